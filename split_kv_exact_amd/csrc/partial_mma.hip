// Partial attention of the split-KV jobs with many query rows (bf16 inputs, fp32 math),
// on the gfx950 matrix cores.
//
// Split-KV page, lede: each context KV block yields a result the size of the queries,
// here for every query row of a unit the block's softmax output O_b and its
// log-sum-exp LSE_b. This kernel runs the jobs whose pass covers at least 8 row tiles
// (128 query rows of one KV head, e.g. long-context and prefill units), where the work
// is a dense contraction: about 2 * rows flops per byte of K and V. The jobs with fewer
// rows, which stream their block, run in partial_bf16.hip.
//
// Execution model
//   * One workgroup of 8 wavefronts (two per SIMD) per workgroup slot of the plan; it
//     walks its list of jobs, each cut into stages of 64 keys. Every wave computes: wave
//     w owns row tiles w and w + 8 of the pass (16 rows each; a pass has 8 to 16 tiles,
//     and a wave whose second tile lies past the pass skips it; rows past the job's last
//     row repeat it and are stored as duplicates of identical values).
//   * Four LDS slots hold stages (a K tile and a V tile each, XOR-swizzled exactly as in
//     the other kernel). Every wave issues one eighth of each stage by direct global->LDS
//     DMA, three stages ahead of the stage computed, after its compute of the current
//     stage (a wave that finishes early issues while the others still compute); the
//     pipeline runs on across job boundaries. One workgroup barrier per stage.
//   * Within a stage a wave takes two steps of 32 keys. The score MFMAs of a step are
//     issued first; the V^T operands of the step are then requested from LDS and their
//     latency passes under the softmax (vector ALU), and the K operands of the next
//     step are requested before the P V MFMAs, under which they arrive.
//   * Q is loaded at the start of a job into registers (global loads; the wait for them
//     also waits for the stage DMA issued before them, once per job).
//   * The arithmetic is that of the other kernel: S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
//     a lane owns one query row and four keys per 16-key tile), online softmax in base 2
//     with a thresholded reference max (p first, the row max only when a lane's sum of
//     p says the reference may move), p rounded to bf16 for O^T += V^T P^T (V^T read
//     with ds_read_b64_tr_b16), O normalised by the MFMA sum of the rounded p, the LSE
//     from the fp32 sum of p. Both kernels give the same result for a job bit for bit.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace splitkv {
namespace {

using namespace lds;

constexpr int NW = 8;    // wavefronts per workgroup, all computing
constexpr int TK = kStageKeys;
constexpr int NST = 4;   // LDS slots
constexpr int AHEAD = 3; // stages in flight ahead of the stage computed
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float RESCALE_LOG2 = 8.f;
constexpr float PSUM_RESCAN = 128.f;  // 2^(RESCALE_LOG2 - 1)
static_assert(TK == 64, "two 32-key steps per stage");
static_assert(AHEAD <= NST - 1, "a slot is refilled after the barrier that ends its last read");

template <int D>
struct Cfg {
  static constexpr int DC = D / 32;                 // 32-dim slices of the QK^T contraction
  static constexpr int DT = D / 16;                 // 16-dim output tiles
  static constexpr int ROWB = 2 * D;                // bytes per key row
  static constexpr int CH = ROWB / 16;              // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;           // rows per 1 KiB DMA instruction
  static constexpr int TILEB = TK * ROWB;           // bytes of a K or V tile
  static constexpr int SLOTB = 2 * TILEB;           // bytes per slot
  static constexpr int KVI = TILEB / 1024 / NW;     // DMA instructions per wave per tile
  static constexpr int NDMA = 2 * KVI;              // DMA instructions per wave per stage
  static constexpr int STORES = DT + 1;             // store instructions per row tile
  static constexpr int LDSB = NST * SLOTB > 96 * 1024 ? NST * SLOTB : 96 * 1024;
  static_assert(KVI >= 1 && KVI * NW * RPI == TK, "DMA covers a tile");
  static_assert(CH <= 16 && 32 % CH == 0, "swizzles repeat every 16 rows");
};

template <int D>
__device__ __forceinline__ int swz_k(int row, int c) { return swz_row<Cfg<D>::CH>(row, c); }
template <int D>
__device__ __forceinline__ int swz_v(int row, int c) { return swz_tr<Cfg<D>::CH>(row, c); }

// Wait until at most n vector-memory instructions of this wave are outstanding, then
// barrier the workgroup. Values past the table wait for everything (always safe).
__device__ __forceinline__ void vm_wait_barrier(int n) {
  switch (__builtin_amdgcn_readfirstlane(n)) {
#define SKV_CASE(N) \
  case N: asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory"); break;
    SKV_CASE(0) SKV_CASE(1) SKV_CASE(2) SKV_CASE(3) SKV_CASE(4) SKV_CASE(5) SKV_CASE(6) SKV_CASE(7)
    SKV_CASE(8) SKV_CASE(9) SKV_CASE(10) SKV_CASE(11) SKV_CASE(12) SKV_CASE(13) SKV_CASE(14) SKV_CASE(15)
    SKV_CASE(16) SKV_CASE(17) SKV_CASE(18) SKV_CASE(19) SKV_CASE(20) SKV_CASE(21) SKV_CASE(22) SKV_CASE(23)
    SKV_CASE(24) SKV_CASE(25) SKV_CASE(26) SKV_CASE(27) SKV_CASE(28) SKV_CASE(29) SKV_CASE(30) SKV_CASE(31)
    SKV_CASE(32) SKV_CASE(33) SKV_CASE(34) SKV_CASE(35) SKV_CASE(36) SKV_CASE(37) SKV_CASE(38) SKV_CASE(39)
    SKV_CASE(40) SKV_CASE(41) SKV_CASE(42) SKV_CASE(43) SKV_CASE(44) SKV_CASE(45) SKV_CASE(46) SKV_CASE(47)
    SKV_CASE(48) SKV_CASE(49) SKV_CASE(50) SKV_CASE(51) SKV_CASE(52) SKV_CASE(53) SKV_CASE(54) SKV_CASE(55)
    SKV_CASE(56) SKV_CASE(57) SKV_CASE(58) SKV_CASE(59) SKV_CASE(60) SKV_CASE(61) SKV_CASE(62)
#undef SKV_CASE
    default: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Transposing V^T reads of one 32-key step, without waiting: the destination
// registers are written when the reads return, and nothing may use them before
// vt_wait. Lane addresses are a[dt] + OFF (keys 0-15 of the step) and + OFF + HI.
template <int OFF, int HI>
__device__ __forceinline__ void vt_issue(i16x4 (&lo)[8], i16x4 (&hi)[8], const unsigned (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\tds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %2, %18 offset:%24\n\tds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %4, %20 offset:%24\n\tds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %22 offset:%24\n\tds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%25\n\tds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%25\n\tds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %20 offset:%25\n\tds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %14, %22 offset:%25\n\tds_read_b64_tr_b16 %15, %23 offset:%25"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(lo[4]), "=&v"(lo[5]), "=&v"(lo[6]),
        "=&v"(lo[7]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]), "=&v"(hi[3]), "=&v"(hi[4]), "=&v"(hi[5]),
        "=&v"(hi[6]), "=&v"(hi[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF),
        "i"(OFF + HI)
      : "memory");
}
template <int OFF, int HI>
__device__ __forceinline__ void vt_issue(i16x4 (&lo)[4], i16x4 (&hi)[4], const unsigned (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\tds_read_b64_tr_b16 %1, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%12\n\tds_read_b64_tr_b16 %3, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n\tds_read_b64_tr_b16 %5, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:%13\n\tds_read_b64_tr_b16 %7, %11 offset:%13"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
        "=&v"(hi[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF), "i"(OFF + HI)
      : "memory");
}
// Every LDS read of this wave has returned. The V^T registers pass through the
// statement, so no use of them can be placed before it.
template <int N>
__device__ __forceinline__ void vt_wait(i16x4 (&lo)[N], i16x4 (&hi)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(lo[i]), "+v"(hi[i]));
}

// Per-lane constant offsets.
template <int D>
struct LaneOff {
  uint32_t dk[Cfg<D>::KVI];  // DMA: this lane's 16 bytes of a full K stage, from the stage's first key
  uint32_t dv[Cfg<D>::KVI];  // the same for V
  int row0;                  // DMA: this lane's row of the stage in its first instruction
  uint32_t kr[Cfg<D>::DC];   // LDS: K operand (key row li, dims 32dc + 8G..+7) of a 16-key tile
  uint32_t vr[Cfg<D>::DT];   // LDS: V^T operand (key row 4G + li/4, dims 16dt + 4(li%4)..+3)
};

template <int D>
__device__ __forceinline__ void lane_offsets(LaneOff<D>& lo, int wave, int lane, uint32_t kst, uint32_t vst) {
  using C = Cfg<D>;
  const int G = lane >> 4, li = lane & 15;
  const int cs = lane % C::CH;
  lo.row0 = wave * C::KVI * C::RPI + lane / C::CH;
#pragma unroll
  for (int in = 0; in < C::KVI; ++in) {
    const int row = lo.row0 + in * C::RPI;
    lo.dk[in] = uint32_t(row) * kst + 16u * swz_k<D>(row, cs);
    lo.dv[in] = uint32_t(row) * vst + 16u * swz_v<D>(row, cs);
  }
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) lo.kr[dc] = li * C::ROWB + 16 * swz_k<D>(li, 4 * dc + G);
  const int e = li >> 2, cc = li & 3, r = 4 * G + e;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) lo.vr[dt] = r * C::ROWB + 16 * swz_v<D>(r, 2 * dt + (cc >> 1)) + 8 * (cc & 1);
}

// The DMA side: the job and stage to issue next.
struct Loader {
  int li;      // position of the job in the workgroup's list
  int stage;   // next stage of that job
  int nst, len, flags;
  const unsigned char* kb;  // K / V address of the next stage's first key
  const unsigned char* vb;
};

// Per-lane byte offsets, from the stage's first key, of this wave's DMA instructions
// for the loader's next stage: K and V rows of its first 1 KiB (parts 0, 1) and of its
// second (parts 2, 3, D = 128 only).
template <int D>
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[4], const Loader& L, const LaneOff<D>& lo,
                                            uint32_t kst, uint32_t vst) {
  using C = Cfg<D>;
  // When the block ends inside the stage, rows past its end re-read its last key
  // (finite data, masked out later): row r reads key min(r, rem - 1), i.e. over rows
  // earlier than the full stage's offset. The swizzle depends on the LDS row only.
  const int last = L.len - L.stage * TK - 1;
#pragma unroll
  for (int in = 0; in < C::KVI; ++in) {
    const uint32_t over = uint32_t(max(lo.row0 + in * C::RPI - last, 0));
    off[2 * in] = lo.dk[in] - over * kst;
    off[2 * in + 1] = lo.dv[in] - over * vst;
  }
}

template <int D>
struct State {
  f32x4 o[2][Cfg<D>::DT];
  bf16x8 q[2][Cfg<D>::DC];
  f32x4 ls[2];   // sum of the bf16-rounded p of this lane's row (every entry equal)
  float m[2];    // running reference max of raw scores
  float thr[2];  // scores above this move the reference: m + RESCALE_LOG2 / c
  float pthr[2]; // a lane whose step sum of p exceeds this looks for such scores
  float nmc[2];  // -m * c (0 while m = -inf)
  float l[2];    // this lane's share of the row sum of the fp32 p
  int lim[2];    // last visible block key of this lane's row
};

template <int D>
__device__ __forceinline__ void reset(State<D>& st) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::DT; ++dt) st.o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m[t] = NEG_INF;
    st.thr[t] = NEG_INF;
    st.pthr[t] = -1.f;
    st.nmc[t] = 0.f;
    st.l[t] = 0.f;
    st.ls[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// K operands of one 32-key step (two 16-key tiles) at byte offset KOFF of the stage.
template <int D, int KOFF>
__device__ __forceinline__ void k_read(bf16x8 (&k)[2][Cfg<D>::DC], const unsigned (&ka)[Cfg<D>::DC]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int dc = 0; dc < Cfg<D>::DC; ++dc)
      k[tt][dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(ka[dc] + KOFF + tt * 16 * Cfg<D>::ROWB));
}

// S^T = K Q^T for the step: s[t][tt] holds row tile t against key tile tt.
template <int D>
__device__ __forceinline__ void scores_tile(f32x4 (&s)[2][2], const State<D>& st, const bf16x8 (&k)[2][Cfg<D>::DC],
                                            int t) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < Cfg<D>::DC; ++dc) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[tt][dc], st.q[t][dc], acc, 0, 0, 0);
    s[t][tt] = acc;
  }
}
// two: the wave's second row tile lies inside the pass (wave-uniform); otherwise its
// work is skipped.
template <int D>
__device__ __forceinline__ void scores(f32x4 (&s)[2][2], const State<D>& st, const bf16x8 (&k)[2][Cfg<D>::DC],
                                       bool two) {
  scores_tile<D>(s, st, k, 0);
  if (two) scores_tile<D>(s, st, k, 1);
}

// Mask, reference max, p = 2^(s*c - m*c): rounded to bf16 into p, fp32 sum into l.
template <int D>
__device__ __forceinline__ void softmax(f32x4 (&s)[2][2], State<D>& st, bf16x4 (&p)[2][2], int key0, bool mask,
                                        bool two, float c, float inv_c) {
  const int G = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t == 1 && !two) break;
    if (mask) {
      // Entry e of key tile tt is step key key0 + 16tt + 4G + e.
      const int d = st.lim[t] - (key0 + 4 * G);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * tt + e > d) s[t][tt][e] = NEG_INF;
    }
    // p first, against the current reference. A score above thr gives p > 2^RESCALE_LOG2,
    // so its lane's sum of p exceeds pthr = 2^(RESCALE_LOG2 - 1) whatever the rounding:
    // only then is the row maximum formed (and the reference moved, and p taken again).
    // While m = -inf, pthr = -1 sends every lane there. The reference therefore moves
    // exactly where a row maximum above thr moves it, without a maximum per step.
    float pe[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[tt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][tt][e], c, st.nmc[t]));
    float ps = ((pe[0][0] + pe[0][1]) + (pe[0][2] + pe[0][3])) + ((pe[1][0] + pe[1][1]) + (pe[1][2] + pe[1][3]));
    if (__any(ps > st.pthr[t])) {
      float mx = fmaxf(fmaxf(s[t][0][0], s[t][0][1]), fmaxf(s[t][0][2], s[t][0][3]));
      mx = fmaxf(mx, fmaxf(fmaxf(s[t][1][0], s[t][1][1]), fmaxf(s[t][1][2], s[t][1][3])));
      mx = max4(mx);
      if (mx > st.thr[t]) {
        const float alpha = st.m[t] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((st.m[t] - mx) * c);
        st.m[t] = mx;
        st.thr[t] = mx + RESCALE_LOG2 * inv_c;
        st.pthr[t] = PSUM_RESCAN;
        st.nmc[t] = -mx * c;
        st.l[t] *= alpha;
        st.ls[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < Cfg<D>::DT; ++dt) st.o[t][dt] *= alpha;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[tt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][tt][e], c, st.nmc[t]));
        ps = ((pe[0][0] + pe[0][1]) + (pe[0][2] + pe[0][3])) + ((pe[1][0] + pe[1][1]) + (pe[1][2] + pe[1][3]));
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) p[t][tt][e] = (__bf16)pe[tt][e];
    st.l[t] += ps;
  }
}

// O^T += V^T P^T for both row tiles, and the rounded p summed on the matrix core.
template <int D>
__device__ __forceinline__ void pv(State<D>& st, const bf16x4 (&p)[2][2], const i16x4 (&vlo)[Cfg<D>::DT],
                                   const i16x4 (&vhi)[Cfg<D>::DT], bool two) {
  const __bf16 one = (__bf16)1.0f;
  const bf16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t == 1 && !two) break;
    const bf16x8 pb = __builtin_shufflevector(p[t][0], p[t][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::DT; ++dt) {
      const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[dt], vhi[dt], 0, 1, 2, 3, 4, 5, 6, 7));
      st.o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb, st.o[t][dt], 0, 0, 0);
    }
    st.ls[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, st.ls[t], 0, 0, 0);
  }
}

// One 64-key stage of this wave (keys key0..key0+63 of the block); mask: some key of
// the stage lies past some row's limit (wave-uniform). The K operands of step A were
// requested before the call.
template <int D>
__device__ __forceinline__ void stage(State<D>& st, bf16x8 (&kA)[2][Cfg<D>::DC], const unsigned (&ka)[Cfg<D>::DC],
                                      const unsigned (&va)[Cfg<D>::DT], int key0, bool mask, bool two, float c,
                                      float inv_c) {
  using C = Cfg<D>;
  f32x4 s[2][2];
  bf16x4 p[2][2];
  i16x4 vlo[C::DT], vhi[C::DT];
  bf16x8 kB[2][C::DC];
  // Step A: scores; this step's V^T requested under the softmax, the next step's K
  // under the P V products. The matrix-core bursts run at raised wave priority, so that
  // of the SIMD's two waves the one with products to issue goes first and the other's
  // softmax fills in behind them (long and mixed 2-3% faster, same GPU).
  __builtin_amdgcn_s_setprio(1);
  scores<D>(s, st, kA, two);
  __builtin_amdgcn_s_setprio(0);
  vt_issue<0, 16 * C::ROWB>(vlo, vhi, va);
  softmax<D>(s, st, p, key0, mask, two, c, inv_c);
  vt_wait(vlo, vhi);
  k_read<D, 32 * C::ROWB>(kB, ka);
  __builtin_amdgcn_s_setprio(1);
  pv<D>(st, p, vlo, vhi, two);
  __builtin_amdgcn_s_setprio(0);
  // Step B.
  __builtin_amdgcn_s_setprio(1);
  scores<D>(s, st, kB, two);
  __builtin_amdgcn_s_setprio(0);
  vt_issue<32 * C::ROWB, 16 * C::ROWB>(vlo, vhi, va);
  softmax<D>(s, st, p, key0 + 32, mask, two, c, inv_c);
  vt_wait(vlo, vhi);
  __builtin_amdgcn_s_setprio(1);
  pv<D>(st, p, vlo, vhi, two);
  __builtin_amdgcn_s_setprio(0);
}

// Query row of tile `tile`, lane row li; rows past the last one repeat it.
__device__ __forceinline__ int tile_row(const JobRec& j, int tile, int li) {
  return min(min(tile, j.tile_lo + j.tile_n - 1) * 16 + li, j.rows - 1);
}

// Normalise and store row tile t (tile index `tile` of the job): DT + 1 store
// instructions with every lane active.
template <int D, bool H16>
__device__ __forceinline__ void write_tile(const State<D>& st, int t, const PartialArgs& a, const JobRec& j, int tile) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float l = sum4(st.l[t]);
  const int row = tile_row(j, tile, li);
  const float ls = st.ls[t][0];
  const float inv = ls > 0.f ? 1.f / ls : 0.f;
  const float lse = l > 0.f ? st.m[t] * a.scale + __builtin_amdgcn_logf(l) * LN2 : NEG_INF;
  float* op;
  float* lp;
  if (a.out != nullptr && (j.flags & kJobSingle)) {
    const int i = row / a.g, hl = row - i * a.g;
    const int64_t idx = (j.q_tok + i) * a.Hq + j.kv * a.g + hl;
    op = a.out + idx * D;
    lp = a.lse + idx;
  } else {
    const int64_t prow = j.ws_row + row;
    if constexpr (H16) {
      store_row_h16<C::DT, false>(st.o[t], inv, lse, reinterpret_cast<_Float16*>(a.ws_o) + prow * D, a.ws_lse + 2 * prow, G);
      return;
    }
    op = a.ws_o + prow * D;
    lp = a.ws_lse + prow;
  }
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
    __builtin_nontemporal_store(st.o[t][dt] * inv, reinterpret_cast<f32x4*>(op + 16 * dt + 4 * G));
  __builtin_nontemporal_store(lse, lp);
}

// PARTIAL: the launch has passes of fewer than 16 row tiles, whose waves skip a second
// tile past the pass; without it every wave always computes two tiles (no branches).
template <int D, bool PARTIAL, bool H16>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void partial_mma_kernel(PartialArgs a, const JobRec* __restrict__ jobs, const int32_t* __restrict__ wjobs,
                        const int32_t* __restrict__ job_ptr, const int32_t* __restrict__ split_ptr) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDSB];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float c = a.scale * LOG2E;
  const float inv_c = 1.f / c;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();

  const uint32_t kst = uint32_t(a.k_st) * 2, vst = uint32_t(a.v_st) * 2;
  LaneOff<D> lo;
  lane_offsets<D>(lo, wave, lane, kst, vst);

  // This workgroup's jobs: wjobs[beg, end).
  const int beg = job_ptr[blockIdx.x];
  const int end = split_ptr[blockIdx.x];

  // Loader: runs AHEAD stages ahead of the compute, across job boundaries.
  Loader L;
  L.li = beg - 1;
  L.stage = L.nst = 0;
  int issued = 0;  // stages issued
  // Vector-memory instructions this wave issued after the DMA of the stage computed next
  // (c[0]) and of the stages after it (c[1], ...), so that a wait drains only what the
  // stage needs. Entries shift by one per stage.
  int cnt[AHEAD + 1] = {};
  auto next_stage = [&]() -> bool {
    if (L.stage >= L.nst) {
      if (L.li + 1 >= end) return false;
      ++L.li;
      const JobRec j = jobs[wjobs[L.li]];
      L.stage = 0;
      L.nst = j.nst;
      L.len = j.len;
      L.flags = j.flags;
      L.kb = reinterpret_cast<const unsigned char*>(a.k) + 2 * (j.kv_tok * a.k_st + int64_t(j.kv) * a.k_sh);
      L.vb = reinterpret_cast<const unsigned char*>(a.v) + 2 * (j.kv_tok * a.v_st + int64_t(j.kv) * a.v_sh);
    }
    return true;
  };
  // Issue the loader's next stage into its slot; false when the list is done.
  auto issue = [&]() -> bool {
    if (!next_stage()) return false;
    unsigned char* slot = smem + (issued % NST) * C::SLOTB;
    uint32_t off[4] = {0, 0, 0, 0};
    if ((L.stage + 1) * TK <= L.len) {
      // A full stage (every stage but a block's ragged last one): the constant offsets.
#pragma unroll
      for (int in = 0; in < C::KVI; ++in) {
        off[2 * in] = lo.dk[in];
        off[2 * in + 1] = lo.dv[in];
      }
    } else {
      dma_offsets<D>(off, L, lo, kst, vst);
    }
#pragma unroll
    for (int part = 0; part < C::NDMA; ++part) {
      const unsigned char* src = ((part & 1) ? L.vb : L.kb) + off[part];
      lds_void* dst = (lds_void*)(slot + ((part & 1) ? C::TILEB : 0) + (wave * C::KVI + (part >> 1)) * 1024);
      // Default cache policy: the passes of a unit (on workgroups of one XCD) share the
      // block through L2; the streaming hint measured 4% slower here.
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
    ++L.stage;
    L.kb += TK * kst;
    L.vb += TK * vst;
    // Every earlier stage now has NDMA more instructions after its own.
#pragma unroll
    for (int x = 0; x <= AHEAD; ++x) cnt[x] += C::NDMA;
    ++issued;
    return true;
  };
  static_assert(AHEAD == 3, "prologue issues three stages");
  if (issue()) {
    cnt[0] = 0;  // the newest issued stage has nothing after it yet
    if (issue()) {
      cnt[1] = 0;
      if (issue()) cnt[2] = 0;
    }
  }

  State<D> st;
  reset<D>(st);
  int ci = beg;  // list position of the job computed
  int jj = 0;    // its stage
  int nst = 0, len = 0;
  int min_lim = 0, max_lim = 0;
  bool two = true;
  for (int s = 0; s < issued; ++s) {
    // Stage s has landed for this wave once only the instructions issued after it are
    // pending; the barrier makes every wave's part visible and frees slot (s - 1) % NST.
    // Steady state: the two stages issued after stage s are all that may be pending.
    if (cnt[0] == (AHEAD - 1) * C::NDMA)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"((AHEAD - 1) * C::NDMA) : "memory");
    else
      vm_wait_barrier(cnt[0]);
#pragma unroll
    for (int x = 0; x < AHEAD; ++x) cnt[x] = cnt[x + 1];
    cnt[AHEAD] = 0;

    if (jj == 0) {
      // Job start: per-row limits and Q operands (global loads, waited for here).
      const JobRec j = jobs[wjobs[ci]];
      nst = j.nst;
      len = j.len;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = tile_row(j, j.tile_lo + wave + 8 * t, li);
        st.lim[t] = min(j.lim0 + row / a.g, j.len - 1);
        const int iq = row / a.g;
        const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (j.q_tok + iq) * a.q_st +
                           int64_t(j.kv * a.g + (row - iq * a.g)) * a.q_sh + 8 * G;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
          st.q[t][dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * dc));
      }
      two = !PARTIAL || wave + 8 < j.tile_n;
      const int r_first = tile_row(j, j.tile_lo + wave, 0);
      const int r_last = tile_row(j, j.tile_lo + wave + 8, 15);
      min_lim = min(j.lim0 + r_first / a.g, j.len - 1);
      max_lim = min(j.lim0 + max(r_first, r_last) / a.g, j.len - 1);
      // Compiler-visible wait for the Q loads (and the DMA issued before them, one stage
      // ahead of this one), before the next stage's DMA is issued.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
      for (int x = 0; x <= AHEAD; ++x) cnt[x] = 0;
    }
    const int key0 = jj * TK;
    if (key0 <= max_lim) {
      const unsigned sb = lds_addr(smem + (s % NST) * C::SLOTB);
      unsigned ka[C::DC], va[C::DT];
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) ka[dc] = sb + lo.kr[dc];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) va[dt] = sb + C::TILEB + lo.vr[dt];
      bf16x8 kA[2][C::DC];
      k_read<D, 0>(kA, ka);
      stage<D>(st, kA, ka, va, key0, key0 + TK - 1 > min_lim, two, c, inv_c);
    }
    if (issue()) cnt[AHEAD - 1] = 0;
    if (++jj == nst) {
      const JobRec j = jobs[wjobs[ci]];
      write_tile<D, H16>(st, 0, a, j, j.tile_lo + wave);
      if (two) write_tile<D, H16>(st, 1, a, j, j.tile_lo + wave + 8);
#pragma unroll
      for (int x = 0; x <= AHEAD; ++x) cnt[x] += (two ? 2 : 1) * C::STORES;
      reset<D>(st);
      ++ci;
      jj = 0;
    }
  }

  if (threadIdx.x == 0 && a.clock != nullptr) {
    a.clock[2 * blockIdx.x] = t_start;
    a.clock[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
#endif
}

}  // namespace

template <int D, bool H16>
static void launch_variant(const PartialArgs& a, bool partial_passes, hipStream_t stream) {
  const dim3 grid(a.num_workers), block(NW * 64);
  if (partial_passes)
    hipLaunchKernelGGL((partial_mma_kernel<D, true, H16>), grid, block, 0, stream, a, a.jobs, a.wjobs, a.job_ptr,
                       a.split_ptr);
  else
    hipLaunchKernelGGL((partial_mma_kernel<D, false, H16>), grid, block, 0, stream, a, a.jobs, a.wjobs, a.job_ptr,
                       a.split_ptr);
}

hipError_t launch_partial_mma(const PartialArgs& a, int head_dim, bool partial_passes, hipStream_t stream) {
  // The partial format is a template parameter, as in the streaming kernel.
  if (head_dim == 128)
    a.h16 ? launch_variant<128, true>(a, partial_passes, stream) : launch_variant<128, false>(a, partial_passes, stream);
  else if (head_dim == 64)
    a.h16 ? launch_variant<64, true>(a, partial_passes, stream) : launch_variant<64, false>(a, partial_passes, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
