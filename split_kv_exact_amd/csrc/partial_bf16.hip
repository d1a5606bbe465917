// Partial attention of split-KV jobs on gfx950 matrix cores (bf16 inputs, fp32 math).
//
// Split-KV page, lede: each context KV block yields a result the size of the
// queries; here that is, for every query row of a unit, the block's softmax output
// O_b and its log-sum-exp LSE_b (natural log). The page describes no kernel; this is
// a CDNA4 design.
//
// Execution model
//   * One workgroup of 8 wavefronts (two per SIMD) per LPT worker, one worker per CU
//     (the LDS footprint admits one workgroup per CU). The planner cuts every unit
//     of the worker into jobs (KV head x pass over at most 256 query rows), and the
//     workgroup walks that job list, each job cut into stages of 64 keys.
//   * A 3-slot LDS pipeline holds stages: each slot has a K tile, a V tile and (for
//     jobs with at most 64 query rows) the job's Q tile. Slots are filled by direct
//     global->LDS DMA (global_load_lds_dwordx4, 16 bytes per lane), issued two stages
//     ahead of the stage being computed and continuing across job boundaries, so
//     about 64 KiB per CU stay in flight without staging registers. A lane's part of
//     a stage sits at a fixed offset from the stage's base address, so issuing a
//     stage costs one scalar add per tensor; only a block's last, partial stage
//     computes clamped offsets.
//   * Only waves 4..7 issue the DMA. Issuing a stage's 32 KiB queues behind the
//     memory pipeline for hundreds of cycles; waves 0..3, which compute every job,
//     never wait there (jobs of fewer than 8 row tiles compute on waves 0..3 alone).
//   * Each stage costs one workgroup barrier. Completion of a stage's DMA is tracked
//     with explicit vmcnt waits: vector-memory instructions complete in issue order,
//     and the kernel counts every one it issues after a stage (the next stage's DMA
//     and the result stores, whose number per finished job is fixed), so a wait never
//     drains more than the stage it needs.
//   * Tiles are stored row-major (one key per 2*D-byte row) with an XOR swizzle of the
//     16-byte chunks, chosen so that both read patterns below are free of LDS bank
//     conflicts and so that a lane's read offsets do not depend on the stage.
//   * Query rows of a KV head are r = i*g + (h - kv*g) (query token i, head h), in
//     16-row tiles. With >= 8 tiles the 8 waves split the tiles (up to 2 each, so 256
//     rows per pass); with 4..7 tiles waves 0..3 split them; with 1..3 tiles waves
//     split the tiles and each stage's keys two ways and merge their results in LDS at
//     the end of the job. Rows past the last query row repeat the last row, so every
//     wave stores whole tiles.
//   * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16, A = 16
//     keys x 32 dims from the K tile, B = 32 dims x 16 rows of Q in registers). A lane
//     then owns one query row and 4 keys per 16-key tile: the row sum needs no
//     cross-lane step until the end of the job.
//   * Output is accumulated transposed, O^T += V^T P^T. P^T comes straight from the
//     score registers (rounded to bf16); V^T is read with ds_read_b64_tr_b16, which
//     hands each lane four keys of one dimension. Pairs of 16-key tiles feed
//     v_mfma_f32_16x16x32_bf16; the key order inside the contraction is permuted
//     identically on both operands, which leaves the sum unchanged.
//   * Softmax runs in base 2 on raw scores: p = 2^(s*c - m*c), c = scale*log2(e), m a
//     running reference max that moves only when a row's scores rise more than 2^8 in
//     p above it. p is taken first; the row max is formed (two cross-lane steps) only
//     when a lane's sum of p exceeds 2^7. The LSE uses the sum of the fp32 p (LSE =
//     scale*m + ln l); O is normalised by the sum of the bf16-rounded p it was
//     accumulated from.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace splitkv {
namespace {

using namespace lds;

constexpr int NW = 8;           // wavefronts per workgroup (two per SIMD)
constexpr int TK = kStageKeys;  // keys per pipeline stage
constexpr int NST = 3;          // pipeline slots
constexpr int RTW = 2;          // row tiles per wave per pass
constexpr int NLW = 4;          // loader waves: waves NW - NLW .. NW - 1 issue all DMA
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float NEG_INF = -__builtin_huge_valf();
static_assert(kPassTiles == NW * RTW, "a pass gives every wave up to RTW row tiles");
static_assert(TK == 64, "a wave's key slice is one or two 32-key steps");

template <int D>
struct Cfg {
  static constexpr int DC = D / 32;                  // 32-dim slices of the QK^T contraction
  static constexpr int DT = D / 16;                  // 16-dim output tiles
  static constexpr int ROWB = 2 * D;                 // bytes per key row
  static constexpr int CH = ROWB / 16;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;            // rows per 1 KiB DMA instruction
  static constexpr int TILEB = TK * ROWB;            // bytes of a K or V tile
  static constexpr int QTILEB = kQTileRows * ROWB;   // bytes of a Q tile
  static constexpr int SLOTB = 2 * TILEB + QTILEB;   // bytes per pipeline slot
  static constexpr int KV_INST = TILEB / 1024 / NLW;  // DMA instructions per loader wave per K (or V) tile
  static constexpr int Q_INST = QTILEB / 1024 / NLW;  // DMA instructions per loader wave per Q tile
  static constexpr int MSLOT = 64 * (DT * 4 + 3);    // floats of one merge record (m, l, ls, O)
  static constexpr int STORES = DT + 1;              // store instructions per finished row tile
  // At least 96 KiB so that a compute unit holds a single workgroup.
  static constexpr int LDSB = NST * SLOTB > 96 * 1024 ? NST * SLOTB : 96 * 1024;
  static_assert(4 * MSLOT * 4 <= SLOTB, "a merge round's records fit in one slot");
  static_assert(KV_INST >= 1 && Q_INST >= 1, "tile sizes");
  static_assert(CH <= 16 && 32 % CH == 0, "swizzles repeat every 16 rows");
};

// XOR swizzles of the 16-byte chunk index within a row: conflict-free 16-lane row
// reads (K, Q) and 32-lane transposing reads (V). Both depend on the row modulo 16
// only, and tiles start at multiples of 16 rows.
template <int D>
__device__ __forceinline__ int swz_k(int row, int c) { return swz_row<Cfg<D>::CH>(row, c); }
template <int D>
__device__ __forceinline__ int swz_v(int row, int c) { return swz_tr<Cfg<D>::CH>(row, c); }

// Wait until at most n vector-memory instructions of this wave are outstanding, then
// barrier the workgroup (no fence: the pipeline's later DMA must stay in flight).
// Values past the table wait for everything, which is always safe.
__device__ __forceinline__ void wait_vm_barrier(int n) {
  switch (n) {
#define SKV_CASE(N) \
  case N: asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory"); break;
    SKV_CASE(0) SKV_CASE(1) SKV_CASE(2) SKV_CASE(3) SKV_CASE(4) SKV_CASE(5) SKV_CASE(6) SKV_CASE(7)
    SKV_CASE(8) SKV_CASE(9) SKV_CASE(10) SKV_CASE(11) SKV_CASE(12) SKV_CASE(13) SKV_CASE(14) SKV_CASE(15)
    SKV_CASE(16) SKV_CASE(17) SKV_CASE(18) SKV_CASE(19) SKV_CASE(20) SKV_CASE(21) SKV_CASE(22) SKV_CASE(23)
    SKV_CASE(24) SKV_CASE(25) SKV_CASE(26) SKV_CASE(27) SKV_CASE(28) SKV_CASE(29) SKV_CASE(30) SKV_CASE(31)
    SKV_CASE(32) SKV_CASE(33) SKV_CASE(34) SKV_CASE(35) SKV_CASE(36) SKV_CASE(37) SKV_CASE(38) SKV_CASE(39)
    SKV_CASE(40) SKV_CASE(41) SKV_CASE(42) SKV_CASE(43) SKV_CASE(44) SKV_CASE(45) SKV_CASE(46) SKV_CASE(47)
#undef SKV_CASE
    default: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// The same, with the two counts of the steady state (a stage's DMA with and without
// a Q tile) tested first.
template <int D>
__device__ __forceinline__ void wait_stage(int n) {
  constexpr int NKV = 2 * Cfg<D>::KV_INST, NQ = Cfg<D>::Q_INST;
  if (n == NKV)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(NKV) : "memory");
  else if (n == NKV + NQ)
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(NKV + NQ) : "memory");
  else
    wait_vm_barrier(__builtin_amdgcn_readfirstlane(n));  // opaque: keeps the tests above out of the switch
}

// LDS writes and reads of this wave done, then barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Per-lane constant offsets.
template <int D>
struct LaneOff {
  uint32_t dk[Cfg<D>::KV_INST];  // DMA: this lane's 16 bytes of a full K stage, from the stage base
  uint32_t dv[Cfg<D>::KV_INST];  // the same for V
  uint32_t kr[Cfg<D>::DC];       // LDS: K operand (key row li, dims 32dc + 8G..+7) in a 16-key tile
  uint32_t vr[Cfg<D>::DT];       // LDS: V^T operand (key row 4G + li/4, dims 16dt + 4(li%4)..+3)
};

// Loader wave index (0..NLW-1), or -1 for a wave that issues no DMA.
__device__ __forceinline__ int loader_index(int wave) { return wave >= NW - NLW ? wave - (NW - NLW) : -1; }

template <int D>
__device__ __forceinline__ void lane_offsets(LaneOff<D>& lo, int wave, int lane, uint32_t kst, uint32_t vst) {
  using C = Cfg<D>;
  const int G = lane >> 4, li = lane & 15;
  const int cs = lane % C::CH;
  const int lw = max(loader_index(wave), 0);
#pragma unroll
  for (int in = 0; in < C::KV_INST; ++in) {
    const int row = (lw * C::KV_INST + in) * C::RPI + lane / C::CH;
    lo.dk[in] = uint32_t(row) * kst + 16u * swz_k<D>(row, cs);
    lo.dv[in] = uint32_t(row) * vst + 16u * swz_v<D>(row, cs);
  }
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) lo.kr[dc] = li * C::ROWB + 16 * swz_k<D>(li, 4 * dc + G);
  const int e = li >> 2, cc = li & 3, r = 4 * G + e;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) lo.vr[dt] = r * C::ROWB + 16 * swz_v<D>(r, 2 * dt + (cc >> 1)) + 8 * (cc & 1);
}

// The DMA side of the pipeline: the job and stage to issue next.
struct Loader {
  int job;       // job being loaded
  int stage;     // next stage of that job
  int nst, len, flags;
  const unsigned char* kb;  // K / V address of the next stage's first key, this job's KV head
  const unsigned char* vb;
};

__device__ __forceinline__ void open_job(Loader& L, const PartialArgs& a, const JobRec* __restrict__ jobs) {
  const JobRec j = jobs[L.job];
  L.stage = 0;
  L.nst = j.nst;
  L.len = j.len;
  L.flags = j.flags;
  L.kb = reinterpret_cast<const unsigned char*>(a.k) + 2 * (j.kv_tok * a.k_st + int64_t(j.kv) * a.k_sh);
  L.vb = reinterpret_cast<const unsigned char*>(a.v) + 2 * (j.kv_tok * a.v_st + int64_t(j.kv) * a.v_sh);
}

// The K and V DMA of one stage with cache policy AUX (0, or 2 = non-temporal).
template <int D, int AUX>
__device__ __forceinline__ void issue_kv(const Loader& L, unsigned char* slot, const LaneOff<D>& lo, int wave,
                                         int lane, uint32_t kst, uint32_t vst) {
  using C = Cfg<D>;
  const int lw = loader_index(wave);
  if (lw < 0) return;
  const int rem = L.len - L.stage * TK;  // keys of the block from this stage's first key on
  if (rem >= TK) {
#pragma unroll
    for (int in = 0; in < C::KV_INST; ++in) {
      const int gi = lw * C::KV_INST + in;
      __builtin_amdgcn_global_load_lds(L.kb + lo.dk[in], (lds_void*)(slot + gi * 1024), 16, 0, AUX);
      __builtin_amdgcn_global_load_lds(L.vb + lo.dv[in], (lds_void*)(slot + C::TILEB + gi * 1024), 16, 0, AUX);
    }
  } else {
    // The block ends inside this stage: rows past its end re-read its last key (finite
    // data, masked out later).
    const int cs = lane % C::CH;
#pragma unroll
    for (int in = 0; in < C::KV_INST; ++in) {
      const int gi = lw * C::KV_INST + in;
      const int row = gi * C::RPI + lane / C::CH;
      const uint32_t t = uint32_t(min(row, rem - 1));
      __builtin_amdgcn_global_load_lds(L.kb + (t * kst + 16u * swz_k<D>(row, cs)), (lds_void*)(slot + gi * 1024),
                                       16, 0, AUX);
      __builtin_amdgcn_global_load_lds(L.vb + (t * vst + 16u * swz_v<D>(row, cs)),
                                       (lds_void*)(slot + C::TILEB + gi * 1024), 16, 0, AUX);
    }
  }
}

// Issue the DMA of the loader's next stage into one pipeline slot (loader waves) and
// advance the loader (every wave); returns the number of vector-memory instructions
// this wave issued.
template <int D>
__device__ __forceinline__ int issue_stage(const PartialArgs& a, const JobRec* __restrict__ jobs, Loader& L,
                                           unsigned char* slot, const LaneOff<D>& lo, int wave, int lane,
                                           uint32_t kst, uint32_t vst) {
  using C = Cfg<D>;
  if (L.flags & kJobStream)
    issue_kv<D, 2>(L, slot, lo, wave, lane, kst, vst);
  else
    issue_kv<D, 0>(L, slot, lo, wave, lane, kst, vst);
  const int lw = loader_index(wave);
  int n = lw >= 0 ? 2 * C::KV_INST : 0;
  if (L.stage == 0 && (L.flags & kJobQTile) && lw >= 0) {
    // The job's query rows (at most 64) ride with its first stage; rows past the last
    // one repeat it.
    const JobRec j = jobs[L.job];
    const unsigned char* qb =
        reinterpret_cast<const unsigned char*>(a.q) + 2 * (j.q_tok * a.q_st + int64_t(j.kv) * a.g * a.q_sh);
    const uint32_t qst = uint32_t(a.q_st) * 2, qsh = uint32_t(a.q_sh) * 2;
    const int cs = lane % C::CH;
#pragma unroll
    for (int in = 0; in < C::Q_INST; ++in) {
      const int gi = lw * C::Q_INST + in;
      const int row = gi * C::RPI + lane / C::CH;
      const int rr = min(row, j.rows - 1);
      const int i = rr / a.g, hl = rr - i * a.g;
      __builtin_amdgcn_global_load_lds(qb + (uint32_t(i) * qst + uint32_t(hl) * qsh + 16u * swz_k<D>(row, cs)),
                                       (lds_void*)(slot + 2 * C::TILEB + gi * 1024), 16, 0, 0);
    }
    n += C::Q_INST;
  }
  ++L.stage;
  L.kb += TK * kst;
  L.vb += TK * vst;
  return n;
}

// The compute side: the job being computed and this wave's share of it. The job's
// record itself is read again where it is needed (scalar loads), which keeps the
// stage loop's scalar registers free.
struct Work {
  int job, nst;          // job index; its stages
  int wr_log, Wk;        // row groups 2^wr_log, key slices Wk
  int rg, ks, nt;        // this wave's row group, key slice, row tiles (<= RTW)
  int tkw, tok_w;        // keys per stage of this wave's slice, and its first key in the stage
  int min_lim, max_lim;  // last visible block key of this wave's first / last row
};

// Query row of tile `tile`, lane row li, with rows past the last repeating it.
__device__ __forceinline__ int tile_row(const JobRec& j, int tile, int li) { return min(tile * 16 + li, j.rows - 1); }

// Start job w.job (record j) and derive this wave's share.
__device__ __forceinline__ void open_work(Work& w, const JobRec& j, int wave, int g) {
  w.nst = j.nst;
  // Waves split the row tiles 2^wr_log ways and each stage's keys Wk ways
  // (2^wr_log * Wk <= NW; the other waves compute nothing in this job). With 4..7
  // tiles only waves 0..3 compute, so that the loader waves 4..7 stay free.
  w.wr_log = j.flags & kJobWrMask;
  w.Wk = w.wr_log >= 2 ? 1 : 2;
  const int Wr = 1 << w.wr_log;
  w.rg = wave & (Wr - 1);
  w.ks = wave >> w.wr_log;
  const int ntw = w.ks < w.Wk ? (j.tile_n - w.rg + Wr - 1) >> w.wr_log : 0;
  w.nt = min(max(ntw, 0), RTW);
  w.tkw = TK / w.Wk;
  w.tok_w = w.ks * w.tkw;
  const int first = tile_row(j, j.tile_lo + w.rg, 0);
  const int last = tile_row(j, j.tile_lo + w.rg + max(w.nt - 1, 0) * Wr, 15);
  w.min_lim = min(j.lim0 + first / g, j.len - 1);
  w.max_lim = min(j.lim0 + last / g, j.len - 1);
}

template <int D>
struct State {
  f32x4 o[RTW][Cfg<D>::DT];
  bf16x8 q[RTW][Cfg<D>::DC];
  f32x4 ls[RTW];   // sum of the bf16-rounded p of this lane's row (every entry equal)
  float m[RTW];    // running reference max of raw scores (row of this lane)
  float thr[RTW];  // scores above this move the reference: m + RESCALE_LOG2 / c
  float pthr[RTW]; // a lane whose step sum of p exceeds this looks for such scores
  float nmc[RTW];  // -m * c (0 while m = -inf)
  float l[RTW];    // this lane's share of the row sum of the fp32 p
  int lim[RTW];    // last visible block key of this lane's row
};

// Empty accumulators for the next job. Done right after a job's results are stored
// (not at the next job's first stage), so that the accumulators flow around the stage
// loop in the same registers.
template <int D>
__device__ __forceinline__ void reset(State<D>& st) {
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
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

// The running reference max m moves only when a row's max exceeds it by more than
// RESCALE_LOG2 in base 2 (then O and l are rescaled); otherwise p = 2^(s*c - m*c) may
// reach 2^RESCALE_LOG2, which fp32 and bf16 hold exactly in range. O, l and LSE all use
// the same reference, so the result does not depend on when it moved.
constexpr float RESCALE_LOG2 = 8.f;
constexpr float PSUM_RESCAN = 128.f;  // 2^(RESCALE_LOG2 - 1)

// One online-softmax step of this wave: its nt row tiles against 32 keys (block keys
// key0..key0+31), in three phases: scores (matrix cores), softmax (vector ALUs),
// P V (matrix cores). ka / va are the stage's K / V operand addresses of the wave's
// first key; the step's keys start KOFF rows later. (Interleaving the two steps of a
// 64-key stage needs more registers than a wave has at two waves per SIMD.)
constexpr int NT = 2;  // 16-key tiles per step

template <int D>
struct Scores {
  f32x4 s[RTW][NT];
};

// S^T = K Q^T for each 16-key tile, shared K operands across the row tiles.
template <int D, int KOFF>
__device__ __forceinline__ void step_scores(Scores<D>& S, const State<D>& st, int nt, const unsigned (&ka)[Cfg<D>::DC]) {
  using C = Cfg<D>;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    bf16x8 kop[C::DC];
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc)
      kop[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(ka[dc] + (KOFF + 16 * tt) * C::ROWB));
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      if (t < nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[dc], st.q[t][dc], acc, 0, 0, 0);
        S.s[t][tt] = acc;
      }
    }
  }
}

// Mask, p = 2^(s*c - m*c) rounded to bf16 for the P V product, the reference max moved
// when a score rises far enough above it; the row sum of the fp32 p goes to l.
template <int D>
__device__ __forceinline__ void step_softmax(Scores<D>& S, State<D>& st, int nt, bf16x4 (&p)[RTW][NT], int key0,
                                             bool need_mask, float c, float inv_c) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4;
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    if (t < nt) {
      if (need_mask) {
        // Entry e of tile tt is block key key0 + 16tt + 4G + e.
        const int d = st.lim[t] - (key0 + 4 * G);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * tt + e > d) S.s[t][tt][e] = NEG_INF;
      }
      // p first, against the current reference. A score above thr gives p > 2^RESCALE_LOG2,
      // so its lane's sum of p exceeds pthr = 2^(RESCALE_LOG2 - 1) whatever the rounding:
      // only then is the row max formed across the row's four lanes, the reference moved
      // (and O, l rescaled) if the max exceeds thr, and p taken again. While m = -inf,
      // pthr = -1 sends every lane there (-inf -> finite always moves). The reference so
      // moves exactly where a per-step row max would move it.
      float pe[NT][4];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[tt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S.s[t][tt][e], c, st.nmc[t]));
      float ps = ((pe[0][0] + pe[0][1]) + (pe[0][2] + pe[0][3])) + ((pe[1][0] + pe[1][1]) + (pe[1][2] + pe[1][3]));
      if (__any(ps > st.pthr[t])) {
        float mx = fmaxf(fmaxf(S.s[t][0][0], S.s[t][0][1]), fmaxf(S.s[t][0][2], S.s[t][0][3]));
        mx = fmaxf(mx, fmaxf(fmaxf(S.s[t][1][0], S.s[t][1][1]), fmaxf(S.s[t][1][2], S.s[t][1][3])));
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
          for (int dt = 0; dt < C::DT; ++dt) st.o[t][dt] *= alpha;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) pe[tt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(S.s[t][tt][e], c, st.nmc[t]));
          ps = ((pe[0][0] + pe[0][1]) + (pe[0][2] + pe[0][3])) + ((pe[1][0] + pe[1][1]) + (pe[1][2] + pe[1][3]));
        }
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[t][tt][e] = (__bf16)pe[tt][e];
      st.l[t] += ps;
    }
  }
}

// O^T += V^T P^T, and the rounded p summed on the matrix core (an all-ones V^T tile:
// exact fp32 accumulation, already reduced across lanes). O is normalised by that sum,
// so it is a convex combination of the values even when one key dominates.
template <int D, int KOFF>
__device__ __forceinline__ void step_pv(State<D>& st, int nt, const bf16x4 (&p)[RTW][NT],
                                        const unsigned (&va)[Cfg<D>::DT]) {
  using C = Cfg<D>;
  i16x4 lo[C::DT], hi[C::DT];
  tr_read<KOFF * C::ROWB, 16 * C::ROWB>(lo, hi, va);
  bf16x8 vop[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
    vop[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[dt], hi[dt], 0, 1, 2, 3, 4, 5, 6, 7));
  const __bf16 one = (__bf16)1.0f;
  const bf16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    if (t < nt) {
      const bf16x8 pb = __builtin_shufflevector(p[t][0], p[t][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        st.o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pb, st.o[t][dt], 0, 0, 0);
      st.ls[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, st.ls[t], 0, 0, 0);
    }
  }
}

// The wave's keys of one stage: 32 keys (one step) or 64 (two steps, interleaved).
template <int D>
__device__ __forceinline__ void stage_compute(State<D>& st, int nt, bool two_steps, const unsigned (&ka)[Cfg<D>::DC],
                                              const unsigned (&va)[Cfg<D>::DT], int key0, bool need_mask, float c,
                                              float inv_c) {
  {
    Scores<D> S;
    bf16x4 p[RTW][NT];
    step_scores<D, 0>(S, st, nt, ka);
    step_softmax<D>(S, st, nt, p, key0, need_mask, c, inv_c);
    step_pv<D, 0>(st, nt, p, va);
  }
  if (two_steps) {
    Scores<D> S;
    bf16x4 p[RTW][NT];
    step_scores<D, 32>(S, st, nt, ka);
    step_softmax<D>(S, st, nt, p, key0 + 32, need_mask, c, inv_c);
    step_pv<D, 32>(st, nt, p, va);
  }
}

// Normalise and store one row tile of a finished job (row li of the tile, dims
// 16dt+4G..+3): Cfg<D>::STORES store instructions with every lane active. Lanes of
// rows past the last query row store that row's values again.
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
      store_row_h16<C::DT, true>(st.o[t], inv, lse, reinterpret_cast<_Float16*>(a.ws_o) + prow * D, a.ws_lse + 2 * prow, G);
      return;
    }
    op = a.ws_o + prow * D;
    lp = a.ws_lse + prow;
  }
#pragma unroll
  // Non-temporal stores: no later job of the launch reads the results, and they leave
  // less for the caches to write back when the kernel ends (measured 2-3% faster).
  for (int dt = 0; dt < C::DT; ++dt)
    __builtin_nontemporal_store(st.o[t][dt] * inv, reinterpret_cast<f32x4*>(op + 16 * dt + 4 * G));
  __builtin_nontemporal_store(lse, lp);
}

// Finish the job right after its last stage: combine its key slices (Wk > 1) through
// the LDS slot that stage used, then store every row tile. The slot is next written by
// DMA only after the following iteration's barrier. Returns the number of store
// instructions this wave issued.
template <int D, bool H16>
__device__ __forceinline__ int finish_job(State<D>& st, const PartialArgs& a, const Work& w, const JobRec& j,
                                          unsigned char* slot, float c) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int Wr = 1 << w.wr_log;
  if (w.Wk == 1) {
#pragma unroll
    for (int t = 0; t < RTW; ++t)
      if (t < w.nt) write_tile<D, H16>(st, t, a, j, j.tile_lo + w.rg + t * Wr);
    return w.nt * C::STORES;
  }
  // Two key slices per row group; one round per tile index (<= Wr records each). The
  // loop is unrolled with compile-time tile indices: a runtime index would put the
  // wave state in scratch memory.
  float* mbuf = reinterpret_cast<float*>(slot);
  const int rounds = (j.tile_n + Wr - 1) >> w.wr_log;
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    if (t >= rounds) break;
    lds_barrier();  // all waves are done with the slot's tiles / the previous round
    if (w.ks == 1 && t < w.nt) {
      float* rec = mbuf + w.rg * C::MSLOT;
      rec[lane] = st.m[t];
      rec[64 + lane] = st.l[t];
      rec[128 + lane] = st.ls[t][0];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) rec[(3 + dt * 4 + q4) * 64 + lane] = st.o[t][dt][q4];
    }
    lds_barrier();
    if (w.ks == 0 && t < w.nt) {
      const float* rec = mbuf + w.rg * C::MSLOT;
      const float m2 = rec[lane];
      const float ms = fmaxf(st.m[t], m2);
      if (ms != NEG_INF) {
        const float a1 = __builtin_amdgcn_exp2f((st.m[t] - ms) * c);
        const float a2 = __builtin_amdgcn_exp2f((m2 - ms) * c);
        st.l[t] = st.l[t] * a1 + rec[64 + lane] * a2;
        const float ls2 = st.ls[t][0] * a1 + rec[128 + lane] * a2;
        st.ls[t] = f32x4{ls2, ls2, ls2, ls2};
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            st.o[t][dt][q4] = st.o[t][dt][q4] * a1 + rec[(3 + dt * 4 + q4) * 64 + lane] * a2;
        st.m[t] = ms;
      }
      write_tile<D, H16>(st, t, a, j, j.tile_lo + w.rg + t * Wr);
    }
  }
  return w.ks == 0 ? w.nt * C::STORES : 0;
}

// Where the workgroup's jobs come from (identical in every wave): first its plan
// worker's list without the jobs of the shared tail; then, with the queue schedule,
// chunks of the tail drawn from the sub-queue counters shared by all workgroups.
struct Feed {
  int sbeg, send;  // the rest of the static list in wjobs
  int cbeg, cend;  // the rest of the current chunk
  int npop;        // pops so far
  int qk;          // sub-queues found empty (they are tried in turn from this workgroup's own)
};

// Compute-side queue of the jobs the loader has started (at most three: the stage
// being computed and two stages in flight can belong to three different jobs).
struct Started {
  int j0, j1, j2, n;
};

__device__ __forceinline__ void started_push(Started& S, int j) {
  if (S.n == 0)
    S.j0 = j;
  else if (S.n == 1)
    S.j1 = j;
  else
    S.j2 = j;
  ++S.n;
}

__device__ __forceinline__ void started_pop(Started& S) {
  S.j0 = S.j1;
  S.j1 = S.j2;
  --S.n;
}

// QUEUE: after its static list, the workgroup draws chunks of the shared tail. A
// template parameter, so that the static kernel holds no queue code at all.
template <int D, bool QUEUE, bool H16>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void partial_bf16_kernel(PartialArgs a, const JobRec* __restrict__ jobs, const int32_t* __restrict__ wjobs,
                         const int32_t* __restrict__ job_ptr, const int32_t* __restrict__ chunk_ptr) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel's signature
  using C = Cfg<D>;
  // One LDS object: the pipeline slots, then two words for drawn chunk numbers. (A
  // separate __shared__ variable makes the compiler wait for the DMA before LDS reads.)
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDSB + 16];
  int* const s_pop = reinterpret_cast<int*>(smem + C::LDSB);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float c = a.scale * LOG2E;
  const float inv_c = 1.f / c;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  constexpr bool queue = QUEUE;

  const uint32_t kst = uint32_t(a.k_st) * 2, vst = uint32_t(a.v_st) * 2;  // bytes per token
  LaneOff<D> lo;
  lane_offsets<D>(lo, wave, lane, kst, vst);

  Feed F;
  F.sbeg = a.split_ptr[blockIdx.x];  // the jobs before it run in the matrix-path launch
  F.send = job_ptr[blockIdx.x + 1];
  F.cbeg = F.cend = 0;
  F.npop = 0;
  F.qk = 0;

  // Vector-memory instructions this wave issued after the most recent stage's DMA (c1)
  // and after the stage before it (c2).
  int c1 = 0, c2 = 0;
  Loader L;
  L.stage = L.nst = 0;  // no job yet
  int issued = 0, slot_l = 0;
  Started S;
  S.n = 0;

  // Next job for the loader, or -1. Drawing a chunk is synchronous: wave 0 waits for
  // its atomic (only its own few memory operations are older than the wait, it issues
  // its share of the DMA afterwards) and the workgroup meets at one barrier. Every
  // wave takes the same branches, so all of them reach that barrier.
  auto next_job = [&]() -> int {
    // Static list; jobs of the shared tail in it are skipped (the tail is drawn below).
    while (F.sbeg < F.send) {
      const int j = wjobs[__builtin_amdgcn_readfirstlane(F.sbeg)];
      ++F.sbeg;
      if (j < a.tail_start) return j;
    }
    if constexpr (queue) {
      while (F.cbeg == F.cend && F.qk < kQueues) {
        const int qi = (int(blockIdx.x) + F.qk) % kQueues;
        if (wave == 0) {
          if (lane == 0)
            s_pop[F.npop & 1] = int(__hip_atomic_fetch_add(a.sched + qi * kSchedStride, 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT));
        }
        lds_barrier();
        const int ch = __builtin_amdgcn_readfirstlane(s_pop[F.npop & 1]) * kQueues + qi;
        ++F.npop;
        if (ch < a.num_chunks) {
          F.cbeg = chunk_ptr[ch];
          F.cend = chunk_ptr[ch + 1];
        } else {
          ++F.qk;  // this sub-queue is empty; try the next one
        }
      }
      if (F.cbeg < F.cend) return F.cbeg++;
    }
    return -1;
  };
  auto ready = [&](int target) {
    if (issued >= target) return false;
    if (L.stage < L.nst) return true;
    const int j = next_job();
    if (j < 0) return false;
    L.job = j;
    open_job(L, a, jobs);
    started_push(S, j);
    return true;
  };
  // Issue stages until `target` stages are issued or the workgroup has no more jobs.
  auto loader_step = [&](int target) {
    while (ready(target)) {
      const int n = issue_stage<D>(a, jobs, L, smem + slot_l * C::SLOTB, lo, wave, lane, kst, vst);
      ++issued;
      slot_l = slot_l == NST - 1 ? 0 : slot_l + 1;
      c2 = c1 + n;
      c1 = 0;
    }
  };

  loader_step(NST - 1);

  Work w;
  State<D> st;
  reset<D>(st);
  int slot_c = 0;  // slot of the stage computed
  int jj = 0;      // stage within the compute job
  for (int i = 0;; ++i) {
    if (i >= issued) break;  // the loader is done and every stage computed
    // Stage i landed (for every wave) once the later stages' DMA and the stores after
    // them are all that is pending; stage i + 1, if issued, is the most recent stage.
    wait_stage<D>(issued > i + 1 ? c2 : c1);
    unsigned char* slot = smem + slot_c * C::SLOTB;

    if (jj == 0) {
      // Job start: this wave's share, per-row limits and Q operands.
      w.job = S.j0;
      const JobRec j = jobs[w.job];
      open_work(w, j, wave, a.g);
      const int Wr = 1 << w.wr_log;
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        const int row = tile_row(j, j.tile_lo + w.rg + t * Wr, li);
        st.lim[t] = min(j.lim0 + row / a.g, j.len - 1);
      }
      if (!(j.flags & kJobQTile)) {
        // Q from HBM, loaded before this iteration's DMA is issued.
#pragma unroll
        for (int t = 0; t < RTW; ++t) {
          const int row = tile_row(j, j.tile_lo + w.rg + t * Wr, li);
          const int iq = row / a.g;
          const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (j.q_tok + iq) * a.q_st +
                             int64_t(j.kv * a.g + (row - iq * a.g)) * a.q_sh + 8 * G;
#pragma unroll
          for (int dc = 0; dc < C::DC; ++dc)
            st.q[t][dc] = t < w.nt ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * dc))
                                   : bf16x8{};
        }
        // Complete these loads here. A compiler-visible wait, so that no load into the Q
        // registers is pending anywhere else in the loop: otherwise every later use of
        // them would wait for all in-flight DMA. Nothing this wave issued is pending
        // after it.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        c1 = 0;
        c2 = 0;
      } else {
        // The Q tile of this slot holds rows 0..63 of the job.
#pragma unroll
        for (int t = 0; t < RTW; ++t) {
          const int tile = j.tile_lo + w.rg + t * Wr;
          const unsigned qa = lds_addr(slot + 2 * C::TILEB) + unsigned(t < w.nt ? tile : 0) * (16 * C::ROWB);
#pragma unroll
          for (int dc = 0; dc < C::DC; ++dc) st.q[t][dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(qa + lo.kr[dc]));
        }
      }
    }

    loader_step(i + NST);

    // This wave's keys of the stage: block keys [key0, key0 + tkw).
    const int key0 = jj * TK + w.tok_w;
    if (w.nt > 0 && key0 <= w.max_lim) {
      const bool need_mask = key0 + w.tkw - 1 > w.min_lim;
      const unsigned sb = lds_addr(slot) + unsigned(w.tok_w) * C::ROWB;
      unsigned ka[C::DC], va[C::DT];
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) ka[dc] = sb + lo.kr[dc];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) va[dt] = sb + C::TILEB + lo.vr[dt];
      stage_compute<D>(st, w.nt, w.tkw == TK, ka, va, key0, need_mask, c, inv_c);
    }
    if (jj + 1 == w.nst) {
      const int s = finish_job<D, H16>(st, a, w, jobs[w.job], slot, c);
      c1 += s;
      c2 += s;
      reset<D>(st);
      started_pop(S);
      jj = 0;
    } else {
      ++jj;
    }
    slot_c = slot_c == NST - 1 ? 0 : slot_c + 1;
  }

  if (threadIdx.x == 0) {
    if (a.clock != nullptr) {
      // After the matrix-path launch, the start is moved back by that launch's busy time,
      // so that end - start is the workgroup's busy time in both launches.
      const uint64_t prev = a.clock_add ? a.clock[2 * blockIdx.x + 1] - a.clock[2 * blockIdx.x] : 0;
      a.clock[2 * blockIdx.x] = t_start - prev;
      a.clock[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
    }
    if constexpr (queue) {
      // The last workgroup to finish (every pop of every workgroup has returned by
      // then) leaves the queue counters zero for the next launch.
      uint32_t* const done_ctr = a.sched + kQueues * kSchedStride;
      const unsigned done = __hip_atomic_fetch_add(done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == gridDim.x - 1) {
        for (int qi = 0; qi < kQueues; ++qi)
          __hip_atomic_store(a.sched + qi * kSchedStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(done_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
#endif
}

}  // namespace

template <int D, bool H16>
static void launch_variant(const PartialArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_workers), block(NW * 64);
  if (a.queue)
    hipLaunchKernelGGL((partial_bf16_kernel<D, true, H16>), grid, block, 0, stream, a, a.jobs, a.wjobs, a.job_ptr,
                       a.chunk_ptr);
  else
    hipLaunchKernelGGL((partial_bf16_kernel<D, false, H16>), grid, block, 0, stream, a, a.jobs, a.wjobs, a.job_ptr,
                       a.chunk_ptr);
}

hipError_t launch_partial_bf16(const PartialArgs& a, int head_dim, hipStream_t stream) {
  // The partial format is a template parameter, so that the store path it selects adds
  // nothing to the streaming loop's scalar registers (the loop runs near the SGPR limit;
  // more live scalars spill to VGPR lanes inside it).
  if (head_dim == 128)
    a.h16 ? launch_variant<128, true>(a, stream) : launch_variant<128, false>(a, stream);
  else if (head_dim == 64)
    a.h16 ? launch_variant<64, true>(a, stream) : launch_variant<64, false>(a, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
