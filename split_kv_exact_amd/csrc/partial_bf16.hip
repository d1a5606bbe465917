// Partial attention of split-KV units on gfx950 matrix cores (bf16 inputs, fp32 math).
//
// Split-KV page, lede: each context KV block yields a result the size of the
// queries; here that is, for every query row of a unit, the block's softmax output
// O_b and its log-sum-exp LSE_b (natural log). The page describes no kernel; this is
// a CDNA4 design.
//
// Execution model
//   * One workgroup (4 wavefronts, one per SIMD) per LPT worker, one worker per CU
//     (the LDS footprint admits one workgroup per CU). The workgroup walks its unit
//     list in plan order as a flat sequence of "jobs" (unit x KV head x row pass),
//     each cut into stages of 64 keys.
//   * A 3-slot LDS pipeline holds stages: each slot has a K tile, a V tile and (for
//     units with at most 64 query rows) the unit's Q tile. Slots are filled by
//     direct global->LDS DMA (global_load_lds_dwordx4, 16 bytes per lane), issued two
//     stages ahead of the stage being computed and continuing across unit
//     boundaries, so about 64 KiB per CU stay in flight without staging registers.
//     Each stage costs one workgroup barrier; completion of a stage's DMA is tracked
//     with explicit vmcnt waits (loads complete in issue order).
//   * Tiles are stored row-major (one key per 2*D-byte row) with an XOR swizzle of the
//     16-byte chunks, chosen so that both read patterns below are free of LDS bank
//     conflicts.
//   * Query rows of a KV head are r = i*g + (h - kv*g) (query token i, head h), in
//     16-row tiles. With >= 4 tiles the 4 waves split the tiles (up to 4 per wave per
//     pass, so 256 rows per pass); with fewer tiles the waves also split each stage's
//     keys two ways and merge their results in LDS at the end of the job.
//   * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16, A = 16
//     keys x 32 dims from the K tile, B = 32 dims x 16 rows of Q in registers). A lane
//     then owns one query row and 4 keys per 16-key tile: the row max needs two
//     cross-lane steps and the row sum none until the end of the job.
//   * Output is accumulated transposed, O^T += V^T P^T. P^T comes straight from the
//     score registers (rounded to bf16); V^T is read with ds_read_b64_tr_b16, which
//     hands each lane four keys of one dimension. Pairs of 16-key tiles feed
//     v_mfma_f32_16x16x32_bf16; the key order inside the contraction is permuted
//     identically on both operands, which leaves the sum unchanged.
//   * Softmax runs in base 2 on raw scores: p = 2^(s*c - m*c), c = scale*log2(e), m a
//     running reference max. The LSE uses the sum of the fp32 p (LSE = scale*m + ln l);
//     O is normalised by the sum of the bf16-rounded p it was accumulated from.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace splitkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int NW = 8;          // wavefronts per workgroup (two per SIMD)
constexpr int TK = 64;         // keys per pipeline stage
constexpr int NST = 3;         // pipeline slots
constexpr int RTW = 2;         // row tiles per wave per pass
constexpr int QLDS_ROWS = 64;  // units with at most this many rows get Q through LDS
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float NEG_INF = -__builtin_huge_valf();

template <int D>
struct Cfg {
  static constexpr int DC = D / 32;                  // 32-dim slices of the QK^T contraction
  static constexpr int DT = D / 16;                  // 16-dim output tiles
  static constexpr int ROWB = 2 * D;                 // bytes per key row
  static constexpr int CH = ROWB / 16;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;            // rows per 1 KiB DMA instruction
  static constexpr int TILEB = TK * ROWB;            // bytes of a K or V tile
  static constexpr int QTILEB = QLDS_ROWS * ROWB;    // bytes of a Q tile
  static constexpr int SLOTB = 2 * TILEB + QTILEB;   // bytes per pipeline slot
  static constexpr int KV_INST = TILEB / 1024 / NW;  // DMA instructions per wave per K (or V) tile
  static constexpr int Q_INST = QTILEB / 1024 / NW;  // DMA instructions per wave per Q tile
  static constexpr int MSLOT = 64 * (DT * 4 + 3);    // floats of one merge record (m, l, ls, O)
  // At least 96 KiB so that a compute unit holds a single workgroup.
  static constexpr int LDSB = NST * SLOTB > 96 * 1024 ? NST * SLOTB : 96 * 1024;
  static_assert(4 * MSLOT * 4 <= SLOTB, "a merge round's records fit in one slot");
  static_assert(KV_INST >= 1 && Q_INST >= 1, "tile sizes");
};

// XOR swizzles of the 16-byte chunk index within a row: conflict-free 16-lane row
// reads (K, Q) and 32-lane transposing reads (V).
template <int D>
__device__ __forceinline__ int swz_k(int row, int c) { return c ^ (row & (Cfg<D>::CH - 1)); }
template <int D>
__device__ __forceinline__ int swz_v(int row, int c) { return c ^ ((2 * row) & (Cfg<D>::CH - 1)); }

// Wait until at most n vector-memory operations of this wave are outstanding, then
// barrier the workgroup (no fence: the pipeline's later DMA must stay in flight).
__device__ __forceinline__ void wait_vm_barrier(int n) {
  switch (n) {
#define SKV_CASE(N) \
  case N: asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory"); break;
    SKV_CASE(0) SKV_CASE(1) SKV_CASE(2) SKV_CASE(3) SKV_CASE(4) SKV_CASE(5) SKV_CASE(6) SKV_CASE(7)
    SKV_CASE(8) SKV_CASE(9) SKV_CASE(10) SKV_CASE(11) SKV_CASE(12)
#undef SKV_CASE
    default: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// Transposing LDS reads (ds_read_b64_tr_b16) issued from inline assembly. Through the
// builtin, the compiler cannot tell that they read a different pipeline slot than the
// in-flight DMA writes, and it drains all of that DMA first. The reads and their
// lgkmcnt wait sit in one asm statement, so no instruction can touch the destination
// registers while the loads are still in flight.
__device__ __forceinline__ unsigned lds_addr(const unsigned char* p) {
  typedef __attribute__((address_space(3))) const unsigned char* lds_cptr;
  return (unsigned)(uintptr_t)(lds_cptr)p;  // 32-bit LDS offset
}

template <int N>
__device__ __forceinline__ void tr_read_all(i16x4 (&lo)[N], i16x4 (&hi)[N], const unsigned (&alo)[N],
                                            const unsigned (&ahi)[N]) {
  if constexpr (N == 8) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %17\n\t"
        "ds_read_b64_tr_b16 %2, %18\n\tds_read_b64_tr_b16 %3, %19\n\t"
        "ds_read_b64_tr_b16 %4, %20\n\tds_read_b64_tr_b16 %5, %21\n\t"
        "ds_read_b64_tr_b16 %6, %22\n\tds_read_b64_tr_b16 %7, %23\n\t"
        "ds_read_b64_tr_b16 %8, %24\n\tds_read_b64_tr_b16 %9, %25\n\t"
        "ds_read_b64_tr_b16 %10, %26\n\tds_read_b64_tr_b16 %11, %27\n\t"
        "ds_read_b64_tr_b16 %12, %28\n\tds_read_b64_tr_b16 %13, %29\n\t"
        "ds_read_b64_tr_b16 %14, %30\n\tds_read_b64_tr_b16 %15, %31\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(lo[4]), "=&v"(lo[5]), "=&v"(lo[6]),
          "=&v"(lo[7]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]), "=&v"(hi[3]), "=&v"(hi[4]), "=&v"(hi[5]),
          "=&v"(hi[6]), "=&v"(hi[7])
        : "v"(alo[0]), "v"(alo[1]), "v"(alo[2]), "v"(alo[3]), "v"(alo[4]), "v"(alo[5]), "v"(alo[6]), "v"(alo[7]),
          "v"(ahi[0]), "v"(ahi[1]), "v"(ahi[2]), "v"(ahi[3]), "v"(ahi[4]), "v"(ahi[5]), "v"(ahi[6]), "v"(ahi[7]));
  } else {
    static_assert(N == 4, "head_dim 64 or 128");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
          "=&v"(hi[3])
        : "v"(alo[0]), "v"(alo[1]), "v"(alo[2]), "v"(alo[3]), "v"(ahi[0]), "v"(ahi[1]), "v"(ahi[2]), "v"(ahi[3]));
  }
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

// Read-only plan records. Passed as separate __restrict__ kernel arguments so the
// compiler can prove no store of the kernel aliases them and read them with scalar
// loads: a vector load here would be counted by vmcnt behind the in-flight DMA and
// waiting for it would drain the whole pipeline.
struct Plan {
  const UnitRec* __restrict__ units;
  const SeqRec* __restrict__ seqs;
};

// One job: (unit, KV head, row pass) and everything derived from it.
struct Job {
  int ui, kv, pass;
  int block, len, lim0, R, nrt, Wr, Wk, npass, tile_lo, tile_hi, nst;
  bool qlds, direct;
  SeqRec sq;
};

__device__ __forceinline__ void describe(const PartialArgs& a, const Plan& P, Job& J) {
  const UnitRec u = P.units[J.ui];
  J.sq = P.seqs[u.seq];
  J.block = u.block;
  const int64_t key0 = int64_t(u.block) * a.B;
  J.len = int(min(int64_t(a.B), J.sq.n - key0));
  // Row r (query token i = r / g) sees block keys t <= lim0 + i; lim0 >= 1 - q.
  J.lim0 = int(min(int64_t(J.len), J.sq.n - J.sq.q - key0));
  J.R = J.sq.rows;
  J.nrt = (J.R + 15) >> 4;
  // Waves split the row tiles Wr ways and each stage's keys Wk ways (Wr * Wk <= NW;
  // the other waves only load). With >= 8 tiles: up to 16 tiles (256 rows) per pass.
  J.Wr = J.nrt >= 8 ? 8 : (J.nrt >= 4 ? 4 : (J.nrt >= 2 ? 2 : 1));
  J.Wk = J.Wr == 8 ? 1 : 2;
  J.npass = J.Wr == 8 ? (J.nrt + NW * RTW - 1) / (NW * RTW) : 1;
  J.tile_lo = J.Wr == 8 ? J.pass * NW * RTW : 0;
  J.tile_hi = min(J.nrt, J.tile_lo + (J.Wr == 8 ? NW * RTW : J.nrt));
  const int rmax = min(J.R, J.tile_hi * 16) - 1;
  const int tmax = a.causal ? min(J.len - 1, J.lim0 + rmax / a.g) : J.len - 1;
  J.nst = tmax < 0 ? 1 : (tmax + TK) / TK;
  J.qlds = J.R <= QLDS_ROWS;
  J.direct = a.out != nullptr && J.sq.nb == 1;
}

// Advance to the next job of the worker; returns false when the list is exhausted.
__device__ __forceinline__ bool next_job(const Plan& P, Job& J, int u_end) {
  if (++J.pass < J.npass) return true;
  J.pass = 0;
  const UnitRec u = P.units[J.ui];
  if (++J.kv < u.kv0 + u.nkv) return true;
  if (++J.ui >= u_end) return false;
  J.kv = P.units[J.ui].kv0;
  return true;
}

// Issue the DMA of stage j of job J into one pipeline slot; returns the number of
// vector-memory instructions this wave issued.
template <int D>
__device__ __forceinline__ int issue_stage(const PartialArgs& a, const Job& J, int j, unsigned char* slot, int wave,
                                           int lane) {
  using C = Cfg<D>;
  const int cs = lane % C::CH;
  const int64_t kv0 = (J.sq.kv_base + int64_t(J.block) * a.B);
  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + kv0 * a.k_st + int64_t(J.kv) * a.k_sh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + kv0 * a.v_st + int64_t(J.kv) * a.v_sh;
#pragma unroll
  for (int in = 0; in < C::KV_INST; ++in) {
    const int gi = wave * C::KV_INST + in;
    const int row = gi * C::RPI + lane / C::CH;
    // Keys past the block end re-read the last key: finite data, masked out later.
    const int tok = min(j * TK + row, J.len - 1);
    const __bf16* ks = kb + int64_t(tok) * a.k_st + 8 * swz_k<D>(row, cs);
    const __bf16* vs = vb + int64_t(tok) * a.v_st + 8 * swz_v<D>(row, cs);
    __builtin_amdgcn_global_load_lds(ks, (lds_void*)(slot + gi * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vs, (lds_void*)(slot + C::TILEB + gi * 1024), 16, 0, 0);
  }
  int n = 2 * C::KV_INST;
  if (J.qlds && j == 0) {
    const __bf16* qb = reinterpret_cast<const __bf16*>(a.q);
#pragma unroll
    for (int in = 0; in < C::Q_INST; ++in) {
      const int gi = wave * C::Q_INST + in;
      const int row = gi * C::RPI + lane / C::CH;
      const int rr = min(row, J.R - 1);  // padding rows repeat the last row
      const int i = rr / a.g, hl = rr - i * a.g;
      const __bf16* qs = qb + (J.sq.q_base + i) * a.q_st + int64_t(J.kv * a.g + hl) * a.q_sh + 8 * swz_k<D>(row, cs);
      __builtin_amdgcn_global_load_lds(qs, (lds_void*)(slot + 2 * C::TILEB + gi * 1024), 16, 0, 0);
    }
    n += C::Q_INST;
  }
  return n;
}

template <int D>
struct State {
  f32x4 o[RTW][Cfg<D>::DT];
  bf16x8 q[RTW][Cfg<D>::DC];
  f32x4 ls[RTW];  // sum of the bf16-rounded p of this lane's row (every entry equal)
  float m[RTW];   // running reference max of raw scores (row of this lane)
  float l[RTW];   // this lane's share of the row sum of the fp32 p
  int lim[RTW];  // last visible block key of this lane's row
};

// One online-softmax step for this wave: its nt row tiles against 32 keys of the
// stage (two 16-key tiles) starting at key `tok` of the stage.
//
// The running reference max m moves only when a row's max exceeds it by more than
// RESCALE_LOG2 in base 2 (then O and l are rescaled); otherwise p = 2^(s*c - m*c) may
// reach 2^RESCALE_LOG2, which fp32 and bf16 hold exactly in range. O, l and LSE all use
// the same reference, so the result does not depend on when it moved.
constexpr float RESCALE_LOG2 = 8.f;

template <int D>
__device__ __forceinline__ void softmax_step(State<D>& st, int nt, const unsigned char* slot, int tok_stage, int tok,
                                             bool need_mask, float c) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const unsigned char* kt = slot;
  const unsigned char* vt = slot + C::TILEB;

  // S^T = K Q^T for each 16-key tile, shared K operands across the row tiles.
  constexpr int NT = 2;
  f32x4 s[RTW][NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int row = tok + 16 * tt + li;
    bf16x8 kop[C::DC];
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc)
      kop[dc] = *reinterpret_cast<const bf16x8*>(kt + row * C::ROWB + 16 * swz_k<D>(row, 4 * dc + G));
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      if (t < nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[dc], st.q[t][dc], acc, 0, 0, 0);
        s[t][tt] = acc;
      }
    }
  }

  bf16x4 p[RTW][NT];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    if (t < nt) {
      if (need_mask) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (tok_stage + tok + 16 * tt + 4 * G + e > st.lim[t]) s[t][tt][e] = NEG_INF;
      }
      float mx = s[t][0][0];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[t][tt][e]);
      // Move the reference (and rescale) only on a large increase; -inf -> finite always
      // moves. The test first uses this lane's own scores: only when some lane would move
      // is the row max formed across the row's four lanes (rare after the first step).
      const bool grow_lane = mx * c > st.m[t] * c + RESCALE_LOG2 || (st.m[t] == NEG_INF && mx != NEG_INF);
      if (__any(grow_lane)) {
        mx = max4(mx);
        const bool grow = mx * c > st.m[t] * c + RESCALE_LOG2 || (st.m[t] == NEG_INF && mx != NEG_INF);
        const float mnew = grow ? mx : st.m[t];
        const float alpha = grow ? (st.m[t] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((st.m[t] - mnew) * c)) : 1.f;
        st.m[t] = mnew;
        st.l[t] *= alpha;
        st.ls[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) st.o[t][dt] *= alpha;
      }
      const float mc = st.m[t] == NEG_INF ? 0.f : st.m[t] * c;
      float psum = 0.f;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][tt][e], c, -mc));
          psum += pe;
          p[t][tt][e] = (__bf16)pe;
        }
      st.l[t] += psum;
    }
  }

  const int e = li >> 2, cc = li & 3;
  const int r0 = tok + 4 * G + e, r1 = r0 + 16;
  i16x4 lo[C::DT], hi[C::DT];
  unsigned alo[C::DT], ahi[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int ch = 2 * dt + (cc >> 1), off = 8 * (cc & 1);
    alo[dt] = lds_addr(vt + r0 * C::ROWB + 16 * swz_v<D>(r0, ch) + off);
    ahi[dt] = lds_addr(vt + r1 * C::ROWB + 16 * swz_v<D>(r1, ch) + off);
  }
  tr_read_all<C::DT>(lo, hi, alo, ahi);
  bf16x8 vop[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
    vop[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[dt], hi[dt], 0, 1, 2, 3, 4, 5, 6, 7));
  // An all-ones V^T tile sums the rounded p of each row on the matrix core (exact fp32
  // accumulation, already reduced across lanes): O is normalised by that sum, so it is a
  // convex combination of the values even when one key dominates.
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

// Normalise and store one row tile of a finished job (row li of the tile, dims
// 16dt+4G..+3).
template <int D>
__device__ __forceinline__ void write_tile(const State<D>& st, int t, const PartialArgs& a, const Job& J, int tile) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float l = sum4(st.l[t]);
  const int row = tile * 16 + li;
  if (row >= J.R) return;
  const float ls = st.ls[t][0];
  const float inv = ls > 0.f ? 1.f / ls : 0.f;
  const float lse = l > 0.f ? st.m[t] * a.scale + __builtin_amdgcn_logf(l) * LN2 : NEG_INF;
  float* op;
  float* lp;
  if (J.direct) {
    const int i = row / a.g, hl = row - i * a.g;
    const int64_t idx = (J.sq.q_base + i) * a.Hq + J.kv * a.g + hl;
    op = a.out + idx * D;
    lp = a.lse + idx;
  } else {
    const int64_t prow = J.sq.row_base + (int64_t(J.kv) * J.sq.nb + J.block) * J.R + row;
    op = a.ws_o + prow * D;
    lp = a.ws_lse + prow;
  }
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * G) = st.o[t][dt] * inv;
  if (G == 0) *lp = lse;
}

// Finish job J right after its last stage: combine its key slices (Wk > 1) through
// the LDS slot that stage used, then store every row tile. The slot is next written by
// DMA only after the following iteration's barrier. (Finishing before that iteration's
// DMA issue instead delays the pipeline more than the stores cost here.)
template <int D>
__device__ __forceinline__ void finish_job(State<D>& st, const PartialArgs& a, const Job& J, unsigned char* slot,
                                           int wave, float c) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int rg = wave % J.Wr, ks = wave / J.Wr;
  const int ntw = ks < J.Wk && J.tile_hi - J.tile_lo - rg > 0 ? (J.tile_hi - J.tile_lo - rg + J.Wr - 1) / J.Wr : 0;
  const int nt = min(ntw, RTW);
  if (J.Wk == 1) {
#pragma unroll
    for (int t = 0; t < RTW; ++t)
      if (t < nt) write_tile<D>(st, t, a, J, J.tile_lo + rg + t * J.Wr);
    return;
  }
  // Two key slices per row group; one round per tile index (<= Wr records each). The
  // loop is unrolled with compile-time tile indices: a runtime index would put the
  // wave state in scratch memory.
  float* mbuf = reinterpret_cast<float*>(slot);
  const int rounds = (J.tile_hi - J.tile_lo + J.Wr - 1) / J.Wr;
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    if (t >= rounds) break;
    lds_barrier();  // all waves are done with the slot's tiles / the previous round
    if (ks == 1 && t < nt) {
      float* rec = mbuf + rg * C::MSLOT;
      rec[lane] = st.m[t];
      rec[64 + lane] = st.l[t];
      rec[128 + lane] = st.ls[t][0];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) rec[(3 + dt * 4 + q4) * 64 + lane] = st.o[t][dt][q4];
    }
    lds_barrier();
    if (ks == 0 && t < nt) {
      const float* rec = mbuf + rg * C::MSLOT;
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
      write_tile<D>(st, t, a, J, J.tile_lo + rg + t * J.Wr);
    }
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void partial_bf16_kernel(PartialArgs a, const UnitRec* __restrict__ units, const SeqRec* __restrict__ seqs,
                         const int32_t* __restrict__ worker_ptr) {
  using C = Cfg<D>;
  const Plan P{units, seqs};
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDSB];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float c = a.scale * LOG2E;

  const int u_beg = worker_ptr[blockIdx.x], u_end = worker_ptr[blockIdx.x + 1];
  if (u_beg >= u_end) return;

  // Loader and compute walk the same job sequence; the loader runs two stages ahead.
  Job L, J;
  L.ui = J.ui = u_beg;
  L.kv = J.kv = P.units[u_beg].kv0;
  L.pass = J.pass = 0;
  describe(a, P, L);
  describe(a, P, J);
  int lj = 0;         // next stage of job L to issue
  bool lmore = true;  // loader has stages left
  int last_cnt = 0;   // vector-memory instructions of the most recently issued stage
  int issued = 0;     // stages issued so far
  for (int k = 0; k < NST - 1 && lmore; ++k) {
    last_cnt = issue_stage<D>(a, L, lj, smem + (issued % NST) * C::SLOTB, wave, lane);
    ++issued;
    if (++lj == L.nst) {
      lj = 0;
      lmore = next_job(P, L, u_end);
      if (lmore) describe(a, P, L);
    }
  }

  State<D> st;
  int jj = 0;  // stage within the compute job
  for (int i = 0;; ++i) {
    // Stage i landed (for every wave) once the later stages are all that is pending.
    // Here at most stage i + 1 was issued after it, and it is the latest one.
    wait_vm_barrier(issued > i + 1 ? last_cnt : 0);

    // This wave's share of the job.
    const int rg = wave % J.Wr, ks = wave / J.Wr;
    const int ntw = ks < J.Wk && J.tile_hi - J.tile_lo - rg > 0 ? (J.tile_hi - J.tile_lo - rg + J.Wr - 1) / J.Wr : 0;
    const int nt = min(ntw, RTW);
    if (jj == 0 && !J.qlds) {
      // Job start with Q from HBM: issued before this iteration's DMA, so that waiting
      // for it leaves the newer stages in flight.
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        const int row = (J.tile_lo + rg + t * J.Wr) * 16 + li;
        const bool ok = t < nt && row < J.R;
        const int iq = ok ? row / a.g : 0;
        const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (J.sq.q_base + iq) * a.q_st +
                           int64_t(J.kv * a.g + (ok ? row - iq * a.g : 0)) * a.q_sh + 8 * G;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
          st.q[t][dc] = ok ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * dc)) : bf16x8{};
      }
      // Complete these loads here (only the previous stage's DMA is older). A compiler-
      // visible wait, so that no load into the Q registers is pending anywhere else in
      // the loop: otherwise every later use of them would wait for all in-flight DMA.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    if (lmore) {
      last_cnt = issue_stage<D>(a, L, lj, smem + (issued % NST) * C::SLOTB, wave, lane);
      ++issued;
      if (++lj == L.nst) {
        lj = 0;
        lmore = next_job(P, L, u_end);
        if (lmore) describe(a, P, L);
      }
    }
    unsigned char* slot = smem + (i % NST) * C::SLOTB;
    if (jj == 0) {
      // Job start: Q operands, accumulators, per-row limits.
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        const int tile = J.tile_lo + rg + t * J.Wr;
        const int row = tile * 16 + li;
        const bool ok = t < nt && row < J.R;
        const int iq = ok ? row / a.g : 0;
        st.lim[t] = a.causal ? min(J.lim0 + iq, J.len - 1) : J.len - 1;
        if (J.qlds) {
          // The Q tile of this slot holds rows 0..63 of the unit (R <= 64 here).
          const int qr = t < nt ? row : 0;
#pragma unroll
          for (int dc = 0; dc < C::DC; ++dc)
            st.q[t][dc] = *reinterpret_cast<const bf16x8*>(slot + 2 * C::TILEB + qr * C::ROWB +
                                                           16 * swz_k<D>(qr, 4 * dc + G));
        }
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) st.o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m[t] = NEG_INF;
        st.l[t] = 0.f;
        st.ls[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

    // Keys of this stage handled by this wave, and whether masking is needed.
    const int tkw = TK / J.Wk;
    const int tok_w = ks * tkw;
    const int tok_stage = jj * TK;
    const int first_row = (J.tile_lo + rg) * 16;
    const int min_lim = a.causal ? J.lim0 + min(first_row, J.R - 1) / a.g : J.len - 1;
    const int last_key = tok_stage + tok_w + tkw - 1;
    const bool need_mask = last_key >= J.len || last_key > min_lim;
    if (nt > 0) {
      for (int h = 0; h < tkw; h += 32) softmax_step<D>(st, nt, slot, tok_stage, tok_w + h, need_mask, c);
    }
    if (jj + 1 == J.nst) {
      finish_job<D>(st, a, J, slot, wave, c);
      jj = 0;
      if (!next_job(P, J, u_end)) break;
      describe(a, P, J);
    } else {
      ++jj;
    }
  }
}

}  // namespace

hipError_t launch_partial_bf16(const PartialArgs& a, int head_dim, hipStream_t stream) {
  dim3 grid(a.num_workers), block(NW * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL(partial_bf16_kernel<128>, grid, block, 0, stream, a, a.units, a.seqs, a.worker_ptr);
  else if (head_dim == 64)
    hipLaunchKernelGGL(partial_bf16_kernel<64>, grid, block, 0, stream, a, a.units, a.seqs, a.worker_ptr);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
