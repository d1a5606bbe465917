// Gradients of split-KV attention on gfx950 matrix cores (bf16 inputs, fp32 math).
//
// Split-KV page, "Timeline": the sharded computation equals the unsharded one. With
// the merged log-sum-exp of every query row, P = e^(S - LSE) is the row's global
// softmax, so each context KV block's share of the backward pass is exact on its own
// (textbook attention gradients, D_i = <dO_i, O_i>):
//   dS = P o (dP - D),  dP = dO V^T,
//   dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i   (complete within the block),
//   dQ_i = scale sum_j dS_ij k_j                              (a query-sized part per block,
//                                                              summed over the blocks).
// The page describes no kernel; this is a CDNA4 design in up to five launches:
//   rowdot:  D_i = <dO_i, O_i> for every query row (one wavefront per row);
//   dq:      one workgroup per forward job (a unit's KV head and up to 256 of its query
//            rows; 4 waves when no pass has more than 128 rows, so that two workgroups
//            share a CU, else 8): its block's keys stream through LDS in stages of 32
//            (direct global->LDS DMA, three stages in flight; stages below the smallest
//            causal limit of a wave's rows skip the causal test); each wave keeps
//            Q, dO and its dQ part of two 16-row tiles in registers. Scores are computed
//            transposed as in the forward (S^T = K Q^T), dP^T = V dO^T the same way, and
//            dQ^T += K^T dS^T with K^T read by transposing LDS loads. The part goes to the
//            workspace row of (block, KV head), or straight to dQ for one-block sequences;
//   dqkv_small: the jobs of sequences with at most 16 query rows per KV head (one row
//            tile holds all of them): the dQ part as dq forms it, and the dK and dV of
//            each stage's keys from the same K/V stream, so those blocks are read once;
//   dqsum:   dQ of a multi-block sequence is the sum of its blocks' parts in block order
//            (one wavefront per row);
//   dkv:     one workgroup of 4 waves per (sequence, KV head, 64-key tile) of the other
//            sequences (the plan's key-tile table); a wave holds
//            its 16 keys' K and V rows in registers and dK^T, dV^T accumulators, and the
//            query rows that see the tile stream through LDS 32 at a time, with their LSE
//            and D (direct global->LDS DMA, two chunks ahead, three buffers, one barrier
//            per chunk; when g divides 32 a lane's loads are a per-chunk scalar base plus
//            constant offsets): S = Q K^T, dP = dO V^T, then dV^T += dO^T P and
//            dK^T += Q^T dS with Q^T and dO^T read by transposing loads. Kept at 168
//            VGPRs or fewer (three workgroups per CU). dK and dV are written once, as
//            fp32 or rounded to bf16.
// P and dS enter the matrix cores rounded to bf16 (as P does in the forward); all sums
// are fp32.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace splitkv {
namespace {

using namespace lds;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

template <int D>
struct BCfg {
  static constexpr int DC = D / 32;      // 32-dim slices of a contraction over dims
  static constexpr int DT = D / 16;      // 16-dim output tiles
  static constexpr int ROWB = 2 * D;     // bytes per bf16 row
  static constexpr int CH = ROWB / 16;   // 16-byte chunks per row
  static constexpr int TILEB = 64 * ROWB;  // 64 rows
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---------------------------------------------------------------- D_i = <dO_i, O_i>
// and the row's LSE in base 2 (LSE_i * log2 e, the product the dK/dV kernel would
// otherwise form for every (row, key) pair).
template <int D>
__global__ __launch_bounds__(256) void rowdot_kernel(BwdArgs a) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // i * Hq + h
  if (row >= a.total_q * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int64_t i = row / a.Hq, h = row - i * a.Hq;
  const __bf16* dop = reinterpret_cast<const __bf16*>(a.dout) + i * a.do_st + h * a.do_sh;
  const float* op = a.out + row * D;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) s += float(dop[lane + 64 * k]) * op[lane + 64 * k];
  s = wave_sum(s);
  if (lane == 0) {
    a.ws_d[row] = s;
    a.ws_l2[row] = LOG2E * a.lse[row];
  }
}

// ---------------------------------------------------------------- dQ parts per job
constexpr int RT = 2;  // row tiles per wave

constexpr int DQ_KEYS = 32;  // keys per stage (one step of the contraction)

constexpr int DQ_BUFS = 4;   // stage buffers: the stage computed and three in flight
template <int D>
struct DqLds {
  unsigned char k[DQ_BUFS][DQ_KEYS * BCfg<D>::ROWB];  // K rows stored for transposing reads
  unsigned char v[DQ_BUFS][DQ_KEYS * BCfg<D>::ROWB];  // V rows stored for row reads
};

// Wait until at most n (0, 2, 4, 6 or 8) vector-memory instructions of this wave are
// outstanding, then barrier (no fence: later stages' DMA stays in flight).
__device__ __forceinline__ void dq_wait_barrier(int n) {
  if (n >= 8)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if (n >= 6)
    asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
  else if (n >= 4)
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else if (n >= 2)
    asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, int W>
__global__ __launch_bounds__(W * 64, 2) void dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[sizeof(DqLds<D>)];
  DqLds<D>& L = *reinterpret_cast<DqLds<D>*>(smem);
  const JobRec j = a.jobs[blockIdx.x];
  if (j.flags & kJobFusedKV) return;  // dqkv_small_kernel's job
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float c = a.scale * LOG2E;

  // This wave's row tiles: tile_lo + wave and tile_lo + wave + W.
  int nt = 0;
  int rowq[RT];  // query row of this lane in each tile (rows past the last repeat it)
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int tile = wave + t * W;
    if (tile < j.tile_n) nt = t + 1;
    rowq[t] = min((j.tile_lo + min(tile, j.tile_n - 1)) * 16 + li, j.rows - 1);
  }
  bf16x8 qop[RT][C::DC], dop[RT][C::DC];
  float lsec[RT], dd[RT];
  int lim[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = rowq[t];
    const int i = r / a.g, hl = r - i * a.g;
    const int64_t tok = j.q_tok + i, head = int64_t(j.kv) * a.g + hl;
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + tok * a.q_st + head * a.q_sh + 8 * G;
    const __bf16* gp = reinterpret_cast<const __bf16*>(a.dout) + tok * a.do_st + head * a.do_sh + 8 * G;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      qop[t][dc] = *reinterpret_cast<const bf16x8*>(qp + 32 * dc);
      dop[t][dc] = *reinterpret_cast<const bf16x8*>(gp + 32 * dc);
    }
    lsec[t] = a.lse[tok * a.Hq + head] * LOG2E;
    dd[t] = a.ws_d[tok * a.Hq + head];
    lim[t] = min(j.lim0 + i, j.len - 1);  // last visible block key of this row
  }
  f32x4 acc[RT][C::DT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage loads: direct global->LDS DMA of 1 KiB per instruction, PW instructions per
  // issuing wave for K and as many for V. LDS position p of a tile (16-byte units) is key
  // row p / CH, slot p % CH; the slot holds chunk swz(row, slot) of the row (XOR
  // swizzles are their own inverse).
  constexpr int NI = DQ_KEYS * C::ROWB / 1024;  // instructions per tile
  constexpr int PW = NI > W ? NI / W : 1;        // per issuing wave
  static_assert(PW * (NI / PW) == NI && NI / PW <= W, "tile split over the waves");
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k) + 2 * (j.kv_tok * a.k_st + int64_t(j.kv) * a.k_sh);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v) + 2 * (j.kv_tok * a.v_st + int64_t(j.kv) * a.v_sh);
  int srow[PW], kcc[PW], vcc[PW];
  uint32_t koff[PW], voff[PW];  // this lane's bytes of a full stage, from its first key
#pragma unroll
  for (int u = 0; u < PW; ++u) {
    const int p = (wave * PW + u) * 64 + lane;
    srow[u] = p / C::CH;
    kcc[u] = swz_tr<C::CH>(srow[u], p % C::CH);
    vcc[u] = swz_row<C::CH>(srow[u], p % C::CH);
    koff[u] = uint32_t(srow[u]) * uint32_t(2 * a.k_st) + 16u * kcc[u];
    voff[u] = uint32_t(srow[u]) * uint32_t(2 * a.v_st) + 16u * vcc[u];
  }
  auto issue_stage = [&](int st) {
    if (wave * PW >= NI) return;
    const int buf = st % DQ_BUFS;
    if ((st + 1) * DQ_KEYS <= j.len) {
      // A full stage: the stage's first key plus the constant per-lane offsets.
      const unsigned char* ks = kbase + int64_t(st * DQ_KEYS) * (2 * a.k_st);
      const unsigned char* vs = vbase + int64_t(st * DQ_KEYS) * (2 * a.v_st);
#pragma unroll
      for (int u = 0; u < PW; ++u) {
        const int gi = wave * PW + u;
        __builtin_amdgcn_global_load_lds(ks + koff[u], (lds_void*)(L.k[buf] + gi * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vs + voff[u], (lds_void*)(L.v[buf] + gi * 1024), 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int key = min(st * DQ_KEYS + srow[u], j.len - 1);  // past the block: its last key (masked)
      const int gi = wave * PW + u;
      __builtin_amdgcn_global_load_lds(kbase + int64_t(key) * (2 * a.k_st) + 16 * kcc[u], (lds_void*)(L.k[buf] + gi * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vbase + int64_t(key) * (2 * a.v_st) + 16 * vcc[u], (lds_void*)(L.v[buf] + gi * 1024), 16, 0, 0);
    }
  };
  // Per-lane LDS offsets within a 16-row tile: row reads (lane: row li, dims 8G + 32 dc)
  // and K^T reads (lane: dims of tile dt, keys 4G + li/4 and 16 more).
  unsigned ok_row[C::DC], ov_row[C::DC], ok_tr[C::DT];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    ok_row[dc] = li * C::ROWB + 16 * swz_tr<C::CH>(li, 4 * dc + G);
    ov_row[dc] = li * C::ROWB + 16 * swz_row<C::CH>(li, 4 * dc + G);
  }
  {
    const int e = li >> 2, cc = li & 3, r = 4 * G + e;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) ok_tr[dt] = r * C::ROWB + 16 * swz_tr<C::CH>(r, 2 * dt + (cc >> 1)) + 8 * (cc & 1);
  }

  // Keys up to the smallest limit of the wave's rows (its first row) are visible to all
  // of them: stages that end there need no causal test.
  const int r_first = min((j.tile_lo + min(wave, j.tile_n - 1)) * 16, j.rows - 1);
  const int wave_min_lim = min(j.lim0 + r_first / a.g, j.len - 1);
  const int nst = j.nst * (kStageKeys / DQ_KEYS);  // the job's stages of visible keys, in 32-key steps
  for (int st = 0; st < DQ_BUFS - 1 && st < nst; ++st) issue_stage(st);
  for (int st = 0; st < nst; ++st) {
    const int buf = st % DQ_BUFS;
    // Stage st has landed once only the (at most two) later stages' DMA is pending.
    dq_wait_barrier(2 * PW * min(DQ_BUFS - 2, nst - 1 - st));
    if (st + DQ_BUFS - 1 < nst) issue_stage(st + DQ_BUFS - 1);  // into the buffer of stage st - 1
    const unsigned kb = lds_addr(L.k[buf]), vb = lds_addr(L.v[buf]);
    {
      const int key0 = st * DQ_KEYS;  // block key of the stage's first key
      const bool all_vis = key0 + DQ_KEYS - 1 <= wave_min_lim;
      if (nt > 0) {
        // Per 16-key tile: S^T and dP^T, then dS^T = P^T (dP^T - D) with
        // P^T = 2^(s c - LSE log2 e); entry e of tile tt is block key key0 + 16 tt + 4 G + e.
        float ds[RT][2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          bf16x8 kop[C::DC], vop[C::DC];
          const unsigned rowoff = unsigned(tt * 16) * C::ROWB;
#pragma unroll
          for (int dc = 0; dc < C::DC; ++dc) {
            kop[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(kb + rowoff + ok_row[dc]));
            vop[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(vb + rowoff + ov_row[dc]));
          }
#pragma unroll
          for (int t = 0; t < RT; ++t) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
            if (t < nt) {
#pragma unroll
              for (int dc = 0; dc < C::DC; ++dc) {
                x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[dc], qop[t][dc], x, 0, 0, 0);
                y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dc], dop[t][dc], y, 0, 0, 0);
              }
            }
            if (all_vis) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                ds[t][tt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -lsec[t])) * (y[e] - dd[t]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int key = key0 + 16 * tt + 4 * G + e;
                const float pr = key <= lim[t] ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -lsec[t])) : 0.f;
                ds[t][tt][e] = pr * (y[e] - dd[t]);
              }
            }
          }
        }
        bf16x8 dsb[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
          dsb[t] = bf16x8{(__bf16)ds[t][0][0], (__bf16)ds[t][0][1], (__bf16)ds[t][0][2], (__bf16)ds[t][0][3],
                          (__bf16)ds[t][1][0], (__bf16)ds[t][1][1], (__bf16)ds[t][1][2], (__bf16)ds[t][1][3]};
        // dQ^T += K^T dS^T over the stage's 32 keys.
        unsigned ka[C::DT];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) ka[dt] = kb + ok_tr[dt];
        i16x4 lo[C::DT], hi[C::DT];
        tr_read<0, 16 * C::ROWB>(lo, hi, ka);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[dt], hi[dt], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < RT; ++t)
            if (t < nt) acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, dsb[t], acc[t][dt], 0, 0, 0);
        }
      }
    }
  }
  // Store the part (lane: row li of the tile, dims 16 dt + 4 G .. + 3).
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if (t < nt) {
      const int r = rowq[t];
      float* dst;
      if (j.flags & kJobSingle) {
        const int i = r / a.g, hl = r - i * a.g;
        dst = a.dq + ((j.q_tok + i) * a.Hq + int64_t(j.kv) * a.g + hl) * D;
      } else {
        dst = a.ws_dq + (j.ws_row + r) * D;
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt + 4 * G) = acc[t][dt] * a.scale;
    }
  }
#endif
}

// ------------------------------------------------- dQ part, dK and dV of few-row jobs
// A job flagged kJobFusedKV holds every query row of its KV head (at most kFusedRows,
// one row tile), so once a stage of keys has been through it, those keys' dK and dV are
// complete: the block's K/V stream serves dQ and dK/dV alike and the block is read once
// (the dK/dV kernel's key-tile table leaves these sequences out). Four waves, 32-key
// stages through the same LDS buffers and swizzles as dq_kernel:
//   wave 0:     the job's dQ part exactly as dq_kernel forms it (S^T, dP^T, dS^T, then
//               dQ^T += K^T dS^T), stored at the end;
//   waves 1, 2: the stage's 16-key tiles 0 and 1: S = Q K^T and dP = dO V^T from the
//               same register and LDS operands with the operands swapped (lane: key li,
//               rows 4 G + e), P and dS, then dV^T = dO^T P and dK^T = Q^T dS as
//               16x16x16 products over the row tile, with Q^T and dO^T held in registers
//               from the job's start; each key's dK and dV are stored at once;
//   waves 0, 3: the stage DMA. The storing waves issue none, so no wait on the DMA
//               counts their stores; they pass the stage barrier without a wait.
__device__ __forceinline__ void small_wait_barrier(int n) {
  if (n >= 16)
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else if (n >= 8)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if (n >= 4)
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
struct SmallLds {
  DqLds<D> s;                        // the stage buffers, as dq_kernel's
  unsigned char t[2][16 * D * 4];    // per dK/dV wave: one gradient tile of its 16 keys, row-major
};

// Store one gradient tile of a dK/dV wave's 16 keys. g[dt] holds this lane's values
// for key li, dims 16 dt + 4 G .. + 3 (the transposed product's layout, in which a
// store instruction writes 32- or 16-byte pieces of 16 rows). The tile goes through
// LDS (16-byte chunks XOR-swizzled by the key's low bits) and leaves as whole rows: a store
// instruction writes four keys' D contiguous values, 16 bytes per lane, with the
// non-temporal hint (nothing in the pass reads them again). Keys at or
// past n_keys are not stored; dst is key 0's row.
template <int D, typename T>
__device__ __forceinline__ void store_tile_rows(const f32x4 (&g)[D / 16], unsigned char* t, T* dst,
                                                int64_t key_stride, int n_keys, int lane) {
  constexpr int RB = D * int(sizeof(T)), NCH = RB / 16;
  static_assert(NCH % 4 == 0, "whole store instructions");
  const int G = lane >> 4, li = lane & 15;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int byte = (16 * dt + 4 * G) * int(sizeof(T));
    const int off = li * RB + 16 * ((byte / 16) ^ (li & (NCH - 1))) + byte % 16;
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<f32x4*>(t + off) = g[dt];
    } else {
      *reinterpret_cast<bf16x4*>(t + off) = bf16x4{(__bf16)g[dt][0], (__bf16)g[dt][1], (__bf16)g[dt][2], (__bf16)g[dt][3]};
    }
  }
#pragma unroll
  for (int u = 0; u < NCH / 4; ++u) {
    const int idx = u * 64 + lane, k = idx / NCH, c = idx % NCH;
    const u32x4 x = *reinterpret_cast<const u32x4*>(t + k * RB + 16 * (c ^ (k & (NCH - 1))));
    if (k < n_keys)
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(dst + k * key_stride) + 16 * c));
  }
}

template <int D, bool BF16OUT>
__global__ __launch_bounds__(256, 2) void dqkv_small_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[sizeof(SmallLds<D>)];
  SmallLds<D>& SL = *reinterpret_cast<SmallLds<D>*>(smem);
  DqLds<D>& L = SL.s;
  const JobRec j = a.jobs[blockIdx.x];
  if (!(j.flags & kJobFusedKV)) return;  // dq_kernel's job
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float c = a.scale * LOG2E;

  // Stage loads by waves 0 and 3 (PW instructions each per tensor), as in dq_kernel.
  constexpr int NI = DQ_KEYS * C::ROWB / 1024;  // instructions per tile
  constexpr int PW = NI / 2;
  static_assert(PW * 2 == NI, "tile split over the two loading waves");
  const int nst = j.nst * (kStageKeys / DQ_KEYS);
  // The stage loop every wave runs: one barrier per stage (the loading waves first wait
  // for their own DMA of the stage), then the next stage's DMA, then body(st, buf).
  auto stages = [&](bool dma, auto&& body) {
    const int iw = wave == 0 ? 0 : 1;
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k) + 2 * (j.kv_tok * a.k_st + int64_t(j.kv) * a.k_sh);
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v) + 2 * (j.kv_tok * a.v_st + int64_t(j.kv) * a.v_sh);
    int srow[PW], kcc[PW], vcc[PW];
    uint32_t koff[PW], voff[PW];
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int p = (iw * PW + u) * 64 + lane;
      srow[u] = p / C::CH;
      kcc[u] = swz_tr<C::CH>(srow[u], p % C::CH);
      vcc[u] = swz_row<C::CH>(srow[u], p % C::CH);
      koff[u] = uint32_t(srow[u]) * uint32_t(2 * a.k_st) + 16u * kcc[u];
      voff[u] = uint32_t(srow[u]) * uint32_t(2 * a.v_st) + 16u * vcc[u];
    }
    auto issue_stage = [&](int st) {
      const int buf = st % DQ_BUFS;
      if ((st + 1) * DQ_KEYS <= j.len) {
        const unsigned char* ks = kbase + int64_t(st * DQ_KEYS) * (2 * a.k_st);
        const unsigned char* vs = vbase + int64_t(st * DQ_KEYS) * (2 * a.v_st);
#pragma unroll
        for (int u = 0; u < PW; ++u) {
          const int gi = iw * PW + u;
          __builtin_amdgcn_global_load_lds(ks + koff[u], (lds_void*)(L.k[buf] + gi * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vs + voff[u], (lds_void*)(L.v[buf] + gi * 1024), 16, 0, 0);
        }
        return;
      }
#pragma unroll
      for (int u = 0; u < PW; ++u) {
        const int key = min(st * DQ_KEYS + srow[u], j.len - 1);  // past the block: its last key (masked)
        const int gi = iw * PW + u;
        __builtin_amdgcn_global_load_lds(kbase + int64_t(key) * (2 * a.k_st) + 16 * kcc[u], (lds_void*)(L.k[buf] + gi * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vbase + int64_t(key) * (2 * a.v_st) + 16 * vcc[u], (lds_void*)(L.v[buf] + gi * 1024), 16, 0, 0);
      }
    };
    if (dma)
      for (int st = 0; st < DQ_BUFS - 1 && st < nst; ++st) issue_stage(st);
    for (int st = 0; st < nst; ++st) {
      const int buf = st % DQ_BUFS;
      if (dma) {
        small_wait_barrier(2 * PW * min(DQ_BUFS - 2, nst - 1 - st));
        if (st + DQ_BUFS - 1 < nst) issue_stage(st + DQ_BUFS - 1);  // into the buffer of stage st - 1
      } else {
        asm volatile("s_barrier" ::: "memory");
      }
      body(st, buf);
    }
  };
  // LDS row-read offsets within a 16-key tile (lane: key li, dims 8 G + 32 dc), K stored
  // for transposing reads, V for row reads, as in dq_kernel.
  unsigned ok_row[C::DC], ov_row[C::DC];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) {
    ok_row[dc] = li * C::ROWB + 16 * swz_tr<C::CH>(li, 4 * dc + G);
    ov_row[dc] = li * C::ROWB + 16 * swz_row<C::CH>(li, 4 * dc + G);
  }
  // Row operands (lane: row li, dims 8 G + 32 dc; rows past the last repeat it): the B
  // operands of S^T = K Q^T and dP^T = V dO^T, and the A operands of S = Q K^T and
  // dP = dO V^T; and the row's LSE * log2 e, D and last visible block key.
  const int rq = min(li, j.rows - 1);
  auto load_rows = [&](bf16x8 (&qop)[C::DC], bf16x8 (&dop)[C::DC], float& lsec, float& dd, int& lim) {
    const int i = rq / a.g, hl = rq - i * a.g;
    const int64_t tok = j.q_tok + i, head = int64_t(j.kv) * a.g + hl;
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + tok * a.q_st + head * a.q_sh + 8 * G;
    const __bf16* gp = reinterpret_cast<const __bf16*>(a.dout) + tok * a.do_st + head * a.do_sh + 8 * G;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      qop[dc] = *reinterpret_cast<const bf16x8*>(qp + 32 * dc);
      dop[dc] = *reinterpret_cast<const bf16x8*>(gp + 32 * dc);
    }
    lsec = a.lse[tok * a.Hq + head] * LOG2E;
    dd = a.ws_d[tok * a.Hq + head];
    lim = min(j.lim0 + i, j.len - 1);
  };

  if (wave == 0) {
    // The job's dQ part, as dq_kernel forms it for a one-tile job.
    bf16x8 qop[C::DC], dop[C::DC];
    float lsec, dd;
    int lim;
    load_rows(qop, dop, lsec, dd, lim);
    unsigned ok_tr[C::DT];
    {
      const int e = li >> 2, cc = li & 3, r = 4 * G + e;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) ok_tr[dt] = r * C::ROWB + 16 * swz_tr<C::CH>(r, 2 * dt + (cc >> 1)) + 8 * (cc & 1);
    }
    f32x4 acc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wave_min_lim = min(j.lim0, j.len - 1);  // row 0's limit, the smallest
    stages(true, [&](int st, int buf) {
      const unsigned kb = lds_addr(L.k[buf]), vb = lds_addr(L.v[buf]);
      const int key0 = st * DQ_KEYS;
      const bool all_vis = key0 + DQ_KEYS - 1 <= wave_min_lim;
      float ds[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 kop[C::DC], vop[C::DC];
        const unsigned rowoff = unsigned(tt * 16) * C::ROWB;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) {
          kop[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(kb + rowoff + ok_row[dc]));
          vop[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(vb + rowoff + ov_row[dc]));
        }
        f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) {
          x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[dc], qop[dc], x, 0, 0, 0);
          y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dc], dop[dc], y, 0, 0, 0);
        }
        if (all_vis) {
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[tt][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -lsec)) * (y[e] - dd);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = key0 + 16 * tt + 4 * G + e;
            const float pr = key <= lim ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -lsec)) : 0.f;
            ds[tt][e] = pr * (y[e] - dd);
          }
        }
      }
      const bf16x8 dsb = {(__bf16)ds[0][0], (__bf16)ds[0][1], (__bf16)ds[0][2], (__bf16)ds[0][3],
                          (__bf16)ds[1][0], (__bf16)ds[1][1], (__bf16)ds[1][2], (__bf16)ds[1][3]};
      unsigned ka[C::DT];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) ka[dt] = kb + ok_tr[dt];
      i16x4 lo[C::DT], hi[C::DT];
      tr_read<0, 16 * C::ROWB>(lo, hi, ka);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[dt], hi[dt], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, dsb, acc[dt], 0, 0, 0);
      }
    });
    // Store the part (lane: row li, dims 16 dt + 4 G .. + 3), as dq_kernel.
    float* dst;
    if (j.flags & kJobSingle) {
      const int i = rq / a.g, hl = rq - i * a.g;
      dst = a.dq + ((j.q_tok + i) * a.Hq + int64_t(j.kv) * a.g + hl) * D;
    } else {
      dst = a.ws_dq + (j.ws_row + rq) * D;
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt + 4 * G) = acc[dt] * a.scale;
  } else if (wave <= 2) {
    // dK and dV of the stage's 16-key tile tt = wave - 1.
    const int tt = wave - 1;
    bf16x8 qop[C::DC], dop[C::DC];
    float lsec, dd;
    int lim;
    load_rows(qop, dop, lsec, dd, lim);
    // Per row 4 G + e (lane: key li): LSE, D and limit (-1 past the last row, which then
    // sees no key); Q^T and dO^T as the A operands of the 16x16x16 products (lane: dim
    // 16 dt + li, rows 4 G .. 4 G + 3; rows past the last read the last row, in bounds,
    // and are zeroed).
    float lsek[4], ddk[4];
    int limk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * G + e;
      lsek[e] = __shfl(lsec, r);
      ddk[e] = __shfl(dd, r);
      limk[e] = r < j.rows ? __shfl(lim, r) : -1;
    }
    i16x4 qtr[C::DT], dtr[C::DT];
    {
      const short* qs[4];
      const short* gs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = min(4 * G + e, j.rows - 1);
        const int i = r / a.g, hl = r - i * a.g;
        const int64_t tok = j.q_tok + i, head = int64_t(j.kv) * a.g + hl;
        qs[e] = reinterpret_cast<const short*>(a.q) + tok * a.q_st + head * a.q_sh + li;
        gs[e] = reinterpret_cast<const short*>(a.dout) + tok * a.do_st + head * a.do_sh + li;
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        short qv[4], gv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool in = 4 * G + e < j.rows;
          qv[e] = in ? qs[e][16 * dt] : short(0);
          gv[e] = in ? gs[e][16 * dt] : short(0);
        }
        qtr[dt] = i16x4{qv[0], qv[1], qv[2], qv[3]};
        dtr[dt] = i16x4{gv[0], gv[1], gv[2], gv[3]};
      }
    }
    const int64_t kstride = int64_t(a.Hkv) * D;
    using OutT = typename std::conditional<BF16OUT, __bf16, float>::type;
    stages(false, [&](int st, int buf) {
      const unsigned kb = lds_addr(L.k[buf]), vb = lds_addr(L.v[buf]);
      const unsigned rowoff = unsigned(tt * 16) * C::ROWB;
      bf16x8 kop[C::DC], vop[C::DC];
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        kop[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(kb + rowoff + ok_row[dc]));
        vop[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(vb + rowoff + ov_row[dc]));
      }
      f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[dc], kop[dc], x, 0, 0, 0);
        y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dop[dc], vop[dc], y, 0, 0, 0);
      }
      // Lane: block key kfirst + li, rows 4 G + e.
      const int kfirst = st * DQ_KEYS + 16 * tt;
      const int key = kfirst + li;
      float pr[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[e] = key <= limk[e] ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -lsek[e])) : 0.f;
        ds[e] = pr[e] * (y[e] - ddk[e]);
      }
      const i16x4 pb = __builtin_bit_cast(i16x4, bf16x4{(__bf16)pr[0], (__bf16)pr[1], (__bf16)pr[2], (__bf16)pr[3]});
      const i16x4 db = __builtin_bit_cast(i16x4, bf16x4{(__bf16)ds[0], (__bf16)ds[1], (__bf16)ds[2], (__bf16)ds[3]});
      // dK^T, then dV^T of the 16 keys (lane: key li, dims 16 dt + 4 G + e), each stored
      // as rows before the next is formed.
      const int nk = min(16, j.len - kfirst);
      const int64_t row0 = ((j.kv_tok + kfirst) * a.Hkv + j.kv) * D;
      f32x4 gr[C::DT];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        gr[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qtr[dt], db, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0) * a.scale;
      store_tile_rows<D, OutT>(gr, SL.t[tt], static_cast<OutT*>(a.dk) + row0, kstride, nk, lane);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        gr[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dtr[dt], pb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      store_tile_rows<D, OutT>(gr, SL.t[tt], static_cast<OutT*>(a.dv) + row0, kstride, nk, lane);
    });
  } else {
    stages(true, [](int, int) {});
  }
#endif
}

// ---------------------------------------------------------------- dQ = sum of the parts
template <int D>
__global__ __launch_bounds__(256) void dqsum_kernel(BwdArgs a) {
  constexpr int DPL = D / 64;
  static_assert(kMergeRowsPerGroup == 4, "four rows per workgroup, as the merge");
  const int64_t gw = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gw >= a.total_rows) return;
  const int lane = threadIdx.x & 63;
  // Sequence with row_base[lo] <= gw < row_base[lo + 1], as the merge finds it.
  const MergeGroup e = a.groups[blockIdx.x];
  int lo = e.lo_cross & ~kMergeCross;
  int sid = e.seq;
  if (e.lo_cross & kMergeCross) {
    while (lo + 1 < a.count && a.row_base[lo + 1] <= gw) ++lo;
    sid = a.seq_ids[lo];
  }
  const SeqRec sq = a.seqs[sid];
  const int64_t rem = gw - a.row_base[lo];
  const int kv = int(rem / sq.rows);
  const int r = int(rem - int64_t(kv) * sq.rows);
  const int64_t r0 = sq.row_base + int64_t(kv) * sq.nb * sq.rows + r;  // block b: r0 + b * rows
  float s[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) s[k] = 0.f;
  for (int b = 0; b < sq.nb; ++b) {
    const float* p = a.ws_dq + (r0 + int64_t(b) * sq.rows) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) s[k] += p[lane + 64 * k];
  }
  const int i = r / a.g, hl = r - i * a.g;
  float* dst = a.dq + ((sq.q_base + i) * a.Hq + int64_t(kv) * a.g + hl) * D;
#pragma unroll
  for (int k = 0; k < DPL; ++k) dst[lane + 64 * k] = s[k];
}

// ---------------------------------------------------------------- dK, dV per key tile
constexpr int KV_WAVES = 4;
constexpr int RCH = 32;     // query rows per chunk
constexpr int KV_BUFS = 3;  // chunk buffers: the chunk computed and two in flight

template <int D>
struct KvLds {
  unsigned char q[KV_BUFS][RCH * BCfg<D>::ROWB];   // Q rows, stored for row and transposing reads
  unsigned char g[KV_BUFS][RCH * BCfg<D>::ROWB];   // dO rows, likewise
  float lse[KV_BUFS][RCH];                          // the rows' LSE * log2 e
  float dd[KV_BUFS][RCH];                           // D_i
};

template <int D, bool BF16OUT>
__global__ __launch_bounds__(256, 3) void dkv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = BCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[sizeof(KvLds<D>)];
  KvLds<D>& L = *reinterpret_cast<KvLds<D>*>(smem);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float c = a.scale * LOG2E;

  // Workgroup -> (KV head kv, key tile): the plan image names the tile's sequence and
  // its index there.
  static_assert(kDkvTileKeys == 16 * KV_WAVES, "16 keys per wave");
  const int64_t wg = blockIdx.x;
  const int kv = int(wg % a.Hkv);
  const KeyTile where = a.tiles[wg / a.Hkv];
  const SeqRec sq = a.seqs[where.seq];
  const int64_t n = sq.n, k0 = int64_t(where.tile) * kDkvTileKeys;
  const int rows = sq.rows;  // q * g
  // This lane's key (the wave's 16 keys) and its K and V rows as B operands
  // (lane: key li, dims 8 G + 32 dc).
  const int64_t key = k0 + 16 * wave + li;
  const int64_t keyc = min(key, n - 1);
  bf16x8 kt[C::DC], vt[C::DC];
  {
    const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + (sq.kv_base + keyc) * a.k_st + int64_t(kv) * a.k_sh + 8 * G;
    const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + (sq.kv_base + keyc) * a.v_st + int64_t(kv) * a.v_sh + 8 * G;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      kt[dc] = *reinterpret_cast<const bf16x8*>(kp + 32 * dc);
      vt[dc] = *reinterpret_cast<const bf16x8*>(vp + 32 * dc);
    }
  }
  f32x4 dk[C::DT], dv[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Rows that see some key of the tile: query tokens i >= k0 - (n - q) when causal. Row r
  // (token r / g) sees this lane's key when r >= r_vis = g (key - (n - q)).
  const int q = sq.q;
  const int64_t i0 = a.causal ? max<int64_t>(0, k0 - (n - q)) : 0;
  const int r_begin = int(i0) * a.g;
  const int nchunk = r_begin < rows ? (rows - r_begin + RCH - 1) / RCH : 0;
  const int r_vis = a.causal ? int(min<int64_t>(max<int64_t>(int64_t(a.g) * (key - (n - q)), 0), rows)) : 0;
  const bool key_in = key < n;
  // The same for the wave's last key (wave-uniform): a chunk whose rows all exist and
  // start at or past r_vis_last is seen by all 16 keys of the wave, and needs no test.
  const int64_t key_last = k0 + 16 * wave + 15;
  const bool keys_in = key_last < n;
  const int r_vis_last =
      a.causal ? int(min<int64_t>(max<int64_t>(int64_t(a.g) * (key_last - (n - q)), 0), rows)) : 0;

  // Chunk loads, all by direct global->LDS DMA: Q and dO rows (1 KiB per instruction,
  // lane l to byte 16 l of it; LDS position p of a tile (16-byte units) is row p / CH,
  // slot p % CH, and holds the row's chunk swz_tr(row, slot), so each lane loads the chunk
  // its position needs), and the rows' LSE and D (wave 0, 4 bytes per lane). Rows past
  // the last re-read it (finite data, not visible).
  constexpr int TILE_INST = RCH * C::ROWB / 1024;      // instructions per tile
  constexpr int PER_WAVE = TILE_INST / KV_WAVES;       // per wave, per tensor
  static_assert(PER_WAVE * KV_WAVES == TILE_INST, "chunk tile split");
  // Vector-memory instructions this wave issues per chunk.
  const int per_chunk = 2 * PER_WAVE + (wave == 0 ? 2 : 0);
  auto row_src = [&](int r, int64_t& tok, int64_t& head) {
    const int i = r / a.g, hl = r - i * a.g;
    tok = sq.q_base + i;
    head = int64_t(kv) * a.g + hl;
  };
  // When g divides the chunk's row count, a lane's row of a chunk is the same (token,
  // head) offset from the chunk's first row in every chunk: the loads are a scalar base
  // per chunk plus per-lane constant offsets. Otherwise, and for a chunk that runs past
  // the last row, each lane computes its row's address.
  const bool fixed = RCH % a.g == 0;
  uint32_t fq[PER_WAVE], fg[PER_WAVE], fs = 0;
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int p = (wave * PER_WAVE + u) * 64 + lane;
    const int row = p / C::CH, cc = swz_tr<C::CH>(row, p % C::CH);
    const int i = row / a.g, hl = row - i * a.g;
    fq[u] = uint32_t(2 * (i * a.q_st + hl * a.q_sh) + 16 * cc);
    fg[u] = uint32_t(2 * (i * a.do_st + hl * a.do_sh) + 16 * cc);
  }
  fs = uint32_t((lane / a.g) * a.Hq + lane % a.g);
  // Addresses of the first row of the next chunk to load (chunks load in order), and
  // their steps per chunk (RCH / g tokens).
  const int64_t tok0 = sq.q_base + r_begin / a.g, head0 = int64_t(kv) * a.g;
  const unsigned char* nq = reinterpret_cast<const unsigned char*>(a.q) + 2 * (tok0 * a.q_st + head0 * a.q_sh);
  const unsigned char* ng = reinterpret_cast<const unsigned char*>(a.dout) + 2 * (tok0 * a.do_st + head0 * a.do_sh);
  int64_t ns = tok0 * a.Hq + head0;
  const int tstep = fixed ? RCH / a.g : 0;
  const int64_t dq_step = 2 * int64_t(tstep) * a.q_st, dg_step = 2 * int64_t(tstep) * a.do_st,
                ds_step = int64_t(tstep) * a.Hq;
  auto load_chunk = [&](int ch, int buf) {
    const int rb = r_begin + ch * RCH;
    if (fixed && rb + RCH <= rows) {
      // Each load is a uniform base plus a 32-bit lane offset. The offsets pass through
      // an empty asm so that the compiler does not keep base + offset as a 64-bit lane
      // address across the loop (registers this kernel does not have).
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const int gi = wave * PER_WAVE + u;
        uint32_t oq = fq[u], og = fg[u];
        asm volatile("" : "+v"(oq), "+v"(og));
        __builtin_amdgcn_global_load_lds(nq + oq, (lds_void*)(L.q[buf] + gi * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(ng + og, (lds_void*)(L.g[buf] + gi * 1024), 16, 0, 0);
      }
      if (wave == 0 && lane < RCH) {
        uint32_t os = 4 * fs;
        asm volatile("" : "+v"(os));
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(a.ws_l2 + ns) + os, (lds_void*)L.lse[buf], 4, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(a.ws_d + ns) + os, (lds_void*)L.dd[buf], 4, 0, 0);
      }
      nq += dq_step;
      ng += dg_step;
      ns += ds_step;
      return;
    }
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int gi = wave * PER_WAVE + u;
      const int p = gi * 64 + lane;
      const int row = p / C::CH, slot = p % C::CH;
      const int cc = swz_tr<C::CH>(row, slot);
      const int r = min(rb + row, rows - 1);
      int64_t tok, head;
      row_src(r, tok, head);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(a.q) + 2 * (tok * a.q_st + head * a.q_sh) + 16 * cc,
                                       (lds_void*)(L.q[buf] + gi * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(a.dout) + 2 * (tok * a.do_st + head * a.do_sh) + 16 * cc,
                                       (lds_void*)(L.g[buf] + gi * 1024), 16, 0, 0);
    }
    if (wave == 0 && lane < RCH) {
      int64_t tok, head;
      row_src(min(rb + lane, rows - 1), tok, head);
      __builtin_amdgcn_global_load_lds(a.ws_l2 + (tok * a.Hq + head), (lds_void*)L.lse[buf], 4, 0, 0);
      __builtin_amdgcn_global_load_lds(a.ws_d + (tok * a.Hq + head), (lds_void*)L.dd[buf], 4, 0, 0);
    }
  };
  // Lane offsets within a 16-row tile of a chunk: row reads (lane: row li, dims 8G + 32dc)
  // and transposing reads (lane: dims of tile dt, rows 4G + li/4 and 16 more).
  unsigned o_row[C::DC], o_tr[C::DT];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) o_row[dc] = li * C::ROWB + 16 * swz_tr<C::CH>(li, 4 * dc + G);
  {
    const int e = li >> 2, cc = li & 3, r = 4 * G + e;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) o_tr[dt] = r * C::ROWB + 16 * swz_tr<C::CH>(r, 2 * dt + (cc >> 1)) + 8 * (cc & 1);
  }

  // The K and V operands first (a compiler-visible wait), so that no wait for them
  // drains the chunk DMA below.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (nchunk > 0) load_chunk(0, 0);
  if (nchunk > 1) load_chunk(1, 1);
  int buf = 0;
  for (int ch = 0; ch < nchunk; ++ch) {
    // Chunk ch has landed for this wave once only chunk ch + 1's loads may be pending;
    // the barrier makes every wave's part visible, and every wave is past its reads of
    // the buffer that chunk ch + 2 now refills (last read for chunk ch - 1).
    dq_wait_barrier(ch + 1 < nchunk ? per_chunk : 0);
    if (ch + 2 < nchunk) load_chunk(ch + 2, buf == 0 ? 2 : buf - 1);
    const int rb = r_begin + ch * RCH;
    const unsigned qb = lds_addr(L.q[buf]), gb = lds_addr(L.g[buf]);
    // S and dP for the chunk's two 16-row tiles (lane: key li, rows 16 t + 4 G + e).
    f32x4 sv[2], pv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 qa[C::DC];
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) qa[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(qb + unsigned(16 * t) * C::ROWB + o_row[dc]));
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[dc], kt[dc], x, 0, 0, 0);
      sv[t] = x;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 ga[C::DC];
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) ga[dc] = *reinterpret_cast<lds_bf16x8>(uintptr_t(gb + unsigned(16 * t) * C::ROWB + o_row[dc]));
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ga[dc], vt[dc], y, 0, 0, 0);
      pv[t] = y;
    }
    // P and dS; a row that does not see the key (or lies past the last row) gives 0.
    // Every p is taken (finite inputs: rows past the last repeat it, keys past the
    // sequence its last key), and only a chunk not wholly visible to the wave selects.
    float pr[2][4], ds[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(&L.lse[buf][16 * t + 4 * G]);
#pragma unroll
      for (int e = 0; e < 4; ++e) pr[t][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t][e], c, -l2[e]));
    }
    if (!(keys_in && rb >= r_vis_last && rb + RCH <= rows)) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rb + 16 * t + 4 * G + e;
          if (!(key_in && r < rows && r >= r_vis)) pr[t][e] = 0.f;
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 dd4 = *reinterpret_cast<const f32x4*>(&L.dd[buf][16 * t + 4 * G]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[t][e] = pr[t][e] * (pv[t][e] - dd4[e]);
    }
    const bf16x8 pb = {(__bf16)pr[0][0], (__bf16)pr[0][1], (__bf16)pr[0][2], (__bf16)pr[0][3],
                       (__bf16)pr[1][0], (__bf16)pr[1][1], (__bf16)pr[1][2], (__bf16)pr[1][3]};
    const bf16x8 db = {(__bf16)ds[0][0], (__bf16)ds[0][1], (__bf16)ds[0][2], (__bf16)ds[0][3],
                       (__bf16)ds[1][0], (__bf16)ds[1][1], (__bf16)ds[1][2], (__bf16)ds[1][3]};
    // dV^T += dO^T P and dK^T += Q^T dS over the chunk's 32 rows.
    // In halves of D/32 dimension tiles, to keep the transposed operands few.
    constexpr int DH = C::DT / 2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      unsigned ga[DH];
#pragma unroll
      for (int d = 0; d < DH; ++d) ga[d] = gb + o_tr[half * DH + d];
      i16x4 lo[DH], hi[DH];
      tr_read<0, 16 * C::ROWB>(lo, hi, ga);
#pragma unroll
      for (int d = 0; d < DH; ++d)
        dv[half * DH + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[d], hi[d], 0, 1, 2, 3, 4, 5, 6, 7)), pb, dv[half * DH + d], 0, 0, 0);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      unsigned qa[DH];
#pragma unroll
      for (int d = 0; d < DH; ++d) qa[d] = qb + o_tr[half * DH + d];
      i16x4 lo[DH], hi[DH];
      tr_read<0, 16 * C::ROWB>(lo, hi, qa);
#pragma unroll
      for (int d = 0; d < DH; ++d)
        dk[half * DH + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[d], hi[d], 0, 1, 2, 3, 4, 5, 6, 7)), db, dk[half * DH + d], 0, 0, 0);
    }
    buf = buf == KV_BUFS - 1 ? 0 : buf + 1;
  }
  // Store (lane: key li, dims 16 dt + 4 G .. + 3) as whole rows through LDS, each wave
  // in its own 16 D-float area of the chunk buffers once every wave is past its last
  // chunk; keys past the sequence are not stored. bf16 outputs take each fp32 sum
  // rounded to nearest even.
  static_assert(KV_WAVES * 16 * D * 4 <= int(sizeof(KvLds<D>)), "transpose areas fit the chunk buffers");
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dk[dt] = dk[dt] * a.scale;
  {
    using OutT = typename std::conditional<BF16OUT, __bf16, float>::type;
    const int64_t kfirst = k0 + 16 * wave;
    const int nk = int(min<int64_t>(16, n - kfirst));
    const int64_t row0 = ((sq.kv_base + kfirst) * a.Hkv + kv) * D, kstride = int64_t(a.Hkv) * D;
    unsigned char* t = smem + wave * (16 * D * 4);
    store_tile_rows<D, OutT>(dk, t, static_cast<OutT*>(a.dk) + row0, kstride, nk, lane);
    store_tile_rows<D, OutT>(dv, t, static_cast<OutT*>(a.dv) + row0, kstride, nk, lane);
  }
#endif
}

template <int D>
hipError_t launch_all(const BwdArgs& a, hipStream_t stream) {
  const int64_t qrows = a.total_q * a.Hq;
  if (qrows > 0) {
    hipLaunchKernelGGL(rowdot_kernel<D>, dim3(unsigned((qrows + 3) / 4)), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  // Both grids cover every job; each kernel returns at once from the other's jobs.
  if (a.num_jobs > a.num_fused_jobs) {
    if (a.dq_waves == 4)
      hipLaunchKernelGGL((dq_kernel<D, 4>), dim3(unsigned(a.num_jobs)), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((dq_kernel<D, 8>), dim3(unsigned(a.num_jobs)), dim3(512), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (a.num_fused_jobs > 0) {
    if (a.dkv_bf16)
      hipLaunchKernelGGL((dqkv_small_kernel<D, true>), dim3(unsigned(a.num_jobs)), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((dqkv_small_kernel<D, false>), dim3(unsigned(a.num_jobs)), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (a.total_rows > 0) {
    hipLaunchKernelGGL(dqsum_kernel<D>, dim3(unsigned((a.total_rows + 3) / 4)), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (a.key_tiles > 0) {
    if (a.dkv_bf16)
      hipLaunchKernelGGL((dkv_kernel<D, true>), dim3(unsigned(a.key_tiles * a.Hkv)), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((dkv_kernel<D, false>), dim3(unsigned(a.key_tiles * a.Hkv)), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward_bf16(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if ((a.total_q * a.Hq + 3) / 4 > 0x7fffffffLL || a.num_jobs > 0x7fffffff || (a.total_rows + 3) / 4 > 0x7fffffffLL ||
      a.key_tiles * a.Hkv > 0x7fffffffLL)
    return hipErrorInvalidValue;
  if (head_dim == 128) return launch_all<128>(a, stream);
  if (head_dim == 64) return launch_all<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace splitkv
