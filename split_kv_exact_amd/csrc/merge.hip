// Log-sum-exp merge of split-KV partials (one wavefront per output row).
//
// Split-KV page, "Timeline": the method is exact, its result equals unsharded
// attention. With block partials (O_b, LSE_b) for b = 0..nb-1 of one query row:
//   M = max_b LSE_b,  w_b = e^(LSE_b - M),  O = sum_b w_b O_b / sum_b w_b,
//   LSE = M + ln sum_b w_b,
// because e^(LSE_b) O_b and e^(LSE_b) are the block's sums of e^s v and e^s.
//
// A workgroup merges kMergeRowsPerGroup consecutive rows; the plan image names the
// sequence of its first row, so a row's sequence costs one load (a group that straddles
// two sequences walks on from there).
// Layout of the work: lane b holds LSE_b (64 blocks at a time), so M and sum_b w_b are
// wave reductions; the output row is then accumulated in block order, each lane owning
// head_dim/64 dimensions, with the loads of 16 blocks issued before they are used (the
// first 16 before the maximum is formed). Block order is fixed, so the result does not
// depend on how the plan spread the blocks over workers. The partials are read once, with
// the non-temporal hint (rows of many blocks merged from cold caches: batch of 8 with
// 512-key blocks 36 -> 23 us, one 1M-key context 165 -> 112 us), and lane b keeps LSE_b of
// the first 64 blocks between the two passes.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace splitkv {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr int WAVES = kMergeRowsPerGroup;
constexpr int UNROLL = 16;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// H16: partials stored as fp16 elements times a per-row scale, with (LSE, scale) pairs;
// a lane then owns D/64 consecutive dimensions (one load per block row), and block b's
// elements enter the sum weighted by w_b * scale_b while the denominator takes w_b.
template <int D, bool H16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int DPL = D / 64;
  const int64_t gw = int64_t(blockIdx.x) * WAVES + (threadIdx.x >> 6);
  if (gw >= a.total_rows) return;
  const int lane = threadIdx.x & 63;
  // Sequence lo with row_base[lo] <= gw < row_base[lo + 1]: the plan names the one of
  // the workgroup's first row; only a group that straddles sequences looks further.
  const MergeGroup e = a.groups[blockIdx.x];
  int lo = e.lo_cross & ~kMergeCross;
  int s = e.seq;
  if (e.lo_cross & kMergeCross) {
    while (lo + 1 < a.count && a.row_base[lo + 1] <= gw) ++lo;
    s = a.seq_ids ? a.seq_ids[lo] : lo;
  }
  const SeqRec sq = a.seqs[s];
  const int64_t rem = gw - a.row_base[lo];
  const int kv = int(rem / sq.rows);
  const int r = int(rem - int64_t(kv) * sq.rows);
  const int i = r / a.g, hl = r - i * a.g;
  const int nb = sq.nb;
  const int64_t r0 = sq.row_base + int64_t(kv) * nb * sq.rows + r;  // block b: r0 + b * rows
  const int64_t rs = sq.rows;
  const _Float16* wh = reinterpret_cast<const _Float16*>(a.ws_o);
  typedef _Float16 f16v __attribute__((ext_vector_type(DPL)));
  typedef float f32v __attribute__((ext_vector_type(2)));

  // M = max_b LSE_b, then W = sum_b e^(LSE_b - M), lanes over blocks. The first blocks'
  // rows are requested before the maximum is formed (they do not depend on it).
  float v[UNROLL][DPL];
  auto load = [&](int b0, int j0, int cnt) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int jb = min(j0 + u, cnt - 1);
      const int64_t row = r0 + (b0 + jb) * rs;
      if constexpr (H16) {
        const f16v h = __builtin_nontemporal_load(reinterpret_cast<const f16v*>(wh + row * D + DPL * lane));
#pragma unroll
        for (int k = 0; k < DPL; ++k) v[u][k] = float(h[k]);
      } else {
        const float* ob = a.ws_o + row * D;
#pragma unroll
        for (int k = 0; k < DPL; ++k) v[u][k] = __builtin_nontemporal_load(ob + lane + 64 * k);
      }
    }
  };
  // Lane b's LSE_b (and row scale) of block b0 + lane.
  auto stats = [&](int b, float& lse_b, float& scale_b) {
    if constexpr (H16) {
      const f32v p = b < nb ? __builtin_nontemporal_load(reinterpret_cast<const f32v*>(a.ws_lse + 2 * (r0 + b * rs)))
                            : f32v{NEG_INF, 0.f};
      lse_b = p[0];
      scale_b = p[1];
    } else {
      lse_b = b < nb ? __builtin_nontemporal_load(a.ws_lse + r0 + b * rs) : NEG_INF;
      scale_b = 1.f;
    }
  };
  load(0, 0, min(64, nb));
  // Lane b keeps LSE_b (and scale_b) of the first 64 blocks for the weights below.
  float lse0, sc0;
  stats(lane, lse0, sc0);
  float M = lse0;
  for (int b0 = 64; b0 < nb; b0 += 64) {
    float lb, sb;
    stats(b0 + lane, lb, sb);
    M = fmaxf(M, lb);
  }
  M = wave_max(M);
  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.f;
  float W = 0.f;
  if (M != NEG_INF) {
    for (int b0 = 0; b0 < nb; b0 += 64) {
      const int b = b0 + lane;
      float lb = lse0, sb = sc0;
      if (b0 > 0) stats(b, lb, sb);
      const float wl = b < nb ? __builtin_amdgcn_exp2f((lb - M) * LOG2E) : 0.f;
      W += wl;
      const float wo = H16 ? wl * sb : wl;  // weight of the block's stored elements
      const int cnt = min(64, nb - b0);
      for (int j0 = 0; j0 < cnt; j0 += UNROLL) {
        if (b0 > 0 || j0 > 0) load(b0, j0, cnt);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          if (j0 + u < cnt) {
            const float wb = __shfl(wo, j0 + u);
#pragma unroll
            for (int k = 0; k < DPL; ++k) o[k] = __builtin_fmaf(wb, v[u][k], o[k]);
          }
        }
      }
    }
    W = wave_sum(W);
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int64_t idx = (sq.q_base + i) * a.Hq + kv * a.g + hl;
  if constexpr (H16) {
#pragma unroll
    for (int k = 0; k < DPL; ++k) a.out[idx * D + DPL * lane + k] = o[k] * inv;
  } else {
#pragma unroll
    for (int k = 0; k < DPL; ++k) a.out[idx * D + lane + 64 * k] = o[k] * inv;
  }
  if (lane == 0) a.lse[idx] = W > 0.f ? M + __builtin_amdgcn_logf(W) * LN2 : NEG_INF;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  if (a.total_rows <= 0) return hipSuccess;
  const int64_t blocks = (a.total_rows + WAVES - 1) / WAVES;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(WAVES * 64);
  if (head_dim == 128 && a.h16)
    hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, stream, a);
  else if (head_dim == 64 && a.h16)
    hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
