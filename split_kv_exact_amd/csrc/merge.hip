// Log-sum-exp merge of split-KV partials (one wavefront per output row).
//
// Split-KV page, "Timeline": the method is exact, its result equals unsharded
// attention. With block partials (O_b, LSE_b) for b = 0..nb-1 of one query row:
//   M = max_b LSE_b,  w_b = e^(LSE_b - M),  O = sum_b w_b O_b / sum_b w_b,
//   LSE = M + ln sum_b w_b,
// because e^(LSE_b) O_b and e^(LSE_b) are the block's sums of e^s v and e^s. Blocks
// are summed in block order by every lane, so the result does not depend on how the
// plan spread the blocks over workers.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace splitkv {
namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr int WAVES = 4;

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int DPL = D / 64;
  const int64_t gw = int64_t(blockIdx.x) * WAVES + (threadIdx.x >> 6);
  if (gw >= a.total_rows) return;
  const int lane = threadIdx.x & 63;
  // Sequence j with row_base[j] <= gw < row_base[j + 1].
  int lo = 0, hi = a.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.row_base[mid] <= gw)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int s = a.seq_ids ? a.seq_ids[lo] : lo;
  const SeqRec sq = a.seqs[s];
  const int64_t rem = gw - a.row_base[lo];
  const int kv = int(rem / sq.rows);
  const int r = int(rem - int64_t(kv) * sq.rows);
  const int i = r / a.g, hl = r - i * a.g;
  const int64_t r0 = sq.row_base + int64_t(kv) * sq.nb * sq.rows + r;  // block b: r0 + b * rows

  float M = NEG_INF;
  for (int b = 0; b < sq.nb; ++b) M = fmaxf(M, a.ws_lse[r0 + int64_t(b) * sq.rows]);
  float W = 0.f;
  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.f;
  if (M != NEG_INF) {
    for (int b = 0; b < sq.nb; ++b) {
      const int64_t rb = r0 + int64_t(b) * sq.rows;
      const float wb = __builtin_amdgcn_exp2f((a.ws_lse[rb] - M) * LOG2E);
      W += wb;
      const float* ob = a.ws_o + rb * D;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] = __builtin_fmaf(wb, ob[lane + 64 * k], o[k]);
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int64_t idx = (sq.q_base + i) * a.Hq + kv * a.g + hl;
#pragma unroll
  for (int k = 0; k < DPL; ++k) a.out[idx * D + lane + 64 * k] = o[k] * inv;
  if (lane == 0) a.lse[idx] = W > 0.f ? M + __builtin_amdgcn_logf(W) * LN2 : NEG_INF;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  if (a.total_rows <= 0) return hipSuccess;
  const int64_t blocks = (a.total_rows + WAVES - 1) / WAVES;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(WAVES * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
