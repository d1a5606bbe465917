// Partial attention of split-KV units for fp32 inputs, on the vector ALUs.
//
// Same contract as the bf16 kernel (Split-KV page, lede: each context KV block
// yields a query-sized result, here O_b and LSE_b per query row). fp32 inputs keep
// full fp32 products, so this path uses plain FMAs rather than matrix cores:
//   * one workgroup (4 wavefronts) per LPT worker, walking its unit list;
//   * each wave takes query rows round-robin; for a row it streams the block's keys
//     64 at a time (one key per lane), forms the score with a dot product, updates
//     the running max and sum with wave reductions, then accumulates P V with each
//     lane owning head_dim/64 output dimensions (coalesced V rows).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace splitkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float NEG_INF = -__builtin_huge_valf();

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

template <int D>
__global__ __launch_bounds__(256) void partial_f32_kernel(PartialArgs a) {
  constexpr int DPL = D / 64;  // output dims per lane
  __shared__ float qrow[NW][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float c = a.scale * LOG2E;
  const int w = blockIdx.x;
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const int u0 = a.worker_ptr[w], u1 = a.worker_ptr[w + 1];
  for (int ui = u0; ui < u1; ++ui) {
    const UnitRec u = a.units[ui];
    const SeqRec sq = a.seqs[u.seq];
    const int64_t key0 = int64_t(u.block) * a.B;
    const int len = int(min(int64_t(a.B), sq.n - key0));
    const int lim0 = int(min(int64_t(len), sq.n - sq.q - key0));
    const bool direct = a.out != nullptr && sq.nb == 1;
    for (int kv = u.kv0; kv < u.kv0 + u.nkv; ++kv) {
      const float* kb = reinterpret_cast<const float*>(a.k) + (sq.kv_base + key0) * a.k_st + int64_t(kv) * a.k_sh;
      const float* vb = reinterpret_cast<const float*>(a.v) + (sq.kv_base + key0) * a.v_st + int64_t(kv) * a.v_sh;
      for (int row = wave; row < sq.rows; row += NW) {
        const int i = row / a.g, hl = row - i * a.g;
        const float* qp = reinterpret_cast<const float*>(a.q) + (sq.q_base + i) * a.q_st + int64_t(kv * a.g + hl) * a.q_sh;
        for (int d = lane; d < D; d += 64) qrow[wave][d] = qp[d];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int last = a.causal ? min(len - 1, lim0 + i) : len - 1;  // last visible key
        float m = NEG_INF, l = 0.f;
        float o[DPL];
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] = 0.f;
        for (int t0 = 0; t0 <= last; t0 += 64) {
          const int t = t0 + lane;
          float s = NEG_INF;
          if (t <= last) {
            const f32x4* kr = reinterpret_cast<const f32x4*>(kb + int64_t(t) * a.k_st);
            float acc = 0.f;
#pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
              const f32x4 kk = kr[d4];
              acc = __builtin_fmaf(qrow[wave][4 * d4 + 0], kk[0], acc);
              acc = __builtin_fmaf(qrow[wave][4 * d4 + 1], kk[1], acc);
              acc = __builtin_fmaf(qrow[wave][4 * d4 + 2], kk[2], acc);
              acc = __builtin_fmaf(qrow[wave][4 * d4 + 3], kk[3], acc);
            }
            s = acc;
          }
          const float mnew = fmaxf(m, wave_max(s));  // finite: key t0 <= last is visible
          const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, c, -mnew * c));
          l = l * alpha + wave_sum(p);
#pragma unroll
          for (int k = 0; k < DPL; ++k) o[k] *= alpha;
          const int nk = min(64, last - t0 + 1);
          for (int j = 0; j < nk; ++j) {
            const float pj = __shfl(p, j);
            const float* vr = vb + int64_t(t0 + j) * a.v_st;
#pragma unroll
            for (int k = 0; k < DPL; ++k) o[k] = __builtin_fmaf(pj, vr[lane + 64 * k], o[k]);
          }
          m = mnew;
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float lse = l > 0.f ? m * a.scale + __builtin_amdgcn_logf(l) * LN2 : NEG_INF;
        float* op;
        float* lp;
        if (direct) {
          const int64_t idx = (sq.q_base + i) * a.Hq + kv * a.g + hl;
          op = a.out + idx * D;
          lp = a.lse + idx;
        } else {
          const int64_t prow = sq.row_base + (int64_t(kv) * sq.nb + u.block) * sq.rows + row;
          op = a.ws_o + prow * D;
          lp = a.ws_lse + prow;
        }
#pragma unroll
        for (int k = 0; k < DPL; ++k) op[lane + 64 * k] = o[k] * inv;
        if (lane == 0) *lp = lse;
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  if (a.clock != nullptr && threadIdx.x == 0) {
    a.clock[2 * w] = t_start;
    a.clock[2 * w + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

}  // namespace

hipError_t launch_partial_f32(const PartialArgs& a, int head_dim, hipStream_t stream) {
  dim3 grid(a.num_workers), block(NW * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL(partial_f32_kernel<128>, grid, block, 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(partial_f32_kernel<64>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
