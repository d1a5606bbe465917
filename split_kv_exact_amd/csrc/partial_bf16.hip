// Partial attention of split-KV units on gfx950 matrix cores (bf16 inputs, fp32 math).
//
// Split-KV page, lede: each context KV block yields a result the size of the
// queries; here that is, for every query row of the unit, the block's softmax output
// O_b and its log-sum-exp LSE_b (natural log). The page describes no kernel; this is
// a CDNA4 design.
//
// Execution model
//   * One workgroup (4 wavefronts) per LPT worker; it walks the worker's unit list in
//     plan order. A unit is (sequence, KV block, KV head[s]).
//   * Query rows of a KV head are r = i*g + (h - kv*g) (query token i, head h), in
//     16-row tiles. Depending on the row count the 4 waves split the tiles (rows) or
//     the unit's key range (tokens), or both; token slices are merged in LDS.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: the
//     A operand is 16 keys x 32 dims read straight from HBM (16 contiguous bytes per
//     lane), the B operand 32 dims x 16 query rows held in registers. Each lane then
//     owns one query row and 4+4 keys of a 32-key chunk, so the row max needs only
//     two cross-lane steps and the row sum none until the end.
//   * Output is accumulated transposed too, O^T += V^T P^T. P^T comes straight from the
//     score registers (rounded to bf16); V^T is read from a wave-private LDS copy of
//     the 32-key chunk with ds_read_b64_tr_b16, which hands each lane four keys of one
//     dimension. The key order inside the MFMA contraction is permuted identically on
//     both operands, which leaves the sum unchanged.
//   * Softmax runs in base 2 on raw scores: p = 2^(s*c - m*c) with c = scale*log2(e)
//     and m the running row max; LSE = scale*m + ln(l).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace splitkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;    // wavefronts per workgroup
constexpr int KT = 32;   // keys per chunk (two 16-key MFMA tiles)
constexpr int RTW = 2;   // at most 2 row tiles (32 rows) per wave at a time
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994531f;
constexpr float NEG_INF = -__builtin_huge_valf();

template <int D>
struct Cfg {
  static constexpr int DC = D / 32;           // 32-dim slices of the QK^T contraction
  static constexpr int DT = D / 16;           // 16-dim output tiles
  static constexpr int VROW = D + 16;         // LDS row stride (elements), 32 bytes of padding
  static constexpr int VCH = D / 8;           // 16-byte pieces per key row
  static constexpr int NV = KT * VCH / 64;    // 16-byte V pieces per lane per chunk
  static constexpr int VSTAGE = KT * VROW;    // elements of one wave's V staging area
  static constexpr int MSLOT = 64 * (DT * 4 + 2);  // floats of one merge slot
  static constexpr int MSLOTS = 4;
};

// Shared memory: V staging (per wave) + merge slots. Sized to at least 96 KiB so a
// compute unit holds one workgroup, i.e. one LPT worker per CU.
constexpr int LDS_BYTES = 96 * 1024;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bf16x8 load16(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float wave_max16x4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum16x4(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int D>
struct WaveState {
  f32x4 o[RTW][Cfg<D>::DT];
  float m[RTW];  // running max of raw scores (row of this lane)
  float l[RTW];  // this lane's share of the row's sum of p
};

// Process one pass: up to RTW row tiles of this wave against key chunks [c0, c1).
template <int D>
__device__ __forceinline__ void run_pass(WaveState<D>& st, const PartialArgs& a, const SeqRec& sq,
                                         int kv, int64_t key0, int len, int lim0, int tile0, int tstride,
                                         int nt, int c0, int c1, __bf16* vst) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const int R = sq.rows, g = a.g;
  const float c = a.scale * LOG2E;

  // Q^T operands (B: 32 dims x 16 rows; lane holds row li, dims 8G..8G+7 of each slice).
  bf16x8 qop[RTW][C::DC];
  int lim[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int row = (tile0 + t * tstride) * 16 + li;
    const bool ok = t < nt && row < R;
    const int i = ok ? row / g : 0;
    lim[t] = lim0 + i;
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (sq.q_base + i) * a.q_st +
                       int64_t(kv * g + (ok ? row - i * g : 0)) * a.q_sh + 8 * G;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      if (ok)
        qop[t][dc] = load16(qp + 32 * dc);
      else
        qop[t][dc] = bf16x8{};
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) st.o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m[t] = NEG_INF;
    st.l[t] = 0.f;
  }

  // Key range this wave's rows can see at all.
  const int last_tile = tile0 + (nt - 1) * tstride;
  const int rmax = min(R - 1, last_tile * 16 + 15);
  const int rmin = tile0 * 16;
  const int tmax = a.causal ? min(len - 1, lim0 + rmax / g) : len - 1;
  const int tmin_lim = a.causal ? lim0 + rmin / g : len - 1;  // smallest row limit
  const int c_end = tmax < 0 ? c0 : min(c1, tmax / KT + 1);

  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + (sq.kv_base + key0) * a.k_st + int64_t(kv) * a.k_sh;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + (sq.kv_base + key0) * a.v_st + int64_t(kv) * a.v_sh;

  for (int ch = c0; ch < c_end; ++ch) {
    const int tok0 = ch * KT;
    // K operands (A: 16 keys x 32 dims; lane holds key li, dims 8G..8G+7).
    bf16x8 kop[2][C::DC];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = tok0 + 16 * tt + li;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        if (tok < len)
          kop[tt][dc] = load16(kb + int64_t(tok) * a.k_st + 32 * dc + 8 * G);
        else
          kop[tt][dc] = bf16x8{};
      }
    }
    // V chunk -> LDS (coalesced 16-byte pieces; rows past the block end are zero).
    u32x4 vreg[C::NV];
#pragma unroll
    for (int it = 0; it < C::NV; ++it) {
      const int p = it * 64 + lane;
      const int row = p / C::VCH, pc = p % C::VCH;
      const int tok = tok0 + row;
      if (tok < len)
        vreg[it] = *reinterpret_cast<const u32x4*>(vb + int64_t(tok) * a.v_st + 8 * pc);
      else
        vreg[it] = u32x4{0u, 0u, 0u, 0u};
    }
    wave_sync();  // previous chunk's LDS reads are done before overwriting
#pragma unroll
    for (int it = 0; it < C::NV; ++it) {
      const int p = it * 64 + lane;
      const int row = p / C::VCH, pc = p % C::VCH;
      *reinterpret_cast<u32x4*>(vst + row * C::VROW + 8 * pc) = vreg[it];
    }
    wave_sync();
    // V^T operands (A: 16 dims x 32 keys) via transposing LDS reads.
    bf16x8 vop[C::DT];
    {
      const int e = li >> 2, cc = li & 3;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const __bf16* p0 = vst + (4 * G + e) * C::VROW + 16 * dt + 4 * cc;
        const __bf16* p1 = p0 + 16 * C::VROW;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p1));
        i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        vop[dt] = __builtin_bit_cast(bf16x8, both);
      }
    }
    const bool need_mask = (tok0 + KT > len) || (a.causal && tok0 + KT - 1 > tmin_lim);

#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      if (t < nt) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) {
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][dc], qop[t][dc], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][dc], qop[t][dc], s1, 0, 0, 0);
        }
        float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        if (need_mask) {
          const int lt = a.causal ? min(lim[t], len - 1) : len - 1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tok = tok0 + (e >> 2) * 16 + 4 * G + (e & 3);
            if (tok > lt) s[e] = NEG_INF;
          }
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
        mx = wave_max16x4(mx);
        const float mnew = fmaxf(st.m[t], mx);
        const float muse = mnew == NEG_INF ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f((st.m[t] - muse) * c);
        st.m[t] = mnew;
        const float mc = muse * c;
        bf16x8 pb;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // The row sum uses the fp32 values (it sets the LSE); only the PV operand is
          // rounded to bf16.
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, -mc));
          pb[e] = (__bf16)pe;
          psum += pe;
        }
        st.l[t] = st.l[t] * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          st.o[t][dt] *= alpha;
          st.o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[dt], pb, st.o[t][dt], 0, 0, 0);
        }
      }
    }
  }
}

// Normalise and write one tile of results (row li of the tile, dims 16dt+4G..+3).
template <int D>
__device__ __forceinline__ void write_tile(const WaveState<D>& st, int t, const PartialArgs& a, const SeqRec& sq,
                                           int kv, int block, int tile, bool direct) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const float l = wave_sum16x4(st.l[t]);
  const int row = tile * 16 + li;
  if (row >= sq.rows) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? st.m[t] * a.scale + __builtin_amdgcn_logf(l) * LN2 : NEG_INF;
  float* op;
  float* lp;
  if (direct) {
    const int i = row / a.g, hl = row - i * a.g;
    const int64_t idx = (sq.q_base + i) * a.Hq + kv * a.g + hl;
    op = a.out + idx * D;
    lp = a.lse + idx;
  } else {
    const int64_t prow = sq.row_base + (int64_t(kv) * sq.nb + block) * sq.rows + row;
    op = a.ws_o + prow * D;
    lp = a.ws_lse + prow;
  }
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    f32x4 v = st.o[t][dt] * inv;
    *reinterpret_cast<f32x4*>(op + 16 * dt + 4 * G) = v;
  }
  if (G == 0) *lp = lse;
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void partial_bf16_kernel(PartialArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
  static_assert(NW * C::VSTAGE * 2 + C::MSLOTS * C::MSLOT * 4 <= LDS_BYTES, "LDS budget");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __bf16* vst = reinterpret_cast<__bf16*>(smem) + wave * C::VSTAGE;
  float* mbuf = reinterpret_cast<float*>(smem + NW * C::VSTAGE * 2);

  const int w = blockIdx.x;
  const int u0 = a.worker_ptr[w], u1 = a.worker_ptr[w + 1];
  for (int ui = u0; ui < u1; ++ui) {
    const UnitRec u = a.units[ui];
    const SeqRec sq = a.seqs[u.seq];
    const int64_t key0 = int64_t(u.block) * a.B;
    const int len = int(min(int64_t(a.B), sq.n - key0));
    // Row r (query token i = r / g) sees block keys t <= lim0 + i. lim0 >= 1 - q_s since
    // the block starts before the context ends; values above len change nothing.
    const int lim0 = int(min(int64_t(len), sq.n - sq.q - key0));
    const int R = sq.rows;
    const bool direct = a.out != nullptr && sq.nb == 1;
    const int nrt = (R + 15) >> 4;
    const int Wr = nrt >= 4 ? 4 : (nrt >= 2 ? 2 : 1);
    const int Wk = NW / Wr;
    const int rg = wave % Wr, ks = wave / Wr;
    const int nc = (len + KT - 1) / KT;
    const int c0 = ks * nc / Wk, c1 = (ks + 1) * nc / Wk;
    const int ntw = rg < nrt ? (nrt - rg + Wr - 1) / Wr : 0;  // tiles of this wave's row group

    for (int kv = u.kv0; kv < u.kv0 + u.nkv; ++kv) {
      if (Wk == 1) {
        for (int pass = 0; pass < ntw; pass += RTW) {
          const int nt = min(RTW, ntw - pass);
          const int tile0 = rg + pass * Wr;
          WaveState<D> st;
          run_pass<D>(st, a, sq, kv, key0, len, lim0, tile0, Wr, nt, c0, c1, vst);
#pragma unroll
          for (int t = 0; t < RTW; ++t)
            if (t < nt) write_tile<D>(st, t, a, sq, kv, u.block, tile0 + t * Wr, direct);
        }
      } else {
        // Every wave holds 1 or 2 tiles here (nrt <= 3), one pass, then a merge of
        // the Wk token slices of each row group through LDS.
        const int nt = ntw;
        const int maxt = Wr == 1 ? 1 : 2;  // merge slots: (ks-1, rg, t) -> at most 4
        WaveState<D> st;
        run_pass<D>(st, a, sq, kv, key0, len, lim0, rg, Wr, nt, c0, c1, vst);
        if (ks > 0) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (t < nt) {
              float* slot = mbuf + (((ks - 1) * Wr + rg) * maxt + t) * C::MSLOT;
              slot[lane] = st.m[t];
              slot[64 + lane] = st.l[t];
#pragma unroll
              for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) slot[(2 + dt * 4 + j) * 64 + lane] = st.o[t][dt][j];
            }
          }
        }
        __syncthreads();
        if (ks == 0) {
          const float c = a.scale * LOG2E;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (t < nt) {
              for (int k2 = 1; k2 < Wk; ++k2) {
                const float* slot = mbuf + (((k2 - 1) * Wr + rg) * maxt + t) * C::MSLOT;
                const float m2 = slot[lane];
                const float ms = fmaxf(st.m[t], m2);
                if (ms == NEG_INF) continue;
                const float a1 = __builtin_amdgcn_exp2f((st.m[t] - ms) * c);
                const float a2 = __builtin_amdgcn_exp2f((m2 - ms) * c);
                st.l[t] = st.l[t] * a1 + slot[64 + lane] * a2;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                  for (int j = 0; j < 4; ++j)
                    st.o[t][dt][j] = st.o[t][dt][j] * a1 + slot[(2 + dt * 4 + j) * 64 + lane] * a2;
                st.m[t] = ms;
              }
              write_tile<D>(st, t, a, sq, kv, u.block, rg + t * Wr, direct);
            }
          }
        }
        __syncthreads();
      }
    }
  }
}

}  // namespace

hipError_t launch_partial_bf16(const PartialArgs& a, int head_dim, hipStream_t stream) {
  dim3 grid(a.num_workers), block(NW * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL(partial_bf16_kernel<128>, grid, block, 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(partial_bf16_kernel<64>, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace splitkv
