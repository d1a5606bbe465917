// LDS tile helpers and the partial-output store shared by the bf16 attention kernels
// (gfx950).
#pragma once
#include <hip/hip_runtime.h>

namespace splitkv {
namespace lds {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8* lds_bf16x8;

// XOR swizzles of the 16-byte chunk index c within a row of CH chunks: swz_row keeps
// 16-lane row reads (one row per lane, 16 bytes each) free of bank conflicts,
// swz_tr the 32-lane transposing reads (ds_read_b64_tr_b16). Both depend on the row
// modulo 16 only, so tiles that start at multiples of 16 rows share lane offsets.
template <int CH>
__device__ __forceinline__ int swz_row(int row, int c) { return c ^ (row & (CH - 1)); }
template <int CH>
__device__ __forceinline__ int swz_tr(int row, int c) { return c ^ ((2 * row) & (CH - 1)); }

// Row-scaled fp16 store of one row of a partial output. o[dt] holds this lane's
// elements of the row, dims 16 dt + 4 G .. + 3 (the transposed accumulator of both
// bf16 kernels; the row's other elements are on the lanes 16 and 32 apart), before
// normalisation by inv. The row's scale is its largest |o * inv|; each element is
// stored as fp16(o / max|o|), so element * scale is within scale * 2^-12 of o * inv,
// and (lse, scale) goes to lp[0..1]. DT + 1 store instructions, as the fp32 form.
// NT: the elements carry the non-temporal hint (the pair always does). Each element
// store writes 32-byte pieces of 16 rows; the matrix-core kernel stores them cached,
// because there non-temporal pieces reached HBM as separate partial-line writes
// (measured: 2.2 times the elements' bytes), while cached ones merge in L2.
template <int DT, bool NT>
__device__ __forceinline__ void store_row_h16(const f32x4 (&o)[DT], float inv, float lse, _Float16* hp, float* lp,
                                              int G) {
  float mx = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(o[dt][e]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float k = mx > 0.f ? 1.f / mx : 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const f16x4 h = {(_Float16)(o[dt][0] * k), (_Float16)(o[dt][1] * k), (_Float16)(o[dt][2] * k),
                     (_Float16)(o[dt][3] * k)};
    if constexpr (NT)
      __builtin_nontemporal_store(h, reinterpret_cast<f16x4*>(hp + 16 * dt + 4 * G));
    else
      *reinterpret_cast<f16x4*>(hp + 16 * dt + 4 * G) = h;
  }
  const f32x2 ls = {lse, mx * inv};
  __builtin_nontemporal_store(ls, reinterpret_cast<f32x2*>(lp));
}

__device__ __forceinline__ unsigned lds_addr(const unsigned char* p) {
  typedef __attribute__((address_space(3))) const unsigned char* lds_cptr;
  return (unsigned)(uintptr_t)(lds_cptr)p;  // 32-bit LDS offset
}

// Transposing LDS reads (ds_read_b64_tr_b16) issued from inline assembly. Through the
// builtin, the compiler cannot tell that they read a different pipeline slot than the
// in-flight DMA writes, and it drains all of that DMA first. The reads and their
// lgkmcnt wait sit in one asm statement, so no instruction can touch the destination
// registers while the loads are still in flight. Lane addresses are a[dt] + OFF (keys
// 0-15 of the step) and a[dt] + OFF + HI (keys 16-31).
template <int OFF, int HI>
__device__ __forceinline__ void tr_read(i16x4 (&lo)[8], i16x4 (&hi)[8], const unsigned (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\tds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %2, %18 offset:%24\n\tds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %4, %20 offset:%24\n\tds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %22 offset:%24\n\tds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%25\n\tds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:%25\n\tds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %20 offset:%25\n\tds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %14, %22 offset:%25\n\tds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(lo[4]), "=&v"(lo[5]), "=&v"(lo[6]),
        "=&v"(lo[7]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]), "=&v"(hi[3]), "=&v"(hi[4]), "=&v"(hi[5]),
        "=&v"(hi[6]), "=&v"(hi[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF),
        "i"(OFF + HI));
}
template <int OFF, int HI>
__device__ __forceinline__ void tr_read(i16x4 (&lo)[4], i16x4 (&hi)[4], const unsigned (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\tds_read_b64_tr_b16 %1, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%12\n\tds_read_b64_tr_b16 %3, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n\tds_read_b64_tr_b16 %5, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:%13\n\tds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
        "=&v"(hi[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF), "i"(OFF + HI));
}
template <int OFF, int HI>
__device__ __forceinline__ void tr_read(i16x4 (&lo)[2], i16x4 (&hi)[2], const unsigned (&a)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\tds_read_b64_tr_b16 %1, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\tds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(hi[0]), "=&v"(hi[1])
      : "v"(a[0]), "v"(a[1]), "i"(OFF), "i"(OFF + HI));
}

}  // namespace lds
}  // namespace splitkv
