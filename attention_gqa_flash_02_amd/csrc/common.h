// Shared device helpers for the gfx950 attention kernels: vector types, MFMA
// wrappers, conversions and wave-level reductions. CDNA4 only (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// Word 3 of a raw buffer resource on gfx950 (32-bit data format; no swizzle, no stride): out of
// range accesses (offset >= num_records) read zero.
constexpr int kBufferFlags = 0x00020000;

// ---- MFMA (matrix cores). Lane layouts, for lane l of the 64-lane wave:
//   16x16xK: A[i][k] at lane (i = l%16), k-slots KPL*(l/16) .. +KPL-1 (KPL = K/4)
//            B[k][j] at lane (j = l%16), same k-slots
//            C[i][j] at lane (j = l%16), acc r <-> row i = 4*(l/16) + r
//   32x32x16: A[i][k] at lane (i = l%32), k-slots 8*(l/32) .. +7; B symmetric;
//            C[i][j] at lane (j = l%32), acc r <-> row i = 8*(r/4) + 4*(l/32) + r%4
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- conversions
// Two OCP e4m3fn codes (bytes 0,1 of the selected 16-bit half of w) -> two bf16, exact
// (every finite e4m3fn value is a bf16 value).
template <bool HI>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}
// Four e4m3fn codes packed in a dword -> four bf16.
__device__ __forceinline__ bf16x4 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = fp8x2_to_bf16x2<false>(w);
  bf16x2 hi = fp8x2_to_bf16x2<true>(w);
  return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}
// Eight e4m3fn codes in two dwords -> eight bf16.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  bf16x4 a = fp8x4_to_bf16x4(w0);
  bf16x4 b = fp8x4_to_bf16x4(w1);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ bf16x4 f32x4_to_bf16x4(f32x4 x) {
  return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

// max(a, b, c) in one v_max3_f32.
__device__ __forceinline__ float max3(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x2 cvt_pk_bf16(float a, float b) {
  return bf16x2{(bf16)a, (bf16)b};
}

// 2^x on the VALU transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max(x, x of lane l ^ 32) in every lane: one cross-half swap on the VALU (v_permlane32_swap
// exchanges lanes 32-63 of its first operand with lanes 0-31 of its second), no LDS round trip.
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---- cross-lane reductions over lanes l, l^16, l^32, l^48 (the four k-slot groups of a
// 16-wide MFMA column).
__device__ __forceinline__ float max_over_quads(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  x = fmaxf(x, __shfl_xor(x, 32, kWave));
  return x;
}
__device__ __forceinline__ float sum_over_quads(float x) {
  x += __shfl_xor(x, 16, kWave);
  x += __shfl_xor(x, 32, kWave);
  return x;
}

// Plain global loads of 16 / 8 / 4 bytes.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }
// Nontemporal loads (the nt bit: the lines are filled evict-first). For data read once, whole
// lines at a time, a stream of these reaches about 7.0 TB/s on MI355X against about 6.3 TB/s for
// plain loads; a line whose other half is read by a later load may have to be fetched twice.
__device__ __forceinline__ u32x4 ld16nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
__device__ __forceinline__ u32x2 ld8nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)); }

template <typename T, typename S>
__device__ __forceinline__ T bitcast(S s) {
  static_assert(sizeof(T) == sizeof(S), "size mismatch");
  return __builtin_bit_cast(T, s);
}

}  // namespace attn
