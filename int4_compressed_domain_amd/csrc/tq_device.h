// Device helpers for the gfx950 kernels: vector types, exact input widening, lane
// exchange, and the nibble -> fp16 operand unpackers used by the matrix-core loops.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define TQ_LOG2E 1.4426950408889634f

// ---- element types of the caller's tensors --------------------------------------------
struct TF32 { typedef float storage; };
struct TBF16 { typedef uint16_t storage; };
struct TF16 { typedef f16 storage; };

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float widen(f16 h) { return (float)h; }

// Load N consecutive elements (N * sizeof(T) a multiple of 4 bytes, naturally aligned)
// and widen them exactly to fp32.
template <typename T, int N>
__device__ __forceinline__ void load_widen(const T* __restrict__ p, float (&out)[N]) {
  constexpr int BYTES = N * (int)sizeof(T);
  if constexpr (BYTES % 16 == 0) {
    T tmp[N];
#pragma unroll
    for (int i = 0; i < BYTES / 16; i++)
      reinterpret_cast<u32x4*>(tmp)[i] = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
    for (int i = 0; i < N; i++) out[i] = widen(tmp[i]);
  } else if constexpr (BYTES % 8 == 0) {
    T tmp[N];
#pragma unroll
    for (int i = 0; i < BYTES / 8; i++)
      reinterpret_cast<u32x2*>(tmp)[i] = reinterpret_cast<const u32x2*>(p)[i];
#pragma unroll
    for (int i = 0; i < N; i++) out[i] = widen(tmp[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N; i++) out[i] = widen(p[i]);
  }
}

// fp32(1/sqrt(D)) for D a power of two, correctly rounded: an even power of two is exact,
// otherwise sqrt(2) rounded once to fp32 (0x3FB504F3) scaled by a power of two.
__host__ __device__ __forceinline__ float tq_rho(int D) {
  int k = 0;
  while ((1 << k) < D) k++;
  float r = (k & 1) ? 1.41421353816986083984375f : 1.0f;
  int e = (k & 1) ? -(k + 1) / 2 : -k / 2;
  return ldexpf(r, e);
}

// fp16 round-to-nearest-even with overflow clamped to +-65504.
__device__ __forceinline__ f16 f16_sat(float x) {
  f16 h = (f16)x;
  uint16_t b = __builtin_bit_cast(uint16_t, h);
  if ((b & 0x7fffu) == 0x7c00u) b = (b & 0x8000u) | 0x7bffu;
  return __builtin_bit_cast(f16, b);
}

// ---- lane exchange -------------------------------------------------------------------
// DPP row rotate right by 8 lanes inside each row of 16: lane i reads lane (i+8) mod 16.
__device__ __forceinline__ float dpp_ror8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, true));
}

// Value of lane ^ st (st = 1, 2, 4, 8: inside a row of 16 lanes) by DPP, no LDS round trip.
template <int ST>
__device__ __forceinline__ float dpp_xor(float x, int lane) {
  const int v = __float_as_int(x);
  if constexpr (ST == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, true));  // quad_perm 1 0 3 2
  else if constexpr (ST == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, true));  // quad_perm 2 3 0 1
  else if constexpr (ST == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, true));  // row_ror 8
  else {  // ST == 4 (row_ror n: lane i reads lane i - n mod 16): i + 4 is row_ror 12, i - 4 row_ror 4
    const int from_up = __builtin_amdgcn_mov_dpp(v, 0x12C, 0xf, 0xf, true);
    const int from_dn = __builtin_amdgcn_mov_dpp(v, 0x124, 0xf, 0xf, true);
    return __int_as_float((lane & 4) ? from_dn : from_up);
  }
}

// lane ^ m for a run-time-constant m in {1, 2, 4, 8} (folds once loops are unrolled)
__device__ __forceinline__ float lane_xor16(float x, int m, int lane) {
  switch (m) {
    case 1: return dpp_xor<1>(x, lane);
    case 2: return dpp_xor<2>(x, lane);
    case 4: return dpp_xor<4>(x, lane);
    default: return dpp_xor<8>(x, lane);
  }
}

// max of floats without the canonicalizing v_max x,x that fmaxf adds under IEEE mode
// (the inputs here are never signaling NaNs).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float xor_shfl(float x, int m) { return __shfl_xor(x, m, 64); }

// Butterfly exchanges across 16-lane rows (lane ^ 16) and wave halves (lane ^ 32) with the
// gfx950 permlane swaps: both outputs of a self-swap hold {x[l], x[l ^ 16|32]} in some
// order, so their max / sum is the reduction over the pair.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// (a & m) | o in one VALU instruction. gfx9 VOP3 encodings take at most one literal or
// SGPR, so the two constants are passed in VGPRs (the caller keeps them in registers).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// ---- nibble -> fp16 operand unpack ----------------------------------------------------
// fp16 0x6400 | n is the exact value 1024 + n for n < 1024; 0x6400 | (n << 4) is
// 1024 + 16 n. Subtracting (or scaling) these back is exact in fp16.
__device__ __forceinline__ f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }

// Offset-binary indices u (value u - 8) at nibble positions 0 and 4 of w.
__device__ __forceinline__ f16x2 nib_p0p4(uint32_t w) {
  const f16x2 off = {(f16)1032.0f, (f16)1032.0f};
  return as_h2((w & 0x000F000Fu) | 0x64006400u) - off;
}
// ... at positions 1 and 5.
__device__ __forceinline__ f16x2 nib_p1p5(uint32_t w) {
  const f16x2 sc = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 off = {(f16)72.0f, (f16)72.0f};
  return as_h2((w & 0x00F000F0u) | 0x64006400u) * sc - off;
}

// K operand, abs-max codec: one dword = indices of dims e = 0..7 (nibble position e) ->
// 8 halves in k-slot order [e0 e4 e1 e5 e2 e6 e3 e7].
__device__ __forceinline__ f16x8 unpack_k_absmax(uint32_t w) {
  f16x2 a = nib_p0p4(w), b = nib_p1p5(w), c = nib_p0p4(w >> 8), d = nib_p1p5(w >> 8);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Byte-wise table lookup: for 4 indices (one per byte of ix, each 0..15) return the 4
// selected bytes of a 16-byte table held in t0..t3 (bytes 0..15).
__device__ __forceinline__ uint32_t lut_bytes16(uint32_t ix, uint32_t t0, uint32_t t1, uint32_t t2,
                                                uint32_t t3) {
  uint32_t i3 = ix & 0x07070707u;
  uint32_t a = __builtin_amdgcn_perm(t1, t0, i3);
  uint32_t b = __builtin_amdgcn_perm(t3, t2, i3);
  uint32_t hb = (ix >> 3) & 0x01010101u;
  uint32_t m = (hb << 8) - hb;  // 0xFF in bytes whose index has bit 3 set
  return (b & m) | (a & ~m);
}

// K operand, Lloyd-Max codec: table lo/hi bytes of the 16 fp16 levels in lo[4], hi[4].
// One dword of indices (dims e = 0..7) -> 8 halves in k-slot order [e0 e2 e4 e6 e1 e3 e5 e7].
__device__ __forceinline__ f16x8 unpack_k_lut(uint32_t w, const uint32_t (&lo)[4], const uint32_t (&hi)[4]) {
  uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
  uint32_t le = lut_bytes16(ev, lo[0], lo[1], lo[2], lo[3]);
  uint32_t he = lut_bytes16(ev, hi[0], hi[1], hi[2], hi[3]);
  uint32_t lodd = lut_bytes16(od, lo[0], lo[1], lo[2], lo[3]);
  uint32_t hodd = lut_bytes16(od, hi[0], hi[1], hi[2], hi[3]);
  f16x2 a = as_h2(__builtin_amdgcn_perm(he, le, 0x05010400u));    // e0 e2
  f16x2 b = as_h2(__builtin_amdgcn_perm(he, le, 0x07030602u));    // e4 e6
  f16x2 c = as_h2(__builtin_amdgcn_perm(hodd, lodd, 0x05010400u)); // e1 e3
  f16x2 d = as_h2(__builtin_amdgcn_perm(hodd, lodd, 0x07030602u)); // e5 e7
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Dim offset (0..7 inside an 8-dim chunk) held by k-slot s of the K operand.
template <int KCODEC>
__host__ __device__ __forceinline__ int kslot_dim(int s) {
  if constexpr (KCODEC == TQ_CODEC_ABSMAX) return (s >> 1) + ((s & 1) << 2);  // 0 4 1 5 2 6 3 7
  else return ((s & 3) << 1) + (s >> 2);                                      // 0 2 4 6 1 3 5 7
}

// Lloyd-Max levels of N(0,1) with 16 cells divided by sqrt(32), rounded to fp16
// (increasing index order). Derived by csrc/gen_lloydmax.py.
#define TQ_LUT16_BITS                                                                  \
  {0xb7bbu, 0xb5dau, 0xb494u, 0xb31bu, 0xb155u, 0xaf6eu, 0xac64u, 0xa5cfu,               \
   0x25cfu, 0x2c64u, 0x2f6eu, 0x3155u, 0x331bu, 0x3494u, 0x35dau, 0x37bbu}
