// Dequantize reference: dense K and V from the packed pool, the first half of the
// dequantize-then-attend baseline [Open-TQ-Metal, arXiv abstract].
// One wavefront per (sequence, kv head, page): it loads the page's block with one set of
// coalesced vector loads, in the block's own lane order, and writes 16 rows of K and V.
// K (4-bit codes): lane l = 16j + t holds token t, dims 32g + 8j + e (e = 0..7, g < D/32).
// fp16 keys: the same lanes and dims, copied as stored (they have no rotated form).
// V: lane 16j + i holds row 16j + m of the value region, m = i ^ 3*bit2(i) (so that every
// cross-lane butterfly partner is one DPP move away): tokens 4j + e (e = 0..3), dims
// 32g + 2m + {0, 1}; packed 3- and 2-bit values are first rebuilt into that 4-bit layout.
// Values (u - 8)*s (4-bit), (u - 4)*s or (u - 2)*s (3- and 2-bit values) or LUT_u*n are
// exact in fp32. The original-basis variant applies the fp32 inverse rotation
// diag(sigma)*rho*H with the forward rotation's stage order: butterflies of stride 1, 2,
// ..., D/2 (each an in-lane pair or a lane-xor pair, as the dims fall), then x rho, then the
// signs. Compiled with -ffp-contract=off.
#include <type_traits>

#include "tq_codec.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace {

// One butterfly stage across lanes (stride bit = lane bit M): the lane whose dim has the
// bit clear keeps own + partner, the other partner - own. Both are fma(s, own, partner) with
// s = +1 or -1: s * own is exact, so the fma rounds once, as the addition it stands for.
// The partner comes by DPP inside a row of 16 lanes, by ds_bpermute across rows.
// Keys: the stride bit is lane bit M (16 or 32), partner by ds_bpermute.
template <int M>
__device__ __forceinline__ float bfly_lane(float y, int lane) {
  return __builtin_fmaf((lane & M) ? -1.0f : 1.0f, y, __shfl_xor(y, M, 64));
}
// Values: lane 16j + i holds row 16j + tq_blk16(i), so the partner whose row differs in bit
// M (1, 2, 4, 8) is one DPP move away (bxor<M>); the stride bit is that bit of the row.
template <int M>
__device__ __forceinline__ float bfly_row(float y, int row16) {
  return __builtin_fmaf((row16 & M) ? -1.0f : 1.0f, y, bxor<M>(y));
}

// The dense outputs are written once and read back by another kernel, so stores are
// non-temporal (streamed past the caches).
template <typename TOut>
__device__ __forceinline__ void store8(TOut* p, const float* y) {
  if constexpr (sizeof(TOut) == 2) {
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; e++) h[e] = (f16)y[e];
    __builtin_nontemporal_store(h, reinterpret_cast<f16x8*>(p));
  } else {
    __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{y[4], y[5], y[6], y[7]}, reinterpret_cast<f32x4*>(p + 4));
  }
}

template <typename TOut>
__device__ __forceinline__ void store2(TOut* p, float a, float b) {
  if constexpr (sizeof(TOut) == 2) {
    __builtin_nontemporal_store(f16x2{(f16)a, (f16)b}, reinterpret_cast<f16x2*>(p));
  } else {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(f32x2{a, b}, reinterpret_cast<f32x2*>(p));
  }
}

template <int D, typename TOut, int KC, int VB>
__global__ __launch_bounds__(256) void dequant_page_kernel(LaunchDequant a) {
  constexpr int G = D / 32;
  __shared__ float lut[16];
  if (threadIdx.x < 16) {
    const uint16_t lb[16] = TQ_LUT16_BITS;
    uint16_t v = lb[0];
#pragma unroll
    for (int i = 1; i < 16; i++) v = threadIdx.x == i ? lb[i] : v;
    lut[threadIdx.x] = (float)__builtin_bit_cast(f16, v);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  // one-dimensional grid: workgroup = (sequence b, kv head h, 4 consecutive pages)
  const uint32_t p4 = (uint32_t)(((a.max_ctx + 15) / 16 + 3) / 4);
  const uint32_t unit = blockIdx.x / p4;
  const int h = (int)(unit % (uint32_t)a.Hkv), b = (int)(unit / (uint32_t)a.Hkv);
  const int p = (int)(blockIdx.x % p4) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = p * 16;
  if (t0 >= a.max_ctx) return;
  // the length and the page id are loaded together: every page of the output (p < max_ctx/16
  // rounded up <= max_pages) has a block-table entry, read whether or not it is used
  const int L = a.context_lens[b];
  int page_id = a.block_table[(int64_t)b * a.max_pages + p];
  uint32_t sgn[G];  // sign words of the rotation
#pragma unroll
  for (int g = 0; g < G; g++) sgn[g] = a.sign_bits[g];
  // keeps these loads above the branch: one wait for all of them
  asm volatile("" : "+s"(page_id));
#pragma unroll
  for (int g = 0; g < G; g++) asm volatile("" : "+s"(sgn[g]));
  const int64_t page = page_id;
  const int nt = min(16, a.max_ctx - t0);  // rows of this page inside the output
  TOut* kout = static_cast<TOut*>(a.k_out) + (((int64_t)b * a.Hkv + h) * a.max_ctx + t0) * D;
  TOut* vout = static_cast<TOut*>(a.v_out) + (((int64_t)b * a.Hkv + h) * a.max_ctx + t0) * D;
  if (t0 >= L) {  // the whole page lies past the context: zero rows
    const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = lane * 8; i < nt * D; i += 512) {
      store8(kout + i, z);
      store8(vout + i, z);
    }
    return;
  }
  constexpr bool kf16 = KC == TQ_CODEC_FP16;
  constexpr bool lutk = KC == TQ_CODEC_LLOYDMAX;
  const int BB = tq_block_bytes(D, KC, a.v_codec);
  const int vbase = kf16 ? 32 * D : 8 * D;
  const int ksb = 8 * D + 2 * VB * D;                    // K scales (4-bit keys)
  const int vsb = kf16 ? 32 * D + 2 * VB * D : ksb + D;  // V scales
  const uint8_t* blk = a.pool + (page * a.Hkv + h) * BB;
  const bool rot = a.original_basis != 0;
  const float rho = tq_rho(D);
  const int j = lane >> 4, t = lane & 15;
  const int m = tq_blk16(lane & 15), vrow = 16 * j + m;  // values: the row this lane holds

  // ---- every load of the page first (no store may come between them: the compiler cannot
  // move a load of the pool above a store to the outputs)
  // keys: lane l = 16j + t, token t, dims 32g + 8j + e
  u32x4 k16[G];  // fp16 keys: 8 dims per group
  uint32_t kw[G];
  f16 ks[G];
  if constexpr (kf16) {
#pragma unroll
    for (int g = 0; g < G; g++) k16[g] = *reinterpret_cast<const u32x4*>(blk + 1024 * g + 16 * lane);
  } else if constexpr (G == 2) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(blk + 8 * lane);
    kw[0] = x[0]; kw[1] = x[1];
    const f16x2 sv = *reinterpret_cast<const f16x2*>(blk + ksb + 4 * t);
    ks[0] = sv[0]; ks[1] = sv[1];
  } else {
#pragma unroll
    for (int c = 0; c < G / 4; c++) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(blk + 4 * G * lane + 16 * c);
      const f16x4 sv = *reinterpret_cast<const f16x4*>(blk + ksb + 2 * G * t + 8 * c);
#pragma unroll
      for (int k = 0; k < 4; k++) { kw[4 * c + k] = x[k]; ks[4 * c + k] = sv[k]; }
    }
  }
  // values: lane 16j + i holds row 16j + m, m = tq_blk16(i): tokens 4j + e, dims 32g + 2m + {0, 1}
  uint32_t nw[G];  // the lane's nibble dwords
  if constexpr (VB == 4) {
    if constexpr (G == 2) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(blk + vbase + 8 * vrow);
      nw[0] = x[0]; nw[1] = x[1];
    } else {
#pragma unroll
      for (int c = 0; c < G / 4; c++) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(blk + vbase + 4 * G * vrow + 16 * c);
#pragma unroll
        for (int k = 0; k < 4; k++) nw[4 * c + k] = x[k];
      }
    }
  } else {
    // X dword i of row l holds the low two bits of nibble dwords 2i (bits 0-1 of every
    // nibble) and 2i + 1 (bits 2-3); Z dword (l*G + g)/4 holds the third bit of nibble
    // dword g at bit (l*G + g) % 4 of every nibble
    constexpr int XD = G / 2;
    uint32_t xw[XD], zw[G];
#pragma unroll
    for (int i = 0; i < XD; i++) xw[i] = *reinterpret_cast<const uint32_t*>(blk + vbase + 4 * (vrow * XD + i));
    if constexpr (VB == 3) {
#pragma unroll
      for (int g = 0; g < G; g++) zw[g] = *reinterpret_cast<const uint32_t*>(blk + vbase + 128 * G + 4 * ((vrow * G + g) >> 2));
    }
#pragma unroll
    for (int g = 0; g < G; g++) {
      nw[g] = (xw[g >> 1] >> (2 * (g & 1))) & 0x33333333u;
      if constexpr (VB == 3) nw[g] |= ((zw[g] >> ((vrow * G + g) & 3)) & 0x11111111u) << 2;
    }
  }
  // scales of tokens 4j .. 4j + 3, every group: 4G contiguous fp16
  f16 vs[4][G];
#pragma unroll
  for (int c = 0; c < G; c++) {
    const f16x4 sv = *reinterpret_cast<const f16x4*>(blk + vsb + 2 * (4 * j * G) + 8 * c);
#pragma unroll
    for (int k = 0; k < 4; k++) vs[(4 * c + k) / G][(4 * c + k) % G] = sv[k];
  }

  // ---- keys
  {
    float y[G][8];
    if constexpr (kf16) {
#pragma unroll
      for (int g = 0; g < G; g++) {
        const f16x8 w = __builtin_bit_cast(f16x8, k16[g]);
#pragma unroll
        for (int e = 0; e < 8; e++) y[g][e] = (float)w[e];
      }
    } else {
      if constexpr (lutk) {
#pragma unroll
        for (int g = 0; g < G; g++)
#pragma unroll
          for (int e = 0; e < 8; e++) y[g][e] = lut[(kw[g] >> (4 * e)) & 15u] * (float)ks[g];
      } else {
        // (u - 8) * s = fma(u, s, -8s): u*s and 8s are exact and so is their difference
#pragma unroll
        for (int g = 0; g < G; g++) {
          const float sc = (float)ks[g], off = -8.0f * sc;
          const uint32_t lo = kw[g] & 0x0F0F0F0Fu, hi = (kw[g] >> 4) & 0x0F0F0F0Fu;  // nibbles 2b, 2b + 1
#pragma unroll
          for (int bb = 0; bb < 4; bb++) {
            y[g][2 * bb] = __builtin_fmaf((float)((lo >> (8 * bb)) & 0xFFu), sc, off);
            y[g][2 * bb + 1] = __builtin_fmaf((float)((hi >> (8 * bb)) & 0xFFu), sc, off);
          }
        }
      }
      if (rot) {
#pragma unroll
        for (int st = 1; st < 8; st <<= 1)
#pragma unroll
          for (int g = 0; g < G; g++)
#pragma unroll
            for (int e = 0; e < 8; e++)
              if (!(e & st)) {
                const float x0 = y[g][e], x1 = y[g][e + st];
                y[g][e] = x0 + x1;
                y[g][e + st] = x0 - x1;
              }
#pragma unroll
        for (int g = 0; g < G; g++)
#pragma unroll
          for (int e = 0; e < 8; e++) y[g][e] = bfly_lane<16>(y[g][e], lane);
#pragma unroll
        for (int g = 0; g < G; g++)
#pragma unroll
          for (int e = 0; e < 8; e++) y[g][e] = bfly_lane<32>(y[g][e], lane);
#pragma unroll
        for (int st = 1; st < G; st <<= 1)
#pragma unroll
          for (int g = 0; g < G; g++)
            if (!(g & st))
#pragma unroll
              for (int e = 0; e < 8; e++) {
                const float x0 = y[g][e], x1 = y[g + st][e];
                y[g][e] = x0 + x1;
                y[g + st][e] = x0 - x1;
              }
#pragma unroll
        for (int g = 0; g < G; g++) {
          const uint32_t sw = sgn[g] >> (8 * j);
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float x = y[g][e] * rho;
            y[g][e] = ((sw >> e) & 1u) ? -x : x;
          }
        }
      }
    }
    if (t < nt) {
      const bool live = t0 + t < L;
#pragma unroll
      for (int g = 0; g < G; g++) {
        if (!live)
#pragma unroll
          for (int e = 0; e < 8; e++) y[g][e] = 0.0f;
        store8(kout + t * D + 32 * g + 8 * j, y[g]);
      }
    }
  }

  // ---- values
  {
    constexpr int QM = VB == 4 ? 7 : (VB == 3 ? 3 : 1);  // largest abs-max level
    float y[4][G][2];
#pragma unroll
    for (int g = 0; g < G; g++) {
      const uint32_t lo = nw[g] & 0x0F0F0F0Fu, hi = (nw[g] >> 4) & 0x0F0F0F0Fu;  // byte e: token 4j + e
#pragma unroll
      for (int e = 0; e < 4; e++) {
        // (u - (QM + 1)) * s = fma(u, s, -(QM + 1)s), exact as for the keys
        const float sc = (float)vs[e][g], off = -(float)(QM + 1) * sc;
        y[e][g][0] = __builtin_fmaf((float)((lo >> (8 * e)) & 0xFFu), sc, off);
        y[e][g][1] = __builtin_fmaf((float)((hi >> (8 * e)) & 0xFFu), sc, off);
      }
    }
    if (rot) {
#pragma unroll
      for (int e = 0; e < 4; e++)
#pragma unroll
        for (int g = 0; g < G; g++) {
          const float x0 = y[e][g][0], x1 = y[e][g][1];
          y[e][g][0] = x0 + x1;
          y[e][g][1] = x0 - x1;
        }
      auto vstage = [&](auto mc) {
        constexpr int M = decltype(mc)::value;
#pragma unroll
        for (int e = 0; e < 4; e++)
#pragma unroll
          for (int g = 0; g < G; g++)
#pragma unroll
            for (int q = 0; q < 2; q++) y[e][g][q] = bfly_row<M>(y[e][g][q], m);
      };
      vstage(std::integral_constant<int, 1>{});
      vstage(std::integral_constant<int, 2>{});
      vstage(std::integral_constant<int, 4>{});
      vstage(std::integral_constant<int, 8>{});
#pragma unroll
      for (int st = 1; st < G; st <<= 1)
#pragma unroll
        for (int e = 0; e < 4; e++)
#pragma unroll
          for (int g = 0; g < G; g++)
            if (!(g & st))
#pragma unroll
              for (int q = 0; q < 2; q++) {
                const float x0 = y[e][g][q], x1 = y[e][g + st][q];
                y[e][g][q] = x0 + x1;
                y[e][g + st][q] = x0 - x1;
              }
#pragma unroll
      for (int g = 0; g < G; g++) {
        const uint32_t sw = sgn[g] >> (2 * m);
#pragma unroll
        for (int e = 0; e < 4; e++)
#pragma unroll
          for (int q = 0; q < 2; q++) {
            const float x = y[e][g][q] * rho;
            y[e][g][q] = ((sw >> q) & 1u) ? -x : x;
          }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int tv = 4 * j + e;
      if (tv < nt) {
        const bool live = t0 + tv < L;
#pragma unroll
        for (int g = 0; g < G; g++)
          store2(vout + tv * D + 32 * g + 2 * m, live ? y[e][g][0] : 0.0f, live ? y[e][g][1] : 0.0f);
      }
    }
  }
}

template <int D, typename TOut, int KC>
hipError_t launch_k(const LaunchDequant& a, dim3 grid, hipStream_t st) {
  switch (tq_value_bits(a.v_codec)) {
    case 4: hipLaunchKernelGGL((dequant_page_kernel<D, TOut, KC, 4>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((dequant_page_kernel<D, TOut, KC, 3>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((dequant_page_kernel<D, TOut, KC, 2>), grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

template <int D, typename TOut>
hipError_t launch_t(const LaunchDequant& a, dim3 grid, hipStream_t st) {
  switch (a.k_codec) {
    case TQ_CODEC_FP16: return launch_k<D, TOut, TQ_CODEC_FP16>(a, grid, st);
    case TQ_CODEC_LLOYDMAX: return launch_k<D, TOut, TQ_CODEC_LLOYDMAX>(a, grid, st);
    default: return launch_k<D, TOut, TQ_CODEC_ABSMAX>(a, grid, st);
  }
}

template <int D>
hipError_t launch_d(const LaunchDequant& a, hipStream_t st) {
  const int64_t pages = (a.max_ctx + 15) / 16;
  dim3 grid((unsigned)((int64_t)a.B * a.Hkv * ((pages + 3) / 4)));  // the caller keeps it < 2^31
  return a.out_dtype == TQ_F32 ? launch_t<D, float>(a, grid, st) : launch_t<D, f16>(a, grid, st);
}

}  // namespace

hipError_t tq_launch_dequant(const LaunchDequant& a, hipStream_t st) {
  if ((int64_t)a.B * a.Hkv * a.max_ctx == 0) return hipSuccess;
  switch (a.D) {
    case 64: return launch_d<64>(a, st);
    case 128: return launch_d<128>(a, st);
    default: return launch_d<256>(a, st);
  }
}
