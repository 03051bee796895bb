// Dequantize reference: dense K and V from the packed pool, the first half of the
// dequantize-then-attend baseline [Open-TQ-Metal, arXiv abstract].
// 16 lanes per (sequence, kv head, token) vector, E = D/16 coordinates per lane; values
// (u - 8)*s (4-bit), (u - 4)*s or (u - 2)*s (3- and 2-bit values) or LUT_u*n are exact in
// fp32. The original-basis variant applies the fp32
// inverse rotation diag(sigma)*rho*H with the forward rotation's stage order.
// fp16 keys are copied as stored (they have no rotated form). Compiled with
// -ffp-contract=off.
#include "tq_device.h"
#include "tq_internal.h"

namespace {

template <int D, typename TOut>
__global__ __launch_bounds__(256) void dequant_kernel(LaunchDequant a) {
  constexpr int E = D / 16, G = D / 32;
  const bool kf16 = a.k_codec == TQ_CODEC_FP16;
  const int BB = tq_block_bytes(D, a.k_codec, a.v_codec);
  const int VB = tq_value_bits(a.v_codec);
  const int QM = VB == 4 ? 7 : (VB == 3 ? 3 : 1);  // largest abs-max level of the values
  const int vbase = kf16 ? 32 * D : 8 * D;
  const int lane = threadIdx.x & 15;
  const int64_t vec = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int64_t per_b = (int64_t)a.Hkv * a.max_ctx;
  if (vec >= (int64_t)a.B * per_b * 2) return;
  const int is_v = (int)(vec & 1);
  const int64_t row = vec >> 1;  // (b * Hkv + h) * max_ctx + t
  const int b = (int)(row / per_b);
  const int h = (int)((row / a.max_ctx) % a.Hkv);
  const int t = (int)(row % a.max_ctx);
  float y[E];
  if (t >= a.context_lens[b]) {
#pragma unroll
    for (int e = 0; e < E; e++) y[e] = 0.0f;
  } else {
    const int64_t page = a.block_table[(int64_t)b * a.max_pages + (t >> 4)];
    const uint8_t* blk = a.pool + (page * a.Hkv + h) * BB;
    const int tt = t & 15;
    uint32_t u[E];
    if (!is_v && kf16) {  // fp16 key, dims lane*E + e: byte 1024g + 16(16j + t) + 2(d % 8)
#pragma unroll
      for (int e = 0; e < E; e++) {
        const int d = lane * E + e;
        y[e] = (float)*reinterpret_cast<const f16*>(blk + 1024 * (d >> 5) + 16 * (16 * ((d >> 3) & 3) + tt) + 2 * (d & 7));
      }
    } else if (!is_v) {
      if constexpr (E >= 8) {
#pragma unroll
        for (int c = 0; c < E / 8; c++) {
          const int q = lane * (E / 8) + c;
          const uint32_t w = *reinterpret_cast<const uint32_t*>(blk + (16 * (q & 3) + tt) * 4 * G + 4 * (q >> 2));
#pragma unroll
          for (int e = 0; e < 8; e++) u[8 * c + e] = (w >> (4 * e)) & 15u;
        }
      } else {
        const int q = lane >> 1;
        const uint32_t w = *reinterpret_cast<const uint16_t*>(blk + (16 * (q & 3) + tt) * 4 * G + 4 * (q >> 2) + 2 * (lane & 1));
#pragma unroll
        for (int e = 0; e < 4; e++) u[e] = (w >> (4 * e)) & 15u;
      }
    } else if (VB == 4) {
#pragma unroll
      for (int k = 0; k < E / 2; k++) {
        const int c = lane * (E / 2) + k;
        const uint32_t byte = blk[vbase + (16 * (tt >> 2) + (c & 15)) * 4 * G + 4 * (c >> 4) + (tt & 3)];
        u[2 * k] = byte & 15u;
        u[2 * k + 1] = byte >> 4;
      }
    } else {
      // packed b-bit values: dim pair c = 16g + m of token tt = 4j + e is row l = 16j + m,
      // dword g of the 4-bit layout; its low bits are in byte e of X dword l*G/2 + g/2
      // (nibble bits 2*(g%2)), its third bits (b = 3) in byte e of Z dword (l*G + g)/4
      // (nibble bit (l*G + g)%4)
      constexpr int XD = G >= 2 ? G / 2 : 1;
#pragma unroll
      for (int k = 0; k < E / 2; k++) {
        const int c = lane * (E / 2) + k, gg = c >> 4;
        const int l = 16 * (tt >> 2) + (c & 15), e = tt & 3;
        const uint32_t xb = blk[vbase + 4 * (l * XD + (gg >> 1)) + e] >> (2 * (gg & 1));
        uint32_t lo = xb & 3u, hi = (xb >> 4) & 3u;
        if (VB == 3) {
          const int z = l * G + gg;
          const uint32_t zb = blk[vbase + 128 * G + 4 * (z >> 2) + e] >> (z & 3);
          lo |= (zb & 1u) << 2;
          hi |= ((zb >> 4) & 1u) << 2;
        }
        u[2 * k] = lo;
        u[2 * k + 1] = hi;
      }
    }
    const int g = (lane * E) / 32;
    const int sbase = (kf16 ? 32 * D : 8 * D) + 2 * VB * D + ((is_v && !kf16) ? D : 0);
    const float sc = (float)*reinterpret_cast<const f16*>(blk + sbase + 2 * (tt * G + g));
    if (!is_v && kf16) {
      // y holds the key already
    } else if (!is_v && a.k_codec == TQ_CODEC_LLOYDMAX) {
      const uint16_t lb[16] = TQ_LUT16_BITS;
#pragma unroll
      for (int e = 0; e < E; e++) y[e] = (float)__builtin_bit_cast(f16, lb[u[e]]) * sc;
    } else {
      const int off = is_v ? QM + 1 : 8;
#pragma unroll
      for (int e = 0; e < E; e++) y[e] = (float)((int)u[e] - off) * sc;
    }
    if (a.original_basis && (is_v || !kf16)) {
#pragma unroll
      for (int s = 1; s < E; s <<= 1)
#pragma unroll
        for (int e = 0; e < E; e++)
          if (!(e & s)) {
            const float x0 = y[e], x1 = y[e + s];
            y[e] = x0 + x1;
            y[e + s] = x0 - x1;
          }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < E; e++) {
          const float o = __shfl_xor(y[e], m, 16);
          y[e] = upper ? (o - y[e]) : (y[e] + o);
        }
      }
      const float rho = tq_rho(D);
      const uint32_t sw = a.sign_bits[(lane * E) >> 5] >> ((lane * E) & 31);
#pragma unroll
      for (int e = 0; e < E; e++) {
        const float x = y[e] * rho;
        y[e] = ((sw >> e) & 1u) ? -x : x;
      }
    }
  }
  TOut* out = static_cast<TOut*>(is_v ? a.v_out : a.k_out) + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; e++) out[e] = (TOut)y[e];
}

template <int D>
hipError_t launch_d(const LaunchDequant& a, hipStream_t st) {
  const int64_t nvec = (int64_t)a.B * a.Hkv * a.max_ctx * 2;
  dim3 grid((unsigned)((nvec + 15) / 16));
  if (a.out_dtype == TQ_F32)
    hipLaunchKernelGGL((dequant_kernel<D, float>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dequant_kernel<D, f16>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
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
