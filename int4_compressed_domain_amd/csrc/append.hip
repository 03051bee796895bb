// Append kernel: rotate, quantize and pack new K/V vectors into the paged pool.
// [Open-TQ-Metal, card abstract: one fused kernel does the sign-randomized rotation, the
//  per-group abs-max and the int4 nibble pack; "TurboQuant on AMD GPUs", section 2: keys
//  may use a LUT quantizer, values a uniform one; section 4: Walsh-Hadamard rotation.]
//
// Work split: 16 lanes per vector, each lane holding E = D/16 consecutive coordinates.
// The butterfly runs stride 1..E/2 inside a lane and stride E..D/2 across lanes (lane
// xor), in ascending order, so every fp32 add/sub pairs the same operands as the plain
// definition; codes are therefore bit-identical to a sequential implementation.
// Compiled with -ffp-contract=off: no multiply may fuse into an add here.
#include "tq_device.h"
#include "tq_internal.h"

namespace {

template <int D, typename TIn, int KCODEC>
__global__ __launch_bounds__(256) void append_kernel(uint8_t* __restrict__ pool,
                                                     const TIn* __restrict__ kin,
                                                     const TIn* __restrict__ vin,
                                                     const int64_t* __restrict__ slots,
                                                     const uint32_t* __restrict__ sign_bits,
                                                     int n_tokens, int Hkv) {
  constexpr int E = D / 16;   // coordinates per lane
  constexpr int G = D / 32;   // groups per vector
  constexpr int LPG = 32 / E; // lanes per group
  constexpr int BB = TQ_BLOCK_BYTES(D);
  const int lane = threadIdx.x & 15;
  const int64_t vec = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (vec >= (int64_t)n_tokens * Hkv * 2) return;  // whole 16-lane groups exit together
  const int is_v = (int)(vec & 1);
  const int64_t th = vec >> 1;  // token * Hkv + head
  const int64_t tok = th / Hkv;
  const int h = (int)(th % Hkv);
  const int64_t slot = slots[tok];
  if (slot < 0) return;

  float y[E];
  load_widen<TIn, E>((is_v ? vin : kin) + th * D + lane * E, y);

  // y = sigma .* x
  const uint32_t sw = sign_bits[(lane * E) >> 5] >> ((lane * E) & 31);
#pragma unroll
  for (int e = 0; e < E; e++)
    if ((sw >> e) & 1u) y[e] = -y[e];
  // butterfly, stride 1 .. E/2 inside the lane
#pragma unroll
  for (int s = 1; s < E; s <<= 1)
#pragma unroll
    for (int e = 0; e < E; e++)
      if (!(e & s)) {
        float a = y[e], b = y[e + s];
        y[e] = a + b;
        y[e + s] = a - b;
      }
  // stride E .. D/2 across lanes: the lower index gets a + b, the upper a - b
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < E; e++) {
      float o = __shfl_xor(y[e], m, 16);
      y[e] = upper ? (o - y[e]) : (y[e] + o);
    }
  }
  const float rho = tq_rho(D);
#pragma unroll
  for (int e = 0; e < E; e++) y[e] = y[e] * rho;

  uint32_t u[E];
  f16 scale;
  if (is_v || KCODEC == TQ_CODEC_ABSMAX) {
    // s = fp16(absmax / 7); c = clamp(rint(y / s), -7, 7); u = c + 8
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < E; e++) a = fmaxf(a, fabsf(y[e]));
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 16));
    scale = f16_sat(a / 7.0f);
    const float sf = (float)scale;
#pragma unroll
    for (int e = 0; e < E; e++) {
      float c = 0.0f;
      if (sf != 0.0f) c = fminf(fmaxf(rintf(y[e] / sf), -7.0f), 7.0f);
      u[e] = (uint32_t)((int)c + 8);
    }
  } else {
    // group L2 norm with the tree t_i += t_{i+off}, off = 16, 8, 4, 2, 1
    float t[E];
#pragma unroll
    for (int e = 0; e < E; e++) t[e] = y[e] * y[e];
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
      if (off >= E) {
#pragma unroll
        for (int e = 0; e < E; e++) t[e] = t[e] + __shfl_xor(t[e], off / E, 16);
      } else {
#pragma unroll
        for (int e = 0; e < E; e++)
          if (e < off) t[e] = t[e] + t[e + off];
      }
    }
    scale = f16_sat(sqrtf(t[0]));
    const float nf = (float)scale;
    const uint16_t lut_bits[16] = TQ_LUT16_BITS;
    float thr[16];
#pragma unroll
    for (int j = 1; j < 16; j++)
      thr[j] = ((float)__builtin_bit_cast(f16, lut_bits[j - 1]) +
                (float)__builtin_bit_cast(f16, lut_bits[j])) * 0.5f;
#pragma unroll
    for (int e = 0; e < E; e++) {
      uint32_t c = 8;
      if (nf != 0.0f) {
        const float v = y[e] / nf;
        c = 0;
#pragma unroll
        for (int j = 1; j < 16; j++) c += (v >= thr[j]) ? 1u : 0u;
      }
      u[e] = c;
    }
  }

  uint8_t* blk = pool + ((slot >> 4) * (int64_t)Hkv + h) * BB;
  const int t = (int)(slot & 15);
  if (!is_v) {
    // K: dims 8q..8q+7 (q = chunk index, g = q/4, j = q%4) -> one dword at (16j+t)*4G + 4g
    if constexpr (E >= 8) {
#pragma unroll
      for (int c = 0; c < E / 8; c++) {
        const int q = lane * (E / 8) + c;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) w |= u[c * 8 + e] << (4 * e);
        *reinterpret_cast<uint32_t*>(blk + (16 * (q & 3) + t) * 4 * G + 4 * (q >> 2)) = w;
      }
    } else {  // E == 4: half a chunk -> 2 bytes
      const int q = lane >> 1;
      uint16_t w = (uint16_t)(u[0] | (u[1] << 4) | (u[2] << 8) | (u[3] << 12));
      *reinterpret_cast<uint16_t*>(blk + (16 * (q & 3) + t) * 4 * G + 4 * (q >> 2) + 2 * (lane & 1)) = w;
    }
  } else {
    // V: byte column c = d/2 = 16g + m of token t = 4j + e -> byte 8D + (16j + m)*4G + 4g + e
#pragma unroll
    for (int k = 0; k < E / 2; k++) {
      const int c = lane * (E / 2) + k;
      blk[8 * D + (16 * (t >> 2) + (c & 15)) * 4 * G + 4 * (c >> 4) + (t & 3)] =
          (uint8_t)(u[2 * k] | (u[2 * k + 1] << 4));
    }
  }
  if ((lane % LPG) == 0) {
    const int g = (lane * E) / 32;
    *reinterpret_cast<f16*>(blk + 16 * D + (is_v ? 32 * G : 0) + 2 * (t * G + g)) = scale;
  }
}

template <int D, typename T>
hipError_t launch_d(const LaunchAppend& a, hipStream_t st) {
  const int64_t nvec = (int64_t)a.n_tokens * a.Hkv * 2;
  dim3 grid((unsigned)((nvec + 15) / 16));
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  if (a.k_codec == TQ_CODEC_LLOYDMAX)
    hipLaunchKernelGGL((append_kernel<D, T, TQ_CODEC_LLOYDMAX>), grid, dim3(256), 0, st, a.pool, k, v,
                       a.slots, a.sign_bits, a.n_tokens, a.Hkv);
  else
    hipLaunchKernelGGL((append_kernel<D, T, TQ_CODEC_ABSMAX>), grid, dim3(256), 0, st, a.pool, k, v,
                       a.slots, a.sign_bits, a.n_tokens, a.Hkv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_t(const LaunchAppend& a, hipStream_t st) {
  switch (a.dtype) {
    case TQ_F32: return launch_d<D, float>(a, st);
    case TQ_BF16: return launch_d<D, uint16_t>(a, st);
    default: return launch_d<D, f16>(a, st);
  }
}

}  // namespace

hipError_t tq_launch_append(const LaunchAppend& a, hipStream_t st) {
  if (a.n_tokens == 0) return hipSuccess;
  switch (a.D) {
    case 64: return launch_t<64>(a, st);
    case 128: return launch_t<128>(a, st);
    default: return launch_t<256>(a, st);
  }
}
