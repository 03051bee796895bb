// Rotation and 4-bit codec of one K or V vector by 16 lanes, and its placement in a block.
// [Open-TQ-Metal, card abstract: one fused step does the sign-randomized rotation, the
//  per-group abs-max and the int4 nibble pack; "TurboQuant on AMD GPUs", section 2: keys
//  may use a LUT quantizer, values a uniform one; section 4: Walsh-Hadamard rotation.]
//
// Work split: 16 lanes per vector, each lane holding E = D/16 consecutive coordinates.
// The butterfly runs stride 1..E/2 inside a lane and stride E..D/2 across lanes (lane
// xor by DPP, so the 16 lanes must be one aligned row), in ascending order, so every fp32
// add/sub pairs the same operands as the plain definition. No multiply may fuse into an add here (contraction is switched off in these
// functions), so codes are bit-identical to a sequential implementation.
#pragma once
#include "tq_device.h"

template <int D>
struct CodecCfg {
  static constexpr int E = D / 16;    // coordinates per lane
  static constexpr int G = D / 32;    // groups per vector
  static constexpr int LPG = 32 / E;  // lanes per group
};

// Sign bits of the lane's E coordinates, bit e = sigma of coordinate lane16 * E + e.
template <int D>
__device__ __forceinline__ uint32_t lane_signs(const uint32_t* sign_bits, int lane16) {
  constexpr int E = CodecCfg<D>::E;
  return sign_bits[(lane16 * E) >> 5] >> ((lane16 * E) & 31);
}

// y: this lane's E coordinates of the vector (already widened to fp32), sw: lane_signs();
// lane16 = lane % 16 of the 16 lanes that hold the vector. Returns the lane's E indices and
// its group's scale (abs-max scale, or the group norm for the LUT codec).
template <int D, int CODEC>
__device__ __forceinline__ void codec_vector(float (&y)[D / 16], uint32_t sw, int lane16,
                                             uint32_t (&u)[D / 16], f16& scale) {
#pragma clang fp contract(off)
  constexpr int E = CodecCfg<D>::E, LPG = CodecCfg<D>::LPG;
  // y = sigma .* x
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
    const bool upper = (lane16 & m) != 0;
#pragma unroll
    for (int e = 0; e < E; e++) {
      float o = lane_xor16(y[e], m, lane16);
      y[e] = upper ? (o - y[e]) : (y[e] + o);
    }
  }
  const float rho = tq_rho(D);
#pragma unroll
  for (int e = 0; e < E; e++) y[e] = y[e] * rho;

  if constexpr (CODEC == TQ_CODEC_ABSMAX) {
    // s = fp16(absmax / 7); c = clamp(rint(y / s), -7, 7); u = c + 8
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < E; e++) a = fmaxf(a, fabsf(y[e]));
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) a = fmaxf(a, lane_xor16(a, m, lane16));
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
        for (int e = 0; e < E; e++) t[e] = t[e] + lane_xor16(t[e], off / E, lane16);
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
}

// Write one lane's indices and (from the group's first lane) the scale of token t into a
// block (pool memory, or a copy of the block in LDS; see the pool format in tq.h). KF16:
// the fp16-key block, whose value regions start at 32D (indices) and 40D (scales).
template <int D, bool KF16 = false>
__device__ __forceinline__ void place_vector(uint8_t* blk, int t, int lane16, bool is_v,
                                             const uint32_t (&u)[D / 16], f16 scale) {
  constexpr int E = CodecCfg<D>::E, G = CodecCfg<D>::G, LPG = CodecCfg<D>::LPG;
  constexpr int VBASE = KF16 ? 32 * D : 8 * D;
  if (!is_v) {
    // K: dims 8q..8q+7 (q = chunk index, g = q/4, j = q%4) -> one dword at (16j+t)*4G + 4g
    if constexpr (E >= 8) {
#pragma unroll
      for (int c = 0; c < E / 8; c++) {
        const int q = lane16 * (E / 8) + c;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) w |= u[c * 8 + e] << (4 * e);
        *reinterpret_cast<uint32_t*>(blk + (16 * (q & 3) + t) * 4 * G + 4 * (q >> 2)) = w;
      }
    } else {  // E == 4: half a chunk -> 2 bytes
      const int q = lane16 >> 1;
      uint16_t w = (uint16_t)(u[0] | (u[1] << 4) | (u[2] << 8) | (u[3] << 12));
      *reinterpret_cast<uint16_t*>(blk + (16 * (q & 3) + t) * 4 * G + 4 * (q >> 2) + 2 * (lane16 & 1)) = w;
    }
  } else {
    // V: byte column c = d/2 = 16g + m of token t = 4j + e -> byte 8D + (16j + m)*4G + 4g + e
#pragma unroll
    for (int k = 0; k < E / 2; k++) {
      const int c = lane16 * (E / 2) + k;
      blk[VBASE + (16 * (t >> 2) + (c & 15)) * 4 * G + 4 * (c >> 4) + (t & 3)] =
          (uint8_t)(u[2 * k] | (u[2 * k + 1] << 4));
    }
  }
  if ((lane16 % LPG) == 0) {
    const int g = (lane16 * E) / 32;
    const int sbase = KF16 ? 40 * D : 16 * D + (is_v ? 32 * G : 0);
    *reinterpret_cast<f16*>(blk + sbase + 2 * (t * G + g)) = scale;
  }
}

// fp16 keys: this lane's E coordinates of the (unrotated) key of token t, rounded to fp16
// (nearest even, overflow saturated), into an fp16-key block: dims 32g + 8j + 0..7 of
// token t are the 16 bytes at 1024g + 16(16j + t).
template <int D>
__device__ __forceinline__ void place_key_f16(uint8_t* blk, int t, int lane16, const float (&y)[D / 16]) {
  constexpr int E = CodecCfg<D>::E;
#pragma unroll
  for (int c = 0; c < (E >= 8 ? E / 8 : 1); c++) {
    const int d0 = lane16 * E + 8 * c;
    uint8_t* dst = blk + 1024 * (d0 >> 5) + 16 * (16 * ((d0 >> 3) & 3) + t) + 2 * (d0 & 7);
    if constexpr (E >= 8) {
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; e++) h[e] = f16_sat(y[8 * c + e]);
      *reinterpret_cast<f16x8*>(dst) = h;
    } else {  // E == 4: half of an 8-dim run
      f16x4 h;
#pragma unroll
      for (int e = 0; e < 4; e++) h[e] = f16_sat(y[e]);
      *reinterpret_cast<f16x4*>(dst) = h;
    }
  }
}
