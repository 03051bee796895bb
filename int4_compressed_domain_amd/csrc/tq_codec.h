// Rotation and codec of one K or V vector by 16 lanes, and its placement in a block.
// [Open-TQ-Metal, card abstract: one fused step does the sign-randomized rotation, the
//  per-group abs-max and the int4 nibble pack; "TurboQuant on AMD GPUs", section 2: keys
//  may use a LUT quantizer, values a uniform one, 2 bits are possible; section 4:
//  Walsh-Hadamard rotation; mlxcel "TurboQuant KV cache" manual, cache-mode table: 3-bit
//  values (fp16+turbo3).]
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
// its group's scale (abs-max scale, or the group norm for the LUT codec). The abs-max
// codecs differ in their largest level QM: 7 (4 bits), 3 (3 bits), 1 (2 bits).
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

  if constexpr (CODEC != TQ_CODEC_LLOYDMAX) {
    // s = fp16(absmax / QM); c = clamp(rint(y / s), -QM, QM); u = c + QM + 1
    constexpr int QM = CODEC == TQ_CODEC_ABSMAX3 ? 3 : (CODEC == TQ_CODEC_ABSMAX2 ? 1 : 7);
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < E; e++) a = fmaxf(a, fabsf(y[e]));
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) a = fmaxf(a, lane_xor16(a, m, lane16));
    scale = f16_sat(a / (float)QM);
    const float sf = (float)scale;
#pragma unroll
    for (int e = 0; e < E; e++) {
      float c = 0.0f;
      if (sf != 0.0f) c = fminf(fmaxf(rintf(y[e] / sf), -(float)QM), (float)QM);
      u[e] = (uint32_t)((int)c + QM + 1);
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

// lane16 ^ m of a 32-bit word (m = 1, 2, 4, 8), by the same DPP moves
__device__ __forceinline__ uint32_t lane_xor16_u(uint32_t x, int m, int lane16) {
  return __builtin_bit_cast(uint32_t, lane_xor16(__builtin_bit_cast(float, x), m, lane16));
}

// Token t's b-bit value indices (b = VB = 3 or 2) into the packed value region vreg (see
// the pool format in tq.h). In the 4-bit layout the indices of dim pair m of group g of
// token t = 4j + e sit in byte e of dword g of row l = 16j + m. Packed: their two low bits
// go to byte e of X dword l*G/2 + g/2 (shifted by 2*(g%2) in each nibble), for b = 3 their
// third bits to byte e of Z dword (l*G + g)/4 (shifted by (l*G + g)%4), Z after the 32*G X
// dwords. This lane holds dim pairs m0 .. m0 + E/2 - 1 of group g; the other groups of a
// byte are in lanes lane16 ^ LG (and ^ 2*LG), LG = 32/E lanes per group, so each byte is
// ORed together by DPP and written once. All 16 lanes of the vector must take part.
template <int D, int VB>
__device__ __forceinline__ void place_v_packed(uint8_t* vreg, int t, int lane16, const uint32_t (&u)[D / 16]) {
  constexpr int E = CodecCfg<D>::E, G = CodecCfg<D>::G, LG = 32 / E;
  constexpr int XD = G >= 2 ? G / 2 : 1;  // X dwords per row
  const int g = lane16 / LG, j = t >> 2, e = t & 3;
  const int m0 = (lane16 % LG) * (E / 2);
  uint32_t zacc = 0;
#pragma unroll
  for (int k = 0; k < E / 2; k++) {
    const uint32_t ue = u[2 * k], uo = u[2 * k + 1];
    const int l = 16 * j + m0 + k;
    uint32_t xb = ((ue & 3u) | ((uo & 3u) << 4)) << (2 * (g & 1));
    xb |= lane_xor16_u(xb, LG, lane16);
    if (!(g & 1)) vreg[4 * (l * XD + (g >> 1)) + e] = (uint8_t)xb;
    if constexpr (VB == 3) {
      const int z = l * G + g;
      const uint32_t zb = (((ue >> 2) & 1u) | (((uo >> 2) & 1u) << 4)) << (z & 3);
      if constexpr (G >= 4) {
        uint32_t zc = zb | lane_xor16_u(zb, LG, lane16);
        zc |= lane_xor16_u(zc, 2 * LG, lane16);
        if ((g & 3) == 0) vreg[128 * G + 4 * (z >> 2) + e] = (uint8_t)zc;
      } else {  // G == 2: this lane's two pairs are rows l, l + 1 of one Z dword
        zacc |= zb;
        if (k == E / 2 - 1) {
          zacc |= lane_xor16_u(zacc, LG, lane16);
          if (g == 0) vreg[128 * G + 4 * (z >> 2) + e] = (uint8_t)zacc;
        }
      }
    }
  }
}

// Write one lane's indices and (from the group's first lane) the scale of token t into a
// block (pool memory, or a copy of the block in LDS; see the pool format in tq.h). KF16:
// the fp16-key block, whose value indices start at 32D. VB: bits per value index (4, 3, 2);
// the value region takes 2*VB*D bytes and the scales follow it.
template <int D, bool KF16 = false, int VB = 4>
__device__ __forceinline__ void place_vector(uint8_t* blk, int t, int lane16, bool is_v,
                                             const uint32_t (&u)[D / 16], f16 scale) {
  constexpr int E = CodecCfg<D>::E, G = CodecCfg<D>::G, LPG = CodecCfg<D>::LPG;
  constexpr int VBASE = KF16 ? 32 * D : 8 * D;
  constexpr int SBASE = VBASE + 2 * VB * D;  // K scales (4-bit keys), then V scales
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
  } else if constexpr (VB == 4) {
    // V: byte column c = d/2 = 16g + m of token t = 4j + e -> byte 8D + (16j + m)*4G + 4g + e
#pragma unroll
    for (int k = 0; k < E / 2; k++) {
      const int c = lane16 * (E / 2) + k;
      blk[VBASE + (16 * (t >> 2) + (c & 15)) * 4 * G + 4 * (c >> 4) + (t & 3)] =
          (uint8_t)(u[2 * k] | (u[2 * k + 1] << 4));
    }
  } else {
    place_v_packed<D, VB>(blk + VBASE, t, lane16, u);
  }
  if ((lane16 % LPG) == 0) {
    const int g = (lane16 * E) / 32;
    const int sbase = SBASE + ((is_v && !KF16) ? D : 0);
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
