// Rotation and codec of one K or V vector by 16 lanes, and its placement in a block.
// [Open-TQ-Metal, card abstract: one fused step does the sign-randomized rotation, the
//  per-group abs-max and the int4 nibble pack; "TurboQuant on AMD GPUs", section 2: keys
//  may use a LUT quantizer, values a uniform one, 2 bits are possible; section 4:
//  Walsh-Hadamard rotation; mlxcel "TurboQuant KV cache" manual, cache-mode table: 3-bit
//  values (fp16+turbo3).]
//
// Work split: 16 lanes per vector, each holding E = D/16 consecutive coordinates: lane
// lane16 holds coordinate block blk = tq_blk16(lane16), coordinates blk*E .. blk*E + E - 1.
// The butterfly runs stride 1..E/2 inside a lane, then stride E..D/2 across lanes, in
// ascending order, so every fp32 add/sub pairs the same operands as the plain definition.
// The map lane -> block is chosen so that the partner block (blk ^ m, m = 1, 2, 4, 8) is
// one DPP move away inside a row of 16: xor 1 and xor 2 of the lane are quad permutes,
// xor 7 a half-row mirror (flipping only bit 2 of the block), xor 8 a row rotation by 8.
// No multiply may fuse into an add here (contraction is switched off in these functions,
// and the rotation's only fused operations are fma with a +-1 factor, which round once
// like the add they stand for; the quantizer's fast estimate is used only where a margin
// proves it decides as the exact quotient does), so codes are bit-identical to a
// sequential implementation.
#pragma once
#include "tq_device.h"

template <int D>
struct CodecCfg {
  static constexpr int E = D / 16;    // coordinates per lane
  static constexpr int G = D / 32;    // groups per vector
  static constexpr int LPG = 32 / E;  // lanes per group
};

// Coordinate block of lane lane16 (an involution of 0..15 keeping bits 2 and 3).
__host__ __device__ __forceinline__ int tq_blk16(int lane16) {
  return lane16 ^ (((lane16 >> 2) & 1) * 3);
}

// Value held by the lane whose block is blk ^ M (M = 1, 2, 4, 8), by one DPP move.
template <int M>
__device__ __forceinline__ float bxor(float x) {
  const int v = __float_as_int(x);
  constexpr int CTRL = M == 1 ? 0xB1 : (M == 2 ? 0x4E : (M == 4 ? 0x141 : 0x128));
  return __int_as_float(__builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float bxor_m(float x, int m) {
  switch (m) {
    case 1: return bxor<1>(x);
    case 2: return bxor<2>(x);
    case 4: return bxor<4>(x);
    default: return bxor<8>(x);
  }
}
__device__ __forceinline__ uint32_t bxor_u(uint32_t x, int m) {
  return __builtin_bit_cast(uint32_t, bxor_m(__builtin_bit_cast(float, x), m));
}

// One cross-lane butterfly stage over the lane's E values: y[e] += s * (y[e] of the lane
// whose block is blk ^ M), each one v_fmac_f32 reading the partner through DPP. The block
// starts with the wait states a DPP read needs after a VALU write (of a VGPR, or of EXEC),
// whatever the compiler placed before it; inside, each instruction reads a register the
// previous ones did not write.
#define TQ_DPP_CTRL_1 "quad_perm:[1,0,3,2]"
#define TQ_DPP_CTRL_2 "quad_perm:[2,3,0,1]"
#define TQ_DPP_CTRL_4 "row_half_mirror"
#define TQ_DPP_CTRL_8 "row_ror:8"
#define TQ_FMAC_DPP(i, c) "v_fmac_f32_dpp %" #i ", %" #i ", %[s] " c " row_mask:0xf bank_mask:0xf\n\t"
#define TQ_FMAC_DPP4(c) TQ_FMAC_DPP(0, c) TQ_FMAC_DPP(1, c) TQ_FMAC_DPP(2, c) TQ_FMAC_DPP(3, c)
#define TQ_FMAC_DPP8(c) TQ_FMAC_DPP4(c) TQ_FMAC_DPP(4, c) TQ_FMAC_DPP(5, c) TQ_FMAC_DPP(6, c) TQ_FMAC_DPP(7, c)
#define TQ_FMAC_DPP16(c)                                                                        \
  TQ_FMAC_DPP8(c) TQ_FMAC_DPP(8, c) TQ_FMAC_DPP(9, c) TQ_FMAC_DPP(10, c) TQ_FMAC_DPP(11, c)     \
  TQ_FMAC_DPP(12, c) TQ_FMAC_DPP(13, c) TQ_FMAC_DPP(14, c) TQ_FMAC_DPP(15, c)

template <int M, int E>
__device__ __forceinline__ void bfly_stage(float (&y)[E], float s) {
  constexpr int X = M == 1 ? 1 : (M == 2 ? 2 : (M == 4 ? 4 : 8));
  static_assert(X == M && (E == 4 || E == 8 || E == 16), "stage 1, 2, 4 or 8 over 4, 8 or 16 values");
#define TQ_STAGE(c)                                                                                  \
  if constexpr (E == 4)                                                                             \
    asm volatile("s_nop 4\n\t" TQ_FMAC_DPP4(c) : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])     \
                 : [s] "v"(s));                                                                      \
  else if constexpr (E == 8)                                                                        \
    asm volatile("s_nop 4\n\t" TQ_FMAC_DPP8(c)                                                      \
                 : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]),         \
                   "+v"(y[6]), "+v"(y[7])                                                           \
                 : [s] "v"(s));                                                                      \
  else                                                                                              \
    asm volatile("s_nop 4\n\t" TQ_FMAC_DPP16(c)                                                     \
                 : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]),         \
                   "+v"(y[6]), "+v"(y[7]), "+v"(y[8]), "+v"(y[9]), "+v"(y[10]), "+v"(y[11]),       \
                   "+v"(y[12]), "+v"(y[13]), "+v"(y[14]), "+v"(y[15])                               \
                 : [s] "v"(s));
  if constexpr (M == 1) { TQ_STAGE(TQ_DPP_CTRL_1) }
  else if constexpr (M == 2) { TQ_STAGE(TQ_DPP_CTRL_2) }
  else if constexpr (M == 4) { TQ_STAGE(TQ_DPP_CTRL_4) }
  else { TQ_STAGE(TQ_DPP_CTRL_8) }
#undef TQ_STAGE
}

// Sign bits of block blk's E coordinates, bit e = sigma of coordinate blk * E + e.
template <int D>
__device__ __forceinline__ uint32_t lane_signs(const uint32_t* sign_bits, int blk) {
  constexpr int E = CodecCfg<D>::E;
  return sign_bits[(blk * E) >> 5] >> ((blk * E) & 31);
}

// y = sigma .* x for the lane's E coordinates (sw: lane_signs()).
template <int D>
__device__ __forceinline__ void apply_signs(float (&y)[D / 16], uint32_t sw) {
#pragma unroll
  for (int e = 0; e < D / 16; e++)
    if ((sw >> e) & 1u) y[e] = -y[e];
}

// The codebook is symmetric (level 15 - i = -level i), so the 15 decision thresholds are
// 0 and +-t_k, k = 1..7, t_k the midpoint of positive levels k - 1 and k.
constexpr bool tq_lut_symmetric() {
  constexpr uint16_t b[16] = TQ_LUT16_BITS;
  for (int i = 0; i < 8; i++)
    if (b[15 - i] != (uint16_t)(b[i] ^ 0x8000u)) return false;
  return true;
}
static_assert(tq_lut_symmetric(), "the key codebook must be symmetric");

// Key codebook thresholds as buckets of width 1/32 over |v| (v = y / n): bucket b covers
// [b/32, (b+1)/32), b = 0..32 (|v| <= 1 + 2^-10 where the table is used, so below 33/32).
// Each holds at most one of the positive thresholds t_1..t_7, none within 2^-12 of its
// edges, so for |v| in bucket b, #{k : t_k <= |v|} = lo[b] + (|v| >= th[b]) (th = +inf
// where the bucket holds none), also for an estimate of |v| that lands in a neighbouring
// bucket. Entry b is {lo[b] + 1, th[b]}.
namespace tq_lutb {
constexpr float f16_value(uint16_t h) {  // exact value of fp16 bits (no inf/NaN here)
  const int e = (h >> 10) & 31, m = h & 1023;
  float v = e ? (float)(1024 + m) : (float)m;
  for (int i = 0; i < 24; i++) v = v * 0.5f;  // v * 2^-24
  for (int i = 0; i < (e ? e - 1 : 0); i++) v = v * 2.0f;
  return (h & 0x8000) ? -v : v;
}
constexpr float tk(int k) {  // k = 1..7: midpoint of positive levels k - 1 and k
  constexpr uint16_t b[16] = TQ_LUT16_BITS;
  return (f16_value(b[7 + k]) + f16_value(b[8 + k])) * 0.5f;
}
constexpr int NB = 33;
struct Table {
  uint32_t lo1[NB];  // lo[b] + 1
  float th[NB];
};
constexpr Table make_table() {
  Table t{};
  for (int bk = 0; bk < NB; bk++) {
    int n = 0;
    float h = __builtin_huge_valf();
    for (int k = 1; k < 8; k++) {
      n += tk(k) < bk / 32.0f ? 1 : 0;
      if (tk(k) >= bk / 32.0f && tk(k) < (bk + 1) / 32.0f) h = tk(k);
    }
    t.lo1[bk] = (uint32_t)n + 1u;
    t.th[bk] = h;
  }
  return t;
}
constexpr bool valid() {
  for (int k = 1; k < 8; k++) {
    if (!(tk(k) > 0.0f) || (k > 1 && !(tk(k) > tk(k - 1)))) return false;  // increasing
    for (int bk = 0; bk <= NB; bk++) {             // away from every edge
      const float d = tk(k) - bk / 32.0f;
      if ((d < 0 ? -d : d) < 0x1p-12f) return false;
    }
  }
  for (int bk = 0; bk < NB; bk++) {  // at most one per bucket
    int c = 0;
    for (int k = 1; k < 8; k++) c += (tk(k) >= bk / 32.0f && tk(k) < (bk + 1) / 32.0f) ? 1 : 0;
    if (c > 1) return false;
  }
  return true;
}
static_assert(valid(), "the key codebook thresholds do not fit the 1/32 buckets");
}  // namespace tq_lutb

// Entry i of the bucket table ({lo + 1, bits of th}; zeros for i >= NB), for the caller to
// write into LDS (NB entries) and synchronize before codec_vector reads it.
__device__ __forceinline__ u32x2 tq_lut_table_entry(int i) {
  constexpr tq_lutb::Table T = tq_lutb::make_table();
  u32x2 w = {0u, 0u};
  if (i < tq_lutb::NB) {
    w[0] = T.lo1[i];
    w[1] = __float_as_uint(T.th[i]);
  }
  return w;
}

// y: this lane's E coordinates of the vector, widened to fp32 and already multiplied by
// sigma; blk = tq_blk16(lane16) of the 16 lanes that hold the vector. Returns the lane's
// E indices and its group's scale (abs-max scale, or the group norm for the LUT codec). The
// abs-max codecs differ in their largest level QM: 7 (4 bits), 3 (3 bits), 1 (2 bits).
// lut_tbl: the LUT codec's bucket table in LDS (tq_lut_table_entry), or null for the
// division-per-coordinate path alone.
template <int D, int CODEC>
__device__ __forceinline__ void codec_vector(float (&y)[D / 16], int blk, uint32_t (&u)[D / 16],
                                             f16& scale, const u32x2* lut_tbl = nullptr) {
#pragma clang fp contract(off)
  constexpr int E = CodecCfg<D>::E, LPG = CodecCfg<D>::LPG;
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
  // stride E .. D/2 across lanes: the lower block gets a + b, the upper a - b. The lane
  // keeps its value times sg, the product of the signs s_m (+1 lower, -1 upper) of the
  // stages done; partners share sg, and sg * s_m * (result) = held + s_m * held_partner
  // is one fma with an exact product, rounded once like the add itself.
  bfly_stage<1>(y, (blk & 1) ? -1.0f : 1.0f);
  bfly_stage<2>(y, (blk & 2) ? -1.0f : 1.0f);
  bfly_stage<4>(y, (blk & 4) ? -1.0f : 1.0f);
  bfly_stage<8>(y, (blk & 8) ? -1.0f : 1.0f);
  // y = held * sg * rho, one rounding as y * rho
  const float rho = (__builtin_popcount(blk & 15) & 1) ? -tq_rho(D) : tq_rho(D);
#pragma unroll
  for (int e = 0; e < E; e++) y[e] = y[e] * rho;

  if constexpr (CODEC != TQ_CODEC_LLOYDMAX) {
    // s = fp16(absmax / QM); c = clamp(rint(y / s), -QM, QM); u = c + QM + 1
    constexpr int QM = CODEC == TQ_CODEC_ABSMAX3 ? 3 : (CODEC == TQ_CODEC_ABSMAX2 ? 1 : 7);
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < E; e++) a = fmaxf(a, fabsf(y[e]));
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) a = fmaxf(a, bxor_m(a, m));
    scale = f16_sat(a / (float)QM);
    const float sf = (float)scale;
    // Fast path: t = y * (1/s) + QM + 1 with the hardware reciprocal (1 ulp). For a normal,
    // unsaturated s, |y / s| <= QM (1 + 2^-11), so no clamp is needed, and t lies within
    // 2^-19 of the exact y / s + QM + 1: when t is further than 2^-16 from a half-integer,
    // rint(t) is the index the rounded quotient gives. s = 0 (an all-zero group) gives
    // t = QM + 1 exactly. Anything else (a subnormal or saturated scale, a value near a
    // decision boundary, a non-finite input) takes the exact path below.
    const float r = sf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sf);
    float dmax = 0.0f;  // largest |t - rint(t)|
#pragma unroll
    for (int e = 0; e < E; e++) {
      const float t = __builtin_fmaf(y[e], r, (float)(QM + 1));
      const float c = rintf(t);
      dmax = fmaxf(dmax, fabsf(t - c));
      u[e] = (uint32_t)c;
    }
    // (fmaxf drops NaNs; a NaN input makes every rotated coordinate NaN, y[0] included)
    const bool fast = (sf == 0.0f || (sf >= 0x1p-14f && sf < 65504.0f)) &&
                      dmax <= 0.5f - 0x1p-16f && y[0] == y[0];
    if (!fast) {
#pragma unroll
      for (int e = 0; e < E; e++) {
        float c = 0.0f;
        if (sf != 0.0f) c = fminf(fmaxf(rintf(y[e] / sf), -(float)QM), (float)QM);
        u[e] = (uint32_t)((int)c + QM + 1);
      }
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
        for (int e = 0; e < E; e++) t[e] = t[e] + bxor_m(t[e], off / E);
      } else {
#pragma unroll
        for (int e = 0; e < E; e++)
          if (e < off) t[e] = t[e] + t[e + off];
      }
    }
    scale = f16_sat(sqrtf(t[0]));
    const float nf = (float)scale;
    // u = #{j in 1..15 : v >= thr_j}, v = y / n, thr_j the midpoint of levels j - 1 and j.
    // With the symmetric codebook: v >= 0 (also -0) passes thr_1..thr_8 = 0, so
    // u = 8 + #{k : v >= t_k}; v < 0 passes thr_{8-k} = -t_k iff |v| <= t_k, so
    // u = 7 - #{k : |v| > t_k}, and |v| > t_k iff the next float below |v| is >= t_k.
    bool fast = false;
    if (lut_tbl != nullptr) {
      // Fast path: v ~ y * (1/n) (hardware reciprocal: within 2^-20 of y / n for |v| <= 1.01),
      // its bucket, one compare with the bucket's threshold; valid when n is a normal,
      // unsaturated fp16 (then every |v| <= 1 + 2^-10, all finite, and the bucket index at
      // most 32) or 0 (all coordinates 0: v = +0, index 8), and no estimate lies within
      // 2^-16 of the threshold it was compared with. (Outside those cases 1/n is replaced by
      // 0, so every table read stays at entry 0, and the result is discarded.) For v < 0 the count of thresholds below |v| is the same as of those
      // strictly below once ties are excluded, so u = 8 + n (v >= 0) or 7 - n (v < 0),
      // computed as (n xor s) + 8 with s = 0 or -1 the sign of v.
      const bool nrange = nf >= 0x1p-14f && nf < 65504.0f;
      const float rn = nrange ? __builtin_amdgcn_rcpf(nf) : 0.0f;  // (0: every index read is 0)
      float dmin = 1.0f;  // smallest |estimate - compared threshold|
#pragma unroll
      for (int e = 0; e < E; e++) {
        const float v = __builtin_fmaf(y[e], rn, 0.0f);  // (+0 for a zero product)
        const float av = fabsf(v);
        const u32x2 w = lut_tbl[(uint32_t)(av * 32.0f)];
        const float d = av - __uint_as_float(w[1]);  // < 0 iff |v| < th (th = +inf: -inf)
        const uint32_t n = w[0] + (uint32_t)((int)__float_as_uint(d) >> 31);
        dmin = fminf(dmin, fabsf(d));
        u[e] = (n ^ (uint32_t)((int)__float_as_uint(v) >> 31)) + 8u;
      }
      fast = (nf == 0.0f || nrange) && dmin > 0x1p-16f;
    }
    if (!fast) {
    const uint16_t lut_bits[16] = TQ_LUT16_BITS;
    float tk[8];
#pragma unroll
    for (int k = 1; k < 8; k++)
      tk[k] = ((float)__builtin_bit_cast(f16, lut_bits[7 + k]) +
               (float)__builtin_bit_cast(f16, lut_bits[8 + k])) * 0.5f;
#pragma unroll
    for (int e = 0; e < E; e++) {
      uint32_t c = 8;
      if (nf != 0.0f) {
        const float v = y[e] / nf;
        const bool nonneg = v >= 0.0f;
        const float av = fabsf(v);
        const float a2 = nonneg ? av : __uint_as_float(__float_as_uint(av) - 1u);
        uint32_t n = 0;
#pragma unroll
        for (int k = 1; k < 8; k++) n += (a2 >= tk[k]) ? 1u : 0u;
        c = nonneg ? 8u + n : (v < 0.0f ? 7u - n : 0u);  // (NaN: below no threshold)
      }
      u[e] = c;
    }
    }
  }
}

// Token t's b-bit value indices (b = VB = 3 or 2) into the packed value region vreg (see
// the pool format in tq.h). In the 4-bit layout the indices of dim pair m of group g of
// token t = 4j + e sit in byte e of dword g of row l = 16j + m. Packed: their two low bits
// go to byte e of X dword l*G/2 + g/2 (shifted by 2*(g%2) in each nibble), for b = 3 their
// third bits to byte e of Z dword (l*G + g)/4 (shifted by (l*G + g)%4), Z after the 32*G X
// dwords. This lane holds dim pairs m0 .. m0 + E/2 - 1 of group g; the other groups of a
// byte are in blocks blk ^ LG (and ^ 2*LG), LG = 32/E lanes per group, so each byte is
// ORed together by DPP and written once. All 16 lanes of the vector must take part.
// blk = tq_blk16(lane16) (the lanes are named by their blocks here).
template <int D, int VB>
__device__ __forceinline__ void place_v_packed(uint8_t* vreg, int t, int blk, const uint32_t (&u)[D / 16]) {
  constexpr int E = CodecCfg<D>::E, G = CodecCfg<D>::G, LG = 32 / E;
  constexpr int XD = G >= 2 ? G / 2 : 1;  // X dwords per row
  const int g = blk / LG, j = t >> 2, e = t & 3;
  const int m0 = (blk % LG) * (E / 2);
  uint32_t zacc = 0;
#pragma unroll
  for (int k = 0; k < E / 2; k++) {
    const uint32_t ue = u[2 * k], uo = u[2 * k + 1];
    const int l = 16 * j + m0 + k;
    uint32_t xb = ((ue & 3u) | ((uo & 3u) << 4)) << (2 * (g & 1));
    xb |= bxor_u(xb, LG);
    if (!(g & 1)) vreg[4 * (l * XD + (g >> 1)) + e] = (uint8_t)xb;
    if constexpr (VB == 3) {
      const int z = l * G + g;
      const uint32_t zb = (((ue >> 2) & 1u) | (((uo >> 2) & 1u) << 4)) << (z & 3);
      if constexpr (G >= 4) {
        uint32_t zc = zb | bxor_u(zb, LG);
        zc |= bxor_u(zc, 2 * LG);
        if ((g & 3) == 0) vreg[128 * G + 4 * (z >> 2) + e] = (uint8_t)zc;
      } else {  // G == 2: this lane's two pairs are rows l, l + 1 of one Z dword
        zacc |= zb;
        if (k == E / 2 - 1) {
          zacc |= bxor_u(zacc, LG);
          if (g == 0) vreg[128 * G + 4 * (z >> 2) + e] = (uint8_t)zacc;
        }
      }
    }
  }
}

// Write one lane's indices and (from the group's first lane) the scale of token t into a
// block (pool memory, or a copy of the block in LDS; see the pool format in tq.h); cb is
// the lane's coordinate block (tq_blk16). KF16: the fp16-key block, whose value indices
// start at 32D. VB: bits per value index (4, 3, 2); the value region takes 2*VB*D bytes
// and the scales follow it.
template <int D, bool KF16 = false, int VB = 4>
__device__ __forceinline__ void place_vector(uint8_t* blk, int t, int cb, bool is_v,
                                             const uint32_t (&u)[D / 16], f16 scale) {
  constexpr int E = CodecCfg<D>::E, G = CodecCfg<D>::G, LPG = CodecCfg<D>::LPG;
  constexpr int VBASE = KF16 ? 32 * D : 8 * D;
  constexpr int SBASE = VBASE + 2 * VB * D;  // K scales (4-bit keys), then V scales
  if (!is_v) {
    // K: dims 8q..8q+7 (q = chunk index, g = q/4, j = q%4) -> one dword at (16j+t)*4G + 4g
    if constexpr (E >= 8) {
#pragma unroll
      for (int c = 0; c < E / 8; c++) {
        const int q = cb * (E / 8) + c;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) w |= u[c * 8 + e] << (4 * e);
        *reinterpret_cast<uint32_t*>(blk + (16 * (q & 3) + t) * 4 * G + 4 * (q >> 2)) = w;
      }
    } else {  // E == 4: half a chunk -> 2 bytes
      const int q = cb >> 1;
      uint16_t w = (uint16_t)(u[0] | (u[1] << 4) | (u[2] << 8) | (u[3] << 12));
      *reinterpret_cast<uint16_t*>(blk + (16 * (q & 3) + t) * 4 * G + 4 * (q >> 2) + 2 * (cb & 1)) = w;
    }
  } else if constexpr (VB == 4) {
    // V: byte column c = d/2 = 16g + m of token t = 4j + e -> byte 8D + (16j + m)*4G + 4g + e
#pragma unroll
    for (int k = 0; k < E / 2; k++) {
      const int c = cb * (E / 2) + k;
      blk[VBASE + (16 * (t >> 2) + (c & 15)) * 4 * G + 4 * (c >> 4) + (t & 3)] =
          (uint8_t)(u[2 * k] | (u[2 * k + 1] << 4));
    }
  } else {
    place_v_packed<D, VB>(blk + VBASE, t, cb, u);
  }
  if ((cb % LPG) == 0) {
    const int g = (cb * E) / 32;
    const int sbase = SBASE + ((is_v && !KF16) ? D : 0);
    *reinterpret_cast<f16*>(blk + sbase + 2 * (t * G + g)) = scale;
  }
}

// fp16 keys: this lane's E coordinates (block cb) of the (unrotated) key of token t, rounded
// to fp16 (nearest even, overflow saturated), into an fp16-key block: dims 32g + 8j + 0..7
// of token t are the 16 bytes at 1024g + 16(16j + t).
template <int D>
__device__ __forceinline__ void place_key_f16(uint8_t* blk, int t, int cb, const float (&y)[D / 16]) {
  constexpr int E = CodecCfg<D>::E;
#pragma unroll
  for (int c = 0; c < (E >= 8 ? E / 8 : 1); c++) {
    const int d0 = cb * E + 8 * c;
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
