/*
 * tq_oracle.c -- plain, slow CPU reference for int4 compressed-domain decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU-baseline
 * leg are the only callers. The GPU library never links, loads or calls this file, and
 * this file shares no code, header, table or constant generator with it.
 *
 * Sources (web pages; cited by title and section):
 *  - Open-TQ-Metal (card abstract): one fused quantize step = sign-randomized rotation,
 *    per-group abs-max, int4 nibble pack; SRFT and SRHT give the same quality.
 *  - Open-TQ-Metal (arXiv abstract): int4 on the fly, attention computed directly on the
 *    compressed representation, no dequantized K/V matrix; attn_scale 1.0 vs 1/sqrt(d).
 *  - "TurboQuant on AMD GPUs" (oracore.dev), section 2 (TQ4/4): keys by rotation + LUT
 *    quantization, values by uniform quantization; section 4: Walsh-Hadamard rotation.
 *  - mlxcel "TurboQuant KV cache" manual, head-dim limitation: power-of-two head dims only.
 *
 * Readings taken where the pages are silent (each is also listed in the design notes):
 *  - R = rho * H * diag(sigma), H the natural-order Sylvester Hadamard matrix, sigma from
 *    sign bits (bit set => -1), fp32 butterfly with stride ascending 1,2,..,D/2, then
 *    multiply by rho = fp32(1/sqrt(D)). No fused multiply-add anywhere.
 *  - abs-max: s = fp16_rne(absmax/7) (saturating at 65504), c = clamp(rint(y/s), -7, 7),
 *    c = 0 when s == 0; the stored 4-bit index is u = c + 8 (offset binary).
 *  - LUT (keys): LUT_j = fp16_rne(m_j/sqrt(32)) with m_j the 16-level Lloyd-Max
 *    centroids of N(0,1); n = fp16_rne(sqrtf(sum of squares, xor-tree 16,8,4,2,1));
 *    u = #{j in 1..15 : y/n >= (LUT_{j-1}+LUT_j)/2}, u = 8 when n == 0 (value 0 is
 *    not a level; index 8 is the smallest positive level, as any index would be).
 *  - Attention in fp64: scores alpha*q'.k^, softmax, weighted sum of v^ in the rotated
 *    basis, then the fp64 inverse rotation rho*sigma.*(H o').
 *  - Pool placement: see the header comment of each placement function below.
 *  - fp16 keys (mlxcel "TurboQuant KV cache" manual, cache-mode table and recommended
 *    mode: keys stay fp16, only values take the 4-bit rotated form): k_codec 2 stores
 *    fp16_rne(k) of the original key, saturating at 65504, with no rotation; scores are
 *    alpha * q.k in the original basis (the query is not rotated for them); values,
 *    the weighted sum and the inverse rotation are as in the 4-bit mode.
 *  - 3-bit and 2-bit values (mlxcel manual, cache-mode table: fp16+turbo3 keeps keys in
 *    fp16 and stores values with 3 bits; TurboQuant on AMD GPUs section 2: 2 bits are
 *    possible): v_codec 3 and 4 are the abs-max codec with the largest level qmax = 3
 *    and 1 instead of 7: s = fp16_rne(absmax/qmax), c = clamp(rint(y/s), -qmax, qmax),
 *    stored index u = c + qmax + 1 (3 and 2 bits). Their packing: see the placement
 *    functions below.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -fno-fast-math -fopenmp (no -march).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_PAGE 16
#define OR_GROUP 32

/* ------------------------------------------------------------------------------------- */
/* fp16 conversion, written from the IEEE 754 binary16 definition (round to nearest even,
 * subnormals kept). A double holds every fp32 value and every fp32 * 2^k exactly, so the
 * rint() below rounds the exact value once. Overflow returns +-inf. */
uint16_t or_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7e00;
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -14)) {                 /* subnormal range: units of 2^-24 */
    double q = rint(ldexp(a, 24));           /* q in [0, 1024]; 1024 is the min normal */
    return sign | (uint16_t)q;
  }
  int e;
  frexp(a, &e);                              /* a = f * 2^e, f in [0.5, 1) */
  e -= 1;                                    /* a = 1.xxx * 2^e */
  double m = rint(ldexp(a, 10 - e));         /* in [1024, 2048] */
  if (m == 2048.0) { m = 1024.0; e += 1; }
  if (e > 15) return sign | 0x7c00;
  return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

double or_f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

static uint16_t f16_saturate(uint16_t h) {   /* +-inf -> +-65504 */
  if ((h & 0x7fff) == 0x7c00) return (h & 0x8000) | 0x7bff;
  return h;
}

/* ------------------------------------------------------------------------------------- */
/* Rotation [Open-TQ-Metal card abstract: "sign-randomized" transform; TurboQuant on AMD
 * GPUs section 4: Walsh-Hadamard]. fp32(1/sqrt(D)) for D = 2^k, correctly rounded. */
static int ilog2i(int D) { int k = 0; while ((1 << k) < D) k++; return k; }

float or_rho_f32(int D) {
  int k = ilog2i(D);
  if ((k & 1) == 0) return ldexpf(1.0f, -k / 2);
  return ldexpf(sqrtf(2.0f), -(k + 1) / 2);      /* sqrtf is correctly rounded (IEEE) */
}

static int sign_of(const uint32_t* sb, int i) { return (sb[i >> 5] >> (i & 31)) & 1u; }

void or_rotate(const float* x, float* y, int D, const uint32_t* sign_bits) {
  for (int i = 0; i < D; i++) y[i] = sign_of(sign_bits, i) ? -x[i] : x[i];
  for (int h = 1; h < D; h <<= 1)
    for (int i = 0; i < D; i++)
      if (!(i & h)) {
        float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
  float rho = or_rho_f32(D);
  for (int i = 0; i < D; i++) y[i] = y[i] * rho;
}

/* fp32 inverse rotation R^-1 = diag(sigma) * H * rho, same stage order. Used for the
 * dense original-basis output of the dequantize reference. */
void or_unrotate_f32(const float* y, float* x, int D, const uint32_t* sign_bits) {
  for (int i = 0; i < D; i++) x[i] = y[i];
  for (int h = 1; h < D; h <<= 1)
    for (int i = 0; i < D; i++)
      if (!(i & h)) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  float rho = or_rho_f32(D);
  for (int i = 0; i < D; i++) {
    float t = x[i] * rho;
    x[i] = sign_of(sign_bits, i) ? -t : t;
  }
}

/* fp64 inverse rotation, for the attention output. */
static void unrotate_f64(const double* y, double* x, int D, const uint32_t* sign_bits) {
  for (int i = 0; i < D; i++) x[i] = y[i];
  for (int h = 1; h < D; h <<= 1)
    for (int i = 0; i < D; i++)
      if (!(i & h)) {
        double a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  double rho = 1.0 / sqrt((double)D);
  for (int i = 0; i < D; i++) x[i] = (sign_of(sign_bits, i) ? -x[i] : x[i]) * rho;
}

/* ------------------------------------------------------------------------------------- */
/* Uniform abs-max int4 for one group of g rotated values [Open-TQ-Metal card abstract:
 * per-group abs-max + int4; TurboQuant on AMD GPUs section 2: uniform V]. */
void or_quant_absmax_q(const float* y, int g, int qmax, uint8_t* u, uint16_t* scale) {
  float a = 0.0f;
  for (int i = 0; i < g; i++) { float t = fabsf(y[i]); if (t > a) a = t; }
  float s32 = a / (float)qmax;
  uint16_t s16 = f16_saturate(or_f64_to_f16((double)s32));
  float sf = (float)or_f16_to_f64(s16);
  float lim = (float)qmax;
  for (int i = 0; i < g; i++) {
    int c = 0;
    if (sf != 0.0f) {
      float r = rintf(y[i] / sf);
      c = r > lim ? qmax : (r < -lim ? -qmax : (int)r);
    }
    u[i] = (uint8_t)(c + qmax + 1);
  }
  *scale = s16;
}

void or_quant_absmax(const float* y, int g, uint8_t* u, uint16_t* scale) {
  or_quant_absmax_q(y, g, 7, u, scale);
}

/* Largest level of the abs-max codecs: v_codec 0 (4 bits), 3 (3 bits), 4 (2 bits). */
#define OR_ABSMAX3 3
#define OR_ABSMAX2 4
static int qmax_of(int codec) { return codec == OR_ABSMAX3 ? 3 : (codec == OR_ABSMAX2 ? 1 : 7); }
static int vbits_of(int codec) { return codec == OR_ABSMAX3 ? 3 : (codec == OR_ABSMAX2 ? 2 : 4); }

/* Lloyd-Max quantizer with 16 levels for N(0,1), by Lloyd's iteration in fp64
 * [TurboQuant on AMD GPUs section 2: keys use a LUT quantizer after the rotation]. */
static double phi(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
static double Phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

void or_lloydmax16(double* m, double* mse_out) {
  double c[16], t[17];
  for (int j = 0; j < 16; j++) c[j] = -3.0 + 6.0 * (j + 0.5) / 16.0;
  for (int it = 0; it < 200000; it++) {
    t[0] = -INFINITY; t[16] = INFINITY;
    for (int j = 1; j < 16; j++) t[j] = 0.5 * (c[j - 1] + c[j]);
    double delta = 0.0;
    for (int j = 0; j < 16; j++) {
      double mass = Phi(t[j + 1]) - Phi(t[j]);
      double nc = (phi(t[j]) - phi(t[j + 1])) / mass;
      delta = fmax(delta, fabs(nc - c[j]));
      c[j] = nc;
    }
    if (delta < 1e-15) break;
  }
  for (int j = 0; j < 8; j++) {               /* the density is even: average the pair */
    double s = 0.5 * (c[15 - j] - c[j]);
    c[j] = -s; c[15 - j] = s;
  }
  if (mse_out) {
    t[0] = -INFINITY; t[16] = INFINITY;
    for (int j = 1; j < 16; j++) t[j] = 0.5 * (c[j - 1] + c[j]);
    double mse = 0.0;
    for (int j = 0; j < 16; j++) {
      double a = t[j], b = t[j + 1];
      double mass = Phi(b) - Phi(a);
      double ap = isinf(a) ? 0.0 : a * phi(a), bp = isinf(b) ? 0.0 : b * phi(b);
      double x2 = mass - (bp - ap);            /* integral of x^2 phi over [a,b] */
      double x1 = phi(a) - phi(b);             /* integral of x phi over [a,b] */
      mse += x2 - 2.0 * c[j] * x1 + c[j] * c[j] * mass;
    }
    *mse_out = mse;
  }
  memcpy(m, c, sizeof c);
}

/* LUT_j = fp16_rne(m_j / sqrt(32)): the coordinates of a unit-norm group of 32 have
 * variance 1/32, so the N(0,1) centroids are scaled by 1/sqrt(32). */
void or_lut16(uint16_t* lut) {
  double m[16];
  or_lloydmax16(m, NULL);
  for (int j = 0; j < 16; j++) lut[j] = or_f64_to_f16(m[j] / sqrt(32.0));
}

void or_quant_lut(const float* y, int g, const uint16_t* lut, uint8_t* u, uint16_t* norm) {
  float t[256];
  for (int i = 0; i < g; i++) t[i] = y[i] * y[i];
  for (int off = g / 2; off >= 1; off >>= 1)
    for (int i = 0; i < off; i++) t[i] = t[i] + t[i + off];
  uint16_t n16 = f16_saturate(or_f64_to_f16((double)sqrtf(t[0])));
  float nf = (float)or_f16_to_f64(n16);
  float thr[16];
  for (int j = 1; j < 16; j++)
    thr[j] = ((float)or_f16_to_f64(lut[j - 1]) + (float)or_f16_to_f64(lut[j])) * 0.5f;
  for (int i = 0; i < g; i++) {
    if (nf == 0.0f) { u[i] = 8; continue; }
    float v = y[i] / nf;
    int c = 0;
    for (int j = 1; j < 16; j++) if (v >= thr[j]) c++;
    u[i] = (uint8_t)c;
  }
  *norm = n16;
}

/* Value of one stored index under each codec. */
static double dequant1(int codec, uint8_t u, uint16_t s16, const uint16_t* lut) {
  double s = or_f16_to_f64(s16);
  if (codec == 1) return or_f16_to_f64(lut[u]) * s;
  return (double)((int)u - qmax_of(codec) - 1) * s;
}

/* Encode n vectors of length D (fp32 input) with group size g: rotate, then quantize each
 * group. Outputs natural-order indices u[n][D] and scales[n][D/g]. codec 0 = abs-max,
 * 1 = LUT, 3 = 3-bit abs-max, 4 = 2-bit abs-max. */
void or_encode(const float* x, int64_t n, int D, int g, const uint32_t* sign_bits, int codec,
               uint8_t* u, uint16_t* scales) {
  uint16_t lut[16];
  if (codec == 1) or_lut16(lut);
#pragma omp parallel for schedule(static)
  for (int64_t v = 0; v < n; v++) {
    float y[512];
    or_rotate(x + v * D, y, D, sign_bits);
    for (int k = 0; k < D / g; k++) {
      if (codec == 1) or_quant_lut(y + k * g, g, lut, u + v * D + k * g, scales + v * (D / g) + k);
      else or_quant_absmax_q(y + k * g, g, qmax_of(codec), u + v * D + k * g, scales + v * (D / g) + k);
    }
  }
}

/* ------------------------------------------------------------------------------------- */
/* Pool placement. A pool is [num_pages][Hkv][block]; a block holds 16 tokens of one KV
 * head: [K indices 8D bytes][V indices 8D bytes][K scales 16*G fp16][V scales 16*G fp16]
 * with G = D/32. Two 4-bit indices share a byte, the first one in the low nibble.
 *  - K byte of (token t, dim d), d = 32g + 8j + e: (16j + t)*4G + 4g + e/2, nibble e%2.
 *  - V byte of (token t, dim d), c = d/2 = 16g + m, t = 4j + e: (16j + m)*4G + 4g + e,
 *    nibble d%2.
 *  - scale of (token t, group g): [t][g] in its scale array. */
int64_t or_block_bytes(int D) { return 16 * D + 64 * (D / 32); }

static int64_t k_byte(int t, int d, int D) {
  int G = D / 32, g = d / 32, j = (d % 32) / 8, e = d % 8;
  return (int64_t)(16 * j + t) * 4 * G + 4 * g + e / 2;
}
static int64_t v_byte(int t, int d, int D) {
  int G = D / 32, c = d / 2, g = c / 16, m = c % 16, j = t / 4, e = t % 4;
  return 8 * (int64_t)D + (int64_t)(16 * j + m) * 4 * G + 4 * g + e;
}
static int64_t ks_off(int t, int k, int D) { return 16 * (int64_t)D + 2 * (t * (D / 32) + k); }
static int64_t vs_off(int t, int k, int D) { return 16 * (int64_t)D + 32 * (D / 32) + 2 * (t * (D / 32) + k); }

static void put_nibble(uint8_t* p, int hi, uint8_t u) {
  *p = hi ? (uint8_t)((*p & 0x0f) | (u << 4)) : (uint8_t)((*p & 0xf0) | (u & 0x0f));
}
static uint8_t get_nibble(const uint8_t* p, int hi) { return hi ? (*p >> 4) : (*p & 0x0f); }

static void put16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }
static uint16_t get16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Store already-encoded natural-order indices/scales of n tokens x Hkv heads into the
 * pool at the given slots (slot = page*16 + offset; negative slots are skipped). */
void or_place(uint8_t* pool, int D, int Hkv, int64_t n, const int64_t* slots,
              const uint8_t* ku, const uint16_t* ks, const uint8_t* vu, const uint16_t* vs) {
  int G = D / 32;
  int64_t bb = or_block_bytes(D);
  for (int64_t i = 0; i < n; i++) {
    if (slots[i] < 0) continue;
    int64_t page = slots[i] / OR_PAGE;
    int t = (int)(slots[i] % OR_PAGE);
    for (int h = 0; h < Hkv; h++) {
      uint8_t* blk = pool + (page * Hkv + h) * bb;
      const uint8_t* kx = ku + (i * Hkv + h) * D;
      const uint8_t* vx = vu + (i * Hkv + h) * D;
      for (int d = 0; d < D; d++) {
        put_nibble(blk + k_byte(t, d, D), (d % 8) & 1, kx[d]);
        put_nibble(blk + v_byte(t, d, D), d & 1, vx[d]);
      }
      for (int k = 0; k < G; k++) {
        put16(blk + ks_off(t, k, D), ks[(i * Hkv + h) * G + k]);
        put16(blk + vs_off(t, k, D), vs[(i * Hkv + h) * G + k]);
      }
    }
  }
}

/* fp16-key blocks (k_codec 2): [K fp16 32D bytes][V indices 8D bytes][V scales 16*G fp16].
 *  - K value of (token t, dim d), d = 32g + 8j + e: byte 1024g + 16(16j + t) + 2e
 *    (for each group, the 16 tokens x 32 dims as four 8-dim chunks per token);
 *  - V byte and V scale as in the 4-bit block, shifted to start at 32D and 40D. */
#define OR_KF16 2

int64_t or_block_bytes_kc(int D, int k_codec) {
  return k_codec == OR_KF16 ? 41 * (int64_t)D : or_block_bytes(D);
}
static int64_t kf16_off(int t, int d) {
  int g = d / 32, j = (d % 32) / 8, e = d % 8;
  return 1024 * (int64_t)g + 16 * (int64_t)(16 * j + t) + 2 * e;
}
static int64_t kf16_v_byte(int t, int d, int D) { return v_byte(t, d, D) + 24 * (int64_t)D; }
static int64_t kf16_vs_off(int t, int k, int D) { return 40 * (int64_t)D + 2 * (t * (D / 32) + k); }

/* Keys to fp16 bits: round to nearest even (or_f64_to_f16), overflow saturated. */
void or_keys_f16(const float* k, int64_t n, uint16_t* kh) {
  for (int64_t i = 0; i < n; i++) kh[i] = f16_saturate(or_f64_to_f16((double)k[i]));
}

/* Store n tokens x Hkv heads into an fp16-key pool: kh [n][Hkv][D] fp16 bits, V indices
 * and scales as for or_place. Negative slots are skipped. */
void or_place_kf16(uint8_t* pool, int D, int Hkv, int64_t n, const int64_t* slots,
                   const uint16_t* kh, const uint8_t* vu, const uint16_t* vs) {
  int G = D / 32;
  int64_t bb = or_block_bytes_kc(D, OR_KF16);
  for (int64_t i = 0; i < n; i++) {
    if (slots[i] < 0) continue;
    int64_t page = slots[i] / OR_PAGE;
    int t = (int)(slots[i] % OR_PAGE);
    for (int h = 0; h < Hkv; h++) {
      uint8_t* blk = pool + (page * Hkv + h) * bb;
      const uint16_t* kx = kh + (i * Hkv + h) * D;
      const uint8_t* vx = vu + (i * Hkv + h) * D;
      for (int d = 0; d < D; d++) {
        put16(blk + kf16_off(t, d), kx[d]);
        put_nibble(blk + kf16_v_byte(t, d, D), d & 1, vx[d]);
      }
      for (int k = 0; k < G; k++) put16(blk + kf16_vs_off(t, k, D), vs[(i * Hkv + h) * G + k]);
    }
  }
}

/* Read back one token of an fp16-key pool: K fp16 bits, V indices and scales. */
void or_fetch_kf16(const uint8_t* pool, int D, int Hkv, int64_t page, int t, int h,
                   uint16_t* kh, uint8_t* vu, uint16_t* vs) {
  int G = D / 32;
  const uint8_t* blk = pool + (page * Hkv + h) * or_block_bytes_kc(D, OR_KF16);
  for (int d = 0; d < D; d++) {
    kh[d] = get16(blk + kf16_off(t, d));
    vu[d] = get_nibble(blk + kf16_v_byte(t, d, D), d & 1);
  }
  for (int k = 0; k < G; k++) vs[k] = get16(blk + kf16_vs_off(t, k, D));
}

/* Blocks in general, by key codec and value codec:
 *   4-bit keys: [K indices 8D][V indices][K scales 16*G fp16][V scales 16*G fp16]
 *   fp16 keys:  [K fp16 32D][V indices][V scales 16*G fp16]
 * with 2*b*D bytes of V indices for b-bit values (b = 4, 3, 2). K bytes as above.
 * b = 4: the V byte of (t, d) as in the 4-bit block. b = 3 or 2: the 4-bit position of
 * (t, d) -- row l = 16j + m, dword g of the row, nibble n = 2e + d%2, where t = 4j + e
 * and d/2 = 16g + m -- decides where the bits of its index go: bits 0-1 to X dword
 * l*G/2 + g/2 at bit 4n + 2*(g%2); for b = 3 bit 2 to Z dword (l*G + g)/4 at bit
 * 4n + (l*G + g)%4, the 16*G Z dwords following the 32*G X dwords. Dwords are
 * little-endian. Every byte of the V region then holds bits of one token only. */
int64_t or_block_bytes_kv(int D, int k_codec, int v_codec) {
  int64_t kpart = k_codec == OR_KF16 ? 32 * (int64_t)D : 8 * (int64_t)D;
  int64_t scales = k_codec == OR_KF16 ? (int64_t)D : 2 * (int64_t)D;
  return kpart + 2 * (int64_t)vbits_of(v_codec) * D + scales;
}
static int64_t vbase_of(int D, int k_codec) { return k_codec == OR_KF16 ? 32 * (int64_t)D : 8 * (int64_t)D; }
static int64_t kv_ks_off(int t, int k, int D, int v_codec) {
  return 8 * (int64_t)D + 2 * (int64_t)vbits_of(v_codec) * D + 2 * (t * (D / 32) + k);
}
static int64_t kv_vs_off(int t, int k, int D, int k_codec, int v_codec) {
  return vbase_of(D, k_codec) + 2 * (int64_t)vbits_of(v_codec) * D + (k_codec == OR_KF16 ? 0 : D) +
         2 * (t * (D / 32) + k);
}
/* bit offsets, inside the V region, of the low two bits (xb) and of bit 2 (zb) of the
 * b-bit index of (t, d), b = 3 or 2 */
static void vbit_pos(int t, int d, int D, int64_t* xb, int64_t* zb) {
  int G = D / 32, c = d / 2, g = c / 16, m = c % 16, j = t / 4, e = t % 4;
  int l = 16 * j + m, n = 2 * e + (d & 1);
  *xb = 32 * ((int64_t)l * (G / 2) + g / 2) + 4 * n + 2 * (g % 2);
  int64_t zi = ((int64_t)l * G + g) / 4, zs = ((int64_t)l * G + g) % 4;
  *zb = 32 * (32 * (int64_t)G + zi) + 4 * n + zs;
}
static void put_bit(uint8_t* reg, int64_t bit, int v) {
  uint8_t* p = reg + bit / 8;
  *p = v ? (uint8_t)(*p | (1u << (bit % 8))) : (uint8_t)(*p & ~(1u << (bit % 8)));
}
static int get_bit(const uint8_t* reg, int64_t bit) { return (reg[bit / 8] >> (bit % 8)) & 1; }
static void put_v(uint8_t* blk, int t, int d, int D, int k_codec, int v_codec, uint8_t u) {
  uint8_t* reg = blk + vbase_of(D, k_codec);
  int b = vbits_of(v_codec);
  if (b == 4) { put_nibble(reg + (v_byte(t, d, D) - 8 * (int64_t)D), d & 1, u); return; }
  int64_t xb, zb;
  vbit_pos(t, d, D, &xb, &zb);
  put_bit(reg, xb, u & 1);
  put_bit(reg, xb + 1, (u >> 1) & 1);
  if (b == 3) put_bit(reg, zb, (u >> 2) & 1);
}
static uint8_t get_v(const uint8_t* blk, int t, int d, int D, int k_codec, int v_codec) {
  const uint8_t* reg = blk + vbase_of(D, k_codec);
  int b = vbits_of(v_codec);
  if (b == 4) return get_nibble(reg + (v_byte(t, d, D) - 8 * (int64_t)D), d & 1);
  int64_t xb, zb;
  vbit_pos(t, d, D, &xb, &zb);
  int u = get_bit(reg, xb) | (get_bit(reg, xb + 1) << 1);
  if (b == 3) u |= get_bit(reg, zb) << 2;
  return (uint8_t)u;
}

/* Store n tokens x Hkv heads into a pool of any (k_codec, v_codec): keys as indices ku and
 * scales ks (4-bit keys) or fp16 bits kh (fp16 keys), values as indices vu, scales vs.
 * Negative slots are skipped. */
void or_place_kv(uint8_t* pool, int D, int Hkv, int k_codec, int v_codec, int64_t n,
                 const int64_t* slots, const uint8_t* ku, const uint16_t* ks, const uint16_t* kh,
                 const uint8_t* vu, const uint16_t* vs) {
  int G = D / 32;
  int64_t bb = or_block_bytes_kv(D, k_codec, v_codec);
  for (int64_t i = 0; i < n; i++) {
    if (slots[i] < 0) continue;
    int64_t page = slots[i] / OR_PAGE;
    int t = (int)(slots[i] % OR_PAGE);
    for (int h = 0; h < Hkv; h++) {
      uint8_t* blk = pool + (page * Hkv + h) * bb;
      int64_t row = i * Hkv + h;
      for (int d = 0; d < D; d++) {
        if (k_codec == OR_KF16) put16(blk + kf16_off(t, d), kh[row * D + d]);
        else put_nibble(blk + k_byte(t, d, D), (d % 8) & 1, ku[row * D + d]);
        put_v(blk, t, d, D, k_codec, v_codec, vu[row * D + d]);
      }
      for (int k = 0; k < G; k++) {
        if (k_codec != OR_KF16) put16(blk + kv_ks_off(t, k, D, v_codec), ks[row * G + k]);
        put16(blk + kv_vs_off(t, k, D, k_codec, v_codec), vs[row * G + k]);
      }
    }
  }
}

/* Read back one token of a pool of any (k_codec, v_codec): key indices and scales (4-bit
 * keys) or key fp16 bits (fp16 keys), value indices and scales. */
void or_fetch_kv(const uint8_t* pool, int D, int Hkv, int k_codec, int v_codec, int64_t page,
                 int t, int h, uint8_t* ku, uint16_t* ks, uint16_t* kh, uint8_t* vu, uint16_t* vs) {
  int G = D / 32;
  const uint8_t* blk = pool + (page * Hkv + h) * or_block_bytes_kv(D, k_codec, v_codec);
  for (int d = 0; d < D; d++) {
    if (k_codec == OR_KF16) kh[d] = get16(blk + kf16_off(t, d));
    else ku[d] = get_nibble(blk + k_byte(t, d, D), (d % 8) & 1);
    vu[d] = get_v(blk, t, d, D, k_codec, v_codec);
  }
  for (int k = 0; k < G; k++) {
    if (k_codec != OR_KF16) ks[k] = get16(blk + kv_ks_off(t, k, D, v_codec));
    vs[k] = get16(blk + kv_vs_off(t, k, D, k_codec, v_codec));
  }
}

/* Append [one fused step per the Open-TQ-Metal card abstract]: encode K and V of n tokens
 * ([n][Hkv][D] fp32) and store them at their slots. */
void or_append(uint8_t* pool, int D, int Hkv, int k_codec, int v_codec, const uint32_t* sign_bits,
               const float* k, const float* v, int64_t n, const int64_t* slots) {
  int G = D / 32;
  int64_t nv = n * Hkv;
  uint8_t* ku = malloc(nv * D);
  uint8_t* vu = malloc(nv * D);
  uint16_t* ks = malloc(nv * (k_codec == OR_KF16 ? D : G) * 2);
  uint16_t* vs = malloc(nv * G * 2);
  or_encode(v, nv, D, OR_GROUP, sign_bits, v_codec, vu, vs);
  if (k_codec == OR_KF16) {  /* keys kept in fp16, original basis */
    or_keys_f16(k, nv * D, ks);
    or_place_kv(pool, D, Hkv, k_codec, v_codec, n, slots, NULL, NULL, ks, vu, vs);
  } else {
    or_encode(k, nv, D, OR_GROUP, sign_bits, k_codec, ku, ks);
    or_place_kv(pool, D, Hkv, k_codec, v_codec, n, slots, ku, ks, NULL, vu, vs);
  }
  free(ku); free(vu); free(ks); free(vs);
}

/* Read back one token's indices and scales (natural order) from the pool. */
void or_fetch(const uint8_t* pool, int D, int Hkv, int64_t page, int t, int h,
              uint8_t* ku, uint16_t* ks, uint8_t* vu, uint16_t* vs) {
  int G = D / 32;
  const uint8_t* blk = pool + (page * Hkv + h) * or_block_bytes(D);
  for (int d = 0; d < D; d++) {
    ku[d] = get_nibble(blk + k_byte(t, d, D), (d % 8) & 1);
    vu[d] = get_nibble(blk + v_byte(t, d, D), d & 1);
  }
  for (int k = 0; k < G; k++) { ks[k] = get16(blk + ks_off(t, k, D)); vs[k] = get16(blk + vs_off(t, k, D)); }
}

/* ------------------------------------------------------------------------------------- */
/* Plain softmax attention in fp64 for one query: out = softmax(alpha * K q) V.
 * [Open-TQ-Metal arXiv abstract: attention on the compressed representation; the values
 * fed here are the dequantized ones, in the rotated basis]. */
void or_attention_f64(const double* q, const double* K, const double* V, int64_t L, int D,
                      double alpha, double* out) {
  double* s = malloc(sizeof(double) * (L > 0 ? L : 1));
  double mx = -INFINITY;
  for (int64_t t = 0; t < L; t++) {
    double acc = 0.0;
    for (int i = 0; i < D; i++) acc += q[i] * K[t * D + i];
    s[t] = alpha * acc;
    if (s[t] > mx) mx = s[t];
  }
  double l = 0.0;
  for (int i = 0; i < D; i++) out[i] = 0.0;
  for (int64_t t = 0; t < L; t++) {
    double w = exp(s[t] - mx);
    l += w;
    for (int i = 0; i < D; i++) out[i] += w * V[t * D + i];
  }
  for (int i = 0; i < D; i++) out[i] = (L > 0) ? out[i] / l : 0.0;
  free(s);
}

/* Decode attention for a list of (b, hq) pairs, reading the pool through the block table.
 * q is fp32 [B][Hq][D] (already widened from its storage type); alpha is the fp32 scale the
 * caller passes, widened exactly to fp64. The query is rotated with
 * the same fp32 rotation as the keys (not at all for fp16 keys, which stay in the original
 * basis); kv head = hq / (Hq/Hkv) [GQA, contiguous groups].
 * out: fp64 [n_pairs][D], original basis. A sequence of length 0 gives zeros. */
void or_decode(const uint8_t* pool, int D, int Hq, int Hkv, int k_codec, int v_codec,
               const uint32_t* sign_bits, const int32_t* block_table, int max_pages,
               const int32_t* context_lens, const float* q, float alpha,
               const int32_t* pairs, int n_pairs, double* out) {
  uint16_t lut[16];
  or_lut16(lut);
  int r = Hq / Hkv, G = D / 32;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < n_pairs; p++) {
    int b = pairs[2 * p], hq = pairs[2 * p + 1], h = hq / r;
    int64_t L = context_lens[b];
    float qr[512];
    double qd[512], o1[512];
    const float* qx = q + ((int64_t)b * Hq + hq) * D;
    if (k_codec == OR_KF16) {  /* fp16 keys are in the original basis: q as given */
      for (int i = 0; i < D; i++) qd[i] = (double)qx[i];
    } else {
      or_rotate(qx, qr, D, sign_bits);
      for (int i = 0; i < D; i++) qd[i] = (double)qr[i];
    }
    double* K = malloc(sizeof(double) * (L > 0 ? L : 1) * D);
    double* V = malloc(sizeof(double) * (L > 0 ? L : 1) * D);
    uint8_t ku[512], vu[512];
    uint16_t ks[16], vs[16], kh[512];
    for (int64_t t = 0; t < L; t++) {
      int64_t page = block_table[(int64_t)b * max_pages + t / OR_PAGE];
      or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
      if (k_codec == OR_KF16) {
        for (int d = 0; d < D; d++) K[t * D + d] = or_f16_to_f64(kh[d]);
      } else {
        for (int d = 0; d < D; d++) K[t * D + d] = dequant1(k_codec, ku[d], ks[d / 32], lut);
      }
      for (int d = 0; d < D; d++) V[t * D + d] = dequant1(v_codec, vu[d], vs[d / 32], lut);
    }
    (void)G;
    or_attention_f64(qd, K, V, L, D, (double)alpha, o1);
    unrotate_f64(o1, out + (int64_t)p * D, D, sign_bits);
    free(K); free(V);
  }
}

/* Sparse values [mlxcel "TurboQuant KV cache" manual, sparse-V threshold: value
 * dequantization is skipped where the attention weight is below the threshold]. For each
 * (b, hq) pair: the exact fp64 softmax weights w_t over all L tokens (as or_decode);
 * out_sparse = R^-1 sum_{t: w_t >= thr} w_t v_t (the terms below the threshold dropped, the
 * normalizer unchanged), and bound = sum_{t: w_t < thr} w_t * max_i |(R^-1 v_t)_i|, which
 * bounds (max norm) the difference from the exact output made by dropping any subset of the
 * terms below the threshold. */
void or_decode_sparse_v(const uint8_t* pool, int D, int Hq, int Hkv, int k_codec, int v_codec,
                        const uint32_t* sign_bits, const int32_t* block_table, int max_pages,
                        const int32_t* context_lens, const float* q, float alpha, double thr,
                        const int32_t* pairs, int n_pairs, double* out_sparse, double* bound) {
  uint16_t lut[16];
  or_lut16(lut);
  int r = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < n_pairs; p++) {
    int b = pairs[2 * p], hq = pairs[2 * p + 1], h = hq / r;
    int64_t L = context_lens[b];
    float qr[512];
    double qd[512], acc[512], vt[512], ut[512];
    const float* qx = q + ((int64_t)b * Hq + hq) * D;
    if (k_codec == OR_KF16) {
      for (int i = 0; i < D; i++) qd[i] = (double)qx[i];
    } else {
      or_rotate(qx, qr, D, sign_bits);
      for (int i = 0; i < D; i++) qd[i] = (double)qr[i];
    }
    double* sc = malloc(sizeof(double) * (L > 0 ? L : 1));
    uint8_t ku[512], vu[512];
    uint16_t ks[16], vs[16], kh[512];
    double mx = -INFINITY;
    for (int64_t t = 0; t < L; t++) {  /* scores */
      int64_t page = block_table[(int64_t)b * max_pages + t / OR_PAGE];
      double dot = 0.0;
      if (k_codec == OR_KF16) {
        or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
        for (int d = 0; d < D; d++) dot += qd[d] * or_f16_to_f64(kh[d]);
      } else {
        or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
        for (int d = 0; d < D; d++) dot += qd[d] * dequant1(k_codec, ku[d], ks[d / 32], lut);
      }
      sc[t] = (double)alpha * dot;
      if (sc[t] > mx) mx = sc[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < L; t++) l += exp(sc[t] - mx);
    for (int i = 0; i < D; i++) acc[i] = 0.0;
    double bnd = 0.0;
    for (int64_t t = 0; t < L; t++) {  /* weighted values, kept or bounded */
      int64_t page = block_table[(int64_t)b * max_pages + t / OR_PAGE];
      or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
      for (int d = 0; d < D; d++) vt[d] = dequant1(v_codec, vu[d], vs[d / 32], lut);
      double w = exp(sc[t] - mx) / l;
      if (w >= thr) {
        for (int d = 0; d < D; d++) acc[d] += w * vt[d];
      } else {
        unrotate_f64(vt, ut, D, sign_bits);
        double m = 0.0;
        for (int d = 0; d < D; d++) m = fmax(m, fabs(ut[d]));
        bnd += w * m;
      }
    }
    if (L > 0) unrotate_f64(acc, out_sparse + (int64_t)p * D, D, sign_bits);
    else for (int d = 0; d < D; d++) out_sparse[(int64_t)p * D + d] = 0.0;
    bound[p] = bnd;
    free(sc);
  }
}

/* Hot/cold cache [mlxcel "TurboQuant KV cache" manual, delegated cache: the most recent
 * tokens are kept in fp16, the older ones in the packed form]. Sequence b attends to its
 * cold tokens 0..cold_lens[b]-1 in the pool (as or_decode) and then to its hot tokens,
 * hot_k / hot_v [B][Hkv][hot_cap][D] fp16 bits in the original basis, hot_lens[b] of them.
 * One softmax over all of them, in fp64; out is in the original basis. */
void or_decode_hotcold(const uint8_t* pool, int D, int Hq, int Hkv, int k_codec, int v_codec,
                       const uint32_t* sign_bits, const int32_t* block_table, int max_pages,
                       const int32_t* cold_lens, const uint16_t* hot_k, const uint16_t* hot_v,
                       const int32_t* hot_lens, int hot_cap, const float* q, float alpha,
                       const int32_t* pairs, int n_pairs, double* out) {
  uint16_t lut[16];
  or_lut16(lut);
  int r = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < n_pairs; p++) {
    int b = pairs[2 * p], hq = pairs[2 * p + 1], h = hq / r;
    int64_t Lc = cold_lens[b], Lh = hot_lens[b], L = Lc + Lh;
    const float* qx = q + ((int64_t)b * Hq + hq) * D;
    float qr[512];
    double qo[512], qc[512], accc[512], acch[512], tmp[512];
    for (int i = 0; i < D; i++) qo[i] = (double)qx[i];
    if (k_codec == OR_KF16) {
      for (int i = 0; i < D; i++) qc[i] = qo[i];
    } else {
      or_rotate(qx, qr, D, sign_bits);
      for (int i = 0; i < D; i++) qc[i] = (double)qr[i];
    }
    double* sc = malloc(sizeof(double) * (L > 0 ? L : 1));
    uint8_t ku[512], vu[512];
    uint16_t ks[16], vs[16], kh[512];
    double mx = -INFINITY;
    for (int64_t t = 0; t < Lc; t++) {  /* cold scores */
      int64_t page = block_table[(int64_t)b * max_pages + t / OR_PAGE];
      double dot = 0.0;
      if (k_codec == OR_KF16) {
        or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
        for (int d = 0; d < D; d++) dot += qc[d] * or_f16_to_f64(kh[d]);
      } else {
        or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
        for (int d = 0; d < D; d++) dot += qc[d] * dequant1(k_codec, ku[d], ks[d / 32], lut);
      }
      sc[t] = (double)alpha * dot;
    }
    const uint16_t* hk = hot_k + (((int64_t)b * Hkv + h) * hot_cap) * D;
    const uint16_t* hv = hot_v + (((int64_t)b * Hkv + h) * hot_cap) * D;
    for (int64_t t = 0; t < Lh; t++) {  /* hot scores: original basis */
      double dot = 0.0;
      for (int d = 0; d < D; d++) dot += qo[d] * or_f16_to_f64(hk[t * D + d]);
      sc[Lc + t] = (double)alpha * dot;
    }
    for (int64_t t = 0; t < L; t++) if (sc[t] > mx) mx = sc[t];
    double l = 0.0;
    for (int i = 0; i < D; i++) { accc[i] = 0.0; acch[i] = 0.0; }
    for (int64_t t = 0; t < Lc; t++) {  /* cold values, rotated basis */
      int64_t page = block_table[(int64_t)b * max_pages + t / OR_PAGE];
      or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
      double w = exp(sc[t] - mx);
      l += w;
      for (int d = 0; d < D; d++) accc[d] += w * dequant1(v_codec, vu[d], vs[d / 32], lut);
    }
    for (int64_t t = 0; t < Lh; t++) {  /* hot values, original basis */
      double w = exp(sc[Lc + t] - mx);
      l += w;
      for (int d = 0; d < D; d++) acch[d] += w * or_f16_to_f64(hv[t * D + d]);
    }
    double* o = out + (int64_t)p * D;
    if (L == 0) {
      for (int d = 0; d < D; d++) o[d] = 0.0;
    } else {
      unrotate_f64(accc, tmp, D, sign_bits);
      for (int d = 0; d < D; d++) o[d] = (tmp[d] + acch[d]) / l;
    }
    free(sc);
  }
}

/* Dense dequantized K and V, [B][Hkv][Lmax][D] fp32, rows past a sequence's length zero.
 * basis 0: rotated (exact c*s products); basis 1: original, via or_unrotate_f32. */
void or_dequant(const uint8_t* pool, int D, int Hkv, int k_codec, int v_codec,
                const uint32_t* sign_bits, const int32_t* block_table, int max_pages,
                const int32_t* context_lens, int B, int Lmax, int basis, float* kout, float* vout) {
  uint16_t lut[16];
  or_lut16(lut);
  for (int b = 0; b < B; b++)
    for (int h = 0; h < Hkv; h++)
      for (int64_t t = 0; t < Lmax; t++) {
        float* kr = kout + (((int64_t)b * Hkv + h) * Lmax + t) * D;
        float* vr = vout + (((int64_t)b * Hkv + h) * Lmax + t) * D;
        if (t >= context_lens[b]) { memset(kr, 0, 4 * D); memset(vr, 0, 4 * D); continue; }
        uint8_t ku[512], vu[512];
        uint16_t ks[16], vs[16], kh[512];
        int64_t page = block_table[(int64_t)b * max_pages + t / OR_PAGE];
        float ky[512], vy[512];
        if (k_codec == OR_KF16) {
          or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
          for (int d = 0; d < D; d++) ky[d] = (float)or_f16_to_f64(kh[d]);
        } else {
          or_fetch_kv(pool, D, Hkv, k_codec, v_codec, page, (int)(t % OR_PAGE), h, ku, ks, kh, vu, vs);
          for (int d = 0; d < D; d++) ky[d] = (float)dequant1(k_codec, ku[d], ks[d / 32], lut);
        }
        for (int d = 0; d < D; d++) vy[d] = (float)dequant1(v_codec, vu[d], vs[d / 32], lut);
        /* fp16 keys have no rotated form: they are returned as stored in both bases */
        if (basis == 0 || k_codec == OR_KF16) memcpy(kr, ky, 4 * D);
        else or_unrotate_f32(ky, kr, D, sign_bits);
        if (basis == 0) memcpy(vr, vy, 4 * D);
        else or_unrotate_f32(vy, vr, D, sign_bits);
      }
}
