// Decode attention directly on the packed int4 cache.
// [Open-TQ-Metal, arXiv abstract: attention computed on the compressed representation,
//  no intermediate dequantized K/V; the split merge follows the online softmax normalizer
//  cited among its references.]
//
// Pass 1, one workgroup of 4 wavefronts per (sequence b, kv head h, context split s):
//  prologue  the r = Hq/Hkv queries of kv head h are rotated into the cache basis with the
//            same fp32 butterfly as the keys, scaled by alpha*log2(e) and a power of two,
//            and split into fp16 hi + lo parts: B operand rows 0..7 hold hi of heads 0..7,
//            rows 8..15 hold lo, so one 16-column MFMA carries ~22 bits of the query.
//  loop      each wave takes every 4th page of the split. Per 16-token page:
//            scores  S^T[t][row] = sum_g sK[t][g] * (K_g codes . q_g)  (4 x 16x16x32 MFMA
//                    at D=128, one per 32-dim group, codes exact in fp16), hi + lo rows
//                    added with a DPP lane rotate;
//            softmax running max/sum per head (log2 domain);
//            values  o'^T[d][row] += sum_t V codes[t][d] * P'[t][row], P' = p * sV (fp16
//                    hi in rows 0..7, lo in rows 8..15), 2 x 16x16x16 MFMA per group.
//  epilogue  the 4 waves merge through LDS; one partial (o', m, l) per split is written.
// Pass 2, one wavefront per (b, q head): merge the splits, divide by the sum, and rotate
//  back to the original basis (fp32 butterfly, times rho, times sigma).
#include "tq_device.h"
#include "tq_internal.h"

namespace {

template <int G>
__device__ __forceinline__ void load_dwords(const uint8_t* __restrict__ p, uint32_t (&w)[G]) {
  if constexpr (G == 2) {
    u32x2 a = *reinterpret_cast<const u32x2*>(p);
    w[0] = a[0]; w[1] = a[1];
  } else {
#pragma unroll
    for (int i = 0; i < G / 4; i++) {
      u32x4 a = reinterpret_cast<const u32x4*>(p)[i];
      w[4 * i] = a[0]; w[4 * i + 1] = a[1]; w[4 * i + 2] = a[2]; w[4 * i + 3] = a[3];
    }
  }
}

// 4 tokens x G fp16 scales (8G bytes, 16-byte aligned for G >= 2).
template <int G>
__device__ __forceinline__ void load_scales(const uint8_t* __restrict__ p, f16 (&s)[4 * G]) {
  uint32_t w[2 * G];
  if constexpr (G == 2) {
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else {
#pragma unroll
    for (int i = 0; i < G / 2; i++) {
      u32x4 a = reinterpret_cast<const u32x4*>(p)[i];
      w[4 * i] = a[0]; w[4 * i + 1] = a[1]; w[4 * i + 2] = a[2]; w[4 * i + 3] = a[3];
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * G; i++) {
    f16x2 h = as_h2(w[i]);
    s[2 * i] = h[0];
    s[2 * i + 1] = h[1];
  }
}

template <int D, typename TQ, int KCODEC>
__global__ __launch_bounds__(64 * TQ_DECODE_WAVES) void decode_pass1(LaunchDecode a) {
  constexpr int G = D / 32, BB = TQ_BLOCK_BYTES(D), NW = TQ_DECODE_WAVES, NT = 64 * NW;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int r = a.Hq / a.Hkv;
  const int L = a.context_lens[b];
  const int npages = (L + 15) >> 4;
  const int p0 = s * a.pages_per_split;
  if (p0 >= npages) return;  // pass 2 reads only the splits that hold pages
  const int p1 = min(p0 + a.pages_per_split, npages);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int jq = lane >> 4, hr = lane & 15;

  __shared__ float qs[8 * D];
  __shared__ f16x8 bq[G * 64];
  __shared__ float red[NW];
  __shared__ float mo[NW][8][D];
  __shared__ float mml[NW][8][2];

  // ---- prologue: rotate and split the queries ------------------------------------------
  const TQ* qb = static_cast<const TQ*>(a.q) + ((int64_t)b * a.Hq + (int64_t)h * r) * D;
  for (int i = tid; i < 8 * D; i += NT) {
    const int hd = i / D, d = i % D;
    float x = 0.0f;
    if (hd < r) {
      x = widen(qb[hd * D + d]);
      if ((a.sign_bits[d >> 5] >> (d & 31)) & 1u) x = -x;
    }
    qs[i] = x;
  }
  for (int st = 1; st < D; st <<= 1) {
    __syncthreads();
    for (int pi = tid; pi < 4 * D; pi += NT) {
      const int hd = pi / (D / 2), k = pi % (D / 2);
      const int lo = (k / st) * 2 * st + (k % st), hi = lo + st;
      const float x0 = qs[hd * D + lo], x1 = qs[hd * D + hi];
      qs[hd * D + lo] = x0 + x1;
      qs[hd * D + hi] = x0 - x1;
    }
  }
  __syncthreads();
  const float rho = tq_rho(D), qmul = a.attn_scale * TQ_LOG2E;
  float mx = 0.0f;
  for (int i = tid; i < 8 * D; i += NT) {
    const float v = (qs[i] * rho) * qmul;
    qs[i] = v;
    mx = fmaxf(mx, fabsf(v));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < NW; w++) mx = fmaxf(mx, red[w]);
  int sh = 0;
  if (mx > 0.0f) sh = min(60, max(-60, 14 - ilogbf(mx)));
  const float up = ldexpf(1.0f, sh), down = ldexpf(1.0f, -sh);
  for (int idx = tid; idx < G * 64; idx += NT) {
    const int g = idx >> 6, l = idx & 63, j = l >> 4, c = l & 15, hd = c & 7;
    f16x8 v;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float x = (hd < r) ? qs[hd * D + 32 * g + 8 * j + kslot_dim<KCODEC>(k)] * up : 0.0f;
      const f16 hi = (f16)x;
      v[k] = (c < 8) ? hi : (f16)(x - (float)hi);
    }
    bq[idx] = v;
  }
  __syncthreads();
  f16x8 bop[G];
#pragma unroll
  for (int g = 0; g < G; g++) bop[g] = bq[g * 64 + lane];

  uint32_t tlo[4] = {0, 0, 0, 0}, thi[4] = {0, 0, 0, 0};
  if constexpr (KCODEC == TQ_CODEC_LLOYDMAX) {
    const uint16_t lb[16] = TQ_LUT16_BITS;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      tlo[i >> 2] |= (uint32_t)(lb[i] & 0xffu) << (8 * (i & 3));
      thi[i >> 2] |= (uint32_t)(lb[i] >> 8) << (8 * (i & 3));
    }
  }

  // ---- main loop over pages --------------------------------------------------------------
  f32x4 acc[2 * G];
#pragma unroll
  for (int t = 0; t < 2 * G; t++) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int p = p0 + wv; p < p1; p += NW) {
    const uint8_t* blk = a.pool + ((int64_t)bt[p] * a.Hkv + h) * BB;
    uint32_t kw[G], vw[G];
    load_dwords<G>(blk + lane * 4 * G, kw);
    load_dwords<G>(blk + 8 * D + lane * 4 * G, vw);
    f16 ks[4 * G], vs[4 * G];
    load_scales<G>(blk + 16 * D + 8 * G * jq, ks);
    load_scales<G>(blk + 16 * D + 32 * G + 8 * G * jq, vs);

    float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < G; g++) {
      f16x8 A;
      if constexpr (KCODEC == TQ_CODEC_LLOYDMAX) A = unpack_k_lut(kw[g], tlo, thi);
      else A = unpack_k_absmax(kw[g]);
      const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bop[g], zero4, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; e++) sc[e] += (float)ks[e * G + g] * c[e];
    }
    const int tb = p * 16 + 4 * jq;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      sc[e] = (sc[e] + dpp_ror8(sc[e])) * down;
      if (tb + e >= L) sc[e] = -INFINITY;
    }
    float cm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    cm = fmaxf(cm, xor_shfl(cm, 16));
    cm = fmaxf(cm, xor_shfl(cm, 32));
    if (cm > m_run) {
      const float f = exp2f(m_run - cm);
      l_run *= f;
#pragma unroll
      for (int t = 0; t < 2 * G; t++) acc[t] *= f;
      m_run = cm;
    }
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; e++) pr[e] = exp2f(sc[e] - m_run);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);

#pragma unroll
    for (int g = 0; g < G; g++) {
      f16x4 P;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int e = (k >> 1) | ((k & 1) << 1);  // k-slot order: tokens 0, 2, 1, 3
        const float x = (tb + e < L) ? pr[e] * (float)vs[e * G + g] : 0.0f;
        const f16 hi = (f16)x;
        P[k] = (hr < 8) ? hi : (f16)(x - (float)hi);
      }
      const uint32_t w = vw[g];
      const f16x2 e0 = nib_p0p4(w), e1 = nib_p0p4(w >> 8);
      const f16x2 o0 = nib_p1p5(w), o1 = nib_p1p5(w >> 8);
      const f16x4 Ae = {e0[0], e0[1], e1[0], e1[1]};
      const f16x4 Ao = {o0[0], o0[1], o1[0], o1[1]};
      acc[2 * g] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ae, P, acc[2 * g], 0, 0, 0);
      acc[2 * g + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ao, P, acc[2 * g + 1], 0, 0, 0);
    }
  }

  // ---- epilogue: per-wave results, then merge the waves of this workgroup ------------------
  l_run += xor_shfl(l_run, 16);
  l_run += xor_shfl(l_run, 32);
#pragma unroll
  for (int t = 0; t < 2 * G; t++)
#pragma unroll
    for (int i = 0; i < 4; i++) acc[t][i] += dpp_ror8(acc[t][i]);
  if (hr < 8) {
#pragma unroll
    for (int g = 0; g < G; g++)
#pragma unroll
      for (int par = 0; par < 2; par++)
#pragma unroll
        for (int i = 0; i < 4; i++) mo[wv][hr][32 * g + 8 * jq + 2 * i + par] = acc[2 * g + par][i];
    if (jq == 0) {
      mml[wv][hr][0] = m_run;
      mml[wv][hr][1] = l_run;
    }
  }
  __syncthreads();
  const int S = a.splits;
  for (int i = tid; i < r * D; i += NT) {
    const int hd = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) M = fmaxf(M, mml[w][hd][0]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const float mw = mml[w][hd][0];
      if (mw != -INFINITY) {
        const float f = exp2f(mw - M);
        o += f * mo[w][hd][d];
        l += f * mml[w][hd][1];
      }
    }
    const int64_t row = ((int64_t)b * a.Hq + (int64_t)h * r + hd) * S + s;
    a.part_o[row * D + d] = o;
    if (d == 0) {
      a.part_ml[2 * row] = M;
      a.part_ml[2 * row + 1] = l;
    }
  }
}

}  // namespace

namespace {
// Pass 2 (also used by the dense baseline with unrotate = false).
template <int D, bool UNROTATE>
__global__ __launch_bounds__(64) void decode_pass2(LaunchDecode a) {
  constexpr int PL = D / 64;
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = a.context_lens[b];
  const int npages = (L + 15) >> 4;
  const int ns = (npages + a.pages_per_split - 1) / a.pages_per_split;
  const int64_t row0 = ((int64_t)b * a.Hq + hq) * a.splits;
  __shared__ float buf[D];
  float M = -INFINITY;
  for (int s = 0; s < ns; s++) M = fmaxf(M, a.part_ml[2 * (row0 + s)]);
  float lsum = 0.0f, v[PL];
#pragma unroll
  for (int k = 0; k < PL; k++) v[k] = 0.0f;
  for (int s = 0; s < ns; s++) {
    const float m = a.part_ml[2 * (row0 + s)];
    if (m == -INFINITY) continue;
    const float f = exp2f(m - M);
    lsum += f * a.part_ml[2 * (row0 + s) + 1];
#pragma unroll
    for (int k = 0; k < PL; k++) v[k] += f * a.part_o[(row0 + s) * D + lane + 64 * k];
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int k = 0; k < PL; k++) buf[lane + 64 * k] = v[k] * inv;
  if constexpr (UNROTATE) {
    for (int st = 1; st < D; st <<= 1) {
      __syncthreads();
      for (int pi = lane; pi < D / 2; pi += 64) {
        const int lo = (pi / st) * 2 * st + (pi % st), hi = lo + st;
        const float x0 = buf[lo], x1 = buf[hi];
        buf[lo] = x0 + x1;
        buf[hi] = x0 - x1;
      }
    }
    __syncthreads();
    const float rho = tq_rho(D);
#pragma unroll
    for (int k = 0; k < PL; k++) {
      const int d = lane + 64 * k;
      float x = buf[d] * rho;
      if ((a.sign_bits[d >> 5] >> (d & 31)) & 1u) x = -x;
      buf[d] = x;
    }
  }
  __syncthreads();
  float* o = a.out + ((int64_t)b * a.Hq + hq) * D;
#pragma unroll
  for (int k = 0; k < PL; k++) o[lane + 64 * k] = buf[lane + 64 * k];
}
}  // namespace

namespace {

// Dense fp16 decode attention, the "attend" half of the dequantize-then-attend baseline
// [Open-TQ-Metal, arXiv abstract]. K, V fp16 [B][Hkv][max_ctx][D] in the original basis;
// q is used unrotated. Plain VALU fp32 arithmetic on 64-token tiles staged in LDS; the
// partial (o', m, l) format is that of the compressed pass 1, merged by pass 2.
template <int D, typename TQ>
__global__ __launch_bounds__(256) void dense_pass1(LaunchDecode a) {
  constexpr int TT = 64, PD = D + 8, DPT = D / 32;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int r = a.Hq / a.Hkv;
  const int L = a.context_lens[b];
  const int npages = (L + 15) >> 4;
  const int p0 = s * a.pages_per_split;
  if (p0 >= npages) return;
  const int t0 = p0 * 16, t1 = min(min(p0 + a.pages_per_split, npages) * 16, L);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ float qf[8][D];
  __shared__ f16 kt[TT][PD];
  __shared__ f16 vt[TT][PD];
  __shared__ float pt[8][TT];
  __shared__ float mrow[8], lrow[8], frow[8];

  const TQ* qb = static_cast<const TQ*>(a.q) + ((int64_t)b * a.Hq + (int64_t)h * r) * D;
  const float qmul = a.attn_scale * TQ_LOG2E;
  for (int i = tid; i < 8 * D; i += 256) {
    const int hd = i / D, d = i % D;
    qf[hd][d] = hd < r ? widen(qb[hd * D + d]) * qmul : 0.0f;
  }
  if (tid < 8) { mrow[tid] = -INFINITY; lrow[tid] = 0.0f; frow[tid] = 1.0f; }
  const f16* kb = static_cast<const f16*>(static_cast<const void*>(a.pool)) +
                  ((int64_t)b * a.Hkv + h) * (int64_t)a.max_ctx * D;
  const f16* vb = static_cast<const f16*>(a.dense_v) + ((int64_t)b * a.Hkv + h) * (int64_t)a.max_ctx * D;
  const int phd = tid >> 5, pd0 = tid & 31;   // PV mapping: head phd, dims pd0 + 32 k
  float o[DPT];
#pragma unroll
  for (int k = 0; k < DPT; k++) o[k] = 0.0f;

  for (int t = t0; t < t1; t += TT) {
    const int n = min(TT, t1 - t);
    __syncthreads();
    for (int i = tid; i < TT * (D / 8); i += 256) {
      const int row = i / (D / 8), c8 = i % (D / 8);
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (row < n) {
        kv = reinterpret_cast<const u32x4*>(kb + (int64_t)(t + row) * D)[c8];
        vv = reinterpret_cast<const u32x4*>(vb + (int64_t)(t + row) * D)[c8];
      }
      *reinterpret_cast<u32x4*>(&kt[row][8 * c8]) = kv;
      *reinterpret_cast<u32x4*>(&vt[row][8 * c8]) = vv;
    }
    __syncthreads();
    for (int hd = wv; hd < r; hd += 4) {
      float sc = -INFINITY;
      if (lane < n) {
        float acc = 0.0f;
#pragma unroll 8
        for (int d = 0; d < D; d++) acc += qf[hd][d] * (float)kt[lane][d];
        sc = acc;
      }
      float cm = sc;
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o2, 64));
      const float m_old = mrow[hd];
      const float m_new = fmaxf(m_old, cm);
      const float p = exp2f(sc - m_new);
      float ps = p;
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) ps += __shfl_xor(ps, o2, 64);
      pt[hd][lane] = p;
      if (lane == 0) {
        const float f = exp2f(m_old - m_new);
        frow[hd] = f;
        lrow[hd] = lrow[hd] * f + ps;
        mrow[hd] = m_new;
      }
    }
    __syncthreads();
    if (phd < r) {
      const float f = frow[phd];
#pragma unroll
      for (int k = 0; k < DPT; k++) o[k] *= f;
      for (int tt = 0; tt < n; tt++) {
        const float p = pt[phd][tt];
#pragma unroll
        for (int k = 0; k < DPT; k++) o[k] += p * (float)vt[tt][pd0 + 32 * k];
      }
    }
  }
  __syncthreads();
  if (phd < r) {
    const int64_t row = ((int64_t)b * a.Hq + (int64_t)h * r + phd) * a.splits + s;
#pragma unroll
    for (int k = 0; k < DPT; k++) a.part_o[row * D + pd0 + 32 * k] = o[k];
    if (pd0 == 0) {
      a.part_ml[2 * row] = mrow[phd];
      a.part_ml[2 * row + 1] = lrow[phd];
    }
  }
}

template <int D, typename TQ>
hipError_t launch_dense_dq(const LaunchDecode& a, hipStream_t st) {
  hipLaunchKernelGGL((dense_pass1<D, TQ>), dim3(a.splits, a.Hkv, a.B), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_pass2<D, false>), dim3(a.Hq, a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dense_d(const LaunchDecode& a, hipStream_t st) {
  switch (a.q_dtype) {
    case TQ_F32: return launch_dense_dq<D, float>(a, st);
    case TQ_BF16: return launch_dense_dq<D, uint16_t>(a, st);
    default: return launch_dense_dq<D, f16>(a, st);
  }
}

template <int D, typename TQ>
hipError_t launch_dq(const LaunchDecode& a, hipStream_t st) {
  dim3 g1(a.splits, a.Hkv, a.B), b1(64 * TQ_DECODE_WAVES);
  if (a.k_codec == TQ_CODEC_LLOYDMAX)
    hipLaunchKernelGGL((decode_pass1<D, TQ, TQ_CODEC_LLOYDMAX>), g1, b1, 0, st, a);
  else
    hipLaunchKernelGGL((decode_pass1<D, TQ, TQ_CODEC_ABSMAX>), g1, b1, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_pass2<D, true>), dim3(a.Hq, a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const LaunchDecode& a, hipStream_t st) {
  switch (a.q_dtype) {
    case TQ_F32: return launch_dq<D, float>(a, st);
    case TQ_BF16: return launch_dq<D, uint16_t>(a, st);
    default: return launch_dq<D, f16>(a, st);
  }
}

}  // namespace

hipError_t tq_launch_decode(const LaunchDecode& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_d<64>(a, st);
    case 128: return launch_d<128>(a, st);
    default: return launch_d<256>(a, st);
  }
}

hipError_t tq_launch_dense_decode(const LaunchDecode& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_dense_d<64>(a, st);
    case 128: return launch_dense_d<128>(a, st);
    default: return launch_dense_d<256>(a, st);
  }
}
