// Dense fp16 decode attention: the "attend" half of the dequantize-then-attend baseline
// [Open-TQ-Metal, arXiv abstract], plus the split merge it uses. Plain VALU fp32
// arithmetic; this is the comparison path, not the product's hot path.
#include "tq_device.h"
#include "tq_internal.h"

namespace {
// Merge of the context splits: m* = max m_s, o = sum_s 2^(m_s - m*) o_s / sum_s 2^(m_s - m*) l_s.
template <int D, bool UNROTATE>
__global__ __launch_bounds__(64) void merge_splits(LaunchDecode a) {
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
// partial (o', m, l) layout is [B][Hq][S][D] and [B][Hq][S][2], merged by merge_splits.
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
  hipLaunchKernelGGL((merge_splits<D, false>), dim3(a.Hq, a.B), dim3(64), 0, st, a);
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

}  // namespace

hipError_t tq_launch_dense_decode(const LaunchDecode& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_dense_d<64>(a, st);
    case 128: return launch_dense_d<128>(a, st);
    default: return launch_dense_d<256>(a, st);
  }
}
