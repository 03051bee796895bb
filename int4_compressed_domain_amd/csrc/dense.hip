// Dense fp16 decode attention: the "attend" half of the dequantize-then-attend baseline
// [Open-TQ-Metal, arXiv abstract], plus the split merge it uses. This is the comparison
// path, not the product's hot path, but it is built to stream its fp16 K and V near the
// memory rate: scores on the matrix cores (16 tokens x 16 columns per MFMA: 8 query heads
// as fp16 hi parts, the same heads' lo parts), values on the VALU with fp32 accumulation.
#include "tq_device.h"
#include "tq_internal.h"

namespace {
// Merge of the context splits: m* = max m_s, o = sum_s 2^(m_s - m*) o_s / sum_s 2^(m_s - m*) l_s.
// One wave per (sequence, q head): the lanes take the splits' (m, l) 64 at a time, so the
// loads of a round are in flight together, and the partial rows are summed eight rows at a
// time, all of their loads issued before the first is used.
template <int D>
__global__ __launch_bounds__(64) void merge_splits(LaunchDecode a) {
  constexpr int PL = D / 64;
  const int hq = (int)(blockIdx.x % (uint32_t)a.Hq), b = (int)(blockIdx.x / (uint32_t)a.Hq), lane = threadIdx.x;
  const int L = a.context_lens[b];
  const int npages = (L + 15) >> 4;
  const int ns = (npages + a.pages_per_split - 1) / a.pages_per_split;
  const int64_t row0 = ((int64_t)b * a.Hq + hq) * a.splits;
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, a.part_ml[2 * (row0 + s)]);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
  float lsum = 0.0f, v[PL];
#pragma unroll
  for (int k = 0; k < PL; k++) v[k] = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    float f = 0.0f, lw = 0.0f;
    if (s0 + lane < ns) {
      const float m = a.part_ml[2 * (row0 + s0 + lane)];
      f = m == -INFINITY ? 0.0f : exp2f(m - M);
      lw = f * a.part_ml[2 * (row0 + s0 + lane) + 1];
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) lw += __shfl_xor(lw, x, 64);
    lsum += lw;
    const int cnt = min(64, ns - s0);
    const float* po = a.part_o + (row0 + s0) * D + lane;
    int i = 0;
    for (; i + 8 <= cnt; i += 8) {  // eight partial rows loaded before any is used
      float x[8][PL];
#pragma unroll
      for (int u = 0; u < 8; u++)
#pragma unroll
        for (int k = 0; k < PL; k++) x[u][k] = po[(int64_t)(i + u) * D + 64 * k];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const float fi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), i + u));
#pragma unroll
        for (int k = 0; k < PL; k++) v[k] += fi * x[u][k];
      }
    }
    for (; i < cnt; i++) {
      const float fi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), i));
#pragma unroll
      for (int k = 0; k < PL; k++) v[k] += fi * po[(int64_t)i * D + 64 * k];
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  float* o = a.out + ((int64_t)b * a.Hq + hq) * D;
#pragma unroll
  for (int k = 0; k < PL; k++) o[lane + 64 * k] = v[k] * inv;
}

// One workgroup of 4 waves per (split, kv head, sequence). The split's tokens are cut into
// 16-token tiles dealt to the waves in turn; each wave keeps its own running max and sum.
// Scores of a tile: A = 16 rows of K (lane l: row l%16, dims 32g + 8(l/16) .. +7, one
// 16-byte load per group straight from the row), B = the query as fp16 hi (columns 0-7)
// and lo (columns 8-15) parts, scaled per head by a power of two that keeps both parts
// normal; lane l gets rows 4(l/16) .. +3 of column l%16, and the hi and lo columns are added
// by a row rotation of 8 lanes. Values: lane l holds G chunks of 8 dims (chunk l % (D/8)) of
// tokens (l + 64k) / (D/8), reads the tile's weights of all heads from LDS and accumulates
// 8 dims x RP heads. The waves' (o', m, l) are merged in LDS into the split's partial.
template <int D, int RP>
__global__ __launch_bounds__(256) void dense_attn(LaunchDecode a) {
  constexpr int G = D / 32, NC = D / 8;
  // one-dimensional grid: workgroup = (split s, kv head h, sequence b)
  const uint32_t unit = blockIdx.x / (uint32_t)a.splits;
  const int s = (int)(blockIdx.x % (uint32_t)a.splits);
  const int h = (int)(unit % (uint32_t)a.Hkv), b = (int)(unit / (uint32_t)a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = a.Hq / a.Hkv;
  __shared__ __align__(16) float Pt[4][16][8];     // per wave: the tile's weights [token][head]
  __shared__ float Ft[4][8];         // per wave: rescale factors of the heads
  __shared__ float Ow[4][RP][D];     // per wave: o' of each head
  __shared__ float MLw[4][RP][2];    // per wave: m, l of each head
  const int L = a.context_lens[b];
  const int npages = (L + 15) >> 4;
  const int p0 = s * a.pages_per_split;
  if (p0 >= npages) return;
  const int t0 = p0 * 16, t1 = min(min(p0 + a.pages_per_split, npages) * 16, L);
  const int ntile = (t1 - t0 + 15) >> 4;
  const f16* kb = reinterpret_cast<const f16*>(a.pool) + ((int64_t)b * a.Hkv + h) * (int64_t)a.max_ctx * D;
  const f16* vb = static_cast<const f16*>(a.dense_v) + ((int64_t)b * a.Hkv + h) * (int64_t)a.max_ctx * D;

  // ---- query operand: column n = lane % 16 is head n % 8 (hi for n < 8, lo otherwise)
  const int n = lane & 15, kq = lane >> 4, hd = n & 7;
  const float qmul = a.attn_scale * TQ_LOG2E;
  float qx[G][8];
  const int64_t qoff = ((int64_t)b * a.Hq + (int64_t)h * r + (hd < r ? hd : 0)) * D + 8 * kq;
  // 8 consecutive elements per group with vector loads, all issued before any is used (the
  // address is valid for every lane; heads past r are zeroed after the load)
  const float keep = hd < r ? qmul : 0.0f;
  if (a.q_dtype == TQ_F32) {
    const float* qp = static_cast<const float*>(a.q) + qoff;
    f32x4 raw[G][2];
#pragma unroll
    for (int g = 0; g < G; g++) {
      raw[g][0] = *reinterpret_cast<const f32x4*>(qp + 32 * g);
      raw[g][1] = *reinterpret_cast<const f32x4*>(qp + 32 * g + 4);
    }
#pragma unroll
    for (int g = 0; g < G; g++)
#pragma unroll
      for (int e = 0; e < 8; e++) qx[g][e] = raw[g][e >> 2][e & 3] * keep;
  } else {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qoff;
    u32x4 raw[G];
#pragma unroll
    for (int g = 0; g < G; g++) raw[g] = *reinterpret_cast<const u32x4*>(qp + 32 * g);
    const bool bf = a.q_dtype == TQ_BF16;
#pragma unroll
    for (int g = 0; g < G; g++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const uint16_t bits = (uint16_t)(raw[g][e >> 1] >> (16 * (e & 1)));
        qx[g][e] = (bf ? widen(bits) : widen(__builtin_bit_cast(f16, bits))) * keep;
      }
  }
  float amax = 0.0f;
#pragma unroll
  for (int g = 0; g < G; g++)
#pragma unroll
    for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(qx[g][e]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  int ex = 0;
  if (amax > 0.0f && amax <= 3.0e38f) (void)frexpf(amax, &ex);
  const float up = ldexpf(1.0f, 15 - ex), down = ldexpf(1.0f, ex - 15);  // amax*up in [2^14, 2^15)
  f16x8 bq[G];
#pragma unroll
  for (int g = 0; g < G; g++)
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float x = qx[g][e] * up;
      const f16 hi = (f16)x;
      bq[g][e] = n < 8 ? hi : (f16)(x - (float)hi);
    }

  float acc[RP][8];
#pragma unroll
  for (int k = 0; k < RP; k++)
#pragma unroll
    for (int e = 0; e < 8; e++) acc[k][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;  // of head hd; l_run is this lane's rows only

  const int chunk = lane % NC;
  auto load_tile = [&](int tile, f16x8* kA, f16x8* vv) {
    const int tt = t0 + 16 * tile;
    const int kr = min(tt + n, L - 1);
#pragma unroll
    for (int g = 0; g < G; g++)
      kA[g] = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(kb + (int64_t)kr * D + 32 * g + 8 * kq));
#pragma unroll
    for (int k = 0; k < G; k++) {
      const int vr = min(tt + (lane + 64 * k) / NC, L - 1);
      vv[k] = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(vb + (int64_t)vr * D + 8 * chunk));
    }
  };
  // NB tiles in registers: the one being computed and NB - 1 in flight (3 at D <= 128, where
  // the registers allow it; 2 at D = 256)
  constexpr int NB = D <= 128 ? 3 : 2;
  f16x8 kbuf[NB][G], vbuf[NB][G];
  auto step = [&](int tile, const f16x8* kA, const f16x8* vv) {
    const int tt = t0 + 16 * tile;
    f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < G; g++) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(kA[g], bq[g], c, 0, 0, 0);
    float sc[4], tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sc[i] = tt + 4 * kq + i < t1 ? (c[i] + dpp_ror8(c[i])) * down : -INFINITY;
      tmax = fmaxf(tmax, sc[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sc[i] = exp2f(sc[i] - m_new);
      ps += sc[i];
    }
    const bool grew = m_new > m_run;
    const float f = exp2f(m_run - m_new);  // 1 where the max did not grow
    l_run = l_run * f + ps;
    m_run = m_new;
    if (n < 8) {
#pragma unroll
      for (int i = 0; i < 4; i++) Pt[w][4 * kq + i][n] = sc[i];
      if (kq == 0) Ft[w][n] = f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (__any(grew)) {
#pragma unroll
      for (int k = 0; k < RP; k++) {
        const float fk = Ft[w][k];
#pragma unroll
        for (int e = 0; e < 8; e++) acc[k][e] *= fk;
      }
    }
#pragma unroll
    for (int k = 0; k < G; k++) {
      const int tk = (lane + 64 * k) / NC;
      const f32x4 p0v = *reinterpret_cast<const f32x4*>(&Pt[w][tk][0]);
      const f32x4 p1v = *reinterpret_cast<const f32x4*>(&Pt[w][tk][4]);
      const float pk[8] = {p0v[0], p0v[1], p0v[2], p0v[3], p1v[0], p1v[1], p1v[2], p1v[3]};
#pragma unroll
      for (int hh = 0; hh < RP; hh++)
#pragma unroll
        for (int e = 0; e < 8; e++) acc[hh][e] = __builtin_fmaf((float)vv[k][e], pk[hh], acc[hh][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  if (w < ntile) {
#pragma unroll
    for (int i = 0; i < NB; i++) load_tile(min(w + 4 * i, ntile - 1), kbuf[i], vbuf[i]);
  }
  for (int tile = w; tile < ntile; tile += 4 * NB) {
    // the loads are issued whether or not their tile exists (the last tile again), so
    // every buffer has the same loads outstanding on every path
#pragma unroll
    for (int i = 0; i < NB; i++) {
      const int ti = tile + 4 * i;
      if (ti < ntile) step(ti, kbuf[i], vbuf[i]);
      load_tile(min(ti + 4 * NB, ntile - 1), kbuf[i], vbuf[i]);
    }
  }
  // ---- the wave's totals: o' summed over the lanes of each dim chunk, l over the row groups
#pragma unroll
  for (int x = NC; x < 64; x <<= 1)
#pragma unroll
    for (int k = 0; k < RP; k++)
#pragma unroll
      for (int e = 0; e < 8; e++) acc[k][e] += __shfl_xor(acc[k][e], x, 64);
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (lane < NC)
#pragma unroll
    for (int k = 0; k < RP; k++)
#pragma unroll
      for (int e = 0; e < 8; e++) Ow[w][k][8 * lane + e] = acc[k][e];
  if (lane < RP) {
    MLw[w][lane][0] = m_run;
    MLw[w][lane][1] = l_run;
  }
  __syncthreads();
  // ---- merge of the 4 waves into the split's partial (o' relative to the split's max)
  for (int i = tid; i < r * D; i += 256) {
    const int k = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; v++) M = fmaxf(M, MLw[v][k][0]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const float mv = MLw[v][k][0];
      if (mv == -INFINITY) continue;
      const float f = exp2f(mv - M);
      o += f * Ow[v][k][d];
      l += f * MLw[v][k][1];
    }
    const int64_t row = ((int64_t)b * a.Hq + (int64_t)h * r + k) * a.splits + s;
    a.part_o[row * D + d] = o;
    if (d == 0) {
      a.part_ml[2 * row] = M;
      a.part_ml[2 * row + 1] = l;
    }
  }
}

template <int D, int RP>
hipError_t launch_dense_dr(const LaunchDecode& a, hipStream_t st) {
  hipLaunchKernelGGL((dense_attn<D, RP>), dim3((unsigned)((int64_t)a.splits * a.Hkv * a.B)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((merge_splits<D>), dim3((unsigned)((int64_t)a.Hq * a.B)), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dense_d(const LaunchDecode& a, hipStream_t st) {
  const int r = a.Hq / a.Hkv;
  if (r <= 1) return launch_dense_dr<D, 1>(a, st);
  if (r <= 2) return launch_dense_dr<D, 2>(a, st);
  if (r <= 4) return launch_dense_dr<D, 4>(a, st);
  return launch_dense_dr<D, 8>(a, st);
}

}  // namespace

hipError_t tq_launch_dense_decode(const LaunchDecode& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_dense_d<64>(a, st);
    case 128: return launch_dense_d<128>(a, st);
    default: return launch_dense_d<256>(a, st);
  }
}
