// Append kernel: rotate, quantize and pack new K/V vectors into the paged pool.
// [Open-TQ-Metal, card abstract: one fused kernel does the sign-randomized rotation, the
//  per-group abs-max and the int4 nibble pack.] The per-vector arithmetic is in tq_codec.h:
// 16 lanes per vector, bit-identical to the plain definition.
#include "tq_codec.h"
#include "tq_internal.h"

namespace {

// One vector (the key or the value of one token and kv head) per 16-lane group, 16 per
// workgroup: workgroup (x, y) takes kv head y of tokens 8x .. 8x + 7, waves 0 and 2 their
// keys, waves 1 and 3 their values, so that every wave runs one codec. A vector's slot
// and input are loaded together; one vector per group keeps each wave's dependent chain
// short (a small append is one pass of latency) while a large one fills every SIMD.
template <int D, typename TIn, int KCODEC, int VCODEC>
__global__ __launch_bounds__(256) void append_kernel(uint8_t* __restrict__ pool,
                                                     const TIn* __restrict__ kin,
                                                     const TIn* __restrict__ vin,
                                                     const int64_t* __restrict__ slots,
                                                     const uint32_t* __restrict__ sign_bits,
                                                     int n_tokens, int Hkv) {
  constexpr int E = D / 16;
  constexpr int BB = tq_block_bytes(D, KCODEC, VCODEC);
  constexpr int VB = tq_value_bits(VCODEC);
  constexpr bool KF16 = KCODEC == TQ_CODEC_FP16;
  constexpr bool KLUT = KCODEC == TQ_CODEC_LLOYDMAX;
  // sigma as a sign mask per coordinate (0 or the fp32 sign bit); the key codebook's
  // bucket table
  __shared__ uint32_t smask[D];
  __shared__ u32x2 lut_tbl[KLUT ? tq_lutb::NB : 1];
  const int cb = tq_blk16(threadIdx.x & 15);
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int tok = blockIdx.x * 8 + (wave >> 1) * 4 + ((threadIdx.x >> 4) & 3);
  const int tc = min(tok, n_tokens - 1);  // (a token past the end loads the last one's)
  const int is_v = wave & 1;
  // the vector's slot and input first, then the sign mask's words: one wait covers all
  const int64_t slot_in = slots[tc];
  float y[E];
  load_widen<TIn, E>((is_v ? vin : kin) + ((size_t)tc * Hkv + h) * D + cb * E, y);
  // (both small loads issued before either is used: one wait covers them and the above)
  const int tid = threadIdx.x;
  const uint32_t sword = tid < D ? sign_bits[tid >> 5] : 0u;
  u32x2 tent = {0u, 0u};
  if constexpr (KLUT) tent = tq_lut_table_entry(tid);
  if (tid < D) smask[tid] = ((sword >> (tid & 31)) & 1u) << 31;
  if (KLUT && tid < tq_lutb::NB) lut_tbl[tid] = tent;
  __syncthreads();
  const int64_t slot = tok < n_tokens ? slot_in : -1;
  if (slot < 0) return;  // a skipped token, or past the end: the same for the 16 lanes
  uint8_t* blk = pool + ((slot >> 4) * (int64_t)Hkv + h) * BB;
  const int t = (int)(slot & 15);
  if (KF16 && !is_v) {  // fp16 keys: stored as given, no rotation
    place_key_f16<D>(blk, t, cb, y);
    return;
  }
#pragma unroll
  for (int e = 0; e < E; e++) y[e] = __uint_as_float(__float_as_uint(y[e]) ^ smask[cb * E + e]);
  uint32_t u[E];
  f16 scale;
  if (is_v) codec_vector<D, VCODEC>(y, cb, u, scale);
  else if (KLUT) codec_vector<D, TQ_CODEC_LLOYDMAX>(y, cb, u, scale, lut_tbl);
  else codec_vector<D, TQ_CODEC_ABSMAX>(y, cb, u, scale);
  place_vector<D, KF16, VB>(blk, t, cb, is_v != 0, u, scale);
}

template <int D, typename T, int VC>
hipError_t launch_v(const LaunchAppend& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.n_tokens + 7) / 8), (unsigned)a.Hkv);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  if (a.k_codec == TQ_CODEC_LLOYDMAX)
    hipLaunchKernelGGL((append_kernel<D, T, TQ_CODEC_LLOYDMAX, VC>), grid, dim3(256), 0, st, a.pool, k, v,
                       a.slots, a.sign_bits, a.n_tokens, a.Hkv);
  else if (a.k_codec == TQ_CODEC_FP16)
    hipLaunchKernelGGL((append_kernel<D, T, TQ_CODEC_FP16, VC>), grid, dim3(256), 0, st, a.pool, k, v,
                       a.slots, a.sign_bits, a.n_tokens, a.Hkv);
  else
    hipLaunchKernelGGL((append_kernel<D, T, TQ_CODEC_ABSMAX, VC>), grid, dim3(256), 0, st, a.pool, k, v,
                       a.slots, a.sign_bits, a.n_tokens, a.Hkv);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_d(const LaunchAppend& a, hipStream_t st) {
  switch (a.v_codec) {
    case TQ_CODEC_ABSMAX3: return launch_v<D, T, TQ_CODEC_ABSMAX3>(a, st);
    case TQ_CODEC_ABSMAX2: return launch_v<D, T, TQ_CODEC_ABSMAX2>(a, st);
    default: return launch_v<D, T, TQ_CODEC_ABSMAX>(a, st);
  }
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
