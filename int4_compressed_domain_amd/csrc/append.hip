// Append kernel: rotate, quantize and pack new K/V vectors into the paged pool.
// [Open-TQ-Metal, card abstract: one fused kernel does the sign-randomized rotation, the
//  per-group abs-max and the int4 nibble pack.] The per-vector arithmetic is in tq_codec.h:
// 16 lanes per vector, bit-identical to the plain definition.
#include "tq_codec.h"
#include "tq_internal.h"

namespace {

// Each 16-lane group takes VPT vectors (index vec = group * VPT + i; even vec: key, odd:
// value, of token-head vec / 2): their slots and inputs are all loaded first, so one group
// keeps several loads in flight and a large append needs few wavefronts.
constexpr int VPT = 4;

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
  const int lane = threadIdx.x & 15;
  const int64_t nvec = (int64_t)n_tokens * Hkv * 2;
  const int64_t vec0 = ((int64_t)blockIdx.x * 16 + (threadIdx.x >> 4)) * VPT;
  if (vec0 >= nvec) return;  // whole 16-lane groups exit together
  int64_t slot[VPT];
  float y[VPT][E];
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t vec = vec0 + i;
    slot[i] = -1;
    if (vec < nvec) {
      const int64_t th = vec >> 1;  // token * Hkv + head
      slot[i] = slots[th / Hkv];
      load_widen<TIn, E>(((vec & 1) ? vin : kin) + th * D + lane * E, y[i]);
    }
  }
  const uint32_t sw = lane_signs<D>(sign_bits, lane);
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    if (slot[i] < 0) continue;  // a skipped token, or past the end: the same for the group
    const int64_t vec = vec0 + i;
    const int is_v = (int)(vec & 1);
    const int h = (int)((vec >> 1) % Hkv);
    uint8_t* blk = pool + ((slot[i] >> 4) * (int64_t)Hkv + h) * BB;
    if (KF16 && !is_v) {  // fp16 keys: stored as given, no rotation
      place_key_f16<D>(blk, (int)(slot[i] & 15), lane, y[i]);
      continue;
    }
    uint32_t u[E];
    f16 scale;
    if (is_v) codec_vector<D, VCODEC>(y[i], sw, lane, u, scale);
    else if (KCODEC == TQ_CODEC_LLOYDMAX) codec_vector<D, TQ_CODEC_LLOYDMAX>(y[i], sw, lane, u, scale);
    else codec_vector<D, TQ_CODEC_ABSMAX>(y[i], sw, lane, u, scale);
    place_vector<D, KF16, VB>(blk, (int)(slot[i] & 15), lane, is_v != 0, u, scale);
  }
}

template <int D, typename T, int VC>
hipError_t launch_v(const LaunchAppend& a, hipStream_t st) {
  const int64_t nvec = (int64_t)a.n_tokens * a.Hkv * 2;
  dim3 grid((unsigned)((nvec + 16 * VPT - 1) / (16 * VPT)));
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
