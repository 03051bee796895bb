// Internal launch descriptors shared by the host API (tq_api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

struct LaunchAppend {
  uint8_t* pool;
  const void* k;
  const void* v;
  const int64_t* slots;
  const uint32_t* sign_bits;
  int D, Hkv, n_tokens, dtype, k_codec, v_codec;
};

// Split-K decode: pass 1 writes, per (b, q head, split), the unnormalized weighted value
// sum o' (rotated basis) and the running max m (log2 units) and sum l; pass 2 merges them.
struct LaunchDecode {
  const uint8_t* pool;       // compressed pool (pass 1), or dense fp16 K (dense path)
  const void* dense_v;       // dense fp16 V (dense path only)
  const void* q;
  const int32_t* block_table;
  const int32_t* context_lens;
  const uint32_t* sign_bits;
  float* out;
  float* part_o;             // [B][Hq][S][D] (= [unit][split][r][D])
  float* part_ml;            // [B][Hq][S][2]
  int* counters;             // per unit (b * Hkv + h) arrival counters, zero between calls
  int D, Hq, Hkv, B, max_pages, max_ctx, q_dtype, k_codec, v_codec;
  int splits, pages_per_split;
  float attn_scale;
  const void* knew;          // optional: K and V of each sequence's last token,
  const void* vnew;          //   [B][Hkv][D] of new_dtype, appended before attending
  int new_dtype;
  int32_t* order;            // optional [B * Hkv]: the unit that workgroup position u takes
  int sparse_v;              // 1: values loaded only where a weight can reach v_thr
  float v_thr;               // sparse values: weight threshold
  unsigned long long* v_skipped;  // optional: pages whose values were skipped (added to)
  const void* hot_k;         // optional fp16 tail [B][Hkv][hot_cap][D] (original basis),
  const void* hot_v;         //   hot_lens[b] tokens attended after the pool's context_lens[b]
  const int32_t* hot_lens;
  int hot_cap;
  int hot_wg;                // 1: split index `splits` of each unit takes the whole tail
};

hipError_t tq_launch_append(const LaunchAppend& a, hipStream_t st);
hipError_t tq_launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t st);
hipError_t tq_launch_decode(const LaunchDecode& a, hipStream_t st);
hipError_t tq_launch_dense_decode(const LaunchDecode& a, hipStream_t st);

struct LaunchDequant {
  const uint8_t* pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  const uint32_t* sign_bits;
  void* k_out;
  void* v_out;
  int D, Hkv, B, max_pages, max_ctx, original_basis, out_dtype, k_codec, v_codec;
};
hipError_t tq_launch_dequant(const LaunchDequant& a, hipStream_t st);

// Wavefronts per fused-decode workgroup; each workgroup owns one (sequence, kv head,
// context split). 16 waves fill a CU when the kernel fits in 128 registers per lane.
// fp16 keys: 8 waves (a staged page is 41*D bytes, three per wave fit the LDS ring).
constexpr int tq_decode_waves(int D, int k_codec = TQ_CODEC_ABSMAX) {
  return (D > 128 || k_codec == TQ_CODEC_FP16) ? 8 : 16;
}
// Bits per value index of a value codec.
constexpr int tq_value_bits(int v_codec) { return TQ_VALUE_BITS(v_codec); }
// Bytes of one block (16 tokens of one kv head).
constexpr int tq_block_bytes(int D, int k_codec, int v_codec = TQ_CODEC_ABSMAX) {
  return TQ_BLOCK_BYTES_KV(D, k_codec, v_codec);
}
constexpr int TQ_DECODE_WAVES = 4;   // dense baseline workgroups
constexpr int TQ_MAX_SPLITS = 128;   // context splits per (sequence, kv head)
constexpr int TQ_MAX_SPLIT_PAGES = 2048;  // pages per split (their ids are staged in LDS)
constexpr int TQ_LPT_MAX_BATCH = 256;    // longest-first workgroup order up to this batch
constexpr int TQ_SPARSE_PAGES_PER_WAVE = 32;  // sparse values: page maxima kept per wave
constexpr int TQ_MAX_HOT = 1024;         // fp16 tail tokens per (sequence, kv head)
constexpr int TQ_MAX_UNITS = 1 << 20;  // sequences x kv heads per call
