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
  int hot_wg;                // > 0: split indices splits + k of each unit take the tail in hot_wg pieces
};

hipError_t tq_launch_append(const LaunchAppend& a, hipStream_t st);
hipError_t tq_launch_decode(const LaunchDecode& a, hipStream_t st);
hipError_t tq_launch_zero_i32(int32_t* p, int n, hipStream_t st);
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

// Bits per value index of a value codec.
constexpr int tq_value_bits(int v_codec) { return TQ_VALUE_BITS(v_codec); }
#ifndef TQ_REG_WAVES
#define TQ_REG_WAVES 8
#endif
#ifndef TQ_REG_PAGES_PER_STEP
#define TQ_REG_PAGES_PER_STEP 2
#endif
// Packed 3- and 2-bit values: 4 pages per step (their pages are ~28% smaller, so two sets
// of 2 keep fewer bytes in flight; 128K with 2-bit values: 32.9 us against 33.7 with 2).
#ifndef TQ_REG_PPS_PACKED
#define TQ_REG_PPS_PACKED 4
#endif
#ifndef TQ_REG_EARLY
#define TQ_REG_EARLY 2
#endif
// Wavefronts per fused-decode workgroup; each workgroup owns one (sequence, kv head,
// context split). Pages staged in LDS (fp16 keys, 3- and 2-bit values, sparse values):
// 16 waves fill a CU when the kernel fits in 128 registers per lane; fp16 keys or D = 256
// take 8 (a staged fp16-key page is 41*D bytes, three per wave fit the LDS ring), fp16 keys
// at D = 256 (10.5 KB a page) 4, one workgroup per CU (the ring takes 123 KB), which limits
// that variant to 4 query heads per kv head (one wave per head in the rotations). Pages
// streamed through registers (abs-max keys, D <= 128): two sets of
// TQ_REG_PAGES_PER_STEP pages per wave, one computed while the other is in flight, need
// more than 128 registers, so 8 waves of up to 256.
#ifndef TQ_REG_LUT
#define TQ_REG_LUT 0
#endif
#ifndef TQ_REG_PACKED
#define TQ_REG_PACKED 1
#endif
// Variants whose pages stream through registers (the others stage pages in LDS): abs-max
// keys at D <= 128 with 4-bit values, or packed 3- and 2-bit ones; sparse values included
// (the first pass streams the keys alone).
constexpr bool tq_decode_reg_path(int D, int k_codec, int value_bits, bool sparse) {
  return D <= 128 && (value_bits == 4 || TQ_REG_PACKED) &&
         (k_codec == TQ_CODEC_ABSMAX || (TQ_REG_LUT && k_codec == TQ_CODEC_LLOYDMAX));
}
constexpr int tq_decode_waves(int D, int k_codec, int v_codec, bool sparse) {
  if (D > 128 && k_codec == TQ_CODEC_FP16) return 4;
  if (D > 128 || k_codec == TQ_CODEC_FP16) return 8;
  if (tq_decode_reg_path(D, k_codec, tq_value_bits(v_codec), sparse)) return TQ_REG_WAVES;
  return 16;
}
// Bytes of one block (16 tokens of one kv head).
constexpr int tq_block_bytes(int D, int k_codec, int v_codec = TQ_CODEC_ABSMAX) {
  return TQ_BLOCK_BYTES_KV(D, k_codec, v_codec);
}
constexpr int TQ_DECODE_WAVES = 4;   // dense baseline workgroups
constexpr int TQ_MAX_SPLITS = 128;   // context splits per (sequence, kv head)
constexpr int TQ_MAX_SPLIT_PAGES = 2048;  // pages per split (their ids are held in registers)
// Pages per split of a variant with nw waves: every wave keeps the ids of its pages in at
// most four registers (256 ids).
constexpr int tq_max_split_pages(int nw) { return 256 * nw < TQ_MAX_SPLIT_PAGES ? 256 * nw : TQ_MAX_SPLIT_PAGES; }
constexpr int TQ_LPT_MAX_BATCH = 256;    // longest-first workgroup order up to this batch
constexpr int TQ_SPARSE_PAGES_PER_WAVE = 32;  // sparse values: page maxima kept per wave
// Sparse values: per-(unit, head) published maxima, 8 words per unit from word 2^19 of the
// workspace's counter area (zero between calls like the arrival counters), so at most
// 2^16 units.
constexpr int TQ_SPARSE_MAX_BASE = 1 << 19;
constexpr int TQ_SPARSE_MAX_UNITS = 1 << 16;
constexpr int TQ_MAX_HOT = 1024;         // fp16 tail tokens per (sequence, kv head)
constexpr int TQ_MAX_UNITS = 1 << 20;  // sequences x kv heads per call
