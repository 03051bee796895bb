// Host side of the C ABI: argument validation (before any device work), launch geometry
// (context split count), workspace sizing and kernel dispatch. Declarations and the
// meaning of every argument are in include/tq.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/tq.h"
#include "tq_internal.h"

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Layout checks shared by every entry point. Non-power-of-two head dims are rejected, as
// the mlxcel TurboQuant manual (head-dim limitation) does at cache initialisation.
int check_layout(const tq_layout* L, bool need_pool_fields) {
  if (!L) return TQ_EINVAL;
  if (!is_pow2(L->head_dim)) return TQ_EINVAL;
  if (L->num_q_heads <= 0 || L->num_kv_heads <= 0) return TQ_EINVAL;
  if (L->num_q_heads % L->num_kv_heads != 0) return TQ_EINVAL;
  if (L->head_dim != 64 && L->head_dim != 128 && L->head_dim != 256) return TQ_EUNSUPPORTED;
  if (L->num_q_heads / L->num_kv_heads > 8) return TQ_EUNSUPPORTED;
  if (!need_pool_fields) return TQ_OK;
  if (L->group_size <= 0 || L->head_dim % L->group_size != 0) return TQ_EINVAL;
  if (L->group_size != 32) return TQ_EUNSUPPORTED;
  if (L->page_size <= 0) return TQ_EINVAL;
  if (L->page_size != 16) return TQ_EUNSUPPORTED;
  if (L->num_pages < 0) return TQ_EINVAL;
  if (L->k_codec != TQ_CODEC_ABSMAX && L->k_codec != TQ_CODEC_LLOYDMAX && L->k_codec != TQ_CODEC_FP16)
    return TQ_EINVAL;
  if (L->v_codec == TQ_CODEC_LLOYDMAX || L->v_codec == TQ_CODEC_FP16)
    return TQ_EUNSUPPORTED;  // the LUT codec and fp16 are for keys
  if (L->v_codec != TQ_CODEC_ABSMAX && L->v_codec != TQ_CODEC_ABSMAX3 && L->v_codec != TQ_CODEC_ABSMAX2)
    return TQ_EINVAL;
  if (!L->sign_bits) return TQ_EINVAL;
  return TQ_OK;
}

bool valid_dtype(int d) { return d == TQ_F32 || d == TQ_BF16 || d == TQ_F16; }

int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Context split of the fused decode: about one 16-wave workgroup (two 8-wave ones at
// D = 256) per compute unit in total, at least four pages per wave where the context has
// them, at most TQ_MAX_SPLITS.
struct Split { int splits, pages_per_split; };

Split make_split(int pages, int S) {
  Split s{1, pages > 0 ? pages : 1};
  if (pages == 0) return s;
  if (S > pages) S = pages;
  if (S < 1) S = 1;
  s.pages_per_split = (pages + S - 1) / S;
  s.splits = (pages + s.pages_per_split - 1) / s.pages_per_split;
  return s;
}

// sparse: the two-pass sparse-value loop keeps at most TQ_SPARSE_PAGES_PER_WAVE pages per
// wave, which sets a smallest split count.
Split choose_split(int B, int Hkv, int D, int k_codec, int v_codec, int max_ctx, int requested,
                   bool sparse = false) {
  const int pages = (max_ctx + 15) / 16;
  const int nw = tq_decode_waves(D, k_codec, v_codec, sparse);
  const int maxp = tq_max_split_pages(nw);
  int min_s = (pages + maxp - 1) / maxp;  // page ids fit the waves' registers
  if (sparse) {
    const int per = TQ_SPARSE_PAGES_PER_WAVE * nw;
    if ((pages + per - 1) / per > min_s) min_s = (pages + per - 1) / per;
  }
  if (requested > 0) {
    int S = requested < TQ_MAX_SPLITS ? requested : TQ_MAX_SPLITS;
    return make_split(pages, S > min_s ? S : min_s);
  }
  const int64_t units = (int64_t)B * Hkv;
  // one workgroup per CU: the page ring takes ~147 KB of a CU's 160 KB of LDS, at every head
  // size (at D = 256, batch 4, 8 kv heads, 32K tokens: 63.4 us against 70.6 us with splits
  // sized for two workgroups per CU)
  const int64_t target = (int64_t)num_cus();
  int64_t want = (target + units - 1) / units;
  // at least ~1.5 pages per wave: below that the split merge costs more than the split
  // saves (1024 tokens, one kv head, 8 waves: 11.2 us with 2 splits, 10.3 with 4, 10.1 with
  // 5 or 6, 10.4 with 8)
  const int64_t cap = 2 * (int64_t)pages / (3 * nw) > 1 ? 2 * (int64_t)pages / (3 * nw) : 1;
  if (want > cap) want = cap;
  if (want < min_s) want = min_s;
  if (want > TQ_MAX_SPLITS) want = TQ_MAX_SPLITS;
  return make_split(pages, (int)want);
}

// The dense baseline uses 4-wave workgroups, two per compute unit (its 8-head kernel at
// head_dim 128 takes 166 registers a lane: two waves per SIMD).
Split choose_split_dense(int B, int Hkv, int max_ctx, int requested) {
  const int pages = (max_ctx + 15) / 16;
  if (requested > 0) return make_split(pages, requested);
  const int64_t units = (int64_t)B * Hkv;
  int64_t want = (2LL * num_cus() + units - 1) / units;
  const int64_t cap = (pages + TQ_DECODE_WAVES - 1) / TQ_DECODE_WAVES;
  if (want > cap) want = cap;
  return make_split(pages, (int)want);
}

size_t partial_bytes(int B, int Hq, int D, int splits) {
  return (size_t)B * Hq * splits * ((size_t)D + 2) * sizeof(float);
}

size_t workspace_bytes(const tq_layout* L, int B, int max_ctx, int requested) {
  const Split f = choose_split(B, L->num_kv_heads, L->head_dim, L->k_codec, L->v_codec, max_ctx, requested);
  const Split sp = choose_split(B, L->num_kv_heads, L->head_dim, L->k_codec, L->v_codec, max_ctx, requested, true);
  const Split d = choose_split_dense(B, L->num_kv_heads, max_ctx, requested);
  int S = f.splits > d.splits ? f.splits : d.splits;
  if (sp.splits > S) S = sp.splits;
  return TQ_DECODE_COUNTER_BYTES + partial_bytes(B, L->num_q_heads, L->head_dim, S) +
         (size_t)B * L->num_kv_heads * sizeof(int32_t);  // + the workgroup order
}

int from_hip(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_EDEVICE; }

// ---- optional validation of device-side preconditions (TQ_VALIDATE=1) -------------------
// Block tables, lengths and slots live in device memory and are normally trusted. With the
// environment variable TQ_VALIDATE set to 1, a call first synchronizes its stream, copies
// them to the host and rejects out-of-range values before launching anything.
bool validating() {
  const char* e = getenv("TQ_VALIDATE");
  return e && e[0] == '1' && e[1] == 0;
}

template <typename T>
int to_host(std::vector<T>& dst, const T* src, size_t n) {
  dst.resize(n);
  if (n == 0) return TQ_OK;
  return from_hip(hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost));
}

// lengths in [0, max_ctx]; the page ids a sequence uses in [0, num_pages); tail lengths
// (hot_lens, when given) in [0, hot_cap]
int validate_tables(const tq_layout* L, int batch, const int32_t* block_table, int max_pages,
                    const int32_t* lens_dev, int max_ctx, const int32_t* hot_lens, int hot_cap,
                    hipStream_t st) {
  if (hipStreamSynchronize(st) != hipSuccess) return TQ_EDEVICE;
  std::vector<int32_t> lens, bt, hl;
  int rc = to_host(lens, lens_dev, (size_t)batch);
  if (rc != TQ_OK) return rc;
  int32_t need = 0;
  for (int b = 0; b < batch; b++) {
    if (lens[b] < 0 || lens[b] > max_ctx) return TQ_EINVAL;
    need = std::max(need, (lens[b] + 15) / 16);
  }
  if (need > 0) {
    if (!block_table) return TQ_EINVAL;
    rc = to_host(bt, block_table, (size_t)batch * max_pages);
    if (rc != TQ_OK) return rc;
    for (int b = 0; b < batch; b++)
      for (int p = 0; p < (lens[b] + 15) / 16; p++) {
        const int32_t id = bt[(size_t)b * max_pages + p];
        if (id < 0 || id >= L->num_pages) return TQ_EINVAL;
      }
  }
  if (hot_lens) {
    rc = to_host(hl, hot_lens, (size_t)batch);
    if (rc != TQ_OK) return rc;
    for (int b = 0; b < batch; b++)
      if (hl[b] < 0 || hl[b] > hot_cap) return TQ_EINVAL;
  }
  return TQ_OK;
}

// slots inside the pool (negative: skipped), no slot twice
int validate_slots(const tq_layout* L, int n, const int64_t* slots, hipStream_t st) {
  if (hipStreamSynchronize(st) != hipSuccess) return TQ_EDEVICE;
  std::vector<int64_t> sl;
  const int rc = to_host(sl, slots, (size_t)n);
  if (rc != TQ_OK) return rc;
  std::vector<int64_t> used;
  for (int64_t x : sl) {
    if (x < 0) continue;
    if (x >= (int64_t)L->num_pages * 16) return TQ_EINVAL;
    used.push_back(x);
  }
  std::sort(used.begin(), used.end());
  return std::adjacent_find(used.begin(), used.end()) == used.end() ? TQ_OK : TQ_EINVAL;
}

int check_decode_common(const tq_layout* L, const void* q, int q_dtype, int batch,
                        const int32_t* context_lens, int max_context_len, float attn_scale,
                        int num_splits, const float* out) {
  if (batch < 0 || max_context_len < 0 || num_splits < 0) return TQ_EINVAL;
  if (!valid_dtype(q_dtype)) return TQ_EINVAL;
  if (!isfinite(attn_scale)) return TQ_EINVAL;
  if (batch > 0 && (!q || !context_lens || !out)) return TQ_EINVAL;
  if ((int64_t)batch * L->num_kv_heads > TQ_MAX_UNITS) return TQ_EUNSUPPORTED;
  (void)L;
  return TQ_OK;
}

}  // namespace

// ---- decode without allocation: the library's own device scratch -----------------------
// One array per GPU (each device holds its own copy of a __device__ variable), looked up
// with hipGetSymbolAddress on the first call on that device and kept per device: in host
// code the array's name is not a device address.
static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int TQ_MAX_DEVICES = 64;
std::atomic<void*> scratch_dev[TQ_MAX_DEVICES];
std::mutex scratch_mu;

int scratch_of_current_device(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= TQ_MAX_DEVICES) return TQ_EDEVICE;
  void* ptr = scratch_dev[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> g(scratch_mu);
    ptr = scratch_dev[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TQ_EDEVICE;
      scratch_dev[dev].store(ptr, std::memory_order_release);
    }
  }
  *p = ptr;
  return TQ_OK;
}
}  // namespace

extern "C" {

const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "TQ_OK";
    case TQ_EINVAL: return "TQ_EINVAL: invalid argument";
    case TQ_EUNSUPPORTED: return "TQ_EUNSUPPORTED: configuration not implemented on the GPU";
    case TQ_ENOSPC: return "TQ_ENOSPC: workspace too small";
    case TQ_EDEVICE: return "TQ_EDEVICE: HIP runtime error";
    default: return "unknown tq_status";
  }
}

size_t tq_page_bytes(const tq_layout* L) {
  if (check_layout(L, true) != TQ_OK) return 0;
  return (size_t)L->num_kv_heads * tq_block_bytes(L->head_dim, L->k_codec, L->v_codec);
}

int tq_kv_append(const tq_layout* L, void* pool, const void* k, const void* v, int32_t in_dtype,
                 int32_t n_tokens, const int64_t* slot_mapping, void* stream) {
  int rc = check_layout(L, true);
  if (rc != TQ_OK) return rc;
  if (n_tokens < 0 || !valid_dtype(in_dtype)) return TQ_EINVAL;
  if (n_tokens == 0) return TQ_OK;
  if (!pool || !k || !v || !slot_mapping) return TQ_EINVAL;
  if (L->num_kv_heads > 65535) return TQ_EUNSUPPORTED;  // (one grid row per kv head)
  if (validating()) {
    rc = validate_slots(L, n_tokens, slot_mapping, static_cast<hipStream_t>(stream));
    if (rc != TQ_OK) return rc;
  }
  LaunchAppend a{static_cast<uint8_t*>(pool), k, v, slot_mapping, L->sign_bits,
                 L->head_dim, L->num_kv_heads, n_tokens, in_dtype, L->k_codec, L->v_codec};
  return from_hip(tq_launch_append(a, static_cast<hipStream_t>(stream)));
}

size_t tq_decode_workspace_size(const tq_layout* L, int32_t batch, int32_t max_context_len,
                                int32_t num_splits) {
  if (check_layout(L, false) != TQ_OK || batch < 0 || max_context_len < 0 || num_splits < 0) return 0;
  return workspace_bytes(L, batch, max_context_len, num_splits);
}

static_assert(((size_t)TQ_SPARSE_MAX_BASE + 8 * (size_t)TQ_SPARSE_MAX_UNITS) * 4 <= TQ_DECODE_COUNTER_BYTES,
              "the sparse maxima must fit the counter area");

// no_alloc: the workspace is the library's static scratch (tq_decode_attn_noalloc): its
// arrival counters are cleared by a fill kernel before the decode, and the TQ_VALIDATE
// host checks (which synchronize and copy to host buffers) are not run.
static int decode_impl(const tq_layout* L, const void* pool, const void* knew, const void* vnew,
                       int32_t new_dtype, const void* q, int32_t q_dtype, int32_t batch,
                       const int32_t* block_table, int32_t max_pages_per_seq,
                       const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                       int32_t num_splits, float* out, void* workspace, size_t workspace_bytes_,
                       void* stream, int sparse_v = 0, float v_thr = 0.0f,
                       unsigned long long* v_skipped = nullptr, const void* hot_k = nullptr,
                       const void* hot_v = nullptr, const int32_t* hot_lens = nullptr,
                       int hot_cap = 0, bool no_alloc = false) {
  int rc = check_layout(L, true);
  if (rc != TQ_OK) return rc;
  rc = check_decode_common(L, q, q_dtype, batch, context_lens, max_context_len, attn_scale,
                           num_splits, out);
  if (rc != TQ_OK) return rc;
  if (max_pages_per_seq < 0 || (int64_t)max_context_len > 16LL * max_pages_per_seq) return TQ_EINVAL;
  const int nw = tq_decode_waves(L->head_dim, L->k_codec, L->v_codec, sparse_v != 0);
  if ((int64_t)max_context_len > 16LL * TQ_MAX_SPLITS * tq_max_split_pages(nw)) return TQ_EUNSUPPORTED;
  if (L->num_q_heads / L->num_kv_heads > nw) return TQ_EUNSUPPORTED;  // one wave per q head
  if (sparse_v && (int64_t)batch * L->num_kv_heads > TQ_SPARSE_MAX_UNITS) return TQ_EUNSUPPORTED;
  if (sparse_v && (int64_t)max_context_len >
                      16LL * TQ_MAX_SPLITS * TQ_SPARSE_PAGES_PER_WAVE * tq_decode_waves(L->head_dim, L->k_codec, L->v_codec, true))
    return TQ_EUNSUPPORTED;
  if (batch == 0) return TQ_OK;
  // with every context empty nothing is read from the pool or the block table (the outputs
  // are zeros, plus a tail's attention for tq_decode_attn_hotcold): they may be NULL then
  if (max_context_len > 0 && (!pool || !block_table)) return TQ_EINVAL;
  Split s = choose_split(batch, L->num_kv_heads, L->head_dim, L->k_codec, L->v_codec, max_context_len,
                         num_splits, sparse_v != 0);
  const int64_t resident = (int64_t)num_cus();  // fused-decode workgroups the chip holds at once
  // fp16 tail: with automatic splits, a grid that fits the chip and at least 8 splits per
  // unit for every 512 tokens of tail capacity, splits are given up for workgroups that take
  // the tail in pieces of at most 512 tokens and run beside the pool's (their cost then
  // hides behind theirs); otherwise every split takes a slice of the tail after its pages.
  // Measured at 128K (one sequence, 8 kv heads, 32 splits): tails of 512 / 640 / 768 / 1024
  // tokens in one workgroup 34.9 / 36.9 / 40.2 / 49.1 us against 38.4 / 38.6 / 38.7 / 38.8
  // us in slices; at D = 256, 4 sequences of 32K (8 splits): 512 tokens 62.8 against 72.2
  // us, 1024 tokens in one workgroup 101 against 77 us. With 16 splits or more, two pieces
  // even for short tails (128K: 256 tokens 34.83 against 35.05 us in one, 512 tokens 34.87
  // against 34.97 us).
  int hot_wg = 0;
  const int hot_pieces = (hot_cap + 511) / 512 < 2 && s.splits >= 16 ? 2 : (hot_cap + 511) / 512;
  if (hot_k && num_splits == 0 && s.splits >= 8 * hot_pieces &&
      (int64_t)batch * L->num_kv_heads * s.splits <= resident &&
      (int64_t)(s.splits - hot_pieces) * tq_max_split_pages(nw) >= (max_context_len + 15) / 16) {
    s = make_split((max_context_len + 15) / 16, s.splits - hot_pieces);
    hot_wg = hot_pieces;
  }
  if (workspace_bytes_ < workspace_bytes(L, batch, max_context_len, num_splits)) return TQ_ENOSPC;
  if (!workspace) return TQ_EINVAL;
  if (!no_alloc && validating()) {
    rc = validate_tables(L, batch, block_table, max_pages_per_seq, context_lens, max_context_len,
                         hot_k ? hot_lens : nullptr, hot_cap, static_cast<hipStream_t>(stream));
    if (rc != TQ_OK) return rc;
  }
  float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + TQ_DECODE_COUNTER_BYTES);
  LaunchDecode a{};
  a.counters = static_cast<int*>(workspace);
  a.pool = static_cast<const uint8_t*>(pool);
  a.q = q;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.sign_bits = L->sign_bits;
  a.out = out;
  const int rows = s.splits + hot_wg;  // partial rows per unit
  a.part_o = ws;
  a.part_ml = ws + (size_t)batch * L->num_q_heads * rows * L->head_dim;
  a.D = L->head_dim; a.Hq = L->num_q_heads; a.Hkv = L->num_kv_heads; a.B = batch;
  a.max_pages = max_pages_per_seq; a.max_ctx = max_context_len;
  a.q_dtype = q_dtype; a.k_codec = L->k_codec; a.v_codec = L->v_codec;
  a.splits = s.splits; a.pages_per_split = s.pages_per_split;
  a.attn_scale = attn_scale;
  a.knew = knew; a.vnew = vnew; a.new_dtype = new_dtype;
  a.sparse_v = sparse_v; a.v_thr = v_thr; a.v_skipped = v_skipped;
  a.hot_k = hot_k; a.hot_v = hot_v; a.hot_lens = hot_lens; a.hot_cap = hot_cap; a.hot_wg = hot_wg;
  // longest-first order pays when the workgroups do not all fit on the chip at once
  if (batch > 1 && batch <= TQ_LPT_MAX_BATCH && (int64_t)batch * L->num_kv_heads * s.splits > resident)
    a.order = reinterpret_cast<int32_t*>(
        a.part_ml + (size_t)batch * L->num_q_heads * rows * 2);
  if (no_alloc) {
    rc = from_hip(tq_launch_zero_i32(a.counters, batch * L->num_kv_heads, static_cast<hipStream_t>(stream)));
    if (rc != TQ_OK) return rc;
  }
  return from_hip(tq_launch_decode(a, static_cast<hipStream_t>(stream)));
}

int tq_decode_attn(const tq_layout* L, const void* pool, const void* q, int32_t q_dtype,
                   int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                   const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                   int32_t num_splits, float* out, void* workspace, size_t workspace_bytes_,
                   void* stream) {
  return decode_impl(L, pool, nullptr, nullptr, 0, q, q_dtype, batch, block_table,
                     max_pages_per_seq, context_lens, max_context_len, attn_scale, num_splits, out,
                     workspace, workspace_bytes_, stream);
}

int tq_decode_attn_noalloc(const tq_layout* L, const void* pool, const void* q, int32_t q_dtype,
                           int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                           const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                           int32_t num_splits, float* out, void* stream) {
  int rc = check_layout(L, true);
  if (rc != TQ_OK) return rc;
  if (batch < 0 || max_context_len < 0 || num_splits < 0) return TQ_EINVAL;
  if (batch > 0 && workspace_bytes(L, batch, max_context_len, num_splits) > TQ_NOALLOC_SCRATCH_BYTES)
    return TQ_ENOSPC;
  void* ws = nullptr;
  if (batch > 0) {
    rc = scratch_of_current_device(&ws);
    if (rc != TQ_OK) return rc;
  }
  return decode_impl(L, pool, nullptr, nullptr, 0, q, q_dtype, batch, block_table, max_pages_per_seq,
                     context_lens, max_context_len, attn_scale, num_splits, out, ws,
                     TQ_NOALLOC_SCRATCH_BYTES, stream, 0, 0.0f, nullptr, nullptr, nullptr, nullptr, 0,
                     true);
}

int tq_append_decode_attn(const tq_layout* L, void* pool, const void* k_last, const void* v_last,
                          int32_t in_dtype, const void* q, int32_t q_dtype, int32_t batch,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                          int32_t num_splits, float* out, void* workspace, size_t workspace_bytes_,
                          void* stream) {
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16 && in_dtype != TQ_F16) return TQ_EINVAL;
  if (batch > 0 && (!k_last || !v_last)) return TQ_EINVAL;
  return decode_impl(L, pool, k_last, v_last, in_dtype, q, q_dtype, batch, block_table,
                     max_pages_per_seq, context_lens, max_context_len, attn_scale, num_splits, out,
                     workspace, workspace_bytes_, stream);
}

int tq_decode_attn_sparse_v(const tq_layout* L, const void* pool, const void* q, int32_t q_dtype,
                            int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                            float v_threshold, int32_t num_splits, float* out, void* workspace,
                            size_t workspace_bytes_, unsigned long long* v_pages_skipped,
                            void* stream) {
  if (!(v_threshold >= 0.0f && v_threshold < 1.0f)) return TQ_EINVAL;
  // a zero threshold drops nothing: the dense decode, bit for bit
  return decode_impl(L, pool, nullptr, nullptr, 0, q, q_dtype, batch, block_table,
                     max_pages_per_seq, context_lens, max_context_len, attn_scale, num_splits, out,
                     workspace, workspace_bytes_, stream, v_threshold > 0.0f ? 1 : 0, v_threshold,
                     v_pages_skipped);
}

int tq_append_decode_attn_sparse_v(const tq_layout* L, void* pool, const void* k_last,
                                   const void* v_last, int32_t in_dtype, const void* q,
                                   int32_t q_dtype, int32_t batch, const int32_t* block_table,
                                   int32_t max_pages_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, float attn_scale, float v_threshold,
                                   int32_t num_splits, float* out, void* workspace,
                                   size_t workspace_bytes_, unsigned long long* v_pages_skipped,
                                   void* stream) {
  if (!(v_threshold >= 0.0f && v_threshold < 1.0f)) return TQ_EINVAL;
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16 && in_dtype != TQ_F16) return TQ_EINVAL;
  if (batch > 0 && (!k_last || !v_last)) return TQ_EINVAL;
  // a zero threshold drops nothing: tq_append_decode_attn, bit for bit
  return decode_impl(L, pool, k_last, v_last, in_dtype, q, q_dtype, batch, block_table,
                     max_pages_per_seq, context_lens, max_context_len, attn_scale, num_splits, out,
                     workspace, workspace_bytes_, stream, v_threshold > 0.0f ? 1 : 0, v_threshold,
                     v_pages_skipped);
}

int tq_decode_attn_hotcold(const tq_layout* L, const void* pool, const void* q, int32_t q_dtype,
                           int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                           const int32_t* cold_lens, int32_t max_cold_len, const void* hot_k,
                           const void* hot_v, const int32_t* hot_lens, int32_t hot_cap,
                           float attn_scale, int32_t num_splits, float* out, void* workspace,
                           size_t workspace_bytes_, void* stream) {
  if (hot_cap < 1 || hot_cap > TQ_MAX_HOT) return TQ_EUNSUPPORTED;
  if (batch > 0 && (!hot_k || !hot_v || !hot_lens)) return TQ_EINVAL;
  return decode_impl(L, pool, nullptr, nullptr, 0, q, q_dtype, batch, block_table,
                     max_pages_per_seq, cold_lens, max_cold_len, attn_scale, num_splits, out,
                     workspace, workspace_bytes_, stream, 0, 0.0f, nullptr, hot_k, hot_v, hot_lens,
                     hot_cap);
}

int tq_dequant_ref(const tq_layout* L, const void* pool, int32_t batch, const int32_t* block_table,
                   int32_t max_pages_per_seq, const int32_t* context_lens, int32_t max_context_len,
                   int32_t to_original_basis, int32_t out_dtype, void* k_out, void* v_out,
                   void* stream) {
  int rc = check_layout(L, true);
  if (rc != TQ_OK) return rc;
  if (batch < 0 || max_context_len < 0 || max_pages_per_seq < 0) return TQ_EINVAL;
  if ((int64_t)max_context_len > 16LL * max_pages_per_seq) return TQ_EINVAL;
  if (out_dtype != TQ_F32 && out_dtype != TQ_F16) return TQ_EINVAL;
  if (to_original_basis != 0 && to_original_basis != 1) return TQ_EINVAL;
  if ((int64_t)batch * max_context_len == 0) return TQ_OK;
  if (!pool || !block_table || !context_lens || !k_out || !v_out) return TQ_EINVAL;
  // one workgroup per (sequence, kv head, 4 pages), in a one-dimensional grid
  if ((int64_t)batch * L->num_kv_heads * (((int64_t)max_context_len + 63) / 64) > INT32_MAX) return TQ_EUNSUPPORTED;
  if (validating()) {
    rc = validate_tables(L, batch, block_table, max_pages_per_seq, context_lens, max_context_len,
                         nullptr, 0, static_cast<hipStream_t>(stream));
    if (rc != TQ_OK) return rc;
  }
  LaunchDequant a{static_cast<const uint8_t*>(pool), block_table, context_lens, L->sign_bits,
                  k_out, v_out, L->head_dim, L->num_kv_heads, batch, max_pages_per_seq,
                  max_context_len, to_original_basis, out_dtype, L->k_codec, L->v_codec};
  return from_hip(tq_launch_dequant(a, static_cast<hipStream_t>(stream)));
}

int tq_dense_decode_attn(const tq_layout* L, const void* k, const void* v, const void* q,
                         int32_t q_dtype, int32_t batch, const int32_t* context_lens,
                         int32_t max_context_len, float attn_scale, int32_t num_splits, float* out,
                         void* workspace, size_t workspace_bytes_, void* stream) {
  int rc = check_layout(L, false);
  if (rc != TQ_OK) return rc;
  rc = check_decode_common(L, q, q_dtype, batch, context_lens, max_context_len, attn_scale,
                           num_splits, out);
  if (rc != TQ_OK) return rc;
  if (batch == 0) return TQ_OK;
  if (!k || !v) return TQ_EINVAL;
  Split s = choose_split_dense(batch, L->num_kv_heads, max_context_len, num_splits);
  if ((int64_t)s.splits * L->num_kv_heads * batch > INT32_MAX) return TQ_EUNSUPPORTED;  // 1-D grid
  if (workspace_bytes_ < workspace_bytes(L, batch, max_context_len, num_splits)) return TQ_ENOSPC;
  if (!workspace) return TQ_EINVAL;
  float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + TQ_DECODE_COUNTER_BYTES);
  LaunchDecode a{};
  a.pool = static_cast<const uint8_t*>(k);
  a.dense_v = v;
  a.q = q;
  a.context_lens = context_lens;
  a.out = out;
  a.part_o = ws;
  a.part_ml = ws + (size_t)batch * L->num_q_heads * s.splits * L->head_dim;
  a.D = L->head_dim; a.Hq = L->num_q_heads; a.Hkv = L->num_kv_heads; a.B = batch;
  a.max_ctx = max_context_len;
  a.q_dtype = q_dtype;
  a.splits = s.splits; a.pages_per_split = s.pages_per_split;
  a.attn_scale = attn_scale;
  return from_hip(tq_launch_dense_decode(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
