/*
 * tq.h -- C ABI of the MI355X (gfx950) int4 compressed-domain decode-attention library.
 *
 * What the library computes (sources are web pages, cited by title and section):
 *  - On append, every key and value vector is rotated with a sign-randomized
 *    Walsh-Hadamard transform, quantized to 4 bits per group of 32 coordinates with an
 *    fp16 scale per group, and nibble-packed into a paged pool [Open-TQ-Metal, card
 *    abstract: rotation + per-group abs-max + int4 nibble pack in one fused kernel;
 *    "TurboQuant on AMD GPUs", section 4: Walsh-Hadamard rotation].
 *  - Keys may instead use a 16-entry Gaussian Lloyd-Max table times the group's L2 norm,
 *    values uniform abs-max ["TurboQuant on AMD GPUs", section 2, TQ4/4].
 *  - Or keys stay in fp16 and only values take the 4-bit rotated form: the asymmetric
 *    mode the mlxcel "TurboQuant KV cache" manual recommends by default (cache-mode table,
 *    fp16+turbo4). Keys are then stored unrotated and scored against the query as given.
 *  - Values may also take 3 or 2 bits (the same rotation, abs-max with fewer levels): the
 *    manual's fp16+turbo3 mode is fp16 keys with 3-bit values; "TurboQuant on AMD GPUs",
 *    section 2, notes that 2 bits are possible.
 *  - Decode attention runs directly on the packed codes: the query is rotated into the
 *    cache basis, scores and the weighted value sum are computed from codes and scales,
 *    the softmax is online, and no dequantized K/V matrix is written [Open-TQ-Metal, arXiv
 *    abstract]. A split over the context is merged in a second pass [online softmax
 *    normalizer, cited among Open-TQ-Metal's references].
 *  - The dequantize reference writes dense K/V, the "dequantize-then-attend" baseline the
 *    arXiv abstract compares against; a dense fp16 decode attention completes it.
 *
 * Numerics (fixed so that codes are reproducible bit for bit):
 *  - R = rho * H * diag(sigma), H the natural-order Sylvester Hadamard matrix
 *    (H_ij = (-1)^popcount(i & j)), sigma_i = -1 iff bit i of sign_bits is set,
 *    rho = fp32(1/sqrt(D)). fp32 butterfly with strides 1, 2, ..., D/2, then times rho.
 *  - abs-max: s = fp16_rne(max|y|/7) (saturating at 65504); c = clamp(rint(y/s), -7, 7)
 *    (c = 0 when s = 0); the stored 4-bit index is u = c + 8. Value = (u - 8) * s.
 *  - Lloyd-Max (keys only): LUT_j = fp16_rne(m_j / sqrt(32)), m_j the 16 Lloyd-Max levels
 *    of N(0,1) in increasing order; n = fp16_rne(sqrtf(sum of squares)) summed by the tree
 *    t_i += t_{i+off}, off = 16, 8, 4, 2, 1; u = #{j in 1..15 : y/n >= (LUT_{j-1}+LUT_j)/2},
 *    u = 8 when n = 0. Value = LUT_u * n.
 *  - fp16 keys: k16 = fp16_rne(k) of the original key (saturating at 65504), no rotation.
 *  - 3-bit and 2-bit values (v_codec TQ_CODEC_ABSMAX3, TQ_CODEC_ABSMAX2): abs-max with the
 *    largest level Q = 3 or 1 in place of 7: s = fp16_rne(max|y|/Q), c = clamp(rint(y/s),
 *    -Q, Q), stored index u = c + Q + 1. Value = (u - Q - 1) * s.
 *
 * Pool format. A pool is one device buffer of num_pages * num_kv_heads * TQ_BLOCK_BYTES(D)
 * bytes, [page][kv head][block]. A block holds 16 tokens of one KV head (G = D/32):
 *     [K indices: 8*D B][V indices: 8*D B][K scales: 16*G fp16][V scales: 16*G fp16]
 * Two 4-bit indices share a byte, the first in the low nibble.
 *     K index of token t, dim d = 32g + 8j + e  ->  byte (16j + t)*4G + 4g + e/2, nibble e%2
 *     V index of token t = 4j + e, dim d, c = d/2 = 16g + m
 *                                            ->  byte 8D + (16j + m)*4G + 4g + e, nibble d%2
 *     scale of token t, group g              ->  element t*G + g of its scale array
 * These orders let one 64-lane wavefront load a block's K (or V) indices with one 16-byte
 * load per lane, already in the operand order of the gfx950 matrix-core instructions.
 * With fp16 keys (k_codec TQ_CODEC_FP16) a block is TQ_BLOCK_BYTES_KF16(D) bytes:
 *     [K fp16: 32*D B][V indices: 8*D B][V scales: 16*G fp16]
 *     K of token t, dim d = 32g + 8j + e     ->  byte 1024g + 16(16j + t) + 2e
 *     V indices and scales as above, their regions starting at 32*D and 40*D
 * (each group's 16 tokens x 32 dims are one 1 KB run, again one 16-byte load per lane).
 * With b-bit values (b = 3 or 2) the V index region takes 2*b*D bytes instead of 8*D and
 * the scale regions follow it (block bytes: TQ_BLOCK_BYTES_KV). Its dwords are derived
 * from the 4-bit V region's, read as 64 rows of G little-endian dwords (row 16j + m,
 * dword g = the indices of dim pair m of group g of tokens 4j..4j+3, byte e = token
 * 4j + e, low nibble the even dim): the two low bits of each nibble of dwords g = 2i and
 * 2i + 1 of row l form X dword l*G/2 + i (dword 2i in bits 0-1 of every nibble, 2i + 1 in
 * bits 2-3); for b = 3 the third bits follow as 16*G Z dwords, bit 2 of each nibble of
 * dword g of row l going to bit (l*G + g) % 4 of that nibble in Z dword (l*G + g) / 4.
 * Every byte then holds bits of one token only.
 * A slot is page * 16 + offset within the page.
 *
 * Conventions.
 *  - Every buffer is allocated and owned by the caller; device pointers unless stated.
 *    The library allocates nothing and keeps no mutable global state.
 *  - Calls are asynchronous on the caller's stream (hipStream_t passed as void*, NULL =
 *    default stream) and never synchronize.
 *  - Arguments are checked on the host before any device work; failures return a
 *    negative tq_status and launch nothing. A launch failure returns TQ_EDEVICE. Device
 *    contents (slots, block tables, context lengths) are preconditions, not checked:
 *    out-of-range values there are undefined behaviour, unless the environment variable
 *    TQ_VALIDATE is 1. Then each call synchronizes its stream, copies these arrays to
 *    the host and returns TQ_EINVAL, launching nothing, for page ids a sequence uses
 *    outside [0, num_pages), lengths outside [0, max_context_len], tail lengths above
 *    hot_cap, and slots outside the pool or given twice (a debugging aid: it costs a
 *    synchronization and host copies per call).
 *  - GPU support: head_dim in {64, 128, 256}, group_size 32, page_size 16,
 *    1 <= num_q_heads / num_kv_heads <= 8, batch * num_kv_heads <= 2^20, appends with
 *    num_kv_heads <= 65535; decode with fp16 keys at head_dim 256 with
 *    num_q_heads / num_kv_heads <= 4; sparse values with batch * num_kv_heads <= 2^16
 *    (TQ_EUNSUPPORTED otherwise).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,        /* malformed argument: null pointer, negative size, bad enum */
  TQ_EUNSUPPORTED = -2,  /* well-formed but outside what the GPU kernels implement */
  TQ_ENOSPC = -3,        /* caller-provided workspace too small */
  TQ_EDEVICE = -4        /* the HIP runtime reported an error */
} tq_status;

typedef enum {
  TQ_CODEC_ABSMAX = 0,    /* 4-bit abs-max (keys or values) */
  TQ_CODEC_LLOYDMAX = 1,  /* 4-bit Lloyd-Max table times the group norm (keys) */
  TQ_CODEC_FP16 = 2,      /* fp16, not rotated (keys) */
  TQ_CODEC_ABSMAX3 = 3,   /* 3-bit abs-max (values) */
  TQ_CODEC_ABSMAX2 = 4    /* 2-bit abs-max (values) */
} tq_codec;
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

#define TQ_BLOCK_BYTES(D) (16 * (D) + 64 * ((D) / 32))
#define TQ_BLOCK_BYTES_KF16(D) (41 * (D))
/* any (k_codec, v_codec): keys 8*D (4-bit) or 32*D (fp16), values 2*b*D, scales D or 2*D */
#define TQ_VALUE_BITS(VC) ((VC) == TQ_CODEC_ABSMAX3 ? 3 : ((VC) == TQ_CODEC_ABSMAX2 ? 2 : 4))
#define TQ_BLOCK_BYTES_KV(D, KC, VC)                                                  \
  (((KC) == TQ_CODEC_FP16 ? 33 * (D) : 10 * (D)) + 2 * TQ_VALUE_BITS(VC) * (D))

/* The first TQ_DECODE_COUNTER_BYTES bytes of a decode workspace hold per-(sequence,
 * kv head) arrival counters. They must be zero before the workspace is first used; every
 * tq_decode_attn call that completes leaves them zero again. A call whose kernel did not
 * complete (a launch error, a device fault, a stream torn down mid-flight) can leave them
 * non-zero, and later calls on that workspace would then merge at the wrong time and return
 * wrong results without an error: clear the first TQ_DECODE_COUNTER_BYTES bytes again (or
 * take a fresh zeroed workspace) after any failed call. How a split is published: its
 * partial results are stored with device-coherent stores, the workgroup waits until the
 * stores are complete, and only then increments the counter (a relaxed atomic); the
 * workgroup that sees the final count reads the partials with device-coherent loads. */
#define TQ_DECODE_COUNTER_BYTES ((size_t)4 << 20)

typedef struct {
  int32_t head_dim;          /* D: a power of two; 64, 128 or 256 on the GPU */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv; Hq % Hkv == 0; q head hq uses kv head hq / (Hq/Hkv) */
  int32_t group_size;        /* quantization group, must be 32 */
  int32_t page_size;         /* tokens per page, must be 16 */
  int32_t num_pages;         /* physical pages in the pool */
  int32_t k_codec;           /* tq_codec for keys: ABSMAX, LLOYDMAX or FP16 */
  int32_t v_codec;           /* tq_codec for values: ABSMAX, ABSMAX3 or ABSMAX2 */
  const uint32_t* sign_bits; /* device, D/32 words; bit i of word i/32 set => sigma_i = -1 */
} tq_layout;

/* Human-readable name of a tq_status (static string, never NULL). */
const char* tq_status_str(int status);

/* Bytes of one physical page of the pool (all KV heads):
 * num_kv_heads * TQ_BLOCK_BYTES_KV(D, k_codec, v_codec). Returns 0 for an invalid layout. */
size_t tq_page_bytes(const tq_layout* layout);

/* Append: rotate, quantize and store n_tokens new K and V vectors.
 *   pool          device, the layout's pool (written at the given slots only)
 *   k, v          device, [n_tokens][num_kv_heads][head_dim] of in_dtype, row-major
 *   slot_mapping  device int64 [n_tokens]: page * 16 + offset; a negative slot skips
 *                 the token. Two tokens of one call must not share a slot.
 * Writes exactly the indices and scales of the given slots; other bytes are untouched.
 * [Open-TQ-Metal, card abstract: the fused quantize kernel] */
int tq_kv_append(const tq_layout* layout, void* pool, const void* k, const void* v,
                 int32_t in_dtype, int32_t n_tokens, const int64_t* slot_mapping, void* stream);

/* Workspace bytes tq_decode_attn needs for this batch and maximum context length:
 * TQ_DECODE_COUNTER_BYTES of counters, the split partials (batch * num_q_heads * splits
 * * (head_dim + 2) floats) and the workgroup order (batch * num_kv_heads int32).
 * num_splits: 0 picks the split count automatically (as tq_decode_attn does); > 0 asks
 * for that many splits of the context (clamped to the number of pages). Returns 0 for
 * invalid arguments. */
size_t tq_decode_workspace_size(const tq_layout* layout, int32_t batch, int32_t max_context_len,
                                int32_t num_splits);

/* Decode attention on the compressed cache, one query per sequence.
 *   q               device, [batch][num_q_heads][head_dim] of q_dtype (original basis)
 *   block_table     device int32 [batch][max_pages_per_seq]: physical page of each
 *                   16-token page of each sequence
 *   context_lens    device int32 [batch]: tokens to attend (0 gives a zero output);
 *                   each <= max_context_len <= 16 * max_pages_per_seq
 *   max_context_len host, an upper bound of context_lens (sizes the launch); when it is
 *                   0, pool and block_table are not read and may be NULL
 *   attn_scale      softmax scale alpha (scores are alpha * q.k)
 *   num_splits      0 = automatic; > 0 forces that many context splits, at most 128
 *                   (results agree across split counts up to rounding)
 *   out             device fp32 [batch][num_q_heads][head_dim], original basis
 *   workspace       device scratch of >= tq_decode_workspace_size(...) bytes (TQ_ENOSPC
 *                   otherwise). Its first TQ_DECODE_COUNTER_BYTES must be zero before the
 *                   first call (a zero-filled allocation); the rest is overwritten freely.
 *                   Two calls that run at the same time must not share a workspace.
 * When the grid is larger than the GPU holds at once (batch * num_kv_heads * splits above
 * the compute-unit count) and batch <= 256, a one-workgroup kernel first ranks the
 * sequences by context_lens and the decode workgroups take them longest first.
 * [Open-TQ-Metal, arXiv abstract: attention directly on the compressed representation] */
int tq_decode_attn(const tq_layout* layout, const void* pool, const void* q, int32_t q_dtype,
                   int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                   const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                   int32_t num_splits, float* out, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Device scratch of tq_decode_attn_noalloc, per GPU, held until the process ends. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* tq_decode_attn without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. It calls no allocating routine; its workspace is the library's own static
 * device array of TQ_NOALLOC_SCRATCH_BYTES bytes on the current device (one per GPU,
 * found on the first call on that device). Arguments, results and errors as
 * tq_decode_attn, except:
 *   - a call whose workspace (tq_decode_workspace_size(layout, batch, max_context_len,
 *     num_splits)) exceeds TQ_NOALLOC_SCRATCH_BYTES returns TQ_ENOSPC before any launch;
 *   - the arrival counters of the array are cleared by a fill kernel on `stream` at the
 *     start of every call, so a call never depends on what an earlier one left there;
 *   - calls that overlap on one GPU (on different streams, or from different threads)
 *     share the array and race: the caller serializes them;
 *   - TQ_VALIDATE does not apply (its checks synchronize and copy to host memory);
 *   - TQ_EDEVICE if the device or the array's address cannot be obtained. */
int tq_decode_attn_noalloc(const tq_layout* layout, const void* pool, const void* q, int32_t q_dtype,
                           int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                           const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                           int32_t num_splits, float* out, void* stream);

/* Append the newest token of every sequence, then decode: the same result as
 *   tq_kv_append(k_last, v_last, slots = position context_lens[b] - 1 of each sequence)
 *   followed by tq_decode_attn(...), in one decode launch. The token of sequence b is the last one
 *   it attends to (position context_lens[b] - 1, in the page block_table[b][(len - 1) / 16]);
 *   sequences with context_lens[b] == 0 append nothing.
 *   pool            device, written at those slots (and read as in tq_decode_attn)
 *   k_last, v_last  device, [batch][num_kv_heads][head_dim] of in_dtype (TQ_F32, TQ_BF16,
 *                   TQ_F16), row-major
 *   other arguments, workspace and errors as tq_decode_attn.
 * The decode of a step reads that page anyway: the new token is quantized by the same
 * kernel and used from on-chip memory, which saves the separate append launch.
 * [Open-TQ-Metal, card abstract: quantize on append; arXiv abstract: attention directly on
 *  the compressed representation] */
int tq_append_decode_attn(const tq_layout* layout, void* pool, const void* k_last,
                          const void* v_last, int32_t in_dtype, const void* q, int32_t q_dtype,
                          int32_t batch, const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float attn_scale,
                          int32_t num_splits, float* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Decode attention with sparse values: as tq_decode_attn, except that the values of a
 * 16-token page (of one kv head) are neither loaded nor used when every weight of it, for
 * every q head of the kv head, is below v_threshold (mlxcel "TurboQuant KV cache" manual,
 * sparse-V threshold: value dequantization is skipped where the attention weight is below
 * it, 1e-6 by default). Each context split first reads the keys of all its pages, then
 * the keys and values of the pages it keeps. The weight compared is exp(score - M), M the
 * largest score the (sequence, kv head) has shown so far: the split's own largest, raised
 * to the largest that the splits done with their keys before it have published (an atomic
 * maximum in the workspace's counter area, cleared again by the split that merges). M never
 * exceeds the final maximum, so exp(score - M) bounds the token's final softmax weight from
 * above, and the result differs from tq_decode_attn only by dropped terms w_t * v_t with
 * every w_t < v_threshold (the softmax normalizer still counts every token). Which pages
 * are dropped depends on the split count and on the order in which splits finish their
 * keys; v_threshold = 0 drops none and is tq_decode_attn, bit for bit. Keys are read twice
 * for kept pages: this pays where attention is peaky. Any value width (4, 3, 2 bits). The
 * split count is at least the context's pages / (32 * waves per workgroup), which
 * tq_decode_workspace_size includes.
 *   v_threshold     in [0, 1), TQ_EINVAL otherwise
 *   v_pages_skipped optional device uint64: the number of (page, kv head) value blocks
 *                   skipped is added to it (NULL: not counted)
 *   other arguments, workspace and errors as tq_decode_attn.
 * [mlxcel manual, sparse-V dequant threshold; Open-TQ-Metal, arXiv abstract] */
int tq_decode_attn_sparse_v(const tq_layout* layout, const void* pool, const void* q,
                            int32_t q_dtype, int32_t batch, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float attn_scale, float v_threshold,
                            int32_t num_splits, float* out, void* workspace,
                            size_t workspace_bytes, unsigned long long* v_pages_skipped,
                            void* stream);

/* Sparse values with the newest token appended in the same launch: the same result as
 *   tq_kv_append(k_last, v_last, slots = position context_lens[b] - 1 of each sequence)
 *   followed by tq_decode_attn_sparse_v(...), as tq_append_decode_attn is to tq_decode_attn.
 * Both passes of the split that holds a sequence's last page use the new token from on-chip
 * memory: its key in the first (so its score counts in the page's maximum and in the
 * normalizer), its key and value in the second if the page is kept. Which pages are dropped
 * follows tq_decode_attn_sparse_v; v_threshold = 0 drops none and is tq_append_decode_attn,
 * bit for bit.
 *   pool, k_last, v_last, in_dtype   as tq_append_decode_attn
 *   v_threshold, v_pages_skipped     as tq_decode_attn_sparse_v
 *   other arguments, workspace and errors as tq_decode_attn_sparse_v.
 * [mlxcel manual, sparse-V threshold; Open-TQ-Metal, card abstract: quantize on append] */
int tq_append_decode_attn_sparse_v(const tq_layout* layout, void* pool, const void* k_last,
                                   const void* v_last, int32_t in_dtype, const void* q,
                                   int32_t q_dtype, int32_t batch, const int32_t* block_table,
                                   int32_t max_pages_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, float attn_scale, float v_threshold,
                                   int32_t num_splits, float* out, void* workspace,
                                   size_t workspace_bytes, unsigned long long* v_pages_skipped,
                                   void* stream);

/* Decode attention over a hot/cold cache: the packed pool holds each sequence's older
 * tokens and an fp16 tail its most recent ones [mlxcel "TurboQuant KV cache" manual,
 * delegated cache: recent tokens in fp16, older ones in the 4-bit form]. Sequence b attends
 * to its cold_lens[b] pool tokens and then to its hot_lens[b] tail tokens, one softmax over
 * both. Each split of the pool also takes an equal slice of the tail and joins it to its
 * partial, so the tail adds no workgroups and its work is spread over the splits; with
 * num_splits = 0 and few enough (sequence, kv head) pairs that the grid has room (at least
 * 8 splits per pair for every 512 tokens of hot_cap), workgroups of their own take the tail
 * instead, one per 512 tokens of hot_cap (at least two with 16 splits or more), beside the
 * pool's splits.
 *   cold_lens       device int32 [batch], as context_lens of tq_decode_attn (may be 0)
 *   max_cold_len    host, an upper bound of cold_lens
 *   hot_k, hot_v    device fp16 [batch][num_kv_heads][hot_cap][head_dim], original basis
 *                   (not rotated); rows >= hot_lens[b] are not read
 *   hot_lens        device int32 [batch], 0 <= hot_lens[b] <= hot_cap
 *   hot_cap         1..1024 (TQ_EUNSUPPORTED otherwise)
 *   other arguments, workspace (tq_decode_workspace_size(layout, batch, max_cold_len,
 *   num_splits)) and errors as tq_decode_attn. A sequence with no tokens at all gets zeros.
 * The caller writes new tokens into the tail as plain fp16 (nothing to quantize) and folds
 * the oldest tail tokens into the pool with tq_kv_append when the tail is full. */
int tq_decode_attn_hotcold(const tq_layout* layout, const void* pool, const void* q,
                           int32_t q_dtype, int32_t batch, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* cold_lens,
                           int32_t max_cold_len, const void* hot_k, const void* hot_v,
                           const int32_t* hot_lens, int32_t hot_cap, float attn_scale,
                           int32_t num_splits, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Dequantize reference: dense K and V, [batch][num_kv_heads][max_context_len][head_dim]
 * of out_dtype (TQ_F32 or TQ_F16), rows at or past a sequence's length set to zero.
 * to_original_basis = 0: values (u-8)*s or LUT_u*n in the rotated basis (exact products,
 * rounded once to out_dtype); 1: times R^-1 = diag(sigma) * rho * H in fp32 (same stage
 * order as the forward rotation), then rounded to out_dtype. fp16 keys have no rotated
 * form: they are written as stored in both cases. TQ_EUNSUPPORTED when batch *
 * num_kv_heads * ceil(max_context_len / 64) (its workgroups) exceeds 2^31 - 1.
 * [Open-TQ-Metal, arXiv abstract: the dequantize-then-attend baseline] */
int tq_dequant_ref(const tq_layout* layout, const void* pool, int32_t batch,
                   const int32_t* block_table, int32_t max_pages_per_seq,
                   const int32_t* context_lens, int32_t max_context_len, int32_t to_original_basis,
                   int32_t out_dtype, void* k_out, void* v_out, void* stream);

/* Dense fp16 decode attention, the "attend" half of the baseline: K and V are fp16
 * [batch][num_kv_heads][max_context_len][head_dim] (e.g. tq_dequant_ref output in the
 * original basis), q as in tq_decode_attn but used unrotated; fp32 accumulation, same
 * split/merge scheme; out fp32 [batch][num_q_heads][head_dim]. Workspace as for
 * tq_decode_attn. Only head_dim, num_q_heads, num_kv_heads of the layout are used.
 * TQ_EUNSUPPORTED when splits * num_kv_heads * batch (its workgroups) exceeds 2^31 - 1.
 * [Open-TQ-Metal, arXiv abstract: dequantize-then-attend] */
int tq_dense_decode_attn(const tq_layout* layout, const void* k, const void* v, const void* q,
                         int32_t q_dtype, int32_t batch, const int32_t* context_lens,
                         int32_t max_context_len, float attn_scale, int32_t num_splits,
                         float* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
