"""Seeded synthetic workloads for int4 compressed-domain decode attention.

This module only draws random inputs (keys, values, queries, sign vectors, page tables,
context lengths). It holds none of the method's arithmetic, so both the GPU path and the
CPU oracle can take their inputs from it. Every array comes from numpy's PCG64
(``default_rng``) with a seed derived from (seed, purpose, sequence), so a sequence's
tokens do not depend on how the caller chunks the generation.

The workloads, named by what they are:

  single_head_1k     1 head, D=128, 1024 cached tokens, fp32, N(0,1) with 4 outlier
                     channels x20 on K and V (q not scaled)
  llama8b_b16_8k     32 q / 8 kv heads, D=128, batch 16, context 8192, bf16,
                     N(0,1) x per-(kv head, channel) lognormal(0,1) scales
  llama70b_b1_128k   64 q / 8 kv heads, D=128, batch 1, context 131072, bf16, as above
                     plus 1% of tokens (all heads) x10
  gemma_d256_32k     16 q / 8 kv heads, D=256, batch 4, context 32768, bf16, as the
                     previous one, attention scale 1.0
  mixed_serving      prefill chunk of 2048 tokens appended to 128 fresh pages, then a
                     decode batch of 64 with contexts uniform in [1024, 32768]; 32 q / 8 kv
                     heads, D=128, keys by the LUT codec, values by abs-max
  llama70b_b1_128k_k16v4
                     the 128K workload with keys kept in fp16 and values in 4 bits (the
                     asymmetric mode); _k16v3 with 3-bit values, _k4v2 with 4-bit keys and
                     2-bit values
  gemma_d256_32k_k16v4
                     the D=256 workload with fp16 keys and 4-bit values

Each step of a workload appends one new token per decoding sequence (its last token;
the other L_b - 1 tokens are the resident cache) plus, for mixed_serving, the 2048-token
prefill chunk, and then decodes one query per sequence over all L_b tokens.
"""
import math
from dataclasses import dataclass, field, replace

import numpy as np

PAGE = 16

CODEC_ABSMAX = 0
CODEC_LUT = 1
CODEC_FP16 = 2   # keys only: kept in fp16 (values stay 4-bit)
CODEC_ABSMAX3 = 3  # values only: 3-bit abs-max
CODEC_ABSMAX2 = 4  # values only: 2-bit abs-max
VALUE_BITS = {CODEC_ABSMAX: 4, CODEC_ABSMAX3: 3, CODEC_ABSMAX2: 2}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    context: int                 # every sequence's length, or the upper bound if ragged
    dtype: str                   # "f32" or "bf16" (storage type of k, v, q)
    attn_scale: float
    k_codec: int = CODEC_ABSMAX
    v_codec: int = CODEC_ABSMAX
    dist: str = "lognormal"      # "outlier", "lognormal", "lognormal_spikes"
    ragged_min: int = 0          # > 0: contexts uniform in [ragged_min, context]
    prefill: int = 0             # extra prefill tokens appended in each step
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def gqa(self):
        return self.q_heads // self.kv_heads

    def scaled(self, context, batch=None, ragged_min=None, prefill=None, name=None):
        """Same distribution and head layout at a smaller size (for oracle-speed tests)."""
        return replace(self, name=name or (self.name + "_small"), context=context,
                       batch=self.batch if batch is None else batch,
                       ragged_min=(min(self.ragged_min, context) if ragged_min is None else ragged_min),
                       prefill=self.prefill if prefill is None else prefill)


WORKLOADS = {
    "single_head_1k": Workload("single_head_1k", 1, 1, 1, 128, 1024, "f32",
                               1.0 / math.sqrt(128), dist="outlier"),
    "llama8b_b16_8k": Workload("llama8b_b16_8k", 16, 32, 8, 128, 8192, "bf16",
                               1.0 / math.sqrt(128)),
    "llama70b_b1_128k": Workload("llama70b_b1_128k", 1, 64, 8, 128, 131072, "bf16",
                                 1.0 / math.sqrt(128), dist="lognormal_spikes"),
    "gemma_d256_32k": Workload("gemma_d256_32k", 4, 16, 8, 256, 32768, "bf16", 1.0,
                               dist="lognormal_spikes"),
    "mixed_serving": Workload("mixed_serving", 64, 32, 8, 128, 32768, "bf16",
                              1.0 / math.sqrt(128), k_codec=CODEC_LUT, ragged_min=1024,
                              prefill=2048),
    "llama70b_b1_128k_k16v4": Workload("llama70b_b1_128k_k16v4", 1, 64, 8, 128, 131072, "bf16",
                                       1.0 / math.sqrt(128), k_codec=CODEC_FP16,
                                       dist="lognormal_spikes"),
    # fp16 keys + 3-bit values (the mlxcel manual's fp16+turbo3 mode)
    "llama70b_b1_128k_k16v3": Workload("llama70b_b1_128k_k16v3", 1, 64, 8, 128, 131072, "bf16",
                                       1.0 / math.sqrt(128), k_codec=CODEC_FP16,
                                       v_codec=CODEC_ABSMAX3, dist="lognormal_spikes"),
    # the D = 256 workload with fp16 keys and 4-bit values (the manual's recommended mode)
    "gemma_d256_32k_k16v4": Workload("gemma_d256_32k_k16v4", 4, 16, 8, 256, 32768, "bf16", 1.0,
                                     k_codec=CODEC_FP16, dist="lognormal_spikes"),
    # 4-bit keys + 2-bit values
    "llama70b_b1_128k_k4v2": Workload("llama70b_b1_128k_k4v2", 1, 64, 8, 128, 131072, "bf16",
                                      1.0 / math.sqrt(128), v_codec=CODEC_ABSMAX2,
                                      dist="lognormal_spikes"),
}

HEADLINE = "llama70b_b1_128k"


def _rng(seed, *keys):
    return np.random.default_rng([seed, *keys])


def bf16_round(x):
    """fp32 -> nearest bf16 (ties to even), returned as (uint16 bits, fp32 values)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    return r, (r.astype(np.uint32) << np.uint32(16)).view(np.float32)


def sign_bits(D, seed=0):
    """D/32 packed words; bit i set means coordinate i is negated."""
    bits = _rng(seed, 1).integers(0, 2, size=D, dtype=np.uint32)
    words = np.zeros(max(1, D // 32), np.uint32)
    for i in range(D):
        words[i // 32] |= np.uint32(bits[i]) << np.uint32(i % 32)
    return words


def context_lens(w: Workload, seed=0):
    if w.ragged_min > 0:
        return _rng(seed, 2).integers(w.ragged_min, w.context, size=w.batch,
                                      endpoint=True).astype(np.int32)
    return np.full(w.batch, w.context, np.int32)


def channel_scales(w: Workload, seed=0):
    """Per-(kv head, channel) multipliers for K and for V ([Hkv, D] each), or outlier mask."""
    if w.dist == "outlier":
        ch = _rng(seed, 3).choice(w.head_dim, 4, replace=False)
        s = np.ones((w.kv_heads, w.head_dim), np.float32)
        s[:, ch] = 20.0
        return s, s.copy()
    r = _rng(seed, 3)
    ks = r.lognormal(0.0, 1.0, size=(w.kv_heads, w.head_dim)).astype(np.float32)
    vs = r.lognormal(0.0, 1.0, size=(w.kv_heads, w.head_dim)).astype(np.float32)
    return ks, vs


def seq_tokens(w: Workload, b, L, seed=0, scales=None):
    """K, V of sequence b's first L tokens: fp32 [L, Hkv, D] values exactly representable
    in the storage type, plus the storage arrays (bf16 bits as uint16, or the fp32)."""
    ks, vs = channel_scales(w, seed) if scales is None else scales
    r = _rng(seed, 4, b)
    shape = (L, w.kv_heads, w.head_dim)
    k = r.standard_normal(shape, dtype=np.float32) * ks[None]
    v = r.standard_normal(shape, dtype=np.float32) * vs[None]
    if w.dist == "lognormal_spikes" and L > 0:
        n = int(round(0.01 * L))
        idx = r.choice(L, n, replace=False)
        k[idx] *= 10.0
        v[idx] *= 10.0
    if w.dtype == "bf16":
        kb, k = bf16_round(k)
        vb, v = bf16_round(v)
        return k, v, kb, vb
    return k, v, k, v


def prefill_tokens(w: Workload, seed=0, scales=None):
    """The prefill chunk's K, V (treated as a sequence of its own, index batch)."""
    return seq_tokens(w, w.batch, w.prefill, seed, scales)


def queries(w: Workload, seed=0):
    """fp32 [B, Hq, D] values and their storage array."""
    q = _rng(seed, 5).standard_normal((w.batch, w.q_heads, w.head_dim), dtype=np.float32)
    if w.dtype == "bf16":
        qb, q = bf16_round(q)
        return q, qb
    return q, q


def page_tables(w: Workload, lens, seed=0):
    """Seeded random permutation of the physical pages over all sequences (and the
    prefill chunk). Returns (block_table [B, max_pages] int32, prefill_pages int32,
    num_pages)."""
    npg = [-(-int(L) // PAGE) for L in lens]
    pre = -(-w.prefill // PAGE)
    total = sum(npg) + pre
    perm = _rng(seed, 6).permutation(total).astype(np.int32)
    maxp = max(max(npg), 1)
    bt = np.zeros((len(lens), maxp), np.int32)
    pos = 0
    for b, n in enumerate(npg):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt, perm[pos:pos + pre], total


def slots_for(bt, b, t0, t1):
    """slot = page*16 + offset for tokens t0..t1-1 of sequence b."""
    t = np.arange(t0, t1, dtype=np.int64)
    return bt[b, t // PAGE].astype(np.int64) * PAGE + t % PAGE


def kv_bytes_per_token(w: Workload):
    """Packed K+V bytes of one token over all kv heads: keys D/2 + 2*D/32 (fp16 keys: 2D),
    values b*D/8 + 2*D/32 for b-bit values, per kv head."""
    D = w.head_dim
    kbytes = 2 * D if w.k_codec == CODEC_FP16 else D // 2 + 2 * (D // 32)
    vbytes = VALUE_BITS[w.v_codec] * D // 8 + 2 * (D // 32)
    return w.kv_heads * (kbytes + vbytes)


def algorithmic_bytes(w: Workload, lens):
    """Packed K+V indices and fp16 scales read by one decode: sum_b L_b * Hkv * (keys:
    D/2 + 2*D/32, or 2D for fp16 keys; values: b*D/8 + 2*D/32 for b-bit values), plus the
    query and the fp32 output."""
    D = w.head_dim
    per_tok = kv_bytes_per_token(w)
    qbytes = w.batch * w.q_heads * D * (4 if w.dtype == "f32" else 2)
    return int(np.sum(lens, dtype=np.int64)) * per_tok + qbytes + w.batch * w.q_heads * D * 4
