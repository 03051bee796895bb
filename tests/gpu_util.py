"""Helpers for the GPU parity tests: run a workload through the C ABI and through the C
oracle on the same seeded inputs, and compare.

Codes and scales must match byte for byte; attention outputs must satisfy
max_i |o_i - o*_i| / max_i |o*_i| <= 2e-3 per (sequence, q head), with o* the oracle's
fp64 result (the normwise reading of "max relative error": elementwise relative error is
undefined near zero).
"""
import math

import numpy as np
import torch

from int4_compressed_domain_amd import tq
from int4_compressed_domain_amd import workloads as W
from oracle import c_oracle

ATTN_TOL = 2e-3
DEV = "cuda:0"


def to_dev(arr_storage, dtype):
    """numpy storage array (fp32 values, or bf16 bits as uint16) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr_storage).view(np.int16)).view(torch.bfloat16).to(DEV)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr_storage, np.float16)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr_storage, np.float32)).to(DEV)


def attn_err(gpu, ref):
    """Per-row normwise relative error, rows = (b, hq)."""
    g = np.asarray(gpu, np.float64).reshape(-1, gpu.shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    den = np.max(np.abs(r), axis=1)
    num = np.max(np.abs(g - r), axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


class Case:
    """One workload resident in a GPU pool and in an oracle pool."""

    def __init__(self, w, seed=0, q_dtype=None, oracle=True, lens=None, fill_last=True):
        self.w = w
        self.seed = seed
        D, Hkv = w.head_dim, w.kv_heads
        self.sb = W.sign_bits(D, seed)
        self.lens = W.context_lens(w, seed) if lens is None else np.asarray(lens, np.int32)
        self.bt, self.prefill_pages, self.npages = W.page_tables(w, self.lens, seed)
        self.sb_dev = torch.from_numpy(self.sb.view(np.int32)).to(DEV)
        self.layout = tq.make_layout(D, w.q_heads, Hkv, self.npages, self.sb_dev.data_ptr(),
                                     w.k_codec, w.v_codec)
        self.page_bytes = tq.tq_page_bytes(self.layout)
        assert self.page_bytes == Hkv * c_oracle.block_bytes(D, w.k_codec, w.v_codec)
        self.pool = torch.zeros(self.npages * self.page_bytes, dtype=torch.uint8, device=DEV)
        self.opool = c_oracle.new_pool(self.npages, Hkv, D, w.k_codec, w.v_codec) if oracle else None
        self.scales = W.channel_scales(w, seed)
        self.q_dtype = q_dtype or w.dtype
        q32, qst = W.queries(w, seed)
        if self.q_dtype == "f16":
            q16 = q32.astype(np.float16)
            self.q32, self.q_dev = q16.astype(np.float32), to_dev(q16, "f16")
        elif self.q_dtype == "f32" and w.dtype == "bf16":
            self.q32, self.q_dev = q32, to_dev(q32, "f32")
        else:
            self.q32, self.q_dev = q32, to_dev(qst, w.dtype)
        self.bt_dev = torch.from_numpy(self.bt).to(DEV)
        self.lens_dev = torch.from_numpy(self.lens).to(DEV)

    def append_seq(self, b, t0, t1, k=None, v=None):
        """Append tokens t0..t1-1 of sequence b on the GPU (and in the oracle pool)."""
        w = self.w
        if k is None:
            k32, v32, kst, vst = W.seq_tokens(w, b, t1, self.seed, self.scales)
            k32, v32, kst, vst = k32[t0:t1], v32[t0:t1], kst[t0:t1], vst[t0:t1]
        else:
            k32, v32, kst, vst = k, v, k, v
        slots = W.slots_for(self.bt, b, t0, t1)
        self.append_raw(k32, v32, kst, vst, slots)

    def append_raw(self, k32, v32, kst, vst, slots):
        w = self.w
        kd, vd = to_dev(kst, w.dtype), to_dev(vst, w.dtype)
        sd = torch.from_numpy(np.ascontiguousarray(slots, np.int64)).to(DEV)
        tq.tq_kv_append(self.layout, self.pool, kd, vd, sd)
        if self.opool is not None:
            c_oracle.append(self.opool, w.head_dim, w.kv_heads, k32, v32, slots, self.sb,
                            w.k_codec, w.v_codec)

    def fill(self, chunk=4096, keep_last=False):
        """Append every sequence's tokens; keep_last: all but the last, which are returned
        (the decode step's new tokens, [B][Hkv][D] fp32 values and storage, and slots)."""
        w = self.w
        last = None
        if keep_last:
            sdt = np.uint16 if w.dtype == "bf16" else np.float32
            last = dict(k32=np.zeros((w.batch, w.kv_heads, w.head_dim), np.float32),
                        kst=np.zeros((w.batch, w.kv_heads, w.head_dim), sdt),
                        slots=np.full(w.batch, -1, np.int64))
            last["v32"], last["vst"] = np.zeros_like(last["k32"]), np.zeros_like(last["kst"])
        for b in range(w.batch):
            L = int(self.lens[b])
            k32, v32, kst, vst = W.seq_tokens(w, b, L, self.seed, self.scales)
            n = L - 1 if keep_last and L > 0 else L
            for t0 in range(0, n, chunk):
                t1 = min(n, t0 + chunk)
                self.append_raw(k32[t0:t1], v32[t0:t1], kst[t0:t1], vst[t0:t1],
                                W.slots_for(self.bt, b, t0, t1))
            if keep_last and L > 0:
                last["k32"][b], last["v32"][b] = k32[L - 1], v32[L - 1]
                last["kst"][b], last["vst"][b] = kst[L - 1], vst[L - 1]
                last["slots"][b] = W.slots_for(self.bt, b, L - 1, L)[0]
        torch.cuda.synchronize()
        return last

    def append_decode_gpu(self, last, num_splits=0):
        """The benchmark's call: tq_append_decode_attn of the new tokens over the whole
        context (automatic split count unless given); the oracle pool gets the same tokens."""
        w = self.w
        maxc = int(self.lens.max())
        ws = torch.zeros(max(tq.tq_decode_workspace_size(self.layout, w.batch, maxc, num_splits), 4) // 4,
                         dtype=torch.float32, device=DEV)
        out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device=DEV)
        tq.tq_append_decode_attn(self.layout, self.pool, to_dev(last["kst"], w.dtype), to_dev(last["vst"], w.dtype),
                                 self.q_dev, self.bt_dev, self.lens_dev, maxc, w.attn_scale, out, ws,
                                 num_splits=num_splits)
        torch.cuda.synchronize()
        keep = last["slots"] >= 0
        if self.opool is not None:
            c_oracle.append(self.opool, w.head_dim, w.kv_heads, last["k32"][keep], last["v32"][keep],
                            last["slots"][keep], self.sb, w.k_codec, w.v_codec)
        return out.cpu().numpy()

    def pool_equal(self):
        return np.array_equal(self.pool.cpu().numpy(), self.opool)

    def decode_gpu(self, num_splits=0, max_ctx=None):
        w = self.w
        max_ctx = int(self.lens.max()) if max_ctx is None else max_ctx
        ws_bytes = tq.tq_decode_workspace_size(self.layout, w.batch, max_ctx, num_splits)
        ws = torch.zeros(max(ws_bytes, 4) // 4, dtype=torch.float32, device=DEV)
        out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device=DEV)
        tq.tq_decode_attn(self.layout, self.pool, self.q_dev, self.bt_dev, self.lens_dev, max_ctx,
                          w.attn_scale, out, ws, num_splits=num_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def decode_oracle(self, pairs=None):
        w = self.w
        return c_oracle.decode(self.opool, w.head_dim, w.q_heads, w.kv_heads, self.sb, self.bt,
                               self.lens, self.q32, w.attn_scale, pairs=pairs,
                               k_codec=w.k_codec, v_codec=w.v_codec)
