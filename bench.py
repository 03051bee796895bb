"""Benchmark: one decode step of int4 compressed-domain attention on one MI355X.

A step = the whole hot path over one batch: the prefill chunk of the mixed-serving
workload is appended to the packed pool (tq_kv_append), then one launch
(tq_append_decode_attn) rotates, quantizes and writes the new token of every decoding
sequence and decodes one query per sequence over its whole context, directly on the
packed codes.
Inputs are resident in HBM before the timed region. To measure HBM rather than the 256 MB
Infinity Cache, the step cycles through several identical copies of the pool (>= 1 GiB
in total), so each step reads a pool that was evicted since its last use.

Prints one JSON line. Metric: effective KV GB/s (algorithmic packed K+V bytes + q + out,
divided by the wall time of the step) and its fraction of the 8 TB/s HBM peak; decode
microseconds per token at 128K context; roofline of the decode kernel (HIP events on the
stream it runs on); the CPU oracle timed on the host; and the fp16
dequantize-then-attend GPU baseline on the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SPREAD_SAMPLES, SPREAD_LAUNCHES = 120, 32
METRIC = "effective KV GB/s (fraction of HBM peak) + decode attn µs/token at 128K ctx"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--splits", type=int, default=0, help="context splits (0 = automatic)")
    ap.add_argument("--min-pool-bytes", type=float, default=1.0 * 2 ** 30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baseline", action="store_true", help="skip the fp16 GPU baseline")
    ap.add_argument("--hot", type=int, default=0, metavar="N",
                    help="hot/cold cache: the last N tokens of each sequence in an fp16 tail, the "
                         "rest in the pool; the step is one tq_decode_attn_hotcold")
    ap.add_argument("--sparse-v", type=float, default=None, metavar="THR",
                    help="decode with sparse values at this weight threshold (the step is then the "
                         "new tokens' append + tq_decode_attn_sparse_v)")
    ap.add_argument("--cpu-oracle-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--profile", type=int, default=0,
                    help="run this many eager steps and exit: for profilers")
    ap.add_argument("--profile-append", type=int, default=0,
                    help="run this many appends of the prefill chunk (mixed_serving) alone and exit: "
                         "for profilers")
    return ap.parse_args()


def to_dev(arr, dtype, dev):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dev)


class Setup:
    """A workload resident on the GPU: filled pool (several copies), step inputs."""

    def __init__(self, w, args, dev):
        import torch
        from int4_compressed_domain_amd import tq
        from int4_compressed_domain_amd import workloads as W
        self.w = w
        D, Hkv = w.head_dim, w.kv_heads
        self.sb = W.sign_bits(D, 0)
        self.lens = W.context_lens(w, 0)
        self.bt, self.prefill_pages, self.npages = W.page_tables(w, self.lens, 0)
        self.sb_dev = torch.from_numpy(self.sb.view(np.int32)).to(dev)
        self.layout = tq.make_layout(D, w.q_heads, Hkv, self.npages, self.sb_dev.data_ptr(),
                                     w.k_codec, w.v_codec)
        pool_bytes = self.npages * tq.tq_page_bytes(self.layout)
        pool = torch.zeros(pool_bytes, dtype=torch.uint8, device=dev)
        scales = W.channel_scales(w, 0)
        self.scales = scales
        # resident cache: every token but the last of each sequence
        # newest token of each sequence, in its storage type (zeros for an empty sequence)
        sdt = np.uint16 if w.dtype == "bf16" else np.float32
        k_last = np.zeros((w.batch, Hkv, D), sdt)
        v_last = np.zeros((w.batch, Hkv, D), sdt)
        t_fill = time.time()
        self.hot = getattr(args, "hot", 0)
        if self.hot:  # hot/cold: the pool holds the first L - hot tokens, the tail the rest
            self.cold_lens = np.maximum(self.lens - self.hot, 0).astype(np.int32)
            self.hot_lens = (self.lens - self.cold_lens).astype(np.int32)
            hk = np.zeros((w.batch, Hkv, self.hot, D), np.float16)
            hv = np.zeros_like(hk)
        for b in range(w.batch):
            L = int(self.lens[b])
            k32, v32, kst, vst = W.seq_tokens(w, b, L, 0, scales)
            nres = int(self.cold_lens[b]) + 1 if self.hot else L   # tokens appended, plus one
            if self.hot:
                c0 = int(self.cold_lens[b])
                hk[b, :, :L - c0] = k32[c0:].transpose(1, 0, 2).astype(np.float16)
                hv[b, :, :L - c0] = v32[c0:].transpose(1, 0, 2).astype(np.float16)
            for t0 in range(0, nres - 1, 16384):
                t1 = min(nres - 1, t0 + 16384)
                tq.tq_kv_append(self.layout, pool, to_dev(kst[t0:t1], w.dtype, dev),
                                to_dev(vst[t0:t1], w.dtype, dev),
                                torch.from_numpy(W.slots_for(self.bt, b, t0, t1)).to(dev))
            if L > 0:
                k_last[b], v_last[b] = kst[L - 1], vst[L - 1]
        self.k_pre = None
        if w.prefill:
            _, _, kst, vst = W.prefill_tokens(w, 0, scales)
            pre = self.prefill_pages.astype(np.int64)
            t = np.arange(w.prefill)
            self.k_pre, self.v_pre = to_dev(kst, w.dtype, dev), to_dev(vst, w.dtype, dev)
            self.slots_pre = torch.from_numpy(pre[t // 16] * 16 + t % 16).to(dev)
            self.pre_stream = torch.cuda.Stream()  # default priority, like every stream here
        torch.cuda.synchronize()
        log("filled %s: %d pages, %.1f MB pool, %.1f s" % (w.name, self.npages, pool_bytes / 1e6,
                                                            time.time() - t_fill))
        self.n_new = int(np.count_nonzero(self.lens)) + w.prefill
        self.k_last = to_dev(k_last, w.dtype, dev)
        self.v_last = to_dev(v_last, w.dtype, dev)
        if self.hot:
            self.hk = torch.from_numpy(hk).to(dev)
            self.hv = torch.from_numpy(hv).to(dev)
            self.cold_dev = torch.from_numpy(self.cold_lens).to(dev)
            self.hot_dev = torch.from_numpy(self.hot_lens).to(dev)
            self.max_cold = int(self.cold_lens.max())
        last = np.array([W.slots_for(self.bt, b, int(L) - 1, int(L))[0] if L > 0 else -1
                         for b, L in enumerate(self.lens)], np.int64)
        self.slots_last = torch.from_numpy(last).to(dev)
        self.sparse_v = args.sparse_v
        self.v_skipped = torch.zeros(1, dtype=torch.int64, device=dev)
        ncopy = max(2, int(math.ceil(args.min_pool_bytes / max(pool_bytes, 1))))
        self.pools = [pool] + [pool.clone() for _ in range(ncopy - 1)]
        self.q32, qst = W.queries(w, 0)
        self.q = to_dev(qst, w.dtype, dev)
        self.bt_dev = torch.from_numpy(self.bt).to(dev)
        self.lens_dev = torch.from_numpy(self.lens).to(dev)
        self.max_ctx = int(self.lens.max())
        self.splits = args.splits
        ws = tq.tq_decode_workspace_size(self.layout, w.batch, self.max_ctx, self.splits)
        self.ws = torch.zeros(max(ws, 4) // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((w.batch, w.q_heads, D), dtype=torch.float32, device=dev)
        self.alg_bytes = W.algorithmic_bytes(w, self.lens)
        if self.hot:  # cold tokens packed, hot tokens fp16 K and V (4D bytes per token and head)
            self.alg_bytes = (W.algorithmic_bytes(w, self.cold_lens)
                              + int(np.sum(self.hot_lens, dtype=np.int64)) * Hkv * 4 * D)
        self.kv_bytes_all = W.algorithmic_bytes(w, self.lens) - W.algorithmic_bytes(w, 0 * self.lens)
        self.kv_bytes = int(np.sum(self.lens, dtype=np.int64)) * Hkv * 2 * (D // 2 + 2 * (D // 32))
        log("pool copies: %d (%.2f GB)" % (ncopy, ncopy * pool_bytes / 1e9))

    def prefill(self, i):
        """The prefill chunk's append (mixed serving only)."""
        from int4_compressed_domain_amd import tq
        if self.k_pre is not None:
            tq.tq_kv_append(self.layout, self.pools[i % len(self.pools)], self.k_pre, self.v_pre,
                            self.slots_pre)

    def decode(self, i):
        """One launch: append every decoding sequence's newest token, then attend (with
        sparse values too)."""
        from int4_compressed_domain_amd import tq
        pool = self.pools[i % len(self.pools)]
        if self.hot:
            tq.tq_decode_attn_hotcold(self.layout, pool, self.q, self.bt_dev, self.cold_dev,
                                      self.max_cold, self.hk, self.hv, self.hot_dev,
                                      self.w.attn_scale, self.out, self.ws, num_splits=self.splits)
            return
        if self.sparse_v is not None:
            tq.tq_append_decode_attn_sparse_v(self.layout, pool, self.k_last, self.v_last, self.q,
                                              self.bt_dev, self.lens_dev, self.max_ctx,
                                              self.w.attn_scale, self.sparse_v, self.out, self.ws,
                                              num_splits=self.splits, v_pages_skipped=self.v_skipped)
            return
        tq.tq_append_decode_attn(self.layout, pool, self.k_last, self.v_last, self.q, self.bt_dev,
                                 self.lens_dev, self.max_ctx, self.w.attn_scale, self.out, self.ws,
                                 num_splits=self.splits)

    def append_last(self, i):
        """tq_kv_append alone: every decoding sequence's newest token (as the fused call
        writes it, so the pool's contents do not change)."""
        from int4_compressed_domain_amd import tq
        tq.tq_kv_append(self.layout, self.pools[i % len(self.pools)], self.k_last, self.v_last,
                        self.slots_last)

    def step(self, i):
        """The prefill chunk's append and the decode. They touch different pages (the chunk
        fills fresh ones), so the append runs on a second stream beside the decode and can
        take the compute units the decode's shorter sequences leave idle."""
        import torch
        if self.k_pre is None:
            self.decode(i)
            return
        cur = torch.cuda.current_stream()
        self.pre_stream.wait_stream(cur)
        self.decode(i)  # first, so that its workgroups (one per CU) take the CUs first
        with torch.cuda.stream(self.pre_stream):
            self.prefill(i)
        cur.wait_stream(self.pre_stream)


def _graph(fn, n):
    """Capture n calls fn(i) into one HIP graph (on a side stream, as torch requires)."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def _time_replays(g, reps):
    """HIP events (on the replay stream) around reps replays; returns (event ms, wall s)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), time.perf_counter() - t0


def time_steps(S, steps, warmup):
    """Each step = (prefill append) + fused append/decode on the next pool copy. The steps
    of one pass over the copies are captured in a HIP graph; K = reps * copies steps are
    timed between synchronizations. A decode-only graph gives the fused kernel's mean
    time, a prefill-only graph the prefill append's (mixed serving)."""
    import torch
    n = len(S.pools)
    for i in range(warmup):
        S.step(i)
    torch.cuda.synchronize()
    eager = S.out.clone()
    graphs = [_graph(S.step, n), _graph(S.decode, n)]
    if S.k_pre is not None:
        graphs.append(_graph(S.prefill, n))
    reps = max(1, -(-steps // n))
    for g in graphs[:2]:
        g.replay()
        torch.cuda.synchronize()
        if S.sparse_v is None:
            same = torch.equal(S.out, eager)
        else:  # which value pages are skipped depends on the order the splits finish their
            # keys: the two runs drop different terms below the threshold (normwise check)
            diff = (S.out - eager).abs().amax(dim=2)
            same = bool((diff <= 2e-3 * eager.abs().amax(dim=2) + 1e-6).all())
        if not same:
            raise RuntimeError("graph replay output differs from the eager step")
    for g in graphs:  # untimed replays, ~0.3 s each: clocks ramp up and settle
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            for _ in range(20):
                g.replay()
            torch.cuda.synchronize()
    ev_ms, wall = _time_replays(graphs[0], reps)
    dec_ms, _ = _time_replays(graphs[1], reps)
    pre_ms = _time_replays(graphs[2], reps)[0] if len(graphs) > 2 else 0.0
    K = reps * n
    # spread: SPREAD_SAMPLES samples, each the mean per-launch time of one replay of a graph
    # of SPREAD_LAUNCHES back-to-back decodes (the pool copies in turn), timed by events on
    # the replay stream; the graph launch itself is spread over those launches
    g32 = _graph(S.decode, SPREAD_LAUNCHES)
    for _ in range(5):
        g32.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(SPREAD_SAMPLES):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g32.replay()
        e1.record()
        per.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in per]) / SPREAD_LAUNCHES * 1e3
    S.decode_pct = [round(float(x), 3) for x in np.percentile(us, [10, 50, 90])]
    # the one-token append alone (the fused call does it inside the decode)
    ga = _graph(S.append_last, n)
    for _ in range(20):
        ga.replay()
    torch.cuda.synchronize()
    S.append_one_us = _time_replays(ga, max(reps, 200 // n + 1))[0] / (max(reps, 200 // n + 1) * n) * 1e3
    return K, wall / K * 1e3, ev_ms / K, dec_ms / K * 1e3, pre_ms / K * 1e3


def stream_read_peak(dev, gib=2.0):
    """Measured HBM read rate of the library's plain streaming-read probe over gib GiB (best
    of 10 after 2 untimed): the practical read peak to set the decode's rate against."""
    import torch
    from int4_compressed_domain_amd import tq
    x = torch.ones(int(gib * 2 ** 30) // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(1 << 19, dtype=torch.int32, device=dev)
    best = float("inf")
    for i in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tq.tq_stream_read_probe(x, sink)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            best = min(best, e0.elapsed_time(e1))
    del x, sink
    torch.cuda.empty_cache()
    return gib * 2 ** 30 / (best * 1e-3) / 1e9


def fp16_baseline(S, steps, warmup, dev):
    """Dequantize to dense fp16 (original basis) then dense fp16 attention, same workload."""
    import torch
    from int4_compressed_domain_amd import tq
    w = S.w
    Lmax = S.max_ctx
    k = torch.empty((w.batch, w.kv_heads, Lmax, w.head_dim), dtype=torch.float16, device=dev)
    v = torch.empty_like(k)
    out = torch.empty_like(S.out)
    ws = torch.zeros(tq.tq_decode_workspace_size(S.layout, w.batch, Lmax, 0) // 4 + 1,
                     dtype=torch.float32, device=dev)
    res = {"dequant": [], "attend": []}
    for i in range(warmup + steps):
        pool = S.pools[i % len(S.pools)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        tq.tq_dequant_ref(S.layout, pool, S.bt_dev, S.lens_dev, Lmax, k, v, to_original_basis=1)
        e[1].record()
        tq.tq_dense_decode_attn(S.layout, k, v, S.q, S.lens_dev, Lmax, w.attn_scale, out, ws)
        e[2].record()
        if i >= warmup:
            res["dequant"].append(e)
    torch.cuda.synchronize()
    dq = np.array([e[0].elapsed_time(e[1]) for e in res["dequant"]]) * 1e3
    at = np.array([e[1].elapsed_time(e[2]) for e in res["dequant"]]) * 1e3
    dense_bytes = 2 * k.numel() * 2  # the dense K and V arrays (every row up to the longest context)
    live_bytes = int(np.sum(S.lens, dtype=np.int64)) * w.kv_heads * w.head_dim * 2 * 2  # rows in a context
    return {"dequant_us": float(np.median(dq)), "attend_us": float(np.median(at)),
            "total_us": float(np.median(dq + at)), "dense_kv_bytes": int(dense_bytes),
            "dense_kv_live_bytes": live_bytes,
            "attend_GBps": live_bytes / (np.median(at) * 1e-6) / 1e9}


KERNEL_SOURCES = ("int4_compressed_domain_amd/csrc/decode.hip", "int4_compressed_domain_amd/csrc/tq_device.h",
                  "int4_compressed_domain_amd/csrc/tq_internal.h", "int4_compressed_domain_amd/csrc/tq_codec.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(workload):
    """HBM bytes per decode dispatch from the committed rocprofv3 counter summary of this
    workload, or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "decode_fused_%s_hbm_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, min_seconds=10.0, one_group=False):
    """The C oracle, as it stands, on the host cores: build its own pool (untimed), then time
    its decode of a bounded sample (whole sequences, every q head over every cached token; with
    one_group, only the q heads of the first sequence's first kv head), repeated until
    min_seconds have passed."""
    from int4_compressed_domain_amd import workloads as W
    from oracle import c_oracle
    D, Hkv = w.head_dim, w.kv_heads
    sb = W.sign_bits(D, 0)
    lens = W.context_lens(w, 0)
    bt, _, npages = W.page_tables(w, lens, 0)
    # bounded sample: whole sequences, until ~2^27 token-heads of KV are covered
    budget = 1 << 24
    nseq = 0
    while nseq < w.batch and int(np.sum(lens[:nseq + 1])) * Hkv <= budget:
        nseq += 1
    nseq = max(nseq, 1)
    opool = c_oracle.new_pool(npages, Hkv, D, w.k_codec, w.v_codec)
    scales = W.channel_scales(w, 0)
    for b in range(nseq):
        k32, v32, _, _ = W.seq_tokens(w, b, int(lens[b]), 0, scales)
        c_oracle.append(opool, D, Hkv, k32, v32, W.slots_for(bt, b, 0, int(lens[b])), sb,
                        w.k_codec, w.v_codec)
    q32, _ = W.queries(w, 0)
    if one_group:
        nseq = 1
        pairs = np.array([(0, h) for h in range(w.gqa)], np.int32)
    else:
        pairs = np.array([(b, h) for b in range(nseq) for h in range(w.q_heads)], np.int32)
    # the sample's decode, repeated until at least min_seconds of host time are covered
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        c_oracle.decode(opool, D, w.q_heads, Hkv, sb, bt, lens, q32, w.attn_scale, pairs=pairs,
                        k_codec=w.k_codec, v_codec=w.v_codec)
        dt += time.perf_counter() - t0
        reps += 1
    # the KV bytes the sample's heads read: a q head group reads one kv head's share
    kv = reps * int(np.sum(lens[:nseq], dtype=np.int64)) * W.kv_bytes_per_token(w)
    if one_group:
        kv //= Hkv
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    heads = "%d q heads of kv head 0" % w.gqa if one_group else "%d q heads" % w.q_heads
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds": dt,
            "sample": "C oracle decode (fp64) of %d of %d sequences x %s (%d tokens in "
                      "the first), repeated %d times" % (nseq, w.batch, heads, int(lens[0]), reps)}


def numpy_oracle_single_head(min_seconds=3.0):
    """The NumPy oracle's decode on the single-head workload (1 head, D = 128, 1024 tokens),
    repeated until min_seconds have passed (pool built untimed)."""
    from int4_compressed_domain_amd import workloads as W
    from oracle import np_oracle
    w = W.WORKLOADS["single_head_1k"]
    D, Hkv = w.head_dim, w.kv_heads
    sb = W.sign_bits(D, 0)
    lens = W.context_lens(w, 0)
    bt, _, npages = W.page_tables(w, lens, 0)
    pool = np_oracle.new_pool(npages, Hkv, D)
    k32, v32, _, _ = W.seq_tokens(w, 0, int(lens[0]), 0, W.channel_scales(w, 0))
    np_oracle.append(pool, D, Hkv, k32, v32, W.slots_for(bt, 0, 0, int(lens[0])), sb)
    q32, _ = W.queries(w, 0)
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        np_oracle.decode(pool, D, w.q_heads, Hkv, sb, bt, lens, q32, w.attn_scale)
        dt += time.perf_counter() - t0
        reps += 1
    kv = reps * int(lens[0]) * W.kv_bytes_per_token(w)
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle (NumPy)",
            "seconds": dt, "sample": "NumPy oracle decode of single_head_1k (1024 tokens, "
                                     "1 head), repeated %d times" % reps}


def one_core_baselines(name):
    """The C oracle on one core (one q head group of the workload) and the NumPy oracle on
    the single-head workload, in a child process limited to one thread."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-oracle-child", "--workload", name],
                       env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-400:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    from int4_compressed_domain_amd import workloads as W
    name = args.workload or W.HEADLINE
    w = W.WORKLOADS[name]
    if args.cpu_oracle_child:  # (one thread, no GPU)
        print(json.dumps({"c_oracle_one_core": cpu_baseline(w, one_group=True),
                          "numpy_oracle_single_head": numpy_oracle_single_head()}))
        return
    import torch
    dev = "cuda:0"
    S = Setup(w, args, dev)
    if args.profile:
        for i in range(args.profile):
            S.step(i)
        torch.cuda.synchronize()
        log("profile mode: %d eager steps done" % args.profile)
        return
    if args.profile_append:
        if S.k_pre is None:
            sys.exit("--profile-append needs a workload with a prefill chunk")
        for i in range(args.profile_append):
            S.prefill(i)
        torch.cuda.synchronize()
        log("profile mode: %d prefill-chunk appends done" % args.profile_append)
        return
    K, ms, ev_ms, dec_mean, pre_mean = time_steps(S, args.steps, args.warmup)
    value = S.alg_bytes / (ms * 1e-3) / 1e9
    achieved = S.alg_bytes / (dec_mean * 1e-6) / 1e9
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": name, "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "context": w.context,
                   "ragged_min": w.ragged_min, "prefill": w.prefill, "page": 16, "group": 32,
                   "k_codec": ["absmax", "lloydmax", "fp16"][w.k_codec], "v_codec": {W.CODEC_ABSMAX: "absmax", W.CODEC_ABSMAX3: "absmax3", W.CODEC_ABSMAX2: "absmax2"}[w.v_codec],
                   "kv_input": w.dtype, "attn_scale": w.attn_scale, "splits": args.splits},
        "hbm_fraction": round(value / HBM_PEAK_GBS, 4),
        "decode_us": round(dec_mean, 3), "prefill_append_us": round(pre_mean, 3),
        "step_us": round(ms * 1e3, 3), "step_us_events": round(ev_ms * 1e3, 3),
        "us_per_token": round(ms * 1e3 / max(1, w.batch), 3),
        "algorithmic_bytes": S.alg_bytes, "new_tokens_per_step": S.n_new,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(name),
                     "kernel": "decode_fused", "mean_us": round(dec_mean, 3)},
        "decode_us_p10_p50_p90": S.decode_pct,
        "decode_spread": "%d samples, each one graph replay of %d back-to-back decodes over the "
                         "pool copies, timed with HIP events, divided by %d"
                         % (SPREAD_SAMPLES, SPREAD_LAUNCHES, SPREAD_LAUNCHES),
        # append cost per head_dim vector (K or V of one kv head of one token)
        "append": {"vector": "one head_dim vector, K or V, of one kv head of one token",
                   "one_token_us": round(S.append_one_us, 3),
                   "one_token_vectors": 2 * w.kv_heads * int(np.count_nonzero(S.lens)),
                   "one_token_ns_per_vector": round(S.append_one_us * 1e3 / max(
                       1, 2 * w.kv_heads * int(np.count_nonzero(S.lens))), 3)},
    }
    if w.prefill:
        nv = 2 * w.kv_heads * w.prefill
        rec["append"].update({"prefill_chunk_us": round(pre_mean, 3), "prefill_chunk_vectors": nv,
                              "prefill_ns_per_vector": round(pre_mean * 1e3 / nv, 4)})
    if S.hot:
        rec["config"]["hot_tail"] = S.hot
        rec["roofline"].update({"traffic": None, "kernel": "decode_fused (hot/cold)"})
    if S.sparse_v is not None:
        # one more decode, counted alone: the share of (page, kv head) value blocks skipped
        S.v_skipped.zero_()
        S.decode(0)
        torch.cuda.synchronize()
        pages = int(np.sum((S.lens + 15) // 16)) * w.kv_heads
        frac = int(S.v_skipped.item()) / max(1, pages)
        D = w.head_dim
        kpart = D * 2 if w.k_codec == W.CODEC_FP16 else D // 2 + 2 * (D // 32)
        vpart = D // 2 + 2 * (D // 32)
        moved = int(np.sum(S.lens, dtype=np.int64)) * w.kv_heads * (kpart + vpart * (1.0 - frac))
        moved += S.alg_bytes - S.kv_bytes_all
        rec["config"]["sparse_v_threshold"] = S.sparse_v  # (value pages skipped below)
        rec["sparse_v"] = {"threshold": S.sparse_v, "value_pages_skipped_frac": round(frac, 4),
                           "bytes_moved_est": int(moved)}
        # the dominant kernel's rate on the bytes it actually moves (keys + values not skipped)
        rec["roofline"].update({"achieved": round(moved / (dec_mean * 1e-6) / 1e9, 2),
                                "frac": round(moved / (dec_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "traffic": None, "kernel": "decode_fused (sparse values)"})
    if not args.no_baseline and not S.hot:
        base = fp16_baseline(S, min(args.steps, 20), 3, dev)
        base["speedup_of_fused"] = round(base["total_us"] / dec_mean, 2)
        rec["fp16_dequant_then_attend"] = base
    del S
    torch.cuda.empty_cache()
    peak_meas = stream_read_peak(dev)
    rec["roofline"]["measured_read_peak"] = round(peak_meas, 1)
    rec["roofline"]["frac_of_measured_peak"] = round(rec["roofline"]["achieved"] / peak_meas, 4)
    if "fp16_dequant_then_attend" in rec:
        # the same baseline's floor: its HBM bytes (packed pool read, dense fp16 K and V written
        # then read) moved at the measured read peak, however fast its kernels were made
        b = rec["fp16_dequant_then_attend"]
        moved = rec["algorithmic_bytes"] + 2 * b["dense_kv_live_bytes"]
        b["floor_us_at_measured_read_peak"] = round(moved / (peak_meas * 1e9) * 1e6, 2)
        b["speedup_of_fused_vs_floor"] = round(b["floor_us_at_measured_read_peak"] / dec_mean, 2)
        # the baseline's own roofline: dequant reads the packed pool and writes dense fp16 K and
        # V (every row of the arrays, zeros past each context); the attend reads the rows inside
        # the contexts back
        dq_bytes = rec["algorithmic_bytes"] + b["dense_kv_bytes"]
        b["dequant_GBps"] = round(dq_bytes / (b["dequant_us"] * 1e-6) / 1e9, 1)
        b["dequant_frac"] = round(b["dequant_GBps"] / HBM_PEAK_GBS, 4)
        b["attend_frac"] = round(b["attend_GBps"] / HBM_PEAK_GBS, 4)
        b["frac"] = round(moved / (b["total_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
        rec["cpu_baseline"].update(one_core_baselines(name))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
