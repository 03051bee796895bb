"""GPU parity: the HIP path through the C ABI against the C oracle on the same seeded inputs.

* append: pools byte-identical (codes and fp16 scales) to the oracle's;
* decode: per (sequence, q head) normwise relative error <= 2e-3 against the fp64 oracle;
* dequantize reference: bit-identical to the oracle's fp32 dequantization;
* dense fp16 baseline: against plain fp64 softmax attention of the same fp16 inputs.
Small cases cover several pages with ragged tails; the full-size cases run the call and
launch configuration the benchmark times and check every (sequence, q head) output, or
one q head of every (sequence, kv head) for the batch of 64.
"""
import math
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from int4_compressed_domain_amd import tq  # noqa: E402
from int4_compressed_domain_amd import workloads as W  # noqa: E402
from oracle import c_oracle  # noqa: E402

from .gpu_util import ATTN_TOL, DEV, Case, attn_err, to_dev  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_case(c, pairs=None, num_splits=0, tol=ATTN_TOL):
    out = c.decode_gpu(num_splits=num_splits)
    if pairs is None:
        ref = c.decode_oracle()
        err = attn_err(out, ref)
    else:
        ref = c.decode_oracle(pairs)
        got = np.stack([out[b, h] for b, h in pairs])
        err = attn_err(got, ref)
    assert np.all(np.isfinite(out)), "non-finite output"
    _say("   max normwise err %.3e" % err.max())
    assert err.max() <= tol, "attention error %.3e > %.1e" % (err.max(), tol)
    return out


SMALL = {
    "single_head_1k": dict(context=1024, batch=1),
    "llama8b_b16_8k": dict(context=700, batch=3),
    "llama70b_b1_128k": dict(context=2000, batch=1),
    "gemma_d256_32k": dict(context=900, batch=2),
    "mixed_serving": dict(context=600, batch=5, ragged_min=17, prefill=100),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workload_parity(name):
    w = W.WORKLOADS[name].scaled(**SMALL[name])
    _say("case", name, w)
    c = Case(w)
    c.fill()
    if w.prefill:
        k32, v32, kst, vst = W.prefill_tokens(w, c.seed, c.scales)
        slots = c.prefill_pages.astype(np.int64).repeat(16)[:w.prefill] * 16 + np.arange(w.prefill) % 16
        c.append_raw(k32, v32, kst, vst, slots)
        torch.cuda.synchronize()
    assert c.pool_equal(), "packed pool differs from the oracle"
    _check_case(c)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("r", [1, 2, 4, 8])
def test_head_dims_and_gqa(D, r):
    base = W.WORKLOADS["llama8b_b16_8k"]
    w = base.scaled(context=300, batch=2)
    w = W.Workload("d%d_r%d" % (D, r), 2, 2 * r, 2, D, 300, "bf16", 1.0 / math.sqrt(D),
                   dist="lognormal_spikes")
    _say("case D=%d r=%d" % (D, r))
    c = Case(w, seed=D + r)
    c.fill()
    assert c.pool_equal()
    _check_case(c)


@pytest.mark.parametrize("D,r", [(64, 1), (64, 4), (64, 8), (128, 1), (128, 4), (128, 8),
                                 (256, 1), (256, 2), (256, 4)])
def test_fp16_keys(D, r):
    """fp16 keys + 4-bit values: pool bytes equal the oracle's (keys as fp16 of the input,
    values rotated and quantized), attention within the tolerance, across split counts."""
    w = W.Workload("k16_d%d_r%d" % (D, r), 3, 2 * r, 2, D, 700, "bf16", 1.0 / math.sqrt(D),
                   k_codec=2, dist="lognormal_spikes")
    _say("case fp16 keys D=%d r=%d" % (D, r))
    c = Case(w, seed=40 + D + r, lens=[700, 33, 260])
    c.fill()
    assert c.pool_equal()
    for splits in (0, 1, 5):
        _check_case(c, num_splits=splits)


V3, V2 = W.CODEC_ABSMAX3, W.CODEC_ABSMAX2


@pytest.mark.parametrize("D,r,k_codec,v_codec", [(64, 4, 0, V3), (128, 8, 0, V3), (128, 8, 2, V3),
                                                 (256, 2, 0, V3), (128, 4, 1, V2), (128, 8, 0, V2),
                                                 (64, 2, 2, V2), (256, 4, 1, V2), (256, 2, 2, V3),
                                                 (256, 4, 2, V2), (64, 2, 0, V2)])
def test_low_bit_values(D, r, k_codec, v_codec):
    """3-bit and 2-bit values with each key codec: packed pool bytes equal the oracle's
    (appends of many tokens into shared pages), attention within the tolerance for edge
    lengths and several split counts."""
    lens = [700, 0, 1, 15, 16, 17, 260]
    w = W.Workload("v%d_d%d_r%d_k%d" % (v_codec, D, r, k_codec), len(lens), 2 * r, 2, D, max(lens), "bf16",
                   1.0 / math.sqrt(D), k_codec=k_codec, v_codec=v_codec, dist="lognormal_spikes")
    _say("case low-bit values D=%d r=%d k_codec=%d v_codec=%d" % (D, r, k_codec, v_codec))
    c = Case(w, seed=60 + D + r + k_codec + v_codec, lens=lens)
    c.fill(chunk=300)
    assert c.pool_equal(), "packed pool differs from the oracle"
    for splits in (0, 1, 5):
        out = _check_case(c, num_splits=splits)
        assert np.all(out[1] == 0.0)


def _sparse_gpu(c, thr, num_splits=0):
    w = c.w
    max_ctx = int(c.lens.max())
    ws = torch.zeros(max(tq.tq_decode_workspace_size(c.layout, w.batch, max_ctx, num_splits), 4) // 4,
                     dtype=torch.float32, device=DEV)
    out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    skipped = torch.zeros(1, dtype=torch.int64, device=DEV)
    tq.tq_decode_attn_sparse_v(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, max_ctx, w.attn_scale,
                               thr, out, ws, num_splits=num_splits, v_pages_skipped=skipped)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(skipped.item())


@pytest.mark.parametrize("name,k_codec,v_codec", [("llama70b_b1_128k", 0, 0), ("gemma_d256_32k", 0, 0),
                                                  ("mixed_serving", 1, 0), ("llama70b_b1_128k", 2, 0),
                                                  ("llama70b_b1_128k", 2, V3), ("llama70b_b1_128k", 0, V2),
                                                  ("gemma_d256_32k", 2, V3), ("llama70b_b1_128k", 0, V3)])
def test_sparse_values(name, k_codec, v_codec):
    """Sparse values: threshold 0 reproduces the dense decode bit for bit; at 1e-6 the
    result stays within the tolerance plus the oracle's bound on the dropped terms
    (sum of w_t |v_t| over weights below the threshold), for several split counts, and
    spiky attention lets most value pages be skipped; 4-, 3- and 2-bit values."""
    base = W.WORKLOADS[name]
    w = W.Workload(name + "_sv", 3, base.q_heads, base.kv_heads, base.head_dim, 3000, base.dtype,
                   base.attn_scale, k_codec=k_codec, v_codec=v_codec, dist="lognormal_spikes")
    _say("case sparse values", name, "k_codec", k_codec, "v_codec", v_codec)
    c = Case(w, seed=23, lens=[3000, 1234, 77])
    c.fill()
    dense = c.decode_gpu()
    out0, sk0 = _sparse_gpu(c, 0.0)
    assert sk0 == 0 and np.array_equal(out0, dense)
    exact = c.decode_oracle()
    _, bound = c_oracle.decode_sparse_v(c.opool, w.head_dim, w.q_heads, w.kv_heads, c.sb, c.bt,
                                        c.lens, c.q32, w.attn_scale, 1e-6, k_codec=w.k_codec,
                                        v_codec=w.v_codec)
    total = int(np.sum((c.lens + 15) // 16)) * w.kv_heads
    for splits in (0, 1, 3):
        out, sk = _sparse_gpu(c, 1e-6, splits)
        err = np.max(np.abs(out - exact), axis=2)
        lim = ATTN_TOL * np.max(np.abs(exact), axis=2) + bound
        _say("   splits %d: skipped %d of %d value pages, max err %.3e" % (splits, sk, total, err.max()))
        assert np.all(np.isfinite(out)) and np.all(err <= lim)
        if splits == 1:
            assert sk > 0, "spiky attention should let value pages be skipped"


def _hot_cold_case(D, r, k_codec, cold, hot, cap, splits_list, seed, v_codec=0, kv=2):
    w = W.Workload("hc_d%d_r%d_k%d" % (D, r, k_codec), len(cold), kv * r, kv, D, max(max(cold), 1), "bf16",
                   1.0 / math.sqrt(D), k_codec=k_codec, v_codec=v_codec, dist="lognormal_spikes")
    _say("case hot/cold D", D, "r", r, "k_codec", k_codec, "tail capacity", cap)
    c = Case(w, seed=seed, lens=cold)
    c.fill()
    hk = np.zeros((w.batch, w.kv_heads, cap, D), np.float16)
    hv = np.zeros_like(hk)
    for b in range(w.batch):
        k32, v32, _, _ = W.seq_tokens(w, b, cold[b] + hot[b], c.seed, c.scales)
        hk[b, :, :hot[b]] = k32[cold[b]:].transpose(1, 0, 2).astype(np.float16)
        hv[b, :, :hot[b]] = v32[cold[b]:].transpose(1, 0, 2).astype(np.float16)
    hl = np.array(hot, np.int32)
    ref = c_oracle.decode_hotcold(c.opool, D, w.q_heads, w.kv_heads, c.sb, c.bt, c.lens, hk, hv, hl,
                                  c.q32, w.attn_scale, k_codec=w.k_codec, v_codec=w.v_codec)
    hk_d = torch.from_numpy(hk).to(DEV)
    hv_d = torch.from_numpy(hv).to(DEV)
    hl_d = torch.from_numpy(hl).to(DEV)
    maxc = int(max(cold))
    outs = []
    for splits in splits_list:
        ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, w.batch, maxc, splits) // 4,
                         dtype=torch.float32, device=DEV)
        out = torch.full((w.batch, w.q_heads, D), float("nan"), dtype=torch.float32, device=DEV)
        tq.tq_decode_attn_hotcold(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, maxc, hk_d, hv_d,
                                  hl_d, w.attn_scale, out, ws, num_splits=splits)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        err = attn_err(o, ref)
        _say("   splits %d: max normwise err %.3e" % (splits, err.max()))
        assert np.all(np.isfinite(o)) and err.max() <= ATTN_TOL
        assert int(ws[:(4 << 20) // 4].view(torch.int32).abs().sum().item()) == 0, "counters not reset"
        outs.append(o)
    return outs


@pytest.mark.parametrize("D,r,k_codec,v_codec", [(128, 8, 0, 0), (128, 4, 1, 0), (128, 8, 2, 0),
                                                 (64, 2, 2, 0), (256, 2, 0, 0), (128, 8, 2, V3)])
def test_hot_cold(D, r, k_codec, v_codec):
    """Hot/cold cache: older tokens in the pool, the most recent in an fp16 tail, one softmax;
    against the oracle for several split counts, with empty pools, empty and full tails, and
    a sequence with no tokens at all."""
    outs = _hot_cold_case(D, r, k_codec, [0, 1, 40, 300, 1000, 0], [5, 0, 64, 17, 1, 0], 64,
                          (0, 1, 3), 90 + D + r + k_codec, v_codec)
    for o in outs:
        assert np.all(o[-1] == 0.0)


@pytest.mark.parametrize("D,kv,cap", [(128, 2, 256), (256, 4, 256), (64, 1, 256), (128, 2, 512),
                                      (256, 2, 512), (64, 1, 512), (128, 2, 1024), (64, 1, 1024),
                                      (128, 8, 256), (128, 8, 512)])
def test_hot_cold_tail_workgroup(D, kv, cap):
    """Few long sequences with automatic splits: the tail gets workgroups of its own per
    (sequence, kv head), one per 512 tokens of capacity and at least two where a unit has 16
    splits or more (pieces of equal length), beside the pool's splits (as many splits fewer);
    with 8 kv heads (8 splits per unit) one workgroup takes the whole tail. Checked against
    the oracle with long, full, short and empty tails and pools."""
    cold = [16384, 0, 9000, 100]
    hot = [200, cap, 0, 17] if cap == 256 else [cap, 333, 0, cap - 1]
    w_outs = _hot_cold_case(D, 4, 0, cold, hot, cap, (0,), 400 + D + cap, kv=kv)
    assert np.all(np.isfinite(w_outs[0]))


@pytest.mark.parametrize("D,r", [(64, 8), (128, 8), (256, 4)])
def test_hot_cold_long_tail(D, r):
    """Tails of up to the largest capacity (1024 tokens), longer than one batch of the value
    loop, with ragged ends; a tail-only sequence (no pool tokens) among them."""
    _hot_cold_case(D, r, 0, [0, 700, 33, 129], [1024, 1023, 517, 64], 1024, (0, 2), 300 + D)


@pytest.mark.parametrize("k_codec", [0, 1, 2])
def test_ragged_edge_lengths(k_codec):
    lens = [0, 1, 15, 16, 17, 33, 48, 250]
    w = W.Workload("edges", len(lens), 8, 2, 128, max(lens), "bf16", 0.125, k_codec=k_codec)
    _say("case edge lengths, k_codec", k_codec)
    c = Case(w, seed=5, lens=lens)
    c.fill()
    assert c.pool_equal()
    out = _check_case(c)
    assert np.all(out[0] == 0.0), "an empty sequence must give a zero output"


@pytest.mark.parametrize("num_splits", [0, 3])
def test_many_ragged_sequences(num_splits):
    """More workgroups than the chip holds at once (40 sequences x 8 kv heads): workgroups
    take sequences longest first. Ties, empty and one-token sequences included."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 400, 40)
    lens[[3, 9, 20]] = 0
    lens[[4, 5, 6]] = 257          # ties
    lens[7] = 1
    lens[8] = 512
    w = W.Workload("many", len(lens), 16, 8, 128, int(lens.max()), "bf16", 0.125,
                   k_codec=1, ragged_min=1)
    _say("case many ragged sequences, splits", num_splits)
    c = Case(w, seed=8, lens=lens)
    c.fill()
    out = _check_case(c, num_splits=num_splits)
    assert np.all(out[[3, 9, 20]] == 0.0)


def test_batch_beyond_longest_first_limit():
    """Batch 300 (past the longest-first limit): plain workgroup order."""
    rng = np.random.default_rng(78)
    lens = rng.integers(0, 40, 300)
    w = W.Workload("wide", len(lens), 4, 2, 64, int(lens.max()), "f32", 0.125, ragged_min=1)
    _say("case batch 300")
    c = Case(w, seed=9, lens=lens)
    c.fill()
    _check_case(c)


@pytest.mark.parametrize("q_dtype", ["f32", "f16"])
def test_query_dtypes(q_dtype):
    w = W.WORKLOADS["llama8b_b16_8k"].scaled(context=200, batch=2)
    _say("case q dtype", q_dtype)
    c = Case(w, seed=3, q_dtype=q_dtype)
    c.fill()
    _check_case(c)


def test_fp32_and_fp16_cache_inputs():
    for dt in ("f32", "f16"):
        w = W.Workload("in_" + dt, 2, 4, 2, 128, 130, "f32", 0.09)
        c = Case(w, seed=9)
        for b in range(w.batch):
            k32, v32, _, _ = W.seq_tokens(w, b, int(c.lens[b]), c.seed, c.scales)
            if dt == "f16":
                k32, v32 = k32.astype(np.float16), v32.astype(np.float16)
                c.w = W.Workload("in_f16", 2, 4, 2, 128, 130, "f16", 0.09)
                c.append_raw(k32.astype(np.float32), v32.astype(np.float32), k32, v32,
                             W.slots_for(c.bt, b, 0, int(c.lens[b])))
                c.w = w
            else:
                c.append_raw(k32, v32, k32, v32, W.slots_for(c.bt, b, 0, int(c.lens[b])))
        torch.cuda.synchronize()
        assert c.pool_equal(), dt


def test_split_count_invariance():
    w = W.WORKLOADS["llama70b_b1_128k"].scaled(context=3000, batch=2)
    _say("case split invariance")
    c = Case(w, seed=11)
    c.fill()
    outs = [c.decode_gpu(num_splits=s) for s in (1, 2, 7, 0, 1000)]
    # P' = p * s_V is rounded to fp16 relative to the running max at the time its page is
    # processed, which depends on the split count, so results differ by those roundings:
    # at worst one fp16 unit roundoff (2^-11) of every weight, all in one direction. They
    # are independent across the 3000 tokens and largely cancel: on MI355X the largest
    # normwise difference of the four split counts is 6.1e-5 (~2^-14), rms ~7e-6, so the
    # bar is 2^-13, twice the largest seen.
    for o in outs[1:]:
        e = attn_err(o, outs[0])
        _say("   split agreement: max %.3e, rms %.3e" % (e.max(), np.sqrt(np.mean(e ** 2))))
        assert e.max() < 2.0 ** -13
    ref = c.decode_oracle()
    for o in outs:
        assert attn_err(o, ref).max() <= ATTN_TOL


@pytest.mark.parametrize("D,r", [(128, 8), (256, 2), (64, 4)])
def test_most_splits(D, r):
    """The largest split count (128 splits of 2 pages): the last workgroup merges the
    partials, in several rounds of loads at D = 128 and 256 (at D = 64 the 16 split groups
    of 16 loads cover 256 splits, so one round); within 2^-11 of one split and within the
    tolerance of the oracle. A second sequence of 33 tokens (3 pages) uses 2 of the 128
    splits."""
    w = W.Workload("most_splits_d%d" % D, 2, 2 * r, 2, D, 4096, "bf16", 1.0 / math.sqrt(D),
                   dist="lognormal_spikes")
    _say("case most splits D", D, "r", r)
    c = Case(w, seed=37, lens=[4096, 33])
    c.fill()
    one, most = c.decode_gpu(num_splits=1), c.decode_gpu(num_splits=128)
    assert attn_err(most, one).max() < 2.0 ** -11
    err = attn_err(most, c.decode_oracle())
    _say("   max normwise err %.3e" % err.max())
    assert np.all(np.isfinite(most)) and err.max() <= ATTN_TOL


def test_negative_slots_and_untouched_bytes():
    w = W.WORKLOADS["llama8b_b16_8k"].scaled(context=64, batch=1)
    c = Case(w, seed=2)
    c.pool.fill_(0xAB)
    c.opool[:] = 0xAB
    k32, v32, kst, vst = W.seq_tokens(w, 0, 40, c.seed, c.scales)
    slots = W.slots_for(c.bt, 0, 0, 40)
    slots[::3] = -1
    c.append_raw(k32, v32, kst, vst, slots)
    torch.cuda.synchronize()
    assert c.pool_equal()


DEQUANT_CASES = [(128, k, v) for k, v in [(0, 0), (1, 0), (2, 0), (0, V3), (2, V3), (1, V2)]] + \
    [(64, 0, 0), (64, 1, V3), (64, 2, V2), (256, 0, 0), (256, 1, V2), (256, 2, V3), (256, 0, V3)]


@pytest.mark.parametrize("D,k_codec,v_codec", DEQUANT_CASES)
@pytest.mark.parametrize("basis", [0, 1])
def test_dequant_reference(D, k_codec, v_codec, basis):
    lens = [37, 0, 50]
    w = W.Workload("dq", 3, 8, 2, D, 50, "bf16", 0.1, k_codec=k_codec, v_codec=v_codec)
    c = Case(w, seed=13, lens=lens)
    c.fill()
    Lmax = 60  # rows past each context (zeros), whole pages of them, a partial last page
    for dt in (torch.float32, torch.float16):
        ko = torch.full((3, 2, Lmax, D), 7.0, dtype=dt, device=DEV)
        vo = torch.full_like(ko, 7.0)
        tq.tq_dequant_ref(c.layout, c.pool, c.bt_dev, c.lens_dev, Lmax, ko, vo, to_original_basis=basis)
        torch.cuda.synchronize()
        rk, rv = c_oracle.dequant(c.opool, D, 2, c.sb, c.bt, c.lens, Lmax, basis, k_codec, v_codec)
        if dt == torch.float16:
            rk, rv = rk.astype(np.float16), rv.astype(np.float16)
        assert np.array_equal(ko.cpu().numpy(), rk)
        assert np.array_equal(vo.cpu().numpy(), rv)


DENSE_CASES = [
    # (head_dim, q heads, kv heads, lengths, splits, q dtype, key codec)
    (256, 16, 8, [500, 333], 0, None, 0),      # the D = 256 workload's shape, r = 2
    (128, 16, 2, [1000, 15, 16, 17], 3, None, 0),  # r = 8 (the 128K shape), edge lengths
    (128, 4, 4, [257, 0, 1], 0, "f32", 1),      # r = 1, an empty and a one-token sequence
    (64, 8, 1, [300, 33], 2, "f16", 0),         # r = 8 at D = 64
    (256, 8, 1, [100, 31], 0, None, 2),         # r = 8 at D = 256, fp16 keys
    (128, 12, 4, [129, 64], 5, None, 0),        # r = 3 (padded to 4 columns)
    (64, 12, 2, [1000, 77], 0, "f32", 1),       # r = 6 (padded to 8 columns)
    (128, 8, 1, [2000, 1500, 0], 100, None, 0),  # 100 splits: the merge takes them in rounds of 64
]


@pytest.mark.parametrize("D,hq,hkv,lens,splits,q_dtype,k_codec", DENSE_CASES)
def test_dense_fp16_baseline(D, hq, hkv, lens, splits, q_dtype, k_codec):
    w = W.Workload("dense", len(lens), hq, hkv, D, max(lens), "bf16", 1.0 if D == 256 else D ** -0.5,
                   k_codec=k_codec)
    c = Case(w, seed=17 + D + hq, lens=lens, q_dtype=q_dtype)
    c.fill()
    Lmax = max(lens)
    B = len(lens)
    ko = torch.zeros((B, hkv, Lmax, D), dtype=torch.float16, device=DEV)
    vo = torch.zeros_like(ko)
    tq.tq_dequant_ref(c.layout, c.pool, c.bt_dev, c.lens_dev, Lmax, ko, vo, to_original_basis=1)
    ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, B, Lmax, splits) // 4, dtype=torch.float32, device=DEV)
    out = torch.full((B, hq, D), 7.0, dtype=torch.float32, device=DEV)
    tq.tq_dense_decode_attn(c.layout, ko, vo, c.q_dev, c.lens_dev, Lmax, w.attn_scale, out, ws,
                            num_splits=splits)
    torch.cuda.synchronize()
    # the reference is the oracle's: its own dequantization (original basis), rounded to
    # fp16 as the baseline stores it, then its fp64 attention
    Ko, Vo = c_oracle.dequant(c.opool, D, hkv, c.sb, c.bt, c.lens, Lmax, 1,
                              k_codec=w.k_codec, v_codec=w.v_codec)
    assert np.array_equal(ko.cpu().numpy(), Ko.astype(np.float16))
    K16 = Ko.astype(np.float16).astype(np.float64)
    V16 = Vo.astype(np.float16).astype(np.float64)
    ref = np.zeros((B, hq, D))
    for b in range(B):
        L = int(c.lens[b])
        if L == 0:
            continue
        for h in range(hq):
            ref[b, h] = c_oracle.attention_f64(c.q32[b, h], K16[b, h // w.gqa, :L], V16[b, h // w.gqa, :L],
                                               w.attn_scale)
    got = out.cpu().numpy()
    assert attn_err(got, ref).max() <= ATTN_TOL
    # how far the baseline's fp16-rounded keys put it from the compressed-domain result
    # (reported, not bounded: at attention scale 1.0 the rounding moves scores visibly)
    exact = c.decode_oracle()
    _say("   dense baseline vs the compressed-domain oracle: max normwise %.3e" % attn_err(got, exact).max())


def test_baseline_batch_beyond_65535():
    """70000 sequences (one kv head, one page each) through the dequant and the dense attend:
    their workgroups fill a one-dimensional grid past 65535. The pool holds 4 filled
    sequences; the block table repeats their rows, so every output row has a known answer."""
    w = W.Workload("bigb", 4, 1, 1, 64, 16, "bf16", 0.125)
    c = Case(w, seed=3, lens=[16, 16, 16, 16])
    c.fill()
    B = 70000
    rep = np.arange(B) % 4
    bt = torch.from_numpy(np.ascontiguousarray(c.bt[rep])).to(DEV)
    lens = torch.full((B,), 16, dtype=torch.int32, device=DEV)
    ko = torch.zeros((B, 1, 16, 64), dtype=torch.float16, device=DEV)
    vo = torch.zeros_like(ko)
    tq.tq_dequant_ref(c.layout, c.pool, bt, lens, 16, ko, vo, to_original_basis=1)
    Ko, Vo = c_oracle.dequant(c.opool, 64, 1, c.sb, c.bt, c.lens, 16, 1)
    K16, V16 = Ko.astype(np.float16), Vo.astype(np.float16)
    assert np.array_equal(ko.cpu().numpy(), K16[rep])
    assert np.array_equal(vo.cpu().numpy(), V16[rep])
    q = c.q_dev[torch.from_numpy(rep).to(DEV)].contiguous()
    ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, B, 16, 0) // 4, dtype=torch.float32, device=DEV)
    out = torch.full((B, 1, 64), 7.0, dtype=torch.float32, device=DEV)
    tq.tq_dense_decode_attn(c.layout, ko, vo, q, lens, 16, w.attn_scale, out, ws)
    torch.cuda.synchronize()
    ref = np.stack([c_oracle.attention_f64(c.q32[b, 0], K16[b, 0].astype(np.float64),
                                           V16[b, 0].astype(np.float64), w.attn_scale) for b in range(4)])
    assert attn_err(out.cpu().numpy()[:, 0], ref[rep]).max() <= ATTN_TOL


# ---- full-size workloads, through the call and launch configuration the benchmark times ----

def _full_size_pairs(w):
    """Every (sequence, q head) pair where that is at most 512 of them; otherwise one q
    head of every (sequence, kv head), taking each head of the group in turn."""
    if w.batch * w.q_heads <= 512:
        return None
    r = w.gqa
    return [(b, h * r + (b + h) % r) for b in range(w.batch) for h in range(w.kv_heads)]


@pytest.mark.parametrize("name", ["single_head_1k", "llama8b_b16_8k", "llama70b_b1_128k",
                                  "gemma_d256_32k", "mixed_serving", "llama70b_b1_128k_k16v4",
                                  "llama70b_b1_128k_k16v3", "llama70b_b1_128k_k4v2",
                                  "gemma_d256_32k_k16v4"])
def test_full_size_workloads(name):
    """The benchmark's step at full size: every token but each sequence's last is resident,
    the mixed-serving prefill chunk is appended with tq_kv_append, and one
    tq_append_decode_attn appends the newest tokens and decodes (automatic split count).
    Pools must equal the oracle's; outputs are checked on every (sequence, q head) pair, or
    on one q head of every (sequence, kv head) for the batch of 64."""
    w = W.WORKLOADS[name]
    _say("case full-size", name)
    c = Case(w)
    last = c.fill(chunk=8192, keep_last=True)
    if w.prefill:
        k32, v32, kst, vst = W.prefill_tokens(w, c.seed, c.scales)
        slots = c.prefill_pages.astype(np.int64).repeat(16)[:w.prefill] * 16 + np.arange(w.prefill) % 16
        c.append_raw(k32, v32, kst, vst, slots)
        torch.cuda.synchronize()
    out = c.append_decode_gpu(last)
    assert c.pool_equal(), "packed pool differs from the oracle"
    _say("   pool bytes equal (%d B)" % c.pool.numel())
    pairs = _full_size_pairs(w)
    assert np.all(np.isfinite(out)), "non-finite output"
    if pairs is None:
        err = attn_err(out, c.decode_oracle())
    else:
        err = attn_err(np.stack([out[b, h] for b, h in pairs]), c.decode_oracle(pairs))
    _say("   %d pairs, max normwise err %.3e" % (err.size, err.max()))
    assert err.max() <= ATTN_TOL, "attention error %.3e > %.1e" % (err.max(), ATTN_TOL)


@pytest.mark.parametrize("D,r,k_codec,dtype,v_codec", [(128, 8, 0, "bf16", 0), (128, 4, 1, "bf16", 0),
                                                       (64, 2, 0, "f32", 0), (256, 2, 0, "bf16", 0),
                                                       (128, 8, 2, "bf16", 0), (64, 4, 2, "f32", 0),
                                                       (128, 8, 2, "bf16", V3), (128, 8, 0, "bf16", V2),
                                                       (64, 4, 2, "f32", V3), (256, 2, 0, "bf16", V3),
                                                       (64, 2, 1, "bf16", V2), (128, 8, 0, "bf16", V3),
                                                       (64, 2, 0, "f32", V3), (64, 4, 0, "bf16", V2)])
def test_append_decode_equals_append_then_decode(D, r, k_codec, dtype, v_codec):
    """The fused entry point writes the same pool bytes as tq_kv_append of each sequence's
    last token and returns the same output, bit for bit, as tq_decode_attn afterwards."""
    lens = [0, 1, 15, 16, 17, 33, 250, 1000]
    w = W.Workload("appdec", len(lens), 2 * r, 2, D, max(lens), dtype, 0.125, k_codec=k_codec,
                   v_codec=v_codec)
    _say("case append+decode D", D, "r", r, "k_codec", k_codec, dtype, "v_codec", v_codec)
    fused = Case(w, seed=31, lens=lens)
    split = Case(w, seed=31, lens=lens, oracle=False)
    for c in (fused, split):  # every token but the last
        for b, L in enumerate(c.lens):
            if L > 1:
                c.append_seq(b, 0, int(L) - 1)
    k_last = np.zeros((w.batch, w.kv_heads, D), np.float32)
    v_last = np.zeros_like(k_last)
    kst = np.zeros(k_last.shape, np.float32 if dtype == "f32" else np.uint16)
    vst = np.zeros_like(kst)
    slots = np.full(w.batch, -1, np.int64)
    for b, L in enumerate(fused.lens):
        if L > 0:
            k32, v32, ks_, vs_ = W.seq_tokens(w, b, int(L), fused.seed, fused.scales)
            k_last[b], v_last[b], kst[b], vst[b] = k32[-1], v32[-1], ks_[-1], vs_[-1]
            slots[b] = W.slots_for(fused.bt, b, int(L) - 1, int(L))[0]
    maxc = int(max(lens))
    outs = []
    for c, use_fused in ((fused, True), (split, False)):
        ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, w.batch, maxc, 0) // 4, dtype=torch.float32, device=DEV)
        out = torch.full((w.batch, w.q_heads, D), float("nan"), dtype=torch.float32, device=DEV)
        if use_fused:
            tq.tq_append_decode_attn(c.layout, c.pool, to_dev(kst, dtype), to_dev(vst, dtype), c.q_dev,
                                     c.bt_dev, c.lens_dev, maxc, w.attn_scale, out, ws)
        else:
            tq.tq_kv_append(c.layout, c.pool, to_dev(kst, dtype), to_dev(vst, dtype),
                            torch.from_numpy(slots).to(DEV))
            tq.tq_decode_attn(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, maxc, w.attn_scale, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    keep = slots >= 0
    c_oracle.append(fused.opool, D, w.kv_heads, k_last[keep], v_last[keep], slots[keep], fused.sb,
                    w.k_codec, w.v_codec)
    assert np.array_equal(fused.pool.cpu().numpy(), split.pool.cpu().numpy())
    assert fused.pool_equal()
    assert np.array_equal(outs[0], outs[1])
    err = attn_err(outs[0], fused.decode_oracle())
    _say("   max normwise err %.3e" % err.max())
    assert err.max() <= ATTN_TOL
    assert np.all(outs[0][0] == 0.0)


@pytest.mark.parametrize("D,r,k_codec,v_codec", [(128, 8, 0, 0), (128, 4, 0, 0), (128, 2, 0, V2),
                                                 (64, 4, 0, V3), (128, 4, 1, 0), (128, 4, 2, 0),
                                                 (256, 2, 0, 0), (256, 2, 2, V3)])
def test_append_sparse_v_equals_append_then_sparse_v(D, r, k_codec, v_codec):
    """The fused sparse-value entry point writes the same pool bytes as tq_kv_append of each
    sequence's last token; with one split (one published maximum per unit, so the pages
    dropped do not depend on timing) it returns the same output and skip count, bit for
    bit, as tq_decode_attn_sparse_v afterwards; with automatic splits it stays within the
    tolerance plus the oracle's bound on the dropped terms."""
    lens = [0, 1, 15, 16, 17, 33, 250, 1000]
    w = W.Workload("appsv", len(lens), 2 * r, 2, D, max(lens), "bf16", 1.0 / math.sqrt(D),
                   k_codec=k_codec, v_codec=v_codec, dist="lognormal_spikes")
    _say("case append+sparse values D", D, "r", r, "k_codec", k_codec, "v_codec", v_codec)
    fused = Case(w, seed=37, lens=lens)
    split = Case(w, seed=37, lens=lens, oracle=False)
    for c in (fused, split):  # every token but the last
        for b, L in enumerate(c.lens):
            if L > 1:
                c.append_seq(b, 0, int(L) - 1)
    k_last = np.zeros((w.batch, w.kv_heads, D), np.float32)
    v_last = np.zeros_like(k_last)
    kst = np.zeros(k_last.shape, np.uint16)
    vst = np.zeros_like(kst)
    slots = np.full(w.batch, -1, np.int64)
    for b, L in enumerate(fused.lens):
        if L > 0:
            k32, v32, ks_, vs_ = W.seq_tokens(w, b, int(L), fused.seed, fused.scales)
            k_last[b], v_last[b], kst[b], vst[b] = k32[-1], v32[-1], ks_[-1], vs_[-1]
            slots[b] = W.slots_for(fused.bt, b, int(L) - 1, int(L))[0]
    maxc = int(max(lens))
    kd, vd = to_dev(kst, "bf16"), to_dev(vst, "bf16")

    def run(c, use_fused, splits):
        ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, w.batch, maxc, splits) // 4, dtype=torch.float32,
                         device=DEV)
        out = torch.full((w.batch, w.q_heads, D), float("nan"), dtype=torch.float32, device=DEV)
        sk = torch.zeros(1, dtype=torch.int64, device=DEV)
        if use_fused:
            tq.tq_append_decode_attn_sparse_v(c.layout, c.pool, kd, vd, c.q_dev, c.bt_dev, c.lens_dev, maxc,
                                              w.attn_scale, 1e-6, out, ws, num_splits=splits, v_pages_skipped=sk)
        else:
            tq.tq_kv_append(c.layout, c.pool, kd, vd, torch.from_numpy(slots).to(DEV))
            tq.tq_decode_attn_sparse_v(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, maxc, w.attn_scale,
                                       1e-6, out, ws, num_splits=splits, v_pages_skipped=sk)
        torch.cuda.synchronize()
        return out.cpu().numpy(), int(sk.item())

    of, skf = run(fused, True, 1)
    os_, sks = run(split, False, 1)
    keep = slots >= 0
    c_oracle.append(fused.opool, D, w.kv_heads, k_last[keep], v_last[keep], slots[keep], fused.sb,
                    w.k_codec, w.v_codec)
    assert np.array_equal(fused.pool.cpu().numpy(), split.pool.cpu().numpy())
    assert fused.pool_equal()
    _say("   one split: skipped %d value pages (fused) and %d (separate append)" % (skf, sks))
    assert skf == sks
    if r <= 4:  # (with 8 q heads per kv head some head keeps nearly every page here)
        assert skf > 0
    assert np.array_equal(of, os_)
    assert np.all(of[0] == 0.0)
    exact = fused.decode_oracle()
    _, bound = c_oracle.decode_sparse_v(fused.opool, D, w.q_heads, w.kv_heads, fused.sb, fused.bt,
                                        fused.lens, fused.q32, w.attn_scale, 1e-6, k_codec=w.k_codec,
                                        v_codec=w.v_codec)
    lim = ATTN_TOL * np.max(np.abs(exact), axis=2) + bound
    for out in (of, run(fused, True, 0)[0]):  # (the second call appends the same bytes again)
        err = np.max(np.abs(out - exact), axis=2)
        _say("   max err %.3e" % err.max())
        assert np.all(np.isfinite(out)) and np.all(err <= lim)
    assert fused.pool_equal()


def test_workspace_reuse_across_calls():
    """The split-arrival counters in the workspace return to zero after every call, so one
    zero-filled workspace serves calls of any batch size and split count in sequence."""
    w = W.WORKLOADS["llama70b_b1_128k"].scaled(context=2500, batch=3)
    c = Case(w, seed=21)
    c.fill()
    ref = c.decode_oracle()
    ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, 3, 2500, 40) // 4 + 16, dtype=torch.float32, device=DEV)
    for it, (nb, splits) in enumerate([(3, 0), (1, 7), (3, 40), (2, 0), (3, 3), (3, 0)]):
        out = torch.full((nb, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device=DEV)
        tq.tq_decode_attn(c.layout, c.pool, c.q_dev[:nb], c.bt_dev[:nb], c.lens_dev[:nb], int(c.lens[:nb].max()),
                          w.attn_scale, out, ws, num_splits=splits)
        torch.cuda.synchronize()
        assert attn_err(out.cpu().numpy(), ref[:nb]).max() <= ATTN_TOL, (it, nb, splits)
    assert int(ws[:(4 << 20) // 4].view(torch.int32).abs().sum().item()) == 0, "counters not reset"


@pytest.mark.parametrize("mode", ["append_then_decode", "fused", "fused_sparse"])
def test_graph_replay_matches_eager(mode):
    """append + decode captured in a HIP graph, replayed several times with eager work and
    synchronizations in between; every replay must equal the eager result bit for bit. The
    step is tq_kv_append then tq_decode_attn, or one tq_append_decode_attn, or one
    tq_append_decode_attn_sparse_v with one split (whose dropped pages do not depend on
    timing)."""
    w = W.WORKLOADS["llama8b_b16_8k"].scaled(context=900, batch=4)
    c = Case(w, seed=23, lens=[900, 899, 450, 17])
    c.fill()
    L = c.lens.copy()
    nsp = 1 if mode == "fused_sparse" else 0
    ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, w.batch, int(L.max()), nsp) // 4, dtype=torch.float32,
                     device=DEV)
    out = torch.zeros((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    # the step re-appends the last token of every sequence, then decodes
    k32, v32, kst, vst, sl = [], [], [], [], []
    for b in range(w.batch):
        kk, vv, ks_, vs_ = W.seq_tokens(w, b, int(L[b]), c.seed, c.scales)
        k32.append(kk[-1:]); v32.append(vv[-1:]); kst.append(ks_[-1:]); vst.append(vs_[-1:])
        sl.append(W.slots_for(c.bt, b, int(L[b]) - 1, int(L[b])))
    kd, vd = to_dev(np.concatenate(kst), w.dtype), to_dev(np.concatenate(vst), w.dtype)
    sd = torch.from_numpy(np.concatenate(sl)).to(DEV)

    def step():
        if mode == "append_then_decode":
            tq.tq_kv_append(c.layout, c.pool, kd, vd, sd)
            tq.tq_decode_attn(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, int(L.max()), w.attn_scale, out, ws)
        elif mode == "fused":
            tq.tq_append_decode_attn(c.layout, c.pool, kd, vd, c.q_dev, c.bt_dev, c.lens_dev, int(L.max()),
                                     w.attn_scale, out, ws)
        else:
            tq.tq_append_decode_attn_sparse_v(c.layout, c.pool, kd, vd, c.q_dev, c.bt_dev, c.lens_dev,
                                              int(L.max()), w.attn_scale, 1e-6, out, ws, num_splits=nsp)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert c.pool_equal()
    exact = c.decode_oracle()
    if mode == "fused_sparse":  # within the tolerance plus the oracle's bound on the dropped terms
        _, bound = c_oracle.decode_sparse_v(c.opool, w.head_dim, w.q_heads, w.kv_heads, c.sb, c.bt, c.lens,
                                            c.q32, w.attn_scale, 1e-6, k_codec=w.k_codec, v_codec=w.v_codec)
        err = np.max(np.abs(eager.cpu().numpy() - exact), axis=2)
        assert np.all(err <= ATTN_TOL * np.max(np.abs(exact), axis=2) + bound)
    else:
        assert attn_err(eager.cpu().numpy(), exact).max() <= ATTN_TOL
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs" % rep
        step()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def _random_config(i):
    rng = np.random.default_rng(1000 + i)
    D = int(rng.choice([64, 128, 256]))
    k_codec = int(rng.choice([0, 1, 2] if D <= 128 else [0, 1]))
    v_codec = int(rng.choice([W.CODEC_ABSMAX, W.CODEC_ABSMAX3, W.CODEC_ABSMAX2]))
    r = int(rng.choice([1, 2, 3, 4, 8]))
    kv = int(rng.choice([1, 2, 3]))
    batch = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 600, batch)]
    if i % 4 == 1:
        lens[-1] = 0
    if i % 4 == 2:
        lens[0] = 16 * int(rng.integers(1, 30))
    q_dtype = str(rng.choice(["bf16", "f32", "f16"]))
    splits = int(rng.choice([0, 0, 1, 2, 7]))
    hot = int(rng.choice([0, 0, 1, 40])) if i % 3 == 0 else 0
    return D, k_codec, v_codec, r, kv, batch, lens, q_dtype, splits, hot


@pytest.mark.parametrize("i", range(24))
def test_random_configurations(i):
    """Seeded random combinations of head dim, key and value codecs, GQA ratio, kv heads,
    ragged lengths, query dtype, split count and (every third case) an fp16 tail: pool bytes
    equal to the oracle's and attention within the tolerance."""
    D, k_codec, v_codec, r, kv, batch, lens, q_dtype, splits, hot = _random_config(i)
    _say("case random %d: D %d k %d v %d r %d kv %d lens %s q %s splits %d hot %d"
         % (i, D, k_codec, v_codec, r, kv, lens, q_dtype, splits, hot))
    if hot:
        hl = [min(hot, 1 + (b * 7) % (hot + 1)) for b in range(batch)]
        _hot_cold_case(D, r, k_codec, [max(L, 1) if b % 2 else L for b, L in enumerate(lens)], hl,
                       max(hot, 1), (splits,), 2000 + i, v_codec=v_codec, kv=kv)
        return
    w = W.Workload("rnd%d" % i, batch, kv * r, kv, D, max(max(lens), 1), "bf16", 1.0 / math.sqrt(D),
                   k_codec=k_codec, v_codec=v_codec, dist="lognormal_spikes")
    c = Case(w, seed=3000 + i, lens=lens, q_dtype=q_dtype)
    c.fill(chunk=257)
    assert c.pool_equal(), "packed pool differs from the oracle"
    out = _check_case(c, num_splits=splits)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(out[b] == 0.0)
    # sparse values with the last token re-appended in the launch (the same bytes again)
    k_last = np.zeros((batch, kv, D), np.uint16)
    v_last = np.zeros_like(k_last)
    for b, L in enumerate(lens):
        if L > 0:
            _, _, ks_, vs_ = W.seq_tokens(w, b, L, c.seed, c.scales)
            k_last[b], v_last[b] = ks_[-1], vs_[-1]
    maxc = max(lens)
    ws = torch.zeros(max(tq.tq_decode_workspace_size(c.layout, batch, maxc, splits), 4) // 4, dtype=torch.float32,
                     device=DEV)
    sp = torch.full((batch, kv * r, D), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_append_decode_attn_sparse_v(c.layout, c.pool, to_dev(k_last, "bf16"), to_dev(v_last, "bf16"), c.q_dev,
                                      c.bt_dev, c.lens_dev, maxc, w.attn_scale, 1e-6, sp, ws, num_splits=splits)
    torch.cuda.synchronize()
    assert c.pool_equal(), "the re-appended tokens changed the pool"
    exact = c.decode_oracle()
    _, bound = c_oracle.decode_sparse_v(c.opool, D, w.q_heads, kv, c.sb, c.bt, c.lens, c.q32, w.attn_scale, 1e-6,
                                        k_codec=k_codec, v_codec=v_codec)
    err = np.max(np.abs(sp.cpu().numpy() - exact), axis=2)
    _say("   fused sparse values: max err %.3e" % err.max())
    assert np.all(err <= ATTN_TOL * np.max(np.abs(exact), axis=2) + bound)


@pytest.mark.parametrize("nbytes", [16, 16 * 12345, 8 << 20])
def test_stream_read_probe_reads_every_word_once(nbytes):
    """The measurement probe (not part of the method): every thread stores the XOR of the
    words it read, so the XOR over the sink equals the XOR over the whole buffer exactly
    when each 16-byte element is read once."""
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.zeros((2 << 20) // 4, dtype=torch.int32, device=DEV)
    tq.tq_stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))


def test_validation_of_device_tables(monkeypatch):
    """TQ_VALIDATE=1: the device-side preconditions are checked on the host before any
    launch. A page id outside the pool, a length above max_context_len, a tail longer than
    its capacity, and a slot outside the pool or given twice return TQ_EINVAL; valid
    tables decode as usual."""
    monkeypatch.setenv("TQ_VALIDATE", "1")
    w = W.Workload("val", 2, 4, 2, 128, 40, "bf16", 0.1)
    c = Case(w, seed=7, lens=[40, 17])
    c.fill()
    _check_case(c)  # valid tables: checked, then decoded
    ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, 2, 40, 0) // 4, dtype=torch.float32, device=DEV)
    out = torch.zeros((2, 4, 128), dtype=torch.float32, device=DEV)

    def decode(bt, lens, maxc=40):
        tq.tq_decode_attn(c.layout, c.pool, c.q_dev, torch.from_numpy(bt).to(DEV),
                          torch.from_numpy(np.asarray(lens, np.int32)).to(DEV), maxc, 0.1, out, ws)

    bt = c.bt.copy()
    bt[1, 1] = c.npages  # page 1 of the 17-token sequence lies outside the pool
    with pytest.raises(tq.TQError) as e:
        decode(bt, c.lens)
    assert e.value.status == tq.TQ_EINVAL
    bt = c.bt.copy()
    bt[1, 2] = -1  # not used by a 17-token sequence: accepted
    decode(bt, c.lens)
    with pytest.raises(tq.TQError) as e:
        decode(c.bt, [41, 17])  # longer than max_context_len
    assert e.value.status == tq.TQ_EINVAL
    hk = torch.zeros((2, 2, 8, 128), dtype=torch.float16, device=DEV)
    with pytest.raises(tq.TQError) as e:
        tq.tq_decode_attn_hotcold(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, 40, hk, hk,
                                  torch.tensor([3, 9], dtype=torch.int32, device=DEV), 0.1, out, ws)
    assert e.value.status == tq.TQ_EINVAL  # a tail of 9 tokens in a capacity of 8
    kv = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device=DEV)
    for slots in ([0, 0], [c.npages * 16, -1]):  # a slot twice; a slot outside the pool
        with pytest.raises(tq.TQError) as e:
            tq.tq_kv_append(c.layout, c.pool, kv, kv, torch.tensor(slots, dtype=torch.int64, device=DEV))
        assert e.value.status == tq.TQ_EINVAL
    before = c.pool.clone()
    tq.tq_kv_append(c.layout, c.pool, kv[:1], kv[:1], torch.tensor([-1], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(before, c.pool)


@pytest.mark.parametrize("D,k_codec,v_codec", [(64, 0, 0), (128, 1, 0), (128, 0, V2), (64, 0, V3), (64, 0, V2)])
def test_sparse_values_full_waves(D, k_codec, v_codec):
    """Sparse values with one split over 8192 tokens (512 pages): each wave holds the most
    pages the first pass keeps maxima for (32). LUT keys stage two key parts per LDS ring
    slot; abs-max keys stream through registers, where 2-bit values (D = 64 and 128) keep the
    second page set's scale blocks in a second ring slot. Within the tolerance plus the
    oracle's bound, value pages skipped."""
    w = W.Workload("sv_full_d%d" % D, 2, 8, 2, D, 8192, "bf16", 1.0 / math.sqrt(D), k_codec=k_codec,
                   v_codec=v_codec, dist="lognormal_spikes")
    _say("case sparse values, full waves, D", D, "k_codec", k_codec, "v_codec", v_codec)
    c = Case(w, seed=29, lens=[8192, 5000])
    c.fill()
    exact = c.decode_oracle()
    _, bound = c_oracle.decode_sparse_v(c.opool, D, w.q_heads, w.kv_heads, c.sb, c.bt, c.lens, c.q32,
                                        w.attn_scale, 1e-6, k_codec=k_codec, v_codec=w.v_codec)
    for splits in (1, 0):
        out, sk = _sparse_gpu(c, 1e-6, splits)
        err = np.max(np.abs(out - exact), axis=2)
        lim = ATTN_TOL * np.max(np.abs(exact), axis=2) + bound
        _say("   splits %d: skipped %d value pages, max err %.3e" % (splits, sk, err.max()))
        assert np.all(np.isfinite(out)) and np.all(err <= lim)
        assert sk > 0


@pytest.mark.parametrize("D,kv,k_codec,v_codec", [(256, 4, 0, 0), (128, 8, 2, V3), (64, 8, 1, 0)])
def test_pool_beyond_4gib(D, kv, k_codec, v_codec):
    """A pool of more than 4.5 GiB whose used pages all lie past the first 4.5 GiB, up to its
    last page: append, fused append+decode, decode, sparse values and the dequantize
    reference write and read the same bytes and results as the oracle's compact pool (same
    pages, shifted ids), and the bytes below the used pages stay untouched."""
    lens = [3000, 1037, 16]
    w = W.Workload("big_d%d" % D, len(lens), 4 * kv, kv, D, max(lens), "bf16", 1.0 / math.sqrt(D),
                   k_codec=k_codec, v_codec=v_codec, dist="lognormal_spikes")
    _say("case pool beyond 4 GiB, D", D, "kv", kv, "k_codec", k_codec, "v_codec", v_codec)
    c = Case(w, seed=41, lens=lens)
    pb = c.page_bytes
    base = -(-(9 << 29) // pb)  # first used page starts at or past 4.5 GiB
    total = base + c.npages
    big = torch.zeros(total * pb, dtype=torch.uint8, device=DEV)
    lay = tq.make_layout(D, w.q_heads, kv, total, c.sb_dev.data_ptr(), k_codec, v_codec)
    bt_big = torch.from_numpy(c.bt.astype(np.int64) + base).to(torch.int32).to(DEV)
    k_last = np.zeros((w.batch, kv, D), np.float32)
    v_last = np.zeros_like(k_last)
    kst, vst = np.zeros(k_last.shape, np.uint16), np.zeros(k_last.shape, np.uint16)
    for b, L in enumerate(lens):  # every token but the last of each sequence
        k32, v32, ks_, vs_ = W.seq_tokens(w, b, L, c.seed, c.scales)
        slots = W.slots_for(c.bt, b, 0, L - 1)
        tq.tq_kv_append(lay, big, to_dev(ks_[:L - 1], "bf16"), to_dev(vs_[:L - 1], "bf16"),
                        torch.from_numpy(slots + base * 16).to(DEV))
        c_oracle.append(c.opool, D, kv, k32[:L - 1], v32[:L - 1], slots, c.sb, k_codec, v_codec)
        k_last[b], v_last[b], kst[b], vst[b] = k32[-1], v32[-1], ks_[-1], vs_[-1]
        c_oracle.append(c.opool, D, kv, k32[-1:], v32[-1:], W.slots_for(c.bt, b, L - 1, L), c.sb,
                        k_codec, v_codec)
    maxc = max(lens)
    ws = torch.zeros(tq.tq_decode_workspace_size(lay, w.batch, maxc, 0) // 4, dtype=torch.float32,
                     device=DEV)
    out = torch.full((w.batch, w.q_heads, D), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_append_decode_attn(lay, big, to_dev(kst, "bf16"), to_dev(vst, "bf16"), c.q_dev, bt_big,
                             c.lens_dev, maxc, w.attn_scale, out, ws)
    out2 = torch.full_like(out, float("nan"))
    tq.tq_decode_attn(lay, big, c.q_dev, bt_big, c.lens_dev, maxc, w.attn_scale, out2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(big[base * pb:].cpu().numpy(), c.opool), "pool bytes differ"
    low = big[:base * pb].view(torch.int32)
    assert int(low.max().item()) == 0 and int(low.min().item()) == 0, "bytes below the pages written"
    del low
    o = out.cpu().numpy()
    assert np.array_equal(o, out2.cpu().numpy())
    exact = c.decode_oracle()
    err = attn_err(o, exact)
    _say("   decode: max normwise err %.3e" % err.max())
    assert np.all(np.isfinite(o)) and err.max() <= ATTN_TOL
    if True:  # sparse values, every value width
        _, bound = c_oracle.decode_sparse_v(c.opool, D, w.q_heads, kv, c.sb, c.bt, c.lens, c.q32,
                                            w.attn_scale, 1e-6, k_codec=k_codec, v_codec=v_codec)
        so = torch.full_like(out, float("nan"))
        skipped = torch.zeros(1, dtype=torch.int64, device=DEV)
        tq.tq_decode_attn_sparse_v(lay, big, c.q_dev, bt_big, c.lens_dev, maxc, w.attn_scale, 1e-6,
                                   so, ws, v_pages_skipped=skipped)
        torch.cuda.synchronize()
        so = so.cpu().numpy()
        lim = ATTN_TOL * np.max(np.abs(exact), axis=2) + bound
        _say("   sparse values: skipped %d value pages" % int(skipped.item()))
        assert np.all(np.isfinite(so)) and np.all(np.max(np.abs(so - exact), axis=2) <= lim)
    ko = torch.full((w.batch, kv, maxc, D), 7.0, dtype=torch.float32, device=DEV)
    vo = torch.full_like(ko, 7.0)
    tq.tq_dequant_ref(lay, big, bt_big, c.lens_dev, maxc, ko, vo, to_original_basis=1)
    torch.cuda.synchronize()
    rk, rv = c_oracle.dequant(c.opool, D, kv, c.sb, c.bt, c.lens, maxc, 1, k_codec, v_codec)
    assert np.array_equal(ko.cpu().numpy(), rk) and np.array_equal(vo.cpu().numpy(), rv)
    del big, ko, vo
    torch.cuda.empty_cache()
