"""GPU parity on the codec's edge cases, built on purpose rather than met by chance.

The vectors are constructed in the rotated basis and carried back through an exact
pre-image of the rotation (D = 64 and 256, where rho is a power of two and every partial
sum of the butterflies is exact in fp32), so that after the GPU's own rotation each group
holds exactly what it is meant to hold:

* abs-max (Open-TQ-Metal card abstract: per-group abs-max, int4 nibble pack), for 4-, 3-
  and 2-bit values: quotients y/s on exact half-integers (round half to even), all-zero
  groups (s = 0), fp16-subnormal scales, scales that underflow to zero, scales above the
  fp16 range (saturated at 65504, codes clamped);
* lookup-table keys ("TurboQuant on AMD GPUs", section 2: rotation plus a table): values
  on exact midpoints between table entries under a unit group norm (ties go up),
  zero-norm groups, subnormal and saturated norms;
* fp16 keys (mlxcel manual, the fp16+turbo4 mode): fp16 rounding ties, subnormals, signed
  zeros and magnitudes above 65504.

D = 128 takes the same kinds directly in the input basis (its rho is irrational, so exact
ties cannot be placed there; zero, tiny and huge inputs still reach those branches).
Both entry points that quantize are checked: tq_kv_append for every token but the last,
tq_append_decode_attn for the last one. Pools must equal the oracle's byte for byte and
attention must stay within 2e-3 (normwise) of the fp64 oracle.

Lossless case (exact agreement, last test): keys and values whose rotations are integer
codes with a +-7 in every group are stored without loss, so the decode must equal plain
softmax attention over the original vectors, computed here in fp64 without the oracle.
"""
import functools
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

V3, V2 = W.CODEC_ABSMAX3, W.CODEC_ABSMAX2
QMAX = {W.CODEC_ABSMAX: 7, V3: 3, V2: 1}


@pytest.fixture(autouse=True, scope="module")
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def _hadamard(D):
    i = np.arange(D)
    return np.array([[(-1) ** bin(a & b).count("1") for b in i] for a in i], dtype=np.float64)


def _sigma(sb, D):
    return np.array([-1.0 if (int(sb[i // 32]) >> (i % 32)) & 1 else 1.0 for i in range(D)])


def _preimage(y, sb):
    """x with R(x) = y exactly: x = sigma * (H y) / sqrt(D) for D = 64, 256 (fp64, exact)."""
    D = y.shape[-1]
    x64 = (y @ _hadamard(D)) / math.sqrt(D) * _sigma(sb, D)
    x32 = x64.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x64), "pre-image not exact in fp32"
    return x32


# ---- rotated-basis rows of each kind ----------------------------------------------------------

def _absmax_row(rng, D, Q, kind):
    """One row (D values, groups of 32) for the abs-max codec with largest level Q."""
    y = np.zeros(D)
    if kind == "zero":
        return y
    for g in range(D // 32):
        if kind == "tie_zero_group" and g == 0:
            continue                                  # s = 0: every index is the zero code
        e = {"tie": (-8, 3), "tie_zero_group": (-8, 3), "subnormal": (-24, -14),
             "underflow": (-27, -26), "saturate": (17, 18)}[kind]
        s = 2.0 ** int(rng.integers(*e))
        k = rng.integers(-Q, Q, size=32)
        vals = (k + 0.5) * s                          # exact half-integer quotients
        m = rng.random(32) < 0.3
        vals[m] = rng.integers(-Q, Q + 1, size=int(m.sum())) * s
        vals[int(rng.integers(32))] = Q * s * (1 if rng.random() < 0.5 else -1)  # the max: s = Q s / Q
        y[32 * g:32 * g + 32] = vals
    return y


def _lut_tables():
    lut = c_oracle.lut16().view(np.float16).astype(np.float64)
    T = np.concatenate(([np.nan], 0.5 * (lut[:-1] + lut[1:])))   # T[j], j = 1..15 (exact)
    return lut, T


def _lut_row(rng, D, kind):
    y = np.zeros(D)
    if kind == "lut_zero":
        return y
    _, T = _lut_tables()
    for g in range(D // 32):
        if kind == "lut_mid_zero_group" and g == 0:
            continue                                  # zero norm: every index is 8
        if kind in ("lut_mid", "lut_mid_zero_group"):
            for _ in range(100):                      # midpoints under a unit norm
                j = rng.choice([5, 6, 7, 8, 9, 10, 11], size=31)
                vals = T[j]
                ss = float(np.sum(vals * vals))
                if ss < 0.9:
                    break
            f = round(math.sqrt(1.0 - ss) * 2 ** 17) / 2 ** 17
            pos = int(rng.integers(32))
            grp = np.insert(vals, pos, f)
            u, nb = c_oracle.quant_lut(grp.astype(np.float32))
            assert nb == 0x3C00, "group norm is not 1.0"
            ties = np.delete(np.arange(32), pos)
            assert np.array_equal(u[ties], j), "midpoints must go up"
            y[32 * g:32 * g + 32] = grp
        elif kind == "lut_subnormal":
            y[32 * g:32 * g + 32] = rng.integers(-64, 65, size=32) * 2.0 ** -26
        elif kind == "lut_saturate":
            y[32 * g:32 * g + 32] = rng.integers(-32, 33, size=32) * 2.0 ** 11
    return y


def _f16_key_row(rng, D):
    """Input keys (stored as fp16, not rotated) on fp16's own edges."""
    x = rng.integers(-512, 513, size=D) * 2.0 ** -8
    k = rng.integers(0, 1024, size=D)
    x[0::7] = (1.0 + (2 * k[0::7] + 1) * 2.0 ** -11) * np.sign(rng.random(len(x[0::7])) - 0.5)  # RNE ties
    x[1::7] = rng.integers(-2000, 2001, size=len(x[1::7])) * 2.0 ** -25     # subnormals and ties
    x[2::11] = 0.0
    x[3::11] = -0.0
    x[4::13] = rng.choice([65504.0, 65519.0, 65520.0, 70000.0, 1e6, -1e6, -65520.0], size=len(x[4::13]))
    return x.astype(np.float32)


ABS_KINDS = ["tie", "tie_zero_group", "subnormal", "underflow", "saturate", "zero", "tie"]
LUT_KINDS = ["lut_mid", "lut_mid_zero_group", "lut_zero", "lut_subnormal", "lut_saturate", "lut_mid"]


def _rows(rng, D, n, sb, kind_list, make):
    """n rows in the input basis: exact pre-images at D = 64, 256; at D = 128 the rows
    are taken as inputs directly (zero, tiny and huge groups keep their meaning)."""
    out = np.zeros((n, D), np.float32)
    for i in range(n):
        y = make(kind_list[i % len(kind_list)])
        if D == 128:
            out[i] = y.astype(np.float32)
        else:
            out[i] = _preimage(y, sb)
            assert np.array_equal(c_oracle.rotate(out[i], sb), y.astype(np.float32)), "R(x) != y"
    return out


def _edge_kv(D, k_codec, v_codec, n, Hkv, sb, seed):
    rng = np.random.default_rng(seed)
    Q = QMAX[v_codec]
    nh = n * Hkv
    if k_codec == W.CODEC_FP16:
        k = np.stack([_f16_key_row(rng, D) for _ in range(nh)])
    elif k_codec == W.CODEC_LUT:
        k = _rows(rng, D, nh, sb, LUT_KINDS, lambda kd: _lut_row(rng, D, kd))
    else:
        k = _rows(rng, D, nh, sb, ABS_KINDS, lambda kd: _absmax_row(rng, D, 7, kd))
    v = _rows(rng, D, nh, sb, ABS_KINDS[::-1], lambda kd: _absmax_row(rng, D, Q, kd))
    return k.reshape(n, Hkv, D), v.reshape(n, Hkv, D)


CASES = [(64, 0, 0), (128, 0, 0), (256, 0, 0), (64, 1, 0), (128, 1, 0), (256, 1, 0),
         (64, 2, 0), (128, 2, 0), (64, 0, V3), (256, 0, V3), (128, 2, V3), (64, 1, V2), (256, 0, V2)]


@pytest.mark.parametrize("D,k_codec,v_codec", CASES)
def test_codec_edge_cases(D, k_codec, v_codec):
    lens = [70, 45]
    Hkv, r = 2, 2
    w = W.Workload("edges_d%d_k%d_v%d" % (D, k_codec, v_codec), len(lens), Hkv * r, Hkv, D, max(lens), "f32",
                   1.0 / math.sqrt(D), k_codec=k_codec, v_codec=v_codec)
    _say("case codec edges D=%d k_codec=%d v_codec=%d" % (D, k_codec, v_codec))
    c = Case(w, seed=77 + D + 3 * k_codec + v_codec, lens=lens)
    kv = [_edge_kv(D, k_codec, v_codec, L, Hkv, c.sb, seed=1000 * b + D + 7 * k_codec + v_codec)
          for b, L in enumerate(lens)]
    # every token but the last through tq_kv_append
    for b, L in enumerate(lens):
        k, v = kv[b]
        c.append_raw(k[:L - 1], v[:L - 1], k[:L - 1], v[:L - 1], W.slots_for(c.bt, b, 0, L - 1))
    torch.cuda.synchronize()
    assert c.pool_equal(), "tq_kv_append: pool differs from the oracle"
    # a query whose scores stay within a few units for every key (|alpha q.k| <= 4)
    rng = np.random.default_rng(5 + D)
    q = rng.standard_normal((len(lens), w.q_heads, D)).astype(np.float64)
    kabs = [np.abs(kv[b][0].astype(np.float64)) for b in range(len(lens))]
    if k_codec == W.CODEC_FP16:
        kabs = [np.minimum(x, 65504.0) for x in kabs]   # stored keys saturate
    kmax = max(float(np.max(np.linalg.norm(x, axis=-1))) for x in kabs)
    q *= 4.0 / (w.attn_scale * kmax * np.linalg.norm(q, axis=-1, keepdims=True))
    c.q32 = q.astype(np.float32)
    c.q_dev = to_dev(c.q32, "f32")
    # the last token of each sequence through the fused append + decode
    k_last = np.stack([kv[b][0][L - 1] for b, L in enumerate(lens)])
    v_last = np.stack([kv[b][1][L - 1] for b, L in enumerate(lens)])
    maxc = max(lens)
    ws = torch.zeros(tq.tq_decode_workspace_size(c.layout, len(lens), maxc, 0) // 4, dtype=torch.float32, device=DEV)
    out = torch.full((len(lens), w.q_heads, D), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_append_decode_attn(c.layout, c.pool, to_dev(k_last, "f32"), to_dev(v_last, "f32"), c.q_dev,
                             c.bt_dev, c.lens_dev, maxc, w.attn_scale, out, ws)
    torch.cuda.synchronize()
    slots = np.array([W.slots_for(c.bt, b, L - 1, L)[0] for b, L in enumerate(lens)], np.int64)
    c_oracle.append(c.opool, D, Hkv, k_last, v_last, slots, c.sb, k_codec, v_codec)
    assert c.pool_equal(), "tq_append_decode_attn: pool differs from the oracle"
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = attn_err(got, c.decode_oracle())
    _say("   pools equal; max normwise err %.3e" % err.max())
    assert err.max() <= ATTN_TOL


def _plain_attention(q, K, V, alpha):
    s = alpha * (K @ q)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("v_codec", [0, V3, V2])
def test_lossless_inputs_equal_plain_attention(D, v_codec):
    """Keys and values whose rotations are integer codes in [-Q, Q] with a +-Q in every
    group are stored exactly (scale 1), so the compressed-domain decode must equal softmax
    attention over the original fp32 vectors (fp64 here, no oracle), within 2e-3."""
    lens = [100, 37]
    Hkv, r = 2, 4
    Q = QMAX[v_codec]
    w = W.Workload("lossless_d%d_v%d" % (D, v_codec), len(lens), Hkv * r, Hkv, D, max(lens), "f32",
                   1.0 / math.sqrt(D), v_codec=v_codec)
    _say("case lossless D=%d v_codec=%d" % (D, v_codec))
    c = Case(w, seed=91 + D, lens=lens)
    rng = np.random.default_rng(D + v_codec)

    def codes(n, q):
        y = rng.integers(-q, q + 1, size=(n, D)).astype(np.float64)
        for g in range(D // 32):
            y[np.arange(n), 32 * g + rng.integers(32, size=n)] = q * rng.choice([-1.0, 1.0], size=n)
        return y

    ks, vs = [], []
    for b, L in enumerate(lens):
        k = np.stack([_preimage(y, c.sb) for y in codes(L * Hkv, 7)]).reshape(L, Hkv, D)
        v = np.stack([_preimage(y, c.sb) for y in codes(L * Hkv, Q)]).reshape(L, Hkv, D)
        c.append_raw(k, v, k, v, W.slots_for(c.bt, b, 0, L))
        ks.append(k)
        vs.append(v)
    torch.cuda.synchronize()
    assert c.pool_equal()
    # the query too is an exact pre-image (of multiples of 2^-7), so that its fp32 rotation
    # is exact and the oracle itself must equal plain attention to rounding of fp64
    yq = rng.integers(-512, 513, size=(len(lens) * w.q_heads, D)) / 128.0
    q = np.stack([_preimage(y, c.sb) for y in yq]).reshape(len(lens), w.q_heads, D)
    c.q32, c.q_dev = q, to_dev(q, "f32")
    got = c.decode_gpu()
    ref = np.zeros((len(lens), w.q_heads, D))
    for b in range(len(lens)):
        for hq in range(w.q_heads):
            h = hq // r
            ref[b, hq] = _plain_attention(q[b, hq].astype(np.float64), ks[b][:, h].astype(np.float64),
                                          vs[b][:, h].astype(np.float64), w.attn_scale)
    err = attn_err(got, ref)
    _say("   max normwise err %.3e against plain attention" % err.max())
    assert err.max() <= ATTN_TOL
    assert attn_err(c.decode_oracle(), ref).max() <= 1e-12
