"""C-ABI checks that need no GPU: the library loads, exports every symbol of include/tq.h,
and host-side validation rejects malformed arguments before any device work."""
import ctypes
import os
import re

import pytest

from int4_compressed_domain_amd import tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions(header="tq.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(tq_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert set(names) == set(tq.EXPORTS), names
    lib = tq.lib()
    for n in names:
        assert hasattr(lib, n), n
    # the measurement aid lives in a library of its own, not in the method's
    pnames = _header_functions("tq_probe.h")
    assert set(pnames) == set(tq.PROBE_EXPORTS), pnames
    for n in pnames:
        assert hasattr(tq.probe_lib(), n), n
        assert not hasattr(lib, n), n


def test_status_strings():
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(tq.lib().tq_status_str(s), bytes)


def _layout(**kw):
    args = dict(head_dim=128, num_q_heads=32, num_kv_heads=8, num_pages=10, sign_bits_ptr=0x1000)
    args.update(kw)
    return tq.make_layout(**args)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _append(layout, n=1, dtype=tq.BF16, pool=FAKE, k=FAKE, v=FAKE, slots=FAKE):
    return tq.lib().tq_kv_append(ctypes.byref(layout), pool, k, v, dtype, n, slots, None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), tq.TQ_EINVAL),             # not a power of two: rejected
    (dict(head_dim=0), tq.TQ_EINVAL),
    (dict(head_dim=32), tq.TQ_EUNSUPPORTED),       # power of two outside 64/128/256
    (dict(head_dim=512), tq.TQ_EUNSUPPORTED),
    (dict(num_q_heads=30), tq.TQ_EINVAL),          # Hq % Hkv != 0
    (dict(num_q_heads=0), tq.TQ_EINVAL),
    (dict(num_q_heads=128), tq.TQ_EUNSUPPORTED),   # GQA ratio 16 > 8
    (dict(group_size=24), tq.TQ_EINVAL),           # does not divide D
    (dict(group_size=64), tq.TQ_EUNSUPPORTED),
    (dict(page_size=32), tq.TQ_EUNSUPPORTED),
    (dict(page_size=0), tq.TQ_EINVAL),
    (dict(num_pages=-1), tq.TQ_EINVAL),
    (dict(k_codec=5), tq.TQ_EINVAL),
    (dict(v_codec=1), tq.TQ_EUNSUPPORTED),         # the LUT codec is for keys only
    (dict(v_codec=2), tq.TQ_EUNSUPPORTED),         # and so is fp16
    (dict(v_codec=5), tq.TQ_EINVAL),
    (dict(k_codec=3), tq.TQ_EINVAL),               # 3- and 2-bit codecs are for values
    (dict(sign_bits_ptr=None), tq.TQ_EINVAL),
])
def test_layout_validation(kw, code):
    assert _append(_layout(**kw)) == code


def test_append_argument_validation():
    L = _layout()
    assert _append(L, n=-1) == tq.TQ_EINVAL
    assert _append(L, dtype=9) == tq.TQ_EINVAL
    assert _append(L, pool=None) == tq.TQ_EINVAL
    assert _append(L, slots=None) == tq.TQ_EINVAL
    assert _append(L, n=0, pool=None) == tq.TQ_OK     # nothing to do


def _decode(L, batch=2, bt=FAKE, maxp=4, ctx=FAKE, maxctx=64, alpha=0.1, splits=0, out=FAKE,
            ws=FAKE, wsb=1 << 30, q=FAKE, qd=tq.BF16, pool=FAKE):
    return tq.lib().tq_decode_attn(ctypes.byref(L), pool, q, qd, batch, bt, maxp, ctx, maxctx,
                                   alpha, splits, out, ws, wsb, None)


def test_decode_argument_validation():
    L = _layout()
    assert _decode(L, batch=-1) == tq.TQ_EINVAL
    assert _decode(L, maxctx=65, maxp=4) == tq.TQ_EINVAL        # more tokens than pages
    assert _decode(L, splits=-2) == tq.TQ_EINVAL
    assert _decode(L, qd=7) == tq.TQ_EINVAL
    assert _decode(L, alpha=float("nan")) == tq.TQ_EINVAL
    assert _decode(L, q=None) == tq.TQ_EINVAL
    assert _decode(L, bt=None) == tq.TQ_EINVAL
    assert _decode(L, wsb=16) == tq.TQ_ENOSPC
    assert _decode(L, batch=0, q=None, out=None) == tq.TQ_OK


def _append_decode(L, batch=2, kl=FAKE, vl=FAKE, kd=tq.BF16, bt=FAKE, maxp=4, ctx=FAKE, maxctx=64,
                   alpha=0.1, splits=0, out=FAKE, ws=FAKE, wsb=1 << 30, q=FAKE, qd=tq.BF16, pool=FAKE):
    return tq.lib().tq_append_decode_attn(ctypes.byref(L), pool, kl, vl, kd, q, qd, batch, bt, maxp,
                                          ctx, maxctx, alpha, splits, out, ws, wsb, None)


def test_append_decode_argument_validation():
    L = _layout()
    assert _append_decode(L, kd=5) == tq.TQ_EINVAL              # bad k/v dtype
    assert _append_decode(L, kl=None) == tq.TQ_EINVAL
    assert _append_decode(L, vl=None) == tq.TQ_EINVAL
    assert _append_decode(L, maxctx=65, maxp=4) == tq.TQ_EINVAL
    assert _append_decode(L, qd=7) == tq.TQ_EINVAL
    assert _append_decode(L, wsb=16) == tq.TQ_ENOSPC
    assert _append_decode(L, pool=None) == tq.TQ_EINVAL
    assert _append_decode(L, batch=0, kl=None, vl=None, q=None, out=None) == tq.TQ_OK


def _sparse(L, thr=1e-6, batch=2, bt=FAKE, maxp=4, ctx=FAKE, maxctx=64, out=FAKE, ws=FAKE,
            wsb=1 << 30, q=FAKE, skipped=None):
    return tq.lib().tq_decode_attn_sparse_v(ctypes.byref(L), FAKE, q, tq.BF16, batch, bt, maxp, ctx,
                                            maxctx, 0.1, thr, 0, out, ws, wsb, skipped, None)


def test_sparse_v_argument_validation():
    L = _layout()
    assert _sparse(L, thr=-1e-6) == tq.TQ_EINVAL
    assert _sparse(L, thr=1.0) == tq.TQ_EINVAL
    assert _sparse(L, thr=float("nan")) == tq.TQ_EINVAL
    assert _sparse(L, q=None) == tq.TQ_EINVAL
    assert _sparse(L, wsb=16) == tq.TQ_ENOSPC
    assert _sparse(L, batch=0, q=None, out=None) == tq.TQ_OK
    # sparse values are implemented for 4-bit values only
    # every value width is accepted (up to the workspace check here)
    assert _sparse(_layout(v_codec=tq.CODEC_ABSMAX3), wsb=16) == tq.TQ_ENOSPC
    assert _sparse(_layout(v_codec=tq.CODEC_ABSMAX2), wsb=16) == tq.TQ_ENOSPC
    # the published maxima take 8 words per (sequence, kv head) of the counter area
    assert _sparse(_layout(), batch=(1 << 16) // 8 + 1) == tq.TQ_EUNSUPPORTED


def _append_sparse(L, thr=1e-6, batch=2, kl=FAKE, vl=FAKE, kd=tq.BF16, q=FAKE, wsb=1 << 30,
                   out=FAKE, pool=FAKE):
    return tq.lib().tq_append_decode_attn_sparse_v(ctypes.byref(L), pool, kl, vl, kd, q, tq.BF16, batch,
                                                   FAKE, 4, FAKE, 64, 0.1, thr, 0, out, FAKE, wsb, None,
                                                   None)


def test_append_sparse_v_argument_validation():
    L = _layout()
    assert _append_sparse(L, thr=-1e-6) == tq.TQ_EINVAL
    assert _append_sparse(L, thr=1.0) == tq.TQ_EINVAL
    assert _append_sparse(L, thr=float("nan")) == tq.TQ_EINVAL
    assert _append_sparse(L, kd=5) == tq.TQ_EINVAL              # bad k/v dtype
    assert _append_sparse(L, kl=None) == tq.TQ_EINVAL
    assert _append_sparse(L, vl=None) == tq.TQ_EINVAL
    assert _append_sparse(L, q=None) == tq.TQ_EINVAL
    assert _append_sparse(L, pool=None) == tq.TQ_EINVAL
    assert _append_sparse(L, wsb=16) == tq.TQ_ENOSPC
    assert _append_sparse(_layout(v_codec=tq.CODEC_ABSMAX2), wsb=16) == tq.TQ_ENOSPC
    assert _append_sparse(L, batch=(1 << 16) // 8 + 1) == tq.TQ_EUNSUPPORTED
    assert _append_sparse(L, batch=0, kl=None, vl=None, q=None, out=None) == tq.TQ_OK


def test_stream_read_probe_validation():
    probe = tq.probe_lib().tq_stream_read_probe
    assert probe(FAKE, 0, None, 0, None) == tq.TQ_OK          # nothing to read
    assert probe(None, 64, FAKE, 1 << 21, None) == tq.TQ_EINVAL
    assert probe(FAKE, 60, FAKE, 1 << 21, None) == tq.TQ_EINVAL  # not a multiple of 16
    assert probe(FAKE, 64, FAKE, 16, None) == tq.TQ_ENOSPC      # sink too small


def test_hotcold_argument_validation():
    L = _layout()
    def hc(cap=16, hk=FAKE, hv=FAKE, hl=FAKE, batch=2, q=FAKE):
        return tq.lib().tq_decode_attn_hotcold(ctypes.byref(L), FAKE, q, tq.BF16, batch, FAKE, 4, FAKE,
                                               64, hk, hv, hl, cap, 0.1, 0, FAKE, FAKE, 1 << 30, None)
    assert hc(cap=0) == tq.TQ_EUNSUPPORTED
    assert hc(cap=1025) == tq.TQ_EUNSUPPORTED
    assert hc(hk=None) == tq.TQ_EINVAL
    assert hc(hl=None) == tq.TQ_EINVAL
    assert hc(q=None) == tq.TQ_EINVAL
    assert hc(batch=0, hk=None, hv=None, hl=None, q=None) == tq.TQ_OK


def test_workspace_size_formula():
    L = _layout()
    for batch, ctx, splits in ((1, 131072, 5), (16, 8192, 1), (3, 100, 100)):
        pages = -(-ctx // 16)
        # the sparse-value decode keeps at most 32 pages per wave (8 waves here: 4-bit keys
        # and values stream through registers)
        splits = max(splits, -(-pages // (32 * 8)))
        pps = -(-pages // min(splits, pages))
        S = -(-pages // pps)
        want = (4 << 20) + batch * 32 * S * (128 + 2) * 4 + batch * 8 * 4  # counters + partials + order
        assert tq.tq_decode_workspace_size(L, batch, ctx, splits) == want
    assert tq.tq_decode_workspace_size(_layout(head_dim=96), 1, 10, 0) == 0


def test_page_bytes():
    assert tq.tq_page_bytes(_layout()) == 8 * (16 * 128 + 64 * 4)
    assert tq.tq_page_bytes(_layout(head_dim=256, num_q_heads=4, num_kv_heads=2)) == 2 * (16 * 256 + 64 * 8)
    assert tq.tq_page_bytes(_layout(head_dim=100)) == 0
    # fp16 keys: [K fp16 32D][V indices 8D][V scales 16 x D/32 fp16]
    assert tq.tq_page_bytes(_layout(k_codec=tq.CODEC_FP16)) == 8 * (32 * 128 + 8 * 128 + 32 * 4)
    assert tq.tq_page_bytes(_layout(head_dim=64, k_codec=tq.CODEC_FP16)) == 8 * 41 * 64
    # b-bit values: 2*b*D bytes of value indices instead of 8*D
    for D in (64, 128, 256):
        for vc, b in ((tq.CODEC_ABSMAX3, 3), (tq.CODEC_ABSMAX2, 2)):
            L = _layout(head_dim=D, num_q_heads=8, num_kv_heads=8, v_codec=vc)
            assert tq.tq_page_bytes(L) == 8 * (8 * D + 2 * b * D + 2 * D)
            L = _layout(head_dim=D, num_q_heads=8, num_kv_heads=8, v_codec=vc, k_codec=tq.CODEC_FP16)
            assert tq.tq_page_bytes(L) == 8 * (32 * D + 2 * b * D + D)


def test_fp16_keys_decode_limits():
    """fp16 keys decode at every head_dim; at 256 (four-wave workgroups, one wave per query
    head in the rotations) with at most 4 query heads per kv head: 8 is rejected before any
    launch, 2 passes validation up to the workspace check."""
    L = _layout(head_dim=256, num_q_heads=64, num_kv_heads=8, k_codec=tq.CODEC_FP16)
    assert _decode(L) == tq.TQ_EUNSUPPORTED
    assert _append_decode(L) == tq.TQ_EUNSUPPORTED
    assert _append(L, pool=None) == tq.TQ_EINVAL     # appending itself is supported
    L2 = _layout(head_dim=256, num_q_heads=16, num_kv_heads=8, k_codec=tq.CODEC_FP16)
    assert _decode(L2, wsb=16) == tq.TQ_ENOSPC
    assert _decode(_layout(k_codec=tq.CODEC_FP16), q=None) == tq.TQ_EINVAL


def test_dequant_and_dense_validation():
    L = _layout()
    lib = tq.lib()
    assert lib.tq_dequant_ref(ctypes.byref(L), FAKE, 1, FAKE, 4, FAKE, 64, 2, tq.F32, FAKE, FAKE, None) == tq.TQ_EINVAL
    assert lib.tq_dequant_ref(ctypes.byref(L), FAKE, 1, FAKE, 4, FAKE, 64, 1, tq.BF16, FAKE, FAKE, None) == tq.TQ_EINVAL
    assert lib.tq_dequant_ref(ctypes.byref(L), FAKE, 1, FAKE, 3, FAKE, 64, 1, tq.F32, FAKE, FAKE, None) == tq.TQ_EINVAL
    assert lib.tq_dense_decode_attn(ctypes.byref(L), FAKE, None, FAKE, tq.BF16, 1, FAKE, 64, 0.1, 0, FAKE, FAKE, 1 << 30, None) == tq.TQ_EINVAL
    assert lib.tq_dense_decode_attn(ctypes.byref(L), FAKE, FAKE, FAKE, tq.BF16, 1, FAKE, 64, 0.1, 0, FAKE, FAKE, 8, None) == tq.TQ_ENOSPC
    # one-dimensional grids: more than 2^31 - 1 workgroups is refused before any launch
    # (dequant: 65536 sequences x 8 kv heads x 2^20 tokens / 64 tokens per workgroup = 2^33)
    assert lib.tq_dequant_ref(ctypes.byref(L), FAKE, 1 << 16, FAKE, 1 << 16, FAKE, 1 << 20, 1, tq.F16,
                              FAKE, FAKE, None) == tq.TQ_EUNSUPPORTED
    # (dense attend: 2^17 requested splits x 8 kv heads x 4096 sequences = 2^32)
    assert lib.tq_dense_decode_attn(ctypes.byref(L), FAKE, FAKE, FAKE, tq.BF16, 4096, FAKE, 1 << 21, 0.1,
                                    1 << 17, FAKE, FAKE, 1 << 62, None) == tq.TQ_EUNSUPPORTED


def test_lut_constant_matches_product_generator():
    """The LUT table compiled into the kernels equals what the library's own generator
    (independent of the oracle) derives from the Lloyd-Max iteration."""
    from int4_compressed_domain_amd.csrc import gen_lloydmax
    text = open(os.path.join(ROOT, "int4_compressed_domain_amd", "csrc", "tq_device.h")).read()
    block = text[text.index("#define TQ_LUT16_BITS"):]
    bits = [int(x, 16) for x in re.findall(r"0x([0-9a-f]{4})u", block)[:16]]
    assert bits == gen_lloydmax.lut_bits()
    # and the tabulated fp16 values of the scaled Gaussian codebook (positive half; the
    # negative half is the same with the sign bit set)
    pos = [0x25CF, 0x2C64, 0x2F6E, 0x3155, 0x331B, 0x3494, 0x35DA, 0x37BB]
    assert bits == [b | 0x8000 for b in pos[::-1]] + pos


def test_algorithmic_bytes_of_the_measured_workloads():
    """Bytes one decode must read (packed K+V, query, fp32 output), as the benchmark counts
    them: 144 B per token and kv head at D = 128 with 4-bit keys and values, 328 with fp16
    keys, 312 with fp16 keys and 3-bit values, 112 with 2-bit values."""
    from int4_compressed_domain_amd import workloads as W
    extra = 64 * 128 * 2 + 64 * 128 * 4  # bf16 query + fp32 output
    for name, per in (("llama70b_b1_128k", 144), ("llama70b_b1_128k_k16v4", 328),
                      ("llama70b_b1_128k_k16v3", 312), ("llama70b_b1_128k_k4v2", 112)):
        w = W.WORKLOADS[name]
        assert W.algorithmic_bytes(w, W.context_lens(w, 0)) == 131072 * 8 * per + extra
    assert W.algorithmic_bytes(W.WORKLOADS["llama70b_b1_128k"], W.context_lens(W.WORKLOADS["llama70b_b1_128k"], 0)) == 151044096
