"""ctypes binding of the C oracle (tq_oracle.c). Test infrastructure only.

Every function here marshals NumPy arrays into the C routines; the arithmetic lives in
tq_oracle.c, whose header lists the passages of the pages it follows.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force=False):
    """Compile tq_oracle.c with gcc (IEEE arithmetic: no FMA contraction, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=gnu11", "-ffp-contract=off",
                           "-fno-fast-math", "-fopenmp", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.or_f64_to_f16.argtypes = [f64]
        L.or_f64_to_f16.restype = ctypes.c_uint16
        L.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_f16_to_f64.restype = f64
        L.or_rho_f32.argtypes = [i32]
        L.or_rho_f32.restype = ctypes.c_float
        L.or_rotate.argtypes = [P, P, i32, P]
        L.or_unrotate_f32.argtypes = [P, P, i32, P]
        L.or_quant_absmax.argtypes = [P, i32, P, P]
        L.or_lloydmax16.argtypes = [P, P]
        L.or_lut16.argtypes = [P]
        L.or_quant_lut.argtypes = [P, i32, P, P, P]
        L.or_encode.argtypes = [P, i64, i32, i32, P, i32, P, P]
        L.or_block_bytes.argtypes = [i32]
        L.or_block_bytes.restype = i64
        L.or_place.argtypes = [P, i32, i32, i64, P, P, P, P, P]
        L.or_append.argtypes = [P, i32, i32, i32, i32, P, P, P, i64, P]
        L.or_fetch.argtypes = [P, i32, i32, i64, i32, i32, P, P, P, P]
        L.or_attention_f64.argtypes = [P, P, P, i64, i32, f64, P]
        L.or_decode.argtypes = [P, i32, i32, i32, i32, i32, P, P, i32, P, P, ctypes.c_float, P, i32, P]
        L.or_dequant.argtypes = [P, i32, i32, i32, i32, P, P, i32, P, i32, i32, i32, P, P]
        L.or_block_bytes_kc.argtypes = [i32, i32]
        L.or_block_bytes_kc.restype = i64
        L.or_keys_f16.argtypes = [P, i64, P]
        L.or_place_kf16.argtypes = [P, i32, i32, i64, P, P, P, P]
        L.or_fetch_kf16.argtypes = [P, i32, i32, i64, i32, i32, P, P, P]
        L.or_quant_absmax_q.argtypes = [P, i32, i32, P, P]
        L.or_block_bytes_kv.argtypes = [i32, i32, i32]
        L.or_block_bytes_kv.restype = i64
        L.or_place_kv.argtypes = [P, i32, i32, i32, i32, i64, P, P, P, P, P, P]
        L.or_fetch_kv.argtypes = [P, i32, i32, i32, i32, i64, i32, i32, P, P, P, P, P]
        L.or_decode_sparse_v.argtypes = [P, i32, i32, i32, i32, i32, P, P, i32, P, P, ctypes.c_float,
                                         f64, P, i32, P, P]
        L.or_decode_hotcold.argtypes = [P, i32, i32, i32, i32, i32, P, P, i32, P, P, P, P, i32, P,
                                        ctypes.c_float, P, i32, P]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def f32_to_f16_bits(x):
    return np.array([lib().or_f64_to_f16(float(v)) for v in np.asarray(x, np.float64).ravel()],
                    np.uint16).reshape(np.shape(x))


def rho_f32(D):
    return np.float32(lib().or_rho_f32(D))


def rotate(x, sign_bits):
    """fp32 rotation of each row of x ([..., D] fp32)."""
    x = _c(x, np.float32)
    D = x.shape[-1]
    sb = _c(sign_bits, np.uint32)
    flat = x.reshape(-1, D)
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        lib().or_rotate(_p(flat[i]), _p(out[i]), D, _p(sb))
    return out.reshape(x.shape)


def unrotate_f32(y, sign_bits):
    y = _c(y, np.float32)
    D = y.shape[-1]
    sb = _c(sign_bits, np.uint32)
    flat = y.reshape(-1, D)
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        lib().or_unrotate_f32(_p(flat[i]), _p(out[i]), D, _p(sb))
    return out.reshape(y.shape)


def quant_absmax(y, qmax=7):
    """One group of rotated fp32 values -> (indices u in 1..2*qmax+1, fp16 scale bits)."""
    y = _c(y, np.float32)
    u = np.empty(y.shape[0], np.uint8)
    s = np.zeros(1, np.uint16)
    if qmax == 7:
        lib().or_quant_absmax(_p(y), y.shape[0], _p(u), _p(s))
    else:
        lib().or_quant_absmax_q(_p(y), y.shape[0], qmax, _p(u), _p(s))
    return u, int(s[0])


def lloydmax16():
    m = np.empty(16, np.float64)
    mse = np.empty(1, np.float64)
    lib().or_lloydmax16(_p(m), _p(mse))
    return m, float(mse[0])


def lut16():
    lut = np.empty(16, np.uint16)
    lib().or_lut16(_p(lut))
    return lut


def quant_lut(y, lut=None):
    y = _c(y, np.float32)
    lut = lut16() if lut is None else _c(lut, np.uint16)
    u = np.empty(y.shape[0], np.uint8)
    n = np.zeros(1, np.uint16)
    lib().or_quant_lut(_p(y), y.shape[0], _p(lut), _p(u), _p(n))
    return u, int(n[0])


def encode(x, sign_bits, codec=0, group=32):
    """Rotate + quantize rows of x ([n, D] fp32) -> (u [n, D] uint8, scales [n, D/group] uint16)."""
    x = _c(x, np.float32)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    n = flat.shape[0]
    u = np.empty((n, D), np.uint8)
    s = np.empty((n, D // group), np.uint16)
    lib().or_encode(_p(flat), n, D, group, _p(_c(sign_bits, np.uint32)), codec, _p(u), _p(s))
    return u.reshape(x.shape[:-1] + (D,)), s.reshape(x.shape[:-1] + (D // group,))


KF16 = 2  # k_codec of the fp16-key mode


ABSMAX3, ABSMAX2 = 3, 4  # v_codec of the 3-bit and 2-bit value modes


def block_bytes(D, k_codec=0, v_codec=0):
    return int(lib().or_block_bytes_kv(D, k_codec, v_codec))


def new_pool(num_pages, Hkv, D, k_codec=0, v_codec=0):
    return np.zeros(num_pages * Hkv * block_bytes(D, k_codec, v_codec), np.uint8)


def place_kv(pool, D, Hkv, slots, vu, vs, ku=None, ks=None, kh=None, k_codec=0, v_codec=0):
    """Store encoded tokens in a pool of any (k_codec, v_codec); keys as ku/ks (indices and
    scales) or kh (fp16 bits, k_codec 2)."""
    slots = _c(slots, np.int64)
    lib().or_place_kv(_p(pool), D, Hkv, k_codec, v_codec, slots.shape[0], _p(slots),
                      None if ku is None else _p(_c(ku, np.uint8)),
                      None if ks is None else _p(_c(ks, np.uint16)),
                      None if kh is None else _p(_c(kh, np.uint16)),
                      _p(_c(vu, np.uint8)), _p(_c(vs, np.uint16)))


def fetch_kv(pool, D, Hkv, page, t, h, k_codec=0, v_codec=0):
    """-> (ku, ks, kh, vu, vs) of one token; the key arrays of the other key form are zero."""
    G = D // 32
    ku, vu = np.zeros(D, np.uint8), np.zeros(D, np.uint8)
    ks, vs = np.zeros(G, np.uint16), np.zeros(G, np.uint16)
    kh = np.zeros(D, np.uint16)
    lib().or_fetch_kv(_p(pool), D, Hkv, k_codec, v_codec, page, t, h, _p(ku), _p(ks), _p(kh),
                      _p(vu), _p(vs))
    return ku, ks, kh, vu, vs


def keys_f16(k):
    """fp16 bits (round to nearest even, overflow saturated) of fp32 keys, any shape."""
    k = _c(k, np.float32)
    out = np.empty(k.shape, np.uint16)
    lib().or_keys_f16(_p(k), k.size, _p(out))
    return out


def place_kf16(pool, D, Hkv, slots, kh, vu, vs):
    slots = _c(slots, np.int64)
    lib().or_place_kf16(_p(pool), D, Hkv, slots.shape[0], _p(slots), _p(_c(kh, np.uint16)),
                        _p(_c(vu, np.uint8)), _p(_c(vs, np.uint16)))


def fetch_kf16(pool, D, Hkv, page, t, h):
    kh, vu, vs = np.empty(D, np.uint16), np.empty(D, np.uint8), np.empty(D // 32, np.uint16)
    lib().or_fetch_kf16(_p(pool), D, Hkv, page, t, h, _p(kh), _p(vu), _p(vs))
    return kh, vu, vs


def place(pool, D, Hkv, slots, ku, ks, vu, vs):
    slots = _c(slots, np.int64)
    lib().or_place(_p(pool), D, Hkv, slots.shape[0], _p(slots), _p(_c(ku, np.uint8)),
                   _p(_c(ks, np.uint16)), _p(_c(vu, np.uint8)), _p(_c(vs, np.uint16)))


def append(pool, D, Hkv, k, v, slots, sign_bits, k_codec=0, v_codec=0):
    """Encode k, v ([n, Hkv, D] fp32) and write them into pool (uint8, in place)."""
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    slots = _c(slots, np.int64)
    lib().or_append(_p(pool), D, Hkv, k_codec, v_codec, _p(_c(sign_bits, np.uint32)),
                    _p(k), _p(v), slots.shape[0], _p(slots))


def fetch(pool, D, Hkv, page, t, h):
    G = D // 32
    ku, vu = np.empty(D, np.uint8), np.empty(D, np.uint8)
    ks, vs = np.empty(G, np.uint16), np.empty(G, np.uint16)
    lib().or_fetch(_p(pool), D, Hkv, page, t, h, _p(ku), _p(ks), _p(vu), _p(vs))
    return ku, ks, vu, vs


def attention_f64(q, K, V, alpha):
    q = _c(q, np.float64)
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    out = np.empty(q.shape[0], np.float64)
    lib().or_attention_f64(_p(q), _p(K), _p(V), K.shape[0], q.shape[0], float(alpha), _p(out))
    return out


def decode(pool, D, Hq, Hkv, sign_bits, block_table, context_lens, q, alpha, pairs=None,
           k_codec=0, v_codec=0):
    """fp64 decode attention for (b, hq) pairs (default: all). q: [B, Hq, D] fp32.
    Returns fp64 [n_pairs, D] (or [B, Hq, D] when pairs is None)."""
    q = _c(q, np.float32)
    B = q.shape[0]
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    full = pairs is None
    if full:
        pairs = np.array([(b, h) for b in range(B) for h in range(Hq)], np.int32)
    pairs = _c(pairs, np.int32).reshape(-1, 2)
    out = np.empty((pairs.shape[0], D), np.float64)
    lib().or_decode(_p(pool), D, Hq, Hkv, k_codec, v_codec, _p(_c(sign_bits, np.uint32)), _p(bt),
                    bt.shape[1], _p(cl), _p(q), float(alpha), _p(pairs), pairs.shape[0], _p(out))
    return out.reshape(B, Hq, D) if full else out


def dequant(pool, D, Hkv, sign_bits, block_table, context_lens, Lmax, basis, k_codec=0, v_codec=0):
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    B = cl.shape[0]
    ko = np.empty((B, Hkv, Lmax, D), np.float32)
    vo = np.empty((B, Hkv, Lmax, D), np.float32)
    lib().or_dequant(_p(pool), D, Hkv, k_codec, v_codec, _p(_c(sign_bits, np.uint32)), _p(bt),
                     bt.shape[1], _p(cl), B, Lmax, basis, _p(ko), _p(vo))
    return ko, vo


def decode_sparse_v(pool, D, Hq, Hkv, sign_bits, block_table, context_lens, q, alpha, thr,
                    pairs=None, k_codec=0, v_codec=0):
    """Exact-weight sparse values: (out_sparse, bound) per (b, hq) pair (default: all), out
    fp64 original basis; see or_decode_sparse_v."""
    q = _c(q, np.float32)
    B = q.shape[0]
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    full = pairs is None
    if full:
        pairs = np.array([(b, h) for b in range(B) for h in range(Hq)], np.int32)
    pairs = _c(pairs, np.int32).reshape(-1, 2)
    out = np.empty((pairs.shape[0], D), np.float64)
    bound = np.empty(pairs.shape[0], np.float64)
    lib().or_decode_sparse_v(_p(pool), D, Hq, Hkv, k_codec, v_codec, _p(_c(sign_bits, np.uint32)),
                             _p(bt), bt.shape[1], _p(cl), _p(q), float(alpha), float(thr), _p(pairs),
                             pairs.shape[0], _p(out), _p(bound))
    if full:
        return out.reshape(B, Hq, D), bound.reshape(B, Hq)
    return out, bound


def decode_hotcold(pool, D, Hq, Hkv, sign_bits, block_table, cold_lens, hot_k, hot_v, hot_lens, q,
                   alpha, pairs=None, k_codec=0, v_codec=0):
    """fp64 decode over cold (pool) + hot tokens; hot_k, hot_v: [B, Hkv, hot_cap, D] fp16 (or
    their uint16 bits), original basis. Returns [B, Hq, D] (or [n_pairs, D])."""
    q = _c(q, np.float32)
    B = q.shape[0]
    bt = _c(block_table, np.int32)
    cl = _c(cold_lens, np.int32)
    hl = _c(hot_lens, np.int32)
    hk = np.ascontiguousarray(hot_k).view(np.uint16)
    hv = np.ascontiguousarray(hot_v).view(np.uint16)
    full = pairs is None
    if full:
        pairs = np.array([(b, h) for b in range(B) for h in range(Hq)], np.int32)
    pairs = _c(pairs, np.int32).reshape(-1, 2)
    out = np.empty((pairs.shape[0], D), np.float64)
    lib().or_decode_hotcold(_p(pool), D, Hq, Hkv, k_codec, v_codec, _p(_c(sign_bits, np.uint32)), _p(bt),
                            bt.shape[1], _p(cl), _p(hk), _p(hv), _p(hl), hk.shape[2], _p(q), float(alpha),
                            _p(pairs), pairs.shape[0], _p(out))
    return out.reshape(B, Hq, D) if full else out
