"""NumPy oracle: a second, separately written CPU reference. Test infrastructure only.

It implements the same readings as tq_oracle.c (listed in that file's header) without
sharing any code with it, so that the two can be compared byte for byte:

  * rotation  [Open-TQ-Metal, card abstract: sign-randomized transform; "TurboQuant on
    AMD GPUs", section 4: Walsh-Hadamard] - fp32, stride-ascending butterfly, then rho;
  * abs-max int4 [Open-TQ-Metal, card abstract; "TurboQuant on AMD GPUs", section 2,
    uniform V] - s = fp16(absmax/7), c = clamp(rint(y/s), -7, 7), index u = c + 8;
  * LUT int4 for keys ["TurboQuant on AMD GPUs", section 2: rotation + LUT] - Lloyd-Max
    N(0,1) centroids / sqrt(32) in fp16 times the fp16 group L2 norm;
  * attention in fp64 on the dequantized rotated values [Open-TQ-Metal, arXiv abstract],
    then the fp64 inverse rotation;
  * fp16 keys (k_codec 2) [mlxcel "TurboQuant KV cache" manual, cache-mode table: keys in
    fp16, values in the 4-bit rotated form] - fp16(k) of the original key, saturated; the
    scores use the query as given (no rotation), the values are as above;
  * 3-bit and 2-bit values (v_codec 3 and 4) [mlxcel manual, cache-mode table: fp16+turbo3;
    "TurboQuant on AMD GPUs", section 2: 2-bit is possible] - abs-max with the largest
    level 3 or 1 instead of 7, index u = c + 4 or c + 2, packed as the block comment
    below describes.

numpy's float32 arithmetic is IEEE single precision and its float16 casts round to
nearest even with subnormals, which is what the readings ask for.
"""
import math

import numpy as np

PAGE = 16
GROUP = 32

F32 = np.float32


def signs(sign_bits, D):
    """+1/-1 per coordinate; bit i of the packed words set means -1."""
    sb = np.asarray(sign_bits, np.uint32)
    bits = (sb[np.arange(D) // 32] >> (np.arange(D) % 32).astype(np.uint32)) & 1
    return np.where(bits == 1, -1.0, 1.0)


def rho32(D):
    return F32(1.0 / math.sqrt(D))


def hadamard_f32(y):
    """Unnormalized Walsh-Hadamard butterfly on the last axis, fp32, stride 1, 2, 4, ..."""
    y = np.array(y, dtype=F32, copy=True)
    D = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < D:
        z = y.reshape(lead + (D // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(lead + (D,))
        h *= 2
    return y


def rotate(x, sign_bits):
    x = np.asarray(x, F32)
    s = signs(sign_bits, x.shape[-1]).astype(F32)
    return hadamard_f32(x * s) * rho32(x.shape[-1])


def unrotate_f32(y, sign_bits):
    y = np.asarray(y, F32)
    s = signs(sign_bits, y.shape[-1]).astype(F32)
    return (hadamard_f32(y) * rho32(y.shape[-1])) * s


def unrotate_f64(y, sign_bits):
    y = np.array(y, dtype=np.float64, copy=True)
    D = y.shape[-1]
    h = 1
    while h < D:
        z = y.reshape(y.shape[:-1] + (D // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape[:-1] + (D,))
        h *= 2
    return y / math.sqrt(D) * signs(sign_bits, D)


def to_f16_sat(x):
    """fp16 round-to-nearest-even, with overflow clamped to the largest finite value."""
    with np.errstate(over="ignore"):
        h = np.asarray(x).astype(np.float16)
    return np.where(np.isinf(h), np.copysign(np.float16(65504.0), h), h).astype(np.float16)


QMAX = {0: 7, 3: 3, 4: 1}    # largest abs-max level per codec (4, 3, 2 bits)
VBITS = {0: 4, 1: 4, 3: 3, 4: 2}


def quant_absmax(y, group=GROUP, qmax=7):
    """y [..., D] rotated fp32 -> (u [..., D] uint8 in 1..2*qmax+1, scales [..., D/group] fp16)."""
    y = np.asarray(y, F32)
    D = y.shape[-1]
    yg = y.reshape(y.shape[:-1] + (D // group, group))
    a = np.max(np.abs(yg), axis=-1)
    s16 = to_f16_sat(a / F32(qmax))
    sf = s16.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint(yg / np.where(sf == 0, F32(1.0), sf))
    c = np.clip(c, -qmax, qmax)
    c = np.where(sf == 0, 0, c)
    u = (c + qmax + 1).astype(np.uint8).reshape(y.shape)
    return u, s16


def lloydmax16(iters=200000, tol=1e-15):
    """16-level Lloyd-Max centroids of N(0,1) by Lloyd's iteration in fp64, and the MSE."""
    from scipy.special import ndtr

    def cdf(x):
        return ndtr(x)

    def pdf(x):
        return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)

    c = np.linspace(-2.8, 2.8, 16)
    for _ in range(iters):
        t = np.concatenate(([-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]))
        pa, pb = pdf(t[:-1]), pdf(t[1:])
        mass = cdf(t[1:]) - cdf(t[:-1])
        nc = (pa - pb) / mass
        done = np.max(np.abs(nc - c)) < tol
        c = nc
        if done:
            break
    c = 0.5 * (c - c[::-1])
    t = np.concatenate(([-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]))
    mass = cdf(t[1:]) - cdf(t[:-1])
    with np.errstate(invalid="ignore"):
        ta = np.where(np.isinf(t[:-1]), 0.0, t[:-1] * pdf(t[:-1]))
        tb = np.where(np.isinf(t[1:]), 0.0, t[1:] * pdf(t[1:]))
    m1 = pdf(t[:-1]) - pdf(t[1:])
    m2 = mass - (tb - ta)
    mse = float(np.sum(m2 - 2 * c * m1 + c * c * mass))
    return c, mse


def lut16():
    c, _ = lloydmax16()
    return (c / math.sqrt(32.0)).astype(np.float16)


def quant_lut(y, lut=None, group=GROUP):
    """y [..., D] -> (u [..., D] uint8 in 0..15, group norms [..., D/group] fp16)."""
    lut = lut16() if lut is None else np.asarray(lut, np.float16)
    y = np.asarray(y, F32)
    D = y.shape[-1]
    yg = y.reshape(y.shape[:-1] + (D // group, group))
    t = yg * yg
    off = group // 2
    while off >= 1:
        t = t[..., :off] + t[..., off:2 * off]
        off //= 2
    n16 = to_f16_sat(np.sqrt(t[..., 0]))
    nf = n16.astype(F32)[..., None]
    lf = lut.astype(F32)
    thr = (lf[:-1] + lf[1:]) * F32(0.5)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = yg / np.where(nf == 0, F32(1.0), nf)
    u = np.sum(v[..., None] >= thr, axis=-1)
    u = np.where(nf == 0, 8, u).astype(np.uint8).reshape(y.shape)
    return u, n16


def encode(x, sign_bits, codec=0, group=GROUP):
    y = rotate(x, sign_bits)
    return quant_lut(y, group=group) if codec == 1 else quant_absmax(y, group, QMAX[codec])


def dequant_values(u, s16, codec=0, lut=None, group=GROUP):
    """Indices + scales -> fp64 values in the rotated basis."""
    u = np.asarray(u)
    D = u.shape[-1]
    s = np.repeat(np.asarray(s16, np.float16).astype(np.float64), group, axis=-1)
    if codec != 1:
        return (u.astype(np.float64) - float(QMAX[codec] + 1)) * s
    lut = lut16() if lut is None else lut
    return lut.astype(np.float64)[u] * s


# ---- pool placement ----------------------------------------------------------------------
# Block of one page and one KV head, G = D/32 groups:
#   [K indices 8D B][V indices 8D B][K scales 16xG fp16][V scales 16xG fp16]
# K index of (t, d = 32g + 8j + e): byte (16j + t)*4G + 4g + e//2, high nibble iff e odd.
# V index of (t = 4j + e, d): column c = d//2 = 16g + m, byte 8D + (16j + m)*4G + 4g + e,
#   high nibble iff d odd.

KF16 = 2


def block_bytes(D, k_codec=0, v_codec=0):
    vb = 2 * VBITS[v_codec] * D  # V index bytes of 16 tokens
    if k_codec == KF16:
        return 32 * D + vb + D   # [K fp16 32D][V indices][V scales 16 x G fp16]
    return 8 * D + vb + 2 * D    # [K indices 8D][V indices][K scales][V scales]


# 3-bit and 2-bit value indices. The 16 tokens' 4-bit V region would be 64 rows of G
# little-endian dwords (row 16j + m, dword g: tokens 4j..4j+3 at bytes 0..3, dims
# 32g + 2m (low nibble) and 32g + 2m + 1 (high nibble)). With b bits, the two low bits of
# each nibble of dwords g = 2i, 2i + 1 of a row share one dword X[row][i] (dword 2i in
# bits 0-1 of every nibble, 2i + 1 in bits 2-3); for b = 3 the third bits of all rows
# follow as dwords Z, where dword g of row r lands in Z[(r*G + g) // 4] at bit
# (r*G + g) % 4 of every nibble.
def _nibble_rows(D):
    """(row, dword g, nibble n) of every (t, d) in the 4-bit V layout, each [16, D]."""
    d = np.arange(D)
    t = np.arange(PAGE)[:, None]
    c = d // 2
    g, m = c // 16, c % 16
    row = 16 * (t // 4) + m
    n = 2 * (t % 4) + d % 2
    return np.broadcast_to(row, (PAGE, D)), np.broadcast_to(g, (PAGE, D)), n


def _vpack(u, D, bits):
    """u [16, D] indices -> the V region bytes for b = 3 or 2."""
    G = D // 32
    row, g, n = _nibble_rows(D)
    u = np.asarray(u, np.uint32)
    X = np.zeros((64, G // 2 if G >= 2 else 1), np.uint32)
    np.bitwise_or.at(X, (row, g // 2), (u & 3) << (4 * n + 2 * (g % 2)).astype(np.uint32))
    out = [X.reshape(-1)]
    if bits == 3:
        z = row * G + g
        Z = np.zeros(16 * G, np.uint32)
        np.bitwise_or.at(Z, z // 4, ((u >> 2) & 1) << (4 * n + z % 4).astype(np.uint32))
        out.append(Z)
    return np.concatenate(out).astype("<u4").view(np.uint8)


def _vunpack(reg, D, bits):
    G = D // 32
    row, g, n = _nibble_rows(D)
    w = np.asarray(reg, np.uint8).copy().view("<u4").astype(np.uint32)
    X = w[:32 * G].reshape(64, -1)
    u = (X[row, g // 2] >> (4 * n + 2 * (g % 2)).astype(np.uint32)) & 3
    if bits == 3:
        z = row * G + g
        Z = w[32 * G:]
        u = u | (((Z[z // 4] >> (4 * n + z % 4).astype(np.uint32)) & 1) << 2)
    return u.astype(np.uint8)


def _k_index(D):
    d = np.arange(D)
    t = np.arange(PAGE)[:, None]
    G = D // 32
    g, j, e = d // 32, (d % 32) // 8, d % 8
    return (16 * j + t) * 4 * G + 4 * g + e // 2, np.broadcast_to(e % 2, (PAGE, D))


def _v_index(D):
    d = np.arange(D)
    t = np.arange(PAGE)[:, None]
    G = D // 32
    c = d // 2
    g, m = c // 16, c % 16
    j, e = t // 4, t % 4
    return 8 * D + (16 * j + m) * 4 * G + 4 * g + e, np.broadcast_to(d % 2, (PAGE, D))


def _kf16_index(D):
    """fp16-key block: byte of K (t, d = 32g + 8j + e) is 1024g + 16(16j + t) + 2e."""
    d = np.arange(D)
    t = np.arange(PAGE)[:, None]
    g, j, e = d // 32, (d % 32) // 8, d % 8
    return 1024 * g + 16 * (16 * j + t) + 2 * e


def new_pool(num_pages, Hkv, D, k_codec=0, v_codec=0):
    return np.zeros(num_pages * Hkv * block_bytes(D, k_codec, v_codec), np.uint8)


def _put_v(blk, base, D, v_codec, t, u):
    """Write token t's value indices into the V region at blk[base:]."""
    bits = VBITS[v_codec]
    if bits == 4:
        vb, vh = _v_index(D)
        vb = vb - 8 * D + base
        lo_sel, hi_sel = vh[t] == 0, vh[t] == 1
        blk[vb[t][lo_sel]] = (blk[vb[t][lo_sel]] & 0xF0) | u[lo_sel]
        blk[vb[t][hi_sel]] = (blk[vb[t][hi_sel]] & 0x0F) | (u[hi_sel] << 4)
        return
    nb = 2 * bits * D
    cur = _vunpack(blk[base:base + nb], D, bits)
    cur[t] = u
    blk[base:base + nb] = _vpack(cur, D, bits)


def _get_v(blk, base, D, v_codec):
    bits = VBITS[v_codec]
    if bits == 4:
        vb, vh = _v_index(D)
        vb = vb - 8 * D + base
        return np.where(vh == 1, blk[vb] >> 4, blk[vb] & 0x0F).astype(np.uint8)
    return _vunpack(blk[base:base + 2 * bits * D], D, bits)


def place_kf16(pool, D, Hkv, slots, kh, vu, vs, v_codec=0):
    """fp16-key pool: kh [n, Hkv, D] fp16 keys, V indices and scales as in place()."""
    G = D // 32
    bb = block_bytes(D, KF16, v_codec)
    kb = _kf16_index(D)
    vsoff = 32 * D + 2 * VBITS[v_codec] * D
    blocks = pool.reshape(-1, Hkv, bb)
    for i, slot in enumerate(np.asarray(slots, np.int64)):
        if slot < 0:
            continue
        page, t = divmod(int(slot), PAGE)
        for h in range(Hkv):
            blk = blocks[page, h]
            kbytes = np.asarray(kh[i, h], np.float16).view(np.uint8)
            blk[kb[t]] = kbytes[0::2]
            blk[kb[t] + 1] = kbytes[1::2]
            _put_v(blk, 32 * D, D, v_codec, t, np.asarray(vu[i, h], np.uint8))
            blk[vsoff + 2 * G * t:vsoff + 2 * G * (t + 1)] = np.asarray(vs[i, h], np.float16).view(np.uint8)


def fetch_block_kf16(pool, D, Hkv, page, h, v_codec=0):
    """fp16 keys [16, D], V indices [16, D] and V scales [16, G] of one fp16-key block."""
    G = D // 32
    blk = pool.reshape(-1, Hkv, block_bytes(D, KF16, v_codec))[page, h]
    kb = _kf16_index(D)
    vsoff = 32 * D + 2 * VBITS[v_codec] * D
    k = (blk[kb].astype(np.uint16) | (blk[kb + 1].astype(np.uint16) << 8)).view(np.float16)
    vu = _get_v(blk, 32 * D, D, v_codec)
    vs = blk[vsoff:vsoff + 32 * G].copy().view(np.float16).reshape(PAGE, G)
    return k, vu, vs


def place(pool, D, Hkv, slots, ku, ks, vu, vs, v_codec=0):
    """Write encoded tokens ([n, Hkv, D] indices, [n, Hkv, G] scales) at their slots."""
    G = D // 32
    bb = block_bytes(D, 0, v_codec)
    kb, kh = _k_index(D)
    ksoff = 8 * D + 2 * VBITS[v_codec] * D
    blocks = pool.reshape(-1, Hkv, bb)
    for i, slot in enumerate(np.asarray(slots, np.int64)):
        if slot < 0:
            continue
        page, t = divmod(int(slot), PAGE)
        for h in range(Hkv):
            blk = blocks[page, h]
            u = np.asarray(ku[i, h], np.uint8)
            lo_sel, hi_sel = kh[t] == 0, kh[t] == 1     # one nibble per byte per pass
            blk[kb[t][lo_sel]] = (blk[kb[t][lo_sel]] & 0xF0) | u[lo_sel]
            blk[kb[t][hi_sel]] = (blk[kb[t][hi_sel]] & 0x0F) | (u[hi_sel] << 4)
            _put_v(blk, 8 * D, D, v_codec, t, np.asarray(vu[i, h], np.uint8))
            kscale = np.asarray(ks[i, h], np.float16).view(np.uint8)
            vscale = np.asarray(vs[i, h], np.float16).view(np.uint8)
            blk[ksoff + 2 * G * t:ksoff + 2 * G * (t + 1)] = kscale
            blk[ksoff + D + 2 * G * t:ksoff + D + 2 * G * (t + 1)] = vscale


def append(pool, D, Hkv, k, v, slots, sign_bits, k_codec=0, v_codec=0):
    vu, vs = encode(v, sign_bits, v_codec)
    if k_codec == KF16:
        place_kf16(pool, D, Hkv, slots, to_f16_sat(np.asarray(k, F32)), vu, vs, v_codec)
        return
    ku, ks = encode(k, sign_bits, k_codec)
    place(pool, D, Hkv, slots, ku, ks, vu, vs, v_codec)


def fetch_block(pool, D, Hkv, page, h, v_codec=0):
    """Indices and scales of the 16 tokens of one block, natural order."""
    G = D // 32
    blk = pool.reshape(-1, Hkv, block_bytes(D, 0, v_codec))[page, h]
    kb, kh = _k_index(D)
    ksoff = 8 * D + 2 * VBITS[v_codec] * D
    ku = np.where(kh == 1, blk[kb] >> 4, blk[kb] & 0x0F).astype(np.uint8)
    vu = _get_v(blk, 8 * D, D, v_codec)
    ks = blk[ksoff:ksoff + 32 * G].copy().view(np.float16).reshape(PAGE, G)
    vs = blk[ksoff + D:ksoff + D + 32 * G].copy().view(np.float16).reshape(PAGE, G)
    return ku, ks, vu, vs


def gather(pool, D, Hkv, block_table, L, b, h, k_codec=0, v_codec=0):
    """Dequantized K, V (fp64; rotated basis, fp16 keys as stored) of the first L tokens of
    sequence b, head h."""
    npg = -(-L // PAGE)
    ks_, vs_ = [], []
    lut = lut16()
    for p in range(npg):
        if k_codec == KF16:
            k16, vu, vs = fetch_block_kf16(pool, D, Hkv, int(block_table[b][p]), h, v_codec)
            ks_.append(k16.astype(np.float64))
        else:
            ku, ks, vu, vs = fetch_block(pool, D, Hkv, int(block_table[b][p]), h, v_codec)
            ks_.append(dequant_values(ku, ks, k_codec, lut))
        vs_.append(dequant_values(vu, vs, v_codec, lut))
    if npg == 0:
        return np.zeros((0, D)), np.zeros((0, D))
    return np.concatenate(ks_)[:L], np.concatenate(vs_)[:L]


def attention_f64(q, K, V, alpha):
    if K.shape[0] == 0:
        return np.zeros(q.shape[-1])
    s = alpha * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def decode(pool, D, Hq, Hkv, sign_bits, block_table, context_lens, q, alpha, k_codec=0,
           v_codec=0):
    """fp64 decode attention for every (b, hq); q [B, Hq, D] fp32. Returns [B, Hq, D]."""
    q = np.asarray(q, F32)
    B = q.shape[0]
    r = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hkv):
            K, V = gather(pool, D, Hkv, block_table, int(context_lens[b]), b, h, k_codec, v_codec)
            for hq in range(h * r, (h + 1) * r):
                if k_codec == KF16:   # fp16 keys stay in the original basis
                    qr = q[b, hq].astype(np.float64)
                else:
                    qr = rotate(q[b, hq], sign_bits).astype(np.float64)
                o1 = attention_f64(qr, K, V, float(np.float32(alpha)))
                out[b, hq] = unrotate_f64(o1, sign_bits)
    return out
