"""NumPy brute force for pinning the CPU oracle on tiny inputs.

An independent formulation of the same rules, written from the format
definitions and the pages' description, not from the oracle's code:

* encoders are a nearest-value search over every code of the right sign
  (argmin of exact distances, each held as a float64 TwoSum pair; ties go to
  the code whose mantissa bit is 0); satfinite falls out because the largest
  finite value is the nearest one for anything beyond it;
* decoders are built from the OCP MX E2M1 / E4M3 value definitions;
* the gather walk is a linear scan over requests for every row;
* entries are assembled as whole byte arrays and scattered with fancy indexing.

Only for small inputs (memory is O(n * codes)).
"""
import numpy as np

from synth import bf16_to_f32

# OCP MX E2M1: magnitudes of codes 0..7.
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e4m3_mag():
    """OCP E4M3FN magnitudes of codes 0..126 (code 127 is NaN)."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        out.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


E4M3_MAG = _e4m3_mag()


def _exact_distance(a, g):
    """|a - g| as an unevaluated pair (s, e) with s + e exact (Knuth's
    TwoSum in float64), so that distances compare exactly even when |a| is
    so large that a - g rounds to the same float64 for every grid value g."""
    b = -g
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    neg = (s < 0) | ((s == 0) & (e < 0))
    return np.where(neg, -s, s), np.where(neg, -e, e)


def _nearest(y, mags, sign_bit):
    y = np.asarray(y, dtype=np.float32).ravel()
    a = np.abs(y.astype(np.float64))
    out = np.empty(y.shape, np.uint8)
    step = max(1, 2_000_000 // mags.size)
    even = (2 - (np.arange(mags.size) % 2))[None, :]
    for lo in range(0, y.size, step):
        s, e = _exact_distance(a[lo:lo + step, None], mags[None, :])
        cand = s == s.min(axis=1, keepdims=True)
        e = np.where(cand, e, np.inf)
        cand &= e == e.min(axis=1, keepdims=True)
        # among equally near codes prefer the even one (mantissa LSB 0)
        out[lo:lo + step] = (cand * even).argmax(axis=1)
    return (out | np.where(np.signbit(y), sign_bit, 0)).astype(np.uint8)


def e2m1_encode(y):
    return _nearest(y, E2M1_MAG, 0x8).reshape(np.shape(y))


def e4m3_encode(y):
    return _nearest(y, E4M3_MAG, 0x80).reshape(np.shape(y))


def e2m1_value(code):
    code = np.asarray(code)
    v = E2M1_MAG[code & 7]
    return np.where(code & 8, -v, v)


def e4m3_value(code):
    code = np.asarray(code).astype(np.int64)
    mag = np.concatenate([E4M3_MAG, [np.nan]])[code & 0x7F]
    return np.where(code & 0x80, -mag, mag)


def to_bf16_bits(x32):
    """float32 -> bf16 bits by exhaustive neighbour choice: compare the value
    with both neighbouring bf16 values in float64, ties to the even pattern."""
    x32 = np.asarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lo = (u >> 16).astype(np.uint64)                 # truncated (toward zero)
    hi = lo + 1                                      # next away from zero
    vlo = ((lo << 16).astype(np.uint32)).view(np.float32).astype(np.float64)
    vhi = ((hi << 16).astype(np.uint32)).view(np.float32).astype(np.float64)
    # IEEE overflow: past the largest finite bf16 the next value counts as
    # 2^128 (rounding there gives infinity, whose pattern hi already is).
    vhi = np.where(np.isinf(vhi), np.copysign(2.0 ** 128, vhi), vhi)
    xv = x32.astype(np.float64)
    dlo, dhi = np.abs(xv - vlo), np.abs(vhi - xv)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


# ---------------------------------------------------------------------------
def walk(total, block_table, ws, seq_starts, block_size):
    """(block id, offset) of every row by linear scan over the requests."""
    B = ws.shape[0]
    blk = np.empty(total, np.int64)
    off = np.empty(total, np.int64)
    for r in range(total):
        req = max(b for b in range(B) if ws[b] <= r)
        pos = int(seq_starts[req]) + r - int(ws[req])
        blk[r] = block_table[req, pos // block_size]
        off[r] = pos % block_size
    return blk, off


def nvfp4_ds_mla_entries(kv_c_bits, k_pe_bits):
    """[T, 352] entries: NoPE nibbles, e4m3 RoPE, e4m3 block scales."""
    x = bf16_to_f32(kv_c_bits).reshape(-1, 32, 16)
    amax = np.abs(x).max(axis=2)
    sf = e4m3_encode(amax / np.float32(6.0))
    s = e4m3_value(sf).astype(np.float32)
    inv = np.where(s == 0, np.float32(0), np.float32(1) / np.where(s == 0, np.float32(1), s))
    q = e2m1_encode(x * inv[:, :, None].astype(np.float32)).reshape(-1, 256, 2)
    nope = (q[:, :, 0] | (q[:, :, 1] << 4)).astype(np.uint8)
    rope = e4m3_encode(bf16_to_f32(k_pe_bits))
    return np.concatenate([nope, rope, sf], axis=1)


def fp8_ds_mla_entries(kv_c_bits, k_pe_bits):
    """[T, 656] entries: e4m3 NoPE, 4 fp32 scales (LE), raw bf16 RoPE (LE)."""
    x = bf16_to_f32(kv_c_bits).reshape(-1, 4, 128)
    sc = (np.abs(x).max(axis=2) / np.float32(448.0)).astype(np.float32)
    inv = np.where(sc == 0, np.float32(0), np.float32(1) / np.where(sc == 0, np.float32(1), sc))
    q = e4m3_encode(x * inv[:, :, None].astype(np.float32)).reshape(-1, 512)
    scb = sc.astype('<f4').view(np.uint8).reshape(-1, 16)
    rb = np.ascontiguousarray(k_pe_bits).astype('<u2').view(np.uint8).reshape(-1, 128)
    return np.concatenate([q, scb, rb], axis=1)


def scatter(cache, entries, slots, block_size, block_stride, entry_stride):
    for t, s in enumerate(slots):
        if s < 0:
            continue
        a = (s // block_size) * block_stride + (s % block_size) * entry_stride
        cache[a:a + entries.shape[1]] = entries[t]


def nvfp4_rows(entries):
    """[R, 352] entries -> bf16 bits [R, 576]; the products are exact."""
    lo, hi = entries[:, :256] & 0xF, entries[:, :256] >> 4
    nib = np.stack([lo, hi], axis=2).reshape(-1, 512)
    sf = np.repeat(entries[:, 320:352], 16, axis=1)
    v = e2m1_value(nib) * e4m3_value(sf)
    rope = e4m3_value(entries[:, 256:320])
    return to_bf16_bits(np.concatenate([v, rope], axis=1).astype(np.float32))


def fp8_rows(entries):
    """[R, 656] entries -> bf16 bits [R, 576]: binary32 product, then bf16."""
    sc = np.ascontiguousarray(entries[:, 512:528]).view('<f4').astype(np.float32)
    v = (e4m3_value(entries[:, :512]).astype(np.float32)
         * np.repeat(sc, 128, axis=1)).astype(np.float32)
    rope = np.ascontiguousarray(entries[:, 528:656]).view('<u2')
    return np.concatenate([to_bf16_bits(v), rope.astype(np.uint16)], axis=1)


def read_entries(cache, blk, off, block_stride, entry_stride, nbytes):
    idx = (blk * block_stride + off * entry_stride)[:, None] + np.arange(nbytes)[None, :]
    return cache[idx]


# ---------------------------------------------------------------------------
def kv_quantize(x_bits, gs):
    """[..., hs] bf16 bits -> (data [..., hs/2], scales [..., hs/16])."""
    hs = x_bits.shape[-1]
    x = bf16_to_f32(x_bits).reshape(-1, hs // 16, 16)
    gs = np.float32(gs)
    amax = np.abs(x).max(axis=2)
    sf = e4m3_encode((amax / np.float32(6.0)) / gs)
    e = (e4m3_value(sf).astype(np.float32) * gs).astype(np.float32)
    inv = np.where(e == 0, np.float32(0), np.float32(1) / np.where(e == 0, np.float32(1), e))
    q = e2m1_encode(x * inv[:, :, None].astype(np.float32)).reshape(-1, hs // 2, 2)
    data = (q[:, :, 0] | (q[:, :, 1] << 4)).astype(np.uint8)
    shape = x_bits.shape[:-1]
    return data.reshape(*shape, hs // 2), sf.reshape(*shape, hs // 16)


def kv_dequant(data, scales, gs):
    """(data [..., hs/2], scales [..., hs/16]) -> bf16 bits [..., hs]."""
    hs = data.shape[-1] * 2
    nib = np.stack([data & 0xF, data >> 4], axis=-1).reshape(*data.shape[:-1], hs)
    prod = (e2m1_value(nib) * e4m3_value(np.repeat(scales, 16, axis=-1))).astype(np.float32)
    return to_bf16_bits((prod * np.float32(gs)).astype(np.float32))
