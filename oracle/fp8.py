"""FP8 (OCP e4m3) pieces of the FP8 attention path, for the CPU oracle.

Test infrastructure only (see the package docstring).

[FA3-report] sections 2.2 and 3.3 describe the FP8 forward:
  * block quantisation -- one scale per Br x d block of Q and per Bc x d block
    of K and V, with the scaling of each S block folded in at no extra cost;
  * incoherent processing -- Q and K are both multiplied by M = diag(+-1) . H,
    a random sign diagonal times a Hadamard matrix, applied in O(d log d);
    M M^T = I so Q K^T is unchanged while outliers are spread over the row.
[FA3-blog] section 3.2: e4m3 is the format for activations.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):
  * M = diag(s) H_d / sqrt(d) with the Sylvester H_d, applied to row vectors:
    x' = x diag(s) H_d / sqrt(d).  V is not rotated.
  * The format is OCP e4m3 (max 448, no infinities), rounding to nearest even,
    saturating at +-448.
  * Block scale: amax of the block / 448.  The 1/sqrt(d) of M is folded into
    the stored scale, so the codes are taken from the unnormalised transform.
    A block whose amax is 0 stores scale 1; its codes are +-0, the sign of
    each zero following IEEE-754 arithmetic through the transform.
  * The quantise decision is taken in fp32, the kernel's precision: the
    transform is the textbook butterfly in fp32 with strides 1, 2, 4, ...,
    r = fp32(448 / amax) and code = e4m3(fp32(y * r)).
  * P = exp(S - m) is rounded to e4m3 against the running max m of the
    online softmax (the value the kernel rounds); l sums the unrounded P.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import kv_head

E4M3_MAX = 448.0
QBLOCK = 128  # rows per quantisation block (Br = Bc = 128, [FA3-blog] section 3.1)


def e4m3_decode_table() -> np.ndarray:
    """float64[256]: the value of every OCP e4m3 code (NaN for S.1111.111).

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field 0
    encodes subnormals m * 2^-9; there is no infinity.
    """
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** -9
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_TABLE = e4m3_decode_table()
_MAGS = _TABLE[:127].copy()  # codes 0x00..0x7E, increasing magnitudes 0 .. 448


def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest e4m3 code, ties to even, saturating at +-448.

    Negative inputs that round to zero give -0 (0x80).  Works on the exact
    value of each float32/float64 input (all midpoints of e4m3 are exact in
    float64).  Returns uint8 codes.  NaN input is rejected.
    """
    a = np.asarray(x, dtype=np.float64)
    if np.isnan(a).any():
        raise ValueError("NaN cannot be encoded")
    mag = np.minimum(np.abs(a), E4M3_MAX)
    hi = np.searchsorted(_MAGS, mag, side="left")  # _MAGS[hi-1] < mag <= _MAGS[hi]
    hi = np.clip(hi, 1, 126)
    lo = hi - 1
    dlo = mag - _MAGS[lo]
    dhi = _MAGS[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(mag == 0.0, 0, np.where(pick_hi, hi, lo)).astype(np.uint8)
    # the sign bit follows the operand, also when the magnitude rounds to zero
    # (IEEE-754 rounding keeps the sign; e4m3 has both +0 and -0)
    return np.where(np.signbit(a), code | 0x80, code).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def fwht(x, axis: int = -1) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along ``axis`` (y = x H_d).

    Textbook in-place butterfly: for stride h = 1, 2, 4, ..., d/2 every pair
    (a, b) = (x[j], x[j+h]) with (j mod 2h) < h becomes (a + b, a - b).  The
    arithmetic stays in the input dtype, so float32 input gives the float32
    rounding of exactly this sequence of adds.
    """
    y = np.moveaxis(np.array(x, copy=True), axis, -1)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(lead + (d,))
        h *= 2
    return np.moveaxis(y, -1, axis)


def sylvester_hadamard(d: int) -> np.ndarray:
    """Dense Sylvester Hadamard matrix H_d (entries +-1), float64."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != d:
        raise ValueError("d must be a power of two")
    return h


def rotate_fp64(x, signs) -> np.ndarray:
    """x M with M = diag(signs) H_d / sqrt(d), in fp64 (dense product)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    m = np.asarray(signs, dtype=np.float64)[:, None] * sylvester_hadamard(d) / math.sqrt(d)
    return x @ m


def _num_blocks(n: int) -> int:
    return (n + QBLOCK - 1) // QBLOCK


def blockquant_hadamard(x, signs=None, block_rows: int = QBLOCK):
    """Emulates the FP8 pre-pass on one BSHD tensor.

    x: float32-valued BSHD array (bf16 inputs upcast).  signs: d values of
    +-1, or None for no rotation (V, and the per-tensor baseline).
    block_rows: 128 for per-block scales, 0 for one scale per tensor.

    Returns (codes uint8 BSHD, scales float32 [B, H, ceil(N/128)]).  The
    dequantised value code * scale approximates x M (or x without rotation).
    With block_rows=0 every slot holds the single tensor-wide scale.
    """
    if block_rows not in (0, QBLOCK):
        raise ValueError("block_rows must be 0 or 128")
    x32 = np.asarray(x, dtype=np.float32)
    B, N, H, d = x32.shape
    if signs is not None:
        y = fwht(x32 * np.asarray(signs, dtype=np.float32), axis=-1)
        kconst = np.float32(1.0 / (E4M3_MAX * math.sqrt(d)))
    else:
        y = x32.copy()
        kconst = np.float32(1.0 / E4M3_MAX)
    nb = _num_blocks(N)
    codes = np.empty(y.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)

    def quant(blk):
        amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
        if amax == 0:  # all (signed) zeros: coded with r = 1, scale 1
            return e4m3_encode(blk), np.float32(1.0)
        r = np.float32(E4M3_MAX) / amax
        return e4m3_encode((blk * r).astype(np.float32)), np.float32(amax * kconst)

    if block_rows == 0:
        c, s = quant(y)
        codes[...] = c
        scales[...] = s
        return codes, scales
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                r0, r1 = j * QBLOCK, min(N, (j + 1) * QBLOCK)
                c, s = quant(y[b, r0:r1, h, :])
                codes[b, r0:r1, h, :] = c
                scales[b, h, j] = s
    return codes, scales


def dequantize(codes, scales) -> np.ndarray:
    """code * scale of its 128-row block, fp64 BSHD."""
    vals = e4m3_decode(codes)
    B, N, H, d = vals.shape
    per_row = np.repeat(np.asarray(scales, np.float64), QBLOCK, axis=2)[:, :, :N]  # [B,H,N]
    return vals * np.transpose(per_row, (0, 2, 1))[..., None]


def fp8_attention_emulation(q8, k8, v8, sq, sk, sv, scale: float, causal: bool,
                            Bc: int = QBLOCK, quantize_p: bool = True, rows=None,
                            observer=None):
    """FP8 attention forward as the FP8 path computes it, in fp64.

    Inputs are e4m3 codes (BSHD) and per-128-row block scales [B,H,ceil(N/128)];
    K/V codes and scales may have H_kv heads (query head h then reads K/V head
    h // (H // H_kv), as in ``oracle.attention.kv_head``).
    The online-softmax recurrence of ``oracle.attention.tiled_attention`` runs
    over key blocks of Bc, with:
      S_j = (Q8 K8_j^T) * sQ * sK_j * scale  (block scaling of S, [FA3-report] 3.3)
      P_j = exp(S_j - m')                     m' = running row max
      l   = exp(m - m') l + rowsum P_j        (unrounded P)
      O   = exp(m - m') O + e4m3(P_j) (V8_j * sV_j)
    Returns (O, LSE) for all rows (O BSHD, LSE [B,H,N]) or, when ``rows``
    ([R,3] of (b,h,i)) is given, (O_rows [R,d], LSE_rows [R]).

    observer: optional callable, called after each key block with
    (b, h, g, qi_idx, keys, s, m_new, p, alpha): the K/V head g, the query
    rows, the block's keys, its scores S_j, the running max m' after it, the
    unrounded P block and the rescale factor exp(m - m').  It only watches
    (the tests derive error bounds from it); the result does not depend on it.
    """
    qv, kv, vv = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    B, N, H, d = qv.shape
    Nk, Hkv = kv.shape[1], kv.shape[2]
    sq = np.asarray(sq, np.float64)
    sk = np.asarray(sk, np.float64)
    sv = np.asarray(sv, np.float64)

    def one(b, h, qi_idx):
        g = kv_head(h, H, Hkv)
        qi = qv[b, qi_idx, h, :]
        sqr = sq[b, h, qi_idx // QBLOCK]
        m = np.full(len(qi_idx), -np.inf)
        l = np.zeros(len(qi_idx))
        acc = np.zeros((len(qi_idx), vv.shape[3]))
        for c0 in range(0, Nk, Bc):
            c1 = min(Nk, c0 + Bc)
            if causal and c0 > qi_idx.max():
                break
            keys = np.arange(c0, c1)
            skc = sk[b, g, keys // QBLOCK]
            svc = sv[b, g, keys // QBLOCK]
            s = (qi @ kv[b, c0:c1, g, :].T) * (sqr[:, None] * skc[None, :]) * scale
            if causal:
                s[keys[None, :] > qi_idx[:, None]] = -np.inf
            m_new = np.maximum(m, np.max(s, axis=1))
            p = np.exp(s - m_new[:, None])
            alpha = np.exp(m - m_new)
            l = alpha * l + np.sum(p, axis=1)
            pq = e4m3_decode(e4m3_encode(p)) if quantize_p else p
            acc = alpha[:, None] * acc + pq @ (vv[b, c0:c1, g, :] * svc[:, None])
            m = m_new
            if observer is not None:
                observer(b, h, g, qi_idx, keys, s, m_new, p, alpha)
        return acc / l[:, None], m + np.log(l)

    if rows is not None:
        rows = np.asarray(rows, np.int64)
        oo = np.empty((rows.shape[0], vv.shape[3]))
        ll = np.empty(rows.shape[0])
        keys_bh = rows[:, 0] * H + rows[:, 1]
        for key in np.unique(keys_bh):
            sel = np.nonzero(keys_bh == key)[0]
            b, h = int(rows[sel[0], 0]), int(rows[sel[0], 1])
            oo[sel], ll[sel] = one(b, h, rows[sel, 2])
        return oo, ll
    o = np.empty((B, N, H, vv.shape[3]))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, QBLOCK):
                idx = np.arange(r0, min(N, r0 + QBLOCK))
                o[b, idx, h, :], lse[b, h, idx] = one(b, h, idx)
    return o, lse
