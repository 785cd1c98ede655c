"""CPU oracle for the rotated W4A4 linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  The GPU library never imports, links or calls it, and it shares
no code with the GPU library (no kernels, tables, constants or helpers).

What it computes, in plain fp64 numpy, following the pages:

    Y = dequant( Q(X . R) . Q(W . R^{-T})^T )   [+ X_out . W_out^T]

Pages cited (title, then the section on it):
  [QS]   "QuaRot & SpinQuant" blog (chenghuawang.github.io): section 1
         "Computational Invariance", section 2 "QuaRot", section 3 "SpinQuant".
  [FQ]   FlatQuant article ("LLM量化新篇章 ... FlatQuant的平坦之道"): section 2.2
         (pivot tokens), section 2.3 "方法概述" (affine transform, Kronecker
         decomposition, per-channel scaling, clipping thresholds), section 3
         "实验结果" (quantization setting).
  [GSR]  "Grouped Sequency-arranged Rotation" abstract page: the English
         abstract and the method summary (sequency-ordered Walsh-Hadamard,
         block-diagonal small Walsh blocks).
  [QUIK] "QUIK: LLM上的一种4-bit推理方法" (CSDN blog): "QUIK量化" part 1
         (workflow: outliers to FP16, per-token asymmetric activations,
         INT4 GEMM, dequant, FP16 outlier GEMM, sum), part 3 (outlier columns
         by infinity norm), part 4 (INT32 accumulation).
  [SQR]  SpinQuant OpenReview discussion (paperhub.cn): first reviewer Q1/A1
         (min-max quantizer range), Q2/A2 (R R^T = I), the QuIP# bound (W1/A1
         of the third reviewer).

Readings where the pages are silent or garbled are listed where they are
used; every one also appears in the design notes.

Pinning: every function here is checked by tests against closed forms,
invariants, special cases or brute force; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

QMAX_SYM4 = 7       # symmetric INT4 range [-7, 7]   ([SQR] Q1/A1, reading c1)
QMAX_ASYM4 = 15     # asymmetric INT4 range [0, 15]  ([QUIK] part 1, reading c4)
QMAX_SYM8 = 127     # the same forms at 8 bits (QUIK-8B; reading r22)
QMAX_ASYM8 = 255


def code_max(bits: int, asym: bool) -> int:
    """Code range of the min-max quantizers at 4 or 8 bits.

    [SQR] Q1/A1: symmetric codes span +-(2^{N-1} - 1); asymmetric codes span
    [0, 2^N - 1] ([QUIK] part 1 form, reading c4).  [QUIK] "QUIK量化" part 3
    and the QUIK-8B experiments: the sensitive down projection runs with
    8-bit weights and activations (reading r22).
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    return (1 << bits) - 1 if asym else (1 << (bits - 1)) - 1


# --------------------------------------------------------------------------
# Rotations R (dense fp64 matrices: the plain definition, no fast transform)
# --------------------------------------------------------------------------

def _popcount(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.int64)
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a >>= 1
    return c


def hadamard(n: int) -> np.ndarray:
    """Normalized Walsh-Hadamard matrix in natural (Sylvester) order.

    H[i, j] = (-1)^popcount(i & j) / sqrt(n).  [QS] section 2: QuaRot inserts
    Hadamard multiplications in the forward pass; the 1/sqrt(n) makes it
    orthogonal, which [QS] section 1 (computational invariance) and [SQR] Q2/A2
    (R R^T = I) require.
    """
    if n <= 0 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(n)
    sign = 1.0 - 2.0 * (_popcount(np.bitwise_and.outer(i, i)) & 1)
    return sign / np.sqrt(float(n))


def sign_changes(rows: np.ndarray) -> np.ndarray:
    """Number of sign changes along each row (the row's sequency)."""
    return np.sum(rows[:, :-1] * rows[:, 1:] < 0, axis=1)


def walsh_sequency(n: int) -> np.ndarray:
    """Sequency-ordered Walsh matrix: Hadamard rows sorted by sign-change count.

    [GSR] abstract: the Walsh-Hadamard transform with sequency ordering; row s
    is the Hadamard row that changes sign exactly s times.
    """
    h = hadamard(n)
    order = np.argsort(sign_changes(h), kind="stable")
    return h[order]


def block_diag(block: np.ndarray, count: int) -> np.ndarray:
    b = block.shape[0]
    r = np.zeros((b * count, b * count))
    for g in range(count):
        r[g * b:(g + 1) * b, g * b:(g + 1) * b] = block
    return r


def gsr_rotation(K: int, block: int) -> np.ndarray:
    """Grouped sequency-arranged rotation: blockdiag(Wal_block, ..., Wal_block).

    [GSR] abstract: block-diagonal matrices built from smaller Walsh blocks.
    Reading c7: activations are multiplied on the right, x' = x . R.
    """
    if K % block:
        raise ValueError("K must be a multiple of the GSR block")
    return block_diag(walsh_sequency(block), K // block)


def kron_affine(p1: np.ndarray, p2: np.ndarray, chan_scale: np.ndarray | None) -> np.ndarray:
    """FlatQuant activation transform R = diag(s) . (P1 kron P2).

    [FQ] section 2.3: a per-layer affine transform, decomposed as a Kronecker
    product of two small matrices, with a per-channel scale.  Reading c8: the
    scale multiplies channels first, the Kronecker product uses numpy's index
    convention, so x' = (x * s) . (P1 kron P2).
    """
    r = np.kron(np.asarray(p1, np.float64), np.asarray(p2, np.float64))
    if chan_scale is not None:
        r = np.asarray(chan_scale, np.float64)[:, None] * r
    return r


def rotation(kind: str, K: int, block: int = 0, p1=None, p2=None, chan_scale=None) -> np.ndarray:
    """Dense fp64 R for one of the online transforms ("none" is the identity)."""
    if kind == "hadamard":
        return hadamard(K)
    if kind == "gsr":
        return gsr_rotation(K, block)
    if kind == "kron":
        return kron_affine(p1, p2, chan_scale)
    if kind == "none":
        return np.eye(K)
    raise ValueError(kind)


def weight_transform(kind: str, K: int, block: int = 0, p1=None, p2=None, chan_scale=None) -> np.ndarray:
    """Matrix G with W' = W . G such that (X R)(W G)^T = X W^T, i.e. G = R^{-T}.

    [QS] section 1 (computational invariance): for an orthogonal Q the weight
    side takes the same rotation, G = R.  [FQ] section 2.3: the affine case
    uses the inverse transform on the weights; with R = diag(s)(P1 kron P2),
    R^{-T} = diag(1/s) (P1^{-T} kron P2^{-T}) (Kronecker inverse/transpose).
    """
    if kind in ("hadamard", "gsr", "none"):
        return rotation(kind, K, block)
    if kind == "kron":
        g = np.kron(np.linalg.inv(np.asarray(p1, np.float64)).T,
                    np.linalg.inv(np.asarray(p2, np.float64)).T)
        if chan_scale is not None:
            g = g / np.asarray(chan_scale, np.float64)[:, None]
        return g
    raise ValueError(kind)


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def quantize_sym(xr: np.ndarray, clip=1.0, qmax: int = QMAX_SYM4):
    """Per-row symmetric min-max quantization.

    [SQR] Q1/A1: min-max scaling onto +-(2^{N-1}-1), so no clip is needed at
    clip = 1.  [FQ] section 3: weights per output channel, activations per
    token, both symmetric.  [FQ] section 2.3: a clipping threshold shrinks the
    range (reading c3: scale = clip * absmax / qmax, codes clamped to +-qmax).
    Scale rounded once to fp32; codes round half to even (reading c2).
    Zero rows get scale 0 and codes 0 (reading c5).

    Returns (codes int8 [rows, K], scale fp32 [rows], pre-round value fp64).
    """
    xr = np.asarray(xr, np.float64)
    clip64 = np.asarray(clip, np.float32).astype(np.float64)   # a scalar, or one ratio per row
    amax = np.max(np.abs(xr), axis=1) if xr.shape[1] else np.zeros(xr.shape[0])
    scale = (clip64 * amax / qmax).astype(np.float32)
    s64 = scale.astype(np.float64)[:, None]
    safe = np.where(s64 > 0, s64, 1.0)
    pre = np.where(s64 > 0, xr / safe, 0.0)
    q = np.clip(np.rint(pre), -qmax, qmax).astype(np.int8)
    return q, scale, pre


def quantize_asym(x: np.ndarray, qmax: int = QMAX_ASYM4):
    """Per-row asymmetric min-max quantization with an integer zero point.

    [QUIK] part 1: activations are quantized per token, asymmetric and
    dynamic.  Reading c4: lo = min(min x, 0), hi = max(max x, 0),
    scale = fp32((hi - lo)/qmax), zero = clamp(rne(-lo/scale), 0, qmax),
    code = clamp(rne(x/scale) + zero, 0, qmax); dequant = (code - zero)*scale.

    Returns (codes uint8, scale fp32, zero int32, pre-round x/scale, pre-round -lo/scale).
    """
    x = np.asarray(x, np.float64)
    rows = x.shape[0]
    if x.shape[1]:
        lo = np.minimum(x.min(axis=1), 0.0)
        hi = np.maximum(x.max(axis=1), 0.0)
    else:
        lo = hi = np.zeros(rows)
    scale = ((hi - lo) / qmax).astype(np.float32)
    s64 = scale.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    zpre = np.where(s64 > 0, -lo / safe, 0.0)
    zero = np.clip(np.rint(zpre), 0, qmax).astype(np.int32)
    pre = np.where(s64[:, None] > 0, x / safe[:, None], 0.0)
    q = np.clip(np.rint(pre) + zero[:, None], 0, qmax).astype(np.uint8)
    return q, scale, zero, pre, zpre


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Codes as stored: two per byte at 4 bits (pack_int4), one byte each at
    8 bits (signed codes as 8-bit two's complement)."""
    if bits == 4:
        return pack_int4(q)
    return np.asarray(q).astype(np.int16).astype(np.uint8)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element 2j in the low nibble, 2j+1 in the high.

    Signed codes are stored as 4-bit two's complement.
    """
    q = np.asarray(q).astype(np.int16)
    if q.shape[-1] % 2:
        raise ValueError("packed rows need an even number of codes")
    u = (q & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray, signed: bool) -> np.ndarray:
    p = np.asarray(p, np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int16)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    if signed:
        q = np.where(q >= 8, q - 16, q)
    return q.astype(np.int8 if signed else np.uint8)


# --------------------------------------------------------------------------
# Integer GEMM and dequantization
# --------------------------------------------------------------------------

def int_gemm_bruteforce(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """acc[t, n] = sum_k a[t, k] * b[n, k] in int64 (plain loops over t)."""
    a = np.asarray(a, np.int64)
    b = np.asarray(b, np.int64)
    out = np.empty((a.shape[0], b.shape[0]), np.int64)
    for t in range(a.shape[0]):
        out[t] = (b * a[t][None, :]).sum(axis=1)
    return out


def int_gemm(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact integer acc[t, n] = sum_k a[t, k] b[n, k], stored int32.

    [QUIK] part 4: INT4 operands, INT32 accumulation.  Computed with an fp64
    matrix product: every operand and every partial sum is an integer below
    2^53 in magnitude (checked), so no rounding happens in any summation order.
    The result must fit int32, as the INT32 accumulator requires.
    """
    a = np.asarray(a)
    b = np.asarray(b)
    K = a.shape[1]
    bound = float(np.max(np.abs(a), initial=0)) * float(np.max(np.abs(b), initial=0)) * K
    if bound >= 2.0 ** 53:
        raise OverflowError("operands too large for an exact fp64 product")
    acc = np.asarray(a, np.float64) @ np.asarray(b, np.float64).T
    acc = acc.astype(np.int64)
    if acc.size and (acc.max() >= 2 ** 31 or acc.min() < -2 ** 31):
        raise OverflowError("accumulator exceeds int32")
    return acc.astype(np.int32)


def to_fp16(y: np.ndarray) -> np.ndarray:
    """Round fp64 once to fp16, round half to even (numpy's direct conversion).

    [QUIK] part 1: the dequantized INT4 product and the FP16 outlier product
    are summed into an FP16 output; reading c14: the sum is formed exactly and
    rounded once.  Values at or above 65520 in magnitude become infinities.
    """
    return np.asarray(y, np.float64).astype(np.float16)


def dequant_sym(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """y = fp16(acc * sx[t] * sw[n]), computed in fp64, rounded once.

    Per-token times per-channel scales factor out of the K-sum, which is what
    keeps the GEMM on matrix units ([SQR] third reviewer A3, token-wise
    quantization).
    """
    y = (np.asarray(acc, np.float64) * np.asarray(sx, np.float64)[:, None]
         * np.asarray(sw, np.float64)[None, :])
    return to_fp16(y)


def dequant_mixed(acc, sx, zx, sw, w_rowsum, x_out=None, w_out=None) -> np.ndarray:
    """QUIK mixed output: y = fp16((acc - z rowsum) sx sw + X_out W_out^T).

    [QUIK] part 1: the INT4 product is dequantized to FP16, the outlier
    columns are multiplied in FP16, and the two are added.  The asymmetric
    zero point comes out of the K-sum as z[t] * sum_k qw[n, k] (exact
    integer).  Reading c14: one fp16 rounding at the end.
    """
    acc2 = np.asarray(acc, np.int64) - np.asarray(zx, np.int64)[:, None] * np.asarray(w_rowsum, np.int64)[None, :]
    y = acc2.astype(np.float64) * np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    if x_out is not None and np.asarray(x_out).shape[1]:
        y = y + np.asarray(x_out, np.float64) @ np.asarray(w_out, np.float64).T
    return to_fp16(y)


# --------------------------------------------------------------------------
# QUIK outlier split
# --------------------------------------------------------------------------

def split_outliers(x: np.ndarray, outlier_idx: np.ndarray):
    """Split columns into (normal columns in their order, outlier columns).

    [QUIK] part 1: outlier columns are kept in FP16 and moved to the end (with
    the matching weight columns); the others go through INT4.
    """
    K = x.shape[1]
    mask = np.zeros(K, bool)
    mask[np.asarray(outlier_idx, np.int64)] = True
    return x[:, ~mask], x[:, mask]


def select_outlier_columns(x: np.ndarray, count: int) -> np.ndarray:
    """Columns with the largest infinity norm, ascending ([QUIK] part 3).

    Ties go to the lower index (reading c13).
    """
    inf = np.max(np.abs(np.asarray(x, np.float64)), axis=0)
    order = np.lexsort((np.arange(inf.size), -inf))
    return np.sort(order[:count]).astype(np.int32)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def rotate_quant(x16: np.ndarray, kind: str, clip: float = 1.0, asym: bool = False,
                 outlier_idx=None, block: int = 0, p1=None, p2=None, chan_scale=None,
                 bits: int = 4) -> dict:
    """Online transform + per-token INT4 (or INT8) quantization of activations.

    Returns codes (unpacked and packed), scale, zero (asymmetric), the fp16
    outlier columns, and the fp64 pre-round values for tolerance checks.
    bits = 8 is QUIK-8B's form for the down projection (reading r22).
    """
    x = np.asarray(x16, np.float16).astype(np.float64)          # exact upcast
    x_out = np.zeros((x.shape[0], 0), np.float16)
    if outlier_idx is not None and len(outlier_idx):
        x, xo = split_outliers(x, outlier_idx)
        x_out = xo.astype(np.float16)                             # exact (fp16 values)
    K = x.shape[1]
    if kind != "none":
        x = x @ rotation(kind, K, block, p1, p2, chan_scale)
    out = {"x_out": x_out, "xr": x}
    if asym:
        q, s, z, pre, zpre = quantize_asym(x, code_max(bits, True))
        out.update(q=q, scale=s, zero=z, pre=pre, zpre=zpre)
    else:
        q, s, pre = quantize_sym(x, clip, code_max(bits, False))
        out.update(q=q, scale=s, zero=None, pre=pre)
    out["packed"] = pack_codes(q, bits)
    return out


def kv_rotate_quant(x16: np.ndarray, group: int = 128, rotate: bool = True) -> dict:
    """The KV-cache path: R3, then group-wise asymmetric INT4.

    [SQR] the authors' answer on the number of rotation matrices: R3 rotates
    the KV cache before its quantization; [SQR] first reviewer Q2/A2 (the two
    R3 of Figure 1): (W_q R3)(W_k R3)^T = W_q W_k^T, so the rotation cancels
    in the attention scores.  Reading: R3 is the normalized Walsh-Hadamard of
    one head's `group` channels, applied to every head (blockdiag(H_group, ...)).
    [FQ] section 3 (quantization setting, after QuaRot): the KV cache is
    quantized group-wise asymmetric with groups of 128; each group takes the
    asymmetric min-max form of reading c4 (quantize_asym, one scale and zero
    point per group).  Codes are packed as in pack_int4.

    Returns q [T, K] uint8, scale and zero [T, K/group], the fp64 rotated
    values xr, pre-round values pre [T, K] and zpre [T, K/group], packed.
    """
    x = np.asarray(x16, np.float16).astype(np.float64)          # exact upcast
    T, K = x.shape
    assert K % group == 0
    if rotate:
        x = x @ block_diag(hadamard(group), K // group)
    q, s, z, pre, zpre = quantize_asym(x.reshape(T * (K // group), group))
    q = q.reshape(T, K)
    return {"q": q, "scale": s.reshape(T, K // group), "zero": z.reshape(T, K // group), "xr": x,
            "pre": pre.reshape(T, K), "zpre": zpre.reshape(T, K // group), "packed": pack_int4(q)}


def search_weight_clip(w16: np.ndarray, outlier_idx=None, bits: int = 4, steps: int = 100) -> dict:
    """QUIK's weight clipping by linear search, per output channel.

    [QUIK] "QUIK量化" part 2: before the weights are quantized, a linear
    search picks the clipping threshold.  Reading r23: the candidates are the
    ratios c = k / steps (rounded to fp32), k = steps, steps - 1, ..., 1; each
    is scored by the squared error sum (w - s_c q_c)^2 of symmetric min-max
    quantization with s_c = fp32(c * max|w| / qmax) over the row's normal
    columns (outlier columns stay fp16 and are not clipped), and the first
    minimum in that order is kept (ties go to the larger ratio).

    Returns clip fp32 [N] and the error table err [N, steps] (column j is
    k = steps - j).
    """
    w = np.asarray(w16, np.float16).astype(np.float64)
    if outlier_idx is not None and len(outlier_idx):
        w, _ = split_outliers(w, outlier_idx)
    qm = code_max(bits, False)
    ratios = [np.float32(k / steps) for k in range(steps, 0, -1)]
    err = np.empty((w.shape[0], steps))
    for j, c in enumerate(ratios):
        q, s, _ = quantize_sym(w, c, qm)
        err[:, j] = ((w - s.astype(np.float64)[:, None] * q) ** 2).sum(axis=1)
    best = np.argmin(err, axis=1)          # first minimum = largest ratio among ties
    clip = np.array([ratios[j] for j in best], np.float32)
    return {"clip": clip, "err": err, "ratios": np.array(ratios, np.float32)}


def prepare_weights(w16: np.ndarray, kind: str, clip: float = 1.0, outlier_idx=None,
                    block: int = 0, p1=None, p2=None, chan_scale=None, bits: int = 4) -> dict:
    """Offline weight side: W' = W . R^{-T}, then per-output-channel symmetric RTN.

    [QS] sections 1-2 (rotation folded into the weights), [FQ] section 3
    (per-channel symmetric weights), [QUIK] part 1 (outlier weight columns
    stay FP16; the scale comes from the normal columns only, reading c12).
    Also returns the code row sums the asymmetric epilogue needs.
    """
    w = np.asarray(w16, np.float16).astype(np.float64)
    w_out = np.zeros((w.shape[0], 0), np.float16)
    if outlier_idx is not None and len(outlier_idx):
        w, wo = split_outliers(w, outlier_idx)
        w_out = wo.astype(np.float16)
    K = w.shape[1]
    if kind != "none":
        w = w @ weight_transform(kind, K, block, p1, p2, chan_scale)
    q, s, pre = quantize_sym(w, clip, code_max(bits, False))
    return {"q": q, "scale": s, "pre": pre, "packed": pack_codes(q, bits),
            "rowsum": q.astype(np.int64).sum(axis=1).astype(np.int32), "w_out": w_out,
            "wr": w}


def linear(xq: dict, wq: dict) -> dict:
    """Integer GEMM of the codes plus the dequant epilogue ([QUIK] parts 1 and 4)."""
    acc = int_gemm(xq["q"], wq["q"])
    if xq.get("zero") is not None or xq["x_out"].shape[1]:
        zero = xq["zero"] if xq.get("zero") is not None else np.zeros(acc.shape[0], np.int32)
        y = dequant_mixed(acc, xq["scale"], zero, wq["scale"], wq["rowsum"],
                          xq["x_out"], wq["w_out"])
    else:
        y = dequant_sym(acc, xq["scale"], wq["scale"])
    return {"acc": acc, "y": y}
