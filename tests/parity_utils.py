"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (fixed for this path):
  - INT32 accumulators: bit-exact on identical codes.
  - Quantized codes: equal, except at most 1 LSB on at most 1e-4 of the
    elements, and only where the oracle's pre-round value lies within 1e-5 of
    a rounding boundary (k + 0.5).  Asymmetric zero points may differ by 1
    only where the oracle's -lo/scale lies within 1e-5 of a boundary.
  - Scales: within 1e-6 relative.
  - fp16 outputs: |y - y_ref| <= 1e-3 + 2e-3 |y_ref|; end-to-end comparisons
    widen this by the effect of the tolerated code flips.
  - KV-cache quantizer (group-wise asymmetric, check_kv_quant): bit-exact
    without rotation; with rotation, the same code, zero-point and scale
    tolerances per group as every other quantizer.
"""
import sys

import numpy as np

from oracle import rq_oracle as o

CODE_FRAC = 1e-4
NEAR_TIE = 1e-5
SCALE_RTOL = 1e-6
Y_ATOL, Y_RTOL = 1e-3, 2e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def near_tie(pre):
    pre = np.asarray(pre, np.float64)
    return np.abs(pre - (np.floor(pre) + 0.5)) < NEAR_TIE


def check_scales(s_gpu, s_ref, what="scale"):
    s_gpu = np.asarray(s_gpu, np.float64)
    s_ref = np.asarray(s_ref, np.float64)
    zero = s_ref == 0
    assert np.array_equal(s_gpu[zero], s_ref[zero]), f"{what}: zero rows differ"
    rel = np.abs(s_gpu - s_ref) / np.where(zero, 1.0, np.abs(s_ref))
    assert rel.max(initial=0) <= SCALE_RTOL, f"{what}: max rel diff {rel.max():.3g}"


def code_flips(q_gpu, q_ref, pre, what="codes"):
    """Check codes; return the per-row count of tolerated flips."""
    q_gpu = np.asarray(q_gpu, np.int64)
    q_ref = np.asarray(q_ref, np.int64)
    diff = q_gpu != q_ref
    if not diff.any():
        return np.zeros(q_ref.shape[0], np.int64)
    bad = diff & ~(near_tie(pre) & (np.abs(q_gpu - q_ref) <= 1))
    assert not bad.any(), (f"{what}: {int(bad.sum())} codes differ away from a rounding boundary; "
                           f"first at {np.argwhere(bad)[0].tolist()} gpu={q_gpu[bad][0]} ref={q_ref[bad][0]}")
    assert diff.sum() <= CODE_FRAC * diff.size, f"{what}: {int(diff.sum())} near-tie flips > {CODE_FRAC:g}"
    return diff.sum(axis=1)


def check_sym_quant(q_packed_gpu, s_gpu, ref, what="x"):
    check_scales(s_gpu, ref["scale"], what + " scale")
    q_gpu = o.unpack_int4(q_packed_gpu, signed=True)
    return code_flips(q_gpu, ref["q"], ref["pre"], what + " codes")


def check_asym_quant(q_packed_gpu, s_gpu, z_gpu, ref, what="x"):
    check_scales(s_gpu, ref["scale"], what + " scale")
    z_gpu = np.asarray(z_gpu, np.int64)
    z_ref = ref["zero"].astype(np.int64)
    zd = z_gpu != z_ref
    assert not (zd & ~(near_tie(ref["zpre"]) & (np.abs(z_gpu - z_ref) <= 1))).any(), "zero points differ"
    q_gpu = o.unpack_int4(q_packed_gpu, signed=False).astype(np.int64)
    q_ref = ref["q"].astype(np.int64)
    # compare codes relative to the zero point; where a zero point flipped,
    # elements clamped on either side are counted as flips instead
    rel_gpu = q_gpu - z_gpu[:, None]
    rel_ref = q_ref - z_ref[:, None]
    ignore = zd[:, None] & ((q_gpu == 0) | (q_gpu == 15) | (q_ref == 0) | (q_ref == 15))
    flips = code_flips(np.where(ignore, rel_ref, rel_gpu), rel_ref, ref["pre"], what + " codes")
    total = flips + ignore.sum(axis=1)
    assert total.sum() <= CODE_FRAC * q_ref.size, f"{what}: {int(total.sum())} flipped codes > {CODE_FRAC:g}"
    return total


def check_y(y_gpu, y_ref, extra=None, what="y"):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite output"
    bound = Y_ATOL + Y_RTOL * np.abs(y_ref)
    if extra is not None:
        bound = bound + extra
    err = np.abs(y_gpu - y_ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst "
                           f"{np.max(err - bound):.4g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def flip_allowance(sx, sw, flips_x, flips_w, qmax_x=15, qmax_w=7):
    """Largest change of y[t, n] the tolerated code flips can cause: a flipped
    activation code moves y by sx*sw*|qw| <= 7 sx sw; a flipped weight code by
    sx*sw*|qx - z| <= 15 sx sw."""
    sx = np.asarray(sx, np.float64)[:, None]
    sw = np.asarray(sw, np.float64)[None, :]
    return sx * sw * (qmax_w * np.asarray(flips_x)[:, None] + qmax_x * np.asarray(flips_w)[None, :]) * 1.001


def check_kv_quant(q_packed_gpu, s_gpu, z_gpu, ref, x16=None, group=128, rotate=True, what="kv"):
    """Compare the KV quantizer's output with the oracle's kv_rotate_quant.

    Without rotation the result must be identical.  With rotation each group
    is one row of check_asym_quant: scales within 1e-6 relative, a zero point
    or a code (relative to its zero point) one step off only where the
    oracle's pre-round value lies within 1e-5 of a rounding boundary, and at
    most 1e-4 of the codes so flipped.  Returns the flips per group.
    """
    T, K = ref["q"].shape
    G = T * (K // group)
    if not rotate:
        assert np.array_equal(np.asarray(q_packed_gpu), ref["packed"]), f"{what}: codes differ"
        assert np.array_equal(np.asarray(s_gpu, np.float64).reshape(G),
                              ref["scale"].reshape(G).astype(np.float64)), f"{what}: scales differ"
        assert np.array_equal(np.asarray(z_gpu, np.int64).reshape(G), ref["zero"].reshape(G)), f"{what}: zero points differ"
        return np.zeros(G, np.int64)
    rows = {"scale": ref["scale"].reshape(G), "zero": ref["zero"].reshape(G),
            "q": ref["q"].reshape(G, group), "pre": ref["pre"].reshape(G, group), "zpre": ref["zpre"].reshape(G)}
    return check_asym_quant(np.asarray(q_packed_gpu).reshape(G, group // 2), np.asarray(s_gpu).reshape(G),
                            np.asarray(z_gpu).reshape(G), rows, what)
