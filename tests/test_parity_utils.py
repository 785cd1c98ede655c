"""CPU checks of the comparison helpers themselves: the KV quantizer's check
admits an evaluation with the rotation rounded once to fp32 (what the GPU
computes) and rejects a code that is wrong away from a rounding boundary, a
scale off by more than 1e-6, and more near-boundary flips than 1e-4 of the
codes."""
import numpy as np
import pytest

import workloads
from oracle import rq_oracle as o
from parity_utils import check_kv_quant


def _sylvester_signs(g):
    h = np.array([[1.0]])
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    return h


def _rotated_fp32(x16, g):
    """Each group's Walsh-Hadamard image, summed exactly (integer multiples of
    2^-24 below 2^48 in fp64), scaled by fp64(1/sqrt(g)) and rounded to fp32."""
    x = x16.astype(np.float64).reshape(-1, g)
    return ((x @ _sylvester_signs(g)) * (1.0 / np.sqrt(g))).astype(np.float32)


def _fp32_quant(v):
    lo = np.minimum(v.min(axis=1), np.float32(0)).astype(np.float64)
    hi = np.maximum(v.max(axis=1), np.float32(0)).astype(np.float64)
    s = ((hi - lo) / 15).astype(np.float32)
    s64 = s.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    z = np.where(s64 > 0, np.clip(np.rint(-lo / safe), 0, 15), 0).astype(np.int64)
    inv = (np.float32(1) / np.where(s > 0, s, np.float32(1))).astype(np.float32)
    prod = v * inv[:, None]                                   # fp32 products, as the fma form rounds them
    q = np.where(s64[:, None] > 0, np.clip(np.rint(prod.astype(np.float64)) + z[:, None], 0, 15), 0).astype(np.uint8)
    return q, s, z


@pytest.mark.parametrize("g", [64, 128, 256])
def test_kv_check_admits_the_rotation_rounded_once(g):
    x = workloads.make_inputs("kv", T=64, K=4096, with_weights=False)["x"]
    T, K = x.shape
    q, s, z = _fp32_quant(_rotated_fp32(x, g))
    ref = o.kv_rotate_quant(x, group=g, rotate=True)
    flips = check_kv_quant(o.pack_int4(q.reshape(T, K)), s.reshape(T, -1), z.reshape(T, -1), ref, x, g, True)
    assert flips.sum() <= 1e-4 * x.size


def test_kv_check_rejects_wrong_codes_scales_and_too_many_flips():
    g = 128
    x = workloads.make_inputs("kv", T=16, K=1024, with_weights=False)["x"]
    ref = o.kv_rotate_quant(x, group=g, rotate=True)
    q, s, z = ref["packed"], ref["scale"], ref["zero"]
    check_kv_quant(q, s, z, ref, x, g, True)
    # a mistake planted in the oracle's result: one code moved by one where
    # its pre-round value is far from a boundary
    bad = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
    frac = np.abs(ref["pre"] - np.floor(ref["pre"]) - 0.5)
    t, j = np.argwhere((frac > 0.2) & (ref["q"] > 0) & (ref["q"] < 15))[0]
    bad["q"][t, j] += 1
    with pytest.raises(AssertionError):
        check_kv_quant(q, s, z, bad, x, g, True)
    with pytest.raises(AssertionError):
        check_kv_quant(q, s, z, bad | {"packed": o.pack_int4(bad["q"])}, x, g, False)
    # a scale 2e-6 off
    s2 = s.copy()
    s2[3, 2] = np.float32(s2[3, 2] * (1 + 2e-6))
    with pytest.raises(AssertionError):
        check_kv_quant(q, s2, z, ref, x, g, True)
    # near-boundary flips on more than 1e-4 of the codes: every code of a
    # window wide enough to hold a few pre-round values, planted as if they
    # were all within 1e-5 of their boundary
    near = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
    inner = (ref["q"] > 0) & (ref["q"] < 15)
    pos = np.argwhere(inner)[:8]
    for tt, jj in pos:
        near["pre"][tt, jj] = np.floor(near["pre"][tt, jj]) + 0.5 + 1e-6
    q3 = ref["q"].copy()
    for tt, jj in pos:
        q3[tt, jj] += 1
    assert len(pos) > 1e-4 * x.size
    with pytest.raises(AssertionError):
        check_kv_quant(o.pack_int4(q3), s, z, near, x, g, True)
