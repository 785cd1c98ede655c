"""CPU checks of the comparison helpers themselves: the KV quantizer's fp32
window admits a plain fp32 evaluation of the same steps and rejects a code
that is wrong away from a rounding boundary."""
import numpy as np
import pytest

import workloads
from oracle import rq_oracle as o
from parity_utils import check_kv_quant


def _fp32_butterflies(x16, g):
    """Walsh-Hadamard of each group by in-place butterflies in float32, then
    one multiply by float32(1/sqrt(g)): the evaluation order the window is
    derived for (any other tree of log2(g) additions has the same bound)."""
    v = x16.astype(np.float32).reshape(-1, g).copy()
    h = 1
    while h < g:
        v = v.reshape(-1, g // (2 * h), 2, h)
        a, b = v[:, :, 0, :].copy(), v[:, :, 1, :].copy()
        v[:, :, 0, :], v[:, :, 1, :] = a + b, a - b
        v = v.reshape(-1, g)
        h *= 2
    return v * np.float32(1.0 / np.sqrt(g))


def _fp32_quant(v):
    lo = np.minimum(v.min(axis=1), np.float32(0))
    hi = np.maximum(v.max(axis=1), np.float32(0))
    s = ((hi - lo) / np.float32(15)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1))
    z = np.where(s > 0, np.clip(np.rint(-lo / safe), 0, 15), 0).astype(np.int64)
    q = np.clip(np.rint(v / safe[:, None]) + z[:, None], 0, 15).astype(np.uint8)
    return q, s, z


@pytest.mark.parametrize("g", [64, 128, 256])
def test_kv_window_admits_fp32_evaluation(g):
    x = workloads.make_inputs("kv", T=64, K=4096, with_weights=False)["x"]
    T, K = x.shape
    q, s, z = _fp32_quant(_fp32_butterflies(x, g))
    ref = o.kv_rotate_quant(x, group=g, rotate=True)
    flips = check_kv_quant(o.pack_int4(q.reshape(T, K)), s.reshape(T, -1), z.reshape(T, -1), ref, x, g, True)
    assert flips.sum() <= 1e-3 * x.size


def test_kv_window_rejects_a_wrong_code():
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
