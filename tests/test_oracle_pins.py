"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types an oracle formula: each checks the oracle against an
independent construction (a recursion, a hand-worked example, an identity, a
special case with a known answer, or brute force), chosen so that a dropped
term, a wrong sign or index, or a transposed operand fails one of them.
"""
import math
import os

import numpy as np
import pytest

from oracle import rq_oracle as o
import workloads


def _rows(path):
    out = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            out.append([p.strip() for p in line.split("|")])
    return out


# ---------------------------------------------------------------- Hadamard

def _sylvester(n):
    """Independent construction: H_1 = [1], H_2n = [[H, H], [H, -H]] / sqrt(2)."""
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]]) / math.sqrt(2.0)
    return h


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 256, 1024])
def test_hadamard_matches_sylvester_recursion(n):
    np.testing.assert_allclose(o.hadamard(n), _sylvester(n), rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [4, 64, 256, 4096])
def test_hadamard_orthogonal_symmetric_involution(n):
    h = o.hadamard(n)
    eye = np.eye(n)
    assert np.abs(h @ h.T - eye).max() < 1e-12          # R R^T = I  (SpinQuant OpenReview Q2/A2)
    assert np.array_equal(h, h.T)
    assert np.abs(h @ h - eye).max() < 1e-12


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        o.hadamard(12)


def test_hadamard_worked_example(golden_dir):
    rows = {r[0]: r for r in _rows(os.path.join(golden_dir, "worked_examples.txt"))}
    x = np.array(rows["hadamard4"][1].split(), float)
    want = np.array(rows["hadamard4"][2].split(), float)
    np.testing.assert_array_equal(x @ o.hadamard(4), want)


def test_hadamard_special_cases():
    n = 256
    h = o.hadamard(n)
    # e_i . H = row i: every entry +-1/sqrt(n), so min-max codes are all +-7
    e = np.zeros((1, n)); e[0, 37] = 1.0
    q, s, _ = o.quantize_sym(e @ h)
    assert np.all(np.abs(q) == 7) and np.isclose(s[0], np.float32(1 / 16 / 7))
    # c * ones . H = c sqrt(n) e_0: one code +-7, the rest 0
    c = 3.0
    q, s, _ = o.quantize_sym(np.full((1, n), c) @ h)
    assert q[0, 0] == 7 and not np.any(q[0, 1:])
    # a single outlier of size m spreads to +-m/sqrt(n) on every channel
    m = 50.0
    x = np.zeros((1, n)); x[0, 5] = m
    np.testing.assert_allclose(np.abs(x @ h), m / 16.0, rtol=0, atol=1e-12)


def test_rotation_preserves_norm_and_rmsnorm_invariance():
    """||x R|| = ||x|| and RMSNorm(X) = RMSNorm(X Q^T) Q ("QuaRot & SpinQuant"
    blog, section 1, with RMSNorm taken as x / ||x|| per row)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 256)) * 3
    x[:, 7] *= 40

    def rmsnorm(a, eps=0.0):
        return a / np.sqrt(np.sum(a * a, axis=1, keepdims=True) + eps)

    for q in (o.hadamard(256), o.gsr_rotation(256, 64)):
        np.testing.assert_allclose(np.linalg.norm(x @ q, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
        np.testing.assert_allclose(rmsnorm(x), rmsnorm(x @ q.T) @ q, rtol=0, atol=1e-13)
    # a non-orthogonal transform breaks the invariance (FlatQuant's affine is
    # not a rotation, so it is never relied on there)
    wl = workloads.get("flat")
    p1, p2, s = workloads.make_affine(wl, np.random.default_rng(0), 16, 16)
    r = o.kron_affine(p1, p2, s)
    assert np.abs(rmsnorm(x) - rmsnorm(x @ np.linalg.inv(r)) @ r).max() > 1e-3


# ---------------------------------------------------------------- Walsh / GSR

def test_walsh8_matches_hand_table(golden_dir):
    table = _rows(os.path.join(golden_dir, "walsh8_sequency.txt"))
    want = np.array([r[1].split() for r in table], float) / math.sqrt(8)
    np.testing.assert_allclose(o.walsh_sequency(8), want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [2, 8, 64, 256])
def test_walsh_sign_changes_are_a_permutation(n):
    w = o.walsh_sequency(n)
    assert list(o.sign_changes(w)) == list(range(n))
    assert np.abs(w @ w.T - np.eye(n)).max() < 1e-12


def _bitrev(v, bits):
    r = 0
    for _ in range(bits):
        r = (r << 1) | (v & 1)
        v >>= 1
    return r


@pytest.mark.parametrize("n", [8, 64])
def test_walsh_rows_follow_bitreversed_gray_code(n):
    """Textbook map from sequency s to natural Hadamard index: bitrev(gray(s))."""
    bits = n.bit_length() - 1
    w = o.walsh_sequency(n)
    h = o.hadamard(n)
    for s in range(n):
        np.testing.assert_array_equal(w[s], h[_bitrev(s ^ (s >> 1), bits)])


def test_gsr_is_block_local():
    r = o.gsr_rotation(256, 64)
    x = np.zeros((1, 256)); x[0, 64:128] = np.arange(64) + 1.0
    y = x @ r
    assert not np.any(y[0, :64]) and not np.any(y[0, 128:])
    np.testing.assert_allclose(y[0, 64:128], (np.arange(64) + 1.0) @ o.walsh_sequency(64), atol=1e-12)
    with pytest.raises(ValueError):
        o.gsr_rotation(100, 64)


def _butterfly_fwht(x):
    """Radix-2 fast Walsh-Hadamard transform in fp64, rows of x, no matrix:
    log2(n) stages of (a, b) -> (a + b, a - b) on pairs h apart, then 1/sqrt(n)."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        v = y.reshape(y.shape[0], n // (2 * h), 2, h)
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        h *= 2
    return y / math.sqrt(n)


def test_butterfly_fwht_cross_checks_the_dense_rotations():
    """The oracle rotates by a dense matrix product; an independent fast
    transform on the same rows must agree to fp64 rounding: the full 4096-point
    transform, and the 64-point block transform reordered by sequency
    (s -> bitrev(gray(s))) for the GSR form."""
    rng = np.random.default_rng(11)
    K = 4096
    x = rng.standard_normal((6, K))
    x[:, rng.choice(K, 16, replace=False)] *= 40.0
    ref = x @ o.rotation("hadamard", K)
    np.testing.assert_allclose(_butterfly_fwht(x), ref, rtol=0, atol=1e-11 * np.abs(x).max())

    g = 64
    perm = np.array([_bitrev(s ^ (s >> 1), 6) for s in range(g)])
    blocks = _butterfly_fwht(x.reshape(-1, g)).reshape(x.shape[0], K // g, g)
    fast = blocks[:, :, perm].reshape(x.shape)
    np.testing.assert_allclose(fast, x @ o.rotation("gsr", K, block=g), rtol=0,
                               atol=1e-12 * np.abs(x).max())


# ---------------------------------------------------------------- Kronecker affine

def test_kron_matches_elementwise_definition_and_matrix_form():
    rng = np.random.default_rng(3)
    n1, n2 = 4, 8
    p1 = rng.standard_normal((n1, n1)); p2 = rng.standard_normal((n2, n2))
    s = rng.uniform(0.5, 2, n1 * n2)
    x = rng.standard_normal((3, n1 * n2))
    y = x @ o.kron_affine(p1, p2, s)
    # brute force: y[j1*n2+j2] = sum_{i1,i2} x[i1*n2+i2] s[.] P1[i1,j1] P2[i2,j2]
    for t in range(3):
        for j1 in range(n1):
            for j2 in range(n2):
                acc = 0.0
                for i1 in range(n1):
                    for i2 in range(n2):
                        acc += x[t, i1 * n2 + i2] * s[i1 * n2 + i2] * p1[i1, j1] * p2[i2, j2]
                assert abs(y[t, j1 * n2 + j2] - acc) < 1e-12
        # per-token matrix form: reshape row-major, P1^T M P2
        m = (x[t] * s).reshape(n1, n2)
        np.testing.assert_allclose(y[t], (p1.T @ m @ p2).reshape(-1), atol=1e-12)


def test_kron_full_size_matrix_form_and_inverse():
    inp = workloads.make_inputs("flat", T=8, with_weights=False)
    p1, p2, s = inp["p1"], inp["p2"], inp["s"]
    r = o.kron_affine(p1, p2, s)
    x = inp["x"].astype(np.float64)
    y = x @ r
    for t in range(8):
        m = (x[t] * s.astype(np.float64)).reshape(64, 64)
        np.testing.assert_allclose(y[t], (p1.astype(np.float64).T @ m @ p2.astype(np.float64)).reshape(-1),
                                   rtol=1e-12, atol=1e-9)
    k = np.kron(p1.astype(np.float64), p2.astype(np.float64))
    kinv = np.kron(np.linalg.inv(p1.astype(np.float64)), np.linalg.inv(p2.astype(np.float64)))
    assert np.abs(k @ kinv - np.eye(4096)).max() < 1e-10
    for p in (p1, p2):
        assert np.linalg.cond(p.astype(np.float64)) <= 1.5


@pytest.mark.parametrize("kind", ["hadamard", "gsr", "kron", "none"])
def test_weight_transform_keeps_the_product(kind):
    """(X R)(W G)^T = X W^T: computational invariance ("QuaRot & SpinQuant"
    blog, section 1) and its affine form (FlatQuant article, section 2.3)."""
    rng = np.random.default_rng(5)
    K = 256
    x = rng.standard_normal((6, K)); w = rng.standard_normal((10, K))
    kw = {}
    if kind == "gsr":
        kw = {"block": 64}
    if kind == "kron":
        wl = workloads.get("flat")
        p1, p2, s = workloads.make_affine(wl, rng, 16, 16)
        kw = {"p1": p1, "p2": p2, "chan_scale": s}
    r = o.rotation(kind, K, **kw)
    g = o.weight_transform(kind, K, **kw)
    ref = x @ w.T
    got = (x @ r) @ (w @ g).T
    assert np.abs(got - ref).max() <= 1e-10 * np.abs(ref).max()


# ---------------------------------------------------------------- quantizers

def test_symmetric_quantizer_worked_examples(golden_dir):
    rows = {r[0]: r for r in _rows(os.path.join(golden_dir, "worked_examples.txt"))}
    for name in ("symq_after_h4", "symq_ties"):
        x = np.array([rows[name][1].split()], float)
        want = np.array(rows[name][2].split(), int)
        q, s, _ = o.quantize_sym(x)
        np.testing.assert_array_equal(q[0], want)
    q, s, _ = o.quantize_sym(np.array([[5.0, -1, -2, 0]]))
    assert s[0] == np.float32(5.0 / 7.0)


def test_symmetric_quantizer_properties():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, (64, 1))
    q, s, pre = o.quantize_sym(x)
    assert q.min() >= -7 and q.max() <= 7
    assert np.all(np.abs(q).max(axis=1) == 7)               # min-max uses the full range
    assert np.abs(pre).max() <= 7 + 1e-6                      # no clamp needed at clip = 1
    err = np.abs(x - q * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 * (1 + 1e-6))
    # clipped: codes saturate at +-7 and the unclipped part keeps the s/2 bound
    q9, s9, pre9 = o.quantize_sym(x, clip=0.9)
    np.testing.assert_allclose(s9, (np.float64(np.float32(0.9)) * np.abs(x).max(1) / 7).astype(np.float32))
    assert q9.min() >= -7 and q9.max() <= 7 and np.abs(pre9).max() > 7
    inside = np.abs(pre9) <= 7
    assert np.all(np.abs(x - q9 * s9.astype(np.float64)[:, None])[inside]
                  <= np.broadcast_to(s9.astype(np.float64)[:, None] / 2 * (1 + 1e-6), x.shape)[inside])
    # zero row: scale 0, codes 0, no NaN
    qz, sz, _ = o.quantize_sym(np.zeros((2, 16)))
    assert not qz.any() and not sz.any()


def test_crafted_ties_through_the_rotation():
    """Rows built as y . H with half-integer y: H is an involution, so the
    rotated row is y again and the quantizer sees exact .5 ties."""
    n = 256
    y = np.zeros((1, n))
    y[0, :6] = [7.0, 0.5, 1.5, 2.5, -2.5, -3.5]
    x = y @ o.hadamard(n)
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x)         # exact in fp16
    r = o.rotate_quant(x16, "hadamard")
    assert r["scale"][0] == np.float32(1.0)
    np.testing.assert_array_equal(r["q"][0, :6], [7, 0, 2, 2, -2, -4])
    assert not r["q"][0, 6:].any()


def test_asymmetric_quantizer_worked_and_properties(golden_dir):
    rows = {r[0]: r for r in _rows(os.path.join(golden_dir, "worked_examples.txt"))}
    x = np.array([rows["asymq"][1].split()], float)
    q, s, z, _, _ = o.quantize_asym(x)
    np.testing.assert_array_equal(q[0], np.array(rows["asymq"][2].split(), int))
    assert z[0] == 5 and s[0] == np.float32(0.2)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 300)) * 5 + rng.uniform(-3, 3, (32, 1))
    x[3] = np.abs(x[3])            # all >= 0: lo = 0 -> zero point 0
    x[4] = -np.abs(x[4])           # all <= 0: hi = 0 -> zero point 15
    q, s, z, pre, zpre = o.quantize_asym(x)
    assert q.min() >= 0 and q.max() <= 15 and z.min() >= 0 and z.max() <= 15
    assert z[3] == 0 and z[4] == 15
    deq = (q.astype(np.float64) - z[:, None]) * s.astype(np.float64)[:, None]
    assert np.all(np.abs(deq - x) <= s.astype(np.float64)[:, None] * (1.0 + 1e-6))
    qz, sz, zz, _, _ = o.quantize_asym(np.zeros((1, 8)))
    assert not qz.any() and not sz.any() and not zz.any()


# ---------------------------------------------------------------- packing, GEMM

def test_pack_worked_example_and_roundtrip(golden_dir):
    rows = {r[0]: r for r in _rows(os.path.join(golden_dir, "worked_examples.txt"))}
    q = np.array([rows["pack"][1].split()], int)
    np.testing.assert_array_equal(o.pack_int4(q)[0], np.array(rows["pack"][2].split(), int))
    rng = np.random.default_rng(1)
    qs = rng.integers(-8, 8, (5, 64))
    np.testing.assert_array_equal(o.unpack_int4(o.pack_int4(qs), signed=True), qs)
    qu = rng.integers(0, 16, (5, 64))
    np.testing.assert_array_equal(o.unpack_int4(o.pack_int4(qu), signed=False), qu)


def test_int_gemm_matches_bruteforce(golden_dir):
    rows = {r[0]: r for r in _rows(os.path.join(golden_dir, "worked_examples.txt"))}
    a, b = [np.array([p.split()], int) for p in rows["dot"][1].split(";")]
    assert o.int_gemm(a, b)[0, 0] == int(rows["dot"][2])
    rng = np.random.default_rng(2)
    for K in (64, 256, 1000):
        a = rng.integers(-7, 8, (9, K)); b = rng.integers(-7, 8, (13, K))
        np.testing.assert_array_equal(o.int_gemm(a, b), o.int_gemm_bruteforce(a, b))
        au = rng.integers(0, 16, (9, K))
        np.testing.assert_array_equal(o.int_gemm(au, b), o.int_gemm_bruteforce(au, b))
    big = np.full((1, 4), 2 ** 20);
    with pytest.raises(OverflowError):
        o.int_gemm(big, big)


def _grid_layer(kind, T=5, N=7, K=256, seed=0):
    """Inputs that quantize losslessly: rotated rows are integer codes times a
    power-of-two scale, so the whole pipeline must reproduce X W^T exactly."""
    rng = np.random.default_rng(seed)
    kw = {"block": 64} if kind == "gsr" else {}
    r = o.rotation(kind, K, **kw)
    qx = rng.integers(-7, 8, (T, K)); qx[:, 0] = 7
    qw = rng.integers(-7, 8, (N, K)); qw[:, 1] = -7
    sx = 2.0 ** rng.integers(-4, 2, T); sw = 2.0 ** rng.integers(-8, -4, N)
    x = (qx * sx[:, None]) @ r.T          # x R = qx sx  (R orthogonal)
    w = (qw * sw[:, None]) @ r.T          # w R = qw sw
    return x, w, qx, qw, sx, sw


@pytest.mark.parametrize("kind", ["hadamard", "gsr", "none"])
def test_lossless_pipeline_reproduces_dense_product(kind):
    x, w, qx, qw, sx, sw = _grid_layer(kind)
    x16, w16 = x.astype(np.float16), w.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x) and np.array_equal(w16.astype(np.float64), w)
    kw = {"block": 64} if kind == "gsr" else {}
    xq = o.rotate_quant(x16, kind, **kw)
    wq = o.prepare_weights(w16, kind, **kw)
    np.testing.assert_array_equal(xq["q"], qx)
    np.testing.assert_array_equal(wq["q"], qw)
    y = o.linear(xq, wq)["y"]
    np.testing.assert_array_equal(y, (x @ w.T).astype(np.float16))


def test_dequant_equals_product_of_dequantized_operands():
    rng = np.random.default_rng(4)
    qx = rng.integers(-7, 8, (6, 128)); qw = rng.integers(-7, 8, (9, 128))
    sx = rng.uniform(0.1, 2, 6).astype(np.float32); sw = rng.uniform(1e-3, 1e-2, 9).astype(np.float32)
    dense = (qx * sx.astype(np.float64)[:, None]) @ (qw * sw.astype(np.float64)[:, None]).T
    np.testing.assert_array_equal(o.dequant_sym(o.int_gemm(qx, qw), sx, sw), dense.astype(np.float16))


def _term(t):
    """'2^-11', '-2^-40', '65504', 'inf' -> float, each exactly representable."""
    if t in ("inf", "-inf"):
        return float(t)
    sign = -1.0 if t.startswith("-") else 1.0
    t = t.lstrip("-")
    if "^" in t:
        b, e = t.split("^")
        assert b == "2"
        return sign * math.ldexp(1.0, int(e))
    return sign * float(t)


def _exact_sum(terms):
    """Sum of powers of two and small integers, exactly (as a Fraction)."""
    from fractions import Fraction
    return sum((Fraction(_term(t)) for t in terms), Fraction(0))


def test_fp16_rounding_hand_worked(golden_dir):
    """Single round-half-to-even fp64 -> fp16 of the output (reading c14), on
    values whose rounding through fp32 would differ: the oracle must round
    the exact value once."""
    from fractions import Fraction
    rows = _rows(os.path.join(golden_dir, "fp16_rounding.txt"))
    plain = [r for r in rows if not r[0].startswith("epilogue")]
    assert len(plain) >= 10
    for name, value, want in plain:
        v = _exact_sum(value.split())
        assert Fraction(float(v)) == v, name            # the value itself is an fp64
        w = want.split()
        expect = float(w[0]) if w[0] in ("inf", "0") else float(_exact_sum(w))
        got = o.to_fp16(np.array([float(v)]))[0]
        assert got.dtype == np.float16
        assert float(got) == expect, f"{name}: got {float(got)!r}, want {expect!r}"
    # the first line is the fp32-detour trap: rounding through fp32 lands on
    # the tie and gives 1, the single rounding gives 1 + 2^-10
    v = float(_exact_sum(plain[0][1].split()))
    assert float(np.float16(np.float32(v))) == 1.0 and float(o.to_fp16(np.array([v]))[0]) == 1 + 2.0 ** -10


def test_fp16_rounding_through_the_epilogues(golden_dir):
    """dequant_sym and dequant_mixed form y exactly and round it once: the
    hand-worked lines give outputs that an fp32 product or sum would miss."""
    rows = {r[0]: r for r in _rows(os.path.join(golden_dir, "fp16_rounding.txt")) if r[0].startswith("epilogue")}
    assert set(rows) == {"epilogue_sym", "epilogue_mixed", "epilogue_outliers_only"}

    def parse(spec):
        out, key = {}, None
        for tok in spec.split():
            if "=" in tok:
                key, tok = tok.split("=")
                out[key] = []
            out[key].append(tok)
        return out

    for name, r in rows.items():
        f = parse(r[1])
        want = float(_exact_sum(r[2].split()))
        acc = np.array([[int(_exact_sum(f["acc"]))]], np.int32)
        sx = np.array([float(_exact_sum(f["sx"]))], np.float32)
        sw = np.array([float(_exact_sum(f["sw"]))], np.float32)
        assert float(sx[0]) == float(_exact_sum(f["sx"])) and float(sw[0]) == float(_exact_sum(f["sw"]))
        if name == "epilogue_sym":
            y = o.dequant_sym(acc, sx, sw)
        else:
            zx = np.array([int(_exact_sum(f["z"]))], np.int32)
            rs = np.array([int(_exact_sum(f["rowsum"]))], np.int32)
            if name == "epilogue_outliers_only":   # one outlier column per term
                xo_v = [float(_exact_sum([t])) for t in f["xo"]]
                wo_v = [float(_exact_sum([t])) for t in f["wo"]]
            else:
                xo_v, wo_v = [float(_exact_sum(f["xo"]))], [float(_exact_sum(f["wo"]))]
            xo, wo = np.array([xo_v], np.float16), np.array([wo_v], np.float16)
            assert xo.astype(np.float64).tolist() == [xo_v] and wo.astype(np.float64).tolist() == [wo_v]
            y = o.dequant_mixed(acc, sx, zx, sw, rs, xo, wo)
        assert y.dtype == np.float16 and float(y[0, 0]) == want, f"{name}: got {float(y[0, 0])!r}, want {want!r}"


# ---------------------------------------------------------------- QUIK split

def test_quik_split_identity_and_zero_point_correction():
    rng = np.random.default_rng(8)
    K, n_out = 512, 16
    x = rng.integers(-50, 50, (4, K)).astype(np.float64)
    w = rng.integers(-50, 50, (6, K)).astype(np.float64)
    idx = np.sort(rng.choice(K, n_out, replace=False))
    xn, xo = o.split_outliers(x, idx); wn, wo = o.split_outliers(w, idx)
    assert xn.shape == (4, K - n_out) and xo.shape == (4, n_out)
    np.testing.assert_array_equal(xn @ wn.T + xo @ wo.T, x @ w.T)
    keep = np.setdiff1d(np.arange(K), idx)
    np.testing.assert_array_equal(xn, x[:, keep])
    # asymmetric codes: sum_k (q - z) qw = acc - z * rowsum (brute force)
    q = rng.integers(0, 16, (4, 64)); z = rng.integers(0, 16, 4)
    qw = rng.integers(-7, 8, (6, 64))
    brute = o.int_gemm_bruteforce(q - z[:, None], qw)
    acc = o.int_gemm(q, qw).astype(np.int64)
    np.testing.assert_array_equal(acc - z[:, None] * qw.sum(1)[None, :], brute)


def test_quik_mixed_pipeline_small():
    """Asymmetric INT4 part + FP16 outlier part against the dense product,
    within the quantization error bound of the INT4 part."""
    inp = workloads.make_inputs("quik_prefill", T=24, K=512, N=40)
    x, w, idx = inp["x"], inp["w"], inp["outlier_ch"][:32]
    xq = o.rotate_quant(x, "none", asym=True, outlier_idx=idx)
    wq = o.prepare_weights(w, "none", outlier_idx=idx)
    y = o.linear(xq, wq)["y"].astype(np.float64)
    xn, xo = o.split_outliers(x.astype(np.float64), idx)
    wn, wo = o.split_outliers(w.astype(np.float64), idx)
    xd = (xq["q"].astype(np.float64) - xq["zero"][:, None]) * xq["scale"].astype(np.float64)[:, None]
    wd = wq["q"] * wq["scale"].astype(np.float64)[:, None]
    exact = xd @ wd.T + xo @ wo.T
    np.testing.assert_allclose(y, exact, rtol=1e-3, atol=1e-3)
    # the quantization error of each operand is bounded by half a step
    assert np.all(np.abs(xd - xn) <= xq["scale"].astype(np.float64)[:, None] * 0.5 * (1 + 1e-6) + 1e-12)
    assert np.all(np.abs(wd - wn) <= wq["scale"].astype(np.float64)[:, None] * 0.5 * (1 + 1e-6) + 1e-12)


def test_outlier_selection_recovers_generator_columns():
    inp = workloads.make_inputs("quik_prefill", T=64, with_weights=False)
    np.testing.assert_array_equal(o.select_outlier_columns(inp["x"], 256), inp["outlier_ch"])


# ---------------------------------------------------------------- statistical sanity

def test_rotation_flattens_outliers_and_quip_bound():
    inp = workloads.make_inputs("llama7b", T=64, N=64)
    x = inp["x"].astype(np.float64)
    xr = x @ o.hadamard(4096)

    def ratio(a):
        return np.max(np.abs(a), axis=1) / np.sqrt(np.mean(a * a, axis=1))
    assert np.all(ratio(xr) < ratio(x))
    # QuIP# incoherence bound quoted in the SpinQuant OpenReview discussion:
    # max |W_ij| <= mu ||W||_F / sqrt(mn), mu = 2 log(4 mn / delta)
    w = inp["w"].astype(np.float64) @ o.hadamard(4096)
    m, n = w.shape
    delta = 0.01
    mu = 2 * math.log(4 * m * n / delta)
    assert np.abs(w).max() <= mu * np.linalg.norm(w) / math.sqrt(m * n)


def test_affine_pipeline_small():
    """FlatQuant path end to end: codes dequantize to X R and W R^{-T} within
    half a step (clipped entries aside), and (X R)(W R^{-T})^T = X W^T."""
    inp = workloads.make_inputs("flat", T=12, K=256, N=20, n1=16, n2=16)
    x, w = inp["x"], inp["w"]
    kw = dict(p1=inp["p1"], p2=inp["p2"], chan_scale=inp["s"])
    xq = o.rotate_quant(x, "kron", clip=0.95, **kw)
    wq = o.prepare_weights(w, "kron", **kw)
    xr = x.astype(np.float64) @ o.rotation("kron", 256, **kw)
    wr = w.astype(np.float64) @ o.weight_transform("kron", 256, **kw)
    np.testing.assert_allclose(xq["xr"], xr, rtol=1e-13, atol=1e-12)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(xr @ wr.T - ref).max() <= 1e-10 * np.abs(ref).max()
    sx = xq["scale"].astype(np.float64)[:, None]
    inside = np.abs(xq["pre"]) <= 7
    assert np.all((np.abs(xq["q"] * sx - xr) <= sx / 2 * (1 + 1e-6))[inside])
    assert np.all(np.abs(xq["q"][~inside]) == 7)
    sw = wq["scale"].astype(np.float64)[:, None]
    assert np.all(np.abs(wq["q"] * sw - wr) <= sw / 2 * (1 + 1e-6))
    y = o.linear(xq, wq)["y"]
    np.testing.assert_array_equal(y, ((xq["q"] * sx) @ (wq["q"] * sw).T).astype(np.float16))


# ----------------------------------------------------------------------------- KV-cache path (R3 + g128)

def _sylvester(n):
    """H_n by the recursion H_2n = [[H, H], [H, -H]] / sqrt(2), built with loops."""
    h = [[1.0]]
    while len(h) < n:
        m = len(h)
        h = [[h[i % m][j % m] * (-1.0 if (i >= m and j >= m) else 1.0) for j in range(2 * m)]
             for i in range(2 * m)]
    return [[v / math.sqrt(n) for v in row] for row in h]


def test_kv_rotate_quant_matches_bruteforce_loops():
    """Tiny case with every step written as plain loops: per group, rotate by
    the recursively built Hadamard, then asymmetric min-max with a zero point."""
    rng = np.random.default_rng(21)
    T, K, g = 3, 16, 4
    x = (rng.standard_normal((T, K)) * 2).astype(np.float16)
    x[1, 4:8] = [0, 0, 0, 0]                       # an all-zero group: scale 0, zero 0, codes 0
    h = _sylvester(g)
    ref = o.kv_rotate_quant(x, group=g)
    for t in range(T):
        for gi in range(K // g):
            xs = [float(x[t, gi * g + i]) for i in range(g)]
            xr = [sum(xs[i] * h[i][j] for i in range(g)) for j in range(g)]
            lo, hi = min(min(xr), 0.0), max(max(xr), 0.0)
            s = float(np.float32((hi - lo) / 15))
            z = int(min(max(round(-lo / s), 0), 15)) if s > 0 else 0
            assert ref["scale"][t, gi] == np.float32(s) and ref["zero"][t, gi] == z
            for j in range(g):
                c = 0 if s == 0 else int(min(max(round(xr[j] / s) + z, 0), 15))   # round(): ties to even
                pre = 0.0 if s == 0 else xr[j] / s
                if abs(pre - math.floor(pre) - 0.5) > 1e-9:                         # away from ties
                    assert ref["q"][t, gi * g + j] == c


def test_kv_rotate_quant_one_hot_closed_form():
    """x = c e_i inside group g: that group becomes c H_128[i, :] = +-a with
    a = |c|/sqrt(128).  For i > 0 both signs occur: S = 2a/15 and s = fp32(S), so
    -lo/s = a/s = 7.5 S/s.  Above 7.5 (s < S) or at 7.5 (ties to even): zero 8,
    codes 15 / 0; below (s > S): zero 7, codes 14 / 0.  Row 0 of H is all +1
    (c > 0): scale fp32(a/15), zero 0, codes 15.  Every other group is all zero
    (scale 0, codes 0)."""
    K, g = 512, 128
    for i, gi, c in ((0, 0, 3.0), (77, 2, -1.5), (127, 3, 0.25)):
        x = np.zeros((1, K), np.float16)
        x[0, gi * g + i] = c
        r = o.kv_rotate_quant(x, group=g)
        signs = np.array([(-1.0) ** bin(i & j).count("1") for j in range(g)]) * np.sign(c)
        a = abs(c) / math.sqrt(g)
        S = (2 * a if i else a) / 15
        sf = float(np.float32(S))
        assert r["scale"][0, gi] == np.float32(S)
        hi_code = 15 if (not i or sf <= S) else 14
        np.testing.assert_array_equal(r["q"][0, gi * g:(gi + 1) * g], np.where(signs > 0, hi_code, 0))
        assert r["zero"][0, gi] == ((8 if sf <= S else 7) if i else 0)
        others = [k for k in range(K // g) if k != gi]
        assert np.all(r["scale"][0, others] == 0) and np.all(r["q"][0, [k * g + j for k in others for j in range(g)]] == 0)


def test_kv_rotate_quant_groups_are_independent_and_roundtrip():
    """Changing one group changes only that group's outputs; dequantized values
    rotated back (H is an involution) recover x within sqrt(g) * s / 2 per group."""
    rng = np.random.default_rng(22)
    T, K, g = 4, 1024, 128
    x = (rng.standard_normal((T, K)) * 3).astype(np.float16)
    r0 = o.kv_rotate_quant(x, group=g)
    x2 = x.copy()
    x2[2, 3 * g:4 * g] *= np.float16(-2)
    r1 = o.kv_rotate_quant(x2, group=g)
    diff = np.argwhere(r0["q"] != r1["q"])
    assert diff.size and np.all(diff[:, 0] == 2) and np.all(diff[:, 1] // g == 3)
    assert np.array_equal(np.argwhere(r0["scale"] != r1["scale"]), [[2, 3]])
    h = o.hadamard(g)
    for t in range(T):
        for gi in range(K // g):
            q = r0["q"][t, gi * g:(gi + 1) * g].astype(np.float64)
            s, z = float(r0["scale"][t, gi]), int(r0["zero"][t, gi])
            back = ((q - z) * s) @ h                   # H = H^T = H^{-1}
            err = np.linalg.norm(back - x[t, gi * g:(gi + 1) * g].astype(np.float64))
            assert err <= math.sqrt(g) * s / 2 * (1 + 1e-6)


def test_kv_rotate_quant_without_rotation_is_groupwise_asymmetric():
    """rotate=False: each group quantized on its own fp16 values; with a single
    group per row it is the per-token asymmetric quantizer."""
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((5, 256)) * 2).astype(np.float16)
    one = o.kv_rotate_quant(x, group=256, rotate=False)
    ref = o.rotate_quant(x, "none", asym=True)
    np.testing.assert_array_equal(one["q"], ref["q"])
    np.testing.assert_array_equal(one["scale"][:, 0], ref["scale"])
    np.testing.assert_array_equal(one["zero"][:, 0], ref["zero"])
    two = o.kv_rotate_quant(x, group=128, rotate=False)
    for gi in range(2):
        part = o.rotate_quant(np.ascontiguousarray(x[:, gi * 128:(gi + 1) * 128]), "none", asym=True)
        np.testing.assert_array_equal(two["q"][:, gi * 128:(gi + 1) * 128], part["q"])


# ---------------------------------------------------------------- 8-bit (QUIK-8B)

from fractions import Fraction


def _fp32_round(fr):
    """Correct rounding of an exact rational to fp32 (ties to even), without
    going through fp64: the two fp32 neighbours, compared exactly."""
    f = np.float32(float(fr))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = sorted(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best[0])


def _rne(fr):
    return round(fr)   # Fraction rounding is round-half-to-even


def _exact_asym8(row):
    xs = [Fraction(float(v)) for v in row]
    lo, hi = min(min(xs), Fraction(0)), max(max(xs), Fraction(0))
    s = _fp32_round((hi - lo) / 255)
    if s == 0:
        return [0] * len(xs), s, 0
    sf = Fraction(float(s))
    z = min(max(_rne(-lo / sf), 0), 255)
    return [min(max(_rne(x / sf) + z, 0), 255) for x in xs], s, z


def _exact_sym8(row, clip=1.0):
    xs = [Fraction(float(v)) for v in row]
    amax = max(abs(x) for x in xs)
    s = _fp32_round(Fraction(float(np.float32(clip))) * amax / 127)
    if s == 0:
        return [0] * len(xs), s
    sf = Fraction(float(s))
    return [min(max(_rne(x / sf), -127), 127) for x in xs], s


def test_8bit_quantizers_match_exact_rational_arithmetic():
    """Per-token asymmetric INT8 activations and per-channel symmetric INT8
    weights against exact rational arithmetic: workload rows with outlier
    columns split off, a row of exact ties (scale 2^-6 exactly), a zero row."""
    inp = workloads.make_inputs("quik_prefill", T=6, K=512, N=5)
    x, w, idx = inp["x"].copy(), inp["w"], inp["outlier_ch"][:32]
    keep = np.setdiff1d(np.arange(512), idx)
    ties = (np.arange(len(keep)) % 255) * 2.0 ** -6 + 2.0 ** -7   # (k + 1/2) s with s = 2^-6
    ties[0], ties[1] = 0.0, 255 * 2.0 ** -6                         # lo = 0, hi = 255 s
    x[4, keep] = ties.astype(np.float16)
    x[5] = 0
    xq = o.rotate_quant(x, "none", asym=True, outlier_idx=idx, bits=8)
    for t in range(6):
        q, s, z = _exact_asym8(x[t, keep].astype(np.float64))
        assert xq["scale"][t] == s and xq["zero"][t] == z
        np.testing.assert_array_equal(xq["q"][t], q)
    assert np.array_equal(xq["packed"], xq["q"].astype(np.uint8))
    assert len(set(xq["q"][4][2:].tolist()) & {0, 2, 4}) and xq["scale"][4] == 2.0 ** -6
    np.testing.assert_array_equal(xq["x_out"], x[:, idx])
    wq = o.prepare_weights(w, "none", outlier_idx=idx, bits=8)
    for n in range(5):
        q, s = _exact_sym8(w[n, keep].astype(np.float64))
        assert wq["scale"][n] == s
        np.testing.assert_array_equal(wq["q"][n], q)
    assert np.array_equal(wq["packed"].view(np.int8), wq["q"].astype(np.int8))
    assert np.array_equal(wq["rowsum"], wq["q"].astype(np.int64).sum(1))


def test_8bit_lossless_pipeline_and_bounds():
    """Operands already on their 8-bit grids go through exactly, and the
    mixed 8-bit pipeline reproduces (q - z) s (qw sw)^T + X_out W_out^T."""
    rng = np.random.default_rng(11)
    T, N, K = 5, 7, 256
    sx = 2.0 ** -3
    qx = rng.integers(0, 256, (T, K)); qx[:, 0], qx[:, 1] = 0, 255   # lo = -z s, hi = (255 - z) s
    z = 100
    x = (qx - z) * sx
    qw = rng.integers(-127, 128, (N, K)); qw[:, 0] = 127
    sw = 2.0 ** -9
    w = qw * sw
    x16, w16 = x.astype(np.float16), w.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x) and np.array_equal(w16.astype(np.float64), w)
    xq = o.rotate_quant(x16, "none", asym=True, bits=8)
    wq = o.prepare_weights(w16, "none", bits=8)
    np.testing.assert_array_equal(xq["q"], qx)
    assert np.all(xq["zero"] == z) and np.all(xq["scale"] == sx)
    np.testing.assert_array_equal(wq["q"], qw)
    y = o.linear(xq, wq)["y"]
    np.testing.assert_array_equal(y, (x @ w.T).astype(np.float16))
    # workload data: codes in range, half-step round trip, int32 accumulators fit
    inp = workloads.make_inputs("quik_prefill", T=8, K=1024, N=6)
    idx = inp["outlier_ch"][:64]
    xq = o.rotate_quant(inp["x"], "none", asym=True, outlier_idx=idx, bits=8)
    wq = o.prepare_weights(inp["w"], "none", outlier_idx=idx, bits=8)
    assert xq["q"].min() >= 0 and xq["q"].max() <= 255
    assert wq["q"].min() >= -127 and wq["q"].max() <= 127
    xn, _ = o.split_outliers(inp["x"].astype(np.float64), idx)
    xd = (xq["q"].astype(np.float64) - xq["zero"][:, None]) * xq["scale"].astype(np.float64)[:, None]
    assert np.all(np.abs(xd - xn) <= xq["scale"].astype(np.float64)[:, None] * 0.5 * (1 + 1e-6) + 1e-12)
    acc = o.linear(xq, wq)["acc"]
    np.testing.assert_array_equal(acc, o.int_gemm_bruteforce(xq["q"], wq["q"]))
    with pytest.raises(ValueError):
        o.code_max(6, True)


# ---------------------------------------------------------------- QUIK clip search

def _bruteforce_clip(row, steps, qmax):
    """The linear search in exact rational arithmetic, one plain loop per candidate."""
    xs = [Fraction(float(v)) for v in row]
    amax = max(abs(x) for x in xs)
    best, best_err = None, None
    for k in range(steps, 0, -1):
        c = np.float32(k / steps)
        s = _fp32_round(Fraction(float(c)) * amax / qmax)
        sf = Fraction(float(s))
        err = Fraction(0)
        for x in xs:
            q = 0 if sf == 0 else min(max(_rne(x / sf), -qmax), qmax)
            err += (x - sf * q) ** 2
        if best_err is None or err < best_err:
            best, best_err = c, err
    return best


def test_clip_search_matches_exact_bruteforce():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((4, 24)) * 0.02).astype(np.float16)
    w[1, 3] = 0.2                                  # one large value: clipping pays
    w[2] = 0                                       # zero row: every ratio ties, the first (1) stays
    for bits, qm in ((4, 7), (8, 127)):
        got = o.search_weight_clip(w, bits=bits, steps=20)["clip"]
        for n in range(4):
            assert got[n] == _bruteforce_clip(w[n].astype(np.float64), 20, qm), (bits, n)
    assert o.search_weight_clip(w, steps=20)["clip"][2] == 1.0


def test_clip_search_special_cases_and_invariances():
    rng = np.random.default_rng(6)
    # a row already on the c = 1 grid has zero error there, and ties keep 1
    grid = (rng.integers(-7, 8, (3, 64)) * 2.0 ** -6).astype(np.float16)
    grid[:, 0] = 7 * 2.0 ** -6
    assert np.all(o.search_weight_clip(grid)["clip"] == 1.0)
    # gaussian rows: clipping lowers the error (the choice is below 1 and
    # strictly better than c = 1)
    w = (rng.standard_normal((6, 4096)) * 0.02).astype(np.float16)
    r = o.search_weight_clip(w)
    assert np.all(r["clip"] < 1.0) and np.all(r["err"].min(axis=1) < r["err"][:, 0])
    # power-of-two scaling and column permutation leave the choice unchanged
    assert np.array_equal(o.search_weight_clip((w.astype(np.float64) * 8).astype(np.float16))["clip"], r["clip"])
    perm = rng.permutation(4096)
    assert np.array_equal(o.search_weight_clip(w[:, perm])["clip"], r["clip"])
    # outlier columns take no part: a huge value there changes nothing
    idx = np.array([5, 900], np.int32)
    w2 = w.copy()
    w2[:, idx] = 60.0
    keep = np.setdiff1d(np.arange(4096), idx)
    np.testing.assert_array_equal(o.search_weight_clip(w2, outlier_idx=idx)["clip"],
                                  o.search_weight_clip(w[:, keep])["clip"])
    # prepare_weights with the chosen per-row ratios equals per-row quantization
    wq = o.prepare_weights(w, "none", clip=r["clip"])
    for n in range(6):
        q1 = o.prepare_weights(w[n:n + 1], "none", clip=float(r["clip"][n]))
        assert np.array_equal(wq["q"][n], q1["q"][0]) and wq["scale"][n] == q1["scale"][0]
