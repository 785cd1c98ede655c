"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every test prints its case before touching the GPU.  Inputs come from the
seeded generators in `workloads`; expected values come from `oracle` only.
"""
import numpy as np
import pytest

import workloads
from oracle import rq_oracle as o
from parity_utils import (check_asym_quant, check_kv_quant, check_scales, check_sym_quant, check_y, dev,
                          flip_allowance, host, note)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
rq = pytest.importorskip("online_rotation_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rq.lib()  # raises if librq.so is missing: no silent fallback


def _rot_args(kind, block=0, inp=None):
    kw = {}
    if kind == "gsr":
        kw["block"] = block
    if kind == "kron":
        kw.update(p1=inp["p1"], p2=inp["p2"], chan_scale=inp["s"])
    return kw


def _gpu_rot(kind, block=0, inp=None):
    if kind == "kron":
        return rq.Rotation("kron", p1=dev(inp["p1"]), p2=dev(inp["p2"]), chan_scale=dev(inp["s"]))
    return rq.Rotation(kind, block=block)


# ----------------------------------------------------------------------------- quantizer

QUANT_CASES = [
    # name, workload, T, K, kind, block, clip, n1
    ("tiny-full", "tiny", None, None, "hadamard", 0, 1.0, 0),
    ("had4096-ragged", "llama7b", 301, 4096, "hadamard", 0, 1.0, 0),
    ("gsr64-4096-clip", "gsr", 301, 4096, "gsr", 64, 0.9, 0),
    ("gsr16-4096", "gsr", 37, 4096, "gsr", 16, 1.0, 0),
    ("gsr256-4096", "gsr", 37, 4096, "gsr", 256, 1.0, 0),
    ("gsr8-4096", "gsr", 37, 4096, "gsr", 8, 1.0, 0),
    ("gsr32-4096-clip", "gsr", 37, 4096, "gsr", 32, 0.9, 0),
    ("gsr128-4096", "gsr", 37, 4096, "gsr", 128, 1.0, 0),
    ("gsr64-1024-rowlds", "gsr", 41, 1024, "gsr", 64, 0.9, 0),
    ("had64-rowlds", "llama7b", 33, 64, "hadamard", 0, 1.0, 0),
    ("had1024-rowlds", "llama7b", 33, 1024, "hadamard", 0, 1.0, 0),
    ("had8192-rowlds", "llama7b", 9, 8192, "hadamard", 0, 1.0, 0),
    ("had32768-rowlds-max", "llama7b", 3, 32768, "hadamard", 0, 1.0, 0),
    ("kron64x64", "flat", 37, 4096, "kron", 0, 0.95, 64),
    ("kron16x16", "flat", 21, 256, "kron", 0, 0.95, 16),
    ("none-sym-512", "llama7b", 19, 512, "none", 0, 1.0, 0),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_rotate_quant_matches_oracle(case):
    name, wl, T, K, kind, block, clip, n1 = case
    note(f"[rotate_quant] {name}")
    inp = workloads.make_inputs(wl, T=T, K=K, with_weights=False, n1=n1 or None, n2=n1 or None)
    x = inp["x"]
    ref = o.rotate_quant(x, kind, clip=clip, **_rot_args(kind, block, inp))
    out = rq.rq_rotate_quant(dev(x), _gpu_rot(kind, block, inp), clip=clip, code_sum=True)
    torch.cuda.synchronize()
    check_sym_quant(host(out["q"]), host(out["scale"]), ref)
    q_gpu = o.unpack_int4(host(out["q"]), signed=True).astype(np.int64)
    assert np.array_equal(host(out["code_sum"]), q_gpu.sum(axis=1))


def test_rotate_quant_strided_rows():
    note("[rotate_quant] strided ldx")
    inp = workloads.make_inputs("llama7b", T=13, K=4096, with_weights=False)
    x = inp["x"]
    big = np.zeros((13, 4096 + 64), np.float16)
    big[:, :4096] = x
    ref = o.rotate_quant(x, "hadamard")
    xt = dev(big)[:, :4096]
    assert xt.stride(0) == 4160
    out = rq.rq_rotate_quant(xt, rq.Rotation("hadamard"))
    torch.cuda.synchronize()
    check_sym_quant(host(out["q"]), host(out["scale"]), ref)
    inp2 = workloads.make_inputs("tiny", T=5, with_weights=False)
    big2 = np.zeros((5, 256 + 8), np.float16)
    big2[:, :256] = inp2["x"]
    out2 = rq.rq_rotate_quant(dev(big2)[:, :256], rq.Rotation("hadamard"))
    torch.cuda.synchronize()
    check_sym_quant(host(out2["q"]), host(out2["scale"]), o.rotate_quant(inp2["x"], "hadamard"))


def _outlier_pattern(inp, K, n_out, pattern):
    if pattern == "workload":
        return np.ascontiguousarray(inp["outlier_ch"][:n_out]).astype(np.int32)
    # clustered: a dense run across word boundaries, both ends, and strays
    rng = np.random.default_rng(K + n_out)
    run = np.arange(K // 2 - 40, K // 2 - 40 + (n_out - 2) // 2)
    rest = np.setdiff1d(np.arange(1, K - 1), run)
    stray = rng.choice(rest, n_out - 2 - run.size, replace=False)
    idx = np.concatenate([[K - 1], run, stray, [0]]).astype(np.int32)
    assert np.unique(idx).size == n_out
    return idx


# The split kernel covers every K % 32 == 0 up to 32768 (1, 2 or 4 words of
# 32 columns per thread); 1100 rows exceed its grid, so its row loop turns over.
@pytest.mark.parametrize("T,K,n_out,pattern", [
    (37, 8192, 256, "workload"), (5, 8192, 0, "workload"), (3, 1024, 64, "workload"),
    (1100, 1024, 64, "clustered"), (29, 8192, 512, "clustered"), (7, 16384, 256, "workload"),
    (9, 16384, 128, "clustered"), (5, 32768, 256, "workload"), (3, 24576, 64, "clustered"),
    (11, 4096, 0, "workload")])
def test_asymmetric_outlier_split_matches_oracle(T, K, n_out, pattern):
    note(f"[rotate_quant] asym T={T} K={K} n_out={n_out} {pattern}")
    inp = workloads.make_inputs("quik_prefill", T=T, K=K, with_weights=False)
    x, idx = inp["x"], _outlier_pattern(inp, K, n_out, pattern)
    ref = o.rotate_quant(x, "none", asym=True, outlier_idx=idx if n_out else None)
    out = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True,
                             outlier_idx=dev(idx) if n_out else None, code_sum=True)
    torch.cuda.synchronize()
    check_asym_quant(host(out["q"]), host(out["scale"]), host(out["zero"]), ref)
    q_gpu = o.unpack_int4(host(out["q"]), signed=False).astype(np.int64)
    assert np.array_equal(host(out["code_sum"]), q_gpu.sum(axis=1))
    if n_out:
        assert np.array_equal(host(out["x_out"]).view(np.uint16), ref["x_out"].view(np.uint16))
        # the order of the index list does not matter
        perm = np.random.default_rng(0).permutation(n_out)
        out2 = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True,
                                  outlier_idx=dev(idx[perm].copy()))
        torch.cuda.synchronize()
        for k in ("q", "scale", "zero", "x_out"):
            assert torch.equal(out[k], out2[k]), k


# ----------------------------------------------------------------------------- weights

WEIGHT_CASES = [
    ("had4096", "llama7b", 200, 4096, "hadamard", 0, 0),
    ("gsr64", "gsr", 130, 4096, "gsr", 64, 0),
    ("kron64", "flat", 70, 4096, "kron", 0, 0),
    ("tiny", "tiny", None, None, "hadamard", 0, 0),
    ("quik-split", "quik_prefill", 100, 8192, "none", 0, 256),
]


@pytest.mark.parametrize("case", WEIGHT_CASES, ids=[c[0] for c in WEIGHT_CASES])
def test_prepare_weights_matches_oracle(case):
    name, wl, N, K, kind, block, n_out = case
    note(f"[prepare_weights] {name}")
    inp = workloads.make_inputs(wl, T=4, K=K, N=N)
    w = inp["w"]
    idx = inp["outlier_ch"][:n_out] if n_out else None
    ref = o.prepare_weights(w, kind, outlier_idx=idx, **_rot_args(kind, block, inp))
    out = rq.rq_prepare_weights(dev(w), _gpu_rot(kind, block, inp),
                                outlier_idx=dev(idx) if n_out else None)
    torch.cuda.synchronize()
    check_sym_quant(host(out["q"]), host(out["scale"]), ref, what="w")
    q_gpu = o.unpack_int4(host(out["q"]), signed=True).astype(np.int64)
    assert np.array_equal(host(out["rowsum"]), q_gpu.sum(axis=1))
    if n_out:
        assert np.array_equal(host(out["w_out"]).view(np.uint16), ref["w_out"].view(np.uint16))


# ----------------------------------------------------------------------------- GEMM

# With K % 128 == 0: T <= 16 runs the 16-channel decode kernel when the
# activation rows fit its 64 KB LDS stage (T * K / 2 bytes; (16, 100, 8192)
# fills it exactly, (16, 70, 8320) overflows it), otherwise and for T <= 32
# the 32-channel decode kernel; T >= 256 the register-A kernel; the rest and
# K % 128 != 0 the LDS-tile kernel.  Ragged N leaves idle wavefronts in the
# last decode workgroup; N > 16384 gives it more than 4 wavefronts (5 here,
# with the stage loaded in one group of 8 chunks per thread, then in two).
# Long rows at small N split each channel block's k-steps over 2 (K = 8192,
# 8320: parts of 33 and 32 steps), 4 (K = 16384) and 8 (K = 32768) wavefronts.
# 17 to 32 rows take the two-half form of the 16-channel kernel: staged in
# one, two or three groups of 8 chunks per thread, K split over two parts
# (T = 24, K = 8192), more than 16384 channels (T = 32, N = 16500); a stage
# above its LDS bound (T = 30, K = 16384) keeps the 32-channel kernel.
GEMM_SHAPES = [(1, 1, 64), (16, 256, 256), (200, 130, 192), (300, 257, 4096), (129, 130, 7936),
               (8, 300, 8192), (300, 129, 4032), (513, 200, 192), (256, 128, 64),
               (32, 513, 4096), (3, 1000, 7936), (17, 96, 128), (31, 33, 384),
               (16, 100, 8192), (16, 70, 8320), (9, 65, 4608), (4, 16500, 128), (16, 16400, 6144),
               (5, 300, 16384), (2, 40, 32768), (3, 70, 65536), (300, 130, 65536),
               (24, 100, 8192), (32, 16500, 1024), (30, 300, 16384), (21, 2000, 7936),
               # the 256-row kernel's k-step counts of 1, 2, 3, 5, 6, 7 and 9 (K / 128): partial
               # last groups of its 4-step schedule, an odd last step without its barrier
               (256, 130, 128), (300, 200, 256), (257, 129, 384), (300, 257, 640), (260, 64, 768),
               (512, 300, 896), (270, 100, 1152)]


@pytest.mark.parametrize("unsigned_x", [False, True])
@pytest.mark.parametrize("T,N,K", GEMM_SHAPES)
def test_gemm_int32_bit_exact(T, N, K, unsigned_x):
    note(f"[gemm_i32] T={T} N={N} K={K} unsigned_x={unsigned_x}")
    rng = np.random.default_rng(T * 7 + N * 3 + K)
    qx = rng.integers(0, 16, (T, K)) if unsigned_x else rng.integers(-8, 8, (T, K))
    qw = rng.integers(-8, 8, (N, K))
    acc = rq.rq_w4a4_gemm_i32(dev(o.pack_int4(qx)), dev(o.pack_int4(qw)), x_unsigned=unsigned_x)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), o.int_gemm(qx, qw))


@pytest.mark.parametrize("K", [128, 384, 640, 896, 4096])
def test_gemm_more_tiles_than_cus(K):
    """264 tiles of the 256-row kernel, more than the 256 CUs (two workgroups
    on some CUs), at 1, 3, 5, 7 and 32 k-steps: raw accumulators and the
    symmetric epilogue."""
    T, N = 2048, 4224
    note(f"[gemm_i32 + w4a4_linear, 264 tiles] T={T} N={N} K={K}")
    rng = np.random.default_rng(K + 1)
    qx = rng.integers(-8, 8, (T, K)); qw = rng.integers(-8, 8, (N, K))
    ref = o.int_gemm(qx, qw)
    acc = rq.rq_w4a4_gemm_i32(dev(o.pack_int4(qx)), dev(o.pack_int4(qw)))
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), ref)
    sx = rng.uniform(0.01, 0.1, T).astype(np.float32); sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    y = rq.rq_w4a4_linear(dev(o.pack_int4(qx)), dev(sx), dev(o.pack_int4(qw)), dev(sw))
    torch.cuda.synchronize()
    check_y(host(y), o.dequant_sym(ref, sx, sw))


@pytest.mark.parametrize("T,N,K", [(16, 256, 256), (300, 257, 4096), (77, 130, 3968), (270, 100, 4032),
                                   (7, 190, 3968), (24, 130, 3968), (32, 300, 8192),
                                   (256, 128, 128), (300, 257, 384), (260, 130, 640), (513, 100, 896)])
def test_linear_epilogue_on_oracle_codes(T, N, K):
    note(f"[w4a4_linear] T={T} N={N} K={K}")
    rng = np.random.default_rng(K + T)
    qx = rng.integers(-7, 8, (T, K)); qw = rng.integers(-7, 8, (N, K))
    sx = rng.uniform(0.01, 40, T).astype(np.float32); sw = rng.uniform(1e-4, 5e-3, N).astype(np.float32)
    y = rq.rq_w4a4_linear(dev(o.pack_int4(qx)), dev(sx), dev(o.pack_int4(qw)), dev(sw))
    torch.cuda.synchronize()
    check_y(host(y), o.dequant_sym(o.int_gemm(qx, qw), sx, sw))


@pytest.mark.parametrize("N,pad,off", [(4096, 0, 0), (260, 0, 0), (4096, 3, 0), (4100, 4, 8), (300, 8, 1)])
def test_large_gemm_output_layouts(N, pad, off):
    """The 256-row GEMM's output paths: 16-byte row stores through LDS when
    y rows are 16-byte aligned (N a multiple of 8, or a partial last chunk),
    element stores otherwise (a row pitch or a start not a multiple of 8
    elements); every layout holds the same values as a dense y."""
    T, K = 300, 1024
    note(f"[w4a4_linear layouts] T={T} N={N} K={K} row pad={pad} start offset={off}")
    rng = np.random.default_rng(N + pad + off)
    qx = rng.integers(-7, 8, (T, K)); qw = rng.integers(-7, 8, (N, K))
    sx = rng.uniform(0.01, 0.1, T).astype(np.float32); sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    args = (dev(o.pack_int4(qx)), dev(sx), dev(o.pack_int4(qw)), dev(sw))
    y = rq.rq_w4a4_linear(*args)
    big = torch.full((T * (N + pad) + off + 64,), float("nan"), dtype=torch.float16, device="cuda")
    view = big[off:off + T * (N + pad)].view(T, N + pad)[:, :N]
    rq.rq_w4a4_linear(*args, out=view)
    torch.cuda.synchronize()
    assert torch.equal(y, view)
    check_y(host(y), o.dequant_sym(o.int_gemm(qx, qw), sx, sw))
    rest = big.clone()
    rest[off:off + T * (N + pad)].view(T, N + pad)[:, :N] = 0
    assert torch.isnan(rest[:off]).all() and torch.isnan(rest[off + T * (N + pad):]).all()
    if pad:
        assert torch.isnan(big[off:off + T * (N + pad)].view(T, N + pad)[:, N:]).all()


@pytest.mark.parametrize("T,N,n_out,asym", [(37, 130, 256, True), (129, 64, 0, True), (20, 70, 32, False),
                                            (300, 150, 256, True), (260, 70, 32, False),
                                            (8, 300, 256, True), (32, 64, 96, True), (1, 40, 32, False),
                                            (15, 64, 96, True), (12, 130, 64, False), (5, 77, 0, True),
                                            (16, 200, 256, True), (24, 300, 256, True), (17, 4500, 64, False),
                                            (32, 1000, 256, True)])
def test_mixed_epilogue_on_oracle_codes(T, N, n_out, asym):
    note(f"[mixed_linear] T={T} N={N} n_out={n_out} asym={asym}")
    K = 7936
    rng = np.random.default_rng(n_out + T)
    qx = rng.integers(0, 16, (T, K)) if asym else rng.integers(-7, 8, (T, K))
    zx = rng.integers(0, 16, T).astype(np.int32) if asym else None
    qw = rng.integers(-7, 8, (N, K))
    rowsum = qw.sum(axis=1).astype(np.int32)
    sx = rng.uniform(0.01, 2, T).astype(np.float32); sw = rng.uniform(1e-4, 5e-3, N).astype(np.float32)
    xo = (rng.standard_normal((T, n_out)) * 40).astype(np.float16)
    wo = (rng.standard_normal((N, n_out)) * 0.02).astype(np.float16)
    y = rq.rq_mixed_outlier_linear(dev(o.pack_int4(qx)), dev(sx), dev(zx) if asym else None,
                                   dev(o.pack_int4(qw)), dev(sw), dev(rowsum) if asym else None,
                                   dev(xo) if n_out else None, dev(wo) if n_out else None)
    torch.cuda.synchronize()
    ref = o.dequant_mixed(o.int_gemm(qx, qw), sx, zx if asym else np.zeros(T, np.int32), sw, rowsum,
                          xo, wo)
    check_y(host(y), ref)


@pytest.mark.parametrize("K", [128, 384, 1152, 1280])
def test_mixed_epilogue_step_counts(K):
    """The QUIK form of the 256-row kernel (a barrier every step, groups of 3
    steps) at k-step counts of 1, 3, 9 and 10: whole and partial last groups."""
    T, N, n_out = 300, 200, 32
    note(f"[mixed_linear steps] T={T} N={N} K={K} n_out={n_out}")
    rng = np.random.default_rng(K)
    qx = rng.integers(0, 16, (T, K)); zx = rng.integers(0, 16, T).astype(np.int32)
    qw = rng.integers(-7, 8, (N, K)); rowsum = qw.sum(axis=1).astype(np.int32)
    sx = rng.uniform(0.01, 2, T).astype(np.float32); sw = rng.uniform(1e-4, 5e-3, N).astype(np.float32)
    xo = (rng.standard_normal((T, n_out)) * 40).astype(np.float16)
    wo = (rng.standard_normal((N, n_out)) * 0.02).astype(np.float16)
    y = rq.rq_mixed_outlier_linear(dev(o.pack_int4(qx)), dev(sx), dev(zx), dev(o.pack_int4(qw)), dev(sw),
                                   dev(rowsum), dev(xo), dev(wo))
    torch.cuda.synchronize()
    check_y(host(y), o.dequant_mixed(o.int_gemm(qx, qw), sx, zx, sw, rowsum, xo, wo))


# ----------------------------------------------------------------------------- fused decode

# The fused decode form against the oracle (codes within the quantizer
# tolerance, y within the output tolerance widened by the tolerated flips) and
# against the two calls it replaces, which here run the same 16-channel decode
# kernel on staged codes: equal bit for bit.  Shapes:
# the QUIK decode rows, T = 1 and the T = 16 maximum (at K = 8192 its LDS
# exceeds 64 KB), asymmetric and symmetric, with and without outliers, a
# clustered outlier run, small K, ragged N and N > 16384 (more than 4
# wavefronts per workgroup).
FUSED_CASES = [
    # T, N, K, n_out, asym, pattern
    (8, 300, 8192, 256, True, "workload"), (1, 64, 8192, 256, True, "workload"),
    (16, 130, 8192, 0, True, "workload"), (16, 130, 4096, 256, True, "clustered"),
    (5, 257, 4096, 0, True, "workload"),
    (7, 100, 4096, 0, False, "workload"), (3, 70, 2048, 128, False, "clustered"),
    (12, 16500, 1024, 128, True, "workload"), (16, 33, 128, 0, False, "workload"),
]


@pytest.mark.parametrize("T,N,K,n_out,asym,pattern", FUSED_CASES)
def test_quant_decode_linear_equals_two_calls(T, N, K, n_out, asym, pattern):
    note(f"[fused decode] T={T} N={N} K={K} n_out={n_out} asym={asym} {pattern}")
    inp = workloads.make_inputs("quik_prefill", T=T, K=K, with_weights=False)
    x = inp["x"]
    idx = _outlier_pattern(inp, K, n_out, pattern) if n_out else None
    w = (np.random.default_rng(N + K).standard_normal((N, K)) * 0.02).astype(np.float16)
    xd, wd = dev(x), dev(w)
    idxd = dev(idx) if n_out else None
    wq = rq.rq_prepare_weights(wd, rq.Rotation("none"), outlier_idx=idxd)
    xq = rq.rq_rotate_quant(xd, rq.Rotation("none"), asym=asym, outlier_idx=idxd)
    if asym or n_out:
        y2 = rq.rq_mixed_outlier_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"],
                                        wq["rowsum"] if asym else None, xq["x_out"], wq["w_out"])
    else:
        y2 = rq.rq_w4a4_linear(xq["q"], xq["scale"], wq["q"], wq["scale"])
    y1 = rq.rq_quant_decode_linear(xd, wq["q"], wq["scale"], wq["rowsum"] if asym else None,
                                   wq["w_out"], asym=asym, outlier_idx=idxd)
    torch.cuda.synchronize()
    _check_fused_against_oracle(x, w, idx, asym, xq, wq, y1)
    assert torch.equal(y1, y2)


def _check_fused_against_oracle(x, w, idx, asym, xq, wq, y1):
    """y of the fused form against o.rotate_quant + o.prepare_weights +
    o.linear; the codes the fused kernel made are those of the standalone
    quantizer (checked bit for bit against it through y above), so their
    tolerated flips widen the output tolerance."""
    ref = o.rotate_quant(x, "none", asym=asym, outlier_idx=idx)
    wr = o.prepare_weights(w, "none", outlier_idx=idx)
    fw = check_sym_quant(host(wq["q"]), host(wq["scale"]), wr, what="w")
    if asym:
        fx = check_asym_quant(host(xq["q"]), host(xq["scale"]), host(xq["zero"]), ref)
    else:
        fx = check_sym_quant(host(xq["q"]), host(xq["scale"]), ref)
    extra = flip_allowance(ref["scale"], wr["scale"], fx, fw)
    check_y(host(y1), o.linear(ref, wr)["y"], extra=extra, what="fused y")


# The rotated fused decode form (K = 4096): the 4096-point Walsh-Hadamard and
# GSR blocks of 64 / 16, with and without a clip ratio below 1, T from 1 to the
# 16-row maximum, N small, ragged and large (GSR's 11008: more than 4
# wavefronts per workgroup is not reached below 16384, so 4 here).  Against
# the oracle (rows' codes within the quantizer tolerance, y widened by their
# flips) and against the two calls bit for bit.
ROT_FUSED_CASES = [
    # T, N, workload, kind, block, clip
    (1, 4096, "llama7b", "hadamard", 0, 1.0), (8, 257, "llama7b", "hadamard", 0, 1.0),
    (16, 130, "llama7b", "hadamard", 0, 0.95), (3, 11008, "gsr", "gsr", 64, 0.9),
    (16, 96, "gsr", "gsr", 16, 1.0), (5, 70, "gsr", "gsr", 8, 0.9),
]


@pytest.mark.parametrize("T,N,wl,kind,block,clip", ROT_FUSED_CASES)
def test_rotate_quant_decode_linear_matches_oracle(T, N, wl, kind, block, clip):
    note(f"[rotated fused decode] T={T} N={N} {kind} block={block} clip={clip}")
    inp = workloads.make_inputs(wl, T=T, K=4096, N=N)
    x, w = inp["x"], inp["w"]
    rot = rq.Rotation(kind, block=block)
    xd, wd = dev(x), dev(w)
    wq = rq.rq_prepare_weights(wd, rot)
    y1 = rq.rq_rotate_quant_decode_linear(xd, rot, wq["q"], wq["scale"], clip=clip)
    xq = rq.rq_rotate_quant(xd, rot, clip=clip)
    y2 = rq.rq_w4a4_linear(xq["q"], xq["scale"], wq["q"], wq["scale"])
    torch.cuda.synchronize()
    kw = {"block": block} if kind == "gsr" else {}
    ref = o.rotate_quant(x, kind, clip=clip, **kw)
    wr = o.prepare_weights(w, kind, **kw)
    fx = check_sym_quant(host(xq["q"]), host(xq["scale"]), ref)
    fw = check_sym_quant(host(wq["q"]), host(wq["scale"]), wr, what="w")
    check_y(host(y1), o.linear(ref, wr)["y"], extra=flip_allowance(ref["scale"], wr["scale"], fx, fw, qmax_x=7),
            what="fused y")
    assert torch.equal(y1, y2)


def test_quant_decode_linear_exact_ties():
    """Rows with exact rounding ties take the exact-quotient path inside the
    fused kernel too."""
    note("[fused decode] exact ties")
    sym, asy = _exact_tie_rows(K=1024)
    w = (np.random.default_rng(3).standard_normal((96, 1024)) * 0.02).astype(np.float16)
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"))
    for rows, asym in ((sym[:16], False), (sym[16:], False), (asy[:8], True), (asy[8:], True)):
        xd = dev(np.ascontiguousarray(rows))
        xq = rq.rq_rotate_quant(xd, rq.Rotation("none"), asym=asym)
        if asym:
            y2 = rq.rq_mixed_outlier_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"], wq["rowsum"])
        else:
            y2 = rq.rq_w4a4_linear(xq["q"], xq["scale"], wq["q"], wq["scale"])
        y1 = rq.rq_quant_decode_linear(xd, wq["q"], wq["scale"], wq["rowsum"] if asym else None, asym=asym)
        torch.cuda.synchronize()
        _check_fused_against_oracle(rows, w, None, asym, xq, wq, y1)
        assert torch.equal(y1, y2)


# ----------------------------------------------------------------------------- end to end

E2E_CASES = [
    # name, workload, T, K, N, kind, block, clip, n1
    ("tiny-full", "tiny", None, None, None, "hadamard", 0, 1.0, 0),
    ("llama7b-small", "llama7b", 300, 4096, 200, "hadamard", 0, 1.0, 0),
    ("gsr-small", "gsr", 150, 4096, 260, "gsr", 64, 0.9, 0),
    ("flat-small", "flat", 70, 4096, 130, "kron", 0, 0.95, 64),
]


def _e2e(inp, kind, block, clip, x_rows=None, w_rows=None):
    """GPU full pipeline; returns GPU results on the requested rows."""
    x, w = inp["x"], inp["w"]
    rot = _gpu_rot(kind, block, inp)
    xd, wd = dev(x), dev(w)
    xq = rq.rq_rotate_quant(xd, rot, clip=clip)
    wq = rq.rq_prepare_weights(wd, rot)
    y = rq.rq_w4a4_linear(xq["q"], xq["scale"], wq["q"], wq["scale"])
    torch.cuda.synchronize()
    return xq, wq, y


@pytest.mark.parametrize("case", E2E_CASES, ids=[c[0] for c in E2E_CASES])
def test_end_to_end_matches_oracle(case):
    name, wl, T, K, N, kind, block, clip, n1 = case
    note(f"[e2e] {name}")
    inp = workloads.make_inputs(wl, T=T, K=K, N=N, n1=n1 or None, n2=n1 or None)
    kw = _rot_args(kind, block, inp)
    xr = o.rotate_quant(inp["x"], kind, clip=clip, **kw)
    wr = o.prepare_weights(inp["w"], kind, **kw)
    yr = o.linear(xr, wr)["y"]
    xq, wq, y = _e2e(inp, kind, block, clip)
    fx = check_sym_quant(host(xq["q"]), host(xq["scale"]), xr)
    fw = check_sym_quant(host(wq["q"]), host(wq["scale"]), wr, what="w")
    check_y(host(y), yr, extra=flip_allowance(xr["scale"], wr["scale"], fx, fw, qmax_x=7))


def test_end_to_end_quik_small():
    note("[e2e] quik small")
    inp = workloads.make_inputs("quik_prefill", T=40, K=8192, N=130)
    x, w, idx = inp["x"], inp["w"], inp["outlier_ch"]
    xr = o.rotate_quant(x, "none", asym=True, outlier_idx=idx)
    wr = o.prepare_weights(w, "none", outlier_idx=idx)
    yr = o.linear(xr, wr)["y"]
    xq = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True, outlier_idx=dev(idx))
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=dev(idx))
    y = rq.rq_mixed_outlier_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"],
                                   wq["rowsum"], xq["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    fx = check_asym_quant(host(xq["q"]), host(xq["scale"]), host(xq["zero"]), xr)
    fw = check_sym_quant(host(wq["q"]), host(wq["scale"]), wr, what="w")
    check_y(host(y), yr, extra=flip_allowance(xr["scale"], wr["scale"], fx, fw))


# ----------------------------------------------------------------------------- full size, sampled

FULL_CASES = [
    # name, workload, kind, block, clip
    ("llama7b", "llama7b", "hadamard", 0, 1.0),
    ("gsr", "gsr", "gsr", 64, 0.9),
    ("flat", "flat", "kron", 0, 0.95),
]


@pytest.mark.parametrize("case", FULL_CASES, ids=[c[0] for c in FULL_CASES])
def test_full_size_sampled(case):
    name, wl, kind, block, clip = case
    note(f"[full] {name}")
    inp = workloads.make_inputs(wl)
    x, w = inp["x"], inp["w"]
    T, N = x.shape[0], w.shape[0]
    rng = np.random.default_rng(99)
    ts = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, 45, replace=False)]))
    ns = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 254, replace=False)]))
    kw = _rot_args(kind, block, inp)
    xr = o.rotate_quant(x[ts], kind, clip=clip, **kw)
    wr = o.prepare_weights(w[ns], kind, **kw)
    yr = o.linear(xr, wr)["y"]
    xq, wq, y = _e2e(inp, kind, block, clip)
    fx = check_sym_quant(host(xq["q"])[ts], host(xq["scale"])[ts], xr)
    fw = check_sym_quant(host(wq["q"])[ns], host(wq["scale"])[ns], wr, what="w")
    check_y(host(y)[np.ix_(ts, ns)], yr, extra=flip_allowance(xr["scale"], wr["scale"], fx, fw, qmax_x=7))


@pytest.mark.parametrize("T", [2049, 5000])
@pytest.mark.parametrize("kind,block,clip", [("hadamard", 0, 1.0), ("gsr", 64, 0.9)])
def test_rotate_quant_several_tokens_per_wavefront(T, kind, block, clip):
    """K = 4096 above 2048 tokens: each wavefront takes an even number of tokens,
    prefetching the next; indices past the end are clamped onto the last row
    (T = 2049 gives most wavefronts such a clamped second token)."""
    note(f"[rotate_quant tpw>1] kind={kind} T={T}")
    x0 = workloads.make_inputs("llama7b", with_weights=False)["x"]
    reps = -(-T // x0.shape[0])
    x = np.concatenate([x0 * np.float16(1.0 + 0.25 * r) for r in range(reps)])[:T]
    rng = np.random.default_rng(T)
    ts = np.unique(np.concatenate([[0, 1, 1020, 1027, 1028, 2047, 2048, T - 2, T - 1],
                                   rng.choice(T, 40, replace=False)]))
    ts = ts[ts < T]
    xr = o.rotate_quant(x[ts], kind, clip=clip, **_rot_args(kind, block))
    xq = rq.rq_rotate_quant(dev(x), _gpu_rot(kind, block), clip=clip)
    torch.cuda.synchronize()
    check_sym_quant(host(xq["q"])[ts], host(xq["scale"])[ts], xr)


@pytest.mark.parametrize("T", [16384, 65536])
@pytest.mark.parametrize("name", ["llama7b", "gsr", "flat", "quik_prefill", "quik8_down"])
def test_rotate_quant_large_token_counts_sampled(name, T):
    """The quantizer at the benchmark's 16K and 64K token sweep in its launch
    configuration (up to 32 tokens per wavefront for the 4096-point transform,
    many rows per workgroup for the others): the workload's rows repeated, each
    copy scaled by its own factor so that a row written to the wrong place
    fails; sampled rows against the oracle."""
    note(f"[rotate_quant sweep] {name} T={T}")
    wl = workloads.get(name)
    inp = workloads.make_inputs(name, with_weights=False)
    x0 = inp["x"]
    T0 = x0.shape[0]
    x = np.concatenate([x0 * np.float16(1.0 + r / 64.0) for r in range(T // T0)])
    assert np.isfinite(x).all()
    rng = np.random.default_rng(T + T0)
    ts = np.unique(np.concatenate([[0, 1, 31, 32, 33, T0 - 1, T0, 2047, 2048, T - 33, T - 2, T - 1],
                                   rng.choice(T, 36, replace=False)]))
    kind, block = wl.rot, wl.block
    idx = inp["outlier_ch"].astype(np.int32) if wl.asym else None
    ref = o.rotate_quant(x[ts], kind, clip=wl.clip_x, asym=wl.asym, outlier_idx=idx, bits=wl.bits,
                         **_rot_args(kind, block, inp))
    out = rq.rq_rotate_quant(dev(x), _gpu_rot(kind, block, inp), clip=wl.clip_x, asym=wl.asym,
                             outlier_idx=None if idx is None else dev(idx), bits=wl.bits)
    torch.cuda.synchronize()
    del x
    sel = torch.from_numpy(ts).cuda()
    q, s = host(out["q"][sel]), host(out["scale"][sel])
    if wl.bits == 8:
        assert np.array_equal(q, ref["packed"]) and np.array_equal(s, ref["scale"])
        assert np.array_equal(host(out["zero"][sel]), ref["zero"])
    elif wl.asym:
        check_asym_quant(q, s, host(out["zero"][sel]), ref)
    else:
        check_sym_quant(q, s, ref)
    if idx is not None:
        assert np.array_equal(host(out["x_out"][sel]), ref["x_out"])


@pytest.mark.parametrize("wl", ["quik_prefill", "quik_decode"])
def test_full_size_quik_sampled(wl):
    note(f"[full] {wl}")
    inp = workloads.make_inputs(wl)
    x, w, idx = inp["x"], inp["w"], inp["outlier_ch"]
    T, N = x.shape[0], w.shape[0]
    rng = np.random.default_rng(7)
    ts = np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(T, 30), replace=False)]))
    ns = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 254, replace=False)]))
    xr = o.rotate_quant(x[ts], "none", asym=True, outlier_idx=idx)
    wr = o.prepare_weights(w[ns], "none", outlier_idx=idx)
    yr = o.linear(xr, wr)["y"]
    xq = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True, outlier_idx=dev(idx))
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=dev(idx))
    y = rq.rq_mixed_outlier_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"],
                                   wq["rowsum"], xq["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    fx = check_asym_quant(host(xq["q"])[ts], host(xq["scale"])[ts], host(xq["zero"])[ts], xr)
    fw = check_sym_quant(host(wq["q"])[ns], host(wq["scale"])[ns], wr, what="w")
    check_y(host(y)[np.ix_(ts, ns)], yr, extra=flip_allowance(xr["scale"], wr["scale"], fx, fw))
    if T <= 16:  # the fused decode form of the same step
        yf = rq.rq_quant_decode_linear(dev(x), wq["q"], wq["scale"], wq["rowsum"], wq["w_out"],
                                       asym=True, outlier_idx=dev(idx))
        torch.cuda.synchronize()
        assert torch.equal(yf, y)


@pytest.mark.parametrize("T,N,K", [(2048, 4096, 4096), (4096, 28672, 7936)])
def test_full_size_gemm_int32_sampled(T, N, K):
    """The bench's GEMM launch shape, on random codes, bit-exact on sampled outputs."""
    note(f"[full gemm_i32] T={T} N={N} K={K}")
    rng = np.random.default_rng(5)
    qx = rng.integers(-8, 8, (T, K), dtype=np.int8)
    qw = rng.integers(-8, 8, (N, K), dtype=np.int8)
    acc = host(rq.rq_w4a4_gemm_i32(dev(o.pack_int4(qx)), dev(o.pack_int4(qw))))
    ts = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 40, replace=False)]))
    ns = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 300, replace=False)]))
    assert np.array_equal(acc[np.ix_(ts, ns)], o.int_gemm(qx[ts], qw[ns]))


# ----------------------------------------------------------------------------- edge cases

def test_edge_rows_zero_constant_onehot_and_ties():
    note("[edge] crafted rows")
    K = 4096
    h = o.hadamard(K)
    rows = np.zeros((8, K))
    rows[1] = 3.0                                   # constant -> one nonzero code
    rows[2, 17] = 5.0                               # one-hot -> all codes +-7
    y = np.zeros(K); y[:6] = [7.0, 0.5, 1.5, 2.5, -2.5, -3.5]
    rows[3] = y @ h                                 # exact ties after rotation
    rows[4] = -rows[3]
    rows[5, :] = 1e-3                               # tiny values
    rows[6] = np.where(np.arange(K) % 2, 1.0, -1.0) * 65504.0 / 64  # large, exact
    rows[7, 4095] = -2.0
    x = rows.astype(np.float16)
    assert np.array_equal(x[3].astype(np.float64), rows[3])
    for kind, block, clip in (("hadamard", 0, 1.0), ("gsr", 64, 1.0), ("hadamard", 0, 0.9)):
        ref = o.rotate_quant(x, kind, clip=clip, block=block)
        out = rq.rq_rotate_quant(dev(x), rq.Rotation(kind, block=block), clip=clip)
        torch.cuda.synchronize()
        check_sym_quant(host(out["q"]), host(out["scale"]), ref)
        qg = o.unpack_int4(host(out["q"]), signed=True)
        assert not qg[0].any() and host(out["scale"])[0] == 0.0
        if kind == "hadamard" and clip == 1.0:
            np.testing.assert_array_equal(qg[3, :6], [7, 0, 2, 2, -2, -4])
            np.testing.assert_array_equal(qg[4, :6], [-7, 0, -2, -2, 2, 4])
    # zero activation row gives a zero output row
    inp = workloads.make_inputs("llama7b", T=4, K=K, N=64)
    xz = inp["x"].copy(); xz[2] = 0
    xq = rq.rq_rotate_quant(dev(xz), rq.Rotation("hadamard"))
    wq = rq.rq_prepare_weights(dev(inp["w"]), rq.Rotation("hadamard"))
    yy = host(rq.rq_w4a4_linear(xq["q"], xq["scale"], wq["q"], wq["scale"]))
    assert not yy[2].any()


def test_edge_asymmetric_rows():
    note("[edge] asymmetric rows")
    K = 1024
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, K))
    x[0] = np.abs(x[0])          # zero point 0
    x[1] = -np.abs(x[1])         # zero point 15
    x[2] = 0.0                   # zero row
    x[3] = 2.5                   # constant positive row
    x16 = x.astype(np.float16)
    ref = o.rotate_quant(x16, "none", asym=True)
    out = rq.rq_rotate_quant(dev(x16), rq.Rotation("none"), asym=True)
    torch.cuda.synchronize()
    check_asym_quant(host(out["q"]), host(out["scale"]), host(out["zero"]), ref)
    assert host(out["zero"])[0] == 0 and host(out["zero"])[1] == 15 and host(out["scale"])[2] == 0


def _wide_rows(T, K, qmax, asym, clip=1.0, seed=5):
    """fp16 rows whose scale numerator needs many bits: a large maximum
    (20..60) beside a tiny negative minimum (-5e-3..-1e-4), so that hi - lo
    (or clip * max) is not exact in fp32.  Columns 0 and 1 hold the bounds
    (hi and lo, or hi and -hi when symmetric); a quarter of each row holds the
    fp16 values of the row's range whose x / s lies closest to a rounding
    boundary (s the oracle's fp32 scale); row 0 holds a reported case: hi =
    39.78, lo = -0.002882, x = 31.28125 (x / s = 200.50001 at 8 bits)."""
    rng = np.random.default_rng(seed)
    all16 = np.arange(65536, dtype=np.uint16).view(np.float16)
    fin = np.unique(all16[np.isfinite(all16)].astype(np.float64))
    rows = []
    for t in range(T):
        if t == 0:
            hi, lo = float(np.float16(39.78)), float(np.float16(-0.002882))
        else:
            hi, lo = float(np.float16(rng.uniform(20, 60))), -float(np.float16(rng.uniform(1e-4, 5e-3)))
        num = (hi - lo) if asym else float(np.float32(clip)) * hi
        s = float(np.float32(num / qmax))
        cand = fin[(fin > lo) & (fin < hi)] if asym else fin[(fin > -hi) & (fin < hi)]
        pre = cand / s
        near = cand[np.argsort(np.abs(pre - np.floor(pre) - 0.5), kind="stable")[:K // 4]]
        body = rng.choice(cand, K - near.size - 3)
        # the bounds and the reported value in columns 0-2, the rest shuffled
        rows.append(np.concatenate([[hi, lo if asym else -hi, 31.28125 if t == 0 else body[0]],
                                    rng.permutation(np.concatenate([near, body]))]))
    x = np.array(rows).astype(np.float16)
    assert np.array_equal(x.astype(np.float64).max(axis=1), [r.max() for r in rows])
    return x


@pytest.mark.parametrize("bits,asym,clip,n_out", [(8, True, 1.0, 0), (8, True, 1.0, 64), (4, True, 1.0, 0),
                                                  (4, True, 1.0, 128), (4, False, 0.9, 0), (4, False, 1.0, 0),
                                                  (8, False, 0.9, 0)])
def test_wide_range_rows_are_exact(bits, asym, clip, n_out):
    """Rows whose scale numerator is not exact in fp32 (ranges spanning more
    than 24 bits, clip ratios below 1), packed with values next to rounding
    boundaries: scales, zero points and codes equal the oracle's exactly."""
    T, K = 9, 2048
    qm = ((1 << bits) - 1) if asym else ((1 << (bits - 1)) - 1)
    note(f"[rotate_quant] wide-range rows bits={bits} asym={asym} clip={clip} n_out={n_out}")
    x = _wide_rows(T, K, qm, asym, clip)
    idx = np.sort(np.random.default_rng(1).choice(np.arange(3, K), n_out, replace=False)).astype(np.int32) \
        if n_out else None
    ref = o.rotate_quant(x, "none", clip=clip, asym=asym, outlier_idx=idx, bits=bits)
    # the trap: with the numerator rounded to fp32 first, some scales differ
    x32 = x.astype(np.float32)
    num32 = (x32.max(axis=1) - np.minimum(x32.min(axis=1), 0)) if asym else np.float32(clip) * np.abs(x32).max(axis=1)
    assert np.any((num32 / np.float32(qm)).astype(np.float32) != ref["scale"]) or n_out or (not asym and clip == 1)
    out = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), clip=clip, asym=asym,
                             outlier_idx=None if idx is None else dev(idx), code_sum=True, bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["scale"]), ref["scale"]), "scales differ"
    if asym:
        assert np.array_equal(host(out["zero"]), ref["zero"]), "zero points differ"
    assert np.array_equal(host(out["q"]), ref["packed"]), "codes differ"
    assert np.array_equal(host(out["code_sum"]), ref["q"].astype(np.int64).sum(axis=1))
    if bits == 4 and asym:  # the fused decode form quantizes the same rows itself
        w = (np.random.default_rng(2).standard_normal((80, K)) * 0.02).astype(np.float16)
        wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=None if idx is None else dev(idx))
        y1 = rq.rq_quant_decode_linear(dev(x), wq["q"], wq["scale"], wq["rowsum"], wq["w_out"], asym=True,
                                       outlier_idx=None if idx is None else dev(idx))
        torch.cuda.synchronize()
        wr = o.prepare_weights(w, "none", outlier_idx=idx)
        assert np.array_equal(host(wq["q"]), wr["packed"])
        check_y(host(y1), o.linear(ref, wr)["y"])


def test_kv_wide_range_groups_are_exact():
    """Unrotated KV groups with a wide range (see _wide_rows): identical to
    the oracle; rotated, within the common tolerance."""
    g, K = 128, 1024
    x = np.concatenate([_wide_rows(8, g, 15, True, seed=s) for s in range(K // g)], axis=1)
    note(f"[kv_rotate_quant] wide-range groups {x.shape}")
    for rot in (False, True):
        ref = o.kv_rotate_quant(x, group=g, rotate=rot)
        out = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=rot)
        torch.cuda.synchronize()
        check_kv_quant(*(host(t) for t in out), ref, x, g, rot)


def _exact_tie_rows(seed=11, K=1024):
    """fp16 rows whose quotients x / S hit rounding boundaries exactly in the
    reals: symmetric rows with elements +-amax/2 (x/S = +-3.5, S = amax/7 not
    representable, so the rounding of S to fp32 decides), symmetric rows with
    S = 2^e representable (true ties, to even), asymmetric rows with hi = -lo
    (zero point -lo/S = 7.5) and asymmetric rows with S = 2^e."""
    rng = np.random.default_rng(seed)
    sym = (rng.standard_normal((24, K)) * 0.3).astype(np.float16)
    for r in range(16):
        amax = np.float16(rng.uniform(0.5, 4.0))
        sym[r] = np.clip(sym[r], -amax * 0.9, amax * 0.9)
        sym[r, 0] = amax if r % 2 else -amax
        sym[r, 1:9] = np.float16(amax / 2) * np.where(np.arange(8) % 2, 1, -1)
    for r in range(16, 24):
        e = 2.0 ** rng.integers(-4, 2)
        sym[r] = np.clip(sym[r], -6.9 * e, 6.9 * e)
        sym[r, 0] = 7 * e
        sym[r, 1:15] = (np.arange(14) % 7 + 0.5) * e * np.where(np.arange(14) < 7, 1, -1)
    asy = (rng.standard_normal((16, K)) * 0.3).astype(np.float16)
    for r in range(8):
        a = np.float16(rng.uniform(0.5, 4.0))
        asy[r] = np.clip(asy[r], -a, a)
        asy[r, 0], asy[r, 1] = a, -a
    for r in range(8, 16):
        e = 2.0 ** rng.integers(-4, 2)
        lo, hi = (-7.5 * e, 7.5 * e) if r % 2 else (-5 * e, 10 * e)
        asy[r] = np.clip(asy[r], lo, hi)
        asy[r, 0], asy[r, 1] = lo, hi
        asy[r, 2:12] = (np.arange(10) - 4.5) * e
    return sym.astype(np.float16), asy.astype(np.float16)


def test_edge_exact_fp16_ties():
    """Unrotated fp16 inputs meet exact rounding boundaries often; the GPU
    must round them as rne(x / fp32 scale) does, code for code."""
    note("[edge] exact ties on fp16 inputs")
    sym, asy = _exact_tie_rows()
    ref = o.rotate_quant(sym, "none")
    assert (np.abs(ref["pre"] - np.round(ref["pre"] - 0.5) - 0.5) < 1e-6).sum() >= 100
    out = rq.rq_rotate_quant(dev(sym), rq.Rotation("none"))
    torch.cuda.synchronize()
    check_scales(host(out["scale"]), ref["scale"])
    np.testing.assert_array_equal(o.unpack_int4(host(out["q"]), signed=True), ref["q"])
    refa = o.rotate_quant(asy, "none", asym=True)
    outa = rq.rq_rotate_quant(dev(asy), rq.Rotation("none"), asym=True)
    torch.cuda.synchronize()
    check_scales(host(outa["scale"]), refa["scale"])
    np.testing.assert_array_equal(host(outa["zero"]), refa["zero"])
    np.testing.assert_array_equal(o.unpack_int4(host(outa["q"]), signed=False), refa["q"])
    # the weight side with an outlier split (outliers away from the crafted columns)
    idx = np.sort(np.random.default_rng(12).choice(np.arange(64, 1024), 64, replace=False)).astype(np.int32)
    wr = o.prepare_weights(sym, "none", outlier_idx=idx)
    wq = rq.rq_prepare_weights(dev(sym), rq.Rotation("none"), outlier_idx=dev(idx))
    torch.cuda.synchronize()
    check_scales(host(wq["scale"]), wr["scale"])
    np.testing.assert_array_equal(o.unpack_int4(host(wq["q"]), signed=True), wr["q"])


def test_empty_and_single_row():
    note("[edge] T=0 and T=1")
    x0 = torch.empty((0, 4096), dtype=torch.float16, device="cuda")
    out = rq.rq_rotate_quant(x0, rq.Rotation("hadamard"))
    assert out["q"].shape == (0, 2048)
    inp = workloads.make_inputs("llama7b", T=1, K=4096, N=130)
    xr = o.rotate_quant(inp["x"], "hadamard"); wr = o.prepare_weights(inp["w"], "hadamard")
    xq, wq, y = _e2e(inp, "hadamard", 0, 1.0)
    fx = check_sym_quant(host(xq["q"]), host(xq["scale"]), xr)
    fw = check_sym_quant(host(wq["q"]), host(wq["scale"]), wr, what="w")
    check_y(host(y), o.linear(xr, wr)["y"], extra=flip_allowance(xr["scale"], wr["scale"], fx, fw, qmax_x=7))
    y0 = rq.rq_w4a4_linear(xq["q"][:0], xq["scale"][:0], wq["q"], wq["scale"])
    torch.cuda.synchronize()
    assert y0.shape == (0, 130)


def test_deterministic_reruns():
    note("[edge] determinism")
    inp = workloads.make_inputs("gsr", T=64, K=4096, N=256)
    a = _e2e(inp, "gsr", 64, 0.9)
    b = _e2e(inp, "gsr", 64, 0.9)
    assert torch.equal(a[0]["q"], b[0]["q"]) and torch.equal(a[2], b[2])


# ----------------------------------------------------------------------------- KV cache

KV_CASES = [
    # name, T, K, group, rotate, tensor
    ("g128-rot-ragged", 301, 4096, 128, True, "x"),
    ("g64-rot", 37, 4096, 64, True, "x"),
    ("g256-rot", 37, 4096, 256, True, "x"),
    ("g128-values-rot", 41, 4096, 128, True, "v"),
    ("g128-plain", 301, 4096, 128, False, "x"),
    ("g64-plain", 19, 1024, 64, False, "x"),
    ("g256-plain-values", 19, 2048, 256, False, "v"),
    ("one-group", 1, 128, 128, True, "x"),
    ("one-group-plain", 1, 64, 64, False, "x"),
    ("three-groups", 3, 384, 128, True, "x"),
    ("wide-8192", 5, 8192, 128, True, "x"),
    ("24-groups-per-row", 77, 3072, 128, True, "x"),
    ("21-groups-per-row", 50, 1344, 64, True, "v"),
    ("21-groups-per-row-plain", 50, 1344, 64, False, "x"),
]


@pytest.mark.parametrize("case", KV_CASES, ids=[c[0] for c in KV_CASES])
def test_kv_rotate_quant_matches_oracle(case):
    name, T, K, g, rot, which = case
    note(f"[kv_rotate_quant] {name} T={T} K={K} group={g} rotate={rot}")
    x = workloads.make_inputs("kv", T=T, K=K, with_weights=False)[which]
    ref = o.kv_rotate_quant(x, group=g, rotate=rot)
    out = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=rot)
    torch.cuda.synchronize()
    check_kv_quant(*(host(t) for t in out), ref, x, g, rot)


def test_kv_rotate_quant_strided_rows_and_degenerate_groups():
    note("[kv_rotate_quant] strided ldx, zero / constant / one-signed groups")
    T, K, g = 6, 1024, 128
    x = workloads.make_inputs("kv", T=T, K=K, with_weights=False)["x"].copy()
    x[0] = 0                      # all-zero rows: scale 0, zero point 0, codes 0
    x[1] = 1.5                    # constant: one nonzero value after R3
    x[2] = -2.0                   # constant negative
    x[3, :g] = np.abs(x[3, :g])   # one-signed groups
    x[4, g:2 * g] = -np.abs(x[4, g:2 * g])
    big = np.zeros((T, K + 64), np.float16)
    big[:, :K] = x
    xt = dev(big)[:, :K]
    assert xt.stride(0) == K + 64
    for rot in (True, False):
        ref = o.kv_rotate_quant(x, group=g, rotate=rot)
        out = rq.rq_kv_rotate_quant(xt, group=g, rotate=rot)
        torch.cuda.synchronize()
        check_kv_quant(*(host(t) for t in out), ref, x, g, rot)
        assert np.all(host(out[1])[0] == 0) and np.all(host(out[2])[0] == 0)


def _tie_inputs(g, s, rng):
    """fp16 rows whose R3 image v is sparse on the grid of odd multiples of
    s/2 with hi - lo = 15 s, so that every nonzero v / scale is an exact tie,
    and whose values x = v . H / sqrt(g) are exact in fp16 (g = 64, 256:
    1/sqrt(g) is a power of two)."""
    from scipy.linalg import hadamard
    rows = []
    for _ in range(8):
        v = np.zeros(g)
        idx = rng.choice(g, 14, replace=False)
        v[idx[:12]] = s * (rng.integers(-7, 7, 12) + 0.5)
        v[idx[12]], v[idx[13]] = 7.5 * s, -7.5 * s
        x = v @ hadamard(g) / np.sqrt(g)
        assert np.array_equal(x.astype(np.float16).astype(np.float64), x)
        rows.append(x)
    return np.array(rows).reshape(2, 4 * g).astype(np.float16)


@pytest.mark.parametrize("g", [64, 256])
def test_kv_rotate_quant_exact_ties(g):
    """Every nonzero rotated value is a tie; the transform is exact, so the
    codes must round half to even exactly as the oracle."""
    note(f"[kv_rotate_quant] exact ties group={g}")
    rng = np.random.default_rng(g)
    x = _tie_inputs(g, 0.5 if g == 64 else 1.0, rng)
    ref = o.kv_rotate_quant(x, group=g, rotate=True)
    assert (np.abs(ref["pre"] - np.floor(ref["pre"]) - 0.5) == 0).sum() > 50
    q, s, z = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), ref["packed"])
    assert np.array_equal(host(s), ref["scale"]) and np.array_equal(host(z), ref["zero"])
    # the same ties without the transform (the inputs on a half-step grid)
    xp = (np.round(x.astype(np.float64) * 2) / 2).astype(np.float16)
    refp = o.kv_rotate_quant(xp, group=g, rotate=False)
    q, s, z = rq.rq_kv_rotate_quant(dev(xp), group=g, rotate=False)
    torch.cuda.synchronize()
    check_kv_quant(host(q), host(s), host(z), refp, xp, g, False)


def test_kv_rotate_quant_full_size_sampled():
    """The kv workload at its full size (2048 tokens x 4096 channels, g=128),
    in the launch the benchmark times: sampled token rows against the oracle,
    the values (no rotation) against it in full."""
    inp = workloads.make_inputs("kv", with_weights=False)
    x, v = inp["x"], inp["v"]
    note(f"[kv_rotate_quant] full size {x.shape}")
    out = rq.rq_kv_rotate_quant(dev(x), group=128, rotate=True)
    outv = rq.rq_kv_rotate_quant(dev(v), group=128, rotate=False)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, x.shape[0] - 1, np.random.default_rng(7).choice(x.shape[0], 125, replace=False)])
    ref = o.kv_rotate_quant(x[rows], group=128, rotate=True)
    check_kv_quant(host(out[0])[rows], host(out[1])[rows], host(out[2])[rows], ref, x[rows], 128, True)
    check_kv_quant(*(host(t) for t in outv), o.kv_rotate_quant(v, group=128, rotate=False), v, 128, False)


def test_kv_rotate_quant_grid_stride():
    """More groups than one grid step covers (4096 wavefronts x 16 groups):
    the grid-stride loop, rows that wrap inside a set (24 groups per row, a
    step of 65536 groups is 2730 rows + 16 groups) and the clamped last set;
    then 64 groups per row over 8200 rows."""
    for T, K, g in ((3000, 3072, 128), (8200, 4096, 64)):
        note(f"[kv_rotate_quant] grid stride T={T} K={K} group={g}")
        x = workloads.make_inputs("kv", T=T, K=K, with_weights=False)["v"]
        q, s, z = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=False)
        torch.cuda.synchronize()
        check_kv_quant(host(q), host(s), host(z), o.kv_rotate_quant(x, group=g, rotate=False), x, g, False)
        rows = np.r_[0:3, 1023:1026, 2729:2733, T - 3:T]
        q, s, z = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=True)
        torch.cuda.synchronize()
        check_kv_quant(host(q)[rows], host(s)[rows], host(z)[rows], o.kv_rotate_quant(x[rows], group=g), x[rows],
                       g, True)


@pytest.mark.parametrize("rot", [True, False])
def test_kv_rotate_quant_widest_rows(rot):
    """K = 2^21 channels (the largest the ABI takes), 16384 groups per row.
    Groups are independent (an oracle pin), so the oracle runs on the rows cut
    into one group each; the keys and values launch gets the same rows."""
    T, K, g = 2, 1 << 21, 128
    note(f"[kv_rotate_quant] widest rows T={T} K={K} group={g} rotate={rot}")
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((T, K)) * np.where(rng.random(K) < 0.01, 30.0, 1.0)).astype(np.float16)
    ref = o.kv_rotate_quant(x.reshape(T * K // g, g), group=g, rotate=rot)
    ref = {"q": ref["q"].reshape(T, K), "scale": ref["scale"].reshape(T, K // g),
           "zero": ref["zero"].reshape(T, K // g), "pre": ref["pre"].reshape(T, K),
           "zpre": ref["zpre"].reshape(T, K // g), "packed": ref["packed"].reshape(T, K // 2)}
    out = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=rot)
    ok_, ov = rq.rq_kv_cache_quant(dev(x), dev(x[::-1].copy()), group=g, rotate_k=rot, rotate_v=rot)
    torch.cuda.synchronize()
    check_kv_quant(*(host(t) for t in out), ref, x, g, rot)
    for a, b in zip(out, ok_):
        assert torch.equal(a, b)
    for a, b in zip(out, ov):   # the values were the same rows in reverse order
        assert torch.equal(a, b.flip(0))


def _offset_codes(T, K, off=4):
    """A dense uint8 [T, K/2] view that starts `off` bytes into its buffer:
    4-byte aligned, not 16-byte aligned."""
    buf = torch.empty(T * (K // 2) + 16, dtype=torch.uint8, device="cuda")
    return buf[off:off + T * (K // 2)].view(T, K // 2)


def _kv_out(T, K, g, q=None):
    return (q if q is not None else torch.empty((T, K // 2), dtype=torch.uint8, device="cuda"),
            torch.empty((T, K // g), dtype=torch.float32, device="cuda"),
            torch.empty((T, K // g), dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("g", [128, 256])
def test_kv_rotate_quant_codes_at_4_byte_alignment(g):
    """Codes buffers that are 4- but not 16-byte aligned take the dword
    stores; the result is the same as with an aligned buffer."""
    T, K = 45, 2048
    note(f"[kv_rotate_quant] codes 4-byte aligned group={g}")
    x = workloads.make_inputs("kv", T=T, K=K, with_weights=False)["x"]
    for rot in (True, False):
        a = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=rot)
        b = rq.rq_kv_rotate_quant(dev(x), group=g, rotate=rot, out=_kv_out(T, K, g, _offset_codes(T, K)))
        torch.cuda.synchronize()
        assert b[0].data_ptr() % 16 == 4
        for u, w in zip(a, b):
            assert torch.equal(u, w)
        check_kv_quant(*(host(t) for t in b), o.kv_rotate_quant(x, group=g, rotate=rot), x, g, rot)


KV_PAIR_CASES = [
    # name, T, K, group, rotate keys, rotate values
    ("g128-ragged", 301, 4096, 128, True, False),
    ("g64-both-rotated", 37, 4096, 64, True, True),
    ("g256", 37, 4096, 256, True, False),
    ("g64-plain", 19, 1024, 64, False, False),
    ("values-rotated-only", 41, 4096, 128, False, True),
    ("one-group", 1, 128, 128, True, False),
    ("24-groups-per-row", 77, 3072, 128, True, False),
    ("grid-stride", 3000, 3072, 128, True, False),
]


@pytest.mark.parametrize("case", KV_PAIR_CASES, ids=[c[0] for c in KV_PAIR_CASES])
def test_kv_cache_quant_pair(case):
    """Keys and values in one launch: each tensor's outputs are those of its
    own rq_kv_rotate_quant call, bit for bit, and match the oracle."""
    name, T, K, g, rk, rv = case
    note(f"[kv_cache_quant] {name} T={T} K={K} group={g} rotate_k={rk} rotate_v={rv}")
    inp = workloads.make_inputs("kv", T=T, K=K, with_weights=False)
    k, v = inp["x"], inp["v"]
    ok_, ov = rq.rq_kv_cache_quant(dev(k), dev(v), group=g, rotate_k=rk, rotate_v=rv)
    sk = rq.rq_kv_rotate_quant(dev(k), group=g, rotate=rk)
    sv = rq.rq_kv_rotate_quant(dev(v), group=g, rotate=rv)
    torch.cuda.synchronize()
    for a, b in zip(ok_ + ov, sk + sv):
        assert torch.equal(a, b)
    rows = np.arange(T) if T <= 400 else np.r_[0:3, 1023:1026, 2729:2733, T - 3:T]
    for x, out, rot in ((k, ok_, rk), (v, ov, rv)):
        check_kv_quant(*(host(t)[rows] for t in out), o.kv_rotate_quant(x[rows], group=g, rotate=rot), x[rows],
                       g, rot)


def test_kv_cache_quant_strided_and_unaligned():
    """Different leading dimensions for keys and values, and a values codes
    buffer that is only 4-byte aligned (every tensor then takes the dword
    stores)."""
    T, K, g = 29, 1024, 128
    note("[kv_cache_quant] strided rows, 4-byte aligned codes")
    inp = workloads.make_inputs("kv", T=T, K=K, with_weights=False)
    k, v = inp["x"], inp["v"]
    kb = np.zeros((T, K + 64), np.float16)
    kb[:, :K] = k
    vb = np.zeros((T, K + 8), np.float16)
    vb[:, :K] = v
    kt, vt = dev(kb)[:, :K], dev(vb)[:, :K]
    ok_, ov = rq.rq_kv_cache_quant(kt, vt, group=g, out_v=_kv_out(T, K, g, _offset_codes(T, K)))
    torch.cuda.synchronize()
    check_kv_quant(*(host(t) for t in ok_), o.kv_rotate_quant(k, group=g, rotate=True), k, g, True)
    check_kv_quant(*(host(t) for t in ov), o.kv_rotate_quant(v, group=g, rotate=False), v, g, False)


def test_kv_cache_quant_full_size_sampled():
    """The kv workload at its full size (keys and values [2048, 4096], g=128)
    in the one launch the benchmark times: sampled key rows against the
    oracle, the values in full."""
    inp = workloads.make_inputs("kv", with_weights=False)
    k, v = inp["x"], inp["v"]
    note(f"[kv_cache_quant] full size {k.shape}")
    ok_, ov = rq.rq_kv_cache_quant(dev(k), dev(v), group=128)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, k.shape[0] - 1, np.random.default_rng(8).choice(k.shape[0], 125, replace=False)])
    check_kv_quant(*(host(t)[rows] for t in ok_), o.kv_rotate_quant(k[rows], group=128, rotate=True), k[rows],
                   128, True)
    check_kv_quant(*(host(t) for t in ov), o.kv_rotate_quant(v, group=128, rotate=False), v, 128, False)


# ----------------------------------------------------------------------------- 8-bit (QUIK-8B)

Q8_CASES = [
    # name, T, K, n_out, pattern, asym, clip
    ("asym-64", 37, 2048, 64, "workload", True, 1.0),
    ("asym-clustered-192", 19, 4096, 192, "clustered", True, 1.0),
    ("sym-clip", 23, 1024, 0, "workload", False, 0.9),
    ("asym-down-proj-width", 5, 28672, 896, "workload", True, 1.0),
    ("sym-32768", 3, 32768, 0, "workload", False, 1.0),
    ("asym-more-rows-than-grid", 2100, 512, 64, "workload", True, 1.0),
]


@pytest.mark.parametrize("case", Q8_CASES, ids=[c[0] for c in Q8_CASES])
def test_rotate_quant_8bit_matches_oracle(case):
    name, T, K, n_out, pattern, asym, clip = case
    note(f"[rotate_quant 8-bit] {name} T={T} K={K} n_out={n_out}")
    inp = workloads.make_inputs("quik8_down", T=T, K=K, with_weights=False)
    x = inp["x"].copy()
    if T >= 4:  # a zero row, a constant row and a row of exact ties (scale 2^-6)
        x[1] = 0
        x[2] = 0.75
        x[3] = ((np.arange(K) % 255) * 2.0 ** -6 + 2.0 ** -7).astype(np.float16)
    idx = _outlier_pattern(inp, K, n_out, pattern) if n_out else None
    if idx is not None and T >= 4:
        keep = np.setdiff1d(np.arange(K), idx)
        x[3, keep[0]], x[3, keep[1]] = 0.0, 255 * 2.0 ** -6
    ref = o.rotate_quant(x, "none", clip=clip, asym=asym, outlier_idx=idx, bits=8)
    out = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), clip=clip, asym=asym,
                             outlier_idx=None if idx is None else dev(idx), code_sum=True, bits=8)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["q"]), ref["packed"]), "codes differ"
    assert np.array_equal(host(out["scale"]), ref["scale"]), "scales differ"
    if asym:
        assert np.array_equal(host(out["zero"]), ref["zero"]), "zero points differ"
    assert np.array_equal(host(out["code_sum"]), ref["q"].astype(np.int64).sum(axis=1))
    if n_out:
        assert np.array_equal(host(out["x_out"]), ref["x_out"])


def test_prepare_weights_8bit_matches_oracle():
    note("[prepare_weights 8-bit] N=70 K=2048 n_out=64")
    inp = workloads.make_inputs("quik8_down", T=4, K=2048, N=70)
    idx = inp["outlier_ch"][:64].astype(np.int32)
    ref = o.prepare_weights(inp["w"], "none", outlier_idx=idx, bits=8)
    wq = rq.rq_prepare_weights(dev(inp["w"]), rq.Rotation("none"), outlier_idx=dev(idx), bits=8)
    torch.cuda.synchronize()
    assert np.array_equal(host(wq["q"]), ref["packed"])
    assert np.array_equal(host(wq["scale"]), ref["scale"])
    assert np.array_equal(host(wq["rowsum"]), ref["rowsum"])
    assert np.array_equal(host(wq["w_out"]), ref["w_out"])


GEMM8_SHAPES = [(300, 1024, 200), (5, 64, 33), (257, 27776, 130), (1, 128, 1), (513, 2048, 257),
                (5, 32768, 70), (260, 32768, 129)]


@pytest.mark.parametrize("shape", GEMM8_SHAPES, ids=[f"{t}x{k}x{n}" for t, k, n in GEMM8_SHAPES])
@pytest.mark.parametrize("unsigned", [True, False], ids=["u8", "s8"])
def test_w8a8_gemm_i32_bit_exact(shape, unsigned):
    T, K, N = shape
    note(f"[w8a8_gemm_i32] T={T} K={K} N={N} unsigned={unsigned}")
    rng = np.random.default_rng(T * 7 + K + N)
    qx = rng.integers(0, 256, (T, K)) if unsigned else rng.integers(-127, 128, (T, K))
    qw = rng.integers(-127, 128, (N, K))
    qx[0, :] = 255 if unsigned else 127   # extremes in the first row and column
    qw[0, :] = -127
    ref = o.int_gemm(qx, qw)
    rowsum = qw.sum(axis=1).astype(np.int32)
    acc = rq.rq_w8a8_gemm_i32(dev(qx.astype(np.int16).astype(np.uint8)), dev(qw.astype(np.int16).astype(np.uint8)),
                              x_unsigned=unsigned, w_rowsum=dev(rowsum) if unsigned else None)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), ref)


# The decode-size 8-bit kernel (T <= 32): K split 4 ways (N < 16384), 2 ways
# (16384 <= N < 32768, or T > 16 with 4 parts over 64 staged rows) and not at
# all (N >= 32768); one or two blocks of 16 tokens; K parts of unequal length
# and steps past the end of a part (K = 27776 = 434 steps, K = 64 = 1 step).
D8_SHAPES = [(1, 27776, 100), (8, 27776, 8192), (16, 1024, 33), (17, 4096, 130), (32, 640, 16400),
             (3, 64, 40000), (5, 4160, 2048), (32, 27776, 257)]


@pytest.mark.parametrize("shape", D8_SHAPES, ids=[f"{t}x{k}x{n}" for t, k, n in D8_SHAPES])
@pytest.mark.parametrize("unsigned", [True, False], ids=["u8", "s8"])
def test_w8a8_decode_gemm_i32_bit_exact(shape, unsigned):
    T, K, N = shape
    note(f"[w8a8_gemm_i32 decode] T={T} K={K} N={N} unsigned={unsigned}")
    rng = np.random.default_rng(T * 11 + K + N)
    qx = rng.integers(0, 256, (T, K)) if unsigned else rng.integers(-127, 128, (T, K))
    qw = rng.integers(-127, 128, (N, K))
    qx[0, :] = 255 if unsigned else -127
    qw[-1, :] = -127
    ref = o.int_gemm(qx, qw)
    rowsum = qw.sum(axis=1).astype(np.int32)
    acc = rq.rq_w8a8_gemm_i32(dev(qx.astype(np.int16).astype(np.uint8)), dev(qw.astype(np.int16).astype(np.uint8)),
                              x_unsigned=unsigned, w_rowsum=dev(rowsum) if unsigned else None)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), ref)


@pytest.mark.parametrize("T,N,n_out", [(8, 8192, 896), (1, 300, 64), (16, 130, 0), (24, 2100, 896),
                                       (32, 64, 64)])
def test_w8a8_linear_decode_kernel(T, N, n_out):
    """The 8-bit linear layer at decode sizes (the decode kernel: codes from
    LDS phases, the outlier product split over the K parts and summed) against
    the oracle, at the down projection's width."""
    K = 28672
    note(f"[w8a8_linear decode] T={T} K={K} N={N} n_out={n_out}")
    inp = workloads.make_inputs("quik8_down", T=T, K=K, N=N)
    x, w = inp["x"], inp["w"]
    idx = inp["outlier_ch"][:n_out].astype(np.int32) if n_out else None
    didx = dev(idx) if n_out else None
    xr = o.rotate_quant(x, "none", asym=True, outlier_idx=idx, bits=8)
    wr = o.prepare_weights(w, "none", outlier_idx=idx, bits=8)
    xq = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True, outlier_idx=didx, bits=8)
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=didx, bits=8)
    y = rq.rq_w8a8_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"], wq["rowsum"],
                          xq["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    assert np.array_equal(host(xq["q"]), xr["packed"]) and np.array_equal(host(wq["q"]), wr["packed"])
    check_y(host(y), o.linear(xr, wr)["y"])
    # symmetric activations (signed codes, no zero point)
    xs = o.rotate_quant(x, "none", outlier_idx=idx, bits=8)
    xqs = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), outlier_idx=didx, bits=8)
    ys = rq.rq_w8a8_linear(xqs["q"], xqs["scale"], None, wq["q"], wq["scale"], wq["rowsum"],
                           xqs["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    check_y(host(ys), o.linear(xs, wr)["y"])


@pytest.mark.parametrize("n_out", [64, 0])
def test_w8a8_linear_end_to_end(n_out):
    note(f"[w8a8_linear] T=70 K=2048 N=96 n_out={n_out}")
    inp = workloads.make_inputs("quik8_down", T=70, K=2048, N=96)
    x, w = inp["x"], inp["w"]
    idx = inp["outlier_ch"][:n_out].astype(np.int32) if n_out else None
    xr = o.rotate_quant(x, "none", asym=True, outlier_idx=idx, bits=8)
    wr = o.prepare_weights(w, "none", outlier_idx=idx, bits=8)
    yr = o.linear(xr, wr)["y"]
    didx = dev(idx) if n_out else None
    xq = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True, outlier_idx=didx, bits=8)
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=didx, bits=8)
    y = rq.rq_w8a8_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"], wq["rowsum"],
                          xq["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    assert np.array_equal(host(xq["q"]), xr["packed"]) and np.array_equal(host(wq["q"]), wr["packed"])
    check_y(host(y), yr)
    # symmetric activations (signed codes, no zero point)
    xs = o.rotate_quant(x, "none", outlier_idx=idx, bits=8)
    xqs = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), outlier_idx=didx, bits=8)
    ys = rq.rq_w8a8_linear(xqs["q"], xqs["scale"], None, wq["q"], wq["scale"], wq["rowsum"],
                           xqs["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    check_y(host(ys), o.linear(xs, wr)["y"])


def test_quik8_full_size_sampled():
    """The quik8_down workload at full size (T=4096, K=28672, N=8192, 896
    outliers) in the benchmark's calls: sampled token rows and weight rows
    against the oracle, and y at their crossings."""
    inp = workloads.make_inputs("quik8_down")
    x, w = inp["x"], inp["w"]
    idx = inp["outlier_ch"].astype(np.int32)
    note(f"[quik8 full size] x {x.shape} w {w.shape} n_out {idx.size}")
    didx = dev(idx)
    xq = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True, outlier_idx=didx, bits=8)
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=didx, bits=8)
    y = rq.rq_w8a8_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"], wq["rowsum"],
                          xq["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    ts = np.unique(np.r_[0, x.shape[0] - 1, rng.choice(x.shape[0], 22, replace=False)])
    ns = np.unique(np.r_[0, w.shape[0] - 1, rng.choice(w.shape[0], 30, replace=False)])
    xr = o.rotate_quant(x[ts], "none", asym=True, outlier_idx=idx, bits=8)
    wr = o.prepare_weights(w[ns], "none", outlier_idx=idx, bits=8)
    assert np.array_equal(host(xq["q"])[ts], xr["packed"])
    assert np.array_equal(host(xq["zero"])[ts], xr["zero"]) and np.array_equal(host(xq["scale"])[ts], xr["scale"])
    assert np.array_equal(host(wq["q"])[ns], wr["packed"]) and np.array_equal(host(wq["rowsum"])[ns], wr["rowsum"])
    check_y(host(y)[np.ix_(ts, ns)], o.linear(xr, wr)["y"])


# ----------------------------------------------------------------------------- QUIK clip search

def _check_clip_choice(clip_gpu, ref, what="clip"):
    """The GPU's ratio is the oracle's, or ties with it: the oracle's error at
    the GPU's ratio is within 1e-12 (relative) of the minimum.  (The GPU sums
    the same fp64 terms in another order.)"""
    clip_gpu = np.asarray(clip_gpu)
    diff = clip_gpu != ref["clip"]
    for n in np.flatnonzero(diff):
        j = int(np.flatnonzero(ref["ratios"] == clip_gpu[n])[0])
        best = ref["err"][n].min()
        assert ref["err"][n, j] <= best * (1 + 1e-12) + 1e-300, f"{what}: row {n} picked {clip_gpu[n]}"
    return int(diff.sum())


CLIP_CASES = [
    # name, workload, N, K, n_out, bits, steps
    ("4bit-outliers", "quik_prefill", 300, 1024, 32, 4, 100),
    ("8bit-outliers", "quik8_down", 70, 2048, 64, 8, 100),
    ("4bit-odd-steps", "llama7b", 41, 4096, 0, 4, 7),
    ("4bit-one-step", "llama7b", 5, 512, 0, 4, 1),
    ("8bit-width-32768", "quik8_down", 3, 32768, 0, 8, 100),
]


@pytest.mark.parametrize("case", CLIP_CASES, ids=[c[0] for c in CLIP_CASES])
def test_clip_search_matches_oracle(case):
    name, wl, N, K, n_out, bits, steps = case
    note(f"[clip search] {name} N={N} K={K} n_out={n_out} bits={bits} steps={steps}")
    inp = workloads.make_inputs(wl, T=4, K=K, N=N)
    w = inp["w"].copy()
    w[1] = 0                                          # zero row: ratio 1
    qm = 127 if bits == 8 else 7
    w[2, :] = (np.arange(K) % (2 * qm + 1) - qm) * 2.0 ** -10   # on the c = 1 grid: ratio 1
    idx = inp["outlier_ch"][:n_out].astype(np.int32) if n_out else None
    ref = o.search_weight_clip(w, outlier_idx=idx, bits=bits, steps=steps)
    clip = rq.rq_search_weight_clip(dev(w), outlier_idx=None if idx is None else dev(idx), bits=bits, steps=steps)
    torch.cuda.synchronize()
    _check_clip_choice(host(clip), ref)
    assert host(clip)[1] == 1.0 and host(clip)[2] == 1.0


@pytest.mark.parametrize("bits", [4, 8])
def test_prepare_weights_with_searched_clip(bits):
    """Weight prep with the searched per-row ratios equals the oracle's
    prepare_weights at those ratios (bit-exact at 8 bits; at 4 bits within
    the quantizer tolerance, whose fp32 scale rounding differs)."""
    wl = "quik8_down" if bits == 8 else "quik_prefill"
    note(f"[prepare_weights searched clip] bits={bits}")
    inp = workloads.make_inputs(wl, T=4, K=2048, N=150)
    w, idx = inp["w"], inp["outlier_ch"][:64].astype(np.int32)
    clip = rq.rq_search_weight_clip(dev(w), outlier_idx=dev(idx), bits=bits)
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=dev(idx), bits=bits, row_clip=clip)
    torch.cuda.synchronize()
    ref = o.prepare_weights(w, "none", clip=host(clip), outlier_idx=idx, bits=bits)
    assert np.any(host(clip) < 1.0)   # gaussian rows: clipping pays (at 8 bits, not on every row)
    if bits == 8:
        assert np.array_equal(host(wq["q"]), ref["packed"]) and np.array_equal(host(wq["scale"]), ref["scale"])
        assert np.array_equal(host(wq["rowsum"]), ref["rowsum"])
    else:
        check_sym_quant(host(wq["q"]), host(wq["scale"]), ref, what="w")
    assert np.array_equal(host(wq["w_out"]), ref["w_out"])


def test_clip_search_full_size_sampled():
    """QUIK's 4-bit weight side at full size: W [28672, 8192] with 256 outlier
    columns (the quik_prefill workload), sampled rows against the oracle."""
    inp = workloads.make_inputs("quik_prefill")
    w, idx = inp["w"], inp["outlier_ch"].astype(np.int32)
    note(f"[clip search full size] w {w.shape}")
    clip = rq.rq_search_weight_clip(dev(w), outlier_idx=dev(idx))
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, w.shape[0] - 1, np.random.default_rng(3).choice(w.shape[0], 30, replace=False)])
    ref = o.search_weight_clip(w[rows], outlier_idx=idx)
    _check_clip_choice(host(clip)[rows], ref)


def test_8bit_quantizer_and_clip_search_strided_rows():
    """Row strides above K (ldx = K + 64) through the 8-bit quantizer, the clip
    search and the weight prep with searched ratios."""
    note("[8-bit / clip search] strided rows")
    inp = workloads.make_inputs("quik8_down", T=9, K=2048, N=11)
    x, w, idx = inp["x"], inp["w"], inp["outlier_ch"][:64].astype(np.int32)
    bx = np.zeros((9, 2048 + 64), np.float16)
    bx[:, :2048] = x
    bw = np.zeros((11, 2048 + 64), np.float16)
    bw[:, :2048] = w
    xt, wt = dev(bx)[:, :2048], dev(bw)[:, :2048]
    assert xt.stride(0) == 2112 and wt.stride(0) == 2112
    xq = rq.rq_rotate_quant(xt, rq.Rotation("none"), asym=True, outlier_idx=dev(idx), bits=8)
    clip = rq.rq_search_weight_clip(wt, outlier_idx=dev(idx), bits=8)
    wq = rq.rq_prepare_weights(wt, rq.Rotation("none"), outlier_idx=dev(idx), bits=8, row_clip=clip)
    torch.cuda.synchronize()
    xr = o.rotate_quant(x, "none", asym=True, outlier_idx=idx, bits=8)
    assert np.array_equal(host(xq["q"]), xr["packed"]) and np.array_equal(host(xq["x_out"]), xr["x_out"])
    _check_clip_choice(host(clip), o.search_weight_clip(w, outlier_idx=idx, bits=8))
    wr = o.prepare_weights(w, "none", clip=host(clip), outlier_idx=idx, bits=8)
    assert np.array_equal(host(wq["q"]), wr["packed"]) and np.array_equal(host(wq["scale"]), wr["scale"])


@pytest.mark.parametrize("T", [1, 8, 16, 33])
def test_w8a8_linear_decode_sizes(T):
    """Decode-sized batches through the 8-bit linear layer, the full
    down-projection width: the decode kernel up to 32 rows, the 256-row tile
    kernel with clamped rows above."""
    note(f"[w8a8_linear] decode T={T}")
    inp = workloads.make_inputs("quik8_down", T=T, K=28672, N=130)
    x, w, idx = inp["x"], inp["w"], inp["outlier_ch"].astype(np.int32)
    xr = o.rotate_quant(x, "none", asym=True, outlier_idx=idx, bits=8)
    wr = o.prepare_weights(w, "none", outlier_idx=idx, bits=8)
    xq = rq.rq_rotate_quant(dev(x), rq.Rotation("none"), asym=True, outlier_idx=dev(idx), bits=8)
    wq = rq.rq_prepare_weights(dev(w), rq.Rotation("none"), outlier_idx=dev(idx), bits=8)
    y = rq.rq_w8a8_linear(xq["q"], xq["scale"], xq["zero"], wq["q"], wq["scale"], wq["rowsum"],
                          xq["x_out"], wq["w_out"])
    torch.cuda.synchronize()
    check_y(host(y), o.linear(xr, wr)["y"])
