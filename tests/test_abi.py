"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/rq.h declares, and its host-side validation rejects bad arguments
with the documented status codes before anything is launched.

Every test runs in both sessions: once unmarked (the CPU session) and once
marked `gpu` (the GPU session, against the library the GPU tests load).  A
missing librq.so is built first, never skipped."""
import ctypes
import os
import re

import pytest

import online_rotation_amd as rq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rq.h")



@pytest.fixture(scope="module", autouse=True,
                params=[pytest.param("host"), pytest.param("gpu-session", marks=pytest.mark.gpu)])
def _library(request):
    if not os.path.exists(rq.LIB_PATH):
        from online_rotation_amd import build
        build.build()
    assert os.path.exists(rq.LIB_PATH), "librq.so is missing"
    return request.param

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rq_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(rq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = rq.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert rq.rq_abi_version() == 2
    assert rq.rq_status_string(0) == "RQ_OK"
    for s in range(1, 5):
        assert rq.rq_status_string(s).startswith("RQ_E")


def _rot(kind="hadamard", block=0, n1=0, n2=0, p1=None, p2=None, cs=None):
    return rq._RotDesc(rq.ROT_KINDS[kind], block, n1, n2, p1, p2, cs)


def _qd(asym=0, clip=1.0, idx=None, n_out=0):
    return rq._QuantDesc(asym, clip, idx, n_out)


def _rotate_quant(T, K, ldx, rot, qd, x=FAKE, q=FAKE, scale=FAKE, zero=None, x_out=None):
    return rq.lib().rq_rotate_quant(x, T, K, ldx, ctypes.byref(rot), ctypes.byref(qd), q, scale,
                                    zero, None, x_out, None)


@pytest.mark.parametrize("T,K,ldx,rot,qd,want", [
    (4, 4096, 4096, _rot("hadamard"), _qd(clip=0.0), rq.RQ_EINVAL),           # clip out of range
    (4, 4096, 4096, _rot("hadamard"), _qd(clip=1.5), rq.RQ_EINVAL),
    (-1, 4096, 4096, _rot("hadamard"), _qd(), rq.RQ_EINVAL),                  # negative T
    (4, 3000, 3000, _rot("hadamard"), _qd(), rq.RQ_ESHAPE),                   # not a power of two
    (4, 65536, 65536, _rot("hadamard"), _qd(), rq.RQ_ESHAPE),                 # too large
    (4, 4096, 4096, _rot("gsr", block=48), _qd(), rq.RQ_ESHAPE),              # block not pow2
    (4, 4096, 4096, _rot("gsr", block=512), _qd(), rq.RQ_ESHAPE),             # block too large
    (4, 4096, 4096, _rot("kron", n1=64, n2=32, p1=FAKE, p2=FAKE), _qd(), rq.RQ_ESHAPE),  # K != n1*n2
    (4, 4096, 4096, _rot("kron", n1=64, n2=64), _qd(), rq.RQ_EINVAL),         # null factors
    (4, 4096, 4096, _rot("hadamard"), _qd(asym=1), rq.RQ_ESHAPE),             # asym + rotation
    (4, 4096, 4096, _rot("hadamard"), _qd(idx=FAKE, n_out=64), rq.RQ_ESHAPE),  # split + rotation
    (4, 8192, 8192, _rot("none"), _qd(idx=FAKE, n_out=100), rq.RQ_ESHAPE),    # K - n_out % 64
    (4, 8192, 8192, _rot("none"), _qd(n_out=256), rq.RQ_EINVAL),              # null idx
    (4, 4096, 4000, _rot("hadamard"), _qd(), rq.RQ_EALIGN),                   # ldx < K
    (4, 4096, 4100, _rot("hadamard"), _qd(), rq.RQ_EALIGN),                   # ldx % 8
    (4, 4096, 4096, _rot("none"), _qd(asym=1, clip=0.9), rq.RQ_EINVAL),       # asym takes clip 1
    (4, 4104, 4104, _rot("none"), _qd(), rq.RQ_ESHAPE),                       # K % 64 with no split
    (4, 32832, 32832, _rot("none"), _qd(idx=FAKE, n_out=64), rq.RQ_ESHAPE),   # K > 32768 unrotated
    (4, 8232, 8232, _rot("none"), _qd(idx=FAKE, n_out=40), rq.RQ_ESHAPE),     # K % 32 unrotated
])
def test_rotate_quant_validation(T, K, ldx, rot, qd, want):
    assert _rotate_quant(T, K, ldx, rot, qd, x_out=FAKE) == want
    assert rq.rq_last_error() != ""


def test_rotate_quant_alignment_and_nulls():
    rot, qd = _rot("hadamard"), _qd()
    assert _rotate_quant(4, 4096, 4096, rot, qd, x=FAKE + 2) == rq.RQ_EALIGN
    assert _rotate_quant(4, 4096, 4096, rot, qd, q=None) == rq.RQ_EINVAL
    assert _rotate_quant(4, 8192, 8192, _rot("none"), _qd(asym=1), zero=None) == rq.RQ_EINVAL
    assert _rotate_quant(4, 8448, 8448, _rot("none"), _qd(idx=FAKE, n_out=256)) == rq.RQ_EINVAL  # x_out
    L = rq.lib()
    assert L.rq_rotate_quant(FAKE, 4, 4096, 4096, None, ctypes.byref(qd), FAKE, FAKE, None, None,
                             None, None) == rq.RQ_EINVAL
    bad = _rot("hadamard"); bad.kind = 9
    assert _rotate_quant(4, 4096, 4096, bad, qd) == rq.RQ_EINVAL


def test_empty_batch_is_a_no_op():
    # T == 0 passes validation and launches nothing, so it is safe without a GPU
    assert _rotate_quant(0, 4096, 4096, _rot("hadamard"), _qd(), x=None, q=None, scale=None) == rq.RQ_OK
    L = rq.lib()
    assert L.rq_w4a4_linear(None, None, 0, 4096, None, None, 16, None, 16, None) == rq.RQ_OK
    assert L.rq_w4a4_gemm_i32(None, 0, 0, 4096, None, 16, None, 16, None) == rq.RQ_OK


def test_gemm_validation():
    L = rq.lib()
    assert L.rq_w4a4_linear(FAKE, FAKE, 8, 100, FAKE, FAKE, 16, FAKE, 16, None) == rq.RQ_ESHAPE  # K % 64
    assert L.rq_w4a4_linear(FAKE, FAKE, 8, 4096, FAKE, FAKE, 0, FAKE, 16, None) == rq.RQ_EINVAL  # N
    assert L.rq_w4a4_linear(FAKE, FAKE, 8, 4096, FAKE, FAKE, 16, FAKE, 12, None) == rq.RQ_EALIGN  # ldy < N
    assert L.rq_w4a4_linear(FAKE, FAKE, 8, 4096, FAKE, FAKE, 16, FAKE + 1, 16, None) == rq.RQ_EALIGN  # fp16 y
    assert L.rq_w4a4_linear(FAKE + 8, FAKE, 8, 4096, FAKE, FAKE, 16, FAKE, 16, None) == rq.RQ_EALIGN
    assert L.rq_w4a4_linear(FAKE, None, 8, 4096, FAKE, FAKE, 16, FAKE, 16, None) == rq.RQ_EINVAL
    assert L.rq_w4a4_linear(FAKE, FAKE, 8, 131072, FAKE, FAKE, 16, FAKE, 16, None) == rq.RQ_ESHAPE
    assert L.rq_w4a4_gemm_i32(FAKE, 0, 8, 4096, FAKE, 16, FAKE + 2, 16, None) == rq.RQ_EALIGN  # int32 acc
    assert L.rq_w4a4_gemm_i32(FAKE, 0, 65535 * 128 + 1, 4096, FAKE, 16, FAKE, 16, None) == rq.RQ_ESHAPE
    assert L.rq_mixed_outlier_linear(FAKE, FAKE, FAKE, 8, 7936, FAKE, FAKE, FAKE, 16, FAKE, FAKE,
                                     100, FAKE, 16, None) == rq.RQ_ESHAPE                    # n_out % 32
    assert L.rq_mixed_outlier_linear(FAKE, FAKE, FAKE, 8, 7936, FAKE, FAKE, None, 16, FAKE, FAKE,
                                     256, FAKE, 16, None) == rq.RQ_EINVAL                    # rowsum
    assert L.rq_mixed_outlier_linear(FAKE, FAKE, None, 8, 7936, FAKE, FAKE, None, 16, None, None,
                                     256, FAKE, 16, None) == rq.RQ_EINVAL                    # outliers


def test_quant_decode_linear_validation():
    L = rq.lib()
    f = L.rq_quant_decode_linear
    qd, qa = _qd(), _qd(asym=1, idx=FAKE, n_out=256)
    args = lambda T, K, qd, rowsum=FAKE, w_out=FAKE, ldy=16: (FAKE, T, K, K, ctypes.byref(qd), FAKE, FAKE, rowsum,
                                                             16, w_out, FAKE, ldy, None)
    assert f(*args(0, 4096, qd)) == rq.RQ_OK                       # T == 0
    assert f(*args(17, 4096, qd)) == rq.RQ_ESHAPE                  # T > 16: the two calls
    assert f(*args(8, 16384, qd)) == rq.RQ_ESHAPE                  # K > 8192
    assert f(*args(8, 4160, qd)) == rq.RQ_ESHAPE                   # K % 128 with n_out = 0
    assert f(*args(8, 8192, qa, rowsum=None)) == rq.RQ_EINVAL      # asymmetric without w_rowsum
    assert f(*args(8, 8192, qa, w_out=None)) == rq.RQ_EINVAL       # outliers without w_out
    assert f(*args(8, 8192, qa, ldy=12)) == rq.RQ_EALIGN           # ldy < N
    assert f(*args(8, 8192, _qd(asym=1, idx=FAKE, n_out=100))) == rq.RQ_ESHAPE  # n_out % 32
    assert f(*args(8, 8192, _qd(asym=1, clip=0.9))) == rq.RQ_EINVAL             # asymmetric clip
    assert f(FAKE, 8, 4096, 4096, None, FAKE, FAKE, None, 16, None, FAKE, 16, None) == rq.RQ_EINVAL


def test_kv_rotate_quant_validation():
    L = rq.lib()
    f = L.rq_kv_rotate_quant
    ok = lambda T=8, K=4096, ldx=4096, g=128, x=FAKE, q=FAKE, s=FAKE, z=FAKE: f(x, T, K, ldx, g, 1, q, s, z, None)
    assert ok(T=0) == rq.RQ_OK                              # empty batch: nothing launched
    assert ok(T=-1) == rq.RQ_EINVAL
    assert ok(g=96) == rq.RQ_ESHAPE                         # group not 64 / 128 / 256
    assert ok(g=32) == rq.RQ_ESHAPE
    assert ok(K=4160) == rq.RQ_ESHAPE                       # K % group
    assert ok(ldx=4090) == rq.RQ_EALIGN                     # ldx < K
    assert ok(ldx=4100) == rq.RQ_EALIGN                     # ldx % 8
    assert ok(x=None) == rq.RQ_EALIGN
    assert ok(x=FAKE + 2) == rq.RQ_EALIGN                   # x 16-byte aligned
    assert ok(q=FAKE + 2) == rq.RQ_EALIGN                   # q 4-byte aligned
    assert ok(s=None) == rq.RQ_EALIGN
    assert ok(z=FAKE + 1) == rq.RQ_EALIGN


def test_kv_cache_quant_validation():
    L = rq.lib()
    MB = 1 << 24
    K_, V_ = FAKE, FAKE + 8 * MB   # keys' and values' buffers, far apart

    def desc(base, x=None, ldx=4096, q=None, s=None, z=None, rot=1):
        return rq._KvTensor(base if x is None else x, ldx, rot, base + MB if q is None else q,
                            base + 2 * MB if s is None else s, base + 3 * MB if z is None else z)

    def call(k=None, v=None, T=8, K=4096, g=128):
        k = desc(K_) if k is None else k
        v = desc(V_, rot=0) if v is None else v
        return L.rq_kv_cache_quant(ctypes.byref(k), ctypes.byref(v), T, K, g, None)

    assert L.rq_kv_cache_quant(None, ctypes.byref(desc(V_)), 8, 4096, 128, None) == rq.RQ_EINVAL
    assert L.rq_kv_cache_quant(ctypes.byref(desc(K_)), None, 8, 4096, 128, None) == rq.RQ_EINVAL
    assert call(T=-1) == rq.RQ_EINVAL
    assert call(g=96) == rq.RQ_ESHAPE
    assert call(K=4160) == rq.RQ_ESHAPE
    assert call(k=desc(K_, ldx=4090)) == rq.RQ_EALIGN            # keys ldx < K
    assert call(v=desc(V_, ldx=4100)) == rq.RQ_EALIGN            # values ldx % 8
    assert call(k=desc(K_, x=FAKE + 2)) == rq.RQ_EALIGN
    assert call(v=desc(V_, q=V_ + MB + 2)) == rq.RQ_EALIGN       # codes 4-byte aligned
    assert call(v=desc(V_, s=0)) == rq.RQ_EALIGN                 # null scale
    assert call(k=desc(K_, z=K_ + 3 * MB + 1)) == rq.RQ_EALIGN
    # outputs shared or overlapping between keys and values
    assert call(v=desc(V_, q=K_ + MB)) == rq.RQ_EINVAL
    assert call(v=desc(V_, s=K_ + 3 * MB)) == rq.RQ_EINVAL          # values' scale on keys' zero points
    assert call(v=desc(V_, q=K_ + MB + 8 * 2048 - 16)) == rq.RQ_EINVAL  # the last 16 bytes of keys' codes
    # T == 0: nothing to check beyond the descriptors, nothing launched
    assert call(T=0) == rq.RQ_OK


def test_prepare_weights_validation_and_workspace():
    L = rq.lib()
    kron = _rot("kron", n1=64, n2=64, p1=FAKE, p2=FAKE)
    assert L.rq_prepare_weights_workspace_bytes(ctypes.byref(kron)) == 2 * 64 * 64 * 4
    assert L.rq_prepare_weights_workspace_bytes(ctypes.byref(_rot("hadamard"))) == 0
    assert L.rq_prepare_weights_workspace_bytes(None) == 0
    qd = _qd()
    # KRON without a workspace
    assert L.rq_prepare_weights(FAKE, 8, 4096, 4096, ctypes.byref(kron), ctypes.byref(qd), FAKE, FAKE,
                                None, None, None, 0, None) == rq.RQ_EINVAL
    # asymmetric weights are not a thing
    assert L.rq_prepare_weights(FAKE, 8, 4096, 4096, ctypes.byref(_rot("none")), ctypes.byref(_qd(asym=1)),
                                FAKE, FAKE, None, None, None, 0, None) == rq.RQ_EINVAL


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 4096), dtype=torch.float16)
    with pytest.raises(ValueError):
        rq.rq_rotate_quant(x, rq.Rotation("hadamard"))


def test_8bit_validation():
    L = rq.lib()
    q8 = rq._QuantDesc(1, 1.0, FAKE, 256, 8)
    bad_bits = rq._QuantDesc(0, 1.0, None, 0, 6)
    assert _rotate_quant(8, 8192, 8192, _rot("none"), bad_bits) == rq.RQ_EINVAL          # bits 6
    assert _rotate_quant(8, 4096, 4096, _rot("hadamard"), rq._QuantDesc(0, 1.0, None, 0, 8)) == rq.RQ_ESHAPE
    assert _rotate_quant(0, 8192, 8192, _rot("none"), q8, zero=FAKE, x_out=FAKE) == rq.RQ_OK
    f = L.rq_w8a8_linear
    assert f(FAKE, FAKE, FAKE, 8, 40000, FAKE, FAKE, FAKE, 16, None, None, 0, FAKE, 16, None) == rq.RQ_ESHAPE
    assert f(FAKE, FAKE, FAKE, 8, 1000, FAKE, FAKE, FAKE, 16, None, None, 0, FAKE, 16, None) == rq.RQ_ESHAPE
    assert f(FAKE, FAKE, FAKE, 8, 1024, FAKE, FAKE, None, 16, None, None, 0, FAKE, 16, None) == rq.RQ_EINVAL
    assert f(FAKE, FAKE, None, 8, 1024, FAKE, FAKE, None, 16, None, None, 32, FAKE, 16, None) == rq.RQ_EINVAL
    assert f(FAKE, FAKE, None, 0, 1024, FAKE, FAKE, None, 16, None, None, 0, FAKE, 16, None) == rq.RQ_OK
    g = L.rq_w8a8_gemm_i32
    assert g(FAKE, 1, 8, 1024, FAKE, None, 16, FAKE, 16, None) == rq.RQ_EINVAL            # unsigned without rowsum
    assert g(FAKE, 0, 8, 40960, FAKE, None, 16, FAKE, 16, None) == rq.RQ_ESHAPE
    d = L.rq_quant_decode_linear
    assert d(FAKE, 8, 4096, 4096, ctypes.byref(rq._QuantDesc(0, 1.0, None, 0, 8)), FAKE, FAKE, FAKE, 16, None,
             FAKE, 16, None) == rq.RQ_ESHAPE


def test_clip_search_and_row_clip_validation():
    L = rq.lib()
    f = L.rq_search_weight_clip
    qd = lambda **kw: ctypes.byref(rq._QuantDesc(kw.get("asym", 0), 1.0, kw.get("idx"), kw.get("n_out", 0),
                                                 kw.get("bits", 4), kw.get("rc")))
    assert f(FAKE, 0, 4096, 4096, qd(), 100, FAKE, None) == rq.RQ_OK            # N == 0
    assert f(FAKE, 8, 4096, 4096, qd(asym=1), 100, FAKE, None) == rq.RQ_EINVAL  # asymmetric weights
    assert f(FAKE, 8, 4096, 4096, qd(), 0, FAKE, None) == rq.RQ_EINVAL          # steps
    assert f(FAKE, 8, 4096, 4096, qd(bits=6), 100, FAKE, None) == rq.RQ_EINVAL
    assert f(FAKE, 8, 4100, 4104, qd(), 100, FAKE, None) == rq.RQ_ESHAPE        # K % 32
    assert f(FAKE, 8, 4096, 4096, qd(n_out=32), 100, FAKE, None) == rq.RQ_EINVAL  # outliers without a list
    assert f(FAKE, 8, 4096, 4096, qd(), 100, None, None) == rq.RQ_EALIGN
    # per-row clip ratios: symmetric codes without a rotation only
    rc = rq._QuantDesc(0, 1.0, None, 0, 4, FAKE)
    assert _rotate_quant(4, 4096, 4096, _rot("hadamard"), rc) == rq.RQ_ESHAPE
    assert _rotate_quant(4, 4096, 4096, _rot("none"), rq._QuantDesc(1, 1.0, None, 0, 4, FAKE)) == rq.RQ_ESHAPE
    assert _rotate_quant(4, 4096, 4096, _rot("none"), rq._QuantDesc(0, 1.0, None, 0, 4, FAKE + 2)) == rq.RQ_EALIGN
    d = L.rq_quant_decode_linear
    assert d(FAKE, 8, 4096, 4096, ctypes.byref(rc), FAKE, FAKE, FAKE, 16, None, FAKE, 16, None) == rq.RQ_ESHAPE


def test_prepare_weights_noalloc_validates_first():
    L = rq.lib()
    qd = _qd()
    # no descriptor
    assert L.rq_prepare_weights_noalloc(FAKE, 4, 4096, 4096, None, ctypes.byref(qd), FAKE, FAKE, FAKE, None,
                                        None) == rq.RQ_EINVAL
    # a shape check of the common path (KRON factors wider than 64) fails before the scratch lookup
    rot = _rot("kron", n1=128, n2=32, p1=FAKE, p2=FAKE)
    assert L.rq_prepare_weights_noalloc(FAKE, 4, 4096, 4096, ctypes.byref(rot), ctypes.byref(qd), FAKE, FAKE,
                                        FAKE, None, None) == rq.RQ_ESHAPE
    # asymmetric weights are rejected as by rq_prepare_weights
    rot = _rot("none")
    qa = _qd(asym=1)
    assert L.rq_prepare_weights_noalloc(FAKE, 4, 4096, 4096, ctypes.byref(rot), ctypes.byref(qa), FAKE, FAKE,
                                        FAKE, None, None) == rq.RQ_EINVAL


def test_rotate_quant_decode_linear_validates_first():
    L = rq.lib()
    qd = _qd()

    def call(rot, qd, T=4, K=4096):
        return L.rq_rotate_quant_decode_linear(FAKE, T, K, K, ctypes.byref(rot) if rot is not None else None,
                                               ctypes.byref(qd), FAKE, FAKE, None, 64, None, FAKE, 64, None)
    assert call(None, qd) == rq.RQ_EINVAL
    assert call(_rot("kron", n1=64, n2=64, p1=FAKE, p2=FAKE), qd) == rq.RQ_ESHAPE
    assert call(_rot("hadamard"), qd, K=2048) == rq.RQ_ESHAPE       # the rotated form is K = 4096 only
    assert call(_rot("gsr", block=4), qd) == rq.RQ_ESHAPE            # GSR blocks of 8 to 64
    assert call(_rot("hadamard"), _qd(asym=1)) == rq.RQ_ESHAPE       # symmetric codes only
    assert call(_rot("hadamard"), qd, T=17) == rq.RQ_ESHAPE          # at most 16 rows
    assert call(_rot("hadamard"), _qd(clip=0.0)) == rq.RQ_EINVAL
    assert call(_rot("hadamard"), qd, T=0) == rq.RQ_OK               # empty batch: nothing launched
