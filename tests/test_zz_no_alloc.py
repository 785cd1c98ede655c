"""rq_prepare_weights_noalloc (the weight side for callers that cannot
allocate) against rq_prepare_weights with a caller workspace, through the C
ABI: two calls in a row on the same GPU, the second with a smaller input
(smaller KRON factors and fewer rows), each equal bit for bit; then a
transform that needs no scratch."""
import ctypes

import numpy as np
import pytest

import workloads
from parity_utils import dev, host, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
rq = pytest.importorskip("online_rotation_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rq.lib()


def _noalloc(w, rot):
    N, K = w.shape
    qw = torch.full((N, K // 2), 0xAB, dtype=torch.uint8, device=w.device)
    sw = torch.full((N,), -1.0, dtype=torch.float32, device=w.device)
    rs = torch.full((N,), -1, dtype=torch.int32, device=w.device)
    rd, qd = rot.desc(), rq._QuantDesc(0, 1.0, None, 0, 4, None)
    st = rq.lib().rq_prepare_weights_noalloc(w.data_ptr(), N, K, w.stride(0), ctypes.byref(rd), ctypes.byref(qd),
                                             qw.data_ptr(), sw.data_ptr(), rs.data_ptr(), None,
                                             torch.cuda.current_stream().cuda_stream)
    assert st == rq.RQ_OK, rq.rq_last_error()
    return {"q": qw, "scale": sw, "rowsum": rs}


@pytest.mark.parametrize("order", ["large-then-small"])
def test_noalloc_weight_prep_equals_workspace_form(order):
    for N, n in ((300, 64), (70, 16)):
        note(f"[prepare_weights_noalloc] kron N={N} factors {n}x{n}")
        inp = workloads.make_inputs("flat", T=2, K=n * n, N=N, n1=n, n2=n)
        w = dev(inp["w"])
        rot = rq.Rotation("kron", p1=dev(inp["p1"]), p2=dev(inp["p2"]), chan_scale=dev(inp["s"]))
        got = _noalloc(w, rot)
        want = rq.rq_prepare_weights(w, rot)
        torch.cuda.synchronize()
        for k in ("q", "scale", "rowsum"):
            assert np.array_equal(host(got[k]), host(want[k])), k
    note("[prepare_weights_noalloc] hadamard N=64 K=1024 (no scratch)")
    w = dev(workloads.make_inputs("llama7b", T=2, K=1024, N=64)["w"])
    got = _noalloc(w, rq.Rotation("hadamard"))
    want = rq.rq_prepare_weights(w, rq.Rotation("hadamard"))
    torch.cuda.synchronize()
    for k in ("q", "scale", "rowsum"):
        assert np.array_equal(host(got[k]), host(want[k])), k


def test_noalloc_binding_matches_and_allocates_nothing_on_the_device():
    """The Python form of the same call writes caller-given tensors, and the
    call itself leaves torch's device allocator untouched."""
    note("[prepare_weights_noalloc] binding, kron 32x32")
    inp = workloads.make_inputs("flat", T=2, K=1024, N=96, n1=32, n2=32)
    w = dev(inp["w"])
    rot = rq.Rotation("kron", p1=dev(inp["p1"]), p2=dev(inp["p2"]), chan_scale=dev(inp["s"]))
    qw = torch.empty((96, 512), dtype=torch.uint8, device=w.device)
    sw = torch.empty((96,), dtype=torch.float32, device=w.device)
    rs = torch.empty((96,), dtype=torch.int32, device=w.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats(w.device).get("allocation.all.allocated", 0)
    rq.rq_prepare_weights_noalloc(w, rot, qw, sw, rs)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats(w.device).get("allocation.all.allocated", 0) == before
    want = rq.rq_prepare_weights(w, rot)
    torch.cuda.synchronize()
    assert torch.equal(qw, want["q"]) and torch.equal(sw, want["scale"]) and torch.equal(rs, want["rowsum"])
