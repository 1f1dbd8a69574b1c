"""The allocation-free backward entry point, mxnorm_bwd_noalloc, against
mxnorm_bwd (the same computation with a caller-owned workspace).

Both run the same kernels in the same summation order, so every output (dx,
the row dot and dgamma) must be bit-identical. Two calls in a row, the second
on a smaller input, show that the second call does not depend on what the
first left in the library's scratch array.
"""

import ctypes

import pytest
import torch

import norm_mx_quantisation_amd as mxq
from norm_mx_quantisation_amd import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mxq.lib()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc_backward(x, g, dy, inv, want_dgamma=True):
    """Outputs of mxnorm_bwd_noalloc, called through the C ABI."""
    T, D = x.shape
    dx = torch.full((T, D), 7.0, dtype=torch.bfloat16, device=DEV)
    row_dot = torch.full((T,), 7.0, dtype=torch.float32, device=DEV)
    dgamma = torch.full((D,), 7.0, dtype=torch.float32, device=DEV) if want_dgamma else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = mxq.mxnorm_bwd_noalloc(_ptr(x), x.stride(0), _ptr(g), _ptr(dy), dy.stride(0), _ptr(inv),
                                T, D, _ptr(dx), _ptr(row_dot), _ptr(dgamma), stream)
    assert st == mxq.MXQ_OK, mxq.mxq_strerror(st)
    return dx, row_dot, dgamma


def case(T, D, seed, gamma=True):
    x = workloads.random_rows(T, D, seed=seed, device=DEV)
    x[T // 2, : min(D, 64)] *= 30.0
    dy = workloads.random_rows(T, D, seed=seed + 1, device=DEV)
    g = workloads.random_gamma(D, seed=seed + 2, device=DEV) if gamma else None
    _, _, inv = mxq.mxnorm(x, g, 2.0)
    return x, g, dy, inv


def check_same(x, g, dy, inv, want_dgamma=True):
    ref = mxq.mxnorm_backward(x, g, dy, inv, want_dgamma=want_dgamma)   # with a workspace
    got = noalloc_backward(x, g, dy, inv, want_dgamma)
    torch.cuda.synchronize()
    assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), "dx"
    assert torch.equal(got[1].view(torch.int32), ref[1].view(torch.int32)), "row_dot"
    if want_dgamma:
        assert torch.equal(got[2].view(torch.int32), ref[2].view(torch.int32)), "dgamma"
    else:
        assert got[2] is None and ref[2] is None


def test_noalloc_backward_matches_the_workspace_entry_point_twice_then_smaller():
    # the first call fills 512 partial rows of 4096 floats; the second, smaller,
    # fills 175 partial rows of 1024 floats of the same array
    check_same(*case(2048, 4096, seed=601))
    check_same(*case(700, 1024, seed=611))


def test_noalloc_backward_widest_rows_and_without_gain_or_dgamma():
    # the largest partial block the array must hold (512 rows of 8192 floats:
    # all 16 MiB), then calls without a gain and without dgamma
    check_same(*case(2048, 8192, seed=621))
    check_same(*case(64, 512, seed=631, gamma=False))
    check_same(*case(33, 2048, seed=641), want_dgamma=False)


def test_noalloc_backward_empty_batch_zeroes_dgamma():
    e = torch.empty(0, 4096, dtype=torch.bfloat16, device=DEV)
    inv = torch.empty(0, dtype=torch.float32, device=DEV)
    _, _, dg = noalloc_backward(e, None, e, inv)
    torch.cuda.synchronize()
    assert (dg == 0).all()


def test_noalloc_backward_in_a_graph_matches_the_workspace_entry_point():
    # the callers this entry point serves capture it: replayed several times,
    # with eager work and synchronisations between replays, the captured call
    # reproduces mxnorm_bwd's outputs bit for bit
    x, g, dy, inv = case(1500, 4096, seed=651)
    ref = mxq.mxnorm_backward(x, g, dy, inv)
    torch.cuda.synchronize()
    T, D = x.shape
    dx = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    row_dot = torch.empty((T,), dtype=torch.float32, device=DEV)
    dgamma = torch.empty((D,), dtype=torch.float32, device=DEV)

    def work():
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = mxq.mxnorm_bwd_noalloc(_ptr(x), x.stride(0), _ptr(g), _ptr(dy), dy.stride(0),
                                    _ptr(inv), T, D, _ptr(dx), _ptr(row_dot), _ptr(dgamma), stream)
        assert st == mxq.MXQ_OK, mxq.mxq_strerror(st)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(4):
        for t in (dx, row_dot, dgamma):
            t.view(torch.uint8).fill_(0x5A + rep)
        check_same(*case(64, 2048, seed=661 + rep))   # other calls use the array in between
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), ref[0].view(torch.int16)), rep
        assert torch.equal(row_dot.view(torch.int32), ref[1].view(torch.int32)), rep
        assert torch.equal(dgamma.view(torch.int32), ref[2].view(torch.int32)), rep
