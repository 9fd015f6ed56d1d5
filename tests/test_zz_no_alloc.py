"""rq_rotq_linear_noalloc (the entry point that allocates nothing; its workspace is the library's
static device scratch) against rq_rotq_linear with a caller workspace: bit-identical outputs on
two calls in a row, the second with a smaller input, and the size limit."""
import numpy as np
import pytest
import torch

import w4a4_integer_quantized_amd as rq
from w4a4_integer_quantized_amd import synth
from tests.gpu_util import dev_from_bits, need_gpu

pytestmark = pytest.mark.gpu


def _noalloc(X, Wq, ws, b, cfg, N):
    M, K = X.shape
    Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    xdt = rq.RQ_F16 if X.dtype == torch.float16 else rq.RQ_BF16
    st = rq.rq_rotq_linear_noalloc(X.data_ptr(), xdt, M, K, Wq.data_ptr(), ws.data_ptr(), N,
                                   b.data_ptr() if b is not None else None, cfg, Y.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    return st, Y


@pytest.mark.parametrize("first,second", [(("vit_attn", 41472), ("single", 256)),
                                          (("dit", 8192), ("vit_mlp", 700))])
def test_noalloc_matches_workspace_entry_point(first, second):
    need_gpu()
    for key, M in (first, second):
        g = synth.generate(key, M=M, with_second_layer=False)
        cfg_ = g["cfg"]
        lin = cfg_.linears[0]
        print("no-alloc case %s M=%d N=%d K=%d" % (key, M, lin.N, lin.K), flush=True)
        X = dev_from_bits(g["x_bits"], cfg_.io)
        Wq, ws = rq.quantize_weights(dev_from_bits(g["W"][lin.name], "f32"), bits=cfg_.bits)
        b = torch.from_numpy(g["bias"][lin.name]).cuda()
        need = rq.workspace_size(M, lin.K, cfg_.bits)
        assert need <= rq.RQ_NOALLOC_SCRATCH_BYTES
        ref = rq.rotq_linear(X, Wq, ws, b, bits=cfg_.bits,
                             workspace=torch.empty((need,), dtype=torch.uint8, device="cuda"))
        st, got = _noalloc(X, Wq, ws, b, rq.make_cfg(cfg_.bits), lin.N)
        assert st == rq.RQ_OK, rq.load().rq_last_error_detail().decode()
        st2, got_nb = _noalloc(X, Wq, ws, None, rq.make_cfg(cfg_.bits), lin.N)
        ref_nb = rq.rotq_linear(X, Wq, ws, None, bits=cfg_.bits)
        torch.cuda.synchronize()
        assert st2 == rq.RQ_OK
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), key
        assert torch.equal(got_nb.view(torch.int16), ref_nb.view(torch.int16)), key


def test_noalloc_rejects_calls_beyond_the_scratch():
    need_gpu()
    K, N = 1024, 64
    M = rq.RQ_NOALLOC_SCRATCH_BYTES // K + 256          # codes alone exceed the scratch
    assert rq.workspace_size(M, K, 8) > rq.RQ_NOALLOC_SCRATCH_BYTES
    small = torch.zeros((16, K), dtype=torch.float16, device="cuda")   # never read: no launch
    Wq = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    ws = torch.zeros(N, device="cuda")
    Y = torch.empty((16, N), dtype=torch.float16, device="cuda")
    st = rq.rq_rotq_linear_noalloc(small.data_ptr(), rq.RQ_F16, M, K, Wq.data_ptr(), ws.data_ptr(), N,
                                   None, rq.make_cfg(8), Y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == rq.RQ_EWORKSPACE
    assert "static scratch" in rq.load().rq_last_error_detail().decode()
    # M == 0 is a no-op, as for rq_rotq_linear.
    st = rq.rq_rotq_linear_noalloc(small.data_ptr(), rq.RQ_F16, 0, K, Wq.data_ptr(), ws.data_ptr(), N,
                                   None, rq.make_cfg(8), Y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == rq.RQ_OK


def test_noalloc_replays_under_graph_capture():
    """Graph capture is one of the uses the entry point is for: a HIP graph holding one
    rq_rotq_linear_noalloc call (the resident-weight GEMM's shape; no allocation and no memset
    inside) is replayed three times, with an eager call on another input, which rewrites the
    shared scratch, and synchronizations between the replays. Every replay gives the eager
    result bit for bit."""
    need_gpu()
    g = synth.generate("vit_attn", M=8192, with_second_layer=False)
    cfg_ = g["cfg"]
    lin = max(cfg_.linears, key=lambda l: l.N)
    X = dev_from_bits(g["x_bits"], cfg_.io)
    Wq, ws = rq.quantize_weights(dev_from_bits(g["W"][lin.name], "f32"), bits=cfg_.bits)
    b = torch.from_numpy(g["bias"][lin.name]).cuda()
    cfg = rq.make_cfg(cfg_.bits)
    st, ref = _noalloc(X, Wq, ws, b, cfg, lin.N)          # eager: also resolves the scratch
    torch.cuda.synchronize()
    assert st == rq.RQ_OK
    other = torch.randn((300, lin.K), device="cuda").half()

    Y = torch.empty_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st = rq.rq_rotq_linear_noalloc(X.data_ptr(), rq.RQ_F16, X.shape[0], lin.K, Wq.data_ptr(),
                                       ws.data_ptr(), lin.N, b.data_ptr(), cfg, Y.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == rq.RQ_OK
    for rep in range(3):
        Y.zero_()
        st_o, _ = _noalloc(other, Wq, ws, b, cfg, lin.N)
        assert st_o == rq.RQ_OK
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), rep
