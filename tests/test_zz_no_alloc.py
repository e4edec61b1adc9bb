"""fp8_linear_run_noalloc: the forward for callers that cannot allocate device memory.

Called through the C ABI. Its output must equal fp8_linear_run's (the same kernels on
the same codes, so bit for bit), and the first output is also held to the oracle's
linear tolerance. Two calls in a row on the shared scratch, the second with fewer
tokens; an input above the scratch size is refused before anything runs; the e4m3fn
kind needs no scratch; the call recorded into a HIP graph and replayed on new inputs.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from fp8_w8a8_quantized_token_amd import _lib
from oracle import linear as ol, quant as oq
from tests._helpers import assert_linear_close, require_gpu
from workloads import bf16_bits, make_case

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(lin, a, kind=_lib.A_BF16, a_scale=None):
    m = a.shape[0]
    out = torch.empty((m, lin.n), dtype=torch.bfloat16, device=a.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(a.device).cuda_stream)
    st = _lib.lib().fp8_linear_run_noalloc(lin._plan, m, _p(a), kind, _p(a_scale), _p(out), stream)
    return st, out


def test_noalloc_matches_run_with_workspace():
    dev = require_gpu()
    big = make_case(1100, 528, 2064, seed=71, kind="outlier")
    lin = fp8.Fp8Linear(big.w.to(dev), big.bias.to(dev))
    small_a = make_case(70, 528, 2064, seed=72, kind="outlier").a
    ref_out = []
    for a in (big.a, small_a):  # two calls in a row on the shared scratch, the second smaller
        ad = a.to(dev)
        st, out = _noalloc(lin, ad)
        assert st == _lib.OK, _lib.status_string(st)
        expect = lin(ad)  # fp8_linear_run with its own workspace
        torch.cuda.synchronize()
        assert torch.equal(out, expect)
        ref_out.append(out)
    qw, sw = oq.quant_weights_per_channel(bf16_bits(big.w))
    for a, out in zip((big.a, small_a), ref_out):
        ref, _, _ = ol.linear_ref(bf16_bits(a), qw, sw, bf16_bits(big.bias))
        assert_linear_close(out, ref, f"noalloc {a.shape[0]} rows")


def test_noalloc_e4m3_input_and_limits():
    dev = require_gpu()
    case = make_case(96, 144, 256, seed=73, kind="outlier")
    lin = fp8.Fp8Linear(case.w.to(dev), case.bias.to(dev))
    a = case.a.to(dev)
    qa, sa = fp8.quant_rows(a)
    st, out = _noalloc(lin, qa, _lib.A_E4M3, sa)
    assert st == _lib.OK
    torch.cuda.synchronize()
    assert torch.equal(out, lin(a))
    # m = 0 is a no-op; a bf16 input whose codes and scales exceed the scratch is refused
    # on the host before any launch (the pointers are never dereferenced)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    assert _lib.lib().fp8_linear_run_noalloc(lin._plan, 0, _p(a), _lib.A_BF16, None, _p(out), stream) == _lib.OK
    too_many = _lib.NOALLOC_SCRATCH_BYTES // 256 + 1
    assert lin.workspace_bytes(too_many) > _lib.NOALLOC_SCRATCH_BYTES
    st = _lib.lib().fp8_linear_run_noalloc(lin._plan, too_many, _p(a), _lib.A_BF16, None, _p(out), stream)
    assert st == _lib.ERR_TOO_LARGE


def test_noalloc_near_the_scratch_size():
    # the 32760-token QKV input [32760, 2048]: 64 MiB of codes plus the scales, most of
    # the scratch; then a small call again
    dev = require_gpu()
    case = make_case(32760, 2048, 2048, seed=74, kind="outlier")
    lin = fp8.Fp8Linear(case.w.to(dev), case.bias.to(dev))
    assert lin.workspace_bytes(32760) <= _lib.NOALLOC_SCRATCH_BYTES
    for a in (case.a, case.a[:300].contiguous()):
        ad = a.to(dev)
        st, out = _noalloc(lin, ad)
        assert st == _lib.OK
        expect = lin(ad)
        torch.cuda.synchronize()
        assert torch.equal(out, expect)


def test_noalloc_replayed_from_a_graph():
    # the use the entry point exists for: recorded once into a HIP graph (no allocation
    # inside the capture), replayed with new inputs copied in between replays; every replay
    # must equal the eager forward on that input, bit for bit
    dev = require_gpu()
    case = make_case(300, 528, 1040, seed=75, kind="outlier")
    lin = fp8.Fp8Linear(case.w.to(dev), case.bias.to(dev))
    a_static = torch.empty((300, 1040), dtype=torch.bfloat16, device=dev)
    out_static = torch.empty((300, 528), dtype=torch.bfloat16, device=dev)
    inputs = [make_case(300, 528, 1040, seed=76 + i, kind="outlier").a.to(dev) for i in range(3)]
    a_static.copy_(inputs[0])
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # first call outside capture: the scratch address is looked up here
        st = _lib.lib().fp8_linear_run_noalloc(lin._plan, 300, _p(a_static), _lib.A_BF16, None, _p(out_static),
                                               ctypes.c_void_p(side.cuda_stream))
        assert st == _lib.OK
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        cap = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        st = _lib.lib().fp8_linear_run_noalloc(lin._plan, 300, _p(a_static), _lib.A_BF16, None, _p(out_static), cap)
    assert st == _lib.OK
    for x in inputs:
        a_static.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        expect = lin(x)  # eager, with its own workspace
        torch.cuda.synchronize()
        assert torch.equal(out_static, expect)
