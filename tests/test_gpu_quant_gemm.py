"""GPU parity of the single-launch quantisation + GEMM.

fp8_quant_gemm quantises the bf16 activation per token into its workspace and runs
the 256 x 256 GEMM on those codes, in one launch. Checked:
- the codes and scales it leaves in the workspace equal the oracle's bit for bit;
- its output equals the oracle's unrounded reference within the linear tolerance,
  and equals bit for bit what the two-launch path (per-token quantiser, then GEMM
  configuration 0) produces: the arithmetic is the same;
- row shares of every size (fewer tokens than workgroups, ragged last shares), every
  register-resident row length and the two-pass long-row quantiser, ragged m / n / k
  tiles, more tiles than compute units (workgroups that start after the shares are
  published), a workspace holding garbage, and back-to-back calls on one workspace
  (the second one smaller).
"""

import dataclasses

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from oracle import linear as ol, quant as oq
from tests._helpers import assert_linear_close_rows, require_gpu
from workloads import bf16_bits, make_case

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _weights(case, dev):
    qw, sw = oq.quant_weights_per_channel(bf16_bits(case.w))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return qw, sw, t(qw), t(sw)


def _check(case, dev, workspace=None, label=""):
    qw, sw, dqw, dsw = _weights(case, dev)
    bias = case.bias.to(dev) if case.bias is not None else None
    a = case.a.to(dev)
    out, codes, scales = fp8.quant_gemm(a, dqw, dsw, bias, workspace=workspace)
    # the two-launch path on the same input
    qa, sa = fp8.quant_rows(a)
    out0 = fp8.gemm_run_config(0, qa, sa, dqw, dsw, bias)
    torch.cuda.synchronize()
    eqa, esa = oq.quant_rows(bf16_bits(case.a))
    assert np.array_equal(codes.cpu().numpy(), eqa), f"{label}: codes differ from the oracle"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), esa.view(np.uint32)), f"{label}: scales"
    assert torch.equal(codes, qa) and torch.equal(scales.view(torch.int32), sa.view(torch.int32))
    assert torch.equal(out, out0), f"{label}: single launch differs from quantiser + configuration 0"
    bias_bits = bf16_bits(case.bias) if case.bias is not None else None
    assert_linear_close_rows(out, lambda r0, r1: ol.linear_ref_fp8(eqa[r0:r1], esa[r0:r1], qw, sw, bias_bits), label)
    return out


SHAPES = [
    (1, 16, 16),        # one token, one tile, one k chunk
    (64, 128, 256),     # the tiny workload's shape
    (26, 2048, 2048),   # the encoder input: fewer tokens than workgroups
    (300, 272, 400),    # ragged m, n and k tiles
    (513, 528, 1040),   # rows of 65 chunks (two register chunks per lane)
    (200, 160, 2064),   # four register chunks
    (130, 144, 4112),   # eight register chunks
    (40, 96, 8208),     # rows too long for registers: the two-pass row quantiser
]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_single_launch_matches_oracle_and_two_launch_path(dev, m, n, k):
    case = make_case(m, n, k, seed=m * 3 + n + k, kind="outlier")
    _check(case, dev, label=f"{m}x{n}x{k}")


def test_no_bias_and_zero_rows(dev):
    case = make_case(257, 272, 512, seed=11, kind="normal", with_bias=False)
    a = case.a.clone()
    a[5] = 0.0  # an all-zero token: scale 0, codes 0
    a[256] = -0.0
    case = dataclasses.replace(case, a=a)
    _check(case, dev, label="no bias, zero rows")


def test_more_tiles_than_compute_units(dev):
    # 17 x 17 = 289 tiles of 256 x 256 (ragged m, n and k): the workgroups beyond the
    # first wave own no share and start once the shares are published
    case = make_case(4100, 4112, 272, seed=21, kind="outlier")
    _check(case, dev, label="more tiles than compute units")


def test_garbage_workspace_and_back_to_back_calls(dev):
    big = make_case(1030, 528, 784, seed=31, kind="outlier")
    small = make_case(300, 528, 784, seed=32, kind="outlier")
    small = dataclasses.replace(small, w=big.w, bias=big.bias)
    ws_bytes = fp8.lib().fp8_quant_gemm_workspace_bytes(1030, 784)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device=dev)
    _check(big, dev, workspace=ws, label="garbage workspace")
    _check(small, dev, workspace=ws, label="second call, fewer tokens")
    _check(big, dev, workspace=ws, label="third call")


@pytest.mark.slow
def test_ffn_up_full_size(dev):
    case = make_case(4096, 8192, 2048, seed=41, kind="outlier")
    _check(case, dev, label="FFN-up")


@pytest.mark.slow
def test_ffn_down_full_size(dev):
    # rows of 8192 in the shares (eight register chunks per lane), 16 tiles of k = 8192
    case = make_case(4096, 2048, 8192, seed=42, kind="gelu")
    _check(case, dev, label="FFN-down")


def test_refused_under_graph_capture(dev):
    # the launch's generation number is chosen on the host per call; a graph would replay
    # it, so a call on a capturing stream is refused and nothing is recorded
    case = make_case(64, 128, 256, seed=51, kind="outlier")
    _, _, dqw, dsw = _weights(case, dev)
    a = case.a.to(dev)
    ws = torch.empty((fp8.lib().fp8_quant_gemm_workspace_bytes(64, 256),), dtype=torch.uint8, device=dev)
    out = torch.empty((64, 128), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    with torch.cuda.graph(g, stream=side):
        with pytest.raises(fp8._lib.Fp8W8A8Error) as err:
            fp8.quant_gemm(a, dqw, dsw, None, out=out, workspace=ws)
    assert err.value.status == fp8._lib.ERR_CAPTURE
    # still usable outside capture afterwards
    _check(case, dev, workspace=ws, label="after a refused capture")
