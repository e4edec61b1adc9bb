"""GPU parity of the FP8 weight-only linear (W8A16) against the float64 oracle.

The weight is quantised per output channel by the library (and checked bit for bit
against the oracle's quantiser); the activation stays bf16. Outputs are compared
with the unrounded float64 reference: |gpu - ref| <= 1e-2 (|ref| + 1) elementwise and
relative Frobenius error <= 2e-3. Covered: the tiny shape in full; every compiled
configuration on ragged m / n / k tails; every finite e4m3fn code through the
in-register fp8 -> bf16 conversion (bit exact); A = 0 (output == bias exactly); no
bias; the selector; full-size FFN shapes on sampled rows.
"""

import dataclasses

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from oracle import e4m3, e5m2, quant as oq, tensor_quant as otq, w8a16 as ow
from tests._helpers import assert_linear_close, assert_linear_close_rows, require_gpu
from workloads import bf16_bits, make_case, make_config

pytestmark = pytest.mark.gpu

try:
    N_CONFIGS = fp8.w8a16_config_count()
except Exception:  # library not built: the tests below report it
    N_CONFIGS = 1

TAIL_SHAPES = [(1, 16, 16), (26, 144, 48), (63, 16, 272), (65, 144, 16), (257, 144, 272), (300, 272, 400),
               (513, 528, 1040)]


def _ref(case, qw=None, sw=None):
    if qw is None:
        qw, sw = oq.quant_weights_per_channel(bf16_bits(case.w))
    b = None if case.bias is None else bf16_bits(case.bias)
    return ow.w8a16_ref(bf16_bits(case.a), qw, sw, b), qw, sw


def test_tiny_full_and_weight_codes():
    dev = require_gpu()
    cfg = make_config("tiny")
    a, w, b = cfg["activations"]["a"], cfg["weights"]["linear"], cfg["biases"]["linear"]
    lin = fp8.Fp8WeightOnlyLinear(w.to(dev), b.to(dev))
    out = lin(a.to(dev))
    torch.cuda.synchronize()
    qw, sw = oq.quant_weights_per_channel(bf16_bits(w))
    assert np.array_equal(lin.w_fp8.cpu().numpy(), qw) and np.array_equal(lin.w_scale.cpu().numpy(), sw)
    assert_linear_close(out, ow.w8a16_ref(bf16_bits(a), qw, sw, bf16_bits(b)), "w8a16 tiny")


@pytest.mark.parametrize("config", range(N_CONFIGS))
@pytest.mark.parametrize("m,n,k", TAIL_SHAPES)
def test_every_config_on_ragged_tails(config, m, n, k):
    dev = require_gpu()
    case = make_case(m, n, k, seed=m + 3 * n + 7 * k, kind="normal")
    ref, qw, sw = _ref(case)
    out = fp8.w8a16_run_config(config, case.a.to(dev), torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev),
                               case.bias.to(dev))
    assert_linear_close(out, ref, f"w8a16 config {config} {m}x{n}x{k}")


@pytest.mark.parametrize("config", range(N_CONFIGS))
def test_every_e4m3_code_through_the_conversion(config):
    _every_code(config, "e4m3fn", np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8))


@pytest.mark.parametrize("config", range(N_CONFIGS))
def test_every_e5m2_code_through_the_conversion(config):
    _every_code(config, "e5m2", np.array([c for c in range(256) if (c & 0x7F) < 0x7C], np.uint8))


def _every_code(config, fmt, codes):
    # one-hot activation rows pick single weight codes: out[t, n] = dec(qw[n, t]) exactly
    dev = require_gpu()
    dec = e4m3.decode if fmt == "e4m3fn" else e5m2.decode
    k = 256
    n = 64
    rng = np.random.default_rng(config + 17 * len(codes))
    qw = np.zeros((n, k), np.uint8)
    for r in range(n):
        qw[r, :len(codes)] = rng.permutation(codes)
    a = torch.eye(k, dtype=torch.bfloat16)[:len(codes)]
    sw = np.ones(n, np.float32)
    out = fp8.w8a16_run_config(config, a.to(dev), torch.from_numpy(qw).to(dev), torch.from_numpy(sw).to(dev),
                               fmt=fmt)
    got = out.float().cpu().numpy()
    exp = dec(qw[:, :len(codes)]).T  # every finite code's value is exact in bf16
    assert np.array_equal(got, exp.astype(np.float32))


def test_zero_activation_gives_bias_and_no_bias():
    dev = require_gpu()
    case = make_case(70, 272, 528, seed=8, kind="normal")
    lin = fp8.Fp8WeightOnlyLinear(case.w.to(dev), case.bias.to(dev))
    zero = torch.zeros((70, 528), dtype=torch.bfloat16, device=dev)
    out = lin(zero)
    assert torch.equal(out, case.bias.to(dev).expand(70, -1))
    nob = fp8.Fp8WeightOnlyLinear(case.w.to(dev))
    ref, _, _ = _ref(dataclasses.replace(case, bias=None))
    assert_linear_close(nob(case.a.to(dev)), ref, "w8a16 no bias")


def test_selector_and_3d_input():
    dev = require_gpu()
    case = make_case(96, 400, 272, seed=9, kind="normal")
    lin = fp8.Fp8WeightOnlyLinear(case.w.to(dev), case.bias.to(dev))
    for m in (1, 26, 64, 300, 4096, 32760):
        cid, tm, tn, wg = lin.config(m)
        assert 0 <= cid < N_CONFIGS and wg == -(-m // tm) * -(-400 // tn)
    out = lin(case.a.to(dev).reshape(4, 24, 272))
    assert out.shape == (4, 24, 400)
    ref, _, _ = _ref(case)
    assert_linear_close(out.reshape(96, 400), ref, "w8a16 3-d input")
    empty = lin(torch.zeros((2, 0, 272), dtype=torch.bfloat16, device=dev))  # no tokens: an empty output
    assert empty.shape == (2, 0, 400)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
def test_per_tensor_weights_from_the_state_dict_converter(fmt):
    # the converter's output (codes + one scale) runs through the weight-only linear
    dev = require_gpu()
    case = make_case(130, 272, 528, seed=12, kind="normal")
    q, s = fp8.quant_tensor(case.w.to(dev), fmt)
    lin = fp8.Fp8WeightOnlyLinear(w_fp8=q, w_scale=s, bias=case.bias.to(dev), fmt=fmt)
    out = lin(case.a.to(dev))
    eq, es = otq.quant_tensor(bf16_bits(case.w), fmt)
    assert np.array_equal(q.cpu().numpy(), eq)
    ref = ow.w8a16_ref(bf16_bits(case.a), eq, np.full(272, es, np.float32), bf16_bits(case.bias), fmt=fmt)
    assert_linear_close(out, ref, f"w8a16 per-tensor {fmt}")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["ffn_up", "ffn_down"])
def test_ffn_full_size(name):
    dev = require_gpu()
    cfg = make_config(name)
    a = cfg["activations"]["a"]
    w, b = cfg["weights"][name], cfg["biases"][name]
    lin = fp8.Fp8WeightOnlyLinear(w.to(dev), b.to(dev))
    out = lin(a.to(dev))
    torch.cuda.synchronize()
    qw, sw = oq.quant_weights_per_channel(bf16_bits(w))
    assert np.array_equal(lin.w_fp8.cpu().numpy(), qw)
    a_bits, b_bits = bf16_bits(a), bf16_bits(b)
    assert_linear_close_rows(out, lambda r0, r1: ow.w8a16_ref(a_bits[r0:r1], qw, sw, b_bits), f"w8a16 {name}")


@pytest.mark.slow
def test_ffn_up_full_size_per_tensor_e5m2():
    # the state-dict converter's e5m2 weight (one scale for the tensor) at the FFN-up shape:
    # the codes and the scale bit for bit, every output element against the oracle
    dev = require_gpu()
    cfg = make_config("ffn_up")
    a, w, b = cfg["activations"]["a"], cfg["weights"]["ffn_up"], cfg["biases"]["ffn_up"]
    q, s = fp8.quant_tensor(w.to(dev), "e5m2")
    lin = fp8.Fp8WeightOnlyLinear(w_fp8=q, w_scale=s, bias=b.to(dev), fmt="e5m2")
    out = lin(a.to(dev))
    torch.cuda.synchronize()
    eq, es = otq.quant_tensor(bf16_bits(w), "e5m2")
    assert np.array_equal(q.cpu().numpy(), eq)
    assert s.cpu().numpy().view(np.uint32)[0] == np.float32(es).view(np.uint32)
    sw = np.full(w.shape[0], es, np.float32)
    a_bits, b_bits = bf16_bits(a), bf16_bits(b)
    assert_linear_close_rows(out, lambda r0, r1: ow.w8a16_ref(a_bits[r0:r1], eq, sw, b_bits, fmt="e5m2"),
                             "w8a16 ffn_up per-tensor e5m2")


@pytest.mark.gpu
def test_w8a16_selector_picks_the_measured_best():
    # timed on MI355X (every configuration interleaved in one process): 256 x 256 at FFN-up,
    # 128 x 256 at FFN-down, 128 x 128 at 512 x 8192 x 2048 and 2048 x 2048 x 8192, 64 x 64 for
    # 26 and 256 rows
    dev = require_gpu()
    if torch.cuda.get_device_properties(dev).multi_processor_count != 256:
        pytest.skip("the picks are measured for a 256-CU device")
    up = fp8.Fp8WeightOnlyLinear(torch.zeros((8192, 2048), dtype=torch.bfloat16, device=dev))
    down = fp8.Fp8WeightOnlyLinear(torch.zeros((2048, 8192), dtype=torch.bfloat16, device=dev))
    assert up.config(4096)[0] == 0 and down.config(4096)[0] == 2
    assert up.config(512)[0] == 3 and down.config(2048)[0] == 3
    assert up.config(256)[0] == 4 and down.config(26)[0] == 4
