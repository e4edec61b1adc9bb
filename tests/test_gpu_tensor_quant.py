"""GPU parity of per-tensor FP8 quantisation (e4m3fn and e5m2) and fp32 dequantisation.

Codes, the scale and the dequantised values are integer / byte results once the
precision is fixed, so every comparison with the oracle is bit for bit. Covered:
random tensors of several sizes (one 16-element group, ragged grid-stride tails, a
weight-sized tensor) in both formats; every finite bf16 value through each format's
conversion (a tensor whose amax equals the format's largest value has scale 1, so
the quotients are the values themselves); zero tensors; tensors whose scale is an
fp32 subnormal (the exact-division path); the dequantisation of every code.
"""

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from oracle import e4m3, e5m2, tensor_quant as otq
from tests._helpers import require_gpu
from workloads import bf16_bits, make_case

pytestmark = pytest.mark.gpu
FMTS = ["e4m3fn", "e5m2"]
FMAX_BITS = {"e4m3fn": 0x43E0, "e5m2": 0x4760}  # bf16 of 448 and of 57344


def _gpu(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)


def _check(bits, fmt, dev):
    q, s = fp8.quant_tensor(_gpu(bits, dev), fmt)
    eq, es = otq.quant_tensor(bits, fmt)
    assert np.array_equal(q.cpu().numpy().reshape(eq.shape), eq), fmt
    assert s.cpu().numpy().view(np.uint32)[0] == np.float32(es).view(np.uint32), fmt
    d = fp8.dequant_tensor(q, s, fmt)
    ed = otq.dequant_tensor(eq, fmt, es)
    assert np.array_equal(d.cpu().numpy().reshape(ed.shape).view(np.uint32), ed.view(np.uint32)), fmt


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(16,), (1008,), (37, 272), (8192, 2048)])
def test_random_tensors(fmt, shape):
    dev = require_gpu()
    rng = np.random.default_rng(sum(shape))
    x = (rng.standard_normal(shape) * np.exp2(rng.integers(-8, 8))).astype(np.float32)
    _check(bf16_bits(torch.from_numpy(x).to(torch.bfloat16)), fmt, dev)


@pytest.mark.parametrize("fmt", FMTS)
def test_every_bf16_value_through_the_conversion(fmt):
    dev = require_gpu()
    mod = e4m3 if fmt == "e4m3fn" else e5m2
    pat = np.arange(1 << 16, dtype=np.uint32)
    mag = pat & 0x7FFF
    keep = mag <= FMAX_BITS[fmt]  # finite and not above fmax, both signs
    bits = pat[keep].astype(np.uint16)
    bits = np.concatenate([bits, np.full((-len(bits)) % 16, FMAX_BITS[fmt], np.uint16)])
    q, s = fp8.quant_tensor(_gpu(bits, dev), fmt)
    assert float(s.item()) == 1.0
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(q.cpu().numpy(), mod.encode(vals))
    _check(bits, fmt, dev)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_and_subnormal_scale_tensors(fmt):
    dev = require_gpu()
    _check(np.zeros(64, np.uint16), fmt, dev)
    z = np.zeros(32, np.uint16)
    z[::3] = 0x8000
    _check(z, fmt, dev)
    rng = np.random.default_rng(7)
    tiny = rng.integers(1, 0x0400, 256).astype(np.uint16) | (rng.integers(0, 2, 256).astype(np.uint16) << 15)
    _check(tiny, fmt, dev)  # amax < 2^-120: the scale is an fp32 subnormal


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_every_code(fmt):
    dev = require_gpu()
    mod = e4m3 if fmt == "e4m3fn" else e5m2
    nfin = 0x7F if fmt == "e4m3fn" else 0x7C
    codes = np.concatenate([np.arange(nfin), np.arange(nfin) | 0x80]).astype(np.uint8)
    codes = np.concatenate([codes, np.zeros((-len(codes)) % 16, np.uint8)])
    scale = np.float32(0.0123)
    out = fp8.dequant_tensor(torch.from_numpy(codes).to(dev), torch.tensor([scale], device=dev), fmt)
    exp = (mod.decode(codes) * float(scale)).astype(np.float32)
    assert np.array_equal(out.cpu().numpy(), exp)


def test_weight_quantised_per_tensor_feeds_nothing_else():
    # the per-tensor and per-channel quantisers agree when the weight has one row
    dev = require_gpu()
    case = make_case(4, 1, 2048, seed=3, kind="normal")
    q1, s1 = fp8.quant_tensor(case.w.to(dev), "e4m3fn")
    q2, s2 = fp8.quant_weights_per_channel(case.w.to(dev))
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
