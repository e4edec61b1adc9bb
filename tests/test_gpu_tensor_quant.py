"""GPU parity of per-tensor FP8 quantisation (e4m3fn and e5m2) and fp32 dequantisation.

Codes, the scale and the dequantised values are integer / byte results once the
precision is fixed, so every comparison with the oracle is bit for bit. Covered:
random tensors of several sizes in both formats, on both kernel forms (one pass: one
16-element group, ragged partial grids, one to four groups per thread, the largest tensor
that fits; two passes: just above it), every form on the same tensors (the one-pass form
also with no workgroup waiting for the others), the maximum held by the first or the last
workgroup only; both forms captured in a HIP graph and replayed with new inputs; every finite bf16 value through each format's
conversion (a tensor whose amax equals the format's largest value has scale 1, so
the quotients are the values themselves); quotients near each format's rounding floor
for every exponent of amax (where the divide-free quotient may be an ulp off); zero
tensors; tensors whose scale is an
fp32 subnormal (the exact-division path), down to the smallest bf16 amax values, whose
e5m2 quotients overflow the format and must saturate; the dequantisation of every code.
"""

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from oracle import e4m3, e5m2, tensor_quant as otq
from oracle.quant import bf16_bits_to_f32
from tests._helpers import require_gpu
from workloads import bf16_bits, make_case

pytestmark = pytest.mark.gpu
FMTS = ["e4m3fn", "e5m2"]
FMAX_BITS = {"e4m3fn": 0x43E0, "e5m2": 0x4760}  # bf16 of 448 and of 57344


def _gpu(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)


def _check(bits, fmt, dev, form="auto"):
    q, s = fp8.quant_tensor(_gpu(bits, dev), fmt, form=form)
    eq, es = otq.quant_tensor(bits, fmt)
    assert np.array_equal(q.cpu().numpy().reshape(eq.shape), eq), fmt
    assert s.cpu().numpy().view(np.uint32)[0] == np.float32(es).view(np.uint32), fmt
    d = fp8.dequant_tensor(q, s, fmt)
    ed = otq.dequant_tensor(eq, fmt, es)
    assert np.array_equal(d.cpu().numpy().reshape(ed.shape).view(np.uint32), ed.view(np.uint32)), fmt


# one pass: one group, ragged partial grids, one group per thread on every CU, two and
# four groups per thread (ragged), the largest one-pass tensor on 256 CUs; two passes: just
# above it
SHAPES = [(16,), (1008,), (37, 272), (2048, 2048), (3000, 2048), (8192, 2048), (8200, 2048)]


def _random_bits(shape, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * np.exp2(rng.integers(-8, 8))).astype(np.float32)
    return bf16_bits(torch.from_numpy(x).to(torch.bfloat16))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES)
def test_random_tensors(fmt, shape):
    dev = require_gpu()
    _check(_random_bits(shape, sum(shape)), fmt, dev)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("form", ["one_pass", "two_pass", "one_pass_no_wait"])
@pytest.mark.parametrize("shape", [(37, 272), (3000, 2048), (8192, 2048)])
def test_every_form_on_the_same_tensors(fmt, form, shape):
    # one_pass_no_wait: every workgroup computes the maximum over the whole input itself,
    # the path a workgroup takes when the others do not arrive in time
    dev = require_gpu()
    _check(_random_bits(shape, 7 + sum(shape)), fmt, dev, form=form)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("where", ["first", "last"])
def test_maximum_in_one_workgroup_only(fmt, where):
    # the scale depends on one element held by the first or the last workgroup
    dev = require_gpu()
    bits = _random_bits((3000, 2048), 11).copy()
    big = np.uint16(0x4580)  # bf16 4096, above every other magnitude here
    if where == "first":
        bits.reshape(-1)[5] = big
    else:
        bits.reshape(-1)[-3] = big | np.uint16(0x8000)
    _check(bits, fmt, dev)


def test_one_pass_refuses_a_tensor_that_does_not_fit():
    dev = require_gpu()
    if torch.cuda.get_device_properties(dev).multi_processor_count != 256:
        pytest.skip("the one-pass capacity is 65536 elements per CU; sized for 256 CUs")
    x = torch.zeros((8200, 2048), dtype=torch.bfloat16, device=dev)
    with pytest.raises(fp8.Fp8W8A8Error, match="shape"):
        fp8.quant_tensor(x, "e4m3fn", form="one_pass")
    q, s = fp8.quant_tensor(x, "e4m3fn", form="two_pass")
    torch.cuda.synchronize()
    assert float(s) == 0.0 and int(q.view(torch.uint8).max()) == 0


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
@pytest.mark.parametrize("amax_bits", range(1, 8))
def test_smallest_subnormal_amax(fmt, amax_bits):
    # amax = amax_bits x 2^-133 (a bf16 subnormal): the scale has only a few significant
    # bits, and for e5m2 with amax_bits <= 3 it rounds down so far that amax / s = 65536
    # lies above the format's largest value and must saturate to 57344 (0x7B).
    dev = require_gpu()
    rng = np.random.default_rng(amax_bits)
    body = rng.integers(0, amax_bits + 1, 96).astype(np.uint16)
    body |= rng.integers(0, 2, 96).astype(np.uint16) << 15
    body[5] = amax_bits
    body[17] = amax_bits | 0x8000
    _check(body, fmt, dev)


@pytest.mark.parametrize("fmt", FMTS)
def test_quotients_near_the_rounding_floor_at_every_scale_exponent(fmt):
    # The kernels form x / s without a divide from amax >= 2^-80 (a reciprocal and one fma
    # correction), which can differ from fl32(x / s) by an ulp where the quotient is tiny.
    # For every bf16 exponent of amax (two mantissas each), every bf16 x whose quotient
    # lies within a few binades of the format's rounding floor (half its smallest
    # subnormal: 2^-10 for e4m3fn, 2^-17 for e5m2), both signs; codes bit for bit.
    dev = require_gpu()
    floor = -10 if fmt == "e4m3fn" else -17
    fmax = 448.0 if fmt == "e4m3fn" else 57344.0
    mant = np.arange(128, dtype=np.uint16)
    for e in range(1, 255):
        for m in (0x00, 0x5B):
            amax_bits = np.uint16((e << 7) | m)
            amax = float(bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0])
            es = int(np.floor(np.log2(np.float32(amax / fmax))))  # exponent of the scale
            fields = [f for f in range(es + floor - 3 + 127, es + floor + 4 + 127) if 0 <= f <= 254]
            if not fields:
                continue
            mags = np.concatenate([(np.uint16(f) << 7) | mant for f in fields])
            bits = np.concatenate([mags, mags | np.uint16(0x8000), [amax_bits, amax_bits | np.uint16(0x8000)]])
            bits = np.concatenate([bits, np.zeros((-len(bits)) % 16, np.uint16)]).astype(np.uint16)
            _check(bits, fmt, dev)


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


@pytest.mark.parametrize("form", ["one_pass", "two_pass"])
def test_graph_replays_with_new_inputs(form):
    # both forms are two kernels with no memset: captured once, each replay (with a new
    # input copied in between and eager work around it) must give that input's codes
    dev = require_gpu()
    shape = (3000, 2048)
    x = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    ws = torch.empty((fp8.lib().fp8_quant_tensor_workspace_bytes(),), dtype=torch.uint8, device=dev)
    x.copy_(_gpu(_random_bits(shape, 100), dev))
    fp8.quant_tensor(x, "e4m3fn", workspace=ws, form=form)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g, stream=side):
        q, s = fp8.quant_tensor(x, "e4m3fn", workspace=ws, form=form)
    torch.cuda.synchronize()
    for rep in range(3):
        bits = _random_bits(shape, 101 + rep)
        if rep == 2:
            bits = bits.copy()
            bits.reshape(-1)[-1] = np.uint16(0x4580)  # a new maximum, in the last workgroup
        x.copy_(_gpu(bits, dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eq, es = otq.quant_tensor(bits, "e4m3fn")
        assert s.cpu().numpy().view(np.uint32)[0] == np.float32(es).view(np.uint32), f"replay {rep}: scale"
        assert np.array_equal(q.cpu().numpy().reshape(eq.shape), eq), f"replay {rep}: codes"
