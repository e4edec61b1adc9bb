"""GPU parity of the activation producers (GELU / SiLU -> bf16, and fused -> per-token FP8).

The oracle (oracle.act) rounds each activation exactly to bf16 and quantises the
result with the pinned per-token quantiser. Everything here is integer or byte work
once the bf16 rounding is fixed, so every comparison is bit for bit: the table on
every finite input pattern, the plain producer's bf16 output, and the fused
producer's codes and scales. The fused producer must also equal the unfused path
(act, then the plain quantiser) on the GPU, and feed the FP8 linear like any other
(codes, scale) pair.
"""

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from oracle import act as oact, cref, linear as ol, quant as oq
from tests._helpers import assert_codes_equal, assert_linear_close, require_gpu
from workloads import bf16_bits, make_case

pytestmark = pytest.mark.gpu

KINDS = oact.ACTS


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def tables(dev):
    t = {k: fp8.act_table(k, dev) for k in KINDS}
    torch.cuda.synchronize()
    return t


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _from_bits(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)


def _normal(m, k, seed, scale=1.0):
    a = make_case(m, 16, k, seed=seed, kind="normal", with_bias=False).a
    return (a.float() * scale).to(torch.bfloat16) if scale != 1.0 else a


@pytest.mark.parametrize("kind", KINDS)
def test_table_every_input_pattern(tables, kind):
    gpu = _u16(tables[kind])
    pats, vals = oact.table(kind)
    bad = np.nonzero(gpu[pats] != vals)[0]
    assert len(bad) == 0, f"{kind}: {len(bad)} entries differ, first patterns {[hex(p) for p in pats[bad[:8]]]}"
    # outside the contract, but defined: NaN -> NaN, +inf -> +inf, -inf -> -0
    assert gpu[0x7F80] == 0x7F80 and gpu[0xFF80] == 0x8000
    assert gpu[0x7FC0] == 0x7FC0 and gpu[0xFFC1] == 0x7FC0


@pytest.mark.parametrize("kind", KINDS)
def test_plain_producer_every_pattern_and_random(dev, tables, kind):
    pats, vals = oact.table(kind)
    x = _from_bits(pats.reshape(255, 256), dev)
    y = fp8.act_rows(x, tables[kind])
    assert np.array_equal(_u16(y).reshape(-1), vals)
    xr = _normal(37, 1040, seed=3, scale=4.0)
    yr = fp8.act_rows(xr.to(dev), tables[kind])
    assert np.array_equal(_u16(yr), oact.act_bf16_bits(bf16_bits(xr), kind))


# rows x cols: one chunk per lane and less, ragged chunk counts, two / four / eight
# register chunks, and rows too long for registers (the two-pass loop)
SHAPES = [(5, 16), (64, 256), (37, 1040), (33, 2064), (17, 4112), (16, 8192), (9, 8208), (3, 16400), (300, 2048)]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_fused_producer_matches_oracle(dev, tables, kind, rows, cols):
    x = _normal(rows, cols, seed=rows * 7 + cols, scale=3.0)
    q, s = fp8.act_quant_rows(x.to(dev), tables[kind])
    eq, es = oact.act_quant_rows(bf16_bits(x), kind)
    assert np.array_equal(q.cpu().numpy(), eq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), es.view(np.uint32))


@pytest.mark.parametrize("kind", KINDS)
def test_fused_producer_special_rows(dev, tables, kind):
    cols = 1024
    rng = np.random.default_rng(5)
    rows = [
        np.zeros(cols, np.uint16),                                  # all +0: scale 0, codes 0
        np.full(cols, 0x8000, np.uint16),                           # all -0
        rng.integers(1, 0x100, cols).astype(np.uint16),             # |x| < 2^-125: the tie inputs
        (rng.integers(1, 0x100, cols) | 0x8000).astype(np.uint16),  # the same, negative
        rng.integers(0x0100, 0x7F80, cols).astype(np.uint16),       # every positive magnitude
        rng.integers(0x8100, 0xFF80, cols).astype(np.uint16),       # every negative magnitude
        np.full(cols, 0xC2B0, np.uint16),                           # -88: SiLU's far tail, GELU's -0
        np.full(cols, 0x7F7F, np.uint16),                           # the largest finite bf16
    ]
    bits = np.stack(rows)
    q, s = fp8.act_quant_rows(_from_bits(bits, dev), tables[kind])
    eq, es = oact.act_quant_rows(bits, kind)
    assert np.array_equal(q.cpu().numpy(), eq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), es.view(np.uint32))


# (2050, 8192) and (1500, 4112) take several iterations of the persistent row loop
# (with a ragged last one) on a 256-CU device
@pytest.mark.parametrize("rows,cols", [(257, 8192), (2050, 8192), (1500, 4112)])
@pytest.mark.parametrize("kind", KINDS)
def test_fused_equals_unfused_on_gpu(dev, tables, kind, rows, cols):
    x = _normal(rows, cols, seed=9 + rows, scale=2.0).to(dev)
    q1, s1 = fp8.act_quant_rows(x, tables[kind])
    q2, s2 = fp8.quant_rows(fp8.act_rows(x, tables[kind]))
    assert torch.equal(q1, q2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


@pytest.mark.parametrize("kind,rows", [("gelu_tanh", 4096), ("gelu_tanh", 32760), ("gelu_erf", 4096),
                                       ("silu", 4096)])
def test_fused_producer_full_size_ffn_down_input(dev, tables, kind, rows):
    # the FFN-down input at the FFN shape [4096, 8192] (every activation) and at the DiT-block
    # size [32760, 8192], every row: the oracle's exact activation table, then the C statement
    # of the per-token quantiser (pinned bit for bit to oracle.quant)
    x = _normal(rows, 8192, seed=21)
    q, s = fp8.act_quant_rows(x.to(dev), tables[kind])
    torch.cuda.synchronize()
    eq, es = cref.quant_rows(oact.act_bf16_bits(bf16_bits(x), kind))
    assert_codes_equal(q, s, eq, es, f"{kind} producer [{rows}, 8192]")


def test_fused_producer_feeds_the_fp8_linear(dev, tables):
    # FFN-down: GELU producer -> (codes, scale) -> FP8 linear against W [2048, 8192]
    case = make_case(96, 2048, 8192, seed=4, kind="normal")
    q, s = fp8.act_quant_rows(case.a.to(dev), tables["gelu_erf"])
    lin = fp8.Fp8Linear(case.w.to(dev), case.bias.to(dev))
    out = lin(q, x_scale=s)
    eq, es = oact.act_quant_rows(bf16_bits(case.a), "gelu_erf")
    qw, sw = oq.quant_weights_per_channel(bf16_bits(case.w))
    ref = ol.linear_ref_fp8(eq, es, qw, sw, bf16_bits(case.bias))
    assert_linear_close(out, ref, "gelu -> fp8 linear")


def test_shared_table_across_calls_and_streams(dev, tables):
    # a table is read-only: two streams may use it at once
    x1 = _normal(64, 2048, seed=30).to(dev)
    x2 = _normal(48, 8192, seed=31).to(dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        r1 = fp8.act_quant_rows(x1, tables["silu"])
    with torch.cuda.stream(s2):
        r2 = fp8.act_quant_rows(x2, tables["silu"])
    torch.cuda.synchronize()
    for x, (q, s) in ((x1, r1), (x2, r2)):
        eq, es = oact.act_quant_rows(bf16_bits(x.cpu()), "silu")
        assert np.array_equal(q.cpu().numpy(), eq) and np.array_equal(s.cpu().numpy(), es)
