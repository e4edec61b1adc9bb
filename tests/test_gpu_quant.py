"""GPU parity of the per-token / per-channel quantiser against the CPU oracle.

Codes and scales must be bit-identical: every config activation and weight,
ragged and edge shapes, special rows (zero, signed zero, tiny amax that takes the
exact-division path, extreme magnitudes, ties), guard bands around the outputs,
and the exhaustive sweep over every pair of finite bf16 values (x, amax).
"""

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from fp8_w8a8_quantized_token_amd import quant_rows, quant_weights_per_channel
from oracle import cref, quant as oq
from tests._helpers import assert_codes_equal, require_gpu
from workloads import CONFIGS, bf16_bits, make_case, make_config

pytestmark = pytest.mark.gpu


def _check(x_cpu, label, rows=None):
    dev = require_gpu()
    q, s = quant_rows(x_cpu.to(dev))
    torch.cuda.synchronize()
    bits = bf16_bits(x_cpu)
    q, s = q.cpu().numpy(), s.cpu().numpy()
    if rows is not None:
        bits, q, s = bits[rows], q[rows], s[rows]
    eq, es = oq.quant_rows(bits)
    assert np.array_equal(s.view(np.uint32), es.view(np.uint32)), f"{label}: scales differ"
    bad = np.argwhere(q != eq)
    assert bad.size == 0, f"{label}: {len(bad)} codes differ, first at {bad[0]}: gpu {q[tuple(bad[0])]:#x} " \
                          f"oracle {eq[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("config", ["tiny", "ffn_up", "ffn_down"])
def test_config_activations_and_weights_bit_exact(config):
    cfg = make_config(config)
    for name, a in cfg["activations"].items():
        _check(a, f"{config}/{name}")
    for layer, w in cfg["weights"].items():
        _check(w, f"{config}/W_{layer}")


@pytest.mark.slow
@pytest.mark.parametrize("config", ["qkv", "dit_block"])
def test_large_config_activations_every_row(config):
    # every row of the 32760-token activations, against the C statement of the oracle
    # (pinned bit for bit to oracle.quant), which handles these sizes in about a second
    dev = require_gpu()
    cfg = make_config(config)
    tensors = dict(cfg["activations"])
    seen = set()
    for layer, w in cfg["weights"].items():
        if id(w) not in seen:
            seen.add(id(w))
            tensors[f"W_{layer}"] = w
    for name, x in tensors.items():
        q, s = quant_rows(x.to(dev))
        torch.cuda.synchronize()
        eq, es = cref.quant_rows(bf16_bits(x))
        assert_codes_equal(q, s, eq, es, f"{config}/{name}")


@pytest.mark.parametrize("rows", [1, 3, 63, 65, 257])
@pytest.mark.parametrize("cols", [16, 48, 272, 1024, 1040, 2064, 4096, 4112, 8192, 8208, 16400, 65536])
def test_edge_shapes(rows, cols):
    if rows * cols > 257 * 16400:
        rows = 3
    x = make_case(rows, 16, cols, seed=rows * 7 + cols, kind="outlier").a
    _check(x, f"{rows}x{cols}")


@pytest.mark.parametrize("cols", [4112, 6160, 8192])
def test_many_long_rows(cols):
    # 16384 rows or more of 4097..8192 elements take eight wavefronts per row: every row
    # against the C statement of the oracle, ragged chunk counts included
    dev = require_gpu()
    x = make_case(16400, 16, cols, seed=cols, kind="outlier").a
    q, s = quant_rows(x.to(dev))
    torch.cuda.synchronize()
    eq, es = cref.quant_rows(bf16_bits(x))
    assert_codes_equal(q, s, eq, es, f"16400x{cols}")


def _bf16(values):
    return torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16)


def test_special_rows():
    rng = np.random.default_rng(1)
    k = 1024
    rows = []
    rows.append(np.zeros(k))                                      # all zero
    z = np.zeros(k); z[::3] = -0.0; rows.append(z)                 # signed zeros only
    rows.append(rng.standard_normal(k) * 2.0 ** -100)              # tiny amax: exact-division path
    rows.append(rng.standard_normal(k) * 2.0 ** -128)              # bf16 subnormals, subnormal scale
    rows.append(rng.standard_normal(k) * 2.0 ** -79)               # just above the fast-path threshold
    rows.append(rng.standard_normal(k) * 2.0 ** 120)               # huge
    rows.append(np.full(k, 3.25))                                  # constant row
    t = rng.choice([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -1.0625, 0.0, -0.0, 7.5 * 2.0 ** -9], k)
    t[0] = 448.0; rows.append(t)                                   # s = 1: quotients land on ties
    u = rng.standard_normal(k); u[5] = -0.0; u[6] = 0.0; rows.append(u)
    v = rng.standard_normal(k) * 1e-3; v[100] = 60000.0; rows.append(v)  # one dominant outlier
    x = _bf16(np.stack(rows))
    _check(x, "special rows")


def test_weight_entry_point_matches_rows_entry_point():
    dev = require_gpu()
    w = make_case(16, 384, 512, seed=5).w.to(dev)
    q1, s1 = quant_weights_per_channel(w)
    q2, s2 = quant_rows(w)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    eq, es = oq.quant_weights_per_channel(bf16_bits(w.cpu()))
    assert np.array_equal(q1.cpu().numpy(), eq) and np.array_equal(s1.cpu().numpy(), es)


def test_outputs_stay_in_bounds():
    """Sentinels around q and scale survive: the kernel writes exactly [rows, cols] and [rows]."""
    from fp8_w8a8_quantized_token_amd import _lib
    import ctypes
    dev = require_gpu()
    rows, cols, pad = 37, 1040, 4096
    x = make_case(rows, 16, cols, seed=2).a.to(dev)
    qbuf = torch.full((pad + rows * cols + pad,), 0xA5, dtype=torch.uint8, device=dev)
    sbuf = torch.full((64 + rows + 64,), -7.0, dtype=torch.float32, device=dev)
    q = qbuf[pad:pad + rows * cols]
    s = sbuf[64:64 + rows]
    st = _lib.lib().fp8_quant_rows(ctypes.c_void_p(x.data_ptr()), rows, cols, ctypes.c_void_p(q.data_ptr()),
                                   ctypes.c_void_p(s.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    qb, sb = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(qb[:pad] == 0xA5) and np.all(qb[pad + rows * cols:] == 0xA5)
    assert np.all(sb[:64] == -7.0) and np.all(sb[64 + rows:] == -7.0)
    eq, es = oq.quant_rows(bf16_bits(x.cpu()))
    assert np.array_equal(q.cpu().numpy().reshape(rows, cols), eq)


@pytest.mark.slow
def test_exhaustive_bf16_pairs():
    """Every finite bf16 amax > 0 against every bf16 x with |x| <= amax (about 1.07e9 pairs).

    Row a holds all 65536 bf16 patterns with magnitudes above amax replaced by +-amax
    and non-finite patterns replaced by zero, so its row maximum is exactly amax. The
    codes and scales must equal the C statement of the oracle (itself pinned to
    oracle.quant) for every element.
    """
    from oracle import cref
    dev = require_gpu()
    cols = 1 << 16
    pat = torch.arange(cols, dtype=torch.int32, device=dev)
    mag = pat & 0x7FFF
    sign = pat & 0x8000
    finite = mag <= 0x7F7F
    amax_bits = torch.arange(1, 0x7F80, dtype=torch.int32, device=dev)  # every positive finite bf16
    chunk = 1024
    mismatches = 0
    for start in range(0, amax_bits.numel(), chunk):
        a = amax_bits[start:start + chunk, None]
        m = torch.where(mag[None, :] > a, a, mag[None, :])
        m = torch.where(finite[None, :], m, torch.zeros_like(m))
        xb = (sign[None, :] | m).to(torch.int16).contiguous().view(torch.bfloat16)
        q, s = quant_rows(xb)
        torch.cuda.synchronize()
        eq, es = cref.quant_rows(xb.view(torch.int16).cpu().numpy().view(np.uint16))
        assert np.array_equal(s.cpu().numpy().view(np.uint32), es.view(np.uint32)), f"scales differ in chunk {start}"
        diff = q.cpu().numpy() != eq
        mismatches += int(diff.sum())
        assert mismatches == 0, f"{mismatches} codes differ (amax chunk starting at bf16 {start + 1:#06x})"


def test_empty_inputs_through_the_bindings():
    # no tokens: empty outputs of the right shapes and nothing launched; the per-tensor
    # converter treats an empty tensor as invalid input
    dev = require_gpu()
    x = torch.zeros((0, 2048), dtype=torch.bfloat16, device=dev)
    q, s = fp8.quant_rows(x)
    assert q.shape == (0, 2048) and s.shape == (0,)
    table = fp8.act_table("gelu_tanh", dev)
    assert fp8.act_rows(x, table).shape == (0, 2048)
    q, s = fp8.act_quant_rows(x, table)
    assert q.shape == (0, 2048) and s.shape == (0,)
    with pytest.raises(ValueError, match="empty"):
        fp8.quant_tensor(x)
    d = fp8.dequant_tensor(torch.zeros((0, 16), dtype=torch.uint8, device=dev), torch.ones((1,), device=dev))
    assert d.shape == (0, 16)
