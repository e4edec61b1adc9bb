"""GPU parity of the grouped linear (several weights on one activation, quantised once).

The retrospective (aigcage.com, section 3.4) feeds one set of hidden states into the
Q, K and V projections. fp8_linear_run_group runs such a group: one per-token
quantisation, then ONE GEMM launch over every problem's tiles when each plan would take
the persistent configuration at this m (or each the skinny one, at a few tokens), else
each plan's own GEMM.
Each output must be bit-identical to the plan's separate fp8_linear_run (same codes,
same products summed in the same order), and rows of it (the first tile row and the
ragged last one) are compared with the float64 oracle under the linear tests' bound.
Covered: groups of 1..4 problems with ragged n (a partial last tile column in each
problem), with and without bias in one group, bf16 and e4m3fn inputs, skinny groups at
1..32 tokens, groups that fall back to per-plan launches (mixed configurations), m = 0,
a grouped call captured in a HIP graph and replayed with new inputs, the C ABI's
shape and workspace checks, and the Q/K/V projections at full size.
"""

import ctypes
from types import SimpleNamespace

import pytest
import torch

from fp8_w8a8_quantized_token_amd import Fp8Linear, Fp8W8A8Error, _lib, group_config, linear_group, quant_rows
from oracle import cref, linear as ol
from tests._helpers import assert_codes_equal, assert_linear_close, require_gpu
from workloads import bf16_bits, make_case, make_config

pytestmark = pytest.mark.gpu

PERSISTENT = 6
SKINNY = 5
SKINNY_WIDE = 7  # the same weight stream with 32 channels per workgroup


def _cus(dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def _layers(ns, k, dev, seed, no_bias=()):
    lins, cases = [], []
    for i, n in enumerate(ns):
        c = make_case(16, n, k, seed=seed + i, with_bias=i not in no_bias)
        lins.append(Fp8Linear(c.w.to(dev), c.bias.to(dev) if c.bias is not None else None))
        cases.append(c)
    return lins, cases


def _bits(t):
    return t.view(torch.int16)


def _check_rows_against_oracle(outs, cases, qa, sa, label):
    """Oracle rows [0, 256) and the last (ragged) tile row of every output."""
    m = qa.shape[0]
    last = (m - 1) // 256 * 256
    for i, (out, c) in enumerate(zip(outs, cases)):
        qw, sw = cref.quant_rows(bf16_bits(c.w))
        bias_bits = None if c.bias is None else bf16_bits(c.bias)
        for r0, r1 in ((0, min(256, m)), (last, m)):
            ref = ol.linear_ref_fp8(qa[r0:r1], sa[r0:r1], qw, sw, bias_bits)
            assert_linear_close(out[r0:r1], ref, f"{label} problem {i} rows {r0}..{r1}")


@pytest.mark.parametrize("a_kind", ["bf16", "e4m3"])
def test_group_in_one_persistent_launch_matches_separate_runs(a_kind):
    dev = require_gpu()
    m, k = 8200, 2048  # a ragged last tile row (8 tokens)
    ns = (4112, 4624, 5136)  # 17, 19, 21 tile columns, each with a 16-column last one
    lins, cases = _layers(ns, k, dev, seed=11, no_bias=(2,))
    if _cus(dev) == 256:
        assert all(lin.config(m)[0] == PERSISTENT for lin in lins)
    a = make_case(m, 16, k, seed=12, kind="outlier").a
    qa, sa = cref.quant_rows(bf16_bits(a))
    if a_kind == "bf16":
        x, xs = a.to(dev), None
    else:
        x, xs = torch.from_numpy(qa).to(dev), torch.from_numpy(sa).to(dev)
    separate = [lin(x, xs) for lin in lins]
    ws = torch.empty((lins[0].workspace_bytes(m),), dtype=torch.uint8, device=dev)
    grouped = linear_group(lins, x, xs, workspace=ws)
    torch.cuda.synchronize()
    if a_kind == "bf16":  # the group's one quantisation, left in the workspace
        cb = (m * k + 255) // 256 * 256
        assert_codes_equal(ws[: m * k].view(m, k), ws[cb: cb + 4 * m].view(torch.float32), qa, sa, "group codes")
    for i, (g, s) in enumerate(zip(grouped, separate)):
        assert g.shape == (m, ns[i])
        assert torch.equal(_bits(g), _bits(s)), f"problem {i}: group and separate run differ"
    _check_rows_against_oracle(grouped, cases, qa, sa, f"group {a_kind}")


def test_groups_of_one_and_of_four():
    dev = require_gpu()
    m, k = 16400, 2048
    ns = (2064, 4112, 2320, 3088)  # 9, 17, 10, 13 tile columns
    lins, cases = _layers(ns, k, dev, seed=21, no_bias=(1,))
    if _cus(dev) == 256:
        assert all(lin.config(m)[0] == PERSISTENT for lin in lins)
    a = make_case(m, 16, k, seed=22, kind="outlier").a
    x = a.to(dev)
    separate = [lin(x) for lin in lins]
    four = linear_group(lins, x)
    one = linear_group(lins[1:2], x)
    # outputs passed in, with guard rows around them
    bufs = [torch.full((m + 2, n), -7.0, dtype=torch.bfloat16, device=dev) for n in ns[:2]]
    two = linear_group(lins[:2], x, outs=[b[1: m + 1] for b in bufs])
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(_bits(four[i]), _bits(separate[i])), f"group of four, problem {i}"
    assert torch.equal(_bits(one[0]), _bits(separate[1])), "group of one"
    for i, b in enumerate(bufs):
        assert torch.equal(_bits(two[i]), _bits(separate[i])), f"group of two, problem {i}"
        assert torch.all(b[0] == -7.0) and torch.all(b[m + 1] == -7.0), "guard rows overwritten"
    qa, sa = cref.quant_rows(bf16_bits(a))
    _check_rows_against_oracle(four, cases, qa, sa, "group of four")


@pytest.mark.parametrize("m", [1, 17, 26, 32])
@pytest.mark.parametrize("a_kind", ["bf16", "e4m3"])
@pytest.mark.parametrize("ns", [(4112, 1040, 2064), (1040, 2064, 528)])
def test_group_of_skinny_problems_in_one_launch(m, a_kind, ns):
    # a few tokens (the 26-row encoder input): every plan takes a skinny form, and the
    # group runs as one launch over all the problems' column blocks (the wide form when
    # their 16-channel blocks together outnumber the CUs: 451 blocks, else 227)
    dev = require_gpu()
    k = 2048
    lins, cases = _layers(ns, k, dev, seed=51, no_bias=(1,))
    assert all(lin.config(m)[0] in (SKINNY, SKINNY_WIDE) for lin in lins)
    a = make_case(m, 16, k, seed=52, kind="outlier").a
    qa, sa = cref.quant_rows(bf16_bits(a))
    if a_kind == "bf16":
        x, xs = a.to(dev), None
    else:
        x, xs = torch.from_numpy(qa).to(dev), torch.from_numpy(sa).to(dev)
    separate = [lin(x, xs) for lin in lins]
    grouped = linear_group(lins, x, xs)
    torch.cuda.synchronize()
    for i, (g, s) in enumerate(zip(grouped, separate)):
        assert torch.equal(_bits(g), _bits(s)), f"m={m} problem {i}"
    _check_rows_against_oracle(grouped, cases, qa, sa, f"skinny group m={m}")


def test_group_reports_its_launch_form():
    # the configuration of the one launch, as the run takes it: the Q/K/V weights at 32760
    # tokens as one persistent launch, their 26-row encoder input as one wide skinny launch
    # (384 16-channel blocks on 256 CUs), a narrow skinny group (227 blocks) in
    # configuration 5, and a narrow weight next to a wide one at 700 tokens as separate GEMMs
    dev = require_gpu()
    if _cus(dev) != 256:
        pytest.skip("the forms are chosen for a 256-CU device")
    qkv, _ = _layers((2048, 2048, 2048), 2048, dev, seed=81)
    assert group_config(qkv, 32760) == PERSISTENT
    assert group_config(qkv, 26) == SKINNY_WIDE
    assert group_config(qkv[:1], 26) == -1 and group_config(qkv, 0) == -1
    narrow, _ = _layers((1040, 2064, 528), 2048, dev, seed=82)
    assert group_config(narrow, 26) == SKINNY
    mixed, _ = _layers((4112, 1040), 2048, dev, seed=83)
    assert group_config(mixed, 700) == -1


@pytest.mark.parametrize("m", [0, 700, 3000, 8200])
def test_group_falls_back_to_each_plans_own_launch(m):
    # at these m the plans do not all take one groupable form (a narrow weight next to a
    # wide one, or neither persistent nor skinny): every plan runs its own GEMM on the
    # shared codes
    dev = require_gpu()
    k = 2048
    lins, cases = _layers((4112, 1040), k, dev, seed=31)
    if m > 0 and _cus(dev) == 256:
        assert lins[1].config(m)[0] not in (PERSISTENT, SKINNY, SKINNY_WIDE)
    a = make_case(max(m, 1), 16, k, seed=32, kind="outlier").a[:m]
    x = a.to(dev)
    separate = [lin(x) for lin in lins]
    grouped = linear_group(lins, x)
    torch.cuda.synchronize()
    for i, (g, s) in enumerate(zip(grouped, separate)):
        assert g.shape == (m, lins[i].n)
        assert torch.equal(_bits(g), _bits(s)), f"m={m} problem {i}"
    if m > 0:
        qa, sa = cref.quant_rows(bf16_bits(a))
        _check_rows_against_oracle(grouped, cases, qa, sa, f"fallback m={m}")


def test_group_abi_checks_plans_before_launching():
    dev = require_gpu()
    a = torch.zeros((64, 2048), dtype=torch.bfloat16, device=dev)
    lins, _ = _layers((2048,), 2048, dev, seed=41)
    other_k, _ = _layers((2048,), 1024, dev, seed=42)
    out = torch.empty((64, 2048), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((lins[0].workspace_bytes(64),), dtype=torch.uint8, device=dev)
    lib = _lib.lib()

    def call(plans, nplans, ws_bytes=None):
        parr = (ctypes.c_void_p * len(plans))(*[p._plan.value for p in plans])
        oarr = (ctypes.c_void_p * len(plans))(*([out.data_ptr()] * len(plans)))
        return lib.fp8_linear_run_group(ctypes.cast(parr, ctypes.c_void_p), nplans, 64, a.data_ptr(), _lib.A_BF16,
                                        None, ctypes.cast(oarr, ctypes.c_void_p), ws.data_ptr(),
                                        ws.numel() if ws_bytes is None else ws_bytes, None)

    out.fill_(3.0)
    torch.cuda.synchronize()
    assert call(lins + other_k, 2) == _lib.ERR_BAD_SHAPE
    assert call(lins + lins, 2, ws_bytes=16) == _lib.ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0), "a rejected call launched something"
    with pytest.raises(ValueError):
        linear_group(lins + other_k, torch.zeros((64, 2048), dtype=torch.bfloat16, device=dev))
    with pytest.raises(Fp8W8A8Error):  # the library's own check (the binding checks k first)
        x1 = torch.zeros((64, 1024), dtype=torch.bfloat16, device=dev)
        linear_group(other_k, x1, workspace=torch.empty((16,), dtype=torch.uint8, device=dev))


@pytest.mark.slow
def test_qkv_group_full_size():
    # the three projections of the 32760-token hidden states in one group, and of the
    # 26-token encoder states (per-plan launches at that m)
    dev = require_gpu()
    cfg = make_config("qkv")
    names = ("q", "k", "v")
    lins = [Fp8Linear(cfg["weights"][n].to(dev), cfg["biases"][n].to(dev)) for n in names]
    for act in ("hidden", "encoder"):
        a = cfg["activations"][act]
        x = a.to(dev)
        separate = [lin(x) for lin in lins]
        grouped = linear_group(lins, x)
        qx, sx = quant_rows(x)
        codes_grouped = linear_group(lins, qx, sx)
        torch.cuda.synchronize()
        for i, name in enumerate(names):
            assert torch.equal(_bits(grouped[i]), _bits(separate[i])), f"{act}/{name}"
            assert torch.equal(_bits(codes_grouped[i]), _bits(separate[i])), f"{act}/{name} e4m3fn input"
        qa, sa = cref.quant_rows(bf16_bits(a))
        assert_codes_equal(qx, sx, qa, sa, f"qkv/{act} codes")
        cases = [SimpleNamespace(w=cfg["weights"][n], bias=cfg["biases"][n]) for n in names]
        _check_rows_against_oracle(grouped, cases, qa, sa, f"qkv group {act}")


@pytest.mark.parametrize("m", [26, 8200])
def test_group_replayed_from_a_graph_with_new_inputs(m):
    # one grouped call (quantisation + one GEMM launch, skinny at 26 tokens, persistent at
    # 8200) captured once and replayed with new inputs copied in between; every replay must
    # equal the eager separate runs on that input, bit for bit
    dev = require_gpu()
    k = 2048
    lins, _ = _layers((4112, 4624), k, dev, seed=61, no_bias=(0,))
    if _cus(dev) == 256:
        assert len({lin.config(m)[0] for lin in lins}) == 1 and lins[0].config(m)[0] in (SKINNY, SKINNY_WIDE, PERSISTENT)
    inputs = [make_case(m, 16, k, seed=62 + i, kind="outlier").a.to(dev) for i in range(3)]
    x = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((lins[0].workspace_bytes(m),), dtype=torch.uint8, device=dev)
    outs = [torch.empty((m, lin.n), dtype=torch.bfloat16, device=dev) for lin in lins]
    x.copy_(inputs[0])
    linear_group(lins, x, outs=outs, workspace=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g, stream=side):
        linear_group(lins, x, outs=outs, workspace=ws)
    torch.cuda.synchronize()
    for inp in inputs:
        x.copy_(inp)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        expect = [lin(inp) for lin in lins]
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, expect)):
            assert torch.equal(_bits(o), _bits(e)), f"m={m} problem {i}"
