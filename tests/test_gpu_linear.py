"""GPU parity of the FP8 W8A8 linear against the float64 CPU oracle.

Every GPU output is compared with the oracle's unrounded reference computed from
the same bf16 inputs (the oracle quantises them itself): elementwise
|gpu - ref| <= 1e-2 (|ref| + 1) and relative Frobenius error <= 2e-3. Quantised
activations and weights are compared bit for bit on the way. Covered: the tiny
config in full; every compiled GEMM configuration on ragged m / n / k tails; the
persistent configuration where each of its workgroups walks several tiles (whole output,
and bit for bit against one workgroup per tile); the selector's plans at the four full-size workloads, every output element against the
oracle (elementwise bound on each, relative Frobenius error over the whole output) and
every activation code and scale bit for bit; the e4m3fn pass-through input on the
oracle's own codes; A = 0 (output == bias exactly); no bias; guard bands.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_token_amd as fp8
from fp8_w8a8_quantized_token_amd import Fp8Linear, gemm_config_count, gemm_run_config, quant_rows
from oracle import cref, linear as ol, quant as oq
from tests._helpers import assert_codes_equal, assert_linear_close, assert_linear_close_rows, require_gpu
from workloads import bf16_bits, make_case, make_config

pytestmark = pytest.mark.gpu


def _oracle_weight(w_cpu):
    return oq.quant_weights_per_channel(bf16_bits(w_cpu))


def _cus(dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def _bias_bits(b):
    return None if b is None else bf16_bits(b)


def test_tiny_config_full():
    dev = require_gpu()
    cfg = make_config("tiny")
    a, w, b = cfg["activations"]["a"], cfg["weights"]["linear"], cfg["biases"]["linear"]
    lin = Fp8Linear(w.to(dev), b.to(dev))
    out = lin(a.to(dev))
    qa, sa = quant_rows(a.to(dev))
    torch.cuda.synchronize()
    qw, sw = _oracle_weight(w)
    assert np.array_equal(lin.w_fp8.cpu().numpy(), qw) and np.array_equal(lin.w_scale.cpu().numpy(), sw)
    ref, eqa, esa = ol.linear_ref(bf16_bits(a), qw, sw, bf16_bits(b))
    assert np.array_equal(qa.cpu().numpy(), eqa) and np.array_equal(sa.cpu().numpy(), esa)
    assert_linear_close(out, ref, "tiny")


try:
    N_CONFIGS = gemm_config_count()
except Exception:  # library not built: the GPU tests below report it
    N_CONFIGS = 1

TAIL_SHAPES = [(1, 16, 16), (26, 144, 48), (63, 16, 272), (65, 144, 16), (257, 144, 272), (300, 272, 400),
               (513, 528, 1040)]


PERSISTENT = 6  # the 256 x 256 tiles walked by one workgroup per CU
SKINNY, SKINNY_WIDE = 5, 7  # the weight stream, 16 and 32 channels per workgroup


@pytest.mark.parametrize("config", range(N_CONFIGS))
@pytest.mark.parametrize("m,n,k", TAIL_SHAPES)
def test_every_config_on_ragged_tails(config, m, n, k):
    dev = require_gpu()
    assert config < gemm_config_count()
    case = make_case(m, n, k, seed=m + n + k, kind="outlier")
    qa, sa = oq.quant_rows(bf16_bits(case.a))
    qw, sw = _oracle_weight(case.w)
    ref = ol.linear_ref_fp8(qa, sa, qw, sw, _bias_bits(case.bias))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    out = gemm_run_config(config, t(qa), t(sa), t(qw), t(sw), case.bias.to(dev))
    torch.cuda.synchronize()
    assert_linear_close(out, ref, f"config {config} {m}x{n}x{k}")


# more tiles than compute units, ragged in m, n and k (a one-stage k among them): every
# workgroup of the persistent configuration walks several tiles, each handing its stage
# ring to the next before its epilogue
PERSISTENT_SHAPES = [(4100, 12304, 272), (8200, 8208, 208), (8197, 8208, 128), (16400, 4112, 144)]


@pytest.mark.parametrize("m,n,k,with_bias", [s + (True,) for s in PERSISTENT_SHAPES] + [(8200, 8208, 208, False)])
def test_persistent_config_walks_many_tiles(m, n, k, with_bias):
    dev = require_gpu()
    tiles = -(-m // 256) * -(-n // 256)
    assert tiles > 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    case = make_case(m, n, k, seed=m + n + k, kind="outlier")
    qa, sa = cref.quant_rows(bf16_bits(case.a))
    qw, sw = _oracle_weight(case.w)
    bias = case.bias if with_bias else None
    bias_bits = _bias_bits(bias)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    args = (t(qa), t(sa), t(qw), t(sw), bias.to(dev) if bias is not None else None)
    out = gemm_run_config(PERSISTENT, *args)
    out0 = gemm_run_config(0, *args)
    torch.cuda.synchronize()
    # the same products summed in the same order as one workgroup per tile
    assert torch.equal(out.view(torch.int16), out0.view(torch.int16))
    assert_linear_close_rows(out, lambda r0, r1: ol.linear_ref_fp8(qa[r0:r1], sa[r0:r1], qw, sw, bias_bits),
                             f"persistent {m}x{n}x{k}")


def test_one_plan_on_two_streams_at_once():
    # a plan is immutable after construction: runs on different streams (each with its
    # own workspace) may overlap, here one on the persistent configuration (4096 tokens)
    # and one on another (700 tokens), plus a second plan on a third stream
    dev = require_gpu()
    case = make_case(4096, 8192, 2048, seed=77, kind="outlier")
    lin = Fp8Linear(case.w.to(dev), case.bias.to(dev))
    other = Fp8Linear(make_case(16, 2048, 2048, seed=78).w.to(dev))
    a1 = case.a.to(dev)
    a2 = make_case(700, 8192, 2048, seed=79, kind="outlier").a.to(dev)
    a3 = make_case(2000, 2048, 2048, seed=80).a.to(dev)
    jobs = [(lin, a1), (lin, a2), (other, a3)]
    assert lin.config(4096)[0] == PERSISTENT or torch.cuda.get_device_properties(dev).multi_processor_count != 256
    serial = []
    for p, a in jobs:
        serial.append(p(a))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(dev) for _ in jobs]
    outs = []
    for _ in range(3):
        torch.cuda.synchronize()
        res = []
        for st, (p, a) in zip(streams, jobs):
            with torch.cuda.stream(st):
                ws = torch.empty((p.workspace_bytes(a.shape[0]),), dtype=torch.uint8, device=dev)
                res.append(p(a, workspace=ws))
        torch.cuda.synchronize()
        outs.append(res)
    for res in outs:
        for got, want in zip(res, serial):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_zero_activation_gives_bias_exactly():
    dev = require_gpu()
    case = make_case(70, 272, 256, seed=3)
    lin = Fp8Linear(case.w.to(dev), case.bias.to(dev))
    out = lin(torch.zeros((70, 256), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    expect = case.bias.expand(70, 272)
    assert torch.equal(out.cpu(), expect)


def test_no_bias_and_gelu_input():
    dev = require_gpu()
    case = make_case(200, 160, 512, seed=4, kind="gelu", with_bias=False)
    lin = Fp8Linear(case.w.to(dev))
    out = lin(case.a.to(dev))
    torch.cuda.synchronize()
    qw, sw = _oracle_weight(case.w)
    ref, _, _ = ol.linear_ref(bf16_bits(case.a), qw, sw, None)
    assert_linear_close(out, ref, "no bias")


def test_fp8_input_passthrough_matches_bf16_path():
    # an input that is already e4m3fn goes straight to the GEMM with the scales passed in;
    # the codes here are the oracle's own (not the GPU quantiser's), so the check of the
    # pass-through against the oracle depends on no other GPU step
    dev = require_gpu()
    case = make_case(333, 384, 1024, seed=6)
    lin = Fp8Linear(case.w.to(dev), case.bias.to(dev))
    eqa, esa = oq.quant_rows(bf16_bits(case.a))
    qw, sw = _oracle_weight(case.w)
    ref = ol.linear_ref_fp8(eqa, esa, qw, sw, bf16_bits(case.bias))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    out_fp8 = lin(t(eqa).view(torch.float8_e4m3fn), t(esa))
    out_u8 = lin(t(eqa), t(esa))
    a = case.a.to(dev)
    out_bf16 = lin(a)
    torch.cuda.synchronize()
    assert_linear_close(out_fp8, ref, "e4m3fn pass-through")
    assert torch.equal(out_fp8, out_u8)
    # the bf16 input quantises to the same codes, so the two forwards agree bit for bit
    assert torch.equal(out_bf16, out_fp8)


def test_three_dim_input_and_out_buffer_guard_band():
    dev = require_gpu()
    case = make_case(2 * 75, 144, 256, seed=8)
    lin = Fp8Linear(case.w.to(dev), case.bias.to(dev))
    m, n = 150, 144
    pad = 1024
    buf = torch.full((pad + m * n + pad,), 12345.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + m * n]
    res = lin(case.a.reshape(2, 75, 256).to(dev), out=out)
    torch.cuda.synchronize()
    assert res.shape == (2, 75, 144)
    b = buf.cpu()
    assert torch.all(b[:pad] == 12345.0) and torch.all(b[pad + m * n:] == 12345.0)
    qw, sw = _oracle_weight(case.w)
    ref, _, _ = ol.linear_ref(bf16_bits(case.a), qw, sw, bf16_bits(case.bias))
    assert_linear_close(out.reshape(m, n), ref, "3-d input")


def _full_size_linear(a_cpu, w_cpu, b_cpu, dev, label, qa_gpu=None, sa_gpu=None, lin=None, oracle_codes=None,
                      oracle_weight=None):
    """Run the plan at full size on the GPU and compare its whole output with the oracle.

    The oracle's codes come from the C statement of the per-token quantiser (pinned bit
    for bit to oracle.quant). A bf16 run leaves its codes and scales in the workspace;
    those are compared bit for bit too. An e4m3fn run (qa_gpu, sa_gpu) takes the codes
    the caller produced and checked."""
    if lin is None:
        lin = Fp8Linear(w_cpu.to(dev), b_cpu.to(dev))
    m, k = a_cpu.shape
    eqa, esa = oracle_codes if oracle_codes is not None else cref.quant_rows(bf16_bits(a_cpu))
    qw, sw = oracle_weight if oracle_weight is not None else cref.quant_rows(bf16_bits(w_cpu))
    if qa_gpu is None:
        ws = torch.empty((lin.workspace_bytes(m),), dtype=torch.uint8, device=dev)
        out = lin(a_cpu.to(dev), workspace=ws)
        torch.cuda.synchronize()
        codes_bytes = (m * k + 255) // 256 * 256
        assert_codes_equal(ws[: m * k].view(m, k), ws[codes_bytes: codes_bytes + 4 * m].view(torch.float32),
                           eqa, esa, f"{label} activation")
    else:
        out = lin(qa_gpu, sa_gpu)
        torch.cuda.synchronize()
    assert np.array_equal(lin.w_fp8.cpu().numpy(), qw), f"{label}: weight codes differ"
    assert np.array_equal(lin.w_scale.cpu().numpy().view(np.uint32), sw.view(np.uint32)), f"{label}: weight scales"
    bias_bits = _bias_bits(b_cpu)
    return assert_linear_close_rows(
        out, lambda r0, r1: ol.linear_ref_fp8(eqa[r0:r1], esa[r0:r1], qw, sw, bias_bits), label)


@pytest.mark.slow
@pytest.mark.parametrize("config", ["ffn_up", "ffn_down"])
def test_ffn_full_size(config):
    dev = require_gpu()
    cfg = make_config(config)
    layer, act = cfg["layers"][0]
    _full_size_linear(cfg["activations"][act], cfg["weights"][layer], cfg["biases"][layer], dev, config)


@pytest.mark.slow
def test_qkv_shared_quantisation_full_size():
    dev = require_gpu()
    cfg = make_config("qkv")
    hidden, enc = cfg["activations"]["hidden"], cfg["activations"]["encoder"]
    qh, sh = quant_rows(hidden.to(dev))  # quantised once, fed to all three projections
    qe, se = quant_rows(enc.to(dev))
    torch.cuda.synchronize()
    codes_h = cref.quant_rows(bf16_bits(hidden))
    codes_e = cref.quant_rows(bf16_bits(enc))
    assert_codes_equal(qh, sh, *codes_h, "qkv/hidden")
    assert_codes_equal(qe, se, *codes_e, "qkv/encoder")
    for layer in ("q", "k", "v"):
        w, b = cfg["weights"][layer], cfg["biases"][layer]
        lin = Fp8Linear(w.to(dev), b.to(dev))
        wq = cref.quant_rows(bf16_bits(w))
        _full_size_linear(hidden, w, b, dev, f"qkv/{layer}", qa_gpu=qh, sa_gpu=sh, lin=lin, oracle_codes=codes_h,
                          oracle_weight=wq)
        _full_size_linear(enc, w, b, dev, f"qkv/{layer}_enc", qa_gpu=qe, sa_gpu=se, lin=lin, oracle_codes=codes_e,
                          oracle_weight=wq)
        # the same plan on the bf16 input quantises it itself, bit for bit the same codes
        _full_size_linear(enc, w, b, dev, f"qkv/{layer}_enc bf16 input", lin=lin, oracle_codes=codes_e,
                          oracle_weight=wq)


@pytest.mark.parametrize("m", [1, 26, 32])
@pytest.mark.parametrize("config", ["ffn_up", "ffn_down"])
def test_few_tokens_through_the_ffn_weights(config, m):
    # a few tokens (the skinny weight stream, configuration 5) against the full FFN weights,
    # bf16 input: every code and every output element against the oracle
    dev = require_gpu()
    cfg = make_config(config)
    layer, act = cfg["layers"][0]
    w, b = cfg["weights"][layer], cfg["biases"][layer]
    lin = Fp8Linear(w.to(dev), b.to(dev))
    # 16-channel blocks of the 8192 FFN-up channels outnumber the CUs: the wide form
    assert lin.config(m)[0] == (SKINNY_WIDE if w.shape[0] // 16 > _cus(dev) else SKINNY)
    _full_size_linear(cfg["activations"][act][:m].contiguous(), w, b, dev, f"{config} m={m}", lin=lin)


@pytest.mark.parametrize("m", [1, 17, 26, 32])
def test_wide_skinny_form_matches_the_narrow_one(m):
    # configurations 5 and 7 (16 and 32 channels per workgroup) split k alike and sum in
    # the same order: bit-identical outputs, here with ragged n (the last 32-channel block
    # half valid) and ragged k, and both against the oracle element by element
    dev = require_gpu()
    n, k = 8208, 2064
    case = make_case(m, n, k, seed=71 + m, kind="outlier")
    qa, sa = oq.quant_rows(bf16_bits(case.a))
    qw, sw = _oracle_weight(case.w)
    ref = ol.linear_ref_fp8(qa, sa, qw, sw, _bias_bits(case.bias))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    args = (t(qa), t(sa), t(qw), t(sw), case.bias.to(dev))
    narrow = gemm_run_config(SKINNY, *args)
    wide = gemm_run_config(SKINNY_WIDE, *args)
    torch.cuda.synchronize()
    assert torch.equal(narrow.view(torch.int16), wide.view(torch.int16)), f"m={m}"
    assert_linear_close(wide, ref, f"wide skinny {m}x{n}x{k}")


@pytest.fixture(scope="module")
def dit_block():
    """The DiT-block config, each activation quantised once on the GPU (codes checked
    against the oracle by the tests that use them) and by the oracle."""
    dev = require_gpu()
    cfg = make_config("dit_block")
    gpu, oracle = {}, {}
    for name, a in cfg["activations"].items():
        gpu[name] = quant_rows(a.to(dev))
        oracle[name] = cref.quant_rows(bf16_bits(a))
    torch.cuda.synchronize()
    return cfg, gpu, oracle


@pytest.mark.slow
@pytest.mark.parametrize("layer", ["q", "k", "v", "out", "ffn_up", "ffn_down"])
def test_dit_block_full_size(dit_block, layer):
    dev = require_gpu()
    cfg, gpu, oracle = dit_block
    act = dict(cfg["layers"])[layer]
    qa, sa = gpu[act]
    assert_codes_equal(qa, sa, *oracle[act], f"dit/{act}")
    w, b = cfg["weights"][layer], cfg["biases"][layer]
    _full_size_linear(cfg["activations"][act], w, b, dev, f"dit/{layer}", qa_gpu=qa, sa_gpu=sa,
                      oracle_codes=oracle[act])


def test_selector_is_fixed_at_construction():
    dev = require_gpu()
    w = torch.zeros((2048, 8192), dtype=torch.bfloat16, device=dev)
    lin = Fp8Linear(w)
    seen = {m: lin.config(m) for m in (1, 26, 64, 65, 4096, 32760)}
    for m, (cid, tm, tn, wg) in seen.items():
        assert 0 <= cid < gemm_config_count()
        assert wg == ((m + tm - 1) // tm) * ((2048 + tn - 1) // tn)
        assert lin.config(m) == (cid, tm, tn, wg)  # same answer every call


def test_selector_picks_the_measured_best_at_the_page_shapes():
    # 256 x 256 tiles for FFN-up and the 32760-token layers, 128 x 256 for FFN-down, the
    # skinny weight stream for the 26-row encoder input: the fastest configuration at each
    # when timed on MI355X
    dev = require_gpu()
    if torch.cuda.get_device_properties(dev).multi_processor_count != 256:
        pytest.skip("the picks are measured for a 256-CU device")
    up = Fp8Linear(torch.zeros((8192, 2048), dtype=torch.bfloat16, device=dev))
    down = Fp8Linear(torch.zeros((2048, 8192), dtype=torch.bfloat16, device=dev))
    qkv = Fp8Linear(torch.zeros((2048, 2048), dtype=torch.bfloat16, device=dev))
    # the persistent form of the 256 x 256 tiles where every CU gets two or more tiles
    # and k is 2048 .. 4096; one workgroup per tile at k = 8192
    assert up.config(4096)[0] == PERSISTENT and up.config(32760)[0] == PERSISTENT
    assert down.config(4096)[0] == 2
    assert qkv.config(32760)[0] == PERSISTENT and down.config(32760)[0] == 0
    assert up.config(1024)[0] != PERSISTENT  # 128 tiles: one round
    assert qkv.config(26)[0] == SKINNY and down.config(26)[0] == SKINNY and up.config(26)[0] == SKINNY_WIDE
    assert qkv.config(64)[0] == 4


def test_errors_are_statuses_not_crashes():
    dev = require_gpu()
    w = torch.zeros((32, 64), dtype=torch.bfloat16, device=dev)
    lin = Fp8Linear(w)
    with pytest.raises(ValueError):
        lin(torch.zeros((4, 48), dtype=torch.bfloat16, device=dev))
    from fp8_w8a8_quantized_token_amd import _lib
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    a = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    out = torch.empty((4, 32), dtype=torch.bfloat16, device=dev)
    st = _lib.lib().fp8_linear_run(lin._plan, 4, ctypes.c_void_p(a.data_ptr()), _lib.A_BF16, None,
                                   ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), 16, None)
    assert st == _lib.ERR_WORKSPACE_TOO_SMALL
    st = _lib.lib().fp8_linear_run(lin._plan, 4, ctypes.c_void_p(a.data_ptr()), _lib.A_E4M3, None,
                                   ctypes.c_void_p(out.data_ptr()), None, 0, None)
    assert st == _lib.ERR_INVALID_ARG
