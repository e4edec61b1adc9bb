"""Python binding of libfp8w8a8: torch tensors in, torch tensors out.

Every function marshals arguments (device pointers, sizes, the current HIP stream)
and calls the C ABI; all arithmetic happens in the library's HIP kernels. torch is
used for device memory and streams only. Shapes follow include/fp8w8a8.h:
activations [m, k] (leading dims are flattened), weights [n, k] k-contiguous
(nn.Linear layout), outputs [m, n] bf16.
"""

import ctypes

import torch

from . import _lib
from ._lib import (A_BF16, A_E4M3, ACT_GELU_ERF, ACT_GELU_TANH, ACT_SILU, ACT_TABLE_BYTES, FMT_E4M3FN, FMT_E5M2,
                   check, lib)

ACTIVATIONS = {"gelu_erf": ACT_GELU_ERF, "gelu_tanh": ACT_GELU_TANH, "silu": ACT_SILU}


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require(t, dtypes, name, dims=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the HIP library is the only implementation)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(device, **tensors):
    """Every given tensor must live on the plan's device (the library launches there)."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the layer's weight on {device}")


def _codes(t):
    """View e4m3fn codes as uint8 (float8_e4m3fn tensors and uint8 tensors are accepted)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t


def quant_rows(x):
    """Per-token quantisation of bf16 x [..., k] -> (codes uint8 [m, k], scales fp32 [m])."""
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    _require(x2, (torch.bfloat16,), "x", 2)
    m, k = x2.shape
    q = torch.empty((m, k), dtype=torch.uint8, device=x2.device)
    s = torch.empty((m,), dtype=torch.float32, device=x2.device)
    if m == 0:  # no tokens (an empty tensor has no device address to pass)
        return q, s
    check(lib().fp8_quant_rows(_ptr(x2), m, k, _ptr(q), _ptr(s), _stream(x2)), "fp8_quant_rows")
    return q, s


def quant_weights_per_channel(w):
    """Per-output-channel quantisation of an nn.Linear weight bf16 [n, k] -> (codes [n, k], scales [n])."""
    _require(w, (torch.bfloat16,), "w", 2)
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    s = torch.empty((n,), dtype=torch.float32, device=w.device)
    check(lib().fp8_quant_weights_per_channel(_ptr(w), n, k, _ptr(q), _ptr(s), _stream(w)),
          "fp8_quant_weights_per_channel")
    return q, s


def act_table(kind, device=None):
    """Build the bf16 -> bf16 table of activation `kind` ("gelu_erf", "gelu_tanh", "silu") on a GPU.

    Returns an int16 tensor [65536] indexed by the input's bit pattern; pass it to
    act_rows / act_quant_rows on the same device and keep it alive while they run.
    """
    if kind not in ACTIVATIONS:
        raise ValueError(f"unknown activation {kind!r}; expected one of {sorted(ACTIVATIONS)}")
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    t = torch.empty(ACT_TABLE_BYTES // 2, dtype=torch.int16, device=device)
    with torch.cuda.device(t.device):
        check(lib().fp8_act_table_build(ACTIVATIONS[kind], _ptr(t), _stream(t)), "fp8_act_table_build")
    return t


def _check_table(table, x):
    _require(table, (torch.int16,), "table", 1)
    if table.numel() != ACT_TABLE_BYTES // 2 or table.device != x.device:
        raise ValueError("table must be the int16 [65536] tensor act_table built on x's device")


def act_rows(x, table, out=None):
    """The unfused producer: bf16 act(x) rounded to bf16, same shape as x."""
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    _require(x2, (torch.bfloat16,), "x", 2)
    _check_table(table, x2)
    m, k = x2.shape
    y = torch.empty((m, k), dtype=torch.bfloat16, device=x2.device) if out is None else out
    _require(y, (torch.bfloat16,), "out")
    if y.numel() != m * k:
        raise ValueError("out must hold as many elements as x")
    if m == 0:
        return y.view(x.shape)
    check(lib().fp8_act_rows(_ptr(x2), m, k, _ptr(table), _ptr(y), _stream(x2)), "fp8_act_rows")
    return y.view(x.shape)


def act_quant_rows(x, table, q=None, scale=None):
    """The fused producer: per-token FP8 (codes uint8 [m, k], scales fp32 [m]) of act(x) rounded to bf16."""
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    _require(x2, (torch.bfloat16,), "x", 2)
    _check_table(table, x2)
    m, k = x2.shape
    q = torch.empty((m, k), dtype=torch.uint8, device=x2.device) if q is None else _codes(q)
    s = torch.empty((m,), dtype=torch.float32, device=x2.device) if scale is None else scale
    _require(q, (torch.uint8,), "q")
    _require(s, (torch.float32,), "scale")
    if q.numel() != m * k or s.numel() != m:
        raise ValueError("q must hold m * k codes and scale m values")
    if m == 0:
        return q, s
    check(lib().fp8_act_quant_rows(_ptr(x2), m, k, _ptr(table), _ptr(q), _ptr(s), _stream(x2)),
          "fp8_act_quant_rows")
    return q, s


FORMATS = {"e4m3fn": FMT_E4M3FN, "e5m2": FMT_E5M2}


def quant_tensor(x, fmt="e4m3fn", workspace=None, form="auto"):
    """Per-tensor quantisation of a bf16 tensor -> (codes uint8 of x's shape, scale fp32 [1]).

    One scale for the whole tensor, s = amax / fmax (448 for e4m3fn, 57344 for e5m2):
    the state-dict conversion of the QuantizeFP8Format page. numel must be a multiple of 16.
    ``form`` picks the kernel form ("auto", "one_pass", "two_pass", "one_pass_no_wait";
    include/fp8w8a8.h, fp8_quant_tensor_form); every form gives the same result.
    """
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(FORMATS)}")
    if form not in _lib.TENSOR_FORMS:
        raise ValueError(f"unknown form {form!r}; expected one of {sorted(_lib.TENSOR_FORMS)}")
    xc = x.contiguous()
    _require(xc, (torch.bfloat16,), "x")
    if xc.numel() == 0:  # the converter treats an empty tensor as invalid input
        raise ValueError("empty tensor: there is nothing to quantise and no scale to derive")
    q = torch.empty(xc.shape, dtype=torch.uint8, device=xc.device)
    s = torch.empty((1,), dtype=torch.float32, device=xc.device)
    ws_bytes = lib().fp8_quant_tensor_workspace_bytes()
    if workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=xc.device)
    check(lib().fp8_quant_tensor_form(_lib.TENSOR_FORMS[form], _ptr(xc), xc.numel(), FORMATS[fmt], _ptr(q), _ptr(s),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(xc)),
          "fp8_quant_tensor_form")
    return q, s


def dequant_tensor(q, scale, fmt="e4m3fn"):
    """fp32 values dec(q) * scale of a per-tensor quantised tensor (q uint8 or float8, scale fp32 [1])."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(FORMATS)}")
    qc = q.contiguous()
    if qc.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        qc = qc.view(torch.uint8)
    _require(qc, (torch.uint8,), "q")
    _require(scale, (torch.float32,), "scale")
    out = torch.empty(qc.shape, dtype=torch.float32, device=qc.device)
    if qc.numel() == 0:
        return out
    check(lib().fp8_dequant_tensor(_ptr(qc), qc.numel(), FORMATS[fmt], _ptr(scale), _ptr(out), _stream(qc)),
          "fp8_dequant_tensor")
    return out


class Fp8Linear:
    """An FP8 W8A8 linear bound at construction (weight quantised once, GEMM config chosen once).

    Construction follows the HunyuanVideo1.5 retrospective (aigcage.com, section 3.3):
    the weight is quantised per output channel and kept in its [n, k] layout, and the
    library picks the kernel configuration from the weight shape and the device. The
    forward is narrow: a bf16 input is quantised per token and multiplied; an input that
    is already e4m3fn (with its per-token scale) goes straight to the GEMM (section 3.5).
    """

    def __init__(self, weight=None, bias=None, *, w_fp8=None, w_scale=None):
        if weight is not None:
            if w_fp8 is not None or w_scale is not None:
                raise ValueError("pass either a bf16 weight or (w_fp8, w_scale), not both")
            w_fp8, w_scale = quant_weights_per_channel(weight)
        if w_fp8 is None or w_scale is None:
            raise ValueError("Fp8Linear needs a bf16 weight or a pre-quantised (w_fp8, w_scale)")
        w_fp8 = _codes(w_fp8)
        _require(w_fp8, (torch.uint8,), "w_fp8", 2)
        _require(w_scale, (torch.float32,), "w_scale", 1)
        n, k = w_fp8.shape
        if w_scale.shape[0] != n:
            raise ValueError("w_scale must have one entry per output channel")
        if bias is not None:
            _require(bias, (torch.bfloat16,), "bias", 1)
            if bias.shape[0] != n:
                raise ValueError("bias must have one entry per output channel")
        self.w_fp8, self.w_scale, self.bias = w_fp8, w_scale, bias  # the plan borrows these
        self.n, self.k = n, k
        self.device = w_fp8.device
        plan = ctypes.c_void_p()
        check(lib().fp8_linear_create(self.device.index or 0, n, k, _ptr(w_fp8), _ptr(w_scale), _ptr(bias),
                                      ctypes.byref(plan)), "fp8_linear_create")
        self._plan = plan
        self._lib = lib()

    def __del__(self):
        plan = getattr(self, "_plan", None)
        if plan is not None and plan.value:
            self._lib.fp8_linear_destroy(plan)
            self._plan = None

    def config(self, m):
        """(config_id, tile_m, tile_n, workgroups) the plan launches for m activation rows."""
        cid, tm, tn, wg = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
        check(lib().fp8_linear_plan_config(self._plan, m, ctypes.byref(cid), ctypes.byref(tm), ctypes.byref(tn),
                                           ctypes.byref(wg)), "fp8_linear_plan_config")
        return cid.value, tm.value, tn.value, wg.value

    def workspace_bytes(self, m):
        return lib().fp8_linear_workspace_bytes(self._plan, m)

    def forward(self, x, x_scale=None, out=None, workspace=None):
        """out [..., n] bf16 from x [..., k] (bf16, or e4m3fn codes with x_scale [m])."""
        lead = x.shape[:-1]
        if x.shape[-1] != self.k:
            raise ValueError(f"input has {x.shape[-1]} features, the weight expects {self.k}")
        fp8_in = x.dtype in (torch.float8_e4m3fn, torch.uint8)
        x2 = _codes(x).reshape(-1, self.k).contiguous()
        m = x2.shape[0]
        if fp8_in:
            if x_scale is None:
                raise ValueError("an e4m3fn input needs its per-token scale")
            _require(x2, (torch.uint8,), "x", 2)
            _require(x_scale, (torch.float32,), "x_scale", 1)
            if x_scale.shape[0] != m:
                raise ValueError("x_scale must have one entry per token")
            kind, ws, ws_bytes = A_E4M3, None, 0
        else:
            _require(x2, (torch.bfloat16,), "x", 2)
            kind = A_BF16
            ws_bytes = self.workspace_bytes(m)
            if workspace is None:
                workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=x2.device)
            ws = workspace
        if out is None:
            out = torch.empty((m, self.n), dtype=torch.bfloat16, device=x2.device)
        else:
            _require(out, (torch.bfloat16,), "out")
            if out.numel() != m * self.n:
                raise ValueError("out has the wrong size")
        _on_device(self.device, x=x2, x_scale=x_scale if fp8_in else None, out=out, workspace=ws)
        if m == 0:  # nothing to compute (an empty tensor has no device address to pass)
            return out.reshape(*lead, self.n)
        check(lib().fp8_linear_run(self._plan, m, _ptr(x2), kind, _ptr(x_scale) if fp8_in else None, _ptr(out),
                                   _ptr(ws), ws_bytes if ws is None else ws.numel(), _stream(x2)),
              "fp8_linear_run")
        return out.reshape(*lead, self.n)

    __call__ = forward


def group_config(linears, m):
    """The GEMM configuration of the single launch linear_group makes for these layers at m
    tokens, or -1 when each layer runs its own GEMM (include/fp8w8a8.h,
    fp8_linear_group_config)."""
    linears = list(linears)
    if not 1 <= len(linears) <= _lib.MAX_GROUP:
        raise ValueError(f"a group takes 1..{_lib.MAX_GROUP} layers, got {len(linears)}")
    plans = (ctypes.c_void_p * len(linears))(*[lin._plan.value for lin in linears])
    cid = ctypes.c_int()
    check(lib().fp8_linear_group_config(plans, len(linears), m, ctypes.byref(cid)), "fp8_linear_group_config")
    return cid.value


def linear_group(linears, x, x_scale=None, outs=None, workspace=None):
    """Several Fp8Linear layers on one input: [out_i [..., n_i]], bit-identical to
    [lin(x) for lin in linears], with x quantised once.

    The retrospective (aigcage.com, section 3.4) feeds one set of hidden states into the
    Q, K and V projections; per-token quantisation of that input serves all of them, and
    when every layer takes the library's persistent GEMM form at this many tokens the
    products run as one launch (include/fp8w8a8.h, fp8_linear_run_group).
    """
    linears = list(linears)
    if not 1 <= len(linears) <= _lib.MAX_GROUP:
        raise ValueError(f"linear_group takes 1..{_lib.MAX_GROUP} layers, got {len(linears)}")
    k = linears[0].k
    if any(lin.k != k for lin in linears):
        raise ValueError("every layer of a group must take the same number of input features")
    if x.shape[-1] != k:
        raise ValueError(f"input has {x.shape[-1]} features, the weights expect {k}")
    lead = x.shape[:-1]
    fp8_in = x.dtype in (torch.float8_e4m3fn, torch.uint8)
    x2 = _codes(x).reshape(-1, k).contiguous()
    m = x2.shape[0]
    if fp8_in:
        if x_scale is None:
            raise ValueError("an e4m3fn input needs its per-token scale")
        _require(x2, (torch.uint8,), "x", 2)
        _require(x_scale, (torch.float32,), "x_scale", 1)
        if x_scale.shape[0] != m:
            raise ValueError("x_scale must have one entry per token")
        kind, ws, ws_bytes = A_E4M3, None, 0
    else:
        _require(x2, (torch.bfloat16,), "x", 2)
        kind = A_BF16
        ws_bytes = linears[0].workspace_bytes(m)
        if workspace is None:
            workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=x2.device)
        ws = workspace
    if outs is None:
        outs = [torch.empty((m, lin.n), dtype=torch.bfloat16, device=x2.device) for lin in linears]
    else:
        outs = list(outs)
        if len(outs) != len(linears):
            raise ValueError("one output per layer")
        for o, lin in zip(outs, linears):
            _require(o, (torch.bfloat16,), "out")
            if o.numel() != m * lin.n:
                raise ValueError("an output has the wrong size")
    dev = linears[0].device
    for i, lin in enumerate(linears):
        if lin.device != dev:
            raise ValueError(f"layer {i} is on {lin.device}, layer 0 on {dev}")
    _on_device(dev, x=x2, x_scale=x_scale if fp8_in else None, workspace=ws)
    for i, o in enumerate(outs):
        _on_device(dev, **{f"outs[{i}]": o})
    if m == 0:  # nothing to compute (an empty tensor has no device address to pass)
        return [o.reshape(*lead, lin.n) for o, lin in zip(outs, linears)]
    g = len(linears)
    plans = (ctypes.c_void_p * g)(*[lin._plan.value for lin in linears])
    optrs = (ctypes.c_void_p * g)(*[o.data_ptr() for o in outs])
    check(lib().fp8_linear_run_group(ctypes.cast(plans, ctypes.c_void_p), g, m, _ptr(x2), kind,
                                     _ptr(x_scale) if fp8_in else None, ctypes.cast(optrs, ctypes.c_void_p),
                                     _ptr(ws), ws_bytes if ws is None else ws.numel(), _stream(x2)),
          "fp8_linear_run_group")
    return [o.reshape(*lead, lin.n) for o, lin in zip(outs, linears)]


class Fp8WeightOnlyLinear:
    """An FP8 weight-only (W8A16) linear: e4m3fn weight with per-channel scales, bf16 activation.

    The FP8 weight-only pipeline of the LongCat avatar comparison page
    (longcat-avatar-compare.pages.dev, speed overview): the weight is quantised per
    output channel once at construction (or passed in as (w_fp8, w_scale)); the
    activation is used as it is, in bf16, and the product runs on the bf16 matrix cores.
    """

    def __init__(self, weight=None, bias=None, *, w_fp8=None, w_scale=None, fmt="e4m3fn"):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(FORMATS)}")
        if weight is not None:
            if w_fp8 is not None or w_scale is not None:
                raise ValueError("pass either a bf16 weight or (w_fp8, w_scale), not both")
            if fmt != "e4m3fn":
                raise ValueError("a bf16 weight is quantised per channel to e4m3fn; pass e5m2 codes as w_fp8")
            w_fp8, w_scale = quant_weights_per_channel(weight)
        if w_fp8 is None or w_scale is None:
            raise ValueError("Fp8WeightOnlyLinear needs a bf16 weight or a pre-quantised (w_fp8, w_scale)")
        if w_fp8.dtype == torch.float8_e5m2:
            w_fp8 = w_fp8.view(torch.uint8)
        w_fp8 = _codes(w_fp8)
        _require(w_fp8, (torch.uint8,), "w_fp8", 2)
        _require(w_scale, (torch.float32,), "w_scale", 1)
        n, k = w_fp8.shape
        if w_scale.numel() == 1 and n > 1:  # a per-tensor scale: repeat it per channel
            w_scale = w_scale.reshape(1).expand(n).contiguous()
        if w_scale.shape[0] != n:
            raise ValueError("w_scale must have one entry per output channel (or a single per-tensor entry)")
        if bias is not None:
            _require(bias, (torch.bfloat16,), "bias", 1)
            if bias.shape[0] != n:
                raise ValueError("bias must have one entry per output channel")
        self.w_fp8, self.w_scale, self.bias = w_fp8, w_scale, bias  # the plan borrows these
        self.n, self.k, self.fmt = n, k, fmt
        self.device = w_fp8.device
        plan = ctypes.c_void_p()
        check(lib().fp8_w8a16_create(self.device.index or 0, n, k, FORMATS[fmt], _ptr(w_fp8), _ptr(w_scale),
                                     _ptr(bias), ctypes.byref(plan)), "fp8_w8a16_create")
        self._plan = plan
        self._lib = lib()

    def __del__(self):
        plan = getattr(self, "_plan", None)
        if plan is not None and plan.value:
            self._lib.fp8_w8a16_destroy(plan)
            self._plan = None

    def config(self, m):
        """(config_id, tile_m, tile_n, workgroups) the plan launches for m activation rows."""
        cid, tm, tn, wg = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
        check(lib().fp8_w8a16_plan_config(self._plan, m, ctypes.byref(cid), ctypes.byref(tm), ctypes.byref(tn),
                                          ctypes.byref(wg)), "fp8_w8a16_plan_config")
        return cid.value, tm.value, tn.value, wg.value

    def forward(self, x, out=None):
        """out [..., n] bf16 from a bf16 x [..., k]."""
        lead = x.shape[:-1]
        if x.shape[-1] != self.k:
            raise ValueError(f"input has {x.shape[-1]} features, the weight expects {self.k}")
        x2 = x.reshape(-1, self.k).contiguous()
        _require(x2, (torch.bfloat16,), "x", 2)
        m = x2.shape[0]
        if out is None:
            out = torch.empty((m, self.n), dtype=torch.bfloat16, device=x2.device)
        else:
            _require(out, (torch.bfloat16,), "out")
            if out.numel() != m * self.n:
                raise ValueError("out has the wrong size")
        _on_device(self.device, x=x2, out=out)
        if m == 0:  # nothing to compute (an empty tensor has no device address to pass)
            return out.reshape(*lead, self.n)
        check(lib().fp8_w8a16_run(self._plan, m, _ptr(x2), _ptr(out), _stream(x2)), "fp8_w8a16_run")
        return out.reshape(*lead, self.n)

    __call__ = forward


def w8a16_config_count():
    return lib().fp8_w8a16_config_count()


def w8a16_run_config(config_id, a, w_fp8, w_scale, bias=None, out=None, fmt="e4m3fn"):
    """Test hook: run W8A16 configuration `config_id` directly (every configuration is held to parity)."""
    if w_fp8.dtype == torch.float8_e5m2:
        w_fp8 = w_fp8.view(torch.uint8)
    w_fp8 = _codes(w_fp8)
    _require(a, (torch.bfloat16,), "a", 2)
    _require(w_fp8, (torch.uint8,), "w_fp8", 2)
    m, k = a.shape
    n = w_fp8.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    check(lib().fp8_w8a16_run_config(config_id, FORMATS[fmt], m, n, k, _ptr(a), _ptr(w_fp8), _ptr(w_scale),
                                     _ptr(bias), _ptr(out), _stream(a)), "fp8_w8a16_run_config")
    return out


def linear(a, w_fp8, w_scale, bias=None, a_scale=None):
    """One-shot FP8 linear (creates, runs and frees a plan): out [m, n] bf16."""
    return Fp8Linear(w_fp8=w_fp8, w_scale=w_scale, bias=bias).forward(a, a_scale)


def gemm_config_count():
    return lib().fp8_gemm_config_count()


def gemm_run_config(config_id, qa, a_scale, w_fp8, w_scale, bias=None, out=None):
    """Launch one named GEMM configuration on already-quantised operands (tests)."""
    qa, w_fp8 = _codes(qa), _codes(w_fp8)
    _require(qa, (torch.uint8,), "qa", 2)
    _require(w_fp8, (torch.uint8,), "w_fp8", 2)
    _require(a_scale, (torch.float32,), "a_scale", 1)
    _require(w_scale, (torch.float32,), "w_scale", 1)
    m, k = qa.shape
    n = w_fp8.shape[0]
    if w_fp8.shape[1] != k or a_scale.shape[0] != m or w_scale.shape[0] != n:
        raise ValueError("operand shapes do not agree")
    if bias is not None:
        _require(bias, (torch.bfloat16,), "bias", 1)
        if bias.shape[0] != n:
            raise ValueError("bias must have n entries")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=qa.device)
    check(lib().fp8_gemm_run_config(config_id, m, n, k, _ptr(qa), _ptr(a_scale), _ptr(w_fp8), _ptr(w_scale),
                                    _ptr(bias), _ptr(out), _stream(qa)), "fp8_gemm_run_config")
    return out


def quant_gemm(a, w_fp8, w_scale, bias=None, out=None, workspace=None):
    """Per-token quantisation and the FP8 GEMM in one launch.

    Returns (out [m, n] bf16, codes [m, k] uint8, scales [m] fp32); codes and scales
    are views of the workspace that the launch wrote them to.
    """
    a2 = a.reshape(-1, a.shape[-1]) if a.dim() != 2 else a
    _require(a2, (torch.bfloat16,), "a", 2)
    w_fp8 = _codes(w_fp8)
    _require(w_fp8, (torch.uint8,), "w_fp8", 2)
    _require(w_scale, (torch.float32,), "w_scale", 1)
    m, k = a2.shape
    n = w_fp8.shape[0]
    if w_fp8.shape[1] != k or w_scale.shape[0] != n:
        raise ValueError("operand shapes do not agree")
    if bias is not None:
        _require(bias, (torch.bfloat16,), "bias", 1)
        if bias.shape[0] != n:
            raise ValueError("bias must have n entries")
    ws_bytes = lib().fp8_quant_gemm_workspace_bytes(m, k)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=a2.device)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a2.device)
    check(lib().fp8_quant_gemm(m, n, k, _ptr(a2), _ptr(w_fp8), _ptr(w_scale), _ptr(bias), _ptr(out),
                               _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(a2)),
          "fp8_quant_gemm")
    codes_bytes = (m * k + 255) // 256 * 256
    codes = workspace[: m * k].view(m, k)
    scales = workspace[codes_bytes: codes_bytes + 4 * m].view(torch.float32)
    return out, codes, scales


__all__ = ["quant_rows", "quant_weights_per_channel", "Fp8Linear", "linear", "linear_group", "gemm_config_count",
           "gemm_run_config", "quant_gemm", "A_BF16", "A_E4M3", "_lib"]
