"""Seeded synthetic linears shaped like the HunyuanVideo1.5 DiT layers the pages describe.

Shapes (HunyuanVideo1.5 BF16->FP8 retrospective, aigcage.com/blog/hunyuanvideo-fp8):
  FFN-up    M=4096,  N=8192, K=2048   (section 3.2)
  FFN-down  M=4096,  N=2048, K=8192   (section 3.2)
  Q/K/V     hidden_states [32760, 2048], encoder_hidden_states [26, 2048],
            three separate [2048, 2048] projections sharing one quantisation (section 3.4)
The pages run trained weights on real prompts; these synthetic tensors stand in
for them (no weights or data are available or needed):

  activation "outlier": N(0, 1) with a fixed set of channels (columns) scaled x50,
                        the same set for every row; round(1% of K) channels unless
                        a config fixes the count
  activation "gelu":    exact-erf GELU of N(0, 1), the FFN-down input
  weight:               N(0, 1/sqrt(K)) in bf16, quantised per output channel by the
                        code under test (not here)
  bias:                 N(0, 0.1) in bf16

Every tensor comes from its own stream numpy.random.default_rng([seed, config_id,
tensor_id]) in float32 and is rounded once to bf16 (round-to-nearest-even, torch's
CPU cast). Nothing here quantises, multiplies or applies an epilogue.
"""

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

# Activation spec: (rows, cols, kind, outlier_count or None, outlier_group)
# Layer spec: (layer_name, activation_name, N)
CONFIGS = {
    "tiny": {
        "id": 1,
        "activations": {"a": (64, 256, "outlier", 2, "a")},
        "layers": [("linear", "a", 128)],
    },
    "ffn_up": {
        "id": 2,
        "activations": {"a": (4096, 2048, "outlier", None, "a")},
        "layers": [("ffn_up", "a", 8192)],
    },
    "ffn_down": {
        "id": 3,
        "activations": {"a": (4096, 8192, "gelu", None, None)},
        "layers": [("ffn_down", "a", 2048)],
    },
    "qkv": {
        "id": 4,
        "activations": {
            "hidden": (32760, 2048, "outlier", None, "hidden"),
            "encoder": (26, 2048, "outlier", None, "hidden"),
        },
        "layers": [
            ("q", "hidden", 2048), ("k", "hidden", 2048), ("v", "hidden", 2048),
            ("q_enc", "encoder", 2048), ("k_enc", "encoder", 2048), ("v_enc", "encoder", 2048),
        ],
        # the encoder projections reuse the hidden projections' weights and biases
        "weight_alias": {"q_enc": "q", "k_enc": "k", "v_enc": "v"},
    },
    "dit_block": {
        "id": 5,
        "activations": {
            "x_qkv": (32760, 2048, "outlier", None, "x_qkv"),
            "x_out": (32760, 2048, "outlier", None, "x_out"),
            "x_up": (32760, 2048, "outlier", None, "x_up"),
            "x_down": (32760, 8192, "outlier", None, "x_down"),
        },
        "layers": [
            ("q", "x_qkv", 2048), ("k", "x_qkv", 2048), ("v", "x_qkv", 2048),
            ("out", "x_out", 2048), ("ffn_up", "x_up", 8192), ("ffn_down", "x_down", 2048),
        ],
    },
}


def _rng(seed: int, config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, config_id, tensor_id])


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a CPU bf16 tensor (a view, no arithmetic)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def outlier_channels(seed: int, config_id: int, group_id: int, cols: int, count: Optional[int]) -> np.ndarray:
    n = int(round(0.01 * cols)) if count is None else int(count)
    n = max(0, min(n, cols))
    return np.sort(_rng(seed, config_id, 1000 + group_id).choice(cols, size=n, replace=False))


def activation(seed: int, config_id: int, tensor_id: int, rows: int, cols: int, kind: str,
               channels: Optional[np.ndarray] = None) -> torch.Tensor:
    z = _rng(seed, config_id, tensor_id).standard_normal((rows, cols), dtype=np.float32)
    if kind == "outlier":
        if channels is not None and len(channels):
            z[:, channels] *= np.float32(50.0)
        return _to_bf16(z)
    if kind == "gelu":
        return torch.nn.functional.gelu(torch.from_numpy(z)).to(torch.bfloat16)
    if kind == "normal":
        return _to_bf16(z)
    raise ValueError(f"unknown activation kind {kind!r}")


def weight(seed: int, config_id: int, tensor_id: int, n: int, k: int) -> torch.Tensor:
    z = _rng(seed, config_id, tensor_id).standard_normal((n, k), dtype=np.float32)
    return _to_bf16(z * np.float32(1.0 / np.sqrt(k)))


def bias(seed: int, config_id: int, tensor_id: int, n: int) -> torch.Tensor:
    z = _rng(seed, config_id, tensor_id).standard_normal((n,), dtype=np.float32)
    return _to_bf16(z * np.float32(0.1))


@dataclass
class LinearCase:
    """One linear's inputs: activation bf16 [M, K], weight bf16 [N, K], bias bf16 [N] or None."""
    name: str
    a: torch.Tensor
    w: torch.Tensor
    bias: Optional[torch.Tensor]
    meta: Dict = field(default_factory=dict)

    @property
    def shape(self) -> Tuple[int, int, int]:
        return self.a.shape[0], self.w.shape[0], self.a.shape[1]


def make_case(m: int, n: int, k: int, seed: int = 0, kind: str = "outlier", with_bias: bool = True,
              outliers: Optional[int] = None, case_id: int = 99) -> LinearCase:
    """A single synthetic linear of any shape (parity tests, edge cases)."""
    ch = outlier_channels(seed, case_id, 0, k, outliers) if kind == "outlier" else None
    a = activation(seed, case_id, 0, m, k, kind, ch)
    w = weight(seed, case_id, 1, n, k)
    b = bias(seed, case_id, 2, n) if with_bias else None
    return LinearCase(f"case_{m}x{n}x{k}", a, w, b, {"outlier_channels": ch})


def layer_specs(config: str) -> List[Tuple[str, str, int, int, int]]:
    """[(layer, activation, M, N, K)] for a named config, without drawing any tensor."""
    spec = CONFIGS[config]
    out = []
    for layer, act, n in spec["layers"]:
        rows, cols = spec["activations"][act][:2]
        out.append((layer, act, rows, n, cols))
    return out


def make_config(config: str, seed: int = 0, activations=None):
    """Draw a named config.

    Returns {"activations": {name: bf16 [M, K]}, "weights": {layer: bf16 [N, K]},
    "biases": {layer: bf16 [N]}, "layers": [(layer, activation_name)]}. Layers listed
    in the config's weight_alias share the aliased layer's weight and bias tensors.
    ``activations`` may restrict which activation tensors are drawn.
    """
    spec = CONFIGS[config]
    cid = spec["id"]
    acts = {}
    groups = {}
    for i, (name, (rows, cols, kind, count, group)) in enumerate(spec["activations"].items()):
        if activations is not None and name not in activations:
            continue
        ch = None
        if kind == "outlier":
            gid = list(spec["activations"]).index(group)
            key = (group, cols)
            if key not in groups:
                groups[key] = outlier_channels(seed, cid, gid, cols, count)
            ch = groups[key]
        acts[name] = activation(seed, cid, i, rows, cols, kind, ch)
    weights, biases = {}, {}
    alias = spec.get("weight_alias", {})
    for j, (layer, act, n) in enumerate(spec["layers"]):
        if layer in alias:
            continue
        k = spec["activations"][act][1]
        weights[layer] = weight(seed, cid, 100 + j, n, k)
        biases[layer] = bias(seed, cid, 200 + j, n)
    for layer, target in alias.items():
        weights[layer] = weights[target]
        biases[layer] = biases[target]
    return {
        "activations": acts,
        "weights": weights,
        "biases": biases,
        "layers": [(layer, act) for layer, act, _ in spec["layers"]],
        "outlier_channels": {g: c for (g, _), c in groups.items()},
    }
