"""Int4Linear: a torch module whose forward is one fused INT4 linear layer.

The engine page ("Build a Blockwise INT4 Inference Engine", Step 4, the Python
runtime) keeps a layer's weights as packed INT4 codes with per-group scales
and zero points and runs the layer as x @ W_dq.T + b followed by a ReLU, with a
two-layer model as its end-to-end example. Its roadmap asks for the quantized
weights to be persisted together with their metadata and checksums. This
module is that layer on the GPU:

* buffers: ``packed`` uint8 [out, ceil(in/2)], ``scales`` float16 [out, G],
  ``zeros`` uint8 [out, G] for affine codes, ``bias`` float32 [out] (optional);
* ``load_weight(w)`` quantizes a float32 weight on the GPU (int4_quantize or
  int4_quantize_affine);
* ``forward(x)`` is one ``int4_linear`` launch: bias and ReLU are applied in
  the kernel's store and the output is written as float16 or float32, so a
  stack of layers passes float16 activations from one to the next with no
  other GPU work.

``save_int4`` / ``load_int4`` write and read every Int4Linear of a module as a
safetensors file (no pickling): the buffers under their state_dict names, and
per layer its configuration and a SHA-256 of each buffer in the metadata,
checked on load.

Nothing here computes on the CPU: the forward raises if its tensors are not on
the GPU, like the binding underneath.
"""
from __future__ import annotations

import hashlib
import json

import torch

from . import (dequantize_int4, int4_linear, num_groups, quantize_int4,
               quantize_int4_affine)

FORMAT = "int4dq-linear/1"
_DTYPES = {"float16": torch.float16, "float32": torch.float32}


class Int4Linear(torch.nn.Module):
    """y = act(x @ dequantize(W).T + b) with W held as INT4 group codes.

    in_features, out_features: K and N of the layer; group: codes per scale
    group along K; bias: whether the layer has a bias; affine: unsigned codes
    with zero points instead of symmetric codes; relu: apply ReLU in the
    store; out_dtype: float16 or float32 output."""

    def __init__(self, in_features: int, out_features: int, group: int = 128, bias: bool = True,
                 affine: bool = False, relu: bool = False, out_dtype: torch.dtype = torch.float32,
                 device=None):
        super().__init__()
        if in_features < 1 or out_features < 1 or group < 1:
            raise ValueError("in_features, out_features and group must be >= 1")
        if out_dtype not in (torch.float16, torch.float32):
            raise ValueError(f"out_dtype must be float16 or float32 (got {out_dtype})")
        self.in_features, self.out_features, self.group = in_features, out_features, group
        self.affine, self.relu, self.out_dtype = affine, relu, out_dtype
        G = num_groups(in_features, group)
        self.register_buffer("packed", torch.zeros((out_features, (in_features + 1) // 2),
                                                   dtype=torch.uint8, device=device))
        self.register_buffer("scales", torch.zeros((out_features, G), dtype=torch.float16, device=device))
        self.register_buffer("zeros", torch.zeros((out_features, G), dtype=torch.uint8, device=device)
                             if affine else None)
        self.register_buffer("bias", torch.zeros(out_features, dtype=torch.float32, device=device)
                             if bias else None)

    # ------------------------------------------------------------ weights
    @torch.no_grad()
    def load_weight(self, weight: torch.Tensor, bias: torch.Tensor | None = None) -> "Int4Linear":
        """Quantize a float32 [out, in] GPU weight into the buffers (and copy the bias)."""
        if tuple(weight.shape) != (self.out_features, self.in_features):
            raise ValueError(f"weight shape {tuple(weight.shape)} != {(self.out_features, self.in_features)}")
        w = weight.contiguous()
        if self.affine:
            p, s, z, _ = quantize_int4_affine(w, self.group)
            self.zeros.copy_(z)
        else:
            p, s, _ = quantize_int4(w, self.group)
        self.packed.copy_(p)
        self.scales.copy_(s)
        if bias is not None:
            if self.bias is None:
                raise ValueError("this layer was built without a bias")
            self.bias.copy_(bias.to(torch.float32))
        return self

    @classmethod
    def from_float(cls, weight: torch.Tensor, bias: torch.Tensor | None = None, group: int = 128,
                   affine: bool = False, relu: bool = False,
                   out_dtype: torch.dtype = torch.float32) -> "Int4Linear":
        """A layer quantized from a float32 [out, in] GPU weight."""
        out_f, in_f = weight.shape
        layer = cls(in_f, out_f, group, bias is not None, affine, relu, out_dtype, weight.device)
        return layer.load_weight(weight, bias)

    def dequantized_weight(self, dtype: torch.dtype = torch.float32) -> torch.Tensor:
        """w_hat [out, in] as the kernels see it (int4_dequantize)."""
        return dequantize_int4(self.packed, self.scales, self.in_features, self.group, dtype,
                               zeros=self.zeros)

    # ------------------------------------------------------------ forward
    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"x has {x.shape[-1]} features, the layer takes {self.in_features}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if not x2.is_contiguous():
            raise ValueError("x must be contiguous in its last dimension")
        y = int4_linear(x2, self.packed, self.scales, self.in_features, self.group, zeros=self.zeros,
                        bias=self.bias, relu=self.relu, out_dtype=self.out_dtype)
        return y.reshape(*lead, self.out_features)

    def config(self) -> dict:
        return {"in_features": self.in_features, "out_features": self.out_features,
                "group": self.group, "bias": self.bias is not None, "affine": self.affine,
                "relu": self.relu, "out_dtype": str(self.out_dtype).replace("torch.", "")}

    def extra_repr(self) -> str:
        c = self.config()
        return ", ".join(f"{k}={v}" for k, v in c.items())


# ---------------------------------------------------------------- persistence

def _digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()).hexdigest()


def _layers(module: torch.nn.Module):
    if isinstance(module, Int4Linear):
        return [("", module)]
    return [(n, m) for n, m in module.named_modules() if isinstance(m, Int4Linear)]


def save_int4(path: str, module: torch.nn.Module) -> None:
    """Write every Int4Linear of ``module`` (or the layer itself) to a
    safetensors file: buffers under ``<layer>.<buffer>``, and in the metadata
    the format tag, each layer's configuration and each buffer's SHA-256."""
    from safetensors.torch import save_file
    tensors, meta = {}, {"format": FORMAT}
    layers = _layers(module)
    if not layers:
        raise ValueError("the module holds no Int4Linear")
    for name, layer in layers:
        key = name or "layer"
        cfg = layer.config()
        digests = {}
        for b in ("packed", "scales", "zeros", "bias"):
            t = getattr(layer, b)
            if t is None:
                continue
            tensors[f"{key}.{b}"] = t.detach().contiguous().cpu()
            digests[b] = _digest(t)
        cfg["sha256"] = digests
        meta[f"layer:{key}"] = json.dumps(cfg, sort_keys=True)
    save_file(tensors, path, metadata=meta)


def load_int4(path: str, module: torch.nn.Module | None = None, device="cuda"):
    """Read a file written by save_int4. With ``module``: fill its Int4Linear
    layers (same names and configurations) in place and return it. Without:
    return {name: Int4Linear} built from the file. Every buffer's SHA-256 is
    checked; a mismatch, a missing layer or a configuration that differs
    raises ValueError."""
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        meta = f.metadata() or {}
        if meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not an {FORMAT} file")
        cfgs = {k[len("layer:"):]: json.loads(v) for k, v in meta.items() if k.startswith("layer:")}
        data = {k: f.get_tensor(k) for k in f.keys()}

    def fill(key, layer):
        cfg = dict(cfgs[key])
        digests = cfg.pop("sha256")
        if cfg != layer.config():
            raise ValueError(f"{path}: layer {key} configuration {cfg} != {layer.config()}")
        for b, h in digests.items():
            t = data[f"{key}.{b}"]
            if _digest(t) != h:
                raise ValueError(f"{path}: checksum mismatch in {key}.{b}")
            getattr(layer, b).copy_(t)

    if module is not None:
        for name, layer in _layers(module):
            key = name or "layer"
            if key not in cfgs:
                raise ValueError(f"{path}: no layer {key}")
            fill(key, layer)
        return module
    out = {}
    for key, cfg in cfgs.items():
        layer = Int4Linear(cfg["in_features"], cfg["out_features"], cfg["group"], cfg["bias"],
                           cfg["affine"], cfg["relu"], _DTYPES[cfg["out_dtype"]], device)
        fill(key, layer)
        out[key] = layer
    return out
