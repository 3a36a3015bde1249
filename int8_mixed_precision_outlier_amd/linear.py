"""A torch module over the C-ABI: an fp16 linear layer whose forward pass is
the LLM.int8() decomposed matmul.

The layer of the brain.gartu.xyz page's practical example ("Exemple
pratique") replaces an nn.Linear (with bias) by an int8 layer with
threshold 6.0 whose forward pass does the mixed-precision decomposition by
itself; this is that layer for this library.  Weights are quantized once,
when the module is built.  All arithmetic runs in the HIP library.
"""
from __future__ import annotations

import torch

from . import (build_outlier_cache, mixed_matmul, mixed_matmul_cached, quantize_weight,
               workspace_size)


class Int8MixedLinear(torch.nn.Module):
    """y = x . W^T + b for fp16 x [..., in_features] on the GPU.

    Buffers: w_i8 (packed int8 weights), w_absmax (fp32 [out]), the source
    of the outlier rows -- either w_kn (the fp16 weights as [in, out]) or,
    with `outlier_dims` given, cache (the fp16 rows of those static dims
    only; dims outside it fall back to dequantized int8 rows and are
    flagged) -- and bias (fp16 [out] or None).  `threshold` is the outlier
    threshold alpha; `n_cap` bounds the outlier columns per call
    (in_features, always enough, by default).
    """

    def __init__(self, weight: torch.Tensor, bias: torch.Tensor | None = None,
                 threshold: float = 6.0, n_cap: int | None = None, outlier_dims=None):
        super().__init__()
        if weight.dim() != 2 or weight.device.type != "cuda":
            raise TypeError("weight must be a 2-D CUDA tensor [out_features, in_features]")
        out_features, in_features = weight.shape
        w_kn = weight.detach().to(torch.float16).t().contiguous()
        w_i8, w_absmax = quantize_weight(w_kn)
        self.register_buffer("w_i8", w_i8)
        self.register_buffer("w_absmax", w_absmax)
        if outlier_dims is None:
            self.register_buffer("w_kn", w_kn)
            self.register_buffer("cache", None)
        else:
            # memory-lean: only the fp16 rows of the static outlier dims stay
            self.register_buffer("w_kn", None)
            self.register_buffer("cache", build_outlier_cache(w_kn, outlier_dims))
            del w_kn
        if bias is not None:
            bias = bias.detach().to(device=weight.device, dtype=torch.float16).contiguous()
        self.register_buffer("bias", bias)
        self.in_features = in_features
        self.out_features = out_features
        self.threshold = float(threshold)
        self.n_cap = in_features if n_cap is None else int(n_cap)

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, threshold: float = 6.0,
                    n_cap: int | None = None, outlier_dims=None) -> "Int8MixedLinear":
        return cls(linear.weight, linear.bias, threshold, n_cap, outlier_dims)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, threshold={self.threshold}, n_cap={self.n_cap}")

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dimension {self.in_features}, got {x.shape[-1]}")
        x2 = x.reshape(-1, self.in_features)
        if x2.dtype != torch.float16 or not x2.is_contiguous():
            x2 = x2.to(torch.float16).contiguous()
        M = x2.shape[0]
        # the caching allocator makes the per-call workspace cheap and
        # keeps concurrent calls on different streams apart
        ws = torch.empty(workspace_size(M, self.in_features, self.out_features, self.n_cap),
                         dtype=torch.uint8, device=x2.device)
        if self.cache is None:
            y = mixed_matmul(x2, self.w_i8, self.w_absmax, self.w_kn, alpha=self.threshold,
                             bias=self.bias, n_cap=self.n_cap, workspace=ws)
        else:
            y = mixed_matmul_cached(x2, self.w_i8, self.w_absmax, self.cache,
                                    alpha=self.threshold, bias=self.bias, n_cap=self.n_cap,
                                    workspace=ws)
        return y.reshape(*x.shape[:-1], self.out_features)


__all__ = ["Int8MixedLinear"]
