"""Int8Linear: an inference linear layer holding an int8 weight (the CB/SCB pair).

[HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit Matrix
Multiplication for transformers at scale ...", section "Usage": the int8
linear module in inference mode (has_fp16_weights=False) quantizes its fp16
weight once, when the weight is placed on the GPU, keeps the int8 codes (CB)
and the per-output-row absmax (SCB), takes fp16 input, and a second
quantization of the same module is an error (section "accelerate is all you
need").
"""

import torch

from . import ops


class Int8Linear(torch.nn.Module):
    def __init__(self, in_features, out_features, bias=False, threshold=ops.DEFAULT_THRESHOLD,
                 device="cuda"):
        super().__init__()
        if in_features % 16 != 0:
            raise ValueError("in_features must be a multiple of 16")
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.threshold = float(threshold)
        self.register_buffer("Wq", torch.zeros((out_features, in_features), dtype=torch.int8,
                                               device=device))
        self.register_buffer("sw", torch.zeros((out_features,), dtype=torch.float32,
                                               device=device))
        self.bias = (torch.zeros((out_features,), dtype=torch.float16, device=device)
                     if bias else None)
        self._quantized = False
        self._ws = None

    @property
    def CB(self):
        return self.Wq

    @property
    def SCB(self):
        return self.sw

    @property
    def quantized(self):
        return self._quantized

    @torch.no_grad()
    def quantize_(self, weight, bias=None):
        """Quantize an fp16 weight [out, in] once. Raises if already quantized."""
        if self._quantized:
            raise RuntimeError("weight is already quantized; quantizing twice is not allowed")
        if weight.shape != (self.out_features, self.in_features):
            raise ValueError("weight shape %s != (%d, %d)" % (tuple(weight.shape),
                                                            self.out_features, self.in_features))
        W = weight.to(device=self.Wq.device, dtype=torch.float16).contiguous()
        ops.int8_quantize_colwise_weight(W, self.Wq, self.sw)
        if bias is not None:
            if self.bias is None:
                raise ValueError("module was built without bias")
            self.bias.copy_(bias.to(torch.float16))
        self._quantized = True
        return self

    def forward(self, x):
        if not self._quantized:
            raise RuntimeError("quantize_() the weight before forward")
        if x.dtype != torch.float16:
            raise TypeError("input must be fp16")
        x = x.contiguous()
        M = x.numel() // self.in_features
        need = ops.workspace_bytes(M, self.in_features, self.out_features)
        if self._ws is None or self._ws.numel() < need or self._ws.device != x.device:
            self._ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
        return ops.linear_int8_mixed(x, self.Wq, self.sw, self.bias, self.threshold, self._ws)

    def extra_repr(self):
        return "in_features=%d, out_features=%d, threshold=%g, quantized=%s" % (
            self.in_features, self.out_features, self.threshold, self._quantized)
