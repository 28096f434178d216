"""Int8Linear: the LLM.int8() linear layer in its two module modes.

[HF-blog] Hugging Face blog "A Gentle Introduction to 8-bit Matrix
Multiplication for transformers at scale ...", section "Usage":

* has_fp16_weights=False (inference): the module quantizes its fp16 weight
  once, when the weight is placed on the GPU, keeps the int8 codes (CB) and
  the per-output-row absmax (SCB), takes fp16 input, and a second
  quantization of the same module is an error (section "accelerate is all you
  need"). The outlier matmul uses weights recovered as CB * SCB / 127.
* has_fp16_weights=True (the default of the pages' module, meant for mixed
  Int8/FP16 training): the module keeps W in fp16; its int8 codes are those of
  the current W, and the outlier matmul uses W's own fp16 columns.
"""

import torch

from . import ops


class Int8Linear(torch.nn.Module):
    def __init__(self, in_features, out_features, bias=False, threshold=ops.DEFAULT_THRESHOLD,
                 has_fp16_weights=False, device="cuda"):
        super().__init__()
        if in_features % 16 != 0:
            raise ValueError("in_features must be a multiple of 16")
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.threshold = float(threshold)
        self.has_fp16_weights = bool(has_fp16_weights)
        self.register_buffer("Wq", torch.zeros((out_features, in_features), dtype=torch.int8,
                                               device=device))
        self.register_buffer("sw", torch.zeros((out_features,), dtype=torch.float32,
                                               device=device))
        self.register_buffer("weight", torch.zeros((out_features, in_features),
                                                   dtype=torch.float16, device=device)
                             if self.has_fp16_weights else None)
        self.bias = (torch.zeros((out_features,), dtype=torch.float16, device=device)
                     if bias else None)
        # fp16-weight mode: re-quantize W at every call (its codes follow W
        # as it changes); set False to re-quantize only after set_weight_.
        self.requantize_every_call = True
        self._quantized = False     # int8 mode: weight quantized; fp16 mode: weight set
        self._codes_current = False
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

    def _set_bias(self, bias):
        if bias is not None:
            if self.bias is None:
                raise ValueError("module was built without bias")
            self.bias.copy_(bias.to(torch.float16))

    def _check_shape(self, weight):
        if weight.shape != (self.out_features, self.in_features):
            raise ValueError("weight shape %s != (%d, %d)" % (tuple(weight.shape),
                                                            self.out_features, self.in_features))

    @torch.no_grad()
    def quantize_(self, weight, bias=None):
        """int8 mode: quantize an fp16 weight [out, in] once. Raises if already
        quantized, and in the fp16-weight mode (use set_weight_)."""
        if self.has_fp16_weights:
            raise RuntimeError("has_fp16_weights=True keeps the fp16 weight: use set_weight_")
        if self._quantized:
            raise RuntimeError("weight is already quantized; quantizing twice is not allowed")
        self._check_shape(weight)
        W = weight.to(device=self.Wq.device, dtype=torch.float16).contiguous()
        ops.int8_quantize_colwise_weight(W, self.Wq, self.sw)
        self._set_bias(bias)
        self._quantized = True
        return self

    @torch.no_grad()
    def set_weight_(self, weight, bias=None):
        """fp16-weight mode: store (or replace) the fp16 weight [out, in]."""
        if not self.has_fp16_weights:
            raise RuntimeError("has_fp16_weights=False quantizes once: use quantize_")
        self._check_shape(weight)
        self.weight.copy_(weight.to(device=self.weight.device, dtype=torch.float16))
        self._set_bias(bias)
        self._quantized = True
        self._codes_current = False
        return self

    def forward(self, x):
        if not self._quantized:
            raise RuntimeError("quantize_() (or set_weight_()) the weight before forward")
        if x.dtype != torch.float16:
            raise TypeError("input must be fp16")
        x = x.contiguous()
        M = x.numel() // self.in_features
        need = ops.workspace_bytes(M, self.in_features, self.out_features)
        if self._ws is None or self._ws.numel() < need or self._ws.device != x.device:
            self._ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
        if not self.has_fp16_weights:
            return ops.linear_int8_mixed(x, self.Wq, self.sw, self.bias, self.threshold, self._ws)
        requantize = self.requantize_every_call or not self._codes_current
        Y = ops.linear_int8_mixed_fp16_weights(x, self.weight, self.Wq, self.sw, requantize,
                                               self.bias, self.threshold, self._ws)
        if M > 0:
            self._codes_current = True
        return Y

    def extra_repr(self):
        return "in_features=%d, out_features=%d, threshold=%g, has_fp16_weights=%s, ready=%s" % (
            self.in_features, self.out_features, self.threshold, self.has_fp16_weights,
            self._quantized)
