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

The quantized pair can be saved and loaded again without re-quantizing
(section "Saving 8-bit state dicts on the Hub" names the missing piece: the
CB and SCB statistics were not kept in the state dict): as a safetensors file
holding CB and SCB under those names, and through the module's state dict,
whose extra state records that the buffers hold a quantized weight.
"""

import threading

import torch

from . import ops

INT8_FORMAT = "llm-int8/per-output-row-absmax/v1"

# One workspace per (device, stream), shared by every module: the layers of a
# model run one after another on a stream, so they can share their scratch
# (outlier flags and columns, row scales, int8 codes, gathered outlier
# activations, and the region of recovered outlier weights, room for 512
# columns per output row). A model then holds one layer's worth of
# workspace, not one per module. Calls on different streams get their own.
# Each call takes the prefix of the layer's own size, so the layer's path
# (and its result bits) do not depend on which layers ran before.
_WS_LOCK = threading.Lock()
_WORKSPACES = {}


def shared_workspace(device, nbytes):
    """The shared workspace of the current stream on `device`, grown to at
    least nbytes (uint8 tensor)."""
    device = torch.device(device)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    with _WS_LOCK:
        ws = _WORKSPACES.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=device)
            _WORKSPACES[key] = ws
        return ws


def save_int8_weight(path, Wq, sw, bias=None, threshold=ops.DEFAULT_THRESHOLD):
    """Write the quantized weight pair to a safetensors file: CB = Wq (int8
    [out, in], the codes), SCB = sw (fp32 [out], the per-output-row absmax),
    optional bias (fp16 [out]); the threshold and the shape go in the
    metadata. Tensors may live on any device."""
    from safetensors.torch import save_file
    if Wq.dtype != torch.int8 or Wq.dim() != 2:
        raise TypeError("Wq must be an int8 [out, in] tensor")
    N, K = Wq.shape
    if sw.dtype != torch.float32 or tuple(sw.shape) != (N,):
        raise TypeError("sw must be a float32 [out] tensor")
    tensors = {"CB": Wq.detach().cpu().contiguous(), "SCB": sw.detach().cpu().contiguous()}
    if bias is not None:
        if tuple(bias.shape) != (N,):
            raise ValueError("bias must be [out]")
        tensors["bias"] = bias.detach().to(torch.float16).cpu().contiguous()
    meta = {"format": INT8_FORMAT, "threshold": repr(float(threshold)),
            "out_features": str(N), "in_features": str(K)}
    save_file(tensors, path, metadata=meta)


def load_int8_weight(path):
    """Read a file written by save_int8_weight (safetensors: no code is run).
    Returns {"CB", "SCB", "bias" (or None), "threshold"} with CPU tensors;
    raises ValueError on a different format or inconsistent tensors."""
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        meta = f.metadata() or {}
        if meta.get("format") != INT8_FORMAT:
            raise ValueError("not an int8 weight file of format %s" % INT8_FORMAT)
        keys = set(f.keys())
        if not {"CB", "SCB"} <= keys or not keys <= {"CB", "SCB", "bias"}:
            raise ValueError("unexpected tensors %s" % sorted(keys))
        CB, SCB = f.get_tensor("CB"), f.get_tensor("SCB")
        bias = f.get_tensor("bias") if "bias" in keys else None
    N, K = int(meta["out_features"]), int(meta["in_features"])
    if CB.dtype != torch.int8 or tuple(CB.shape) != (N, K):
        raise ValueError("CB must be int8 [%d, %d]" % (N, K))
    if SCB.dtype != torch.float32 or tuple(SCB.shape) != (N,):
        raise ValueError("SCB must be float32 [%d]" % N)
    if bias is not None and (bias.dtype != torch.float16 or tuple(bias.shape) != (N,)):
        raise ValueError("bias must be float16 [%d]" % N)
    return {"CB": CB, "SCB": SCB, "bias": bias, "threshold": float(meta["threshold"])}


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
        self.register_buffer("bias", torch.zeros((out_features,), dtype=torch.float16,
                                                 device=device) if bias else None)
        # fp16-weight mode: re-quantize W at every call (its codes follow W
        # as it changes); set False to re-quantize only after set_weight_.
        self.requantize_every_call = True
        self._quantized = False     # int8 mode: weight quantized; fp16 mode: weight set
        self._codes_current = False

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
        nbytes = ops.workspace_bytes(M, self.in_features, self.out_features)
        ws = shared_workspace(x.device, nbytes)[:nbytes]
        if not self.has_fp16_weights:
            return ops.linear_int8_mixed(x, self.Wq, self.sw, self.bias, self.threshold, ws)
        requantize = self.requantize_every_call or not self._codes_current
        Y = ops.linear_int8_mixed_fp16_weights(x, self.weight, self.Wq, self.sw, requantize,
                                               self.bias, self.threshold, ws)
        if M > 0:
            self._codes_current = True
        return Y

    # ---- saving and loading the quantized pair
    def save_int8(self, path):
        """Write CB, SCB (and bias) to a safetensors file (int8 mode, quantized)."""
        if self.has_fp16_weights:
            raise RuntimeError("has_fp16_weights=True keeps the fp16 weight; save its state_dict")
        if not self._quantized:
            raise RuntimeError("nothing to save: the weight is not quantized")
        save_int8_weight(path, self.Wq, self.sw, self.bias, self.threshold)

    @classmethod
    def from_int8_file(cls, path, device="cuda"):
        """A quantized int8-mode module from a save_int8 file (no re-quantization)."""
        d = load_int8_weight(path)
        N, K = d["CB"].shape
        m = cls(K, N, bias=d["bias"] is not None, threshold=d["threshold"], device=device)
        with torch.no_grad():
            m.Wq.copy_(d["CB"])
            m.sw.copy_(d["SCB"])
            if d["bias"] is not None:
                m.bias.copy_(d["bias"])
        m._quantized = True
        return m

    def get_extra_state(self):
        # the buffers alone cannot tell a quantized weight from the zeros of a
        # fresh module
        return {"format": INT8_FORMAT, "quantized": bool(self._quantized),
                "has_fp16_weights": self.has_fp16_weights, "threshold": self.threshold}

    def set_extra_state(self, state):
        if state.get("format") != INT8_FORMAT:
            raise ValueError("state of a different format")
        if bool(state["has_fp16_weights"]) != self.has_fp16_weights:
            raise ValueError("state of the other weight mode")
        self.threshold = float(state["threshold"])
        self._quantized = bool(state["quantized"])
        self._codes_current = False

    def extra_repr(self):
        return "in_features=%d, out_features=%d, threshold=%g, has_fp16_weights=%s, ready=%s" % (
            self.in_features, self.out_features, self.threshold, self.has_fp16_weights,
            self._quantized)
