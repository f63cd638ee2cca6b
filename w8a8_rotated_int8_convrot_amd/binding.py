"""Python binding of ``libconvrot.so`` (C ABI: ``include/convrot.h``).

Argument marshalling only: every function here allocates its torch outputs
(device memory is PyTorch's job), passes raw device pointers and the current
HIP stream to the entry point of the same name, and raises on a non-zero
status.  Every step of the layer runs in the library's HIP kernels; there is
no other implementation to fall back to, and importing this module without a
built library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconvrot.so")

CONVROT_F32 = 0
CONVROT_BF16 = 1
CONVROT_F16 = 2
CONVROT_SCALE_TENSOR = 0
CONVROT_SCALE_ROW = 1

STATUS = {0: "CONVROT_OK", -1: "CONVROT_EINVAL", -2: "CONVROT_EUNSUPPORTED",
          -3: "CONVROT_EALIGN", -4: "CONVROT_EWORKSPACE", -5: "CONVROT_EHIP"}

# Every symbol include/convrot.h declares, with (argtypes, restype).
_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "convrot_abi_version": ([], _I),
    "convrot_last_error": ([], ctypes.c_char_p),
    "convrot_prepare_weight_workspace": ([_I64, _I64], _SZ),
    "convrot_prepare_weight": ([_P, _I, _I64, _I64, _I, _P, _P, _P, _SZ, _P], _I),
    "convrot_linear_workspace": ([_I64, _I64, _I64], _SZ),
    "convrot_linear": ([_P, _I64, _I64, _P, _P, _I64, _I, _P, _P, _P, _SZ, _P], _I),
    "convrot_linear_noalloc": ([_P, _I64, _I64, _P, _P, _I64, _I, _P, _P, _P], _I),
    "convrot_rotate_quant": ([_P, _I64, _I64, _I, _P, _P, _P], _I),
    "convrot_gemm_i32": ([_P, _P, _I64, _I64, _I64, _P, _P], _I),
    "convrot_gemm_dequant": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], _I),
    "convrot_probe_mfma_i8": ([_P, _I64, _P, _I64, _I, _I, _P, _P], _I),
    "convrot_probe_stream": ([_P, _I64, _P, _P], _I),
    "convrot_prepare_weight_ex": ([_P, _I, _I64, _I64, _I, _I, _P, _P, _P, _SZ, _P], _I),
    "convrot_rotate_quant_ex": ([_P, _I, _I64, _I64, _I, _P, _P, _P], _I),
    "convrot_gemm_dequant_ex": ([_P, _P, _P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _P], _I),
    "convrot_linear_ex": ([_P, _I, _I64, _I64, _P, _P, _I, _I64, _I, _P, _P, _P, _SZ, _P], _I),
    "convrot_stream_slot_bytes": ([_P, _I], _SZ),
    "convrot_linear_streamed": ([_P, _I, _P, _SZ, _P, _SZ, _P, _P], _I),
    "convrot_default_workspace": ([_I64, _I64], _SZ),
    "convrot_unpack_weight": ([_P, _P, _I, _I64, _I64, _I, _I, _P, _P], _I),
    "convrot_default_linear": ([_P, _I, _I64, _I64, _P, _P, _I, _I64, _I, _P, _P, _P, _SZ, _P], _I),
    "convrot_guarded_workspace": ([_I64, _I64, _I64], _SZ),
    "convrot_linear_guarded": ([_P, _I, _I64, _I64, _P, _P, _I, _I64, _I, _P, _P, _P, _SZ, _P], _I),
    "convrot_guard_query": ([_I, _P], _I),
    "convrot_guard_reset": ([_I], _I),
    "convrot_guard_configure": ([ctypes.c_double, _I], _I),
    "convrot_guard_inject": ([_I, _I], _I),
}

CONVROT_FAULT_NONE = 0
CONVROT_FAULT_MISMATCH = 1
CONVROT_FAULT_KERNEL = 2


class ConvrotError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m w8a8_rotated_int8_convrot_amd.build` first")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise ConvrotError(name, rc, last_error())
    return rc


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, name, ndim=None):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} CUDA tensor, got "
                         f"{t.dtype} on {t.device} (contiguous={t.is_contiguous()})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dimensions, got {t.dim()}")


def convrot_last_error() -> str:
    return lib().convrot_last_error().decode()


last_error = convrot_last_error


def convrot_abi_version() -> int:
    return lib().convrot_abi_version()


def convrot_prepare_weight_workspace(N: int, K: int) -> int:
    return lib().convrot_prepare_weight_workspace(N, K)


def convrot_linear_workspace(M: int, K: int, N: int) -> int:
    return lib().convrot_linear_workspace(M, K, N)


def convrot_prepare_weight(w: torch.Tensor, group: int):
    """fp32 or bf16 weight [N, K] -> (int8 codes [N, K], fp32 scale [1])."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("convrot_prepare_weight: weight must be float32 or bfloat16")
    _need(w, w.dtype, "w", 2)
    N, K = w.shape
    wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    s = torch.empty(1, dtype=torch.float32, device=w.device)
    ws_bytes = convrot_prepare_weight_workspace(N, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=w.device)
    dt = CONVROT_F32 if w.dtype == torch.float32 else CONVROT_BF16
    _call("convrot_prepare_weight", _ptr(w), dt, N, K, group, _ptr(wq), _ptr(s), _ptr(ws),
          ws_bytes, _stream(w))
    return wq, s


def convrot_rotate_quant(x: torch.Tensor, group: int, q=None, s=None):
    """bf16 [M, K] -> (int8 codes [M, K], fp32 scales [M])."""
    _need(x, torch.bfloat16, "x", 2)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    s = torch.empty(M, dtype=torch.float32, device=x.device) if s is None else s
    _need(q, torch.int8, "q", 2)
    _need(s, torch.float32, "s", 1)
    if tuple(q.shape) != (M, K) or s.numel() != M:
        raise ValueError("convrot_rotate_quant: output shape mismatch")
    _call("convrot_rotate_quant", _ptr(x), M, K, group, _ptr(q), _ptr(s), _stream(x))
    return q, s


def convrot_gemm_i32(xq: torch.Tensor, wq: torch.Tensor) -> torch.Tensor:
    """int8 [M, K] x int8 [N, K]^T -> int32 [M, N]."""
    _need(xq, torch.int8, "xq", 2)
    _need(wq, torch.int8, "wq", 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("convrot_gemm_i32: K mismatch")
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    _call("convrot_gemm_i32", _ptr(xq), _ptr(wq), M, N, K, _ptr(acc), _stream(xq))
    return acc


def convrot_gemm_dequant(xq, x_scale, wq, w_scale, bias=None, out=None) -> torch.Tensor:
    """int8 codes and scales -> bf16 [M, N] (GEMM + dequant + bias)."""
    _need(xq, torch.int8, "xq", 2)
    _need(wq, torch.int8, "wq", 2)
    _need(x_scale, torch.float32, "x_scale", 1)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or x_scale.numel() != M:
        raise ValueError("convrot_gemm_dequant: shape mismatch")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", 1)
        if bias.numel() != N:
            raise ValueError("convrot_gemm_dequant: bias must have N elements")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device) if out is None else out
    _need(y, torch.bfloat16, "out", 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("convrot_gemm_dequant: output shape mismatch")
    _call("convrot_gemm_dequant", _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), _ptr(bias),
          _ptr(y), M, N, K, _stream(xq))
    return y


def convrot_probe_mfma_i8(a, b, blocks, iters, out=None) -> torch.Tensor:
    """Measurement aid: register-only int8 MFMA loop on fragments of the int8
    tensors a and b (see include/convrot.h); returns the int32 checksums
    [blocks * 768].  Integer ops: blocks * 12 * iters * 16 * 32768."""
    _need(a, torch.int8, "a", None)
    _need(b, torch.int8, "b", None)
    o = torch.empty(blocks * 768, dtype=torch.int32, device=a.device) if out is None else out
    _need(o, torch.int32, "out", 1)
    if o.numel() < blocks * 768:
        raise ValueError("convrot_probe_mfma_i8: out needs blocks * 768 elements")
    _call("convrot_probe_mfma_i8", _ptr(a), a.numel(), _ptr(b), b.numel(), blocks, iters, _ptr(o),
          _stream(a))
    return o


def convrot_probe_stream(x, out=None) -> torch.Tensor:
    """Measurement aid: the traffic of rotate + quant without its arithmetic
    (see include/convrot.h); x is a contiguous 16-bit CUDA tensor, returns the
    int8 tensor of its high bytes, same shape."""
    if x.dtype not in (torch.bfloat16, torch.float16, torch.int16) or not x.is_cuda or not x.is_contiguous():
        raise ValueError("convrot_probe_stream: x must be a contiguous 16-bit CUDA tensor")
    q = torch.empty(x.shape, dtype=torch.int8, device=x.device) if out is None else out
    _need(q, torch.int8, "out", x.dim())
    if q.shape != x.shape:
        raise ValueError("convrot_probe_stream: out shape mismatch")
    _call("convrot_probe_stream", _ptr(x), x.numel(), _ptr(q), _stream(x))
    return q


def convrot_linear(x, wq, w_scale, group, bias=None, out=None, workspace=None) -> torch.Tensor:
    """The whole layer: bf16 x [M, K], int8 wq [N, K] (+ scale) -> bf16 y [M, N].

    ``workspace`` (uint8 CUDA tensor) defaults to convrot_linear_workspace
    bytes; a smaller one makes the library process the tokens in more
    slices (same result)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(wq, torch.int8, "wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("convrot_linear: K mismatch")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", 1)
        if bias.numel() != N:
            raise ValueError("convrot_linear: bias must have N elements")
    if workspace is None:
        workspace = torch.empty(max(convrot_linear_workspace(M, K, N), 1), dtype=torch.uint8,
                                device=x.device)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, torch.bfloat16, "out", 2)
    _need(workspace, torch.uint8, "workspace")
    if tuple(y.shape) != (M, N):
        raise ValueError("convrot_linear: output shape mismatch")
    _call("convrot_linear", _ptr(x), M, K, _ptr(wq), _ptr(w_scale), N, group, _ptr(bias), _ptr(y),
          _ptr(workspace), workspace.numel(), _stream(x))
    return y


def convrot_linear_noalloc(x, wq, w_scale, group, bias=None, out=None) -> torch.Tensor:
    """convrot_linear without a workspace: the library keeps the slice's codes
    and scales in its own device array (see include/convrot.h), so the call
    allocates nothing when ``out`` is given."""
    _need(x, torch.bfloat16, "x", 2)
    _need(wq, torch.int8, "wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("convrot_linear_noalloc: K mismatch")
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", 1)
        if bias.numel() != N:
            raise ValueError("convrot_linear_noalloc: bias must have N elements")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, torch.bfloat16, "out", 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("convrot_linear_noalloc: output shape mismatch")
    _call("convrot_linear_noalloc", _ptr(x), M, K, _ptr(wq), _ptr(w_scale), N, group, _ptr(bias), _ptr(y),
          _stream(x))
    return y


# ---------------------------------------------------------------- variants (fp16 I/O, row-wise weight scales)

_IO = {torch.bfloat16: CONVROT_BF16, torch.float16: CONVROT_F16}


def _io_of(t, name):
    if t.dtype not in _IO:
        raise ValueError(f"{name}: expected bfloat16 or float16, got {t.dtype}")
    return _IO[t.dtype]


def convrot_prepare_weight_ex(w: torch.Tensor, group: int, scale_mode: str = "tensor"):
    """fp32, bf16 or fp16 weight [N, K] -> (int8 codes [N, K], fp32 scales [1] or [N]).

    scale_mode "tensor": one scale; "row": one per output channel."""
    dt = {torch.float32: CONVROT_F32, torch.bfloat16: CONVROT_BF16, torch.float16: CONVROT_F16}.get(w.dtype)
    if dt is None:
        raise ValueError("convrot_prepare_weight_ex: weight must be float32, bfloat16 or float16")
    if scale_mode not in ("tensor", "row"):
        raise ValueError("convrot_prepare_weight_ex: scale_mode is 'tensor' or 'row'")
    _need(w, w.dtype, "w", 2)
    N, K = w.shape
    wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    s = torch.empty(N if scale_mode == "row" else 1, dtype=torch.float32, device=w.device)
    ws_bytes = convrot_prepare_weight_workspace(N, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=w.device)
    mode = CONVROT_SCALE_ROW if scale_mode == "row" else CONVROT_SCALE_TENSOR
    _call("convrot_prepare_weight_ex", _ptr(w), dt, N, K, group, mode, _ptr(wq), _ptr(s), _ptr(ws),
          ws_bytes, _stream(w))
    return wq, s


def convrot_rotate_quant_ex(x: torch.Tensor, group: int, q=None, s=None):
    """bf16 or fp16 [M, K] -> (int8 codes [M, K], fp32 scales [M])."""
    io = _io_of(x, "x")
    _need(x, x.dtype, "x", 2)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    s = torch.empty(M, dtype=torch.float32, device=x.device) if s is None else s
    _need(q, torch.int8, "q", 2)
    _need(s, torch.float32, "s", 1)
    _call("convrot_rotate_quant_ex", _ptr(x), io, M, K, group, _ptr(q), _ptr(s), _stream(x))
    return q, s


def _scale_mode_of(w_scale, N, who):
    if w_scale.numel() == 1:
        return CONVROT_SCALE_TENSOR
    if w_scale.numel() == N:
        return CONVROT_SCALE_ROW
    raise ValueError(f"{who}: w_scale must hold 1 or N scales")


def convrot_gemm_dequant_ex(xq, x_scale, wq, w_scale, bias=None, out=None,
                            out_dtype=torch.bfloat16) -> torch.Tensor:
    """int8 codes and scales -> bf16 or fp16 [M, N]; w_scale holds 1 or N scales,
    bias (nullable) has the output dtype."""
    _need(xq, torch.int8, "xq", 2)
    _need(wq, torch.int8, "wq", 2)
    _need(x_scale, torch.float32, "x_scale", 1)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or x_scale.numel() != M:
        raise ValueError("convrot_gemm_dequant_ex: shape mismatch")
    mode = _scale_mode_of(w_scale, N, "convrot_gemm_dequant_ex")
    y = torch.empty((M, N), dtype=out_dtype, device=xq.device) if out is None else out
    io = _io_of(y, "out")
    _need(y, y.dtype, "out", 2)
    if bias is not None:
        _need(bias, y.dtype, "bias", 1)
        if bias.numel() != N:
            raise ValueError("convrot_gemm_dequant_ex: bias must have N elements")
    if tuple(y.shape) != (M, N):
        raise ValueError("convrot_gemm_dequant_ex: output shape mismatch")
    _call("convrot_gemm_dequant_ex", _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), mode, _ptr(bias),
          _ptr(y), io, M, N, K, _stream(xq))
    return y


def convrot_linear_ex(x, wq, w_scale, group, bias=None, out=None, workspace=None) -> torch.Tensor:
    """The whole layer in bf16 or fp16 (x, bias and y share x's dtype), with one
    weight scale or one per output channel (w_scale of 1 or N floats)."""
    io = _io_of(x, "x")
    _need(x, x.dtype, "x", 2)
    _need(wq, torch.int8, "wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("convrot_linear_ex: K mismatch")
    mode = _scale_mode_of(w_scale, N, "convrot_linear_ex")
    if bias is not None:
        _need(bias, x.dtype, "bias", 1)
        if bias.numel() != N:
            raise ValueError("convrot_linear_ex: bias must have N elements")
    if workspace is None:
        workspace = torch.empty(max(convrot_linear_workspace(M, K, N), 1), dtype=torch.uint8,
                                device=x.device)
    y = torch.empty((M, N), dtype=x.dtype, device=x.device) if out is None else out
    _need(y, x.dtype, "out", 2)
    _need(workspace, torch.uint8, "workspace")
    if tuple(y.shape) != (M, N):
        raise ValueError("convrot_linear_ex: output shape mismatch")
    _call("convrot_linear_ex", _ptr(x), io, M, K, _ptr(wq), _ptr(w_scale), mode, N, group, _ptr(bias),
          _ptr(y), _ptr(workspace), workspace.numel(), _stream(x))
    return y


# ---------------------------------------------------------------- streamed weights

class StreamLayer(ctypes.Structure):
    """Mirror of ``convrot_stream_layer`` (include/convrot.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64),
                ("N", ctypes.c_int64), ("wq_host", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("group", ctypes.c_int), ("bias", ctypes.c_void_p), ("y", ctypes.c_void_p)]


def _stream_layers(layers):
    arr = (StreamLayer * len(layers))()
    for i, L in enumerate(layers):
        x, wq_host, w_scale, y = L["x"], L["wq_host"], L["w_scale"], L["out"]
        M, K = x.shape
        N = wq_host.shape[0]
        arr[i] = StreamLayer(_ptr(x), M, K, N, wq_host.data_ptr(), _ptr(w_scale), L["group"],
                             _ptr(L.get("bias")), _ptr(y))
    return arr


def convrot_stream_slot_bytes(layers) -> int:
    """Bytes of one weight slot for these layers (dicts as for convrot_linear_streamed)."""
    arr = _stream_layers(layers)
    return lib().convrot_stream_slot_bytes(arr, len(layers))


def convrot_linear_streamed(layers, slots=None, workspace=None, copy_stream=None):
    """Run layers whose int8 weights are in pinned host memory (see include/convrot.h).

    ``layers``: list of dicts with ``x`` (bf16 CUDA [M, K]), ``wq_host`` (pinned CPU
    int8 [N, K]), ``w_scale`` (CUDA fp32 [1]), ``group``, optional ``bias`` (bf16
    [N]) and ``out`` (bf16 CUDA [M, N], allocated if absent).  Compute runs on the
    current stream, the weight copies on ``copy_stream`` (a new stream if None).
    Returns the outputs."""
    if not layers:
        return []
    dev = layers[0]["x"].device
    for L in layers:
        _need(L["x"], torch.bfloat16, "x", 2)
        if L["wq_host"].dtype != torch.int8 or L["wq_host"].is_cuda or not L["wq_host"].is_contiguous():
            raise ValueError("wq_host: expected a contiguous int8 CPU tensor (pinned)")
        if "out" not in L or L["out"] is None:
            L["out"] = torch.empty((L["x"].shape[0], L["wq_host"].shape[0]), dtype=torch.bfloat16, device=dev)
    arr = _stream_layers(layers)
    slot_bytes = lib().convrot_stream_slot_bytes(arr, len(layers))
    if slots is None:
        slots = torch.empty(2 * slot_bytes, dtype=torch.uint8, device=dev)
    if workspace is None:
        need = max(convrot_linear_workspace(L["x"].shape[0], L["x"].shape[1], L["wq_host"].shape[0])
                   for L in layers)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=dev)
    _call("convrot_linear_streamed", arr, len(layers), _ptr(slots), slots.numel() // 2, _ptr(workspace),
          workspace.numel(), copy_stream.cuda_stream, torch.cuda.current_stream(dev).cuda_stream)
    return [L["out"] for L in layers]


# ---------------------------------------------------------------- default path and guarded layer

def convrot_default_workspace(K: int, N: int) -> int:
    return lib().convrot_default_workspace(K, N)


def convrot_guarded_workspace(M: int, K: int, N: int) -> int:
    return lib().convrot_guarded_workspace(M, K, N)


def convrot_unpack_weight(wq, w_scale, group, out_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """int8 codes [N, K] and 1 or N scales -> the unpacked weight [N, K] in bf16 or fp16."""
    _need(wq, torch.int8, "wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    N, K = wq.shape
    mode = _scale_mode_of(w_scale, N, "convrot_unpack_weight")
    wu = torch.empty((N, K), dtype=out_dtype, device=wq.device) if out is None else out
    io = _io_of(wu, "out")
    _need(wu, wu.dtype, "out", 2)
    if tuple(wu.shape) != (N, K):
        raise ValueError("convrot_unpack_weight: output shape mismatch")
    _call("convrot_unpack_weight", _ptr(wq), _ptr(w_scale), mode, N, K, group, io, _ptr(wu), _stream(wq))
    return wu


def _layer_args(who, x, wq, w_scale, bias, out):
    io = _io_of(x, "x")
    _need(x, x.dtype, "x", 2)
    _need(wq, torch.int8, "wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError(f"{who}: K mismatch")
    mode = _scale_mode_of(w_scale, N, who)
    if bias is not None:
        _need(bias, x.dtype, "bias", 1)
        if bias.numel() != N:
            raise ValueError(f"{who}: bias must have N elements")
    y = torch.empty((M, N), dtype=x.dtype, device=x.device) if out is None else out
    _need(y, x.dtype, "out", 2)
    if tuple(y.shape) != (M, N):
        raise ValueError(f"{who}: output shape mismatch")
    return io, M, K, N, mode, y


def convrot_default_linear(x, wq, w_scale, group, bias=None, out=None, workspace=None) -> torch.Tensor:
    """The default (dequantizing) path: unpack the weight, y = x . Wu^T + bias in
    x's dtype (bf16 or fp16) with fp32 accumulation."""
    io, M, K, N, mode, y = _layer_args("convrot_default_linear", x, wq, w_scale, bias, out)
    if workspace is None:
        workspace = torch.empty(max(convrot_default_workspace(K, N), 1), dtype=torch.uint8, device=x.device)
    _need(workspace, torch.uint8, "workspace")
    _call("convrot_default_linear", _ptr(x), io, M, K, _ptr(wq), _ptr(w_scale), mode, N, group, _ptr(bias),
          _ptr(y), _ptr(workspace), workspace.numel(), _stream(x))
    return y


def convrot_linear_guarded(x, wq, w_scale, group, bias=None, out=None, workspace=None) -> torch.Tensor:
    """The int8 layer, checked against the default path on its first call per
    layer shape and token bucket, with a sticky per-device fallback."""
    io, M, K, N, mode, y = _layer_args("convrot_linear_guarded", x, wq, w_scale, bias, out)
    if workspace is None:
        workspace = torch.empty(max(convrot_guarded_workspace(M, K, N), 1), dtype=torch.uint8,
                                device=x.device)
    _need(workspace, torch.uint8, "workspace")
    _call("convrot_linear_guarded", _ptr(x), io, M, K, _ptr(wq), _ptr(w_scale), mode, N, group, _ptr(bias),
          _ptr(y), _ptr(workspace), workspace.numel(), _stream(x))
    return y


class GuardInfo(ctypes.Structure):
    """Mirror of ``convrot_guard_info`` (include/convrot.h)."""
    _fields_ = [("fallback", ctypes.c_int), ("checked", ctypes.c_int64), ("checks_run", ctypes.c_int64),
                ("last_error", ctypes.c_double), ("message", ctypes.c_char * 256)]


def convrot_guard_query(device: int = 0) -> dict:
    info = GuardInfo()
    _call("convrot_guard_query", device, ctypes.byref(info))
    return {"fallback": bool(info.fallback), "checked": info.checked, "checks_run": info.checks_run,
            "last_error": info.last_error, "message": info.message.decode()}


def convrot_guard_reset(device: int = 0) -> None:
    _call("convrot_guard_reset", device)


def convrot_guard_configure(tol: float = 0.1, log_to_stderr: bool = True) -> None:
    _call("convrot_guard_configure", float(tol), 1 if log_to_stderr else 0)


def convrot_guard_inject(device: int, fault: str) -> None:
    """Arm one host-side fault ("none", "mismatch" or "kernel") for the next guarded call."""
    codes = {"none": CONVROT_FAULT_NONE, "mismatch": CONVROT_FAULT_MISMATCH, "kernel": CONVROT_FAULT_KERNEL}
    if fault not in codes:
        raise ValueError("convrot_guard_inject: fault is 'none', 'mismatch' or 'kernel'")
    _call("convrot_guard_inject", device, codes[fault])
