"""CPU oracle for the INT8 ConvRot linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with them.

The arithmetic lives in ``convrot_oracle.c`` (plain single-threaded C99, built
with ``gcc -O2 -std=c99 -ffp-contract=off``); this module only marshals numpy
arrays through ctypes.  The steps and their sources:

* O1 Hadamard, O2 rotation -- page "int8 Compute" (InvokeAI docs), opening
  section and "What stays on the default path" (group-wise rotation, groups of
  256 in published builds); page "Explanation of INT8 ConvRot", "What is INT8
  ConvRot?" (rotation applied block after block).
* O3 tensorwise weight scale -- page "int8 Compute", opening section
  (int8_tensorwise: int8 values plus one scale).
* O4 per-token activation quantization, O5 int8 x int8 products -- page
  "int8 Compute", opening section.
* O6 dequantize with act_scale * weight_scale plus bias to bf16 -- page
  "int8 Compute", "What stays on the default path" (BF16 compute).
* Variants: fp16 in place of bf16 for the activation, the bias and the output
  (same page and section: compute is offered in BF16 or FP16), and one weight
  scale per output channel (page "Explanation of INT8 ConvRot", the format
  table's row-wise scaling).
* Default path, against which the guarded layer checks its first result per
  shape and token bucket -- page "int8 Compute", "When something goes wrong"
  and "What stays on the default path" (such layers keep unpacking the
  weight): the int8 weight dequantized and rotated back, times the activation.

Two side outputs are computed here in float64 with numpy, not in C: the
unquantized product ``x . W^T + bias`` (``reference_fp64``) and the NRMSE
(relative Frobenius error) used as the error metric on the page "INT8 ConvRot
on 2xT4 (Turing)" (kernel table and its 0.05 screening gate).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convrot_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` next to its source (gcc, host only)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        F = ctypes.c_float
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = F
        lib.oracle_f32_to_bf16.argtypes = [F]
        lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_rot_scale.argtypes = [I]
        lib.oracle_rot_scale.restype = F
        lib.oracle_hadamard.argtypes = [I, P]
        lib.oracle_rotate_rows.argtypes = [P, I64, I64, I]
        lib.oracle_quant_weight.argtypes = [P, I64, I64, I, P, P, P]
        lib.oracle_quant_act.argtypes = [P, I64, I64, I, P, P, P]
        lib.oracle_gemm_i32.argtypes = [P, P, I64, I64, I64, P]
        lib.oracle_epilogue.argtypes = [P, P, F, P, I64, I64, P]
        lib.oracle_linear_rows.argtypes = [P, I64, I64, P, I64, P, F, I64, I, P, P, P, P]
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = F
        lib.oracle_f32_to_f16.argtypes = [F]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_quant_weight_rows.argtypes = [P, I64, I64, I, P, P, P]
        lib.oracle_quant_act_ex.argtypes = [P, I, I64, I64, I, P, P, P]
        lib.oracle_epilogue_ex.argtypes = [P, P, P, I, P, I, I64, I64, P]
        lib.oracle_linear_rows_ex.argtypes = [P, I, I64, I64, P, I64, P, P, I, I64, I, P, P, P, P]
        lib.oracle_unpack_weight.argtypes = [P, P, I, I64, I64, I, I, P]
        lib.oracle_default_rows.argtypes = [P, I, I64, I64, P, I64, P, I64, P, P, P, P]
        for name in ("oracle_unpack_weight", "oracle_default_rows", "oracle_hadamard", "oracle_rotate_rows", "oracle_quant_weight",
                     "oracle_quant_act", "oracle_gemm_i32", "oracle_epilogue",
                     "oracle_linear_rows", "oracle_quant_weight_rows", "oracle_quant_act_ex",
                     "oracle_epilogue_ex", "oracle_linear_rows_ex"):
            getattr(lib, name).restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc == -2:
        raise OverflowError(f"{what}: an int32 accumulator overflowed")
    if rc != 0:
        raise ValueError(f"{what}: bad arguments (rc={rc})")


# ---------------------------------------------------------------- bf16 bits

def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(f) -> int:
    """Round one float32 to bf16 (RNE) through the C oracle."""
    return int(_load().oracle_f32_to_bf16(float(np.float32(f))))


def f16_bits_to_f32(h) -> np.ndarray:
    """Widen IEEE binary16 bit patterns (uint16) to float32 through the C oracle."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    f = _load().oracle_f16_to_f32
    return np.array([f(int(v)) for v in h.ravel()], dtype=np.float32).reshape(h.shape)


def f32_to_f16_bits(x) -> np.ndarray:
    """Round float32 values to IEEE binary16 bits (RNE) through the C oracle."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().oracle_f32_to_f16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def _io(io: str) -> int:
    if io not in ("bf16", "f16"):
        raise ValueError(f"io must be 'bf16' or 'f16', got {io!r}")
    return 1 if io == "f16" else 0


def rot_scale(g: int) -> np.float32:
    """c_g: the float32 nearest to 1/sqrt(g)."""
    return np.float32(_load().oracle_rot_scale(int(g)))


# ---------------------------------------------------------------- O1 .. O6

def hadamard(g: int) -> np.ndarray:
    H = np.empty((g, g), dtype=np.int32)
    _check(_load().oracle_hadamard(int(g), _ptr(H)), "hadamard")
    return H


def rotate(v: np.ndarray, g: int) -> np.ndarray:
    """O2 on every row of a float32 [rows, K] array; returns a new array."""
    v = np.array(v, dtype=np.float32, order="C", copy=True)
    rows, K = (1, v.shape[0]) if v.ndim == 1 else v.shape
    _check(_load().oracle_rotate_rows(_ptr(v), rows, K, int(g)), "rotate")
    return v


def quant_weight(w: np.ndarray, g: int, return_rot: bool = False):
    """O3: fp32 [N, K] -> (int8 [N, K], float32 scale[, rotated fp32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wq = np.empty((N, K), dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    rot = np.empty((N, K), dtype=np.float32) if return_rot else None
    _check(_load().oracle_quant_weight(_ptr(w), N, K, int(g), _ptr(wq), _ptr(s), _ptr(rot)),
           "quant_weight")
    return (wq, np.float32(s[0]), rot) if return_rot else (wq, np.float32(s[0]))


def quant_weight_rows(w: np.ndarray, g: int, return_rot: bool = False):
    """Row-wise O3: fp32 [N, K] -> (int8 [N, K], float32 scales [N][, rotated fp32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wq = np.empty((N, K), dtype=np.int8)
    s = np.zeros(N, dtype=np.float32)
    rot = np.empty((N, K), dtype=np.float32) if return_rot else None
    _check(_load().oracle_quant_weight_rows(_ptr(w), N, K, int(g), _ptr(wq), _ptr(s), _ptr(rot)),
           "quant_weight_rows")
    return (wq, s, rot) if return_rot else (wq, s)


def quant_act(x_bits: np.ndarray, g: int, return_rot: bool = False, io: str = "bf16"):
    """O4: bf16 (or fp16, io="f16") bits [M, K] -> (int8 [M, K], float32 [M][, rotated fp32])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    rot = np.empty((M, K), dtype=np.float32) if return_rot else None
    _check(_load().oracle_quant_act_ex(_ptr(x_bits), _io(io), M, K, int(g), _ptr(q), _ptr(s),
                                       _ptr(rot)), "quant_act")
    return (q, s, rot) if return_rot else (q, s)


def gemm_i32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """O5: int8 [M, K] x int8 [N, K]^T -> int32 [M, N] (exact)."""
    a = np.ascontiguousarray(a, dtype=np.int8)
    b = np.ascontiguousarray(b, dtype=np.int8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    acc = np.empty((M, N), dtype=np.int32)
    _check(_load().oracle_gemm_i32(_ptr(a), _ptr(b), M, N, K, _ptr(acc)), "gemm_i32")
    return acc


def epilogue(acc: np.ndarray, s_x: np.ndarray, s_w, bias_bits=None, io: str = "bf16") -> np.ndarray:
    """O6: int32 [M, N] -> bf16 (or fp16) bits [M, N].

    s_w: one scale (tensorwise) or an array of N (one per output channel)."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    M, N = acc.shape
    bias = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
    y = np.empty((M, N), dtype=np.uint16)
    sw = np.atleast_1d(np.ascontiguousarray(s_w, dtype=np.float32))
    row = sw.size > 1 or (np.ndim(s_w) == 1 and N == 1)
    if row and sw.size != N:
        raise ValueError("epilogue: s_w must hold 1 or N scales")
    if not row and io == "bf16":
        _check(_load().oracle_epilogue(_ptr(acc), _ptr(s_x), float(sw[0]), _ptr(bias),
                                       M, N, _ptr(y)), "epilogue")
    else:
        _check(_load().oracle_epilogue_ex(_ptr(acc), _ptr(s_x), _ptr(sw), int(row), _ptr(bias),
                                          _io(io), M, N, _ptr(y)), "epilogue")
    return y


def linear(x_bits, wq, s_w, g, bias_bits=None, io: str = "bf16"):
    """The whole layer on every token: O4 -> O5 -> O6.

    Returns (y bits [M, N], q_x int8 [M, K], s_x float32 [M]); x, bias and y
    are bf16 bits, or fp16 bits with io="f16"; s_w has 1 or N scales."""
    q, s = quant_act(x_bits, g, io=io)
    acc = gemm_i32(q, wq)
    return epilogue(acc, s, s_w, bias_bits, io=io), q, s


def linear_rows(x_bits, rows, wq, s_w, g, bias_bits=None):
    """The whole layer evaluated on the token rows listed in ``rows`` only.

    Returns (y bf16 bits [R, N], q int8 [R, K], s float32 [R])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    M, K = x_bits.shape
    N = wq.shape[0]
    R = rows.shape[0]
    bias = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
    y = np.empty((R, N), dtype=np.uint16)
    q = np.empty((R, K), dtype=np.int8)
    s = np.empty(R, dtype=np.float32)
    _check(_load().oracle_linear_rows(_ptr(x_bits), M, K, _ptr(rows), R, _ptr(wq),
                                      float(np.float32(s_w)), N, int(g), _ptr(bias),
                                      _ptr(y), _ptr(q), _ptr(s)), "linear_rows")
    return y, q, s


def linear_rows_ex(x_bits, rows, wq, s_w, g, bias_bits=None, io: str = "bf16"):
    """linear_rows with the variants (io = "bf16" | "f16"; s_w: 1 or N scales)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    M, K = x_bits.shape
    N = wq.shape[0]
    R = rows.shape[0]
    sw = np.atleast_1d(np.ascontiguousarray(s_w, dtype=np.float32))
    row = sw.size > 1 or (np.ndim(s_w) == 1 and N == 1)
    bias = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
    y = np.empty((R, N), dtype=np.uint16)
    q = np.empty((R, K), dtype=np.int8)
    s = np.empty(R, dtype=np.float32)
    _check(_load().oracle_linear_rows_ex(_ptr(x_bits), _io(io), M, K, _ptr(rows), R, _ptr(wq),
                                         _ptr(sw), int(row), N, int(g), _ptr(bias), _ptr(y),
                                         _ptr(q), _ptr(s)), "linear_rows_ex")
    return y, q, s


# ---------------------------------------------------------------- default path

def unpack_weight(wq, s_w, g, io: str = "bf16") -> np.ndarray:
    """The default path's unpacked weight: bf16 (or fp16) bits [N, K] of
    rnd(O2(s_w * q)), each int8 row dequantized and rotated back (s_w: one
    scale or one per row)."""
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    N, K = wq.shape
    sw = np.atleast_1d(np.ascontiguousarray(s_w, dtype=np.float32))
    row = sw.size > 1 or (np.ndim(s_w) == 1 and N == 1)
    if row and sw.size != N:
        raise ValueError("unpack_weight: s_w must hold 1 or N scales")
    wu = np.empty((N, K), dtype=np.uint16)
    _check(_load().oracle_unpack_weight(_ptr(wq), _ptr(sw), int(row), N, K, int(g), _io(io),
                                        _ptr(wu)), "unpack_weight")
    return wu


def default_rows(x_bits, rows, wu_bits, bias_bits=None, io: str = "bf16"):
    """The default-path layer on the token rows listed.

    Returns (y bits [R, N], exact float64 [R, N], mag float64 [R, N]): the
    rounded output, the fp64 value it rounds, and sum |x * wu| + |bias|."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    wu_bits = np.ascontiguousarray(wu_bits, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    M, K = x_bits.shape
    N, K2 = wu_bits.shape
    assert K == K2
    R = rows.shape[0]
    bias = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
    y = np.empty((R, N), dtype=np.uint16)
    exact = np.empty((R, N), dtype=np.float64)
    mag = np.empty((R, N), dtype=np.float64)
    _check(_load().oracle_default_rows(_ptr(x_bits), _io(io), M, K, _ptr(rows), R, _ptr(wu_bits),
                                       N, _ptr(bias), _ptr(y), _ptr(exact), _ptr(mag)),
           "default_rows")
    return y, exact, mag


# ---------------------------------------------------------------- fp64 side outputs

def reference_fp64(x_bits, w, bias_bits=None) -> np.ndarray:
    """Unquantized x . W^T + bias in float64 (no rotation: R R^T = I)."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    y = x @ np.asarray(w, dtype=np.float64).T
    if bias_bits is not None:
        y = y + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return y


def nrmse(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F in float64."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))
