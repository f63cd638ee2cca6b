"""Seeded synthetic inputs for the ConvRot linear workloads.

This module only draws random numbers and shapes them; it holds none of the
layer's arithmetic (no rotation, no quantization, no product).  It is the one
module that both the HIP-path tests/benchmark and the CPU oracle's tests use,
so that both sides see the same bytes.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) used as a counter-based generator -- output i
of stream ``seed`` is the SplitMix64 finalizer applied to
``seed + (i + 1) * 0x9E3779B97F4A7C15``; uniforms take the top 53 bits;
normals come from the Box-Muller transform (cosine branch).  Every stream is
keyed by ``0xC0517 + 1000 * config + 10 * layer + tensor_id``.

Workloads (the pages describe DiT and text-encoder linears of diffusion
models; the trained layers are not available, so these seeded tensors stand in
for them): activations are bf16 (Gaussian or Student-t with outlier
channels), weights fp32 ~ N(0, 0.02^2), bias bf16 ~ N(0, 0.01^2), rotation
group 128 unless stated.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

SEED_BASE = 0xC0517

# tensor ids inside a stream key
T_X, T_W, T_BIAS, T_CHAN, T_FACTOR, T_ROWAMAX, T_ROWS = range(7)


def stream_seed(config: int, layer: int, tensor_id: int) -> int:
    return SEED_BASE + 1000 * config + 10 * layer + tensor_id


_CHUNK = 1 << 20


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset+n-1 of the counter-based SplitMix64 stream."""
    out = np.empty(n, dtype=np.uint64)
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        for a in range(0, n, _CHUNK):
            b = min(n, a + _CHUNK)
            z = out[a:b]
            z[:] = np.arange(offset + a + 1, offset + b + 1, dtype=np.uint64)
            z *= _GOLDEN
            z += s
            z ^= z >> np.uint64(30)
            z *= _M1
            z ^= z >> np.uint64(27)
            z *= _M2
            z ^= z >> np.uint64(31)
    return out


def uniform(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """float64 uniforms in [0, 1)."""
    z = splitmix64(seed, n, offset)
    z >>= np.uint64(11)
    u = z.astype(np.float64)
    u *= 2.0 ** -53
    return u


def normal(seed: int, n: int) -> np.ndarray:
    """float64 standard normals (Box-Muller, cosine branch; 2 uniforms each)."""
    u = uniform(seed, 2 * n).reshape(n, 2)
    out = np.empty(n, dtype=np.float64)
    for a in range(0, n, _CHUNK):
        b = min(n, a + _CHUNK)
        r = np.log(1.0 - u[a:b, 0])      # 1 - u in (0, 1]
        r *= -2.0
        np.sqrt(r, out=r)
        c = np.cos(2.0 * np.pi * u[a:b, 1])
        np.multiply(r, c, out=out[a:b])
    return out


def student_t4(seed: int, n: int) -> np.ndarray:
    """Student-t with 4 degrees of freedom: Z / sqrt(chi2_4 / 4), where
    chi2_4 = -2 ln(U_a U_b) (a sum of two chi2_2 = exponential(1/2) draws)."""
    z = normal(seed, n)
    u = uniform(seed ^ 0x5A5A5A5A, 2 * n)
    chi2 = -2.0 * (np.log(1.0 - u[0::2]) + np.log(1.0 - u[1::2]))
    return z / np.sqrt(chi2 / 4.0)


def pick_channels(seed: int, K: int, count: int) -> np.ndarray:
    """``count`` distinct channel indices in [0, K), seeded."""
    return np.sort(np.argsort(uniform(seed, K), kind="stable")[:count]).astype(np.int64)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float -> bf16 (round to nearest even, by torch's CPU conversion) as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_float(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits -> float32 (exact), by torch's CPU conversion."""
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


@dataclasses.dataclass
class Layer:
    """One linear layer's synthetic inputs."""
    name: str
    M: int
    K: int
    N: int
    g: int
    x_bits: np.ndarray      # uint16 [M, K] bf16 activation
    w: np.ndarray           # float32 [N, K] weight (unrotated, unquantized)
    bias_bits: np.ndarray   # uint16 [N] bf16 bias


def _weight(cfg: int, layer: int, N: int, K: int) -> np.ndarray:
    return (0.02 * normal(stream_seed(cfg, layer, T_W), N * K)).astype(np.float32).reshape(N, K)


def _bias(cfg: int, layer: int, N: int) -> np.ndarray:
    return to_bf16_bits(0.01 * normal(stream_seed(cfg, layer, T_BIAS), N))


def _gauss_outliers(cfg, layer, M, K, count, factor):
    x = normal(stream_seed(cfg, layer, T_X), M * K).reshape(M, K)
    ch = pick_channels(stream_seed(cfg, layer, T_CHAN), K, count)
    x[:, ch] *= factor
    return x


def _t4_outliers(cfg, layer, M, K, count, factors):
    x = student_t4(stream_seed(cfg, layer, T_X), M * K).reshape(M, K)
    ch = pick_channels(stream_seed(cfg, layer, T_CHAN), K, count)
    x[:, ch] *= np.asarray(factors, dtype=np.float64)[None, :]
    return x


def _gelu_tanh(z):
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def _row_absmax(cfg, layer, M, K):
    """N(0,1) rows rescaled so that row m's absmax is a_m ~ U[5, 30]."""
    x = normal(stream_seed(cfg, layer, T_X), M * K).reshape(M, K)
    a = 5.0 + 25.0 * uniform(stream_seed(cfg, layer, T_ROWAMAX), M)
    return x * (a / np.abs(x).max(axis=1))[:, None]


# name -> (config number, M, K, N)
SHAPES = {
    "tiny":      (1, 128, 512, 512),
    "qkv":       (2, 4608, 3072, 9216),
    "mlp_up":    (3, 4608, 3072, 12288),
    "mlp_down":  (3, 4608, 12288, 3072),
    "hires_up":  (4, 16896, 3072, 12288),
    "small_m":   (4, 16, 4096, 12288),
}

# the four linears of one block of the 60-block denoising-step stack (M = 4608)
STACK_LAYERS = (("qkv", 3072, 9216), ("out", 3072, 3072), ("up", 3072, 12288), ("down", 12288, 3072))
STACK_BLOCKS = 60
STACK_M = 4608


def make_layer(name: str, g: int = 128, M: int | None = None) -> Layer:
    """Build one workload's inputs.  ``M`` optionally truncates the token count
    (the rows are then the first M rows of the full workload's activation
    distribution, drawn with the same seeds at that size)."""
    if name.startswith("stack_"):
        return make_stack_layer(name, g=g, M=M)
    cfg, M0, K, N = SHAPES[name]
    M = M0 if M is None else M
    layer = 1 if name == "mlp_down" else 0
    if name == "tiny":
        x = _gauss_outliers(cfg, layer, M, K, 4, 20.0)
    elif name == "qkv":
        x = _t4_outliers(cfg, layer, M, K, 30, np.full(30, 30.0))
    elif name == "mlp_up":
        f = 1.0 + 49.0 * uniform(stream_seed(cfg, layer, T_FACTOR), 30)
        f[0] = 50.0
        x = _t4_outliers(cfg, layer, M, K, 30, f)
    elif name == "mlp_down":
        # the down projection reads GELU(tanh form) of an up-projection-shaped
        # tensor: a bf16 Student-t field with outlier channels, then GELU in
        # float32, then bf16.
        f = 1.0 + 49.0 * uniform(stream_seed(cfg, layer, T_FACTOR), 30)
        f[0] = 50.0
        z = _t4_outliers(cfg, layer, M, K, 30, f)
        z = bf16_bits_to_float(to_bf16_bits(z)).astype(np.float32)
        x = _gelu_tanh(z.astype(np.float32)).astype(np.float32)
    elif name in ("hires_up", "small_m"):
        x = _gauss_outliers(cfg, layer, M, K, 4, 20.0)
    else:
        raise KeyError(name)
    return Layer(name, M, K, N, g, to_bf16_bits(x), _weight(cfg, layer, N, K), _bias(cfg, layer, N))


def make_stack_layer(name: str, g: int = 128, M: int | None = None) -> Layer:
    """``stack_b<block>_<qkv|out|up|down>``: one linear of the 60-block stack."""
    _, b, kind = name.split("_")
    block = int(b[1:])
    idx = [k for k, _, _ in STACK_LAYERS].index(kind)
    _, K, N = STACK_LAYERS[idx]
    layer = 4 * block + idx
    M = STACK_M if M is None else M
    x = _row_absmax(5, layer, M, K)
    return Layer(name, M, K, N, g, to_bf16_bits(x), _weight(5, layer, N, K), _bias(5, layer, N))


def stack_weight_device(block: int, li: int, dev) -> tuple:
    """The benchmark's device-drawn stack: layer li (index into STACK_LAYERS)
    of block ``block``: fp32 weight N(0, 0.02^2) [N, K] and bf16 bias
    N(0, 0.01^2) [N], from torch's generator on ``dev`` seeded per layer, so
    that 6.79 GB of weights never pass through the host."""
    _, K, N = STACK_LAYERS[li]
    gen = torch.Generator(device=dev)
    gen.manual_seed(0xC0517 + 5000 + 10 * (4 * block + li))
    w = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
    bias = (torch.randn(N, generator=gen, device=dev) * 0.01).to(torch.bfloat16)
    return w, bias


def stack_tokens_device(which: int, dev):
    """The stack's bf16 token rows [STACK_M, 3072] on ``dev`` (which = 1: the
    block input, 2: the attention-output stand-in): N(0, 1) rows rescaled so
    that each row's absmax is drawn from U[5, 30]."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(0xC0517 + 5000 + which)
    x = torch.randn((STACK_M, 3072), generator=gen, device=dev)
    a = 5.0 + 25.0 * torch.rand((STACK_M, 1), generator=gen, device=dev)
    return (x * (a / x.abs().amax(dim=1, keepdim=True))).to(torch.bfloat16)


def sample_rows(M: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct token rows for sampled checks; always holds 0 and M-1."""
    r = np.argsort(uniform(seed, M), kind="stable")[:min(count, M)]
    return np.unique(np.concatenate([r, [0, M - 1]])).astype(np.int64)
