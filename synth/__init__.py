"""Seeded synthetic inputs for the sharded-GEMM path.

This module is the only code that both the CPU oracle's tests and the GPU
path use.  It holds none of the method's arithmetic: it draws random
numbers, turns them into the stored bit patterns of fp32 / bf16 / fp16
arrays, and packs 4-bit affine weights into the stored (q, scale, bias)
triple.  Every consumer (oracle and GPU kernels alike) decodes those bit
patterns with its own code.

Recipe (one generator per tensor, so tensors are independent of each
other's sizes):

* ``numpy.random.default_rng(seed)`` (PCG64), drawn in float64;
* cast to float32 (round-to-nearest-even), then, for 16-bit dtypes,
  round-to-nearest-even to bfloat16 / float16;
* large tensors are drawn in row chunks from the same generator, which
  yields the same stream as one big draw.

The workload shapes follow the pages: the MLX worked example (input (4, 2),
two outputs, two devices) and the Llama-style gated MLP of "MLX 张量并行
实战指南" section 5.2; the OPT-175B vocabulary head of "拆解EnergonAI的张量并行
实现" (hidden 12288, vocabulary 50272); and the q x q SUMMA grid of
"ColossalAI 2D 张量并行" (SUMMA section).  No public dataset is involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32, BF16, F16 = "f32", "bf16", "f16"
_CHUNK = 1 << 22  # elements per draw chunk


# ---------------------------------------------------------------------------
# stored bit patterns
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 bit pattern (uint16); numpy's cast rounds to nearest even."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(a64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 draw -> stored array: float32 values, or uint16 bit patterns."""
    a32 = a64.astype(np.float32)
    if dtype == F32:
        return a32
    if dtype == BF16:
        return f32_to_bf16_bits(a32)
    if dtype == F16:
        return f32_to_f16_bits(a32)
    raise ValueError(dtype)


def bits_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array -> float32 values (for host-side statistics only)."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits_to_f32(a)
    if dtype == F16:
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------
def _draw(seed: int, shape, kind: str, a: float, b: float, dtype: str) -> np.ndarray:
    rng = np.random.default_rng(seed)
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out_dt = np.float32 if dtype == F32 else np.uint16
    out = np.empty(n, dtype=out_dt)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        if kind == "normal":
            v = rng.standard_normal(m) * b + a
        else:
            v = rng.uniform(a, b, m)
        out[s:s + m] = to_bits(v, dtype)
    return out.reshape(shape)


def normal(seed: int, shape, std: float = 1.0, dtype: str = BF16) -> np.ndarray:
    return _draw(seed, shape, "normal", 0.0, std, dtype)


def uniform(seed: int, shape, bound: float, dtype: str = BF16) -> np.ndarray:
    """U(-bound, +bound)."""
    return _draw(seed, shape, "uniform", -bound, bound, dtype)


def small_ints(seed: int, shape, lo: int, hi: int, dtype: str) -> np.ndarray:
    """Integers in [lo, hi] stored in ``dtype`` (exact in every dtype here)."""
    rng = np.random.default_rng(seed)
    v = rng.integers(lo, hi + 1, size=tuple(shape)).astype(np.float64)
    return to_bits(v, dtype)


# ---------------------------------------------------------------------------
# 4-bit affine packing (stored format shared by both sides)
# ---------------------------------------------------------------------------
def quantize_q4(w: np.ndarray, group_size: int = 64):
    """Min/max 4-bit affine quantizer and packer.

    For each output row and each group of ``group_size`` consecutive input
    elements: ``scale = fp16(( max - min ) / 15)``, ``bias = fp16(min)``,
    ``q = clamp(rne((w - bias) / scale), 0, 15)`` computed with the rounded
    scale and bias (q = 0 when scale is 0).  Eight codes go in one uint32
    along the input axis, element k in bits [4 (k mod 8), 4 (k mod 8) + 4).

    The pages give only the defaults (group_size 64, bits 4, mode affine) of
    the MLX quantizer ("MLX 张量并行实战指南" section 2.3); this layout is this
    library's own and both the oracle and the kernels decode it themselves.

    Returns (packed uint32 (out, in/8), scales fp16 bits (out, in/gs),
    biases fp16 bits (out, in/gs), q uint8 (out, in)).
    """
    w = np.asarray(w, dtype=np.float32)
    out, inn = w.shape
    assert inn % group_size == 0 and inn % 8 == 0
    g = w.reshape(out, inn // group_size, group_size).astype(np.float64)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    scale = ((mx - mn) / 15.0).astype(np.float32).astype(np.float16)
    bias = mn.astype(np.float32).astype(np.float16)
    s64 = scale.astype(np.float64)[..., None]
    b64 = bias.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(s64 > 0, np.rint((g - b64) / np.where(s64 > 0, s64, 1.0)), 0.0)
    q = np.clip(qf, 0, 15).astype(np.uint8).reshape(out, inn)
    packed = pack_q4(q)
    return packed, scale.view(np.uint16), bias.view(np.uint16), q


def e4m3_encode(v) -> np.ndarray:
    """Round-to-nearest-even, saturating encode of float values to FP8 E4M3
    (OCP: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinity;
    0x7F / 0xFF are NaN, so the largest finite magnitude 448 = 0x7E)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    _, e2 = np.frexp(np.where(a > 0, a, 1.0))          # a = m 2^e2, m in [0.5, 1)
    ex = np.clip(e2 - 1, -6, 8)                         # exponent; -6 also covers subnormals
    q = np.rint(a / np.ldexp(1.0, ex - 3))              # significand in units of 2^(ex-3)
    carry = q >= 16
    ex = np.where(carry, ex + 1, ex)
    q = np.where(carry, 8.0, q)
    code = np.where(q >= 8, ((ex + 7) << 3) | (q.astype(np.int64) - 8), q.astype(np.int64))
    code = np.minimum(code, 0x7E)
    return (code | (sign << 7)).astype(np.uint8)


def quantize_mxfp8(w: np.ndarray, block: int = 32):
    """MX FP8 quantizer (OCP Microscaling: FP8 E4M3 elements, one E8M0 scale
    per block of ``block`` consecutive inputs of a row).  Per block:
    ``X = floor(log2(max |w|)) - 8`` (8 = exponent of E4M3's largest normal),
    clamped to [-127, 127]; scale byte ``X + 127``; elements
    ``e4m3_rne_saturating(w / 2^X)``.  An all-zero block gets X = -127.

    The pages name the mode ("MLX 张量并行实战指南" section 2.3: non-affine
    modes such as mode="mxfp8"; section 4: an mxfp8 layer has no biases) but
    not its format; this is the OCP MX reading, and both the oracle and the
    kernels decode it themselves.

    Returns (codes uint8 (out, in), scales uint8 (out, in / block))."""
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    out, inn = w.shape
    assert inn % block == 0
    g = w.reshape(out, inn // block, block)
    amax = np.abs(g).max(axis=2)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, np.clip(e2 - 1 - 8, -127, 127), -127)
    codes = e4m3_encode(g / np.ldexp(1.0, X)[..., None])
    return codes.reshape(out, inn), (X + 127).astype(np.uint8)


def pack_q4(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint32)
    out, inn = q.shape
    q8 = q.reshape(out, inn // 8, 8)
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    return np.bitwise_or.reduce(q8 << shifts, axis=2).astype(np.uint32)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass
class MLPInputs:
    """Gated MLP: W_gate, W_up (F, D); W_down (D, F); X (B, D).  MLX layout
    (out, in), y = x W^T."""
    B: int
    D: int
    F: int
    P: int
    dtype: str
    X: np.ndarray
    Wg: np.ndarray
    Wu: np.ndarray
    Wd: np.ndarray
    extra: dict = field(default_factory=dict)


def mlp_inputs(B, D, F, P, dtype=BF16, seed=0, w_bound=None) -> MLPInputs:
    """X ~ N(0, 1); W_gate, W_up ~ U(+-1/sqrt(D)); W_down ~ U(+-1/sqrt(F))
    (fan-in rule) unless ``w_bound`` fixes one bound for all three.
    Seeds: X seed, gate seed+1, up seed+2, down seed+3."""
    bg = w_bound if w_bound is not None else 1.0 / math.sqrt(D)
    bd = w_bound if w_bound is not None else 1.0 / math.sqrt(F)
    X = normal(seed, (B, D), 1.0, dtype)
    Wg = uniform(seed + 1, (F, D), bg, dtype)
    Wu = uniform(seed + 2, (F, D), bg, dtype)
    Wd = uniform(seed + 3, (D, F), bd, dtype)
    return MLPInputs(B, D, F, P, dtype, X, Wg, Wu, Wd)


def worked_example(seed=0):
    """The MLX two-layer example: x (4, 2), l1 all-to-sharded (2 -> 2),
    l2 sharded-to-all (2 -> 2), no bias, two devices; fp32.
    X ~ N(0,1) seed; W1 ~ U(+-1/sqrt 2) seed+1; W2 seed+2."""
    X = normal(seed, (4, 2), 1.0, F32)
    W1 = uniform(seed + 1, (2, 2), 1.0 / math.sqrt(2.0), F32)
    W2 = uniform(seed + 2, (2, 2), 1.0 / math.sqrt(2.0), F32)
    return X, W1, W2


def qkv_weight(D=4096, heads=32, head_dim=128, seed=10, dtype=BF16):
    """Fused [Wq; Wk; Wv] ((3 * heads * head_dim), D) ~ U(+-1/sqrt(D))."""
    return uniform(seed, (3 * heads * head_dim, D), 1.0 / math.sqrt(D), dtype)


def q4_mlp_weights(D=4096, F=14336, seed=20, group_size=64):
    """Three fp32 matrices ~ U(+-1/sqrt(D)) quantized to 4-bit affine.
    Returns dict name -> (packed, scales, biases, q)."""
    bound = 1.0 / math.sqrt(D)
    out = {}
    for i, (name, shape) in enumerate((("gate", (F, D)), ("up", (F, D)), ("down", (D, F)))):
        w = uniform(seed + i, shape, bound, F32)
        out[name] = quantize_q4(w, group_size)
    return out


def summa_inputs(n=8192, seed=30, dtype=BF16):
    """X, A (n, n) ~ N(0, variance 1/sqrt(n)), i.e. std n^(-1/4)."""
    std = n ** -0.25
    return normal(seed, (n, n), std, dtype), normal(seed + 1, (n, n), std, dtype)


def vocab_head_inputs(B=32, H=12288, V=50272, seed=40, dtype=F16):
    """X (B, H) ~ N(0,1); W (V, H) ~ U(+-1/sqrt(H))."""
    return normal(seed, (B, H), 1.0, dtype), uniform(seed + 1, (V, H), 1.0 / math.sqrt(H), dtype)
