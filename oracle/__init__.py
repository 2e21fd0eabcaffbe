"""CPU oracle for the sharded GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, OpenMP over
independent outputs, no BLAS); this module builds it with gcc, decodes the
stored bit patterns of the inputs with the C decoders, and exposes one
Python function per oracle step:

==========  =====================================================  ============================
function    computes                                               pinned by (tests/test_oracle)
==========  =====================================================  ============================
slice_      rank r's shard of a weight, segments rule               index-encoded weights, golden
col         all-to-sharded linear, sharded or gathered output       brute force, unsharded identity
swiglu      silu(g) * u, rounded once to the activation dtype       closed forms
row         sharded-to-all linear: partials, rank-order sum, bias   brute force, unsharded identity
deq4        4-bit affine dequantisation                             hand-packed words, round trip
deq_mx8     MX FP8 dequantisation (E4M3 x E8M0 per 32)              closed forms, hand bytes
summa       q-step block accumulation Y_ij += X_it A_tj             brute force, q-independence
mlp         col(gate), col(up) -> swiglu -> row(down)               composition of the above
col_bwd     VJP of all_to_sharded: dx = all_sum of dY_r W_r, dW_r   finite differences of col,
            = dY_r^T X                                              unsharded identity
row_bwd     VJP of sharded_to_all: dX_r = dY W_r, dW_r = dY^T X_r   finite differences of row,
                                                                    unsharded identity
summa_abt   SUMMA backward dX = dY A^T in q steps (Matmul_ABT_2D)  finite differences of summa
summa_atb   SUMMA backward dA = X^T dY in q steps (Matmul_ATB_2D)  finite differences of summa
all_gather  input shards (P, B, k) -> (B, P k), rank order          index arrays, brute force
reduce_     summed (B, n) result -> (P, B, n/P), rank r's columns   index arrays, brute force
 scatter
==========  =====================================================  ============================

Every function accepts stored arrays (float32, float64, or uint16 bit
patterns with a dtype tag) and returns float64.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F16, F64 = 0, 1, 2, 3
_DT = {"f32": F32, "bf16": BF16, "f16": F16, "f64": F64}


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"oracle {what} failed with status {code}")
        self.code = code


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (C11, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        P, I64, I = C.c_void_p, C.c_int64, C.c_int
        sig = {
            "or_decode": [P, I, I64, P],
            "or_slice": [P, I64, I64, I64, I, I, I, I, P],
            "or_col": [P, I64, I64, P, I64, P, I, I, I, P],
            "or_swiglu": [P, P, I64, I, P],
            "or_row": [P, I64, I64, P, I64, P, I, P, P],
            "or_deq4": [P, P, P, I64, I64, I, P],
            "or_deqmx8": [P, P, I64, I64, I, P],
            "or_summa": [P, P, I64, I64, I64, I, P],
            "or_mlp": [P, I64, I64, I64, P, P, P, I, I, P],
            "or_col_bwd": [P, I64, I64, P, I64, P, I, I, P, P],
            "or_row_bwd": [P, I64, I64, P, I64, P, I, P, P],
            "or_summa_abt": [P, P, I64, I64, I64, I, P],
            "or_summa_atb": [P, P, I64, I64, I64, I, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.or_threads.argtypes = []
        L.or_threads.restype = C.c_int
        L.or_round.argtypes = [C.c_double, C.c_int]
        L.or_round.restype = C.c_double
        for name in ("or_e4m3", "or_e8m0"):
            getattr(L, name).argtypes = [C.c_uint8]
            getattr(L, name).restype = C.c_double
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc:
        raise OracleError(rc, what)


def _dtag(a, dtype):
    if dtype is None:
        if a.dtype == np.float32:
            return F32
        if a.dtype == np.float64:
            return F64
        raise ValueError("16-bit inputs need an explicit dtype tag")
    return _DT[dtype] if isinstance(dtype, str) else dtype


def decode(a, dtype=None) -> np.ndarray:
    """Stored array -> float64 using the oracle's own decoders."""
    a = np.ascontiguousarray(a)
    t = _dtag(a, dtype)
    out = np.empty(a.shape, dtype=np.float64)
    _check(lib().or_decode(_p(a), t, a.size, _p(out)), "decode")
    return out


def _f64(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float64:  # already values (e.g. dequantized weights)
        return a
    return decode(a, dtype)


def threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return lib().or_threads()


def round_to(x: float, dtype) -> float:
    return lib().or_round(float(x), _DT[dtype] if isinstance(dtype, str) else dtype)


def slice_(W, axis, S, P, r) -> np.ndarray:
    """Rank r's shard of a 2-D (or 1-D, axis 0) array; bit-exact bytes."""
    W = np.ascontiguousarray(W)
    W2 = W.reshape(W.shape[0], -1) if W.ndim == 1 else W
    rows, cols = W2.shape
    dim = rows if axis == 0 else cols
    if dim % S or (dim // S) % P:
        raise OracleError(3, "slice")
    shape = (rows // P, cols) if axis == 0 else (rows, cols // P)
    out = np.empty(shape, dtype=W.dtype)
    _check(lib().or_slice(_p(W2), W.itemsize, rows, cols, axis, S, P, r, _p(out)), "slice")
    return out.reshape(-1) if W.ndim == 1 else out


def col(X, W, P, S=1, bias=None, gather=False, dtype=None) -> np.ndarray:
    """All-to-sharded: (P, B, out/P), or (B, out) when gathered."""
    X, W, b = _f64(X, dtype), _f64(W, dtype), _f64(bias, dtype)
    B, inn = X.shape
    out = W.shape[0]
    if out % S or (out // S) % P:
        raise OracleError(3, "col")
    Y = np.empty((B, out) if gather else (P, B, out // P), dtype=np.float64)
    _check(lib().or_col(_p(X), B, inn, _p(W), out, _p(b), S, P, int(gather), _p(Y)), "col")
    return Y


def swiglu(g, u, round_dtype="f64") -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    h = np.empty_like(g)
    _check(lib().or_swiglu(_p(g), _p(u), g.size, _DT[round_dtype], _p(h)), "swiglu")
    return h


def row(Xs, W, P, bias=None, dtype=None, partials=False):
    """Sharded-to-all: Xs (P, B, in/P) -> Y (B, out) [and Z (P, B, out)]."""
    Xs, W, b = _f64(Xs, dtype), _f64(W, dtype), _f64(bias, dtype)
    Pp, B, kl = Xs.shape
    assert Pp == P
    out, inn = W.shape
    if inn % P:
        raise OracleError(3, "row")
    Y = np.empty((B, out), dtype=np.float64)
    Z = np.empty((P, B, out), dtype=np.float64) if partials else None
    _check(lib().or_row(_p(Xs), B, inn, _p(W), out, _p(b), P, _p(Y), _p(Z)), "row")
    return (Y, Z) if partials else Y


def deq4(packed, scales, biases, group_size=64) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    out = packed.shape[0]
    inn = packed.shape[1] * 8
    W = np.empty((out, inn), dtype=np.float64)
    _check(lib().or_deq4(_p(packed), _p(scales), _p(biases), out, inn, group_size, _p(W)), "deq4")
    return W


def e4m3(b: int) -> float:
    return float(lib().or_e4m3(int(b)))


def e8m0(x: int) -> float:
    return float(lib().or_e8m0(int(x)))


def deq_mx8(codes, scales, block=32) -> np.ndarray:
    """w[o, k] = 2^(scales[o, k / block] - 127) * e4m3(codes[o, k])."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out, inn = codes.shape
    W = np.empty((out, inn), dtype=np.float64)
    _check(lib().or_deqmx8(_p(codes), _p(scales), out, inn, block, _p(W)), "deq_mx8")
    return W


def summa(X, A, q, dtype=None) -> np.ndarray:
    X, A = _f64(X, dtype), _f64(A, dtype)
    M, K = X.shape
    K2, N = A.shape
    assert K == K2
    Y = np.empty((M, N), dtype=np.float64)
    _check(lib().or_summa(_p(X), _p(A), M, K, N, q, _p(Y)), "summa")
    return Y


def mlp(X, Wg, Wu, Wd, P, round_dtype="bf16", dtype=None) -> np.ndarray:
    X, Wg, Wu, Wd = (_f64(a, dtype) for a in (X, Wg, Wu, Wd))
    B, D = X.shape
    F = Wg.shape[0]
    Y = np.empty((B, D), dtype=np.float64)
    _check(lib().or_mlp(_p(X), B, D, F, _p(Wg), _p(Wu), _p(Wd), P, _DT[round_dtype], _p(Y)), "mlp")
    return Y


def col_bwd(X, W, dY, P, S=1, dtype=None):
    """Vector-Jacobian product of the all-to-sharded layer Y_r = X W_r^T (MLX
    tensor-parallel guide, section 2.1 and its sum_gradients wrapper): the
    input X is used by every rank, so its gradient is the all_sum over ranks
    of dY_r W_r (each rank's product formed whole, then summed in rank order);
    rank r's weight gradient is dY_r^T X.  dY: (P, B, out/P) in the layer's
    output layout.  Returns (dx (B, in), dW (P, out/P, in)); dW[r] is laid out
    as slice_(W, 0, S, P, r).  Plain fp64 loops (oracle.c or_col_bwd)."""
    X, W, dY = _f64(X, dtype), _f64(W, dtype), _f64(dY, dtype)
    B, inn = X.shape
    out = W.shape[0]
    if out % S or (out // S) % P:
        raise OracleError(3, "col_bwd")
    dY = np.ascontiguousarray(dY).reshape(P, B, out // P)
    dx = np.empty((B, inn))
    dW = np.empty((P, out // P, inn))
    _check(lib().or_col_bwd(_p(X), B, inn, _p(W), out, _p(dY), S, P, _p(dx), _p(dW)), "col_bwd")
    return dx, dW


def row_bwd(Xs, W, dY, P, dtype=None):
    """Vector-Jacobian product of the sharded-to-all layer Y = sum_r Xs_r W_r^T
    (+ b) (MLX guide, section 2.2): the gradient reaching every rank is the
    full dY, so rank r's input gradient is dY W_r (no communication: it stays
    sharded like Xs) and its weight gradient dY^T Xs_r.  Xs: (P, B, in/P),
    dY: (B, out).  Returns (dXs (P, B, in/P), dW (P, out, in/P)).  Plain fp64
    loops (oracle.c or_row_bwd)."""
    Xs, W, dY = _f64(Xs, dtype), _f64(W, dtype), _f64(dY, dtype)
    out, inn = W.shape
    if inn % P:
        raise OracleError(3, "row_bwd")
    B = dY.shape[0]
    Xs = np.ascontiguousarray(Xs).reshape(P, B, inn // P)
    dXs = np.empty((P, B, inn // P))
    dW = np.empty((P, out, inn // P))
    _check(lib().or_row_bwd(_p(Xs), B, inn, _p(W), out, _p(dY), P, _p(dXs), _p(dW)), "row_bwd")
    return dXs, dW


def summa_abt(dY, A, q, dtype=None) -> np.ndarray:
    """Backward of Y = X A for X: dX = dY A^T, accumulated over the q blocks
    of the shared inner dimension N in order t = 0..q-1 (ColossalAI 2D SUMMA
    page, its Matmul_ABT_2D): dX_ik += dY_it A_kt^T.  dY (M, N), A (K, N).
    Plain fp64 loops (oracle.c or_summa_abt)."""
    dY, A = _f64(dY, dtype), _f64(A, dtype)
    M, N = dY.shape
    K = A.shape[0]
    if A.shape[1] != N:
        raise OracleError(1, "summa_abt")
    dX = np.empty((M, K))
    _check(lib().or_summa_abt(_p(dY), _p(A), M, K, N, q, _p(dX)), "summa_abt")
    return dX


def summa_atb(X, dY, q, dtype=None) -> np.ndarray:
    """Backward of Y = X A for A: dA = X^T dY over the q blocks of the token
    dimension M in order (the page's Matmul_ATB_2D): dA_kj += X_tk^T dY_tj.
    X (M, K), dY (M, N).  Plain fp64 loops (oracle.c or_summa_atb)."""
    X, dY = _f64(X, dtype), _f64(dY, dtype)
    M, K = X.shape
    N = dY.shape[1]
    if dY.shape[0] != M:
        raise OracleError(1, "summa_atb")
    dA = np.empty((K, N))
    _check(lib().or_summa_atb(_p(X), _p(dY), M, K, N, q, _p(dA)), "summa_atb")
    return dA


def all_gather(Xs) -> np.ndarray:
    """AllGather of activation shards ("Sharded Matrices and How to Multiply
    Them", Case 2 and the collective-primitive table: AllGather_X(A[I, J_X])
    -> A[I, J]): Xs (P, B, k), shard r holding feature columns [r k, (r+1) k),
    -> (B, P k).  A pure copy, so stored bit patterns pass through unchanged."""
    Xs = np.asarray(Xs)
    P, B, k = Xs.shape
    out = np.empty((B, P * k), dtype=Xs.dtype)
    for r in range(P):
        out[:, r * k:(r + 1) * k] = Xs[r]
    return out


def reduce_scatter(Y, P) -> np.ndarray:
    """ReduceScatter of the summed result (same page, Case 3 and the primitive
    table: ReduceScatter_{X,K}(C[I, K]{U_X}) -> C[I, K_X]): the reduction is
    done by ``row``; this hands rank r the output columns [r n/P, (r+1) n/P)
    as slice r of (P, B, n/P)."""
    Y = np.asarray(Y)
    B, n = Y.shape
    if n % P:
        raise OracleError(3, "reduce_scatter")
    k = n // P
    out = np.empty((P, B, k), dtype=Y.dtype)
    for r in range(P):
        out[r] = Y[:, r * k:(r + 1) * k]
    return out


# ---------------------------------------------------------------------------
# error metrics for comparing a device result with the fp64 reference
# ---------------------------------------------------------------------------
def ulp(r: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of ``dtype`` numbers around |r| (its unit in the last place)."""
    bits, emin = {"f32": (24, -125), "bf16": (8, -125), "f16": (11, -13)}[dtype]
    a = np.abs(np.asarray(r, dtype=np.float64))
    _, e = np.frexp(a)
    e = np.maximum(e, emin)
    return np.ldexp(1.0, e - bits)


def metrics(y, ref, out_dtype: str) -> dict:
    """relL2, raw max-abs error, rms(ref), and max-abs error in excess of half
    an output ulp (the error a correctly rounded output cannot avoid)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(y - ref)
    nr = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(y - ref)) / nr if nr > 0 else float(np.linalg.norm(y - ref))
    excess = np.maximum(0.0, d - 0.5 * ulp(ref, out_dtype)) if out_dtype != "f64" else d
    return {
        "relL2": rel,
        "maxabs": float(d.max()) if d.size else 0.0,
        "maxabs_ulp": float(excess.max()) if d.size else 0.0,
        "rms": float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0,
    }


def within(m: dict, out_dtype: str) -> bool:
    """Tolerances: fp32 outputs relL2 <= 1e-5; 16-bit outputs relL2 <= 4e-3
    and max error beyond the output's half ulp <= 1e-2 * rms(ref)."""
    if out_dtype in ("f32", "f64"):
        return m["relL2"] <= 1e-5
    return m["relL2"] <= 4e-3 and m["maxabs_ulp"] <= 1e-2 * m["rms"]
