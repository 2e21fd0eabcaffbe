"""Python binding of libshardgemm: the sharded GEMMs of 1-D tensor parallelism
(all-to-sharded, sharded-to-all, their 4-bit affine variants) and SUMMA's
q-step block accumulation, with all P shards of a layer on one MI355X GPU.

This module only marshals arguments: torch supplies device memory and the
current HIP stream, every step of the computation runs in the library's
kernels.  The entry points mirror include/shardgemm.h one to one:

    shard_linear               sg_shard_linear
    shard_quantized_linear     sg_shard_quantized_linear
    shard_mxfp8_linear         sg_shard_mxfp8_linear
    all_to_sharded             sg_all_to_sharded_ex (sg_all_to_sharded's layouts + a sharded input)
    sharded_to_all             sg_sharded_to_all_ex (+ sg_sharded_to_all_workspace; all-reduce or
                               reduce-scatter output)
    mlp                        sg_mlp (+ sg_mlp_workspace): gate|up with SwiGLU, then down
    all_to_sharded_backward    sg_all_to_sharded_backward (dx = rank-order all_sum, dw)
    sharded_to_all_backward    sg_sharded_to_all_backward (sharded dx, dw)
    summa_matmul               sg_summa_matmul (+ sg_summa_workspace)
    summa_backward             sg_summa_backward (Matmul_ABT_2D / Matmul_ATB_2D)
    Layer.info / Layer.shard   sg_layer_info / sg_layer_copy_shard
    time_next_launch           sg_time_next_launch (profiling)

There is no fallback: if the library is not built, importing works but the
first call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libshardgemm.so")

ALL_TO_SHARDED, SHARDED_TO_ALL = 0, 1
IN_FULL, IN_SHARDED = 0, 1
OUT_FULL, OUT_SHARDED = 0, 1
_MODES = {"all-to-sharded": ALL_TO_SHARDED, "sharded-to-all": SHARDED_TO_ALL}
F32, BF16, F16 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_TORCH_DT = {v: k for k, v in _DT.items()}
EPI_NONE, EPI_SWIGLU = 0, 1

OK, ERR_INVALID_ARG, ERR_BAD_MODE, ERR_NOT_DIVISIBLE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_OOM, ERR_HIP = range(8)


class ShardGemmError(RuntimeError):
    """A non-zero sg_status; `code` holds it, the message is sg_last_error()."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[sg_status {code}] {message}")
        self.code = code


class ShardGemmNotBuilt(RuntimeError):
    pass


_lib = None


def lib():
    """The loaded library (ctypes.CDLL) with every entry point typed."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ShardGemmNotBuilt(
                f"{LIB_PATH} is missing: build it first (python -m sharded_gemm_alltosharded_amd._build)")
        L = C.CDLL(LIB_PATH)
        P, I64, I, SZ = C.c_void_p, C.c_int64, C.c_int, C.c_size_t
        PP = C.POINTER(C.c_void_p)
        sig = {
            "sg_shard_linear": ([P, I, I64, I64, P, I, I, I, P, PP], I),
            "sg_shard_quantized_linear": ([P, P, P, I64, I64, I, I, I, P, I, I, I, P, PP], I),
            "sg_shard_mxfp8_linear": ([P, P, I64, I64, I, P, I, I, I, P, PP], I),
            "sg_all_to_sharded": ([P, P, I64, P, I, I, I, P], I),
            "sg_all_to_sharded_ex": ([P, P, I, I64, P, I, I, I, P], I),
            "sg_sharded_to_all": ([P, P, I64, P, I, P, SZ, P], I),
            "sg_sharded_to_all_ex": ([P, P, I64, P, I, I, P, SZ, P], I),
            "sg_all_to_sharded_backward": ([P, P, P, I64, P, I, P, I, P, SZ, P], I),
            "sg_sharded_to_all_backward": ([P, P, P, I64, P, I, P, I, P, SZ, P], I),
            "sg_layer_backward_workspace": ([P, I64], SZ),
            "sg_summa_backward": ([P, P, P, I, I64, I64, I64, I, P, P, P, SZ, P], I),
            "sg_summa_backward_workspace": ([I, I64, I64, I64, I], SZ),
            "sg_mlp": ([P, P, P, I64, P, I, P, SZ, P], I),
            "sg_mlp_workspace": ([P, P, I64], SZ),
            "sg_mlp_static": ([P, P, P, I64, P, I, P], I),
            "sg_sharded_to_all_workspace": ([P, I64], SZ),
            "sg_summa_matmul": ([P, P, I, I64, I64, I64, I, P, I, I, P, SZ, P], I),
            "sg_summa_workspace": ([I, I64, I64, I], SZ),
            "sg_layer_info": ([P, P, P, P, P, P, P, P], I),
            "sg_layer_copy_shard": ([P, I, I, P, SZ, P], I),
            "sg_layer_free": ([P], None),
            "sg_time_next_launch": ([P, P], I),
            "sg_last_error": ([], C.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise ShardGemmError(rc, lib().sg_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device=None):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _mode(sharding) -> int:
    if isinstance(sharding, int):
        return sharding
    # unknown strings reach the library as an invalid mode, which rejects them
    return _MODES.get(sharding, -1)


def time_next_launch(start: "torch.cuda.Event", stop: "torch.cuda.Event"):
    """Arm two timing events for the next kernel this thread launches
    through the library (sg_time_next_launch): they are recorded at that
    kernel's own start and end."""
    for e in (start, stop):
        if e.cuda_event == 0:  # torch creates events lazily
            e.record()
    _check(lib().sg_time_next_launch(C.c_void_p(start.cuda_event), C.c_void_p(stop.cuda_event)))


class Layer:
    """A sharded layer owned by the library (sg_layer*)."""

    def __init__(self, handle: C.c_void_p, device: torch.device):
        self._h = handle
        self.device = device
        o, i, m, s, p, d, q = (C.c_int64(), C.c_int64(), C.c_int(), C.c_int(), C.c_int(), C.c_int(), C.c_int())
        _check(lib().sg_layer_info(self._h, C.byref(o), C.byref(i), C.byref(m), C.byref(s), C.byref(p),
                                   C.byref(d), C.byref(q)))
        self.out_dims, self.in_dims = o.value, i.value
        self.mode, self.segments, self.P = m.value, s.value, p.value
        self.dtype = _TORCH_DT[d.value]
        self.quantized = bool(q.value)
        self.mx = q.value == 2  # MX FP8 layer

    @property
    def handle(self):
        return self._h

    def free(self):
        if self._h is not None and _lib is not None:
            _lib.sg_layer_free(self._h)
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def shard(self, r: int, what: int = 0) -> torch.Tensor:
        """Copy of rank r's stored tensor: 0 weight, 1 bias, 2 scales, 3 biases."""
        if what == 0:
            if self.mx:
                shape, dt = self._wshape(1), torch.uint8
            elif self.quantized:
                shape, dt = self._wshape(8), torch.int32
            else:
                shape, dt = self._wshape(1), self.dtype
        elif what == 1:
            n = self.out_dims // self.P if self.mode == ALL_TO_SHARDED else self.out_dims
            shape, dt = (n,), self.dtype
        elif self.mx:
            shape, dt = self._wshape(32), torch.uint8
        else:
            shape, dt = self._wshape(64), torch.int16
        out = torch.empty(shape, dtype=dt, device=self.device)
        _check(lib().sg_layer_copy_shard(self._h, r, what, _ptr(out), out.numel() * out.element_size(),
                                         _stream(self.device)))
        return out

    def _wshape(self, per):
        if self.mode == ALL_TO_SHARDED:
            return (self.out_dims // self.P, self.in_dims // per)
        return (self.out_dims, self.in_dims // self.P // per)


def shard_linear(weight: torch.Tensor, sharding, segments: int = 1, P: int = 1, bias=None) -> Layer:
    """Shard a dense (out, in) weight over P ranks (sg_shard_linear)."""
    dt = _DT.get(weight.dtype, -1)
    out_dims, in_dims = weight.shape
    weight = weight.contiguous()
    bias = None if bias is None else bias.contiguous()
    h = C.c_void_p()
    dev = weight.device
    _check(lib().sg_shard_linear(_ptr(weight), dt, out_dims, in_dims, _ptr(bias), _mode(sharding), segments, P,
                                 _stream(dev) if dev.type == "cuda" else None, C.byref(h)))
    return Layer(h, dev if dev.type == "cuda" else torch.device("cuda", torch.cuda.current_device()))


def shard_mxfp8_linear(codes: torch.Tensor, scales: torch.Tensor, sharding, segments: int = 1, P: int = 1,
                       act_dtype=torch.bfloat16, bias=None) -> Layer:
    """Shard an MX FP8 layer (sg_shard_mxfp8_linear).  codes: (out, in) uint8
    E4M3; scales: (out, in/32) uint8 E8M0."""
    out_dims, in_dims = codes.shape
    codes, scales = codes.contiguous(), scales.contiguous()
    bias = None if bias is None else bias.contiguous()
    dev = codes.device
    h = C.c_void_p()
    _check(lib().sg_shard_mxfp8_linear(_ptr(codes), _ptr(scales), out_dims, in_dims, _DT.get(act_dtype, -1),
                                       _ptr(bias), _mode(sharding), segments, P,
                                       _stream(dev) if dev.type == "cuda" else None, C.byref(h)))
    return Layer(h, dev if dev.type == "cuda" else torch.device("cuda", torch.cuda.current_device()))


def shard_quantized_linear(wq: torch.Tensor, scales: torch.Tensor, qbiases: torch.Tensor, in_dims: int, sharding,
                           segments: int = 1, P: int = 1, group_size: int = 64, bits: int = 4,
                           act_dtype=torch.bfloat16, bias=None) -> Layer:
    """Shard a 4-bit affine layer (sg_shard_quantized_linear).  wq: (out, in/8)
    int32 words; scales, qbiases: (out, in/group_size) 16-bit fp16 patterns."""
    out_dims = wq.shape[0]
    wq, scales, qbiases = wq.contiguous(), scales.contiguous(), qbiases.contiguous()
    bias = None if bias is None else bias.contiguous()
    dev = wq.device
    h = C.c_void_p()
    _check(lib().sg_shard_quantized_linear(_ptr(wq), _ptr(scales), _ptr(qbiases), out_dims, in_dims, group_size, bits,
                                           _DT.get(act_dtype, -1), _ptr(bias), _mode(sharding), segments, P,
                                           _stream(dev) if dev.type == "cuda" else None, C.byref(h)))
    return Layer(h, dev if dev.type == "cuda" else torch.device("cuda", torch.cuda.current_device()))


def all_to_sharded(layer: Layer, x: torch.Tensor, gather: bool = False, swiglu: bool = False,
                   out_dtype=None, out: torch.Tensor | None = None, x_sharded: bool = False) -> torch.Tensor:
    """x (B, in) -> (P, B, n/P) sharded, or (B, n) gathered; n = out_dims, or
    out_dims/2 with the fused SwiGLU epilogue.  x_sharded: x is (P, B, in/P),
    all-gathered inside the matmul."""
    B = x.shape[1] if x_sharded else x.shape[0]
    n = layer.out_dims // 2 if swiglu else layer.out_dims
    out_dtype = out_dtype or layer.dtype
    if out is None:
        shape = (B, n) if gather else (layer.P, B, n // layer.P)
        out = torch.empty(shape, dtype=out_dtype, device=x.device)
    _check(lib().sg_all_to_sharded_ex(layer.handle, _ptr(x), IN_SHARDED if x_sharded else IN_FULL, B, _ptr(out),
                                      OUT_FULL if gather else OUT_SHARDED, EPI_SWIGLU if swiglu else EPI_NONE,
                                      _DT.get(out.dtype, -1), _stream(x.device)))
    return out


_workspaces: dict = {}


def workspace(layer: Layer, B: int, device) -> torch.Tensor | None:
    """A workspace shared by calls on one device (no initial contents needed)."""
    need = lib().sg_sharded_to_all_workspace(layer.handle, B)
    if need == 0:
        return None
    key = torch.device(device)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=key)
        _workspaces[key] = ws
    return ws


def sharded_to_all(layer: Layer, x_partial: torch.Tensor, out_dtype=None, out: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None, scatter: bool = False) -> torch.Tensor:
    """x_partial (P, B, in/P) -> (B, out): the rank partials summed in rank
    order, bias added once; scatter: the reduce-scatter (P, B, out/P)."""
    B = x_partial.shape[1]
    out_dtype = out_dtype or layer.dtype
    if out is None:
        shape = (layer.P, B, layer.out_dims // layer.P) if scatter else (B, layer.out_dims)
        out = torch.empty(shape, dtype=out_dtype, device=x_partial.device)
    if ws is None:
        ws = workspace(layer, B, x_partial.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sg_sharded_to_all_ex(layer.handle, _ptr(x_partial), B, _ptr(out), OUT_SHARDED if scatter else OUT_FULL,
                                      _DT.get(out.dtype, -1), _ptr(ws), nbytes, _stream(x_partial.device)))
    return out


_mlp_workspaces: dict = {}


def mlp_workspace(gate_up: Layer, down: Layer, B: int, device) -> torch.Tensor | None:
    """A workspace for mlp(), shared by calls on one device (None
    when the layers do not form a gate|up, down pair: sg_mlp then says why)."""
    need = int(lib().sg_mlp_workspace(gate_up.handle, down.handle, B))
    if need == 0:
        return None
    key = torch.device(device)
    ws = _mlp_workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=key)
        _mlp_workspaces[key] = ws
    return ws


def mlp(gate_up: Layer, down: Layer, x: torch.Tensor, out_dtype=None, out: torch.Tensor | None = None,
        ws: torch.Tensor | None = None) -> torch.Tensor:
    """(B, in) -> (B, out): down(silu(x W_gate^T) * (x W_up^T)) through sg_mlp,
    the sharded h kept in the workspace."""
    B = x.shape[0]
    out_dtype = out_dtype or down.dtype
    if out is None:
        out = torch.empty((B, down.out_dims), dtype=out_dtype, device=x.device)
    if ws is None:
        ws = mlp_workspace(gate_up, down, B, x.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sg_mlp(gate_up.handle, down.handle, _ptr(x), B, _ptr(out), _DT.get(out.dtype, -1), _ptr(ws),
                        nbytes, _stream(x.device)))
    return out


MLP_STATIC_SCRATCH_BYTES = 16 << 20  # SG_MLP_STATIC_SCRATCH_BYTES


def mlp_static(gate_up: Layer, down: Layer, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """sg_mlp_static: mlp() without a workspace, for callers that cannot
    allocate (the library's per-device static scratch holds h).  The caller
    passes the output; this wrapper allocates nothing."""
    _check(lib().sg_mlp_static(gate_up.handle, down.handle, _ptr(x), x.shape[0], _ptr(out), _DT.get(out.dtype, -1),
                               _stream(x.device)))
    return out


def _bwd_ws(layer: Layer, B: int, ws, device):
    """The weight-gradient workspace: "auto" takes sg_layer_backward_workspace
    bytes from torch's caching allocator (stream-ordered), None runs the
    weight gradient on the vector units, or a uint8 device tensor."""
    if isinstance(ws, str):
        n = int(lib().sg_layer_backward_workspace(layer.handle, B))
        ws = torch.empty(n, dtype=torch.uint8, device=device) if n else None
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def all_to_sharded_backward(layer: Layer, x: torch.Tensor | None, dy: torch.Tensor, need_dx: bool = True,
                            need_dw: bool = True, dx_dtype=None, dw_dtype=torch.float32, ws="auto"):
    """Backward of an all-to-sharded layer (sg_all_to_sharded_backward): dy
    (P, B, out/P) -> (dx (B, in) = the rank-order all_sum of dy[r] W_r,
    dw (P, out/P, in), dw[r] = dy[r]^T x); either may be skipped (None)."""
    B = dy.shape[1]
    dx = torch.empty((B, layer.in_dims), dtype=dx_dtype or layer.dtype, device=dy.device) if need_dx else None
    dw = torch.empty((layer.P, layer.out_dims // layer.P, layer.in_dims), dtype=dw_dtype,
                     device=dy.device) if need_dw else None
    ws, nbytes = _bwd_ws(layer, B, ws if need_dw else None, dy.device)
    _check(lib().sg_all_to_sharded_backward(layer.handle, _ptr(x), _ptr(dy), B, _ptr(dx),
                                            _DT.get(dx.dtype if dx is not None else layer.dtype, -1), _ptr(dw),
                                            _DT.get(dw_dtype, -1), _ptr(ws), nbytes, _stream(dy.device)))
    return dx, dw


def sharded_to_all_backward(layer: Layer, x_partial: torch.Tensor | None, dy: torch.Tensor, need_dx: bool = True,
                            need_dw: bool = True, dx_dtype=None, dw_dtype=torch.float32, ws="auto"):
    """Backward of a sharded-to-all layer (sg_sharded_to_all_backward): dy
    (B, out) -> (dx_partial (P, B, in/P), slice r = dy W_r; dw (P, out, in/P),
    dw[r] = dy^T x_partial[r]); either may be skipped (None)."""
    B = dy.shape[0]
    dx = torch.empty((layer.P, B, layer.in_dims // layer.P), dtype=dx_dtype or layer.dtype,
                     device=dy.device) if need_dx else None
    dw = torch.empty((layer.P, layer.out_dims, layer.in_dims // layer.P), dtype=dw_dtype,
                     device=dy.device) if need_dw else None
    ws, nbytes = _bwd_ws(layer, B, ws if need_dw else None, dy.device)
    _check(lib().sg_sharded_to_all_backward(layer.handle, _ptr(x_partial), _ptr(dy), B, _ptr(dx),
                                            _DT.get(dx.dtype if dx is not None else layer.dtype, -1), _ptr(dw),
                                            _DT.get(dw_dtype, -1), _ptr(ws), nbytes, _stream(dy.device)))
    return dx, dw


def summa_backward(X: torch.Tensor, A: torch.Tensor, dY: torch.Tensor, q: int, need_dx: bool = True,
                   need_da: bool = True, ws="auto"):
    """Gradients of Y = X A in q SUMMA steps (sg_summa_backward): dX = dY A^T
    (M, K) and dA = X^T dY (K, N), both fp32; either may be skipped (None).
    ws: "auto" (sg_summa_backward_workspace bytes from torch's allocator), None
    (dA on the vector units) or a uint8 device tensor."""
    M, K = X.shape
    N = A.shape[1]
    dX = torch.empty((M, K), dtype=torch.float32, device=dY.device) if need_dx else None
    dA = torch.empty((K, N), dtype=torch.float32, device=dY.device) if need_da else None
    if isinstance(ws, str):
        n = int(lib().sg_summa_backward_workspace(_DT.get(X.dtype, -1), M, K, N, q)) if need_da else 0
        ws = torch.empty(n, dtype=torch.uint8, device=dY.device) if n else None
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sg_summa_backward(_ptr(X), _ptr(A), _ptr(dY), _DT.get(X.dtype, -1), M, K, N, q, _ptr(dX), _ptr(dA),
                                   _ptr(ws), nbytes, _stream(dY.device)))
    return dX, dA


def summa_workspace(dtype: torch.dtype, K: int, N: int, q: int) -> int:
    """Bytes of workspace summa_matmul can use (0: it reads A in place)."""
    return int(lib().sg_summa_workspace(_DT.get(dtype, -1), K, N, q))


def summa_matmul(X: torch.Tensor, A: torch.Tensor, q: int, out: torch.Tensor | None = None,
                 accumulate: bool = False, fused: bool = True, workspace="auto") -> torch.Tensor:
    """Y (M, N) fp32 = X A (or Y += X A) on a q x q block grid.

    workspace: "auto" takes summa_workspace(...) bytes from torch's caching
    allocator for this call (stream-ordered, so the memory is reused only by
    later work on the same stream); None makes the kernels read A in place; or
    a uint8 device tensor of at least that size."""
    M, K = X.shape
    N = A.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        need = summa_workspace(X.dtype, K, N, q)
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device) if need else None
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sg_summa_matmul(_ptr(X), _ptr(A), _DT.get(X.dtype, -1), M, K, N, q, _ptr(out), int(accumulate),
                                 int(fused), ws_ptr, ws_bytes, _stream(X.device)))
    return out
