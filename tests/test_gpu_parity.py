"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.  Shapes are small enough for the oracle but span several
tiles with ragged tails, and exercise every kernel family (generic, MFMA
tiles 256/128 with and without the rank split, the streaming kernel, the
4-bit kernel) and every epilogue (sharded / gathered store, SwiGLU, fused
rank sum, fp32 accumulate)."""
import numpy as np
import pytest
import torch

import oracle
import sharded_gemm_alltosharded_amd as sg
import synth
from gpu_util import assert_close, bits, dev, to_dev, to_np

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sg.lib()


def _print_case(**kw):
    print("case:", ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# ---------------------------------------------------------------------------
# slicing: stored shards are the oracle's slices, bit for bit
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mode,out,inn,S,P", [
    (0, 24, 16, 1, 2), (0, 48, 8, 3, 4), (0, 12, 5, 2, 3), (1, 6, 32, 1, 4), (1, 5, 24, 3, 2), (1, 4, 16, 2, 2)])
def test_slicing_bit_exact(dtype, mode, out, inn, S, P):
    _print_case(dtype=dtype, mode=mode, out=out, inn=inn, S=S, P=P)
    W = synth.uniform(1, (out, inn), 1.0, dtype)
    b = synth.uniform(2, (out,), 1.0, dtype)
    layer = sg.shard_linear(to_dev(W, dtype), mode, segments=S, P=P, bias=to_dev(b, dtype))
    for r in range(P):
        np.testing.assert_array_equal(bits(layer.shard(r, 0)), oracle.slice_(W, mode, S, P, r))
        want_b = oracle.slice_(b, 0, S, P, r) if mode == 0 else b
        np.testing.assert_array_equal(bits(layer.shard(r, 1)), want_b)


@pytest.mark.parametrize("mode,out,inn,S,P", [(0, 64, 256, 1, 4), (0, 96, 128, 3, 2), (1, 32, 512, 1, 4), (1, 16, 512, 2, 2),
                                               (1, 64, 1024, 1, 4), (0, 128, 512, 2, 2)])
def test_slicing_q4_bit_exact(mode, out, inn, S, P):
    _print_case(mode=mode, out=out, inn=inn, S=S, P=P)
    packed, s, b, _ = synth.quantize_q4(synth.uniform(3, (out, inn), 0.1, "f32"), 64)
    layer = sg.shard_quantized_linear(torch.from_numpy(packed.view(np.int32)).to(dev()),
                                      torch.from_numpy(s.view(np.int16)).to(dev()),
                                      torch.from_numpy(b.view(np.int16)).to(dev()), inn, mode, segments=S, P=P)
    for r in range(P):
        np.testing.assert_array_equal(layer.shard(r, 0).cpu().numpy().view(np.uint32), oracle.slice_(packed, mode, S, P, r))
        np.testing.assert_array_equal(bits(layer.shard(r, 2)), oracle.slice_(s, mode, S, P, r))
        np.testing.assert_array_equal(bits(layer.shard(r, 3)), oracle.slice_(b, mode, S, P, r))


# ---------------------------------------------------------------------------
# config 1: the worked example and the small fp32 MLP
# ---------------------------------------------------------------------------
def test_worked_example_fp32():
    X, W1, W2 = synth.worked_example(seed=0)
    l1 = sg.shard_linear(to_dev(W1, "f32"), "all-to-sharded", P=2)
    l2 = sg.shard_linear(to_dev(W2, "f32"), "sharded-to-all", P=2)
    y1 = sg.all_to_sharded(l1, to_dev(X, "f32"))
    assert tuple(y1.shape) == (2, 4, 1)  # each device: (4, 1)
    y2 = sg.sharded_to_all(l2, y1)  # the sharded output feeds the next layer as is
    assert tuple(y2.shape) == (4, 2)
    r1 = oracle.col(X, W1, P=2)
    assert_close(y1, r1, "f32", "l1")
    assert_close(y2, oracle.row(r1, W2, P=2), "f32", "l2")
    # and the chain equals the unsharded model
    assert_close(y2, X.astype(np.float64) @ W1.T.astype(np.float64) @ W2.T.astype(np.float64), "f32", "unsharded")


def test_config1_mlp_fp32():
    inp = synth.mlp_inputs(8, 64, 256, 2, "f32", seed=0)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), "f32"), "all-to-sharded", segments=2, P=2)
    dn = sg.shard_linear(to_dev(inp.Wd, "f32"), "sharded-to-all", P=2)
    h = sg.all_to_sharded(gu, to_dev(inp.X, "f32"), swiglu=True)
    y = sg.sharded_to_all(dn, h)
    ref = oracle.mlp(inp.X, inp.Wg, inp.Wu, inp.Wd, 2, round_dtype="f32")
    assert_close(y, ref, "f32", "mlp fp32")


# ---------------------------------------------------------------------------
# all-to-sharded
# ---------------------------------------------------------------------------
COL_CASES = [
    # dtype, B, in, out, S, P   (path chosen by B: <= 16 streaming; 17-256 the few-token tiles of
    # 64, 128 or 256 tokens when K is a multiple of 32, else streaming up to 32 tokens and the
    # 128 x 128 tiles beyond; beyond 256 the ping-pong kernel)
    ("bf16", 1, 256, 96, 1, 2), ("bf16", 5, 512, 192, 3, 2), ("bf16", 16, 4096, 448, 1, 8), ("bf16", 32, 200, 64, 2, 2),
    ("f16", 17, 1024, 320, 1, 4), ("bf16", 33, 264, 384, 1, 3), ("bf16", 130, 512, 640, 1, 4),
    ("bf16", 50, 1024, 512, 2, 4), ("f16", 100, 256, 384, 1, 2),
    ("bf16", 64, 256, 200, 1, 2),  # out % 16 != 0: row-major weights on the few-token tiles (32-wide k)
    ("bf16", 70, 96, 256, 1, 2),   # K = 96: the few-token tiles' 32-wide k tiles (64-wide elsewhere)
    ("f16", 300, 128, 1000, 1, 5), ("bf16", 520, 640, 768, 3, 2), ("bf16", 777, 256, 1100, 1, 2),
    ("bf16", 12, 24, 40, 1, 2), ("bf16", 3, 10, 4, 1, 2),  # K not a multiple of 8: generic path
]


@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("case", COL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_all_to_sharded(case, gather):
    dtype, B, inn, out, S, P = case
    _print_case(dtype=dtype, B=B, inn=inn, out=out, S=S, P=P, gather=gather)
    X = synth.normal(5, (B, inn), 1.0, dtype)
    W = synth.uniform(6, (out, inn), 1 / np.sqrt(inn), dtype)
    bias = synth.uniform(7, (out,), 0.5, dtype) if B % 2 else None
    layer = sg.shard_linear(to_dev(W, dtype), "all-to-sharded", segments=S, P=P,
                            bias=None if bias is None else to_dev(bias, dtype))
    ref = oracle.col(X, W, P=P, S=S, bias=bias, gather=gather, dtype=dtype)
    y32 = sg.all_to_sharded(layer, to_dev(X, dtype), gather=gather, out_dtype=torch.float32)
    assert_close(y32, ref, "f32", "fp32 out")
    y = sg.all_to_sharded(layer, to_dev(X, dtype), gather=gather)
    assert_close(y, ref, dtype, "16-bit out")


SWIGLU_CASES = [("bf16", 1, 256, 128, 2), ("bf16", 16, 512, 448, 4), ("f16", 31, 256, 96, 3),
                ("f16", 24, 200, 96, 3),  # K = 200: streaming with two token tiles
                ("bf16", 40, 256, 512, 2), ("bf16", 600, 384, 640, 4), ("f16", 513, 128, 384, 2),
                ("f16", 120, 512, 768, 4), ("bf16", 100, 256, 400, 4),  # few-token tiles (100 outputs per rank)
                ("f16", 200, 512, 768, 4)]  # few-token 256-token tiles


@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("case", SWIGLU_CASES, ids=lambda c: "-".join(map(str, c)))
def test_swiglu_epilogue(case, gather):
    dtype, B, D, F, P = case
    _print_case(dtype=dtype, B=B, D=D, F=F, P=P, gather=gather)
    inp = synth.mlp_inputs(B, D, F, P, dtype, seed=8)
    layer = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), dtype), "all-to-sharded", segments=2, P=P)
    x = to_dev(inp.X, dtype)
    g = oracle.col(inp.X, inp.Wg, P=P, gather=gather, dtype=dtype)
    u = oracle.col(inp.X, inp.Wu, P=P, gather=gather, dtype=dtype)
    h32 = sg.all_to_sharded(layer, x, gather=gather, swiglu=True, out_dtype=torch.float32)
    assert_close(h32, oracle.swiglu(g, u, "f64"), "f32", "fp32 h")
    h = sg.all_to_sharded(layer, x, gather=gather, swiglu=True)
    assert_close(h, oracle.swiglu(g, u, "f64"), dtype, "16-bit h")  # against the exact product


# ---------------------------------------------------------------------------
# sharded-to-all (fused rank sum)
# ---------------------------------------------------------------------------
ROW_CASES = [
    ("bf16", 1, 512, 96, 2), ("bf16", 16, 14336 // 4, 256, 8), ("f16", 29, 768, 200, 3), ("bf16", 8, 256, 64, 1),
    ("bf16", 24, 200, 128, 5),     # 40 inputs per rank: streaming with two token tiles
    ("bf16", 20, 1024, 4096, 8),   # few-token 64-token tiles from 17 tokens, rank split
    ("bf16", 100, 512, 256, 4),    # few-token 128-token tiles, rank split (2 tiles, 4 groups)
    ("bf16", 40, 1024, 4096, 8),   # few-token 64-token tiles, rank split (32 tiles, 8 groups)
    ("f16", 200, 512, 1024, 4),    # few-token 256-token tiles, rank split (8 tiles, 4 groups)
    ("bf16", 256, 128, 9216, 2),   # few-token 256-token tiles, 72 tiles: split into 2 groups
    ("bf16", 96, 256, 36864, 2),   # few-token 128-token tiles, 288 tiles: no split
    ("f16", 600, 256, 512, 4),     # ping-pong tile, rank split
    ("bf16", 1000, 1024, 4096, 8),  # ping-pong tile, 64 tiles: split into 4 groups of 2 ranks (256 CUs)
    ("f16", 1800, 256, 4096, 4),   # ping-pong tile, 128 tiles: split into 2 groups of 2 ranks (256 CUs)
    ("bf16", 1100, 320, 4096, 8),  # rank width 40 (not a multiple of 32): register-staged 256 tile, 4 groups
    ("bf16", 2304, 128, 4096, 2),  # ping-pong tile, no split (144 tiles)
    ("bf16", 7, 12, 9, 2),         # generic
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "-".join(map(str, c)))
def test_sharded_to_all(case):
    dtype, B, inn, out, P = case
    _print_case(dtype=dtype, B=B, inn=inn, out=out, P=P)
    Xf = synth.normal(9, (B, inn), 1.0, dtype)
    W = synth.uniform(10, (out, inn), 1 / np.sqrt(inn), dtype)
    bias = synth.uniform(11, (out,), 0.5, dtype) if B % 2 == 0 else None
    kl = inn // P
    Xs = np.ascontiguousarray(np.stack([Xf[:, r * kl:(r + 1) * kl] for r in range(P)]))
    layer = sg.shard_linear(to_dev(W, dtype), "sharded-to-all", P=P, bias=None if bias is None else to_dev(bias, dtype))
    ref = oracle.row(Xs, W, P=P, bias=bias, dtype=dtype)
    xs = to_dev(Xs, dtype)
    y32 = sg.sharded_to_all(layer, xs, out_dtype=torch.float32)
    assert_close(y32, ref, "f32", "fp32 out")
    y = sg.sharded_to_all(layer, xs)
    assert_close(y, ref, dtype, "16-bit out")
    # deterministic: the same bits on a second call
    y2 = sg.sharded_to_all(layer, xs, out_dtype=torch.float32)
    assert torch.equal(y32, y2)


def test_mlp_chain_bf16():
    """column (gate|up, SwiGLU) -> row (down): one fused reduction for the chain."""
    B, D, F, P = 16, 512, 1024, 8
    inp = synth.mlp_inputs(B, D, F, P, "bf16", seed=12)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), "bf16"), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, "bf16"), "sharded-to-all", P=P)
    y = sg.sharded_to_all(dn, sg.all_to_sharded(gu, to_dev(inp.X, "bf16"), swiglu=True))
    ref = oracle.mlp(inp.X, inp.Wg, inp.Wu, inp.Wd, P, round_dtype="bf16", dtype="bf16")
    assert_close(y, ref, "bf16", "mlp")


# sg_mlp: the same chain with h kept (fragment-major on the streaming path) in
# the workspace.  The kernels and their arithmetic are those of the separate
# calls, so the results must agree bit for bit; B = 40 takes the tile kernels
# and the row-major h.
MLP_CASES = [("bf16", 1, 512, 1024, 4), ("bf16", 16, 512, 1024, 8), ("f16", 20, 256, 512, 2),
             ("bf16", 32, 512, 1024, 4), ("bf16", 7, 256, 768, 3), ("bf16", 40, 256, 512, 2)]


@pytest.mark.parametrize("case", MLP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_mlp_entry_point(case):
    dtype, B, D, F, P = case
    _print_case(dtype=dtype, B=B, D=D, F=F, P=P)
    inp = synth.mlp_inputs(B, D, F, P, dtype, seed=31)
    bd = synth.uniform(32, (D,), 0.5, dtype)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), dtype), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, dtype), "sharded-to-all", P=P, bias=to_dev(bd, dtype))
    x = to_dev(inp.X, dtype)
    y = sg.mlp(gu, dn, x, out_dtype=torch.float32)
    h = sg.all_to_sharded(gu, x, swiglu=True)
    assert torch.equal(y, sg.sharded_to_all(dn, h, out_dtype=torch.float32))
    assert torch.equal(y, sg.mlp(gu, dn, x, out_dtype=torch.float32))  # the workspace carries no state
    g = oracle.col(inp.X, inp.Wg, P=P, dtype=dtype)
    u = oracle.col(inp.X, inp.Wu, P=P, dtype=dtype)
    ref = oracle.row(oracle.swiglu(g, u, dtype), inp.Wd, P=P, bias=bd, dtype=dtype)
    assert_close(y, ref, "f32", "mlp")
    y16 = sg.mlp(gu, dn, x)
    assert torch.equal(y16, sg.sharded_to_all(dn, h))


@pytest.mark.parametrize("B", [1, 8, 16, 32, 40, 200])
def test_mlp_entry_point_quantized(B):
    """MX FP8 and 4-bit layers against the separate calls, bitwise: up to 32
    tokens the streaming kernels with h fragment-major in each down kernel's k
    order, beyond that the tile kernels (the 4-bit down layer split by rank
    through the fused call's workspace)."""
    D, F, P = 512, 1024, 4
    _print_case(B=B, D=D, F=F, P=P)
    ws = [synth.uniform(33 + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    X = to_dev(synth.normal(36, (B, D), 1.0, "bf16"), "bf16")
    gu, _, _, _ = _mx_layer(np.concatenate([ws[0], ws[1]]), 0, P, S=2)
    dn, _, _, _ = _mx_layer(ws[2], 1, P)
    assert torch.equal(sg.mlp(gu, dn, X), sg.sharded_to_all(dn, sg.all_to_sharded(gu, X, swiglu=True)))
    qgu, _ = _q4_layer(np.concatenate([ws[0], ws[1]]), 0, P, S=2)
    qdn, _ = _q4_layer(ws[2], 1, P)
    assert torch.equal(sg.mlp(qgu, qdn, X), sg.sharded_to_all(qdn, sg.all_to_sharded(qgu, X, swiglu=True)))


def test_mlp_shared_workspace_across_sizes():
    """One workspace for calls of different B: the fallback path at B = 40
    (its down layer splits by rank, partial tiles at the workspace's start)
    and the fragment-major path at B = 16 alternate; every call matches the
    separate calls bit for bit."""
    D, F, P = 256, 512, 2
    inp = synth.mlp_inputs(40, D, F, P, "bf16", seed=40)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), "bf16"), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, "bf16"), "sharded-to-all", P=P)
    need = max(sg.lib().sg_mlp_workspace(gu.handle, dn.handle, b) for b in (16, 40))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    for B in (40, 16, 40, 16, 40):
        _print_case(B=B)
        x = to_dev(inp.X[:B], "bf16")
        y = sg.mlp(gu, dn, x, out_dtype=torch.float32, ws=ws)
        ref = sg.sharded_to_all(dn, sg.all_to_sharded(gu, x, swiglu=True), out_dtype=torch.float32)
        assert torch.equal(y, ref), B


def test_mlp_rejections():
    D, F = 256, 512
    w = to_dev(synth.uniform(37, (2 * F, D), 1 / 16, "bf16"), "bf16")
    wd = to_dev(synth.uniform(38, (D, F), 1 / 16, "bf16"), "bf16")
    gu = sg.shard_linear(w, "all-to-sharded", segments=2, P=2)
    dn = sg.shard_linear(wd, "sharded-to-all", P=2)
    x = to_dev(synth.normal(39, (4, D), 1.0, "bf16"), "bf16")
    for a, b in [(dn, gu), (gu, sg.shard_linear(wd, "sharded-to-all", P=4)),
                 (sg.shard_linear(w, "all-to-sharded", segments=1, P=2), dn)]:
        with pytest.raises(sg.ShardGemmError):
            sg.mlp(a, b, x)
    need = sg.lib().sg_mlp_workspace(gu.handle, dn.handle, 4)
    assert need > 0
    with pytest.raises(sg.ShardGemmError, match="workspace"):
        sg.mlp(gu, dn, x, ws=torch.zeros(need - 16, dtype=torch.uint8, device=dev()))


def test_qkv_segments():
    """Fused [Wq; Wk; Wv] with segments = 3: rank r holds [Q_r; K_r; V_r]."""
    B, D, heads, hd, P = 64, 256, 8, 32, 4
    W = synth.uniform(13, (3 * heads * hd, D), 1 / 16, "bf16")
    X = synth.normal(14, (B, D), 1.0, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "all-to-sharded", segments=3, P=P)
    y = sg.all_to_sharded(layer, to_dev(X, "bf16"), out_dtype=torch.float32)
    assert tuple(y.shape) == (P, B, 3 * heads * hd // P)
    assert_close(y, oracle.col(X, W, P=P, S=3, dtype="bf16"), "f32", "qkv")
    # rank r's first heads/P*hd columns are its query heads
    q_full = oracle.col(X, W[:heads * hd], P=P, dtype="bf16")
    assert_close(y[:, :, :heads * hd // P], q_full, "f32", "q heads")


# ---------------------------------------------------------------------------
# 4-bit affine
# ---------------------------------------------------------------------------
def _q4_layer(w, mode, P, S=1, act=torch.bfloat16):
    packed, s, b, _ = synth.quantize_q4(w, 64)
    layer = sg.shard_quantized_linear(torch.from_numpy(packed.view(np.int32)).to(dev()),
                                      torch.from_numpy(s.view(np.int16)).to(dev()),
                                      torch.from_numpy(b.view(np.int16)).to(dev()), w.shape[1], mode,
                                      segments=S, P=P, act_dtype=act)
    return layer, oracle.deq4(packed, s, b, 64)


@pytest.mark.parametrize("B", [1, 8, 13, 32, 40, 100, 300])  # > 32 tokens: the 4-bit tile kernel
def test_q4_all_to_sharded(B):
    _print_case(B=B)
    D, out, P = 512, 384, 4
    layer, Wd = _q4_layer(synth.uniform(15, (out, D), 1 / np.sqrt(D), "f32"), 0, P)
    X = synth.normal(16, (B, D), 1.0, "bf16")
    ref = oracle.col(X, Wd, P=P, dtype="bf16")
    assert_close(sg.all_to_sharded(layer, to_dev(X, "bf16"), out_dtype=torch.float32), ref, "f32", "q4 col")


@pytest.mark.parametrize("B", [1, 8, 13, 24, 32, 48, 300])
def test_q4_swiglu_and_row(B):
    _print_case(B=B)
    D, F, P = 512, 1024, 4
    ws = [synth.uniform(17 + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    gu, Wgu = _q4_layer(np.concatenate([ws[0], ws[1]]), 0, P, S=2)
    dn, Wdn = _q4_layer(ws[2], 1, P)
    X = synth.normal(20, (B, D), 1.0, "bf16")
    h = sg.all_to_sharded(gu, to_dev(X, "bf16"), swiglu=True)
    g = oracle.col(X, Wgu[:F], P=P, dtype="bf16")
    u = oracle.col(X, Wgu[F:], P=P, dtype="bf16")
    h_ref = oracle.swiglu(g, u, "bf16")  # what the next layer consumes
    assert_close(h, oracle.swiglu(g, u, "f64"), "bf16", "q4 h")
    # the chain against the oracle's own chain (h stored in bf16 on both sides)
    y = sg.sharded_to_all(dn, h)
    assert_close(y, oracle.row(h_ref, Wdn, P=P), "bf16", "q4 down")


# ---------------------------------------------------------------------------
# SUMMA
# ---------------------------------------------------------------------------
SUMMA_CASES = [("bf16", 256, 256, 256, 2), ("bf16", 512, 384, 768, 4), ("f16", 320, 512, 256, 1),
               ("bf16", 1024, 512, 512, 4), ("bf16", 600, 256, 272, 2), ("bf16", 96, 64, 48, 2),
               ("bf16", 12, 6, 10, 2)]


@pytest.mark.parametrize("ws", ["auto", None], ids=["transposed-copy", "in-place"])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("case", SUMMA_CASES, ids=lambda c: "-".join(map(str, c)))
def test_summa(case, fused, ws):
    """Both operand paths: A copied to fragment-major A_t^T blocks in a
    workspace (where the sizes allow), or read in place."""
    dtype, M, K, N, q = case
    _print_case(dtype=dtype, M=M, K=K, N=N, q=q, fused=fused, ws=ws)
    X = synth.normal(21, (M, K), K ** -0.25, dtype)
    A = synth.normal(22, (K, N), K ** -0.25, dtype)
    ref = oracle.summa(X, A, q, dtype=dtype)
    y = sg.summa_matmul(to_dev(X, dtype), to_dev(A, dtype), q, fused=fused, workspace=ws)
    assert_close(y, ref, "f32", "summa")
    C0 = synth.normal(23, (M, N), 1.0, "f32")
    yc = to_dev(C0, "f32")
    sg.summa_matmul(to_dev(X, dtype), to_dev(A, dtype), q, out=yc, accumulate=True, fused=fused, workspace=ws)
    assert_close(yc, ref + C0.astype(np.float64), "f32", "summa accumulate")


def test_summa_workspace_reuse():
    """One workspace tensor serves calls of different shapes (no initialisation needed)."""
    ws = torch.full((sg.summa_workspace(torch.bfloat16, 512, 768, 4),), 0x7f, dtype=torch.uint8, device=dev())
    for (M, K, N, q) in ((512, 512, 768, 4), (256, 256, 256, 2)):
        X = synth.normal(31, (M, K), K ** -0.25, "bf16")
        A = synth.normal(32, (K, N), K ** -0.25, "bf16")
        y = sg.summa_matmul(to_dev(X, "bf16"), to_dev(A, "bf16"), q, workspace=ws)
        assert_close(y, oracle.summa(X, A, q, dtype="bf16"), "f32", "summa")


# ---------------------------------------------------------------------------
# exactness on small integers: every product and partial sum is exact in
# fp32, so the GPU result must equal the oracle bit for bit
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B", [4, 32, 96, 640])
def test_integer_exact_dense(B):
    _print_case(B=B)
    inn, out, P = 256, 512, 4
    X = synth.small_ints(24, (B, inn), -2, 2, "bf16")
    W = synth.small_ints(25, (out, inn), -2, 2, "bf16")
    lc = sg.shard_linear(to_dev(W, "bf16"), "all-to-sharded", P=P)
    y = sg.all_to_sharded(lc, to_dev(X, "bf16"), gather=True, out_dtype=torch.float32)
    np.testing.assert_array_equal(to_np(y), oracle.col(X, W, P=P, gather=True, dtype="bf16"))
    lr = sg.shard_linear(to_dev(W, "bf16"), "sharded-to-all", P=P)
    Xs = np.ascontiguousarray(np.stack([X[:, r * 64:(r + 1) * 64] for r in range(P)]))
    y = sg.sharded_to_all(lr, to_dev(Xs, "bf16"), out_dtype=torch.float32)
    np.testing.assert_array_equal(to_np(y), oracle.row(Xs, W, P=P, dtype="bf16"))


def test_integer_exact_summa():
    X = synth.small_ints(26, (512, 512), -2, 2, "bf16")
    A = synth.small_ints(27, (512, 256), -2, 2, "bf16")
    for fused in (True, False):
        for ws in ("auto", None):
            y = sg.summa_matmul(to_dev(X, "bf16"), to_dev(A, "bf16"), 4, fused=fused, workspace=ws)
            np.testing.assert_array_equal(to_np(y), oracle.summa(X, A, 4, dtype="bf16"))


@pytest.mark.parametrize("B", [8, 24, 40, 300])
def test_q4_fp16_activations(B):
    """fp16 activations (the codes expand to 1024 + q): streaming kernels up to
    32 tokens, the 4-bit tile kernel beyond (the down layer split by rank)."""
    _print_case(B=B)
    D, F, P = 512, 1024, 4
    ws = [synth.uniform(80 + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    gu, Wgu = _q4_layer(np.concatenate([ws[0], ws[1]]), 0, P, S=2, act=torch.float16)
    dn, Wdn = _q4_layer(ws[2], 1, P, act=torch.float16)
    X = synth.normal(83, (B, D), 1.0, "f16")
    h = sg.all_to_sharded(gu, to_dev(X, "f16"), swiglu=True)
    g = oracle.col(X, Wgu[:F], P=P, dtype="f16")
    u = oracle.col(X, Wgu[F:], P=P, dtype="f16")
    assert_close(h, oracle.swiglu(g, u, "f64"), "f16", "q4 fp16 h")
    # the down layer alone, on the h it was given, in the activation dtype: with
    # fp16 the codes expand to 1024 + q, so the fp32 group sums carry rounding
    # of order 1024 * 2^-24 relative to the activations (measured relL2 ~1.6e-5
    # on fp32 outputs, above the fp32 bound; far inside the fp16 one)
    y = sg.sharded_to_all(dn, h)
    assert_close(y, oracle.row(to_np(h), Wdn, P=P), "f16", "q4 fp16 down")


@pytest.mark.parametrize("B", [1, 8, 32, 64, 520])
def test_integer_exact_q4(B):
    """Power-of-two scales, integer biases and integer activations: exact."""
    out, D, P = 128, 512, 2
    rng = np.random.default_rng(28)
    q = rng.integers(0, 16, size=(out, D)).astype(np.uint8)
    packed = synth.pack_q4(q)
    s = np.float16(rng.choice([0.5, 1.0, 2.0], size=(out, D // 64))).view(np.uint16)
    b = np.float16(rng.integers(-8, 8, size=(out, D // 64))).view(np.uint16)
    X = synth.small_ints(29, (B, D), -2, 2, "bf16")
    for mode in (0, 1):
        layer = sg.shard_quantized_linear(torch.from_numpy(packed.view(np.int32)).to(dev()),
                                          torch.from_numpy(s.view(np.int16)).to(dev()),
                                          torch.from_numpy(b.view(np.int16)).to(dev()), D, mode, P=P)
        Wd = oracle.deq4(packed, s, b, 64)
        if mode == 0:
            y = sg.all_to_sharded(layer, to_dev(X, "bf16"), gather=True, out_dtype=torch.float32)
            ref = oracle.col(X, Wd, P=P, gather=True, dtype="bf16")
        else:
            Xs = np.ascontiguousarray(np.stack([X[:, r * (D // P):(r + 1) * (D // P)] for r in range(P)]))
            y = sg.sharded_to_all(layer, to_dev(Xs, "bf16"), out_dtype=torch.float32)
            ref = oracle.row(Xs, Wd, P=P, dtype="bf16")
        np.testing.assert_array_equal(to_np(y), ref)


def test_fp16_subnormal_weights_not_flushed():
    """fp16 weights k * 2^-24 (subnormal) times small integers: exact results
    only if the MFMA keeps subnormal operands."""
    B, inn, out = 32, 256, 256
    rng = np.random.default_rng(30)
    W = (rng.integers(-3, 4, size=(out, inn)).astype(np.float64) * 2.0 ** -24)
    Wb = W.astype(np.float16).view(np.uint16)
    X = synth.small_ints(31, (B, inn), -3, 3, "f16")
    for Bt in (B, 64):
        Xt = np.ascontiguousarray(np.resize(X, (Bt, inn)))
        layer = sg.shard_linear(to_dev(Wb, "f16"), "all-to-sharded", P=2)
        y = sg.all_to_sharded(layer, to_dev(Xt, "f16"), gather=True, out_dtype=torch.float32)
        np.testing.assert_array_equal(to_np(y), oracle.col(Xt, Wb, P=2, gather=True, dtype="f16"))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_empty_batch_is_noop():
    W = synth.uniform(32, (64, 64), 0.1, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "all-to-sharded", P=2)
    y = torch.full((2, 0, 32), 7.0, dtype=torch.bfloat16, device=dev())
    sg.all_to_sharded(layer, torch.empty((0, 64), dtype=torch.bfloat16, device=dev()), out=y)
    lr = sg.shard_linear(to_dev(W, "bf16"), "sharded-to-all", P=2)
    y2 = sg.sharded_to_all(lr, torch.empty((2, 0, 32), dtype=torch.bfloat16, device=dev()))
    assert y2.shape == (0, 64)


def test_p1_is_the_plain_linear():
    X = synth.normal(33, (48, 128), 1.0, "bf16")
    W = synth.uniform(34, (96, 128), 0.1, "bf16")
    y = sg.all_to_sharded(sg.shard_linear(to_dev(W, "bf16"), "all-to-sharded", P=1), to_dev(X, "bf16"),
                          out_dtype=torch.float32)
    assert_close(y[0], oracle.decode(X, "bf16") @ oracle.decode(W, "bf16").T, "f32", "P=1")


def test_workspace_too_small_is_rejected():
    # 100 tokens x 256 outputs: two 128 x 128 tiles, so the ranks are split
    # over workgroups and reduced through the workspace
    W = synth.uniform(35, (256, 512), 0.1, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "sharded-to-all", P=4)
    xs = to_dev(synth.normal(36, (4, 100, 128), 1.0, "bf16"), "bf16")
    assert sg.lib().sg_sharded_to_all_workspace(layer.handle, 100) > 16
    ws = torch.zeros(16, dtype=torch.uint8, device=dev())
    with pytest.raises(sg.ShardGemmError) as e:
        sg.sharded_to_all(layer, xs, ws=ws)
    assert e.value.code == sg.ERR_WORKSPACE


def test_wrong_layer_mode_is_rejected():
    W = synth.uniform(37, (64, 64), 0.1, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "sharded-to-all", P=2)
    with pytest.raises(sg.ShardGemmError):
        sg.all_to_sharded(layer, to_dev(synth.normal(38, (4, 64), 1.0, "bf16"), "bf16"))
    with pytest.raises(sg.ShardGemmError) as e:
        sg.shard_linear(to_dev(W, "bf16"), "column", P=2)
    assert e.value.code == sg.ERR_BAD_MODE


# ---------------------------------------------------------------------------
# collective layouts ("Sharded Matrices and How to Multiply Them", Cases 2 and
# 3): an all-to-sharded layer fed sharded activations (all-gathered inside the
# K loop), and a sharded-to-all layer whose summed output is reduce-scattered
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B", [1, 16, 24, 40, 600])
@pytest.mark.parametrize("P", [2, 4])
def test_all_gather_input(B, P):
    _print_case(B=B, P=P)
    out, inn = 512, 1024
    Xs = synth.normal(45, (P, B, inn // P), 1.0, "bf16")
    W = synth.uniform(46, (out, inn), inn ** -0.5, "bf16")
    b = synth.uniform(47, (out,), 0.5, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "all-to-sharded", P=P, bias=to_dev(b, "bf16"))
    xg = oracle.all_gather(Xs)
    for gather in (False, True):
        y = sg.all_to_sharded(layer, to_dev(Xs, "bf16"), x_sharded=True, gather=gather, out_dtype=torch.float32)
        assert_close(y, oracle.col(xg, W, P=P, bias=b, gather=gather, dtype="bf16"), "f32", "gathered-input col")
    # the same numbers as gathering first, bit for bit only where the same kernel runs both
    yb = sg.all_to_sharded(layer, to_dev(Xs, "bf16"), x_sharded=True)
    assert_close(yb, oracle.col(xg, W, P=P, bias=b, dtype="bf16"), "bf16", "gathered-input col bf16")


@pytest.mark.parametrize("B", [16, 100, 600])
def test_all_gather_input_swiglu(B):
    _print_case(B=B)
    D, F, P = 512, 1024, 4
    Wg = synth.uniform(48, (F, D), D ** -0.5, "bf16")
    Wu = synth.uniform(49, (F, D), D ** -0.5, "bf16")
    Xs = synth.normal(50, (P, B, D // P), 1.0, "bf16")
    gu = sg.shard_linear(to_dev(np.concatenate([Wg, Wu]), "bf16"), "all-to-sharded", segments=2, P=P)
    h = sg.all_to_sharded(gu, to_dev(Xs, "bf16"), x_sharded=True, swiglu=True)
    xg = oracle.all_gather(Xs)
    ref = oracle.swiglu(oracle.col(xg, Wg, P=P, dtype="bf16"), oracle.col(xg, Wu, P=P, dtype="bf16"), "f64")
    assert_close(h, ref, "bf16", "gathered-input swiglu")


def test_all_gather_input_row_major_weights():
    """out % 16 != 0: the weights stay row-major."""
    B, out, inn, P = 24, 72, 256, 2
    Xs = synth.normal(51, (P, B, inn // P), 1.0, "bf16")
    W = synth.uniform(52, (out, inn), inn ** -0.5, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "all-to-sharded", P=P)
    y = sg.all_to_sharded(layer, to_dev(Xs, "bf16"), x_sharded=True, out_dtype=torch.float32)
    assert_close(y, oracle.col(oracle.all_gather(Xs), W, P=P, dtype="bf16"), "f32", "row-major gathered input")


@pytest.mark.parametrize("B", [5, 60])
def test_all_gather_input_q4(B):
    """A 4-bit all-to-sharded layer fed its input as rank shards ([HSYM] Case
    2): the 4-bit tile kernel walks the P input slices as K segments."""
    _print_case(B=B)
    D, out, P = 1024, 384, 4
    layer, Wd = _q4_layer(synth.uniform(66, (out, D), 1 / np.sqrt(D), "f32"), 0, P)
    Xs = synth.normal(67, (P, B, D // P), 1.0, "bf16")
    ref = oracle.col(oracle.all_gather(Xs), Wd, P=P, dtype="bf16")
    y = sg.all_to_sharded(layer, to_dev(Xs, "bf16"), x_sharded=True, out_dtype=torch.float32)
    assert_close(y, ref, "f32", "q4 all-gather input")


@pytest.mark.parametrize("B", [1, 16, 24, 100, 600])
def test_all_gather_input_mx(B):
    """An MX FP8 all-to-sharded layer fed its input as rank shards ([HSYM]
    Case 2): the streaming kernel, the MX few-token tiles or (row-major codes,
    out % 16 != 0) the generic kernel walk the P input slices as K segments."""
    _print_case(B=B)
    D, out, P = 1024, 384, 4
    layer, _, _, Wd = _mx_layer(synth.uniform(68, (out, D), 1 / np.sqrt(D), "f32"), 0, P)
    Xs = synth.normal(69, (P, B, D // P), 1.0, "bf16")
    xg = oracle.all_gather(Xs)
    for gather in (False, True):
        y = sg.all_to_sharded(layer, to_dev(Xs, "bf16"), x_sharded=True, gather=gather, out_dtype=torch.float32)
        assert_close(y, oracle.col(xg, Wd, P=P, gather=gather, dtype="bf16"), "f32", "mx all-gather input")
    # SwiGLU over the gathered input
    F = 512
    ws = [synth.uniform(70 + i, (F, D), 1 / np.sqrt(D), "f32") for i in range(2)]
    gu, _, _, Wgu = _mx_layer(np.concatenate(ws), 0, P, S=2)
    h = sg.all_to_sharded(gu, to_dev(Xs, "bf16"), x_sharded=True, swiglu=True)
    ref = oracle.swiglu(oracle.col(xg, Wgu[:F], P=P, dtype="bf16"), oracle.col(xg, Wgu[F:], P=P, dtype="bf16"), "f64")
    assert_close(h, ref, "bf16", "mx all-gather input swiglu")
    # row-major codes (72 outputs: not whole 16-row blocks per rank)
    lr, _, _, Wr = _mx_layer(synth.uniform(72, (72, D), 1 / np.sqrt(D), "f32"), 0, 2)
    Xr = synth.normal(73, (2, B, D // 2), 1.0, "bf16")
    y = sg.all_to_sharded(lr, to_dev(Xr, "bf16"), x_sharded=True, gather=True, out_dtype=torch.float32)
    assert_close(y, oracle.col(oracle.all_gather(Xr), Wr, P=2, gather=True, dtype="bf16"), "f32", "mx row-major")


def test_all_gather_input_rejections():
    W = synth.uniform(53, (64, 96), 0.1, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "all-to-sharded", P=2)  # in / P = 48: not 32-aligned
    with pytest.raises(sg.ShardGemmError) as e:
        sg.all_to_sharded(layer, to_dev(synth.normal(54, (2, 4, 48), 1.0, "bf16"), "bf16"), x_sharded=True)
    assert e.value.code == sg.ERR_UNSUPPORTED
    layer3 = sg.shard_linear(to_dev(synth.uniform(55, (66, 64), 0.1, "bf16"), "bf16"), "all-to-sharded", P=3)
    with pytest.raises(sg.ShardGemmError) as e:  # 64 input features over 3 ranks
        sg.all_to_sharded(layer3, to_dev(synth.normal(56, (3, 4, 21), 1.0, "bf16"), "bf16"), x_sharded=True)
    assert e.value.code == sg.ERR_NOT_DIVISIBLE
    lq, _ = _q4_layer(synth.uniform(57, (128, 256), 1 / 16, "f32"), 0, 2)
    with pytest.raises(sg.ShardGemmError) as e:
        sg.all_to_sharded(lq, to_dev(synth.normal(58, (2, 4, 128), 1.0, "bf16"), "bf16"), x_sharded=True)
    assert e.value.code == sg.ERR_UNSUPPORTED
    lm, _, _, _ = _mx_layer(synth.uniform(59, (128, 384), 1 / 16, "f32"), 0, 2)  # fragment-major, 192 per shard
    with pytest.raises(sg.ShardGemmError) as e:
        sg.all_to_sharded(lm, to_dev(synth.normal(60, (2, 4, 192), 1.0, "bf16"), "bf16"), x_sharded=True)
    assert e.value.code == sg.ERR_UNSUPPORTED


@pytest.mark.parametrize("B", [1, 16, 24, 100, 600, 2048])
@pytest.mark.parametrize("P", [2, 4])
def test_reduce_scatter_output(B, P):
    """B = 100 and 2048 take the rank-split workspace path of the tile kernels."""
    _print_case(B=B, P=P)
    out, inn = 512, 1024
    Xs = synth.normal(59, (P, B, inn // P), 1.0, "bf16")
    W = synth.uniform(60, (out, inn), inn ** -0.5, "bf16")
    b = synth.uniform(61, (out,), 0.5, "bf16")
    layer = sg.shard_linear(to_dev(W, "bf16"), "sharded-to-all", P=P, bias=to_dev(b, "bf16"))
    ref = oracle.reduce_scatter(oracle.row(Xs, W, P=P, bias=b, dtype="bf16"), P)
    y = sg.sharded_to_all(layer, to_dev(Xs, "bf16"), scatter=True, out_dtype=torch.float32)
    assert tuple(y.shape) == (P, B, out // P)
    assert_close(y, ref, "f32", "reduce-scatter")
    # the same rank-order sum as the all-reduce output, bit for bit
    yf = sg.sharded_to_all(layer, to_dev(Xs, "bf16"), out_dtype=torch.float32)
    for r in range(P):
        assert torch.equal(y[r], yf[:, r * (out // P):(r + 1) * (out // P)])


@pytest.mark.parametrize("B", [1, 8, 32, 100])
def test_reduce_scatter_q4(B):
    _print_case(B=B)
    D, F, P = 512, 1024, 4
    dn, Wdn = _q4_layer(synth.uniform(62, (D, F), 1 / np.sqrt(F), "f32"), 1, P)
    Xs = synth.normal(63, (P, B, F // P), 1.0, "bf16")
    y = sg.sharded_to_all(dn, to_dev(Xs, "bf16"), scatter=True, out_dtype=torch.float32)
    assert_close(y, oracle.reduce_scatter(oracle.row(Xs, Wdn, P=P, dtype="bf16"), P), "f32", "q4 reduce-scatter")


def test_reduce_scatter_rejections():
    layer = sg.shard_linear(to_dev(synth.uniform(64, (66, 64), 0.1, "bf16"), "bf16"), "sharded-to-all", P=4)
    with pytest.raises(sg.ShardGemmError) as e:  # 66 outputs over 4 ranks
        sg.sharded_to_all(layer, to_dev(synth.normal(65, (4, 4, 16), 1.0, "bf16"), "bf16"), scatter=True)
    assert e.value.code == sg.ERR_NOT_DIVISIBLE


@pytest.mark.parametrize("B", [4, 600])
def test_attention_projections_end_to_end(B):
    """Fused QKV column shards (segments = 3: rank r holds heads of Q, K and V)
    feeding the row-sharded output projection with a bias, as in the MLX
    attention example ([MLX] 5.4).  The attention core is not on this path:
    rank r's V shard stands in for its heads' attention output, which has the
    same layout (tokens, D/P) per rank."""
    _print_case(B=B)
    D, heads, hd, P = 512, 8, 64, 4
    X = synth.normal(66, (B, D), 1.0, "bf16")
    Wqkv = synth.uniform(67, (3 * D, D), D ** -0.5, "bf16")
    Wo = synth.uniform(68, (D, D), D ** -0.5, "bf16")
    bo = synth.uniform(69, (D,), 0.5, "bf16")
    qkv = sg.shard_linear(to_dev(Wqkv, "bf16"), "all-to-sharded", segments=3, P=P)
    wo = sg.shard_linear(to_dev(Wo, "bf16"), "sharded-to-all", P=P, bias=to_dev(bo, "bf16"))
    y = sg.all_to_sharded(qkv, to_dev(X, "bf16"))            # (P, B, 3 D / P) = [Q_r | K_r | V_r]
    v = y[:, :, 2 * D // P:].contiguous()                   # (P, B, D / P)
    out = sg.sharded_to_all(wo, v, out_dtype=torch.float32)
    # oracle: V_r = X Wv_r^T from the segments rule, then the rank-order sum + bias
    ref_qkv = oracle.col(X, Wqkv, P=P, S=3, dtype="bf16")
    assert_close(y, ref_qkv, "bf16", "qkv")
    v_ref = np.ascontiguousarray(ref_qkv[:, :, 2 * D // P:])
    Wv = Wqkv[2 * D:]
    np.testing.assert_array_equal(v_ref, oracle.col(X, Wv, P=P, dtype="bf16"))  # segment 2 of every rank is V
    # the row layer consumes V as stored between the layers (bf16)
    ref = oracle.row(bits(v), Wo, P=P, bias=bo, dtype="bf16")
    assert_close(out, ref, "f32", "wo(v)")


# ---------------------------------------------------------------------------
# MX FP8 layers ("MLX 张量并行实战指南" 2.3 mode "mxfp8"; OCP MX reading:
# E4M3 codes, one E8M0 scale per 32 inputs, no biases)
# ---------------------------------------------------------------------------
def _mx_layer(w, mode, P, S=1, bias=None):
    codes, scales = synth.quantize_mxfp8(w)
    layer = sg.shard_mxfp8_linear(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()), mode,
                                  segments=S, P=P, bias=bias)
    return layer, codes, scales, oracle.deq_mx8(codes, scales)


@pytest.mark.parametrize("mode,out,inn,S,P", [(0, 384, 512, 1, 4), (0, 768, 256, 3, 2), (1, 256, 1024, 1, 4),
                                              (0, 72, 128, 1, 2), (1, 40, 256, 2, 2)])
def test_slicing_mx_bit_exact(mode, out, inn, S, P):
    _print_case(mode=mode, out=out, inn=inn, S=S, P=P)
    w = synth.uniform(73, (out, inn), inn ** -0.5, "f32")
    layer, codes, scales, _ = _mx_layer(w, mode, P, S)
    for r in range(P):
        np.testing.assert_array_equal(to_np(layer.shard(r, 0)).astype(np.uint8), oracle.slice_(codes, mode, S, P, r))
        np.testing.assert_array_equal(to_np(layer.shard(r, 2)).astype(np.uint8), oracle.slice_(scales, mode, S, P, r))
    with pytest.raises(sg.ShardGemmError):
        layer.shard(0, 3)  # no quantization biases


# beyond 32 tokens: the few-token tiles (codes converted after the LDS), 64- or 128-token tiles
@pytest.mark.parametrize("B", [1, 8, 16, 32, 40, 100, 200, 600, 1100])
def test_mx_all_to_sharded(B):
    _print_case(B=B)
    D, out, P = 512, 384, 4
    layer, _, _, Wd = _mx_layer(synth.uniform(74, (out, D), 1 / np.sqrt(D), "f32"), 0, P)
    X = synth.normal(75, (B, D), 1.0, "bf16")
    for gather in (False, True):
        y = sg.all_to_sharded(layer, to_dev(X, "bf16"), gather=gather, out_dtype=torch.float32)
        assert_close(y, oracle.col(X, Wd, P=P, gather=gather, dtype="bf16"), "f32", "mx col")


@pytest.mark.parametrize("B", [1, 16, 32, 48, 128, 250, 520])
def test_mx_swiglu_and_row(B):
    _print_case(B=B)
    D, F, P = 512, 1024, 4
    ws = [synth.uniform(76 + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    bd = synth.uniform(79, (D,), 0.5, "bf16")
    gu, _, _, Wgu = _mx_layer(np.concatenate([ws[0], ws[1]]), 0, P, S=2)
    dn, _, _, Wdn = _mx_layer(ws[2], 1, P, bias=to_dev(bd, "bf16"))
    X = synth.normal(80, (B, D), 1.0, "bf16")
    h = sg.all_to_sharded(gu, to_dev(X, "bf16"), swiglu=True)
    g, u = oracle.col(X, Wgu[:F], P=P, dtype="bf16"), oracle.col(X, Wgu[F:], P=P, dtype="bf16")
    assert_close(h, oracle.swiglu(g, u, "f64"), "bf16", "mx h")
    y = sg.sharded_to_all(dn, h, out_dtype=torch.float32)
    assert_close(y, oracle.row(bits(h), Wdn, P=P, bias=bd, dtype="bf16"), "f32", "mx y")


@pytest.mark.parametrize("B", [40, 600])
def test_mx_tile_kernel(B):
    """Inputs per rank not a multiple of 128 (480): the MX few-token tiles do
    not take the layer, the 128 x 128 tile kernel with the FP8 loader does."""
    _print_case(B=B)
    D, out, P = 480, 256, 2
    layer, _, _, Wd = _mx_layer(synth.uniform(85, (out, D), 1 / np.sqrt(D), "f32"), 0, P)
    X = synth.normal(86, (B, D), 1.0, "bf16")
    y = sg.all_to_sharded(layer, to_dev(X, "bf16"), gather=True, out_dtype=torch.float32)
    assert_close(y, oracle.col(X, Wd, P=P, gather=True, dtype="bf16"), "f32", "mx tile kernel")


def test_mx_row_major_layout():
    """out % 16 != 0: codes stay row-major and the generic kernel runs."""
    B, out, D, P = 4, 72, 256, 2
    layer, _, _, Wd = _mx_layer(synth.uniform(81, (out, D), D ** -0.5, "f32"), 0, P)
    X = synth.normal(82, (B, D), 1.0, "bf16")
    y = sg.all_to_sharded(layer, to_dev(X, "bf16"), gather=True, out_dtype=torch.float32)
    assert_close(y, oracle.col(X, Wd, P=P, gather=True, dtype="bf16"), "f32", "mx row-major")


@pytest.mark.parametrize("B", [1, 8, 32, 64, 100, 520])
def test_integer_exact_mx(B):
    """Integer-valued E4M3 codes at scale 2^0 and 2^1, integer activations: exact."""
    out, D, P = 128, 512, 2
    rng = np.random.default_rng(83)
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4], dtype=np.uint8)  # 0, 1, 2, 3, 4, -1, -2, -3
    codes = ints[rng.integers(0, len(ints), size=(out, D))]
    scales = rng.choice(np.array([127, 128], dtype=np.uint8), size=(out, D // 32))
    X = synth.small_ints(84, (B, D), -2, 2, "bf16")
    for mode in (0, 1):
        layer = sg.shard_mxfp8_linear(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()), mode, P=P)
        Wd = oracle.deq_mx8(codes, scales)
        if mode == 0:
            y = sg.all_to_sharded(layer, to_dev(X, "bf16"), gather=True, out_dtype=torch.float32)
            ref = oracle.col(X, Wd, P=P, gather=True, dtype="bf16")
        else:
            Xs = np.ascontiguousarray(np.stack([X[:, r * (D // P):(r + 1) * (D // P)] for r in range(P)]))
            y = sg.sharded_to_all(layer, to_dev(Xs, "bf16"), out_dtype=torch.float32)
            ref = oracle.row(Xs, Wd, P=P, dtype="bf16")
        np.testing.assert_array_equal(to_np(y), ref)


def test_mx_rejections():
    codes = torch.zeros((64, 96), dtype=torch.uint8, device=dev())
    scales = torch.full((64, 3), 127, dtype=torch.uint8, device=dev())
    with pytest.raises(sg.ShardGemmError) as e:  # a scale block would straddle the two ranks (96 / 2 = 48)
        sg.shard_mxfp8_linear(codes, scales, "sharded-to-all", P=2)
    assert e.value.code == sg.ERR_NOT_DIVISIBLE
    with pytest.raises(sg.ShardGemmError) as e:
        sg.shard_mxfp8_linear(codes, scales, "all-to-sharded", P=2, act_dtype=torch.float16)
    assert e.value.code == sg.ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# backward (sum_gradients VJP of the all-to-sharded layer; the sharded-to-all VJP)
# ---------------------------------------------------------------------------
BWD_CASES = [("bf16", 8, 256, 512, 1, 4), ("bf16", 5, 96, 72, 1, 2), ("f16", 3, 128, 256, 2, 2),
             ("f32", 4, 64, 96, 1, 3), ("bf16", 1, 512, 128, 1, 1),
             ("bf16", 4, 64, 48, 1, 2),  # 24 rows per rank: the fragment-major stack crosses rank boundaries
             ("f16", 5, 128, 256, 1, 4),  # fp16 with one segment: the sharded-to-all backward in fp16 too
             ("bf16", 40, 256, 512, 1, 4),  # input gradients on the 128 x 128 tile kernel, 64 padded tokens
             ("bf16", 520, 256, 512, 2, 2)]  # the 256 x 256 tile kernels, 544 padded tokens
# ws: "auto" = weight gradients on the matrix cores over the transposed
# operands in a workspace; None = the vector-unit weight-gradient kernel


@pytest.mark.parametrize("ws", ["auto", None])
@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_all_to_sharded_backward(case, ws):
    dtype, B, inn, out, S, P = case
    _print_case(dtype=dtype, B=B, inn=inn, out=out, S=S, P=P, ws=ws)
    W = synth.uniform(90, (out, inn), inn ** -0.5, dtype)
    X = synth.normal(91, (B, inn), 1.0, dtype)
    G = synth.normal(92, (P, B, out // P), 1.0, dtype)
    layer = sg.shard_linear(to_dev(W, dtype), "all-to-sharded", segments=S, P=P)
    dx, dw = sg.all_to_sharded_backward(layer, to_dev(X, dtype), to_dev(G, dtype), dx_dtype=torch.float32, ws=ws)
    rdx, rdw = oracle.col_bwd(X, W, G, P=P, S=S, dtype=dtype)
    assert_close(dx, rdx, "f32", "dx")
    assert_close(dw, rdw, "f32", "dw")
    dx2, _ = sg.all_to_sharded_backward(layer, None, to_dev(G, dtype), need_dw=False, dx_dtype=torch.float32)
    assert torch.equal(dx, dx2)  # the rank-order sum is deterministic
    if dtype != "f32":
        dx16, _ = sg.all_to_sharded_backward(layer, None, to_dev(G, dtype), need_dw=False)
        assert_close(dx16, rdx, dtype, "dx 16-bit")


@pytest.mark.parametrize("ws", ["auto", None])
@pytest.mark.parametrize("case", [c for c in BWD_CASES if c[4] == 1], ids=lambda c: "-".join(map(str, c)))
def test_sharded_to_all_backward(case, ws):
    dtype, B, inn, out, S, P = case  # one segment: the down-projection layers these cases stand for
    inn, out = out, inn  # a down-projection shape: in = the wide side
    _print_case(dtype=dtype, B=B, inn=inn, out=out, P=P, ws=ws)
    W = synth.uniform(93, (out, inn), inn ** -0.5, dtype)
    Xs = synth.normal(94, (P, B, inn // P), 1.0, dtype)
    G = synth.normal(95, (B, out), 1.0, dtype)
    layer = sg.shard_linear(to_dev(W, dtype), "sharded-to-all", P=P)
    dxs, dw = sg.sharded_to_all_backward(layer, to_dev(Xs, dtype), to_dev(G, dtype), dx_dtype=torch.float32, ws=ws)
    rdxs, rdw = oracle.row_bwd(Xs, W, G, P=P, dtype=dtype)
    assert_close(dxs, rdxs, "f32", "dx_partial")
    assert_close(dw, rdw, "f32", "dw")
    if dtype != "f32":
        dxs16, dw16 = sg.sharded_to_all_backward(layer, to_dev(Xs, dtype), to_dev(G, dtype), dw_dtype=DT[dtype], ws=ws)
        assert_close(dxs16, rdxs, dtype, "dx_partial 16-bit")
        assert_close(dw16, rdw, dtype, "dw 16-bit")


def test_backward_rejections():
    w = to_dev(synth.uniform(96, (64, 64), 1 / 8, "bf16"), "bf16")
    col = sg.shard_linear(w, "all-to-sharded", P=2)
    row = sg.shard_linear(w, "sharded-to-all", P=2)
    dy = torch.zeros((2, 4, 32), dtype=torch.bfloat16, device=dev())
    with pytest.raises(sg.ShardGemmError):
        sg.all_to_sharded_backward(row, None, dy, need_dw=False)  # wrong mode
    with pytest.raises(sg.ShardGemmError, match="forward input"):
        sg.all_to_sharded_backward(col, None, dy)  # dw without x
    with pytest.raises(sg.ShardGemmError):
        sg.sharded_to_all_backward(col, None, torch.zeros((4, 64), dtype=torch.bfloat16, device=dev()), need_dw=False)
    assert sg.lib().sg_layer_backward_workspace(col.handle, 4) == 0  # few tokens: dw reads dy and x in place
    x = torch.zeros((200, 64), dtype=torch.bfloat16, device=dev())
    dy2 = torch.zeros((2, 200, 32), dtype=torch.bfloat16, device=dev())
    need = sg.lib().sg_layer_backward_workspace(col.handle, 200)
    assert need > 0
    with pytest.raises(sg.ShardGemmError, match="workspace"):
        sg.all_to_sharded_backward(col, x, dy2, ws=torch.zeros(need - 256, dtype=torch.uint8, device=dev()))


SUMMA_BWD_CASES = [("bf16", 256, 128, 512, 4), ("bf16", 64, 96, 48, 2), ("f16", 512, 256, 256, 1),
                   ("f32", 24, 12, 18, 3), ("bf16", 48, 66, 30, 3),
                   ("bf16", 128, 768, 272, 2)]  # dA on the 256 x 256 tile kernel, a ragged N tile


@pytest.mark.parametrize("ws", ["auto", None])
@pytest.mark.parametrize("case", SUMMA_BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_summa_backward(case, ws):
    """Matmul_ABT_2D / Matmul_ATB_2D: dX = dY A^T and dA = X^T dY in q steps."""
    dtype, M, K, N, q = case
    _print_case(dtype=dtype, M=M, K=K, N=N, q=q, ws=ws)
    X = synth.normal(110, (M, K), K ** -0.25, dtype)
    A = synth.normal(111, (K, N), K ** -0.25, dtype)
    G = synth.normal(112, (M, N), 1.0, dtype)
    dX, dA = sg.summa_backward(to_dev(X, dtype), to_dev(A, dtype), to_dev(G, dtype), q, ws=ws)
    assert_close(dX, oracle.summa_abt(G, A, q, dtype=dtype), "f32", "dX")
    assert_close(dA, oracle.summa_atb(X, G, q, dtype=dtype), "f32", "dA")
    with pytest.raises(sg.ShardGemmError):
        sg.summa_backward(to_dev(X, dtype), to_dev(A, dtype), to_dev(G, dtype), q + 5)
