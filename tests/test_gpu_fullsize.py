"""Full-size parity: every workload at the shapes bench.py times, in the same
launch configuration (same layers, same kernels), against the oracle on all
tokens where the oracle finishes in seconds, else on sampled tokens / rows
(the oracle computes those rows exactly; rows are independent)."""
import numpy as np
import pytest
import torch

import oracle
import sharded_gemm_alltosharded_amd as sg
import synth
from gpu_util import assert_close, dev, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sg.lib()


def _case(msg):
    print("case:", msg, flush=True)


def test_decode_mlp_full():
    """B=16, D=4096, F=14336, P=8, bf16: every token against the oracle."""
    _case("decode MLP B=16 D=4096 F=14336 P=8")
    B, D, F, P = 16, 4096, 14336, 8
    inp = synth.mlp_inputs(B, D, F, P, "bf16", seed=0)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), "bf16"), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, "bf16"), "sharded-to-all", P=P)
    x = to_dev(inp.X, "bf16")
    h = sg.all_to_sharded(gu, x, swiglu=True)
    y = sg.sharded_to_all(dn, h)
    X, Wg, Wu, Wd = (oracle.decode(a, "bf16") for a in (inp.X, inp.Wg, inp.Wu, inp.Wd))
    g, u = oracle.col(X, Wg, P=P), oracle.col(X, Wu, P=P)
    # h against the exact product; the next layer's reference consumes h rounded
    # to bf16 once, as stored between the layers
    assert_close(h, oracle.swiglu(g, u, "f64"), "bf16", "h")
    assert_close(y, oracle.row(oracle.swiglu(g, u, "bf16"), Wd, P=P), "bf16", "y")
    # the fused rank sum is deterministic
    y2 = sg.sharded_to_all(dn, h)
    assert torch.equal(y, y2)
    # the fused MLP entry point bench.py times: bit for bit the chain above
    assert torch.equal(sg.mlp(gu, dn, x), y)


@pytest.mark.parametrize("B", [64, 256])
def test_decode_mlp_more_tokens(B):
    """The decode-MLP layers at 64 and 256 tokens (the few-token tiles; the
    down layer split into rank groups, their partial tiles summed by the second
    kernel): eight sampled tokens against the oracle, the fused entry point bit
    for bit against the two calls."""
    _case(f"decode MLP B={B} D=4096 F=14336 P=8")
    D, F, P = 4096, 14336, 8
    inp = synth.mlp_inputs(B, D, F, P, "bf16", seed=1)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), "bf16"), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, "bf16"), "sharded-to-all", P=P)
    x = to_dev(inp.X, "bf16")
    h = sg.all_to_sharded(gu, x, swiglu=True)
    y = sg.sharded_to_all(dn, h)
    idx = sorted({0, 1, B // 2, B - 1, *np.random.default_rng(B).choice(B, 4, replace=False).tolist()})
    X, Wg, Wu, Wd = (oracle.decode(a, "bf16") for a in (inp.X[idx], inp.Wg, inp.Wu, inp.Wd))
    g, u = oracle.col(X, Wg, P=P), oracle.col(X, Wu, P=P)
    assert_close(h[:, idx], oracle.swiglu(g, u, "f64"), "bf16", "h")
    assert_close(y[idx], oracle.row(oracle.swiglu(g, u, "bf16"), Wd, P=P), "bf16", "y")
    assert torch.equal(sg.mlp(gu, dn, x), y)


@pytest.mark.parametrize("B", [16, 512])
def test_mxfp8_mlp_full(B):
    """MX FP8 decode MLP (the layers bench.py times for it): D=4096, F=14336,
    P=8, E4M3 codes with E8M0 scales per 32 inputs.  16 tokens (the streaming
    kernels): every token; 512 tokens (the MX few-token tiles, the down layer
    split into rank groups): eight sampled tokens."""
    _case(f"MX FP8 decode MLP B={B} D=4096 F=14336 P=8")
    D, F, P = 4096, 14336, 8
    X = synth.normal(90, (B, D), 1.0, "bf16")
    ws = [synth.uniform(91 + i, shp, 1 / 64, "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    gc, gs = synth.quantize_mxfp8(np.concatenate([ws[0], ws[1]]))
    dc, ds = synth.quantize_mxfp8(ws[2])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    gu = sg.shard_mxfp8_linear(t(gc), t(gs), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_mxfp8_linear(t(dc), t(ds), "sharded-to-all", P=P)
    h = sg.all_to_sharded(gu, to_dev(X, "bf16"), swiglu=True)
    y = sg.sharded_to_all(dn, h)
    idx = list(range(B)) if B <= 16 else sorted({0, 1, B // 2, B - 1, *np.random.default_rng(B).choice(B, 4, replace=False).tolist()})
    Wgu, Wd = oracle.deq_mx8(gc, gs), oracle.deq_mx8(dc, ds)
    Xd = oracle.decode(X[idx], "bf16")
    g, u = oracle.col(Xd, Wgu[:F], P=P), oracle.col(Xd, Wgu[F:], P=P)
    assert_close(h[:, idx], oracle.swiglu(g, u, "f64"), "bf16", "h")
    assert_close(y[idx], oracle.row(oracle.swiglu(g, u, "bf16"), Wd, P=P), "bf16", "y")
    assert torch.equal(sg.mlp(gu, dn, to_dev(X, "bf16")), y)  # the entry point bench.py times


def test_prefill_full_sampled():
    """B=4096, P=4: QKV (segments 3) + MLP on the full batch; 8 sampled tokens."""
    _case("prefill B=4096 D=4096 F=14336 P=4 + QKV")
    B, D, F, P = 4096, 4096, 14336, 4
    inp = synth.mlp_inputs(B, D, F, P, "bf16", seed=0)
    wqkv = synth.qkv_weight(D, 32, 128, seed=10)
    x = to_dev(inp.X, "bf16")
    qkv = sg.all_to_sharded(sg.shard_linear(to_dev(wqkv, "bf16"), "all-to-sharded", segments=3, P=P), x)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), "bf16"), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, "bf16"), "sharded-to-all", P=P)
    h = sg.all_to_sharded(gu, x, swiglu=True)
    y = sg.sharded_to_all(dn, h)
    idx = np.array([0, 1, 255, 256, 1000, 2047, 3333, 4095])
    Xs = oracle.decode(inp.X[idx], "bf16")
    Wg, Wu, Wd, Wq = (oracle.decode(a, "bf16") for a in (inp.Wg, inp.Wu, inp.Wd, wqkv))
    assert_close(qkv[:, idx, :], oracle.col(Xs, Wq, P=P, S=3), "bf16", "qkv")
    g, u = oracle.col(Xs, Wg, P=P), oracle.col(Xs, Wu, P=P)
    assert_close(h[:, idx, :], oracle.swiglu(g, u, "f64"), "bf16", "h")
    assert_close(y[idx], oracle.row(oracle.swiglu(g, u, "bf16"), Wd, P=P), "bf16", "y")


@pytest.fixture(scope="module")
def q4_weights():
    return synth.q4_mlp_weights(4096, 14336, seed=20)


@pytest.mark.parametrize("B", [1, 8, 32, 64, 512])
def test_q4_mlp_full(q4_weights, B):
    """4-bit affine MLP, D=4096, F=14336, P=4 (sampled tokens beyond 8): the
    streaming kernels up to 32 tokens, the 4-bit tile kernels beyond (at 64
    tokens the down layer split by rank, summed by the second kernel)."""
    _case(f"4-bit MLP B={B}")
    D, F, P = 4096, 14336, 4
    q = q4_weights

    def t32(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(dev())

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev())

    gu = sg.shard_quantized_linear(t32(np.concatenate([q["gate"][0], q["up"][0]])),
                                   t16(np.concatenate([q["gate"][1], q["up"][1]])),
                                   t16(np.concatenate([q["gate"][2], q["up"][2]])), D, "all-to-sharded",
                                   segments=2, P=P)
    dn = sg.shard_quantized_linear(t32(q["down"][0]), t16(q["down"][1]), t16(q["down"][2]), F, "sharded-to-all", P=P)
    X = synth.normal(0, (B, D), 1.0, "bf16")
    h = sg.all_to_sharded(gu, to_dev(X, "bf16"), swiglu=True)
    y = sg.sharded_to_all(dn, h)
    idx = np.arange(B) if B <= 8 else np.array(sorted({0, 5, 16, 31, B // 2 + 3, B - 1}))
    W = {k: oracle.deq4(*q[k][:3], 64) for k in ("gate", "up", "down")}
    Xs = oracle.decode(X[idx], "bf16")
    g, u = oracle.col(Xs, W["gate"], P=P), oracle.col(Xs, W["up"], P=P)
    assert_close(h[:, idx, :], oracle.swiglu(g, u, "f64"), "bf16", "h")
    assert_close(y[idx], oracle.row(oracle.swiglu(g, u, "bf16"), W["down"], P=P), "bf16", "y")
    assert torch.equal(sg.mlp(gu, dn, to_dev(X, "bf16")), y)  # the entry point bench.py times


@pytest.mark.parametrize("fused", [True, False])
def test_summa_full_sampled(fused):
    """Y = X A, 8192^3 bf16, q = 4, fp32 Y: 8 sampled rows (two per block row)."""
    _case(f"SUMMA 8192 q=4 fused={fused}")
    n, q = 8192, 4
    Xh, Ah = synth.summa_inputs(n, seed=30)
    Y = sg.summa_matmul(to_dev(Xh, "bf16"), to_dev(Ah, "bf16"), q, fused=fused)
    idx = np.array([0, 2047, 2048, 4000, 4096, 6143, 6144, 8191])
    ref = oracle.summa(oracle.decode(Xh[idx], "bf16"), oracle.decode(Ah, "bf16"), q)
    assert_close(Y[idx], ref, "f32", "summa")


def test_summa_backward_full_sampled():
    """SUMMA backward as bench.py times it (--config 5c): 8192^3, q = 4;
    sampled rows of dX = dY A^T and of dA = X^T dY (rows k of dA need all of
    X's column k)."""
    _case("SUMMA backward 8192 q=4")
    n, q = 8192, 4
    Xh, Ah = synth.summa_inputs(n, seed=30)
    Gh = synth.normal(113, (n, n), 1.0, "bf16")
    dX, dA = sg.summa_backward(to_dev(Xh, "bf16"), to_dev(Ah, "bf16"), to_dev(Gh, "bf16"), q)
    idx = np.array([0, 2047, 2048, 4000, 4096, 6143, 6144, 8191])
    A, G = oracle.decode(Ah, "bf16"), oracle.decode(Gh, "bf16")
    assert_close(dX[idx], oracle.summa_abt(G[idx], A, q), "f32", "dX")
    Xc = oracle.decode(np.ascontiguousarray(Xh[:, idx]), "bf16")
    assert_close(dA[idx], oracle.summa_atb(Xc, G, q), "f32", "dA")


def test_vocab_head_full_sampled():
    """fp16 vocabulary head, 32 x 12288 against 50272 x 12288, P = 8 ranks of
    6284 rows, gathered logits: 3 sampled tokens, every vocabulary entry."""
    _case("vocab head B=32 H=12288 V=50272 P=8")
    B, H, V, P = 32, 12288, 50272, 8
    Xh, Wh = synth.vocab_head_inputs(B, H, V, seed=40)
    layer = sg.shard_linear(to_dev(Wh, "f16"), "all-to-sharded", P=P)
    logits = sg.all_to_sharded(layer, to_dev(Xh, "f16"), gather=True)
    assert tuple(logits.shape) == (B, V)
    idx = np.array([0, 17, 31])
    ref = oracle.col(oracle.decode(Xh[idx], "f16"), oracle.decode(Wh, "f16"), P=P, gather=True)
    assert_close(logits[idx], ref, "f16", "logits")
    # the gathered columns of rank r are rank r's sharded output
    sharded = sg.all_to_sharded(layer, to_dev(Xh, "f16"))
    for r in (0, 7):
        assert torch.equal(sharded[r], logits[:, r * (V // P):(r + 1) * (V // P)])


def test_mlp_backward_full():
    """The backward bench.py times (--config 7): decode MLP shapes, B=16,
    D=4096, F=14336, P=8, bf16 in, fp32 weight gradients; every output."""
    _case("MLP backward B=16 D=4096 F=14336 P=8")
    B, D, F, P = 16, 4096, 14336, 8
    inp = synth.mlp_inputs(B, D, F, P, "bf16", seed=0)
    Wgu = np.concatenate([inp.Wg, inp.Wu])
    gu = sg.shard_linear(to_dev(Wgu, "bf16"), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, "bf16"), "sharded-to-all", P=P)
    hs = synth.normal(100, (P, B, F // P), 1.0, "bf16")
    dy = synth.normal(101, (B, D), 1.0, "bf16")
    dg = synth.normal(102, (P, B, 2 * F // P), 1.0, "bf16")
    dh, dWd = sg.sharded_to_all_backward(dn, to_dev(hs, "bf16"), to_dev(dy, "bf16"), dx_dtype=torch.float32)
    rdh, rdWd = oracle.row_bwd(hs, inp.Wd, dy, P=P, dtype="bf16")
    assert_close(dh, rdh, "f32", "dh")
    assert_close(dWd, rdWd, "f32", "dW_down")
    dx, dWgu = sg.all_to_sharded_backward(gu, to_dev(inp.X, "bf16"), to_dev(dg, "bf16"), dx_dtype=torch.float32)
    rdx, rdWgu = oracle.col_bwd(inp.X, Wgu, dg, P=P, S=2, dtype="bf16")
    assert_close(dx, rdx, "f32", "dx")
    assert_close(dWgu, rdWgu, "f32", "dW_gate_up")
