"""sg_mlp_static, the gated-MLP entry point that allocates nothing (its
workspace is the library's per-device static scratch), against sg_mlp with a
caller workspace: the same kernels, so the results must agree bit for bit.
Each case makes two calls in a row, the second with fewer tokens, so the
second call runs on whatever the first left in the scratch."""
import numpy as np
import pytest
import torch

import oracle
import sharded_gemm_alltosharded_amd as sg
import synth
from gpu_util import assert_close, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sg.lib()


def _layers(B, D, F, P, dtype, seed):
    inp = synth.mlp_inputs(B, D, F, P, dtype, seed=seed)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), dtype), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, dtype), "sharded-to-all", P=P)
    return inp, gu, dn


# (dtype, D, F, P, first B, second B): streaming kernels with the fragment-major
# h; the fallback pair whose down layer splits by rank through partial tiles
# in the scratch; fp16
CASES = [("bf16", 512, 1024, 8, 16, 5), ("bf16", 256, 512, 2, 40, 16), ("f16", 256, 768, 3, 32, 8),
         ("bf16", 4096, 14336, 8, 16, 1)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_mlp_static_matches_mlp(case):
    dtype, D, F, P, B1, B2 = case
    print(f"case: dtype={dtype} D={D} F={F} P={P} B={B1},{B2}", flush=True)
    inp, gu, dn = _layers(B1, D, F, P, dtype, seed=61)
    for B in (B1, B2):
        x = to_dev(inp.X[:B], dtype)
        y = torch.empty((B, D), dtype=torch.float32, device=dev())
        before = torch.cuda.memory_allocated()
        sg.mlp_static(gu, dn, x, y)
        assert torch.cuda.memory_allocated() == before
        ref = sg.mlp(gu, dn, x, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), B
        y16 = torch.empty((B, D), dtype=x.dtype, device=dev())
        assert torch.equal(sg.mlp_static(gu, dn, x, y16), sg.mlp(gu, dn, x)), B
        if D <= 512:
            g = oracle.col(inp.X[:B], inp.Wg, P=P, dtype=dtype)
            u = oracle.col(inp.X[:B], inp.Wu, P=P, dtype=dtype)
            assert_close(y, oracle.row(oracle.swiglu(g, u, dtype), inp.Wd, P=P, dtype=dtype), "f32", "mlp_static")


def test_mlp_static_rejects_beyond_the_scratch():
    D, F, P = 256, 8192, 2
    inp, gu, dn = _layers(8, D, F, P, "bf16", seed=62)
    B = 1024  # h alone is 1024 x 8192 x 2 bytes = 16 MiB, past the scratch
    assert sg.lib().sg_mlp_workspace(gu.handle, dn.handle, B) > sg.MLP_STATIC_SCRATCH_BYTES
    x = torch.zeros((B, D), dtype=torch.bfloat16, device=dev())
    y = torch.empty((B, D), dtype=torch.bfloat16, device=dev())
    with pytest.raises(sg.ShardGemmError, match="static scratch"):
        sg.mlp_static(gu, dn, x, y)
    # the largest B that fits still runs, and matches sg_mlp
    Bf = 1
    while sg.lib().sg_mlp_workspace(gu.handle, dn.handle, Bf * 2) <= sg.MLP_STATIC_SCRATCH_BYTES:
        Bf *= 2
    xf = to_dev(synth.normal(63, (Bf, D), 1.0, "bf16"), "bf16")
    yf = torch.empty((Bf, D), dtype=torch.float32, device=dev())
    sg.mlp_static(gu, dn, xf, yf)
    assert torch.equal(yf, sg.mlp(gu, dn, xf, out_dtype=torch.float32))


def _q4(w, mode, P, S=1):
    packed, s, b, _ = synth.quantize_q4(w, 64)
    return sg.shard_quantized_linear(torch.from_numpy(packed.view(np.int32)).to(dev()),
                                     torch.from_numpy(s.view(np.int16)).to(dev()),
                                     torch.from_numpy(b.view(np.int16)).to(dev()), w.shape[1], mode,
                                     segments=S, P=P)


@pytest.mark.parametrize("Bs", [(100, 24), (24, 64)], ids=lambda b: "-".join(map(str, b)))
def test_mlp_static_quantized(Bs):
    """4-bit layers: the tile kernels (the down layer split by rank through
    partial tiles in the scratch) and the streaming kernels (h
    fragment-major in the scratch), two calls in a row."""
    D, F, P = 512, 1024, 4
    print(f"case: q4 D={D} F={F} P={P} B={Bs}", flush=True)
    ws = [synth.uniform(70 + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    gu, dn = _q4(np.concatenate([ws[0], ws[1]]), 0, P, S=2), _q4(ws[2], 1, P)
    X = synth.normal(73, (max(Bs), D), 1.0, "bf16")
    for B in Bs:
        x = to_dev(X[:B], "bf16")
        y = torch.empty((B, D), dtype=torch.float32, device=dev())
        before = torch.cuda.memory_allocated()
        sg.mlp_static(gu, dn, x, y)
        assert torch.cuda.memory_allocated() == before
        ref = sg.mlp(gu, dn, x, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), B


def _mx(w, mode, P, S=1):
    codes, scales = synth.quantize_mxfp8(w)
    return sg.shard_mxfp8_linear(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()), mode,
                                 segments=S, P=P)


@pytest.mark.parametrize("Bs", [(100, 24), (16, 8)], ids=lambda b: "-".join(map(str, b)))
def test_mlp_static_mx(Bs):
    """MX FP8 layers: the MX few-token tiles (the down layer split by rank
    through partial tiles in the scratch) and the FP8 streaming kernel (h
    fragment-major in the scratch), two calls in a row."""
    D, F, P = 512, 1024, 4
    print(f"case: mx D={D} F={F} P={P} B={Bs}", flush=True)
    ws = [synth.uniform(80 + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    gu, dn = _mx(np.concatenate([ws[0], ws[1]]), 0, P, S=2), _mx(ws[2], 1, P)
    X = synth.normal(83, (max(Bs), D), 1.0, "bf16")
    for B in Bs:
        x = to_dev(X[:B], "bf16")
        y = torch.empty((B, D), dtype=torch.float32, device=dev())
        before = torch.cuda.memory_allocated()
        sg.mlp_static(gu, dn, x, y)
        assert torch.cuda.memory_allocated() == before
        ref = sg.mlp(gu, dn, x, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), B
