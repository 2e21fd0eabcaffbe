"""HIP-graph capture of the fused MLP entry points.  sg_mlp and sg_mlp_static
launch kernels only (no allocation, no memset, no host synchronisation), so a
caller can capture them.  Each case captures one call, then replays the graph
several times with eager calls on other inputs (sharing the workspace or the
static scratch) in between, and requires every replay to match the eager
result bit for bit: first for the captured input, then after the input buffer
was overwritten in place with another batch."""
import numpy as np
import pytest
import torch

import sharded_gemm_alltosharded_amd as sg
import synth
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sg.lib()


def _dense(D, F, P, dtype, seed):
    inp = synth.mlp_inputs(8, D, F, P, dtype, seed=seed)
    gu = sg.shard_linear(to_dev(np.concatenate([inp.Wg, inp.Wu]), dtype), "all-to-sharded", segments=2, P=P)
    dn = sg.shard_linear(to_dev(inp.Wd, dtype), "sharded-to-all", P=P)
    return gu, dn


def _q4(w, mode, P, S=1):
    packed, s, b, _ = synth.quantize_q4(w, 64)
    return sg.shard_quantized_linear(torch.from_numpy(packed.view(np.int32)).to(dev()),
                                     torch.from_numpy(s.view(np.int16)).to(dev()),
                                     torch.from_numpy(b.view(np.int16)).to(dev()), w.shape[1], mode,
                                     segments=S, P=P)


def _quantized(D, F, P, seed):
    ws = [synth.uniform(seed + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    return _q4(np.concatenate([ws[0], ws[1]]), "all-to-sharded", P, S=2), _q4(ws[2], "sharded-to-all", P)


def _mx_pair(D, F, P, seed):
    ws = [synth.uniform(seed + i, shp, 1 / np.sqrt(D), "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    gc, gs = synth.quantize_mxfp8(np.concatenate([ws[0], ws[1]]))
    dc, ds = synth.quantize_mxfp8(ws[2])
    return (sg.shard_mxfp8_linear(t(gc), t(gs), "all-to-sharded", segments=2, P=P),
            sg.shard_mxfp8_linear(t(dc), t(ds), "sharded-to-all", P=P))


# (kind, D, F, P, B): the few-token tiles with the down layer split by rank
# (partial tiles, then the rank-order sum kernel); the streaming kernels with a
# fragment-major h; the 4-bit tile kernels with the split down layer; the MX
# FP8 few-token tiles with the split down layer
CASES = [("bf16", 256, 512, 2, 64), ("bf16", 512, 1024, 8, 16), ("q4", 512, 1024, 4, 40),
         ("mx", 512, 1024, 4, 40)]


def _replays(call, xs, out, x1, x2, ref1, ref2, eager2):
    call()  # eager warm-up: every lazily set-up state exists before capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    for r in range(3):
        xs.copy_(x1)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref1), f"replay {r}"
        assert torch.equal(eager2(), ref2), f"eager call after replay {r}"
        xs.copy_(x2)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref2), f"replay {r} on the second batch"


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("static", [False, True], ids=["mlp", "mlp_static"])
def test_mlp_graph_replays(case, static):
    kind, D, F, P, B = case
    print(f"case: {kind} D={D} F={F} P={P} B={B} static={static}", flush=True)
    if kind == "q4":
        gu, dn = _quantized(D, F, P, seed=90)
    elif kind == "mx":
        gu, dn = _mx_pair(D, F, P, seed=94)
    else:
        gu, dn = _dense(D, F, P, kind, seed=91)
    x1 = to_dev(synth.normal(92, (B, D), 1.0, "bf16"), "bf16")
    x2 = to_dev(synth.normal(93, (B, D), 1.0, "bf16"), "bf16")
    ref1 = sg.mlp(gu, dn, x1, out_dtype=torch.float32)
    ref2 = sg.mlp(gu, dn, x2, out_dtype=torch.float32)
    xs = x1.clone()
    out = torch.empty((B, D), dtype=torch.float32, device=dev())
    if static:
        out2 = torch.empty_like(out)
        call = lambda: sg.mlp_static(gu, dn, xs, out)
        eager2 = lambda: sg.mlp_static(gu, dn, x2, out2)
    else:
        ws = sg.mlp_workspace(gu, dn, B, dev())
        call = lambda: sg.mlp(gu, dn, xs, out=out, ws=ws)
        eager2 = lambda: sg.mlp(gu, dn, x2, out_dtype=torch.float32, ws=ws)
    _replays(call, xs, out, x1, x2, ref1, ref2, eager2)
