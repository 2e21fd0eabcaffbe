#!/usr/bin/env python3
"""Throughput of the sharded-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|3|4|5a|5b|5c|6|7|1]

A step is one pass of the workload's whole sharded path over one batch of
synthetic inputs already resident in HBM.  The default workload is the
Llama-style gated MLP decode step (B=16 tokens, D=4096, F=14336, P=8 ranks on
one GPU, bf16): gate/up all-to-sharded with the fused SwiGLU epilogue, then
down sharded-to-all with the fused rank sum, through the fused MLP entry point
(sg_mlp, the sharded h kept in its workspace); --batch sets other token
counts (17-256 run the few-token tile kernel).  Other workloads:

    3   prefill: B=4096, P=4, fused QKV column shard (segments=3) + the MLP
    4   4-bit affine MLP (group 64), B in {1, 8, 32} (--batch; beyond 32 tokens the
        4-bit tile kernel, its roofline on the matrix cores), P=4
    5a  SUMMA Y = X A, 8192^3 bf16, q=4 (--summa fused|steps)
    5b  vocabulary-parallel head, fp16, 32 x 12288 . (50272 x 12288)^T, P=8
    5c  SUMMA backward at 8192^3, q=4: dX = dY A^T and dA = X^T dY
    6   the decode MLP of the default workload with MX FP8 weights (E4M3 codes,
        one E8M0 scale per 32 inputs)
    7   backward of the decode MLP's two sharded layers (input and weight
        gradients, the input-gradient all_sum fused)
    1   the fp32 worked example + the D=64 MLP (launch-bound, for completeness)

Prints ONE JSON line on stdout; progress goes to stderr.  Weight copies are
rotated so that the bytes of one step exceed the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sharded_gemm_alltosharded_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="2", choices=["1", "2", "3", "4", "5a", "5b", "5c", "6", "7"])
    ap.add_argument("--batch", type=int, default=None,
                    help="tokens: the 4-bit workload (1, 8 or 32, default 1; more runs the 4-bit tile kernel) or "
                         "the decode MLP (default 16; 17-256 run the few-token tile kernel)")
    ap.add_argument("--summa", default="fused", choices=["fused", "steps"])
    ap.add_argument("--rank-share", action="store_true",
                    help="configs 2, 3, 4, 5b: only rank 0's share of the layers (P = 1, the per-GPU shapes "
                         "of a deployment with one rank per GPU; the rank-order reduction across GPUs is not run)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MiB",
                    help="instead of a workload, time a plain device copy of this size (counter calibration)")
    return ap.parse_args()


def src_sha(*files):
    """Hash of the kernel sources' code: comments and blank lines removed, so
    a comment edit does not retire a traffic record (the kernel is the same)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            code = line.split("//", 1)[0].strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
class Workload:
    name = ""
    metric = ""
    unit = "GB/s"
    dtype = "bf16"
    bound = "hbm"
    rotate = 1
    steps, warmup = 200, 20
    dominant = ""          # kernel the roofline describes
    dominant_src = ()      # sources it is built from (traffic is void once they change)
    roof_unit = None       # the dominant kernel's roofline unit when it differs from `unit`

    def config(self):
        return {"workload": self.name}

    # The call that launches only the dominant kernel (same kernel, shapes and
    # weights as in the step), for timing it in a back-to-back burst; None when
    # no call launches it alone (its own start/end events are used instead).
    dominant_call = None

    # rank 0's share alone (--rank-share): what one GPU of a one-rank-per-GPU
    # deployment computes locally; None where the workload has no such form
    rank_share = None

    def _share(self, copies_bytes):
        """Shrink to P = 1 and rotate enough weight copies (>= 512 MB) that the
        Infinity Cache cannot hold them; copies_bytes = one copy's weight bytes."""
        self.share_of = self.P
        self.P = 1
        self.rotate = max(2, -(-(512 << 20) // copies_bytes))
        self.name += "-rank-share"


def _dev_tensor(a, dtype):
    import numpy as np
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


class DecodeMLP(Workload):
    """Gated MLP decode: B=16 (or --batch), D=4096, F=14336, P=8, bf16."""
    B, D, F, P = 16, 4096, 14336, 8
    name = "llama-mlp-decode"
    metric = "sharded-MLP decode GB/s (% HBM peak)"
    rotate = 2
    dominant = "skinny_kernel (gate|up all-to-sharded + SwiGLU)"
    dominant_src = ("skinny.hip", "internal.h")

    def __init__(self, B=16):
        self.B = B
        if B > 16:  # beyond one token tile of the streaming kernel
            self.dominant = "tile_nw64_kernel (gate|up all-to-sharded + SwiGLU, few-token tiles)"
            self.dominant_src = ("tile_dma.hip", "internal.h")

    def setup(self):
        import numpy as np
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        B, D, F, P = self.B, self.D, self.F, self.P
        self.inp = inp = synth.mlp_inputs(B, D, F, P, synth.BF16, seed=0)
        self.x = _dev_tensor(inp.X, "bf16")
        gu_w = _dev_tensor(np.concatenate([inp.Wg, inp.Wu]), "bf16")
        dn_w = _dev_tensor(inp.Wd, "bf16")
        self.gu = [sg.shard_linear(gu_w, "all-to-sharded", segments=2, P=P) for _ in range(self.rotate)]
        self.dn = [sg.shard_linear(dn_w, "sharded-to-all", P=P) for _ in range(self.rotate)]
        del gu_w, dn_w
        self.y = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
        self.ws = sg.mlp_workspace(self.gu[0], self.dn[0], B, "cuda")  # the down workspace, then the sharded h
        self.hbuf = torch.empty((P, B, F // P), dtype=torch.bfloat16, device="cuda")
        self.sg = sg
        w = 2 * (2 * F * D + D * F)  # weight bytes, read once
        a = 2 * (B * D + 2 * B * F + B * D)  # x in, h out and back in, y out
        self.units = w + a
        self.dom_units = 2 * (2 * F * D) + 2 * (B * D + B * F)

    def step(self, i, ev=None):
        sg = self.sg
        k = i % self.rotate
        if ev:
            sg.time_next_launch(*ev)
        sg.mlp(self.gu[k], self.dn[k], self.x, out=self.y, ws=self.ws)

    def dominant_call(self, i):
        # the gate|up layer alone (the step stores h fragment-major in the
        # workspace; here row-major, the same kernel and weight stream)
        self.sg.all_to_sharded(self.gu[i % self.rotate], self.x, swiglu=True, out=self.hbuf)

    def rank_share(self):
        self.F //= self.P
        self._share(2 * 3 * self.F * self.D)

    def config(self):
        c = {"workload": self.name, "tokens": self.B, "D": self.D, "F": self.F, "P": self.P,
             "weight_copies_rotated": self.rotate}
        if getattr(self, "share_of", None):
            c["share_of_ranks"] = self.share_of
        return c

    def cpu_baseline(self):
        import oracle
        inp = self.inp
        t0 = time.perf_counter()
        Wg, Wu, Wd = (oracle.decode(w, "bf16") for w in (inp.Wg, inp.Wu, inp.Wd))
        X = oracle.decode(inp.X, "bf16")
        t_dec = time.perf_counter() - t0
        S = 4
        t0 = time.perf_counter()
        oracle.mlp(X[:S], Wg, Wu, Wd, self.P, round_dtype="bf16")
        t_cmp = time.perf_counter() - t0
        t_step = t_dec + t_cmp * self.B / S
        return self.units / t_step / 1e9, t_step, (
            f"oracle MLP on {S} of {self.B} tokens ({t_cmp:.2f} s) scaled x{self.B // S}, plus the fp64 decode "
            f"of all weights ({t_dec:.2f} s); step-equivalent {t_step:.2f} s")


class PrefillMLP(Workload):
    """Prefill: B=4096, QKV (segments 3) + MLP, P=4, bf16."""
    B, D, F, P, H, HD = 4096, 4096, 14336, 4, 32, 128
    name = "llama-prefill-qkv-mlp"
    metric = "sharded-MLP prefill TFLOP/s (% MFMA peak)"
    unit = "TFLOP/s"
    bound = "mfma"
    steps, warmup = 20, 3
    dominant = "tile_pp_kernel 256x256 (gate|up all-to-sharded + SwiGLU)"
    dominant_src = ("tile_dma.hip", "internal.h")

    def setup(self):
        import numpy as np
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        B, D, F, P = self.B, self.D, self.F, self.P
        self.inp = inp = synth.mlp_inputs(B, D, F, P, synth.BF16, seed=0)
        self.wqkv = synth.qkv_weight(D, self.H, self.HD, seed=10)
        self.x = _dev_tensor(inp.X, "bf16")
        self.qkv = sg.shard_linear(_dev_tensor(self.wqkv, "bf16"), "all-to-sharded", segments=3, P=P)
        self.gu = sg.shard_linear(_dev_tensor(np.concatenate([inp.Wg, inp.Wu]), "bf16"), "all-to-sharded",
                                  segments=2, P=P)
        self.dn = sg.shard_linear(_dev_tensor(inp.Wd, "bf16"), "sharded-to-all", P=P)
        nq = 3 * self.H * self.HD
        self.q_out = torch.empty((P, B, nq // P), dtype=torch.bfloat16, device="cuda")
        self.h = torch.empty((P, B, F // P), dtype=torch.bfloat16, device="cuda")
        self.y = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
        self.ws = sg.workspace(self.dn, B, "cuda")
        self.sg = sg
        self.units = 2 * B * D * nq + 2 * B * D * 2 * F + 2 * B * F * D  # FLOP
        self.dom_units = 2 * B * D * 2 * F

    def step(self, i, ev=None):
        sg = self.sg
        sg.all_to_sharded(self.qkv, self.x, out=self.q_out)
        if ev:
            sg.time_next_launch(*ev)
        sg.all_to_sharded(self.gu, self.x, swiglu=True, out=self.h)
        sg.sharded_to_all(self.dn, self.h, out=self.y, ws=self.ws)

    def dominant_call(self, i):
        self.sg.all_to_sharded(self.gu, self.x, swiglu=True, out=self.h)

    def rank_share(self):
        self.F //= self.P
        self.H //= self.P
        self._share(2 * (3 * self.H * self.HD + 3 * self.F) * self.D)

    def config(self):
        c = {"workload": self.name, "tokens": self.B, "D": self.D, "F": self.F, "P": self.P,
             "qkv": f"{self.H} heads x {self.HD}, segments=3"}
        if getattr(self, "share_of", None):
            c["share_of_ranks"] = self.share_of
        return c

    def cpu_baseline(self):
        import oracle
        inp = self.inp
        t0 = time.perf_counter()
        Wg, Wu, Wd, Wq = (oracle.decode(w, "bf16") for w in (inp.Wg, inp.Wu, inp.Wd, self.wqkv))
        X = oracle.decode(inp.X, "bf16")
        t_dec = time.perf_counter() - t0
        S = 32
        t0 = time.perf_counter()
        oracle.col(X[:S], Wq, P=self.P, S=3)
        oracle.mlp(X[:S], Wg, Wu, Wd, self.P, round_dtype="bf16")
        t_cmp = time.perf_counter() - t0
        t_step = t_dec + t_cmp * self.B / S
        return self.units / t_step / 1e12, t_step, (
            f"oracle QKV + MLP on {S} of {self.B} tokens ({t_cmp:.2f} s) scaled x{self.B // S}, plus the fp64 "
            f"decode of all weights ({t_dec:.2f} s); step-equivalent {t_step:.1f} s")


class Q4MLP(Workload):
    """4-bit affine MLP (group 64), D=4096, F=14336, P=4, B tokens."""
    D, F, P = 4096, 14336, 4
    name = "llama-mlp-q4"
    metric = "4-bit sharded-MLP GB/s (% HBM peak)"
    rotate = 6
    dominant = "q4_kernel (gate|up all-to-sharded + SwiGLU)"
    dominant_src = ("q4.hip", "q4_stream.h", "q4_wide.hip", "internal.h")

    def __init__(self, B):
        self.B = B
        if B > 32:  # beyond the streaming kernels: the 4-bit tile kernel, a matrix-core roofline
            self.bound, self.roof_unit = "mfma", "TFLOP/s"
            self.dominant = "q4_tile_dma_kernel 64 x 128 (gate|up all-to-sharded + SwiGLU)"
            self.dominant_src = ("q4tile.hip", "internal.h")

    def setup(self):
        import numpy as np
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        B, D, F, P = self.B, self.D, self.F, self.P
        t0 = time.perf_counter()
        q = synth.q4_mlp_weights(D, F, seed=20)
        log(f"quantized weights in {time.perf_counter() - t0:.1f} s")
        self.q = q
        self.X = synth.normal(0, (B, D), 1.0, synth.BF16)
        self.x = _dev_tensor(self.X, "bf16")

        def dev32(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()

        def dev16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

        gu = [np.concatenate([q["gate"][i], q["up"][i]]) for i in range(3)]
        gt = (dev32(gu[0]), dev16(gu[1]), dev16(gu[2]))
        dt = (dev32(q["down"][0]), dev16(q["down"][1]), dev16(q["down"][2]))
        self.gu = [sg.shard_quantized_linear(*gt, D, "all-to-sharded", segments=2, P=P) for _ in range(self.rotate)]
        self.dn = [sg.shard_quantized_linear(*dt, F, "sharded-to-all", P=P) for _ in range(self.rotate)]
        del gt, dt
        self.y = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
        self.ws = sg.mlp_workspace(self.gu[0], self.dn[0], B, "cuda")  # the down workspace, then the sharded h
        self.hbuf = torch.empty((P, B, F // P), dtype=torch.bfloat16, device="cuda")
        self.sg = sg
        wbytes = lambda rows, cols: rows * cols // 2 + 2 * 2 * rows * (cols // 64)
        self.units = wbytes(2 * F, D) + wbytes(D, F) + 2 * (B * D + 2 * B * F + B * D)
        self.dom_units = wbytes(2 * F, D) + 2 * (B * D + B * F)
        if self.bound == "mfma":
            self.dom_units = 2 * B * D * 2 * F

    def step(self, i, ev=None):
        sg = self.sg
        k = i % self.rotate
        if ev:
            sg.time_next_launch(*ev)
        sg.mlp(self.gu[k], self.dn[k], self.x, out=self.y, ws=self.ws)

    def dominant_call(self, i):
        self.sg.all_to_sharded(self.gu[i % self.rotate], self.x, swiglu=True, out=self.hbuf)

    def rank_share(self):
        self.F //= self.P
        self._share(3 * self.F * self.D * 9 // 16)  # 4.5 bits per weight

    def config(self):
        c = {"workload": self.name, "tokens": self.B, "D": self.D, "F": self.F, "P": self.P,
             "group_size": 64, "bits": 4, "weight_copies_rotated": self.rotate}
        if getattr(self, "share_of", None):
            c["share_of_ranks"] = self.share_of
        return c

    def cpu_baseline(self):
        import oracle
        q = self.q
        t0 = time.perf_counter()
        W = {k: oracle.deq4(*q[k][:3], 64) for k in ("gate", "up", "down")}
        X = oracle.decode(self.X, "bf16")
        t_dec = time.perf_counter() - t0
        S = min(self.B, 4)
        t0 = time.perf_counter()
        oracle.mlp(X[:S], W["gate"], W["up"], W["down"], self.P, round_dtype="bf16")
        t_cmp = time.perf_counter() - t0
        t_step = t_dec + t_cmp * self.B / S
        return self.units / t_step / 1e9, t_step, (
            f"oracle dequantisation of all weights ({t_dec:.2f} s) + MLP on {S} of {self.B} tokens "
            f"({t_cmp:.2f} s, scaled x{self.B / S:g}); step-equivalent {t_step:.2f} s")


class Summa(Workload):
    """SUMMA: X, A (8192, 8192) bf16, q = 4, Y fp32."""
    n, q = 8192, 4
    name = "summa-8192-q4"
    metric = "SUMMA TFLOP/s (% MFMA peak)"
    unit = "TFLOP/s"
    bound = "mfma"
    steps, warmup = 20, 3
    dominant_src = ("tile_dma.hip", "internal.h")

    def __init__(self, fused):
        self.fused = fused
        self.dominant = ("tile_pp_kernel 256x256 on the A_t^T copy (one launch, q steps in registers)" if fused
                         else "whole call: A_t^T copy + q in-place tile_pp_kernel step launches")

    def setup(self):
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        self.Xh, self.Ah = synth.summa_inputs(self.n, seed=30)
        self.X, self.A = _dev_tensor(self.Xh, "bf16"), _dev_tensor(self.Ah, "bf16")
        self.Y = torch.empty((self.n, self.n), dtype=torch.float32, device="cuda")
        # the A_t^T copy's workspace is allocated once, as a caller that reuses it would
        self.ws = torch.empty(sg.summa_workspace(torch.bfloat16, self.n, self.n, self.q), dtype=torch.uint8,
                              device="cuda")
        self.sg = sg
        self.units = 2 * self.n ** 3
        self.dom_units = self.units

    def step(self, i, ev=None):
        if ev and self.fused:
            self.sg.time_next_launch(*ev)
        elif ev:
            ev[0].record()
        self.sg.summa_matmul(self.X, self.A, self.q, out=self.Y, fused=self.fused, workspace=self.ws)
        if ev and not self.fused:
            ev[1].record()

    def config(self):
        return {"workload": self.name, "M": self.n, "K": self.n, "N": self.n, "q": self.q,
                "variant": "fused" if self.fused else "q in-place steps", "Y": "fp32"}

    def cpu_baseline(self):
        import oracle
        t0 = time.perf_counter()
        X, A = oracle.decode(self.Xh, "bf16"), oracle.decode(self.Ah, "bf16")
        t_dec = time.perf_counter() - t0
        S = 8
        t0 = time.perf_counter()
        oracle.summa(X[:S], A, 4 if S % 4 == 0 else 1)
        t_cmp = time.perf_counter() - t0
        t_step = t_dec + t_cmp * self.n / S
        return self.units / t_step / 1e12, t_step, (
            f"oracle SUMMA on {S} of {self.n} rows ({t_cmp:.2f} s) scaled x{self.n // S}, plus decode "
            f"({t_dec:.2f} s); step-equivalent {t_step:.0f} s")


class SummaBackward(Workload):
    """Backward of the SUMMA product Y = X A at 8192^3, q = 4, bf16 in, fp32
    out: dX = dY A^T (Matmul_ABT_2D, matrix-core tile kernels with the q steps
    as K segments) and dA = X^T dY (Matmul_ATB_2D, the same kernels over X^T
    and dY's transposed step blocks in a workspace)."""
    n, q = 8192, 4
    name = "summa-8192-q4-backward"
    metric = "SUMMA backward TFLOP/s (% MFMA peak)"
    unit = "TFLOP/s"
    bound = "mfma"
    steps, warmup = 10, 2
    dominant = "tile_pp_kernel 256x256 (dA = X^T dY over the transposed copies, q steps in registers)"
    dominant_src = ("tile_dma.hip", "internal.h")

    def setup(self):
        import sharded_gemm_alltosharded_amd as sg
        import synth
        self.Xh, self.Ah = synth.summa_inputs(self.n, seed=30)
        self.Gh = synth.normal(113, (self.n, self.n), 1.0, synth.BF16)
        self.X, self.A, self.G = (_dev_tensor(a, "bf16") for a in (self.Xh, self.Ah, self.Gh))
        import torch
        n = sg.lib().sg_summa_backward_workspace(sg.BF16, self.n, self.n, self.n, self.q)
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")  # X^T and dY's transposed step blocks
        self.sg = sg
        self.units = 2 * 2 * self.n ** 3
        self.dom_units = 2 * self.n ** 3

    def step(self, i, ev=None):
        self.sg.summa_backward(self.X, self.A, self.G, self.q, need_da=False)
        if ev:
            self.sg.time_next_launch(*ev)
        self.sg.summa_backward(self.X, self.A, self.G, self.q, need_dx=False, ws=self.ws)

    def config(self):
        return {"workload": self.name, "M": self.n, "K": self.n, "N": self.n, "q": self.q, "grads": "fp32"}

    def cpu_baseline(self):
        import oracle
        t0 = time.perf_counter()
        X, A, G = (oracle.decode(a, "bf16") for a in (self.Xh, self.Ah, self.Gh))
        t_dec = time.perf_counter() - t0
        S = 8
        t0 = time.perf_counter()
        oracle.summa_abt(G[:S], A, 4 if S % 4 == 0 else 1)
        oracle.summa_atb(X[:S], G[:S], 4 if S % 4 == 0 else 1)
        t_cmp = time.perf_counter() - t0
        t_step = t_dec + t_cmp * self.n / S
        return self.units / t_step / 1e12, t_step, (
            f"oracle dX and dA on {S} of {self.n} token rows ({t_cmp:.2f} s) scaled x{self.n // S}, plus decode "
            f"({t_dec:.2f} s); step-equivalent {t_step:.0f} s")


class VocabHead(Workload):
    """Vocabulary-parallel head: X (32, 12288) fp16, W (50272, 12288) fp16, P = 8."""
    B, Hd, V, P = 32, 12288, 50272, 8
    name = "opt175b-vocab-head"
    metric = "vocab-parallel head GB/s (% HBM peak)"
    dtype = "f16"
    steps, warmup = 50, 5
    dominant = "skinny_kernel (all-to-sharded, gathered logits)"
    dominant_src = ("skinny.hip", "internal.h")

    def setup(self):
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        self.Xh, Wh = synth.vocab_head_inputs(self.B, self.Hd, self.V, seed=40)
        self.x = _dev_tensor(self.Xh, "f16")
        wt = _dev_tensor(Wh, "f16")
        self.Wh = Wh
        self.layers = [sg.shard_linear(wt, "all-to-sharded", P=self.P) for _ in range(self.rotate)]
        del wt
        self.y = torch.empty((self.B, self.V), dtype=torch.float16, device="cuda")
        self.sg = sg
        self.units = 2 * (self.V * self.Hd + self.B * self.Hd + self.B * self.V)
        self.dom_units = self.units

    def step(self, i, ev=None):
        if ev:
            self.sg.time_next_launch(*ev)
        self.sg.all_to_sharded(self.layers[i % self.rotate], self.x, gather=True, out=self.y)

    def dominant_call(self, i):
        self.sg.all_to_sharded(self.layers[i % self.rotate], self.x, gather=True, out=self.y)

    def rank_share(self):
        self.V //= self.P
        self._share(2 * self.V * self.Hd)

    def config(self):
        c = {"workload": self.name, "tokens": self.B, "hidden": self.Hd, "vocab": self.V, "P": self.P,
             "rows_per_rank": self.V // self.P}
        if getattr(self, "share_of", None):
            c["share_of_ranks"] = self.share_of
        return c

    def cpu_baseline(self):
        import oracle
        t0 = time.perf_counter()
        W = oracle.decode(self.Wh, "f16")
        X = oracle.decode(self.Xh, "f16")
        t_dec = time.perf_counter() - t0
        S = 2
        t0 = time.perf_counter()
        oracle.col(X[:S], W, P=self.P, gather=True)
        t_cmp = time.perf_counter() - t0
        t_step = t_dec + t_cmp * self.B / S
        return self.units / t_step / 1e9, t_step, (
            f"oracle head on {S} of {self.B} tokens ({t_cmp:.2f} s) scaled x{self.B // S}, plus decode "
            f"({t_dec:.2f} s); step-equivalent {t_step:.1f} s")


class Tiny(Workload):
    """fp32 worked example ((4,2) x (2,2), two ranks) + D=64 F=256 MLP, P=2."""
    name = "worked-example-fp32"
    metric = "fp32 plumbing GB/s (launch-bound)"
    dtype = "f32"
    dominant = "generic_kernel (MLP gate|up + SwiGLU)"
    dominant_src = ("generic.hip", "internal.h")

    def setup(self):
        import numpy as np
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        self.sg = sg
        X, W1, W2 = synth.worked_example(seed=0)
        self.x0 = _dev_tensor(X, "f32")
        self.l1 = sg.shard_linear(_dev_tensor(W1, "f32"), "all-to-sharded", P=2)
        self.l2 = sg.shard_linear(_dev_tensor(W2, "f32"), "sharded-to-all", P=2)
        self.inp = inp = synth.mlp_inputs(8, 64, 256, 2, "f32", seed=0)
        self.x = _dev_tensor(inp.X, "f32")
        self.gu = sg.shard_linear(_dev_tensor(np.concatenate([inp.Wg, inp.Wu]), "f32"), "all-to-sharded",
                                  segments=2, P=2)
        self.dn = sg.shard_linear(_dev_tensor(inp.Wd, "f32"), "sharded-to-all", P=2)
        self.units = 4 * (4 + 4 + 8 + 4 * 2 + 8) + 4 * (3 * 64 * 256 + 8 * 64 * 2 + 8 * 256 * 2)
        self.dom_units = 4 * (2 * 64 * 256 + 8 * 64 + 8 * 256)

    def step(self, i, ev=None):
        sg = self.sg
        sg.sharded_to_all(self.l2, sg.all_to_sharded(self.l1, self.x0))
        if ev:
            sg.time_next_launch(*ev)
        h = sg.all_to_sharded(self.gu, self.x, swiglu=True)
        sg.sharded_to_all(self.dn, h)

    def cpu_baseline(self):
        import oracle
        inp = self.inp
        X, W1, W2 = __import__("synth").worked_example(seed=0)
        t0 = time.perf_counter()
        n = 200
        for _ in range(n):
            oracle.row(oracle.col(X, W1, P=2), W2, P=2)
            oracle.mlp(inp.X, inp.Wg, inp.Wu, inp.Wd, 2, round_dtype="f32")
        t_step = (time.perf_counter() - t0) / n
        return self.units / t_step / 1e9, t_step, f"the whole step x{n}"


class MxfpDecodeMLP(Workload):
    """Gated MLP decode with MX FP8 weights (E4M3 + E8M0 per 32): B=16, D=4096,
    F=14336, P=8, bf16 activations -- the decode shape of config 2 on the
    quantized mode the MLX pages name besides affine."""
    B, D, F, P = 16, 4096, 14336, 8
    name = "llama-mlp-mxfp8-decode"
    metric = "sharded-MLP decode GB/s (% HBM peak)"
    rotate = 2
    dominant = "skinny_kernel FP8 (gate|up all-to-sharded + SwiGLU)"
    dominant_src = ("skinny.hip", "internal.h")

    def setup(self):
        import numpy as np
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        B, D, F, P = self.B, self.D, self.F, self.P
        self.X = synth.normal(90, (B, D), 1.0, synth.BF16)
        self.x = _dev_tensor(self.X, "bf16")
        ws = [synth.uniform(91 + i, shp, 1 / 64, "f32") for i, shp in enumerate([(F, D), (F, D), (D, F)])]
        gc, gs = synth.quantize_mxfp8(np.concatenate([ws[0], ws[1]]))
        dc, ds = synth.quantize_mxfp8(ws[2])
        self.q = (gc, gs, dc, ds)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.gu = [sg.shard_mxfp8_linear(t(gc), t(gs), "all-to-sharded", segments=2, P=P) for _ in range(self.rotate)]
        self.dn = [sg.shard_mxfp8_linear(t(dc), t(ds), "sharded-to-all", P=P) for _ in range(self.rotate)]
        self.y = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
        self.ws = sg.mlp_workspace(self.gu[0], self.dn[0], B, "cuda")  # the down workspace, then the sharded h
        self.hbuf = torch.empty((P, B, F // P), dtype=torch.bfloat16, device="cuda")
        self.sg = sg
        codes = 2 * F * D + D * F
        w = codes + codes // 32  # E4M3 codes + E8M0 scales, read once
        a = 2 * (B * D + 2 * B * F + B * D)
        self.units = w + a
        self.dom_units = (2 * F * D) * 33 // 32 + 2 * (B * D + B * F)

    def step(self, i, ev=None):
        sg = self.sg
        k = i % self.rotate
        if ev:
            sg.time_next_launch(*ev)
        sg.mlp(self.gu[k], self.dn[k], self.x, out=self.y, ws=self.ws)

    def dominant_call(self, i):
        self.sg.all_to_sharded(self.gu[i % self.rotate], self.x, swiglu=True, out=self.hbuf)

    def config(self):
        return {"workload": self.name, "tokens": self.B, "D": self.D, "F": self.F, "P": self.P,
                "weights": "mxfp8 (E4M3, E8M0 per 32)", "weight_copies_rotated": self.rotate}

    def cpu_baseline(self):
        import oracle
        gc, gs, dc, ds = self.q
        t0 = time.perf_counter()
        Wgu, Wd = oracle.deq_mx8(gc, gs), oracle.deq_mx8(dc, ds)
        X = oracle.decode(self.X, "bf16")
        t_dec = time.perf_counter() - t0
        S = 4
        t0 = time.perf_counter()
        oracle.mlp(X[:S], Wgu[:self.F], Wgu[self.F:], Wd, self.P, round_dtype="bf16")
        t_cmp = time.perf_counter() - t0
        t_step = t_dec + t_cmp * self.B / S
        return self.units / t_step / 1e9, t_step, (
            f"oracle MLP on {S} of {self.B} tokens ({t_cmp:.2f} s) scaled x{self.B // S}, plus the fp64 "
            f"dequantisation of all weights ({t_dec:.2f} s); step-equivalent {t_step:.2f} s")


class BackwardMLP(Workload):
    """Backward of the decode MLP's two sharded layers (B=16, D=4096, F=14336,
    P=8, bf16; fp32 weight gradients): the sharded-to-all down layer (dh_r =
    dY W_down,r and dW_down,r = dY^T h_r) and the all-to-sharded gate|up layer
    (dx = the rank-order all_sum of dG_r W_gu,r, and dW_gu,r = dG_r^T x), with
    synthetic upstream gradients dY and dG (the SwiGLU derivative between them
    is elementwise and not part of the sharded path)."""
    B, D, F, P = 16, 4096, 14336, 8
    name = "llama-mlp-backward"
    metric = "sharded-MLP backward GB/s (% HBM peak)"
    steps, warmup = 20, 3
    dominant = "dw_small_kernel (gate|up weight gradient, fp32, streaming writes)"
    dominant_src = ("backward.hip", "internal.h")

    def setup(self):
        import numpy as np
        import torch
        import sharded_gemm_alltosharded_amd as sg
        import synth
        B, D, F, P = self.B, self.D, self.F, self.P
        self.inp = inp = synth.mlp_inputs(B, D, F, P, synth.BF16, seed=0)
        self.x = _dev_tensor(inp.X, "bf16")
        self.gu = sg.shard_linear(_dev_tensor(np.concatenate([inp.Wg, inp.Wu]), "bf16"), "all-to-sharded",
                                  segments=2, P=P)
        self.dn = sg.shard_linear(_dev_tensor(inp.Wd, "bf16"), "sharded-to-all", P=P)
        self.hs = _dev_tensor(synth.normal(100, (P, B, F // P), 1.0, synth.BF16), "bf16")
        self.dy = _dev_tensor(synth.normal(101, (B, D), 1.0, synth.BF16), "bf16")
        self.dg = _dev_tensor(synth.normal(102, (P, B, 2 * F // P), 1.0, synth.BF16), "bf16")
        n = max(sg.lib().sg_layer_backward_workspace(l.handle, B) for l in (self.gu, self.dn))
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")  # transposed operands of the weight gradients
        self.sg = sg
        self.f32 = torch.float32
        w = 2 * (2 * F * D + D * F)              # weights read once by the input-gradient products
        g = 4 * (2 * F * D + D * F)              # fp32 weight gradients written once
        a = 2 * (B * D + B * F + 2 * B * F + B * D + B * F)  # x, h, dG, dY in; dh out (bf16)
        self.units = w + g + a + 4 * B * D       # + dx (fp32)
        self.dom_units = 4 * (2 * F * D) + 2 * (2 * B * F + B * D)  # dW_gu (fp32) out; dG, x in

    def step(self, i, ev=None):
        sg = self.sg
        sg.sharded_to_all_backward(self.dn, self.hs, self.dy, dx_dtype=None, ws=self.ws)
        sg.all_to_sharded_backward(self.gu, None, self.dg, need_dw=False, dx_dtype=self.f32)
        if ev:
            sg.time_next_launch(*ev)
        sg.all_to_sharded_backward(self.gu, self.x, self.dg, need_dx=False, ws=self.ws)

    def dominant_call(self, i):
        self.sg.all_to_sharded_backward(self.gu, self.x, self.dg, need_dx=False, ws=self.ws)

    def config(self):
        return {"workload": self.name, "tokens": self.B, "D": self.D, "F": self.F, "P": self.P,
                "weight_gradients": "fp32"}

    def cpu_baseline(self):
        import numpy as np
        import oracle
        import synth
        inp = self.inp
        t0 = time.perf_counter()
        X = oracle.decode(inp.X, "bf16")
        Wgu = oracle.decode(np.concatenate([inp.Wg, inp.Wu]), "bf16")
        Wd = oracle.decode(inp.Wd, "bf16")
        hs = oracle.decode(synth.normal(100, (self.P, self.B, self.F // self.P), 1.0, synth.BF16), "bf16")
        dy = oracle.decode(synth.normal(101, (self.B, self.D), 1.0, synth.BF16), "bf16")
        dg = oracle.decode(synth.normal(102, (self.P, self.B, 2 * self.F // self.P), 1.0, synth.BF16), "bf16")
        oracle.row_bwd(hs, Wd, dy, P=self.P)
        oracle.col_bwd(X, Wgu, dg, P=self.P, S=2)
        t_step = time.perf_counter() - t0
        return self.units / t_step / 1e9, t_step, (
            f"oracle backward of both layers on the whole step, weight decode included ({t_step:.1f} s)")


def make(args) -> Workload:
    wl = {"1": lambda: Tiny(), "2": lambda: DecodeMLP(args.batch or 16), "3": lambda: PrefillMLP(),
          "4": lambda: Q4MLP(args.batch or 1), "5a": lambda: Summa(args.summa == "fused"),
          "5b": lambda: VocabHead(), "6": lambda: MxfpDecodeMLP(), "7": lambda: BackwardMLP(),
          "5c": lambda: SummaBackward()}[args.config]()
    if getattr(args, "rank_share", False):
        if wl.rank_share is None:
            raise SystemExit(f"--rank-share: config {args.config} has no per-rank form (configs 2, 3, 4, 5b)")
        wl.rank_share()
    return wl


# ---------------------------------------------------------------------------
# counter-derived traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE, see profiles/)
# ---------------------------------------------------------------------------
def load_traffic(wl: Workload, tag: str):
    path = os.path.join(PROFILES, f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != src_sha(*wl.dominant_src):
        return None  # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def calib_copy(mib: int, steps: int):
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "ms_per_copy": ms,
                      "GBps": 2 * n / ms / 1e6}), flush=True)


def time_graph(wl: Workload, K: int, W: int):
    """The same steps replayed from HIP graphs: one graph per rotated weight
    copy holding a single step, and one holding S consecutive steps (cycling
    the copies), S = 8 rounded to whole rotations.  K steps = K // S replays
    of the long graph plus K % S single-step replays; host launch overhead
    and most inter-kernel gaps of the eager path are gone.  None if capture is
    not possible for the workload."""
    import torch
    S = wl.rotate * max(1, 8 // wl.rotate)
    try:
        cap = torch.cuda.Stream()
        singles = []
        for r in range(wl.rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                wl.step(r)
            singles.append(g)
        block = torch.cuda.CUDAGraph()
        with torch.cuda.graph(block, stream=cap):
            for i in range(S):
                wl.step(i)
    except Exception as e:  # capture unsupported for this workload
        log(f"[bench] graph capture failed: {e}")
        return None

    def run(n):
        for _ in range(n // S):
            block.replay()
        for i in range(n % S):
            singles[i % len(singles)].replay()

    run(W)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    run(K)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / K


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: every rank of a sharded layer is emulated on a single MI355X, and "
              "no multi-GPU path is built; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sharded_gemm_alltosharded_amd as sg

    sg.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.calib_copy:
        calib_copy(args.calib_copy, args.steps or 50)
        return

    wl = make(args)
    K = args.steps if args.steps is not None else wl.steps
    W = args.warmup if args.warmup is not None else wl.warmup
    t0 = time.perf_counter()
    wl.setup()
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: setup {time.perf_counter() - t0:.1f} s; warmup {W}, steps {K}")

    for i in range(W):
        wl.step(i)
    torch.cuda.synchronize()

    # The timed loop launches nothing but the steps themselves.  The dominant
    # kernel's own start / end events (armed through sg_time_next_launch, which
    # records them from inside that launch) are taken afterwards, in a
    # separate pass of the same steps, so that arming them never adds to the
    # step time.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        wl.step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    n_samp = max(8, min(25, K))
    if wl.dominant_call is not None:
        # the dominant kernel's call alone, n_samp launches back to back
        # between two events (a launch queued behind a running one starts as
        # soon as it ends, so the per-launch time is the kernel's duration
        # plus the short gap between dependent launches)
        for i in range(3):
            wl.dominant_call(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(n_samp):
            wl.dominant_call(i)
        b.record()
        torch.cuda.synchronize()
        dom_ms = a.elapsed_time(b) / n_samp
        how = f"{n_samp} back-to-back launches of its call alone"
    else:
        # the kernel's own start / end events (sg_time_next_launch), armed in
        # a pass of n_samp steps after the timed ones
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_samp)]
        for a, b in evs:  # create the events before they are armed
            a.record()
            b.record()
        torch.cuda.synchronize()
        for i in range(n_samp):
            wl.step(K + i, evs[i])
        torch.cuda.synchronize()
        dom_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        how = f"its own start/end events, {n_samp} sampled steps after the timed ones"
    log(f"[bench] {ms * 1e3:.1f} us/step; dominant kernel {dom_ms * 1e3:.1f} us ({how})")

    graph_ms = None
    if not args.no_graph:
        graph_ms = time_graph(wl, K, W)
        if graph_ms:
            log(f"[bench] graph replay {graph_ms * 1e3:.1f} us/step")

    scale = 1e9 if wl.unit == "GB/s" else 1e12
    value = wl.units / (ms / 1e3) / scale
    ru = wl.roof_unit or wl.unit  # the dominant kernel's roofline unit
    rscale = 1e9 if ru == "GB/s" else 1e12
    achieved = wl.dom_units / (dom_ms / 1e3) / rscale
    peak = HBM_PEAK_GBS if wl.bound == "hbm" else MFMA_PEAK_TFLOPS[wl.dtype]
    tag = wl.name + (f"-b{wl.B}" if isinstance(wl, Q4MLP) or (isinstance(wl, DecodeMLP) and wl.B != 16) else "") + (
        "-steps" if isinstance(wl, Summa) and not wl.fused else "")
    traffic = load_traffic(wl, tag)
    roofline = {"bound": wl.bound, "achieved": round(achieved, 2), "peak": peak, "unit": ru,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": wl.dominant,
                "kernel_us": round(dom_ms * 1e3, 2), "kernel_samples": n_samp, "kernel_timing": how,
                "algorithmic": f"{wl.dom_units / rscale:.4g} "
                               f"{'GB' if ru == 'GB/s' else 'TFLOP'} per launch"}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        v, t_step, sample = wl.cpu_baseline()
        log(f"[bench] cpu baseline {time.perf_counter() - t0:.1f} s")
        cpu = {"value": round(v, 4), "unit": wl.unit, "cores": oracle.threads(), "kind": "oracle",
               "sample": sample}

    rec = {"metric": wl.metric, "value": round(value, 3), "unit": wl.unit, "n_gpus": 1, "steps": K,
           "warmup": W, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded; shapes of the pages' workloads)",
           "config": wl.config(), "roofline": roofline, "cpu_baseline": cpu,
           "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
           "graph_value": None if graph_ms is None else round(wl.units / (graph_ms / 1e3) / scale, 3)}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
