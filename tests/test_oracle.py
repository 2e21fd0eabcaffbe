"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself -- values and shapes the pages fix, closed forms,
invariants the method guarantees, and brute force in exact rational
arithmetic on tiny inputs."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# brute force in exact arithmetic (pure Python, tiny sizes)
# ---------------------------------------------------------------------------
def _fr(a):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a, dtype=np.float64)]


def bf_linear(X, W, b=None):
    """y[i][j] = sum_k X[i][k] * W[j][k] (+ b[j]) exactly."""
    return [[sum((x * w for x, w in zip(xr, wr)), Fraction(0)) + (b[j] if b else 0)
             for j, wr in enumerate(W)] for xr in X]


def bf_matmul(X, A):
    return [[sum((X[i][k] * A[k][j] for k in range(len(A))), Fraction(0))
             for j in range(len(A[0]))] for i in range(len(X))]


def _ints(seed, shape, lo=-3, hi=3):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float64)


# ---------------------------------------------------------------------------
# (a) the worked example's shapes
# ---------------------------------------------------------------------------
def test_worked_example_shapes():
    g = _gold("worked_example.json")
    X, W1, W2 = synth.worked_example(seed=0)
    assert list(X.shape) == g["input_shape"]
    N = g["N"]
    for r in range(N):
        assert list(oracle.slice_(W1, 0, 1, N, r).shape) == g["all_to_sharded"]["weight_slice"]
        assert list(oracle.slice_(W2, 1, 1, N, r).shape) == g["sharded_to_all"]["weight_slice"]
    y1 = oracle.col(X, W1, P=N)
    assert list(y1.shape[1:]) == g["all_to_sharded"]["local_output"]
    y2, z = oracle.row(y1, W2, P=N, partials=True)
    assert list(z.shape[1:]) == g["sharded_to_all"]["local_result"]
    assert list(y2.shape) == g["sharded_to_all"]["final_output"]
    # the chain equals the unsharded two-layer model: one reduction, no gather
    ref = bf_linear(bf_linear(_fr(X), _fr(W1)), _fr(W2))
    np.testing.assert_allclose(y2, np.array(ref, dtype=np.float64), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# slicing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", _gold("slices.json")["cases"], ids=lambda c: f"d{c['dim']}S{c['S']}P{c['P']}")
def test_slice_golden(case):
    dim, S, P = case["dim"], case["S"], case["P"]
    cols = 3
    W = np.arange(dim * cols, dtype=np.int32).reshape(dim, cols)  # entry encodes (row, col)
    for r, rows in enumerate(case["shards"]):
        got = oracle.slice_(W, 0, S, P, r)
        np.testing.assert_array_equal(got, W[rows])
        got_t = oracle.slice_(np.ascontiguousarray(W.T), 1, S, P, r)
        np.testing.assert_array_equal(got_t, W.T[:, rows])


@pytest.mark.parametrize("dim,S,P", [(24, 3, 4), (16, 2, 8), (30, 3, 5), (7, 1, 7)])
def test_slice_partition(dim, S, P):
    """Shards partition the dimension; each shard takes one contiguous run of
    every segment, in segment order (numpy array_split as a second reading)."""
    W = np.arange(dim, dtype=np.int64).reshape(dim, 1)
    seen = []
    for r in range(P):
        sh = oracle.slice_(W, 0, S, P, r).ravel()
        want = np.concatenate([np.array_split(seg, P)[r] for seg in np.array_split(np.arange(dim), S)])
        np.testing.assert_array_equal(sh, want)
        seen.extend(sh.tolist())
    assert sorted(seen) == list(range(dim))


def test_slice_bit_exact_16bit():
    W = synth.uniform(3, (12, 8), 1.0, synth.BF16)
    for r in range(2):
        np.testing.assert_array_equal(oracle.slice_(W, 0, 3, 2, r).view(np.uint16),
                                      W[[x for s in range(3) for x in range(s * 4 + r * 2, s * 4 + r * 2 + 2)]])


# ---------------------------------------------------------------------------
# (c) divisibility rules
# ---------------------------------------------------------------------------
def test_rejects_output_not_divisible():
    X = np.zeros((4, 2))
    with pytest.raises(oracle.OracleError) as e:
        oracle.col(X, np.zeros((3, 2)), P=2)  # out = 3 over 2 devices
    assert e.value.code == 3
    for P in (2, 4, 8):  # 4096 shards over 2, 4, 8
        assert oracle.slice_(np.zeros((4096, 1), np.float32), 0, 1, P, 0).shape == (4096 // P, 1)


def test_rejects_input_not_divisible():
    with pytest.raises(oracle.OracleError) as e:
        oracle.row(np.zeros((3, 1, 1)), np.zeros((2, 5)), P=3)
    assert e.value.code == 3


def test_rejects_segments_not_divisible():
    with pytest.raises(oracle.OracleError):
        oracle.col(np.zeros((1, 2)), np.zeros((12, 2)), P=4, S=2)  # 12/2 = 6 not / 4
    with pytest.raises(oracle.OracleError):
        oracle.col(np.zeros((1, 2)), np.zeros((10, 2)), P=1, S=3)


def test_summa_rejects_bad_grid():
    with pytest.raises(oracle.OracleError):
        oracle.summa(np.zeros((6, 4)), np.zeros((4, 4)), q=4)


# ---------------------------------------------------------------------------
# (e) brute force: column / row / summa in exact arithmetic
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,inn,out,S,P,gather,bias", [
    (3, 5, 4, 1, 2, False, False), (2, 4, 12, 3, 2, False, True), (3, 3, 12, 2, 3, True, True),
    (1, 7, 6, 1, 3, True, False), (4, 2, 2, 1, 1, False, True)])
def test_col_bruteforce(B, inn, out, S, P, gather, bias):
    X, W = _ints(1, (B, inn)), _ints(2, (out, inn))
    b = _ints(3, (out,), 1, 3) if bias else None  # non-zero so a doubled or dropped bias shows
    got = oracle.col(X, W, P=P, S=S, bias=b, gather=gather)
    nl = out // P
    for r in range(P):
        rows = [s * (out // S) + r * (out // S // P) + i for s in range(S) for i in range(out // S // P)]
        ref = bf_linear(_fr(X), _fr(W[rows]), [Fraction(float(v)) for v in b[rows]] if bias else None)
        ref = np.array(ref, dtype=np.float64)
        blk = got[:, r * nl:(r + 1) * nl] if gather else got[r]
        np.testing.assert_array_equal(blk, ref)


@pytest.mark.parametrize("B,inn,out,P,bias", [(3, 6, 5, 2, False), (2, 8, 3, 4, True), (4, 3, 3, 3, True), (1, 5, 2, 1, False)])
def test_row_bruteforce(B, inn, out, P, bias):
    Xf, W = _ints(4, (B, inn)), _ints(5, (out, inn))
    b = _ints(6, (out,), 1, 3) if bias else None
    kl = inn // P
    Xs = np.stack([Xf[:, r * kl:(r + 1) * kl] for r in range(P)])
    Y, Z = oracle.row(Xs, W, P=P, bias=b, partials=True)
    for r in range(P):
        zr = bf_linear(_fr(Xf[:, r * kl:(r + 1) * kl]), _fr(W[:, r * kl:(r + 1) * kl]))
        np.testing.assert_array_equal(Z[r], np.array(zr, dtype=np.float64))
    # bias enters once, after the sum
    ref = bf_linear(_fr(Xf), _fr(W), [Fraction(float(v)) for v in b] if bias else None)
    np.testing.assert_array_equal(Y, np.array(ref, dtype=np.float64))


# ---------------------------------------------------------------------------
# collective layouts of "Sharded Matrices and How to Multiply Them": AllGather
# of the input shards (Case 2) and ReduceScatter of the summed output (Case 3)
# ---------------------------------------------------------------------------
def test_all_gather_index_layout():
    P, B, k = 3, 2, 4
    Xs = np.array([[[100 * r + 10 * b + j for j in range(k)] for b in range(B)] for r in range(P)], dtype=np.float64)
    got = oracle.all_gather(Xs)
    assert got.shape == (B, P * k)
    for b in range(B):
        for c in range(P * k):
            assert got[b, c] == 100 * (c // k) + 10 * b + c % k  # column c of shard c // k


def test_reduce_scatter_index_layout():
    P, B, n = 4, 3, 8
    Y = np.array([[10 * b + c for c in range(n)] for b in range(B)], dtype=np.float64)
    got = oracle.reduce_scatter(Y, P)
    assert got.shape == (P, B, n // P)
    for r in range(P):
        for b in range(B):
            for j in range(n // P):
                assert got[r, b, j] == 10 * b + r * (n // P) + j
    with pytest.raises(oracle.OracleError):
        oracle.reduce_scatter(np.zeros((2, 6)), 4)


@pytest.mark.parametrize("B,inn,out,P", [(3, 6, 4, 2), (2, 9, 6, 3), (1, 8, 8, 4)])
def test_all_gather_then_col_bruteforce(B, inn, out, P):
    """Case 2: y_r = AllGather(x) W_r^T, written out as a sum over the input
    shards straight from the shard arrays."""
    k = inn // P
    Xs, W = _ints(40, (P, B, k)), _ints(41, (out, inn))
    got = oracle.col(oracle.all_gather(Xs), W, P=P)
    nl = out // P
    for r in range(P):
        for i in range(B):
            for j in range(nl):
                ref = sum((Fraction(float(Xs[s, i, kk])) * Fraction(float(W[r * nl + j, s * k + kk]))
                           for s in range(P) for kk in range(k)), Fraction(0))
                assert got[r, i, j] == float(ref)


@pytest.mark.parametrize("B,inn,out,P", [(2, 6, 4, 2), (3, 6, 9, 3)])
def test_row_then_reduce_scatter_bruteforce(B, inn, out, P):
    """Case 3 with ReduceScatter: rank r receives its output columns of the
    rank-order sum, the bias added once."""
    k = inn // P
    Xs, W, b = _ints(42, (P, B, k)), _ints(43, (out, inn)), _ints(44, (out,), 1, 3)
    got = oracle.reduce_scatter(oracle.row(Xs, W, P=P, bias=b), P)
    nl = out // P
    for r in range(P):
        for i in range(B):
            for j in range(nl):
                c = r * nl + j
                ref = sum((Fraction(float(Xs[s, i, kk])) * Fraction(float(W[c, s * k + kk]))
                           for s in range(P) for kk in range(k)), Fraction(0)) + Fraction(float(b[c]))
                assert got[r, i, j] == float(ref)


@pytest.mark.parametrize("M,K,N,q", [(4, 6, 2, 2), (3, 3, 6, 3), (4, 4, 4, 1), (8, 4, 4, 4)])
def test_summa_bruteforce(M, K, N, q):
    X, A = _ints(7, (M, K)), _ints(8, (K, N))
    ref = np.array(bf_matmul(_fr(X), _fr(A)), dtype=np.float64)
    np.testing.assert_array_equal(oracle.summa(X, A, q), ref)


def test_summa_steps_are_equations_1_and_2():
    """q = 2: the two step products (1) and (2) of the SUMMA derivation, summed
    block by block, give Y; each block depends only on its own row / column
    panels."""
    X, A = _ints(9, (4, 4)), _ints(10, (4, 4))
    Y = oracle.summa(X, A, 2)
    step1 = np.zeros((4, 4))
    step2 = np.zeros((4, 4))
    for i in range(2):
        for j in range(2):
            Xi0, Xi1 = X[2 * i:2 * i + 2, 0:2], X[2 * i:2 * i + 2, 2:4]
            A0j, A1j = A[0:2, 2 * j:2 * j + 2], A[2:4, 2 * j:2 * j + 2]
            step1[2 * i:2 * i + 2, 2 * j:2 * j + 2] = np.array(bf_matmul(_fr(Xi0), _fr(A0j)), dtype=float)
            step2[2 * i:2 * i + 2, 2 * j:2 * j + 2] = np.array(bf_matmul(_fr(Xi1), _fr(A1j)), dtype=float)
    np.testing.assert_array_equal(Y, step1 + step2)


# ---------------------------------------------------------------------------
# (b) sharded == unsharded on float data, and (d) the SUMMA identity
# ---------------------------------------------------------------------------
def test_sharded_equals_unsharded_float():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((8, 64))
    Wg, Wu = rng.uniform(-1 / 8, 1 / 8, (256, 64)), rng.uniform(-1 / 8, 1 / 8, (256, 64))
    Wd = rng.uniform(-1 / 16, 1 / 16, (64, 256))
    for P in (1, 2, 4, 8):
        g = oracle.col(X, Wg, P=P, gather=True)
        np.testing.assert_allclose(g, X @ Wg.T, rtol=1e-12, atol=1e-13)
        ys = oracle.mlp(X, Wg, Wu, Wd, P=P, round_dtype="f64")
        gf, uf = X @ Wg.T, X @ Wu.T
        h = gf / (1 + np.exp(-gf)) * uf
        np.testing.assert_allclose(ys, h @ Wd.T, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("q", [1, 2, 4, 8])
def test_summa_identity_float(q):
    rng = np.random.default_rng(12)
    X, A = rng.standard_normal((16, 24)), rng.standard_normal((24, 32))
    np.testing.assert_allclose(oracle.summa(X, A, q), X @ A, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# SwiGLU closed forms
# ---------------------------------------------------------------------------
def test_swiglu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 2.5, -7.0, 40.0, -40.0])
    s = oracle.swiglu(z, np.ones_like(z))
    assert s[0] == 0.0
    assert abs(s[1] - 0.7310585786300049) < 1e-15  # 1 / (1 + 1/e)
    np.testing.assert_allclose(s[[1, 3]] - oracle.swiglu(-z[[1, 3]], np.ones(2)), z[[1, 3]], rtol=1e-14)  # silu(z) - silu(-z) = z
    assert abs(s[5] - 40.0) < 1e-15 * 40 + 1e-15 and abs(s[6]) < 1e-15
    assert np.all(s[[2, 4]] < 0) and np.all(s[[2, 4]] > -0.3)  # silu is bounded below (min ~ -0.278)
    u = np.array([2.0, -3.0, 0.5, 1.0, 1.0, 1.0, 1.0])
    np.testing.assert_allclose(oracle.swiglu(z, u), s * u, rtol=1e-15)


def test_round_matches_independent_rne():
    rng = np.random.default_rng(13)
    v = rng.standard_normal(2000).astype(np.float32)
    v = np.concatenate([v, np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 6e-41, -3e-39, 65520.0 / 65536])])
    want_bf = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v)).astype(np.float64)
    got_bf = np.array([oracle.round_to(float(x), "bf16") for x in v])
    np.testing.assert_array_equal(got_bf, want_bf)
    w = v[np.abs(v) < 60000]
    want_h = w.astype(np.float16).astype(np.float64)
    got_h = np.array([oracle.round_to(float(x), "f16") for x in w])
    np.testing.assert_array_equal(got_h, want_h)


def test_swiglu_rounds_once_to_activation_dtype():
    rng = np.random.default_rng(14)
    g, u = rng.standard_normal(500), rng.standard_normal(500)
    h = oracle.swiglu(g, u, "bf16")
    exact = oracle.swiglu(g, u, "f64")
    assert np.all(np.abs(h - exact) <= 0.5 * oracle.ulp(exact, "bf16") * (1 + 1e-12))
    hb = synth.f32_to_bf16_bits(h.astype(np.float32))
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(hb).astype(np.float64), h)


# ---------------------------------------------------------------------------
# 4-bit affine
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", _gold("q4_words.json")["cases"], ids=lambda c: c["word"])
def test_deq4_hand_words(case):
    gs = 8
    packed = np.array([[int(case["word"], 16)]], dtype=np.uint32)
    s = np.array([[int(case["scale_f16"], 16)]], dtype=np.uint16)
    b = np.array([[int(case["bias_f16"], 16)]], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.deq4(packed, s, b, group_size=gs)[0], np.array(case["w"], dtype=np.float64))


def test_deq4_round_trip_and_groups():
    w = synth.uniform(15, (6, 256), 1 / 64, synth.F32)
    w[2, 64:128] = np.float32(0.0123)  # a constant group
    packed, s, b, q = synth.quantize_q4(w, 64)
    assert q.min() >= 0 and q.max() <= 15
    d = oracle.deq4(packed, s, b, 64)
    sc = np.repeat(s.view(np.float16).astype(np.float64), 64, axis=1)
    bi = np.repeat(b.view(np.float16).astype(np.float64), 64, axis=1)
    # error of a min/max 4-bit code: half a step, plus the fp16 rounding of scale and bias
    bound = 0.5 * sc + 15 * sc * 2 ** -11 + np.abs(bi) * 2 ** -11 + 1e-12
    assert np.all(np.abs(d - w.astype(np.float64)) <= bound)
    assert np.all(d[2, 64:128] == np.float64(np.float16(np.float32(0.0123))))
    # group boundaries: each group uses its own (scale, bias)
    assert np.all((d[:, :64] - bi[:, :64]) / np.where(sc[:, :64] > 0, sc[:, :64], 1) == q[:, :64])


def test_deq4_then_linear_matches_bruteforce():
    packed, s, b, q = synth.quantize_q4(synth.uniform(16, (4, 64), 1 / 8, synth.F32), 64)
    Wd = oracle.deq4(packed, s, b, 64)
    X = _ints(17, (2, 64))
    ref = bf_linear(_fr(X), _fr(Wd))
    np.testing.assert_array_equal(oracle.col(X, Wd, P=2, gather=True), np.array(ref, dtype=np.float64))


# ---------------------------------------------------------------------------
# decoders and metrics
# ---------------------------------------------------------------------------
def test_decoders():
    bits = np.array([0x3C00, 0xC000, 0x0001, 0x03FF, 0x7BFF, 0x0400], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.decode(bits, "f16"),
                                  [1.0, -2.0, 2.0 ** -24, 1023 * 2.0 ** -24, 65504.0, 2.0 ** -14])
    bb = np.array([0x3F80, 0xBF00, 0x4049, 0x0001], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.decode(bb, "bf16"), [1.0, -0.5, 3.140625, 2.0 ** -133])


def test_ulp_and_metrics():
    np.testing.assert_array_equal(oracle.ulp(np.array([1.0, 1.5, 0.75]), "bf16"), [2 ** -7, 2 ** -7, 2 ** -8])
    assert oracle.ulp(np.array([1.0]), "f16")[0] == 2 ** -10
    assert oracle.ulp(np.array([1.0]), "f32")[0] == 2 ** -23
    ref = np.array([1.0, -2.0, 0.5])
    m = oracle.metrics(ref + np.array([2 ** -9, 0, 0]), ref, "bf16")  # within half an ulp
    assert m["maxabs_ulp"] == 0.0 and m["maxabs"] == 2 ** -9
    assert oracle.within(m, "bf16")


def test_within_rejects_outside_the_tolerances():
    """The acceptance rule of every parity test: fp32 outputs relL2 <= 1e-5;
    16-bit outputs relL2 <= 4e-3 and error beyond half an output ulp
    <= 1e-2 * rms(ref).  Each bound is checked on both sides, and each part
    of the 16-bit rule alone must reject."""
    ok16 = {"relL2": 3.9e-3, "maxabs_ulp": 0.9e-2 * 0.25, "rms": 0.25, "maxabs": 0.0}
    assert oracle.within(ok16, "bf16") and oracle.within(ok16, "f16")
    assert not oracle.within(dict(ok16, relL2=4.1e-3), "bf16")       # relL2 bound alone
    assert not oracle.within(dict(ok16, relL2=5e-3), "f16")
    assert not oracle.within(dict(ok16, maxabs_ulp=1.1e-2 * 0.25), "bf16")  # excess bound alone
    # the excess bound scales with rms(ref): 0.05 passes at rms 10, fails at rms 1
    assert oracle.within(dict(ok16, maxabs_ulp=0.05, rms=10.0), "bf16")
    assert not oracle.within(dict(ok16, maxabs_ulp=0.05, rms=1.0), "bf16")
    assert not oracle.within(dict(ok16, maxabs_ulp=5e-3, rms=0.1), "bf16")
    ok32 = {"relL2": 0.9e-5, "maxabs_ulp": 1.0, "rms": 1.0, "maxabs": 1.0}
    assert oracle.within(ok32, "f32")
    assert not oracle.within(dict(ok32, relL2=1.1e-5), "f32")
    assert not oracle.within(dict(ok32, relL2=4e-3), "f32")  # the 16-bit bound is not the fp32 one


def test_within_on_perturbed_outputs():
    """The same rule through metrics(): perturb a reference by known amounts."""
    ref = np.linspace(-2.0, 2.0, 1001)
    nr = np.linalg.norm(ref)
    d = np.zeros_like(ref)
    d[10] = 1.0
    assert oracle.within(oracle.metrics(ref + 0.9e-5 * nr * d, ref, "f32"), "f32")
    assert not oracle.within(oracle.metrics(ref + 1.1e-5 * nr * d, ref, "f32"), "f32")
    rms = float(np.sqrt(np.mean(ref * ref)))
    half = 0.5 * oracle.ulp(ref, "bf16")
    # one element off by half an ulp plus 1.1e-2 rms: relL2 stays tiny, the excess rule rejects
    bad = ref.copy()
    bad[500] += half[500] + 1.1e-2 * rms
    m = oracle.metrics(bad, ref, "bf16")
    assert m["relL2"] < 4e-3 and not oracle.within(m, "bf16")
    good = ref.copy()
    good[500] += half[500] + 0.9e-2 * rms
    assert oracle.within(oracle.metrics(good, ref, "bf16"), "bf16")


# ---------------------------------------------------------------------------
# the gated MLP rounds the sharded h once to the activation dtype
# ---------------------------------------------------------------------------
def _rne(x: Fraction, bits: int, emin: int) -> Fraction:
    """x rounded to `bits` significant bits (minimum normal exponent emin),
    ties to even, in exact rational arithmetic."""
    if x == 0:
        return x
    s = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a)) + 1  # a = f 2^e, 1/2 <= f < 1 (fixed up below)
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    while Fraction(2) ** e <= a:
        e += 1
    e = max(e, emin)
    scaled = a * Fraction(2) ** (bits - e)
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * Fraction(n) * Fraction(2) ** (e - bits)


def test_mlp_rounds_h_once_closed_form():
    """One token, one feature per rank, P = 2: g_r = 40, u_0 = 1 + 2^-7,
    u_1 = 1 + 3 2^-7, so silu(g) u = 40.3125 and 40.9375 up to 2e-16.  The
    stored h is their bf16 rounding (spacing 0.25 in [32, 64)): 40.25 and 41;
    with W_down = [1, 1/2] the output is exactly 60.75, and 60.78125 - 3e-16
    without the rounding."""
    X = np.array([[1.0]])
    Wg = np.array([[40.0], [40.0]])
    Wu = np.array([[1.0078125], [1.0234375]])
    Wd = np.array([[1.0, 0.5]])
    assert oracle.mlp(X, Wg, Wu, Wd, P=2, round_dtype="bf16")[0, 0] == 60.75
    exact = oracle.mlp(X, Wg, Wu, Wd, P=2, round_dtype="f64")[0, 0]
    assert abs(exact - 60.78125) < 1e-12
    # fp16 (11 significant bits, spacing 2^-5 in [32, 64)) keeps both products
    assert oracle.mlp(X, Wg, Wu, Wd, P=2, round_dtype="f16")[0, 0] == 60.78125


def test_mlp_bruteforce_rounded_h():
    """Brute force of the whole chain on tiny bf16-valued inputs: g and u in
    exact rational arithmetic (not rounded), silu in fp64, h rounded once to
    bf16 by an exact rational RNE, the down layer's rank partials summed
    exactly.  Equal bit for bit to oracle.mlp(round_dtype='bf16')."""
    rng = np.random.default_rng(21)
    B, D, F, P = 3, 8, 16, 2
    # bf16-exact inputs: integers and halves scaled so g, u are generally not bf16 values
    X = rng.integers(-8, 9, (B, D)) / 8.0
    Wg = rng.integers(-16, 17, (F, D)) / 16.0
    Wu = rng.integers(-16, 17, (F, D)) / 16.0
    Wd = rng.integers(-8, 9, (D, F)) / 8.0
    g = bf_linear(_fr(X), _fr(Wg))
    u = bf_linear(_fr(X), _fr(Wu))
    h = [[_rne(Fraction(float(gv) / (1.0 + math.exp(-float(gv)))) * uv, 8, -125) for gv, uv in zip(gr, ur)]
         for gr, ur in zip(g, u)]
    ref = np.array(bf_linear(h, _fr(Wd)), dtype=np.float64)
    got = oracle.mlp(X, Wg, Wu, Wd, P=P, round_dtype="bf16")
    np.testing.assert_array_equal(got, ref)
    # the rounding matters on these inputs: the unrounded chain differs
    assert not np.array_equal(oracle.mlp(X, Wg, Wu, Wd, P=P, round_dtype="f64"), ref)


# ---------------------------------------------------------------------------
# MX FP8 ("MLX 张量并行实战指南" 2.3 mode "mxfp8", read as OCP MX: E4M3 elements,
# one E8M0 scale per 32 inputs, no biases)
# ---------------------------------------------------------------------------
def test_e4m3_closed_forms():
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x09: 1.125 * 2.0 ** -6,
             0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for b, v in table.items():
        assert oracle.e4m3(b) == v, hex(b)
    assert math.isnan(oracle.e4m3(0x7F)) and math.isnan(oracle.e4m3(0xFF))


def test_e4m3_monotone_over_every_finite_code():
    vals = [oracle.e4m3(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))          # no gap or overlap between binades
    assert [oracle.e4m3(0x80 | b) for b in range(0x7F)] == [-v for v in vals]


def test_e8m0():
    assert oracle.e8m0(127) == 1.0 and oracle.e8m0(128) == 2.0 and oracle.e8m0(120) == 2.0 ** -7
    assert oracle.e8m0(0) == 2.0 ** -127 and oracle.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0(255))


def test_deq_mx8_hand_bytes():
    codes = np.array([[0x38, 0xB8] + [0x00] * 30 + [0x7E] + [0x01] * 31], dtype=np.uint8)  # 1 row, 2 blocks
    scales = np.array([[126, 130]], dtype=np.uint8)                                          # 2^-1, 2^3
    W = oracle.deq_mx8(codes, scales)
    assert W[0, 0] == 0.5 and W[0, 1] == -0.5 and W[0, 2] == 0.0
    assert W[0, 32] == 448.0 * 8 and W[0, 33] == 2.0 ** -9 * 8


def test_quantize_mxfp8_bounds():
    w = synth.uniform(70, (6, 128), 1 / 64, "f32").astype(np.float64)
    w[2, 32:64] = 0.0                                      # an all-zero block
    codes, scales = synth.quantize_mxfp8(w)
    assert codes.shape == (6, 128) and scales.shape == (6, 4)
    assert not np.any((codes & 0x7F) == 0x7F)               # never NaN
    assert scales[2, 1] == 0 and np.all(codes[2, 32:64] & 0x7F == 0)
    W = oracle.deq_mx8(codes, scales)
    X = scales.astype(np.int64) - 127
    for o in range(6):
        for blk in range(4):
            g = w[o, 32 * blk:32 * (blk + 1)]
            if not np.any(g):
                continue
            amax = np.abs(g).max()
            assert 2.0 ** (X[o, blk] + 8) <= amax < 2.0 ** (X[o, blk] + 9)   # block max in E4M3's top binade
            for k in range(32):
                a = abs(g[k])
                e = max(math.floor(math.log2(a)), X[o, blk] - 6) if a > 0 else X[o, blk] - 6
                # half a unit in the last place of the element's binade (3 mantissa bits);
                # the block max may also saturate from (448, 512) x 2^X down to 448 x 2^X
                bound = max(2.0 ** (e - 4), amax - 448 * 2.0 ** X[o, blk])
                assert abs(W[o, 32 * blk + k] - g[k]) <= bound


def test_deq_mx8_then_linear_matches_bruteforce():
    codes = np.random.default_rng(71).integers(0, 0x7F, size=(4, 64)).astype(np.uint8)
    codes[1, 5] = 0x80 | 0x3C
    scales = np.array([[120, 134], [127, 127], [122, 131], [127, 125]], dtype=np.uint8)  # sums stay exact in fp64
    X = _ints(72, (3, 64))
    W = oracle.deq_mx8(codes, scales)
    got = oracle.col(X, W, P=2)
    Wf = [[Fraction(oracle.e4m3(codes[o, k])) * Fraction(2) ** (int(scales[o, k // 32]) - 127) for k in range(64)]
          for o in range(4)]
    ref = bf_linear(_fr(X), Wf)
    for r in range(2):
        np.testing.assert_array_equal(got[r], np.array([row[2 * r:2 * r + 2] for row in ref], dtype=np.float64))


# ---------------------------------------------------------------------------
# Backward ("MLX 张量并行实战指南" sections 2.1-2.2: sum_gradients; the VJPs of
# the two layers).  Pinned to the forward oracle by central finite differences
# of the linear loss L = sum(G * Y): the layers are linear in X and in W, so
# the difference quotient equals the gradient up to rounding.
# ---------------------------------------------------------------------------
def _fd(f, A, h=0.5):
    g = np.zeros_like(A)
    for idx in np.ndindex(*A.shape):
        Ap, Am = A.copy(), A.copy()
        Ap[idx] += h
        Am[idx] -= h
        g[idx] = (f(Ap) - f(Am)) / (2 * h)
    return g


@pytest.mark.parametrize("S,P", [(1, 2), (2, 2), (1, 3), (1, 1)])
def test_col_bwd_finite_differences(S, P):
    rng = np.random.default_rng(50 + S + 10 * P)
    B, inn, out = 3, 5, 12
    X, W = rng.standard_normal((B, inn)), rng.standard_normal((out, inn))
    G = rng.standard_normal((P, B, out // P))
    loss_x = lambda Xv: float(np.sum(G * oracle.col(Xv, W, P=P, S=S)))
    loss_w = lambda Wv: float(np.sum(G * oracle.col(X, Wv, P=P, S=S)))
    dx, dW = oracle.col_bwd(X, W, G, P=P, S=S)
    np.testing.assert_allclose(dx, _fd(loss_x, X), rtol=1e-10, atol=1e-10)
    gW = _fd(loss_w, W)
    for r in range(P):
        np.testing.assert_allclose(dW[r], oracle.slice_(gW, 0, S, P, r), rtol=1e-10, atol=1e-10)


def test_col_bwd_unsharded_identity():
    """The all_sum of the rank gradients is the unsharded gradient dY W."""
    rng = np.random.default_rng(60)
    B, inn, out, P = 4, 8, 16, 4
    X, W, dYf = rng.standard_normal((B, inn)), rng.standard_normal((out, inn)), rng.standard_normal((B, out))
    G = dYf.reshape(B, P, out // P).transpose(1, 0, 2)  # rank r holds columns [r out/P, (r+1) out/P)
    dx, dW = oracle.col_bwd(X, W, G, P=P)
    np.testing.assert_allclose(dx, dYf @ W, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(list(dW)), dYf.T @ X, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P", [1, 2, 4])
def test_row_bwd_finite_differences(P):
    rng = np.random.default_rng(70 + P)
    B, inn, out = 3, 8, 5
    Xs, W = rng.standard_normal((P, B, inn // P)), rng.standard_normal((out, inn))
    G = rng.standard_normal((B, out))
    loss_x = lambda Xv: float(np.sum(G * oracle.row(Xv, W, P=P)))
    loss_w = lambda Wv: float(np.sum(G * oracle.row(Xs, Wv, P=P)))
    dXs, dW = oracle.row_bwd(Xs, W, G, P=P)
    np.testing.assert_allclose(dXs, _fd(loss_x, Xs), rtol=1e-10, atol=1e-10)
    gW = _fd(loss_w, W)
    for r in range(P):
        np.testing.assert_allclose(dW[r], oracle.slice_(gW, 1, 1, P, r), rtol=1e-10, atol=1e-10)


def test_row_bwd_unsharded_identity():
    rng = np.random.default_rng(80)
    B, inn, out, P = 4, 12, 6, 3
    X, W, dY = rng.standard_normal((B, inn)), rng.standard_normal((out, inn)), rng.standard_normal((B, out))
    Xs = X.reshape(B, P, inn // P).transpose(1, 0, 2)
    dXs, dW = oracle.row_bwd(Xs, W, dY, P=P)
    np.testing.assert_allclose(np.concatenate(list(dXs), axis=1), dY @ W, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(list(dW), axis=1), dY.T @ X, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("q", [1, 2, 3])
def test_summa_backward_finite_differences(q):
    """Matmul_ABT_2D / Matmul_ATB_2D of the SUMMA page: the gradients of
    L = sum(G * summa(X, A, q)) with respect to X and A."""
    rng = np.random.default_rng(90 + q)
    M, K, N = 3 * q, 2 * q, 4 * q
    X, A, G = rng.standard_normal((M, K)), rng.standard_normal((K, N)), rng.standard_normal((M, N))
    np.testing.assert_allclose(oracle.summa_abt(G, A, q),
                               _fd(lambda Xv: float(np.sum(G * oracle.summa(Xv, A, q))), X), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(oracle.summa_atb(X, G, q),
                               _fd(lambda Av: float(np.sum(G * oracle.summa(X, Av, q))), A), rtol=1e-10, atol=1e-10)


def test_backward_bruteforce_exact():
    """The backward products on small integers, in exact rational arithmetic:
    every sum is exact in fp64, so the oracle's loops must match bit for bit
    (a transposed operand, a wrong rank slice or a dropped step changes them)."""
    B, inn, out, P, S = 3, 6, 8, 2, 2
    X, W = _ints(101, (B, inn)), _ints(102, (out, inn))
    G = _ints(103, (P, B, out // P))
    dx, dW = oracle.col_bwd(X, W, G, P=P, S=S)
    want_dx = [[Fraction(0)] * inn for _ in range(B)]
    for r in range(P):
        Wr = _fr(oracle.slice_(W, 0, S, P, r))
        prod = bf_matmul(_fr(G[r]), Wr)
        want_dx = [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(want_dx, prod)]
        np.testing.assert_array_equal(dW[r], np.array(bf_matmul([list(c) for c in zip(*_fr(G[r]))], _fr(X)),
                                                      dtype=np.float64))
    np.testing.assert_array_equal(dx, np.array(want_dx, dtype=np.float64))

    Xs, Wt, dY = _ints(104, (P, B, inn // P)), _ints(105, (out, inn)), _ints(106, (B, out))
    dXs, dWr = oracle.row_bwd(Xs, Wt, dY, P=P)
    for r in range(P):
        Wr = _fr(oracle.slice_(Wt, 1, 1, P, r))
        np.testing.assert_array_equal(dXs[r], np.array(bf_matmul(_fr(dY), Wr), dtype=np.float64))
        np.testing.assert_array_equal(dWr[r], np.array(bf_matmul([list(c) for c in zip(*_fr(dY))], _fr(Xs[r])),
                                                       dtype=np.float64))

    M, K, N, q = 4, 6, 8, 2
    Xm, A, Gm = _ints(107, (M, K)), _ints(108, (K, N)), _ints(109, (M, N))
    np.testing.assert_array_equal(oracle.summa_abt(Gm, A, q),
                                  np.array(bf_matmul(_fr(Gm), [list(c) for c in zip(*_fr(A))]), dtype=np.float64))
    np.testing.assert_array_equal(oracle.summa_atb(Xm, Gm, q),
                                  np.array(bf_matmul([list(c) for c in zip(*_fr(Xm))], _fr(Gm)), dtype=np.float64))
