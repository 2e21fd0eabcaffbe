"""Planted mistakes.  Each test swaps one oracle function for a plausibly
wrong version (on the CPU, through monkeypatch: nothing else runs it) and
checks that the pins in test_oracle.py covering that function then fail, so
the pins are not vacuous."""
import numpy as np
import pytest

import oracle
import test_oracle as pins


def _fails(pin, *args):
    with pytest.raises(Exception):
        pin(*args)


def test_wrong_slice_index(monkeypatch):
    o = oracle.slice_
    monkeypatch.setattr(oracle, "slice_", lambda W, axis, S, P, r: o(W, axis, S, P, (r + 1) % P))
    _fails(pins.test_slice_partition, 24, 3, 4)


def test_bias_sign(monkeypatch):
    o = oracle.col
    monkeypatch.setattr(oracle, "col", lambda X, W, P, S=1, bias=None, gather=False, dtype=None: o(
        X, W, P=P, S=S, bias=None if bias is None else -np.asarray(bias, dtype=np.float64), gather=gather, dtype=dtype))
    _fails(pins.test_col_bruteforce, 2, 4, 12, 3, 2, False, True)


def test_bias_added_by_every_rank(monkeypatch):
    o = oracle.row

    def bad(Xs, W, P, bias=None, dtype=None, partials=False):
        res = o(Xs, W, P=P, bias=bias, dtype=dtype, partials=partials)
        if bias is None:
            return res
        extra = (P - 1) * np.asarray(bias, dtype=np.float64)
        return (res[0] + extra, res[1]) if partials else res + extra

    monkeypatch.setattr(oracle, "row", bad)
    _fails(pins.test_row_bruteforce, 2, 8, 3, 4, True)


def test_transposed_summa_operand(monkeypatch):
    o = oracle.summa
    monkeypatch.setattr(oracle, "summa", lambda X, A, q, dtype=None: o(X, np.ascontiguousarray(np.asarray(A).T), q,
                                                                     dtype=dtype))
    _fails(pins.test_summa_bruteforce, 4, 4, 4, 1)


def test_nibble_order(monkeypatch):
    o = oracle.deq4

    def bad(packed, scales, biases, group_size=64):
        p = np.asarray(packed, dtype=np.uint32)
        rev = np.zeros_like(p)
        for k in range(8):
            rev |= ((p >> np.uint32(4 * k)) & np.uint32(0xF)) << np.uint32(4 * (7 - k))
        return o(rev, scales, biases, group_size)

    monkeypatch.setattr(oracle, "deq4", bad)
    failed = 0
    for case in pins._gold("q4_words.json")["cases"]:
        try:
            pins.test_deq4_hand_words(case)
        except AssertionError:
            failed += 1
    assert failed > 0


def test_silu_sign(monkeypatch):
    o = oracle.swiglu
    monkeypatch.setattr(oracle, "swiglu", lambda g, u, round_dtype="f64": o(-np.asarray(g, dtype=np.float64), u,
                                                                          round_dtype))
    _fails(pins.test_swiglu_closed_forms)


def test_gather_rank_order(monkeypatch):
    o = oracle.col

    def bad(X, W, P, S=1, bias=None, gather=False, dtype=None):
        y = o(X, W, P=P, S=S, bias=bias, gather=gather, dtype=dtype)
        if not gather or P < 2:
            return y
        nl = y.shape[1] // P
        return np.concatenate([y[:, r * nl:(r + 1) * nl] for r in [1, 0] + list(range(2, P))], axis=1)

    monkeypatch.setattr(oracle, "col", bad)
    _fails(pins.test_col_bruteforce, 3, 3, 12, 2, 3, True, True)


def test_subnormals_flushed(monkeypatch):
    o = oracle.decode
    monkeypatch.setattr(oracle, "decode", lambda a, dtype=None: np.where(np.abs(o(a, dtype)) < 2.0 ** -14, 0.0,
                                                                         o(a, dtype)))
    _fails(pins.test_decoders)


def test_col_bwd_wrong_rank_weight(monkeypatch):
    sl = oracle.slice_

    def bad(X, W, dY, P, S=1, dtype=None):
        X, W, dY = (np.asarray(a, dtype=np.float64) for a in (X, W, dY))
        dx = sum(dY[r] @ sl(W, 0, S, P, (r + 1) % P) for r in range(P))
        return dx, np.stack([dY[r].T @ X for r in range(P)])

    monkeypatch.setattr(oracle, "col_bwd", bad)
    _fails(pins.test_col_bwd_finite_differences, 1, 2)


def test_row_bwd_wrong_rank_input(monkeypatch):
    o = oracle.row_bwd

    def bad(Xs, W, dY, P, dtype=None):
        dXs, _ = o(Xs, W, dY, P=P, dtype=dtype)
        Xs64, dY64 = np.asarray(Xs, dtype=np.float64), np.asarray(dY, dtype=np.float64)
        return dXs, np.stack([dY64.T @ Xs64[(r + 1) % P] for r in range(P)])

    monkeypatch.setattr(oracle, "row_bwd", bad)
    _fails(pins.test_row_bwd_finite_differences, 2)


def test_summa_atb_drops_last_step(monkeypatch):
    def bad(X, dY, q, dtype=None):
        X, dY = np.asarray(X, dtype=np.float64), np.asarray(dY, dtype=np.float64)
        b = X.shape[0] // q
        return sum((X[t * b:(t + 1) * b].T @ dY[t * b:(t + 1) * b] for t in range(q - 1)),
                   np.zeros((X.shape[1], dY.shape[1])))

    monkeypatch.setattr(oracle, "summa_atb", bad)
    _fails(pins.test_summa_backward_finite_differences, 2)


def test_summa_abt_wrong_sign(monkeypatch):
    o = oracle.summa_abt
    monkeypatch.setattr(oracle, "summa_abt", lambda dY, A, q, dtype=None: -o(dY, A, q, dtype=dtype))
    _fails(pins.test_summa_backward_finite_differences, 2)


def _within_or(m, out_dtype):
    if out_dtype in ("f32", "f64"):
        return m["relL2"] <= 1e-5
    return m["relL2"] <= 4e-3 or m["maxabs_ulp"] <= 1e-2 * m["rms"]


def _within_no_rms(m, out_dtype):
    if out_dtype in ("f32", "f64"):
        return m["relL2"] <= 1e-5
    return m["relL2"] <= 4e-3 and m["maxabs_ulp"] <= 1e-2


def _within_typo(m, out_dtype):
    if out_dtype in ("f32", "f64"):
        return m["relL2"] <= 1e-5
    return m["relL2"] <= 4e-2 and m["maxabs_ulp"] <= 1e-2 * m["rms"]


def _within_f32_loose(m, out_dtype):
    if out_dtype in ("f32", "f64"):
        return m["relL2"] <= 1e-4
    return m["relL2"] <= 4e-3 and m["maxabs_ulp"] <= 1e-2 * m["rms"]


@pytest.mark.parametrize("bad", [_within_or, _within_no_rms, _within_typo, _within_f32_loose])
def test_within_mutants(monkeypatch, bad):
    monkeypatch.setattr(oracle, "within", bad)
    failed = 0
    for pin in (pins.test_within_rejects_outside_the_tolerances, pins.test_within_on_perturbed_outputs):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0


def test_mlp_skips_rounding_h(monkeypatch):
    o = oracle.mlp
    monkeypatch.setattr(oracle, "mlp", lambda X, Wg, Wu, Wd, P, round_dtype="bf16", dtype=None: o(
        X, Wg, Wu, Wd, P, round_dtype="f64", dtype=dtype))
    _fails(pins.test_mlp_rounds_h_once_closed_form)
    _fails(pins.test_mlp_bruteforce_rounded_h)


def test_mlp_rounds_g_and_u_too(monkeypatch):
    """Rounding the fused gate and up results to the activation dtype before
    SwiGLU (they never leave the kernel, so they must not be rounded)."""
    def bad(X, Wg, Wu, Wd, P, round_dtype="bf16", dtype=None):
        g = oracle.col(X, Wg, P=P, dtype=dtype)
        u = oracle.col(X, Wu, P=P, dtype=dtype)
        rg = np.vectorize(lambda v: oracle.round_to(v, round_dtype))
        h = oracle.swiglu(rg(g), rg(u), round_dtype)
        return oracle.row(h, Wd, P=P, dtype=dtype)

    monkeypatch.setattr(oracle, "mlp", bad)
    _fails(pins.test_mlp_bruteforce_rounded_h)


def test_mlp_rounds_h_twice(monkeypatch):
    """silu(g) rounded on its own before the product with u."""
    def bad(X, Wg, Wu, Wd, P, round_dtype="bf16", dtype=None):
        g = oracle.col(X, Wg, P=P, dtype=dtype)
        u = oracle.col(X, Wu, P=P, dtype=dtype)
        s = oracle.swiglu(g, np.ones_like(g), round_dtype)
        h = np.vectorize(lambda v: oracle.round_to(v, round_dtype))(s * u)
        return oracle.row(h, Wd, P=P, dtype=dtype)

    monkeypatch.setattr(oracle, "mlp", bad)
    _fails(pins.test_mlp_bruteforce_rounded_h)
