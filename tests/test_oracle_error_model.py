"""Pins of the oracle's tolerance aids: the first-order sensitivity of the
attention outputs and gradients to the rounding of the logits.

The parity tests accept an element of dQ~, dK~ or dV~ (and of the token
gradients) when its error is within a small multiple of u = 2^-24 times
C + C_L.  C is the sum of absolute values of the element's terms; C_L bounds
how far the element moves when each logit s_ij = q_i . k_j / sqrt(d) of
Eq. (1) moves by at most Lam_ij = sum_e |q_ie k_je| / sqrt(d).  Any
computation of the logits in precision u carries such an error, times u.

The pin checks C_L against the oracle's own outputs under an exact
perturbation.  With L = 1 the sub-sequence is the token sequence.  Scaling
every q_ie by (1 + eps sigma_ie), with sigma_ie = +-1 and eps = 2^-15, moves
each logit by at most eps Lam_ij.  Inputs have 8-bit significands, so the
scaled values are exact in fp32.  Every output must then move by at most
eps (C_L + the direct term) to first order; a 5 % margin covers the second
order.  The direct term is C for the product whose other operand is the one
perturbed: dK = dS^T Q for q, and dQ = dS K for k.  The checks also require
that C_L is not a gross overestimate.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si

EPS = 2.0 ** -15


def _inputs(seed, N=96, d=16, scale="student_t3"):
    x = si.make_inputs(N, 1, d, "bf16", seed=seed, scale=scale, with_dout=True, threads=2)
    return {k: si.bf16_to_f32(x[k]) for k in ("q", "k", "v", "dout")}


def _run(q, k, v, do):
    N = q.shape[0]
    r = oracle.forward(q, k, v, 4, 1, 0, "fp32", want=("sel", "ot"))
    b = oracle.backward(q, k, v, do, 4, 1, 0, (r["start"], r["level"]), "fp32", want=("sub", "cond"))
    assert r["start"].shape[1] == N
    return r, b


@pytest.mark.parametrize("seed,scale", [(3, "student_t3"), (4, "lognormal"), (5, "student_t3")])
@pytest.mark.parametrize("which", ["q", "k"])
def test_logit_sensitivity_bounds_the_change_of_every_output(seed, scale, which):
    x = _inputs(seed, scale=scale)
    r0, b0 = _run(x["q"], x["k"], x["v"], x["dout"])
    sigma = np.where(np.random.default_rng(seed + 100).random(x[which].shape) < 0.5, -1.0, 1.0)
    y = dict(x)
    pert = (x[which].astype(np.float64) * (1.0 + EPS * sigma)).astype(np.float32)
    assert np.array_equal(pert.astype(np.float64), x[which].astype(np.float64) * (1.0 + EPS * sigma))
    y[which] = pert
    r1, b1 = _run(y["q"], y["k"], y["v"], y["dout"])
    direct_dq = b0["cdQ"] if which == "k" else 0.0     # dQ = dS K: K itself moved
    direct_dk = b0["cdK"] if which == "q" else 0.0     # dK = dS^T Q: Q itself moved
    checks = (("O~", r1["Ot"] - r0["Ot"], b0["lO"]),
              ("dQ~", b1["dQt"] - b0["dQt"], b0["ldQ"] + direct_dq),
              ("dK~", b1["dKt"] - b0["dKt"], b0["ldK"] + direct_dk),
              ("dV~", b1["dVt"] - b0["dVt"], b0["ldV"]))
    for name, delta, bound in checks:
        ratio = np.abs(delta) / (EPS * bound + 1e-300)
        live = bound > 1e-12 * np.abs(bound).max()
        assert np.all(np.abs(delta)[~live] <= 1e-12), name
        assert ratio[live].max() <= 1.05, (name, float(ratio[live].max()))
        # the bound is attained within a modest factor somewhere (not a trivially large one)
        assert ratio[live].max() >= 0.02, (name, float(ratio[live].max()))


def test_logit_terms_dominate_where_logits_are_large():
    """Heavy-tailed rows make the logits, and so C_L, large against C.  With
    tiny inputs (logits near 0) only the rounding of each row's log-sum-exp
    (|lse| ~ log N) is left in C_L, a few times C at most."""
    big = _inputs(3, scale="student_t3")
    _, b = _run(big["q"], big["k"], big["v"], big["dout"])
    heavy = (b["ldQ"] / np.maximum(b["cdQ"], 1e-300)).max()
    small = {k: (v * np.float32(2.0 ** -6)).astype(np.float32) if k in ("q", "k") else v for k, v in big.items()}
    _, b = _run(small["q"], small["k"], small["v"], small["dout"])
    tiny = (b["ldQ"] / np.maximum(b["cdQ"], 1e-300)).max()
    assert heavy > 10.0 and tiny < 2 * np.log(big["q"].shape[0]) and heavy > 5 * tiny


def test_lse_term_closed_form_at_zero_logits():
    """q = k = 0: every logit is 0, so P_ij = 1 / (i + 1), lse_i = log(i + 1) and
    Lam = 0.  Only the row's log-sum-exp term is left: ldV_j = sum_{i >= j}
    log(i + 1) / (i + 1) |dO_i| elementwise, and ldQ = ldK = lO = 0."""
    N, d = 40, 16
    x = _inputs(9, N=N, d=d, scale="lognormal")
    z = np.zeros_like(x["q"])
    r, b = _run(z, z, x["v"], x["dout"])
    i = np.arange(N, dtype=np.float64)
    w = np.log(i + 1) / (i + 1)                               # P_ij |lse_i| for every j <= i
    dO = np.abs(x["dout"][:, 0, :].astype(np.float64))
    want = np.cumsum((w[:, None] * dO)[::-1], axis=0)[::-1]   # sum over i >= j
    np.testing.assert_allclose(b["ldV"][0], want, rtol=1e-12, atol=0)
    for key in ("ldQ", "ldK", "lO"):
        assert np.all(b[key] == 0.0), key
