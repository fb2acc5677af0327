"""Pins of the oracle's alternative scores (what the parameter-free l2 score is
taken of: Sec. 1 "bidirectional", Fig. 2 "qk scores kq" on the Lighthouse
paper's page), each tied to the default score, which tests/test_oracle_pins.py
pins, or to invariances that the definition fixes."""
import numpy as np
import pytest

import oracle
import synth_inputs as si

QK, KO, QO, PROD = 0, 1, 2, 3


def _x(dtype="bf16", seed=21, N=2048, H=2, d=64):
    return si.make_inputs(N, H, d, dtype, seed=seed, threads=2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_single_sided_scores_equal_default_with_other_side_zero(dtype):
    """||k||^2 alone equals ||q||^2 + ||k||^2 at q = 0 bit for bit (x + 0 = x), and likewise for q."""
    x = _x(dtype)
    zero = np.zeros_like(x["q"])
    assert np.array_equal(oracle.leaf_scores(x["q"], x["k"], dtype, KO).view(np.uint32),
                          oracle.leaf_scores(zero, x["k"], dtype, QK).view(np.uint32))
    assert np.array_equal(oracle.leaf_scores(x["q"], x["k"], dtype, QO).view(np.uint32),
                          oracle.leaf_scores(x["q"], zero, dtype, QK).view(np.uint32))


def test_product_score_is_one_rounded_multiply_of_the_two_sums():
    x = _x()
    sq = oracle.leaf_scores(x["q"], x["k"], "bf16", QO).astype(np.float64)
    sk = oracle.leaf_scores(x["q"], x["k"], "bf16", KO).astype(np.float64)
    want = (sq * sk).astype(np.float32)            # exact product, rounded once to fp32
    assert np.array_equal(oracle.leaf_scores(x["q"], x["k"], "bf16", PROD).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("mode,fixed,changed", [(KO, "k", "q"), (QO, "q", "k")])
def test_single_sided_selection_ignores_the_other_side(mode, fixed, changed):
    N, H, d, p, L, K = 4096, 2, 64, 4, 4, 8
    a = _x(N=N, H=H, d=d, seed=3)
    b = _x(N=N, H=H, d=d, seed=4)
    y = dict(a)
    y[changed] = b[changed]
    r1 = oracle.forward(a["q"], a["k"], a["v"], p, L, K, "bf16", score_mode=mode)
    r2 = oracle.forward(y["q"], y["k"], y["v"], p, L, K, "bf16", score_mode=mode)
    assert np.array_equal(r1["start"], r2["start"]) and np.array_equal(r1["level"], r2["level"])
    r3 = oracle.forward(y["q"], y["k"], y["v"], p, L, K, "bf16", score_mode=QK)
    assert not np.array_equal(r1["start"], r3["start"])      # the default score does see both sides


def test_modes_select_by_their_own_norms():
    """The top-level selection of each mode is the K largest of its fp64 norm (max over each block's
    leaves), whenever the K-th and (K+1)-th are well separated."""
    N, H, d, p, L, K = 4096, 2, 64, 4, 2, 16
    x = _x(N=N, H=H, d=d, seed=9)
    qf = si.to_f32(x["q"], "bf16").astype(np.float64)
    kf = si.to_f32(x["k"], "bf16").astype(np.float64)
    nq, nk = (qf ** 2).sum(-1), (kf ** 2).sum(-1)          # [N, H]
    norms = {QK: nq + nk, KO: nk, QO: nq, PROD: np.sqrt(nq) * np.sqrt(nk)}
    for mode, n in norms.items():
        r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", score_mode=mode)
        for h in range(H):
            blk = n[:, h].reshape(-1, p).max(axis=1)             # level-1 score = max over p leaves
            order = np.argsort(-blk, kind="stable")
            assert blk[order[K - 1]] > blk[order[K]] * (1 + 1e-5)
            chosen = set(order[:K].tolist())
            st, lv = r["start"][h], r["level"][h]
            refined = {int(s // p) for s, l in zip(st, lv) if l == 0}   # level-1 entries replaced by leaves
            assert refined == chosen, (mode, h)
