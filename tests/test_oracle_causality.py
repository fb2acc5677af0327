"""Pins of what the oracle's reading of the attention step implies for
causality, and of its near-tie report.

Causality.  "Long Context Pre-Training with Lighthouse Attention" (Abstract;
Sec. 1, contribution (ii)) says that symmetric pooling keeps left-to-right
causality.  The oracle's plain reading of Sec. 3 (iii) and Eq. (1) (the
ordinary lower-triangular mask over the position-ordered kept entries, each
entry's output copied to all of its tokens by Sec. 3 (iv)) keeps it between
entries only:
  * a token's output depends on the later tokens of its own coarse entry,
    whose q, k and v enter the entry's means;
  * it does not depend on the q, k or v of tokens in later entries once the
    selection is fixed;
  * it does depend on later tokens through the selection, which ranks every
    entry of a level against every other (Fig. 2, selection step).
The three tests below pin each half, so a change of reading (a shift, a mask
of the diagonal) cannot pass unnoticed.

Near ties.  The oracle reports selection boundaries whose fp64 scores lie
within 1e-6 relative of each other (the K-th and the (K+1)-th candidate of a
level); planted cases fix where it must and must not fire.
"""
import numpy as np

import oracle

P, L, K = 4, 3, 1


def _base(seed=3, N=64, H=1, d=16):
    g = np.random.default_rng(seed)
    q, k, v = (g.standard_normal((N, H, d)).astype(np.float32) for _ in range(3))
    return q, k, v


def _fwd(q, k, v, selection=None, K_=K):
    return oracle.forward(q, k, v, P, L, K_, "fp32", want=("sel", "o"), selection=selection)


def _entry_of(res, t, h=0):
    st, lv = res["start"][h], res["level"][h]
    i = int(np.searchsorted(st, t, side="right") - 1)
    return int(st[i]), int(lv[i])


def _coarse_token(res, h=0):
    """First token of a kept entry of level >= 1 with an entry before it (so its
    softmax has more than one key) and one after it."""
    st, lv = res["start"][h], res["level"][h]
    N = int(st[-1]) + P ** int(lv[-1])
    for i in range(1, len(st)):
        s, l = int(st[i]), int(lv[i])
        if l >= 1 and s + P ** l < N:
            return s, l
    raise AssertionError("no coarse entry with a later one")


def test_output_depends_on_later_tokens_of_its_coarse_entry():
    """v of the second token of a coarse entry moves the first token's output."""
    q, k, v = _base()
    r0 = _fwd(q, k, v)
    t, lev = _coarse_token(r0)
    assert lev >= 1
    v2 = v.copy()
    v2[t + 1, 0] += np.float32(1.0)
    r1 = _fwd(q, k, v2)
    assert np.array_equal(r1["start"], r0["start"]) and np.array_equal(r1["level"], r0["level"])
    # o_t = O~_e, and the entry's mean v carries 1/p^l of the change, weighted by
    # the entry's attention to itself (positive under the causal mask)
    delta = np.abs(r1["O"][t, 0] - r0["O"][t, 0]).max()
    assert delta > 1e-3, delta
    # q and k of a later token of the same entry move it as well, with the selection held
    q2 = q.copy()
    q2[t + 1, 0] *= np.float32(-1.0)
    r2 = _fwd(q2, k, v, selection=(r0["start"], r0["level"]))
    assert np.abs(r2["O"][t, 0] - r0["O"][t, 0]).max() > 1e-4


def test_output_ignores_later_entries_when_the_selection_is_fixed():
    """q, k, v of every token after the end of t's entry leave o_t unchanged, bit for bit."""
    q, k, v = _base(seed=5)
    r0 = _fwd(q, k, v)
    t, lev = _coarse_token(r0)
    end = t + P ** lev
    g = np.random.default_rng(11)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[end:] = g.standard_normal(x[end:].shape).astype(np.float32) * np.float32(3.0)
    r1 = _fwd(q2, k2, v2, selection=(r0["start"], r0["level"]))
    assert np.array_equal(r1["O"][:end], r0["O"][:end])
    # and a later token's own output does move (the perturbation is not a no-op)
    assert not np.array_equal(r1["O"][end:], r0["O"][end:])


def test_output_depends_on_later_scores_through_the_selection():
    """Raising the score of a token in a later top-level block takes the refinement
    away from an earlier block: the earlier token's entry, and so its output, change."""
    N, d = 64, 16
    q, k, v = _base(seed=7, N=N, d=d)
    top = P ** (L - 1)                      # 16 tokens per top-level block
    q[:top] *= np.float32(3.0)              # block 0 holds the largest scores
    k[:top] *= np.float32(3.0)
    r0 = _fwd(q, k, v)
    t = 0
    s0, l0 = _entry_of(r0, t)
    assert l0 < L - 1                       # block 0 was refined
    q2, k2 = q.copy(), k.copy()
    late = 3 * top + 5                      # a token of the last block
    q2[late] *= np.float32(20.0)
    k2[late] *= np.float32(20.0)
    r1 = _fwd(q2, k2, v)
    s1, l1 = _entry_of(r1, t)
    assert l1 == L - 1 and s1 == 0          # block 0 is now kept whole
    assert np.abs(r1["O"][t, 0] - r0["O"][t, 0]).max() > 1e-3


# ------------------------------------------------------------------ near ties

def _tie_inputs(second_sq):
    """16 tokens, d = 8: q = k = 0 except token 5 (block 1) with ||q||^2 = 1e6 and
    token 9 (block 2) with ||q||^2 = 1e6 + second_sq (fp32 components)."""
    N, H, d = 16, 1, 8
    q = np.zeros((N, H, d), np.float32)
    k = np.zeros((N, H, d), np.float32)
    v = np.ones((N, H, d), np.float32)
    q[5, 0, 0] = 1000.0
    q[9, 0, 0] = 1000.0
    q[9, 0, 1] = np.sqrt(np.float32(second_sq), dtype=np.float32)
    return q, k, v


def _ties(q, k, v, K_):
    r = oracle.forward(q, k, v, 4, 2, K_, "fp32", want=("sel",))
    return int(r["near_ties"].sum()), r


def test_near_tie_report_fires_at_the_selection_boundary():
    # relative gap 5e-7: the K-th (block 2) and (K+1)-th (block 1) candidates are near
    n, r = _ties(*_tie_inputs(0.5), K_=1)
    assert n == 1
    # block 2 wins in fp32 as well (1e6 + 0.5 is representable): it is the refined one
    assert list(r["level"][0]).count(0) == 4 and r["start"][0][2] == 8
    # relative gap 2e-6: not near
    n, _ = _ties(*_tie_inputs(2.0), K_=1)
    assert n == 0
    # exact tie: reported (and decided by the lower index: block 1 is refined)
    n, r = _ties(*_tie_inputs(0.0), K_=1)
    assert n == 1 and r["start"][0][1] == 4 and r["level"][0][1] == 0
    # with K = 2 both near candidates are selected; the boundary (2nd vs 3rd,
    # 1e6 vs 0) is far apart, so nothing is reported
    n, _ = _ties(*_tie_inputs(0.5), K_=2)
    assert n == 0


def test_near_tie_report_sees_ties_that_fp32_rounds_away():
    """1e8 and 1e8 + 1 are one fp32 value (spacing 8 there): the selection falls to the
    lower index, and the fp64 report flags the boundary (relative gap 1e-8)."""
    N, H, d = 16, 1, 8
    q = np.zeros((N, H, d), np.float32)
    k = np.zeros((N, H, d), np.float32)
    v = np.ones((N, H, d), np.float32)
    q[5, 0, 0] = 10000.0
    q[9, 0, 0] = 10000.0
    q[9, 0, 1] = 1.0
    assert np.float32(1e8) + np.float32(1.0) == np.float32(1e8)
    r = oracle.forward(q, k, v, 4, 2, 1, "fp32", want=("sel",))
    assert int(r["near_ties"].sum()) == 1
    assert r["start"][0][1] == 4 and r["level"][0][1] == 0   # block 1 (lower index) refined
