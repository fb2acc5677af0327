"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, a hand-worked
example (tests/golden), a library routine the method reduces to in a special
case (torch fp64 scaled_dot_product_attention with autograd), a theorem about
the selection, or an invariant stated for the method.  A plausible mistake in
the oracle (a dropped score term, a reversed sort or tie-break, sum instead of
mean, a transposed operand, a wrong scatter, a dropped gradient term) fails at
least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(x, dtype):
    return si.to_f32(x, dtype).astype(np.float64)


def _inputs(N, H, d, dtype, seed, scale="lognormal", dup=0.0, dout=False):
    return si.make_inputs(N, H, d, dtype, seed=seed, scale=scale, dup=dup, with_dout=dout, threads=4)


# ----------------------------------------------------------------- sizes


def test_subseq_len_closed_form():
    """S = N/p^(L-1) + (L-1)(p-1)K whenever K <= every candidate count
    (each selection replaces one entry by p children); S = N when K covers all."""
    for idx, w in si.WORKLOADS.items():
        N, p, L, K = w["N"], w["p"], w["L"], w["K"]
        top = N // p ** (L - 1)
        assert K <= top
        assert oracle.subseq_len(N, p, L, K) == top + (L - 1) * (p - 1) * K
    expected = {1: 224, 2: 1088, 3: 2688, 4: 3584, 5: 2944}
    for idx, S in expected.items():
        w = si.WORKLOADS[idx]
        assert oracle.subseq_len(w["N"], w["p"], w["L"], w["K"]) == S
    assert oracle.subseq_len(2048, 4, 3, 512) == 2048
    assert oracle.subseq_len(2048, 4, 3, 10 ** 6) == 2048
    assert oracle.subseq_len(2048, 4, 3, 0) == 2048 // 16
    assert oracle.subseq_len(2048, 4, 1, 5) == 2048
    assert oracle.subseq_len(2047, 4, 3, 5) == -1


# ----------------------------------------------------------------- pyramid


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_pyramid_equals_direct_mean_of_leaves(dtype):
    """Level l entry j is the mean of the p^l tokens it covers and the mean of its p children."""
    N, H, d, p, L = 256, 3, 16, 4, 4
    x = _inputs(N, H, d, dtype, 7)["q"]
    lev = oracle.pyramid(x, p, L, dtype)
    leaves = _f64(x, dtype)
    prev = leaves
    for l in range(1, L):
        direct = leaves.reshape(N // p ** l, p ** l, H, d).mean(axis=1)
        np.testing.assert_allclose(lev[l - 1], direct, rtol=1e-12, atol=1e-14)
        children = prev.reshape(N // p ** l, p, H, d).mean(axis=1)
        np.testing.assert_allclose(lev[l - 1], children, rtol=1e-12, atol=1e-14)
        prev = lev[l - 1]


# ----------------------------------------------------------------- scores


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128), ("bf16", 16)])
def test_leaf_score_is_squared_norm_of_q_and_k(dtype, d):
    """Score = ||q_t||^2 + ||k_t||^2 (per head); fp32 result within a few fp32 ulps of exact."""
    N, H = 97, 3
    x = _inputs(N, H, d, dtype, 11)
    s = oracle.leaf_scores(x["q"], x["k"], dtype)
    exact = (_f64(x["q"], dtype) ** 2).sum(-1) + (_f64(x["k"], dtype) ** 2).sum(-1)   # [N, H]
    rel = np.abs(s.T.astype(np.float64) - exact) / exact
    assert rel.max() < (d / 8 + 8 + 2) * 2.0 ** -24


def test_leaf_score_exact_on_integers():
    """Small integer inputs: every partial sum is exact in fp32, so the score is the integer sum."""
    rng = np.random.default_rng(3)
    N, H, d = 40, 2, 128
    q = rng.integers(-8, 9, size=(N, H, d)).astype(np.float32)
    k = rng.integers(-8, 9, size=(N, H, d)).astype(np.float32)
    s = oracle.leaf_scores(q, k, "fp32")
    exact = (q.astype(np.int64) ** 2).sum(-1) + (k.astype(np.int64) ** 2).sum(-1)
    assert np.array_equal(s.T.astype(np.int64), exact)


def _fma32(x, y, a):
    """Correctly rounded fp32 fma via exact rationals."""
    exact = Fraction(float(x)) * Fraction(float(y)) + Fraction(float(a))
    return _round_f32(exact)


def _round_f32(fr):
    if fr == 0:
        return np.float32(0.0)
    f64 = float(fr)                       # correctly rounded to fp64
    lo = np.float32(f64)
    # fix a possible double-rounding error by checking neighbours exactly
    cands = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_leaf_score_fixed_reduction_order():
    """The fp32 rounding follows the stated order (8-element fma groups, xor butterfly over
    groups), recomputed here with exact rational arithmetic for the fma and the adds."""
    N, H, d = 6, 2, 64
    x = _inputs(N, H, d, "fp32", 5)
    s = oracle.leaf_scores(x["q"], x["k"], "fp32")
    for t in range(N):
        for h in range(H):
            tot = []
            for name in ("q", "k"):
                r = x[name][t, h]
                G = d // 8
                a = []
                for g in range(G):
                    acc = np.float32(0.0)
                    for e in range(8):
                        acc = _fma32(r[8 * g + e], r[8 * g + e], acc)
                    a.append(acc)
                off = G // 2
                while off >= 1:
                    a = [_round_f32(Fraction(float(a[g])) + Fraction(float(a[g ^ off]))) for g in range(G)]
                    off //= 2
                tot.append(a[0])
            want = _round_f32(Fraction(float(tot[0])) + Fraction(float(tot[1])))
            assert np.float32(s[h, t]).view(np.uint32) == np.float32(want).view(np.uint32)


def test_score_levels_are_max_over_covered_leaves():
    """Level-l score = max of the p^l leaf scores below it (max-pool is exact)."""
    N, H, d, p, L = 1024, 2, 64, 4, 4
    x = _inputs(N, H, d, "bf16", 9)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, 8, "bf16", want=("levels",))
    lev = r["levels"]
    for l in range(L):
        direct = lev[0].reshape(H, N // p ** l, p ** l).max(axis=2)
        assert np.array_equal(lev[l], direct)


# ----------------------------------------------------------------- selection


def _selected_sets(start, level, N, p, L):
    """Entries (l, j) that were refined: ancestors of some kept entry below them."""
    sel = [set() for _ in range(L)]
    for a, l in zip(start.tolist(), level.tolist()):
        for m in range(l + 1, L):
            sel[m].add(a // p ** m)
    return sel


def _check_partition(start, level, N, p):
    sizes = p ** level.astype(np.int64)
    assert np.all(np.diff(start.astype(np.int64)) > 0)            # strictly increasing
    assert start[0] == 0
    assert np.all(start[:-1].astype(np.int64) + sizes[:-1] == start[1:])   # hole-free
    assert int(start[-1]) + int(sizes[-1]) == N                     # covers [0, N)
    assert np.all(start.astype(np.int64) % sizes == 0)              # aligned blocks


def _rank_key(levels, l, j):
    return (-float(levels[l][j]), j)


@pytest.mark.parametrize("seed,N,p,L,K,dup", [(1, 1024, 4, 4, 5, 0.0), (2, 512, 2, 6, 3, 0.0),
                                              (3, 729, 3, 4, 4, 0.3), (4, 2048, 4, 3, 16, 0.0),
                                              (5, 256, 4, 4, 0, 0.0), (6, 256, 4, 1, 7, 0.0)])
def test_selection_properties(seed, N, p, L, K, dup):
    """Partition, size law, and the defining property of each level's choice: exactly
    min(K, #candidates) entries are refined, and each ranks above every unrefined candidate."""
    H, d = 2, 16
    x = _inputs(N, H, d, "bf16", seed, dup=dup)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", want=("levels", "sel"))
    S = oracle.subseq_len(N, p, L, K)
    for h in range(H):
        st, lv = r["start"][h], r["level"][h]
        _check_partition(st, lv, N, p)
        levels = [r["levels"][l][h] for l in range(L)]
        sel = _selected_sets(st, lv, N, p, L)
        cand = set(range(N // p ** (L - 1)))
        for l in range(L - 1, 0, -1):
            assert sel[l] <= cand
            assert len(sel[l]) == min(K, len(cand))
            unsel = cand - sel[l]
            if sel[l] and unsel:
                worst_sel = max(_rank_key(levels, l, j) for j in sel[l])
                best_unsel = min(_rank_key(levels, l, j) for j in unsel)
                assert worst_sel < best_unsel
            cand = {p * j + c for j in sel[l] for c in range(p)}
        assert len(st) == S


def test_selection_contains_global_topk_leaves():
    """Theorem: with max-pooled scores and the lower-index tie-break, the K best leaves
    (score descending, index ascending) always survive to level 0 as single tokens."""
    rng = np.random.default_rng(0)
    for trial in range(60):
        p = int(rng.integers(2, 5))
        L = int(rng.integers(2, 5))
        N = p ** (L - 1) * int(rng.integers(1, 9))
        K = int(rng.integers(0, 6))
        d = 8
        q = rng.integers(0, 3, size=(N, 1, d)).astype(np.float32)   # small integers: heavy ties
        k = np.zeros_like(q)
        r = oracle.forward(q, k, q, p, L, K, "fp32", want=("levels", "sel"))
        s0 = r["levels"][0][0]
        order = sorted(range(N), key=lambda t: (-float(s0[t]), t))
        leaves = set(r["start"][0][r["level"][0] == 0].tolist())
        for t in order[:min(K, N)]:
            assert t in leaves, (trial, p, L, N, K, t)


def test_selection_all_ties_refines_the_prefix():
    """All scores equal: the lower-index tie-break picks entries 0..K-1 at every level, so the
    kept entries are a closed form: leaves [0, pK), then at level l the entries
    K..pK-1, and at the top every entry from K on."""
    N, H, d, p, L, K = 1024, 1, 8, 4, 4, 3
    q = np.ones((N, H, d), np.float32)
    r = oracle.forward(q, q, q, p, L, K, "fp32", want=("sel",))
    want = [(t, 0) for t in range(p * K)]
    for l in range(1, L - 1):
        want += [(j * p ** l, l) for j in range(K, p * K)]
    want += [(j * p ** (L - 1), L - 1) for j in range(K, N // p ** (L - 1))]
    want.sort()
    assert r["start"][0].tolist() == [a for a, _ in want]
    assert r["level"][0].tolist() == [l for _, l in want]


# ----------------------------------------------------------------- golden


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example_n8.json")))
    P = g["params"]
    N, d = P["N"], P["d"]
    q = np.zeros((N, 1, d), np.float32)
    v = np.zeros((N, 1, d), np.float32)
    dout = np.zeros((N, 1, d), np.float32)
    q[:, 0, 0] = g["inputs"]["q_dim0"]
    v[:, 0, 0] = g["inputs"]["v_dim0"]
    dout[:, 0, 0] = g["inputs"]["dout_dim0"]
    k = np.zeros_like(q)
    r = oracle.forward(q, k, v, P["p"], P["L"], P["K"], "fp32", want=("sel", "o"))
    e = g["expected"]
    assert r["start"][0].tolist() == e["start"]
    assert r["level"][0].tolist() == e["level"]
    O = r["O"][:, 0, :]
    np.testing.assert_allclose(O[:, 0], [float(Fraction(s)) for s in e["O_dim0"]], rtol=1e-14)
    assert np.all(O[:, 1:] == 0)
    b = oracle.backward(q, k, v, dout, P["p"], P["L"], P["K"], (r["start"], r["level"]), "fp32",
                        want=("full",))
    np.testing.assert_allclose(b["dv"][:, 0, 0], [float(Fraction(s)) for s in e["dv_dim0"]], rtol=1e-14)
    np.testing.assert_allclose(b["dk"][:, 0, 0] * math.sqrt(8),
                               [float(Fraction(s)) for s in e["dk_dim0_times_sqrt8"]], rtol=1e-13)
    assert np.all(b["dq"] == 0)
    assert np.all(b["dv"][:, :, 1:] == 0) and np.all(b["dk"][:, :, 1:] == 0)


# ------------------------------------------------- reductions to library routines


def _torch_sdpa(q, k, v):
    """[S, H, d] fp64 -> causal SDPA [S, H, d] (torch CPU, math path)."""
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2).unsqueeze(0), k.permute(1, 0, 2).unsqueeze(0),
        v.permute(1, 0, 2).unsqueeze(0), is_causal=True)
    return o.squeeze(0).permute(1, 0, 2)


def _leaf_tensors(x, dtype, dout=True):
    t = {n: torch.tensor(_f64(x[n], dtype), requires_grad=True) for n in ("q", "k", "v")}
    if dout:
        t["dout"] = torch.tensor(_f64(x["dout"], dtype))
    return t


def _grads(out, t):
    out.backward(t["dout"])
    return {n: t[n].grad.numpy() for n in ("q", "k", "v")}


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_k_covers_everything_equals_causal_sdpa(dtype):
    """K >= N/p: every token is kept as a leaf, the sub-sequence is the identity permutation
    and the layer is full causal attention (forward and gradients)."""
    N, H, d, p, L = 256, 2, 16, 4, 3
    K = N // p
    x = _inputs(N, H, d, dtype, 21, dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, dtype, want=("sel", "o"))
    assert np.array_equal(r["start"], np.tile(np.arange(N, dtype=np.int32), (H, 1)))
    assert np.all(r["level"] == 0)
    t = _leaf_tensors(x, dtype)
    o = _torch_sdpa(t["q"], t["k"], t["v"])
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    g = _grads(o, t)
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (r["start"], r["level"]), dtype,
                        want=("full",))
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(b["d" + n], g[n], rtol=1e-9, atol=1e-11)


def test_single_level_is_sdpa():
    """L = 1: no pooling and no selection; the layer is causal SDPA."""
    N, H, d = 128, 2, 32
    x = _inputs(N, H, d, "fp32", 22, dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], 4, 1, 3, "fp32", want=("sel", "o"))
    t = _leaf_tensors(x, "fp32")
    o = _torch_sdpa(t["q"], t["k"], t["v"])
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("p,L", [(4, 3), (2, 4)])
def test_k_zero_is_pooled_sdpa_repeated(p, L):
    """K = 0: only the top level is kept: O = repeat(SDPA(avgpool_{p^(L-1)}(q, k, v))),
    with gradients through the average pool."""
    N, H, d = 256, 2, 16
    B = p ** (L - 1)
    x = _inputs(N, H, d, "fp32", 23, dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, 0, "fp32", want=("sel", "o"))
    t = _leaf_tensors(x, "fp32")
    pooled = [t[n].reshape(N // B, B, H, d).mean(dim=1) for n in ("q", "k", "v")]
    o = _torch_sdpa(*pooled).repeat_interleave(B, dim=0)
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    g = _grads(o, t)
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, 0, (r["start"], r["level"]), "fp32",
                        want=("full",))
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(b["d" + n], g[n], rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("dtype,seed,N,p,L,K", [("fp32", 31, 512, 4, 4, 3), ("bf16", 32, 243, 3, 4, 2),
                                                ("fp32", 33, 256, 2, 5, 4)])
def test_mixed_levels_match_torch_autograd(dtype, seed, N, p, L, K):
    """Given the oracle's kept entries, rebuild the layer from torch ops (block means, SDPA,
    index copy) and let autograd differentiate it: forward and all gradients must agree."""
    H, d = 2, 16
    x = _inputs(N, H, d, dtype, seed, dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, dtype, want=("sel", "o", "sub", "ot"))
    t = _leaf_tensors(x, dtype)
    outs = []
    for h in range(H):
        st, lv = r["start"][h].tolist(), r["level"][h].tolist()
        g = [torch.stack([t[n][a:a + p ** l, h].mean(dim=0) for a, l in zip(st, lv)]) for n in ("q", "k", "v")]
        o_sub = _torch_sdpa(*(z.unsqueeze(1) for z in g)).squeeze(1)
        slot = torch.tensor(np.repeat(np.arange(len(st)), [p ** l for l in lv]))
        outs.append(o_sub.index_select(0, slot))
    o = torch.stack(outs, dim=1)
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    gr = _grads(o, t)
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (r["start"], r["level"]), dtype,
                        want=("full", "sub"))
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(b["d" + n], gr[n], rtol=1e-9, atol=1e-11)


def test_backward_finite_differences_frozen_selection():
    """Central differences (step 2^-12, exact in fp32 for these inputs) with the selection frozen."""
    N, H, d, p, L, K = 64, 1, 8, 2, 3, 2
    x = _inputs(N, H, d, "fp32", 41, scale="none", dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "fp32", want=("sel", "o"))
    sel = (r["start"], r["level"])
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, sel, "fp32", want=("full",))
    dout = x["dout"].astype(np.float64)
    eps = 2.0 ** -12
    rng = np.random.default_rng(1)
    for name in ("q", "k", "v"):
        for _ in range(6):
            t, e = int(rng.integers(0, N)), int(rng.integers(0, d))
            vals = []
            for sgn in (1, -1):
                z = {n: x[n].copy() for n in ("q", "k", "v")}
                z[name][t, 0, e] = np.float32(z[name][t, 0, e] + sgn * eps)
                o = oracle.forward(z["q"], z["k"], z["v"], p, L, K, "fp32", want=("o",), selection=sel)["O"]
                vals.append(float((o * dout).sum()))
            fd = (vals[0] - vals[1]) / (2 * eps)
            an = b["d" + name][t, 0, e]
            assert abs(fd - an) <= 2e-5 * max(1.0, abs(an)), (name, t, e, fd, an)


def test_adjoints_conserve_mass():
    """Scatter adjoint: sum_i dO~_i = sum_t dO_t.  Pool adjoint: the tokens of an entry
    receive gradients that sum to that entry's gradient."""
    N, H, d, p, L, K = 1024, 2, 16, 4, 4, 6
    x = _inputs(N, H, d, "bf16", 51, dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", want=("sel",))
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (r["start"], r["level"]), "bf16",
                        want=("full", "sub"))
    dout = _f64(x["dout"], "bf16")
    for h in range(H):
        np.testing.assert_allclose(b["dOt"][h].sum(0), dout[:, h].sum(0), rtol=1e-10, atol=1e-9)
        for i, (a, l) in enumerate(zip(r["start"][h].tolist(), r["level"][h].tolist())):
            for n, sub in (("dq", "dQt"), ("dk", "dKt"), ("dv", "dVt")):
                np.testing.assert_allclose(b[n][a:a + p ** l, h].sum(0), b[sub][h, i], rtol=1e-10, atol=1e-12)


def test_condition_sums_bound_and_match_nonnegative_cases():
    """The absolute term sums used for tolerances bound each output, and equal it when
    every term is nonnegative (v >= 0 gives cO = O; dO >= 0 gives cdV = dV)."""
    N, H, d, p, L, K = 256, 2, 16, 4, 3, 4
    x = _inputs(N, H, d, "fp32", 61, dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "fp32", want=("sel", "ot"))
    sel = (r["start"], r["level"])
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, sel, "fp32", want=("sub", "cond"))
    assert np.all(b["cO"] >= np.abs(r["Ot"]) * (1 - 1e-12))
    assert np.all(b["cdQ"] >= np.abs(b["dQt"]) * (1 - 1e-12))
    assert np.all(b["cdK"] >= np.abs(b["dKt"]) * (1 - 1e-12))
    assert np.all(b["cdV"] >= np.abs(b["dVt"]) * (1 - 1e-12))
    vpos = np.abs(x["v"])
    dpos = np.abs(x["dout"])
    r2 = oracle.forward(x["q"], x["k"], vpos, p, L, K, "fp32", want=("sel", "ot"))
    b2 = oracle.backward(x["q"], x["k"], vpos, dpos, p, L, K, (r2["start"], r2["level"]), "fp32",
                         want=("sub", "cond"))
    np.testing.assert_allclose(b2["cO"], r2["Ot"], rtol=1e-12)
    np.testing.assert_allclose(b2["cdV"], b2["dVt"], rtol=1e-12)
