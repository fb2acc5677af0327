"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs, read its intermediates, and compare with the oracle.

Tolerances (from the acceptance criteria of the layer):
  * integer / index results: bit-exact;
  * bf16 outputs: max |err| / max(1, |ref|) <= 2e-2 and mean|err| / mean|ref| <= 5e-3;
  * fp32 outputs: max |err| / max(1, |ref|) <= 1e-5, and mean|err| / mean|ref| <= 1e-5
    (the criteria give one fp32 figure; it is read as both bounds).
The max-abs bound is applied to values scaled to unit magnitude because a
bf16 value above 4 is spaced 2^-5 or more apart, so rounding even the exact
result to bf16 can move it by more than 2e-2 in absolute terms.

Gradient allowance.  An element of the attention gradients (dQ~, dK~, dV~ and
the token gradients dq, dk, dv made from them) can be so ill-conditioned
that no fp32 evaluation of Eq. (1)'s gradient meets the elementwise bound.
Two effects cause it.  dS = P o (dP - D) cancels.  On heavy-tailed rows the
logits q.k/sqrt(d) are large, so their own rounding moves P.  The oracle
returns, per element, C (the sum of absolute values of its terms) and C_L
(its first-order sensitivity to the rounding of the logits).  Both are
pinned in tests/test_oracle_error_model.py.  For these tensors only, an
element beyond the plain bound is accepted when
    |err| <= out_round * |ref| + KAPPA * u * (C + C_L),   u = 2^-24,
where out_round is the rounding of the type `got` is stored in.  KAPPA
reflects the matrix instruction.  v_mfma_f32_16x16x32_f16 does not round its
33-term sum correctly.  test_gpu_mfma_rounding measures its error at up to
11.3 ulps (and bounds it at 16 ulps = 32u) of the largest addend, the
accumulator included, with no bias.  A gradient element depends on about four
such roundings at the scale of its own terms: the logit, P V for O~ (through
D = dO~ . O~), dP, and the gradient product.  So KAPPA = 4 * 32 = 128.  The
largest ratio measured over all workloads is about 69 (dQ~ of the
heavy-tailed 1M-token workload).
Every other tensor (o, O~, lse, the gathered rows, dO~) must meet the plain
bound.  Every comparison is recorded, and a per-tensor summary is printed at
the end of the run (conftest.pytest_terminal_summary).
"""
from __future__ import annotations

import os
import re
import sys

import numpy as np
import torch

import oracle
import synth_inputs as si

TOL = {"bf16": dict(max_scaled=2e-2, mean_rel=5e-3), "fp32": dict(max_scaled=1e-5, mean_rel=1e-5)}
U32 = 2.0 ** -24
KAPPA = 128.0

# one record per comparison: the per-tensor table at the end of the run reads these
RESULTS: list[dict] = []


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def lib():
    import hierarchical_selection_attention_amd as lh
    return lh


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _base_name(what: str) -> str:
    return re.sub(r"\s*\(\d+ sampled rows\)", "", what).strip()


def compare(got, ref, dtype, what="", allow=None, stored="fp32"):
    """Compare `got` with `ref` at the tolerance of `dtype`.

    allow: None, or (C, C_L) arrays shaped like `ref` for the attention gradients:
    elements beyond the plain bound are then accepted within
    out_round * |ref| + KAPPA * u * (C + C_L), where out_round is the relative
    rounding of the type `got` is stored in (2^-8 for bf16 token rows, 2^-24 for
    the fp32 sub-sequence tensors).  The reported ratio is the largest
    (|err| - out_round |ref|) / (u (C + C_L)) over all elements: how far the
    kernel is from the rounding level of its inputs.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    t = TOL[dtype]
    err = np.abs(got - ref)
    scaled_all = err / np.maximum(1.0, np.abs(ref))
    scaled = float(scaled_all.max()) if err.size else 0.0
    denom = float(np.abs(ref).mean()) if ref.size else 0.0
    mean_rel = float(err.mean() / denom) if denom > 0 else float(err.mean())
    over = scaled_all > t["max_scaled"]
    n_over = int(over.sum())
    ratio = None
    if allow is not None:
        c, cl = (np.asarray(a, dtype=np.float64) for a in allow)
        budget = U32 * (c + cl)
        rnd = (2.0 ** -8 if stored == "bf16" else 2.0 ** -24) * np.abs(ref)
        excess = np.maximum(err - rnd, 0.0) / np.maximum(budget, 1e-300)
        ratio = float(excess.max()) if err.size else 0.0
        bad = over & (excess > KAPPA)
    else:
        bad = over
    n_allowed = n_over - int(bad.sum())
    rec = dict(test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what=_base_name(what),
               dtype=dtype, n=int(err.size), max_scaled=scaled, mean_rel=mean_rel, n_over=n_over,
               n_allowed=n_allowed, ratio=ratio, ok=not bad.any() and mean_rel <= t["mean_rel"])
    RESULTS.append(rec)
    if ratio is not None and ratio > KAPPA / 4 and os.environ.get("LH_PARITY_DEBUG"):
        flat = np.argsort(excess, axis=None)[-5:][::-1]
        for f in flat:
            i = np.unravel_index(int(f), err.shape)
            say(f"      worst {i}: got {got[i]:.8g} ref {ref[i]:.8g} C {c[i]:.4g} C_L {cl[i]:.4g} "
                f"err/(u(C+C_L)) {excess[i]:.2f}")
    say(f"    {what}: max_scaled={scaled:.3e} mean_rel={mean_rel:.3e}"
        + (f" err/(u(C+C_L)) max={ratio:.2f}" if ratio is not None else "")
        + (f" (beyond the plain bound, within the gradient allowance: {n_allowed})" if n_allowed else ""))
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, scaled_all, -1))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond tolerance; worst at {i}: "
                             f"got {got[i]:.6g} ref {ref[i]:.6g} scaled err {scaled_all[i]:.3e}")
    assert mean_rel <= t["mean_rel"], f"{what}: mean relative error {mean_rel:.3e} > {t['mean_rel']}"
    return scaled, mean_rel


GEMM_KAPPA = 2.0


def compare_product(got, A, B, what, out_dtype):
    """got ~= A @ B for fp64 A, B holding the exact values of the GPU's own operands.

    A GEMM that accumulates in fp32 and rounds once to `out_dtype` is within
        out_round * |ref| + GEMM_KAPPA * sqrt(k) * u * C,   C = |A| @ |B|,
    elementwise (out_round = 2^-8 for bf16, 2^-24 for fp32; k = the contraction
    length; sqrt(k) u C is the size of the accumulated rounding error of a sum of
    k terms).  Far below what one dropped or doubled contraction row would
    change at the small sizes (about C / k), so such a mistake fails it.
    """
    got = np.asarray(got, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    ref = A @ B
    C = np.abs(A) @ np.abs(B)
    k = A.shape[-1]
    out_round = 2.0 ** -8 if out_dtype == "bf16" else 2.0 ** -24
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    excess = np.maximum(err - out_round * np.abs(ref), 0.0) / np.maximum(U32 * C, 1e-300)
    ratio = float(excess.max() / np.sqrt(k)) if err.size else 0.0
    bad = excess > GEMM_KAPPA * np.sqrt(k)
    scaled = float((err / np.maximum(1.0, np.abs(ref))).max()) if err.size else 0.0
    denom = float(np.abs(ref).mean()) if ref.size else 0.0
    mean_rel = float(err.mean() / denom) if denom > 0 else float(err.mean())
    RESULTS.append(dict(test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what=what, dtype=out_dtype,
                        n=int(err.size), max_scaled=scaled, mean_rel=mean_rel, n_over=int(bad.sum()), n_allowed=0,
                        ratio=ratio, ok=not bad.any()))
    say(f"    {what}: GEMM check k={k}: max (err - rounding)/(sqrt(k) u C)={ratio:.3f} (bound {GEMM_KAPPA:g}); "
        f"max_scaled={scaled:.3e} mean_rel={mean_rel:.3e}")
    if bad.any():
        i = np.unravel_index(int(np.argmax(excess)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond the GEMM bound; worst at {i}: got {got[i]:.6g} "
                             f"ref {ref[i]:.6g} excess {excess[i] / np.sqrt(k):.3g} sqrt(k) u C")


def write_summary(write_line):
    """Per-tensor table of every comparison of the run (worst case over the checks)."""
    groups: dict[tuple, list] = {}
    for r in RESULTS:
        groups.setdefault((r["what"], r["dtype"]), []).append(r)
    write_line("parity summary: worst over all checks of each tensor "
               "(bound: bf16 max_scaled 2e-2, mean_rel 5e-3; fp32 1e-5; gradient allowance "
               f"{KAPPA:g}*u*(C+C_L), u=2^-24)")
    write_line(f"{'tensor':<26}{'dtype':<6}{'checks':>7}{'max_scaled':>12}{'mean_rel':>11}"
               f"{'beyond':>9}{'allowed':>9}{'err/u(C+CL)':>13}  worst check")
    order = sorted(groups.items(), key=lambda kv: (kv[0][0].startswith("d"), max(r["n_allowed"] for r in kv[1]),
                                                   max(r["max_scaled"] for r in kv[1])))
    for (what, dt), rs in order:
        w = max(rs, key=lambda r: r["max_scaled"])
        ratios = [r["ratio"] for r in rs if r["ratio"] is not None]
        write_line(f"{what[:25]:<26}{dt:<6}{len(rs):>7}{w['max_scaled']:>12.3e}"
                   f"{max(r['mean_rel'] for r in rs):>11.2e}{sum(r['n_over'] for r in rs):>9}"
                   f"{sum(r['n_allowed'] for r in rs):>9}"
                   f"{(max(ratios) if ratios else float('nan')):>13.2f}  {w['test'].split('::')[-1][:48]}")


class Run:
    """One forward (+ optional backward) of the HIP path with its workspace kept."""

    def __init__(self, x, dtype, p, L, K, backward=False, mode=0, label="", score_mode=0, keep_leaves=True):
        lh = lib()
        self.dtype, self.p, self.L, self.K = dtype, p, L, K
        self.keep_leaves = keep_leaves
        self.N, self.H, self.d = x["q"].shape
        self.code = 0 if dtype == "bf16" else 1
        self.S = int(lh.lh_subseq_len(self.N, p, L, K))
        self.Sp = (self.S + 63) // 64 * 64
        say(f"  GPU run {label}: N={self.N} H={self.H} d={self.d} {dtype} p={p} L={L} K={K} "
            f"S={self.S} backward={backward} mode={mode} score_mode={score_mode} keep_leaves={keep_leaves}")
        self.q, self.k, self.v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
        self.o, self.ws = lh.forward(self.q, self.k, self.v, p, L, K, score_mode=score_mode,
                                     keep_leaf_scores=keep_leaves)
        if backward:
            self.dout = to_dev(x["dout"], dtype)
            self.grads = lh.backward(self.dout, p, L, K, self.ws, mode=mode, keep_sub_grads=True)
        torch.cuda.synchronize()
        say("  GPU run done")

    def view(self, name):
        lh = lib()
        return lh.workspace_tensor(self.ws, self.N, self.H, self.d, self.p, self.L, self.K, self.code, name)

    def scores(self):
        flat = self.view("scores").cpu().numpy()
        out, off = [], 0
        for l in range(self.L):
            n = self.N // self.p ** l
            out.append(flat[off: off + n * self.H].reshape(self.H, n))
            off += n * self.H
        return out

    def selection(self):
        return (self.view("sel_start").cpu().numpy(), self.view("sel_level").cpu().numpy().astype(np.int8))

    def sub(self, name):
        t = self.view(name)
        return to_f64(t[:, : self.S])


def check_selection(run: Run, ref: dict):
    st, lv = run.selection()
    assert np.array_equal(st, ref["start"]), "selected starts differ from the oracle"
    assert np.array_equal(lv, ref["level"]), "selected levels differ from the oracle"
    ties = int(np.sum(ref["near_ties"]))
    if ties:
        say(f"    near-ties at selection boundaries (reported, not failed): {ties}")


def check_scores(run: Run, ref: dict):
    """Every level of the score view bit for bit; level 0 only when the run stored it (the
    layer's default path leaves it out: the selection ranks levels >= 1, and level 1 is the
    max-pool of the leaves)."""
    g = run.scores()
    for l in range(run.L):
        if l == 0 and run.L > 1 and not run.keep_leaves:
            continue
        a = np.ascontiguousarray(g[l]).view(np.uint32)
        b = np.ascontiguousarray(ref["levels"][l]).view(np.uint32)
        bad = int(np.sum(a != b))
        assert bad == 0, f"level {l}: {bad} scores differ bitwise from the oracle"


def slot_index(start_h: np.ndarray, level_h: np.ndarray, p: int) -> np.ndarray:
    """Token -> slot map of one head (each kept entry covers p^level tokens)."""
    return np.repeat(np.arange(start_h.size), p ** level_h.astype(np.int64))


def check_full_rows(got_dev: torch.Tensor, ref_sub: np.ndarray, sel, p, dtype, what, divide=False,
                    sample=None, rng=None, allow_sub=None):
    """got [N, H, d] vs ref_sub[h][slot(t)] (optionally / p^level) for every token, or a sample.
    allow_sub: the (C, C_L) sums of the sub-sequence tensor for the gradient allowance, or None."""
    N, H, d = got_dev.shape
    st, lv = sel
    if sample is None:
        t = np.arange(N).repeat(H)
        h = np.tile(np.arange(H), N)
        got = to_f64(got_dev).reshape(N * H, d)
    else:
        t = rng.integers(0, N, size=sample)
        h = rng.integers(0, H, size=sample)
        got = to_f64(got_dev[torch.from_numpy(t).cuda(), torch.from_numpy(h).cuda()])
    ref = np.empty((t.size, d))
    allow = None if allow_sub is None else (np.empty((t.size, d)), np.empty((t.size, d)))
    for hh in range(H):
        msk = h == hh
        slot = np.searchsorted(st[hh], t[msk], side="right") - 1
        div = (p ** lv[hh][slot].astype(np.int64))[:, None] if divide else 1.0
        ref[msk] = ref_sub[hh][slot] / div
        if allow is not None:
            for a, src in zip(allow, allow_sub):
                a[msk] = src[hh][slot] / div
    label = what if sample is None else what + f" ({sample} sampled rows)"
    return compare(got, ref, dtype, label, allow=allow, stored=dtype)


def grad_allow(b: dict, name: str):
    """(C, C_L) of a sub-sequence gradient from an oracle backward result: name in dQt/dKt/dVt."""
    k = name[1]   # Q, K or V
    return b["cd" + k], b["ld" + k]
