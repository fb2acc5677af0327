"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs, read its intermediates, and compare with the oracle.

Tolerances (from the acceptance criteria of the layer):
  * integer / index results: bit-exact;
  * bf16 outputs: max |err| / max(1, |ref|) <= 2e-2 and mean|err| / mean|ref| <= 5e-3;
  * fp32 outputs: max |err| / max(1, |ref|) <= 1e-5.
The max-abs bound is applied to values scaled to unit magnitude because a
bf16 value above 4 is spaced 2^-5 or more apart, so rounding even the exact
result to bf16 can move it by more than 2e-2 in absolute terms.

Where an output is a sum of terms that cancel (the attention gradients on
heavy-tailed inputs), any fp32 evaluation of the formula carries an error of
order n*u*C, with C the sum of absolute values of its terms (u = 2^-24, n the
dot-product length); the oracle returns C.  Such elements are also accepted
when |err| <= 2 d u C; the number of elements that needed it is reported.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth_inputs as si

TOL = {"bf16": dict(max_scaled=2e-2, mean_rel=5e-3), "fp32": dict(max_scaled=1e-5, mean_rel=1e-6)}


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


U32 = 2.0 ** -24


def compare(got, ref, dtype, what="", cond=None, d=128, cond_unit=None):
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
    n_cond = 0
    if cond is not None and over.any():
        allow = (2.0 * d * U32 if cond_unit is None else cond_unit) * np.asarray(cond, dtype=np.float64)
        bad = over & (err > allow)
        n_cond = int(over.sum() - bad.sum())
        worst = float((err / np.maximum(t["max_scaled"] * np.maximum(1.0, np.abs(ref)), allow))[over].max())
    else:
        bad = over
        worst = scaled / t["max_scaled"]
    say(f"    {what}: max_scaled={scaled:.3e} mean_rel={mean_rel:.3e}"
        + (f" (elements within the cancellation bound only: {n_cond}, worst/allowed={worst:.2f})"
           if n_cond else ""))
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, scaled_all, -1))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond tolerance; worst at {i}: "
                             f"got {got[i]:.6g} ref {ref[i]:.6g} scaled err {scaled_all[i]:.3e}")
    assert mean_rel <= t["mean_rel"], f"{what}: mean relative error {mean_rel:.3e} > {t['mean_rel']}"
    return scaled, mean_rel


class Run:
    """One forward (+ optional backward) of the HIP path with its workspace kept."""

    def __init__(self, x, dtype, p, L, K, backward=False, mode=0, label="", score_mode=0):
        lh = lib()
        self.dtype, self.p, self.L, self.K = dtype, p, L, K
        self.N, self.H, self.d = x["q"].shape
        self.code = 0 if dtype == "bf16" else 1
        self.S = int(lh.lh_subseq_len(self.N, p, L, K))
        self.Sp = (self.S + 63) // 64 * 64
        say(f"  GPU run {label}: N={self.N} H={self.H} d={self.d} {dtype} p={p} L={L} K={K} "
            f"S={self.S} backward={backward} mode={mode} score_mode={score_mode}")
        self.q, self.k, self.v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
        self.o, self.ws = lh.forward(self.q, self.k, self.v, p, L, K, score_mode=score_mode)
        if backward:
            self.dout = to_dev(x["dout"], dtype)
            self.grads = lh.backward(self.dout, p, L, K, self.ws, mode=mode)
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
    g = run.scores()
    for l in range(run.L):
        a = np.ascontiguousarray(g[l]).view(np.uint32)
        b = np.ascontiguousarray(ref["levels"][l]).view(np.uint32)
        bad = int(np.sum(a != b))
        assert bad == 0, f"level {l}: {bad} scores differ bitwise from the oracle"


def slot_index(start_h: np.ndarray, level_h: np.ndarray, p: int) -> np.ndarray:
    """Token -> slot map of one head (each kept entry covers p^level tokens)."""
    return np.repeat(np.arange(start_h.size), p ** level_h.astype(np.int64))


def check_full_rows(got_dev: torch.Tensor, ref_sub: np.ndarray, sel, p, dtype, what, divide=False,
                    sample=None, rng=None, cond_sub=None):
    """got [N, H, d] vs ref_sub[h][slot(t)] (optionally / p^level) for every token, or a sample."""
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
    cond = None if cond_sub is None else np.empty((t.size, d))
    for hh in range(H):
        msk = h == hh
        slot = np.searchsorted(st[hh], t[msk], side="right") - 1
        div = (p ** lv[hh][slot].astype(np.int64))[:, None] if divide else 1.0
        ref[msk] = ref_sub[hh][slot] / div
        if cond is not None:
            cond[msk] = cond_sub[hh][slot] / div
    label = what if sample is None else what + f" ({sample} sampled rows)"
    return compare(got, ref, dtype, label, cond=cond, d=d)
