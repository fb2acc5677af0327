"""GPU parity of the HIP path against the CPU oracle, element by element, on
seeded inputs small enough for the oracle to finish in seconds while spanning
several tiles, ragged tails and the degenerate cases of the method.  All calls
go through the C ABI (liblighthouse.so).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import Run, check_full_rows, check_scores, check_selection, compare, grad_allow, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

# (label, N, H, d, dtype, p, L, K, scale, dup, backward)
CASES = [
    ("tiny_fp32_k16", 2048, 2, 64, "fp32", 4, 3, 16, "lognormal", 0.0, True),
    ("tiny_fp32_kall", 2048, 2, 64, "fp32", 4, 3, 512, "lognormal", 0.0, True),
    ("bf16_d128", 4096, 4, 128, "bf16", 4, 4, 8, "lognormal", 0.0, True),
    ("bf16_d64_h3_p3_ragged", 1080, 3, 64, "bf16", 3, 4, 5, "lognormal", 0.0, True),
    ("bf16_single_level", 512, 2, 128, "bf16", 4, 1, 7, "lognormal", 0.0, True),
    ("bf16_k0", 2048, 2, 128, "bf16", 4, 3, 0, "lognormal", 0.0, True),
    ("bf16_kall", 1024, 2, 128, "bf16", 4, 3, 256, "lognormal", 0.0, True),
    ("bf16_pool_up", 8192, 2, 128, "bf16", 4, 6, 4, "lognormal", 0.0, True),
    ("bf16_chunked_topk", 16384, 2, 64, "bf16", 2, 3, 100, "lognormal", 0.0, True),
    ("bf16_h32_head_groups", 1024, 32, 128, "bf16", 4, 3, 8, "lognormal", 0.0, True),
    ("bf16_p2_deep", 4096, 2, 128, "bf16", 2, 8, 3, "lognormal", 0.0, True),
    ("bf16_ties_heavy_tail", 4096, 2, 128, "bf16", 4, 4, 16, "student_t3", 0.3, True),
    ("fp32_d128", 1024, 2, 128, "fp32", 4, 3, 6, "lognormal", 0.0, True),
    # N = p^(L-1): one top entry, one head
    ("bf16_single_top_h1", 256, 1, 128, "bf16", 4, 5, 2, "lognormal", 0.0, True),
    # a wide pooling factor: p^2 = 64 tokens per top entry
    ("bf16_p8", 4096, 2, 64, "bf16", 8, 3, 3, "lognormal", 0.0, True),
    ("fp32_p8_h1", 512, 1, 64, "fp32", 8, 3, 4, "lognormal", 0.0, True),
    # 8192 top-level candidates: the selection's per-level arrays exceed what it keeps in
    # LDS, so it works on the workspace arrays instead
    ("bf16_topk_arrays_in_memory", 32768, 1, 64, "bf16", 4, 2, 64, "lognormal", 0.0, True),
]


def _inputs(case, seed):
    label, N, H, d, dtype, p, L, K, scale, dup, bwd = case
    return si.make_inputs(N, H, d, dtype, seed=seed, scale=scale, dup=dup, with_dout=bwd, threads=8)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", [0, 1], ids=["fp_atomic", "deterministic"])
def test_parity_small(case, mode):
    label, N, H, d, dtype, p, L, K, scale, dup, bwd = case
    seed = 500 + CASES.index(case)
    say(f"case {label} mode={mode} seed={seed}")
    x = _inputs(case, seed)
    ref = oracle.forward(x["q"], x["k"], x["v"], p, L, K, dtype, want=("levels", "sel", "sub", "ot"))
    run = Run(x, dtype, p, L, K, backward=bwd, mode=mode, label=label)
    check_scores(run, ref)
    check_selection(run, ref)
    for name, key in (("qsub", "Qt"), ("ksub", "Kt"), ("vsub", "Vt")):
        compare(run.sub(name), ref[key], dtype, name)
    lse = run.view("lse").cpu().numpy()[:, : run.S]
    compare(lse, ref["lse"], dtype, "lse")
    dout = x["dout"] if bwd else np.zeros_like(x["q"])
    b = oracle.backward(x["q"], x["k"], x["v"], dout, p, L, K, (ref["start"], ref["level"]), dtype,
                        want=("sub", "full", "cond"))
    compare(run.sub("osub"), ref["Ot"], dtype, "osub")
    sel = (ref["start"], ref["level"])
    check_full_rows(run.o, ref["Ot"], sel, p, dtype, "o")
    if bwd:
        compare(run.sub("dosub"), b["dOt"], dtype, "dosub")
        for name, key in (("dqsub", "dQt"), ("dksub", "dKt"), ("dvsub", "dVt")):
            compare(run.sub(name), b[key], dtype, name, allow=grad_allow(b, key))
        for g, key, sub in zip(run.grads, ("dq", "dk", "dv"), ("dQt", "dKt", "dVt")):
            check_full_rows(g, b[sub], sel, p, dtype, key, divide=True, allow_sub=grad_allow(b, sub))


def test_deterministic_scatter_is_bit_reproducible():
    """Deterministic mode: identical bits over repeated runs (and close to the fp-atomic mode)."""
    case = ("rep", 8192, 4, 128, "bf16", 4, 4, 16, "lognormal", 0.0, True)
    x = _inputs(case, 77)
    say("case deterministic-mode reproducibility N=8192 H=4 d=128 p=4 L=4 K=16")
    runs = [Run(x, "bf16", 4, 4, 16, backward=True, mode=1, label=f"rep{i}") for i in range(5)]
    ref = [g.view(torch.int16).cpu() for g in runs[0].grads]
    dos = runs[0].view("dosub").cpu()
    for r in runs[1:]:
        assert torch.equal(r.view("dosub").cpu(), dos)
        for g, g0 in zip(r.grads, ref):
            assert torch.equal(g.view(torch.int16).cpu(), g0)
    fp = Run(x, "bf16", 4, 4, 16, backward=True, mode=0, label="fp")
    compare(to_f64(fp.view("dosub")), to_f64(runs[0].view("dosub")), "bf16", "fp vs int dosub")
    for g, g0 in zip(fp.grads, runs[0].grads):
        compare(to_f64(g), to_f64(g0), "bf16", "fp vs int grads")


@pytest.mark.parametrize("N,H,d", [(1024, 2, 128), (512, 3, 64)])
def test_dense_attention_matches_oracle(N, H, d):
    """The comparison kernel (same MFMA kernels at full length) is plain causal attention:
    the oracle with a single level."""
    import hierarchical_selection_attention_amd as lh
    x = si.make_inputs(N, H, d, "bf16", seed=900 + d, with_dout=True, threads=8)
    say(f"case dense N={N} H={H} d={d}")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    o, lse, ws = lh.dense_forward(q, k, v)
    dq, dk, dv = lh.dense_backward(q, k, v, o, lse, do, ws)
    torch.cuda.synchronize()
    ref = oracle.forward(x["q"], x["k"], x["v"], 4, 1, 0, "bf16", want=("sel", "o", "ot"))
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], 4, 1, 0, (ref["start"], ref["level"]), "bf16",
                        want=("full", "cond"))
    # with a single level the sub-sequence is the token sequence: [H, N, d] -> [N, H, d]
    tr = lambda z: np.ascontiguousarray(z.transpose(1, 0, 2))
    compare(to_f64(o), ref["O"], "bf16", "dense o")
    compare(lse.cpu().numpy(), ref["lse"], "bf16", "dense lse")
    for g, key, sub in zip((dq, dk, dv), ("dq", "dk", "dv"), ("dQt", "dKt", "dVt")):
        compare(to_f64(g), b[key], "bf16", "dense " + key, allow=tuple(tr(a) for a in grad_allow(b, sub)),
                stored="bf16")


def test_workspace_is_reusable_across_shapes():
    """A workspace sized for a larger call serves a smaller one; outputs do not depend on
    what an earlier call left in it."""
    import hierarchical_selection_attention_amd as lh
    big = si.make_inputs(4096, 4, 128, "bf16", seed=61, with_dout=True, threads=8)
    small = si.make_inputs(1024, 4, 128, "bf16", seed=62, with_dout=True, threads=8)
    say("case workspace reuse")
    nb = lh.lh_workspace_bytes(4096, 4, 128, 4, 4, 8, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    qb, kb, vb = (to_dev(big[n], "bf16") for n in ("q", "k", "v"))
    lh.forward(qb, kb, vb, 4, 4, 8, ws=ws)
    qs, ks, vs = (to_dev(small[n], "bf16") for n in ("q", "k", "v"))
    o1, _ = lh.forward(qs, ks, vs, 4, 3, 5, ws=ws)
    o2, _ = lh.forward(qs, ks, vs, 4, 3, 5)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# shapes whose top entries span several pooling blocks (p^(L-1) > 256 tokens), so the
# deterministic mode combines per-block partial sums; one fp32 case
SCALE_CASES = [("bf16_pool_up", 8192, 2, 128, "bf16", 4, 6, 4),
               ("bf16_p2_deep", 4096, 2, 64, "bf16", 2, 10, 3),
               ("fp32_pool_up", 4096, 1, 64, "fp32", 4, 6, 3)]


@pytest.mark.parametrize("case", SCALE_CASES, ids=[c[0] for c in SCALE_CASES])
@pytest.mark.parametrize("k", [-20, 20])
def test_deterministic_scatter_over_the_fp32_range(case, k):
    """dO scaled by 2^k.  Every scale in the gradient path is a power of two, so
    the deterministic mode's gradients are those of the unscaled dO times 2^k,
    bit for bit.  Times 2^-k they match the oracle's gradients of the unscaled
    dO at the dtype's bound, and the fp-atomic mode's at the same bound."""
    import hierarchical_selection_attention_amd as lh
    label, N, H, d, dtype, p, L, K = case
    seed = 600 + SCALE_CASES.index(case)
    say(f"case {label} dO x 2^{k} seed={seed}")
    x = si.make_inputs(N, H, d, dtype, seed=seed, scale="student_t3", with_dout=True, threads=8)
    f = 2.0 ** k
    do_s = x["dout"]
    if dtype == "bf16":
        do_s = si.bf16_bits(si.bf16_to_f32(x["dout"]) * np.float32(f))
        assert np.array_equal(si.bf16_to_f32(do_s), si.bf16_to_f32(x["dout"]) * np.float32(f))
    else:
        do_s = (x["dout"] * np.float32(f)).astype(np.float32)
    q, k_, v, do0, do1 = (to_dev(a, dtype) for a in (x["q"], x["k"], x["v"], x["dout"], do_s))
    o, ws = lh.forward(q, k_, v, p, L, K)
    g0 = [t.clone() for t in lh.backward(do0, p, L, K, ws, mode=lh.LH_SCATTER_DETERMINISTIC)]
    g1 = [t.clone() for t in lh.backward(do1, p, L, K, ws, mode=lh.LH_SCATTER_DETERMINISTIC)]
    gf = [t.clone() for t in lh.backward(do1, p, L, K, ws, mode=lh.LH_SCATTER_FP_ATOMIC)]
    torch.cuda.synchronize()
    for a, b, name in zip(g0, g1, ("dq", "dk", "dv")):
        want = (a.double() * f).to(a.dtype)
        assert torch.equal(b, want), f"{name}: gradients of 2^{k} dO are not 2^{k} times those of dO"
    ref = oracle.forward(x["q"], x["k"], x["v"], p, L, K, dtype, want=("sel",))
    bw = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (ref["start"], ref["level"]), dtype,
                         want=("sub", "cond"))
    sel = (ref["start"], ref["level"])
    for gg, key in zip(g1, ("dQt", "dKt", "dVt")):
        back = (gg.double() / f).to(gg.dtype)
        check_full_rows(back, bw[key], sel, p, dtype, f"d{key[1].lower()} (dO x 2^{k}, deterministic)", divide=True,
                        allow_sub=grad_allow(bw, key))
    for a, b, name in zip(gf, g1, ("dq", "dk", "dv")):
        compare(to_f64(a) / f, to_f64(b) / f, dtype, f"{name} fp-atomic vs deterministic (dO x 2^{k})",
                stored=dtype)
