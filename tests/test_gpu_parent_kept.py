"""GPU parity of the "parent kept" selection (lh_forward_sel / lh_backward_sel
with LH_SELECT_PARENT_KEPT: the overlapping reading of Fig. 2 step 3 on the
Lighthouse paper's page, outputs of overlapping entries summed) against the
oracle: the kept entries bit for bit, o, dq, dk, dv at the bf16 tolerance, and
both scatter modes giving the same bits."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import compare, lib, say, to_dev, to_f64

pytestmark = pytest.mark.gpu
PK = 1

# (label, N, H, d, p, L, K, planted)
CASES = [("bf16_d128", 4096, 4, 128, 4, 4, 8, 0.0),
         ("bf16_d64_h3_p3_ragged", 1080, 3, 64, 3, 4, 5, 0.0),
         ("bf16_pool_up", 8192, 2, 128, 4, 6, 4, 0.0),
         ("bf16_k0", 2048, 2, 128, 4, 3, 0, 0.0),
         ("bf16_kall", 1024, 2, 128, 4, 3, 256, 0.0),
         ("llama530m_attn_n98304", 98304, 16, 128, 4, 4, 128, 0.01)]


def _token_sum(sub, start, level, p, N, divide):
    """[N, H, d]: for every token, the sum over the kept entries covering it of sub[h][slot]
    (divided by p^level when `divide`)."""
    H, S, d = sub.shape
    out = np.zeros((N, H, d))
    for h in range(H):
        lens = p ** level[h].astype(np.int64)
        tok = np.concatenate([np.arange(a, a + n) for a, n in zip(start[h].tolist(), lens.tolist())])
        slot = np.repeat(np.arange(S), lens)
        rows = sub[h][slot] / (lens[slot][:, None] if divide else 1.0)
        np.add.at(out[:, h], tok, rows)
    return out


def _check(got, ref, allow, what, rows=None):
    """allow: None, or the (C, C_L) sums summed over the covering entries like the output."""
    if rows is not None:
        got, ref = got[rows], ref[rows]
        allow = None if allow is None else tuple(a[rows] for a in allow)
    d = ref.shape[-1]
    compare(got.reshape(-1, d), ref.reshape(-1, d), "bf16", what,
            allow=None if allow is None else tuple(a.reshape(-1, d) for a in allow), stored="bf16")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_parent_kept_parity(case):
    lh = lib()
    label, N, H, d, p, L, K, planted = case
    seed = 1300 + CASES.index(case)
    say(f"case {label} parent kept seed={seed}")
    x = si.make_inputs(N, H, d, "bf16", seed=seed, planted=planted, with_dout=True, threads=8)
    ref = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", want=("sel", "o"), select_mode=PK)
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (ref["start"], ref["level"]), "bf16",
                        want=("full", "cond"), select_mode=PK)
    say(f"  oracle done, S={ref['S']}")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    o, ws = lh.forward(q, k, v, p, L, K, select_mode=PK)
    grads = lh.backward(do, p, L, K, ws, select_mode=PK)
    torch.cuda.synchronize()
    say("  GPU done")
    st, lv = lh.read_selection(ws, N, H, d, p, L, K, 0, select_mode=PK)
    assert np.array_equal(st.cpu().numpy(), ref["start"]), "kept starts differ from the oracle"
    assert np.array_equal(lv.cpu().numpy().astype(np.int8), ref["level"]), "kept levels differ from the oracle"
    rows = None
    if N * H > 65536:
        rows = np.random.default_rng(seed).choice(N, size=4096, replace=False)
    sel = (ref["start"], ref["level"])
    _check(to_f64(o), ref["O"], None, "o", rows)
    for g, name, X in zip(grads, ("dq", "dk", "dv"), "QKV"):
        allow = (_token_sum(b["cd" + X], *sel, p, N, True), _token_sum(b["ld" + X], *sel, p, N, True))
        _check(to_f64(g), b[name], allow, name, rows)


def test_parent_kept_scatter_modes_give_identical_bits():
    lh = lib()
    N, H, d, p, L, K = 4096, 4, 128, 4, 4, 8
    x = si.make_inputs(N, H, d, "bf16", seed=1399, with_dout=True, threads=8)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    res = []
    for mode in (0, 1, 0):
        o, ws = lh.forward(q, k, v, p, L, K, select_mode=PK)
        g = lh.backward(do, p, L, K, ws, mode=mode, select_mode=PK)
        res.append([t.clone() for t in (o, *g)])
    torch.cuda.synchronize()
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
    for a, b in zip(res[0], res[2]):
        assert torch.equal(a, b)


def _sampled_token_sum(sub, start, level, p, t, h, divide):
    """Rows [len(t), d]: for token t[i] of head h[i], the sum over the kept entries covering
    it of sub[h][slot] (divided by p^level when `divide`)."""
    H, S, d = sub.shape
    out = np.zeros((t.size, d))
    for hh in range(H):
        msk = h == hh
        tt = t[msk]
        lens = p ** level[hh].astype(np.int64)
        st = start[hh].astype(np.int64)
        acc = np.zeros((tt.size, d))
        # the entries covering a token: at most one per level
        for l in np.unique(level[hh]):
            sl = np.nonzero(level[hh] == l)[0]                    # slots of level l, starts ascending
            i = np.searchsorted(st[sl], tt, side="right") - 1
            ok = (i >= 0) & (tt < st[sl][np.maximum(i, 0)] + p ** int(l))
            rows = sub[hh][sl[np.maximum(i, 0)]] / (p ** int(l) if divide else 1.0)
            acc += np.where(ok[:, None], rows, 0.0)
        out[msk] = acc
    return out


def _gpu_token_sums(sub_dev, start, level, p, N, divide):
    """[N, H, d] fp32 sums, in the kernel's order (finest level first, each row times
    p^-level for the pool adjoint), of the GPU's own fp32 entry rows."""
    H = start.shape[0]
    d = sub_dev.shape[-1]
    out = torch.zeros((N, H, d), dtype=torch.float32, device="cuda")
    for h in range(H):
        lv = torch.from_numpy(level[h].astype(np.int64)).cuda()
        st = torch.from_numpy(start[h].astype(np.int64)).cuda()
        for l in range(int(level[h].max()) + 1):
            sl = torch.nonzero(lv == l).flatten()
            if sl.numel() == 0:
                continue
            n = p ** l
            tok = (st[sl][:, None] + torch.arange(n, device="cuda")[None, :]).flatten()
            rows = sub_dev[h][sl]
            if divide:
                rows = rows * np.float32(1.0 / n)
            out[tok, h] = out[tok, h] + rows.repeat_interleave(n, dim=0)
    return out


@pytest.mark.timeout(900)
def test_parent_kept_at_512k_as_benched():
    """The 512K workload with the parent-kept reading, as bench.py --select parent_kept times
    it: kept entries bit for bit; O~, dQ~, dK~, dV~ on every row; 200k sampled token rows of
    o, dq, dk, dv against the oracle; and, over all tokens, every token row equal bit for bit
    to the fp32 sum (finest level first) of its covering entries' rows, rounded once."""
    lh = lib()
    w = si.WORKLOADS[4]
    N, H, d, p, L, K = w["N"], w["H"], w["d"], w["p"], w["L"], w["K"]
    say(f"case parent kept 512K: N={N} H={H} d={d} p={p} L={L} K={K}")
    x = si.workload_inputs(4, with_dout=True, threads=16)
    say("  oracle ...")
    ref = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", want=("sel", "ot"), select_mode=PK)
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (ref["start"], ref["level"]), "bf16",
                        want=("sub", "cond"), select_mode=PK)
    S = ref["S"]
    say(f"  oracle done, S={S}")
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    o, ws = lh.forward(q, k, v, p, L, K, select_mode=PK)
    grads = lh.backward(do, p, L, K, ws, select_mode=PK)
    torch.cuda.synchronize()
    st, lv = lh.read_selection(ws, N, H, d, p, L, K, 0, select_mode=PK)
    st, lv = st.cpu().numpy(), lv.cpu().numpy().astype(np.int8)
    assert np.array_equal(st, ref["start"]) and np.array_equal(lv, ref["level"]), "kept entries differ"
    view = lambda name: lh.workspace_tensor(ws, N, H, d, p, L, K, 0, name, select_mode=PK)[:, :S]
    compare(to_f64(view("osub")), ref["Ot"], "bf16", "parent kept 512K osub")
    for name, key in (("dqsub", "dQt"), ("dksub", "dKt"), ("dvsub", "dVt")):
        compare(to_f64(view(name)), b[key], "bf16", "parent kept 512K " + name, allow=(b["cd" + key[1]], b["ld" + key[1]]))
    rng = np.random.default_rng(44)
    t = rng.integers(0, N, size=200_000)
    h = rng.integers(0, H, size=200_000)
    ti, hi = torch.from_numpy(t).cuda(), torch.from_numpy(h).cuda()
    compare(to_f64(o[ti, hi]), _sampled_token_sum(ref["Ot"], st, lv, p, t, h, False), "bf16",
            "parent kept 512K o (200000 sampled rows)", stored="bf16")
    for g, key in zip(grads, ("dQt", "dKt", "dVt")):
        X = key[1]
        allow = (_sampled_token_sum(b["cd" + X], st, lv, p, t, h, True),
                 _sampled_token_sum(b["ld" + X], st, lv, p, t, h, True))
        compare(to_f64(g[ti, hi]), _sampled_token_sum(b[key], st, lv, p, t, h, True), "bf16",
                f"parent kept 512K d{X.lower()} (200000 sampled rows)", allow=allow, stored="bf16")
    # every token: the summed copies reproduce the GPU's own entry rows bit for bit
    for got, name, div in ((o, "osub", False), (grads[0], "dqsub", True), (grads[1], "dksub", True),
                           (grads[2], "dvsub", True)):
        want = _gpu_token_sums(view(name), st, lv, p, N, div).to(torch.bfloat16)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{name}: token sums differ"
    say("  every token row equals its covering entries' sum")
