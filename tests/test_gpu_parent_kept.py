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
