"""Pins of the oracle's "parent kept" selection (the overlapping reading of
Fig. 2 step 3 on the Lighthouse paper's page: a selected entry stays beside its
children, overlapping outputs are summed), tied to the pinned partition
reading, to its size law, and to torch fp64 autograd of the same layer."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si

PK = 1


def _inputs(N, H, d, dtype, seed, dout=False):
    return si.make_inputs(N, H, d, dtype, seed=seed, with_dout=dout, threads=2)


def _f64(x, dtype):
    return si.to_f32(x, dtype).astype(np.float64)


@pytest.mark.parametrize("N,p,L,K", [(1024, 4, 4, 5), (512, 2, 6, 3), (2048, 4, 3, 16), (256, 4, 4, 0),
                                     (256, 4, 1, 7), (243, 3, 4, 100)])
def test_size_law(N, p, L, K):
    """Every candidate of every level is kept: N/p^(L-1) top entries plus p * min(K, #candidates)
    children per selecting level."""
    n = N // p ** (L - 1)
    S, cand = n, n
    for _ in range(L - 1):
        sel = min(K, cand)
        S += p * sel
        cand = p * sel
    assert oracle.subseq_len(N, p, L, K, PK) == S


@pytest.mark.parametrize("seed,N,p,L,K,dup", [(1, 1024, 4, 4, 5, 0.0), (2, 512, 2, 6, 3, 0.0),
                                              (3, 729, 3, 4, 4, 0.3), (4, 2048, 4, 3, 16, 0.0)])
def test_kept_entries_are_the_partition_closed_under_ancestors(seed, N, p, L, K, dup):
    """Parent kept = the partition's entries plus every ancestor of each of them (the refined
    entries), ordered by first token with the coarser entry first."""
    H, d = 2, 16
    x = _inputs(N, H, d, "bf16", seed)
    part = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16")
    pk = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", select_mode=PK)
    for h in range(H):
        want = set()
        for a, l in zip(part["start"][h].tolist(), part["level"][h].tolist()):
            for m in range(l, L):
                want.add(((a // p ** m) * p ** m, m))
        got = list(zip(pk["start"][h].tolist(), pk["level"][h].tolist()))
        assert set(got) == want and len(got) == len(want)
        assert got == sorted(got, key=lambda e: (e[0], -e[1]))


@pytest.mark.parametrize("N,p,L,K", [(256, 4, 4, 0), (256, 4, 1, 7)])
def test_no_selection_means_no_overlap(N, p, L, K):
    """With K = 0 or a single level nothing is refined, so both readings keep the same entries."""
    x = _inputs(N, 2, 16, "fp32", 7, dout=True)
    a = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "fp32", want=("sel", "o"))
    b = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "fp32", want=("sel", "o"), select_mode=PK)
    assert np.array_equal(a["start"], b["start"]) and np.array_equal(a["level"], b["level"])
    assert np.array_equal(a["O"], b["O"])


def _torch_sdpa(q, k, v):
    o = torch.nn.functional.scaled_dot_product_attention(
        q.permute(1, 0, 2).unsqueeze(0), k.permute(1, 0, 2).unsqueeze(0),
        v.permute(1, 0, 2).unsqueeze(0), is_causal=True)
    return o.squeeze(0).permute(1, 0, 2)


@pytest.mark.parametrize("dtype,seed,N,p,L,K", [("fp32", 41, 512, 4, 4, 3), ("bf16", 42, 243, 3, 4, 2),
                                                ("fp32", 43, 256, 2, 5, 4)])
def test_overlapping_layer_matches_torch_autograd(dtype, seed, N, p, L, K):
    """Given the kept entries, rebuild the layer from torch ops (block means, causal SDPA, and a
    sum of each entry's output into its tokens) and let autograd differentiate it."""
    H, d = 2, 16
    x = _inputs(N, H, d, dtype, seed, dout=True)
    r = oracle.forward(x["q"], x["k"], x["v"], p, L, K, dtype, want=("sel", "o"), select_mode=PK)
    t = {n: torch.tensor(_f64(x[n], dtype), requires_grad=True) for n in ("q", "k", "v")}
    outs = []
    for h in range(H):
        st, lv = r["start"][h].tolist(), r["level"][h].tolist()
        g = [torch.stack([t[n][a:a + p ** l, h].mean(dim=0) for a, l in zip(st, lv)]) for n in ("q", "k", "v")]
        o_sub = _torch_sdpa(*(z.unsqueeze(1) for z in g)).squeeze(1)
        tok = torch.tensor(np.concatenate([np.arange(a, a + p ** l) for a, l in zip(st, lv)]))
        slot = torch.tensor(np.repeat(np.arange(len(st)), [p ** l for l in lv]))
        outs.append(torch.zeros(N, d, dtype=torch.float64).index_add(0, tok, o_sub.index_select(0, slot)))
    o = torch.stack(outs, dim=1)
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    o.backward(torch.tensor(_f64(x["dout"], dtype)))
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (r["start"], r["level"]), dtype,
                        want=("full",), select_mode=PK)
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(b["d" + n], t[n].grad.numpy(), rtol=1e-9, atol=1e-11)
