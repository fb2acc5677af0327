"""GPU checks of the descriptor read-out, the achievable-peak probes, concurrent
layers on two streams and the backward's optional sub-sequence gradients, called
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def test_read_selection_matches_oracle_and_view():
    import hierarchical_selection_attention_amd as lh
    N, H, d, p, L, K = 4096, 4, 128, 4, 4, 8
    say(f"case read_selection N={N} H={H} d={d} p={p} L={L} K={K}")
    x = si.make_inputs(N, H, d, "bf16", seed=71, with_dout=False, threads=8)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    _, ws = lh.forward(q, k, v, p, L, K)
    start, level = lh.read_selection(ws, N, H, d, p, L, K, 0)
    torch.cuda.synchronize()
    ref = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", want=("sel",))
    assert np.array_equal(start.cpu().numpy(), ref["start"])
    assert np.array_equal(level.cpu().numpy(), ref["level"])
    assert torch.equal(start, lh.workspace_tensor(ws, N, H, d, p, L, K, 0, "sel_start"))


def test_peak_probes_move_the_right_bytes():
    import hierarchical_selection_attention_amd as lh
    rng = np.random.default_rng(72)
    n = (3 << 20) + 4096                         # three full 1 MiB chunks and a ragged one
    say(f"case peak probes n={n}")
    host = rng.integers(0, 2 ** 32, size=n // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    # read: XOR fold of the 16-byte words of each 1 MiB chunk into that chunk's 16 bytes of dst
    nchunk = (n + (1 << 20) - 1) >> 20
    acc = torch.zeros(4 * nchunk, dtype=torch.int32, device="cuda")
    lh.peak_probe(0, src, acc, n)
    torch.cuda.synchronize()
    words = host.reshape(-1, 4)
    want = np.stack([np.bitwise_xor.reduce(words[c * 65536:(c + 1) * 65536], axis=0) for c in range(nchunk)])
    assert np.array_equal(acc.cpu().numpy().view(np.uint32).reshape(nchunk, 4), want)
    # copy
    dst = torch.zeros_like(src)
    lh.peak_probe(2, src, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    # write: word w holds {1.0f bits, its 256 KiB chunk, thread = w % 256, 0}
    out = torch.zeros_like(src)
    lh.peak_probe(1, None, out, n)
    torch.cuda.synchronize()
    words = out.cpu().numpy().view(np.uint32).reshape(-1, 4)
    idx = np.arange(words.shape[0])
    assert np.all(words[:, 0] == 0x3F800000)
    assert np.array_equal(words[:, 1], (idx // 16384).astype(np.uint32))
    assert np.array_equal(words[:, 2], (idx % 256).astype(np.uint32))
    assert np.all(words[:, 3] == 0)
    # token-row write pattern: the word of token t, head h, chunk c holds
    # {1.0f bits, workgroup 16 (t / 16384) + h, thread 16 (t % 16) + c, 0}
    nt = 128 << 20
    tokw = torch.zeros(nt // 4, dtype=torch.int32, device="cuda")
    lh.peak_probe(5, None, tokw, nt)
    torch.cuda.synchronize()
    words = tokw.cpu().numpy().view(np.uint32).reshape(-1, 16, 16, 4)   # [token][head][chunk]
    t = np.arange(words.shape[0])[:, None, None]
    h = np.arange(16)[None, :, None]
    c = np.arange(16)[None, None, :]
    assert np.all(words[..., 0] == 0x3F800000)
    assert np.array_equal(words[..., 1], np.broadcast_to(16 * (t // 16384) + h, words.shape[:3]).astype(np.uint32))
    assert np.array_equal(words[..., 2], np.broadcast_to(16 * (t % 16) + c, words.shape[:3]).astype(np.uint32))
    assert np.all(words[..., 3] == 0)
    # MFMA loop: every workgroup runs the same operands, so all 1024 checksums agree
    chk = torch.zeros((1024, 4), dtype=torch.int32, device="cuda")
    lh.peak_probe(3, None, chk, 16)
    torch.cuda.synchronize()
    assert torch.equal(chk, chk[:1].expand_as(chk))


def test_concurrent_layers_on_two_user_streams():
    """Two independent forward + backward passes, enqueued interleaved on two
    caller streams with two workspaces: each matches the oracle.  The library
    keeps no per-device stream or event state; every call runs on its own
    stream and reads and writes only its own workspace."""
    import hierarchical_selection_attention_amd as lh
    from gpu_util import check_full_rows, grad_allow
    cases = [(4096, 4, 128, 4, 4, 8, 81), (2048, 8, 128, 4, 3, 5, 82)]
    say("case two user streams: " + ", ".join(f"N={c[0]} H={c[1]}" for c in cases))
    runs = []
    for N, H, d, p, L, K, seed in cases:
        x = si.make_inputs(N, H, d, "bf16", seed=seed, with_dout=True, threads=8)
        t = {n: to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout")}
        ws = lh.alloc_workspace(N, H, d, p, L, K, 0)
        o = torch.empty_like(t["q"])
        g = tuple(torch.empty_like(t["q"]) for _ in range(3))
        runs.append((x, t, ws, o, g, (N, H, d, p, L, K)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]          # default priority
    for (x, t, ws, o, g, (N, H, d, p, L, K)), s in zip(runs, streams):
        lh.forward(t["q"], t["k"], t["v"], p, L, K, ws=ws, out=o, stream=s)
    for (x, t, ws, o, g, (N, H, d, p, L, K)), s in zip(runs, streams):
        lh.backward(t["dout"], p, L, K, ws, grads=g, stream=s)
    torch.cuda.synchronize()
    for x, t, ws, o, g, (N, H, d, p, L, K) in runs:
        ref = oracle.forward(x["q"], x["k"], x["v"], p, L, K, "bf16", want=("sel", "ot"))
        b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (ref["start"], ref["level"]), "bf16",
                            want=("sub", "cond"))
        sel = (ref["start"], ref["level"])
        check_full_rows(o, ref["Ot"], sel, p, "bf16", f"two streams o (N={N})")
        for gg, key in zip(g, ("dQt", "dKt", "dVt")):
            check_full_rows(gg, b[key], sel, p, "bf16", f"two streams d{key[1].lower()} (N={N})", divide=True,
                            allow_sub=grad_allow(b, key))


def test_backward_without_sub_gradients_writes_the_same_tokens():
    """The default backward stores no fp32 dQ~, dK~, dV~ rows on the bf16 partition path
    (LH_BWD_KEEP_SUB asks for them): its dq, dk, dv token rows equal, bit for bit, those of
    a backward that stores them, and the views it does not write keep their contents."""
    import hierarchical_selection_attention_amd as lh
    N, H, d, p, L, K = 8192, 4, 128, 4, 4, 16
    say(f"case backward keep-sub N={N} H={H} d={d} p={p} L={L} K={K}")
    x = si.make_inputs(N, H, d, "bf16", seed=910, with_dout=True, threads=8)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "dout"))
    o, ws = lh.forward(q, k, v, p, L, K)
    for mode in (lh.LH_SCATTER_FP_ATOMIC, lh.LH_SCATTER_DETERMINISTIC):
        kept = [g.clone() for g in lh.backward(do, p, L, K, ws, mode=mode, keep_sub_grads=True)]
        subs = [lh.workspace_tensor(ws, N, H, d, p, L, K, 0, n) for n in ("dqsub", "dksub", "dvsub")]
        for t in subs:
            t.fill_(1234.5)
        plain = lh.backward(do, p, L, K, ws, mode=mode)
        torch.cuda.synchronize()
        for a, b, name in zip(kept, plain, ("dq", "dk", "dv")):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs (mode {mode})"
        for t, name in zip(subs, ("dqsub", "dksub", "dvsub")):
            assert bool((t == 1234.5).all()), f"{name} was written without LH_BWD_KEEP_SUB"

