"""GPU checks of the descriptor read-out and of the achievable-peak probes,
called through the C ABI."""
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
    # MFMA loop: every workgroup runs the same operands, so all 1024 checksums agree
    chk = torch.zeros((1024, 4), dtype=torch.int32, device="cuda")
    lh.peak_probe(3, None, chk, 16)
    torch.cuda.synchronize()
    assert torch.equal(chk, chk[:1].expand_as(chk))
