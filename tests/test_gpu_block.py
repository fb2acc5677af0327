"""GPU parity of the attention block (projections around the layer, Sec. 3.1
Eq. (1) and Fig. 1 of the Lighthouse paper) against the block oracle, through
the C ABI (lh_block_forward / lh_block_backward).

The block inputs sit on fixed-point grids on which the projections are exact in
fp32, so q, k, v and dO must match the oracle bit for bit, and with them the
selection; y, dx and the weight gradients are compared at the bf16 tolerances.

Both sides round the layer's outputs o, dq, dk, dv to bf16, from values that
agree to about 1e-6 but not exactly, so now and then one element rounds to the
neighbouring bf16 value (one ulp = 2^-8 relative).  A product with such an
operand can move by up to 2^-8 times its sum of absolute terms C, which
exceeds the plain tolerance where the sum cancels (dW sums over all tokens,
and a coarse entry repeats its gradient on up to p^l tokens).  Elements beyond
the plain tolerance are therefore also accepted within 2^-8 C; the number of
such elements is reported.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import compare, lib, say, to_f64

pytestmark = pytest.mark.gpu
ULP = 2.0 ** -8     # one bf16 ulp, relative


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _block_qkv(ws, N, H, d, p, L, K):
    lh = lib()
    off = (lh.lh_workspace_bytes(N, H, d, p, L, K, 0) + 255) // 256 * 256
    n = 3 * N * H * d
    return ws[off: off + 2 * n].view(torch.bfloat16).view(N, 3, H, d).transpose(0, 1)


def _block_dout(ws, N, H, d, p, L, K):
    lh = lib()
    off = (lh.lh_workspace_bytes(N, H, d, p, L, K, 0) + 255) // 256 * 256
    off = (off + 2 * 3 * N * H * d + 255) // 256 * 256
    return ws[off: off + 2 * N * H * d].view(torch.bfloat16).view(N, H, d)


def _run_block(b, N, dm, H, d, p, L, K, mode, rows, cols_qkv, cols_o, label):
    lh = lib()
    say(f"  block {label}: N={N} dm={dm} H={H} d={d} p={p} L={L} K={K} mode={mode}")
    x, wqkv, wo, dy = _dev(b["x"]), _dev(b["w_qkv"]), _dev(b["w_o"]), _dev(b["dy"])
    y, o, ws = lh.block_forward(x, wqkv, wo, H, d, p, L, K)
    qkv = _block_qkv(ws, N, H, d, p, L, K).float().cpu().numpy()    # the backward reuses this region
    dx, dwqkv, dwo = lh.block_backward(x, wqkv, wo, o, dy, H, d, p, L, K, ws, mode=mode)
    torch.cuda.synchronize()
    say("  GPU block done; oracle ...")
    f = oracle.block_forward(b["x"], b["w_qkv"], b["w_o"], H, d, p, L, K, rows=rows, cond=True)
    g = oracle.block_backward(f, b["x"], b["w_qkv"], b["w_o"], b["dy"], H, d, p, L, K, rows=rows,
                              cols_qkv=cols_qkv, cols_o=cols_o, cond=True)
    say("  oracle done")
    bad = int(np.sum(qkv != f["qkv"]))
    assert bad == 0, f"{bad} projected q/k/v values differ from the oracle's bf16 rounding"
    bad = int(np.sum(_block_dout(ws, N, H, d, p, L, K).float().cpu().numpy() != g["dO"]))
    assert bad == 0, f"{bad} values of dO = dy W_O^T differ from the oracle's bf16 rounding"
    st, lv = lh.read_selection(ws, N, H, d, p, L, K, 0)
    assert np.array_equal(st.cpu().numpy(), f["start"]), "selected starts differ from the oracle"
    assert np.array_equal(lv.cpu().numpy().astype(np.int8), f["level"]), "selected levels differ"
    sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
    compare(to_f64(y[sel]), f["y"], "bf16", "y", cond=f["cy"], cond_unit=ULP)
    compare(to_f64(dx[sel]), g["dx"], "bf16", "dx", cond=g["cdx"], cond_unit=ULP)
    cq = slice(None) if cols_qkv is None else torch.from_numpy(cols_qkv).cuda()
    co = slice(None) if cols_o is None else torch.from_numpy(cols_o).cuda()
    compare(to_f64(dwqkv[:, cq]), g["dw_qkv"], "bf16", "dW_QKV", cond=g["cdw_qkv"], cond_unit=ULP)
    compare(to_f64(dwo[:, co]), g["dw_o"], "bf16", "dW_O", cond=g["cdw_o"], cond_unit=ULP)


@pytest.mark.parametrize("mode", [0, 1])
def test_block_small_all_outputs(mode):
    N, dm, H, d, p, L, K = 2048, 128, 2, 64, 4, 3, 16
    b = si.make_block_inputs(N, dm, H, d, seed=77, planted=0.01, with_dy=True)
    _run_block(b, N, dm, H, d, p, L, K, mode, None, None, None, "small")


@pytest.mark.parametrize("dm", [192, 64])
def test_block_non_square_projections(dm):
    """d_model != H*d: every GEMM has distinct M, N and K, so a transposed operand cannot go unseen."""
    N, H, d, p, L, K = 2048, 2, 64, 4, 3, 16
    b = si.make_block_inputs(N, dm, H, d, seed=78 + dm, planted=0.01, with_dy=True)
    _run_block(b, N, dm, H, d, p, L, K, 0, None, None, None, f"dm{dm}")


def test_block_530m_shape_sampled():
    w = si.BLOCK_WORKLOAD
    N, dm, H, d, p, L, K = w["N"], w["dm"], w["H"], w["d"], w["p"], w["L"], w["K"]
    b = si.block_inputs(with_dy=True)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(N, size=384, replace=False))
    cols_qkv = np.sort(rng.choice(3 * H * d, size=48, replace=False))
    cols_o = np.sort(rng.choice(dm, size=32, replace=False))
    _run_block(b, N, dm, H, d, p, L, K, 0, rows, cols_qkv, cols_o, w["name"])
