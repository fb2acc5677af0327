"""GPU parity of the attention block through the C ABI (lh_block_forward /
lh_block_backward).  The block is the projections around the layer: Sec. 3.1
Eq. (1) and Fig. 1 of the Lighthouse paper.

Each stage is checked against its own definition, on the GPU's own inputs to
that stage:
  * the six GEMMs: q k v = x W_QKV, y = o W_O, dO = dy W_O^T,
    dx = [dq dk dv] W_QKV^T, dW_QKV = x^T [dq dk dv] and dW_O = o^T dy.
    Each is compared with the fp64 product of the exact values of the bf16
    operands the GPU used (including its own o, dO and dq, dk, dv).  The bound
    is fp32 accumulation plus one rounding of the output (compare_product);
  * the layer.  The layer oracle runs on the GPU's q, k, v and dO.  The
    selection must match bit for bit, o must meet the plain bf16 bound, and
    dq, dk, dv the bound with the gradient allowance (gpu_util).
On the fixed-point grid inputs, x W_QKV and dy W_O^T are exact in fp32 in any
order.  There, q, k, v and dO must also equal the block oracle's bf16
roundings bit for bit.  The non-grid inputs (plain bf16 roundings of the same
distributions) exercise the GEMMs' ordinary rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_util import check_full_rows, compare, compare_product, grad_allow, lib, say, to_f64

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _region(ws, N, H, d, p, L, K):
    """[N, 3, H, d] bf16 region after the layer's workspace: q, k, v after the forward,
    dq, dk, dv after the backward."""
    lh = lib()
    off = (lh.lh_workspace_bytes(N, H, d, p, L, K, 0) + 255) // 256 * 256
    n = 3 * N * H * d
    return ws[off: off + 2 * n].view(torch.bfloat16).view(N, 3, H, d)


def _block_dout(ws, N, H, d, p, L, K):
    lh = lib()
    off = (lh.lh_workspace_bytes(N, H, d, p, L, K, 0) + 255) // 256 * 256
    off = (off + 2 * 3 * N * H * d + 255) // 256 * 256
    return ws[off: off + 2 * N * H * d].view(torch.bfloat16).view(N, H, d)


def _bits(t):
    return np.ascontiguousarray(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def _run_block(b, N, dm, H, d, p, L, K, mode, rows, cols_qkv, cols_o, label, grid):
    lh = lib()
    say(f"  block {label}: N={N} dm={dm} H={H} d={d} p={p} L={L} K={K} mode={mode} grid={grid}")
    x, wqkv, wo, dy = _dev(b["x"]), _dev(b["w_qkv"]), _dev(b["w_o"]), _dev(b["dy"])
    y, o, ws = lh.block_forward(x, wqkv, wo, H, d, p, L, K)
    qkv = _bits(_region(ws, N, H, d, p, L, K))                        # [N, 3, H, d] bf16 bits
    dx, dwqkv, dwo = lh.block_backward(x, wqkv, wo, o, dy, H, d, p, L, K, ws, mode=mode)
    torch.cuda.synchronize()
    G = _bits(_region(ws, N, H, d, p, L, K))                          # dq, dk, dv
    dO = _bits(_block_dout(ws, N, H, d, p, L, K))
    o_b = _bits(o)
    say("  GPU block done")
    X, Wq, Wo, dY = (si.bf16_to_f32(b[n]).astype(np.float64) for n in ("x", "w_qkv", "w_o", "dy"))
    hd = H * d
    r = slice(None) if rows is None else rows
    cq = slice(None) if cols_qkv is None else cols_qkv
    co = slice(None) if cols_o is None else cols_o
    f64 = lambda bits: si.bf16_to_f32(bits).astype(np.float64)
    Q3, Gm, Om, dOm = f64(qkv).reshape(N, 3 * hd), f64(G).reshape(N, 3 * hd), f64(o_b).reshape(N, hd), \
        f64(dO).reshape(N, hd)
    # the six GEMMs on the GPU's own operands
    compare_product(Q3[r], X[r], Wq, "block GEMM qkv = x W_QKV", "bf16")
    compare_product(to_f64(y)[r], Om[r], Wo, "block GEMM y = o W_O", "bf16")
    compare_product(dOm[r], dY[r], Wo.T, "block GEMM dO = dy W_O^T", "bf16")
    compare_product(to_f64(dx)[r], Gm[r], Wq.T, "block GEMM dx = G W_QKV^T", "bf16")
    compare_product(to_f64(dwqkv)[:, cq], X.T, Gm[:, cq], "block GEMM dW_QKV = x^T G", "fp32")
    compare_product(to_f64(dwo)[:, co], Om.T, dY[:, co], "block GEMM dW_O = o^T dy", "fp32")
    # the layer on the GPU's own q, k, v and dO
    q, k, v = (np.ascontiguousarray(qkv[:, j]) for j in range(3))
    say("  layer oracle ...")
    ref = oracle.forward(q, k, v, p, L, K, "bf16", want=("sel", "ot"))
    bw = oracle.backward(q, k, v, dO, p, L, K, (ref["start"], ref["level"]), "bf16", want=("sub", "cond"))
    st, lv = lh.read_selection(ws, N, H, d, p, L, K, 0)
    assert np.array_equal(st.cpu().numpy(), ref["start"]), "selected starts differ from the oracle"
    assert np.array_equal(lv.cpu().numpy().astype(np.int8), ref["level"]), "selected levels differ"
    sel = (ref["start"], ref["level"])
    sample = None if rows is None else 4 * len(rows)
    rng = np.random.default_rng(N + dm)
    check_full_rows(o, ref["Ot"], sel, p, "bf16", "block layer o", sample=sample, rng=rng)
    Gd = _region(ws, N, H, d, p, L, K)
    for j, key in enumerate(("dQt", "dKt", "dVt")):
        check_full_rows(Gd[:, j], bw[key], sel, p, "bf16", "block layer d" + key[1].lower(), divide=True,
                        sample=sample, rng=rng, allow_sub=grad_allow(bw, key))
    if grid:
        # exact products on the grids: the layer's inputs are the block oracle's roundings bit for bit
        f = oracle.block_forward(b["x"], b["w_qkv"], b["w_o"], H, d, p, L, K, rows=rows)
        g = oracle.block_backward(f, b["x"], b["w_qkv"], b["w_o"], b["dy"], H, d, p, L, K, rows=rows,
                                  cols_qkv=cols_qkv, cols_o=cols_o)
        got_qkv = si.bf16_to_f32(qkv).reshape(N, 3, H, d).transpose(1, 0, 2, 3)
        assert int(np.sum(got_qkv != f["qkv"])) == 0, "projected q/k/v differ from the block oracle's bf16 rounding"
        assert int(np.sum(si.bf16_to_f32(dO) != g["dO"])) == 0, "dO = dy W_O^T differs from the oracle's rounding"
        assert np.array_equal(ref["start"], f["start"]) and np.array_equal(ref["level"], f["level"])
        compare(to_f64(y)[r], f["y"], "bf16", "block y vs block oracle")


@pytest.mark.parametrize("grid", [True, False], ids=["grid", "plain"])
@pytest.mark.parametrize("mode", [0, 1])
def test_block_small_all_outputs(mode, grid):
    N, dm, H, d, p, L, K = 2048, 128, 2, 64, 4, 3, 16
    b = si.make_block_inputs(N, dm, H, d, seed=77, planted=0.01, with_dy=True, grid=grid)
    _run_block(b, N, dm, H, d, p, L, K, mode, None, None, None, "small", grid)


@pytest.mark.parametrize("dm", [192, 64])
def test_block_non_square_projections(dm):
    """d_model != H*d: every GEMM has distinct M, N and K, so a transposed operand cannot go unseen."""
    N, H, d, p, L, K = 2048, 2, 64, 4, 3, 16
    b = si.make_block_inputs(N, dm, H, d, seed=78 + dm, planted=0.01, with_dy=True, grid=False)
    _run_block(b, N, dm, H, d, p, L, K, 0, None, None, None, f"dm{dm}", False)


@pytest.mark.parametrize("grid", [True, False], ids=["grid", "plain"])
def test_block_530m_shape_sampled(grid):
    w = si.BLOCK_WORKLOAD
    N, dm, H, d, p, L, K = w["N"], w["dm"], w["H"], w["d"], w["p"], w["L"], w["K"]
    b = si.make_block_inputs(N, dm, H, d, si.workload_seed(6), w["planted"], True, grid=grid)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(N, size=384, replace=False))
    cols_qkv = np.sort(rng.choice(3 * H * d, size=48, replace=False))
    cols_o = np.sort(rng.choice(dm, size=32, replace=False))
    _run_block(b, N, dm, H, d, p, L, K, 0, rows, cols_qkv, cols_o, w["name"], grid)
