"""Pins of the block oracle (the projections around the layer, Sec. 3.1 Eq. (1)
and Fig. 1 of the Lighthouse paper) against results fixed independently of it:
permutation weights that reduce the block to the layer oracle by indexing, the
homogeneity identities of the gradients, and central finite differences."""
import numpy as np
import pytest

import oracle
import synth_inputs as si


def _layer_on(q, k, v, p, L, K):
    return oracle.forward(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), p, L, K, "fp32",
                          want=("sel", "o"))


def test_permutation_weights_reduce_block_to_layer():
    """W_Q, W_K, W_V, W_O = permutation matrices: q = x[:, pi_q] etc., y[:, pi_o] = O
    rounded to bf16 (the layer's output type)."""
    N, H, d, p, L, K = 512, 2, 16, 2, 3, 4
    hd = H * d
    dm = hd
    rng = np.random.default_rng(7)
    x = si.bf16_bits(rng.standard_normal((N, dm)).astype(np.float32) * rng.lognormal(0, 0.5, (N, 1)).astype(np.float32))
    perms = [rng.permutation(dm) for _ in range(4)]
    w_qkv = np.zeros((dm, 3 * hd), np.float32)
    for j in range(3):
        w_qkv[perms[j], j * hd + np.arange(hd)] = 1.0     # column c of block j picks input perms[j][c]
    w_o = np.zeros((hd, dm), np.float32)
    w_o[np.arange(hd), perms[3]] = 1.0                   # row i of O goes to output column perms[3][i]
    f = oracle.block_forward(x, si.bf16_bits(w_qkv), si.bf16_bits(w_o), H, d, p, L, K)
    xf = si.bf16_to_f32(x).astype(np.float64)
    q, k, v = (xf[:, perms[j]].reshape(N, H, d) for j in range(3))
    ref = _layer_on(q, k, v, p, L, K)
    assert np.array_equal(f["start"], ref["start"]) and np.array_equal(f["level"], ref["level"])
    y_ref = np.empty((N, dm))
    y_ref[:, perms[3]] = si.bf16_to_f32(si.bf16_bits(ref["O"].astype(np.float32))).reshape(N, hd)
    assert np.array_equal(f["y"], y_ref)
    for j, t in enumerate((q, k, v)):
        assert np.array_equal(f["qkv"][j], t.astype(np.float32))


def _small(seed, N=256, H=2, d=16, dm=24):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, dm)) * rng.lognormal(0, 0.5, (N, 1))
    w_qkv = rng.standard_normal((dm, 3 * H * d)) / np.sqrt(dm)
    w_o = rng.standard_normal((H * d, dm)) / np.sqrt(H * d)
    dy = rng.standard_normal((N, dm))
    return x, w_qkv, w_o, dy


def _run(x, w_qkv, w_o, dy, H, d, p, L, K):
    f = oracle.block_forward(x, w_qkv, w_o, H, d, p, L, K, round_io=False)
    b = oracle.block_backward(f, x, w_qkv, w_o, dy, H, d, p, L, K)
    return f, b


@pytest.mark.parametrize("seed", [1, 2])
def test_gradient_homogeneity_identities(seed):
    """y is linear in W_O and in W_V (the selection and the attention weights do
    not depend on v), so <dW_O, W_O> = <dW_V, W_V> = <dy, y>; scaling W_Q or
    W_K scales the logits alike, so <dW_Q, W_Q> = <dW_K, W_K>; and x W_QKV is
    bilinear, so <dx, x> = <dW_QKV, W_QKV>."""
    H, d, p, L, K = 2, 16, 2, 3, 4
    hd = H * d
    x, w_qkv, w_o, dy = _small(seed, H=H, d=d)
    f, b = _run(x, w_qkv, w_o, dy, H, d, p, L, K)
    ydy = float(np.sum(f["y"] * dy))
    assert abs(float(np.sum(b["dw_o"] * w_o)) - ydy) <= 1e-9 * abs(ydy) + 1e-12
    wv = w_qkv[:, 2 * hd:]
    assert abs(float(np.sum(b["dw_qkv"][:, 2 * hd:] * wv)) - ydy) <= 1e-5 * abs(ydy)
    gq = float(np.sum(b["dw_qkv"][:, :hd] * w_qkv[:, :hd]))
    gk = float(np.sum(b["dw_qkv"][:, hd:2 * hd] * w_qkv[:, hd:2 * hd]))
    assert abs(gq - gk) <= 1e-5 * (abs(gq) + abs(gk)) + 1e-9
    assert abs(gq) > 1e-3          # the identity is not vacuous
    a1 = float(np.sum(b["dx"] * x))
    a2 = float(np.sum(b["dw_qkv"] * w_qkv))
    assert abs(a1 - a2) <= 1e-9 * (abs(a1) + abs(a2))


@pytest.mark.parametrize("which", ["x", "w_qkv", "w_o"])
def test_gradients_match_central_differences(which):
    """<grad, u> equals (f(theta + e u) - f(theta - e u)) / 2e for f = <dy, y>,
    along a random direction u, with the selection unchanged at both points."""
    H, d, p, L, K = 2, 16, 2, 3, 4
    x, w_qkv, w_o, dy = _small(11, H=H, d=d)
    f, b = _run(x, w_qkv, w_o, dy, H, d, p, L, K)
    args = {"x": x, "w_qkv": w_qkv, "w_o": w_o}
    grad = {"x": b["dx"], "w_qkv": b["dw_qkv"], "w_o": b["dw_o"]}[which]
    u = np.random.default_rng(3).standard_normal(args[which].shape)
    eps = 1e-3
    vals = []
    for sgn in (1, -1):
        a = dict(args)
        a[which] = args[which] + sgn * eps * u
        g = oracle.block_forward(a["x"], a["w_qkv"], a["w_o"], H, d, p, L, K, round_io=False)
        assert np.array_equal(g["start"], f["start"]) and np.array_equal(g["level"], f["level"])
        vals.append(float(np.sum(g["y"] * dy)))
    fd = (vals[0] - vals[1]) / (2 * eps)
    an = float(np.sum(grad * u))
    assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (fd, an)


def test_rounded_projection_is_round_to_nearest_even_of_exact_product():
    """On the block input grids the products are exact in fp32, so the oracle's
    q equals the exact integer-grid product rounded once to bf16."""
    b = si.make_block_inputs(64, 32, 2, 16, seed=3)
    f = oracle.block_forward(b["x"], b["w_qkv"], b["w_o"], 2, 16, 2, 3, 4)
    a = np.rint(si.bf16_to_f32(b["x"]).astype(np.float64) * si.X_GRID).astype(np.int64)
    g = si.w_grid(32)
    w = np.rint(si.bf16_to_f32(b["w_qkv"]).astype(np.float64) * g).astype(np.int64)
    exact = (a @ w).astype(np.float64) / (si.X_GRID * g)                # integer matmul, exact
    want = si.bf16_to_f32(si.bf16_bits(exact.astype(np.float32)))
    got = np.concatenate([f["qkv"][j].reshape(64, -1) for j in range(3)], axis=1)
    assert np.array_equal(got, want)
