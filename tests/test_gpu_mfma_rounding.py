"""The rounding of the attention kernels' matrix instruction, measured
(lh_peak_probe kind 4): v_mfma_f32_16x16x32_f16 adds 32 exact fp16 products
and an fp32 accumulator, and its result is not the correctly rounded sum.

The error model of the gradient allowance (gpu_util.KAPPA) rests on what this
test checks on random trials, against sums computed on the host in fp64
(exact here to far below one fp32 ulp):
  * per instruction, the error is at most 16 fp32 ulps of the largest of its 33
    addends (the accumulator counts as an addend);
  * the error has no bias: its mean over the trials is below 0.1 ulp.
The trials span three cases: a zero accumulator, accumulators near the size
of the products, and accumulators a thousand times larger.  The products
span a wide range of magnitudes.  Only a correct guess of the lane layout
gives errors this small, so the test also pins that layout.
"""
import numpy as np
import pytest
import torch

from gpu_util import lib, say

pytestmark = pytest.mark.gpu


def _trials(n, seed):
    g = np.random.default_rng(seed)
    a = g.standard_normal((n, 64, 8))
    a *= np.exp(2.0 * g.standard_normal((n, 1, 1)) * (np.arange(n) % 3 == 2)[:, None, None])
    b = g.standard_normal((n, 64, 8))
    cs = np.array([0.0, 10.0, 1000.0])[np.arange(n) % 3]
    c = g.standard_normal((n, 64, 4)) * cs[:, None, None]
    return a.astype(np.float16), b.astype(np.float16), c.astype(np.float32)


def test_mfma_16x16x32_f16_rounding_is_bounded_and_unbiased():
    lh = lib()
    n = 3000
    a, b, c = _trials(n, 2024)
    rec = np.zeros((n, 3072), np.uint8)
    rec[:, :1024] = a.view(np.uint8).reshape(n, 1024)
    rec[:, 1024:2048] = b.view(np.uint8).reshape(n, 1024)
    rec[:, 2048:] = c.view(np.uint8).reshape(n, 1024)
    src = torch.from_numpy(rec).cuda()
    dst = torch.empty((n, 64, 4), dtype=torch.float32, device="cuda")
    lh.peak_probe(4, src, dst, n)
    torch.cuda.synchronize()
    d = dst.cpu().numpy().astype(np.float64)
    # exact sums: out[i][j] = sum_{g<4, e<8} A[lane i + 16 g][e] B[lane j + 16 g][e] + C
    A = a.astype(np.float64).reshape(n, 4, 16, 8)        # [t][g][row i][e]
    B = b.astype(np.float64).reshape(n, 4, 16, 8)        # [t][g][col j][e]
    prod = np.einsum("tgie,tgje->tijge", A, B).reshape(n, 16, 16, 32)
    # C and D: lane l = j + 16 (i // 4) holds rows 4 (l // 16) + r
    Cm = c.astype(np.float64).reshape(n, 4, 16, 4).transpose(0, 1, 3, 2).reshape(n, 16, 16)
    Dm = d.reshape(n, 4, 16, 4).transpose(0, 1, 3, 2).reshape(n, 16, 16)
    exact = prod.sum(axis=-1) + Cm
    big = np.maximum(np.abs(prod).max(axis=-1), np.abs(Cm))
    ulp = np.ldexp(1.0, np.floor(np.log2(np.where(big > 0, big, 1.0))).astype(int) - 23)
    err = (Dm - exact) / ulp
    rne = Dm == exact.astype(np.float32).astype(np.float64)
    say(f"    MFMA 16x16x32 f16: {rne.mean() * 100:.1f}% of results equal the rounded exact sum; "
        f"max |error| {np.abs(err).max():.2f} ulp of the largest addend; mean error {err.mean():+.4f} ulp")
    assert np.abs(err).max() <= 16.0
    assert abs(err.mean()) <= 0.1
