"""Seeded synthetic inputs for the Lighthouse attention layer.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the layer's arithmetic, so the CPU oracle (``oracle/``) and
the GPU path can both be fed from it without sharing any of the method.

Recipe (one seed per workload, numpy PCG64 streams):

* ``SeedSequence(seed).spawn(5)`` gives independent streams for q, k, v,
  dO and the per-token scale.
* Each [N, H, d] tensor is drawn as i.i.d. N(0, 1) in float32, chunk by chunk
  (``CHUNK`` elements per chunk, chunk i from the i-th child of the tensor's
  stream), so the bytes do not depend on the thread count.
* q, k and v are multiplied by a per-token scale c_t shared by all heads and
  all three tensors: LogNormal(0, 0.5), or |Student-t(3)| for the heavy-tailed
  workload.  Optionally a fraction of tokens (chosen without replacement) has
  its scale multiplied by 4 ("planted" tokens), and optionally a fraction of
  positions (without replacement) is overwritten by exact copies of the q, k
  and v rows of other, uniformly chosen positions, which forces score ties.
* dO is plain N(0, 1).
* bf16 storage rounds the float32 draw to nearest-even and is returned as the
  raw uint16 bit pattern; fp32 storage returns float32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

# The five workloads.  Sizes, p/L/K and distributions follow the paper's
# settings: a tiny fp32 case, a 32K bandwidth case, the 530M model's attention
# shape at 98,304 tokens, 512K kernel-level context and 1M tokens on one GPU.
WORKLOADS = {
    1: dict(name="tiny_fp32_n2048", N=2048, H=2, d=64, dtype="fp32", p=4, L=3, K=16,
            scale="lognormal", planted=0.0, dup=0.0, backward=False),
    2: dict(name="fwd_n32768", N=32768, H=16, d=128, dtype="bf16", p=4, L=4, K=64,
            scale="lognormal", planted=0.0, dup=0.0, backward=False),
    3: dict(name="llama530m_attn_n98304", N=98304, H=16, d=128, dtype="bf16", p=4, L=4, K=128,
            scale="lognormal", planted=0.01, dup=0.0, backward=True),
    4: dict(name="long_ctx_n524288", N=524288, H=16, d=128, dtype="bf16", p=4, L=5, K=128,
            scale="lognormal", planted=0.0, dup=0.0, backward=True),
    5: dict(name="heavy_tail_ties_n1048576", N=1048576, H=8, d=128, dtype="bf16", p=4, L=6, K=128,
            scale="student_t3", planted=0.0, dup=0.05, backward=True),
}


def workload_seed(index: int) -> int:
    return 1000 + int(index)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32, exact."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_normal(shape, ss: np.random.SeedSequence, token_scale, dtype: str, threads: int):
    """Draw an [N, H, d] tensor chunk-wise, scale rows by token_scale (or not)."""
    N, H, d = shape
    total = N * H * d
    row = H * d
    out = np.empty(total, dtype=np.uint16 if dtype == "bf16" else np.float32)
    nchunk = (total + CHUNK - 1) // CHUNK
    children = ss.spawn(nchunk)

    def work(i):
        lo = i * CHUNK
        hi = min(total, lo + CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        z = g.standard_normal(hi - lo, dtype=np.float32)
        if token_scale is not None:
            t0 = lo // row
            t1 = (hi - 1) // row + 1
            c = np.repeat(token_scale[t0:t1], row)[lo - t0 * row: hi - t0 * row]
            z *= c
        out[lo:hi] = bf16_bits(z) if dtype == "bf16" else z

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(nchunk)))
    return out.reshape(N, H, d)


def make_inputs(N: int, H: int, d: int, dtype: str = "bf16", seed: int = 0,
                scale: str = "lognormal", planted: float = 0.0, dup: float = 0.0,
                with_dout: bool = False, threads: int | None = None) -> dict:
    """Return {"q","k","v"[,"dout"]} as [N, H, d] arrays (uint16 bf16 bits or float32).

    Also returns "token_scale" (float32 [N]) and, when dup > 0, "dup_dst"/"dup_src".
    """
    if dtype not in ("bf16", "fp32"):
        raise ValueError("dtype must be 'bf16' or 'fp32'")
    threads = threads or _threads()
    ss_q, ss_k, ss_v, ss_do, ss_c = np.random.SeedSequence(seed).spawn(5)
    gc = np.random.Generator(np.random.PCG64(ss_c))
    if scale == "lognormal":
        c = gc.lognormal(0.0, 0.5, size=N).astype(np.float32)
    elif scale == "student_t3":
        c = np.abs(gc.standard_t(3, size=N)).astype(np.float32)
    elif scale == "none":
        c = np.ones(N, np.float32)
    else:
        raise ValueError(f"unknown scale {scale!r}")
    if planted > 0.0:
        idx = gc.choice(N, size=int(round(planted * N)), replace=False)
        c[idx] *= np.float32(4.0)
    out = {"token_scale": c}
    for name, ss in (("q", ss_q), ("k", ss_k), ("v", ss_v)):
        out[name] = _fill_normal((N, H, d), ss, c, dtype, threads)
    if dup > 0.0 and N > 1:
        dst = gc.choice(N, size=int(round(dup * N)), replace=False)
        src = (dst + 1 + gc.integers(0, N - 1, size=dst.size)) % N
        for name in ("q", "k", "v"):
            x = out[name]
            x[dst] = x[src]          # right side is evaluated first: copies of the pre-copy rows
        out["dup_dst"] = dst
        out["dup_src"] = src
    if with_dout:
        out["dout"] = _fill_normal((N, H, d), ss_do, None, dtype, threads)
    return out


# The attention block around the layer at the 530M model's shape (d_model 2048,
# 16 heads of 128, 98,304 tokens; the layer's settings of workload 3).
BLOCK_WORKLOAD = dict(name="llama530m_block_n98304", N=98304, dm=2048, H=16, d=128, p=4, L=4, K=128,
                      planted=0.01)

X_GRID, GRID_MAX = 16, 256   # x and dy on the grid a / 16 with |a| <= 256


def w_grid(fan_in: int) -> int:
    """Grid 1/G of a weight drawn as N(0, 1/fan_in): G = 2^ceil(log2(16 sqrt(fan_in))), so the
    grid integers have a standard deviation of 16 to 23 and |b| <= 256 clips nothing below 11 sigma."""
    return 1 << int(np.ceil(np.log2(16.0 * np.sqrt(fan_in))))


def _on_grid(z: np.ndarray, grid: float) -> np.ndarray:
    return np.clip(np.rint(z * np.float32(grid)), -GRID_MAX, GRID_MAX).astype(np.float32)


def _exact_fp32_sums(a: np.ndarray, b: np.ndarray) -> bool:
    """Every partial sum of a @ b (integer grids) is below 2^24 in magnitude, by Cauchy-Schwarz:
    max_t |a_t| * max_j |b_j| bounds sum_i |a_ti b_ij|."""
    return float(np.sqrt(np.square(a, dtype=np.float64).sum(axis=1).max())
                 * np.sqrt(np.square(b, dtype=np.float64).sum(axis=0).max())) < 2.0 ** 24


def make_block_inputs(N: int, dm: int, H: int, d: int, seed: int = 0, planted: float = 0.0,
                      with_dy: bool = False, threads: int | None = None, grid: bool = True) -> dict:
    """Inputs of the attention block, all bf16 bit patterns (uint16).

    x [N, dm] = c_t z with z ~ N(0, 1) and the per-token LogNormal(0, 0.5) scale
    of the layer's workloads (optionally a fraction of tokens scaled x4), and
    dy [N, dm] ~ N(0, 1), both on the grid a / 16 with |a| <= 256; w_qkv
    [dm, 3*H*d] ~ N(0, 1/dm) and w_o [H*d, dm] ~ N(0, 1/(H*d)) on the grids
    b / w_grid(fan_in) with |b| <= 256.  On these grids the products x w_qkv
    and dy w_o^T are exact in fp32 whatever the order of summation (checked,
    see _exact_fp32_sums), so both sides round the same values to bf16 where
    they enter the layer.

    grid=False draws the same distributions without the grids: each value is
    the float32 draw rounded to bf16, so the products carry ordinary fp32
    rounding.
    """
    threads = threads or _threads()
    hd = H * d
    ss_x, ss_w, ss_o, ss_dy, ss_c = np.random.SeedSequence(seed).spawn(5)
    gc = np.random.Generator(np.random.PCG64(ss_c))
    c = gc.lognormal(0.0, 0.5, size=N).astype(np.float32)
    if planted > 0.0:
        idx = gc.choice(N, size=int(round(planted * N)), replace=False)
        c[idx] *= np.float32(4.0)
    if not grid:
        out = {"x": _fill_normal((N, 1, dm), ss_x, c, "bf16", threads).reshape(N, dm),
               "w_qkv": bf16_bits(_fill_normal((dm, 1, 3 * hd), ss_w, None, "fp32", threads).reshape(dm, 3 * hd)
                                  / np.float32(np.sqrt(dm))),
               "w_o": bf16_bits(_fill_normal((hd, 1, dm), ss_o, None, "fp32", threads).reshape(hd, dm)
                                / np.float32(np.sqrt(hd))),
               "token_scale": c}
        if with_dy:
            out["dy"] = _fill_normal((N, 1, dm), ss_dy, None, "bf16", threads).reshape(N, dm)
        return out
    a = _on_grid(_fill_normal((N, 1, dm), ss_x, c, "fp32", threads).reshape(N, dm), X_GRID)
    gq, go = w_grid(dm), w_grid(hd)
    b = _on_grid(_fill_normal((dm, 1, 3 * hd), ss_w, None, "fp32", threads).reshape(dm, 3 * hd) / np.sqrt(dm), gq)
    bo = _on_grid(_fill_normal((hd, 1, dm), ss_o, None, "fp32", threads).reshape(hd, dm) / np.sqrt(hd), go)
    if not _exact_fp32_sums(a, b):
        raise ValueError("block inputs too large for exact fp32 sums")
    out = {"x": bf16_bits(a / np.float32(X_GRID)), "w_qkv": bf16_bits(b / np.float32(gq)),
           "w_o": bf16_bits(bo / np.float32(go)), "token_scale": c}
    if with_dy:
        ady = _on_grid(_fill_normal((N, 1, dm), ss_dy, None, "fp32", threads).reshape(N, dm), X_GRID)
        if not _exact_fp32_sums(ady, bo.T):
            raise ValueError("block inputs too large for exact fp32 sums")
        out["dy"] = bf16_bits(ady / np.float32(X_GRID))
    return out


def block_inputs(with_dy: bool = True, threads: int | None = None) -> dict:
    w = BLOCK_WORKLOAD
    return make_block_inputs(w["N"], w["dm"], w["H"], w["d"], workload_seed(6), w["planted"], with_dy, threads)


def workload_inputs(index: int, with_dout: bool | None = None, threads: int | None = None) -> dict:
    w = WORKLOADS[index]
    wd = w["backward"] if with_dout is None else with_dout
    return make_inputs(w["N"], w["H"], w["d"], w["dtype"], workload_seed(index), w["scale"],
                       w["planted"], w["dup"], wd, threads)
