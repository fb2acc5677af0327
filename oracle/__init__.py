"""CPU oracle for the Lighthouse attention layer (ctypes wrapper over lh_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg.  The GPU path never imports it and has no
fallback to it.  Every function follows the steps listed in lh_oracle.c, which
cite the source pages.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lh_oracle.c")
_LIB = os.path.join(_HERE, "liblh_oracle.so")
_lib = None

DTYPES = {"bf16": 0, "fp32": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
                        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        vp, i32, i64, dp, fp = C.c_void_p, C.c_int, C.c_int64, C.POINTER(C.c_double), C.c_void_p
        L.lho_subseq_len.restype = i64
        L.lho_subseq_len.argtypes = [i32, i32, i32, i32]
        L.lho_pyramid.restype = i32
        L.lho_pyramid.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp]
        L.lho_leaf_scores.restype = i32
        L.lho_leaf_scores.argtypes = [vp, vp, i32, i32, i32, i32, vp]
        L.lho_forward.restype = i32
        L.lho_forward.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                  vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        L.lho_backward.restype = i32
        L.lho_backward.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp,
                                   vp, vp, vp, vp, vp, vp, vp, vp, i32]
        _lib = L
        del dp, fp
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _in(x, dtype):
    want = np.uint16 if dtype == "bf16" else np.float32
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"expected {want} array for dtype {dtype}, got {x.dtype}")
    return x


def subseq_len(N, p, L, K) -> int:
    return int(lib().lho_subseq_len(N, p, L, K))


def score_level_sizes(N, p, L):
    return [N // p ** l for l in range(L)]


def pyramid(x, p, L, dtype="bf16"):
    """Levels 1..L-1 of the mean pyramid, fp64, as a list of [N/p^l, H, d] arrays."""
    x = _in(x, dtype)
    N, H, d = x.shape
    sizes = [N // p ** l for l in range(1, L)]
    out = np.zeros(sum(sizes) * H * d, np.float64)
    rc = lib().lho_pyramid(_ptr(x), N, H, d, DTYPES[dtype], p, L, _ptr(out))
    if rc:
        raise ValueError(f"lho_pyramid failed ({rc})")
    res, off = [], 0
    for n in sizes:
        res.append(out[off: off + n * H * d].reshape(n, H, d))
        off += n * H * d
    return res


def leaf_scores(q, k, dtype="bf16"):
    """fp32 leaf scores [H, N] in the fixed reduction order."""
    q = _in(q, dtype)
    k = _in(k, dtype)
    N, H, d = q.shape
    out = np.zeros((H, N), np.float32)
    rc = lib().lho_leaf_scores(_ptr(q), _ptr(k), N, H, d, DTYPES[dtype], _ptr(out))
    if rc:
        raise ValueError(f"lho_leaf_scores failed ({rc})")
    return out


def forward(q, k, v, p, L, K, dtype="bf16", want=("sel",), selection=None, nthreads=0):
    """Run the oracle forward pass.

    want: any of "levels", "sel", "sub" (Qt, Kt, Vt), "ot" (Ot, lse), "o" (full O).
    selection: optional (start, level) arrays [H, S] to freeze the selection.
    Returns a dict.
    """
    q, k, v = _in(q, dtype), _in(k, dtype), _in(v, dtype)
    N, H, d = q.shape
    S = subseq_len(N, p, L, K)
    if S < 0:
        raise ValueError("invalid (N, p, L, K)")
    res = {"S": S}
    if selection is not None:
        st = np.ascontiguousarray(selection[0], dtype=np.int32).reshape(H, S)
        lv = np.ascontiguousarray(selection[1], dtype=np.int8).reshape(H, S)
        given = 1
    else:
        st = np.zeros((H, S), np.int32)
        lv = np.zeros((H, S), np.int8)
        given = 0
    levels = None
    if "levels" in want:
        levels = np.zeros(sum(score_level_sizes(N, p, L)) * H, np.float32)
    sub = "sub" in want
    Qt = np.zeros((H, S, d)) if sub else None
    Kt = np.zeros((H, S, d)) if sub else None
    Vt = np.zeros((H, S, d)) if sub else None
    ot = "ot" in want
    Ot = np.zeros((H, S, d)) if ot else None
    lse = np.zeros((H, S)) if ot else None
    O = np.zeros((N, H, d)) if "o" in want else None
    ties = np.zeros(H, np.int32)
    rc = lib().lho_forward(_ptr(q), _ptr(k), _ptr(v), N, H, d, DTYPES[dtype], p, L, K, given,
                           _ptr(levels), _ptr(st), _ptr(lv), _ptr(Qt), _ptr(Kt), _ptr(Vt), _ptr(Ot),
                           _ptr(lse), _ptr(O), _ptr(ties), nthreads)
    if rc:
        raise RuntimeError(f"lho_forward failed ({rc})")
    res["start"], res["level"] = st, lv
    res["near_ties"] = ties
    if levels is not None:
        lev, off = [], 0
        for n in score_level_sizes(N, p, L):
            lev.append(levels[off: off + n * H].reshape(H, n))
            off += n * H
        res["levels"] = lev
    if sub:
        res["Qt"], res["Kt"], res["Vt"] = Qt, Kt, Vt
    if ot:
        res["Ot"], res["lse"] = Ot, lse
    if O is not None:
        res["O"] = O
    return res


def backward(q, k, v, dout, p, L, K, selection, dtype="bf16", want=("sub",), nthreads=0):
    """Oracle backward with a given selection.

    want: "sub" (dOt, dQt, dKt, dVt), "full" (dq, dk, dv), "cond" (absolute term sums
    cO, cdQ, cdK, cdV [H, S, d]: the scale of the rounding error of each output, used
    only to set comparison tolerances).
    """
    q, k, v, dout = _in(q, dtype), _in(k, dtype), _in(v, dtype), _in(dout, dtype)
    N, H, d = q.shape
    S = subseq_len(N, p, L, K)
    st = np.ascontiguousarray(selection[0], dtype=np.int32).reshape(H, S)
    lv = np.ascontiguousarray(selection[1], dtype=np.int8).reshape(H, S)
    sub = "sub" in want
    full = "full" in want
    dOt, dQt, dKt, dVt = ((np.zeros((H, S, d)) if sub else None) for _ in range(4))
    dq, dk, dv = ((np.zeros((N, H, d)) if full else None) for _ in range(3))
    cond = np.zeros((4, H, S, d)) if "cond" in want else None
    rc = lib().lho_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), N, H, d, DTYPES[dtype], p, L, K,
                            _ptr(st), _ptr(lv), _ptr(dOt), _ptr(dQt), _ptr(dKt), _ptr(dVt),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cond), nthreads)
    if rc:
        raise RuntimeError(f"lho_backward failed ({rc})")
    res = {"S": S}
    if sub:
        res.update(dOt=dOt, dQt=dQt, dKt=dKt, dVt=dVt)
    if full:
        res.update(dq=dq, dk=dk, dv=dv)
    if cond is not None:
        res.update(cO=cond[0], cdQ=cond[1], cdK=cond[2], cdV=cond[3])
    return res
