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
# A separately built copy of the same source (the sanitizer build in the tests)
# can be loaded instead by naming it here; it is never built from anything else.
_LIB_OVERRIDE = os.environ.get("LH_ORACLE_LIB")
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
        if _LIB_OVERRIDE:
            path = _LIB_OVERRIDE
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            path = _LIB
        L = C.CDLL(path)
        vp, i32, i64, dp, fp = C.c_void_p, C.c_int, C.c_int64, C.POINTER(C.c_double), C.c_void_p
        L.lho_subseq_len.restype = i64
        L.lho_subseq_len.argtypes = [i32, i32, i32, i32]
        L.lho_subseq_len_sel.restype = i64
        L.lho_subseq_len_sel.argtypes = [i32, i32, i32, i32, i32]
        L.lho_pyramid.restype = i32
        L.lho_pyramid.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp]
        L.lho_leaf_scores.restype = i32
        L.lho_leaf_scores.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp]
        L.lho_forward.restype = i32
        L.lho_forward.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                  vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        L.lho_backward.restype = i32
        L.lho_backward.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp,
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


SELECT_MODES = {"partition": 0, "parent_kept": 1}


def subseq_len(N, p, L, K, select_mode=0) -> int:
    return int(lib().lho_subseq_len_sel(N, p, L, K, int(select_mode)))


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


SCORE_MODES = {"qk": 0, "k": 1, "q": 2, "qk_product": 3}


def leaf_scores(q, k, dtype="bf16", score_mode=0):
    """fp32 leaf scores [H, N] in the fixed reduction order (score_mode: see SCORE_MODES)."""
    q = _in(q, dtype)
    k = _in(k, dtype)
    N, H, d = q.shape
    out = np.zeros((H, N), np.float32)
    rc = lib().lho_leaf_scores(_ptr(q), _ptr(k), N, H, d, DTYPES[dtype], int(score_mode), _ptr(out))
    if rc:
        raise ValueError(f"lho_leaf_scores failed ({rc})")
    return out


def forward(q, k, v, p, L, K, dtype="bf16", want=("sel",), selection=None, nthreads=0, score_mode=0,
            select_mode=0):
    """Run the oracle forward pass.

    select_mode: 0 = the kept entries partition [0, N) (default reading), 1 = a
    selected parent stays beside its children and outputs of overlapping
    entries are summed (see SELECT_MODES).

    score_mode: 0 = |q|^2 + |k|^2 (the default reading), 1 = |k|^2, 2 = |q|^2,
    3 = |q|^2 * |k|^2 (see SCORE_MODES).
    want: any of "levels", "sel", "sub" (Qt, Kt, Vt), "ot" (Ot, lse), "o" (full O).
    selection: optional (start, level) arrays [H, S] to freeze the selection.
    Returns a dict.
    """
    q, k, v = _in(q, dtype), _in(k, dtype), _in(v, dtype)
    N, H, d = q.shape
    S = subseq_len(N, p, L, K, select_mode)
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
    rc = lib().lho_forward(_ptr(q), _ptr(k), _ptr(v), N, H, d, DTYPES[dtype], p, L, K, int(score_mode),
                           int(select_mode), given,
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


def backward(q, k, v, dout, p, L, K, selection, dtype="bf16", want=("sub",), nthreads=0, select_mode=0):
    """Oracle backward with a given selection.

    want: "sub" (dOt, dQt, dKt, dVt), "full" (dq, dk, dv), "cond" (absolute term sums
    cO, cdQ, cdK, cdV [H, S, d]: the scale of the rounding error of each output; and
    lO, ldQ, ldK, ldV [H, S, d]: how far each output moves, to first order, when each
    logit q.k/sqrt(d) moves by at most sum |q||k|/sqrt(d); both used only to set
    comparison tolerances).
    """
    q, k, v, dout = _in(q, dtype), _in(k, dtype), _in(v, dtype), _in(dout, dtype)
    N, H, d = q.shape
    S = subseq_len(N, p, L, K, select_mode)
    st = np.ascontiguousarray(selection[0], dtype=np.int32).reshape(H, S)
    lv = np.ascontiguousarray(selection[1], dtype=np.int8).reshape(H, S)
    sub = "sub" in want
    full = "full" in want
    dOt, dQt, dKt, dVt = ((np.zeros((H, S, d)) if sub else None) for _ in range(4))
    dq, dk, dv = ((np.zeros((N, H, d)) if full else None) for _ in range(3))
    cond = np.zeros((8, H, S, d)) if "cond" in want else None
    rc = lib().lho_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), N, H, d, DTYPES[dtype], p, L, K,
                            int(select_mode), _ptr(st), _ptr(lv), _ptr(dOt), _ptr(dQt), _ptr(dKt), _ptr(dVt),
                            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cond), nthreads)
    if rc:
        raise RuntimeError(f"lho_backward failed ({rc})")
    res = {"S": S}
    if sub:
        res.update(dOt=dOt, dQt=dQt, dKt=dKt, dVt=dVt)
    if full:
        res.update(dq=dq, dk=dk, dv=dv)
    if cond is not None:
        res.update(cO=cond[0], cdQ=cond[1], cdK=cond[2], cdV=cond[3],
                   lO=cond[4], ldQ=cond[5], ldK=cond[6], ldV=cond[7])
    return res


# ------------------------------------------------------------------ the block
# The attention block around the layer: Sec. 3.1 Eq. (1) of the Lighthouse
# paper gives q = x W_Q, k = x W_K, v = x W_V for the layer's input, and Fig. 1
# shows the projections feeding the pyramid pool; the block output is the
# layer output times the output projection W_O (the Llama-style models of
# Sec. 4).  Everything is fp64 except at the layer's boundary: the layer's
# I/O type is bf16, so every tensor that crosses it (q, k, v and dO = dy W_O^T
# in; o, dq, dk, dv out) is rounded to bf16, to nearest with ties to even.  The
# rounding of q and k decides the selection, so it must be taken in the same
# precision as on the GPU.  With round_io=False nothing is rounded to bf16 (the
# layer's oracle then reads fp32 values), which makes the block a smooth
# function of its inputs away from selection changes (used by the gradient
# pins).

def _bf16_f64(bits):
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def _round_bf16(x64):
    """fp64 -> nearest bf16 value (ties to even) via fp32; exact when x64 is an fp32 value."""
    b = np.ascontiguousarray(x64, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def block_forward(x, w_qkv, w_o, H, d, p, L, K, rows=None, round_io=True, cond=False, nthreads=0):
    """y = Lighthouse(x W_Q, x W_K, x W_V) W_O for bf16 bit arrays x [N, dm],
    w_qkv [dm, 3Hd] (columns: W_Q | W_K | W_V), w_o [Hd, dm].

    Returns {"qkv": [3, N, H, d] fp32 layer inputs, "O": [N, H, d] the layer
    output (bf16 values unless round_io=False), "y": [N or len(rows), dm] fp64,
    "start", "level", "near_ties", "round_io"}; with cond=True also "cy" =
    |O| |W_O|, the sums of absolute terms of y (only used to size comparison
    tolerances: one bf16 ulp of every element of O moves y by up to 2^-8 cy).
    """
    X = _bf16_f64(x) if x.dtype == np.uint16 else np.asarray(x, np.float64)
    Wq = _bf16_f64(w_qkv) if w_qkv.dtype == np.uint16 else np.asarray(w_qkv, np.float64)
    Wo = _bf16_f64(w_o) if w_o.dtype == np.uint16 else np.asarray(w_o, np.float64)
    N, hd = X.shape[0], H * d
    proj = X @ Wq                                   # [N, 3Hd]
    qkv = np.empty((3, N, H, d), np.float32)
    for j in range(3):
        part = proj[:, j * hd:(j + 1) * hd]
        qkv[j] = (_round_bf16(part) if round_io else part.astype(np.float32)).reshape(N, H, d)
    r = forward(qkv[0], qkv[1], qkv[2], p, L, K, "fp32", want=("sel", "o"), nthreads=nthreads)
    O = _round_bf16(r["O"]).astype(np.float64) if round_io else r["O"]
    Of = O.reshape(N, hd)
    Or = Of if rows is None else Of[rows]
    res = {"qkv": qkv, "O": O, "y": Or @ Wo, "start": r["start"], "level": r["level"], "near_ties": r["near_ties"],
           "round_io": round_io}
    if cond:
        res["cy"] = np.abs(Or) @ np.abs(Wo)
    return res


def block_backward(fwd, x, w_qkv, w_o, dy, H, d, p, L, K, rows=None, cols_qkv=None, cols_o=None, cond=False,
                   nthreads=0):
    """Gradients of the block for upstream gradient dy [N, dm] (bf16 bits or float).

    fwd is block_forward's result for the same inputs.  dO = dy W_O^T enters the
    layer's backward (Sec. 3: through the scatter, the attention, the gather and
    the pool; the selection carries no gradient), then
    dx = [dq dk dv] W_QKV^T, dW_QKV = x^T [dq dk dv], dW_O = O^T dy.
    rows / cols_qkv / cols_o select the rows of dx and the columns of the weight
    gradients to return (None = all).  cond=True adds the sums of absolute
    terms "cdx", "cdw_qkv", "cdw_o" of the same elements (tolerance sizing only).
    """
    X = _bf16_f64(x) if x.dtype == np.uint16 else np.asarray(x, np.float64)
    Wq = _bf16_f64(w_qkv) if w_qkv.dtype == np.uint16 else np.asarray(w_qkv, np.float64)
    Wo = _bf16_f64(w_o) if w_o.dtype == np.uint16 else np.asarray(w_o, np.float64)
    dY = _bf16_f64(dy) if dy.dtype == np.uint16 else np.asarray(dy, np.float64)
    N, hd = X.shape[0], H * d
    rnd = fwd["round_io"]
    dO = dY @ Wo.T
    dO = (_round_bf16(dO) if rnd else dO.astype(np.float32)).reshape(N, H, d)
    qkv = fwd["qkv"]
    g = backward(qkv[0], qkv[1], qkv[2], dO, p, L, K, (fwd["start"], fwd["level"]), "fp32", want=("full",),
                 nthreads=nthreads)
    G = np.concatenate([g["dq"].reshape(N, hd), g["dk"].reshape(N, hd), g["dv"].reshape(N, hd)], axis=1)
    if rnd:
        G = _round_bf16(G).astype(np.float64)
    Of = fwd["O"].reshape(N, hd)
    Gr = G if rows is None else G[rows]
    Gc = G if cols_qkv is None else G[:, cols_qkv]
    dYc = dY if cols_o is None else dY[:, cols_o]
    res = {"dx": Gr @ Wq.T, "dw_qkv": X.T @ Gc, "dw_o": Of.T @ dYc, "dO": dO, "G": G}
    if cond:
        res["cdx"] = np.abs(Gr) @ np.abs(Wq.T)
        res["cdw_qkv"] = np.abs(X.T) @ np.abs(Gc)
        res["cdw_o"] = np.abs(Of.T) @ np.abs(dYc)
    return res
