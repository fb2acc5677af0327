"""ctypes binding of liblighthouse.so (include/lighthouse.h).

The raw functions keep the C names and take plain integers (device pointers as
ints, stream handle as int).  The helpers below them only marshal torch tensors
into those pointers; every step of the layer runs in the HIP kernels.  There is
no fallback: if the library is missing, importing raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblighthouse.so")

LH_OK, LH_ERR_ARG, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE, LH_ERR_HIP, LH_ERR_GEMM = 0, -1, -2, -3, -4, -5, -6
LH_ERR_SCRATCH = -7
LH_STATIC_SCRATCH_BYTES = 64 << 20
LH_BF16, LH_FP32 = 0, 1
LH_SCATTER_FP_ATOMIC, LH_SCATTER_INT_ATOMIC = 0, 1
LH_SCATTER_DETERMINISTIC = LH_SCATTER_INT_ATOMIC
LH_SCORE_QK, LH_SCORE_K, LH_SCORE_Q, LH_SCORE_QK_PRODUCT = 0, 1, 2, 3
LH_SCORE_KEEP_LEAVES = 0x100   # option bit: also store the level-0 scores (score view)
LH_BWD_KEEP_SUB = 0x100        # option bit of scatter_mode: also store dQ~, dK~, dV~ (fp32 views)
LH_SELECT_PARTITION, LH_SELECT_PARENT_KEPT = 0, 1
VIEWS = {"scores": 0, "sel_start": 1, "sel_level": 2, "qsub": 3, "ksub": 4, "vsub": 5, "osub": 6,
         "lse": 7, "dosub": 8, "dqsub": 9, "dksub": 10, "dvsub": 11, "block_first": 12}

EXPORTS = ("lh_subseq_len", "lh_workspace_bytes", "lh_forward", "lh_backward", "lh_workspace_view",
           "lh_dense_workspace_bytes", "lh_dense_attn_fwd", "lh_dense_attn_bwd", "lh_stage_timing",
           "lh_stage_timing_read", "lh_stage_name", "lh_status_str", "lh_read_selection", "lh_peak_probe",
           "lh_block_workspace_bytes", "lh_block_forward", "lh_block_backward", "lh_forward_scored",
           "lh_subseq_len_sel", "lh_workspace_bytes_sel", "lh_forward_sel", "lh_backward_sel",
           "lh_workspace_view_sel", "lh_read_selection_sel", "lh_forward_static")


class LighthouseError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python hierarchical_selection_attention_amd/build.py`")
    L = C.CDLL(LIB_PATH)
    i, i64, sz, vp = C.c_int, C.c_int64, C.c_size_t, C.c_void_p
    sig = {
        "lh_subseq_len": (i64, [i, i, i, i]),
        "lh_workspace_bytes": (sz, [i, i, i, i, i, i, i]),
        "lh_forward": (i, [vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]),
        "lh_forward_static": (i, [vp, vp, vp, vp, i, i, i, i, i, i, i, vp]),
        "lh_forward_scored": (i, [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]),
        "lh_subseq_len_sel": (i64, [i, i, i, i, i]),
        "lh_workspace_bytes_sel": (sz, [i, i, i, i, i, i, i, i]),
        "lh_forward_sel": (i, [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp, sz, vp]),
        "lh_backward_sel": (i, [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp, sz, vp]),
        "lh_workspace_view_sel": (i, [vp, i, i, i, i, i, i, i, i, i, C.POINTER(vp), C.POINTER(sz)]),
        "lh_read_selection_sel": (i, [vp, i, i, i, i, i, i, i, i, vp, vp, vp]),
        "lh_backward": (i, [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]),
        "lh_workspace_view": (i, [vp, i, i, i, i, i, i, i, i, C.POINTER(vp), C.POINTER(sz)]),
        "lh_read_selection": (i, [vp, i, i, i, i, i, i, i, vp, vp, vp]),
        "lh_peak_probe": (i, [i, vp, vp, sz, vp]),
        "lh_dense_workspace_bytes": (sz, [i, i, i, i]),
        "lh_dense_attn_fwd": (i, [vp, vp, vp, vp, vp, i, i, i, i, vp, sz, vp]),
        "lh_dense_attn_bwd": (i, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, sz, vp]),
        "lh_block_workspace_bytes": (sz, [i, i, i, i, i, i, i]),
        "lh_block_forward": (i, [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp]),
        "lh_block_backward": (i, [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]),
        "lh_stage_timing": (i, [i]),
        "lh_stage_timing_read": (i, [C.POINTER(C.c_double), C.POINTER(C.c_int), i]),
        "lh_stage_name": (C.c_char_p, [i]),
        "lh_status_str": (C.c_char_p, [i]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_L = _load()

# ---------------------------------------------------------------- raw C names
lh_subseq_len = _L.lh_subseq_len
lh_workspace_bytes = _L.lh_workspace_bytes
lh_forward = _L.lh_forward
lh_forward_static = _L.lh_forward_static
lh_forward_scored = _L.lh_forward_scored
lh_subseq_len_sel = _L.lh_subseq_len_sel
lh_workspace_bytes_sel = _L.lh_workspace_bytes_sel
lh_forward_sel = _L.lh_forward_sel
lh_backward_sel = _L.lh_backward_sel
lh_backward = _L.lh_backward
lh_dense_workspace_bytes = _L.lh_dense_workspace_bytes
lh_dense_attn_fwd = _L.lh_dense_attn_fwd
lh_dense_attn_bwd = _L.lh_dense_attn_bwd
lh_stage_timing = _L.lh_stage_timing
lh_read_selection = _L.lh_read_selection
lh_peak_probe = _L.lh_peak_probe
lh_block_workspace_bytes = _L.lh_block_workspace_bytes
lh_block_forward = _L.lh_block_forward
lh_block_backward = _L.lh_block_backward


def lh_status_str(rc: int) -> str:
    return _L.lh_status_str(rc).decode()


def lh_stage_name(stage: int) -> str:
    return _L.lh_stage_name(stage).decode()


def lh_workspace_view(ws_ptr, N, H, d, p, L, K, dtype, view, select_mode=LH_SELECT_PARTITION):
    ptr, nbytes = C.c_void_p(), C.c_size_t()
    rc = _L.lh_workspace_view_sel(ws_ptr, N, H, d, p, L, K, dtype, select_mode, view, C.byref(ptr),
                                  C.byref(nbytes))
    _check(rc, "lh_workspace_view")
    return ptr.value, nbytes.value


def lh_stage_timing_read(n: int = 32):
    ms = (C.c_double * n)()
    cnt = (C.c_int * n)()
    rc = _L.lh_stage_timing_read(ms, cnt, n)
    if rc < 0:
        raise LighthouseError(f"lh_stage_timing_read: {lh_status_str(rc)}")
    return {lh_stage_name(s): (ms[s], cnt[s]) for s in range(min(rc, n)) if cnt[s] > 0}


def _check(rc, what):
    if rc != LH_OK:
        raise LighthouseError(f"{what} failed: {lh_status_str(rc)} ({rc})")


# ------------------------------------------------------- torch marshalling
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LH_BF16
    if t.dtype == torch.float32:
        return LH_FP32
    raise LighthouseError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev_tensor_check(*ts):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise LighthouseError("tensors must be contiguous device tensors")


def alloc_workspace(N, H, d, p, L, K, dtype, device="cuda", select_mode=LH_SELECT_PARTITION):
    torch = _torch()
    nbytes = lh_workspace_bytes_sel(N, H, d, p, L, K, dtype, select_mode)
    if nbytes == 0:
        raise LighthouseError("invalid layer parameters")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def forward(q, k, v, p, L, K, ws=None, out=None, stream=None, score_mode=LH_SCORE_QK,
            select_mode=LH_SELECT_PARTITION, keep_leaf_scores=False):
    """o = Lighthouse layer(q, k, v) for [N, H, d] tensors.  Returns (o, ws).

    score_mode / select_mode other than the defaults use the alternative readings
    (lh_forward_scored / lh_forward_sel); keep_leaf_scores also stores level 0 of
    the score view (LH_SCORE_KEEP_LEAVES)."""
    torch = _torch()
    _dev_tensor_check(q, k, v)
    N, H, d = q.shape
    dt = dtype_code(q)
    if ws is None:
        ws = alloc_workspace(N, H, d, p, L, K, dt, q.device, select_mode)
    if out is None:
        out = torch.empty_like(q)
    if keep_leaf_scores:
        score_mode |= LH_SCORE_KEEP_LEAVES
    if select_mode != LH_SELECT_PARTITION:
        rc = lh_forward_sel(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), N, H, d, p, L, K, dt,
                            score_mode, select_mode, ws.data_ptr(), ws.numel(), _stream_handle(stream))
    elif score_mode == LH_SCORE_QK and not keep_leaf_scores:
        rc = lh_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), N, H, d, p, L, K, dt,
                        ws.data_ptr(), ws.numel(), _stream_handle(stream))
    else:
        rc = lh_forward_scored(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), N, H, d, p, L, K, dt,
                               score_mode, ws.data_ptr(), ws.numel(), _stream_handle(stream))
    _check(rc, "lh_forward")
    return out, ws


def forward_static(q, k, v, p, L, K, out=None, stream=None):
    """lh_forward_static: o of the layer with the library's static per-device workspace
    (no allocation in the library; the output is allocated here unless `out` is given)."""
    torch = _torch()
    _dev_tensor_check(q, k, v)
    N, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    rc = lh_forward_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), N, H, d, p, L, K,
                           dtype_code(q), _stream_handle(stream))
    _check(rc, "lh_forward_static")
    return out


def backward(dout, p, L, K, ws, mode=LH_SCATTER_FP_ATOMIC, grads=None, stream=None,
             select_mode=LH_SELECT_PARTITION, keep_sub_grads=False):
    """(dq, dk, dv) of the Lighthouse layer; ws must come from the matching forward().
    keep_sub_grads: also store dQ~, dK~, dV~ in the workspace (LH_BWD_KEEP_SUB)."""
    torch = _torch()
    _dev_tensor_check(dout)
    N, H, d = dout.shape
    dt = dtype_code(dout)
    if keep_sub_grads:
        mode |= LH_BWD_KEEP_SUB
    if grads is None:
        grads = tuple(torch.empty_like(dout) for _ in range(3))
    dq, dk, dv = grads
    if select_mode == LH_SELECT_PARTITION:
        rc = lh_backward(dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), N, H, d, p, L, K, dt, mode,
                         ws.data_ptr(), ws.numel(), _stream_handle(stream))
    else:
        rc = lh_backward_sel(dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), N, H, d, p, L, K, dt,
                             mode, select_mode, ws.data_ptr(), ws.numel(), _stream_handle(stream))
    _check(rc, "lh_backward")
    return dq, dk, dv


def workspace_tensor(ws, N, H, d, p, L, K, dtype, view, select_mode=LH_SELECT_PARTITION):
    """A typed torch view of one intermediate inside the workspace (see lh_view)."""
    torch = _torch()
    vid = VIEWS[view] if isinstance(view, str) else int(view)
    ptr, nbytes = lh_workspace_view(ws.data_ptr(), N, H, d, p, L, K, dtype, vid, select_mode)
    off = ptr - ws.data_ptr()
    raw = ws[off: off + nbytes]
    S = int(lh_subseq_len_sel(N, p, L, K, select_mode))
    Sp = (S + 63) // 64 * 64
    name = [k for k, v in VIEWS.items() if v == vid][0]
    if name == "scores":
        return raw.view(torch.float32)
    if name == "sel_start":
        return raw.view(torch.int32).view(H, S)
    if name == "sel_level":
        return raw.view(H, S)
    if name in ("qsub", "ksub", "vsub", "osub"):
        return raw.view(torch.float32).view(H, Sp, d)
    if name == "lse":
        return raw.view(torch.float32).view(H, Sp)
    if name in ("dosub", "dqsub", "dksub", "dvsub"):
        return raw.view(torch.float32).view(H, Sp, d)
    if name == "block_first":
        return raw.view(torch.int32).view(H, -1)
    raise LighthouseError(f"unknown view {view}")


def read_selection(ws, N, H, d, p, L, K, dtype, stream=None, select_mode=LH_SELECT_PARTITION):
    """Copies of the kept entries' (start int32 [H][S], level uint8 [H][S])."""
    torch = _torch()
    S = int(lh_subseq_len_sel(N, p, L, K, select_mode))
    if S < 0:
        raise LighthouseError("invalid layer parameters")
    start = torch.empty((H, S), dtype=torch.int32, device=ws.device)
    level = torch.empty((H, S), dtype=torch.uint8, device=ws.device)
    rc = _L.lh_read_selection_sel(ws.data_ptr(), N, H, d, p, L, K, dtype, select_mode, start.data_ptr(),
                                  level.data_ptr(), _stream_handle(stream))
    _check(rc, "lh_read_selection")
    return start, level


def block_workspace(N, H, d, dm, p, L, K, device="cuda"):
    torch = _torch()
    nbytes = lh_block_workspace_bytes(N, H, d, dm, p, L, K)
    if nbytes == 0:
        raise LighthouseError("invalid block parameters")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def block_forward(x, w_qkv, w_o, H, d, p, L, K, ws=None, o=None, y=None, stream=None):
    """y = Lighthouse(x W_Q, x W_K, x W_V) W_O for bf16 x [N, dm], w_qkv [dm, 3Hd], w_o [Hd, dm].

    Returns (y, o, ws); o [N, H, d] and ws are needed by block_backward."""
    torch = _torch()
    _dev_tensor_check(x, w_qkv, w_o)
    N, dm = x.shape
    if x.dtype != torch.bfloat16 or w_qkv.dtype != torch.bfloat16 or w_o.dtype != torch.bfloat16:
        raise LighthouseError("the block takes bf16 tensors")
    if tuple(w_qkv.shape) != (dm, 3 * H * d) or tuple(w_o.shape) != (H * d, dm):
        raise LighthouseError("weight shapes do not match x, H and d")
    if ws is None:
        ws = block_workspace(N, H, d, dm, p, L, K, x.device)
    if o is None:
        o = torch.empty((N, H, d), dtype=torch.bfloat16, device=x.device)
    if y is None:
        y = torch.empty((N, dm), dtype=torch.bfloat16, device=x.device)
    rc = lh_block_forward(x.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr(), o.data_ptr(), y.data_ptr(), N, H, d, dm,
                          p, L, K, ws.data_ptr(), ws.numel(), _stream_handle(stream))
    _check(rc, "lh_block_forward")
    return y, o, ws


def block_backward(x, w_qkv, w_o, o, dy, H, d, p, L, K, ws, mode=LH_SCATTER_FP_ATOMIC, grads=None, stream=None):
    """(dx bf16 [N, dm], dw_qkv fp32 [dm, 3Hd], dw_o fp32 [Hd, dm]) of the block."""
    torch = _torch()
    _dev_tensor_check(x, w_qkv, w_o, o, dy)
    N, dm = x.shape
    if grads is None:
        grads = (torch.empty_like(x), torch.empty(w_qkv.shape, dtype=torch.float32, device=x.device),
                 torch.empty(w_o.shape, dtype=torch.float32, device=x.device))
    dx, dwqkv, dwo = grads
    rc = lh_block_backward(x.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr(), o.data_ptr(), dy.data_ptr(),
                           dx.data_ptr(), dwqkv.data_ptr(), dwo.data_ptr(), N, H, d, dm, p, L, K, mode,
                           ws.data_ptr(), ws.numel(), _stream_handle(stream))
    _check(rc, "lh_block_backward")
    return dx, dwqkv, dwo


def peak_probe(kind, src, dst, n, stream=None):
    """Enqueue one achievable-peak probe (see lh_peak_probe); src/dst are device tensors."""
    rc = lh_peak_probe(kind, src.data_ptr() if src is not None else None, dst.data_ptr(), n,
                       _stream_handle(stream))
    _check(rc, "lh_peak_probe")


def dense_forward(q, k, v, ws=None, out=None, lse=None, stream=None):
    torch = _torch()
    _dev_tensor_check(q, k, v)
    N, H, d = q.shape
    dt = dtype_code(q)
    if ws is None:
        ws = torch.empty(lh_dense_workspace_bytes(N, H, d, dt), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, N), dtype=torch.float32, device=q.device)
    rc = lh_dense_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), N, H, d, dt,
                           ws.data_ptr(), ws.numel(), _stream_handle(stream))
    _check(rc, "lh_dense_attn_fwd")
    return out, lse, ws


def dense_backward(q, k, v, o, lse, dout, ws, grads=None, stream=None):
    torch = _torch()
    N, H, d = q.shape
    dt = dtype_code(q)
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(3))
    dq, dk, dv = grads
    rc = lh_dense_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), N, H, d, dt, ws.data_ptr(), ws.numel(),
                           _stream_handle(stream))
    _check(rc, "lh_dense_attn_bwd")
    return dq, dk, dv
