"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and validates arguments before any launch (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

import oracle
import synth_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lh():
    import hierarchical_selection_attention_amd as lh
    return lh


def test_library_exports_every_declared_function():
    lh = _lh()
    header = open(os.path.join(ROOT, "include", "lighthouse.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    declared = set(re.findall(r"\b(lh_[a-z_]+)\s*\(", header))
    assert declared, "no declarations found"
    raw = C.CDLL(lh.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(raw, name), f"{name} declared in lighthouse.h but not exported"
    assert declared == set(lh.EXPORTS)


@pytest.mark.parametrize("N,p,L,K", [(2048, 4, 3, 16), (2048, 4, 3, 512), (524288, 4, 5, 128), (1048576, 4, 6, 128),
                                     (1080, 3, 4, 5), (16384, 2, 3, 100), (512, 4, 1, 7), (2048, 4, 3, 0),
                                     (4096, 2, 8, 3), (98304, 4, 4, 128), (32768, 4, 4, 64)])
def test_subseq_len_matches_oracle(N, p, L, K):
    lh = _lh()
    assert lh.lh_subseq_len(N, p, L, K) == oracle.subseq_len(N, p, L, K)


def test_subseq_len_and_workspace_reject_bad_arguments():
    lh = _lh()
    assert lh.lh_subseq_len(2047, 4, 3, 5) == lh.LH_ERR_SHAPE       # p^(L-1) does not divide N
    assert lh.lh_subseq_len(64, 4, 5, 5) == lh.LH_ERR_SHAPE         # p^(L-1) > N
    assert lh.lh_subseq_len(2048, 1, 3, 5) == lh.LH_ERR_ARG         # p < 2
    assert lh.lh_subseq_len(2048, 4, 0, 5) == lh.LH_ERR_ARG         # L < 1
    assert lh.lh_subseq_len(2048, 4, 3, -1) == lh.LH_ERR_ARG        # K < 0
    assert lh.lh_workspace_bytes(2048, 2, 96, 4, 3, 16, 0) == 0     # d not in {64, 128}
    assert lh.lh_workspace_bytes(2048, 2, 64, 4, 3, 16, 7) == 0     # unknown dtype
    assert lh.lh_workspace_bytes(2048, 128, 128, 4, 3, 16, 0) == 0  # H*d > 8192
    assert lh.lh_workspace_bytes(1 << 20, 2, 64, 2, 3, 4096, 0) == 0  # K > 2048 with a real choice
    for idx, w in si.WORKLOADS.items():
        code = 0 if w["dtype"] == "bf16" else 1
        assert lh.lh_workspace_bytes(w["N"], w["H"], w["d"], w["p"], w["L"], w["K"], code) > 0


def test_entry_points_validate_before_launching():
    """Invalid calls return their status without touching the GPU (this runs on a CPU host)."""
    lh = _lh()
    N, H, d, p, L, K = 2048, 2, 64, 4, 3, 16
    nb = lh.lh_workspace_bytes(N, H, d, p, L, K, 1)
    fake = 1 << 20          # never dereferenced: every call below fails validation first
    aligned_ws = 1 << 24
    assert lh.lh_forward(None, fake, fake, fake, N, H, d, p, L, K, 1, aligned_ws, nb, None) == lh.LH_ERR_ARG
    assert lh.lh_forward(fake, fake, fake, fake, N, H, 96, p, L, K, 1, aligned_ws, nb, None) == lh.LH_ERR_SHAPE
    assert lh.lh_forward(fake, fake, fake, fake, 2047, H, d, p, L, K, 1, aligned_ws, nb, None) == lh.LH_ERR_SHAPE
    assert lh.lh_forward(fake, fake, fake, fake, N, H, d, p, L, K, 3, aligned_ws, nb, None) == lh.LH_ERR_DTYPE
    assert lh.lh_forward(fake, fake, fake, fake, N, H, d, p, L, K, 1, aligned_ws, nb - 1, None) == lh.LH_ERR_WORKSPACE
    assert lh.lh_forward(fake, fake, fake, fake, N, H, d, p, L, K, 1, aligned_ws + 16, nb, None) == lh.LH_ERR_WORKSPACE
    assert lh.lh_forward(fake, fake, fake, fake, N, H, d, p, L, K, 1, None, nb, None) == lh.LH_ERR_WORKSPACE
    assert lh.lh_forward(fake + 2, fake, fake, fake, N, H, d, p, L, K, 1, aligned_ws, nb, None) == lh.LH_ERR_ARG
    assert lh.lh_backward(fake, fake, fake, fake, N, H, d, p, L, K, 1, 2, aligned_ws, nb, None) == lh.LH_ERR_DTYPE
    assert lh.lh_backward(fake, None, fake, fake, N, H, d, p, L, K, 1, 0, aligned_ws, nb, None) == lh.LH_ERR_ARG
    assert lh.lh_backward(fake, fake, fake, fake, N, H, d, p, L, K, 1, 0, aligned_ws, 0, None) == lh.LH_ERR_WORKSPACE
    # the keep-sub-gradients bit is accepted beside either scatter mode (the call then fails
    # at the workspace check); other bits are not
    for mode in (0, 1):
        assert lh.lh_backward(fake, fake, fake, fake, N, H, d, p, L, K, 1, mode | lh.LH_BWD_KEEP_SUB, aligned_ws, 0,
                              None) == lh.LH_ERR_WORKSPACE
    assert lh.lh_backward(fake, fake, fake, fake, N, H, d, p, L, K, 1, 0x200, aligned_ws, nb, None) == lh.LH_ERR_DTYPE
    assert lh.lh_dense_workspace_bytes(1000, 2, 64, 0) == 0          # N not a multiple of 64
    assert lh.lh_dense_workspace_bytes(1024, 2, 64, 1) == 0          # dense path is bf16
    assert lh.lh_dense_attn_fwd(fake, fake, fake, fake, fake, 1000, 2, 64, 0, aligned_ws, 1 << 30, None) \
        == lh.LH_ERR_SHAPE
    assert lh.lh_read_selection(None, N, H, d, p, L, K, 1, fake, fake, None) == lh.LH_ERR_ARG
    assert lh.lh_read_selection(aligned_ws, N, H, d, p, L, K, 1, None, None, None) == lh.LH_ERR_ARG
    assert lh.lh_read_selection(aligned_ws, 2047, H, d, p, L, K, 1, fake, fake, None) == lh.LH_ERR_SHAPE
    assert lh.lh_read_selection(aligned_ws, N, H, d, p, L, K, 7, fake, fake, None) == lh.LH_ERR_DTYPE
    assert lh.lh_peak_probe(6, fake, fake, 1 << 20, None) == lh.LH_ERR_ARG        # unknown kind
    assert lh.lh_peak_probe(5, None, fake, 16 << 20, None) == lh.LH_ERR_ARG       # token rows: whole 64 MiB groups
    assert lh.lh_peak_probe(5, None, fake + 8, 64 << 20, None) == lh.LH_ERR_ARG   # misaligned
    assert lh.lh_peak_probe(5, None, fake, (1 << 40) + (64 << 20), None) == lh.LH_ERR_ARG
    assert lh.lh_peak_probe(4, fake, fake, (1 << 20) + 1, None) == lh.LH_ERR_ARG  # too many rounding trials
    assert lh.lh_peak_probe(0, fake, fake, 17, None) == lh.LH_ERR_ARG             # not a multiple of 16
    assert lh.lh_peak_probe(0, None, fake, 1 << 20, None) == lh.LH_ERR_ARG        # read needs a source
    assert lh.lh_peak_probe(2, fake + 4, fake, 1 << 20, None) == lh.LH_ERR_ARG    # misaligned
    assert lh.lh_peak_probe(1, None, None, 1 << 20, None) == lh.LH_ERR_ARG
    assert lh.lh_peak_probe(3, None, fake, (1 << 30) + 1, None) == lh.LH_ERR_ARG


def test_workspace_views_are_inside_the_workspace():
    lh = _lh()
    for idx, w in si.WORKLOADS.items():
        code = 0 if w["dtype"] == "bf16" else 1
        args = (w["N"], w["H"], w["d"], w["p"], w["L"], w["K"], code)
        nb = lh.lh_workspace_bytes(*args)
        base = 1 << 32
        for name, vid in lh.VIEWS.items():
            ptr, n = lh.lh_workspace_view(base, *args, vid)
            assert base <= ptr and ptr + n <= base + nb, name
            assert (ptr - base) % 256 == 0


def test_status_strings_and_stage_names():
    lh = _lh()
    for rc in (0, -1, -2, -3, -4, -5):
        assert lh.lh_status_str(rc) and lh.lh_status_str(rc) != "unknown status"
    assert lh.lh_stage_name(0) == "pool_score"
    assert lh.lh_stage_name(99) == "unknown"


def test_block_entry_points_validate_before_launching():
    """The block's host checks return their status without touching the GPU."""
    lh = _lh()
    N, H, d, dm, p, L, K = 2048, 2, 64, 128, 4, 3, 16
    nb = lh.lh_block_workspace_bytes(N, H, d, dm, p, L, K)
    assert nb > lh.lh_workspace_bytes(N, H, d, p, L, K, 0)
    assert lh.lh_block_workspace_bytes(N, H, d, 100, p, L, K) == 0       # dm not a multiple of 8
    assert lh.lh_block_workspace_bytes(N, H, 96, dm, p, L, K) == 0       # d not in {64, 128}
    assert lh.lh_block_workspace_bytes(2047, H, d, dm, p, L, K) == 0     # p^(L-1) does not divide N
    fake = 1 << 20                                                       # never dereferenced
    args = (fake, fake, fake, fake, fake)
    assert lh.lh_block_forward(*args, N, H, d, 100, p, L, K, fake * 256, nb, None) == lh.LH_ERR_SHAPE
    assert lh.lh_block_forward(None, fake, fake, fake, fake, N, H, d, dm, p, L, K, fake * 256, nb,
                               None) == lh.LH_ERR_ARG
    assert lh.lh_block_forward(*args, N, H, d, dm, p, L, K, fake * 256, nb - 1, None) == lh.LH_ERR_WORKSPACE
    assert lh.lh_block_forward(fake + 8, fake, fake, fake, fake, N, H, d, dm, p, L, K, fake * 256, nb,
                               None) == lh.LH_ERR_ARG                    # misaligned x
    bargs = (fake,) * 8
    assert lh.lh_block_backward(*bargs, N, H, d, dm, p, L, K, 5, fake * 256, nb, None) == lh.LH_ERR_DTYPE
    assert lh.lh_block_backward(*bargs, N, H, d, dm, p, L, K, 0, fake * 256, nb - 1, None) == lh.LH_ERR_WORKSPACE
    assert lh.lh_status_str(lh.LH_ERR_GEMM).startswith("GEMM")


def test_scored_forward_rejects_unknown_score_mode():
    lh = _lh()
    fake = 1 << 20                                                       # never dereferenced
    nb = lh.lh_workspace_bytes(2048, 2, 64, 4, 3, 16, 1)
    assert lh.lh_forward_scored(fake, fake, fake, fake, 2048, 2, 64, 4, 3, 16, 1, 7, fake * 256, nb,
                                None) == lh.LH_ERR_DTYPE
    assert lh.lh_forward_scored(fake, fake, fake, fake, 2048, 2, 64, 4, 3, 16, 1, -1, fake * 256, nb,
                                None) == lh.LH_ERR_DTYPE
    # the keep-leaves option bit does not make an unknown mode valid
    assert lh.lh_forward_scored(fake, fake, fake, fake, 2048, 2, 64, 4, 3, 16, 1, lh.LH_SCORE_KEEP_LEAVES | 7,
                                fake * 256, nb, None) == lh.LH_ERR_DTYPE


def test_keep_leaves_bit_matches_the_header():
    lh = _lh()
    hdr = open(os.path.join(ROOT, "include", "lighthouse.h")).read()
    m = re.search(r"#define\s+LH_SCORE_KEEP_LEAVES\s+(0x[0-9a-fA-F]+|\d+)", hdr)
    assert m and int(m.group(1), 0) == lh.LH_SCORE_KEEP_LEAVES
    assert lh.LH_SCORE_KEEP_LEAVES & 0xff == 0   # clear of every score mode


def test_keep_sub_gradients_bit_matches_the_header():
    lh = _lh()
    hdr = open(os.path.join(ROOT, "include", "lighthouse.h")).read()
    m = re.search(r"#define\s+LH_BWD_KEEP_SUB\s+(0x[0-9a-fA-F]+|\d+)", hdr)
    assert m and int(m.group(1), 0) == lh.LH_BWD_KEEP_SUB
    assert lh.LH_BWD_KEEP_SUB & (lh.LH_SCATTER_FP_ATOMIC | lh.LH_SCATTER_INT_ATOMIC) == 0


@pytest.mark.parametrize("N,p,L,K", [(2048, 4, 3, 16), (2048, 4, 3, 512), (524288, 4, 5, 128), (1080, 3, 4, 5),
                                     (4096, 2, 8, 3), (256, 4, 4, 0), (512, 4, 1, 7)])
def test_parent_kept_subseq_len_matches_oracle(N, p, L, K):
    lh = _lh()
    assert lh.lh_subseq_len_sel(N, p, L, K, 1) == oracle.subseq_len(N, p, L, K, 1)
    assert lh.lh_subseq_len_sel(N, p, L, K, 0) == lh.lh_subseq_len(N, p, L, K)


def test_select_mode_validation():
    lh = _lh()
    assert lh.lh_subseq_len_sel(2048, 4, 3, 16, 2) == lh.LH_ERR_DTYPE                  # unknown mode
    assert lh.lh_workspace_bytes_sel(2048, 2, 64, 4, 3, 16, 1, 1) == 0                # parent kept is bf16 only
    assert lh.lh_workspace_bytes_sel(2048, 2, 64, 4, 3, 16, 0, 1) > 0
    fake = 1 << 20                                                                     # never dereferenced
    nb = lh.lh_workspace_bytes_sel(2048, 2, 64, 4, 3, 16, 0, 1)
    assert lh.lh_forward_sel(fake, fake, fake, fake, 2048, 2, 64, 4, 3, 16, 1, 0, 1, fake * 256, nb,
                             None) == lh.LH_ERR_DTYPE
    assert lh.lh_forward_sel(fake, fake, fake, fake, 2048, 2, 64, 4, 3, 16, 0, 0, 3, fake * 256, nb,
                             None) == lh.LH_ERR_DTYPE
    assert lh.lh_backward_sel(fake, fake, fake, fake, 2048, 2, 64, 4, 3, 16, 0, 0, 1, fake * 256, nb - 1,
                              None) == lh.LH_ERR_WORKSPACE


def test_forward_static_rejects_before_any_launch():
    """lh_forward_static validates on the host: bad shapes, and shapes whose forward state
    exceeds its static array (LH_ERR_SCRATCH), return before touching a device."""
    import hierarchical_selection_attention_amd as lh
    fake = 1 << 20
    assert lh.lh_forward_static(fake, fake, fake, fake, 524288, 16, 128, 4, 5, 128, 0, None) == lh.LH_ERR_SCRATCH
    assert lh.lh_forward_static(fake, fake, fake, fake, 2048, 2, 96, 4, 3, 16, 0, None) == lh.LH_ERR_SHAPE
    assert lh.lh_forward_static(fake, fake, fake, fake, 2047, 2, 64, 4, 3, 16, 0, None) == lh.LH_ERR_SHAPE
    assert lh.lh_forward_static(fake, fake, fake, fake, 2048, 2, 64, 4, 3, 16, 7, None) == lh.LH_ERR_DTYPE
    assert "static array" in lh.lh_status_str(lh.LH_ERR_SCRATCH)


def test_workspace_plan_accepts_every_valid_shape():
    """Every shape lh_subseq_len accepts gets a workspace in both selection modes, over a
    sweep that includes K = 0, K above every candidate count, one level and deep
    pyramids."""
    lh = _lh()
    n_ok = 0
    for p in (2, 3, 4, 8):
        for L in range(1, 9):
            top = p ** (L - 1)
            for mult in (1, 3, 16):
                N = top * mult * (64 if top < 64 else 1)
                if N > (1 << 22):
                    continue
                for K in (0, 1, 5, 64, 300, N):
                    if lh.lh_subseq_len(N, p, L, K) < 0:
                        continue
                    for H, d in ((1, 64), (3, 64), (16, 128)):
                        assert lh.lh_workspace_bytes(N, H, d, p, L, K, 0) > 0, (N, H, d, p, L, K)
                        assert lh.lh_workspace_bytes_sel(N, H, d, p, L, K, 0, 1) > 0, (N, H, d, p, L, K)
                        n_ok += 1
    assert n_ok > 500
