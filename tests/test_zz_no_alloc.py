"""lh_forward_static, the forward that allocates nothing (its workspace is the
library's static per-device array), against lh_forward through the C ABI:
the same output bit for bit on two calls in a row, the second with a smaller
input, so what the first left in the shared array cannot matter."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

# (N, H, d, dtype, p, L, K): the first fills most of the 64 MiB array
CASES = [(16384, 16, 128, "bf16", 4, 4, 32), (2048, 4, 128, "bf16", 4, 3, 8), (1024, 2, 64, "fp32", 4, 3, 6)]


def test_forward_static_equals_forward_on_consecutive_calls():
    import hierarchical_selection_attention_amd as lh
    for i, (N, H, d, dtype, p, L, K) in enumerate(CASES):
        say(f"case lh_forward_static N={N} H={H} d={d} {dtype} p={p} L={L} K={K}")
        x = si.make_inputs(N, H, d, dtype, seed=1500 + i, threads=8)
        q, k, v = (to_dev(x[n], dtype) for n in ("q", "k", "v"))
        o_st = lh.forward_static(q, k, v, p, L, K)
        o_ref, _ = lh.forward(q, k, v, p, L, K)
        torch.cuda.synchronize()
        same = torch.equal(o_st.view(torch.int16), o_ref.view(torch.int16)) if dtype == "bf16" \
            else torch.equal(o_st, o_ref)
        assert same, f"lh_forward_static differs from lh_forward (case {i})"


def test_forward_static_rejects_a_shape_beyond_its_array():
    import hierarchical_selection_attention_amd as lh
    q = torch.zeros((98304, 16, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lh.LighthouseError, match="static array"):
        lh.forward_static(q, q, q, 4, 4, 128)
