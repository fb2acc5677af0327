"""GPU parity of the alternative scores (lh_forward_scored; what the l2 score is
taken of, Sec. 1 and Fig. 2 of the Lighthouse paper's page) against the oracle:
scores of every level and the selection bit for bit, the layer's output and
gradients at the dtype's tolerance."""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_util import Run, check_full_rows, check_scores, check_selection, compare, grad_allow, say

pytestmark = pytest.mark.gpu

MODES = {"k": 1, "q": 2, "qk_product": 3}
# (label, N, H, d, dtype, p, L, K)
CASES = [("tiny_fp32", 2048, 2, 64, "fp32", 4, 3, 16),
         ("bf16_pool_up", 8192, 2, 128, "bf16", 4, 6, 4),
         ("fwd_n32768", 32768, 16, 128, "bf16", 4, 4, 64)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", list(MODES), ids=list(MODES))
def test_score_mode_parity(case, mode):
    label, N, H, d, dtype, p, L, K = case
    sm = MODES[mode]
    seed = 900 + 10 * CASES.index(case) + sm
    say(f"case {label} score_mode={mode} seed={seed}")
    x = si.make_inputs(N, H, d, dtype, seed=seed, with_dout=True, threads=8)
    ref = oracle.forward(x["q"], x["k"], x["v"], p, L, K, dtype, want=("levels", "sel", "ot"), score_mode=sm)
    run = Run(x, dtype, p, L, K, backward=True, label=label, score_mode=sm)
    check_scores(run, ref)
    check_selection(run, ref)
    b = oracle.backward(x["q"], x["k"], x["v"], x["dout"], p, L, K, (ref["start"], ref["level"]), dtype,
                        want=("sub", "cond"))
    compare(run.sub("osub"), ref["Ot"], dtype, "osub")
    sel = (ref["start"], ref["level"])
    rng = np.random.default_rng(seed)
    sample = None if N * H <= 65536 else 20000
    check_full_rows(run.o, ref["Ot"], sel, p, dtype, "o", sample=sample, rng=rng)
    for g, key in zip(run.grads, ("dQt", "dKt", "dVt")):
        check_full_rows(g, b[key], sel, p, dtype, "d" + key[1].lower(), divide=True, sample=sample, rng=rng,
                        allow_sub=grad_allow(b, key))

