"""The element-wise surface bounds of tests/harness.py, on the CPU: they hold for a pipeline
that accumulates in fp32 and stores in bf16 (torch's CPU bf16 -> fp32 products), and a planted
mistake in such a result (a shifted column, another expert's weight, a wrong scale block, a
dropped K slice) fails them.  The mistakes are planted in the simulated result, never in the
oracle."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe_oracle as O
from tests import harness as Hn

BF = W.MIXTRAL_BF16.with_(T=64, H=512, I=384, N=2)
F8 = W.DEEPSEEKV3_FP8.with_(T=64, H=512, I=384, N=2)


def _pipeline(x_bf, w13_bf, w2_bf):
    """fp32 accumulation, bf16 stores: W13 output, activation, W2 output."""
    I = w13_bf.shape[0] // 2
    u = x_bf.float() @ w13_bf.float().T
    a = (torch.nn.functional.silu(u[:, :I]) * u[:, I:]).to(torch.bfloat16)
    y = (a.float() @ w2_bf.float().T).to(torch.bfloat16)
    return u.to(torch.bfloat16), a, y


def _inputs(w, e=0):
    x = W.hidden_states(w)
    if w.expert_dtype == W.FP8:
        q13, s13 = W.expert_weight(w, "w13", e)
        q2, s2 = W.expert_weight(w, "w2", e)
        d13 = O.dequantize_blocks(q13.numpy(), s13.double().numpy(), 128)
        d2 = O.dequantize_blocks(q2.numpy(), s2.double().numpy(), 128)
        w13_bf = torch.from_numpy(O.round_bf16(d13)).to(torch.bfloat16)
        w2_bf = torch.from_numpy(O.round_bf16(d2)).to(torch.bfloat16)
        return x, w13_bf, w2_bf, d13, d2
    w13 = W.expert_weight(w, "w13", e)
    w2 = W.expert_weight(w, "w2", e)
    return x, w13, w2, Hn.f64(w13), Hn.f64(w2)


@pytest.mark.parametrize("w", [BF, F8], ids=["bf16", "fp8"])
def test_bounds_hold_for_an_fp32_accumulating_bf16_pipeline(w):
    x, w13_bf, w2_bf, w13_exact, w2_exact = _inputs(w)
    u, a, y = _pipeline(x, w13_bf, w2_bf)
    xs = Hn.f64(x)
    lines = []
    Hn.check_expert_rows(w, xs, np.zeros(w.T, np.int64), lambda e: w13_exact, lambda e: w2_exact, Hn.f64(a),
                         Hn.f64(y), got_w13=Hn.f64(u), say=lines.append)
    # the bounds are not vacuous: the measured errors use a visible share of them
    worst = [float(t.split()[-1]) for t in lines[0].split(":")[1].split(",")]
    assert all(0.02 < v <= 1.0 for v in worst), lines


def _expect_fail(fn):
    with pytest.raises(AssertionError):
        fn()


@pytest.mark.parametrize("w", [BF, F8], ids=["bf16", "fp8"])
def test_bounds_catch_planted_mistakes(w):
    x, w13_bf, w2_bf, w13_exact, w2_exact = _inputs(w)
    xs = Hn.f64(x)
    W13 = Hn.effective_weights(w, lambda e: w13_exact)(0)
    W2 = Hn.effective_weights(w, lambda e: w2_exact)(0)
    u, a, y = _pipeline(x, w13_bf, w2_bf)
    I = w.I
    # W13 output with two columns swapped
    bad = Hn.f64(u).copy()
    bad[:, [5, 6]] = bad[:, [6, 5]]
    _expect_fail(lambda: Hn.check_product_surface(w, bad, xs, W13))
    # another expert's weights
    _, w13_other, w2_other, _, _ = _inputs(w, e=1)
    u1, a1, y1 = _pipeline(x, w13_other, w2_bf)
    _expect_fail(lambda: Hn.check_product_surface(w, Hn.f64(u1), xs, W13))
    _expect_fail(lambda: Hn.check_activation_surface(w, Hn.f64(a1), xs, W13))
    # gate and up halves exchanged
    sw = torch.cat([w13_bf[I:], w13_bf[:I]])
    _, a_sw, _ = _pipeline(x, sw, w2_bf)
    _expect_fail(lambda: Hn.check_activation_surface(w, Hn.f64(a_sw), xs, W13))
    # the last 128-wide K slice left out of the W2 product
    a32 = a.float()
    y_short = (a32[:, :-128] @ w2_bf.float()[:, :-128].T).to(torch.bfloat16)
    _expect_fail(lambda: Hn.check_product_surface(w, Hn.f64(y_short), Hn.f64(a), W2))
    if w.expert_dtype == W.FP8:
        # one 128 x 128 weight block with its neighbour's scale
        q2, s2 = W.expert_weight(w, "w2", 0)
        s_bad = s2.clone()
        s_bad[0, 0] = s2[0, 1]
        d_bad = O.round_bf16(O.dequantize_blocks(q2.numpy(), s_bad.double().numpy(), 128))
        y_bad = (a.float() @ torch.from_numpy(d_bad).float().T).to(torch.bfloat16)
        if not torch.equal(s2[0, 0], s2[0, 1]):
            _expect_fail(lambda: Hn.check_product_surface(w, Hn.f64(y_bad), Hn.f64(a), W2))
