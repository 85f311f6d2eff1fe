"""Host logic of the GPU comparisons, run on the CPU: the bf16 token rule
(accept a different token only at an oracle near-tie, at most once per row,
then compare the rest of the walk against the oracle continued from the
GPU's token).  The "GPU" outputs here are the oracle's own with planted
differences."""
import numpy as np
import pytest

import datagen
import oracle
from oracle.fp import bf16_rne
from gpu_helpers import assert_bf16_close


def _tie_inputs():
    # E = 0: every latent is zero, so the logits are the base logits; step 1
    # has two equal maxima (rows 5 and 9), step 3 a unique maximum far above
    # the rest
    d = datagen.make_inputs(16, 8, 2, 5, wtype="bf16", seed=61)
    d["E"][:] = 0
    d["base"][:] = bf16_rne(np.float32(-1.0))
    for t in range(5):
        d["base"][:, t, t + 2] = bf16_rne(np.float32(1.0))
    d["base"][0, 1, 5] = d["base"][0, 1, 9] = bf16_rne(np.float32(3.0))
    d["base"][:, 3, 11] = bf16_rne(np.float32(8.0))
    return d


def _ref(d):
    return oracle.walk(d["W"], d["E"], d["base"], d["x0"], wtype="bf16", keep_z=True)


def test_near_tie_swap_accepted_once_and_rest_compared():
    d = _tie_inputs()
    ref = _ref(d)
    assert ref["tokens"][0, 1] == 5
    got = {"tokens": ref["tokens"].copy(), "logits": ref["logits"].copy()}
    got["tokens"][0, 1] = 9                       # the other of two equal maxima
    assert assert_bf16_close(got, ref, "tie", d=d) == 1


def test_swap_without_near_tie_rejected():
    d = _tie_inputs()
    ref = _ref(d)
    got = {"tokens": ref["tokens"].copy(), "logits": ref["logits"].copy()}
    got["tokens"][1, 3] = 2                       # 8.0 against 1.0: no near-tie
    with pytest.raises(AssertionError, match="gap"):
        assert_bf16_close(got, ref, "far", d=d)


def test_second_near_tie_in_a_row_rejected():
    d = _tie_inputs()
    d["base"][0, 4, 6] = d["base"][0, 4, 7] = bf16_rne(np.float32(3.0))
    ref = _ref(d)
    got = {"tokens": ref["tokens"].copy(), "logits": ref["logits"].copy()}
    got["tokens"][0, 1] = 9
    got["tokens"][0, 4] = 7
    with pytest.raises(AssertionError, match="second accepted"):
        assert_bf16_close(got, ref, "twice", d=d)


def test_logit_outside_tolerance_rejected():
    d = _tie_inputs()
    ref = _ref(d)
    got = {"tokens": ref["tokens"].copy(), "logits": ref["logits"].copy()}
    got["logits"][1, 2, 0] = bf16_rne(np.float32(-1.5))   # -1.5 against -1.0
    with pytest.raises(AssertionError, match="rel err"):
        assert_bf16_close(got, ref, "logit", d=d)


def test_continuation_follows_the_gpu_token():
    # Markov head with real embeddings: row `alt` is a copy of the step-1
    # winner x1 (same W row and base logits, so they tie exactly) with its own
    # embedding row, so a walk that takes `alt` at step 1 goes elsewhere.  A
    # "GPU" walk that takes `alt` and then follows the oracle restarted from
    # it passes; one that keeps the original walk's later tokens does not.
    d = datagen.make_inputs(64, 8, 1, 6, wtype="bf16", seed=62)
    x1 = int(_ref(d)["tokens"][0, 1])
    alt = 63 if x1 != 63 else 62
    d["W"][alt] = d["W"][x1]
    d["base"][:, :, alt] = d["base"][:, :, x1]
    if alt < x1:
        x1, alt = alt, x1
    ref = _ref(d)
    assert ref["tokens"][0, 1] == x1
    cont = oracle.walk(d["W"], d["E"], d["base"][:, 2:], np.array([alt], np.int32), wtype="bf16", keep_z=True,
                       step_offset=2)
    assert not np.array_equal(cont["tokens"], ref["tokens"][:, 2:])
    got = {"tokens": np.concatenate([ref["tokens"][:, :1], [[alt]], cont["tokens"]], 1),
           "logits": np.concatenate([ref["logits"][:, :2], cont["logits"]], 1)}
    assert assert_bf16_close(got, ref, "continued", d=d) == 1
    stale = {"tokens": got["tokens"].copy(), "logits": got["logits"]}
    stale["tokens"][:, 2:] = ref["tokens"][:, 2:]
    with pytest.raises(AssertionError):
        assert_bf16_close(stale, ref, "not continued", d=d)
