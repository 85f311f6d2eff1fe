"""GPU parity of the fixed-latent probe (Fig. 13b) and of the per-step log
normaliser output (the draft distribution a T=1 walk samples from).

Probe, int8 W: tokens and logits bit-identical to the oracle's probe, in
every execution mode.  Log normaliser: within LSE_RTOL of the float64
normaliser of the logits the same walk returned; asking for it changes no
token or logit.
"""
import numpy as np
import pytest

import datagen
from gpu_helpers import (make_head, run, oracle_walk, assert_exact, assert_bf16_close,
                         assert_lse_close)
from conftest import cached_inputs

pytestmark = pytest.mark.gpu


def _print_case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# ---- fixed-latent probe -------------------------------------------------------

@pytest.mark.parametrize("exec_", ["resident", "stream", "stepwise"])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 16])
@pytest.mark.parametrize("T", [0, 1])
def test_fixed_latent_markov_exact(exec_, B, T):
    d = datagen.make_inputs(4099, 256, B, 6, seed=31)
    _print_case(test="fixed_latent_markov", V=4099, B=B, T=T, exec=exec_)
    h, t = make_head(d)
    got = run(h, t, exec=exec_, temperature=T, seed=7, fixed_latent=True)
    assert_exact(got, oracle_walk(d, temperature=T, seed=7, fixed_latent=True), f"probe B={B} T={T} {exec_}")
    h.close()


def test_fixed_latent_headline_size_exact():
    # the headline workload: V = 151,936, B = 1, gamma = 16 (staged-candidate kernel)
    d = cached_inputs(1)
    _print_case(test="fixed_latent_headline", V=d["V"], B=1, gamma=16)
    h, t = make_head(d)
    got = run(h, t, fixed_latent=True)
    ref = oracle_walk(d, fixed_latent=True)
    assert_exact(got, ref, "probe headline")
    # the probe really holds the latent: the normal walk differs from it
    normal = run(h, t, logits=False)
    assert not np.array_equal(normal["tokens"], got["tokens"])
    h.close()


@pytest.mark.parametrize("B", [1, 4])
@pytest.mark.parametrize("T", [0, 1])
def test_fixed_latent_recurrent_exact(B, T):
    d = datagen.make_inputs(3001, 256, B, 5, head="recurrent", seed=32)
    _print_case(test="fixed_latent_recurrent", V=3001, B=B, T=T)
    h, t = make_head(d)
    got = run(h, t, temperature=T, seed=3, fixed_latent=True)
    assert_exact(got, oracle_walk(d, temperature=T, seed=3, fixed_latent=True), f"probe recurrent B={B}")
    h.close()


@pytest.mark.parametrize("exec_", ["resident", "stepwise"])
def test_fixed_latent_bf16_close(exec_):
    d = datagen.make_inputs(5000, 256, 2, 5, wtype="bf16", seed=33)
    _print_case(test="fixed_latent_bf16", V=5000, B=2, exec=exec_)
    h, t = make_head(d)
    got = run(h, t, exec=exec_, fixed_latent=True)
    assert_bf16_close(got, oracle_walk(d, keep_z=True, fixed_latent=True), f"probe bf16 {exec_}", d=d,
                      fixed_latent=True)
    h.close()


# ---- per-step log normaliser --------------------------------------------------

@pytest.mark.parametrize("exec_", ["resident", "stream", "stepwise"])
@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("T", [0, 1])
def test_lse_markov_int8(exec_, B, T):
    d = datagen.make_inputs(4099, 256, B, 5, seed=34)
    _print_case(test="lse_markov_int8", V=4099, B=B, T=T, exec=exec_)
    h, t = make_head(d)
    got = run(h, t, exec=exec_, temperature=T, seed=9, lse=True)
    ref = oracle_walk(d, temperature=T, seed=9, keep_lse=True)
    assert_exact(got, ref, f"lse walk B={B} T={T} {exec_}")
    assert_lse_close(got["lse"], got["logits"], f"lse B={B} T={T} {exec_}")
    h.close()


@pytest.mark.parametrize("V", [1, 15, 33, 260])
def test_lse_ragged_vocab(V):
    # fewer rows than workgroups: most workgroups contribute empty pairs
    d = datagen.make_inputs(V, 256, 3, 4, seed=35)
    _print_case(test="lse_ragged", V=V, B=3)
    h, t = make_head(d)
    for exec_ in ("resident", "stepwise"):
        got = run(h, t, exec=exec_, temperature=1, seed=1, lse=True)
        assert_exact(got, oracle_walk(d, temperature=1, seed=1), f"lse ragged V={V} {exec_}")
        assert_lse_close(got["lse"], got["logits"], f"lse ragged V={V} {exec_}")
    h.close()


@pytest.mark.parametrize("B", [1, 4, 16])
def test_lse_bf16(B):
    d = datagen.make_inputs(6007, 256, B, 4, wtype="bf16", seed=36)
    _print_case(test="lse_bf16", V=6007, B=B)
    h, t = make_head(d)
    got = run(h, t, temperature=1, seed=5, lse=True)
    assert_bf16_close(got, oracle_walk(d, temperature=1, seed=5, keep_z=True), f"lse bf16 B={B}", d=d,
                      temperature=1, seed=5)
    assert_lse_close(got["lse"], got["logits"], f"lse bf16 B={B}")
    h.close()


@pytest.mark.parametrize("B", [1, 4])
def test_lse_recurrent(B):
    d = datagen.make_inputs(3001, 256, B, 5, head="recurrent", seed=37)
    _print_case(test="lse_recurrent", V=3001, B=B)
    h, t = make_head(d)
    got = run(h, t, temperature=1, seed=2, lse=True)
    assert_exact(got, oracle_walk(d, temperature=1, seed=2), f"lse recurrent B={B}")
    assert_lse_close(got["lse"], got["logits"], f"lse recurrent B={B}")
    h.close()


@pytest.mark.parametrize("exec_", ["resident", "stepwise"])
def test_lse_full_size(exec_):
    # V = 151,936, B = 4, gamma = 16, T = 1: every (row, step) against the oracle's normaliser
    d = cached_inputs(2, B=4, gamma=16)
    _print_case(test="lse_full_size", V=d["V"], B=4, gamma=16, exec=exec_)
    h, t = make_head(d)
    got = run(h, t, exec=exec_, temperature=1, seed=0, lse=True)
    ref = oracle_walk(d, temperature=1, seed=0, keep_lse=True)
    assert_exact(got, ref, f"lse full {exec_}")
    err = np.abs(got["lse"].astype(np.float64) - ref["lse"])
    assert np.all(err <= 1e-5 * np.maximum(1.0, np.abs(ref["lse"]))), err.max()
    h.close()


def test_lse_walks_in_a_row():
    # the per-walk completion counter alternates with the walk parity: walks
    # with and without the output, and a step-wise walk, interleaved
    d = datagen.make_inputs(2053, 256, 2, 4, seed=38)
    _print_case(test="lse_in_a_row", V=2053, B=2)
    h, t = make_head(d)
    ref = oracle_walk(d, temperature=1, seed=4, keep_lse=True)
    for i, (lse, exec_) in enumerate([(True, "resident"), (True, "resident"), (False, "resident"),
                                      (True, "stepwise"), (True, "resident"), (False, "stepwise"),
                                      (True, "resident")]):
        got = run(h, t, exec=exec_, temperature=1, seed=4, lse=lse)
        assert_exact(got, ref, f"walk {i}")
        if lse:
            err = np.abs(got["lse"].astype(np.float64) - ref["lse"])
            assert np.all(err <= 1e-5 * np.maximum(1.0, np.abs(ref["lse"]))), (i, err.max())
    h.close()
