"""Seeded random sweep of small walks against the oracle, through the C ABI:
vocabulary sizes with ragged last tiles and workgroups, every batch size up to
16, short and long walks, both temperatures, both W types, both heads, every
execution mode and smaller grids, each drawn from a fixed seed so that a
failure names a reproducible case.  int8 W must match bit for bit; bf16 W
under the bf16 rule (logits within 1e-2, tokens equal but at near-ties)."""
import random

import numpy as np
import pytest

import datagen
from gpu_helpers import make_head, run, oracle_walk, assert_exact, assert_bf16_close

N_CASES = 48


def _draw(i):
    rng = random.Random(7919 * i + 17)
    head = "recurrent" if rng.random() < 0.25 else "markov"
    wtype = "bf16" if rng.random() < 0.35 else "int8"
    V = rng.choice([rng.randrange(1, 64), rng.randrange(64, 5000), rng.randrange(5000, 70000)])
    B = rng.randrange(1, 17)
    gamma = rng.randrange(1, 9)
    T = rng.randrange(2)
    modes = ["resident", "stream"] + (["stepwise"] if head == "markov" else [])
    exec_ = rng.choice(modes)
    grid = rng.choice([0, 0, 0, rng.randrange(1, 257)])
    return dict(head=head, wtype=wtype, V=V, B=B, gamma=gamma, T=T, exec=exec_, grid=grid,
                seed=rng.randrange(1 << 30), walk_seed=rng.randrange(1 << 62))


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_walk_matches_oracle(i):
    from serial_draft_head_persistent_amd import WtsError
    c = _draw(i)
    print("CASE", i, c, flush=True)
    d = datagen.make_inputs(c["V"], 256, c["B"], c["gamma"], wtype=c["wtype"], head=c["head"], seed=c["seed"])
    try:
        h, t = make_head(d, grid=c["grid"])
    except WtsError as e:                       # a grid over which some workgroup would own > 65,535 rows
        assert "UNSUPPORTED" in str(e) and c["grid"] > 0
        pytest.skip(f"grid {c['grid']} refused for V={c['V']}")
    try:
        h.plan(c["B"], exec=c["exec"], temperature=c["T"])
    except WtsError as e:                       # T=1 noise of a small grid that does not fit LDS
        assert "UNSUPPORTED" in str(e)
        h.close()
        pytest.skip("plan refused: " + str(e))
    got = run(h, t, temperature=c["T"], seed=c["walk_seed"], exec=c["exec"])
    ref = oracle_walk(d, temperature=c["T"], seed=c["walk_seed"], keep_z=c["wtype"] == "bf16")
    if c["wtype"] == "int8":
        assert_exact(got, ref, f"case {i}")
    else:
        assert_bf16_close(got, ref, f"case {i}", d=d, temperature=c["T"], seed=c["walk_seed"],
                          max_total=c["B"])
    h.close()


def test_sweep_draws_cover_the_space():
    cases = [_draw(i) for i in range(N_CASES)]
    assert {c["head"] for c in cases} == {"markov", "recurrent"}
    assert {c["wtype"] for c in cases} == {"int8", "bf16"}
    assert {c["exec"] for c in cases} == {"resident", "stream", "stepwise"}
    assert {c["T"] for c in cases} == {0, 1}
    assert any(c["V"] < 64 for c in cases) and any(c["V"] >= 5000 for c in cases)
    assert any(c["grid"] > 0 for c in cases)
    assert any(c["B"] > 8 for c in cases) and any(c["B"] == 1 or c["B"] % 2 for c in cases)
