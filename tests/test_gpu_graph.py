"""Walks captured once in a HIP graph and replayed (the step-wise baseline
under graph replay is the analogue of the serving engine's graph replay,
Fig. 3b).  Between replays the inputs change and eager walks run; every
replay must give the eager walk's bits for its inputs."""
import numpy as np
import pytest

import datagen
from gpu_helpers import make_head

pytestmark = pytest.mark.gpu


def _case(**kw):
    print("CASE", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _host(o):
    import torch
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy().copy() for k, v in o.items()}


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("exec_,head", [("resident", "markov"), ("stepwise", "markov"), ("stream", "markov"),
                                        ("resident", "recurrent")])
def test_graph_replays_match_eager(exec_, head, noalloc):
    import torch
    _case(test="graph_replay", exec=exec_, head=head, noalloc=noalloc)
    sets = [datagen.make_inputs(20011, 256, 3, 6, head=head, seed=120 + i) for i in range(3)]
    # one head (W, E, A, c of the first set); the later sets contribute base, x0, h0
    h, t = make_head(sets[0])
    dev = t["base"].device
    bases = [torch.from_numpy(s["base"].view(np.int16)).view(torch.bfloat16).to(dev) for s in sets]
    x0s = [torch.from_numpy(s["x0"].astype(np.int32)).to(dev) for s in sets]
    h0s = [torch.from_numpy(s["h0"]).to(dev) if head == "recurrent" else None for s in sets]
    kw = dict(exec=exec_, temperature=1, seed=4, logits=True, lse=True, noalloc=noalloc,
              state=head == "recurrent")

    def eager(i):
        o = h.walk(bases[i], x0s[i], h0=h0s[i], **kw)
        torch.cuda.synchronize()
        assert h.error() == "WTS_OK"
        return _host(o)

    refs = [eager(i) for i in range(3)]
    sb, sx = bases[0].clone(), x0s[0].clone()
    sh = h0s[0].clone() if head == "recurrent" else None
    out = h.walk(sb, sx, h0=sh, **kw)          # buffers the graph writes
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.walk(sb, sx, h0=sh, out=out, **kw)   # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.walk(sb, sx, h0=sh, out=out, **kw)
    torch.cuda.synchronize()
    for rep in range(6):
        i = (rep + 1) % 3
        sb.copy_(bases[i])
        sx.copy_(x0s[i])
        if sh is not None:
            sh.copy_(h0s[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert h.error() == "WTS_OK"
        got = _host(out)
        for k in refs[i]:
            assert np.array_equal(got[k], refs[i][k]), f"replay {rep} (inputs {i}): {k} differs"
        # eager work between replays, on the same control block
        e = eager((i + 1) % 3)
        for k in refs[0]:
            assert np.array_equal(e[k], refs[(i + 1) % 3][k]), f"eager after replay {rep}: {k} differs"
    del g
    h.close()
