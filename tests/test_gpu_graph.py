"""The denoising step under HIP graph capture.

A step allocates nothing and synchronises nothing (its scratch is the
caller's workspace, or the library's own device array for
dg_denoise_step_static), so a caller can capture it into a graph and replay
it.  A replay re-runs the captured launches with their captured arguments
-- the step number and temperature included -- so each replay here starts
from the same saved canvas state and must give the eager step's results bit
for bit, with eager work and synchronisations between the replays.
"""
import pytest
import torch

from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D
from uniform_state_discrete_dg_amd import workloads as W

pytestmark = pytest.mark.gpu


def _state(cv):
    return [cv.tokens, cv.probs, cv.stats, cv.entropy, cv.argmax, cv.accept, cv.status]


@pytest.mark.parametrize("static", [False, True])
def test_captured_step_replays_bit_exact(static):
    c = W.config(2, V=16384)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp)
    den.init_canvas(5, 0)
    g_nats = c["gamma"]

    def step(T):
        if static:
            B.dg_denoise_step_static(den.cfg, den.w.s, den.cache.s, den.canvas.s, T, g_nats)
        else:
            den.step(T, g_nats)

    step(D.temperature(c["sched"], c["T0"], c["T1"], 0, c["steps"]))  # step 0: no self-conditioning
    torch.cuda.synchronize()
    saved = [t.clone() for t in _state(den.canvas)]
    host = (den.canvas.s.step, den.canvas.s.has_prev)

    def restore():
        for t, s in zip(_state(den.canvas), saved):
            t.copy_(s)
        den.canvas.s.step, den.canvas.s.has_prev = host
        torch.cuda.synchronize()

    T1 = D.temperature(c["sched"], c["T0"], c["T1"], 1, c["steps"])
    step(T1)  # the eager self-conditioned step
    torch.cuda.synchronize()
    ref = [t.clone() for t in _state(den.canvas)]
    host_after = (den.canvas.s.step, den.canvas.s.has_prev)
    assert not torch.equal(ref[0], saved[0]) or not torch.equal(ref[1], saved[1])

    restore()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(T1)
    assert (den.canvas.s.step, den.canvas.s.has_prev) == host_after  # host fields advance at capture
    for r in range(3):
        restore()
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(_state(den.canvas), ref)):
            assert torch.equal(a, b), (static, r, k)
        # the program's own eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        assert torch.isfinite(x.sum()).item()
    del graph, den
    torch.cuda.empty_cache()
