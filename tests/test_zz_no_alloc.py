"""dg_denoise_step_static: the step with the library's own device scratch
instead of a caller workspace (for callers that cannot allocate).  It must
give exactly what dg_denoise_step gives -- every canvas buffer bit for bit --
on two calls in a row, the second with a smaller input (the scratch keeps
the first call's contents), and reject a configuration whose scratch need
exceeds the array before doing anything."""
import pytest
import torch

from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D
from uniform_state_discrete_dg_amd import workloads as W

pytestmark = pytest.mark.gpu


def _state(cv):
    return [cv.tokens, cv.probs, cv.stats, cv.entropy, cv.argmax, cv.accept, cv.status]


@pytest.mark.parametrize("steps", [3])
def test_static_scratch_step_equals_workspace_step(steps):
    cases = [W.config(3), W.config(2, N=64, V=4096, L=100)]   # the second smaller than the first
    for c in cases:
        inp = W.make_inputs(c)
        den = D.Denoiser(c, inp)                  # workspace path
        cv2 = B.DeviceCanvas(den.cfg)             # same weights and cache, own canvas
        assert B.dg_workspace_bytes(den.cfg, 0) <= B.DG_STATIC_SCRATCH_BYTES
        den.init_canvas(7, 1)
        B.dg_canvas_init(den.cfg, cv2.s, 7, 1)
        for s in range(steps):
            T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
            den.step(T, c["gamma"])
            B.dg_denoise_step_static(den.cfg, den.w.s, den.cache.s, cv2.s, T, c["gamma"])
            torch.cuda.synchronize()
            for a, b in zip(_state(den.canvas), _state(cv2)):
                assert torch.equal(a, b), (c["name"], s)
            assert (cv2.s.step, cv2.s.has_prev) == (den.canvas.s.step, den.canvas.s.has_prev)
        del den, cv2
        torch.cuda.empty_cache()


def test_static_scratch_rejects_oversized_configuration():
    c = W.config(3, d=4096, F=65536)
    cfg = B.make_config(c)
    assert B.dg_validate_config(cfg) == B.DG_OK
    assert B.dg_workspace_bytes(cfg, 0) > B.DG_STATIC_SCRATCH_BYTES
    cv = B.DeviceCanvas(B.make_config(W.config(2)))
    w = B.dg_weights()
    with pytest.raises(B.DgError) as e:
        B.dg_denoise_step_static(cfg, w, B.dg_kv_cache(), cv.s, 1.0, 8.0)
    assert e.value.status == B.DG_ERR_WORKSPACE
