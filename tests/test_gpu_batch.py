"""Batched canvases (dg_denoise_step_batch, GPU).

Several users' canvases, each with its own KV cache, seed and step counter,
stepped in one call ([P5] current limitations: per-user denoising passes).
Every canvas must end each step in exactly the state the single-canvas step
gives it (bit for bit: tokens, probabilities, statistics, entropies,
argmax, accept mask, status), which carries the single step's parity with
the oracle over; a lock-step run also checks the batch against the oracle
directly (entropy within 2e-3 nats, decisions replayed bit-exactly).
"""
import numpy as np
import pytest
import torch

import oracle
from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D
from uniform_state_discrete_dg_amd import workloads as W
from parity_util import rel_frob, replay_select

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.empty_cache()


def prefixes(c, inp, nb):
    """Canvas b's prefix K/V: the workload's own for b = 0, then shorter
    prefixes with values of their own (seeded normal, like the workload's)."""
    out = [(inp["k_prefix"], inp["v_prefix"])]
    g = torch.Generator().manual_seed(9100 + c["N"])
    for b in range(1, nb):
        L = max(1, c["L"] - 37 * b)
        shape = (c["Hkv"], L, c["hd"])
        k = torch.randn(shape, generator=g)
        v = torch.randn(shape, generator=g)
        if c["dtype"] == "bf16":
            k, v = k.bfloat16().float(), v.bfloat16().float()
        out.append((k, v))
    return out


class Batch:
    """nb canvases stepped by the batched call, and a twin of each stepped
    by dg_denoise_step with its own workspace."""

    def __init__(self, c, inp, nb, candidate_rule=B.DG_CANDIDATE_ARGMAX, sampler=B.DG_SAMPLER_UNIFORM):
        self.c = c
        self.cfg = B.make_config(c, candidate_rule=candidate_rule, sampler=sampler)
        self.w = B.DeviceWeights(self.cfg, inp)
        self.pre = prefixes(c, inp, nb)
        self.caches = [B.DeviceCache(self.cfg, max(k.shape[1], 1), "cuda", k, v) for k, v in self.pre]
        self.cv = [B.DeviceCanvas(self.cfg) for _ in range(nb)]
        self.twin = [B.DeviceCanvas(self.cfg) for _ in range(nb)]
        self.ws = torch.empty(B.dg_workspace_bytes_batch(self.cfg, nb), dtype=torch.uint8, device="cuda")
        self.ws1 = B.workspace(self.cfg)
        self.seeds = [W.canvas_seed(c.get("id", 0)) + 17 * b for b in range(nb)]

    def init(self):
        for b, (x, y) in enumerate(zip(self.cv, self.twin)):
            B.dg_canvas_init(self.cfg, x.s, self.seeds[b], 3 * b + 1)
            B.dg_canvas_init(self.cfg, y.s, self.seeds[b], 3 * b + 1)

    def step(self, T, gamma):
        B.dg_denoise_step_batch(self.cfg, self.w.s, [k.s for k in self.caches], [x.s for x in self.cv],
                                T, gamma, self.ws)
        for y, k in zip(self.twin, self.caches):
            B.dg_denoise_step(self.cfg, self.w.s, k.s, y.s, T, gamma, self.ws1)
        torch.cuda.synchronize()

    def assert_equal(self, tag):
        for b, (x, y) in enumerate(zip(self.cv, self.twin)):
            for name in ("tokens", "probs", "stats", "entropy", "argmax", "accept", "status"):
                assert torch.equal(getattr(x, name), getattr(y, name)), (tag, b, name)
            assert (x.s.step, x.s.has_prev) == (y.s.step, y.s.has_prev), (tag, b)


def run_equal(c, inp, nb, nsteps, **kw):
    bt = Batch(c, inp, nb, **kw)
    bt.init()
    for s in range(nsteps):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        bt.step(T, c["gamma"])
        bt.assert_equal(s)
    return bt


@pytest.mark.parametrize("case", ["cfg2_n256_b3", "cfg2_n256_b1", "n128_b3", "n128_b2", "ragged_n100_b4",
                                  "ragged_n200_b2", "cfg1_f32_b3", "n16_b16_max"])
def test_batch_equals_single_steps(case):
    """N = 256 (one row block per canvas), N <= 128 (two canvases share a
    256-row block in both table-streaming contractions; an odd count leaves
    the last block half its own padding), N = 200 (canvases straddle the LM
    head's row blocks), and the fp32 configuration (canvas after canvas)."""
    if case == "cfg2_n256_b3":
        c, nb = W.config(2), 3
    elif case == "cfg2_n256_b1":
        c, nb = W.config(2), 1
    elif case == "n128_b3":
        c, nb = W.config(2, N=128, V=16384), 3
    elif case == "n128_b2":
        c, nb = W.config(2, N=128, V=16384), 2
    elif case == "n16_b16_max":  # the largest batch the library takes
        c, nb = W.config(2, N=16, L=40, V=8192, d=1024, F=1024), B.DG_MAX_BATCH
    elif case == "ragged_n100_b4":
        c, nb = W.config(2, N=100, L=60, V=8192, d=1024, F=1024), 4
    elif case == "ragged_n200_b2":
        c, nb = W.config(2, N=200, L=100, V=8192, d=1024, F=1024), 2
    else:
        c, nb = W.config(1), 3
    run_equal(c, W.make_inputs(c, seed=W.weight_seed(2) + len(case)), nb, 3)


def test_batch_canvases_at_different_steps():
    """Canvases that joined at different times: canvas b has run b + 1
    single steps before the batch takes over (its own step counter feeds its
    Philox counters and, under the multinomial rule, its draws); the batch
    must still match each canvas's single-step twin bit for bit."""
    c = W.config(2, V=16384)
    inp = W.make_inputs(c, seed=5151)
    bt = Batch(c, inp, 3, candidate_rule=B.DG_CANDIDATE_MULTINOMIAL)
    bt.init()
    for b in range(3):
        for s in range(b + 1):
            T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
            for cv in (bt.cv[b], bt.twin[b]):
                B.dg_denoise_step(bt.cfg, bt.w.s, bt.caches[b].s, cv.s, T, c["gamma"], bt.ws1)
    torch.cuda.synchronize()
    bt.assert_equal("joined")
    assert [x.s.step for x in bt.cv] == [1, 2, 3]
    for s in range(3, 6):
        bt.step(D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"]), c["gamma"])
        bt.assert_equal(s)
    assert [x.s.step for x in bt.cv] == [4, 5, 6]


def test_batch_multinomial_and_masked_equal_single():
    c = W.config(2, V=16384)
    inp = W.make_inputs(c, seed=4242)
    run_equal(c, inp, 2, 3, candidate_rule=B.DG_CANDIDATE_MULTINOMIAL)
    run_equal(c, inp, 2, 3, sampler=B.DG_SAMPLER_MASKED)


@pytest.mark.parametrize("cfg_id,nb", [(3, 2), (4, 3)])
def test_batch_full_vocab_equal_single(cfg_id, nb):
    """V = 262144, d = 2816, GQA 16/8: the large-vocabulary canvas (N = 256)
    and the latency-sensitive one (N = 128, prefix 4096, canvases paired in
    the contractions), canvases with different prefixes, two steps (the
    second self-conditioned)."""
    c = W.config(cfg_id)
    run_equal(c, W.make_inputs(c), nb, 2)


def test_batch_oracle_lockstep():
    """Each canvas of a batch against the oracle run on its own cache: every
    entropy within 2e-3 nats, probabilities within 1e-2 relative Frobenius,
    the selection replayed bit-exactly on the GPU's entropies."""
    c = W.config(2)
    inp = W.make_inputs(c)
    nb = 2
    bt = Batch(c, inp, nb)
    bt.init()
    om = oracle.model_from_inputs(inp)
    caches = []
    for k, v in bt.pre:
        caches.append((k.double().numpy(), v.double().numpy(), k.shape[1]))
    p_prev = [None] * nb
    stable = [0] * nb
    for s in range(3):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        tok_in = [x.tokens.cpu().numpy() for x in bt.cv]
        bt.step(T, c["gamma"])
        bt.assert_equal(s)
        for b in range(nb):
            kc, vc, L = caches[b]
            o = om.denoise_forward(tok_in[b], p_prev[b], kc, vc, L, float(np.float32(T)))
            H = bt.cv[b].entropy.cpu().numpy()
            assert np.max(np.abs(H - o["entropy"])) <= 2e-3, (s, b)

            class _D:  # the replay helper reads a Denoiser's canvas and config
                cfg = bt.cfg
                canvas = bt.cv[b]
            fl = replay_select(_D, tok_in[b], stable[b], s, c["gamma"], 0)
            stable[b] = fl["stable"]
            p = bt.cv[b].probabilities(bt.cfg).float()
            a, pa = bt.cv[b].top(bt.cfg)
            p[torch.arange(c["N"], device=p.device), a.long()] = pa
            assert rel_frob(p.cpu().double().numpy(), o["probs"]) <= 1e-2, (s, b)
            p_prev[b] = o["probs"]
