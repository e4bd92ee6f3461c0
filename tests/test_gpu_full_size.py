"""Float parity at the full vocabulary (V = 262144, d = 2816, GQA 16/8 x 128)
for the step the benchmark times: the self-conditioned step.

The oracle runs its own first step over every canvas row (its probabilities
feed its self-conditioning), then the second step; the GPU runs the same two
steps through dg_denoise_step.  Compared on every row where the oracle has
them cheaply (h0, the first step's entropies and probabilities) and on
sampled rows otherwise (attention output, h1, logits, entropy, the
self-conditioning vector).  Tolerances: 1e-2 relative Frobenius on floats,
2e-3 nats on entropies; decisions replayed bit-exactly.  Each test runs the
oracle for 0.5-1.5 minutes on the host.
"""
import numpy as np
import pytest
import torch

import oracle
from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D
from uniform_state_discrete_dg_amd import workloads as W
from parity_util import check_argmax, gpu_probs, oracle_cache, rel_frob, replay_select, ws_view

pytestmark = pytest.mark.gpu


@pytest.fixture
def logits_dump():
    B.dg_test_set_logits_dump(True)
    yield
    B.dg_test_set_logits_dump(False)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.empty_cache()


def _compare_rows(den, o, rows, c, tag):
    """attention output, h1, logits (dump), entropy, argmax of the sampled rows."""
    N, V, d, qw = c["N"], c["V"], c["d"], c["Hq"] * c["hd"]
    attn = ws_view(den, "attn", torch.float32, (N, qw)).cpu().numpy()
    h1 = ws_view(den, "h1", torch.float32, (N, d)).cpu().numpy()
    zr = ws_view(den, "logits", torch.float32, (N, V))[rows].cpu().numpy()
    H = den.canvas.entropy.cpu().numpy()
    am = den.canvas.argmax.cpu().numpy()
    errs = dict(attn=rel_frob(attn[rows], o["attn"][rows]), h1=rel_frob(h1[rows], o["h1"][rows]),
                logits=rel_frob(zr, o["logits"][rows]),
                dH=float(np.max(np.abs(H[rows] - o["entropy"][rows]))))
    for k in ("attn", "h1", "logits"):
        assert errs[k] <= 1e-2, (tag, k, errs)
    assert errs["dH"] <= 2e-3, (tag, errs)
    for k, r in enumerate(rows):   # the argmax replayed on the GPU's own logits
        assert oracle.argmax(np.ascontiguousarray(zr[k])) == am[r]
    check_argmax([o["logits"][r] for r in rows], o["argmax"], am, rows, 2e-2)
    return errs


@pytest.mark.usefixtures("logits_dump")
@pytest.mark.parametrize("cfg_id,lowT", [(3, False), (4, False), (4, True)])
def test_full_size_selfcond_step(cfg_id, lowT):
    """Steps 0 and 1 of a canvas at the configuration's full shapes (lowT:
    a constant temperature of 0.05, so that tiles sit hundreds of nats below
    their row's maximum and the power-of-two tile exponents reach their cap
    of 255).  Checks: step 0 entropies and probabilities on every row; the
    kept state's self-conditioning vector (dg_test_selfcond_canvas, the
    production contraction with exponents, row factors and the dominant-token
    correction) against the oracle's contraction of the GPU's kept
    probabilities (1e-4) and of the oracle's own (1e-2); step 1's h0 on every
    row and its attention output, h1, logits and entropies on sampled rows;
    both steps' decisions replayed."""
    c = W.config(cfg_id, sched="const", T0=0.05, T1=0.05) if lowT else W.config(cfg_id)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, logits_dump=True)
    om = oracle.model_from_inputs(inp)
    kc, vc = oracle_cache(inp)
    N, d = c["N"], c["d"]
    rows = sorted({0, 1, N // 3, N // 2 + 1, N - 2, N - 1})
    sel = np.zeros(N, np.uint8)
    sel[rows] = 1
    den.init_canvas(W.canvas_seed(cfg_id), 0)

    # step 0 (no self-conditioning): the oracle over every row
    T0 = D.temperature(c["sched"], c["T0"], c["T1"], 0, c["steps"])
    tok0 = den.canvas.tokens.cpu().numpy()
    den.step(T0, c["gamma"])
    torch.cuda.synchronize()
    o0 = om.denoise_forward(tok0, None, kc, vc, c["L"], float(np.float32(T0)), want_logits=False)
    H0 = den.canvas.entropy.cpu().numpy()
    assert np.max(np.abs(H0 - o0["entropy"])) <= 2e-3
    pg = gpu_probs(den)
    assert rel_frob(pg, o0["probs"]) <= 1e-2
    stable = replay_select(den, tok0, 0, 0, c["gamma"], 0)["stable"]

    # the self-conditioning vector the next step will use, from the kept state
    S = torch.empty((N, d), dtype=torch.float32, device="cuda")
    B.dg_test_selfcond_canvas(den.cfg, den.w.s, den.canvas.s, S, den.ws)
    torch.cuda.synchronize()
    Sg = S.cpu().numpy()
    S_kept = np.stack([om.selfcond_row(pg[r]) for r in rows])
    S_orc = np.stack([om.selfcond_row(o0["probs"][r]) for r in rows])
    assert rel_frob(Sg[rows], S_kept) <= 1e-4
    assert rel_frob(Sg[rows], S_orc) <= 1e-2
    ex = den.canvas.exponents(den.cfg).cpu().numpy()
    if lowT:
        assert (ex[:, rows] == 255).any(), int(ex[:, rows].max())
    del pg

    # step 1 (self-conditioned), the oracle fed its own step-0 probabilities
    T1 = D.temperature(c["sched"], c["T0"], c["T1"], 1, c["steps"])
    tok1 = den.canvas.tokens.cpu().numpy()
    den.step(T1, c["gamma"])
    torch.cuda.synchronize()
    assert torch.equal(ws_view(den, "selfcond", torch.float32, (N, d)), S)  # the step used that vector
    o1 = om.denoise_forward(tok1, o0["probs"], kc, vc, c["L"], float(np.float32(T1)), row_sel=sel,
                            want_probs=False)
    h0 = ws_view(den, "h0", torch.float32, (N, d)).cpu().numpy()
    assert rel_frob(h0, o1["h0"]) <= 1e-2
    errs = _compare_rows(den, o1, rows, c, "step 1")
    replay_select(den, tok1, stable, 1, c["gamma"], 0)
    print(cfg_id, lowT, errs, "h0", rel_frob(h0, o1["h0"]))


@pytest.mark.usefixtures("logits_dump")
def test_block_diffusion_full_size_floats():
    """Configuration 5 at full size: the 1024-token prompt prefilled causally
    (keys/values of every position and the causal attention output against
    the oracle's own prefill), then step 0 of the first canvas over that cache
    on sampled rows, two more steps replayed, and the canvas appended (its
    256 keys/values against the oracle's append of the same tokens)."""
    c = W.config(5)
    inp = W.make_inputs(c)
    P = c["prompt"]
    den = D.Denoiser(c, inp, capacity=c["cap"], max_prefill=P, logits_dump=True)
    om = oracle.model_from_inputs(inp)
    Hkv, hd, qw, N = c["Hkv"], c["hd"], c["Hq"] * c["hd"], c["N"]
    cap = c["cap"]
    kc, vc = np.zeros((Hkv, cap, hd)), np.zeros((Hkv, cap, hd))
    prompt = inp["prompt"]
    attn = torch.zeros((P, qw), dtype=torch.float32, device="cuda")
    den.prefill(prompt.cuda(), attn)
    torch.cuda.synchronize()
    a_ref = om.prefill_append(prompt.numpy(), kc, vc, 0)
    assert rel_frob(den.cache.k_f32()[:, :P].cpu().numpy(), kc[:, :P]) <= 1e-4
    assert rel_frob(den.cache.v_f32()[:, :P].cpu().numpy(), vc[:, :P]) <= 1e-4
    assert rel_frob(attn.cpu().numpy(), a_ref) <= 1e-4
    rows = sorted({0, 5, N // 2, N - 1})
    sel = np.zeros(N, np.uint8)
    sel[rows] = 1
    den.init_canvas(W.canvas_seed(5), 0)
    stable = 0
    for s in range(3):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        tok = den.canvas.tokens.cpu().numpy()
        den.step(T, c["gamma"])
        torch.cuda.synchronize()
        if s == 0:
            o = om.denoise_forward(tok, None, kc, vc, P, float(np.float32(T)), row_sel=sel, want_probs=False)
            h0 = ws_view(den, "h0", torch.float32, (N, c["d"])).cpu().numpy()
            assert rel_frob(h0, o["h0"]) == 0.0     # embedding rows are exact
            _compare_rows(den, o, rows, c, "canvas 0 step 0")
        stable = replay_select(den, tok, stable, s, c["gamma"], 0)["stable"]
    fin = den.canvas.tokens.clone()
    den.prefill(fin)
    torch.cuda.synchronize()
    om.prefill_append(fin.cpu().numpy(), kc, vc, P, want_attn=False)
    L1 = P + N
    assert den.cache.length == L1
    assert rel_frob(den.cache.k_f32()[:, P:L1].cpu().numpy(), kc[:, P:L1]) <= 1e-4
    assert rel_frob(den.cache.v_f32()[:, P:L1].cpu().numpy(), vc[:, P:L1]) <= 1e-4
