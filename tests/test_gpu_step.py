"""Whole-step parity of dg_denoise_step / dg_prefill_append (GPU) against the
oracle, lock-step: each step the oracle is given the canvas the GPU produced
(integer state already verified by the replay of the previous step) and its
own previous-step probabilities.

Floats: fp32 configuration <= 1e-4 relative Frobenius; bf16 configurations
<= 1e-2 on logits and attention output, <= 2e-3 nats on every entropy.
Decisions (accept set, re-noised tokens, flags): bit-exact when the oracle
replays the selection on the GPU's entropy vector and argmax.
"""
import numpy as np
import pytest
import torch

import oracle
from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D
from uniform_state_discrete_dg_amd import workloads as W
from parity_util import (CONF_EPS_F32, check_argmax, gpu_probs, oracle_cache, rel_frob,
                         replay_select, ws_view)

pytestmark = pytest.mark.gpu


@pytest.fixture
def logits_dump():
    """The bf16 path writes its fp32 LM-head accumulators to the workspace."""
    B.dg_test_set_logits_dump(True)
    yield
    B.dg_test_set_logits_dump(False)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.empty_cache()


def lockstep(c, inp, nsteps, rule=0, seed=None, cid=0, masked=False, stop=False):
    """Runs nsteps GPU steps and checks each against the oracle (all rows);
    masked: the masked-diffusion sampler ([MASK] = id V); stop: after every
    step the library's adaptive-stop test (dg_should_stop, c["stable_n"])
    must agree with the oracle's on the replayed flags, and the loop ends
    when it fires."""
    f32 = c["dtype"] == "f32"
    tol = 1e-4 if f32 else 1e-2
    den = D.Denoiser(c, inp, accept_rule=rule, logits_dump=True,
                     sampler=B.DG_SAMPLER_MASKED if masked else B.DG_SAMPLER_UNIFORM)
    om = oracle.model_from_inputs(inp)
    kc, vc = oracle_cache(inp)
    N, V, d, qw = c["N"], c["V"], c["d"], c["Hq"] * c["hd"]
    seed = W.canvas_seed(c.get("id", 0)) if seed is None else seed
    den.init_canvas(seed, cid)
    np.testing.assert_array_equal(den.canvas.tokens.cpu().numpy(),
                                  oracle.canvas_init(seed, cid, N, V, masked=masked))
    p_prev = None
    stable = 0
    report = []
    for s in range(nsteps):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        assert abs(T - oracle.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])) < 1e-12
        tokens_in = den.canvas.tokens.cpu().numpy()
        den.step(T, c["gamma"])
        torch.cuda.synchronize()
        o = om.denoise_forward(tokens_in, p_prev, kc, vc, c["L"], float(np.float32(T)))
        h0 = ws_view(den, "h0", torch.float32, (N, d)).cpu().numpy()
        h1 = ws_view(den, "h1", torch.float32, (N, d)).cpu().numpy()
        attn = ws_view(den, "attn", torch.float32, (N, qw)).cpu().numpy()
        z = ws_view(den, "logits", torch.float32, (N, V)).cpu().numpy()
        H = den.canvas.entropy.cpu().numpy()
        am = den.canvas.argmax.cpu().numpy()
        errs = dict(h0=rel_frob(h0, o["h0"]), attn=rel_frob(attn, o["attn"]),
                    h1=rel_frob(h1, o["h1"]), logits=rel_frob(z, o["logits"]),
                    probs=rel_frob(gpu_probs(den), o["probs"]),
                    dH=float(np.max(np.abs(H - o["entropy"]))))
        report.append(errs)
        for k in ("h0", "attn", "h1", "logits", "probs"):
            assert errs[k] <= tol, (s, k, errs)
        if f32:
            assert rel_frob(H, o["entropy"]) <= 1e-4, (s, errs)
        else:
            assert errs["dH"] <= 2e-3, (s, errs)
        # argmax: replayed on the GPU's own fp32 logits (exact), and against
        # the oracle's wherever the oracle's top-2 gap exceeds the float error
        for r in range(N):
            assert oracle.argmax(np.ascontiguousarray(z[r])) == am[r]
        gap = 1e-4 if f32 else 2e-2
        check_argmax(o["logits"], o["argmax"], am, range(N), gap)
        fl = replay_select(den, tokens_in, stable, s, c["gamma"], rule)
        stable = fl["stable"]
        p_prev = o["probs"]
        if stop:
            halt, st = den.should_stop(c["stable_n"])
            assert halt == oracle.should_stop(fl, c["stable_n"]), (s, fl)
            report[-1]["stop"] = halt
            if halt:
                break
    return den, report


@pytest.mark.usefixtures("logits_dump")
def test_config1_fp32_lockstep():
    c = W.config(1)
    inp = W.make_inputs(c)
    den, rep = lockstep(c, inp, c["steps"])
    print(rep)


@pytest.mark.usefixtures("logits_dump")
@pytest.mark.parametrize("shape", [
    dict(N=37, V=1024, d=96, Hq=6, Hkv=3, hd=32, F=200, L=45),     # ragged rows, columns and keys, GQA
    dict(N=70, V=2048, d=256, Hq=2, Hkv=1, hd=128, F=96, L=130),   # the largest fp32 head, MQA
])
def test_fp32_matrix_core_path_ragged_lockstep(shape):
    """The fp32 configuration's contractions and attention run on the fp32
    matrix cores (16x16x4 tiles); shapes that are multiples of none of the
    tile sizes, head dims 32 and 128, three steps in lock-step with the
    oracle at 1e-4."""
    c = W.config(1, **shape)
    lockstep(c, W.make_inputs(c, seed=19), 3)


def test_config1_fp32_independent_decisions():
    """fp32 config: the oracle's own decisions equal the GPU's when no two
    entropies (or a prefix sum and the threshold) are within float error."""
    c = W.config(1)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp)
    om = oracle.model_from_inputs(inp)
    kc, vc = oracle_cache(inp)
    seed = W.canvas_seed(1)
    den.init_canvas(seed, 0)
    tok_o = oracle.canvas_init(seed, 0, c["N"], c["V"])
    p_prev, stable = None, 0
    for s in range(c["steps"]):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        den.step(T, c["gamma"])
        o = om.denoise_forward(tok_o, p_prev, kc, vc, c["L"], T)
        Hs = np.sort(o["entropy"])
        sums = np.concatenate([[0.0], np.cumsum(Hs)])
        if np.min(np.diff(Hs)) < 1e-5 or np.min(np.abs(sums - c["gamma"])) < 1e-5:
            pytest.skip("near-tie in the oracle's entropies")
        acc, tok_o, fl = oracle.select(o["entropy"].astype(np.float32), o["argmax"], tok_o, c["V"],
                                       c["gamma"], 0, seed, 0, s, stable, CONF_EPS_F32)
        stable = fl["stable"]
        p_prev = o["probs"]
        np.testing.assert_array_equal(den.canvas.accept.cpu().numpy(), acc)
        np.testing.assert_array_equal(den.canvas.tokens.cpu().numpy(), tok_o)


@pytest.mark.usefixtures("logits_dump")
@pytest.mark.parametrize("rule", [0, 1])
def test_config2_bf16_lockstep(rule):
    c = W.config(2)
    inp = W.make_inputs(c)
    den, rep = lockstep(c, inp, 3, rule=rule)
    print(rep)


@pytest.mark.usefixtures("logits_dump")
def test_config2_bf16_lockstep_full_budget_adaptive_stop():
    """Configuration 2 over its whole 16-step budget (cosine 1.5 -> 0.3), every
    step in lock-step with the oracle, with the adaptive stop (all entropies
    below 0.005, or the predictions stable for 3 steps) tested after each
    step against the oracle's decision on the replayed flags."""
    c = W.config(2)
    den, rep = lockstep(c, W.make_inputs(c), c["steps"], stop=True)
    print(len(rep), "steps;", rep[-1])


@pytest.mark.usefixtures("logits_dump")
def test_config1_fp32_masked_sampler_lockstep():
    c = W.config(1)
    den, rep = lockstep(c, W.make_inputs(c), c["steps"], masked=True)
    tok = den.canvas.tokens.cpu().numpy()
    assert (tok == c["V"]).sum() < c["N"]        # some positions decided, and locked


@pytest.mark.usefixtures("logits_dump")
def test_config2_bf16_masked_sampler_lockstep():
    c = W.config(2)
    lockstep(c, W.make_inputs(c), 3, masked=True)


@pytest.mark.usefixtures("logits_dump")
def test_config2_bf16_lockstep_low_temperature():
    """T = 0.05: peaked rows whose tiles sit hundreds of nats below the row
    maximum, so the self-conditioning contraction's power-of-two tile
    exponents span the whole uint8 range (including the cap that flushes a
    tile to zero) at steps 1 and 2."""
    c = W.config(2, sched="const", T0=0.05, T1=0.05)
    inp = W.make_inputs(c)
    den, rep = lockstep(c, inp, 3)
    shift = den.canvas.exponents(den.cfg)
    assert int(shift.max()) == 255 and int(shift.min()) == 0, (int(shift.min()), int(shift.max()))
    print(rep)


@pytest.mark.usefixtures("logits_dump")
def test_config3_dims_reduced_vocab_lockstep():
    """Config-3 model dims (d 2816, GQA 16/8, F 2816, L 2048, N 256) with a
    16384-token vocabulary so the oracle finishes in seconds."""
    c = W.config(3, V=16384)
    inp = W.make_inputs(c, seed=W.weight_seed(3))
    den, rep = lockstep(c, inp, 2)
    print(rep)


@pytest.mark.usefixtures("logits_dump")
def test_ragged_canvas_lockstep():
    """A canvas that is not a multiple of any tile (N = 200, 40 rows past the
    last 32-row block), short prefix not a multiple of 64."""
    c = W.config(2, N=200, L=100, V=8192, d=1024, F=1024)
    inp = W.make_inputs(c, seed=77)
    den, rep = lockstep(c, inp, 2)
    print(rep)


@pytest.mark.usefixtures("logits_dump")
@pytest.mark.parametrize("table", ["bf16", "fp8", "fp4"])
def test_partial_column_tile_lockstep(table):
    """A model width that is not a multiple of 256 (d = 320 = 10 column
    blocks of 32): the self-conditioning contraction's last 256-column tile
    reads E transposed with 6 of its 8 column blocks past the table (their
    reads clamped, their columns never stored); lock-step against the oracle
    over three steps (two self-conditioned), in each table form (the
    quantised ones on their grids)."""
    c = W.config(2, N=96, V=4096, d=320, F=448, Hq=4, Hkv=2, L=130)
    if table != "bf16":
        c = dict(c, table=table, table_exp=8 if table == "fp8" else 0)
    inp = W.make_inputs(c, seed=91)
    den, rep = lockstep(c, inp, 3)
    print(rep)


@pytest.mark.usefixtures("logits_dump")
@pytest.mark.parametrize("cfg_id", [3, 4])
def test_full_size_step_sampled(cfg_id):
    """Full vocabulary (262144) at the configuration's canvas and prefix:
    first step checked on sampled rows (attention keys use every row), then
    three more self-conditioned steps checked by decision replay and by the
    argmax replay on the logits dump."""
    c = W.config(cfg_id)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, logits_dump=True)
    om = oracle.model_from_inputs(inp)
    kc, vc = oracle_cache(inp)
    N, V, d = c["N"], c["V"], c["d"]
    seed = W.canvas_seed(cfg_id)
    den.init_canvas(seed, 0)
    rows = sorted({0, 1, N // 3, N // 2 + 1, N - 1})
    sel = np.zeros(N, np.uint8)
    sel[rows] = 1
    stable = 0
    for s in range(4):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        tokens_in = den.canvas.tokens.cpu().numpy()
        den.step(T, c["gamma"])
        torch.cuda.synchronize()
        zg = ws_view(den, "logits", torch.float32, (N, V))
        am = den.canvas.argmax.cpu().numpy()
        zr = zg[rows].cpu().numpy()
        for k, r in enumerate(rows):
            assert oracle.argmax(np.ascontiguousarray(zr[k])) == am[r]
        if s == 0:
            o = om.denoise_forward(tokens_in, None, kc, vc, c["L"], float(np.float32(T)),
                                   row_sel=sel, want_probs=False)
            qw = c["Hq"] * c["hd"]
            attn = ws_view(den, "attn", torch.float32, (N, qw)).cpu().numpy()
            h1 = ws_view(den, "h1", torch.float32, (N, d)).cpu().numpy()
            h0 = ws_view(den, "h0", torch.float32, (N, d)).cpu().numpy()
            assert rel_frob(h0, o["h0"]) == 0.0  # embedding rows are exact
            assert rel_frob(attn[rows], o["attn"][rows]) <= 1e-2
            assert rel_frob(h1[rows], o["h1"][rows]) <= 1e-2
            assert rel_frob(zr, o["logits"][rows]) <= 1e-2
            H = den.canvas.entropy.cpu().numpy()
            assert np.max(np.abs(H[rows] - o["entropy"][rows])) <= 2e-3
            check_argmax([o["logits"][r] for r in rows], o["argmax"], am, rows, 2e-2)
        fl = replay_select(den, tokens_in, stable, s, c["gamma"], 0)
        stable = fl["stable"]


def multinomial_steps(c, inp, nsteps, cid=5, den=None):
    """Steps under the multinomial candidate rule ([P3] §5.3): each step's
    candidates equal the oracle's two-level Gumbel-max draw replayed on the
    step's own tile statistics and stored weights, bit for bit, and the
    selection replays on them.  Returns the number of rows whose candidate
    differs from the argmax."""
    den = den or D.Denoiser(c, inp, candidate_rule=B.DG_CANDIDATE_MULTINOMIAL)
    cfg = den.cfg
    N = c["N"]
    seed = W.canvas_seed(c.get("id", 0))
    den.init_canvas(seed, cid)
    stable, differ = 0, 0
    for s in range(nsteps):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        tokens_in = den.canvas.tokens.cpu().numpy()
        den.step(T, c["gamma"])
        torch.cuda.synchronize()
        zmax, l, _, tcol = (t.cpu().numpy() for t in den.canvas.tile_stats(cfg))
        wgt = den.canvas.weights(cfg).cpu().numpy()
        inv_T = np.float32(1.0) / np.float32(T)
        cand = oracle.multinomial_candidates(zmax, l, wgt, inv_T, seed, s, cid, np.full(N, -1, np.int32))
        gpu = den.canvas.argmax.cpu().numpy()
        np.testing.assert_array_equal(gpu, cand, err_msg=f"step {s}")
        # the argmax from the same statistics (lowest column among equal maxima)
        for r in range(N):
            best = np.flatnonzero(zmax[r] == zmax[r].max())
            differ += int(cand[r] != tcol[r, best].min())
        fl = replay_select(den, tokens_in, stable, s, c["gamma"], 0)
        stable = fl["stable"]
    return differ


def test_config1_fp32_multinomial_draw_replays():
    c = W.config(1)
    differ = multinomial_steps(c, W.make_inputs(c), c["steps"])
    assert differ > c["N"]          # T = 1 over 512 tokens: the draw mostly differs from the argmax


def test_config2_bf16_multinomial_draw_replays():
    c = W.config(2)
    differ = multinomial_steps(c, W.make_inputs(c), 4)
    assert differ > 0


def test_masked_sampler_with_multinomial_draw_replays():
    """The two variants together (configuration 2): masked canvas, drawn candidates."""
    c = W.config(2)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, candidate_rule=B.DG_CANDIDATE_MULTINOMIAL, sampler=B.DG_SAMPLER_MASKED)
    multinomial_steps(c, inp, 4, den=den)
    assert int(den.canvas.status[B.DG_ST_MASKED]) < c["N"]


def test_full_size_multinomial_draw_replays():
    """V = 262144, d = 2816, 256 rows: two steps (the second self-conditioned)."""
    c = W.config(3)
    multinomial_steps(c, W.make_inputs(c), 2)


def test_determinism_bitwise():
    c = W.config(2)
    inp = W.make_inputs(c)
    outs = []
    for _ in range(2):
        den = D.Denoiser(c, inp)
        den.init_canvas(3, 1)
        for s in range(3):
            den.step(D.temperature("cosine", 1.5, 0.3, s, 16), 8.0)
        torch.cuda.synchronize()
        outs.append((den.canvas.entropy.clone(), den.canvas.probs.clone(),
                     den.canvas.tokens.clone(), den.canvas.stats.clone()))
        del den
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_cache_untouched_by_denoise():
    c = W.config(2)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, capacity=c["L"] + 64)
    k0, v0 = den.cache.k.clone(), den.cache.v.clone()
    den.init_canvas(1, 0)
    for s in range(2):
        den.step(1.0, 8.0)
    torch.cuda.synchronize()
    assert torch.equal(den.cache.k, k0) and torch.equal(den.cache.v, v0)
    assert den.cache.length == c["L"]


@pytest.mark.parametrize("dtype,masked", [("bf16", False), ("f32", False), ("bf16", True), ("f32hd64", False)])
def test_prefill_append_incremental(dtype, masked):
    """Causal prefill of 300 tokens then 77 more (ragged), against the oracle;
    masked: the masked sampler's [MASK] id V among them reads its own row."""
    if dtype == "bf16":
        c = W.config(2, L=0, V=8192, d=1024, F=1024, Hq=8, Hkv=4)
    elif dtype == "f32hd64":
        c = W.config(1, L=0, d=128, Hq=4, Hkv=2, hd=64)
    else:
        c = W.config(1, L=0)
    cap = 400
    inp = W.make_inputs(c, seed=11)
    den = D.Denoiser(c, inp, capacity=cap, max_prefill=300,
                     sampler=B.DG_SAMPLER_MASKED if masked else B.DG_SAMPLER_UNIFORM)
    om = oracle.model_from_inputs(inp)
    Hkv, hd, qw = c["Hkv"], c["hd"], c["Hq"] * c["hd"]
    kc, vc = np.zeros((Hkv, cap, hd)), np.zeros((Hkv, cap, hd))
    g = torch.Generator().manual_seed(5)
    toks = torch.randint(0, c["V"], (377,), generator=g, dtype=torch.int32)
    if masked:
        toks[::7] = c["V"]
    tol = 1e-4
    L = 0
    for lo, hi in [(0, 300), (300, 377)]:
        n = hi - lo
        attn = torch.zeros((n, qw), dtype=torch.float32, device="cuda")
        den.prefill(toks[lo:hi].cuda(), attn)
        torch.cuda.synchronize()
        a_ref = om.prefill_append(toks[lo:hi].numpy(), kc, vc, L)
        L += n
        assert den.cache.length == L
        assert rel_frob(den.cache.k_f32()[:, :L].cpu().numpy(), kc[:, :L]) <= tol
        assert rel_frob(den.cache.v_f32()[:, :L].cpu().numpy(), vc[:, :L]) <= tol
        assert rel_frob(attn.float().cpu().numpy(), a_ref) <= tol
    assert not den.cache.k_f32()[:, L:].any()
    # keys/values of a token depend on the token only: a one-shot append, with no attention output
    # requested (the incremental one asked for it), is bitwise equal
    den2 = D.Denoiser(c, inp, capacity=cap, max_prefill=377, sampler=den.cfg.sampler)
    den2.prefill(toks.cuda())
    assert torch.equal(den2.cache.k, den.cache.k) and torch.equal(den2.cache.v, den.cache.v)
    # capacity overflow is rejected without touching the cache
    with pytest.raises(B.DgError) as e:
        den.prefill(toks[:cap].cuda())
    assert e.value.status == B.DG_ERR_CAPACITY and den.cache.length == L


def test_block_diffusion_reduced_vocab():
    """Block diffusion (prompt 1024, chained canvases of 256) at config-5 model
    dims with a 16384-token vocabulary: each step replayed bit-exactly, each
    finished canvas appended causally and checked against the oracle."""
    c = W.config(5, V=16384)
    inp = W.make_inputs(c, seed=W.weight_seed(5))
    cap = 1024 + 2 * 256
    den = D.Denoiser(c, inp, capacity=cap, max_prefill=1024)
    om = oracle.model_from_inputs(inp)
    Hkv, hd = c["Hkv"], c["hd"]
    kc, vc = np.zeros((Hkv, cap, hd)), np.zeros((Hkv, cap, hd))
    prompt = inp["prompt"]
    den.prefill(prompt.cuda())
    om.prefill_append(prompt.numpy(), kc, vc, 0, want_attn=False)
    seed = W.canvas_seed(5)
    for b in range(2):
        den.init_canvas(seed, b)
        stable = 0
        for s in range(2):
            T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
            tokens_in = den.canvas.tokens.cpu().numpy()
            den.step(T, c["gamma"])
            fl = replay_select(den, tokens_in, stable, s, c["gamma"], 0)
            stable = fl["stable"]
        L0 = den.cache.length
        fin = den.canvas.tokens.clone()
        den.prefill(fin)
        om.prefill_append(fin.cpu().numpy(), kc, vc, L0, want_attn=False)
        L1 = den.cache.length
        assert L1 == L0 + 256
        assert rel_frob(den.cache.k_f32()[:, :L1].cpu().numpy(), kc[:, :L1]) <= 1e-2
        assert rel_frob(den.cache.v_f32()[:, :L1].cpu().numpy(), vc[:, :L1]) <= 1e-2


def test_block_diffusion_full_size_short():
    """Config 5 at full size: prompt 1024 prefilled, one canvas of 256 for three
    steps (decisions replayed bit-exactly), appended (cache 1024 -> 1280)."""
    c = W.config(5)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, capacity=c["cap"], max_prefill=1024)
    den.prefill(inp["prompt"].cuda())
    assert den.cache.length == 1024
    den.init_canvas(W.canvas_seed(5), 0)
    stable = 0
    for s in range(3):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        tokens_in = den.canvas.tokens.cpu().numpy()
        den.step(T, c["gamma"])
        stable = replay_select(den, tokens_in, stable, s, c["gamma"], 0)["stable"]
    den.prefill(den.canvas.tokens.clone())
    assert den.cache.length == 1280


@pytest.mark.parametrize("cfg_id,stop", [(2, True), (2, False), (1, True)])
def test_run_canvas_native_matches_host_loop(cfg_id, stop):
    """dg_run_canvas (the loop inside the library, one status readback per
    step) gives the same canvas, step count and stop as the host loop of
    dg_denoise_step + dg_should_stop, bit for bit."""
    c = W.config(cfg_id)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp)
    seed = W.canvas_seed(cfg_id)
    steps = min(c["steps"], 12)
    a = den.run_canvas(seed, 3, steps, c["sched"], c["T0"], c["T1"], c["gamma"], stop, c["stable_n"])
    ent_a = den.canvas.entropy.clone()
    b = den.run_canvas_native(seed, 3, steps, c["sched"], c["T0"], c["T1"], c["gamma"], stop,
                              c["stable_n"])
    torch.cuda.synchronize()
    assert (a.steps, a.stop_reason) == (b.steps, b.stop_reason)
    assert torch.equal(a.tokens, b.tokens)
    assert torch.equal(ent_a, den.canvas.entropy)
    assert den.canvas.s.step == b.steps and den.canvas.s.has_prev == (1 if b.steps else 0)
    # a zero-step call only initialises the canvas
    n, stopped = B.dg_run_canvas(den.cfg, den.w.s, den.cache.s, den.canvas.s, seed, 4, [], c["gamma"],
                                 True, 3, den.ws)
    assert (n, stopped) == (0, False) and den.canvas.s.step == 0
    with pytest.raises(B.DgError) as e:
        B.dg_run_canvas(den.cfg, den.w.s, den.cache.s, den.canvas.s, seed, 4, [1.0, float("nan")],
                        c["gamma"], True, 3, den.ws)
    assert e.value.status == B.DG_ERR_INVALID_ARG


@pytest.mark.parametrize("cfg_id,budget", [(1, 40), (2, 400)])
def test_masked_sampler_runs_until_unmasked(cfg_id, budget):
    """Masked sampler ([P3] §3.1): the loop ends when no [MASK] is left, every
    position then holds a vocabulary token, and the library's loop equals the
    host loop bit for bit."""
    c = W.config(cfg_id)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, sampler=B.DG_SAMPLER_MASKED)
    seed = W.canvas_seed(cfg_id)
    a = den.run_canvas(seed, 2, budget, c["sched"], c["T0"], c["T1"], c["gamma"], True, 0)
    b = den.run_canvas_native(seed, 2, budget, c["sched"], c["T0"], c["T1"], c["gamma"], True, 0)
    torch.cuda.synchronize()
    assert (a.steps, a.stop_reason) == (b.steps, b.stop_reason)
    assert torch.equal(a.tokens, b.tokens)
    assert a.stop_reason in ("unmasked", "confident"), a.stop_reason
    assert int((b.tokens >= c["V"]).sum()) == 0 and int((b.tokens < 0).sum()) == 0
    assert int(den.canvas.status[B.DG_ST_MASKED]) == 0
    # masks only ever resolve: the per-step counts of the host loop never grow
    counts = [st.masked for st in a.stats]
    assert all(x >= y for x, y in zip(counts, counts[1:])) and counts[-1] == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multinomial_draw_law(dtype):
    """[P3] §5.3 logits scheduler: the candidate drawn at each position follows
    softmax(z / T) -- the law, not just the replay.  The canvas is held fixed
    (every step a first step, so the logits are fixed) while the step counter,
    which keys the draw's Philox counters, runs over K values; the K draws of
    each row are tested by chi-square against the probabilities the oracle
    computes from its own float64 logits (bins of expected count >= 5, the
    tail merged), and the same counts must reject the untempered softmax(z)."""
    from scipy import stats
    # temperatures at which the own-token logit the random-init model echoes
    # back does not swamp the row (a broad law, many chi-square bins)
    if dtype == "f32":
        c = W.config(1, sched="const", T0=1.5, T1=1.5)
    else:
        c = W.config(2, N=32, V=1024, d=256, Hq=2, Hkv=2, F=256, L=64, sched="const", T0=2.0, T1=2.0)
    inp = W.make_inputs(c, seed=404)
    den = D.Denoiser(c, inp, candidate_rule=B.DG_CANDIDATE_MULTINOMIAL)
    N, V, T = c["N"], c["V"], c["T0"]
    den.init_canvas(W.canvas_seed(1), 9)
    tok = den.canvas.tokens.clone()
    K = 4000
    draws = torch.empty((K, N), dtype=torch.int32, device="cuda")
    for k in range(K):
        den.canvas.tokens.copy_(tok)
        den.canvas.s.step, den.canvas.s.has_prev = k, 0
        den.step(T, c["gamma"])
        draws[k].copy_(den.canvas.argmax)
    torch.cuda.synchronize()
    d_np = draws.cpu().numpy()
    om = oracle.model_from_inputs(inp)
    kc, vc = oracle_cache(inp)
    o = om.denoise_forward(tok.cpu().numpy(), None, kc, vc, c["L"], T)
    o1 = om.denoise_forward(tok.cpu().numpy(), None, kc, vc, c["L"], 1.0)

    def chi2(probs):
        x2, dof = 0.0, 0
        for i in range(N):
            cnt = np.bincount(d_np[:, i], minlength=V).astype(np.float64)
            e = K * probs[i]
            order = np.argsort(-e)
            big = order[e[order] >= 5.0]
            rest = np.setdiff1d(np.arange(V), big)
            obs = list(cnt[big]) + ([cnt[rest].sum()] if rest.size else [])
            exp = list(e[big]) + ([e[rest].sum()] if rest.size else [])
            obs, exp = np.array(obs), np.array(exp)
            if exp.size < 2:
                continue
            x2 += float(((obs - exp) ** 2 / np.maximum(exp, 1e-300)).sum())
            dof += exp.size - 1
        return x2, dof

    x2, dof = chi2(o["probs"])
    p_val = stats.chi2.sf(x2, dof)
    assert p_val > 1e-4, (x2, dof, p_val)
    x2w, dofw = chi2(o1["probs"])
    assert stats.chi2.sf(x2w, dofw) < 1e-6, (x2w, dofw)
    # the draw differs from the argmax often: it is a draw
    assert (d_np != o["argmax"][None, :]).mean() > 0.2
    print(dtype, "chi2", x2, "dof", dof, "p", p_val)


def test_nan_weights_never_accepted_or_stop():
    """A NaN in the self-conditioning FFN's output weights (w_sc2): the first
    step is unaffected; from the first self-conditioned step every entropy is
    NaN, and then no position is accepted (every one is re-noised), none
    counts as confident, the stability counter stays 0 under both rules and
    the adaptive stop never fires; the decisions replay bit-exactly."""
    for srule in (B.DG_STABLE_PREDICTIONS, B.DG_STABLE_CANVAS):
        c = W.config(2, N=64, V=4096, d=512, Hq=4, Hkv=4, F=512, L=64, stable_rule=srule)
        inp = W.make_inputs(c, seed=31)
        inp["w2"] = inp["w2"].clone()
        inp["w2"][3, 7] = float("nan")
        den = D.Denoiser(c, inp)
        N = c["N"]
        den.init_canvas(5, 0)
        stable = 0
        for s in range(4):
            tok = den.canvas.tokens.cpu().numpy()
            den.step(1.0, 1e6)
            torch.cuda.synchronize()
            H = den.canvas.entropy.cpu().numpy()
            fl = replay_select(den, tok, stable, s, 1e6, 0)
            stable = fl["stable"]
            halt, st = den.should_stop(1)
            if s == 0:
                assert np.isfinite(H).all() and st.accepted == N
                continue
            assert np.isnan(H).all()
            assert st.accepted == 0 and st.allconf == 0 and st.stable == 0 and not halt
            assert int(den.canvas.status[B.DG_ST_NAN]) == N
            expect = [oracle.uniform_token(5, i, s, 0, 1, c["V"]) for i in range(N)]
            np.testing.assert_array_equal(den.canvas.tokens.cpu().numpy(), expect)
