"""Kernel-level parity of the HIP library against the oracle (GPU)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import workloads as W
from parity_util import CONF_EPS_F32, rel_frob

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_matches_oracle_and_kat():
    kat = json.load(open(os.path.join(GOLD, "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        ctr = torch.tensor([int(x, 16) for x in v["ctr"]], dtype=torch.int64).to(torch.int32).cuda()
        out = torch.zeros(4, dtype=torch.int32, device="cuda")
        k = [int(x, 16) for x in v["key"]]
        B.dg_test_philox(ctr, k[0], k[1], out, 1)
        got = [int(x) & 0xFFFFFFFF for x in out.cpu().tolist()]
        assert got == [int(x, 16) for x in v["out"]]
    rng = np.random.default_rng(0)
    n = 4096
    ctr = rng.integers(0, 2**32, (n, 4), dtype=np.uint64).astype(np.uint32)
    key = [int(x) for x in rng.integers(0, 2**32, 2, dtype=np.uint64)]
    out = torch.zeros(n * 4, dtype=torch.int32, device="cuda")
    B.dg_test_philox(torch.from_numpy(ctr.view(np.int32).copy()).cuda(), key[0], key[1], out, n)
    got = out.cpu().numpy().view(np.uint32).reshape(n, 4)
    for i in range(0, n, 97):
        np.testing.assert_array_equal(got[i], oracle.philox4x32_10(ctr[i], key))


def test_multinomial_pieces_bit_exact():
    """The multinomial draw's single-precision log and Gumbel transform on the
    device equal the oracle's bit for bit (random words and edge values)."""
    rng = np.random.default_rng(3)
    words = np.concatenate([rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32),
                            np.array([0, 1, 511, 512, 513, 2**31, 2**32 - 512, 2**32 - 1], np.uint32)])
    # positive normal floats for the log: random exponents and mantissas, plus edges
    xs = np.concatenate([
        (rng.integers(1, 255, 20000, dtype=np.uint64).astype(np.uint32) << 23)
        | rng.integers(0, 2**23, 20000, dtype=np.uint64).astype(np.uint32),
        np.array([1.0, 2.0, 0.5, 1.4142135, 1.4142137, 0.70710677, 1.1754944e-38, 3.4028235e38,
                  5.9604645e-8, 0.99999994, 16.635532], np.float32).view(np.uint32)])
    for mode, src in ((1, words), (0, xs)):
        n = src.size
        w = torch.from_numpy(src.view(np.int32).copy()).cuda()
        out = torch.zeros(n, dtype=torch.float32, device="cuda")
        B.dg_test_gumbel(w, n, mode, out)
        got = out.cpu().numpy()
        fn = oracle.gumbel_f32 if mode == 1 else (lambda b: oracle.ln_f32(np.uint32(b).view(np.float32)))
        ref = np.array([fn(int(b)) for b in src], np.float32)
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,V", [(16, 512), (128, 262144), (256, 32768)])
def test_canvas_init_matches_oracle(N, V):
    c = dict(N=N, V=V, d=1024, Hq=8, Hkv=8, hd=128, F=1024, dtype="bf16")
    cfg = B.make_config(c)
    cv = B.DeviceCanvas(cfg)
    for seed, cid in [(1, 0), (4, 7), (2**40 + 3, 123)]:
        B.dg_canvas_init(cfg, cv.s, seed, cid)
        np.testing.assert_array_equal(cv.tokens.cpu().numpy(), oracle.canvas_init(seed, cid, N, V))
        assert cv.s.step == 0 and cv.s.has_prev == 0
        assert int(cv.status[B.DG_ST_STABLE]) == 0 and int(cv.status[B.DG_ST_MASKED]) == -1
    # masked sampler: [MASK] (id V) everywhere, all N counted as masked
    cfg.sampler = B.DG_SAMPLER_MASKED
    B.dg_canvas_init(cfg, cv.s, 5, 1)
    np.testing.assert_array_equal(cv.tokens.cpu().numpy(), oracle.canvas_init(5, 1, N, V, masked=True))
    assert int(cv.status[B.DG_ST_MASKED]) == N


def _select_cases():
    rng = np.random.default_rng(1)
    for N in (1, 5, 16, 128, 255, 256):
        for kind in ("spread", "ties", "edge"):
            if kind == "spread":
                H = rng.random(N).astype(np.float32) * 12
            elif kind == "ties":
                H = (np.floor(rng.random(N) * 6) / 2).astype(np.float32)
            else:
                H = rng.random(N).astype(np.float32) * 3
                if N >= 5:
                    H[0] = np.nan
                    H[1] = -0.0
                    H[2] = -3.0
                    H[3] = np.inf
                    H[4] = 3e6
            yield N, H


def _set_predictions(cv, cfg, pred, prev):
    """Writes a step's predictions (top tokens) and the previous step's into
    the canvas's stats buffer, where the selection kernel reads them."""
    N = cfg.canvas_len
    o = B.stats_offsets(cfg)
    top = cv.stats[o["top"]:o["top"] + N * 8].view(torch.int32).view(N, 2)
    top[:, 0] = torch.from_numpy(pred).to(top.device)
    cv.pred_prev(cfg).copy_(torch.from_numpy(prev))


@pytest.mark.parametrize("rule,masked", [(0, False), (1, False), (0, True), (1, True)])
def test_select_kernel_bit_exact(rule, masked):
    """Selection kernel vs the oracle, bit-exact: uniform-state re-noise, and
    the masked sampler ([MASK] = id V at ~60% of the positions, the rest
    locked); both stability rules, predictions equal to or differing from the
    previous step's, step 0 (no previous predictions) included."""
    V = 32768
    c = dict(N=256, V=V, d=1024, Hq=8, Hkv=8, hd=128, F=1024, dtype="bf16")
    rng = np.random.default_rng(2 + rule + 4 * masked)
    for N, H in _select_cases():
        c["N"] = N
        for srule in (B.DG_STABLE_PREDICTIONS, B.DG_STABLE_CANVAS):
            cfg = B.make_config(c, accept_rule=rule, stable_rule=srule,
                                sampler=B.DG_SAMPLER_MASKED if masked else B.DG_SAMPLER_UNIFORM)
            cv = B.DeviceCanvas(cfg)
            am = rng.integers(0, V, N).astype(np.int32)
            tin = rng.integers(0, V, N).astype(np.int32)
            if masked:
                tin[rng.random(N) < 0.6] = V
            for gamma in (0.0, 0.75, 3.0, 16.0, 1e30):
                step, cid, seed, stable_in = int(rng.integers(0, 64)), int(rng.integers(0, 8)), 99, 2
                if gamma == 0.75:
                    step = 0
                pred = rng.integers(0, V, N).astype(np.int32)
                prev = pred.copy()
                if gamma in (3.0, 1e30):     # one position's prediction moved
                    prev[int(rng.integers(0, N))] ^= 1
                cv.entropy.copy_(torch.from_numpy(H))
                cv.argmax.copy_(torch.from_numpy(am))
                cv.tokens.copy_(torch.from_numpy(tin))
                _set_predictions(cv, cfg, pred, prev)
                cv.status.zero_()
                cv.status[B.DG_ST_STABLE] = stable_in
                cv.s.step, cv.s.canvas_id, cv.s.seed = step, cid, seed
                B.dg_test_select(cfg, cv.s, gamma)
                acc, tout, fl = oracle.select(H, am, tin, V, gamma, rule, seed, cid, step, stable_in,
                                              CONF_EPS_F32, mask_id=V if masked else -1, stable_rule=srule,
                                              pred=pred, pred_prev=None if step == 0 else prev)
                np.testing.assert_array_equal(cv.accept.cpu().numpy(), acc, err_msg=f"{N} {gamma}")
                np.testing.assert_array_equal(cv.tokens.cpu().numpy(), tout)
                st = cv.status.cpu().numpy()
                assert (st[B.DG_ST_ALLCONF], st[B.DG_ST_CHANGED], st[B.DG_ST_STABLE], st[B.DG_ST_ACCEPTED],
                        st[B.DG_ST_MASKED], st[B.DG_ST_PRED_CHANGED]) == (
                    fl["allconf"], fl["changed"], fl["stable"], fl["accepted"], fl["masked"], fl["pred_changed"])
                # the kernel keeps this step's predictions for the next comparison
                np.testing.assert_array_equal(cv.pred_prev(cfg).cpu().numpy(), pred)


def test_stop_on_stable_predictions_under_renoise():
    """[P3] §5.3 / [P5]: the predictions held fixed while only one position is
    accepted per step (the canvas keeps changing through re-noise): the
    prediction rule counts 1, 2, 3 and stops; the canvas rule never does."""
    V, N = 4096, 64
    c = dict(N=N, V=V, d=1024, Hq=8, Hkv=8, hd=128, F=1024, dtype="bf16")
    rng = np.random.default_rng(3)
    pred = rng.integers(0, V, N).astype(np.int32)
    for srule, want in ((B.DG_STABLE_PREDICTIONS, [0, 1, 2, 3]), (B.DG_STABLE_CANVAS, [0, 0, 0, 0])):
        cfg = B.make_config(c, stable_rule=srule)
        cv = B.DeviceCanvas(cfg)
        B.dg_canvas_init(cfg, cv.s, 5, 0)
        cv.entropy.fill_(1.0)
        for k in range(4):
            _set_predictions(cv, cfg, pred, cv.pred_prev(cfg).cpu().numpy())
            cv.argmax.copy_(torch.from_numpy(pred))
            cv.s.step = k
            B.dg_test_select(cfg, cv.s, 0.5)     # sum - max: exactly one accepted
            stop, st = B.dg_should_stop(cfg, cv.s, 3)
            assert st.accepted == 1 and st.changed == 1 and st.stable == want[k], (srule, k)
            assert stop == (want[k] >= 3)


def test_stop_flags_on_constructed_canvas():
    """All entropies 0 and argmax == canvas: unchanged, confident; the stable
    counter (canvas rule) counts up and dg_should_stop fires on either criterion."""
    V, N = 4096, 64
    c = dict(N=N, V=V, d=1024, Hq=8, Hkv=8, hd=128, F=1024, dtype="bf16")
    cfg = B.make_config(c, stable_rule=B.DG_STABLE_CANVAS)
    cv = B.DeviceCanvas(cfg)
    B.dg_canvas_init(cfg, cv.s, 5, 0)
    cv.argmax.copy_(cv.tokens)
    cv.entropy.fill_(0.01)  # confident at no position (>= 0.005)
    for k in range(1, 4):
        B.dg_test_select(cfg, cv.s, 1e30)
        stop, st = B.dg_should_stop(cfg, cv.s, 3)
        assert st.stable == k and st.changed == 0 and st.allconf == 0 and st.accepted == N
        assert stop == (k >= 3)
    cv.entropy.fill_(0.001)
    B.dg_test_select(cfg, cv.s, 0.0)  # only one accepted, the rest re-noised
    stop, st = B.dg_should_stop(cfg, cv.s, 0)
    assert st.allconf == 1 and stop and st.accepted == 1 and st.changed == 1


@pytest.mark.parametrize("cfg_id,N", [(2, 256), (3, 256), (4, 128)])
def test_selfcond_contraction(cfg_id, N):
    """S = P E at full vocabulary size through the production contraction
    (the instance the step runs, exponents 0), sampled rows against the
    oracle on the same bf16 probabilities: only the accumulation differs."""
    c = W.config(cfg_id)
    inp = W.make_inputs(c)
    cfg = B.make_config(c)
    w = B.DeviceWeights(cfg, inp)
    Pm = W.random_row_weights(N, c["V"], seed=7).to(torch.bfloat16)
    S = torch.zeros((N, c["d"]), dtype=torch.float32, device="cuda")
    ws = B.workspace(cfg, logits_dump=True)
    Pt = B.rows_to_tiled(Pm.cuda())
    B.dg_test_selfcond(cfg, w.s, Pt, S, ws)
    torch.cuda.synchronize()
    om = oracle.model_from_inputs(inp)
    Pf = Pm.float().numpy()
    rows = [0, 1, N // 2 + 3, N - 1]
    ref = np.stack([om.selfcond_row(Pf[r]) for r in rows])
    got = S.cpu().numpy()[rows]
    assert rel_frob(got, ref) <= 1e-4
    # determinism: a second run is bit-identical
    S2 = torch.zeros_like(S)
    B.dg_test_selfcond(cfg, w.s, Pt, S2, ws)
    assert torch.equal(S, S2)


def test_selfcond_one_hot_gathers_rows():
    """One-hot P: S = E[t] exactly (sum of one product, bf16 round trip)."""
    c = W.config(2)
    inp = W.make_inputs(c)
    cfg = B.make_config(c)
    w = B.DeviceWeights(cfg, inp)
    N, V = c["N"], c["V"]
    t = torch.randint(0, V, (N,), generator=torch.Generator().manual_seed(3))
    Pm = torch.zeros((N, V), dtype=torch.bfloat16)
    Pm[torch.arange(N), t] = 1.0
    S = torch.zeros((N, c["d"]), dtype=torch.float32, device="cuda")
    B.dg_test_selfcond(cfg, w.s, B.rows_to_tiled(Pm.cuda()), S, B.workspace(cfg, logits_dump=True))
    assert torch.equal(S.cpu(), inp["E"][t].float())


def test_copy_kernel():
    n = 1 << 20
    a = torch.randint(0, 1000, (n,), dtype=torch.int32, device="cuda")
    b = torch.zeros_like(a)
    B.dg_test_copy(a, b, n * 4)
    assert torch.equal(a, b)


@pytest.mark.parametrize("V,d", [(4096, 1024), (2048, 320)])
def test_bf16_pack_is_the_one_tiled_copy(V, d):
    """dg_pack_embedding (bf16): E_pack is E once in the documented tiled
    layout (the host formula of rows_to_tiled), nothing else; d = 320 leaves
    a partial set of 32-column slices per block row."""
    g = torch.Generator().manual_seed(21)
    E = (torch.randn(V, d, generator=g) * 0.05).to(torch.bfloat16)
    cfg = B.make_config(W.config(2, V=V, d=d))
    nb = B.dg_embedding_pack_bytes(cfg)
    assert nb == V * d * 2
    packed = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    B.dg_pack_embedding(cfg, E.cuda(), packed)
    torch.cuda.synchronize()
    got = packed.cpu().view(torch.bfloat16)
    assert torch.equal(got, B.rows_to_tiled(E))
    assert torch.equal(B.tiled_to_rows(got, V, d), E)
