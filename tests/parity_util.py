"""Shared helpers of the GPU parity tests: lock-step comparison of the HIP
path (through the C ABI) with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D

CONF_EPS_F32 = float(np.float32(0.005))  # the decision is taken on float32 values


def rel_frob(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def ws_view(den: D.Denoiser, name: str, dtype, shape):
    off = getattr(B.dg_test_ws_offsets(den.cfg), name)
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    return den.ws[off:off + n].view(dtype).view(*shape)


def gpu_probs(den: D.Denoiser) -> np.ndarray:
    cfg = den.cfg
    N = cfg.canvas_len
    p = den.canvas.probabilities(cfg).float().clone()
    if cfg.dtype == B.DG_BF16:  # the dominant token's probability is kept exactly
        a, pa = den.canvas.top(cfg)
        p[torch.arange(N, device=p.device), a.long()] = pa
    return p.cpu().double().numpy()


def oracle_cache(inp: dict, cap: int | None = None):
    kp = inp["k_prefix"].double().numpy()
    vp = inp["v_prefix"].double().numpy()
    Hkv, L, hd = kp.shape
    cap = L if cap is None else cap
    kc = np.zeros((Hkv, max(cap, 1), hd))
    vc = np.zeros((Hkv, max(cap, 1), hd))
    kc[:, :L] = kp
    vc[:, :L] = vp
    return kc, vc


def check_argmax(z_oracle_rows, am_oracle, am_gpu, rows, gap_tol):
    """The argmax is unique unless two logits are within the float error; a
    mismatch is allowed only where the oracle's own gap is below gap_tol."""
    mism = 0
    for r, zr in zip(rows, z_oracle_rows):
        if am_oracle[r] != am_gpu[r]:
            gap = abs(zr[am_oracle[r]] - zr[am_gpu[r]])
            assert gap <= gap_tol, (r, am_oracle[r], am_gpu[r], gap)
            mism += 1
    return mism


def replay_select(den: D.Denoiser, tokens_in, stable_in, step, gamma, rule):
    """Oracle selection on the GPU's own entropies, candidates and
    predictions: must be bit-exact.  The previous step's predictions are the
    ones this helper saw at the canvas's previous step (call it for every
    step of a canvas, from step 0)."""
    cfg = den.cfg
    H = den.canvas.entropy.cpu().numpy()
    am = den.canvas.argmax.cpu().numpy()
    pred = den.canvas.predictions(cfg).cpu().numpy()
    prev = None if step == 0 else den.canvas.replay_pred
    assert step == 0 or prev is not None, "replay every step of the canvas from step 0"
    mask_id = cfg.vocab if cfg.sampler == B.DG_SAMPLER_MASKED else -1
    acc, tout, fl = oracle.select(H, am, tokens_in, cfg.vocab, gamma, rule, den.canvas.s.seed,
                                  den.canvas.s.canvas_id, step, stable_in, CONF_EPS_F32, mask_id=mask_id,
                                  stable_rule=cfg.stable_rule, pred=pred, pred_prev=prev)
    den.canvas.replay_pred = pred
    st = den.canvas.status.cpu().numpy()
    assert st[B.DG_ST_PRED_CHANGED] == fl["pred_changed"]
    np.testing.assert_array_equal(den.canvas.accept.cpu().numpy(), acc)
    np.testing.assert_array_equal(den.canvas.tokens.cpu().numpy(), tout)
    assert st[B.DG_ST_ALLCONF] == fl["allconf"]
    assert st[B.DG_ST_CHANGED] == fl["changed"]
    assert st[B.DG_ST_STABLE] == fl["stable"]
    assert st[B.DG_ST_ACCEPTED] == fl["accepted"]
    assert st[B.DG_ST_MASKED] == fl["masked"]
    return fl
