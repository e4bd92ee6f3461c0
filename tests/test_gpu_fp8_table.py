"""The fp8 packed table (DG_TABLE_FP8, GPU).

The table the two streaming contractions read is stored as fp8 e4m3
q = E * 2^e and turned back into bf16 exactly, so on a table that lies on
that grid (the quantised-table inputs) the step must equal the bf16-table
step bit for bit, and the oracle, given the same table, within the bf16
tolerances.  The packed bytes are checked against torch's own e4m3
conversion placed in the 8-byte-chunk tiled layout.
"""
import numpy as np
import pytest
import torch

import oracle
from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D
from uniform_state_discrete_dg_amd import workloads as W
from parity_util import oracle_cache, rel_frob, replay_select
from test_gpu_step import lockstep

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.empty_cache()


@pytest.fixture
def logits_dump():
    B.dg_test_set_logits_dump(True)
    yield
    B.dg_test_set_logits_dump(False)


def tiled8_positions(R: int, K: int) -> torch.Tensor:
    """Byte index of X[r][k] in the fp8 tiled layout: blocks of 256 x 32,
    block (b, s) at (b * K/32 + s) * 8192, 8-byte chunk of row r and chunk c
    at slot 4 r + (c ^ w(r)), w(r) = (bit 2 xor bit 4 of r) + 2 bit 3 of r."""
    r = torch.arange(R).view(R, 1)
    k = torch.arange(K).view(1, K)
    b, rr, s, kk = r // 256, r % 256, k // 32, k % 32
    c = kk // 8
    w = (((rr >> 2) ^ (rr >> 4)) & 1) | (((rr >> 3) & 1) << 1)
    slot = rr * 4 + (c ^ w)
    return ((b * (K // 32) + s) * 1024 + slot) * 8 + kk % 8


@pytest.mark.parametrize("exp", [8, 5])
def test_pack_bytes_match_torch_e4m3(exp):
    """dg_pack_embedding (fp8): the one packed copy byte-exact against
    torch's float8_e4m3fn of E * 2^exp (saturated at 448) in the tiled
    layout, for a table on the grid and one that is not (rounding to
    nearest even)."""
    V, d = 4096, 1024
    g = torch.Generator().manual_seed(11)
    E = (torch.randn(V, d, generator=g) * 0.08).to(torch.bfloat16)
    E[0, :8] = torch.tensor([1e4, -1e4, 0.0, -0.0, 1e-9, 448 * 2.0 ** -exp, 465 * 2.0 ** -exp, 3e-3])
    c = W.config(2, V=V, d=d, table="fp8", table_exp=exp)
    cfg = B.make_config(c)
    packed = torch.zeros(B.dg_embedding_pack_bytes(cfg), dtype=torch.uint8, device="cuda")
    B.dg_pack_embedding(cfg, E.cuda(), packed)
    torch.cuda.synchronize()
    got = packed.cpu()
    q = (E.float() * 2.0 ** exp).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    want = torch.zeros(V * d, dtype=torch.uint8)
    want[tiled8_positions(V, d).reshape(-1)] = q.reshape(-1)
    assert torch.equal(got, want)


def step_outputs(c, inp, nsteps, table):
    """Runs nsteps steps with the given table format; returns every canvas
    buffer after each step."""
    c = dict(c, table=table, table_exp=8)
    den = D.Denoiser(c, inp)
    den.init_canvas(W.canvas_seed(c.get("id", 0)), 0)
    out = []
    for s in range(nsteps):
        den.step(D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"]), c["gamma"])
        torch.cuda.synchronize()
        cv = den.canvas
        out.append({k: getattr(cv, k).clone() for k in ("tokens", "probs", "stats", "entropy", "argmax",
                                                          "accept", "status")})
    return out


@pytest.mark.parametrize("cfg_id,V", [(2, 32768), (3, 16384), (4, 16384)])
def test_fp8_table_equals_bf16_table_bitwise(cfg_id, V):
    """On a table that lies on the fp8 grid, the fp8-table step and the
    bf16-table step are the same computation: every canvas buffer equal bit
    for bit over three steps (the second and third self-conditioned)."""
    c = W.config(cfg_id, V=V, table="fp8", table_exp=8)
    inp = W.make_inputs(c)
    a = step_outputs(c, inp, 3, "bf16")
    b = step_outputs(c, inp, 3, "fp8")
    for s, (x, y) in enumerate(zip(a, b)):
        for k in x:
            assert torch.equal(x[k], y[k]), (s, k)


@pytest.mark.usefixtures("logits_dump")
def test_fp8_table_lockstep_oracle():
    """The bf16 configuration with a quantised table against the oracle given
    that table: logits, attention, probabilities within 1e-2 relative
    Frobenius, every entropy within 2e-3 nats, decisions replayed exactly."""
    c = W.config(2, table="fp8", table_exp=8)
    den, rep = lockstep(c, W.make_inputs(c), 3)
    print(rep)


@pytest.mark.usefixtures("logits_dump")
def test_fp8_table_full_vocab_sampled():
    """V = 262144, d = 2816 with a quantised table: the first step on sampled
    rows against the oracle, the next ones by decision replay."""
    c = W.config(3, table="fp8", table_exp=8)
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, logits_dump=True)
    om = oracle.model_from_inputs(inp)
    kc, vc = oracle_cache(inp)
    N, V = c["N"], c["V"]
    seed = W.canvas_seed(3)
    den.init_canvas(seed, 0)
    rows = [0, 7, N // 2, N - 1]
    sel = np.zeros(N, np.uint8)
    sel[rows] = 1
    stable = 0
    for s in range(3):
        T = D.temperature(c["sched"], c["T0"], c["T1"], s, c["steps"])
        tokens_in = den.canvas.tokens.cpu().numpy()
        den.step(T, c["gamma"])
        torch.cuda.synchronize()
        if s == 0:
            o = om.denoise_forward(tokens_in, None, kc, vc, c["L"], float(np.float32(T)), row_sel=sel,
                                   want_probs=False)
            off = B.dg_test_ws_offsets(den.cfg).logits
            z = den.ws[off:off + N * V * 4].view(torch.float32).view(N, V)[rows].cpu().numpy()
            assert rel_frob(z, o["logits"][rows]) <= 1e-2
            H = den.canvas.entropy.cpu().numpy()
            assert np.max(np.abs(H[rows] - o["entropy"][rows])) <= 2e-3
        fl = replay_select(den, tokens_in, stable, s, c["gamma"], 0)
        stable = fl["stable"]


def test_fp8_table_batch_equals_single():
    """Batched canvases on the fp8 table (256-token canvases one per block,
    128-token canvases paired) equal their single-canvas twins bit for bit."""
    from test_gpu_batch import run_equal
    for c, nb in ((W.config(2, V=16384, table="fp8", table_exp=8), 2),
                  (W.config(2, N=128, V=16384, table="fp8", table_exp=8), 3)):
        run_equal(c, W.make_inputs(c, seed=777), nb, 3)
