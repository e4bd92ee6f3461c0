"""The block-scaled fp4 packed table (DG_TABLE_FP4, GPU).

The table the two streaming contractions read is stored as e2m1 codes with
one power-of-two scale byte per 32 x 32 block and turned back into bf16
exactly, so on a table that lies on that grid (the fp4-table inputs) the
step must equal the bf16-table step bit for bit, and the oracle, given the
same table, within the bf16 tolerances.  The packed codes and scale bytes
are checked against the host quantiser of the inputs (round to nearest,
ties to the even code) placed in the 4-byte-chunk tiled layout.
"""
import numpy as np
import pytest
import torch

import oracle
from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import driver as D
from uniform_state_discrete_dg_amd import workloads as W
from parity_util import oracle_cache, rel_frob, replay_select
from test_gpu_fp8_table import step_outputs
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


def packed_fp4(X: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """X [R][K] (R a multiple of 32) in the fp4 tiled layout: the code bytes
    (blocks of 256 x 32 at (b * K/32 + s) * 4096; block row r stored as row
    q = r with bits 3 and 4 swapped, the 4 bytes of its columns 8c .. 8c + 7
    at unit 4 q + 2 ((c % 2) xor (bit 3 xor bit 4 of q)) + c / 2, value
    8c + 2i in the low nibble of byte i) and the scale bytes (8 per block,
    one per 32-row group), rows past R zero codes with scale 127."""
    R, K = X.shape
    Rp = (R + 255) // 256 * 256
    codes = torch.zeros(Rp, K, dtype=torch.int64)
    codes[:R] = W.fp4_codes(X).to(torch.int64)
    u = torch.full((Rp // 32, K // 32), 127, dtype=torch.int64)
    u[:R // 32] = W.fp4_scale_bytes(X)
    r = torch.arange(Rp).view(Rp, 1)
    k = torch.arange(K).view(1, K)
    b, rr, s, kk = r // 256, r % 256, k // 32, k % 32
    c = kk // 8
    q = (rr & ~0x18) | ((rr >> 1) & 0x8) | ((rr << 1) & 0x10)
    slot = q * 4 + 2 * ((c % 2) ^ (((q >> 3) ^ (q >> 4)) & 1)) + c // 2
    byte = ((b * (K // 32) + s) * 1024 + slot) * 4 + (kk % 8) // 2
    out = torch.zeros(Rp * K // 2, dtype=torch.int64)
    even = (kk % 2 == 0).expand(Rp, K)
    out[byte[even]] = codes[even]
    out[byte[~even]] |= codes[~even] << 4
    g = torch.arange(Rp // 32).view(-1, 1)
    sidx = ((g // 8) * (K // 32) + torch.arange(K // 32).view(1, -1)) * 8 + g % 8
    sc = torch.zeros(Rp // 32 * K // 32, dtype=torch.int64)
    sc[sidx.reshape(-1)] = u.reshape(-1)
    return out.to(torch.uint8), sc.to(torch.uint8)


@pytest.mark.parametrize("d", [1024, 320])
def test_pack_bytes_match_host_quantiser(d):
    """dg_pack_embedding (fp4): codes and scale bytes byte-exact against the
    host quantiser in the tiled layout, for a table off the grid (rounding,
    ties, saturation) with an all-zero block, a block of subnormal-range
    values and one with a huge value; the scale of a 32 x 32 block is the
    same whichever way the block is read (E against E^T)."""
    V = 4096
    g = torch.Generator().manual_seed(12)
    E = (torch.randn(V, d, generator=g) * 0.08).to(torch.bfloat16)
    E[0:32, 0:32] = 0.0
    E[32:64, 0:32] = (torch.randn(32, 32, generator=g) * 1e-38).to(torch.bfloat16)
    E[64, 32] = 3e38
    E[96, 64:72] = torch.tensor([4.5, 0.25, 0.26, -0.75, 1.25, 1.75, 2.5, -3.5])
    c = W.config(2, V=V, d=d, table="fp4")
    cfg = B.make_config(c)
    nb = B.dg_embedding_pack_bytes(cfg)
    packed = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    B.dg_pack_embedding(cfg, E.cuda(), packed)
    torch.cuda.synchronize()
    got = packed.cpu()
    ce, se = packed_fp4(E)
    want = torch.cat([ce, se])
    assert got.numel() == want.numel()
    assert torch.equal(got[:ce.numel()], ce)
    assert torch.equal(got, want)
    # square blocks: the transposed table's scale bytes are the same set
    assert torch.equal(W.fp4_scale_bytes(E.t().contiguous()), W.fp4_scale_bytes(E).t())


@pytest.mark.parametrize("cfg_id,V", [(2, 32768), (3, 16384), (4, 16384)])
def test_fp4_table_equals_bf16_table_bitwise(cfg_id, V):
    """On a table that lies on the fp4 grid, the fp4-table step and the
    bf16-table step are the same computation: every canvas buffer equal bit
    for bit over three steps (the second and third self-conditioned)."""
    c = W.config(cfg_id, V=V, table="fp4")
    inp = W.make_inputs(c)
    a = step_outputs(c, inp, 3, "bf16")
    b = step_outputs(c, inp, 3, "fp4")
    for s, (x, y) in enumerate(zip(a, b)):
        for k in x:
            assert torch.equal(x[k], y[k]), (s, k)


@pytest.mark.usefixtures("logits_dump")
def test_fp4_table_lockstep_oracle():
    """The bf16 configuration with an fp4-grid table against the oracle given
    that table: logits, attention, probabilities within 1e-2 relative
    Frobenius, every entropy within 2e-3 nats, decisions replayed exactly."""
    c = W.config(2, table="fp4")
    den, rep = lockstep(c, W.make_inputs(c), 3)
    print(rep)


@pytest.mark.usefixtures("logits_dump")
def test_fp4_table_full_vocab_sampled():
    """V = 262144, d = 2816 with an fp4-grid table: the first step on sampled
    rows against the oracle, the next ones by decision replay."""
    c = W.config(3, table="fp4")
    inp = W.make_inputs(c)
    den = D.Denoiser(c, inp, logits_dump=True)
    om = oracle.model_from_inputs(inp)
    kc, vc = oracle_cache(inp)
    N, V = c["N"], c["V"]
    den.init_canvas(W.canvas_seed(3), 0)
    rows = [0, 5, N // 2 + 1, N - 1]
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


def test_fp4_table_batch_equals_single():
    """Batched canvases on the fp4 table (256-token canvases one per block,
    128-token canvases paired) equal their single-canvas twins bit for bit."""
    from test_gpu_batch import run_equal
    for c, nb in ((W.config(2, V=16384, table="fp4"), 2),
                  (W.config(2, N=128, V=16384, table="fp4"), 3)):
        run_equal(c, W.make_inputs(c, seed=778), nb, 3)
