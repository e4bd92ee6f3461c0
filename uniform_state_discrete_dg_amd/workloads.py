"""Seeded synthetic workloads: the configuration table and input generators.

This module is shared by the HIP path's driver, the tests and the benchmark
as a source of *inputs only*: it draws random weights, prefix keys/values and
prompt tokens with a CPU ``torch.Generator`` and rounds them to the compute
dtype.  It holds none of the method's arithmetic (no embedding, attention,
softmax, sampling or canvas initialisation -- the canvas is drawn by each side
from its own Philox implementation).

The pages describe one trained 26B model on chat/code prompts; no dataset or
trained weights stand behind these inputs.  The shapes follow the pages'
workload (a 256-token canvas, 128 for the latency-sensitive setting, a causal
prefix and chained canvases), the values are random-init:
  E rows ~ N(0, 1/d)  (std 1/sqrt(fan_in), fan_in = d)
  every projection W[out][in] ~ N(0, 1/in)
  RMSNorm gains = 1
  prefix K/V ~ N(0, 1) (configurations that start from a given cache)
  prompt tokens ~ uniform over the vocabulary (the block-diffusion config)
"""
from __future__ import annotations

import math

import torch

# Each entry: canvas N, vocabulary V, model dim d, query/KV heads, head dim,
# self-conditioning FFN hidden F, prefix length L, dtype, temperature
# schedule (kind, T0, T1), max steps, accept threshold gamma (nats),
# adaptive stop (stable steps; 0 = never stop early).
CONFIGS: dict[int, dict] = {
    1: dict(name="tiny-fp32-n16-v512", N=16, V=512, d=64, Hq=4, Hkv=4, hd=16, F=128, L=32,
            dtype="f32", sched="const", T0=1.0, T1=1.0, steps=4, gamma=2.0,
            stop=False, stable_n=0),
    2: dict(name="bf16-n256-v32k-d1024", N=256, V=32768, d=1024, Hq=8, Hkv=8, hd=128, F=2048,
            L=512, dtype="bf16", sched="cosine", T0=1.5, T1=0.3, steps=16, gamma=8.0,
            stop=True, stable_n=3),
    3: dict(name="bf16-n256-v262k-d2816-gqa16x8-l2048", N=256, V=262144, d=2816, Hq=16, Hkv=8,
            hd=128, F=2816, L=2048, dtype="bf16", sched="cosine", T0=1.5, T1=0.3, steps=32,
            gamma=16.0, stop=True, stable_n=3),
    4: dict(name="bf16-n128-v262k-d2816-gqa16x8-l4096", N=128, V=262144, d=2816, Hq=16, Hkv=8,
            hd=128, F=2816, L=4096, dtype="bf16", sched="linear", T0=1.2, T1=0.5, steps=12,
            gamma=8.0, stop=True, stable_n=3),
    5: dict(name="bf16-block-8x256-v262k-d2816-prompt1024", N=256, V=262144, d=2816, Hq=16,
            Hkv=8, hd=128, F=2816, L=0, prompt=1024, canvases=8, dtype="bf16", sched="cosine",
            T0=1.5, T1=0.3, steps=64, gamma=16.0, stop=True, stable_n=3),
}

CONF_EPS = 0.005      # confidence threshold on entropy (nats)
RMS_EPS = 1e-6


def config(cfg_id: int, **overrides) -> dict:
    c = dict(CONFIGS[cfg_id])
    c["id"] = cfg_id
    c.setdefault("prompt", 0)
    c.setdefault("canvases", 1)
    c["rms_eps"] = RMS_EPS
    c.update(overrides)
    c["cap"] = c.get("cap") or max(1, c["L"] + c["prompt"] + (c["canvases"] * c["N"]
                                                               if c["prompt"] else 0))
    return c


def weight_seed(cfg_id: int) -> int:
    return 20260611 + int(cfg_id)


def canvas_seed(cfg_id: int) -> int:
    return 1 + int(cfg_id)


def _round(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.contiguous()


def make_inputs(cfg: dict, seed: int | None = None) -> dict:
    """Draw every input of a configuration on the CPU.

    Returns a dict with the config under "cfg" and tensors in the compute
    dtype (bf16 or fp32): E, w1, w2, wq, wk, wv, wo, g_attn, g_final,
    k_prefix/v_prefix ([Hkv][L][hd], fp32 or bf16), prompt (int32) and
    mask_emb ([d], the [MASK] token's row for the masked sampler).
    """
    c = cfg
    if seed is None:
        seed = weight_seed(c.get("id", 0))
    g = torch.Generator().manual_seed(int(seed))
    V, d, F, Hq, Hkv, hd = c["V"], c["d"], c["F"], c["Hq"], c["Hkv"], c["hd"]
    dt = c["dtype"]

    def w(rows, cols):
        x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
        x.mul_(1.0 / math.sqrt(cols))
        return _round(x, dt)

    out = dict(cfg=c)
    out["E"] = w(V, d)
    if c.get("table") == "fp8":
        out["E"] = fp8_grid(out["E"], c["table_exp"])
    elif c.get("table") == "fp4":
        out["E"] = fp4_grid(out["E"])
    out["w1"] = w(F, d)
    out["w2"] = w(d, F)
    out["wq"] = w(Hq * hd, d)
    out["wk"] = w(Hkv * hd, d)
    out["wv"] = w(Hkv * hd, d)
    out["wo"] = w(d, Hq * hd)
    out["g_attn"] = _round(torch.ones(d), dt)
    out["g_final"] = _round(torch.ones(d), dt)
    L = c["L"]
    out["k_prefix"] = _round(torch.randn(Hkv, L, hd, generator=g), dt)
    out["v_prefix"] = _round(torch.randn(Hkv, L, hd, generator=g), dt)
    P = c.get("prompt", 0)
    out["prompt"] = torch.randint(0, V, (P,), generator=g, dtype=torch.int64).to(torch.int32)
    # the [MASK] token's embedding row (id V) for the masked sampler, drawn
    # like a row of E and last, so the inputs above do not depend on it
    out["mask_emb"] = w(1, d).view(d)
    return out


def fp8_grid(E: torch.Tensor, exp: int) -> torch.Tensor:
    """A quantised table: every entry replaced by the nearest value of the
    form q * 2^-exp with q an fp8 e4m3 number (round to nearest even,
    saturated at +-448), returned in E's dtype (exactly: such values are bf16
    numbers).  This is an input of the fp8-table configurations, drawn before
    either side sees it."""
    q = (E.float() * (2.0 ** exp)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).float()
    return (q * (2.0 ** -exp)).to(E.dtype)


FP4_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # e2m1 magnitudes, codes 0..7


def fp4_scale_bytes(E: torch.Tensor) -> torch.Tensor:
    """The scale byte u of each 32 x 32 block of E [R][K] (R, K multiples of
    32): floor(log2 of the block's largest magnitude) - 2 + 127 read off the
    float32 exponent field, clamped to [2, 252]; 127 for an all-zero block.
    Returns int64 [R/32][K/32]."""
    R, K = E.shape
    a = E.float().abs().view(R // 32, 32, K // 32, 32).amax(dim=(1, 3)).contiguous()
    ef = (a.view(torch.int32) >> 23) & 0xFF
    u = (ef.to(torch.int64) - 2).clamp(2, 252)
    return torch.where(a == 0, torch.full_like(u, 127), u)


def fp4_codes(E: torch.Tensor) -> torch.Tensor:
    """The e2m1 code (sign in bit 3) of every entry of E [R][K] under its
    block's scale: the magnitude over 2^(u - 127) rounded to the nearest
    value of FP4_VALUES, ties to the even code, saturated at 6; a value
    rounded to zero is +0.  Returns uint8 [R][K]."""
    R, K = E.shape
    u = fp4_scale_bytes(E).repeat_interleave(32, 0).repeat_interleave(32, 1)
    y = E.float() * torch.pow(2.0, (127 - u).float())
    a = y.abs()
    # thresholds are the midpoints; a midpoint goes to the even code
    code = torch.full(a.shape, 7, dtype=torch.int64)
    for c, (hi, incl) in reversed(list(enumerate(((0.25, True), (0.75, False), (1.25, True), (1.75, False),
                                                  (2.5, True), (3.5, False), (5.0, True))))):
        code = torch.where((a <= hi) if incl else (a < hi), torch.full_like(code, c), code)
    neg = torch.signbit(y) & (code != 0)
    return (code | (neg.to(torch.int64) << 3)).to(torch.uint8)


def fp4_grid(E: torch.Tensor) -> torch.Tensor:
    """A block-scaled fp4 table: every entry replaced by code value x
    2^(u - 127) (fp4_codes, fp4_scale_bytes), returned in E's dtype (exactly:
    such values are bf16 numbers).  An input of the fp4-table
    configurations, drawn before either side sees it."""
    R, K = E.shape
    q = fp4_codes(E).to(torch.int64)
    mag = torch.tensor(FP4_VALUES, dtype=torch.float32)[q & 7]
    val = torch.where((q & 8) != 0, -mag, mag)
    u = fp4_scale_bytes(E).repeat_interleave(32, 0).repeat_interleave(32, 1)
    return (val * torch.pow(2.0, (u - 127).float())).to(E.dtype)


def random_row_weights(N: int, V: int, seed: int) -> torch.Tensor:
    """Random non-negative matrix [N][V] with entries ~ U(0, 2/V) (so rows sum
    to about 1), a stand-in previous-step distribution for kernel-level tests
    of the self-conditioning contraction."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.rand(N, V, generator=g, dtype=torch.float32) * (2.0 / V)
