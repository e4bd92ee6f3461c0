"""CPU oracle for the uniform-state text-diffusion denoising step.

TEST INFRASTRUCTURE ONLY.  This package wraps ``libdgoracle.so`` (plain C,
double precision, built from ``dg_oracle.c`` with gcc).  It is the slow,
obviously-correct reference that the HIP library is checked against; only the
tests, the smoke check and the benchmark's CPU-baseline leg import it.  It
shares no code with the HIP path: it never imports the product package, and
the product package never imports it.

Each wrapper states the passage of the DiffusionGemma pages it follows (see
``dg_oracle.c``).  Pins: every function is checked by ``tests/test_oracle_*``
against closed forms, library routines on small inputs, invariants and the
published Philox4x32-10 known-answer vectors.  The trained model's behaviour
(convergence, quality, step counts) is "parity unpinned": the pages print no
worked numeric example and no trained weights exist here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dg_oracle.c")
_LIB = os.path.join(_HERE, "libdgoracle.so")

_c_i32 = ctypes.c_int32
_c_u32 = ctypes.c_uint32
_c_u64 = ctypes.c_uint64
_c_dbl = ctypes.c_double
_vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (portable x86-64 code, OpenMP)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.orc_philox4x32_10.argtypes = [_vp, _vp, _vp]
        L.orc_uniform_token.argtypes = [_c_u64, _c_u32, _c_u32, _c_u32, _c_u32, _c_i32]
        L.orc_uniform_token.restype = _c_i32
        L.orc_canvas_init.argtypes = [_c_u64, _c_u32, _c_i32, _c_i32, _vp]
        L.orc_gelu.argtypes = [_c_dbl]
        L.orc_gelu.restype = _c_dbl
        L.orc_rmsnorm.argtypes = [_vp, _vp, _c_i32, _c_dbl, _vp]
        L.orc_matmul_nt.argtypes = [_vp, _vp, _c_i32, _c_i32, _c_i32, _vp]
        L.orc_softmax_entropy.argtypes = [_vp, _c_i32, _vp, _vp]
        L.orc_argmax.argtypes = [_vp, _c_i32]
        L.orc_argmax.restype = _c_i32
        L.orc_argmax_f32.argtypes = [_vp, _c_i32]
        L.orc_argmax_f32.restype = _c_i32
        L.orc_ln_f32.argtypes = [ctypes.c_float]
        L.orc_ln_f32.restype = ctypes.c_float
        L.orc_gumbel_f32.argtypes = [_c_u32]
        L.orc_gumbel_f32.restype = ctypes.c_float
        L.orc_multinomial_candidates.argtypes = [_vp, _vp, _c_i32, _c_i32, _vp, ctypes.c_float, _c_u64,
                                                 _c_u32, _c_u32, _vp, _vp]
        L.orc_attention.argtypes = [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_i32, _c_i32, _vp]
        L.orc_select.argtypes = [_c_i32, _c_i32, _vp, _vp, _vp, _c_dbl, _c_i32, _c_u64,
                                 _c_u32, _c_u32, _c_i32, _c_dbl, _c_i32, _vp, _vp, _c_i32,
                                 _vp, _vp, _vp]
        L.orc_denoise_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_dbl,
                                          _vp, _vp]
        L.orc_denoise_forward.restype = ctypes.c_int
        L.orc_selfcond_row.argtypes = [_vp, _vp, _vp]
        L.orc_prefill_append.argtypes = [_vp, _vp, _c_i32, _vp, _vp, _c_i32, _c_i32, _vp]
        L.orc_prefill_append.restype = ctypes.c_int
        L.orc_temperature.argtypes = [_c_i32, _c_dbl, _c_dbl, _c_i32, _c_i32]
        L.orc_temperature.restype = _c_dbl
        L.orc_should_stop.argtypes = [_vp, _c_i32]
        L.orc_should_stop.restype = _c_i32
        L.orc_num_threads.restype = _c_i32
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_vp)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float32)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def num_threads() -> int:
    return int(lib().orc_num_threads())


# --------------------------------------------------------------------------
# Philox and canvas initialisation
# --------------------------------------------------------------------------
def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def uniform_token(seed: int, pos: int, step: int, canvas_id: int, stream: int, V: int) -> int:
    return int(lib().orc_uniform_token(seed, pos, step, canvas_id, stream, V))


def canvas_init(seed: int, canvas_id: int, N: int, V: int, masked: bool = False) -> np.ndarray:
    """[P3] §5.4 canvas initialisation: uniform tokens from Philox stream 0;
    the masked sampler ([P3] §3.1) starts from [MASK] (id V) everywhere."""
    if masked:
        return np.full(N, V, dtype=np.int32)
    out = np.zeros(N, dtype=np.int32)
    lib().orc_canvas_init(seed, canvas_id, N, V, _p(out))
    return out


# --------------------------------------------------------------------------
# Building blocks
# --------------------------------------------------------------------------
def gelu(x: float) -> float:
    return float(lib().orc_gelu(float(x)))


def rmsnorm(x, g, eps: float) -> np.ndarray:
    x = _f64(x)
    g = _f32(g)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.shape[-1], eps, _p(out))
    return out


def matmul_nt(a, b) -> np.ndarray:
    a = _f64(a)
    b = _f32(b)
    rows, k = a.shape
    cols = b.shape[0]
    assert b.shape[1] == k
    y = np.empty((rows, cols), dtype=np.float64)
    lib().orc_matmul_nt(_p(a), _p(b), rows, cols, k, _p(y))
    return y


def softmax_entropy(y):
    y = _f64(y)
    p = np.empty_like(y)
    H = ctypes.c_double(0.0)
    lib().orc_softmax_entropy(_p(y), y.shape[0], _p(p), ctypes.byref(H))
    return p, H.value


def argmax(z) -> int:
    z = np.asarray(z)
    if z.dtype == np.float32:
        z = np.ascontiguousarray(z)
        return int(lib().orc_argmax_f32(_p(z), z.shape[0]))
    z = _f64(z)
    return int(lib().orc_argmax(_p(z), z.shape[0]))


def ln_f32(x) -> np.float32:
    """The fixed single-precision natural log of the multinomial draw."""
    return np.float32(lib().orc_ln_f32(float(np.float32(x))))


def gumbel_f32(w: int) -> np.float32:
    """Standard Gumbel variable of one 32-bit Philox word (multinomial draw)."""
    return np.float32(lib().orc_gumbel_f32(int(w) & 0xFFFFFFFF))


def multinomial_candidates(tile_zmax, tile_l, num, inv_T, seed: int, step: int, canvas_id: int,
                           fallback) -> np.ndarray:
    """[P3] §5.3 multinomial candidates drawn in two levels (tile by its mass
    l_t e^(zmax_t inv_T), then the column by its numerator) with Gumbel-max,
    replayable bit for bit.  tile_zmax, tile_l: float32 [N][ntiles]; num:
    float32 numerators [N][64 ntiles]; inv_T the float32 the kernels use."""
    tz = np.ascontiguousarray(tile_zmax, dtype=np.float32)
    tl = np.ascontiguousarray(tile_l, dtype=np.float32)
    nm = np.ascontiguousarray(num, dtype=np.float32)
    N, nt = tz.shape
    assert tl.shape == (N, nt) and nm.shape == (N, 64 * nt)
    fb = _i32(fallback)
    out = np.zeros(N, dtype=np.int32)
    lib().orc_multinomial_candidates(_p(tz), _p(tl), N, nt, _p(nm), float(np.float32(inv_T)), seed, step,
                                     canvas_id, _p(fb), _p(out))
    return out


def attention(q, k, v, Hq: int, Hkv: int, causal: bool = False, q_pos0: int = 0) -> np.ndarray:
    """q: [nq][Hq*hd]; k, v: [Hkv][nk][hd] -> [nq][Hq*hd]."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    nq = q.shape[0]
    nk, hd = k.shape[1], k.shape[2]
    out = np.empty((nq, Hq * hd), dtype=np.float64)
    lib().orc_attention(_p(q), _p(k), _p(v), nq, nk, Hq, Hkv, hd, int(causal), q_pos0, _p(out))
    return out


# --------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------
ACCEPT_SUM_MINUS_MAX = 0
ACCEPT_CUMSUM = 1
STABLE_PREDICTIONS = 0
STABLE_CANVAS = 1


class _Flags(ctypes.Structure):
    _fields_ = [("allconf", _c_i32), ("changed", _c_i32), ("stable", _c_i32),
                ("accepted", _c_i32), ("masked", _c_i32), ("pred_changed", _c_i32)]


def select(H, argmax_tokens, tokens_in, V: int, gamma: float, rule: int, seed: int,
           canvas_id: int, step: int, stable_in: int, conf_eps: float = 0.005,
           mask_id: int = -1, stable_rule: int = STABLE_CANVAS, pred=None, pred_prev=None):
    """[P3] §5.4 entropy-bounded acceptance + re-noise; [P3] §5.3 / [P5] stop flags.

    H is float32 (the decision is taken in the precision the kernel produces
    its entropies in; conf_eps is compared as a float32 too).  argmax_tokens:
    the candidate token of each position.  mask_id >= 0 selects the masked
    sampler ([P1] §1, [P3] §3.1): only positions holding mask_id take part;
    accepted ones lock, rejected ones stay mask_id.  stable_rule: what the
    stable counter counts -- STABLE_PREDICTIONS (the predictions `pred`, each
    position's most likely token, equal to the previous step's `pred_prev`;
    None at a canvas's first step) or STABLE_CANVAS (the canvas unchanged).
    Returns (accept uint8[N], tokens_out int32[N], flags dict).
    """
    Hf = np.ascontiguousarray(H, dtype=np.float32)
    am = _i32(argmax_tokens)
    tin = _i32(tokens_in)
    N = Hf.shape[0]
    pr = am if pred is None else _i32(pred)
    pp = None if pred_prev is None else _i32(pred_prev)
    acc = np.zeros(N, dtype=np.uint8)
    tout = np.zeros(N, dtype=np.int32)
    fl = _Flags()
    lib().orc_select(N, V, _p(Hf), _p(am), _p(tin), float(gamma), int(rule), seed, canvas_id,
                     step, stable_in, float(conf_eps), int(mask_id), _p(pr), _p(pp), int(stable_rule),
                     _p(acc), _p(tout), ctypes.byref(fl))
    flags = dict(allconf=fl.allconf, changed=fl.changed, stable=fl.stable, accepted=fl.accepted,
                 masked=fl.masked, pred_changed=fl.pred_changed)
    return acc, tout, flags


def should_stop(flags: dict, stable_steps: int) -> bool:
    fl = _Flags(flags["allconf"], flags["changed"], flags["stable"], flags.get("accepted", 0),
                flags.get("masked", -1), flags.get("pred_changed", 1))
    return bool(lib().orc_should_stop(ctypes.byref(fl), stable_steps))


SCHED_CONST, SCHED_LINEAR, SCHED_COSINE = 0, 1, 2
_SCHED = {"const": SCHED_CONST, "linear": SCHED_LINEAR, "cosine": SCHED_COSINE}


def temperature(kind, T0: float, T1: float, s: int, S: int) -> float:
    k = _SCHED[kind] if isinstance(kind, str) else int(kind)
    return float(lib().orc_temperature(k, T0, T1, s, S))


# --------------------------------------------------------------------------
# Model-level calls
# --------------------------------------------------------------------------
class _Model(ctypes.Structure):
    _fields_ = [("N", _c_i32), ("V", _c_i32), ("d", _c_i32), ("Hq", _c_i32), ("Hkv", _c_i32),
                ("hd", _c_i32), ("F", _c_i32), ("rms_eps", _c_dbl),
                ("E", _vp), ("w1", _vp), ("w2", _vp), ("wq", _vp), ("wk", _vp), ("wv", _vp),
                ("wo", _vp), ("g_attn", _vp), ("g_final", _vp), ("mask_emb", _vp)]


class _StepOut(ctypes.Structure):
    _fields_ = [("h0", _vp), ("q", _vp), ("k_canvas", _vp), ("v_canvas", _vp), ("attn", _vp),
                ("h1", _vp), ("logits", _vp), ("probs", _vp), ("entropy", _vp),
                ("argmax", _vp)]


class Model:
    """Holds float32 copies of the weights (values as the GPU receives them)."""

    def __init__(self, N, V, d, Hq, Hkv, hd, F, E, w1, w2, wq, wk, wv, wo, g_attn, g_final,
                 rms_eps: float = 1e-6, mask_emb=None):
        self.N, self.V, self.d, self.Hq, self.Hkv, self.hd, self.F = N, V, d, Hq, Hkv, hd, F
        self.rms_eps = rms_eps
        self._arrs = dict(E=_f32(E), w1=_f32(w1), w2=_f32(w2), wq=_f32(wq), wk=_f32(wk),
                          wv=_f32(wv), wo=_f32(wo), g_attn=_f32(g_attn), g_final=_f32(g_final))
        if mask_emb is not None:       # the [MASK] token's row (id V), masked sampler
            self._arrs["mask_emb"] = _f32(mask_emb)
            assert self._arrs["mask_emb"].shape == (d,)
        a = self._arrs
        assert a["E"].shape == (V, d)
        assert a["w1"].shape == (F, d) and a["w2"].shape == (d, F)
        assert a["wq"].shape == (Hq * hd, d) and a["wk"].shape == (Hkv * hd, d)
        assert a["wv"].shape == (Hkv * hd, d) and a["wo"].shape == (d, Hq * hd)
        self._s = _Model(N, V, d, Hq, Hkv, hd, F, rms_eps, *(_p(a[k]) for k in
                         ("E", "w1", "w2", "wq", "wk", "wv", "wo", "g_attn", "g_final")),
                         _p(a.get("mask_emb")))

    @property
    def E(self) -> np.ndarray:
        return self._arrs["E"]

    def with_canvas(self, N: int) -> "Model":
        a = self._arrs
        return Model(N, self.V, self.d, self.Hq, self.Hkv, self.hd, self.F, a["E"], a["w1"],
                     a["w2"], a["wq"], a["wk"], a["wv"], a["wo"], a["g_attn"], a["g_final"],
                     self.rms_eps, a.get("mask_emb"))

    def selfcond_row(self, p_row) -> np.ndarray:
        p = _f64(p_row)
        out = np.empty(self.d, dtype=np.float64)
        lib().orc_selfcond_row(ctypes.byref(self._s), _p(p), _p(out))
        return out

    def denoise_forward(self, tokens, p_prev, k_cache, v_cache, L: int, T: float,
                        row_sel=None, want_logits: bool = True, want_probs: bool = True):
        """Steps 1-8 of one denoising step; see ``orc_denoise_forward``.

        k_cache/v_cache: float64 [Hkv][cap][hd].  Returns a dict of arrays.
        """
        N, V, d = self.N, self.V, self.d
        qw, kw = self.Hq * self.hd, self.Hkv * self.hd
        tok = _i32(tokens)
        assert tok.shape == (N,)
        kc = _f64(k_cache)
        vc = _f64(v_cache)
        cap = kc.shape[1]
        pp = None if p_prev is None else _f64(p_prev)
        if pp is not None:
            assert pp.shape == (N, V)
        rs = None if row_sel is None else np.ascontiguousarray(row_sel, dtype=np.uint8)
        out = dict(
            h0=np.zeros((N, d)), q=np.zeros((N, qw)),
            k_canvas=np.zeros((self.Hkv, N, self.hd)), v_canvas=np.zeros((self.Hkv, N, self.hd)),
            attn=np.full((N, qw), np.nan), h1=np.full((N, d), np.nan),
            logits=np.full((N, V), np.nan) if want_logits else None,
            probs=np.full((N, V), np.nan) if want_probs else None,
            entropy=np.full(N, np.nan), argmax=np.full(N, -1, dtype=np.int32))
        so = _StepOut(*(_p(out[k]) for k in ("h0", "q", "k_canvas", "v_canvas", "attn", "h1",
                                               "logits", "probs", "entropy", "argmax")))
        rc = lib().orc_denoise_forward(ctypes.byref(self._s), _p(tok), _p(pp), _p(kc), _p(vc),
                                       L, cap, float(T), _p(rs), ctypes.byref(so))
        if rc != 0:
            raise ValueError(f"orc_denoise_forward failed ({rc})")
        return out

    def prefill_append(self, tokens, k_cache: np.ndarray, v_cache: np.ndarray, L: int,
                       want_attn: bool = True):
        """Causal append of tokens' K/V at [L, L+n) (in place); returns attn or None."""
        tok = _i32(tokens)
        n = tok.shape[0]
        assert k_cache.dtype == np.float64 and k_cache.flags["C_CONTIGUOUS"]
        assert v_cache.dtype == np.float64 and v_cache.flags["C_CONTIGUOUS"]
        cap = k_cache.shape[1]
        attn = np.zeros((n, self.Hq * self.hd)) if want_attn else None
        rc = lib().orc_prefill_append(ctypes.byref(self._s), _p(tok), n, _p(k_cache),
                                      _p(v_cache), L, cap, _p(attn))
        if rc != 0:
            raise ValueError(f"orc_prefill_append failed ({rc})")
        return attn


def model_from_inputs(inp: dict, N: int | None = None) -> Model:
    """Build an oracle Model from a workload input dict (torch or numpy arrays)."""
    def f(x):
        if hasattr(x, "detach"):
            return x.detach().float().numpy()
        return np.asarray(x, dtype=np.float32)
    c = inp["cfg"]
    return Model(N if N is not None else c["N"], c["V"], c["d"], c["Hq"], c["Hkv"], c["hd"],
                 c["F"], f(inp["E"]), f(inp["w1"]), f(inp["w2"]), f(inp["wq"]), f(inp["wk"]),
                 f(inp["wv"]), f(inp["wo"]), f(inp["g_attn"]), f(inp["g_final"]),
                 c.get("rms_eps", 1e-6), f(inp["mask_emb"]) if "mask_emb" in inp else None)
