"""ctypes binding of libdgdenoise (include/dgdenoise.h): same entry-point
names, argument marshalling only.  PyTorch supplies device memory (tensors
whose data_ptr() is passed down) and streams; every step of the compute
path runs in the library's HIP kernels.

The library must have been built (``python -m uniform_state_discrete_dg_amd.build``
or ``__graft_entry__.build()``); loading fails loudly otherwise -- there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdgdenoise.so")

c_i32, c_u32, c_u64, c_f32, c_sz, vp = (ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64,
                                        ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p)

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_CAPACITY, DG_ERR_WORKSPACE, DG_ERR_HIP = range(6)
DG_F32, DG_BF16 = 0, 1
DG_ACCEPT_SUM_MINUS_MAX, DG_ACCEPT_CUMSUM = 0, 1
DG_CANDIDATE_ARGMAX, DG_CANDIDATE_MULTINOMIAL = 0, 1
DG_SAMPLER_UNIFORM, DG_SAMPLER_MASKED = 0, 1
DG_TABLE_BF16, DG_TABLE_FP8, DG_TABLE_FP4 = 0, 1, 2
DG_STABLE_PREDICTIONS, DG_STABLE_CANVAS = 0, 1
DG_STATUS_WORDS = 16
DG_MAX_BATCH = 16
(DG_ST_ALLCONF, DG_ST_CHANGED, DG_ST_STABLE, DG_ST_ACCEPTED, DG_ST_NAN, DG_ST_STEP, DG_ST_HMIN,
 DG_ST_HMAX, DG_ST_HMEAN, DG_ST_MASKED, DG_ST_PRED_CHANGED) = range(11)
TILE_V = 64  # vocabulary columns per softmax-statistics tile


class dg_config(ctypes.Structure):
    _fields_ = [("canvas_len", c_i32), ("vocab", c_i32), ("d_model", c_i32), ("n_q_heads", c_i32),
                ("n_kv_heads", c_i32), ("head_dim", c_i32), ("ffn_hidden", c_i32), ("dtype", c_i32),
                ("rms_eps", c_f32), ("conf_eps", c_f32), ("accept_rule", c_i32), ("candidate_rule", c_i32),
                ("sampler", c_i32), ("table_format", c_i32), ("table_exp", c_i32), ("stable_rule", c_i32)]


class dg_weights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("E", "E_pack", "w_sc1", "w_sc2", "wq", "wk", "wv", "wo", "g_attn",
                                  "g_final", "mask_emb")]


class dg_kv_cache(ctypes.Structure):
    _fields_ = [("k", vp), ("v", vp), ("length", c_i32), ("capacity", c_i32)]


class dg_canvas(ctypes.Structure):
    _fields_ = [("tokens", vp), ("probs", vp), ("stats", vp), ("entropy", vp), ("argmax", vp),
                ("accept", vp), ("status", vp), ("step", c_i32), ("has_prev", c_i32),
                ("seed", c_u64), ("canvas_id", c_u32)]


class dg_step_stats(ctypes.Structure):
    _fields_ = [("accepted", c_i32), ("stable", c_i32), ("allconf", c_i32), ("changed", c_i32),
                ("h_min", c_f32), ("h_mean", c_f32), ("h_max", c_f32), ("masked", c_i32)]


class dg_ws_offsets(ctypes.Structure):
    _fields_ = [("h0", c_sz), ("attn", c_sz), ("h1", c_sz), ("selfcond", c_sz), ("logits", c_sz)]


P = ctypes.POINTER
# name -> (restype, argtypes); mirrors include/dgdenoise.h
SIGNATURES = {
    "dg_abi_version": (c_i32, []),
    "dg_status_string": (ctypes.c_char_p, [c_i32]),
    "dg_validate_config": (c_i32, [P(dg_config)]),
    "dg_workspace_bytes": (c_sz, [P(dg_config), c_i32]),
    "dg_stats_bytes": (c_sz, [P(dg_config)]),
    "dg_embedding_pack_bytes": (c_sz, [P(dg_config)]),
    "dg_probs_bytes": (c_sz, [P(dg_config)]),
    "dg_pack_embedding": (c_i32, [P(dg_config), vp, vp, vp]),
    "dg_canvas_init": (c_i32, [P(dg_config), P(dg_canvas), c_u64, c_u32, vp]),
    "dg_prefill_append": (c_i32, [P(dg_config), P(dg_weights), P(dg_kv_cache), vp, c_i32, vp, vp,
                                  c_sz, vp]),
    "dg_denoise_step": (c_i32, [P(dg_config), P(dg_weights), P(dg_kv_cache), P(dg_canvas), c_f32,
                                c_f32, vp, c_sz, vp]),
    "dg_denoise_step_static": (c_i32, [P(dg_config), P(dg_weights), P(dg_kv_cache), P(dg_canvas), c_f32,
                                       c_f32, vp]),
    "dg_workspace_bytes_batch": (c_sz, [P(dg_config), c_i32]),
    "dg_denoise_step_batch": (c_i32, [P(dg_config), P(dg_weights), P(dg_kv_cache), P(dg_canvas), c_i32,
                                      c_f32, c_f32, vp, c_sz, vp]),
    "dg_should_stop": (c_i32, [P(dg_config), P(dg_canvas), c_i32, P(c_i32), P(dg_step_stats), vp]),
    "dg_run_canvas": (c_i32, [P(dg_config), P(dg_weights), P(dg_kv_cache), P(dg_canvas), c_u64, c_u32,
                              P(c_f32), c_i32, c_f32, c_i32, c_i32, vp, c_sz, vp, P(c_i32), P(c_i32)]),
    "dg_test_ws_offsets": (c_i32, [P(dg_config), P(dg_ws_offsets)]),
    "dg_test_set_logits_dump": (None, [c_i32]),
    "dg_test_logits_ws_bytes": (c_sz, [P(dg_config)]),
    "dg_test_selfcond": (c_i32, [P(dg_config), P(dg_weights), vp, vp, vp, c_sz, vp]),
    "dg_test_selfcond_canvas": (c_i32, [P(dg_config), P(dg_weights), P(dg_canvas), vp, vp, c_sz, vp]),
    "dg_test_select": (c_i32, [P(dg_config), P(dg_canvas), c_f32, vp]),
    "dg_test_philox": (c_i32, [vp, c_u32, c_u32, vp, c_i32, vp]),
    "dg_test_gumbel": (c_i32, [vp, c_i32, c_i32, vp, vp]),
    "dg_test_copy": (c_i32, [vp, vp, c_sz, vp]),
    "dg_profile_enable": (None, [c_i32]),
    "dg_profile_read": (c_i32, [P(c_f32), P(c_i32), P(c_f32), P(c_i32)]),
}

_lib = None


def lib():
    """Load libdgdenoise.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m uniform_state_discrete_dg_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class DgError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib().dg_status_string(status).decode()} ({status})")


def _check(fn: str, st: int) -> None:
    if st != DG_OK:
        raise DgError(fn, st)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def dg_abi_version() -> int:
    return int(lib().dg_abi_version())


def dg_validate_config(cfg: dg_config) -> int:
    return int(lib().dg_validate_config(ctypes.byref(cfg)))


def dg_workspace_bytes(cfg: dg_config, max_prefill_tokens: int = 0) -> int:
    return int(lib().dg_workspace_bytes(ctypes.byref(cfg), max_prefill_tokens))


def dg_stats_bytes(cfg: dg_config) -> int:
    return int(lib().dg_stats_bytes(ctypes.byref(cfg)))


def dg_embedding_pack_bytes(cfg: dg_config) -> int:
    return int(lib().dg_embedding_pack_bytes(ctypes.byref(cfg)))


def dg_probs_bytes(cfg: dg_config) -> int:
    return int(lib().dg_probs_bytes(ctypes.byref(cfg)))


def dg_pack_embedding(cfg: dg_config, E: torch.Tensor, E_pack: torch.Tensor | None, stream=None) -> None:
    _check("dg_pack_embedding", lib().dg_pack_embedding(ctypes.byref(cfg), _ptr(E), _ptr(E_pack),
                                                        _stream(stream)))


def dg_canvas_init(cfg: dg_config, canvas: dg_canvas, seed: int, canvas_id: int, stream=None) -> None:
    _check("dg_canvas_init", lib().dg_canvas_init(ctypes.byref(cfg), ctypes.byref(canvas), seed,
                                                  canvas_id, _stream(stream)))


def dg_prefill_append(cfg: dg_config, w: dg_weights, cache: dg_kv_cache, tokens: torch.Tensor,
                      n_tokens: int, attn_out: torch.Tensor | None, ws: torch.Tensor,
                      stream=None) -> None:
    _check("dg_prefill_append", lib().dg_prefill_append(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), _ptr(tokens), n_tokens,
        _ptr(attn_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dg_denoise_step(cfg: dg_config, w: dg_weights, cache: dg_kv_cache, canvas: dg_canvas,
                    temperature: float, accept_threshold_nats: float, ws: torch.Tensor,
                    stream=None) -> None:
    _check("dg_denoise_step", lib().dg_denoise_step(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), ctypes.byref(canvas),
        temperature, accept_threshold_nats, _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


DG_STATIC_SCRATCH_BYTES = 160 << 20


def dg_denoise_step_static(cfg: dg_config, w: dg_weights, cache: dg_kv_cache, canvas: dg_canvas,
                           temperature: float, accept_threshold_nats: float, stream=None) -> None:
    """dg_denoise_step with the library's own device scratch (no workspace)."""
    _check("dg_denoise_step_static", lib().dg_denoise_step_static(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), ctypes.byref(canvas), temperature,
        accept_threshold_nats, _stream(stream)))


def dg_workspace_bytes_batch(cfg: dg_config, n_canvases: int) -> int:
    return int(lib().dg_workspace_bytes_batch(ctypes.byref(cfg), n_canvases))


def dg_denoise_step_batch(cfg: dg_config, w: dg_weights, caches, canvases, temperature: float,
                          accept_threshold_nats: float, ws: torch.Tensor, stream=None) -> None:
    """caches, canvases: equal-length sequences of dg_kv_cache / dg_canvas.
    The canvases' host fields (step, has_prev) are updated in place."""
    n = len(canvases)
    if len(caches) != n:
        raise ValueError("one cache descriptor per canvas")
    ca = (dg_kv_cache * max(n, 1))(*caches)
    cv = (dg_canvas * max(n, 1))(*canvases)
    _check("dg_denoise_step_batch", lib().dg_denoise_step_batch(
        ctypes.byref(cfg), ctypes.byref(w), ca, cv, n, temperature, accept_threshold_nats, _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    for i in range(n):
        canvases[i].step = cv[i].step
        canvases[i].has_prev = cv[i].has_prev


def dg_should_stop(cfg: dg_config, canvas: dg_canvas, stable_steps: int, stream=None):
    stop = c_i32(0)
    stats = dg_step_stats()
    _check("dg_should_stop", lib().dg_should_stop(ctypes.byref(cfg), ctypes.byref(canvas),
                                                  stable_steps, ctypes.byref(stop),
                                                  ctypes.byref(stats), _stream(stream)))
    return bool(stop.value), stats


def dg_run_canvas(cfg: dg_config, w: dg_weights, cache: dg_kv_cache, canvas: dg_canvas, seed: int,
                  canvas_id: int, temps, accept_threshold_nats: float, adaptive_stop: bool,
                  stable_steps: int, ws: torch.Tensor, stream=None):
    """Returns (steps run, whether the adaptive stop ended the loop)."""
    n = len(temps)
    arr = (c_f32 * max(n, 1))(*temps)
    steps, stopped = c_i32(0), c_i32(0)
    _check("dg_run_canvas", lib().dg_run_canvas(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), ctypes.byref(canvas), seed, canvas_id,
        arr, n, accept_threshold_nats, 1 if adaptive_stop else 0, stable_steps, _ptr(ws), ws.numel(),
        _stream(stream), ctypes.byref(steps), ctypes.byref(stopped)))
    return int(steps.value), bool(stopped.value)


def dg_test_ws_offsets(cfg: dg_config) -> dg_ws_offsets:
    o = dg_ws_offsets()
    _check("dg_test_ws_offsets", lib().dg_test_ws_offsets(ctypes.byref(cfg), ctypes.byref(o)))
    return o


def dg_test_set_logits_dump(on: bool) -> None:
    lib().dg_test_set_logits_dump(1 if on else 0)


def dg_test_logits_ws_bytes(cfg: dg_config) -> int:
    return int(lib().dg_test_logits_ws_bytes(ctypes.byref(cfg)))


def dg_test_selfcond(cfg: dg_config, w: dg_weights, Pm: torch.Tensor, S: torch.Tensor,
                     ws: torch.Tensor, stream=None) -> None:
    _check("dg_test_selfcond", lib().dg_test_selfcond(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(Pm), _ptr(S), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def dg_test_selfcond_canvas(cfg: dg_config, w: dg_weights, canvas: dg_canvas, S: torch.Tensor,
                            ws: torch.Tensor, stream=None) -> None:
    _check("dg_test_selfcond_canvas", lib().dg_test_selfcond_canvas(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(canvas), _ptr(S), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def dg_test_select(cfg: dg_config, canvas: dg_canvas, accept_threshold_nats: float,
                   stream=None) -> None:
    _check("dg_test_select", lib().dg_test_select(ctypes.byref(cfg), ctypes.byref(canvas),
                                                  accept_threshold_nats, _stream(stream)))


def dg_test_philox(ctr: torch.Tensor, k0: int, k1: int, out: torch.Tensor, n: int,
                   stream=None) -> None:
    _check("dg_test_philox", lib().dg_test_philox(_ptr(ctr), k0, k1, _ptr(out), n, _stream(stream)))


def dg_test_gumbel(w: torch.Tensor, n: int, mode: int, out: torch.Tensor, stream=None) -> None:
    _check("dg_test_gumbel", lib().dg_test_gumbel(_ptr(w), n, mode, _ptr(out), _stream(stream)))


def dg_test_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int, stream=None) -> None:
    _check("dg_test_copy", lib().dg_test_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def dg_profile_enable(mask: int) -> None:
    """1: time the LM head, 2: the self-conditioning contraction, 3: both, 0: off."""
    lib().dg_profile_enable(int(mask))


def dg_profile_read():
    a, b = c_f32(0), c_f32(0)
    na, nb = c_i32(0), c_i32(0)
    _check("dg_profile_read", lib().dg_profile_read(ctypes.byref(a), ctypes.byref(na),
                                                    ctypes.byref(b), ctypes.byref(nb)))
    return a.value, na.value, b.value, nb.value


# ---------------------------------------------------------------------------
# device-side holders (torch allocations wrapped in the C structs)
# ---------------------------------------------------------------------------
def make_config(c: dict, accept_rule: int = DG_ACCEPT_SUM_MINUS_MAX,
                conf_eps: float = 0.005, candidate_rule: int = DG_CANDIDATE_ARGMAX,
                sampler: int = DG_SAMPLER_UNIFORM, stable_rule: int = DG_STABLE_PREDICTIONS) -> dg_config:
    """The C config of a workload dict; c["table"] == "fp8" selects the fp8
    packed table with scale exponent c["table_exp"], "fp4" the block-scaled
    fp4 table; c["stable_rule"], when present, overrides stable_rule."""
    table = {"fp8": DG_TABLE_FP8, "fp4": DG_TABLE_FP4}.get(c.get("table"), DG_TABLE_BF16)
    return dg_config(c["N"], c["V"], c["d"], c["Hq"], c["Hkv"], c["hd"], c["F"],
                     DG_BF16 if c["dtype"] == "bf16" else DG_F32, c.get("rms_eps", 1e-6),
                     conf_eps, accept_rule, candidate_rule, sampler,
                     table, c.get("table_exp", 0) if table == DG_TABLE_FP8 else 0,
                     c.get("stable_rule", stable_rule))


def stats_offsets(cfg: dg_config) -> dict:
    """Byte offsets inside a canvas's `stats` buffer (the library's layout):
    float4 tile statistics [N][V/64], float tile factors [N][V/64] (fp32
    path), float2 top [N], float row factor [N], int32 previous predictions
    [N], then, 256-byte aligned, uint8 tile exponents [V/64][256]."""
    N, nt = cfg.canvas_len, cfg.vocab // TILE_V
    o = dict(tstats=0, tscale=N * nt * 16)
    o["top"] = o["tscale"] + N * nt * 4
    o["rscale"] = o["top"] + N * 8
    o["pred"] = o["rscale"] + N * 4
    o["shift"] = (o["pred"] + N * 4 + 255) // 256 * 256
    return o


def torch_dtype(cfg: dg_config):
    return torch.bfloat16 if cfg.dtype == DG_BF16 else torch.float32


def _tiled_perm(device):
    """Chunk positions of the tiled layout: position p holds block row p // 4
    and logical 8-column chunk (p % 4) ^ ((p // 16) % 4)."""
    p = torch.arange(1024, device=device)
    r = p // 4
    return r, (p % 4) ^ ((r // 4) % 4)


def rows_to_tiled(X: torch.Tensor) -> torch.Tensor:
    """Row-major [R][K] -> the tiled layout (flat, rows padded to 256 with zeros)."""
    R, K = X.shape
    Rp = (R + 255) // 256 * 256
    Xp = torch.zeros((Rp, K), dtype=X.dtype, device=X.device)
    Xp[:R] = X
    r, c = _tiled_perm(X.device)
    Y = Xp.view(Rp // 256, 256, K // 32, 4, 8).permute(0, 2, 1, 3, 4)[:, :, r, c, :]
    return Y.contiguous().view(-1)


def tiled_to_rows(T: torch.Tensor, R: int, K: int) -> torch.Tensor:
    """The tiled layout (flat) -> row-major [R][K]."""
    Rp = (R + 255) // 256 * 256
    r, c = _tiled_perm(T.device)
    Y = T.view(Rp // 256, K // 32, 1024, 8)
    out = torch.empty((Rp // 256, K // 32, 256, 4, 8), dtype=T.dtype, device=T.device)
    out[:, :, r, c, :] = Y
    return out.permute(0, 2, 1, 3, 4).reshape(Rp, K)[:R]


class DeviceWeights:
    """Moves a workload's weights to the GPU and packs the table once.  The
    bf16 configuration keeps only the packed copy of E (the row-major one is
    freed once packed and the step is given a null E); the fp32 one keeps E
    row-major."""

    def __init__(self, cfg: dg_config, inp: dict, device="cuda", stream=None):
        dt = torch_dtype(cfg)
        t = {k: inp[k].to(device=device, dtype=dt).contiguous()
             for k in ("E", "w1", "w2", "wq", "wk", "wv", "wo", "g_attn", "g_final", "mask_emb") if k in inp}
        nb = dg_embedding_pack_bytes(cfg)
        if nb:
            t["E_pack"] = torch.empty(nb, dtype=torch.uint8, device=device)
            dg_pack_embedding(cfg, t["E"], t["E_pack"], stream)
            if stream is None:
                torch.cuda.current_stream(device).synchronize()
            else:
                stream.synchronize()
            del t["E"]
        self.t = t
        self.s = dg_weights(*(t[k].data_ptr() if k in t else None
                              for k in ("E", "E_pack", "w1", "w2", "wq", "wk", "wv", "wo", "g_attn",
                                        "g_final", "mask_emb")))


def split_pair(x: torch.Tensor) -> torch.Tensor:
    """fp32 values -> [2, *x.shape] bf16: hi = bf16(x), lo = bf16(x - hi)
    (round to nearest even, as the library writes them)."""
    x = x.to(torch.float32)
    hi = x.to(torch.bfloat16)
    lo = (x - hi.to(torch.float32)).to(torch.bfloat16)
    return torch.stack((hi, lo))


def join_pair(p: torch.Tensor) -> torch.Tensor:
    """[2, ...] bf16 split pair -> the fp32 values hi + lo (exact)."""
    return p[0].to(torch.float32) + p[1].to(torch.float32)


class DeviceCache:
    """Keys and values of the prefix, [Hkv][capacity][hd] each: fp32 for a
    DG_F32 model; for DG_BF16 split pairs, bf16 [2][Hkv][capacity][hd] (the
    hi terms, then the lo terms; the same bytes as fp32).  k_f32() / v_f32()
    give the values as fp32 [Hkv][capacity][hd] either way."""

    def __init__(self, cfg: dg_config, capacity: int, device="cuda", k_prefix=None, v_prefix=None):
        self.pair = cfg.dtype == DG_BF16
        shape = (cfg.n_kv_heads, capacity, cfg.head_dim)
        if self.pair:
            self.k = torch.zeros((2,) + shape, dtype=torch.bfloat16, device=device)
        else:
            self.k = torch.zeros(shape, dtype=torch.float32, device=device)
        self.v = torch.zeros_like(self.k)
        L = 0
        if k_prefix is not None:
            L = k_prefix.shape[1]
            for dst, src in ((self.k, k_prefix), (self.v, v_prefix)):
                if self.pair:
                    dst[:, :, :L] = split_pair(src.to(device=device))
                else:
                    dst[:, :L] = src.to(device=device, dtype=torch.float32)
        self.s = dg_kv_cache(self.k.data_ptr(), self.v.data_ptr(), L, capacity)

    def k_f32(self) -> torch.Tensor:
        return join_pair(self.k) if self.pair else self.k

    def v_f32(self) -> torch.Tensor:
        return join_pair(self.v) if self.pair else self.v

    @property
    def length(self) -> int:
        return self.s.length


class DeviceCanvas:
    def __init__(self, cfg: dg_config, device="cuda"):
        N, V = cfg.canvas_len, cfg.vocab
        dt = torch_dtype(cfg)
        self.tokens = torch.zeros(N, dtype=torch.int32, device=device)
        self.probs = torch.zeros(dg_probs_bytes(cfg), dtype=torch.uint8, device=device)
        self.stats = torch.zeros(dg_stats_bytes(cfg), dtype=torch.uint8, device=device)
        self.entropy = torch.zeros(N, dtype=torch.float32, device=device)
        self.argmax = torch.zeros(N, dtype=torch.int32, device=device)
        self.accept = torch.zeros(N, dtype=torch.uint8, device=device)
        self.status = torch.zeros(DG_STATUS_WORDS, dtype=torch.int32, device=device)
        self.replay_pred = None  # host-side note of the tests' decision replay
        self.s = dg_canvas(self.tokens.data_ptr(), self.probs.data_ptr(), self.stats.data_ptr(),
                           self.entropy.data_ptr(), self.argmax.data_ptr(),
                           self.accept.data_ptr(), self.status.data_ptr(), 0, 0, 0, 0)

    def probabilities(self, cfg: dg_config) -> torch.Tensor:
        """The last step's probabilities as float32 [N][V] (row-major)."""
        N, V = cfg.canvas_len, cfg.vocab
        if cfg.dtype == DG_BF16:
            num = tiled_to_rows(self.probs.view(torch.bfloat16), N, V).float()
            return (num.view(N, V // TILE_V, TILE_V) * self.tile_scale(cfg).unsqueeze(-1)).view(N, V)
        return self.probs.view(torch.float32).view(N, V)

    def tile_scale(self, cfg: dg_config) -> torch.Tensor:
        """Per-(row, tile) factors of the last step ([N][V/64] f32) that turn
        the stored values into probabilities.  bf16: 2^-exponent x the row
        factor (the library keeps those two, not the product)."""
        N, nt = cfg.canvas_len, cfg.vocab // TILE_V
        o = stats_offsets(cfg)
        if cfg.dtype == DG_BF16:
            g = self.stats[o["rscale"]:o["rscale"] + N * 4].view(torch.float32)
            e = self.exponents(cfg).t().float()
            return torch.exp2(-e) * g.unsqueeze(1)
        return self.stats[o["tscale"]:o["top"]].view(torch.float32).view(N, nt)

    def exponents(self, cfg: dg_config) -> torch.Tensor:
        """bf16 path: the per-(tile, row) power-of-two exponents R - r_t
        (uint8 [V/64][N]) the next step's contraction applies."""
        N, nt = cfg.canvas_len, cfg.vocab // TILE_V
        base = stats_offsets(cfg)["shift"]
        return self.stats[base:base + nt * 256].view(nt, 256)[:, :N]

    def predictions(self, cfg: dg_config) -> torch.Tensor:
        """The step's predictions (each position's most likely token), int32 [N]."""
        return self.top(cfg)[0]

    def pred_prev(self, cfg: dg_config) -> torch.Tensor:
        """The predictions the stability test compares against (int32 [N],
        rewritten by every step's selection)."""
        o = stats_offsets(cfg)
        return self.stats[o["pred"]:o["pred"] + cfg.canvas_len * 4].view(torch.int32)

    def tile_stats(self, cfg: dg_config):
        """The last step's per-(row, 64-column tile) statistics as stored:
        (zmax, l = sum e^(y - m), s = sum e^(y - m)(y - m), argmax column),
        float32 [N][V/64] each (the argmax as int32)."""
        N, nt = cfg.canvas_len, cfg.vocab // TILE_V
        t = self.stats[:N * nt * 16].view(torch.float32).view(N, nt, 4)
        return t[..., 0], t[..., 1], t[..., 2], t[..., 3].contiguous().view(torch.int32)

    def weights(self, cfg: dg_config) -> torch.Tensor:
        """The stored per-column weights as float32 [N][V] (row-major): the
        bf16 numerators (probabilities up to a factor per (row, tile)) or the
        fp32 configuration's probabilities."""
        N, V = cfg.canvas_len, cfg.vocab
        if cfg.dtype == DG_BF16:
            return tiled_to_rows(self.probs.view(torch.bfloat16), N, V).float()
        return self.probs.view(torch.float32).view(N, V)

    def top(self, cfg: dg_config):
        """Each row's dominant token and its exact probability (last step)."""
        N = cfg.canvas_len
        o = stats_offsets(cfg)["top"]
        t = self.stats[o:o + N * 8].view(torch.float32).view(N, 2)
        return t[:, 0].contiguous().view(torch.int32), t[:, 1].contiguous()


def workspace(cfg: dg_config, max_prefill: int = 0, device="cuda", logits_dump=False):
    n = dg_workspace_bytes(cfg, max_prefill)
    if logits_dump:
        n = max(n, dg_test_logits_ws_bytes(cfg))
    if n == 0:
        raise DgError("dg_workspace_bytes", dg_validate_config(cfg))
    return torch.empty(n, dtype=torch.uint8, device=device)
