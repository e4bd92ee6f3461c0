"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch
(the rejected calls change no host-visible state)."""
import ctypes
import os
import re

import pytest
import torch

from uniform_state_discrete_dg_amd import binding as B
from uniform_state_discrete_dg_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgdenoise.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from uniform_state_discrete_dg_amd import build
        build.build()
    return B.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    # the binding wraps every declared entry point under the same name
    assert set(names) == set(B.SIGNATURES)


def test_abi_version_and_strings(lib):
    assert B.dg_abi_version() == 9
    for s in range(6):
        assert lib.dg_status_string(s)


def cfg_of(i, **kw):
    c = W.config(i)
    c.update(kw)
    return B.make_config(c)


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_shipped_configs_supported(lib, i):
    cfg = cfg_of(i)
    assert B.dg_validate_config(cfg) == B.DG_OK
    assert B.dg_workspace_bytes(cfg, 0) > 0
    assert B.dg_workspace_bytes(cfg, 1024) >= B.dg_workspace_bytes(cfg, 0)
    # float4 tile stats + float tile scale per (row, tile), float2 top, float
    # row scale and int32 previous prediction per row, then (256-byte aligned)
    # a uint8 exponent per (tile, 256 rows)
    nt = cfg.vocab // 64
    head = cfg.canvas_len * (nt * 20 + 8 + 4 + 4)
    assert B.dg_stats_bytes(cfg) == (head + 255) // 256 * 256 + nt * 256
    assert B.stats_offsets(cfg)["shift"] == (head + 255) // 256 * 256


@pytest.mark.parametrize("kw,st", [
    (dict(V=1000), B.DG_ERR_UNSUPPORTED),        # vocabulary not a power of two
    (dict(V=128), B.DG_ERR_UNSUPPORTED),         # smaller than one statistics tile
    (dict(N=257), B.DG_ERR_UNSUPPORTED),         # canvas longer than one workgroup
    (dict(hd=64), B.DG_ERR_UNSUPPORTED),         # bf16 kernels are head_dim 128
    (dict(d=1000), B.DG_ERR_UNSUPPORTED),        # K slices of 64
    (dict(d=4160), B.DG_ERR_UNSUPPORTED),        # row combine holds a d-row in 16 values per thread
    (dict(Hq=12, Hkv=8), B.DG_ERR_UNSUPPORTED),  # GQA groups must divide
    (dict(N=0), B.DG_ERR_INVALID_ARG),
    (dict(stable_rule=2), B.DG_ERR_INVALID_ARG),   # no such stability rule
    (dict(rms_eps=-1.0), B.DG_ERR_INVALID_ARG),
])
def test_config_rejections(lib, kw, st):
    c = W.config(2)
    c.update(kw)
    assert B.dg_validate_config(B.make_config(c)) == st
    assert B.dg_workspace_bytes(B.make_config(c), 0) == 0


def test_bad_enums(lib):
    cfg = cfg_of(2)
    cfg.dtype = 7
    assert B.dg_validate_config(cfg) == B.DG_ERR_INVALID_ARG
    cfg = cfg_of(2)
    cfg.accept_rule = 9
    assert B.dg_validate_config(cfg) == B.DG_ERR_INVALID_ARG
    cfg = cfg_of(2)
    cfg.sampler = 5
    assert B.dg_validate_config(cfg) == B.DG_ERR_INVALID_ARG
    cfg.sampler = B.DG_SAMPLER_MASKED
    assert B.dg_validate_config(cfg) == B.DG_OK
    cfg = cfg_of(2)
    cfg.candidate_rule = 2
    assert B.dg_validate_config(cfg) == B.DG_ERR_INVALID_ARG
    cfg.candidate_rule = B.DG_CANDIDATE_MULTINOMIAL
    assert B.dg_validate_config(cfg) == B.DG_OK
    # the draw needs no buffer of its own: sizes do not depend on the rule
    assert B.dg_stats_bytes(cfg) == B.dg_stats_bytes(cfg_of(2))
    assert B.dg_workspace_bytes(cfg, 0) == B.dg_workspace_bytes(cfg_of(2), 0)


def test_gumbel_export_rejects_bad_arguments(lib):
    assert lib.dg_test_gumbel(None, 4, 1, None, None) == B.DG_ERR_INVALID_ARG
    assert lib.dg_test_gumbel(FAKE, 4, 2, FAKE, None) == B.DG_ERR_INVALID_ARG
    assert lib.dg_test_gumbel(FAKE, -1, 0, FAKE, None) == B.DG_ERR_INVALID_ARG


FAKE = 0x10000  # a non-null address; validation must fail before it is used


def fake_weights():
    return B.dg_weights(*([FAKE] * 11))


def fake_canvas():
    return B.dg_canvas(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1, 5, 0)


def call_step(cfg, w, cache, cv, T, g, ws_bytes):
    return B.lib().dg_denoise_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache),
                                   ctypes.byref(cv), T, g, ctypes.c_void_p(FAKE), ws_bytes, None)


def test_denoise_step_validation(lib):
    cfg = cfg_of(2)
    need = B.dg_workspace_bytes(cfg, 0)
    cache = B.dg_kv_cache(FAKE, FAKE, 512, 512)
    cv = fake_canvas()
    w = fake_weights()
    cases = [
        (dict(T=0.0), B.DG_ERR_INVALID_ARG),
        (dict(T=-1.0), B.DG_ERR_INVALID_ARG),
        (dict(T=float("nan")), B.DG_ERR_INVALID_ARG),
        (dict(T=float("inf")), B.DG_ERR_INVALID_ARG),
        (dict(g=-0.5), B.DG_ERR_INVALID_ARG),
        (dict(g=float("nan")), B.DG_ERR_INVALID_ARG),
        (dict(ws=need - 1), B.DG_ERR_WORKSPACE),
    ]
    for kw, st in cases:
        r = call_step(cfg, w, cache, cv, kw.get("T", 1.0), kw.get("g", 8.0), kw.get("ws", need))
        assert r == st, (kw, r)
        assert (cv.step, cv.has_prev) == (3, 1)
    w2 = fake_weights()
    w2.E_pack = None
    assert call_step(cfg, w2, cache, cv, 1.0, 8.0, need) == B.DG_ERR_INVALID_ARG
    # the bf16 step reads only the packed copy: a null row-major E passes
    # validation (the call then fails only on the workspace, checked after)
    w4 = fake_weights()
    w4.E = None
    assert call_step(cfg, w4, cache, cv, 1.0, 8.0, need - 1) == B.DG_ERR_WORKSPACE
    # the fp32 step reads the row-major table
    cfg1 = cfg_of(1)
    w5 = fake_weights()
    w5.E = None
    assert call_step(cfg1, w5, cache, cv, 1.0, 8.0, B.dg_workspace_bytes(cfg1, 0)) == B.DG_ERR_INVALID_ARG
    cv2 = fake_canvas()
    cv2.status = None
    assert call_step(cfg, w, cache, cv2, 1.0, 8.0, need) == B.DG_ERR_INVALID_ARG
    bad_cache = B.dg_kv_cache(FAKE, FAKE, 600, 512)
    assert call_step(cfg, w, bad_cache, cv, 1.0, 8.0, need) == B.DG_ERR_INVALID_ARG
    # the masked sampler needs the [MASK] row, 16-byte aligned
    cfg_m = cfg_of(2)
    cfg_m.sampler = B.DG_SAMPLER_MASKED
    w3 = fake_weights()
    w3.mask_emb = None
    assert call_step(cfg_m, w3, cache, cv, 1.0, 8.0, need) == B.DG_ERR_INVALID_ARG
    w3.mask_emb = FAKE + 8
    assert call_step(cfg_m, w3, cache, cv, 1.0, 8.0, need) == B.DG_ERR_INVALID_ARG
    assert call_step(cfg_m, w, cache, cv, 1.0, 8.0, need - 1) == B.DG_ERR_WORKSPACE
    assert (cv.step, cv.has_prev) == (3, 1)


def test_static_scratch_step_validation(lib):
    """The entry point that allocates nothing rejects, before any device work:
    a configuration whose scratch need exceeds the library's array, and every
    argument error of dg_denoise_step."""
    def call(cfg, w, cache, cv, T, g):
        return B.lib().dg_denoise_step_static(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache),
                                              ctypes.byref(cv), T, g, None)
    cache = B.dg_kv_cache(FAKE, FAKE, 512, 512)
    cv, w = fake_canvas(), fake_weights()
    big = cfg_of(3, d=4096, F=65536)
    assert B.dg_validate_config(big) == B.DG_OK
    assert B.dg_workspace_bytes(big, 0) > B.DG_STATIC_SCRATCH_BYTES
    assert call(big, w, cache, cv, 1.0, 8.0) == B.DG_ERR_WORKSPACE
    for i in range(1, 6):   # the shipped configurations fit
        assert B.dg_workspace_bytes(cfg_of(i), 0) <= B.DG_STATIC_SCRATCH_BYTES
    cfg = cfg_of(2)
    for T, g in [(0.0, 8.0), (float("nan"), 8.0), (1.0, -1.0), (1.0, float("nan"))]:
        assert call(cfg, w, cache, cv, T, g) == B.DG_ERR_INVALID_ARG
    cv2 = fake_canvas()
    cv2.status = None
    assert call(cfg, w, cache, cv2, 1.0, 8.0) == B.DG_ERR_INVALID_ARG
    bad = cfg_of(2)
    bad.canvas_len = 0
    assert call(bad, w, cache, cv, 1.0, 8.0) == B.DG_ERR_INVALID_ARG
    assert (cv.step, cv.has_prev) == (3, 1)


def test_prefill_validation(lib):
    cfg = cfg_of(5)
    w = fake_weights()
    L = B.lib()
    cache = B.dg_kv_cache(FAKE, FAKE, 3000, 3072)
    r = L.dg_prefill_append(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache),
                            ctypes.c_void_p(FAKE), 256, None, ctypes.c_void_p(FAKE), 1 << 40, None)
    assert r == B.DG_ERR_CAPACITY and cache.length == 3000
    cache = B.dg_kv_cache(FAKE, FAKE, 0, 3072)
    need = B.dg_workspace_bytes(cfg, 1024)
    r = L.dg_prefill_append(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache),
                            ctypes.c_void_p(FAKE), 1024, None, ctypes.c_void_p(FAKE), need // 4, None)
    assert r == B.DG_ERR_WORKSPACE and cache.length == 0
    r = L.dg_prefill_append(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), None, 4, None,
                            ctypes.c_void_p(FAKE), need, None)
    assert r == B.DG_ERR_INVALID_ARG
    r = L.dg_prefill_append(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache),
                            ctypes.c_void_p(FAKE), -1, None, ctypes.c_void_p(FAKE), need, None)
    assert r == B.DG_ERR_INVALID_ARG
    # zero tokens is a no-op that succeeds without touching the device
    r = L.dg_prefill_append(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache),
                            None, 0, None, None, 0, None)
    assert r == B.DG_OK and cache.length == 0


def test_other_entry_point_validation(lib):
    L = B.lib()
    cfg = cfg_of(2)
    cv = fake_canvas()
    stop = ctypes.c_int32(0)
    assert L.dg_should_stop(ctypes.byref(cfg), ctypes.byref(cv), 3, None, None, None) == \
        B.DG_ERR_INVALID_ARG
    assert L.dg_pack_embedding(ctypes.byref(cfg), None, ctypes.c_void_p(FAKE), None) == \
        B.DG_ERR_INVALID_ARG
    cv.tokens = None
    assert L.dg_canvas_init(ctypes.byref(cfg), ctypes.byref(cv), 1, 0, None) == \
        B.DG_ERR_INVALID_ARG
    assert L.dg_test_copy(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 15, None) == \
        B.DG_ERR_INVALID_ARG
    assert L.dg_test_philox(None, 0, 0, None, -1, None) == B.DG_ERR_INVALID_ARG
    bad = cfg_of(2)
    bad.vocab = 1000
    assert L.dg_should_stop(ctypes.byref(bad), ctypes.byref(fake_canvas()), 3,
                            ctypes.byref(stop), None, None) == B.DG_ERR_UNSUPPORTED


def test_pack_and_probs_bytes(lib):
    """Packed table = E once, tiled (rows padded to 256); bf16 probs are one
    tiled block of 256 rows; fp32 probs are row-major; unsupported
    configurations give 0."""
    def tl(R, K):
        return (R + 255) // 256 * 256 * K
    for i in (2, 3):
        cfg = cfg_of(i)
        V, d = cfg.vocab, cfg.d_model
        assert B.dg_embedding_pack_bytes(cfg) == 2 * tl(V, d)
        assert B.dg_probs_bytes(cfg) == 2 * tl(cfg.canvas_len, V)
    cfg = cfg_of(1)
    assert B.dg_embedding_pack_bytes(cfg) == 0
    assert B.dg_probs_bytes(cfg) == 4 * cfg.canvas_len * cfg.vocab
    bad = cfg_of(2)
    bad.vocab = 1000
    assert B.dg_embedding_pack_bytes(bad) == 0 and B.dg_probs_bytes(bad) == 0


def test_tiled_layout_helpers():
    """rows_to_tiled / tiled_to_rows follow the documented formula: element
    (row, col) of X [R][K] sits at ((b * K/32 + s) * 1024 + p) * 8 + col % 8
    with b, r = divmod(row, 256), s = col // 32, c = (col % 32) // 8 and
    p = 4 r + (c ^ ((r // 4) % 4)); padding rows are zero."""
    import torch
    g = torch.Generator().manual_seed(0)
    X = torch.randn(300, 96, generator=g)
    T = B.rows_to_tiled(X)
    assert T.numel() == 512 * 96
    assert torch.equal(B.tiled_to_rows(T, 300, 96), X)
    for row in (0, 1, 5, 17, 255, 256, 299):
        for col in (0, 7, 8, 31, 32, 63, 95):
            b, r = divmod(row, 256)
            s, c = col // 32, (col % 32) // 8
            p = 4 * r + (c ^ ((r // 4) % 4))
            assert T[((b * 3 + s) * 1024 + p) * 8 + col % 8] == X[row, col]
    pad = B.tiled_to_rows(T, 512, 96)[300:]
    assert not pad.any()


def distinct_canvas(k, step=3, has_prev=1):
    base = FAKE * (k + 2)
    return B.dg_canvas(base, base + 0x100, base + 0x200, base + 0x300, base + 0x400, base + 0x500,
                       base + 0x600, step, has_prev, 5, k)


def call_batch(cfg, w, caches, cvs, T, g, ws_bytes, n=None):
    n = len(cvs) if n is None else n
    ca = (B.dg_kv_cache * max(len(caches), 1))(*caches)
    cv = (B.dg_canvas * max(len(cvs), 1))(*cvs)
    r = B.lib().dg_denoise_step_batch(ctypes.byref(cfg), ctypes.byref(w), ca, cv, n, T, g,
                                      ctypes.c_void_p(FAKE), ws_bytes, None)
    return r, [(c.step, c.has_prev) for c in cv[:len(cvs)]]


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_batch_workspace_bytes(lib, i):
    cfg = cfg_of(i)
    one = B.dg_workspace_bytes(cfg, 0)
    sizes = [B.dg_workspace_bytes_batch(cfg, n) for n in range(1, B.DG_MAX_BATCH + 1)]
    assert sizes[0] >= one - (cfg.canvas_len * cfg.vocab * 4 if cfg.dtype == B.DG_F32 else 0)
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    assert sizes[-1] > sizes[0]
    assert B.dg_workspace_bytes_batch(cfg, 0) == 0
    assert B.dg_workspace_bytes_batch(cfg, B.DG_MAX_BATCH + 1) == 0


def test_batch_step_validation(lib):
    cfg = cfg_of(2)
    w = fake_weights()
    need = B.dg_workspace_bytes_batch(cfg, 3)
    caches = [B.dg_kv_cache(FAKE, FAKE, 512, 512)] * 3
    ok = [distinct_canvas(k) for k in range(3)]
    before = [(3, 1)] * 3
    # a workspace one byte short: the whole call is rejected, nothing stepped
    assert call_batch(cfg, w, caches, ok, 1.0, 8.0, need - 1) == (B.DG_ERR_WORKSPACE, before)
    assert call_batch(cfg, w, caches, ok, 1.0, 8.0, need, n=0)[0] == B.DG_ERR_INVALID_ARG
    assert call_batch(cfg, w, caches, ok, 0.0, 8.0, need) == (B.DG_ERR_INVALID_ARG, before)
    assert call_batch(cfg, w, caches, ok, 1.0, float("nan"), need)[0] == B.DG_ERR_INVALID_ARG
    # mixed has_prev: the batch shares one self-conditioning pass
    mixed = [distinct_canvas(0), distinct_canvas(1, has_prev=0), distinct_canvas(2)]
    assert call_batch(cfg, w, caches, mixed, 1.0, 8.0, need)[0] == B.DG_ERR_INVALID_ARG
    # two canvases on the same buffers
    twin = [distinct_canvas(0), distinct_canvas(1), distinct_canvas(1)]
    assert call_batch(cfg, w, caches, twin, 1.0, 8.0, need) == (B.DG_ERR_INVALID_ARG, before)
    for field in ("tokens", "probs", "stats", "entropy", "argmax", "accept", "status"):
        shared = [distinct_canvas(0), distinct_canvas(1), distinct_canvas(2)]
        setattr(shared[2], field, getattr(shared[0], field))
        assert call_batch(cfg, w, caches, shared, 1.0, 8.0, need) == (B.DG_ERR_INVALID_ARG, before), field
    bad = [distinct_canvas(0), distinct_canvas(1), distinct_canvas(2)]
    bad[2].status = None
    assert call_batch(cfg, w, caches, bad, 1.0, 8.0, need)[0] == B.DG_ERR_INVALID_ARG
    over = [B.dg_kv_cache(FAKE, FAKE, 512, 512), B.dg_kv_cache(FAKE, FAKE, 600, 512),
            B.dg_kv_cache(FAKE, FAKE, 512, 512)]
    assert call_batch(cfg, w, over, ok, 1.0, 8.0, need)[0] == B.DG_ERR_INVALID_ARG
    many = [distinct_canvas(k) for k in range(B.DG_MAX_BATCH + 1)]
    many_c = [caches[0]] * len(many)
    big = B.dg_workspace_bytes_batch(cfg, B.DG_MAX_BATCH)
    assert call_batch(cfg, w, many_c, many, 1.0, 8.0, big)[0] == B.DG_ERR_INVALID_ARG


def test_fp8_table_config_and_sizes(lib):
    """The fp8 packed table: accepted for DG_BF16 with a scale exponent in
    [-32, 32], half the bytes of the bf16 pack, same workspace and canvas
    buffers; bad formats and exponents rejected."""
    for i in (2, 3, 4):
        cfg = cfg_of(i)
        c8 = cfg_of(i, table="fp8", table_exp=8)
        assert c8.table_format == B.DG_TABLE_FP8 and c8.table_exp == 8
        assert B.dg_validate_config(c8) == B.DG_OK
        assert 2 * B.dg_embedding_pack_bytes(c8) == B.dg_embedding_pack_bytes(cfg)
        assert B.dg_embedding_pack_bytes(c8) == cfg.vocab * cfg.d_model
        assert B.dg_workspace_bytes(c8, 0) == B.dg_workspace_bytes(cfg, 0)
        assert B.dg_probs_bytes(c8) == B.dg_probs_bytes(cfg)
    c8 = cfg_of(2, table="fp8", table_exp=33)
    assert B.dg_validate_config(c8) == B.DG_ERR_INVALID_ARG
    c8.table_exp = -33
    assert B.dg_validate_config(c8) == B.DG_ERR_INVALID_ARG
    c8.table_exp = -32
    assert B.dg_validate_config(c8) == B.DG_OK
    c8.table_format = 3
    assert B.dg_validate_config(c8) == B.DG_ERR_INVALID_ARG
    # the fp32 configuration ignores the table format (it reads E directly)
    c1 = cfg_of(1, table="fp8", table_exp=8)
    assert B.dg_validate_config(c1) == B.DG_OK
    assert B.dg_embedding_pack_bytes(c1) == 0


def test_fp8_grid_quantiser():
    """The quantised-table input: every entry is q 2^-exp with q an fp8 e4m3
    number (nearest even, saturating), idempotent, and exact in bf16."""
    import torch
    g = torch.Generator().manual_seed(3)
    E = (torch.randn(64, 256, generator=g) * 0.05).to(torch.bfloat16)
    Q = W.fp8_grid(E, 8)
    q = Q.float() * 256
    assert torch.equal(q.to(torch.float8_e4m3fn).float(), q)
    assert torch.equal(W.fp8_grid(Q, 8), Q)
    assert (Q.float() - E.float()).abs().max().item() <= 0.0625 * E.float().abs().max().item() + 2 ** -17
    big = torch.tensor([[1e6, -1e6, 0.0, 3.0]], dtype=torch.bfloat16)
    assert W.fp8_grid(big, 0).float().tolist() == [[448.0, -448.0, 0.0, 3.0]]


def test_fp4_table_config_and_sizes(lib):
    """The fp4 packed table: accepted for DG_BF16 with table_exp 0 (its
    scales are per block); codes are half a byte per element of E and every
    1024 elements add one scale byte; same workspace and canvas buffers."""
    for i in (2, 3, 4):
        cfg = cfg_of(i)
        c4 = cfg_of(i, table="fp4")
        assert c4.table_format == B.DG_TABLE_FP4 and c4.table_exp == 0
        assert B.dg_validate_config(c4) == B.DG_OK
        n = cfg.vocab * cfg.d_model  # d multiple of 256 here: no padding rows
        assert B.dg_embedding_pack_bytes(c4) == n // 2 + n // 1024
        assert B.dg_workspace_bytes(c4, 0) == B.dg_workspace_bytes(cfg, 0)
        assert B.dg_probs_bytes(c4) == B.dg_probs_bytes(cfg)
    c4 = cfg_of(2, table="fp4")
    c4.table_exp = 1
    assert B.dg_validate_config(c4) == B.DG_ERR_INVALID_ARG
    c1 = cfg_of(1, table="fp4")
    assert B.dg_validate_config(c1) == B.DG_OK
    assert B.dg_embedding_pack_bytes(c1) == 0


def test_fp4_grid_quantiser():
    """The block-scaled fp4 input: each 32 x 32 block holds code values
    times one power of two, the block's largest magnitude maps into
    [4, 6] (saturating above 6), rounding is to the nearest value with ties
    to the even code, the grid is idempotent and exact in bf16."""
    import torch
    g = torch.Generator().manual_seed(5)
    E = (torch.randn(64, 96, generator=g) * 0.05).to(torch.bfloat16)
    Q = W.fp4_grid(E)
    u = W.fp4_scale_bytes(E)
    assert u.shape == (2, 3)
    full = u.repeat_interleave(32, 0).repeat_interleave(32, 1)
    y = Q.float() * torch.pow(2.0, (127 - full).float())
    assert set(y.abs().unique().tolist()) <= set(W.FP4_VALUES)
    amax = E.float().abs().view(2, 32, 3, 32).amax(dim=(1, 3))
    r = amax * torch.pow(2.0, (127 - u).float())
    assert bool(((r >= 4) & (r < 8)).all())
    assert torch.equal(W.fp4_grid(Q), Q)
    assert torch.equal(W.fp4_scale_bytes(Q), u)
    # error bound: half the largest gap (2 units of 2^(u-127)) or the saturation
    err = (Q.float() - E.float()).abs() * torch.pow(2.0, (127 - full).float())
    assert err.max().item() <= 2.0
    # hand-worked block: scale byte 127 (largest magnitude 4.5, floor(log2) = 2)
    blk = torch.zeros(32, 32)
    vals = [4.5, 0.25, 0.26, -0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, -7.9, -0.1, 0.74]
    blk[0, :len(vals)] = torch.tensor(vals)
    want = [4.0, 0.0, 0.5, -1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -6.0, 0.0, 0.5]
    got = W.fp4_grid(blk.to(torch.bfloat16)).float()[0, :len(vals)].tolist()
    assert W.fp4_scale_bytes(blk).item() == 127
    assert got == want
    codes = W.fp4_codes(blk)[0, :len(vals)].tolist()
    assert codes == [6, 0, 1, 8 | 2, 2, 4, 4, 6, 6, 7, 8 | 7, 0, 1]   # -0.1 -> +0
    # an all-zero block has scale byte 127; tiny and huge blocks clamp
    z = torch.zeros(32, 32)
    assert W.fp4_scale_bytes(z).item() == 127
    assert W.fp4_scale_bytes(torch.full((32, 32), 2.0 ** -130)).item() == 2
    assert W.fp4_scale_bytes(torch.full((32, 32), 2.0 ** 126)).item() == 126 - 2 + 127


def test_cache_split_pair_roundtrip():
    """The host's split-pair form of a bf16 model's KV cache: hi = bf16(x)
    (round to nearest even), lo = bf16(x - hi); hi + lo keeps 16
    significant bits, and a bf16 value has lo = 0."""
    g = torch.Generator().manual_seed(7)
    x = torch.randn(3, 17, 128, generator=g) * torch.exp(torch.randn(3, 17, 128, generator=g) * 4)
    p = B.split_pair(x)
    assert p.shape == (2, 3, 17, 128) and p.dtype == torch.bfloat16
    assert torch.equal(p[0], x.to(torch.bfloat16))
    assert torch.equal(p[1], (x - p[0].float()).to(torch.bfloat16))
    y = B.join_pair(p)
    assert ((y - x).abs() <= x.abs() * 2.0 ** -16).all()
    xb = x.to(torch.bfloat16).float()
    pb = B.split_pair(xb)
    assert not pb[1].float().any() and torch.equal(B.join_pair(pb), xb)
