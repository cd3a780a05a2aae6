"""The C ABI library loads, exports every symbol include/ec.h declares, and rejects bad
arguments before touching the GPU (CPU-only: no compute call is made)."""
import ctypes as C
import math
import os
import re

import pytest

from entropy_guided_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "ec.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ec_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libec.so is not built; run `python -m entropy_guided_kv_amd.build`")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ec.h but not exported"
    assert set(_lib.EXPORTS) <= set(names)


def test_library_resolves_every_symbol_at_load():
    # RTLD_NOW: an unresolved symbol (e.g. a kernel stub the compiler dropped) fails here
    C.CDLL(_lib.LIB_PATH, mode=os.RTLD_NOW)


def test_version_and_error_string(lib):
    assert lib.ec_version() == 10200
    assert isinstance(lib.ec_last_error(), bytes)


def test_workspace_queries_are_host_only(lib):
    # single-launch reduction: four tagged 64-bit words per slice state, four slices per row
    # at 64 rows of 126464, plus one published entropy word per row
    assert lib.ec_entropy_max_workspace_size(64, 126464) >= (64 * 4 * 4 + 64) * 8
    assert lib.ec_entropy_max_workspace_size(1, 126464) >= (62 * 4 + 1) * 8
    assert lib.ec_entropy_max_workspace_size(0, 10) == 0
    assert lib.ec_partial_attn_workspace_size(1, 1024, 32, 128) > 0  # split-L partials
    assert lib.ec_partial_attn_workspace_size(1024, 1024, 32, 128) == 0
    assert lib.ec_state_plan_words(1024, 16) >= 8 + 16 + 4 * 1024
    assert lib.ec_state_plan_words(0, 16) == 0


def test_attention_plan_query(lib):
    """Host-only launch plan of the bf16 attention at 32 heads and L = 1024: the 64-query shape
    for the rows of a skip step, over whole key ranges from a few hundred rows and with the
    keys split below that (fewer query tiles, each workgroup's chain of K/V tiles shortened),
    the 128-query shape at refresh size, and the workspace query agreeing."""
    def plan(r, L, H):
        qt, sp = C.c_int32(0), C.c_int32(0)
        assert lib.ec_partial_attn_plan(r, L, H, 128, C.byref(qt), C.byref(sp)) == _lib.EC_OK
        return qt.value, sp.value
    for r in (256, 384, 512):
        assert plan(r, 1024, 32) == (64, 1)
    for r in (96, 128, 147):
        qt, sp = plan(r, 1024, 32)
        assert qt == 64 and sp > 1
    assert plan(1024, 1024, 32) == (128, 1)
    assert plan(4096, 4096, 32)[0] == 128
    qt, sp = plan(17, 1024, 32)
    assert qt == 64 and sp > 1  # one query tile per head: the keys are split to fill the CUs
    for r, L, H in ((1, 1024, 32), (17, 1024, 32), (256, 1024, 32), (1024, 1024, 32), (40, 700, 8),
                    (3, 1250, 2), (1, 33, 1)):
        qt, sp = plan(r, L, H)
        ws = lib.ec_partial_attn_workspace_size(r, L, H, 128)
        assert (ws > 0) == (sp > 1)
        if sp > 1:
            assert ws >= sp * r * H * 130 * 4
    qt, sp = C.c_int32(0), C.c_int32(0)
    assert lib.ec_partial_attn_plan(16, 1024, 32, 64, C.byref(qt), C.byref(sp)) == _lib.EC_ERR_UNSUPPORTED
    assert lib.ec_partial_attn_plan(0, 1024, 32, 128, C.byref(qt), C.byref(sp)) == _lib.EC_ERR_ARG
    assert lib.ec_partial_attn_plan(16, 1024, 32, 128, None, C.byref(sp)) == _lib.EC_ERR_ARG


def test_bf16_attention_cases_cover_both_shapes():
    """Host only: the bf16 cases of the attention parity test reach both workgroup shapes, with and without key
    splits, every merge width from 2 to 16, and caches shorter than one tile."""
    import entropy_guided_kv_amd as ek
    from tests.test_gpu_attn_scatter import BF16_ATTN_CASES
    plans = {c: ek.ec_partial_attn_plan(*c) for c in BF16_ATTN_CASES}
    narrow = {sp for (qt, sp) in plans.values() if qt == 64}
    wide = {sp for (qt, sp) in plans.values() if qt == 128}
    assert 1 in narrow and len(narrow - {1}) >= 4, plans
    assert 1 in wide and len(wide - {1}) >= 8, plans
    assert set(range(2, 17)) <= (narrow | wide), plans
    assert plans[(150, 65, 4)] == (64, 1) and plans[(100, 97, 8)] == (64, 1)
    assert plans[(7, 29, 3)] == (128, 1) and plans[(1024, 1024, 32)] == (128, 1)


def _model_desc(dtype=_lib.EC_BF16, d=4096, H=32, Dh=128, F=12288, V=126464, n_layers=32):
    lw = (_lib.ec_layer_weights * n_layers)()
    for i in range(n_layers):
        for f in ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            setattr(lw[i], f, 0x1000)  # non-null; never dereferenced by the size queries
    m = _lib.ec_model_desc()
    m.struct_size = C.sizeof(_lib.ec_model_desc)
    m.dtype = dtype
    m.n_layers, m.d_model, m.n_heads, m.head_dim, m.ffn_dim, m.vocab = n_layers, d, H, Dh, F, V
    m.rms_eps = 1e-5
    m.embed = m.final_norm = m.lm_head = m.rope_cos = m.rope_sin = 0x1000
    m.layers = C.cast(lw, C.POINTER(_lib.ec_layer_weights))
    m.rope_max_pos = 4096
    m.weight_layout = _lib.EC_LAYOUT_PACKED if dtype == _lib.EC_BF16 else _lib.EC_LAYOUT_PLAIN
    return m, lw


def _params(L=1024, P=768, k=16, n=1, B=32, tau=1.0, mask=126463):
    p = _lib.ec_params()
    p.struct_size = C.sizeof(_lib.ec_params)
    p.tau, p.k_recent, p.tokens_per_step, p.block_len = tau, k, n, B
    p.prompt_len, p.seq_len, p.mask_id = P, L, mask
    return p


def test_step_workspace_size_for_the_8b_config(lib):
    m, _keep = _model_desc()
    p = _params()
    ws = lib.ec_step_workspace_size(C.byref(m), C.byref(p))
    # h fp32 + 3 bf16 [L, d] buffers + SwiGLU [L, F] + logits [B, V] at least
    assert ws >= 1024 * 4096 * 4 + 3 * 1024 * 4096 * 2 + 1024 * 12288 * 2 + 32 * 126464 * 2
    assert ws < 512 << 20


def test_unsupported_shapes_and_bad_params_are_rejected(lib):
    m, _keep = _model_desc(Dh=64, H=64)  # bf16 path needs head_dim 128
    p = _params()
    assert lib.ec_step_workspace_size(C.byref(m), C.byref(p)) == 0
    m2, _keep2 = _model_desc()
    bad = _params(n=0)
    assert lib.ec_step_workspace_size(C.byref(m2), C.byref(bad)) == 0
    bad = _params(tau=math.nan)
    assert lib.ec_step_workspace_size(C.byref(m2), C.byref(bad)) == 0
    # bf16 models must come in the packed weight layout
    m3, _keep3 = _model_desc()
    m3.weight_layout = _lib.EC_LAYOUT_PLAIN
    assert lib.ec_step_workspace_size(C.byref(m3), C.byref(_params())) == 0
    assert b"weight_layout" in lib.ec_last_error()
    # device arrays must be 16-byte aligned (the kernels move 16-byte vectors)
    m4, _keep4 = _model_desc()
    m4.final_norm = 0x1008
    assert lib.ec_step_workspace_size(C.byref(m4), C.byref(_params())) == 0
    assert b"aligned" in lib.ec_last_error()
    m5, keep5 = _model_desc()
    keep5[3].w_down = 0x1004
    assert lib.ec_step_workspace_size(C.byref(m5), C.byref(_params())) == 0
    assert b"layer 3" in lib.ec_last_error()


def test_shapes_beyond_the_32bit_buffer_range_are_rejected(lib):
    """The bf16 kernels address weights, activations and caches with 32-bit byte offsets:
    a matrix over 2 GiB is refused up front instead of wrapping."""
    ok, _k0 = _model_desc()
    assert lib.ec_step_workspace_size(C.byref(ok), C.byref(_params())) > 0
    # LM head of 262144 x 4096 bf16 = 2 GiB: one byte past the range
    big_v, _k1 = _model_desc(V=262144)
    assert lib.ec_step_workspace_size(C.byref(big_v), C.byref(_params(mask=0))) == 0
    assert b"2 GiB" in lib.ec_last_error()
    # just inside: 262016 x 4096 x 2 bytes < 2^31
    fits_v, _k2 = _model_desc(V=262016)
    assert lib.ec_step_workspace_size(C.byref(fits_v), C.byref(_params(mask=0))) > 0
    # activations [L, F]: 65536 rows of F = 16384 bf16 = 2 GiB
    wide, _k3 = _model_desc(F=16384)
    wide.rope_max_pos = 1 << 17
    assert lib.ec_step_workspace_size(C.byref(wide), C.byref(_params(L=65536, P=65536 - 256))) == 0
    assert b"rows" in lib.ec_last_error()
    # fp32 models take the 64-bit-indexed kernels: no such limit
    f32, _k4 = _model_desc(dtype=_lib.EC_F32, V=262144)
    assert lib.ec_step_workspace_size(C.byref(f32), C.byref(_params(mask=0))) > 0


def test_argument_errors_return_before_any_gpu_work(lib):
    E = _lib
    # bad dtype / sizes: rejected by the host checks, nothing is launched
    assert lib.ec_entropy_max(None, 7, 1, 10, 10, None, 0, None, None, None, None, None, 0, None) == E.EC_ERR_DTYPE
    assert lib.ec_entropy_max(None, E.EC_BF16, 1, 10, 5, None, 0, None, None, None, None, None, 0, None) == E.EC_ERR_ARG
    assert lib.ec_entropy_max(0x1000, E.EC_BF16, 4, 10, 10, None, 0, 0x1000, 0x1000, 0x1000, None, None, 0, None) == E.EC_ERR_WORKSPACE
    assert lib.ec_cache_scatter(None, None, 10, 8, E.EC_F32, None, None, None, 3, None) == E.EC_ERR_ARG
    assert lib.ec_cache_scatter(None, None, 10, 8, E.EC_F32, None, None, None, 0, None) == E.EC_OK
    assert lib.ec_partial_attn(None, None, None, 4, 16, 2, 128, 1.0, E.EC_BF16, None, None, 0, None) == E.EC_ERR_ARG
    # sizes past the kernels' 32-bit buffer offsets (2 GiB per cache) and head sizes the bf16
    # kernel does not take: refused before anything is enqueued (fake pointers, never read)
    big = lib.ec_partial_attn_workspace_size(1, 1 << 17, 128, 128)
    assert lib.ec_partial_attn(0x1000, 0x1000, 0x1000, 1, 1 << 17, 128, 128, 1.0, E.EC_BF16, 0x1000, 0x1000,
                               big, None) == E.EC_ERR_UNSUPPORTED
    assert b"2 GiB" in lib.ec_last_error()
    assert lib.ec_partial_attn(0x1000, 0x1000, 0x1000, 4, 16, 2, 64, 1.0, E.EC_BF16, 0x1000, None, 0,
                               None) == E.EC_ERR_UNSUPPORTED
    assert lib.ec_step(None, None, None, None, None, 0, None, None) == E.EC_ERR_ARG
    assert b"model" in lib.ec_last_error()
    m, _keep = _model_desc()
    assert lib.ec_forward(C.byref(m), None, None, None, 0, None, 0, None, None, None, 0, None) == E.EC_ERR_ARG
    assert lib.ec_rope_table(None, None, 16, 128, 10000.0, None) == E.EC_ERR_ARG
    # packing: bad dtype, missing inputs, sizes the layout cannot take
    assert lib.ec_pack_weights(5, 256, 128, 512, None, None, None, None, None, None) == E.EC_ERR_DTYPE
    assert lib.ec_pack_weights(E.EC_BF16, 256, 128, 512, None, None, None, 0x1000, None, None) == E.EC_ERR_ARG
    assert lib.ec_pack_weights(E.EC_BF16, 256, 48, 512, 0x1000, None, None, 0x1000, None, None) == E.EC_ERR_ARG
    assert lib.ec_pack_weights(E.EC_BF16, 256, 128, 520, None, 0x1000, 0x1000, None, 0x1000, None) == E.EC_ERR_ARG
    assert lib.ec_pack_weights(E.EC_BF16, 256, 128, 512, None, None, None, None, None, None) == E.EC_OK
    st = _lib.ec_state()
    st.struct_size = C.sizeof(_lib.ec_state)
    assert lib.ec_state_reset(C.byref(st), C.byref(_params()), None) == E.EC_ERR_ARG
    # batched step: sequence count and null arrays are rejected before any GPU work
    assert lib.ec_step_batch(C.byref(m), 0, None, None, C.byref(_params()), None, 0, None, None) == E.EC_ERR_ARG
    assert lib.ec_step_batch(C.byref(m), E.EC_MAX_SEQ + 1, None, None, C.byref(_params()), None, 0, None,
                             None) == E.EC_ERR_ARG
    assert lib.ec_step_batch(C.byref(m), 2, None, None, C.byref(_params()), None, 0, None, None) == E.EC_ERR_ARG
    assert lib.ec_step_batch_workspace_size(C.byref(m), 0, C.byref(_params())) == 0
    ws1 = lib.ec_step_batch_workspace_size(C.byref(m), 1, C.byref(_params()))
    ws4 = lib.ec_step_batch_workspace_size(C.byref(m), 4, C.byref(_params()))
    assert ws1 > 0 and ws4 > 3 * ws1 // 2


def test_noalloc_entropy_rejects_before_any_gpu_work(lib):
    """ec_entropy_max_noalloc: bad arguments and inputs whose scratch need exceeds the
    library's array are rejected on the host, before any device call."""
    rows, V = 40000, 4096
    assert lib.ec_entropy_max_workspace_size(rows, V) > _lib.EC_ENTROPY_NOALLOC_SCRATCH_BYTES
    p = 0x1000  # never dereferenced: every case fails its checks first
    assert lib.ec_entropy_max_noalloc(p, _lib.EC_BF16, rows, V, V, None, 0, p, p, p, p, None) == _lib.EC_ERR_UNSUPPORTED
    assert lib.ec_entropy_max_noalloc(p, 7, 4, V, V, None, 0, p, p, p, p, None) == _lib.EC_ERR_DTYPE
    assert lib.ec_entropy_max_noalloc(p, _lib.EC_BF16, 4, V, V - 1, None, 0, p, p, p, p, None) == _lib.EC_ERR_ARG
    assert lib.ec_entropy_max_noalloc(None, _lib.EC_BF16, 4, V, V, None, 0, p, p, p, p, None) == _lib.EC_ERR_ARG
