"""Host-side tests of the C ABI (no GPU needed): exported symbols, validation rules
and status codes.  Every call here fails validation before anything touches a device,
so fake non-null pointers are safe."""
import ctypes
import re

import pytest

import head_latent_attention_dkv_amd as M
import mla_synth as S

FAKE = 0x1000  # non-null, never dereferenced: validation fails first


def _lib_or_skip():
    try:
        return M.lib()
    except RuntimeError as e:  # library not built
        pytest.skip(str(e))


def test_exports_match_header():
    L = _lib_or_skip()
    with open(M.HEADER_PATH) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(mla_\w+)\s*\(", text, flags=re.M))
    assert declared == set(M.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def _declaration_comments(text):
    """{entry point: the block comment right above its declaration}"""
    out = {}
    for m in re.finditer(r"/\*((?:[^*]|\*(?!/))*)\*/\s*(?:const\s+)?\w+\*?\s+(mla_\w+)\s*\(", text):
        out[m.group(2)] = m.group(1)
    return out


def test_every_declaration_cites_its_source():
    """Each entry point's comment names the page section that defines the operation (a
    [... page] tag followed by a ``function`` or ``Class.method``), or says that it is the
    library's own."""
    with open(M.HEADER_PATH) as f:
        text = f.read()
    comments = _declaration_comments(text)
    assert set(comments) == set(M.EXPORTS)
    cite = re.compile(r"\[(MLA|MLRA|DSV2|CCA) page\]\s+``[\w.]+``")
    for name, body in comments.items():
        flat = " ".join(re.sub(r"(?m)^\s*\*", " ", body).split())
        assert cite.search(flat) or "library's own" in flat, f"{name}: no source passage"


def test_status_strings():
    _lib_or_skip()
    for code in range(7):
        assert M.mla_status_str(code).startswith("MLA_")
    assert M.mla_status_str(0) == "MLA_OK"


@pytest.mark.parametrize("name", list(S.CONFIGS))
def test_configs_validate(name):
    _lib_or_skip()
    d = M.dims_from_cfg(S.CONFIGS[name])
    assert M.mla_validate(d) == M.MLA_OK
    cfg = S.CONFIGS[name]
    if cfg.mode == "prefill":
        assert M.mla_workspace_bytes(d, M.MLA_OP_PREFILL, cfg.batch, cfg.seq) > 0
        assert M.mla_workspace_bytes(d, M.MLA_OP_PREFILL_ATTENTION, cfg.batch, cfg.seq) > 0
    else:
        assert M.mla_workspace_bytes(d, M.MLA_OP_DECODE, cfg.batch, cfg.seq) > 0
        assert M.mla_workspace_bytes(d, M.MLA_OP_DECODE_ATTENTION, cfg.batch, cfg.seq) > 0
    assert M.mla_workspace_bytes(d, M.MLA_OP_CACHE_APPEND, cfg.batch, cfg.seq) == 0


def _dims(**kw):
    base = dict(family="decoupled", d_model=64, n_heads=4, d_nope=16, d_rope=8, r_kv=32, r_q=16)
    base.update(kw)
    return M.make_dims(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads=0), M.MLA_ERR_INVALID_ARG),
    (dict(r_kv=-1), M.MLA_ERR_INVALID_ARG),
    (dict(d_rope=7), M.MLA_ERR_SHAPE),                           # odd rotary dim
    (dict(family="mlra", d_rope=0, r_kv=30, n_latent_heads=4), M.MLA_ERR_SHAPE),   # L does not divide r
    (dict(family="mlra", d_rope=0, n_heads=6, n_latent_heads=4), M.MLA_ERR_SHAPE),  # L does not divide H
    (dict(n_latent_heads=2), M.MLA_ERR_UNSUPPORTED),             # partitioned latent with RoPE
    (dict(d_nope=12), M.MLA_ERR_UNSUPPORTED),                    # 8-element staging chunks
    (dict(d_rope=128), M.MLA_ERR_UNSUPPORTED),
    (dict(family="fullrope", d_rope=0, d_nope=48), M.MLA_ERR_UNSUPPORTED),  # 128 % 48 != 0
    (dict(r_kv=1024), M.MLA_ERR_UNSUPPORTED),                    # latent block > 512
])
def test_validate_rejects(kw, code):
    _lib_or_skip()
    assert M.mla_validate(_dims(**kw)) == code


def test_validate_rejects_bad_enums_and_scale():
    _lib_or_skip()
    d = _dims()
    d.dtype = 7
    assert M.mla_validate(d) == M.MLA_ERR_INVALID_ARG
    d = _dims()
    d.rope_mode = 9
    assert M.mla_validate(d) == M.MLA_ERR_INVALID_ARG
    d = _dims()
    d.softmax_scale = float("nan")
    assert M.mla_validate(d) == M.MLA_ERR_INVALID_ARG
    d = _dims()
    d.d_v = 8
    assert M.mla_validate(d) == M.MLA_ERR_UNSUPPORTED
    assert M.lib().mla_validate(None) == M.MLA_ERR_INVALID_ARG


def _weights_all():
    return M.mla_weights(*([FAKE] * 9))


def test_entry_points_report_errors_before_launch():
    L = _lib_or_skip()
    d = _dims()
    w = _weights_all()
    cache = M.mla_cache(FAKE, FAKE, 2, 16)
    by = ctypes.byref
    # capacity: batch beyond max_batch, positions beyond max_seq
    assert L.mla_cache_append(by(d), by(w), FAKE, 3, 1, FAKE, 0, by(cache), None) == M.MLA_ERR_CAPACITY
    assert L.mla_cache_append(by(d), by(w), FAKE, 2, 4, FAKE, 13, by(cache), None) == M.MLA_ERR_CAPACITY
    assert L.mla_decode(by(d), by(w), FAKE, 2, FAKE, 16, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_CAPACITY
    assert L.mla_prefill(by(d), by(w), FAKE, 2, 17, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_CAPACITY
    assert L.mla_decode_attention(by(d), FAKE, FAKE, 3, FAKE, 4, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_CAPACITY
    assert L.mla_decode_attention(by(d), FAKE, FAKE, 2, FAKE, 16, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_CAPACITY
    # null pointers
    assert L.mla_cache_append(by(d), by(w), None, 2, 1, FAKE, 0, by(cache), None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_decode(by(d), by(w), FAKE, 2, None, 4, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_INVALID_ARG
    w_missing = _weights_all()
    w_missing.w_kr = None
    assert L.mla_cache_append(by(d), by(w_missing), FAKE, 2, 1, FAKE, 0, by(cache), None) == M.MLA_ERR_INVALID_ARG
    no_kr = M.mla_cache(FAKE, None, 2, 16)
    assert L.mla_cache_append(by(d), by(w), FAKE, 2, 1, FAKE, 0, by(no_kr), None) == M.MLA_ERR_INVALID_ARG
    # workspace too small
    need = M.mla_workspace_bytes(d, M.MLA_OP_DECODE, 2, 8)
    assert need > 0
    assert L.mla_decode(by(d), by(w), FAKE, 2, FAKE, 8, by(cache), FAKE, FAKE, need - 1, None) == M.MLA_ERR_WORKSPACE
    assert L.mla_decode(by(d), by(w), FAKE, 2, FAKE, 8, by(cache), FAKE, None, need, None) == M.MLA_ERR_WORKSPACE
    need = M.mla_workspace_bytes(d, M.MLA_OP_PREFILL, 2, 16)
    assert L.mla_prefill(by(d), by(w), FAKE, 2, 16, None, FAKE, FAKE, need - 1, None) == M.MLA_ERR_WORKSPACE
    # continued prefill: capacity (start_pos + T beyond max_seq, batch beyond max_batch),
    # null pointers, negative start, workspace sized for start_pos + T
    assert L.mla_prefill_chunk(by(d), by(w), FAKE, 2, 4, 13, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_CAPACITY
    assert L.mla_prefill_chunk(by(d), by(w), FAKE, 3, 4, 0, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_CAPACITY
    assert L.mla_prefill_chunk(by(d), by(w), None, 2, 4, 0, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_prefill_chunk(by(d), by(w), FAKE, 2, 4, -1, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_INVALID_ARG
    assert L.mla_prefill_chunk(by(d), by(w), FAKE, 2, 4, 8, None, FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_INVALID_ARG
    need = M.mla_workspace_bytes(d, M.MLA_OP_PREFILL_CHUNK, 2, 12)
    assert need > M.mla_workspace_bytes(d, M.MLA_OP_PREFILL, 2, 12)
    assert L.mla_prefill_chunk(by(d), by(w), FAKE, 2, 4, 8, by(cache), FAKE, FAKE, need - 1, None) == M.MLA_ERR_WORKSPACE
    # decode of the half-split family is not absorbable
    dr = _dims(family="fullrope", d_rope=0, d_nope=16)
    assert L.mla_decode(by(dr), by(w), FAKE, 2, FAKE, 8, by(cache), FAKE, FAKE, 1 << 30, None) == M.MLA_ERR_UNSUPPORTED
    assert M.mla_workspace_bytes(dr, M.MLA_OP_DECODE, 2, 8) == 0


def test_workspace_grows_with_problem():
    _lib_or_skip()
    d = M.dims_from_cfg(S.CONFIGS["dsv2_decode"])
    a = M.mla_workspace_bytes(d, M.MLA_OP_DECODE, 64, 4096)
    b = M.mla_workspace_bytes(d, M.MLA_OP_DECODE, 64, 8192)
    c = M.mla_workspace_bytes(d, M.MLA_OP_DECODE_ATTENTION, 64, 4096)
    assert 0 < c < a <= b
    assert M.mla_workspace_bytes(d, 99, 64, 4096) == 0
    assert M.mla_workspace_bytes(d, M.MLA_OP_DECODE, 0, 4096) == 0


# ---------------------------------------------------------------------------
# Compressed convolutional attention entry points
# ---------------------------------------------------------------------------
def _cca(**kw):
    base = dict(d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, num_conv_layers=2, conv_kernel_seq=4,
                conv_kernel_ch=3, qk_mean=1, value_shift=1, dtype=M.MLA_DTYPE_BF16, rope_base=10000.0)
    base.update(kw)
    return M.mla_cca_dims(*[base[f] for f, _ in M.mla_cca_dims._fields_])


@pytest.mark.parametrize("name", list(S.CCA_CONFIGS))
def test_cca_configs_validate(name):
    _lib_or_skip()
    cfg = S.CCA_CONFIGS[name]
    d = M.cca_dims_from_cfg(cfg)
    assert M.mla_cca_validate(d) == M.MLA_OK
    assert M.mla_cca_workspace_bytes(d, cfg.batch, cfg.seq) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=66), M.MLA_ERR_SHAPE),                 # E not divisible by the heads
    (dict(n_kv_heads=3), M.MLA_ERR_SHAPE),               # key heads do not divide query heads
    (dict(head_dim=15), M.MLA_ERR_SHAPE),                # odd latent head width (RoPE)
    (dict(num_conv_layers=3), M.MLA_ERR_SHAPE),          # 0, 1 or 2 convolutions
    (dict(n_kv_heads=1), M.MLA_ERR_SHAPE),               # value shift needs an even key-head count
    (dict(head_dim=256), M.MLA_ERR_UNSUPPORTED),
    (dict(conv_kernel_seq=9), M.MLA_ERR_UNSUPPORTED),
    (dict(n_heads=0), M.MLA_ERR_INVALID_ARG),
    (dict(dtype=9), M.MLA_ERR_INVALID_ARG),
])
def test_cca_validate_rejects(kw, code):
    _lib_or_skip()
    assert M.mla_cca_validate(_cca(**kw)) == code


def test_cca_validate_accepts_variants():
    _lib_or_skip()
    assert M.mla_cca_validate(_cca(n_kv_heads=1, value_shift=0)) == M.MLA_OK      # odd key heads, no shift
    assert M.mla_cca_validate(_cca(num_conv_layers=0, conv_kernel_seq=0, conv_kernel_ch=0)) == M.MLA_OK
    assert M.mla_cca_validate(_cca(n_kv_heads=4)) == M.MLA_OK                       # CCA


def test_cca_prefill_errors_before_launch():
    L = _lib_or_skip()
    d = _cca()
    w = M.mla_cca_weights(FAKE, FAKE, FAKE, FAKE, FAKE, 0.0)
    n = M.mla_cca_workspace_bytes(d, 2, 8)
    assert n > 0

    def call(dims, wts, x=FAKE, B=2, S_=8, y=FAKE, ws=FAKE, nb=n):
        return L.mla_cca_prefill(ctypes.byref(dims), ctypes.byref(wts) if wts is not None else None, x, B, S_, y,
                                 ws, nb, None)

    assert call(d, w, nb=n - 1) == M.MLA_ERR_WORKSPACE
    assert call(d, w, ws=None) == M.MLA_ERR_WORKSPACE
    assert call(d, w, x=None) == M.MLA_ERR_INVALID_ARG
    assert call(d, None) == M.MLA_ERR_INVALID_ARG
    assert call(d, M.mla_cca_weights(FAKE, FAKE, FAKE, None, FAKE, 0.0)) == M.MLA_ERR_INVALID_ARG   # conv filters
    assert call(d, M.mla_cca_weights(FAKE, FAKE, FAKE, FAKE, FAKE, float("nan"))) == M.MLA_ERR_INVALID_ARG
    assert call(d, w, S_=0) == M.MLA_ERR_INVALID_ARG
    assert call(_cca(head_dim=15), w) == M.MLA_ERR_SHAPE


def test_noalloc_decode_attention_rejects_before_any_device_call():
    """The no-allocation entry point checks its fixed scratch size on the host: a shape that
    needs more is refused with MLA_ERR_WORKSPACE before anything touches a device."""
    L = _lib_or_skip()
    cfg = S.CONFIGS["dsv2_decode"]
    d = M.dims_from_cfg(cfg)
    cap = M.mla_decode_attention_noalloc_max_bytes()
    assert cap == 96 << 20
    assert M.mla_workspace_bytes(d, M.MLA_OP_DECODE_ATTENTION, 64, 4096) <= cap    # the decode workload fits
    B, max_ctx = 512, 100
    assert M.mla_workspace_bytes(d, M.MLA_OP_DECODE_ATTENTION, B, max_ctx) > cap
    c = M.mla_cache(FAKE, FAKE, B, max_ctx + 1)
    st = L.mla_decode_attention_noalloc(ctypes.byref(d), FAKE, FAKE, B, FAKE, max_ctx, ctypes.byref(c), FAKE, None)
    assert st == M.MLA_ERR_WORKSPACE
    c = M.mla_cache(FAKE, FAKE, B, max_ctx)                                           # capacity checked first
    assert L.mla_decode_attention_noalloc(ctypes.byref(d), FAKE, FAKE, B, FAKE, max_ctx, ctypes.byref(c), FAKE,
                                          None) == M.MLA_ERR_CAPACITY
