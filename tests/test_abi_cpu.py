"""The C ABI without a GPU: the library builds and loads, exports every
function include/rpa.h declares, and rejects invalid static arguments with
the documented status before touching device memory."""
import ctypes
import os
import re

import pytest

import ragged_paged_attention_rpa_amd as rpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rpa.h")
PROBE_HEADER = os.path.join(ROOT, "include", "rpa_probe.h")

RPA_E_INVALID, RPA_E_SHAPE, RPA_E_DTYPE, RPA_E_UNSUPPORTED, RPA_E_WORKSPACE = 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rpa.library_path()):
        from ragged_paged_attention_rpa_amd import build
        build.build()
    return rpa.load_library()


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\*?\s+\*?([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_operations():
    names = _declared_functions()
    for op in ("rpa_forward", "kv_cache_update", "mla_rpa_forward", "sparse_mla_forward"):
        assert op in names
    assert set(names) == set(rpa.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions() + _declared_functions(PROBE_HEADER):
        assert hasattr(lib, name), f"{name} not exported by librpa.so"


def test_probe_header_declares_the_four_probes():
    assert _declared_functions(PROBE_HEADER) == ["rpa_probe_chain", "rpa_probe_issue",
                                                 "rpa_probe_rate", "rpa_probe_stream"]


def test_probes_reject_invalid_arguments(lib):
    from ragged_paged_attention_rpa_amd import probes
    probes._lib()
    fake, st = 0x10000, None
    assert lib.rpa_probe_stream(None, 1 << 30, 256, 1, st) == RPA_E_INVALID
    assert lib.rpa_probe_stream(fake, 1 << 30, 0, 1, st) == RPA_E_INVALID
    assert lib.rpa_probe_stream(fake, 1 << 30, 65537, 0, st) == RPA_E_INVALID
    assert lib.rpa_probe_stream(fake, 32 * 1024 * 256 - 1, 256, 1, st) == RPA_E_INVALID
    assert lib.rpa_probe_stream(fake, 1 << 30, 256, 8, st) == RPA_E_INVALID
    assert lib.rpa_probe_stream(fake, 1 << 30, 256, -1, st) == RPA_E_INVALID
    assert lib.rpa_probe_rate(4, 256, fake, st) == RPA_E_INVALID
    assert lib.rpa_probe_rate(-1, 256, fake, st) == RPA_E_INVALID
    assert lib.rpa_probe_rate(0, 256, None, st) == RPA_E_INVALID
    for mode in (1, 3, 16, -2):
        assert lib.rpa_probe_chain(mode, 256, fake, fake, st) == RPA_E_INVALID
    assert lib.rpa_probe_chain(0, 0, fake, fake, st) == RPA_E_INVALID
    assert lib.rpa_probe_chain(0, 256, None, fake, st) == RPA_E_INVALID
    for kind, waves, count, wg, nbytes in [(2, 4, 16, 256, 1 << 20), (-1, 4, 16, 256, 1 << 20),
                                           (0, 0, 16, 256, 1 << 20), (0, 9, 16, 256, 1 << 20),
                                           (1, 4, 8, 256, 1 << 20), (1, 4, 16, 0, 1 << 20),
                                           (0, 4, 16, 65537, 1 << 20), (0, 4, 16, 256, 16383)]:
        assert lib.rpa_probe_issue(kind, waves, count, wg, fake, nbytes, fake, fake, st) == \
            RPA_E_INVALID, (kind, waves, count, wg, nbytes)
    assert lib.rpa_probe_issue(0, 4, 4, 256, None, 1 << 20, fake, fake, st) == RPA_E_INVALID
    assert lib.rpa_probe_issue(0, 4, 4, 256, fake, 1 << 20, None, fake, st) == RPA_E_INVALID
    assert lib.rpa_probe_issue(0, 4, 4, 256, fake, 1 << 20, fake, None, st) == RPA_E_INVALID


def _meta(S=4, pps=8, T=16):
    m = rpa._Meta()
    fake = 0x10000
    m.cu_q_lens = m.kv_lens = m.page_indices = m.num_seqs = fake
    m.max_num_seqs, m.pages_per_seq, m.max_num_tokens = S, pps, T
    return m


def _opts(lib, **kw):
    o = rpa._Opts()
    lib.rpa_opts_init(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def test_opts_defaults(lib):
    o = _opts(lib)
    assert (o.sm_scale, o.sliding_window, o.soft_cap, o.k_scale, o.v_scale, o.debug_validate,
            o.split_keys, o.q_scale) == (1.0, 0, 0.0, 1.0, 1.0, 0, 0, 1.0)


FAKE = ctypes.c_void_p(0x10000)


def _fwd(lib, Hq=8, D=128, Hkv=2, ps=16, P=32, qd=1, kvd=1, meta=None, opts=None, ws=None,
         ws_bytes=0):
    meta = meta or _meta()
    opts = opts or _opts(lib)
    return lib.rpa_forward(FAKE, qd, Hq, D, FAKE, kvd, P, ps, Hkv, None, ctypes.byref(meta),
                           ctypes.byref(opts), FAKE, ws, ws_bytes, None)


def test_rpa_forward_static_rejections(lib):
    assert _fwd(lib, Hq=6, Hkv=4) == RPA_E_SHAPE
    assert "divisible" in lib.rpa_last_error().decode()
    assert _fwd(lib, D=0) == RPA_E_SHAPE
    assert _fwd(lib, ps=0) == RPA_E_SHAPE
    assert _fwd(lib, qd=5) == RPA_E_DTYPE
    assert _fwd(lib, qd=2, D=64) == RPA_E_UNSUPPORTED  # fp8 queries: MFMA path only
    assert "MFMA path" in lib.rpa_last_error().decode()
    assert _fwd(lib, qd=2) == RPA_E_WORKSPACE        # fp8 queries accepted there
    assert _fwd(lib, kvd=3) == RPA_E_WORKSPACE       # int8 pools accepted
    # int4 pools pass the dtype check (an fp8 query is then turned away by the
    # path rule, which comes later) and need an even head_dim
    assert _fwd(lib, kvd=4, qd=2) == RPA_E_UNSUPPORTED
    assert _fwd(lib, kvd=4, D=63) == RPA_E_SHAPE
    assert "even head_dim" in lib.rpa_last_error().decode()
    assert _fwd(lib, kvd=7) == RPA_E_DTYPE
    assert _fwd(lib, opts=_opts(lib, q_scale=float("inf"))) == RPA_E_INVALID
    assert _fwd(lib, opts=_opts(lib, sliding_window=-1)) == RPA_E_INVALID
    assert _fwd(lib, opts=_opts(lib, soft_cap=float("inf"))) == RPA_E_INVALID
    assert _fwd(lib, opts=_opts(lib, sm_scale=float("nan"))) == RPA_E_INVALID
    assert _fwd(lib, meta=_meta(S=0)) == RPA_E_SHAPE
    # bf16 MFMA path without workspace
    assert _fwd(lib) == RPA_E_WORKSPACE
    assert "workspace" in lib.rpa_last_error().decode()


def test_workspace_size_depends_only_on_capacities(lib):
    a = lib.rpa_workspace_size(ctypes.byref(_meta(S=128, pps=512, T=128)), 32, 8, 128)
    b = lib.rpa_workspace_size(ctypes.byref(_meta(S=128, pps=512, T=128)), 32, 8, 128)
    c = lib.rpa_workspace_size(ctypes.byref(_meta(S=256, pps=512, T=128)), 32, 8, 128)
    assert a == b > 0 and c > a


def test_kv_update_static_rejections(lib):
    m = _meta()
    f = lib.kv_cache_update
    assert f(9, FAKE, FAKE, FAKE, None, 1, 4, 16, 2, 128, 0, 0, 0, 4, ctypes.byref(m), None, 0,
             None) == RPA_E_INVALID
    assert f(1, FAKE, FAKE, FAKE, None, 1, 4, 16, 0, 512, 64, 512, 128, 4, ctypes.byref(m), None,
             0, None) == RPA_E_INVALID    # split layout without cache_b
    assert f(1, FAKE, FAKE, FAKE, FAKE, 1, 4, 16, 0, 512, 64, 512, 32, 4, ctypes.byref(m), None,
             0, None) == RPA_E_SHAPE      # stride_b < dim_b
    assert f(2, FAKE, FAKE, FAKE, None, 1, 4, 16, 0, 512, 64, 512, 0, 4, None, FAKE, 0,
             None) == RPA_E_SHAPE         # fused stride < 576
    assert f(0, FAKE, FAKE, FAKE, None, 5, 4, 16, 2, 128, 0, 0, 0, 4, ctypes.byref(m), None, 0,
             None) != 0                   # unknown dtype


def test_mla_static_rejections(lib):
    m = _meta()
    o = _opts(lib)
    f = lib.mla_rpa_forward
    args = lambda **k: [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k.get("dt", 1), 128, k.get("dl", 512),
                        64, 512, 128, 64, 64, ctypes.byref(m), ctypes.byref(o), FAKE, None, 0, None]
    assert f(*args(dt=0)) == RPA_E_UNSUPPORTED
    assert f(*args(dl=256)) == RPA_E_UNSUPPORTED
    assert f(*args()) == RPA_E_WORKSPACE


def test_sparse_static_rejections(lib):
    f = lib.sparse_mla_forward
    base = dict(seq_len=100, S=4, H=16, K=8, RB=64, ps=64, P=4, C=640, ptw=4, kl=512, rd=64, sc=0.07)

    def call(**k):
        a = {**base, **k}
        return f(FAKE, FAKE, FAKE, FAKE, FAKE, a["seq_len"], a["S"], a["H"], a["K"], a["RB"],
                 a["ps"], a["P"], a["C"], a["ptw"], a["kl"], a["rd"], a["sc"], FAKE, None)

    assert call(sc=0.0) == RPA_E_INVALID       # sm_scale is required
    assert call(RB=24) == RPA_E_INVALID        # read_block % 16
    assert call(ps=96) == RPA_E_INVALID        # page_size % read_block
    assert call(C=512) == RPA_E_SHAPE          # cache narrower than the latent
    assert call(kl=256) == RPA_E_UNSUPPORTED


def test_sparse_ragged_static_rejections(lib):
    """The packed-ragged sparse entry shares the single-sequence checks and
    adds its own (request arrays present, at least one request); all of them
    return before any launch."""
    f = lib.sparse_mla_forward_ragged
    base = dict(ptw=8, R=2, T=5, H=16, K=8, RB=64, ps=64, P=8, C=640, kl=512, rd=64, sc=0.07,
                cu=FAKE, sl=FAKE, ck=FAKE)

    def call(**k):
        a = {**base, **k}
        return f(FAKE, FAKE, FAKE, a["ptw"], FAKE, FAKE, a["cu"], a["sl"], a["ck"], a["R"], a["T"],
                 a["H"], a["K"], a["RB"], a["ps"], a["P"], a["C"], a["kl"], a["rd"], a["sc"], FAKE,
                 None)

    assert call(sc=float("nan")) == RPA_E_INVALID
    assert call(RB=24) == RPA_E_INVALID
    assert call(C=512) == RPA_E_SHAPE
    assert call(kl=256) == RPA_E_UNSUPPORTED
    assert call(R=0) == RPA_E_SHAPE
    assert call(cu=None) == RPA_E_INVALID
    assert call(ck=None) == RPA_E_INVALID
    assert call(K=300) == RPA_E_UNSUPPORTED
    assert call(T=0) == 0                      # nothing to do, nothing launched


def test_noalloc_rejects_capacities_beyond_its_scratch_before_any_launch(lib):
    """rpa_forward_noalloc checks the capacities against its static scratch
    array on the host and returns RPA_E_WORKSPACE without touching the GPU."""
    cap = lib.rpa_noalloc_scratch_bytes()
    assert cap == 96 << 20
    big = _meta(S=4096, pps=512, T=4096)
    assert lib.rpa_workspace_size(ctypes.byref(big), 32, 8, 128) > cap
    st = lib.rpa_forward_noalloc(FAKE, 1, 32, 128, FAKE, 1, 64, 16, 8, None, ctypes.byref(big),
                                 ctypes.byref(_opts(lib)), FAKE, None)
    assert st == RPA_E_WORKSPACE
    assert "rpa_forward_noalloc holds at most" in lib.rpa_last_error().decode()
    small = _meta(S=128, pps=512, T=128)
    assert lib.rpa_workspace_size(ctypes.byref(small), 32, 8, 128) <= cap


def test_tile_table_rows_and_override():
    """rpa_tile_config reports the table row a call would use (host values
    only), and a caller's split_keys overrides it; invalid values are refused."""
    import torch
    bf16 = rpa.tile_config(rpa.TILE_DECODE_SPLIT, torch.bfloat16, 32, 8, 128, 16, 512)
    fp8 = rpa.tile_config(rpa.TILE_DECODE_SPLIT, torch.float8_e4m3fn, 32, 8, 128, 16, 512)
    assert bf16[0] == 1024 and bf16[1] == 16 and bf16[2] >= 0
    assert fp8[0] == 2048 and fp8[2] >= 0 and fp8[2] != bf16[2]
    mla = rpa.tile_config(rpa.TILE_MLA_SHARE, torch.bfloat16, 128, 1, 576, 64, 512)
    assert mla[0] % 32 == 0 and mla[1] == 0 and mla[2] >= 0
    assert rpa.tile_config(rpa.TILE_DECODE_SPLIT, torch.bfloat16, 32, 8, 128, 16, 512,
                           split_keys=320) == (320, 16, -2)
    for bad in (32, 100, (1 << 20) + 64):
        with pytest.raises(rpa.RpaError):
            rpa.tile_config(rpa.TILE_DECODE_SPLIT, torch.bfloat16, 32, 8, 128, 16, 512,
                            split_keys=bad)
    with pytest.raises(rpa.RpaError):
        rpa.tile_config(7, torch.bfloat16, 32, 8, 128, 16, 512)
