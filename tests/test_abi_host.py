"""Host-side checks of libgdr.so: it loads, exports every symbol gdr.h
declares, and its validation returns the documented status codes before any
HIP call (so these run without a GPU; no compute call is made)."""
import ctypes
import os
import re

import pytest

from channel_wise_gated_amd import gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(gdr.LIB_PATH):
        pytest.skip("libgdr.so not built (run __graft_entry__.build())")
    return gdr.load()


def test_header_symbols_are_exported():
    lib = _lib()
    with open(os.path.join(ROOT, "include", "gdr.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", header))
    assert declared == set(gdr.SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    _lib()
    assert gdr.gdr_status_string(0) == "GDR_OK"
    for code in range(1, 5):
        assert gdr.gdr_status_string(code).startswith("GDR_ERR_")
    assert "unknown" in gdr.gdr_status_string(99)
    assert gdr.load().gdr_version() >= 100


def ws(desc):
    n = ctypes.c_size_t(123)
    rc = gdr.load().gdr_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    return rc, n.value


GOOD = dict(B=2, H=4, T=256, dk=128, dv=128, chunk=64)


@pytest.mark.parametrize("field,value,code", [
    ("dk", 96, gdr.GDR_ERR_UNSUPPORTED),
    ("dk", 0, gdr.GDR_ERR_INVALID_ARG),
    ("dv", 64, gdr.GDR_ERR_UNSUPPORTED),          # dk != dv
    ("chunk", 32, gdr.GDR_ERR_INVALID_ARG),
    ("T", -64, gdr.GDR_ERR_INVALID_ARG),
    ("B", -1, gdr.GDR_ERR_INVALID_ARG),
    ("in_dtype", 7, gdr.GDR_ERR_INVALID_ARG),
    ("out_dtype", -1, gdr.GDR_ERR_INVALID_ARG),
    ("alpha_mode", gdr.ZEROS, gdr.GDR_ERR_INVALID_ARG),
    ("b_mode", 9, gdr.GDR_ERR_INVALID_ARG),
    ("normalize_qk", 2, gdr.GDR_ERR_INVALID_ARG),
    ("scale", float("nan"), gdr.GDR_ERR_INVALID_ARG),
])
def test_workspace_query_validation(field, value, code):
    _lib()
    kw = dict(GOOD)
    kw[field] = value
    assert ws(gdr.make_desc(**kw))[0] == code


def test_workspace_query_sizes():
    _lib()
    rc, n = ws(gdr.make_desc(**GOOD))
    assert rc == gdr.GDR_OK
    nch = 2 * 4 * (256 // 64)
    # Q', M and the chunk-start states as two bf16 planes, O_bar and N in fp32
    per_chunk = 2 * 64 * 128 * 2 + 2 * 128 * 128 * 2 + 64 * 128 * 4 + 128 * 128 * 4 + 2 * 128 * 128 * 2
    handoff = 2 * 4 * 128 * 128 * 4  # fp32 states carried between segments
    assert n == nch * per_chunk + handoff
    rc, n0 = ws(gdr.make_desc(**dict(GOOD, T=0)))
    assert rc == gdr.GDR_OK and n0 == 0
    # a ragged length takes one (short) chunk more per stream
    rc, nr = ws(gdr.make_desc(**dict(GOOD, T=257)))
    assert rc == gdr.GDR_OK and nr == (nch + 2 * 4) * per_chunk + handoff
    # fp32 mode needs three planes; C = D = 128 does not fit the LDS budget
    assert ws(gdr.make_desc(**dict(GOOD, chunk=128, in_dtype=gdr.GDR_F32)))[0] == gdr.GDR_ERR_UNSUPPORTED
    assert ws(gdr.make_desc(**dict(GOOD, chunk=128)))[0] == gdr.GDR_OK
    assert gdr.load().gdr_chunk_fwd_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == \
        gdr.GDR_ERR_INVALID_ARG
    assert gdr.load().gdr_chunk_fwd_workspace_size(ctypes.byref(gdr.make_desc(**GOOD)), None) == \
        gdr.GDR_ERR_INVALID_ARG


def _call_chunk(desc, ptrs, ws_bytes=1 << 30):
    p = dict(q=16, k=32, v=48, la=64, b=80, w=96, gamma=None, z=None, S0=None, o=112, ST=128,
             ws=256)
    p.update(ptrs)
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return gdr.load().gdr_chunk_fwd(ctypes.byref(desc), c(p["q"]), c(p["k"]), c(p["v"]), c(p["la"]),
                                    c(p["b"]), c(p["w"]), c(p["gamma"]), c(p["z"]), c(p["S0"]),
                                    c(p["o"]), c(p["ST"]), c(p["ws"]), ws_bytes, None)


@pytest.mark.parametrize("ptrs,code", [
    (dict(q=None), gdr.GDR_ERR_INVALID_ARG),
    (dict(o=None), gdr.GDR_ERR_INVALID_ARG),
    (dict(k=40), gdr.GDR_ERR_INVALID_ARG),        # misaligned
    (dict(la=None), gdr.GDR_ERR_INVALID_ARG),     # per-channel alpha needs a pointer
    (dict(z=8), gdr.GDR_ERR_INVALID_ARG),
    (dict(S0=4), gdr.GDR_ERR_INVALID_ARG),
    (dict(ws=None), gdr.GDR_ERR_WORKSPACE),
    (dict(ws=272), gdr.GDR_ERR_WORKSPACE),        # not 256-byte aligned
])
def test_chunk_fwd_rejects_before_launch(ptrs, code):
    _lib()
    assert _call_chunk(gdr.make_desc(**GOOD), ptrs) == code


def _call_gated(desc, ptrs, eps=1e-6, ws_bytes=1 << 30):
    p = dict(q=16, k=32, v=48, la=64, b=80, w=96, gamma=None, z=None, S0=None, g=112, nw=None, y=128,
             o=None, ST=144, ws=256)
    p.update(ptrs)
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return gdr.load().gdr_chunk_fwd_gated(ctypes.byref(desc), c(p["q"]), c(p["k"]), c(p["v"]), c(p["la"]),
                                          c(p["b"]), c(p["w"]), c(p["gamma"]), c(p["z"]), c(p["S0"]),
                                          c(p["g"]), c(p["nw"]), eps, c(p["y"]), c(p["o"]), c(p["ST"]), c(p["ws"]),
                                          ws_bytes, None)


@pytest.mark.parametrize("ptrs,eps,code", [
    (dict(g=None), 1e-6, gdr.GDR_ERR_INVALID_ARG),
    (dict(y=None), 1e-6, gdr.GDR_ERR_INVALID_ARG),
    (dict(g=120), 1e-6, gdr.GDR_ERR_INVALID_ARG),   # misaligned
    (dict(nw=8), 1e-6, gdr.GDR_ERR_INVALID_ARG),
    ({}, -1.0, gdr.GDR_ERR_INVALID_ARG),
    ({}, float("nan"), gdr.GDR_ERR_INVALID_ARG),
    ({}, float("inf"), gdr.GDR_ERR_INVALID_ARG),
    (dict(q=None), 1e-6, gdr.GDR_ERR_INVALID_ARG),
    (dict(ws=None), 1e-6, gdr.GDR_ERR_WORKSPACE),
])
def test_chunk_fwd_gated_rejects_before_launch(ptrs, eps, code):
    _lib()
    assert _call_gated(gdr.make_desc(**GOOD), ptrs, eps) == code


def test_chunk_fwd_workspace_too_small():
    _lib()
    assert _call_chunk(gdr.make_desc(**GOOD), {}, ws_bytes=1024) == gdr.GDR_ERR_WORKSPACE


def test_chunk_fwd_gate_pointers_optional_for_constant_modes():
    _lib()
    # ONES / ZEROS gates need no pointer; validation then fails only on the
    # deliberately missing q, proving the gate checks passed.
    d = gdr.make_desc(**dict(GOOD, alpha_mode=gdr.ONES, b_mode=gdr.ZEROS, w_mode=gdr.ONES))
    assert _call_chunk(d, dict(la=None, b=None, w=None, q=None)) == gdr.GDR_ERR_INVALID_ARG
    d = gdr.make_desc(**dict(GOOD, b_mode=gdr.PER_CHANNEL))
    assert _call_chunk(d, dict(b=None)) == gdr.GDR_ERR_INVALID_ARG


def test_empty_batch_is_a_noop():
    _lib()
    d = gdr.make_desc(**dict(GOOD, B=0))
    assert _call_chunk(d, dict(q=None, ws=None)) == gdr.GDR_OK
    dd = gdr.make_desc(**dict(GOOD, H=0))
    c = lambda x: ctypes.c_void_p(x)
    assert gdr.load().gdr_decode_step(ctypes.byref(dd), None, None, None, None, None, None, None,
                                      None, None, None, None) == gdr.GDR_OK


def test_decode_rejects_before_launch():
    _lib()
    lib = gdr.load()
    d = gdr.make_desc(B=4, H=2, T=1, dk=128, dv=128)
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    args = [16, 32, 48, 64, 80, 96, 112, None, None, 128]   # S q k v la b w gamma z o
    def call(**over):
        names = ["S", "q", "k", "v", "la", "b", "w", "gamma", "z", "o"]
        vals = dict(zip(names, args))
        vals.update(over)
        return lib.gdr_decode_step(ctypes.byref(d), *[c(vals[n]) for n in names], None)
    assert call(S=None) == gdr.GDR_ERR_INVALID_ARG
    assert call(S=20) == gdr.GDR_ERR_INVALID_ARG
    assert call(v=None) == gdr.GDR_ERR_INVALID_ARG
    assert call(gamma=24) == gdr.GDR_ERR_INVALID_ARG
    bad = gdr.make_desc(B=4, H=2, T=1, dk=80, dv=80)
    assert lib.gdr_decode_step(ctypes.byref(bad), *[c(x) for x in args], None) == gdr.GDR_ERR_UNSUPPORTED
    assert lib.gdr_decode_step(None, *[c(x) for x in args], None) == gdr.GDR_ERR_INVALID_ARG


def test_varlen_validation():
    lib = _lib()
    d = gdr.make_desc(B=1, H=4, T=300, dk=128, dv=128, chunk=64)
    n = ctypes.c_size_t(0)
    assert lib.gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(d), 3, ctypes.byref(n)) == gdr.GDR_OK
    # per head ceil(300 / 64) + 3 chunk slots, plus the chunk list and offsets
    per_head = 5 + 3
    slots = 4 * per_head
    maps = slots * (2 * 64 * 128 * 2 + 2 * 128 * 128 * 2 + 64 * 128 * 4 + 128 * 128 * 4 + 2 * 128 * 128 * 2)
    assert n.value == maps + 256 + 256     # 8 x 16-byte entries and 4 offsets, each padded to 256
    assert lib.gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == \
        gdr.GDR_ERR_INVALID_ARG
    d2 = gdr.make_desc(B=2, H=4, T=300, dk=128, dv=128, chunk=64)
    assert lib.gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(d2), 3, ctypes.byref(n)) == \
        gdr.GDR_ERR_INVALID_ARG
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    def call(cu, nseq=3):
        return lib.gdr_chunk_fwd_varlen(ctypes.byref(d), nseq, c(cu), c(16), c(32), c(48), c(64), c(80),
                                        c(96), None, None, None, c(112), c(128), c(256), 1 << 30, None)
    assert call(None) == gdr.GDR_ERR_INVALID_ARG
    assert call(1026) == gdr.GDR_ERR_INVALID_ARG   # misaligned offsets
    assert call(1024, nseq=0) == gdr.GDR_ERR_INVALID_ARG


GATE = dict(B=2, T=100, d_model=256, H=2, d=128, ranks=(64, 64, 128, 128, 128))


def _gate_ws(**kw):
    p = dict(GATE)
    p.update(kw)
    desc = gdr.make_gate_desc(p["B"], p["T"], p["d_model"], p["H"], p["d"], p["ranks"])
    n = ctypes.c_size_t(0)
    return gdr.load().gdr_gate_proj_workspace_size(ctypes.byref(desc), ctypes.byref(n)), n.value


def test_gate_proj_workspace_and_validation():
    _lib()
    rc, n = _gate_ws()
    assert rc == gdr.GDR_OK and n == 2 * 100 * 512 * 4      # the latent h, fp32
    assert _gate_ws(d_model=100)[0] == gdr.GDR_ERR_INVALID_ARG       # not a multiple of 32
    assert _gate_ws(ranks=(64, 64, 128, 100, 128))[0] == gdr.GDR_ERR_INVALID_ARG
    assert _gate_ws(ranks=(64, 64, 128, 256, 128))[0] == gdr.GDR_ERR_UNSUPPORTED
    assert _gate_ws(d=96)[0] == gdr.GDR_ERR_UNSUPPORTED
    assert _gate_ws(H=0)[0] == gdr.GDR_ERR_INVALID_ARG
    assert _gate_ws(T=0) == (gdr.GDR_OK, 0)
    assert _gate_ws(T=1 << 29)[0] == gdr.GDR_ERR_INVALID_ARG             # B T H >= 2^31 (row index)
    desc = gdr.make_gate_desc(2, 100, 256, 2, 128, (64, 64, 128, 128, 128))
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    call = lambda x, wd, wu, ws, nb: gdr.load().gdr_gate_proj(
        ctypes.byref(desc), c(x), c(wd), c(wu), None, c(4096), None, None, None, None, c(ws), nb, None)
    assert call(None, 1024, 2048, 8192, 1 << 30) == gdr.GDR_ERR_INVALID_ARG   # no input
    assert call(1032, 1024, 2048, 8192, 1 << 30) == gdr.GDR_ERR_INVALID_ARG   # misaligned
    assert call(1024, 1288, 2048, 8192, 1 << 30) == gdr.GDR_ERR_INVALID_ARG
    assert call(1024, 1280, 2048, None, 1 << 30) == gdr.GDR_ERR_WORKSPACE
    assert call(1024, 1280, 2048, 8192, 1000) == gdr.GDR_ERR_WORKSPACE


def test_chunk_bwd_workspace_and_validation():
    _lib()
    lib = gdr.load()
    n = ctypes.c_size_t(0)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(gdr.make_desc(**GOOD)), ctypes.byref(n)) == gdr.GDR_OK
    assert n.value > 0
    d0 = gdr.make_desc(**dict(GOOD, T=0))
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(d0), ctypes.byref(n)) == gdr.GDR_OK and n.value == 0
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(gdr.make_desc(**dict(GOOD, dk=96))),
                                            ctypes.byref(n)) == gdr.GDR_ERR_UNSUPPORTED
    c = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(dO=512, q=16, ws=1 << 20, nbytes=1 << 40, dq=None):
        p = [q, 32, 48, 64, 80, 96, None, None, None, dO, None, dq] + [None] * 8
        return lib.gdr_chunk_bwd(ctypes.byref(gdr.make_desc(**GOOD)), *[c(x) for x in p], c(ws), nbytes, None)
    assert call(dO=None) == gdr.GDR_ERR_INVALID_ARG
    assert call(dO=520) == gdr.GDR_ERR_INVALID_ARG      # misaligned
    assert call(q=None) == gdr.GDR_ERR_INVALID_ARG
    assert call(dq=8) == gdr.GDR_ERR_INVALID_ARG
    assert call(ws=None) == gdr.GDR_ERR_WORKSPACE
    assert call(nbytes=1000) == gdr.GDR_ERR_WORKSPACE


def test_chunk_bwd_varlen_workspace_and_validation():
    _lib()
    lib = gdr.load()
    n = ctypes.c_size_t(0)
    one = gdr.make_desc(**dict(GOOD, B=1))
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(one), 3, ctypes.byref(n)) == gdr.GDR_OK
    n_uniform = ctypes.c_size_t(0)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(one), ctypes.byref(n_uniform)) == gdr.GDR_OK
    assert n.value > n_uniform.value  # room for the chunk list and one partial chunk per sequence
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(one), 0, ctypes.byref(n)) == gdr.GDR_ERR_INVALID_ARG
    two = gdr.make_desc(**dict(GOOD, B=2))
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(two), 3, ctypes.byref(n)) == gdr.GDR_ERR_INVALID_ARG
    c = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(nseq=3, cu=4096, desc=one):
        p = [16, 32, 48, 64, 80, 96, None, None, None, 512, None] + [None] * 9
        return lib.gdr_chunk_bwd_varlen(ctypes.byref(desc), nseq, c(cu), *[c(x) for x in p], c(1 << 20), 1 << 40, None)
    assert call(nseq=0) == gdr.GDR_ERR_INVALID_ARG
    assert call(cu=None) == gdr.GDR_ERR_INVALID_ARG
    assert call(cu=4098) == gdr.GDR_ERR_INVALID_ARG      # misaligned offsets
    assert call(desc=two) == gdr.GDR_ERR_INVALID_ARG     # a packed batch has B = 1


def test_output_gate_bwd_workspace_and_validation():
    _lib()
    lib = gdr.load()
    n = ctypes.c_size_t(0)
    desc = gdr.make_desc(**GOOD)
    assert lib.gdr_output_gate_bwd_workspace_size(ctypes.byref(desc), 1, ctypes.byref(n)) == gdr.GDR_OK
    assert n.value == 2 * 4 * ((256 + 63) // 64) * 128 * 4  # B H token-blocks dv fp32
    assert lib.gdr_output_gate_bwd_workspace_size(ctypes.byref(desc), 0, ctypes.byref(n)) == gdr.GDR_OK and n.value == 0
    c = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(o=16, g=32, nw=48, eps=1e-6, dy=64, d_o=80, dnw=96, ws=1 << 20, nbytes=1 << 30):
        return lib.gdr_output_gate_bwd(ctypes.byref(desc), c(o), c(g), c(nw), eps, c(dy), c(d_o), None, c(dnw),
                                       c(ws), nbytes, None)
    assert call(o=None) == gdr.GDR_ERR_INVALID_ARG
    assert call(d_o=None) == gdr.GDR_ERR_INVALID_ARG
    assert call(dy=72) == gdr.GDR_ERR_INVALID_ARG       # misaligned
    assert call(eps=-1.0) == gdr.GDR_ERR_INVALID_ARG
    assert call(eps=float("nan")) == gdr.GDR_ERR_INVALID_ARG
    assert call(ws=None) == gdr.GDR_ERR_WORKSPACE
    assert call(nbytes=1024) == gdr.GDR_ERR_WORKSPACE


# ---------------------------------------------------------------- chunk list of a packed batch
def chunk_table_model(cu, T, C, cap):
    """The device chunk-list builder of a packed batch, step for step on the
    host: offsets clamped to [0, T], a sequence's end to no less than its
    start, entries written only below `cap` (the list's length in the
    workspace, ceil(T / C) + n_seqs) and the offsets capped there too.
    Returns (coff, writes) with writes = [(index, n, c, row, valid)]."""
    nseq = len(cu) - 1
    coff, writes, excl = [], [], 0
    for n in range(nseq + 1):
        cnt, r0, ln = 0, 0, 0
        if n < nseq:
            r0 = min(max(cu[n], 0), T)
            r1 = min(max(cu[n + 1], r0), T)
            ln = r1 - r0
            cnt = (ln + C - 1) // C
        coff.append(min(excl, cap))
        for j in range(excl, min(excl + cnt, cap)):
            c = j - excl
            writes.append((j, n, c, r0 + c * C, min(C, ln - c * C)))
        excl += cnt
    return coff, writes


@pytest.mark.parametrize("cu", [
    [0, 10, 300, 300, 1000],                 # valid
    [0, 900, 100, 1000],                     # decreasing offsets
    [0, 5000, 1000],                         # past T
    [-50, 40, -7, 1000],                     # negative offsets
    [0, 1000, 0, 1000, 0, 1000, 0, 1000],    # overlapping: more chunks than the list holds
])
def test_chunk_table_logic_stays_in_bounds(cu):
    T, C = 1000, 64
    cap = (T + C - 1) // C + len(cu) - 1
    coff, writes = chunk_table_model(cu, T, C, cap)
    assert all(0 <= a <= b <= cap for a, b in zip(coff, coff[1:]))
    for j, n, c, row, valid in writes:
        assert 0 <= j < cap and 1 <= valid <= C and 0 <= row and row + valid <= T
        assert coff[n] <= j < coff[n + 1]           # the chain walks exactly these entries
    if cu == sorted(cu) and 0 <= cu[0] and cu[-1] <= T:
        # valid offsets: every token is covered once, in sequence order
        cover = sorted((row, valid) for _, _, _, row, valid in writes)
        assert sum(v for _, v in cover) == cu[-1] - cu[0]
        assert all(coff[n + 1] - coff[n] == -(-(cu[n + 1] - cu[n]) // C) for n in range(len(cu) - 1))


def test_static_forward_rejects_problems_beyond_its_scratch():
    """gdr_chunk_fwd_static returns GDR_ERR_UNSUPPORTED, before any launch,
    when one chunk per stream of B*H streams does not fit its static scratch
    (64 MiB); a descriptor error still comes first."""
    lib = _lib()
    big = gdr.make_desc(**dict(GOOD, B=64, H=16, T=4096, dk=128, dv=128, chunk=128))
    n = [None] * 11
    assert lib.gdr_chunk_fwd_static(ctypes.byref(big), *n, None) == gdr.GDR_ERR_UNSUPPORTED
    bad = gdr.make_desc(**dict(GOOD, B=64, H=16, T=4096, dk=96, dv=96))
    assert lib.gdr_chunk_fwd_static(ctypes.byref(bad), *n, None) == gdr.GDR_ERR_UNSUPPORTED
    bad = gdr.make_desc(**dict(GOOD, chunk=32))
    assert lib.gdr_chunk_fwd_static(ctypes.byref(bad), *n, None) == gdr.GDR_ERR_INVALID_ARG


def test_segment_chunks_query():
    """Segment length of the whole call: one pass for a small problem, whole
    rounds of the 256 compute units (and at least 8 chunks) for the
    long-context shape, 0 without tokens; validation as the workspace query."""
    _lib()
    small = gdr.make_desc(**GOOD)
    assert gdr.gdr_chunk_fwd_segment_chunks(small) == 256 // 64
    stress = gdr.make_desc(B=1, H=16, T=32768, dk=128, dv=128, chunk=128)
    seg = gdr.gdr_chunk_fwd_segment_chunks(stress)
    assert 8 <= seg < 256 and (16 * seg) % 256 == 0
    assert gdr.gdr_chunk_fwd_segment_chunks(gdr.make_desc(**dict(GOOD, T=0))) == 0
    with pytest.raises(gdr.GdrError):
        gdr.gdr_chunk_fwd_segment_chunks(gdr.make_desc(**dict(GOOD, chunk=32)))
