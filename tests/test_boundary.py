"""The C ABI boundary on a host without a GPU.

libfa.so must load, export every function include/fa.h declares, and reject
invalid arguments with the documented status before making any HIP call (so
these calls never touch a device).  No call here passes valid arguments: each
one is rejected, so nothing is ever launched (the fake addresses below are
never dereferenced).
"""

import ctypes
import math
import os
import re

import pytest

import exact_tiled_attention_10_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def _header_enum():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(FA_[A-Z_]+)\s*=\s*(\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        import exact_tiled_attention_10_amd.build as b
        b.build()
    return fa.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_gqa", "fa_fwd_kv", "fa_fwd_kv_workspace_size",
                          "fa_fwd_fp8", "fa_fwd_f32", "fa_bwd", "fa_bwd_gqa", "fa_bwd_kv",
                          "fa_bwd_workspace_size", "fa_bwd_kv_workspace_size",
                          "fa_status_string", "fa_bwd_preprocess", "fa_bwd_main",
                          "fa_bwd_finalize", "fa_bwd_noalloc"}
    for nm in names:
        assert hasattr(lib, nm), nm


def test_status_codes_match_header(lib):
    enum = _header_enum()
    for name, val in enum.items():
        assert getattr(fa, name) == val, name
        assert fa.fa_status_string(val) not in ("", "unknown status")
    assert fa.fa_status_string(999) == "unknown status"
    m = re.search(r"#define FA_MAX_N \(1 << (\d+)\)", open(HEADER).read())
    assert fa.FA_MAX_N == 1 << int(m.group(1))


A = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
MB = 1 << 24


def _fwd(lib, q=A, k=A + MB, v=A + 2 * MB, o=A + 3 * MB, lse=A + 4 * MB, B=1, H=2, N=100,
         d=64, causal=0, scale=0.125, f32=False):
    fn = lib.fa_fwd_f32 if f32 else lib.fa_fwd
    return fn(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("f32", [False, True])
def test_forward_rejects_bad_arguments(lib, f32):
    assert _fwd(lib, d=32, f32=f32) == fa.FA_ERR_HEADDIM
    assert _fwd(lib, d=0, f32=f32) == fa.FA_ERR_HEADDIM
    assert _fwd(lib, N=-1, f32=f32) == fa.FA_ERR_SHAPE
    assert _fwd(lib, B=-2, f32=f32) == fa.FA_ERR_SHAPE
    assert _fwd(lib, H=-1, f32=f32) == fa.FA_ERR_SHAPE
    assert _fwd(lib, N=fa.FA_MAX_N + 1, f32=f32) == fa.FA_ERR_SHAPE
    assert _fwd(lib, B=1 << 20, H=1 << 12, f32=f32) == fa.FA_ERR_SHAPE
    assert _fwd(lib, scale=math.nan, f32=f32) == fa.FA_ERR_SCALE
    assert _fwd(lib, scale=math.inf, f32=f32) == fa.FA_ERR_SCALE
    assert _fwd(lib, q=None, f32=f32) == fa.FA_ERR_NULL
    assert _fwd(lib, lse=None, f32=f32) == fa.FA_ERR_NULL
    assert _fwd(lib, v=A + 2 * MB + 2, f32=f32) == fa.FA_ERR_ALIGN
    assert _fwd(lib, lse=A + 4 * MB + 4, f32=f32) == fa.FA_ERR_ALIGN
    assert _fwd(lib, o=A + 16, f32=f32) == fa.FA_ERR_ALIAS           # o overlaps q
    assert _fwd(lib, lse=A + 3 * MB + 64, f32=f32) == fa.FA_ERR_ALIAS  # lse inside o
    assert _fwd(lib, o=A + 2 * MB, f32=f32) == fa.FA_ERR_ALIAS       # o is v


@pytest.mark.parametrize("f32", [False, True])
def test_forward_empty_is_noop(lib, f32):
    # B*H*N == 0 returns OK before any pointer check or HIP call
    assert _fwd(lib, N=0, q=None, k=None, v=None, o=None, lse=None, f32=f32) == fa.FA_OK
    assert _fwd(lib, B=0, f32=f32) == fa.FA_OK
    assert _fwd(lib, H=0, f32=f32) == fa.FA_OK


def test_workspace_size(lib):
    assert lib.fa_bwd_workspace_size(1, 2, 100, 32) == 0
    assert lib.fa_bwd_workspace_size(1, 2, -1, 64) == 0
    for (B, H, N, d) in ((1, 2, 100, 64), (4, 16, 2048, 64), (1, 8, 32768, 128),
                         (1, 2, 300, 256)):
        ws = lib.fa_bwd_workspace_size(B, H, N, d)
        # L2 and D (fp32 per row), plus the fp32 dQ accumulator where dQ is
        # accumulated with atomics (d = 64)
        need = 2 * B * H * N * 4 + (B * H * N * d * 4 if d == 64 else 0)
        assert ws >= need
        assert ws % 16 == 0


def test_bwd_kv_workspace_size(lib):
    """The grouped-query backward's workspace: the plain one, plus float32
    partial dK and dV ([2][s][B*Hkv][Nk][d]) when the plan splits each group's
    query heads over s workgroups."""
    assert lib.fa_bwd_kv_workspace_size(1, 2, 1, 100, 100, 32) == 0
    assert lib.fa_bwd_kv_workspace_size(1, 6, 4, 100, 100, 64) == 0    # H % Hkv != 0
    assert lib.fa_bwd_kv_workspace_size(1, 2, 1, 100, -1, 64) == 0
    # no grouping, or enough key / value heads to fill the chip: no split
    for (B, H, Hkv, Nq, Nk, d) in ((1, 2, 2, 100, 100, 64), (4, 16, 16, 2048, 2048, 64),
                                   (4, 32, 8, 4096, 4096, 128)):
        assert (lib.fa_bwd_kv_workspace_size(B, H, Hkv, Nq, Nk, d)
                == lib.fa_bwd_workspace_size(B, H, Nq, d))
    # Llama-3.1-8B heads at batch 1: key tile 0 holds 4 heads x 64 query
    # blocks, twice the average per compute unit; halves of the group fit
    base = lib.fa_bwd_workspace_size(1, 32, 4096, 128)
    assert lib.fa_bwd_kv_workspace_size(1, 32, 8, 4096, 4096, 128) == base + 2 * 2 * 8 * 4096 * 128 * 4
    # one key / value head, a short sequence: every head on its own
    base = lib.fa_bwd_workspace_size(1, 8, 256, 64)
    assert lib.fa_bwd_kv_workspace_size(1, 8, 1, 256, 256, 64) == base + 2 * 8 * 1 * 256 * 64 * 4


def test_kv_workspace_size_is_a_split_of_the_group(lib):
    """Over many shapes: the grouped-query workspace is the plain one plus
    float32 partials [2][s][B*Hkv][Nk][d] for a divisor s of the group (s = 1:
    nothing added), and the split never goes past the group."""
    import random
    rng = random.Random(5)
    for _ in range(300):
        d = rng.choice((64, 128, 256))
        Hkv = rng.choice((1, 2, 4, 8))
        group = rng.choice((1, 2, 3, 4, 8))
        B = rng.choice((1, 2, 4))
        Nq = rng.choice((1, 63, 300, 2048, 4096))
        Nk = rng.choice((1, 100, 2048, 4096, 8192))
        H = Hkv * group
        base = lib.fa_bwd_workspace_size(B, H, Nq, d)
        kv = lib.fa_bwd_kv_workspace_size(B, H, Hkv, Nq, Nk, d)
        extra = kv - base
        assert extra >= 0
        if extra == 0:
            continue
        unit = 2 * B * Hkv * Nk * d * 4
        splits = [s for s in range(2, group + 1) if group % s == 0
                  and (s * unit + 255) // 256 * 256 == extra]
        assert splits, (B, H, Hkv, Nq, Nk, d, extra)
        assert group > 1


def _bwd(lib, ws_bytes=None, **kw):
    B, H, N, d = kw.get("B", 1), kw.get("H", 2), kw.get("N", 100), kw.get("d", 64)
    ptrs = dict(q=A, k=A + MB, v=A + 2 * MB, o=A + 3 * MB, dout=A + 4 * MB, lse=A + 5 * MB,
                dq=A + 6 * MB, dk=A + 7 * MB, dv=A + 8 * MB, ws=A + 9 * MB)
    ptrs.update({k: v for k, v in kw.items() if k in ptrs})
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(1, 2, 100, 64)
    return lib.fa_bwd(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["dout"], ptrs["lse"],
                      ptrs["dq"], ptrs["dk"], ptrs["dv"], ptrs["ws"], ws_bytes, B, H, N, d,
                      kw.get("causal", 1), kw.get("scale", 0.125), None)


def test_backward_rejects_bad_arguments(lib):
    assert _bwd(lib, d=96) == fa.FA_ERR_HEADDIM
    assert _bwd(lib, N=-5) == fa.FA_ERR_SHAPE
    assert _bwd(lib, scale=math.nan) == fa.FA_ERR_SCALE
    assert _bwd(lib, dout=None) == fa.FA_ERR_NULL
    assert _bwd(lib, ws=None) == fa.FA_ERR_NULL
    assert _bwd(lib, dk=A + 7 * MB + 8) == fa.FA_ERR_ALIGN
    assert _bwd(lib, ws_bytes=16) == fa.FA_ERR_WORKSPACE
    assert _bwd(lib, dq=A + 3 * MB) == fa.FA_ERR_ALIAS                # dq is o
    assert _bwd(lib, dv=A + 6 * MB + 32) == fa.FA_ERR_ALIAS           # dv inside dq
    assert _bwd(lib, ws=A + 8 * MB + 64) == fa.FA_ERR_ALIAS           # ws inside dv
    assert _bwd(lib, dk=A + 5 * MB) == fa.FA_ERR_ALIAS                # dk over lse
    assert _bwd(lib, N=0, q=None, ws=None) == fa.FA_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """The binding has no fallback: a missing libfa.so raises."""
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "library_path", lambda: str(tmp_path / "libfa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fa.load_library()


def test_backward_stages_reject_bad_arguments(lib):
    ws = lib.fa_bwd_workspace_size(1, 2, 100, 64)
    o, g, L, w = A, A + MB, A + 5 * MB, A + 9 * MB
    assert lib.fa_bwd_preprocess(o, g, L, w, 8, 1, 2, 100, 64, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd_preprocess(None, g, L, w, ws, 1, 2, 100, 64, None) == fa.FA_ERR_NULL
    assert lib.fa_bwd_preprocess(o, g, None, w, ws, 1, 2, 100, 64, None) == fa.FA_ERR_NULL
    assert lib.fa_bwd_preprocess(o, g, L, o + 64, ws, 1, 2, 100, 64, None) == fa.FA_ERR_ALIAS
    assert lib.fa_bwd_preprocess(o, g, L, L + 16, ws, 1, 2, 100, 64, None) == fa.FA_ERR_ALIAS
    assert lib.fa_bwd_preprocess(o, g, L + 4, w, ws, 1, 2, 100, 64, None) == fa.FA_ERR_ALIGN
    assert lib.fa_bwd_preprocess(o, g, L, w, ws, 1, 2, 100, 48, None) == fa.FA_ERR_HEADDIM
    assert lib.fa_bwd_preprocess(o, g, L, w, ws, 1, 2, 0, 64, None) == fa.FA_OK
    mk = lambda **kw: lib.fa_bwd_main(  # noqa: E731
        kw.get("q", A), A + MB, A + 2 * MB, A + 4 * MB, kw.get("dk", A + 7 * MB),
        A + 8 * MB, kw.get("ws", w), kw.get("wsb", ws), 1, 2, 100, 64, 1,
        kw.get("scale", 0.125), None)
    assert mk(q=None) == fa.FA_ERR_NULL
    assert mk(wsb=4) == fa.FA_ERR_WORKSPACE
    assert mk(dk=A + 8 * MB + 16) == fa.FA_ERR_ALIAS        # dk overlaps dv
    assert mk(ws=A + MB) == fa.FA_ERR_ALIAS                 # workspace over k
    assert mk(scale=math.inf) == fa.FA_ERR_SCALE
    fin = lambda dq, wsp, wsb, d=64, q=None, k=None, v=None, g=None: lib.fa_bwd_finalize(  # noqa
        q, k, v, g, dq, wsp, wsb, 1, 2, 100, d, 1, 0.125, None)
    assert fin(A + 6 * MB, w, 4) == fa.FA_ERR_WORKSPACE
    assert fin(None, w, ws) == fa.FA_ERR_NULL
    assert fin(w + 16, w, ws) == fa.FA_ERR_ALIAS
    assert fin(A + 6 * MB + 2, w, ws) == fa.FA_ERR_ALIGN
    # d = 128: the query-tile dQ kernel needs q, k, v and dout
    ws128 = lib.fa_bwd_workspace_size(1, 2, 100, 128)
    assert fin(A + 6 * MB, w, ws128, d=128) == fa.FA_ERR_NULL
    assert fin(A + 6 * MB, w, ws128, d=128, q=A, k=A + MB, v=A + 2 * MB,
               g=A + 6 * MB + 64) == fa.FA_ERR_ALIAS          # dq over dout
    # only the d = 64 path keeps a dQ accumulator in the workspace
    assert ws128 < lib.fa_bwd_workspace_size(1, 2, 100, 64) * 2
    assert lib.fa_bwd_workspace_size(1, 2, 100, 256) == ws128


def test_gqa_entry_points_reject_bad_head_counts(lib):
    f = lambda H, Hkv, **kw: lib.fa_fwd_gqa(  # noqa: E731
        kw.get("q", A), kw.get("k", A + MB), A + 2 * MB, kw.get("o", A + 3 * MB), A + 4 * MB,
        1, H, Hkv, 100, 64, 1, 0.125, None)
    assert f(4, 0) == fa.FA_ERR_SHAPE
    assert f(4, 3) == fa.FA_ERR_SHAPE            # 4 query heads do not split over 3
    assert f(4, 8) == fa.FA_ERR_SHAPE            # more key/value heads than query heads
    assert f(4, -1) == fa.FA_ERR_SHAPE
    assert f(0, 1) == fa.FA_OK                   # no query heads: nothing to do
    assert f(4, 2, q=None) == fa.FA_ERR_NULL
    assert f(4, 2, o=A + 16) == fa.FA_ERR_ALIAS  # o over q
    # k holds 2 heads of 100 x 64 bf16 (25.6 KB, not the 4 query heads'
    # 51.2 KB): an o that starts 16 bytes before k's end overlaps it
    assert f(4, 2, k=A + 3 * MB - 2 * 100 * 64 * 2 + 16) == fa.FA_ERR_ALIAS
    ws = lib.fa_bwd_workspace_size(1, 4, 100, 64)
    b = lambda H, Hkv, **kw: lib.fa_bwd_gqa(  # noqa: E731
        A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB, A + 6 * MB,
        kw.get("dk", A + 7 * MB), A + 8 * MB, A + 9 * MB, kw.get("wsb", ws), 1, H, Hkv, 100, 64,
        1, 0.125, None)
    assert b(4, 3) == fa.FA_ERR_SHAPE
    assert b(4, 0) == fa.FA_ERR_SHAPE
    assert b(4, 2, wsb=16) == fa.FA_ERR_WORKSPACE
    assert b(4, 2, dk=A + 8 * MB - 16) == fa.FA_ERR_ALIAS   # dk runs into dv
    assert b(0, 2) == fa.FA_OK


def test_fwd_kv_workspace_size(lib):
    # plenty of query tiles: no key split, no workspace
    assert lib.fa_fwd_kv_workspace_size(1, 32, 32, 4096, 4096, 128) == 0
    assert lib.fa_fwd_kv_workspace_size(1, 2, 2, 100, -1, 64) == 0
    assert lib.fa_fwd_kv_workspace_size(1, 2, 2, 100, 100, 96) == 0
    assert lib.fa_fwd_kv_workspace_size(1, 4, 3, 1, 4096, 128) == 0   # 4 heads over 3
    # decode (one query row per head): the keys are split, partials need room
    ws = lib.fa_fwd_kv_workspace_size(1, 2, 2, 1, 4096, 128)
    assert ws > 0 and ws % 4 == 0
    assert ws >= 2 * 2 * 1 * (128 + 1) * 4       # at least two ranges of O and lse


def test_kv_forward_rejects_bad_arguments(lib):
    ws_need = lib.fa_fwd_kv_workspace_size(1, 2, 2, 1, 4096, 128)
    W = A + 9 * MB

    def f(**kw):
        g = dict(q=A, k=A + MB, v=A + 2 * MB, o=A + 3 * MB, lse=A + 4 * MB, ws=W,
                 wsb=ws_need, B=1, H=2, Hkv=2, Nq=1, Nk=4096, d=128, causal=1, scale=0.1)
        g.update(kw)
        return lib.fa_fwd_kv(g["q"], g["k"], g["v"], g["o"], g["lse"], g["ws"], g["wsb"],
                             g["B"], g["H"], g["Hkv"], g["Nq"], g["Nk"], g["d"], g["causal"],
                             g["scale"], None)
    assert f(Nk=-1) == fa.FA_ERR_SHAPE
    assert f(Nk=fa.FA_MAX_N + 1) == fa.FA_ERR_SHAPE
    assert f(Nq=-1) == fa.FA_ERR_SHAPE
    assert f(Hkv=3) == fa.FA_ERR_SHAPE
    assert f(d=80) == fa.FA_ERR_HEADDIM
    assert f(scale=math.nan) == fa.FA_ERR_SCALE
    assert f(k=None) == fa.FA_ERR_NULL
    assert f(ws=None) == fa.FA_ERR_NULL
    assert f(wsb=ws_need - 4) == fa.FA_ERR_WORKSPACE
    assert f(ws=W + 8) == fa.FA_ERR_ALIGN
    assert f(ws=A + MB + 64) == fa.FA_ERR_ALIAS      # workspace over k
    assert f(lse=A + 3 * MB + 16) == fa.FA_ERR_ALIAS  # lse inside o
    assert f(Nq=0, q=None, o=None) == fa.FA_OK        # nothing to compute
    # with no keys, k and v may be NULL: the call gets past the pointer checks
    assert f(Nk=0, k=None, v=None, ws=None, wsb=0, d=96) == fa.FA_ERR_HEADDIM


def test_kv_backward_rejects_bad_arguments(lib):
    ws = lib.fa_bwd_workspace_size(1, 2, 10, 64)

    def b(**kw):
        g = dict(q=A, k=A + MB, v=A + 2 * MB, o=A + 3 * MB, dout=A + 4 * MB, lse=A + 5 * MB,
                 dq=A + 6 * MB, dk=A + 7 * MB, dv=A + 8 * MB, ws=A + 9 * MB, wsb=ws, B=1, H=2,
                 Hkv=1, Nq=10, Nk=300, d=64, causal=1, scale=0.125)
        g.update(kw)
        return lib.fa_bwd_kv(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"], g["dq"],
                             g["dk"], g["dv"], g["ws"], g["wsb"], g["B"], g["H"], g["Hkv"],
                             g["Nq"], g["Nk"], g["d"], g["causal"], g["scale"], None)
    assert b(Nk=-3) == fa.FA_ERR_SHAPE
    assert b(Hkv=3) == fa.FA_ERR_SHAPE
    assert b(wsb=ws - 16) == fa.FA_ERR_WORKSPACE
    assert b(dk=None) == fa.FA_ERR_NULL
    assert b(q=None) == fa.FA_ERR_NULL
    # k holds 1 head of 300 x 64 bf16 (38400 bytes): a dk starting inside it aliases
    assert b(dk=A + MB + 38400 - 16) == fa.FA_ERR_ALIAS
    # no queries and no keys: a no-op with no pointers at all
    assert b(Nq=0, Nk=0, q=None, k=None, v=None, o=None, dout=None, lse=None, dq=None,
             dk=None, dv=None, ws=None, wsb=0) == fa.FA_OK
    # no queries: the query-side pointers are not needed (the call would then
    # zero dk and dv on the device, so only a rejected form is tried here)
    assert b(Nq=0, q=None, o=None, dout=None, lse=None, dq=None, ws=None, dk=None) == \
        fa.FA_ERR_NULL


def test_head_dim_256_only_on_the_bf16_entry_points(lib):
    # the bf16 forwards and backwards get past the head-dim check (then stop at
    # a NULL pointer); the fp32 and fp8 forwards reject d = 256
    assert _fwd(lib, d=256, q=None) == fa.FA_ERR_NULL
    assert _fwd(lib, d=256, q=None, f32=True) == fa.FA_ERR_HEADDIM
    assert lib.fa_fwd_gqa(None, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, 1, 2, 1, 100, 256,
                          1, 0.1, None) == fa.FA_ERR_NULL
    assert lib.fa_fwd_kv(None, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, None, 0, 1, 2, 2, 10,
                         100, 256, 1, 0.1, None) == fa.FA_ERR_NULL
    assert _bwd(lib, d=256, dout=None) == fa.FA_ERR_NULL    # the backward takes 256 too
    assert lib.fa_bwd_workspace_size(1, 2, 100, 256) > 0
    assert _fwd(lib, d=512) == fa.FA_ERR_HEADDIM


def test_fp8_forward_rejects_bad_arguments(lib):
    def f(**kw):
        g = dict(q=A, k=A + MB, v=A + 2 * MB, o=A + 3 * MB, lse=A + 5 * MB, qs=0.01, ks=0.01,
                 vs=0.01, B=1, H=2, N=100, d=128, causal=1, scale=0.09)
        g.update(kw)
        return lib.fa_fwd_fp8(g["q"], g["k"], g["v"], g["o"], g["lse"], g["qs"], g["ks"],
                              g["vs"], g["B"], g["H"], g["N"], g["d"], g["causal"], g["scale"],
                              None)
    assert f(d=64) == fa.FA_ERR_HEADDIM
    assert f(d=256) == fa.FA_ERR_HEADDIM
    assert f(qs=math.inf) == fa.FA_ERR_SCALE
    assert f(vs=math.nan) == fa.FA_ERR_SCALE
    assert f(qs=1e30, ks=1e30) == fa.FA_ERR_SCALE      # the product overflows
    assert f(q=None) == fa.FA_ERR_NULL
    assert f(k=A + MB + 4) == fa.FA_ERR_ALIGN
    # q holds 2 x 100 x 128 bytes = 25600: an o starting inside it aliases
    assert f(o=A + 25600 - 16) == fa.FA_ERR_ALIAS
    assert f(N=0, q=None) == fa.FA_OK


def test_noalloc_backward_rejects_bad_arguments(lib):
    """fa_bwd_noalloc checks like fa_bwd, and refuses (before any HIP call) a
    problem whose workspace would not fit the static scratch buffer."""
    m = re.search(r"#define FA_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert fa.FA_STATIC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))

    def b(**kw):
        g = dict(q=A, k=A + MB, v=A + 2 * MB, o=A + 3 * MB, dout=A + 4 * MB, lse=A + 5 * MB,
                 dq=A + 6 * MB, dk=A + 7 * MB, dv=A + 8 * MB, B=1, H=2, N=100, d=64,
                 causal=1, scale=0.125)
        g.update(kw)
        return lib.fa_bwd_noalloc(g["q"], g["k"], g["v"], g["o"], g["dout"], g["lse"],
                                  g["dq"], g["dk"], g["dv"], g["B"], g["H"], g["N"], g["d"],
                                  g["causal"], g["scale"], None)
    assert b(d=96) == fa.FA_ERR_HEADDIM
    assert b(N=-1) == fa.FA_ERR_SHAPE
    assert b(scale=math.nan) == fa.FA_ERR_SCALE
    assert b(dq=None) == fa.FA_ERR_NULL
    assert b(lse=A + 5 * MB + 4) == fa.FA_ERR_ALIGN
    assert b(dk=A + 4 * MB) == fa.FA_ERR_ALIAS               # dk is dout
    assert b(dv=A + 7 * MB + 16) == fa.FA_ERR_ALIAS          # dv inside dk
    assert b(N=0, q=None) == fa.FA_OK
    # d = 64 keeps a float32 dQ accumulator: 4 x 16 x 8192 rows need 129 MiB
    big = dict(B=4, H=16, N=8192, d=64, q=A, k=A + (1 << 30), v=A + (2 << 30),
               o=A + (3 << 30), dout=A + (4 << 30), lse=A + (5 << 30), dq=A + (6 << 30),
               dk=A + (7 << 30), dv=A + (8 << 30))
    assert lib.fa_bwd_workspace_size(4, 16, 8192, 64) > fa.FA_STATIC_SCRATCH_BYTES
    assert b(**big) == fa.FA_ERR_SCRATCH
    assert "static" in fa.fa_status_string(fa.FA_ERR_SCRATCH)
