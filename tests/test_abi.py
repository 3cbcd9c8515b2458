"""The C ABI on the CPU: the library loads, exports what include/diffqkv.h
declares, and its host-side checks reject bad arguments before any launch.

Every call here fails validation (or is a pure host query), so no HIP call is
made; fake device pointers are 16-byte-aligned integers never dereferenced.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffqkv.h")

dq = pytest.importorskip("asymmetric_head_kv_amd")

OK, NULL, SHAPE, UNSUP, WS, HIP, ALIGN = 0, -1, -2, -3, -4, -5, -6
FAKE = 1 << 20  # aligned, never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dq.lib_path):
        pytest.skip("libdiffqkv.so not built")
    return dq.load()


def test_header_declares_the_entry_points():
    names = _declared()
    assert {"diffqkv_decode", "diffqkv_prefill", "kv_append", "diffqkv_decode_workspace",
            "diffqkv_decode_chunk", "dqkv_status_str"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(dq.SIGNATURES) == _declared()


def test_status_strings(lib):
    for code, name in dq.STATUS.items():
        assert lib.dqkv_status_str(code).decode().startswith(name)
    assert b"unknown" in lib.dqkv_status_str(42)


def _decode(lib, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, l_cap=1024,
            max_ctx=1024, scale=0.125, q=FAKE, k=FAKE, v=FAKE, ctx=FAKE, out=FAKE,
            lse=None, chunk=0, ws=FAKE, ws_bytes=0):
    return lib.diffqkv_decode(n_q, n_k, n_v, d_k, d_v, dtype, B, l_cap, max_ctx, scale,
                              q, k, v, ctx, out, lse, chunk, ws, ws_bytes, None)


@pytest.mark.parametrize("heads,code", [
    ((16, 3, 16), SHAPE),   # n_q not a multiple of n_k
    ((16, 4, 6), SHAPE),    # n_q not a multiple of n_v
    ((16, 32, 16), SHAPE),  # more K heads than query heads
    ((16, 4, 32), SHAPE),   # more V heads than query heads
    ((0, 1, 1), SHAPE),
    ((16, 0, 16), SHAPE),
])
def test_decode_rejects_bad_head_counts(lib, heads, code):
    n_q, n_k, n_v = heads
    assert _decode(lib, n_q=n_q, n_k=n_k, n_v=n_v) == code


def test_decode_rejects_unsupported_and_bad_sizes(lib):
    assert _decode(lib, d_k=48) == UNSUP
    assert _decode(lib, d_v=96) == UNSUP
    assert _decode(lib, dtype=7) == UNSUP
    assert _decode(lib, dtype=0, d_k=256) == UNSUP
    assert _decode(lib, max_ctx=2048, l_cap=1024) == SHAPE
    assert _decode(lib, B=-1) == SHAPE
    assert _decode(lib, scale=-0.125) == SHAPE
    assert _decode(lib, scale=float("nan")) == SHAPE
    assert _decode(lib, scale=float("inf")) == SHAPE
    # 0 selects the library's default 1/sqrt(d_k): validation goes on to the
    # next check (here the workspace size).
    assert _decode(lib, scale=0.0, ws_bytes=0) == WS
    assert _decode(lib, chunk=100) == SHAPE   # not a multiple of 64
    assert _decode(lib, chunk=-64) == SHAPE


def test_decode_null_alignment_and_workspace(lib):
    assert _decode(lib, q=None) == NULL
    assert _decode(lib, ctx=None) == NULL
    assert _decode(lib, ws=None) == NULL
    assert _decode(lib, k=FAKE + 8) == ALIGN
    assert _decode(lib, out=FAKE + 2) == ALIGN
    need = dq.decode_workspace_bytes(16, 4, 16, 64, 128, 1, 1024)
    assert _decode(lib, ws_bytes=need - 1) == WS
    assert _decode(lib, B=0) == OK  # nothing to do, nothing launched


def test_workspace_and_chunk_plan(lib):
    # Partials: (m, l) then acc[d_v], fp32, per (sequence, query head, chunk).
    # The automatic chunk of diffqkv_decode (contiguous caches) and that of
    # diffqkv_decode_paged (half as long for batches under 8 sequences); the
    # workspace query covers both.
    for (B, n_q, d_v, ctx, S_contig, S_paged) in [(1, 16, 128, 32768, 512, 256),
                                                  (16, 16, 128, 32769, 640, 640),
                                                  (4, 16, 128, 65536, 4608, 2048),
                                                  (1, 4, 64, 256, 64, 64)]:
        S = dq.decode_chunk(n_q, 4 if n_q > 4 else 1, n_q, 64, d_v, B, ctx)
        assert S == S_contig
        C = max(-(-ctx // S), -(-ctx // S_paged))
        parts = B * n_q * C
        expect = -(-parts * 8 // 256) * 256 + parts * d_v * 4
        assert dq.decode_workspace_bytes(n_q, 4 if n_q > 4 else 1, n_q, 64, d_v, B, ctx) == expect
    # Long single sequence: one four-wave workgroup per CU (4 K groups x 64
    # chunks).  Large batches (lengths unknown to the host, possibly ragged)
    # plan about seven times more chunks than a small batch would.
    assert 32768 // dq.decode_chunk(16, 4, 16, 64, 128, 1, 32768) == 64
    # One-round plans with chunks of 4096+ rows aim at 15/16 of the CUs in
    # 512-row steps when d_k <= 64 (4 x 64k: 15 chunks of 4608 rows), and keep
    # one workgroup per CU at larger d_k.
    assert dq.decode_chunk(16, 4, 16, 64, 128, 4, 65536) == 4608
    assert dq.decode_chunk(16, 4, 16, 128, 128, 4, 65536) == 4096
    assert dq.decode_chunk(16, 16, 16, 128, 128, 4, 65536) == 4096
    assert -(-32769 // dq.decode_chunk(16, 4, 16, 64, 128, 16, 32769)) >= 32
    # Layouts whose four-wave workgroup loads under 24Ki elements per 64-row
    # tile plan two workgroups per CU: the pages' SIGMA-1.5B attention (32 /
    # 4 / 16 heads, d 64: one K head and four V heads, 20Ki elements) gets
    # twice the chunks of one round; the standard GQA model (32 / 16 / 16,
    # four K and four V heads, 32Ki) and the 16 / 4 / 16 layout (36Ki) keep
    # one workgroup per CU.  The plan does not depend on the dtype.
    assert 32768 // dq.decode_chunk(32, 4, 16, 64, 64, 1, 32768) == 128
    assert 32768 // dq.decode_chunk(32, 16, 16, 64, 64, 1, 32768) == 64
    assert 16384 // dq.decode_chunk(32, 4, 16, 64, 64, 1, 16384) == 128
    # Explicit chunk lengths are honoured.
    assert dq.decode_workspace_bytes(16, 4, 16, 64, 128, 1, 4096, 64) == \
        -(-16 * 64 * 8 // 256) * 256 + 16 * 64 * 128 * 4
    with pytest.raises(dq.DQKVError):
        dq.decode_workspace_bytes(16, 4, 16, 64, 128, 1, 1 << 30, 64)  # too many chunks


def test_kv_append_validation(lib):
    def call(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=2, T=1, l_cap=100,
                 kn=FAKE, vn=FAKE, pos=FAKE, kc=FAKE, vc=FAKE)
        a.update(kw)
        return lib.kv_append(a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"],
                             a["B"], a["T"], a["l_cap"], a["kn"], a["vn"], a["pos"], a["kc"],
                             a["vc"], None)
    assert call(n_k=5) == SHAPE
    assert call(d_v=100) == UNSUP
    assert call(pos=None) == NULL
    assert call(vc=FAKE + 4) == ALIGN
    assert call(T=0) == OK and call(B=0) == OK
    assert call(T=-1) == SHAPE


def test_prefill_validation(lib):
    def call(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, T=128, l_cap=1024,
                 scale=0.125, q=FAKE, kc=FAKE, vc=FAKE, ctx=FAKE, out=FAKE, lse=None)
        a.update(kw)
        return lib.diffqkv_prefill(a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"],
                                   a["B"], a["T"], a["l_cap"], a["scale"], a["q"], a["kc"],
                                   a["vc"], a["ctx"], a["out"], a["lse"], None, 0, None)
    assert call(dtype=0) == UNSUP
    assert call(d_k=32) == UNSUP
    assert call(d_v=256) == UNSUP
    assert call(n_v=5) == SHAPE
    assert call(out=None) == NULL
    assert call(q=FAKE + 2) == ALIGN
    assert call(T=0) == OK


def test_prefill_workspace_plan(lib):
    # 2048 rows x 16 heads = 256 workgroups of 128 rows: two key splits so
    # that every CU gets two workgroups; large launches run unsplit.
    need = dq.prefill_workspace_bytes(16, 4, 16, 64, 128, 1, 2048)
    rows = 2048 * 16
    assert need == -(-2 * rows * 128 * 4 // 256) * 256 + 2 * rows * 4
    assert dq.prefill_workspace_bytes(16, 4, 16, 64, 128, 8, 4096) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 4, 32)
    k = torch.zeros(1, 1, 8, 32)
    v = torch.zeros(1, 4, 8, 64)
    with pytest.raises(ValueError):
        dq.decode(q, k, v, torch.zeros(1, dtype=torch.int32))


def test_selective_workspace_and_validation(lib):
    def layout(B, n_q, ctx, k):
        # Local-selection ranges of 4096 rows, or 2048 when 4096-row ranges
        # would give fewer (sequence, head, range) workgroups than 256 CUs.
        ld = max(64, -(-ctx // 64) * 64)
        rows = 2048 if B * n_q * max(1, -(-ctx // 4096)) < 256 else 4096
        nr = max(1, -(-ctx // rows))
        a = lambda x: -(-x // 256) * 256
        return a(B * n_q * ld * 4) + a(B * n_q * nr * 8) + a(B * n_q * nr * k * 4) + B * n_q * nr * k * 4

    for B, n_q, ctx, k in [(1, 16, 32768, 100), (4, 16, 65536, 100), (3, 32, 5001, 1024),
                           (2, 8, 0, 1)]:
        assert dq.selective_workspace_bytes(n_q, 4 if n_q > 4 else 1, n_q, 64, 128, B, ctx,
                                            k) == layout(B, n_q, ctx, k)
    for k, code in [(0, SHAPE), (-3, SHAPE), (1025, UNSUP)]:
        with pytest.raises(dq.DQKVError) as e:
            dq.selective_workspace_bytes(16, 4, 16, 64, 128, 1, 1024, k)
        assert e.value.status == code

    need = layout(1, 16, 1024, 100)

    def call(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, l_cap=1024,
                 max_ctx=1024, scale=0.125, top_k=100, q=FAKE, kn=None, vn=None, kc=FAKE,
                 vc=FAKE, ctx=FAKE, out=FAKE, lse=None, sel=None, ws=FAKE, ws_bytes=need)
        a.update(kw)
        return lib.diffqkv_decode_selective(
            a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"], a["B"], a["l_cap"],
            a["max_ctx"], a["scale"], a["top_k"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"],
            a["ctx"], a["out"], a["lse"], a["sel"], a["ws"], a["ws_bytes"], None)
    assert call(n_k=3) == SHAPE
    assert call(d_k=48) == UNSUP
    assert call(top_k=0) == SHAPE and call(top_k=2000) == UNSUP
    assert call(max_ctx=2048) == SHAPE
    assert call(scale=-1.0) == SHAPE
    assert call(kn=FAKE) == NULL          # k_new without v_new
    assert call(out=None) == NULL and call(ws=None) == NULL
    assert call(q=FAKE + 4) == ALIGN and call(kn=FAKE, vn=FAKE + 2) == ALIGN
    assert call(ws_bytes=need - 1) == WS
    assert call(B=0) == OK


def test_paged_and_compat_validation(lib):
    def dec(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, P=64, N=16, MB=16,
                 max_ctx=1024, scale=0.125, q=FAKE, kn=None, vn=None, kp=FAKE, vp=FAKE,
                 tab=FAKE, ctx=FAKE, out=FAKE, lse=None, chunk=0, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.diffqkv_decode_paged(
            a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"], a["B"], a["P"],
            a["N"], a["MB"], a["max_ctx"], a["scale"], a["q"], a["kn"], a["vn"], a["kp"],
            a["vp"], a["tab"], a["ctx"], a["out"], a["lse"], a["chunk"], a["ws"],
            a["ws_bytes"], None)
    for P in (0, 16, 32, 96, 100):
        assert dec(P=P) == SHAPE, P          # pages: a power of two >= 64 rows
    assert dec(N=0) == SHAPE and dec(MB=0) == SHAPE
    assert dec(max_ctx=16 * 64 + 1) == SHAPE  # beyond max_blocks * page_rows
    assert dec(tab=None) == NULL and dec(kn=FAKE) == NULL
    assert dec(kp=FAKE + 8) == ALIGN
    assert dec(n_k=3) == SHAPE
    assert dec(ws_bytes=0) == WS
    assert dec(B=0) == OK

    def app(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=2, T=1, P=64, N=8, MB=4,
                 kn=FAKE, vn=FAKE, pos=FAKE, tab=FAKE, kp=FAKE, vp=FAKE)
        a.update(kw)
        return lib.kv_append_paged(a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"],
                                   a["B"], a["T"], a["P"], a["N"], a["MB"], a["kn"], a["vn"],
                                   a["pos"], a["tab"], a["kp"], a["vp"], None)
    assert app(P=48) == SHAPE and app(N=0) == SHAPE
    assert app(tab=None) == NULL and app(vp=FAKE + 4) == ALIGN
    assert app(T=0) == OK and app(d_k=40) == UNSUP

    def pre(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, T=64, P=64, N=16, MB=16,
                 scale=0.125, q=FAKE, kp=FAKE, vp=FAKE, tab=FAKE, ctx=FAKE, out=FAKE, lse=None,
                 ws=None, ws_bytes=0)
        a.update(kw)
        return lib.diffqkv_prefill_paged(
            a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"], a["B"], a["T"], a["P"],
            a["N"], a["MB"], a["scale"], a["q"], a["kp"], a["vp"], a["tab"], a["ctx"], a["out"],
            a["lse"], a["ws"], a["ws_bytes"], None)
    assert pre(P=96) == SHAPE and pre(N=0) == SHAPE and pre(MB=0) == SHAPE
    assert pre(tab=None) == NULL and pre(q=None) == NULL
    assert pre(vp=FAKE + 8) == ALIGN and pre(dtype=0) == UNSUP and pre(d_k=32) == UNSUP
    assert pre(scale=-1.0) == SHAPE and pre(T=0) == OK and pre(B=0, tab=None) == OK

    def sel(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, P=64, N=16, MB=16,
                 max_ctx=1024, scale=0.125, k=100, q=FAKE, kn=None, vn=None, kp=FAKE, vp=FAKE,
                 tab=FAKE, ctx=FAKE, out=FAKE, lse=None, idx=None, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.diffqkv_decode_selective_paged(
            a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"], a["B"], a["P"],
            a["N"], a["MB"], a["max_ctx"], a["scale"], a["k"], a["q"], a["kn"], a["vn"],
            a["kp"], a["vp"], a["tab"], a["ctx"], a["out"], a["lse"], a["idx"], a["ws"],
            a["ws_bytes"], None)
    assert sel(P=32) == SHAPE and sel(N=0) == SHAPE and sel(max_ctx=16 * 64 + 1) == SHAPE
    assert sel(tab=None) == NULL and sel(kn=FAKE) == NULL and sel(vp=FAKE + 4) == ALIGN
    assert sel(k=0) == SHAPE and sel(k=1025) == UNSUP and sel(ws_bytes=0) == WS
    assert sel(B=0, tab=None) == OK

    def grp(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, cap=256, k=FAKE,
                 v=FAKE, ko=FAKE, vo=FAKE)
        a.update(kw)
        return lib.kv_group_sharing(a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"],
                                    a["dtype"], a["B"], a["cap"], a["k"], a["v"], a["ko"],
                                    a["vo"], None)
    assert grp(n_k=5) == SHAPE and grp(dtype=3) == UNSUP
    assert grp(ko=None) == NULL and grp(vo=FAKE + 2) == ALIGN
    assert grp(B=0) == OK and grp(cap=0) == OK


def test_augq_validation(lib):
    def call(**kw):
        a = dict(M=4, d_m=2048, d_i=3072, d_out=2048, h=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, q=FAKE,
                 ws=FAKE, ws_bytes=4 * 3072 * 2)
        a.update(kw)
        return lib.augq_forward(a["M"], a["d_m"], a["d_i"], a["d_out"], a["h"], a["wg"], a["wu"],
                                a["wd"], a["q"], a["ws"], a["ws_bytes"], None)
    assert call(M=-1) == SHAPE and call(d_out=0) == SHAPE
    assert call(d_m=1000) == UNSUP and call(d_i=3000) == UNSUP and call(d_out=100) == UNSUP
    assert call(wd=None) == NULL and call(h=FAKE + 2) == ALIGN and call(q=FAKE + 8) == ALIGN
    assert call(ws_bytes=4 * 3072 * 2 - 1) == WS
    assert call(M=0) == OK
    size = ctypes.c_size_t()
    assert lib.augq_workspace(7, 2048, 3072, 2048, ctypes.byref(size)) == OK
    assert size.value == 7 * 3072 * 2
    assert lib.augq_pack(24, 64, FAKE, FAKE, None) == UNSUP      # n_out % 16
    assert lib.augq_pack(32, 48, FAKE, FAKE, None) == UNSUP      # n_in % 32
    assert lib.augq_pack(32, 64, None, FAKE, None) == NULL
    assert lib.augq_pack(32, 64, FAKE, FAKE + 8, None) == ALIGN
    assert lib.augq_pack(0, 64, None, None, None) == OK


def test_decode_noalloc_validation(lib):
    # Host-side checks run before the library looks up its static scratch,
    # so none of these touches a device.
    def call(**kw):
        a = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128, dtype=1, B=1, l_cap=1024,
                 max_ctx=1024, scale=0.0, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE,
                 ctx=FAKE, out=FAKE, lse=None, chunk=0)
        a.update(kw)
        return lib.diffqkv_decode_append_noalloc(
            a["n_q"], a["n_k"], a["n_v"], a["d_k"], a["d_v"], a["dtype"], a["B"], a["l_cap"],
            a["max_ctx"], a["scale"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["ctx"],
            a["out"], a["lse"], a["chunk"], None)
    assert call(n_k=3) == SHAPE
    assert call(d_k=48) == UNSUP
    assert call(kn=None) == NULL          # k_new and v_new: both or neither
    assert call(q=None, kn=None, vn=None) == NULL
    assert call(vn=FAKE + 8) == ALIGN
    assert call(scale=-1.0) == SHAPE
    assert call(B=0) == OK
    # Partials beyond the 16 MiB static scratch: 16 sequences x 16 heads x
    # 8192 chunks of 64 rows need far more.
    assert call(B=16, l_cap=8192 * 64, max_ctx=8192 * 64, chunk=64) == WS

