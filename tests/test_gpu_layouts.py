"""GPU parity of the cache layouts: the kv_group_sharing expansion, and the
paged cache (decode, fused append and kv_append through a page table).

The expansion is a copy and must be bit-exact; decoding the expanded layout
must give bit-identical results to the native one (same kernels, same rows,
same order).  A paged decode with the same chunking must be bit-identical to
the contiguous decode of the gathered caches, and within the usual tolerance
of the oracle, whose paged_to_contiguous defines the layout.  Pages are
assigned in a seeded random order, with spare pages and unused table
entries, so any wrong table lookup shows up.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, assert_lse_close, ints_to_dev, raw_host, to_dev, to_host, upload

pytestmark = pytest.mark.gpu
dq = pytest.importorskip("asymmetric_head_kv_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dq.load()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_pages(k, v, lens, P, seed, spare=3, extra_blocks=1):
    """Scatter head-major caches (raw host arrays) into shuffled pages.
    Returns (k_pages, v_pages, table); unused table entries are -1."""
    B, n_k, cap, d_k = k.shape
    n_v, d_v = v.shape[1], v.shape[3]
    need = [-(-int(L) // P) for L in lens]
    n_pages = sum(need) + spare
    order = np.random.default_rng(seed).permutation(n_pages)
    max_blocks = max(need + [1]) + extra_blocks
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    kp = np.zeros((n_pages, n_k, P, d_k), dtype=k.dtype)
    vp = np.zeros((n_pages, n_v, P, d_v), dtype=v.dtype)
    nxt = 0
    for b in range(B):
        for blk in range(need[b]):
            page = int(order[nxt])
            nxt += 1
            table[b, blk] = page
            r0, r1 = blk * P, min((blk + 1) * P, cap)
            kp[page, :, :r1 - r0] = k[b, :, r0:r1]
            vp[page, :, :r1 - r0] = v[b, :, r0:r1]
    return kp, vp, table


# ------------------------------------------------------------ kv_group_sharing

@pytest.mark.parametrize("dtype,heads", [("bf16", (16, 4, 16)), ("f32", (8, 8, 2)),
                                         ("bf16", (32, 4, 16))])
def test_kv_group_sharing_bit_exact_and_decode_unchanged(dtype, heads):
    n_q, n_k, n_v = heads
    case = synth.make_case(401, dtype=dtype, batch=2, n_q=n_q, n_k=n_k, n_v=n_v, d_k=64,
                           d_v=128 if dtype == "bf16" else 64, ctx_len=[700, 300], l_cap=704)
    _say("kv_group_sharing", dtype, heads)
    q, k, v, ctx = upload(case)
    kx, vx = dq.kv_group_sharing(k, v, n_q=n_q)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_group_sharing(case.k_cache, case.v_cache)
    np.testing.assert_array_equal(raw_host(kx), ek)
    np.testing.assert_array_equal(raw_host(vx), ev)
    lse_a = torch.empty((2, n_q), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    out_a, _ = dq.decode(q, k, v, ctx, scale=case.scale, lse=lse_a)
    out_b, _ = dq.decode(q, kx, vx, ctx, scale=case.scale, lse=lse_b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out_a), raw_host(out_b))
    np.testing.assert_array_equal(lse_a.cpu().numpy(), lse_b.cpu().numpy())


# ------------------------------------------------------------------ paged cache

PAGED = [
    # dtype, n_q, n_k, n_v, d_k, d_v, lengths, page rows
    ("bf16", 16, 4, 16, 64, 128, [5000, 777, 64, 1], 64),
    ("bf16", 32, 4, 16, 64, 64, [3000, 2049], 128),
    ("bf16", 16, 16, 16, 128, 128, [1500], 256),
    ("f32", 8, 2, 4, 64, 32, [900, 65, 129], 64),
]


def run_paged(case, P, seed, k_new=None, v_new=None, chunk=0):
    kp, vp, table = make_pages(case.k_cache, case.v_cache, case.ctx_len, P, seed)
    kp_d, vp_d = to_dev(kp, case.dtype), to_dev(vp, case.dtype)
    tab = ints_to_dev(table)
    q = to_dev(case.q, case.dtype)
    ctx = ints_to_dev(case.ctx_len)
    lse = torch.empty((case.batch, case.n_q), dtype=torch.float32, device="cuda")
    out, _ = dq.decode_paged(q, kp_d, vp_d, tab, ctx, max_ctx=case.l_cap, scale=case.scale,
                             lse=lse, chunk_tokens=chunk, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    return out, lse, (kp_d, vp_d, table)


@pytest.mark.parametrize("cfg", PAGED, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-P{c[7]}")
def test_paged_decode_matches_contiguous_and_oracle(cfg):
    dtype, n_q, n_k, n_v, d_k, d_v, lens, P = cfg
    cap = max(lens)
    case = synth.make_case(402, dtype=dtype, batch=len(lens), n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=cap)
    _say("paged decode", cfg)
    # Same chunking: bit-identical (the contiguous default, and 192 rows).
    S0 = dq.decode_chunk(n_q, n_k, n_v, d_k, d_v, len(lens), cap)
    for chunk in (S0, 192):
        out_p, lse_p, _ = run_paged(case, P, seed=P + chunk, chunk=chunk)
        q, k, v, ctx = upload(case)
        lse_c = torch.empty_like(lse_p)
        out_c, _ = dq.decode(q, k, v, ctx, scale=case.scale, lse=lse_c, chunk_tokens=chunk)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(raw_host(out_p), raw_host(out_c))
        np.testing.assert_array_equal(lse_p.cpu().numpy(), lse_c.cpu().numpy())
    # The paged path's own default chunking, against the oracle.
    out_p, lse_p, _ = run_paged(case, P, seed=P)
    qw, kw, vw = case.widened()
    ref, ref_lse = oracle.decode(qw, kw, vw, case.ctx_len, case.scale)
    err = assert_close(to_host(out_p), ref, dtype, f"paged {cfg}")
    assert_lse_close(to_host(lse_p), ref_lse, dtype, f"paged {cfg}")
    _say(f"  normwise rel err {err:.2e}")


def test_paged_fused_append_matches_separate_append():
    lens = [3001, 128, 1]
    case = synth.make_case(403, dtype="bf16", batch=3, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=lens, l_cap=3072)
    kn, vn = synth.new_rows(403, dtype="bf16", batch=3, t_new=1, n_k=4, n_v=16, d_k=64, d_v=128)
    kn_d, vn_d = to_dev(kn, "bf16"), to_dev(vn, "bf16")
    _say("paged fused append")
    out_f, lse_f, (kp_f, vp_f, table) = run_paged(case, 64, seed=7, k_new=kn_d, v_new=vn_d)
    kp, vp, _ = make_pages(case.k_cache, case.v_cache, case.ctx_len, 64, seed=7)
    kp_s, vp_s = to_dev(kp, "bf16"), to_dev(vp, "bf16")
    tab = ints_to_dev(table)
    dq.kv_append_paged(kn_d, vn_d, ints_to_dev(np.asarray(lens) - 1), tab, kp_s, vp_s, n_q=16)
    lse_s = torch.empty_like(lse_f)
    out_s, _ = dq.decode_paged(to_dev(case.q, "bf16"), kp_s, vp_s, tab,
                               ints_to_dev(case.ctx_len), max_ctx=3072, scale=case.scale,
                               lse=lse_s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(kp_f), raw_host(kp_s))
    np.testing.assert_array_equal(raw_host(vp_f), raw_host(vp_s))
    np.testing.assert_array_equal(raw_host(out_f), raw_host(out_s))
    np.testing.assert_array_equal(lse_f.cpu().numpy(), lse_s.cpu().numpy())
    # And the appended rows are where the layout says.
    kc, vc = oracle.paged_to_contiguous(raw_host(kp_f), raw_host(vp_f), table, case.ctx_len,
                                        l_cap=3072)
    for b, L in enumerate(lens):
        np.testing.assert_array_equal(kc[b, :, L - 1], kn[b, 0])
        np.testing.assert_array_equal(vc[b, :, L - 1], vn[b, 0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_append_paged_against_oracle(dtype):
    B, T, n_k, n_v, d_k, d_v, P = 3, 70, 2, 8, 64, 64, 64
    lens = np.array([200, 64, 0])          # rows already cached
    cap = 320
    case = synth.make_case(404, dtype=dtype, batch=B, n_q=8, n_k=n_k, n_v=n_v, d_k=d_k,
                           d_v=d_v, ctx_len=lens + T, l_cap=cap)
    kn, vn = synth.new_rows(404, dtype=dtype, batch=B, t_new=T, n_k=n_k, n_v=n_v, d_k=d_k,
                            d_v=d_v)
    kp, vp, table = make_pages(case.k_cache, case.v_cache, lens + T, P, seed=11)
    kp_d, vp_d = to_dev(kp, dtype), to_dev(vp, dtype)
    _say("kv_append_paged", dtype)
    dq.kv_append_paged(to_dev(kn, dtype), to_dev(vn, dtype), ints_to_dev(lens),
                       ints_to_dev(table), kp_d, vp_d, n_q=8)
    torch.cuda.synchronize()
    got_k, got_v = oracle.paged_to_contiguous(raw_host(kp_d), raw_host(vp_d), table, lens + T,
                                              l_cap=cap)
    want_k, want_v = oracle.kv_append(case.k_cache, case.v_cache, kn, vn, lens)
    for b in range(B):
        L = int(lens[b]) + T
        np.testing.assert_array_equal(got_k[b, :, :L].view(np.uint8), want_k[b, :, :L].view(np.uint8))
        np.testing.assert_array_equal(got_v[b, :, :L].view(np.uint8), want_v[b, :, :L].view(np.uint8))
    # Pages no sequence uses are untouched.
    used = set(int(x) for x in table.ravel() if x >= 0)
    for page in set(range(kp.shape[0])) - used:
        np.testing.assert_array_equal(raw_host(kp_d)[page], kp[page])


@pytest.mark.parametrize("P", [64, 256])
def test_paged_full_workload(P):
    case = synth.make_case(**synth.workload("decode32k_asym"))
    _say("paged full workload decode32k_asym, page rows", P)
    # With the contiguous default chunking: bit-identical to the contiguous
    # decode; with its own default: within tolerance of the oracle.
    S0 = dq.decode_chunk(case.n_q, case.n_k, case.n_v, case.d_k, case.d_v, case.batch, case.l_cap)
    out_p, lse_p, _ = run_paged(case, P, seed=P, chunk=S0)
    q, k, v, ctx = upload(case)
    lse_c = torch.empty_like(lse_p)
    out_c, _ = dq.decode(q, k, v, ctx, scale=case.scale, lse=lse_c)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out_p), raw_host(out_c))
    out_p, lse_p, _ = run_paged(case, P, seed=P)
    qw, kw, vw = case.widened()
    ref, ref_lse = oracle.decode(qw, kw, vw, case.ctx_len, case.scale)
    err = assert_close(to_host(out_p), ref, "bf16", "paged 32k")
    assert_lse_close(to_host(lse_p), ref_lse, "bf16", "paged 32k")
    _say(f"  normwise rel err {err:.2e}")


def test_binding_rejects_mismatched_paged_arguments():
    # The binding checks dtypes and shapes before anything is launched: one
    # dtype code travels over the C ABI, so a mismatch would be misread.
    q = torch.zeros((1, 4, 64), dtype=torch.float32, device="cuda")
    kp = torch.zeros((2, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros((2, 4, 64, 64), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    ctx = torch.full((1,), 64, dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        dq.decode_paged(q, kp, vp, table, ctx)
    qb = q.to(torch.bfloat16)
    with pytest.raises(ValueError):
        dq.decode_paged(qb, kp, vp, table, ctx, out=torch.empty((1, 4, 32), dtype=torch.bfloat16,
                                                                 device="cuda"))
    with pytest.raises(ValueError):
        dq.decode_paged(qb, kp, vp, table, ctx, lse=torch.empty((1, 4), dtype=torch.bfloat16,
                                                                 device="cuda"))
    kn = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        dq.kv_append_paged(kn.view(1, 1, 1, 64), kn.new_zeros((1, 1, 4, 64)),
                           ctx, table, kp, vp)



@pytest.mark.parametrize("P,lens,t_new", [(64, [1000, 333], 200), (256, [2048, 1100], 300)])
def test_paged_prefill_matches_contiguous(P, lens, t_new):
    # The same rows in pages of P rows, in a seeded random page order: the
    # paged prefill reads the same keys in the same order, so its output (and
    # lse) equals the contiguous prefill's bit for bit; the contiguous one is
    # itself checked against the oracle elsewhere, and here on a sample.
    _say("paged prefill", P, lens, t_new)
    B = len(lens)
    case = synth.make_case(970 + P, dtype="bf16", batch=B, n_q=16, n_k=4, n_v=16, d_k=64,
                           d_v=128, ctx_len=lens, l_cap=max(lens), t_new=t_new)
    q, k, v, ctx = upload(case)
    rng = np.random.default_rng(P)
    need = [-(-L // P) for L in lens]
    n_pages = sum(need) + 3
    order = rng.permutation(n_pages)
    table = np.full((B, max(need) + 1), -1, dtype=np.int32)
    kp = np.zeros((n_pages, 4, P, 64), dtype=case.k_cache.dtype)
    vp = np.zeros((n_pages, 16, P, 128), dtype=case.v_cache.dtype)
    nxt = 0
    for b, L in enumerate(lens):
        for blk in range(need[b]):
            page = int(order[nxt])
            nxt += 1
            table[b, blk] = page
            r1 = min((blk + 1) * P, L)
            kp[page, :, :r1 - blk * P] = case.k_cache[b, :, blk * P:r1]
            vp[page, :, :r1 - blk * P] = case.v_cache[b, :, blk * P:r1]
    lse_c = torch.empty((B, t_new, 16), dtype=torch.float32, device="cuda")
    lse_p = torch.empty_like(lse_c)
    out_c, _ = dq.prefill(q, k, v, ctx, scale=case.scale, lse=lse_c)
    out_p, _ = dq.prefill_paged(q, to_dev(kp, "bf16"), to_dev(vp, "bf16"), ints_to_dev(table),
                                ctx, scale=case.scale, lse=lse_p)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out_p), raw_host(out_c))
    np.testing.assert_array_equal(raw_host(lse_p), raw_host(lse_c))
    # A sample of rows against the oracle.
    qw, kw, vw = case.widened()
    ref, _ = oracle.prefill(qw[:, -4:], kw, vw, case.ctx_len, case.scale)
    assert_close(to_host(out_p)[:, -4:], ref, "bf16", "paged prefill, last rows")



@pytest.mark.parametrize("fused", [False, True])
def test_paged_selective_matches_contiguous(fused):
    # Selective V over 64-row pages in a random order: the same logits, the
    # same chosen rows and the same sums as on the contiguous cache, bit for
    # bit; with the fused append both caches receive the same new row.
    lens, P, top_k = [3000, 1234], 64, 100
    B = len(lens)
    _say("paged selective", "fused" if fused else "plain", lens)
    case = synth.make_case(990 + fused, dtype="bf16", batch=B, n_q=16, n_k=4, n_v=16, d_k=64,
                           d_v=128, ctx_len=lens, l_cap=max(lens))
    q, k, v, ctx = upload(case)
    rng = np.random.default_rng(7 + fused)
    need = [-(-L // P) for L in lens]
    n_pages = sum(need) + 2
    order = rng.permutation(n_pages)
    table = np.full((B, max(need)), -1, dtype=np.int32)
    kp = np.zeros((n_pages, 4, P, 64), dtype=case.k_cache.dtype)
    vp = np.zeros((n_pages, 16, P, 128), dtype=case.v_cache.dtype)
    nxt = 0
    for b, L in enumerate(lens):
        for blk in range(need[b]):
            page = int(order[nxt])
            nxt += 1
            table[b, blk] = page
            r1 = min((blk + 1) * P, L)
            kp[page, :, :r1 - blk * P] = case.k_cache[b, :, blk * P:r1]
            vp[page, :, :r1 - blk * P] = case.v_cache[b, :, blk * P:r1]
    kp_d, vp_d, tab_d = to_dev(kp, "bf16"), to_dev(vp, "bf16"), ints_to_dev(table)
    kw_ = vw_ = None
    if fused:
        kn, vn = synth.new_rows(991, dtype="bf16", batch=B, t_new=1, n_k=4, n_v=16, d_k=64,
                                d_v=128)
        kw_, vw_ = to_dev(kn, "bf16"), to_dev(vn, "bf16")
    outs = []
    for paged in (False, True):
        lse = torch.empty((B, 16), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, 16, top_k), dtype=torch.int32, device="cuda")
        if paged:
            o, _, _ = dq.decode_selective_paged(q, kp_d, vp_d, tab_d, ctx, top_k=top_k,
                                                max_ctx=max(lens), scale=case.scale, lse=lse,
                                                sel_idx=idx, k_new=kw_, v_new=vw_)
        else:
            o, _, _ = dq.decode_selective(q, k, v, ctx, top_k=top_k, scale=case.scale, lse=lse,
                                          sel_idx=idx, k_new=kw_, v_new=vw_)
        outs.append((o, lse, idx))
    torch.cuda.synchronize()
    for a, b_ in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(raw_host(a), raw_host(b_))
    if fused:
        # The appended rows landed in the right page slots.
        kph, vph = raw_host(kp_d), raw_host(vp_d)
        kh, vh = raw_host(k), raw_host(v)
        for b, L in enumerate(lens):
            page, slot = table[b, (L - 1) // P], (L - 1) % P
            np.testing.assert_array_equal(kph[page, :, slot], kh[b, :, L - 1])
            np.testing.assert_array_equal(vph[page, :, slot], vh[b, :, L - 1])



def test_paged_decode_full_size_matches_contiguous():
    # The 32k single-sequence workload in 64-row pages (a seeded random page
    # order, as the benchmark's paged leg): bit-identical to the contiguous
    # decode, whose full-size parity with the oracle is tested elsewhere.
    wl = synth.workload("decode32k_asym")
    L = int(np.asarray(wl["ctx_len"]).reshape(-1)[0])
    case = synth.make_case(17, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[L], l_cap=L)
    q, k, v, ctx = upload(case)
    P = 64
    n_pg = -(-L // P)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(n_pg)).to("cuda")
    kp = torch.empty((n_pg, 4, P, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty((n_pg, 16, P, 128), dtype=torch.bfloat16, device="cuda")
    kp[perm] = k[0].view(4, n_pg, P, 64).permute(1, 0, 2, 3)
    vp[perm] = v[0].view(16, n_pg, P, 128).permute(1, 0, 2, 3)
    table = perm.to(torch.int32).view(1, n_pg)
    _say("paged decode, full size", L, "pages", n_pg)
    S0 = dq.decode_chunk(16, 4, 16, 64, 128, 1, L)  # the same chunking for both
    out_p, _ = dq.decode_paged(q, kp, vp, table, ctx, max_ctx=L, scale=case.scale,
                               chunk_tokens=S0)
    out_c, _ = dq.decode(q, k, v, ctx, scale=case.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out_p), raw_host(out_c))
