"""GPU checks of the fused appends' guards and of the default softmax scale.

A fused append (the decode and selective-V entry points that take k_new /
v_new) must write nothing for a sequence whose length lies past the launch's
bound (the length is clamped for reading, and the row it would overwrite is
history), and nothing through a page-table entry that names no page (such a
write would land in another sequence's page).  kv_append skips such rows in
the same way.  scale = 0 (the binding's default) selects 1/sqrt(d_k).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, ints_to_dev, raw_host, to_dev, to_host, upload

pytestmark = pytest.mark.gpu
dq = pytest.importorskip("asymmetric_head_kv_amd")

SHAPE = dict(n_q=16, n_k=4, n_v=16, d_k=64, d_v=128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dq.load()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _pages(k, v, lens, P, seed):
    """Head-major host caches -> shuffled pages (every block of l_cap rows
    mapped) and the table."""
    B, n_k, cap, d_k = k.shape
    n_v, d_v = v.shape[1], v.shape[3]
    nblk = -(-cap // P)
    n_pages = B * nblk + 2
    order = np.random.default_rng(seed).permutation(n_pages)
    table = np.zeros((B, nblk), dtype=np.int32)
    kp = np.zeros((n_pages, n_k, P, d_k), dtype=k.dtype)
    vp = np.zeros((n_pages, n_v, P, d_v), dtype=v.dtype)
    for b in range(B):
        for blk in range(nblk):
            page = int(order[b * nblk + blk])
            table[b, blk] = page
            r0, r1 = blk * P, min((blk + 1) * P, cap)
            kp[page, :, :r1 - r0] = k[b, :, r0:r1]
            vp[page, :, :r1 - r0] = v[b, :, r0:r1]
    return kp, vp, table


@pytest.mark.parametrize("path", ["decode", "selective"])
def test_fused_append_skips_a_length_past_max_ctx(path):
    # Sequence 0 claims max_ctx + 1 rows: it attends the first max_ctx rows
    # of the unchanged cache and appends nothing; sequence 1 appends as usual.
    cap = 704
    lens = np.array([cap + 1, 500])
    case = synth.make_case(611, dtype="bf16", batch=2, ctx_len=[cap, 500], l_cap=cap, **SHAPE)
    kn, vn = synth.new_rows(611, dtype="bf16", batch=2, t_new=1, n_k=4, n_v=16, d_k=64, d_v=128)
    q, k, v, _ = upload(case)
    ctx = ints_to_dev(lens)
    _say("fused append, length past max_ctx,", path)
    if path == "decode":
        out, _ = dq.decode(q, k, v, ctx, max_ctx=cap, k_new=to_dev(kn, "bf16"),
                           v_new=to_dev(vn, "bf16"))
    else:
        out, _, _ = dq.decode_selective(q, k, v, ctx, top_k=cap, max_ctx=cap,
                                        k_new=to_dev(kn, "bf16"), v_new=to_dev(vn, "bf16"))
    torch.cuda.synchronize()
    want_k, want_v = oracle.kv_append(case.k_cache[1:], case.v_cache[1:], kn[1:], vn[1:], [499])
    gk, gv = raw_host(k), raw_host(v)
    np.testing.assert_array_equal(gk[0], case.k_cache[0])
    np.testing.assert_array_equal(gv[0], case.v_cache[0])
    np.testing.assert_array_equal(gk[1], want_k[0])
    np.testing.assert_array_equal(gv[1], want_v[0])
    # Both sequences attend what the cache holds (top_k = all rows: full decode).
    kw = synth.bf16_bits_to_f32(gk).astype(np.float64)
    vw = synth.bf16_bits_to_f32(gv).astype(np.float64)
    qw = synth.bf16_bits_to_f32(case.q).astype(np.float64)
    ref, _ = oracle.decode(qw, kw, vw, [cap, 500], case.scale)
    assert_close(to_host(out), ref, "bf16", f"{path}, clamped length")


@pytest.mark.parametrize("path", ["decode", "selective"])
def test_paged_fused_append_skips_a_missing_page(path):
    # The table entry of sequence 0's newest row is -1: its new row must not
    # be written anywhere (reads clamp the entry; its output is not checked).
    # Sequence 1 appends normally; every other page byte stays as it was.
    P, cap = 64, 768
    lens = [700, 300]
    case = synth.make_case(612, dtype="bf16", batch=2, ctx_len=lens, l_cap=cap, **SHAPE)
    kn, vn = synth.new_rows(612, dtype="bf16", batch=2, t_new=1, n_k=4, n_v=16, d_k=64, d_v=128)
    kp, vp, table = _pages(case.k_cache, case.v_cache, lens, P, seed=5)
    table[0, (lens[0] - 1) // P] = -1
    kp_d, vp_d, tab_d = to_dev(kp, "bf16"), to_dev(vp, "bf16"), ints_to_dev(table)
    q, ctx = to_dev(case.q, "bf16"), ints_to_dev(lens)
    _say("paged fused append, missing page,", path)
    if path == "decode":
        out, _ = dq.decode_paged(q, kp_d, vp_d, tab_d, ctx, max_ctx=cap,
                                 k_new=to_dev(kn, "bf16"), v_new=to_dev(vn, "bf16"))
    else:
        out, _, _ = dq.decode_selective_paged(q, kp_d, vp_d, tab_d, ctx, top_k=100, max_ctx=cap,
                                              k_new=to_dev(kn, "bf16"), v_new=to_dev(vn, "bf16"))
    torch.cuda.synchronize()
    want_k, want_v = kp.copy(), vp.copy()
    page, slot = table[1, (lens[1] - 1) // P], (lens[1] - 1) % P
    want_k[page, :, slot] = kn[1, 0]
    want_v[page, :, slot] = vn[1, 0]
    np.testing.assert_array_equal(raw_host(kp_d), want_k)
    np.testing.assert_array_equal(raw_host(vp_d), want_v)
    if path == "decode":
        kc, vc = oracle.kv_append(case.k_cache[1:], case.v_cache[1:], kn[1:], vn[1:], [299])
        ref, _ = oracle.decode(synth.bf16_bits_to_f32(case.q[1:]).astype(np.float64),
                               synth.bf16_bits_to_f32(kc).astype(np.float64),
                               synth.bf16_bits_to_f32(vc).astype(np.float64), [300], case.scale)
        assert_close(to_host(out)[1:], ref, "bf16", "paged decode, intact sequence")


@pytest.mark.parametrize("d_k", [64, 128])
def test_default_scale_is_inverse_sqrt_dk(d_k):
    # scale=None passes 0 over the C ABI, which the library reads as
    # 1/sqrt(d_k) in fp32: the same bits as passing that value explicitly.
    case = synth.make_case(613, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16, d_k=d_k, d_v=128,
                           ctx_len=[900], l_cap=960)
    q, k, v, ctx = upload(case)
    s32 = float(np.float32(1) / np.sqrt(np.float32(d_k)))
    _say("default scale, d_k", d_k)
    a, _ = dq.decode(q, k, v, ctx)
    b, _ = dq.decode(q, k, v, ctx, scale=s32)
    pa, _ = dq.prefill(q.view(1, 1, 16, d_k), k, v, ctx)
    pb, _ = dq.prefill(q.view(1, 1, 16, d_k), k, v, ctx, scale=s32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(a), raw_host(b))
    np.testing.assert_array_equal(raw_host(pa), raw_host(pb))
    qw, kw, vw = case.widened()
    ref, _ = oracle.decode(qw, kw, vw, case.ctx_len)   # the oracle's own default scale
    assert_close(to_host(a), ref, "bf16", f"default scale d_k={d_k}")
