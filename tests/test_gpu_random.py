"""Seeded random sweeps of the decode entry points against the fp64 oracle:
head layouts (either side the smaller one), head dimensions, dtypes, batch
sizes, ragged lengths (1 row .. several chunks, ragged tails) and chunk
lengths; selective V with random top_k; the paged cache with random page
sizes; the causal prefill over random head layouts, head dimensions, new-row
counts (rows with no visible key included), scales, key splits, paged
caches and planted logits far above the first key tile's.  Every
configuration is printed before it runs."""

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


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def random_config(rng):
    dtype = ["f32", "bf16"][rng.integers(2)]
    n_q = int(rng.choice([4, 6, 8, 12, 16, 32]))
    n_k = int(rng.choice(_divisors(n_q)))
    n_v = int(rng.choice(_divisors(n_q)))
    dims = [32, 64, 128] + ([256] if dtype == "bf16" else [])
    d_k = int(rng.choice(dims))
    d_v = int(rng.choice([32, 64, 128, 256]))
    B = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 2500, size=B)]
    cap = max(lens) + int(rng.integers(0, 100))
    chunk = int(rng.choice([0, 64, 128, 320]))
    return dtype, n_q, n_k, n_v, d_k, d_v, lens, cap, chunk


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_shapes(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype, n_q, n_k, n_v, d_k, d_v, lens, cap, chunk = random_config(rng)
    _say("random decode", seed, dtype, (n_q, n_k, n_v, d_k, d_v), lens, cap, chunk)
    case = synth.make_case(700 + seed, dtype=dtype, batch=len(lens), n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=cap, poison_tail=True)
    q, k, v, ctx = upload(case)
    lse = torch.empty((case.batch, n_q), dtype=torch.float32, device="cuda")
    out, _ = dq.decode(q, k, v, ctx, scale=case.scale, lse=lse, chunk_tokens=chunk)
    torch.cuda.synchronize()
    qw, kw, vw = case.widened()
    ref, ref_lse = oracle.decode(qw, kw, vw, case.ctx_len, case.scale)
    err = assert_close(to_host(out), ref, dtype, f"seed {seed}")
    assert_lse_close(to_host(lse), ref_lse, dtype, f"seed {seed}")
    _say(f"  normwise rel err {err:.2e}")


@pytest.mark.parametrize("seed", range(6))
def test_selective_random_shapes(seed):
    rng = np.random.default_rng(2000 + seed)
    dtype, n_q, n_k, n_v, d_k, d_v, lens, cap, _ = random_config(rng)
    lens = [int(x) for x in rng.integers(1, 9000, size=len(lens))]
    cap = max(lens)
    top_k = int(rng.choice([1, 7, 100, 333, 1024]))
    _say("random selective", seed, dtype, (n_q, n_k, n_v, d_k, d_v), lens, top_k)
    case = synth.make_case(800 + seed, dtype=dtype, batch=len(lens), n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=cap, poison_tail=True)
    q, k, v, ctx = upload(case)
    sel = torch.empty((case.batch, n_q, top_k), dtype=torch.int32, device="cuda")
    out, _, _ = dq.decode_selective(q, k, v, ctx, top_k=top_k, scale=case.scale, sel_idx=sel)
    torch.cuda.synchronize()
    qw, kw, vw = case.widened()
    got_sel = sel.cpu().numpy()
    ref = np.zeros((case.batch, n_q, d_v))
    for b, L in enumerate(lens):
        kk = min(top_k, L)
        for i in range(n_q):
            rows = got_sel[b, i, :kk]
            assert (got_sel[b, i, kk:] == -1).all() and (np.diff(rows) > 0).all()
            hk, hv = i * n_k // n_q, i * n_v // n_q
            logits = case.scale * (kw[b, hk, :L].astype(np.float64) @ qw[b, i].astype(np.float64))
            if kk < L:
                mask = np.zeros(L, bool)
                mask[rows] = True
                assert logits[mask].min() >= logits[~mask].max() - 1e-4, (b, i)
            ref[b, i], _ = oracle.attend_selective_one(qw[b, i], kw[b, hk, :L], vw[b, hv, :L],
                                                       case.scale, top_k, rows=rows)
    err = assert_close(to_host(out), ref, dtype, f"seed {seed}")
    _say(f"  normwise rel err {err:.2e}")


@pytest.mark.parametrize("seed", range(6))
def test_paged_random_shapes(seed):
    rng = np.random.default_rng(3000 + seed)
    dtype, n_q, n_k, n_v, d_k, d_v, lens, _, chunk = random_config(rng)
    P = int(rng.choice([64, 128, 256, 512]))
    _say("random paged", seed, dtype, (n_q, n_k, n_v, d_k, d_v), lens, "page rows", P)
    case = synth.make_case(900 + seed, dtype=dtype, batch=len(lens), n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=max(lens))
    need = [-(-L // P) for L in lens]
    n_pages = sum(need) + 2
    order = rng.permutation(n_pages)
    table = np.full((len(lens), max(need) + 1), -1, dtype=np.int32)
    kp = np.zeros((n_pages, n_k, P, d_k), dtype=case.k_cache.dtype)
    vp = np.zeros((n_pages, n_v, P, d_v), dtype=case.v_cache.dtype)
    nxt = 0
    for b, L in enumerate(lens):
        for blk in range(need[b]):
            page = int(order[nxt])
            nxt += 1
            table[b, blk] = page
            r1 = min((blk + 1) * P, L)
            kp[page, :, :r1 - blk * P] = case.k_cache[b, :, blk * P:r1]
            vp[page, :, :r1 - blk * P] = case.v_cache[b, :, blk * P:r1]
    out, _ = dq.decode_paged(to_dev(case.q, dtype), to_dev(kp, dtype), to_dev(vp, dtype),
                             ints_to_dev(table), ints_to_dev(case.ctx_len), max_ctx=max(lens),
                             scale=case.scale, chunk_tokens=chunk)
    q, k, v, ctx = upload(case)
    ref_gpu, _ = dq.decode(q, k, v, ctx, scale=case.scale, chunk_tokens=chunk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out), raw_host(ref_gpu))
    qw, kw, vw = case.widened()
    ref, _ = oracle.decode(qw, kw, vw, case.ctx_len, case.scale)
    err = assert_close(to_host(out), ref, dtype, f"seed {seed}")
    _say(f"  normwise rel err {err:.2e}")


@pytest.mark.parametrize("seed", range(2))
def test_decode_large_ragged_batch(seed):
    # Batches of eight or more sequences plan smaller chunks (the lengths are
    # not known on the host): many chunks are empty for the short sequences.
    rng = np.random.default_rng(4000 + seed)
    B = int(rng.integers(8, 17))
    lens = [int(x) for x in rng.integers(1, 3000, size=B)]
    lens[int(rng.integers(B))] = 3000
    dtype = ["bf16", "f32"][seed % 2]
    _say("large ragged batch", seed, dtype, B, lens)
    case = synth.make_case(950 + seed, dtype=dtype, batch=B, n_q=16, n_k=4, n_v=16, d_k=64,
                           d_v=128, ctx_len=lens, l_cap=3000, poison_tail=True)
    q, k, v, ctx = upload(case)
    lse = torch.empty((B, 16), dtype=torch.float32, device="cuda")
    out, _ = dq.decode(q, k, v, ctx, scale=case.scale, lse=lse)
    torch.cuda.synchronize()
    qw, kw, vw = case.widened()
    ref, ref_lse = oracle.decode(qw, kw, vw, case.ctx_len, case.scale)
    err = assert_close(to_host(out), ref, dtype, f"seed {seed}")
    assert_lse_close(to_host(lse), ref_lse, dtype, f"seed {seed}")
    _say(f"  normwise rel err {err:.2e}")


def _pages_of(case, P, rng):
    """The case's cache rows in pages of P rows, in a seeded random page
    order, with one table entry past each sequence's last page set to -1."""
    B = case.batch
    lens = [int(x) for x in case.ctx_len]
    need = [max(1, -(-L // P)) for L in lens]
    n_pages = sum(need) + 2
    order = rng.permutation(n_pages)
    table = np.full((B, max(need) + 1), -1, dtype=np.int32)
    kp = np.zeros((n_pages,) + case.k_cache.shape[1:2] + (P,) + case.k_cache.shape[3:],
                  dtype=case.k_cache.dtype)
    vp = np.zeros((n_pages,) + case.v_cache.shape[1:2] + (P,) + case.v_cache.shape[3:],
                  dtype=case.v_cache.dtype)
    nxt = 0
    for b, L in enumerate(lens):
        for blk in range(need[b]):
            page = int(order[nxt])
            nxt += 1
            table[b, blk] = page
            r1 = min((blk + 1) * P, L)
            if r1 > blk * P:
                kp[page, :, :r1 - blk * P] = case.k_cache[b, :, blk * P:r1]
                vp[page, :, :r1 - blk * P] = case.v_cache[b, :, blk * P:r1]
    return kp, vp, table


@pytest.mark.parametrize("seed", range(10))
def test_prefill_random_shapes(seed):
    rng = np.random.default_rng(3000 + seed)
    n_q = int(rng.choice([4, 8, 12, 16, 32]))
    n_k = int(rng.choice(_divisors(n_q)))
    n_v = int(rng.choice(_divisors(n_q)))
    d_k = int(rng.choice([64, 128]))
    d_v = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 4))
    T = int(rng.integers(1, 330))
    lens = [int(x) for x in rng.integers(max(1, T // 2), T + 1400, size=B)]
    cap = max(lens) + int(rng.integers(0, 70))
    scale = None if rng.random() < 0.5 else float(rng.uniform(0.03, 0.4))
    spike = rng.random() < 0.4
    _say("random prefill", seed, (n_q, n_k, n_v, d_k, d_v), "T", T, lens, cap, "scale", scale,
         "spike", spike)
    case = synth.make_case(800 + seed, dtype="bf16", batch=B, n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=cap, t_new=T,
                           poison_tail=True, scale=scale)
    if spike:
        # q = 1 everywhere and, late in each sequence, one key row of 6.0 per
        # K head: its logit lies far above every first key tile's max.
        case.q[...] = 0x3F80
        for b, L in enumerate(lens):
            j = int(rng.integers(L // 2, L))
            case.k_cache[b, :, j, :] = 0x40C0
    qw, kw, vw = case.widened()
    ref, ref_lse = oracle.prefill_all_rows(qw, kw, vw, case.ctx_len, case.scale)
    q, k, v, ctx = upload(case)
    outs = {}
    for with_lse in (True, False):
        for split in (True, False):
            lse = (torch.empty((B, T, n_q), dtype=torch.float32, device="cuda")
                   if with_lse else None)
            ws = None if split else torch.empty(0, dtype=torch.uint8, device="cuda")
            out, lse = dq.prefill(q, k, v, ctx, scale=case.scale, lse=lse, workspace=ws)
            torch.cuda.synchronize()
            what = f"seed {seed} lse={with_lse} split={split}"
            got = to_host(out)
            assert np.isfinite(got).all(), what
            assert_close(got, ref, "bf16", what)
            if with_lse:
                assert_lse_close(to_host(lse), ref_lse, "bf16", what)
                outs[split] = (raw_host(out), raw_host(lse))
    # The same prefill over a paged copy of the cache: bit-identical.
    P = int(rng.choice([64, 128, 256]))
    kp, vp, table = _pages_of(case, P, rng)
    lse_p = torch.empty((B, T, n_q), dtype=torch.float32, device="cuda")
    out_p, _ = dq.prefill_paged(q, to_dev(kp, "bf16"), to_dev(vp, "bf16"), ints_to_dev(table),
                                ctx, scale=case.scale, lse=lse_p)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out_p), outs[True][0])
    np.testing.assert_array_equal(raw_host(lse_p), outs[True][1])
