"""GPU parity of kv_append (bit-exact) and of the MFMA causal prefill."""

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


def _bits(shape, seed):
    return np.random.default_rng(seed).integers(0, 65536, shape, dtype=np.uint16)


# ----------------------------------------------------------------- kv_append

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_append_bit_exact(dtype):
    B, T, n_k, n_v, d_k, d_v, cap = 3, 5, 4, 16, 64, 128, 100
    if dtype == "bf16":
        kc, vc = _bits((B, n_k, cap, d_k), 1), _bits((B, n_v, cap, d_v), 2)
        kn, vn = _bits((B, T, n_k, d_k), 3), _bits((B, T, n_v, d_v), 4)
    else:  # arbitrary 32-bit patterns, NaNs included, must survive unchanged
        rng = np.random.default_rng(5)
        kc, vc = (rng.integers(0, 2**32, s, dtype=np.uint32).view(np.float32)
                  for s in ((B, n_k, cap, d_k), (B, n_v, cap, d_v)))
        kn, vn = (rng.integers(0, 2**32, s, dtype=np.uint32).view(np.float32)
                  for s in ((B, T, n_k, d_k), (B, T, n_v, d_v)))
    pos = np.array([0, 40, cap - T])
    _say("kv_append", dtype)
    k, v = to_dev(kc, dtype), to_dev(vc, dtype)
    dq.kv_append(to_dev(kn, dtype), to_dev(vn, dtype), ints_to_dev(pos), k, v, n_q=16)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_append(kc, vc, kn, vn, pos)
    gk, gv = raw_host(k), raw_host(v)
    np.testing.assert_array_equal(gk.view(np.uint8), np.asarray(ek).view(np.uint8))
    np.testing.assert_array_equal(gv.view(np.uint8), np.asarray(ev).view(np.uint8))


def test_kv_append_skips_rows_outside_cache():
    B, T, n_k, n_v, d_k, d_v, cap = 2, 4, 1, 2, 32, 64, 10
    kc, vc = _bits((B, n_k, cap, d_k), 6), _bits((B, n_v, cap, d_v), 7)
    kn, vn = _bits((B, T, n_k, d_k), 8), _bits((B, T, n_v, d_v), 9)
    pos = np.array([8, -3])  # rows 8, 9 fit; 10, 11 and every row of b=1 do not
    _say("kv_append out-of-range rows")
    k, v = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    dq.kv_append(to_dev(kn, "bf16"), to_dev(vn, "bf16"), ints_to_dev(pos), k, v, n_q=2)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_append(kc[:1], vc[:1], kn[:1, :2], vn[:1, :2], pos[:1])
    gk, gv = raw_host(k), raw_host(v)
    np.testing.assert_array_equal(gk[:1], ek)
    np.testing.assert_array_equal(gv[:1], ev)
    np.testing.assert_array_equal(gk[1], kc[1])
    np.testing.assert_array_equal(gv[1], vc[1])


# ------------------------------------------------------------------- prefill

def run_prefill(case, with_lse=True, split=True):
    """Prefill on the GPU.  split=False passes an empty workspace (one key
    split); with_lse=False takes the path that sums the rounded weights."""
    q, k, v, ctx = upload(case)
    lse = None
    if with_lse:
        lse = torch.empty((case.batch, case.t_new, case.n_q), dtype=torch.float32, device="cuda")
    ws = None if split else torch.empty(0, dtype=torch.uint8, device="cuda")
    out, lse = dq.prefill(q, k, v, ctx, scale=case.scale, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return to_host(out), (to_host(lse) if with_lse else None)


PREFILL = [
    # n_q, n_k, n_v, d_k, d_v, t_new, lengths (after append), l_cap
    (16, 4, 16, 64, 128, 200, [700, 200], 704),
    (16, 4, 16, 64, 128, 128, [4000], 4000),
    (32, 4, 16, 64, 64, 70, [333], 340),
    (16, 16, 16, 128, 128, 129, [600], 640),
    (8, 2, 8, 128, 64, 256, [1000, 300], 1024),
]


@pytest.mark.parametrize("cfg", PREFILL, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-{c[3]}x{c[4]}-t{c[5]}")
def test_prefill_small_matches_oracle(cfg):
    n_q, n_k, n_v, d_k, d_v, T, lens, cap = cfg
    case = synth.make_case(202, dtype="bf16", batch=len(lens), n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=cap, t_new=T,
                           poison_tail=True)
    q, k, v = case.widened()
    ref, ref_lse = oracle.prefill(q, k, v, case.ctx_len, case.scale)
    for with_lse, split in ((True, True), (False, True), (True, False), (False, False)):
        _say("prefill small", cfg, "lse" if with_lse else "no lse", "split" if split else "unsplit")
        got, lse = run_prefill(case, with_lse, split)
        err = assert_close(got, ref, "bf16", f"{cfg} lse={with_lse} split={split}")
        if with_lse:
            assert_lse_close(lse, ref_lse, "bf16", str(cfg))
        _say(f"prefill {cfg} normwise rel err {err:.2e}")


def test_prefill_rows_without_visible_keys():
    # ctx_len < t_new: the first t_new - ctx_len rows see nothing.
    case = synth.make_case(203, dtype="bf16", batch=1, n_q=8, n_k=2, n_v=8, d_k=64, d_v=128,
                           ctx_len=[50], l_cap=64, t_new=80, poison_tail=True)
    _say("prefill rows without keys")
    got, _ = run_prefill(case, with_lse=False, split=False)
    assert (got[0, :30] == 0).all()
    got, lse = run_prefill(case)
    assert (got[0, :30] == 0).all() and np.isneginf(lse[0, :30]).all()
    q, k, v = case.widened()
    ref, ref_lse = oracle.prefill(q, k, v, case.ctx_len, case.scale,
                                  rows=[(0, r) for r in range(30, 80)])
    assert_close(got[0, 30:], ref[0, 30:], "bf16", "rows with keys")
    assert_lse_close(lse[0, 30:], ref_lse[0, 30:], "bf16", "rows with keys")


@pytest.mark.parametrize("with_lse", [True, False], ids=["lse", "no-lse"])
def test_prefill_logits_far_above_the_first_tile(with_lse):
    # The kernel keeps each row's max from the first key tile of its split;
    # keys whose scaled logits lie ~100 and ~190 (log2 units) above it make
    # the later weights overflow 2^64 and fp32, which its guard must catch.
    # q = 1 everywhere; two cache rows per K head are set to 9.0 and 17.0.
    case = synth.make_case(204, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[1500], l_cap=1536, t_new=600, poison_tail=True)
    case.q[...] = 0x3F80                      # bf16 1.0
    case.k_cache[:, :, 1000, :] = 0x4110      # bf16 9.0: 2^104 above a typical row max
    case.k_cache[:, :, 1300, :] = 0x4188      # bf16 17.0: 2^196, past fp32's range
    q, k, v = case.widened()
    rows = [(0, r) for r in range(0, 600, 7)] + [(0, 599)]
    ref, ref_lse = oracle.prefill(q, k, v, case.ctx_len, case.scale, rows=rows)
    _say("prefill logits far above the first tile", "lse" if with_lse else "no lse")
    for split in (True, False):
        got, lse = run_prefill(case, with_lse, split)
        idx = [r for _, r in rows]
        assert np.isfinite(got).all()
        assert_close(got[0, idx], ref[0, idx], "bf16", f"spiked logits split={split}")
        if with_lse:
            assert_lse_close(lse[0, idx], ref_lse[0, idx], "bf16", f"spiked logits split={split}")


def test_prefill_full_workload_every_row():
    # The benchmark's prefill (2048 new rows on 30720 cached, 16 query heads,
    # key splits as the benchmark runs it), every one of the 2048 x 16 rows
    # against the oracle, on the lse path and on the path without lse.
    case = synth.make_case(**synth.workload("prefill2k_on_30k"))
    _say("prefill full workload 2048 on 30720: GPU (split, lse and no lse)")
    got_nolse, _ = run_prefill(case, with_lse=False)
    got, lse = run_prefill(case)
    _say("  oracle, all 2048 rows x 16 heads")
    q, k, v = case.widened()
    ref, ref_lse = oracle.prefill_all_rows(q, k, v, case.ctx_len, case.scale)
    err = assert_close(got_nolse, ref, "bf16", "prefill full, no lse")
    _say(f"  no lse: normwise rel err {err:.2e} over every row")
    err = assert_close(got, ref, "bf16", "prefill full")
    assert_lse_close(lse, ref_lse, "bf16", "prefill full")
    _say(f"  lse: normwise rel err {err:.2e} over every row")


def test_prefill_last_row_matches_decode():
    case = synth.make_case(204, dtype="bf16", batch=2, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[3000, 2500], l_cap=3008, t_new=64)
    _say("prefill last row vs decode")
    got, _ = run_prefill(case)
    q, k, v, ctx = upload(case)
    out, _ = dq.decode(q[:, -1].contiguous(), k, v, ctx, scale=case.scale)
    torch.cuda.synchronize()
    dec = to_host(out)
    assert_close(got[:, -1], dec, "bf16", "last row")


TINY = [
    # t_new, lengths (after append), l_cap: one new row of a 100-row sequence
    # (two key tiles over four key splits, so two splits see no key), one
    # row on a one-row cache, and a batch whose second sequence is shorter
    # than a tile.
    (1, [100], 128),
    (1, [1], 64),
    (3, [3000, 65], 3008),
]


@pytest.mark.parametrize("cfg", TINY, ids=lambda c: f"t{c[0]}-L{'-'.join(map(str, c[1]))}")
def test_prefill_tiny_and_empty_key_splits(cfg):
    T, lens, cap = cfg
    case = synth.make_case(205, dtype="bf16", batch=len(lens), n_q=16, n_k=4, n_v=16, d_k=64,
                           d_v=128, ctx_len=lens, l_cap=cap, t_new=T, poison_tail=True)
    q, k, v = case.widened()
    ref, ref_lse = oracle.prefill(q, k, v, case.ctx_len, case.scale)
    for with_lse, split in ((True, True), (False, True), (True, False)):
        _say("prefill tiny", cfg, "lse" if with_lse else "no lse", "split" if split else "unsplit")
        got, lse = run_prefill(case, with_lse, split)
        assert_close(got, ref, "bf16", f"{cfg} lse={with_lse} split={split}")
        if with_lse:
            assert_lse_close(lse, ref_lse, "bf16", str(cfg))
