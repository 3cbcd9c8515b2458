"""GPU parity of selective-V decode against the fp64 oracle.

Which rows are selected is decided on the kernel's fp32 logits, so the
chosen set is checked for what is unique: it must be a valid top-k of the
fp64 logits up to fp32 logit rounding (every chosen row at least as large as
every row left out, within LOGIT_TOL), and must equal the oracle's set
wherever the fp64 gap at the k-th place is wider than that.  The output is
then compared, at the usual tolerance, with the oracle's selective sum over
the set the kernel chose.  Ties are exact in both precisions when rows are
identical, and there the lower rows must win bit for bit.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, assert_lse_close, ints_to_dev, raw_host, to_dev, to_host, upload

pytestmark = pytest.mark.gpu
dq = pytest.importorskip("asymmetric_head_kv_amd")

# Largest error of a logit scale * q.k in fp32 (natural-log units) for the
# sizes used here: |q.k| stays below ~60 and fp32 dot products of <= 128
# terms are far inside 1e-4 of that.
LOGIT_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dq.load()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_selective(case, top_k, k_new=None, v_new=None, tensors=None):
    q, k, v, ctx = tensors if tensors is not None else upload(case)
    B, n_q = case.batch, case.n_q
    lse = torch.empty((B, n_q), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, n_q, top_k), dtype=torch.int32, device="cuda")
    out, lse, sel = dq.decode_selective(q, k, v, ctx, top_k=top_k, scale=case.scale, lse=lse,
                                        sel_idx=sel, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    return out, lse, sel


def check_selective(case, top_k, out, lse, sel, what=""):
    """Validity and uniqueness of the chosen rows; output and lse parity."""
    q, K, V = case.widened()
    got = to_host(out)
    got_lse = to_host(lse)
    got_sel = sel.cpu().numpy()
    ref = np.zeros_like(got)
    ref_lse = np.full(got_lse.shape, -math.inf)
    exact = 0
    for b in range(case.batch):
        L = int(case.ctx_len[b])
        kk = min(top_k, L)
        for i in range(case.n_q):
            hk = oracle.group_sharing_index(i, case.n_q, case.n_k)
            hv = oracle.group_sharing_index(i, case.n_q, case.n_v)
            s = got_sel[b, i]
            assert (s[kk:] == -1).all(), f"{what}: b={b} i={i} padding"
            s = s[:kk]
            assert (np.diff(s) > 0).all() and (s.size == 0 or (s[0] >= 0 and s[-1] < L)), \
                f"{what}: b={b} i={i} indices not ascending in range"
            if L == 0:
                continue
            logits = case.scale * (np.asarray(K[b, hk, :L], np.float64) @ np.asarray(q[b, i], np.float64))
            mask = np.zeros(L, bool)
            mask[s] = True
            if kk < L:
                lo_in, hi_out = logits[mask].min(), logits[~mask].max()
                assert lo_in >= hi_out - LOGIT_TOL, \
                    f"{what}: b={b} i={i} chose {lo_in} but left out {hi_out}"
                top = oracle.top_k_rows(logits, kk)
                srt = np.sort(logits)[::-1]
                if srt[kk - 1] - srt[kk] > 2 * LOGIT_TOL:
                    np.testing.assert_array_equal(s, top, err_msg=f"{what}: b={b} i={i} set")
                    exact += 1
            ref[b, i], _ = oracle.attend_selective_one(q[b, i], K[b, hk, :L], V[b, hv, :L],
                                                       case.scale, top_k, rows=s)
            _, ref_lse[b, i] = oracle.attention_weights(q[b, i], K[b, hk, :L], case.scale)
    err = assert_close(got, ref, case.dtype, what)
    assert_lse_close(got_lse, ref_lse, case.dtype, what)
    return err, exact


SMALL = [
    # dtype, n_q, n_k, n_v, d_k, d_v, lengths, l_cap
    ("bf16", 16, 4, 16, 64, 128, [5000, 777], 5000),
    ("bf16", 32, 4, 16, 64, 64, [9000], 9000),
    ("bf16", 16, 16, 16, 128, 128, [4200, 4096, 4097], 4224),
    ("bf16", 8, 2, 8, 256, 32, [1500], 1536),
    ("f32", 8, 2, 4, 64, 64, [4500, 64], 4608),
    ("f32", 4, 1, 4, 32, 256, [300], 320),
    # 24 query heads on one K head: two groups of query heads (16 + 8) per
    # K tile in the bf16 logit kernel.
    ("bf16", 24, 1, 8, 32, 64, [3000, 2999], 3008),
    # 5 ranges: with top_k = 1024 the 5120 candidates exceed what the final
    # selection holds in registers and it takes its global-memory passes.
    ("bf16", 8, 2, 8, 64, 128, [20000], 20032),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}x{c[5]}")
@pytest.mark.parametrize("top_k", [1, 100, 1024])
def test_selective_small_matches_oracle(cfg, top_k):
    dtype, n_q, n_k, n_v, d_k, d_v, lens, cap = cfg
    case = synth.make_case(301, dtype=dtype, batch=len(lens), n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=cap, poison_tail=True)
    _say("selective small", cfg, "top_k", top_k)
    out, lse, sel = run_selective(case, top_k)
    err, exact = check_selective(case, top_k, out, lse, sel, f"{cfg} k={top_k}")
    _say(f"  normwise rel err {err:.2e}; {exact} sets checked exactly")


def test_selective_with_k_at_least_length_equals_full_decode():
    case = synth.make_case(302, dtype="bf16", batch=3, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[90, 100, 1], l_cap=128, poison_tail=True)
    _say("selective k >= L")
    out, lse, sel = run_selective(case, 100)
    q, k, v = case.widened()
    ref, ref_lse = oracle.decode(q, k, v, case.ctx_len, case.scale)
    assert_close(to_host(out), ref, "bf16", "k >= L vs full decode")
    assert_lse_close(to_host(lse), ref_lse, "bf16", "k >= L")
    s = sel.cpu().numpy()
    for b, L in enumerate(case.ctx_len):
        assert (s[b, :, :L] == np.arange(L)).all() and (s[b, :, L:] == -1).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_selective_ties_go_to_lower_rows(dtype):
    # Every K row equals k0 except a few rows equal to 2 k0, and q = k0: the
    # logits are exactly |k0|^2 scale (ties) or twice that.  The selection
    # must be the doubled rows plus the lowest-indexed tied rows, across
    # several 4096-row ranges.
    n_q, n_k, n_v, d_k, d_v, L, top_k = 4, 1, 2, 64, 64, 9000, 100
    base = synth.make_case(303, dtype=dtype, batch=1, n_q=n_q, n_k=n_k, n_v=n_v, d_k=d_k,
                           d_v=d_v, ctx_len=[L])
    k0 = base.k_cache[0, 0, 0].copy()
    k = np.broadcast_to(k0, (1, n_k, L, d_k)).copy()
    big = np.array([17, 4095, 4096, 5000, 8999])
    if dtype == "bf16":
        k[0, 0, big] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(k0) * 2)
    else:
        k[0, 0, big] = k0 * 2
    q = np.broadcast_to(k0, (1, n_q, d_k)).copy()
    case = synth.DecodeCase(dtype, n_q, n_k, n_v, d_k, d_v, q, k, base.v_cache,
                            base.ctx_len, base.scale)
    _say("selective ties", dtype)
    out, lse, sel = run_selective(case, top_k)
    want = np.sort(np.concatenate([big, np.setdiff1d(np.arange(L), big)[:top_k - len(big)]]))
    s = sel.cpu().numpy()
    for i in range(n_q):
        np.testing.assert_array_equal(s[0, i], want)
    qw, kw, vw = case.widened()
    for i in range(n_q):
        ref, rows = oracle.attend_selective_one(qw[0, i], kw[0, 0], vw[0, i * n_v // n_q],
                                                case.scale, top_k)
        np.testing.assert_array_equal(rows, want)
        assert_close(to_host(out)[0, i], ref, dtype, f"ties head {i}")


def test_selective_logits_far_above_the_rest():
    # q = 1; a few K rows far larger than the rest: they must be chosen, and
    # their weights (full softmax, fp32 logits ~100 and ~190 log2 units above
    # the others) dominate the output.
    case = synth.make_case(612, dtype="bf16", batch=2, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[5000, 2100], l_cap=5000, poison_tail=True)
    case.q[...] = 0x3F80
    case.k_cache[0, :, 4100, :] = 0x4110
    case.k_cache[0, :, 17, :] = 0x4188
    case.k_cache[1, :, 2099, :] = 0x4188
    _say("selective logits far above the rest")
    out, lse, sel = run_selective(case, 100)
    s = sel.cpu().numpy()
    assert (s[0] == 17).any(axis=1).all() and (s[0] == 4100).any(axis=1).all()
    assert (s[1] == 2099).any(axis=1).all()
    check_selective(case, 100, out, lse, sel, "spiked selective")


def test_selective_empty_context():
    case = synth.make_case(304, dtype="bf16", batch=2, n_q=8, n_k=2, n_v=8, d_k=64, d_v=128,
                           ctx_len=[0, 300], l_cap=320, poison_tail=True)
    _say("selective empty context")
    out, lse, sel = run_selective(case, 100)
    assert (to_host(out)[0] == 0).all() and np.isneginf(to_host(lse)[0]).all()
    assert (sel.cpu().numpy()[0] == -1).all()
    check_selective(case, 100, out, lse, sel, "empty + 300")


def test_selective_fused_append_matches_separate_append():
    case = synth.make_case(305, dtype="bf16", batch=3, n_q=32, n_k=4, n_v=16, d_k=64, d_v=64,
                           ctx_len=[5001, 4096, 1], l_cap=5120)
    kn, vn = synth.new_rows(305, dtype="bf16", batch=3, t_new=1, n_k=4, n_v=16, d_k=64, d_v=64)
    _say("selective fused append")
    q, k, v, ctx = upload(case)
    k2, v2 = k.clone(), v.clone()
    kn_d, vn_d = to_dev(kn, "bf16"), to_dev(vn, "bf16")
    out_f, lse_f, sel_f = run_selective(case, 100, k_new=kn_d, v_new=vn_d,
                                        tensors=(q, k, v, ctx))
    dq.kv_append(kn_d, vn_d, ints_to_dev(case.ctx_len - 1), k2, v2, n_q=32)
    out_s, lse_s, sel_s = run_selective(case, 100, tensors=(q, k2, v2, ctx))
    np.testing.assert_array_equal(raw_host(k), raw_host(k2))
    np.testing.assert_array_equal(raw_host(v), raw_host(v2))
    np.testing.assert_array_equal(sel_f.cpu().numpy(), sel_s.cpu().numpy())
    np.testing.assert_array_equal(raw_host(out_f), raw_host(out_s))
    np.testing.assert_array_equal(lse_f.cpu().numpy(), lse_s.cpu().numpy())
    appended = synth.DecodeCase("bf16", 32, 4, 16, 64, 64, case.q, raw_host(k2), raw_host(v2),
                                case.ctx_len, case.scale)
    check_selective(appended, 100, out_f, lse_f, sel_f, "fused append")


@pytest.mark.parametrize("name", ["decode32k_asym", "decode64k_dk64"])
def test_selective_full_workload(name):
    case = synth.make_case(**synth.workload(name))
    _say("selective full workload", name, "top_k 100")
    out, lse, sel = run_selective(case, 100)
    err, exact = check_selective(case, 100, out, lse, sel, name)
    _say(f"  {name}: normwise rel err {err:.2e}; {exact} of {case.batch * case.n_q} sets exact")
