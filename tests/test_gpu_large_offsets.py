"""GPU parity with caches whose element offsets pass 2^31.

On a 288 GB device a head-major cache or a page pool easily holds more than
2^31 elements, where any 32-bit product of (sequence, head, row, column)
would wrap.  Each case fills only the last sequence of a batch (all others
empty) so that its cache plane starts at or beyond element 2^31:

* asymmetric 16/4/16 heads, d_k 64 / d_v 128, 33 sequences of 65536 rows:
  the last sequence's V plane starts at element 2^32;
* symmetric 16/16/16, d 128, 17 sequences: its K and V planes both start at
  element 2^31.

On that sequence the decode step with a fused append, selective V, an
8-row prefill and a plain kv_append are checked against the fp64 oracle (and
the append bit for bit); the empty sequences give zero output and -inf lse.
The same caches, copied into a page pool whose used pages start at element
2^31 (64-row pages in a seeded random order), give bit-identical decode,
selective and prefill results through the paged entry points.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_close, assert_lse_close, ints_to_dev, raw_host, to_dev,
                      to_host)
from test_gpu_selective import check_selective

pytestmark = pytest.mark.gpu
dq = pytest.importorskip("asymmetric_head_kv_amd")

CAP = 65536          # rows per sequence
L = CAP - 29         # rows attended after the fused append (ragged last tile)
T_PF = 8             # prefill rows (the last T_PF rows of the context)
P = 64               # page rows
PAGE0 = 16384        # first used page: 16384 * 16 heads * 64 rows * 128 = 2^31
CASES = {
    # name: (n_q, n_k, n_v, d_k, d_v, batch)
    "asym_v_at_2^32": (16, 4, 16, 64, 128, 33),
    "sym_kv_at_2^31": (16, 16, 16, 128, 128, 17),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dq.load()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16(shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda")


@pytest.mark.parametrize("name", list(CASES))
def test_caches_past_2_31_elements(name):
    n_q, n_k, n_v, d_k, d_v, B = CASES[name]
    last = B - 1
    assert last * n_v * CAP * d_v >= 2 ** 31
    seed = 4100 + len(name)
    case = synth.make_case(seed, dtype="bf16", batch=1, n_q=n_q, n_k=n_k, n_v=n_v, d_k=d_k,
                           d_v=d_v, ctx_len=[L], l_cap=CAP, poison_tail=True)
    kn, vn = synth.new_rows(seed + 1, dtype="bf16", batch=1, t_new=1, n_k=n_k, n_v=n_v,
                            d_k=d_k, d_v=d_v)
    # The oracle's caches: row L-1 replaced by the appended token.
    kh, vh = oracle.kv_append(case.k_cache, case.v_cache, kn, vn, np.array([L - 1]))
    lens = np.array([L], np.int32)
    appended = synth.DecodeCase("bf16", n_q, n_k, n_v, d_k, d_v, case.q, kh, vh, lens,
                                case.scale)

    _say(name, "allocating", B, "sequences of", CAP, "rows")
    k = torch.empty((B, n_k, CAP, d_k), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((B, n_v, CAP, d_v), dtype=torch.bfloat16, device="cuda")
    k[last].copy_(to_dev(case.k_cache[0], "bf16"))
    v[last].copy_(to_dev(case.v_cache[0], "bf16"))
    q = _bf16((B, n_q, d_k))
    q[last].copy_(to_dev(case.q[0], "bf16"))
    k_new, v_new = _bf16((B, n_k, d_k)), _bf16((B, n_v, d_v))
    k_new[last].copy_(to_dev(kn[0, 0], "bf16"))
    v_new[last].copy_(to_dev(vn[0, 0], "bf16"))
    ctx = ints_to_dev([0] * last + [L])

    # Decode with the fused append.
    _say(name, "decode + fused append")
    lse = torch.empty((B, n_q), dtype=torch.float32, device="cuda")
    out, lse = dq.decode(q, k, v, ctx, scale=case.scale, lse=lse, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(k[last]), kh[0])
    np.testing.assert_array_equal(raw_host(v[last]), vh[0])
    q_w, k_w, v_w = appended.widened()
    ref, ref_lse = oracle.decode(q_w, k_w, v_w, lens, case.scale)
    got, got_lse = to_host(out), to_host(lse)
    assert (got[:last] == 0).all() and np.isneginf(got_lse[:last]).all()
    assert_close(got[last:], ref, "bf16", f"{name} decode")
    assert_lse_close(got_lse[last:], ref_lse, "bf16", f"{name} decode")

    # Selective V over the appended caches.
    _say(name, "selective V, top_k 100")
    lse_s = torch.empty((B, n_q), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, n_q, 100), dtype=torch.int32, device="cuda")
    out_s, lse_s, sel = dq.decode_selective(q, k, v, ctx, top_k=100, scale=case.scale,
                                            lse=lse_s, sel_idx=sel)
    torch.cuda.synchronize()
    assert (sel[:last].cpu().numpy() == -1).all()
    assert (to_host(out_s[:last]) == 0).all()
    check_selective(appended, 100, out_s[last:], lse_s[last:], sel[last:], f"{name} selective")

    # Prefill of the context's last T_PF rows.
    _say(name, "prefill", T_PF, "rows")
    q_pf_h = synth.normal(seed + 2, synth.S_Q, (1, T_PF, n_q, d_k), "bf16")
    q_pf = _bf16((B, T_PF, n_q, d_k))
    q_pf[last].copy_(to_dev(q_pf_h[0], "bf16"))
    lse_pf = torch.empty((B, T_PF, n_q), dtype=torch.float32, device="cuda")
    out_pf, lse_pf = dq.prefill(q_pf, k, v, ctx, scale=case.scale, lse=lse_pf)
    torch.cuda.synchronize()
    ref_pf, ref_pf_lse = oracle.prefill(synth.bf16_bits_to_f32(q_pf_h), k_w, v_w, lens,
                                        case.scale)
    got_pf, got_pf_lse = to_host(out_pf), to_host(lse_pf)
    assert (got_pf[:last] == 0).all() and np.isneginf(got_pf_lse[:last]).all()
    assert_close(got_pf[last:], ref_pf, "bf16", f"{name} prefill")
    assert_lse_close(got_pf_lse[last:], ref_pf_lse, "bf16", f"{name} prefill")

    # Page pool: the last sequence's rows in pages PAGE0 .. PAGE0 + n_pg - 1
    # (seeded random order); the empty sequences' table rows are -1.
    n_pg = CAP // P
    _say(name, "paged: pool of", PAGE0 + n_pg, "pages")
    perm = PAGE0 + torch.from_numpy(np.random.default_rng(seed).permutation(n_pg)).to("cuda")
    kp = torch.empty((PAGE0 + n_pg, n_k, P, d_k), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty((PAGE0 + n_pg, n_v, P, d_v), dtype=torch.bfloat16, device="cuda")
    kp[perm] = k[last].view(n_k, n_pg, P, d_k).permute(1, 0, 2, 3)
    vp[perm] = v[last].view(n_v, n_pg, P, d_v).permute(1, 0, 2, 3)
    table = torch.full((B, n_pg), -1, dtype=torch.int32, device="cuda")
    table[last] = perm.to(torch.int32)
    S0 = dq.decode_chunk(n_q, n_k, n_v, d_k, d_v, B, CAP)
    out_c, _ = dq.decode(q, k, v, ctx, scale=case.scale, chunk_tokens=S0)
    out_p, _ = dq.decode_paged(q, kp, vp, table, ctx, max_ctx=CAP, scale=case.scale,
                               chunk_tokens=S0)
    # The same outputs requested as above, lse included: with lse the
    # prefill's row sums add the fp32 weights, without it the bf16-rounded
    # ones of the P.V product, so the two forms may differ by an ulp.
    sel_p, lse_sp = torch.empty_like(sel), torch.empty_like(lse_s)
    out_sp, lse_sp, sel_p = dq.decode_selective_paged(q, kp, vp, table, ctx, top_k=100,
                                                      max_ctx=CAP, scale=case.scale,
                                                      lse=lse_sp, sel_idx=sel_p)
    out_pfp, lse_pfp = dq.prefill_paged(q_pf, kp, vp, table, ctx, scale=case.scale,
                                        lse=torch.empty_like(lse_pf))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out_p), raw_host(out_c))
    np.testing.assert_array_equal(raw_host(out_sp), raw_host(out_s))
    np.testing.assert_array_equal(raw_host(lse_sp), raw_host(lse_s))
    np.testing.assert_array_equal(sel_p.cpu().numpy(), sel.cpu().numpy())
    np.testing.assert_array_equal(raw_host(out_pfp), raw_host(out_pf))
    np.testing.assert_array_equal(raw_host(lse_pfp), raw_host(lse_pf))
    del kp, vp

    # Plain kv_append of one more row at row L (the others' positions are -1:
    # skipped).
    _say(name, "kv_append at row", L)
    kn2, vn2 = synth.new_rows(seed + 3, dtype="bf16", batch=1, t_new=1, n_k=n_k, n_v=n_v,
                              d_k=d_k, d_v=d_v)
    k_add, v_add = _bf16((B, 1, n_k, d_k)), _bf16((B, 1, n_v, d_v))
    k_add[last].copy_(to_dev(kn2[0], "bf16"))
    v_add[last].copy_(to_dev(vn2[0], "bf16"))
    dq.kv_append(k_add, v_add, ints_to_dev([-1] * last + [L]), k, v, n_q=n_q)
    torch.cuda.synchronize()
    kh2, vh2 = oracle.kv_append(kh, vh, kn2, vn2, np.array([L]))
    np.testing.assert_array_equal(raw_host(k[last]), kh2[0])
    np.testing.assert_array_equal(raw_host(v[last]), vh2[0])
    del k, v
    torch.cuda.empty_cache()
