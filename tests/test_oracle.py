"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-derives the oracle's own formula: each compares it with a
printed worked example, an independent library routine, a closed form, a
brute-force evaluation or an invariant.  ``test_pins_catch_planted_mistakes``
plants plausible mistakes in a copy of the oracle and checks that some pin
fails for each.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(seed, B, n_q, n_k, n_v, d_k, d_v, L):
    q = _rand(seed, B, n_q, d_k)
    k = _rand(seed + 1, B, n_k, L, d_k)
    v = _rand(seed + 2, B, n_v, L, d_v)
    return q, k, v, np.full(B, L, dtype=np.int64)


# ---------------------------------------------------------------- head maps

def test_flexheadfa_index_worked_example(golden):
    rows = golden("flexheadfa_index_example.txt")
    assert len(rows) == 3
    for n_q, n_k, n_v, iq, ik, iv in (map(int, r) for r in rows):
        assert oracle.group_sharing_index(iq, n_q, n_k) == ik
        assert oracle.group_sharing_index(iq, n_q, n_v) == iv


def test_group_sharing_sigma15b_ratios():
    # Sigma architecture page, §3.4 Step 3: with 32 Q heads, each of the 4 K
    # heads serves 8 consecutive Q heads (K head floor(i/8)) and each of the
    # 16 V heads serves 2 (V head floor(i/2)).
    for i in range(32):
        assert oracle.group_sharing_index(i, 32, 4) == i // 8
        assert oracle.group_sharing_index(i, 32, 16) == i // 2
    # MHA special case: identity map.
    assert [oracle.group_sharing_index(i, 16, 16) for i in range(16)] == list(range(16))
    # MQA special case: everything reads head 0.
    assert {oracle.group_sharing_index(i, 16, 1) for i in range(16)} == {0}


# ------------------------------------------------ reductions to MHA/GQA/MQA

def _sdpa_reference(q, k, v, L, scale=None):
    """Textbook attention via torch's scaled_dot_product_attention in fp64
    (one query token per head; K/V heads repeated to the query head count)."""
    n_q, n_k = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).unsqueeze(2)                  # [B][n_q][1][d]
    kt = torch.from_numpy(np.ascontiguousarray(k[:, :, :L]))
    vt = torch.from_numpy(np.ascontiguousarray(v[:, :, :L]))
    kt = kt.repeat_interleave(n_q // n_k, dim=1)
    vt = vt.repeat_interleave(n_q // v.shape[1], dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o.squeeze(2).numpy()


@pytest.mark.parametrize("n_q,n_kv,d,L", [
    (4, 4, 16, 37),    # MHA: n_q = n_k = n_v, d_q = d_k = d_v
    (8, 1, 32, 50),    # MQA: n_k = n_v = 1
    (8, 2, 8, 64),     # GQA: 1 < n_k = n_v < n_q
    (16, 4, 64, 129),  # GQA at the decode head counts
])
def test_reduces_to_textbook_attention(n_q, n_kv, d, L):
    # Sigma architecture page, §3.4 "Generalized Formulation": MHA, MQA and
    # GQA are the special cases n_k = n_v with d_q = d_k = d_v.  torch's
    # default scale is 1/sqrt(d), the page's 1/sqrt(d_k).
    q, k, v, lens = _case(7, 2, n_q, n_kv, n_kv, d, d, L)
    out, _ = oracle.decode(q, k, v, lens)
    ref = _sdpa_reference(q, k, v, L)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_asymmetric_matches_per_head_sdpa():
    # With n_k != n_v and d_k != d_v each query head is still ordinary
    # single-head attention on its own K head and V head.
    n_q, n_k, n_v, d_k, d_v, L = 16, 4, 8, 32, 48, 75
    q, k, v, lens = _case(11, 1, n_q, n_k, n_v, d_k, d_v, L)
    out, _ = oracle.decode(q, k, v, lens)
    for i in range(n_q):
        qt = torch.from_numpy(q[0, i]).view(1, 1, d_k)
        kt = torch.from_numpy(np.ascontiguousarray(k[0, i // (n_q // n_k), :L]))[None]
        vt = torch.from_numpy(np.ascontiguousarray(v[0, i // (n_q // n_v), :L]))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).view(-1)
        np.testing.assert_allclose(out[0, i], ref.numpy(), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- softmax

@pytest.mark.parametrize("scale", [None, 0.3, 5.0])
def test_weights_sum_to_one(scale):
    q = _rand(3, 24) * 4.0
    K = _rand(4, 500, 24)
    alpha, _ = oracle.attention_weights(q, K, 1 / math.sqrt(24) if scale is None else scale)
    assert abs(alpha.sum() - 1.0) < 1e-12
    assert (alpha >= 0).all()


def test_brute_force_explicit_softmax():
    # Pure-Python loops, softmax without any max shift: exp(s)/sum(exp(s)).
    n_q, n_k, n_v, d_k, d_v, L = 4, 2, 4, 3, 5, 7
    q, k, v, lens = _case(21, 2, n_q, n_k, n_v, d_k, d_v, L)
    out, lse = oracle.decode(q, k, v, lens)
    scale = 1.0 / math.sqrt(d_k)
    for b in range(2):
        for i in range(n_q):
            kh, vh = i * n_k // n_q, i * n_v // n_q
            s = [scale * sum(q[b, i, d] * k[b, kh, j, d] for d in range(d_k)) for j in range(L)]
            e = [math.exp(x) for x in s]
            z = sum(e)
            for d in range(d_v):
                o = sum(e[j] / z * v[b, vh, j, d] for j in range(L))
                assert abs(out[b, i, d] - o) < 1e-12
            assert abs(lse[b, i] - math.log(z)) < 1e-12


def test_default_scale_is_inverse_sqrt_dk():
    q, k, v, lens = _case(5, 1, 4, 2, 4, 16, 64, 40)
    a, _ = oracle.decode(q, k, v, lens)
    b, _ = oracle.decode(q, k, v, lens, scale=1 / math.sqrt(16))
    c, _ = oracle.decode(q, k, v, lens, scale=1 / math.sqrt(64))
    np.testing.assert_array_equal(a, b)
    assert np.abs(a - c).max() > 1e-3


# ---------------------------------------------------------------- closed forms

def test_single_key_returns_its_value_row():
    q, k, v, _ = _case(9, 1, 8, 2, 8, 16, 32, 5)
    out, lse = oracle.decode(q, k, v, np.array([1]))
    for i in range(8):
        np.testing.assert_array_equal(out[0, i], v[0, i, 0])
        s0 = (q[0, i] @ k[0, i // 4, 0]) / 4.0
        assert abs(lse[0, i] - s0) < 1e-14


def test_zero_scale_is_mean_of_value_rows():
    L = 33
    q, k, v, lens = _case(10, 1, 4, 1, 4, 8, 16, L)
    out, lse = oracle.decode(q, k, v, lens, scale=0.0)
    np.testing.assert_allclose(out[0], v[0, :, :L].mean(axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(L), rtol=1e-15)


def test_two_keys_with_chosen_logits():
    # Scores 0 and ln 3 give weights 1/4 and 3/4.
    q = np.zeros((1, 1, 2)); q[0, 0] = [1.0, 0.0]
    k = np.zeros((1, 1, 2, 2)); k[0, 0, 1, 0] = math.log(3.0)
    v = np.array([[[[2.0, -4.0], [6.0, 8.0]]]])
    out, lse = oracle.decode(q, k, v, np.array([2]), scale=1.0)
    np.testing.assert_allclose(out[0, 0], [0.25 * 2 + 0.75 * 6, 0.25 * -4 + 0.75 * 8], rtol=1e-15)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-15


def test_joint_key_permutation_invariance():
    q, k, v, lens = _case(12, 1, 8, 2, 4, 16, 24, 90)
    perm = np.random.default_rng(0).permutation(90)
    a, la = oracle.decode(q, k, v, lens)
    b, lb = oracle.decode(q, k[:, :, perm], v[:, :, perm], lens)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_kv_group_sharing_equivalence():
    # Sigma architecture page, FlexHeadFA section (kv_group_sharing): copying
    # each K head n_v/n_k times turns the layout into GQA with n_k = n_v and
    # leaves the attention unchanged.
    n_q, n_k, n_v = 16, 4, 16
    q, k, v, lens = _case(13, 2, n_q, n_k, n_v, 32, 64, 70)
    a, la = oracle.decode(q, k, v, lens)
    k_dup = np.repeat(k, n_v // n_k, axis=1)
    b, lb = oracle.decode(q, k_dup, v, lens)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
    # The oracle's expansion is that duplication, and (SIGMA's 4 -> 16) it
    # repeats each K head four times; V is untouched.
    k_exp, v_exp = oracle.kv_group_sharing(k, v)
    np.testing.assert_array_equal(k_exp, k_dup)
    np.testing.assert_array_equal(v_exp, v)
    assert k_exp.shape[1] == 16 and all(
        (k_exp[:, 4 * g + r] == k[:, g]).all() for g in range(4) for r in range(4))


@pytest.mark.parametrize("heads", [(12, 2, 6), (8, 8, 2), (6, 3, 6), (8, 4, 1)])
def test_kv_group_sharing_leaves_attention_unchanged(heads):
    # Either side may be the smaller one: expanding it must not change the
    # output of any query head (the wrapper's purpose, FlexHeadFA section).
    n_q, n_k, n_v = heads
    q, k, v, lens = _case(21, 2, n_q, n_k, n_v, 16, 8, 33)
    k_exp, v_exp = oracle.kv_group_sharing(k, v)
    assert k_exp.shape[1] == v_exp.shape[1] == max(n_k, n_v)
    a, la = oracle.decode(q, k, v, lens)
    b, lb = oracle.decode(q, k_exp, v_exp, lens)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def _to_pages(k, v, lens, P, seed):
    """Scatter contiguous caches into shuffled pages (test helper)."""
    B = k.shape[0]
    need = [-(-int(L) // P) for L in lens]
    n_pages = sum(need) + 3
    order = np.random.default_rng(seed).permutation(n_pages)
    table = np.full((B, max(need + [1])), -1, dtype=np.int64)
    kp = np.zeros((n_pages, k.shape[1], P, k.shape[3]))
    vp = np.zeros((n_pages, v.shape[1], P, v.shape[3]))
    nxt = 0
    for b in range(B):
        for blk in range(need[b]):
            page = order[nxt]
            nxt += 1
            table[b, blk] = page
            rows = slice(blk * P, min((blk + 1) * P, int(lens[b])))
            n = rows.stop - rows.start
            kp[page, :, :n] = k[b, :, rows]
            vp[page, :, :n] = v[b, :, rows]
    return kp, vp, table


def test_paged_layout_round_trip_and_decode():
    q, k, v, _ = _case(22, 3, 8, 2, 4, 16, 8, 150)
    lens = np.array([150, 64, 1])
    for P in (16, 64):
        kp, vp, table = _to_pages(k, v, lens, P, seed=P)
        kc, vc = oracle.paged_to_contiguous(kp, vp, table, lens, l_cap=150)
        for b, L in enumerate(lens):
            np.testing.assert_array_equal(kc[b, :, :L], k[b, :, :L])
            np.testing.assert_array_equal(vc[b, :, :L], v[b, :, :L])
            assert (kc[b, :, L:] == 0).all()
        a, la = oracle.decode_paged(q, kp, vp, table, lens)
        ref, lref = oracle.decode(q, k, v, lens)
        np.testing.assert_array_equal(a, ref)
        np.testing.assert_array_equal(la, lref)


def test_ragged_batch_and_empty_context():
    q, k, v, _ = _case(14, 3, 4, 2, 4, 8, 8, 40)
    lens = np.array([40, 17, 0])
    out, lse = oracle.decode(q, k, v, lens)
    for b, L in enumerate(lens[:2]):
        o1, l1 = oracle.decode(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], np.array([L]))
        np.testing.assert_array_equal(out[b], o1[0])
        np.testing.assert_array_equal(lse[b], l1[0])
    assert (out[2] == 0).all() and np.isneginf(lse[2]).all()


# -------------------------------------------------------------------- prefill

def test_prefill_row_equals_decode_at_its_position():
    B, T, L = 2, 5, 30
    n_q, n_k, n_v, d_k, d_v = 8, 2, 4, 16, 24
    qp = _rand(15, B, T, n_q, d_k)
    _, k, v, _ = _case(16, B, n_q, n_k, n_v, d_k, d_v, L)
    lens = np.array([L, L - 3])
    out, lse = oracle.prefill(qp, k, v, lens)
    for b in range(B):
        for r in range(T):
            ctx = lens[b] - T + r + 1
            o, l = oracle.decode(qp[:, r], k, v, np.full(B, ctx))
            np.testing.assert_array_equal(out[b, r], o[b])
            np.testing.assert_array_equal(lse[b, r], l[b])


def test_prefill_causal_mask():
    B, T, L = 1, 6, 20
    qp = _rand(17, B, T, 4, 8)
    _, k, v, _ = _case(18, B, 4, 1, 4, 8, 8, L)
    lens = np.array([L])
    base, _ = oracle.prefill(qp, k, v, lens)
    r = 2
    p = L - T + r
    k2, v2 = k.copy(), v.copy()
    k2[:, :, p + 1:] += 10.0
    v2[:, :, p + 1:] -= 7.0
    after, _ = oracle.prefill(qp, k2, v2, lens)
    np.testing.assert_array_equal(after[0, :r + 1], base[0, :r + 1])
    assert np.abs(after[0, r + 1:] - base[0, r + 1:]).max() > 1e-3
    v3 = v.copy()
    v3[:, :, p] += 1.0          # the row's own key is visible
    own, _ = oracle.prefill(qp, k, v3, lens)
    assert np.abs(own[0, r] - base[0, r]).max() > 1e-6


def test_prefill_row_subset():
    qp = _rand(19, 1, 4, 4, 8)
    _, k, v, _ = _case(20, 1, 4, 2, 4, 8, 8, 12)
    full, _ = oracle.prefill(qp, k, v, np.array([12]))
    part, _ = oracle.prefill(qp, k, v, np.array([12]), rows=[(0, 3)])
    np.testing.assert_array_equal(part[0, 3], full[0, 3])
    assert np.isnan(part[0, :3]).all()


def test_prefill_all_rows_equals_row_by_row():
    # The matrix form over all new rows of a head against the row-by-row
    # definition: a ragged batch whose second sequence is shorter than the
    # prefill (its first rows see no key), asymmetric heads, both head maps.
    B, T = 3, 7
    n_q, n_k, n_v, d_k, d_v = 8, 2, 4, 16, 24
    qp = _rand(21, B, T, n_q, d_k)
    _, k, v, _ = _case(22, B, n_q, n_k, n_v, d_k, d_v, 40)
    lens = np.array([40, 4, 7])
    ref, ref_lse = oracle.prefill(qp, k, v, lens, 0.3)
    out, lse = oracle.prefill_all_rows(qp, k, v, lens, 0.3)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)
    assert (out[1, :3] == 0).all() and np.isneginf(lse[1, :3]).all()


def test_prefill_all_rows_matches_masked_sdpa():
    # An independent library routine: torch's scaled_dot_product_attention in
    # fp64 with an explicit bottom-right causal mask (row r of T sees keys
    # 0 .. L - T + r) on K / V heads repeated to the query heads.
    B, T, L = 1, 9, 25
    n_q, n_k, n_v, d_k, d_v = 8, 2, 8, 32, 16
    qp = _rand(23, B, T, n_q, d_k)
    _, k, v, _ = _case(24, B, n_q, n_k, n_v, d_k, d_v, L)
    out, lse = oracle.prefill_all_rows(qp, k, v, np.array([L]))
    kx = torch.from_numpy(k[0][[i * n_k // n_q for i in range(n_q)]])
    vx = torch.from_numpy(v[0][[i * n_v // n_q for i in range(n_q)]])
    qt = torch.from_numpy(qp[0]).transpose(0, 1).contiguous()      # [n_q][T][d_k]
    mask = torch.arange(L)[None, :] <= (L - T + torch.arange(T))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kx, vx, attn_mask=mask)
    np.testing.assert_allclose(out[0], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    s = (qt @ kx.transpose(1, 2)) / math.sqrt(d_k)
    ref_lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    np.testing.assert_allclose(lse[0], ref_lse.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- kv_append

def test_kv_append_is_step2_concatenation():
    # Step 2 of §3.4: K_t = [K_{t-1}; k_t]; with the cache filled to pos[b]
    # the appended cache equals the concatenation along time.
    B, n_k, n_v, d_k, d_v, cap, T = 2, 4, 16, 8, 16, 12, 3
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 65536, (B, n_k, cap, d_k), dtype=np.uint16)
    vc = rng.integers(0, 65536, (B, n_v, cap, d_v), dtype=np.uint16)
    kn = rng.integers(0, 65536, (B, T, n_k, d_k), dtype=np.uint16)
    vn = rng.integers(0, 65536, (B, T, n_v, d_v), dtype=np.uint16)
    pos = np.array([5, 9])
    k2, v2 = oracle.kv_append(kc, vc, kn, vn, pos)
    for b in range(B):
        p = pos[b]
        kcat = np.concatenate([kc[b, :, :p], kn[b].transpose(1, 0, 2)], axis=1)
        vcat = np.concatenate([vc[b, :, :p], vn[b].transpose(1, 0, 2)], axis=1)
        np.testing.assert_array_equal(k2[b, :, :p + T], kcat)
        np.testing.assert_array_equal(v2[b, :, :p + T], vcat)
        np.testing.assert_array_equal(k2[b, :, p + T:], kc[b, :, p + T:])
        np.testing.assert_array_equal(v2[b, :, p + T:], vc[b, :, p + T:])
    np.testing.assert_array_equal(kc, kc.copy())  # inputs untouched


# ------------------------------------------------------------ mutation check

def test_pins_catch_planted_mistakes(monkeypatch):
    """Each planted mistake in the oracle must make at least one pin fail."""
    import oracle.attention as A

    pins = [
        lambda g: test_flexheadfa_index_worked_example(g),
        lambda g: test_reduces_to_textbook_attention(16, 4, 64, 129),
        lambda g: test_asymmetric_matches_per_head_sdpa(),
        lambda g: test_brute_force_explicit_softmax(),
        lambda g: test_two_keys_with_chosen_logits(),
        lambda g: test_prefill_row_equals_decode_at_its_position(),
        lambda g: test_prefill_causal_mask(),
        lambda g: test_default_scale_is_inverse_sqrt_dk(),
        lambda g: test_zero_scale_is_mean_of_value_rows(),
        lambda g: test_prefill_all_rows_equals_row_by_row(),
        lambda g: test_prefill_all_rows_matches_masked_sdpa(),
    ]
    from conftest import read_golden

    real_gsi, real_weights, real_prefill = A.group_sharing_index, A.attention_weights, A.prefill
    real_all_rows = A.prefill_all_rows

    def ceil_map(i, n_q, n_h):
        return -((-int(i) * int(n_h)) // int(n_q))

    def wrong_sign(q_i, K_i, scale):
        return real_weights(q_i, K_i, -scale)

    def unnormalised(q_i, K_i, scale):
        s = scale * (np.asarray(K_i, float) @ np.asarray(q_i, float))
        w = np.exp(s - s.max())
        return w / w.sum() * (1 + 1e-3), float(s.max() + math.log(w.sum()))

    def dv_scale(d_k):
        return 1.0 / math.sqrt(2 * d_k)

    def strict_causal(q, k_cache, v_cache, ctx_len, scale=None, rows=None):
        return real_prefill(q, k_cache, v_cache, np.asarray(ctx_len) - 1, scale, rows)

    def all_rows_strict_causal(q, k_cache, v_cache, ctx_len, scale=None):
        return real_all_rows(q, k_cache, v_cache, np.asarray(ctx_len) - 1, scale)

    def all_rows_top_left(q, k_cache, v_cache, ctx_len, scale=None):
        # causal mask aligned to the first key instead of the newest row
        T = q.shape[1]
        o, l = real_all_rows(q, k_cache, v_cache, np.full(len(ctx_len), T), scale)
        return o, l

    mutants = {
        "ceil head map": ("group_sharing_index", ceil_map),
        "round-robin head map": ("group_sharing_index", lambda i, n_q, n_h: int(i) % int(n_h)),
        "negated scores": ("attention_weights", wrong_sign),
        "weights not normalised": ("attention_weights", unnormalised),
        "scale 1/sqrt(d_v)": ("default_scale", dv_scale),
        "causal off by one": ("prefill", strict_causal),
        "all-rows causal off by one": ("prefill_all_rows", all_rows_strict_causal),
        "all-rows top-left causal mask": ("prefill_all_rows", all_rows_top_left),
    }
    for name, (attr, fn) in mutants.items():
        with monkeypatch.context() as m:
            m.setattr(A, attr, fn)
            m.setattr(oracle, attr, fn)
            caught = False
            for pin in pins:
                try:
                    pin(read_golden)
                except AssertionError:
                    caught = True
                    break
            assert caught, f"no pin caught the planted mistake: {name}"
    assert A.group_sharing_index is real_gsi


# ------------------------------------------------------------- selective V

def test_selective_with_k_at_least_length_is_full_decode():
    q, k, v, lens = _case(31, 2, 8, 2, 4, 16, 32, 50)
    full, _ = oracle.decode(q, k, v, lens)
    for top_k in (50, 51, 1000):
        sel, rows = oracle.decode_selective(q, k, v, lens, top_k)
        np.testing.assert_allclose(sel, full, rtol=1e-13, atol=1e-15)
        assert all(len(r) == 50 for rb in rows for r in rb)


def test_selective_top1_is_the_argmax_row():
    q, k, v, lens = _case(32, 1, 4, 1, 4, 16, 8, 40)
    sel, rows = oracle.decode_selective(q, k, v, lens, 1)
    scale = 1 / math.sqrt(16)
    for i in range(4):
        s = scale * (k[0, 0, :40] @ q[0, i])
        j = int(np.argmax(s))
        alpha_j = math.exp(s[j]) / np.exp(s).sum()
        assert list(rows[0][i]) == [j]
        np.testing.assert_allclose(sel[0, i], alpha_j * v[0, i, j], rtol=1e-13)


def test_selective_brute_force_tiny():
    n_q, n_k, n_v, d_k, d_v, L, top_k = 4, 2, 2, 3, 5, 9, 4
    q, k, v, lens = _case(33, 1, n_q, n_k, n_v, d_k, d_v, L)
    sel, _ = oracle.decode_selective(q, k, v, lens, top_k)
    scale = 1.0 / math.sqrt(d_k)
    for i in range(n_q):
        kh, vh = i * n_k // n_q, i * n_v // n_q
        s = [scale * sum(q[0, i, d] * k[0, kh, j, d] for d in range(d_k)) for j in range(L)]
        z = sum(math.exp(x) for x in s)
        a = [math.exp(x) / z for x in s]
        best = sorted(range(L), key=lambda j: (-a[j], j))[:top_k]
        for d in range(d_v):
            assert abs(sel[0, i, d] - sum(a[j] * v[0, vh, j, d] for j in best)) < 1e-12


def test_selective_ties_go_to_lower_rows():
    # All keys equal: every weight is 1/L; the first k rows are selected.
    q = _rand(34, 1, 2, 8)
    k = np.repeat(_rand(35, 1, 1, 1, 8), 30, axis=2)
    v = _rand(36, 1, 2, 30, 4)
    sel, rows = oracle.decode_selective(q, k, v, np.array([30]), 7)
    for i in range(2):
        assert list(rows[0][i]) == list(range(7))
        np.testing.assert_allclose(sel[0, i], v[0, i, :7].sum(axis=0) / 30, rtol=1e-13)
