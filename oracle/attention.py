"""fp64 CPU oracle for DiffQKV attention -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU library never calls it and it never calls the GPU
library: the two share no code.

This is the plain definition of the attention that the Sigma pages describe,
written for a reader to check against them by eye.  Citations name the page
("Sigma architecture page" = the paper-graph-ui.vercel.app architecture
summary of arXiv 2501.13629 "Sigma: Differential Rescaling of Query, Key and
Value for Efficient Language Models"; "Pith review page" = pith.science's
review of the same paper) and the section or equation on it.

Everything is computed in float64 from inputs widened exactly from their
storage type.  The softmax is two-pass (maximum, then normalised exponentials)
and unchunked: it deliberately shares no structure with the split/online GPU
kernels.  numpy's matrix-vector product is the only library step.

Readings taken where the pages are silent:
* scale defaults to 1/sqrt(d_k)                (architecture page, §3.4 Step 4)
* head maps are floor(i * n_h / n_q), 0-based  (§3.4 Step 3; FlexHeadFA section)
* the newest token attends to itself: ctx_len counts the rows after the
  append of Step 2                              (§3.4 Steps 2 and 5)
* prefill rows use a bottom-right causal mask: new row r of a sequence with
  L rows attends keys 0 .. L - t_new + r       (not on the pages)
* an empty context yields o = 0, lse = -inf    (never arises in a decoder)

Selective-V decode (architecture page, "Selective V Cache Fetching") keeps
the full softmax weights and sums only the V rows of the k largest; ties go
to the lower row index (a reading: the page does not say).  Two layouts are
defined as copies: the kv_group_sharing expansion (FlexHeadFA section) and a
paged cache with separate K and V page pools under one block table.

Pins (tests/test_oracle.py): the FlexHeadFA index worked example, reduction
to textbook MHA / GQA / MQA (torch's scaled_dot_product_attention in fp64),
weights summing to 1, brute-force softmax without max-shift on tiny shapes,
the kv_group_sharing equivalence, closed forms (one key, zero scale, two keys
with chosen logits), key-permutation invariance, prefill/decode consistency
and causal masking, Step 2's concatenation for the append, and for
selective V: k >= L equals full decode, k = 1 is the arg-max row times its
weight, brute force on tiny shapes, and ties resolved to lower indices; for
the layouts: attention unchanged under kv_group_sharing (both directions),
the page's 4 -> 16 replication count, and paged gather / scatter round trips
with decode over shuffled pages equal to decode over the contiguous cache.
"""

from __future__ import annotations

import math

import numpy as np


def group_sharing_index(i: int, n_q: int, n_h: int) -> int:
    """Index of the K (or V) head that query head ``i`` reads.

    Sigma architecture page, §3.4 Step 3 (GroupSharing): query head i uses
    head floor(i * n_h / n_q); the FlexHeadFA section gives the same address
    rule idx_h = idx_q * n_h / n_q with 0-based indices (query heads 0 and 1
    read K head 0 and V head 0, query head 2 reads V head 1, for 32/4/16).
    """
    return (int(i) * int(n_h)) // int(n_q)


def default_scale(d_k: int) -> float:
    """1/sqrt(d_k): the divisor of the Attend scores in §3.4 Step 4."""
    return 1.0 / math.sqrt(d_k)


def attention_weights(q_i: np.ndarray, K_i: np.ndarray, scale: float):
    """alpha = Softmax(scale * Attend(q_i, K_i)) and its log-sum-exp.

    §3.4 Step 4: Attend is the inner product of the d_k-dimensional query head
    with every key row.  Two passes: the largest score, then exponentials of
    the shifted scores normalised by their sum (subtracting a constant leaves
    the softmax unchanged in exact arithmetic).

    Returns ``(alpha[L], lse)`` with ``lse = log(sum_j exp(scale * q.k_j))``.
    """
    q64 = np.asarray(q_i, dtype=np.float64)
    K64 = np.asarray(K_i, dtype=np.float64)
    s = scale * (K64 @ q64)
    m = s.max()
    w = np.exp(s - m)
    z = w.sum()
    return w / z, float(m + math.log(z))


def attend_one(q_i, K_i, V_i, scale: float):
    """o = sum_j alpha_j V_j for one query head (§3.4 Step 5)."""
    if K_i.shape[0] == 0:
        return np.zeros(V_i.shape[1], dtype=np.float64), -math.inf
    alpha, lse = attention_weights(q_i, K_i, scale)
    return alpha @ np.asarray(V_i, dtype=np.float64), lse


def decode(q, k_cache, v_cache, ctx_len, scale: float | None = None):
    """One decode step of DiffQKV attention.

    Shapes: ``q[B][n_q][d_k]``, ``k_cache[B][n_k][l_cap][d_k]``,
    ``v_cache[B][n_v][l_cap][d_v]``, ``ctx_len[B]`` (rows attended, newest
    included).  Query head i of sequence b attends rows 0..L_b-1 of K head
    floor(i*n_k/n_q) and weights rows of V head floor(i*n_v/n_q)
    (§3.4 Steps 3-5).  Returns ``(out[B][n_q][d_v], lse[B][n_q])`` in float64.
    """
    B, n_q, d_k = q.shape
    n_k = k_cache.shape[1]
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if scale is None:
        scale = default_scale(d_k)
    out = np.zeros((B, n_q, d_v), dtype=np.float64)
    lse = np.full((B, n_q), -math.inf, dtype=np.float64)
    for b in range(B):
        L = int(ctx_len[b])
        for i in range(n_q):
            g = group_sharing_index(i, n_q, n_k)
            hv = group_sharing_index(i, n_q, n_v)
            out[b, i], lse[b, i] = attend_one(q[b, i], k_cache[b, g, :L],
                                              v_cache[b, hv, :L], scale)
    return out, lse


def prefill(q, k_cache, v_cache, ctx_len, scale: float | None = None,
            rows=None):
    """Causal attention of ``t_new`` new query rows against the cache.

    ``q[B][t_new][n_q][d_k]``; ``ctx_len[B]`` counts cache rows *after* the
    new rows were appended (so ``ctx_len[b] >= t_new``).  New row r of
    sequence b sits at position p = ctx_len[b] - t_new + r and attends keys
    0..p: each token attends every earlier token and itself (§3.4 Steps 2 and
    5, applied token by token).

    ``rows`` optionally restricts the computation to a list of ``(b, r)``;
    the other rows are returned as NaN.  Returns ``(out[B][t_new][n_q][d_v],
    lse[B][t_new][n_q])`` in float64.
    """
    B, T, n_q, d_k = q.shape
    n_k = k_cache.shape[1]
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if scale is None:
        scale = default_scale(d_k)
    if rows is None:
        rows = [(b, r) for b in range(B) for r in range(T)]
    out = np.full((B, T, n_q, d_v), np.nan, dtype=np.float64)
    lse = np.full((B, T, n_q), np.nan, dtype=np.float64)
    for b, r in rows:
        p = int(ctx_len[b]) - T + r
        n_vis = max(p + 1, 0)      # keys 0..p; none when the row sits before key 0
        for i in range(n_q):
            g = group_sharing_index(i, n_q, n_k)
            hv = group_sharing_index(i, n_q, n_v)
            out[b, r, i], lse[b, r, i] = attend_one(
                q[b, r, i], k_cache[b, g, :n_vis], v_cache[b, hv, :n_vis], scale)
    return out, lse


def prefill_all_rows(q, k_cache, v_cache, ctx_len, scale: float | None = None):
    """Every row of :func:`prefill`, with one matrix product per head.

    The same definition written over all new rows of a (sequence, query
    head) at once: S = scale * Q_i K_g^T over the L_b cache rows (t_new x
    L_b), score (r, j) dropped (set to -inf) when key j lies past row r's
    position p_r = L_b - t_new + r, then per row the two-pass softmax of
    :func:`attention_weights` (row maximum, exponentials, normalisation) and
    the weighted sum W V (section 3.4 Steps 4 and 5, row by row).  Rows with
    p_r < 0 see no key: o = 0, lse = -inf.  numpy's matrix product is the
    only library step; it trades the per-row loop for memory (two t_new x
    L_b float64 matrices per head), which makes full-size prefills feasible.
    Returns ``(out[B][t_new][n_q][d_v], lse[B][t_new][n_q])`` in float64.
    """
    B, T, n_q, d_k = q.shape
    n_k = k_cache.shape[1]
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if scale is None:
        scale = default_scale(d_k)
    out = np.zeros((B, T, n_q, d_v), dtype=np.float64)
    lse = np.full((B, T, n_q), -math.inf, dtype=np.float64)
    for b in range(B):
        L = int(ctx_len[b])
        p = L - T + np.arange(T)              # position of each new row
        seen = p >= 0                         # rows that see at least key 0
        if not seen.any():
            continue
        # visible[r, j]: key j at or before row r's position.
        visible = np.arange(L)[None, :] <= p[:, None]
        for i in range(n_q):
            g = group_sharing_index(i, n_q, n_k)
            hv = group_sharing_index(i, n_q, n_v)
            Q = np.asarray(q[b, :, i, :], dtype=np.float64)
            K = np.asarray(k_cache[b, g, :L], dtype=np.float64)
            V = np.asarray(v_cache[b, hv, :L], dtype=np.float64)
            S = scale * (Q @ K.T)
            S[~visible] = -math.inf
            m = S[seen].max(axis=1, keepdims=True)
            W = np.exp(S[seen] - m)
            Z = W.sum(axis=1)
            out[b, seen, i] = (W @ V) / Z[:, None]
            lse[b, seen, i] = m[:, 0] + np.log(Z)
    return out, lse


def kv_append(k_cache, v_cache, k_new, v_new, pos):
    """Step 2 of §3.4: K_t = [K_{t-1}; k_t], V_t = [V_{t-1}; v_t].

    The K and V caches are separate arrays with their own head counts and
    head dimensions (architecture page §3.2 item 3).  ``k_new[B][T][n_k][d_k]``
    and ``v_new[B][T][n_v][d_v]`` are token-major; token t of sequence b is
    written at cache row ``pos[b] + t`` of every head.  Works on raw storage
    (bf16 bit patterns or float32) and returns new arrays; a pure copy.
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    B, T = k_new.shape[0], k_new.shape[1]
    for b in range(B):
        for t in range(T):
            row = int(pos[b]) + t
            k[b, :, row, :] = k_new[b, t]
            v[b, :, row, :] = v_new[b, t]
    return k, v


def top_k_rows(alpha: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest weights, ties to the lower index, ascending.

    Reading of the architecture page's TopK (section "Selective V Cache
    Fetching"), which leaves ties open: the lower row index wins.
    """
    order = np.argsort(-np.asarray(alpha, dtype=np.float64), kind="stable")
    return np.sort(order[:min(int(k), alpha.shape[0])])


def attend_selective_one(q_i, K_i, V_i, scale: float, k: int, rows=None):
    """o ~= sum over TopK(alpha) of alpha_j V_j, for one query head.

    Architecture page, "Selective V Cache Fetching": alpha is the full
    softmax over every visible row (the whole K cache is read); only the V
    rows of the k largest weights are fetched and the others count as zero,
    without renormalising.  ``rows`` overrides the selected set (to evaluate
    the formula on a given set).  Returns ``(o, selected_rows)``.
    """
    if K_i.shape[0] == 0:
        return np.zeros(V_i.shape[1], dtype=np.float64), np.zeros(0, dtype=np.int64)
    alpha, _ = attention_weights(q_i, K_i, scale)
    sel = top_k_rows(alpha, k) if rows is None else np.asarray(rows, dtype=np.int64)
    return alpha[sel] @ np.asarray(V_i[sel], dtype=np.float64), sel


def decode_selective(q, k_cache, v_cache, ctx_len, top_k: int, scale: float | None = None):
    """Selective-V decode: per sequence and query head, the weighted sum of
    the V rows with the top_k largest attention weights (architecture page,
    "Selective V Cache Fetching"; head maps and scale as in :func:`decode`).
    Returns ``(out[B][n_q][d_v], selected)`` with ``selected[b][i]`` the
    ascending row indices."""
    B, n_q, d_k = q.shape
    n_k = k_cache.shape[1]
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if scale is None:
        scale = default_scale(d_k)
    out = np.zeros((B, n_q, d_v), dtype=np.float64)
    selected = [[None] * n_q for _ in range(B)]
    for b in range(B):
        L = int(ctx_len[b])
        for i in range(n_q):
            g = group_sharing_index(i, n_q, n_k)
            hv = group_sharing_index(i, n_q, n_v)
            out[b, i], selected[b][i] = attend_selective_one(
                q[b, i], k_cache[b, g, :L], v_cache[b, hv, :L], scale, top_k)
    return out, selected


def kv_group_sharing(k_cache, v_cache):
    """The compatibility expansion for frameworks that need n_k = n_v.

    Architecture page, FlexHeadFA section (the kv_group_sharing wrapper of
    the paper's Appendix E): the side with fewer heads is duplicated up to
    the other's head count -- with n_k < n_v each K head is repeated
    n_v / n_k times, with n_k > n_v each V head n_k / n_v times.  Expanded
    head h' copies original head floor(h' * n_small / n_large), i.e. the
    copies of one head are adjacent, which is the order under which the
    query-head maps of both layouts pick the same rows (pinned by the
    decode-equivalence test).  A pure copy of raw storage.
    """
    k = np.asarray(k_cache)
    v = np.asarray(v_cache)
    n_k, n_v = k.shape[1], v.shape[1]
    n_h = max(n_k, n_v)
    k_idx = [group_sharing_index(h, n_h, n_k) for h in range(n_h)]
    v_idx = [group_sharing_index(h, n_h, n_v) for h in range(n_h)]
    return k[:, k_idx].copy(), v[:, v_idx].copy()


def paged_to_contiguous(k_pages, v_pages, block_table, ctx_len, l_cap=None):
    """Gather a paged cache into the contiguous head-major layout.

    Definition of the paged layout (a serving layout, not on the pages: the
    architecture page names vLLM's paged attention as prior art that treats
    K and V alike; here K and V keep separate page pools with their own row
    shapes and share one block table): row j of sequence b lives in page
    block_table[b][j // P], slot j % P, where P is the page size in rows;
    ``k_pages[num_pages][n_k][P][d_k]``, ``v_pages[num_pages][n_v][P][d_v]``.
    Rows at or past ctx_len[b] are left as zeros.  A pure copy.
    """
    kp = np.asarray(k_pages)
    vp = np.asarray(v_pages)
    table = np.asarray(block_table)
    B = table.shape[0]
    P = kp.shape[2]
    if l_cap is None:
        l_cap = max([int(x) for x in ctx_len] + [1])
    k = np.zeros((B, kp.shape[1], l_cap, kp.shape[3]), dtype=kp.dtype)
    v = np.zeros((B, vp.shape[1], l_cap, vp.shape[3]), dtype=vp.dtype)
    for b in range(B):
        for j in range(int(ctx_len[b])):
            page = int(table[b, j // P])
            k[b, :, j, :] = kp[page, :, j % P, :]
            v[b, :, j, :] = vp[page, :, j % P, :]
    return k, v


def decode_paged(q, k_pages, v_pages, block_table, ctx_len, scale: float | None = None):
    """Decode over a paged cache: :func:`decode` on the gathered rows."""
    k, v = paged_to_contiguous(k_pages, v_pages, block_table, ctx_len)
    return decode(q, k, v, ctx_len, scale)
