"""GPU parity of the split-KV decode + combine kernels against the fp64 oracle.

Small cases run the oracle on every output; they span several 64-row tiles
and chunks with ragged tails, every supported head dimension, both dtypes,
ragged batches and empty / single-row contexts.  The full-size workloads
(32k single sequence with its symmetric twin, the ragged batch of 16 with an
append, and 64k batch 4 with outlier channels) run in the launch
configuration the benchmark times and are checked in full.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (assert_close, assert_lse_close, ints_to_dev, raw_host, to_dev,
                      to_host, upload)

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


def run_decode(case, chunk=0, max_ctx=None):
    q, k, v, ctx = upload(case)
    B, n_q = case.batch, case.n_q
    lse = torch.empty((B, n_q), dtype=torch.float32, device="cuda")
    out, lse = dq.decode(q, k, v, ctx, max_ctx=max_ctx or case.l_cap, scale=case.scale,
                         lse=lse, chunk_tokens=chunk)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


def oracle_decode(case):
    q, k, v = case.widened()
    return oracle.decode(q, k, v, case.ctx_len, case.scale)


SMALL = [
    # dtype, n_q, n_k, n_v, d_k, d_v, lengths, l_cap
    ("f32", 4, 1, 4, 32, 64, [256], 256),
    ("f32", 8, 2, 4, 64, 32, [1000, 37], 1024),
    ("f32", 16, 16, 16, 128, 128, [300], 320),
    ("f32", 6, 3, 2, 64, 64, [130, 129, 1], 140),
    ("f32", 4, 2, 4, 32, 256, [200], 200),
    ("bf16", 16, 4, 16, 64, 128, [5000, 1, 64, 65, 129], 5000),
    ("bf16", 32, 4, 16, 64, 64, [3000, 700], 3072),     # SIGMA-1.5B heads
    ("bf16", 32, 16, 16, 64, 64, [2100, 64], 2112),     # the pages' standard GQA
    ("bf16", 16, 16, 16, 128, 128, [2000], 2048),
    ("bf16", 16, 1, 16, 256, 256, [500], 512),
    ("bf16", 8, 8, 2, 32, 256, [777], 800),
    ("bf16", 16, 4, 16, 128, 128, [1500, 333], 1536),
    ("bf16", 12, 4, 12, 64, 128, [999], 1000),
    ("bf16", 8, 4, 4, 64, 64, [1000, 3], 1024),          # head pairs share K and V
    ("bf16", 12, 2, 6, 64, 128, [700], 704),            # pairs, last workgroup half full
    ("f32", 8, 2, 4, 64, 64, [300], 320),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_logits_far_above_the_rest(dtype):
    # q = 1 everywhere; a few K rows far larger than the rest, in different
    # chunks: their logits lie ~100 and ~190 (log2 units) above every other
    # row's, past fp32's exponent range for the second.  Each chunk's running
    # max and the combine's merge must keep the result finite and exact.
    case = synth.make_case(611, dtype=dtype, batch=2, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[3000, 1700], l_cap=3072, poison_tail=True)
    one, nine, seventeen = (0x3F80, 0x4110, 0x4188) if dtype == "bf16" else (1.0, 9.0, 17.0)
    case.q[...] = one
    case.k_cache[0, :, 2100, :] = nine
    case.k_cache[0, :, 2950, :] = seventeen
    case.k_cache[1, :, 77, :] = seventeen
    ref, ref_lse = oracle_decode(case)
    for chunk in (0, 64, 320):
        _say("decode logits far above the rest", dtype, "chunk", chunk)
        got, lse = run_decode(case, chunk=chunk)
        assert np.isfinite(got).all()
        assert_close(got, ref, dtype, f"spiked decode chunk={chunk}")
        assert_lse_close(lse, ref_lse, dtype, f"spiked decode chunk={chunk}")


def _log2_score_rows(case, level):
    """Set every K row so that its (scaled, log2-unit) logit against an
    all-ones q is level[j] (d_k equal elements per row)."""
    d_k = case.d_k
    c = np.asarray(level, dtype=np.float64) / (np.log2(np.e) * case.scale * d_k)
    row = np.repeat(c[:, None], d_k, axis=1).astype(np.float32)
    if case.dtype == "bf16":
        case.q[...] = 0x3F80
        row = synth.f32_to_bf16_bits(row)
    else:
        case.q[...] = 1.0
    case.k_cache[:, :, : len(level), :] = row[None, None]


@pytest.mark.parametrize("jump", [7.9, 8.1])
@pytest.mark.parametrize("chunk", [128, 512])
def test_decode_logits_step_up_after_first_tile(jump, chunk):
    # Every chunk's first 64-row tile has logits near 0 (log2 units), the
    # rest lie `jump` higher.  Below the kernel's margin of 8 the chunk keeps
    # the first tile's reference and its weights stay just under 2^8 over
    # every later tile; above it the reference moves once per chunk.
    case = synth.make_case(612, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16, d_k=64,
                           d_v=128, ctx_len=[2000], l_cap=2048, poison_tail=True)
    j = np.arange(2000)
    _log2_score_rows(case, np.where(j % chunk < 64, 0.0, jump) + 0.01 * (j % 7))
    ref, ref_lse = oracle_decode(case)
    _say("decode logits step up", jump, "chunk", chunk)
    got, lse = run_decode(case, chunk=chunk)
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", f"step-up decode jump={jump} chunk={chunk}")
    assert_lse_close(lse, ref_lse, "bf16", f"step-up decode jump={jump} chunk={chunk}")


@pytest.mark.parametrize("slope", [7.9 / 64, 8.1 / 64, 0.5])
def test_decode_logits_rising_ramp_f32(slope):
    # fp32 cache, logits rising by `slope` (log2 units) per row over 3000
    # rows up to 0 at the last one (from -1500 at most, so lse stays small
    # enough for its absolute tolerance): the running reference lags the
    # maximum by up to the margin, or moves on every tile.
    case = synth.make_case(613, dtype="f32", batch=1, n_q=8, n_k=2, n_v=8, d_k=32, d_v=64,
                           ctx_len=[3000], l_cap=3072, poison_tail=True)
    _log2_score_rows(case, slope * (np.arange(3000) - 2999))
    ref, ref_lse = oracle_decode(case)
    for chunk in (0, 256):
        _say("decode rising ramp f32", slope, "chunk", chunk)
        got, lse = run_decode(case, chunk=chunk)
        assert np.isfinite(got).all()
        assert_close(got, ref, "f32", f"ramp decode slope={slope} chunk={chunk}")
        assert_lse_close(lse, ref_lse, "f32", f"ramp decode slope={slope} chunk={chunk}")


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}x{c[5]}")
def test_decode_small_matches_oracle(cfg):
    dtype, n_q, n_k, n_v, d_k, d_v, lens, cap = cfg
    case = synth.make_case(101, dtype=dtype, batch=len(lens), n_q=n_q, n_k=n_k, n_v=n_v,
                           d_k=d_k, d_v=d_v, ctx_len=lens, l_cap=cap, poison_tail=True)
    _say("decode small", cfg)
    ref, ref_lse = oracle_decode(case)
    for chunk in (0, 64, 192):
        got, lse = run_decode(case, chunk=chunk)
        assert_close(got, ref, dtype, f"{cfg} chunk={chunk}")
        assert_lse_close(lse, ref_lse, dtype, f"{cfg} chunk={chunk}")


def test_decode_tiny_f32_workload():
    case = synth.make_case(**synth.workload("tiny_f32"))
    _say("decode tiny_f32")
    ref, ref_lse = oracle_decode(case)
    got, lse = run_decode(case)
    err = assert_close(got, ref, "f32", "tiny_f32")
    assert_lse_close(lse, ref_lse, "f32", "tiny_f32")
    _say(f"tiny_f32 normwise rel err {err:.2e}")


def test_empty_context_gives_zero_and_neg_inf():
    case = synth.make_case(5, dtype="bf16", batch=3, n_q=8, n_k=2, n_v=8, d_k=64, d_v=128,
                           ctx_len=[0, 70, 0], l_cap=128, poison_tail=True)
    _say("decode empty contexts")
    got, lse = run_decode(case)
    ref, ref_lse = oracle_decode(case)
    assert (got[0] == 0).all() and (got[2] == 0).all()
    assert np.isneginf(lse[0]).all() and np.isneginf(lse[2]).all()
    assert_close(got, ref, "bf16", "empty")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_row_context_is_exact(dtype):
    # One visible row: weight exactly 1, so the output is that V row.
    case = synth.make_case(6, dtype=dtype, batch=2, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[1, 1], l_cap=64, poison_tail=True)
    _say("decode single row", dtype)
    q, k, v, ctx = upload(case)
    out, _ = dq.decode(q, k, v, ctx, scale=case.scale)
    torch.cuda.synchronize()
    got = raw_host(out)
    for b in range(2):
        for i in range(16):
            np.testing.assert_array_equal(got[b, i], case.v_cache[b, i, 0])


def test_chunk_length_invariance():
    case = synth.make_case(7, dtype="f32", batch=2, n_q=8, n_k=2, n_v=8, d_k=64, d_v=128,
                           ctx_len=[3000, 1234], l_cap=3072)
    _say("decode chunk invariance")
    outs = [run_decode(case, chunk=c)[0] for c in (64, 128, 640, 3072)]
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=0, atol=2e-6 * np.abs(outs[0]).max())


def test_kv_group_sharing_equivalence_gpu():
    # Copying every K head n_v/n_k times (the pages' compatibility shim) must
    # give bit-identical results: each query head reads the same K bytes.
    case = synth.make_case(8, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[4000], l_cap=4096)
    _say("decode kv_group_sharing equivalence")
    a, la = run_decode(case)
    dup = synth.DecodeCase(**{**case.__dict__, "n_k": 16,
                              "k_cache": np.repeat(case.k_cache, 4, axis=1)})
    b, lb = run_decode(dup)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


FUSED = [
    # dtype, n_q, n_k, n_v, d_k, d_v, lengths after the append, l_cap, chunk
    ("bf16", 16, 4, 16, 64, 128, [65, 1, 128, 300, 4097], 4100, 0),
    ("bf16", 16, 4, 16, 64, 128, [65, 1, 128, 300, 4097], 4100, 64),
    ("bf16", 32, 4, 16, 64, 64, [700, 64], 704, 128),
    ("bf16", 16, 16, 16, 128, 128, [1000, 999], 1024, 0),
    ("f32", 8, 2, 4, 32, 64, [257, 2], 260, 64),
]


@pytest.mark.parametrize("cfg", FUSED, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}x{c[5]}-c{c[8]}")
def test_fused_append_equals_append_then_decode(cfg):
    dtype, n_q, n_k, n_v, d_k, d_v, lens, cap, chunk = cfg
    B = len(lens)
    case = synth.make_case(303, dtype=dtype, batch=B, n_q=n_q, n_k=n_k, n_v=n_v, d_k=d_k,
                           d_v=d_v, ctx_len=lens, l_cap=cap, poison_tail=True)
    k_new, v_new = synth.new_rows(303, dtype=dtype, batch=B, t_new=1, n_k=n_k, n_v=n_v,
                                  d_k=d_k, d_v=d_v)
    _say("fused append", cfg)
    lens = np.asarray(lens)
    # Two-kernel-launch reference: kv_append, then decode.
    q, k1, v1, ctx = upload(case)
    kn, vn = to_dev(k_new, dtype), to_dev(v_new, dtype)
    dq.kv_append(kn, vn, ints_to_dev(lens - 1), k1, v1, n_q=n_q)
    lse1 = torch.empty((B, n_q), dtype=torch.float32, device="cuda")
    out1, _ = dq.decode(q, k1, v1, ctx, lse=lse1, chunk_tokens=chunk)
    # Fused.
    _, k2, v2, _ = upload(case)
    lse2 = torch.empty((B, n_q), dtype=torch.float32, device="cuda")
    out2, _ = dq.decode(q, k2, v2, ctx, lse=lse2, chunk_tokens=chunk,
                        k_new=kn.view(B, n_k, d_k), v_new=vn.view(B, n_v, d_v))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(raw_host(out2), raw_host(out1))
    np.testing.assert_array_equal(raw_host(lse2), raw_host(lse1))
    np.testing.assert_array_equal(raw_host(k2), raw_host(k1))
    np.testing.assert_array_equal(raw_host(v2), raw_host(v1))
    # And both match the oracle of Step 2 followed by Steps 3-5.
    kh, vh = oracle.kv_append(case.k_cache, case.v_cache, k_new, v_new, lens - 1)
    wid = (lambda a: synth.bf16_bits_to_f32(a)) if dtype == "bf16" else (lambda a: a)
    ref, ref_lse = oracle.decode(wid(case.q), wid(kh), wid(vh), lens, case.scale)
    assert_close(to_host(out2), ref, dtype, str(cfg))
    assert_lse_close(to_host(lse2), ref_lse, dtype, str(cfg))


# ------------------------------------------------------------ full workloads

@pytest.mark.parametrize("name", ["decode32k_asym", "decode32k_sym"])
def test_decode_32k_full(name):
    case = synth.make_case(**synth.workload(name))
    _say("decode full", name)
    ref, ref_lse = oracle_decode(case)
    got, lse = run_decode(case)
    err = assert_close(got, ref, "bf16", name)
    assert_lse_close(lse, ref_lse, "bf16", name)
    _say(f"{name} normwise rel err {err:.2e}")


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "kv_append"])
def test_ragged_batch_append_then_decode_full(fused):
    kw = synth.workload("ragged16")
    old = np.asarray(kw["ctx_len"])
    case = synth.make_case(**{**kw, "poison_tail": True})
    k_new, v_new = synth.new_rows(kw["seed"], dtype="bf16", batch=16, t_new=1, n_k=4, n_v=16,
                                  d_k=64, d_v=128)
    _say("ragged16: append + decode, fused", fused, "lengths", old.min(), old.max())
    q, k, v, _ = upload(case)
    kn, vn = to_dev(k_new, "bf16"), to_dev(v_new, "bf16")
    ctx = ints_to_dev(old + 1)
    lse = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    if fused:
        out, lse = dq.decode(q, k, v, ctx, max_ctx=case.l_cap, lse=lse,
                             k_new=kn.view(16, 4, 64), v_new=vn.view(16, 16, 128))
    else:
        dq.kv_append(kn, vn, ints_to_dev(old), k, v, n_q=16)
        out, lse = dq.decode(q, k, v, ctx, max_ctx=case.l_cap, lse=lse)
    torch.cuda.synchronize()
    kh, vh = oracle.kv_append(case.k_cache, case.v_cache, k_new, v_new, old)
    np.testing.assert_array_equal(raw_host(k), kh)
    del k
    np.testing.assert_array_equal(raw_host(v), vh)
    del v
    ref, ref_lse = oracle.decode(synth.bf16_bits_to_f32(case.q), synth.bf16_bits_to_f32(kh),
                                 synth.bf16_bits_to_f32(vh), old + 1, case.scale)
    err = assert_close(to_host(out), ref, "bf16", "ragged16")
    assert_lse_close(to_host(lse), ref_lse, "bf16", "ragged16")
    _say(f"ragged16 normwise rel err {err:.2e}")


@pytest.mark.parametrize("name", ["decode64k_dk64", "decode64k_dk128", "decode64k_sym"])
def test_decode_64k_full(name):
    case = synth.make_case(**synth.workload(name))
    _say("decode full", name, "outliers", case.outliers)
    got, lse = run_decode(case)
    ref, ref_lse = oracle_decode(case)
    err = assert_close(got, ref, "bf16", name)
    assert_lse_close(lse, ref_lse, "bf16", name)
    _say(f"{name} normwise rel err {err:.2e}")
