"""GPU check of diffqkv_decode_append_noalloc, the decode entry point that
takes no workspace (its partial results live in the library's static device
scratch): through the C ABI, against diffqkv_decode_append with a caller
workspace, bit for bit, on two calls in a row whose second is smaller."""

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_util import ints_to_dev, raw_host, to_dev

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


def _inputs(seed, B, lens, cap):
    case = synth.make_case(seed, dtype="bf16", batch=B, n_q=16, n_k=4, n_v=16, d_k=64,
                           d_v=128, ctx_len=lens, l_cap=cap)
    kn, vn = synth.new_rows(seed, dtype="bf16", batch=B, t_new=1, n_k=4, n_v=16, d_k=64,
                            d_v=128)
    return case, to_dev(kn, "bf16"), to_dev(vn, "bf16")


def _run(case, kn, vn, noalloc, fused):
    """One decode step through the C ABI; returns (out, lse, k, v) on the host."""
    lib = dq.load()
    B = case.batch
    q = to_dev(case.q, "bf16")
    k, v = to_dev(case.k_cache, "bf16"), to_dev(case.v_cache, "bf16")
    ctx = ints_to_dev(case.ctx_len)
    out = torch.empty((B, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 16), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = (16, 4, 16, 64, 128, dq.BF16, B, case.l_cap, case.l_cap, 0.0, q.data_ptr(),
            kn.data_ptr() if fused else None, vn.data_ptr() if fused else None,
            k.data_ptr(), v.data_ptr(), ctx.data_ptr(), out.data_ptr(), lse.data_ptr(), 0)
    if noalloc:
        st = lib.diffqkv_decode_append_noalloc(*args, stream)
        assert st == 0, dq.status_str(st)
    else:
        ws_bytes = dq.decode_workspace_bytes(16, 4, 16, 64, 128, B, case.l_cap)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        fn = lib.diffqkv_decode_append if fused else lib.diffqkv_decode
        if fused:
            st = fn(*args, ws.data_ptr(), ws_bytes, stream)
        else:
            st = fn(*args[:10], args[10], args[13], args[14], args[15], args[16], args[17],
                    args[18], ws.data_ptr(), ws_bytes, stream)
        assert st == 0, dq.status_str(st)
    torch.cuda.synchronize()
    return raw_host(out), lse.cpu().numpy(), raw_host(k), raw_host(v)


@pytest.mark.parametrize("fused", [True, False])
def test_noalloc_matches_workspace_decode_twice(fused):
    # First a ragged batch of three sequences, then one shorter sequence: the
    # second call reuses the scratch that still holds the first call's partials.
    calls = [(_inputs(711, 3, [5000, 1234, 64], 5056)), (_inputs(712, 1, [700], 704))]
    for n, (case, kn, vn) in enumerate(calls):
        _say(f"noalloc decode call {n + 1}: batch {case.batch}, lengths {list(case.ctx_len)}, "
             f"fused append {fused}")
        got = _run(case, kn, vn, noalloc=True, fused=fused)
        want = _run(case, kn, vn, noalloc=False, fused=fused)
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g, w)
        assert np.isfinite(got[1]).all()
