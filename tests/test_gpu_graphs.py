"""The entry points under HIP graph capture: each replay must reproduce the
eager result bit for bit (every kernel here is deterministic), with eager
work and synchronisations between the replays."""

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_util import ints_to_dev, raw_host, to_dev, upload

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


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        fn()
    return g


def _replay_and_check(g, outs, want, noise):
    for rep in range(4):
        for o in outs:
            o.fill_(7)  # stale values must not survive a replay
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            np.testing.assert_array_equal(raw_host(o), w, err_msg=f"replay {rep}")
        noise()  # eager work between replays
        torch.cuda.synchronize()


def test_decode_paths_under_graph_replay():
    case = synth.make_case(601, dtype="bf16", batch=2, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[3000, 1500], l_cap=3072)
    kn, vn = synth.new_rows(601, dtype="bf16", batch=2, t_new=1, n_k=4, n_v=16, d_k=64,
                            d_v=128)
    q, k, v, ctx = upload(case)
    kn_d, vn_d = to_dev(kn, "bf16"), to_dev(vn, "bf16")
    B, n_q = 2, 16
    out = torch.empty((B, n_q, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, n_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.decode_workspace_bytes(16, 4, 16, 64, 128, B, 3072), dtype=torch.uint8,
                     device="cuda")
    s_out = torch.empty_like(out)
    s_lse = torch.empty_like(lse)
    s_idx = torch.empty((B, n_q, 100), dtype=torch.int32, device="cuda")
    s_ws = torch.empty(dq.selective_workspace_bytes(16, 4, 16, 64, 128, B, 3072, 100),
                       dtype=torch.uint8, device="cuda")

    def work():
        dq.decode(q, k, v, ctx, scale=case.scale, out=out, lse=lse, workspace=ws, k_new=kn_d,
                  v_new=vn_d)
        dq.decode_selective(q, k, v, ctx, top_k=100, scale=case.scale, out=s_out, lse=s_lse,
                            sel_idx=s_idx, workspace=s_ws, k_new=kn_d, v_new=vn_d)

    _say("graph: fused decode + selective decode")
    work()
    torch.cuda.synchronize()
    want = [raw_host(t) for t in (out, lse, s_out, s_lse, s_idx)]
    g = _capture(work)
    scratch = torch.empty_like(k)

    def noise():
        scratch.copy_(k)
        dq.kv_append(kn_d.view(B, 1, 4, 64), vn_d.view(B, 1, 16, 128), ints_to_dev([0, 1]),
                     scratch, torch.empty_like(v), n_q=16)

    _replay_and_check(g, [out, lse, s_out, s_lse, s_idx], want, noise)


def test_paged_decode_and_prefill_under_graph_replay():
    case = synth.make_case(602, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16, d_k=64, d_v=128,
                           ctx_len=[2048], l_cap=2048, t_new=256)
    q, k, v, ctx = upload(case)
    out = torch.empty((1, 256, 16, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(16, dq.prefill_workspace_bytes(16, 4, 16, 64, 128, 1, 256)),
                     dtype=torch.uint8, device="cuda")
    # Paged view of the same cache: 64-row pages in reverse order.
    n_pg = 2048 // 64
    perm = torch.arange(n_pg - 1, -1, -1, device="cuda")
    kp = k[0].view(4, n_pg, 64, 64).permute(1, 0, 2, 3)[perm.argsort()].contiguous()
    vp = v[0].view(16, n_pg, 64, 128).permute(1, 0, 2, 3)[perm.argsort()].contiguous()
    table = perm.to(torch.int32).view(1, n_pg)
    q_dec = q[:, -1].contiguous()
    p_out = torch.empty((1, 16, 128), dtype=torch.bfloat16, device="cuda")
    p_ws = torch.empty(dq.decode_workspace_bytes(16, 4, 16, 64, 128, 1, 2048), dtype=torch.uint8,
                       device="cuda")

    def work():
        dq.prefill(q, k, v, ctx, scale=case.scale, out=out, workspace=ws)
        dq.decode_paged(q_dec, kp, vp, table, ctx, max_ctx=2048, scale=case.scale, out=p_out,
                        workspace=p_ws)

    _say("graph: prefill + paged decode")
    work()
    torch.cuda.synchronize()
    want = [raw_host(t) for t in (out, p_out)]
    g = _capture(work)
    junk = torch.randn(1 << 20, device="cuda")
    _replay_and_check(g, [out, p_out], want, lambda: junk.mul_(1.0001).sum())
