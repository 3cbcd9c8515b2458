"""GPU parity of the augmented-Q projection against the fp64 oracle.

The kernel rounds the gated intermediate to bf16 once (as the next product's
operand); the oracle keeps it exact, so the outputs are compared at the bf16
tolerance.  The intermediate itself is checked too (it is the workspace)."""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, to_dev, to_host

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


def intermediate(ws, M, d_i):
    """The gated intermediate from the workspace as [M][d_i]: up to 16 tokens
    the library keeps it chunk-major, [d_i / 8][M][8], beyond that row-major."""
    a = to_host(ws.view(torch.bfloat16)[:M * d_i])
    if M <= 16:
        return a.reshape(d_i // 8, M, 8).transpose(1, 0, 2).reshape(M, d_i)
    return a.reshape(M, d_i)


SHAPES = [
    # M, d_m, d_i, d_out
    (1, 1024, 1024, 256),
    (5, 2048, 3072, 2048),     # SIGMA-1.5B, a few decode tokens
    (12, 2048, 3072, 2048),    # the gate/up operand staged through LDS, rows 12-15 empty
    (16, 1024, 2048, 512),
    (17, 1024, 1024, 64),      # first size that takes 64-row workgroups
    (64, 1024, 2048, 128),     # last size on the 64-row workgroups
    (65, 1024, 1024, 64),      # first size on the LDS-tiled product, one ragged tile
    (200, 2048, 3072, 2048),   # LDS-tiled: a full 128-row tile and a ragged tail
    (300, 1024, 2048, 192),    # three row tiles, three 64-column down tiles
    (130, 1024, 1024, 80),     # d_out not a multiple of 64: the down product stays untiled
    (1100, 1024, 3072, 256),   # eight-wave tiles for both products, ragged last row tile
    (1030, 1024, 1024, 128),   # d_i not a multiple of 96: four-wave gate/up, eight-wave down
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_augq_matches_oracle(shape):
    M, d_m, d_i, d_out = shape
    case = synth.make_augq(501, M=M, d_m=d_m, d_i=d_i, d_out=d_out)
    _say("augq", shape)
    h = to_dev(case.h, "bf16")
    wg, wu, wd = (dq.augq_pack(to_dev(x, "bf16")) for x in (case.w_gate, case.w_up, case.w_down))
    ws = torch.empty(M * d_i * 2, dtype=torch.uint8, device="cuda")
    q = dq.augq(h, wg, wu, wd, workspace=ws)
    torch.cuda.synchronize()
    ref_q, ref_a = oracle.augq(*case.widened())
    act = intermediate(ws, M, d_i)
    err_a = assert_close(act, ref_a, "bf16", f"augq intermediate {shape}")
    err_q = assert_close(to_host(q), ref_q, "bf16", f"augq {shape}")
    _say(f"  normwise rel err: intermediate {err_a:.2e}, q {err_q:.2e}")


def test_augq_pack_is_the_fragment_permutation():
    # Unpacking with the documented element map restores the weight bit for
    # bit (the pack moves every element once and nowhere else).
    w = synth.normal(503, 1, (48, 96), "bf16")
    wp = dq.augq_pack(to_dev(w, "bf16"))
    torch.cuda.synchronize()
    p = wp.view(torch.int16).cpu().numpy().view(np.uint16)
    assert p.shape == (3, 3, 64, 8)
    back = np.zeros_like(w)
    for nb in range(3):
        for kb in range(3):
            for lane in range(64):
                r, k = 16 * nb + lane % 16, 32 * kb + 8 * (lane // 16)
                back[r, k:k + 8] = p[nb, kb, lane]
    np.testing.assert_array_equal(back, w)


def test_augq_rows_are_independent():
    # Each token's query depends on that token alone: the 64-row path equals
    # the single-row path row by row, bit for bit.
    case = synth.make_augq(502, M=40, d_m=1024, d_i=1024, d_out=128)
    h = to_dev(case.h, "bf16")
    wg, wu, wd = (dq.augq_pack(to_dev(x, "bf16")) for x in (case.w_gate, case.w_up, case.w_down))
    q_all = dq.augq(h, wg, wu, wd)
    q_one = torch.cat([dq.augq(h[r:r + 1].contiguous(), wg, wu, wd) for r in (0, 17, 39)])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q_all[[0, 17, 39]].view(torch.int16).cpu().numpy(),
                                  q_one.view(torch.int16).cpu().numpy())


def test_augq_tiled_rows_do_not_depend_on_the_batch():
    # On the LDS-tiled path a row's result depends on that row alone: the
    # first 130 rows of a 260-row call equal a 130-row call bit for bit
    # (same tile positions, different tile count and tail).
    case = synth.make_augq(504, M=260, d_m=1024, d_i=2048, d_out=256)
    h = to_dev(case.h, "bf16")
    wg, wu, wd = (dq.augq_pack(to_dev(x, "bf16")) for x in (case.w_gate, case.w_up, case.w_down))
    q_all = dq.augq(h, wg, wu, wd)
    q_part = dq.augq(h[:130].contiguous(), wg, wu, wd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q_all[:130].view(torch.int16).cpu().numpy(),
                                  q_part.view(torch.int16).cpu().numpy())
    ref_q, _ = oracle.augq(*case.widened())
    assert_close(to_host(q_all), ref_q, "bf16", "augq 260 rows")



def test_augq_full_size_every_row():
    # The SIGMA-1.5B shape at 2048 tokens, in the configuration the benchmark
    # times (eight-wave tiled products): every row against the oracle.
    sh = synth.AUGQ_SIGMA15B
    case = synth.make_augq(7, M=2048, **sh)
    h = to_dev(case.h, "bf16")
    wg, wu, wd = (dq.augq_pack(to_dev(x, "bf16")) for x in (case.w_gate, case.w_up, case.w_down))
    q = dq.augq(h, wg, wu, wd)
    torch.cuda.synchronize()
    ref_q, _ = oracle.augq(*case.widened())
    err = assert_close(to_host(q), ref_q, "bf16", "augq 2048 tokens, every row")
    _say(f"  normwise rel err (all 2048 rows): {err:.2e}")
