"""Helpers for the GPU parity tests: move seeded host inputs to the device,
bring results back, and measure the error against the fp64 oracle."""

import numpy as np
import torch

import synth

# Tolerances: max normwise relative error max|gpu - ref| / max|ref| per output
# tensor, for fp32 inputs and for bf16 inputs with fp32 accumulation.
TOL = {"f32": 1e-5, "bf16": 2e-2}
# lse is an fp32 log-sum-exp of scores computed exactly from the inputs; its
# absolute error is bounded by fp32 rounding of scores of size ~|s|.
LSE_TOL = {"f32": 2e-5, "bf16": 2e-4}


def to_dev(a: np.ndarray, dtype: str):
    """Host array (float32, or uint16 bf16 bits) -> contiguous GPU tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda").contiguous()


def ints_to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def to_host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> float64 host array (bf16 widened exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)


def raw_host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> host array of its raw bits (uint16 for bf16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(case: synth.DecodeCase):
    return (to_dev(case.q, case.dtype), to_dev(case.k_cache, case.dtype),
            to_dev(case.v_cache, case.dtype), ints_to_dev(case.ctx_len))


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def assert_close(got, ref, dtype, what=""):
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    err = normwise_err(got, ref)
    assert err <= TOL[dtype], f"{what}: normwise rel err {err:.3e} > {TOL[dtype]:.0e}"
    return err


def assert_lse_close(got, ref, dtype, what=""):
    finite = np.isfinite(ref)
    assert (np.isneginf(got) == np.isneginf(ref)).all(), f"{what}: -inf pattern differs"
    if finite.any():
        err = float(np.abs(got[finite] - ref[finite]).max())
        assert err <= LSE_TOL[dtype], f"{what}: lse abs err {err:.3e}"
