"""Helpers for the GPU parity tests: move seeded host inputs to the device,
bring results back, and measure the error against the fp64 oracle."""

import numpy as np
import torch

import synth

# Tolerances: max normwise relative error max|gpu - ref| / max|ref| per output
# tensor, for fp32 inputs and for bf16 inputs with fp32 accumulation.
TOL = {"f32": 1e-5, "bf16": 2e-2}
# Regression bounds, well inside the contract, so that a kernel that loses a
# few bits fails a test even while it still meets TOL:
#  bf16: 4 * 2^-9.  One 2^-9 is the bf16 rounding of each output element
#  (round to nearest even: relative error <= 2^-9, so <= 2^-9 of the largest
#  element); up to three more cover the bf16 rounding of the weights that
#  enter fp32-accumulated products (the decode's probabilities, the prefill's
#  P tile, augmented Q's gated intermediate), each term off by <= 2^-9
#  relative, whose effect on an element grows where the weighted sum
#  cancels.  Measured: at most 4.7e-3 (the 70-row 32/4/16 prefill).
#  f32: 32 * 2^-24, for the hardware base-2 exponential (about one unit in
#  the last place), the rounding of scores of magnitude up to ~10 and the
#  fp32 accumulation.  Measured: at most 6.2e-7.
REGRESS_TOL = {"f32": 32 * 2.0 ** -24, "bf16": 4 * 2.0 ** -9}
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


def elementwise_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    """Element-wise error figures reported beside the normwise one: the
    largest and mean absolute error, and the largest relative error over the
    elements whose reference is at least a tenth of the largest (relative
    error is ill-posed for elements near zero)."""
    d = np.abs(got - ref)
    a = np.abs(ref)
    big = a >= 0.1 * a.max() if a.size else a
    rel = float((d[big] / a[big]).max()) if a.size and big.any() else 0.0
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "mean_abs": float(d.mean()) if d.size else 0.0,
            "max_rel_big": rel}


def assert_close(got, ref, dtype, what=""):
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    err = normwise_err(got, ref)
    st = elementwise_stats(got, ref)
    print(f"[err] {what}: normwise {err:.3e}, max abs {st['max_abs']:.3e}, "
          f"mean abs {st['mean_abs']:.3e}, max rel (|ref| >= max/10) {st['max_rel_big']:.3e}",
          flush=True)
    assert err <= TOL[dtype], f"{what}: normwise rel err {err:.3e} > {TOL[dtype]:.0e}"
    assert err <= REGRESS_TOL[dtype], (
        f"{what}: normwise rel err {err:.3e} meets the {TOL[dtype]:.0e} contract but exceeds "
        f"the regression bound {REGRESS_TOL[dtype]:.2e}")
    return err


def assert_lse_close(got, ref, dtype, what=""):
    finite = np.isfinite(ref)
    assert (np.isneginf(got) == np.isneginf(ref)).all(), f"{what}: -inf pattern differs"
    if finite.any():
        err = float(np.abs(got[finite] - ref[finite]).max())
        assert err <= LSE_TOL[dtype], f"{what}: lse abs err {err:.3e}"
