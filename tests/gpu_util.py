"""Helpers shared by the GPU parity tests: conversions between torch device
tensors and the numpy arrays the oracle takes, and the tolerance checks.

Tolerances (written once here, used by every GPU test):
  * integer / index / byte outputs: bit-exact;
  * fp32 outputs: max |y - y_ref| <= 1e-4 * max(|y_ref|, RMS(y_ref)) elementwise;
  * bf16 outputs: max |y - y_ref| <= 2e-2 * RMS(y_ref);
  * FP8 outputs: max |y - y_ref| <= 5e-2 * RMS(y_ref) against the fp64 oracle
    of the same dequantised formula.
"""
import numpy as np
import torch

DEV = "cuda"


def np_of(t: torch.Tensor) -> np.ndarray:
    """Device/host tensor -> numpy array in the oracle's convention
    (float32 as float32, bf16 as uint16 bit patterns, ints/uint8 as is)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def f64_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rms(a) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def assert_bf16_close(got, ref, rel=2e-2, what="output"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s has non-finite values" % what
    err = np.abs(got - ref).max() if ref.size else 0.0
    tol = rel * rms(ref)
    assert err <= tol, "%s: max abs err %.3e > %.3e (= %g x RMS %.3e)" % (what, err, tol, rel,
                                                                          rms(ref))


def assert_f32_close(got, ref, rel=1e-4, what="output"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "%s has non-finite values" % what
    floor = np.maximum(np.abs(ref), rms(ref))
    bad = np.abs(got - ref) > rel * floor
    assert not bad.any(), "%s: %d elements off, worst rel err %.3e" % (
        what, int(bad.sum()), float((np.abs(got - ref) / floor).max()))


def offsets_from_sizes(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def sample_rows(offsets, per_group=3, seed=0):
    """A few rows from every non-empty group: first, last and random ones."""
    rng = np.random.default_rng(seed)
    out = []
    for g in range(len(offsets) - 1):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if b > a:
            pick = {a, b - 1}
            pick.update(rng.integers(a, b, size=max(per_group - 2, 0)).tolist())
            out.extend(sorted(pick))
    return np.array(out, dtype=np.int64)


# ----------------------------------------------------------------------------
# tolerances derived from the arithmetic, for single-kernel GEMM tests
# ----------------------------------------------------------------------------

U32 = 2.0 ** -24        # unit roundoff of binary32


def abs_bf16_bits(a):
    return (np.asarray(a, dtype=np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)


def abs_operand(a):
    """|a| for an oracle operand (fp32, bf16 bits or E4M3 codes)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return abs_bf16_bits(a)
    if a.dtype == np.uint8:
        return (a & np.uint8(0x7F)).astype(np.uint8)
    return np.abs(a)


def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu_bound(g, u, eg, eu, store_rel):
    """Elementwise bound on |h_gpu - h| for h = silu(g) u, given bounds eg,
    eu on the errors of g and u: |silu'| <= 1.1, a few roundings in the
    fp32 epilogue, and one rounding of the stored value (store_rel)."""
    h = silu(g) * u
    return (1.1 * np.abs(u) * eg + (np.abs(silu(g)) + 1.1 * eg) * eu
            + (8 * U32 + store_rel) * np.abs(h)), h


def assert_within(got, ref, bound, what="output"):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), "%s has non-finite values" % what
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), "%s: %d of %d elements outside the bound; worst excess %.3e" % (
        what, int(bad.sum()), bad.size, float((err - bound).max()))
