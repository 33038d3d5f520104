"""Parity bounds of the GPU path against the oracle.  numpy only: the CPU
tests use the same checker to show that it rejects plausible wrong results.

Bounds (max-abs 1e-5 for fp32 storage, 2e-2 for bf16 storage on outputs of
unit scale) and how each is applied:

* Outputs, elementwise: fp32 ``|got - want| <= 1e-5``; bf16
  ``|got - want| <= 2e-2 * max(1, |want|)``.  Every bf16 rounding on the way
  (stored K/V, the probabilities fed to the second product, the output
  itself) is relative, so above unit scale the bound grows with |want|.
* Outputs, scale-aware (bf16, for workloads whose outputs are far below unit
  scale: an output over 2^20 keys of random values is ~1e-2): per row
  (token, head), the relative error of the row as a vector,
  ``||got - want||_2 <= 2e-2 * ||want||_2``.  Each bf16 rounding on the way
  (the stored K, hence the logits; the stored V; the probabilities fed to
  the second product; the output) perturbs a row by a random fraction of
  its own norm, about 4e-3 per element measured over the 8K workload.  A
  lost or mis-weighted part of the keys moves it by a sizeable fraction
  (about 0.25 for one of 16 splits of a 2^20-key decode) and fails.  An
  elementwise bound scaled to the row does not fit: it is set by the tail
  of 10^7 such noise samples (up to ~0.04 of the row's RMS on single
  elements), and a tolerance that admits that tail admits real mistakes.
* lse: absolute, ``1e-5`` (fp32) or ``2e-2`` (bf16).  lse is computed in
  fp32 either way; in bf16 it moves only through the rounding of the stored
  keys (about 1e-3 in the logits).
* FP8 matrix products (``check_p8``): the oracle computes the attention on
  the same quantised queries, keys and values, and bounds what rounding the
  softmax probabilities to E4M3 can move (``relattn_prefill_p8_bounds``):
  every output within that bound plus bf16 output rounding
  (``2^-8 |want| + 1e-4``), every lse within its bound plus 1e-4, and the
  root mean square of the errors, in units of the predicted spread, below 2.
"""

import numpy as np

TOL = {"fp32": 1e-5, "bf16": 2e-2}


def _arrays(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    return got, want


def _verdict(err, allowed, got, want, what):
    ratio = err / np.maximum(allowed, 1e-300)
    i = np.unravel_index(np.argmax(ratio), err.shape)
    assert ratio[i] <= 1.0, (f"{what}: err {err[i]:.3e} at {i} > allowed {allowed[i]:.3e} "
                             f"(got {got[i]}, want {want[i]})")
    return float(err.max())


def check_close(got, want, tol, what="", relative=False):
    """max |got - want| <= tol, or, with ``relative``, <= tol * max(1, |want|)."""
    got, want = _arrays(got, want)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - want)
    allowed = tol * np.maximum(1.0, np.abs(want)) if relative else np.full(err.shape, tol)
    return _verdict(err, allowed, got, want, what)


def check_out(got, want, dtype, what="out"):
    """Elementwise output bound of the storage dtype."""
    return check_close(got, want, TOL[dtype], what, relative=(dtype == "bf16"))


def row_rel_l2(got, want):
    """||got - want||_2 / ||want||_2 per row over the last axis."""
    got, want = _arrays(got, want)
    num = np.sqrt(np.sum((got - want) ** 2, axis=-1))
    den = np.sqrt(np.sum(want * want, axis=-1))
    return num / np.maximum(den, 1e-300)


def check_out_scaled(got, want, what="out"):
    """Scale-aware bf16 output bound: relative L2 error of every row (last
    axis) <= 2e-2.  Returns the largest row's relative error."""
    got, want = _arrays(got, want)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    rel = row_rel_l2(got, want)
    i = np.unravel_index(np.argmax(rel), rel.shape)
    assert rel[i] <= TOL["bf16"], (f"{what} (scale-aware): row {i} relative L2 error "
                                   f"{rel[i]:.3e} > {TOL['bf16']:.0e} (|want| "
                                   f"{np.sqrt(np.sum(want[i] ** 2)):.3e})")
    return float(rel[i])


def check_lse(got, want, dtype, what="lse"):
    """Absolute lse bound of the storage dtype."""
    return check_close(got, want, TOL[dtype], what, relative=False)


def check_attention(got_o, want_o, got_l, want_l, dtype, what="", scale_aware=False):
    """All bounds that apply to one attention result; returns the max errors
    (out, lse) and, with ``scale_aware`` (bf16), the largest row relative L2
    error as a third value."""
    e_o = check_out(got_o, want_o, dtype, what + " out")
    rel = None
    if scale_aware and dtype == "bf16":
        rel = check_out_scaled(got_o, want_o, what + " out")
    e_l = check_lse(got_l, want_l, dtype, what + " lse")
    if scale_aware:
        print(f"[parity] {what}: max |out err| {e_o:.3e}, max |lse err| {e_l:.3e}"
              + (f", max row relative L2 {rel:.3e}" if rel is not None else ""), flush=True)
    return (e_o, e_l) if rel is None else (e_o, e_l, rel)


def check_p8(got_o, got_l, exp, what="fp8 products"):
    """Bounds for FP8 matrix products; ``exp`` = the six arrays of
    ``oracle.relattn_prefill_p8_bounds`` (out, lse, bound_o, sigma_o,
    bound_l, sigma_l)."""
    o, l, bo, so, bl, sl = (np.asarray(x, dtype=np.float64) for x in exp)
    got_o, o = _arrays(got_o, o)
    got_l, l = _arrays(got_l, l)
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all(), f"{what}: non-finite values"
    err = got_o - o
    _verdict(np.abs(err), bo + 2.0 ** -8 * np.abs(o) + 1e-4, got_o, o, f"{what} out")
    z = err / (so + 2.0 ** -9 * np.abs(o) / np.sqrt(3.0) + 1e-6)
    rms = float(np.sqrt(np.mean(z ** 2)))
    assert rms < 2.0, f"{what}: output errors are {rms:.2f} predicted spreads (rms)"
    el = got_l - l
    _verdict(np.abs(el), bl + 1e-4, got_l, l, f"{what} lse")
    rmsl = float(np.sqrt(np.mean((el / (sl + 2e-5)) ** 2)))
    assert rmsl < 2.0, f"{what}: lse errors are {rmsl:.2f} predicted spreads (rms)"
    return rms, rmsl
