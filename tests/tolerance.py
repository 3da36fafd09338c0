"""Element-wise comparison of a HIP result with the binary64 oracle.

Bound for each element (u = 2^-24, the binary32 unit roundoff):

    |gpu - ref| <= rtol * |ref| + (n_terms + slack) * u * S + atol

* rtol: 1e-5 for binary32 results, 2e-2 for half-precision results (fp32
  accumulation either way); it also absorbs the single rounding of a
  half-precision output (<= 2^-9 relative for bf16, 2^-11 for fp16).
* S: the oracle's sum of |terms| of this element, n_terms the number of terms.
  n_terms*u*S is the textbook bound for summing n_terms products in binary32
  in any order; `slack` (default 32) covers the few binary32 roundings inside
  each term: bilinear weights (2-3 multiplies), 1 - fraction, and for softmax
  the exponential and the normalisation.  This floor only matters where the
  terms cancel (|ref| much smaller than S).
* atol: 2^-24 for fp16 outputs, whose subnormal spacing is 2^-24.
Both sides form the sampling coordinates in the same binary32 order, so they
take the same floor() branch and no coordinate-rounding term is needed.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24
RTOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
ATOL = {"f32": 0.0, "f16": 2.0 ** -24, "bf16": 0.0}


# unit roundoff of the storage formats (a result rounded to one of them, or
# summed by atomics in it, carries this relative error per rounding)
U_STORE = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def bound(ref, S, n_terms, dtype, slack=32, store_roundings=0, atol=None):
    """store_roundings: how many times a partial sum of magnitude <= S may be
    rounded to the storage format besides the final rounding (half-precision
    atomics add that many).  atol overrides the dtype's absolute floor (for
    results that reach the subnormal range of binary32 or bfloat16, whose
    spacing there is 2^-149 and 2^-133)."""
    return (RTOL[dtype] * np.abs(ref) + (np.asarray(n_terms, np.float64) + slack) * U * S
            + (ATOL[dtype] if atol is None else atol) + store_roundings * U_STORE[dtype] * S)


def compare(gpu, ref, S, n_terms, dtype, slack=32, store_roundings=0, atol=None):
    """Returns a dict of statistics; 'ok' is True when every element is within bound."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    b = bound(ref, S, n_terms, dtype, slack, store_roundings, atol)
    err = np.abs(gpu - ref)
    finite = np.isfinite(gpu)
    ratio = np.where(b > 0, err / np.where(b > 0, b, 1.0), np.where(err > 0, np.inf, 0.0))
    nref = float(np.linalg.norm(ref.ravel()))
    out = dict(ok=bool(np.all(finite) and np.all(err <= b)),
               max_ratio=float(np.max(ratio)) if ratio.size else 0.0,
               norm_rel=float(np.linalg.norm((gpu - ref).ravel()) / nref) if nref > 0 else 0.0,
               n_bad=int(np.sum(~(err <= b))), n=int(err.size))
    if not out["ok"] and err.size:
        k = int(np.argmax(np.where(finite, ratio, np.inf)))
        out["worst"] = dict(index=np.unravel_index(k, err.shape), gpu=float(gpu.ravel()[k]),
                            ref=float(ref.ravel()[k]), bound=float(b.ravel()[k]))
    return out
