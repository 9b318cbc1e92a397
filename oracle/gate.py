"""The parity gate between a GEMM result and the oracle (test infrastructure only).

Normalised error per output entry:
    err(i,j) = |C(i,j) - Cref(i,j)| / (D(i,j) + |beta * C_in(i,j)|)
with D = sum_k |a(i,k) b(k,j)| over the dequantised inputs.  A result passes when
    max err <= K * 2^-23 + u_out,
u_out being the unit roundoff of the output format (2^-24 fp32, 2^-11 fp16, 2^-8 bf16; the
fp8 path writes bf16).  K * 2^-23 is twice the first-order bound K*u_fp32 of any fp32
accumulation order; u_out covers the single final rounding.  The test is written as
`not (err <= tol)` so that NaN or Inf fails.  Where the denominator is zero (an all-zero row of
op(A) or column of op(B) with beta = 0) the entry must instead satisfy
|C - Cref| <= u_out * |Cref|.

"Rigel" (arXiv 2606.12765), section 3, names a per-dtype tolerance against a float64 reference
built from the same quantised bytes but prints no values; the bound above is the one this
implementation adopts.
"""
from __future__ import annotations

import dataclasses

import numpy as np

UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# max over x of d/dx [x Phi(x)] = Phi(sqrt 2) + sqrt 2 phi(sqrt 2)
GELU_MAX_SLOPE = 1.1289


def tolerance(K: int, c_type: str, roundings: int = 1) -> float:
    """K * 2^-23 + u_out.  With `roundings` = 2 (an unfused GEMM that rounds to the output type
    and then a separate bias+GELU pass that rounds again) the first rounding passes through
    GELU (slope <= 1.129) before the second: K * 2^-23 + (1 + 1.129) * u_out."""
    u = UNIT_ROUNDOFF[c_type]
    if roundings == 1:
        return K * 2.0 ** -23 + u
    return K * 2.0 ** -23 + (1.0 + GELU_MAX_SLOPE) * u


@dataclasses.dataclass
class GateResult:
    ok: bool
    max_err: float
    tol: float
    frac_of_tol: float
    argmax: tuple
    n_checked: int

    def __str__(self):
        return (f"max_err={self.max_err:.3e} tol={self.tol:.3e} "
                f"({100 * self.frac_of_tol:.1f}% of tol) at {self.argmax}, n={self.n_checked}, "
                f"{'PASS' if self.ok else 'FAIL'}")


def check(C: np.ndarray, Cref: np.ndarray, D: np.ndarray, tol: float, c_type: str,
          beta: float = 0.0, Cin: np.ndarray | None = None) -> GateResult:
    """Apply the gate to decoded results C (float64) against the oracle's Cref and D."""
    C = np.asarray(C, dtype=np.float64)
    denom = np.asarray(D, dtype=np.float64).copy()
    if beta != 0.0 and Cin is not None:
        denom = denom + np.abs(beta * np.asarray(Cin, dtype=np.float64))
    diff = np.abs(C - Cref)
    zero = denom == 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(zero, 0.0, diff / np.where(zero, 1.0, denom))
    err = np.where(np.isfinite(C), err, np.inf)
    zero_bad = zero & ~(diff <= UNIT_ROUNDOFF[c_type] * np.abs(Cref))
    err = np.where(zero_bad, np.inf, err)
    if err.size == 0:
        return GateResult(True, 0.0, tol, 0.0, (), 0)
    idx = int(np.argmax(np.where(np.isnan(err), np.inf, err)))
    max_err = float(err.reshape(-1)[idx])
    ok = bool(np.all(err <= tol))
    return GateResult(ok, max_err, tol, max_err / tol if tol > 0 else float("inf"),
                      tuple(int(x) for x in np.unravel_index(idx, err.shape)), int(err.size))
