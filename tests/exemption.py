"""The near-threshold exemption of the parity contract (no GPU, no torch).

Two implementations of the quantizer that agree on the updated state S' and
the scales must produce the same codes, except possibly where the exact
pre-rounding value lies within NEAR code units (1e-6 of a scale step) of a
point where the code changes; there a one-code difference is accepted, and
the count of such elements must stay below RATE of all checked elements.
The distance per element is the reference's (oracle threshold distance)."""

from __future__ import annotations

import numpy as np

NEAR = 1e-6
RATE = 1e-5


class ParityError(AssertionError):
    pass


def classify(gpu_codes: np.ndarray, ref_codes: np.ndarray, tdist: np.ndarray, where: str = ""):
    """Indices of the elements whose codes differ, all of them exempt; raises
    ParityError if any differing element is not exempt (more than one code
    apart, or at least NEAR from its threshold)."""
    a = np.asarray(gpu_codes).ravel()
    r = np.asarray(ref_codes).ravel()
    d = np.asarray(tdist, dtype=np.float64).ravel()
    assert a.shape == r.shape == d.shape
    bad = np.nonzero(a != r)[0]
    if bad.size == 0:
        return bad
    far = (d[bad] >= NEAR) | (np.abs(a[bad].astype(np.int64) - r[bad].astype(np.int64)) != 1)
    if np.any(far):
        i = bad[np.argmax(far)]
        raise ParityError(f"{where}: {bad.size} codes differ, element {i} gpu {a[i]} ref {r[i]} "
                          f"threshold distance {d[i]:.3g} code units")
    return bad


def check_rate(exempt: int, elements: int, where: str = ""):
    if exempt > RATE * elements:
        raise ParityError(f"{where}: {exempt} near-threshold exemptions in {elements} elements "
                          f"(limit {RATE:g} of them)")
