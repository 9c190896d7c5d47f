"""Shared helpers of the tests: tolerance checks and tensor conversions."""
import re
import sys

import numpy as np

# Floating-point parity bar for every float output: relative Frobenius error
# <= 5e-3 and max |delta| <= 3e-2 * max |ref|.
REL_FRO = 5e-3
MAX_ABS_REL = 3e-2


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    d = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(d) / max(nref, 1e-30)
    mx = np.abs(d).max() if d.size else 0.0
    bound = MAX_ABS_REL * (np.abs(ref).max() if ref.size else 0.0)
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert mx <= bound + 1e-30, f"{what}: max |delta| {mx:.3e} > {bound:.3e}"
    return rel, mx


def header_symbols(path):
    """Function names declared in a C header (kos_*)."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kos_[a-z0-9_]+)\s*\(", src)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
