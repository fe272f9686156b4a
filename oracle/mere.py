"""Mean element-wise relative error (MERE).

Test infrastructure only (see the package docstring).

Source: [LoKA] section II-C ("Error Analysis"): the error of a low-precision
linear layer against a high-precision reference is the mean, over the M x N
outputs, of |out - ref| / |ref|.  The pages' formula is garbled in the
extraction; reading R10 takes the mean over the entries with ref != 0 (the
ratio is undefined elsewhere) and reports how many entries that is.  The
pages' reference was TF32; here it is the unquantized bf16 inputs taken
exactly in fp64 (forward.reference_forward).
"""

import numpy as np


def mere(out, ref):
    """Returns (MERE, number of entries with ref != 0)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sel = ref != 0
    n = int(sel.sum())
    if n == 0:
        return 0.0, 0
    return float(np.mean(np.abs(out[sel] - ref[sel]) / np.abs(ref[sel]))), n
