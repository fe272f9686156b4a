"""Recipe selection of the Dispatch runtime ([LoKA] section III-C, "Library
and Recipe Selection").

Test infrastructure only (see the package docstring).

The pages' rule, per GEMM operation: candidate implementations are first
filtered by accuracy (the expected error from the Probe's MERE analysis must
stay below a conservative threshold, typically MERE < 0.2) and by speed (the
speedup must exceed a minimum factor, typically 1.05x); from what remains the
one with the highest measured throughput is chosen.

Readings (reading R17):
  * speedup = baseline time / candidate time, with the high-precision path
    as the baseline; both comparisons are strict, as the pages write them;
  * "highest measured throughput" for one operation is the shortest time;
    equal times keep the earlier candidate;
  * when no candidate passes both filters the operation stays on the
    high-precision path (returned as -1);
  * a candidate whose MERE or time is not a finite number never passes.
"""

import math


def select(candidates, baseline_us, mere_max=0.2, min_speedup=1.05):
    """candidates: sequence of (time_us, mere).  Returns the chosen index, or
    -1 for the high-precision baseline."""
    best, best_us = -1, None
    for i, (us, mere) in enumerate(candidates):
        if not (math.isfinite(us) and math.isfinite(mere)) or us <= 0:
            continue
        if not mere < mere_max:
            continue
        if not baseline_us / us > min_speedup:
            continue
        if best_us is None or us < best_us:
            best, best_us = i, us
    return best
