"""Grouped forward: independent blocks, each exactly the single forward.

Test infrastructure only (see the package docstring).

Source: [LoKA] section I (recommendation models combine wide ensembles of
small layers) and [GEM] "Expert Parallelism" (each rank holds one expert);
[GEM] "Generalized Dot-Product Attention" (tile lists precomputed on the
CPU) is how the GPU side schedules them, which does not change the result.
A grouped launch is a scheduling choice: each group's output is the single
forward of that group, so the oracle is just the list of forwards.
"""

from .forward import gemm_ln_forward


def grouped_forward(groups, eps=1e-5, recipe="row"):
    """groups: list of dicts with keys x, w, bias, gamma, beta (bf16 bit
    patterns; bias/gamma/beta may be None).  Returns one forward dict per group."""
    return [gemm_ln_forward(g["x"], g["w"], g.get("bias"), g.get("gamma"), g.get("beta"),
                            eps=eps, recipe=recipe) for g in groups]
