"""The kernel variants bench.py times fit their registers: no VGPR spills
(scratch traffic would add HBM bytes and time that no other check sees,
since the results stay correct).  Reads the per-kernel resource table the
build writes (the compiler's resource remarks for every kernel)."""

import csv
import os

import pytest

TABLE = os.path.join(os.path.dirname(__file__), "..", "fp8_precision_gemm_amd", "_build", "resource_usage.tsv")

# workload -> kernels its timed launches run
TIMED = {
    "rowwise forward 16384x512x512": ["loka::fwd::k_fwd_xl<1, 4, 4, false, true>"],
    "tensor forward 512x256x256": ["loka::fwd::k_fwd_xl<0, 2, 2, false, false>"],
    "MX forward 65536x1024x256": ["loka::fwd::k_fwd_res<3, 2, 8, false, true>"],
    "BlockNorm forward": ["loka::fwd::k_fwd_bn<4, 4, false, true>"],
    "square-block forward 16384x512x512": ["loka::fwd::k_fwd_res<4, 4, 4, false, true>"],
    "square-block X quantization": ["loka::k_cast_tile<0, 0, 5, 0>"],
    "backward 16384x512x512": ["loka::k_bwd_main<4, 4, 0, true, 8, false>", "loka::k_amax_col<0>",
                               "loka::k_col_scales_pair<0, 1>", "loka::k_cast_col_pair<0, 0, 1, 1>",
                               "loka::k_wgrad<false>", "loka::k_finalize_vectors"],
    "square-block backward 16384x512x512": ["loka::k_relayout_sq", "loka::k_bwd_main<4, 4, 0, true, 8, true>",
                                            "loka::k_wgrad<true>", "loka::k_finalize_vectors"],
    "grouped 64 x 8192": ["loka::fwd::k_grouped_mixed<false>"],
}


def load():
    if not os.path.exists(TABLE):
        pytest.skip("the library has not been built here (no resource table)")
    with open(TABLE) as f:
        return {row["kernel"]: row for row in csv.DictReader(f, delimiter="\t")}


@pytest.mark.parametrize("workload", sorted(TIMED))
def test_timed_kernels_do_not_spill(workload):
    table = load()
    for k in TIMED[workload]:
        assert k in table, f"{workload}: kernel {k} not in the build"
        spill = int(table[k]["VGPRs Spill"] or 0)
        assert spill == 0, f"{workload}: {k} spills {spill} VGPRs ({table[k]['VGPRs']} used)"


def test_table_covers_every_source():
    table = load()
    sources = {row["source"] for row in table.values()}
    for s in ("quant.hip", "fwd_row.hip", "fwd_mx.hip", "fwd_mxsq.hip", "fwd_tensor.hip", "fwd_blocknorm.hip",
              "gemm_bwd.hip", "grouped.hip", "probe.hip", "mere.hip"):
        assert s in sources, s
