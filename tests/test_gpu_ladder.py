"""The ladder tool's own sampled check, run on the GPU.

Every record the measurement tool prints carries a check of sampled elements
of its result against float64 dot products on the host.  Here the tool runs
over the two small workloads and every rung, and each record must carry a
passing check (equality on the integer-valued workload); the tool's exit
status is non-zero if any record fails.
"""
from __future__ import annotations

import json

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_ladder_records_carry_passing_checks(capsys):
    from tiled_fp32_gemm_03_amd import ladder

    variants = "naive,tiled,tiled32,tiled32_pad,valu,prod,splitk,bf16,f16"
    print("case: ladder on square_256, square_1024_int", flush=True)
    rc = ladder.main(["--workloads", "square_256,square_1024_int", "--variants", variants,
                      "--reps", "2", "--warmup", "1"])
    out = capsys.readouterr().out
    recs = [json.loads(line) for line in out.splitlines() if line.startswith("{")]
    assert rc == 0
    assert len(recs) == 2 * len(variants.split(","))
    for r in recs:
        c = r["check"]
        assert c["pass"] and c["samples"] == 2052, r
        if r["workload"] == "square_1024_int":
            assert c["max_abs_err"] == 0.0, r
