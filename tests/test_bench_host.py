"""bench.py's host side: the CPU oracle baseline runs every stage of the step
on a sample of each workload (small batch and vocabulary), from probability
rows and, where the bench offers it, from logits."""
import pytest

import bench
import workloads


@pytest.mark.parametrize("name,logits", [("c1", False), ("c2", False), ("c2", True), ("c3", False), ("c4", False),
                                         ("c4", True), ("c5", False)])
def test_cpu_baseline_runs_every_stage(name, logits):
    over = {} if name == "c1" else {"B": 2}
    if name not in ("c1", "c5"):
        over["V"] = 3000                  # c5's vocabularies come with its intersection map
    cfg = workloads.get_config(name, **over)
    inp = workloads.generate(cfg, with_logits=logits)
    out = bench.cpu_baseline(cfg, inp, 1, threads=1, logits=logits)
    assert out["value"] > 0 and out["cores"] == 1 and out["kind"] == "oracle"
    assert out["unit"] == "verified draft tokens/s"
