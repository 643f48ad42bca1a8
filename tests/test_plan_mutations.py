"""The planner checks have teeth: plausible mistakes planted in a copy of
csrc/pa_plan.cpp (a long-item threshold that lists items twice, merge rows
missing two-partition sequences, sequences of a prefill plan in the wrong
order, split chunks sharing one workspace slot, a partition halved past a
batch that already fills the GPU, a dropped last partition) each make
tests/native/plan_check.cpp fail.  The mutants are built with g++ in a
temporary directory; the package's source is never changed.  No GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_05_amd", "csrc")
SOURCE = os.path.join(CSRC, "pa_plan.cpp")
CHECKER = os.path.join(ROOT, "tests", "native", "plan_check.cpp")

MUTATIONS = {
    "long-threshold-inclusive": ("if ((long long)e[i].tokens > long_item) tmp[n_long++]",
                                 "if ((long long)e[i].tokens >= long_item) tmp[n_long++]"),
    "merge-rows-miss-two-partitions": ("if (np > 1) merge_rows->item", "if (np > 2) merge_rows->item"),
    "prefill-sequence-order": ("seq_weight[a] > seq_weight[b] : sa < sb",
                               "seq_weight[a] > seq_weight[b] : sa > sb"),
    "split-chunks-share-a-slot": ("(slot + (uint32_t)c) << 8", "(slot) << 8"),
    "partition-halved-regardless": ("if (items >= kPlanTargetItems || next < kPlanMinPartition) break;",
                                    "if (next < kPlanMinPartition) break;"),
    "last-partition-dropped": ("const int np = c == 0 ? 1 : (c + part - 1) / part;\n    if (b > 0xffff",
                               "const int np = c == 0 ? 1 : c / part + (c < part);\n    if (b > 0xffff"),
}


def build_and_run(tmp, name):
    src = open(SOURCE).read()
    if name is not None:
        old, new = MUTATIONS[name]
        assert src.count(old) == 1, f"mutation {name!r} does not match pa_plan.cpp once"
        src = src.replace(old, new)
    path = os.path.join(tmp, "pa_plan.cpp")
    with open(path, "w") as f:
        f.write(src)
    shutil.copy(os.path.join(CSRC, "pa_plan.h"), tmp)
    exe = os.path.join(tmp, "plan_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", tmp, "-I", os.path.join(ROOT, "include"),
                    CHECKER, path, os.path.join(CSRC, "pa_manager.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return subprocess.run([exe, "1"], capture_output=True, text=True, timeout=300)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_unmutated_planners_pass(tmp_path):
    res = build_and_run(str(tmp_path), None)
    assert res.returncode == 0, res.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_planner_mistake_is_caught(tmp_path, name):
    res = build_and_run(str(tmp_path), name)
    assert res.returncode != 0 and "FAIL" in res.stderr, f"mutant {name} survived"
