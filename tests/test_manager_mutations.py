"""The step-loop pins have teeth against the block manager: plausible
mistakes planted in a copy of csrc/pa_manager.cpp (no copy-on-write, a fork
that does not count its sharers, a block freed while still referenced, a
reversed copy pair, an off-by-one slot, a copy of the wrong block; in the
swap: ids not rewritten, a shared block moved twice, references left on the
source pool, reversed pairs) each make the managed-step check against dense
attention (tests/test_step_loop.py), the preemption program
(tests/test_swap.py) or a worked example of tests/test_manager.py fail.  The mutants are host-only
C++ built with g++ in a temporary directory; the package's source is never
changed.  No GPU."""
import ctypes
import os
import subprocess

import pytest

import workloads as W
from test_step_loop import run_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "paged_kv_cache_05_amd", "csrc", "pa_manager.cpp")

MUTATIONS = {
    "no-copy-on-write": ("if (m->dev.refcount[block] > 1) {  // shared: copy before writing",
                         "if (false) {"),
    "fork-without-count": ("for (int32_t b : copy.blocks) ++m->dev.refcount[b];",
                           "for (int32_t b : copy.blocks) (void)b;"),
    "free-while-shared": ("if (refcount[b] == 0) freed.push_back(b);", "freed.push_back(b);"),
    "reversed-copy-pair": ("copy_pairs[2 * pairs] = block;\n        copy_pairs[2 * pairs + 1] = fresh;",
                           "copy_pairs[2 * pairs] = fresh;\n        copy_pairs[2 * pairs + 1] = block;"),
    "slot-off-by-one": ("slots[i] = (int64_t)block * B + offset;",
                        "slots[i] = (int64_t)block * B + (offset + 1) % B;"),
    "copy-first-block": ("copy_pairs[2 * pairs] = block;",
                         "copy_pairs[2 * pairs] = q.blocks.front();"),
    "swap-keeps-old-ids": ("for (int32_t &b : q.blocks) b = moved[b];", "(void)moved;"),
    "swap-moves-shared-block-twice": ("if (refs[b]++ == 0) order.push_back(b);",
                                      "{ refs[b]++; order.push_back(b); }"),
    "swap-keeps-source-references": ("from.release(b, refs[b]);", "(void)from;"),
    "swap-reversed-pairs": ("pairs[2 * p] = b;\n      pairs[2 * p + 1] = t;",
                            "pairs[2 * p] = t;\n      pairs[2 * p + 1] = b;"),
}


def build(tmp, name=None):
    src = open(SOURCE).read()
    if name is not None:
        old, new = MUTATIONS[name]
        assert src.count(old) == 1, f"mutation {name!r} does not match pa_manager.cpp once"
        src = src.replace(old, new)
    path = os.path.join(tmp, "pa_manager_mutant.cpp")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmp, f"libmanager_{name or 'copy'}.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-I",
                    os.path.join(ROOT, "include"), "-o", lib, path], check=True)
    return ctypes.CDLL(lib)


class Bound:
    """The manager module with BlockManager bound to another build."""

    def __init__(self, M, lib):
        self.OutOfBlocks, self.PAError = M.OutOfBlocks, M.PAError
        self.BlockManager = lambda *a, **kw: M.BlockManager(*a, lib=lib, **kw)


PROGRAMS = [dict(dtype=W.F32, num_heads=2, head_dim=16, block_size=4),
            dict(dtype=W.F16, num_heads=2, head_dim=16, block_size=8, churn=0.9, seed=5)]


def caught(oracle, M, lib):
    import test_manager
    import test_swap
    found = []
    try:
        test_swap.test_preempted_run_equals_dense_and_unpressed_run(oracle, Bound(M, lib),
                                                                    test_swap.PROGRAMS[0])
    except Exception as e:  # noqa: BLE001
        found.append(f"preemption program: {type(e).__name__}")
    for i, kw in enumerate(PROGRAMS):
        try:
            run_oracle(oracle, Bound(M, lib), W.generation(**kw))
        except Exception as e:  # noqa: BLE001
            found.append(f"program {i}: {type(e).__name__}")
    for name in ("test_cow_worked_example", "test_sharing_diagram", "test_free_at_zero_and_reuse",
                 "test_swap_out_and_in_keep_sharing"):
        try:
            getattr(test_manager, name)(Bound(M, lib))
        except Exception as e:  # noqa: BLE001
            found.append(f"{name}: {type(e).__name__}")
    return found


@pytest.fixture(scope="module")
def M(pa):
    from paged_kv_cache_05_amd import manager
    return manager


def test_unmutated_copy_passes(tmp_path, oracle_lib, M):
    assert caught(oracle_lib, M, build(str(tmp_path))) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_manager_mistake_is_caught(tmp_path, oracle_lib, M, name):
    assert caught(oracle_lib, M, build(str(tmp_path), name)), f"{name!r} not caught"
