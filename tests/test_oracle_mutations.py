"""The pins have teeth: plausible mistakes planted in a copy of the oracle's C
source (a dropped token, a reversed offset, a transposed layout, a missing
scale, a wrong sign, a wrong operand, a missing normalisation, a shifted
index, a wrong exponent bias, swapped block/offset, half a copy, mirrored
heads; in the swap: only K, a missed offset, mirrored heads, only the first
pair; in the prefill: the query's own token left out, the cached prefix
ignored, the query row taken within its chunk) each make at least one pin of tests/test_oracle_pins.py fail.  The
mutants are built in a temporary directory on the CPU; oracle/oracle.c is
never changed.  No GPU."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins
import workloads as W

# (exact fragment of oracle.c, replacement) -- each must occur in the source.
MUTATIONS = {
    "drop-last-token": ("const int filled = (n - j * B < B) ? (n - j * B) : B;\n        for (int o = 0; o < filled; ++o) {\n            double dot",
                        "const int filled = (n - j * B < B) ? (n - j * B - 1) : B;\n        for (int o = 0; o < filled; ++o) {\n            double dot"),
    "reversed-offset": ("return ((block * H + head) * (int64_t)B + offset) * D + dim;",
                        "return ((block * H + head) * (int64_t)B + (B - 1 - offset)) * D + dim;"),
    "transposed-layout": ("return ((block * H + head) * (int64_t)B + offset) * D + dim;",
                          "return ((block * B + offset) * (int64_t)H + head) * D + dim;"),
    "missing-scale": ("s[j * B + o] = scale * dot;", "s[j * B + o] = dot;"),
    "wrong-sign": ("z += exp(s[t] - m);", "z += exp(m - s[t]);"),
    "v-from-k-pool": ("out[d] += w * load_elem(v_pool,", "out[d] += w * load_elem(k_pool,"),
    "unnormalised": ("const double w = exp(s[j * B + o] - m) / z;",
                     "const double w = exp(s[j * B + o] - m);"),
    "shifted-table-index": ("const int32_t p = block_tables[(int64_t)b * MB + j];",
                            "const int32_t p = block_tables[(int64_t)b * MB + (j + 1) % nblk];"),
    "half-exponent-bias": ("v = ldexp((double)(1024 + frac), expo - 25);",
                           "v = ldexp((double)(1024 + frac), expo - 24);"),
    "swapped-block-offset": ("const int64_t block = slot / B;\n        const int offset = (int)(slot % B);",
                             "const int64_t block = slot % B;\n        const int offset = (int)(slot / B);"),
    "copy-k-only": ("memcpy((char *)v_pool + dst * block_bytes, (const char *)v_pool + src * block_bytes, block_bytes);",
                    ";"),
    "mirrored-heads-in-write": ("const int64_t src = ((int64_t)i * H + h) * D;",
                                "const int64_t src = ((int64_t)i * H + (H - 1 - h)) * D;"),
    "prefill-excludes-own-token": ("const int32_t visible = n - m + (row - query_start[b]) + 1;",
                                   "const int32_t visible = n - m + (row - query_start[b]);"),
    "prefill-ignores-prefix": ("const int32_t visible = n - m + (row - query_start[b]) + 1;",
                               "const int32_t visible = (row - query_start[b]) + 1;"),
    "prefill-query-row-in-chunk": ("(const char *)q + (int64_t)row * H * D * elem_bytes(dtype),",
                                   "(const char *)q + (int64_t)(row - query_start[b]) * H * D * elem_bytes(dtype),"),
    "swap-k-only": ("memcpy((char *)dst_v + to * es, (const char *)src_v + from * es, es);", ";"),
    "swap-misses-last-offset": ("            for (int o = 0; o < B; ++o)\n                for (int d = 0; d < D; ++d) {\n                    const int64_t from",
                                "            for (int o = 0; o < B - 1; ++o)\n                for (int d = 0; d < D; ++d) {\n                    const int64_t from"),
    "swap-mirrored-heads": ("const int64_t from = pool_index(src, h, o, d, H, B, D);",
                            "const int64_t from = pool_index(src, H - 1 - h, o, d, H, B, D);"),
    "swap-first-pair-only": ("    for (int i = 0; i < num_pairs; ++i) {\n        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];\n        for (int h",
                             "    for (int i = 0; i < 1 && i < num_pairs; ++i) {\n        const int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];\n        for (int h"),
}

# The pins, each run against a mutant; any AssertionError or oracle error
# counts as the pin catching it.
PINS = {
    "half-decoder": lambda o: pins.test_half_decoder_exhaustive(o),
    "dense-tiny": lambda o: pins.test_dense_attention_after_gather(o, lambda: W.tiny_fp32()),
    "dense-short-b8": lambda o: pins.test_dense_attention_after_gather(
        o, lambda: W.short_rows(block_size=8, num_seqs=8, num_heads=2)),
    "decimal": lambda o: [pins.test_decimal_brute_force(o, s) for s in range(6)],
    "one-token": lambda o: pins.test_single_token_returns_v_exactly(o),
    "weights": lambda o: pins.test_weights_sum_to_one(o),
    "two-tokens": lambda o: pins.test_two_tokens_logistic(o),
    "translation": lambda o: [pins.test_translation_matches_append_process(o, B) for B in (4, 16)],
    "cow-example": lambda o: pins.test_cow_worked_example(o),
    "step-tiny": lambda o: pins.test_step_reproduces_placement(o, lambda: W.tiny_fp32()),
    "write-read-back": lambda o: pins.test_write_then_read_back(o),
    "sharing-diagram": lambda o: pins.test_sharing_diagram(o),
    "prefill-sdpa": lambda o: [pins.test_prefill_equals_causal_sdpa(o, c) for c in range(3)],
    "prefill-one-token": lambda o: pins.test_prefill_of_one_token_is_decode(o),
    "swap-round-trip": lambda o: pins.test_swap_round_trip_leaves_decode_unchanged(o),
    "swap-block-slices": lambda o: pins.test_swap_equals_whole_block_slices(o),
    "swap-is-copy-in-one-pool": lambda o: pins.test_swap_within_one_pool_is_copy_blocks(o),
}


def build_mutant(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation {name!r} does not match oracle.c exactly once"
    path = os.path.join(tmp_path, "oracle_mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp_path, f"liboracle_{name}.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lib, path,
                    "-lm"], check=True)
    return oracle.Oracle(lib)


def caught_by(mutant):
    caught = []
    for name, pin in PINS.items():
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, oracle.OracleError):
            caught.append(name)
    return caught


def test_unmutated_source_passes_every_pin(tmp_path):
    src = open(oracle.SOURCE).read()
    path = os.path.join(tmp_path, "oracle_copy.c")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmp_path, "liboracle_copy.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lib, path,
                    "-lm"], check=True)
    assert caught_by(oracle.Oracle(lib)) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(tmp_path, name):
    caught = caught_by(build_mutant(str(tmp_path), name))
    assert caught, f"no pin caught the planted mistake {name!r}"
