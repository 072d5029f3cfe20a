"""Plants plausible mistakes in copies of the oracle's C source and checks that
the pins catch every one (so a passing pin set means something). CPU only;
the planted builds live in a temporary directory and are never used
elsewhere."""
import os

import pytest

import oracle
from oracle import build as oracle_build

import oracle_pins as P

# (name, exact text in msa_oracle.c, replacement)
MUTATIONS = [
    ("mask_off_by_one", "return p < seq_len && p <= pos;", "return p < seq_len && p < pos;"),
    ("normal_exponent", "(int64_t)(8 + mantissa) << (exponent - 1)",
     "(int64_t)(8 + mantissa) << exponent"),
    ("subnormal_as_normal", "magnitude_units = mantissa;", "magnitude_units = 8 + mantissa;"),
    ("dropped_sign", "        acc += prod;\n", "        acc += prod < 0 ? -prod : prod;\n"),
    ("max_becomes_min", "if (!*have || u > *best)", "if (!*have || u < *best)"),
    ("page_row_index", "((page * page_size) + (p % page_size))",
     "((page * page_size) + (p % ORACLE_BLOCK))"),
    ("unpadded_columns", "return (blocks + 3) / 4 * 4;", "return blocks;"),
    ("rounding_scale", "(float)ldexp((double)units, -18)", "(float)ldexp((double)units, -17)"),
    ("tie_break_reversed",
     "    if (a->score < b->score)\n        return 1;\n    return (a->id > b->id) - (a->id < b->id);",
     "    if (a->score < b->score)\n        return 1;\n    return (a->id < b->id) - (a->id > b->id);"),
    ("forced_end_off_by_one", "return id < init_blocks || id >= n - local_blocks;",
     "return id < init_blocks || id > n - local_blocks;"),
    ("range_width_floor", "return ((int64_t)cols + num_ranges - 1) / num_ranges;",
     "return (int64_t)cols / num_ranges;"),
    ("merge_budget", "ORACLE_TOPK - (int)expected_forced, cand",
     "ORACLE_TOPK - (int)expected_forced - 1, cand"),
    ("amax_signed", "acc_abs += prod < 0 ? -prod : prod;", "acc_abs += prod;"),
    ("ascending_by_score", "qsort(chosen, (size_t)m, sizeof(entry), id_cmp);",
     "qsort(chosen, (size_t)m, sizeof(entry), rank_cmp);"),
    # row-sharded scoring and the column -> global id mapping
    ("shard_rank_offset_dropped", "int64_t p = c * page_size + (int64_t)rank * rows + i;",
     "int64_t p = c * page_size + i;"),
    ("shard_key_row", "index_k_shard + (page * rows + i) * ORACLE_DIM",
     "index_k_shard + (page * rows + (rows - 1 - i)) * ORACLE_DIM"),
    ("sharded_columns_unpadded", "return (pages + 3) / 4 * 4;", "return pages;"),
    ("sharded_columns_in_blocks", "int64_t pages = (seq_len + page_size - 1) / page_size;",
     "int64_t pages = (seq_len + ORACLE_BLOCK - 1) / ORACLE_BLOCK;"),
    ("mapped_offset_dropped", "int64_t id = (int64_t)index_scale * c + index_offset;",
     "int64_t id = (int64_t)index_scale * c;"),
    # prefill chunks
    ("prefill_position_from_chunk_start", "int64_t pos = seq_len - q_len + j;",
     "int64_t pos = seq_len - q_len + j - 1;"),
    ("prefill_request_lookup", "while (qo_indptr[b + 1] <= t)", "while (qo_indptr[b + 1] < t)"),
    ("prefill_head_row", "index_q + (t * ORACLE_HEADS + h) * ORACLE_DIM",
     "index_q + (t * ORACLE_HEADS) * ORACLE_DIM"),
    ("mapped_forced_on_columns",
     "entry e = {srow[c], (int32_t)id};\n                    if (is_forced(id, n,",
     "entry e = {srow[c], (int32_t)id};\n                    if (is_forced(c, n,"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle_build.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation anchor for {name} not unique/absent"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(source.replace(old, new))
    lib = oracle_build.build(src=str(src), out=str(tmp_path / f"libmut_{name}.so"))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name}"
