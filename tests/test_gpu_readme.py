"""The README's Python example runs as written (the code block under
"Use from Python"), and its merged rows equal the oracle's select + merge on
the plane it computed."""
from __future__ import annotations

import pathlib
import re

import pytest
import torch

import oracle
from parity import assert_rows_equal

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

README = pathlib.Path(__file__).resolve().parent.parent / "README.md"


def example_code() -> str:
    text = README.read_text()
    section = text.split("## Use from Python", 1)[1]
    m = re.search(r"```python\n(.*?)```", section, re.S)
    assert m, "no python block under 'Use from Python'"
    return m.group(1)


def test_readme_example_runs():
    env: dict = {}
    exec(compile(example_code(), str(README), "exec"), env)
    msa = env["msa"]
    plane = env["plane"].cpu().numpy()
    nvp = env["num_valid_pages"].numpy()
    rows = env["rows"].cpu()
    s, i, bad = oracle.top16_select(plane, nvp, init_blocks=1, local_blocks=2, num_ranges=2)
    assert bad == 0
    s, i, missing = oracle.top16_merge(s, i, nvp, init_blocks=1, local_blocks=2)
    assert missing == 0
    assert_rows_equal(msa.row_scores(rows).numpy(), msa.row_ids(rows).numpy(), s, i,
                      "README example vs oracle")
