"""The README's usage example compiles and every name it takes from the
binding exists (CPU; the GPU test runs it)."""
import re

import blockwise_fp8_zero_amd as bfz
from tests.test_gpu_readme import _example


def test_readme_example_names():
    src = _example()
    compile(src, "README.md", "exec")
    names = set(re.findall(r"\bbfz\.(\w+)", src))
    assert {"Plan", "AdamW", "pack_shard", "fold_adamw_fp8_step_unpack"} <= names
    missing = [n for n in sorted(names) if not hasattr(bfz, n)]
    assert not missing, missing
