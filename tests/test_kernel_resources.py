"""Compile-time resource check of every HIP kernel (no GPU needed): no kernel
may use scratch (private) memory.  Register arrays that the compiler fails
to keep in registers land in scratch and serialize the memory pipeline."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources():
    from prefill_gemm_amd import build
    return [s for s in build.sources() if s.endswith(".hip")]


@pytest.mark.parametrize("src", _sources(), ids=os.path.basename)
def test_no_scratch(src, tmp_path):
    from prefill_gemm_amd import build
    cmd = ["hipcc", "-x", "hip", *build.HIP_FLAGS, "-c", src, "-o", str(tmp_path / "k.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    names = re.findall(r"Function Name: (\S+)", out)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out)]
    assert names and len(names) == len(scratch)
    bad = [(n, s) for n, s in zip(names, scratch) if s]
    assert not bad, f"kernels using scratch: {bad}"
