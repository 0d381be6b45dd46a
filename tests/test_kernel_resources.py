"""Every gfx950 kernel of the library compiles without scratch memory (no register spills, no
private arrays left in memory): the compiler's resource-usage report for each HIP source, built
with the library's own flags.  CPU only (hipcc cross-compiles); skipped without hipcc."""
import pathlib
import re
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

from speculative_decoding_verification_specdec_amd import build as B  # noqa: E402

HIP_SOURCES = [p for p in B.SOURCES if p.suffix == ".hip"]


def _usage(src: pathlib.Path, tmp: pathlib.Path):
    flags = [f for f in B.FLAGS if f not in ("-shared",)]
    cmd = [B.hipcc(), *flags, f"-I{ROOT / 'include'}", "-c", str(src), "-o",
           str(tmp / (src.stem + ".o")), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None:
            kernels[name] = int(m.group(1))
    return kernels


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not pathlib.Path(B.hipcc()).exists(),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", HIP_SOURCES, ids=[p.name for p in HIP_SOURCES])
def test_no_kernel_uses_scratch(src, tmp_path):
    kernels = _usage(src, tmp_path)
    if src.name != "noalloc.hip":  # (that file holds the device scratch array and host code only)
        assert kernels, f"no kernel resource report for {src.name}"
    spilled = {k: v for k, v in kernels.items() if v != 0}
    assert not spilled, spilled
