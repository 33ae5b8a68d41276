"""Register budget of the attention kernels (CPU only: the compiler's
resource report, no GPU).

Every instance of fwd_mfma_kernel must fit two waves per SIMD with no VGPR
spills and no scratch memory: a spill inside the tile loop costs a scratch
round trip per step, and a spill anywhere makes every launch allocate
scratch.  The report comes from compiling each fwd_mfma_*.hip file with
-Rpass-analysis=kernel-resource-usage, with the library's own flags."""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from masked_bidirectional_attention_amd import build as B  # noqa: E402

SOURCES = sorted(f for f in os.listdir(B.CSRC) if f.startswith("fwd_mfma_") and f.endswith(".hip"))


def _report(src, tmpdir):
    obj = os.path.join(tmpdir, src + ".o")
    cmd = [B.HIPCC, *B.CFLAGS, "-c", os.path.join(B.CSRC, src), "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr


def _parse(text):
    """{kernel name: {field: value}} from the remarks of one compile."""
    out = {}
    for blk in text.split("Function Name: ")[1:]:
        name = blk.split()[0]
        if "fwd_mfma_kernel" not in name:
            continue
        vals = {}
        for key, pat in (("vgpr", r"VGPRs: (\d+)"), ("agpr", r"AGPRs: (\d+)"), ("vspill", r"VGPRs Spill: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"), ("occ", r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, blk)
            vals[key] = int(m.group(1)) if m else None
        out[name] = vals
    return out


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not available")
def test_attention_kernels_fit_two_waves_without_spills(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _report(s, str(tmp_path)), SOURCES))
    kernels = {}
    for t in texts:
        kernels.update(_parse(t))
    # 2 element types x 2 head dims x 4 mask kinds x (1 stream, 2 streams,
    # in-kernel K interleaved, in-kernel K half split)
    assert len(kernels) == 64, sorted(kernels)
    bad = {n: v for n, v in kernels.items()
           if v["vspill"] != 0 or v["scratch"] != 0 or v["occ"] is None or v["occ"] < 2}
    assert not bad, bad
