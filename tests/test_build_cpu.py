"""Sources that only the instrumented build compiles: the wall-clock marks of
csrc/gdn_timeline.h (GDN_TIMELINE) expand to code in every kernel that uses
them, and the product build compiles them to nothing, so a kernel that uses
the marks without declaring them (GDN_TL_BEGIN) would break only the
instrumented library.  A syntax-only device compile of each such source with
the marks on catches that here, in seconds, without a GPU.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_verify_gdn_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def marked_sources():
    return sorted(f for f in glob.glob(os.path.join(CSRC, "*.hip")) if "GDN_TL(" in open(f).read())


def test_some_sources_carry_marks():
    names = [os.path.basename(f) for f in marked_sources()]
    assert "gdn_step.hip" in names and "gdn_prefill_c64.hip" in names


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", [os.path.basename(f) for f in marked_sources()])
def test_instrumented_source_compiles(src):
    text = open(os.path.join(CSRC, src)).read()
    # every kernel that takes marks declares them and writes them out
    assert text.count("GDN_TL_BEGIN()") >= 1 and text.count("GDN_TL_END()") >= 1, src
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fsyntax-only", "-DGDN_TIMELINE",
                        "-I" + os.path.join(ROOT, "include"), os.path.join(CSRC, src)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
