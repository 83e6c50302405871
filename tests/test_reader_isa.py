"""Host-side check of the ordinary readers' staging wait (no GPU needed: hipcc compiles the
library to gfx950 assembly).

The ordinary and the routed readers copy the image columns into LDS with direct global-to-LDS
loads issued as inline assembly, issue their first weight loads, and then wait with an explicit
`s_waitcnt vmcnt(N)`: N must equal the number of vector-memory loads issued after the last
copy, since the counter retires in order (a smaller N only waits longer; a larger N would let
the wave read LDS before the copies land). N is derived in the source from the loads each step
issues; this test reads the compiled code of every reader instantiation and checks that the
compiler emitted exactly that many loads between the last copy and the wait.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "q8_activation_quant_amd", "csrc", "qimg.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "qimg.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-S", "--offload-device-only", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def kernels(asm_text, pattern):
    """{mangled name: list of instruction lines} of the kernels whose name matches."""
    res = {}
    for m in re.finditer(r"^(_Z\w*%s\w*):" % pattern, asm_text, flags=re.M):
        body = asm_text[m.end():]
        body = body[: body.find("s_endpgm")]
        res[m.group(1)] = [ln.strip() for ln in body.splitlines() if ln.strip() and not ln.strip().startswith(";")]
    return res


VMEM_LOAD = re.compile(r"^(buffer_load_|global_load_(?!lds))")


MARKER = "; routed staging copies issued"


def kernel_lines(asm_text, pattern):
    """Like kernels(), keeping the routed reader's marker comment."""
    res = {}
    for m in re.finditer(r"^(_Z\w*%s\w*):" % pattern, asm_text, flags=re.M):
        body = asm_text[m.end():]
        body = body[: body.find("s_endpgm")]
        res[m.group(1)] = [ln.strip() for ln in body.splitlines()
                           if ln.strip() and (not ln.strip().startswith(";") or ln.strip() == MARKER)]
    return res


def test_staging_wait_counts_the_loads_issued_after_the_copies(asm):
    ks = kernels(asm, "mmvq_tiled_kernel")
    assert len(ks) >= 16, "reader instantiations not found"
    routed = kernel_lines(asm, "mmvq_routed_kernel")
    assert routed, "routed reader not found"
    ks.update(routed)
    for name, lines in ks.items():
        copies = [i for i, ln in enumerate(lines) if ln.startswith("global_load_lds")]
        assert copies, name
        # the routed reader's copies sit in loops whose blocks the compiler may place after
        # the code that follows them; its marker stands after the last copy in program order
        marks = [i for i, ln in enumerate(lines) if ln == MARKER]
        last = marks[0] if marks else copies[-1]
        loads = 0
        for ln in lines[last + 1:]:
            if VMEM_LOAD.match(ln):
                loads += 1
            m = re.match(r"s_waitcnt vmcnt\((\d+)\)", ln)
            # the staging wait is the first one after the prologue's weight loads (a wait the
            # compiler places before any of them only waits longer)
            if m and int(m.group(1)) > 0 and loads > 0:
                assert int(m.group(1)) == loads, (
                    "%s: staging wait vmcnt(%s) but %d loads were issued after the last copy"
                    % (name, m.group(1), loads))
                break
        else:
            pytest.fail("%s: no staging wait after the copies" % name)
