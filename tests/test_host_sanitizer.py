"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

tests/native/host_boundary.cpp drives every entry point down its host-only paths: seeded
sweeps of the config validation of the drafter, the batch and the target (edge values of
every field), the create refusals one defect at a time, every call on a NULL handle, and the
width controller over long schedules. It is linked with dflash.cpp and controller.cpp as
g++ compiles them with both sanitizers, which stop the run at the first report (an
out-of-bounds access, a use after free, a leak, a signed overflow, a bad shift or cast). The
HIP kernels are linked as the library's build compiles them, without sanitizers, and are
never launched. The controller's transcript is then replayed through the oracle's
controller, decision by decision.
"""
import os
import shutil
import subprocess

import pytest

from block_drafting_dflash_amd import build as B
from oracle.width_controller import WidthController

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "native", "host_boundary.cpp")
OUT = os.path.join(B.BUILD, "host_sanitize")
HIP_LIB = "/opt/rocm/lib"
SAN = ["-fsanitize=address,undefined", "-fsanitize=float-cast-overflow", "-fno-sanitize-recover=all"]
CXXFLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-D__HIP_PLATFORM_AMD__",
            "-I", "/opt/rocm/include", "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC, *SAN]
HOST_SOURCES = [os.path.join(B.CSRC, "dflash.cpp"), os.path.join(B.CSRC, "controller.cpp"), DRIVER]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(HIP_LIB, "libamdhip64.so")),
                                reason="needs g++ and the HIP runtime library")


def _newest_header() -> float:
    hs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith(".h")]
    return max(os.path.getmtime(h) for h in hs + [os.path.join(B.ROOT, "include", "dflash.h")])


def _kernel_objects():
    """The library build's kernel objects, recompiled where a source or header is newer."""
    objs = []
    newest = _newest_header()
    for src in B.SOURCES:
        if not src.endswith(".hip"):
            continue
        obj = os.path.join(B.BUILD, src + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < max(newest, os.path.getmtime(os.path.join(B.CSRC, src))):
            os.makedirs(B.BUILD, exist_ok=True)
            obj = B._compile(src)
        objs.append(obj)
    return objs


def _build_driver() -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run(["g++", *CXXFLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = os.path.join(OUT, "host_boundary")
    r = subprocess.run(["g++", *SAN, *objs, *_kernel_objects(), f"-L{HIP_LIB}", "-lamdhip64",
                        f"-Wl,-rpath,{HIP_LIB}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.fixture(scope="module")
def driver_run():
    exe = _build_driver()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    return r


def test_host_paths_run_clean_under_the_sanitizers(driver_run):
    r = driver_run
    err = r.stderr
    assert "runtime error" not in err and "AddressSanitizer" not in err and "LeakSanitizer" not in err, err[-4000:]
    assert r.returncode == 0, err[-4000:]
    last = r.stdout.strip().splitlines()[-1].split()
    assert last[0] == "checks" and int(last[1]) > 100000 and last[3] == "0", last
    print(err)


def test_controller_transcript_matches_the_oracle(driver_run):
    """Every round the sanitized controller ran, replayed through the oracle's controller: the
    same width asked for at every round, the same final incumbent, challenges and adoptions."""
    ctl, rounds, finals = {}, 0, 0
    for line in driver_run.stdout.splitlines():
        f = line.split()
        if f[0] == "C":
            ctl[int(f[1])] = WidthController(*(int(x) for x in f[2:6]))
        elif f[0] == "T":
            w = ctl[int(f[1])]
            block, committed, ms = int(f[2]), int(f[3]), float(f[4])
            assert w.width() == block, (f[1], rounds)
            w.record(block, committed, ms)
            rounds += 1
        elif f[0] == "F":
            w = ctl[int(f[1])]
            adopted = sum(1 for d in w.decisions if d[3])
            assert (w.incumbent, w.challenger, len(w.decisions), adopted) == tuple(int(x) for x in f[2:6]), line
            finals += 1
    assert finals == len(ctl) == 6 and rounds > 10000
    # the schedules reach both widths and both outcomes of a challenge
    assert any(sum(d[3] for d in w.decisions) > 0 for w in ctl.values())
    assert any(sum(not d[3] for d in w.decisions) > 0 for w in ctl.values())
