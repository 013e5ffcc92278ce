"""Host logic of the launch splitting (fa_internal.h, `launch_by_heads`), on the CPU.

The kernels take a 1-D grid of tiles x heads, and a dispatch counts each grid dimension in
32-bit work-items, so a grid past 2^32 - 1 work-items goes out as several launches over
consecutive heads. This compiles the header's helper into a small host program whose
launcher only prints each grid and head range (and whose `hipGetLastError` is a stub), and
checks, for shapes up to the front end's limits: the launches cover every head once, in
order; each fits a dispatch; no more launches than needed; a launch error stops the loop
and is returned; a single head too large for one dispatch is refused without a launch.
"""
import os
import shutil
import subprocess

import pytest

from exact_io_aware_46_amd import build as fabuild

LIMIT = 2 ** 32 - 1
PROGRAM = r"""
#include "fa_internal.h"
#include <cstdio>
#include <cstdlib>
static hipError_t g_err = hipSuccess;
extern "C" hipError_t hipGetLastError() { return g_err; }
int main(int argc, char** argv) {
  fa::BwdParams p{};
  p.B = atoi(argv[1]);
  p.H = atoi(argv[2]);
  const long long tiles = atoll(argv[3]);
  const int threads = atoi(argv[4]);
  g_err = (hipError_t)atoi(argv[5]);
  const hipError_t e = fa::launch_by_heads(p, tiles, threads, [&](dim3 g, const fa::BwdParams& q) {
    printf("launch %u %u %u %d %d\n", g.x, g.y, g.z, q.bh0, q.nbh);
  });
  printf("rc %d\n", (int)e);
  return 0;
}
"""


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    cxx = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(cxx):
        cxx = shutil.which("clang++")
    if cxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no clang++ or HIP headers")
    d = tmp_path_factory.mktemp("launch_split")
    src, exe = d / "t.cpp", d / "t"
    src.write_text(PROGRAM)
    r = subprocess.run([cxx, "-std=c++17", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", f"-I{fabuild.CSRC}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return str(exe)


def run(prog, B, H, tiles, threads, err=0):
    out = subprocess.run([prog, str(B), str(H), str(tiles), str(threads), str(err)],
                         capture_output=True, text=True, check=True).stdout.split("\n")
    launches = [tuple(int(x) for x in l.split()[1:]) for l in out if l.startswith("launch")]
    rc = int([l for l in out if l.startswith("rc")][0].split()[1])
    return launches, rc


@pytest.mark.parametrize("B,H,tiles,threads", [
    (1, 16, 64, 512),                # the long causal workload's forward: one launch
    (4097, 4096, 1, 512),            # 2^24 + 2^12 heads of one tile: three launches
    (4097, 4096, 1, 256),            # two launches
    (1, 128, 65536, 512),            # 2^31 - 128 rows at d = 8: heads 0..126, then 127
    (1, 1, (1 << 28) // 256, 512),   # the longest head the front end accepts (d = 8)
    (2147483647, 1, 1, 512),         # the most heads: 2^31 - 1 of one tile
    (65535, 32767, 1, 256),
])
def test_launches_cover_every_head_once_and_fit_a_dispatch(prog, B, H, tiles, threads):
    launches, rc = run(prog, B, H, tiles, threads)
    assert rc == 0
    bh = B * H
    per = LIMIT // (tiles * threads)
    assert len(launches) == -(-bh // per)                 # no more launches than needed
    nxt = 0
    for gx, gy, gz, bh0, nbh in launches:
        assert (gy, gz) == (1, 1)
        assert bh0 == nxt and 1 <= nbh <= per
        assert gx == tiles * nbh
        assert gx * threads <= LIMIT
        nxt = bh0 + nbh
    assert nxt == bh


def test_a_launch_error_stops_the_loop_and_is_returned(prog):
    launches, rc = run(prog, 4097, 4096, 1, 512, err=98)
    assert rc == 98
    assert len(launches) == 1


def test_a_head_too_large_for_one_dispatch_is_refused_without_a_launch(prog):
    launches, rc = run(prog, 1, 1, (1 << 32) // 256, 512)   # 2^32 work-items for one head
    assert launches == [] and rc != 0
