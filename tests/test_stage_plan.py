"""Host logic of the staged prefill (CPU only): the chunk stages chosen by
gated_delta_rule_fwd_amd/csrc/kda_stage_plan.h, compiled with the host C++
compiler into a small driver.  Checks that the stages partition the chunk
range, respect the stage count and minimum size, appear only where the
overlap can pay, follow the growth direction of the cost ratio, and that the
64K-token, 96-head prefill gets the four stages its kernel trace shows."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_fwd_amd", "csrc")

DRIVER = r"""
#include "kda_stage_plan.h"
#include <cstdio>
int main()
{
    int nck, chains, cus;
    while (std::scanf("%d %d %d", &nck, &chains, &cus) == 3) {
        int b[kda::kMaxStages + 1];
        const int n = kda::plan_stages(nck, chains, cus, b);
        std::printf("%d", n);
        for (int i = 0; i <= n; ++i) std::printf(" %d", b[i]);
        std::printf("\n");
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def plan(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("plan")
    src, exe = d / "plan.cpp", d / "plan"
    src.write_text(DRIVER)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)

    def run(cases):
        text = "".join("%d %d %d\n" % c for c in cases)
        out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
        res = []
        for line in out[:len(cases)]:
            v = [int(x) for x in line.split()]
            assert len(v) == v[0] + 2
            res.append(v[1:])
        return res
    return run


def _pays(nck, chains):
    return nck >= 256 and nck * chains >= 8192


def test_headline_plan(plan):
    # 64K tokens x 96 heads on 256 CUs: the stages of the committed kernel trace
    assert plan([(1024, 96, 256)]) == [[0, 657, 893, 978, 1024]]


def test_partition_and_limits(plan):
    cases = [(nck, ch, cus) for nck in (1, 63, 64, 255, 256, 257, 1000, 1024, 4219, 17188, 2 ** 20)
             for ch in (1, 2, 16, 32, 64, 96, 112, 120, 256, 4096) for cus in (256, 304, 80)]
    for (nck, ch, cus), b in zip(cases, plan(cases)):
        assert b[0] == 0 and b[-1] == nck, (nck, ch, cus, b)
        n = len(b) - 1
        assert 1 <= n <= 6, (nck, ch, cus, b)
        assert all(y > x for x, y in zip(b, b[1:])), (nck, ch, cus, b)
        idle = cus - 16 * ((ch + 7) // 8)
        if not _pays(nck, ch) or idle < 32:
            assert n == 1, (nck, ch, cus, b)
        if n > 1:
            assert min(y - x for x, y in zip(b, b[1:])) >= 16, (nck, ch, cus, b)


def test_stage_sizes_follow_the_cost_ratio(plan):
    # many chains on few idle CUs: pass 1 is slow there, so the stages shrink;
    # few chains on many idle CUs: the stages grow
    shrink, grow = plan([(1024, 96, 256), (1024, 16, 256)])
    s = [y - x for x, y in zip(shrink, shrink[1:])]
    g = [y - x for x, y in zip(grow, grow[1:])]
    assert all(a >= b for a, b in zip(s, s[1:-1])), s
    assert all(a <= b for a, b in zip(g, g[1:])), g
    assert s[0] > 512 and g[0] == 16
