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


JOIN_DRIVER = r"""
#include "kda_stage_plan.h"
#include <cstdio>
int main()
{
    int launched, recorded, capturing;
    while (std::scanf("%d %d %d", &launched, &recorded, &capturing) == 3) {
        const kda::StageJoin j = kda::plan_join(launched, recorded, capturing != 0);
        std::printf("%d %d\n", j.wait_stage, j.sync_side ? 1 : 0);
    }
    return 0;
}
"""


def test_join_after_failures(tmp_path):
    """The join at the end of a staged call: the calling stream waits on the
    last recorded pass-2 event; when a stage was enqueued on the second stream
    but its event failed to record, the second stream is drained on the host
    (outside a capture) so nothing of the call outlives it unordered."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    src, exe = tmp_path / "join.cpp", tmp_path / "join"
    src.write_text(JOIN_DRIVER)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    cases = [
        (-1, -1, 0, (-1, 0)),   # nothing reached the second stream
        (-1, -1, 1, (-1, 0)),
        (3, 3, 0, (3, 0)),      # every stage recorded: wait on the last
        (3, 3, 1, (3, 0)),
        (0, -1, 0, (-1, 1)),    # stage 0 enqueued, its event failed: drain
        (2, 1, 0, (1, 1)),      # stage 2's event failed: wait on stage 1 and drain
        (2, 1, 1, (1, 0)),      # under capture: no host synchronisation
    ]
    text = "".join("%d %d %d\n" % c[:3] for c in cases)
    out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    for c, line in zip(cases, out):
        assert tuple(int(x) for x in line.split()) == c[3], (c, line)


SEG_DRIVER = r"""
#include "kda_stage_plan.h"
#include <cstdio>
int main()
{
    std::printf("%d %d %d %d\n", kda::kMaxSegments, kda::kMinSegChunks, kda::kMaxSegChains, kda::kSegBudget);
    int nck, chains, cus, paired;
    while (std::scanf("%d %d %d %d", &nck, &chains, &cus, &paired) == 4)
        std::printf("%d\n", kda::plan_segments(nck, chains, cus, paired != 0));
    return 0;
}
"""


def test_segment_plan(tmp_path):
    """Segments of the sequential pass: phase C's 2 * chains * P workgroups
    fit the CUs one per CU and phase A's 2 * chains * (2P - 3) two per CU
    (paired) or one per CU, every segment has at least the minimum number of
    chunks, P * chains stays within the budget the workspace reserves for,
    P is the largest such count up to the cap, and 1 (no segments) wherever
    fewer than 3 segments fit.  On 256 CUs the 64K-token, 16-head prefill
    takes 8 segments paired and 5 unpaired; one or four chains of 4096 chunks
    take 32."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    src, exe = tmp_path / "seg.cpp", tmp_path / "seg"
    src.write_text(SEG_DRIVER)
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    cases = [(nck, chains, cus, paired) for nck in (1, 47, 48, 64, 95, 96, 100, 160, 200, 512, 1024, 4096)
             for chains in (1, 2, 3, 4, 8, 12, 16, 24, 32, 42, 43, 96) for cus in (80, 256, 304, 1024)
             for paired in (0, 1)]
    text = "".join("%d %d %d %d\n" % c for c in cases)
    out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    pmax, minc, maxch, budget = (int(x) for x in out[0].split())

    def fits(p, nck, chains, cus, paired):
        return (p <= pmax and p * chains <= budget and nck // p >= minc and 2 * chains * p <= cus and
                2 * chains * (2 * p - 3) <= (2 * cus if paired else cus))

    for (nck, chains, cus, paired), line in zip(cases, out[1:]):
        p = int(line)
        if p == 1:
            assert chains > maxch or not fits(3, nck, chains, cus, paired), (nck, chains, cus, paired)
        else:
            assert p >= 3 and fits(p, nck, chains, cus, paired), (nck, chains, cus, paired, p)
            assert not fits(p + 1, nck, chains, cus, paired), (nck, chains, cus, paired, p)
    got = dict(zip(cases, (int(x) for x in out[1:])))
    assert got[(1024, 16, 256, 1)] == 8 and got[(1024, 16, 256, 0)] == 5
    assert got[(64, 32, 256, 1)] == 4 and got[(64, 32, 256, 0)] == 3
    assert got[(1024, 96, 256, 1)] == 1 and got[(47, 1, 256, 1)] == 1 and got[(1024, 43, 256, 1)] == 1
    assert got[(4096, 1, 256, 1)] == 32 and got[(4096, 4, 256, 1)] == 32 and got[(1024, 8, 256, 1)] == 16
    assert got[(1024, 12, 256, 1)] == 10 and got[(4096, 1, 1024, 1)] == 32 and got[(4096, 8, 1024, 1)] == 16
