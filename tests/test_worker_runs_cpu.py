"""The split of a worker-fastest launch into runs of workers
(error_compensated_bit_02_amd/csrc/worker_runs.h): the runs cover the
worker range once, in ascending order, and each run's grid fits the limit.
Large worker counts on large lists take this path; no GPU test list reaches
it, so the arithmetic is checked here on the host."""
import os
import shutil
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "error_compensated_bit_02_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include "worker_runs.h"
int main() {
  long long w0, w1, chunks, max_grid;
  while (std::scanf("%lld %lld %lld %lld", &w0, &w1, &chunks, &max_grid) == 4) {
    ob::worker_runs(static_cast<int>(w0), static_cast<int>(w1), chunks, max_grid,
                    [](int b0, int b1) { std::printf("%d %d\n", b0, b1); });
    std::printf("end\n");
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("worker_runs")
    src, exe = d / "driver.cpp", d / "driver"
    src.write_text(DRIVER)
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return str(exe)


def _runs(driver, cases):
    text = "".join(f"{w0} {w1} {c} {m}\n" for w0, w1, c, m in cases)
    out = subprocess.run([driver], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
    result, cur = [], []
    for line in out:
        if line == "end":
            result.append(cur)
            cur = []
        elif line:
            b0, b1 = map(int, line.split())
            cur.append((b0, b1))
    return result


def test_runs_cover_the_range_in_order_within_the_limit(driver):
    max_grid = 0xFFFFFFFF // 256   # the library's grid limit in workgroups of 256
    cases = []
    for w0, w1 in [(0, 1), (0, 8), (3, 17), (0, 4096), (100, 4096), (5, 5)]:
        for chunks in [1, 7, 8 * 41_000, 8 * 160_215, max_grid // 200, max_grid // 2 + 1, max_grid]:
            cases.append((w0, w1, chunks, max_grid))
    for w0 in range(0, 6):            # small limits, every shape
        for w1 in range(w0, 12):
            for chunks in range(1, 9):
                for m in range(chunks, 3 * chunks + 2):
                    cases.append((w0, w1, chunks, m))
    for (w0, w1, chunks, m), runs in zip(cases, _runs(driver, cases)):
        got = [w for b0, b1 in runs for w in range(b0, b1)]
        assert got == list(range(w0, w1)), (w0, w1, chunks, m, runs)
        assert all(b1 > b0 and chunks * (b1 - b0) <= m for b0, b1 in runs), (w0, w1, chunks, m, runs)
        # as few launches as the limit allows
        per = m // chunks
        assert len(runs) == (-(-(w1 - w0) // per) if w1 > w0 else 0), (w0, w1, chunks, m, runs)
