"""Host-side layout helpers of the kernels, compiled for the CPU from
zero_kernels.h: the shift reduce's block order (shift_block) is a bijection on
[0, n) for every grid size, hands each XCD (workgroups b = x mod 8) consecutive
blocks in groups of G, and leaves a last, partial set of 8 groups in the plain
order; G is kRedShiftGroupRuns wave-runs for the kernel's shapes."""
import os
import shutil
import subprocess

from conftest import ROOT

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "zero_kernels.h"
template <unsigned G>
static int check() {
    const unsigned set = 8u * G;
    for (unsigned n = 1; n <= 5000; n += (n < 600 ? 1 : 37)) {
        std::vector<int> seen(n, 0);
        for (unsigned b = 0; b < n; ++b) {
            const unsigned m = zk::shift_block<G>(b, n);
            if (m >= n || seen[m]++) { std::printf("not a bijection G=%u n=%u b=%u\n", G, n, b); return 1; }
            const unsigned s0 = b - b % set;
            if (G > 1 && s0 + set <= n) {
                // within a full set, XCD b % 8 takes G consecutive blocks
                const unsigned j = b - s0;
                if (m != s0 + (j % 8u) * G + j / 8u) { std::printf("order G=%u n=%u b=%u\n", G, n, b); return 1; }
                if (b >= 8 && b - 8 >= s0 && zk::shift_block<G>(b - 8, n) + 1 != m) {
                    std::printf("not consecutive G=%u n=%u b=%u\n", G, n, b); return 1;
                }
            } else if (m != b) {
                std::printf("reordered G=%u n=%u b=%u\n", G, n, b); return 1;
            }
        }
    }
    return 0;
}
int main() {
    if (check<1>() || check<16>() || check<zk::shift_group<64, 2>()>() ||
        check<zk::shift_group<64, 1>()>())
        return 1;
    std::printf("ok %u %u %u\n", zk::shift_group<64, 1>(), zk::shift_group<64, 2>(),
                zk::shift_group<256, 1>());
    return 0;
}
"""


def test_shift_block_order(tmp_path):
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    src = tmp_path / "layout.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "layout"
    r = subprocess.run([hipcc, "-O1", "-std=c++17",
                        f"-I{os.path.join(ROOT, 'zero_dp_sharded_amd', 'csrc')}",
                        f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout
    # 64 wave-runs: 64 one-wave workgroups of one run, 32 of two, 16 of four waves
    assert out.stdout.startswith("ok 64 32 16")
