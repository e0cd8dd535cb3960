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


LAYOUT_PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>
#include "zero_kernels.h"
#include "zero_layout.h"

#define CHECK(c, ...) do { if (!(c)) { std::printf(__VA_ARGS__); std::printf("\n"); return 1; } } while (0)

// The word indexes a shift-kernel launch of nvec runs reads and the runs it
// writes, from the kernel's index expressions: workgroup b takes block
// shift_block(b), lane t its runs v0 + u * BS (v0 = block * BS * U + t), each
// load clamped to word nvec, and the last lane of each wave one more word
// when its last run is inside the body.
template <unsigned G>
static int walk(int64_t nvec, int U, int BS, std::vector<int>& hit)
{
    const int64_t vblocks = (nvec + (int64_t)BS * U - 1) / ((int64_t)BS * U);
    hit.assign((size_t)nvec, 0);
    for (int64_t b = 0; b < vblocks; ++b) {
        const int64_t blk = zk::shift_block<G>((unsigned)b, (unsigned)vblocks);
        CHECK(blk >= 0 && blk < vblocks, "block %lld of %lld", (long long)blk, (long long)vblocks);
        for (int t = 0; t < BS; ++t) {
            const int64_t v0 = blk * BS * U + t;
            for (int u = 0; u < U; ++u) {
                const int64_t vi = v0 + (int64_t)u * BS;
                const int64_t w = vi <= nvec ? vi : nvec;
                CHECK(w >= 0 && w <= nvec, "word %lld past %lld", (long long)w, (long long)nvec);
                if (vi < nvec) hit[(size_t)vi]++;
            }
            if ((t & 63) == 63 && v0 + (int64_t)(U - 1) * BS < nvec)
                CHECK(v0 + (int64_t)(U - 1) * BS + 1 <= nvec, "extra word past %lld", (long long)nvec);
        }
    }
    for (int64_t vi = 0; vi < nvec; ++vi)
        CHECK(hit[(size_t)vi] == 1, "run %lld written %d times", (long long)vi, hit[(size_t)vi]);
    return 0;
}

int main() {
    std::mt19937_64 rng(20261203);
    long nvec_cases = 0, nshift = 0, nelem = 0, nwalk = 0;
    std::vector<int> hit;
    for (int trial = 0; trial < 300000; ++trial) {
        const int esz = (rng() & 1) ? 2 : 4;
        const int W = 16 / esz;
        const int R = 1 + (int)(rng() % 24);
        const int size_class = (int)(rng() % 60);
        const int64_t n = size_class < 20 ? 1 + (int64_t)(rng() % 48)
                          : size_class < 59 ? 1 + (int64_t)(rng() % 20000)
                                            : 1 + (int64_t)(rng() % 1200000);   // full block sets
        std::vector<uintptr_t> base(R + 1), addr(R + 1);
        for (int k = 0; k <= R; ++k) {
            base[k] = (uintptr_t)(k + 1) << 24;                 // separate allocations
            addr[k] = base[k] + (uintptr_t)(rng() % (16 / esz)) * esz;
        }
        const int mode = (int)(rng() % 8);
        if (mode == 0)                                          // one common phase
            for (int k = 0; k < R; ++k) addr[k] = base[k] + (addr[R] & 15u);
        if (mode == 1) addr[0] = addr[R];                       // reduce in place
        if (mode == 2 && esz == 2) addr[R] += 1;                // output not element-aligned
        const zl::ReduceLayout L = zl::reduce_layout(addr.data(), R, esz, n);
        if (!L.vec_ok) {
            CHECK(L.head == 0 && L.nvec == 0 && L.shift == 0, "element-wise layout");
            nelem++;
            continue;
        }
        const int64_t tail = n - L.head - L.nvec * W;
        CHECK(L.head >= 0 && L.nvec >= 0 && tail >= 0, "partition n=%lld head=%lld nvec=%lld",
              (long long)n, (long long)L.head, (long long)L.nvec);
        if (L.nvec > 0)
            CHECK(((addr[R] + (uintptr_t)L.head * esz) & 15u) == 0, "output runs not aligned");
        if (!L.shift) {
            nvec_cases++;
            CHECK(L.head < 8, "head %lld", (long long)L.head);
            if (L.nvec > 0)
                for (int k = 0; k < R; ++k)
                    CHECK(((addr[k] + (uintptr_t)L.head * esz) & 15u) == 0, "contribution %d not aligned", k);
            continue;
        }
        nshift++;
        // head and tail go element-wise, one per lane of the last workgroup
        CHECK(L.head < W + 8 && (L.nvec == 0 || tail < 2 * W), "head %lld tail %lld",
              (long long)L.head, (long long)tail);
        if (L.nvec == 0) continue;
        for (int r = 0; r < R; ++r) {
            const uintptr_t p = addr[r] + (uintptr_t)L.head * esz;   // run 0 of contribution r
            const uintptr_t w0 = p & ~(uintptr_t)15;                   // its word 0
            CHECK(w0 >= addr[r], "word 0 of contribution %d starts before it", r);
            CHECK(w0 + 16 * (uintptr_t)(L.nvec + 1) <= addr[r] + (uintptr_t)n * esz,
                  "word nvec of contribution %d ends past it (n=%lld head=%lld nvec=%lld)", r,
                  (long long)n, (long long)L.head, (long long)L.nvec);
        }
        if ((L.nvec <= 5000 && trial % 7 == 0) || size_class == 59) {
            for (int small = 0; small < 2; ++small) {
                const int U = zk::red_runs(R, L.nvec, small != 0, true);
                const int BS = zk::red_block(R, small != 0);
                int rc;
                if (BS == 64 && U == 1) rc = walk<zk::shift_group<64, 1>()>(L.nvec, U, BS, hit);
                else if (BS == 64 && U == 2) rc = walk<zk::shift_group<64, 2>()>(L.nvec, U, BS, hit);
                else if (BS == 256 && U == 1) rc = walk<zk::shift_group<256, 1>()>(L.nvec, U, BS, hit);
                else CHECK(false, "shape U=%d BS=%d not modelled", U, BS);
                if (rc) return rc;
                nwalk++;
            }
        }
    }
    CHECK(nshift > 1000 && nvec_cases > 1000 && nelem > 100 && nwalk > 1000,
          "too few cases %ld %ld %ld %ld", nvec_cases, nshift, nelem, nwalk);
    std::printf("ok aligned %ld shift %ld element-wise %ld walks %ld\n", nvec_cases, nshift, nelem, nwalk);
    return 0;
}
"""


def test_reduce_layout_reads_stay_inside_every_bucket(tmp_path):
    """For 300,000 random bucket layouts (2- and 4-byte elements, 1-24
    contributions at random phases, some sharing one phase, some reducing in
    place, some with an output off its element size), the host's layout
    (zero_layout.h) partitions the bucket into head, 16-byte output runs and
    tail; the aligned kernel gets only addresses that share the output's
    phase; and for the shift kernel word 0 of every contribution starts inside
    it and word nvec, the last one its loads reach, ends inside it.  For
    a sample of layouts, up to 150,000 runs (several full sets of the XCD
    block order), the kernel's own index expressions (block order, lanes, runs
    per lane, the clamp and the last lane's extra word) are walked in every
    launch shape: no word index passes nvec and every output run is written
    exactly once."""
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    src = tmp_path / "layout2.cpp"
    src.write_text(LAYOUT_PROGRAM)
    exe = tmp_path / "layout2"
    r = subprocess.run([hipcc, "-O2", "-std=c++17",
                        f"-I{os.path.join(ROOT, 'zero_dp_sharded_amd', 'csrc')}",
                        f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout[-2000:]
    assert out.stdout.startswith("ok aligned"), out.stdout
