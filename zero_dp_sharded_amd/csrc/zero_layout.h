// Host-side layout of the streamed arrays: how many leading elements a kernel
// peels so that its vector runs are 16-byte aligned, and for a bucket reduce
// whether the aligned kernel, the shift kernel or the element-wise kernel runs
// and over which runs.  Used by zero_shard.cpp and compiled on the CPU by the
// layout tests.  Not part of the public ABI.
#pragma once

#include <stdint.h>

namespace zl {

// Leading elements to peel so that every listed address, advanced by that many
// elements of size elt[k], is aligned to align[k] bytes; -1 if none below 8
// exists.
inline int64_t common_head(const uintptr_t* addr, const int* elt, const int* align, int count)
{
    for (int64_t h = 0; h < 8; ++h) {
        bool ok = true;
        for (int k = 0; k < count && ok; ++k)
            ok = ((addr[k] + (uintptr_t)h * elt[k]) % (uintptr_t)align[k]) == 0;
        if (ok) return h;
    }
    return -1;
}

// Layout of n elements for a kernel working on runs of `run` elements:
// `head` scalar elements, then nrun aligned runs, then a scalar tail.
// head < 0 (no common alignment) selects the element-wise path.
inline void split(int64_t n, int64_t head, int64_t run, int64_t* out_head, int64_t* out_nrun,
                  int32_t* vec_ok)
{
    if (head < 0) {
        *vec_ok = 0;
        *out_head = 0;
        *out_nrun = 0;
        return;
    }
    if (head > n) head = n;
    *vec_ok = 1;
    *out_head = head;
    *out_nrun = (n - head) / run;
}

// Smallest h < 8 such that every one of the `count` addresses advanced by h
// elements of esz bytes is 16-byte aligned; -1 if there is none.
inline int64_t head16(const uintptr_t* addr, int count, int esz)
{
    for (int64_t h = 0; h < 8; ++h) {
        bool ok = true;
        for (int k = 0; k < count && ok; ++k) ok = ((addr[k] + (uintptr_t)h * esz) & 15u) == 0;
        if (ok) return h;
    }
    return -1;
}

struct ReduceLayout {
    int32_t shift;    // 1: the shift kernel (contributions off the output's phase)
    int32_t vec_ok;   // 0: every element element-wise
    int64_t head;     // leading elements reduced element-wise
    int64_t nvec;     // 16-byte output runs of W elements after the head
};

// A bucket reduce of n elements of esz bytes from R contributions at
// addr[0 .. R) into the output at addr[R], in runs of W = 16 / esz elements:
//  - every address sharing one phase modulo 16 bytes: whole aligned runs after
//    the common head;
//  - else, with the output element-aligned: the shift kernel.  The output runs
//    are aligned from head h, and contribution r's run vi lies s_r elements
//    past the aligned word vi of its base (s_r = its phase at h, in elements).
//    h is the output's own head, raised by one run when some s_r exceeds it,
//    so that word 0 starts inside every contribution; the body keeps one whole
//    run after it (nvec = whole runs - 1), so that word nvec, which the last
//    run reads, ends inside every contribution;
//  - else element-wise.
inline ReduceLayout reduce_layout(const uintptr_t* addr, int R, int esz, int64_t n)
{
    const int W = 16 / esz;
    ReduceLayout lay{0, 0, 0, 0};
    const int64_t common = head16(addr, R + 1, esz);
    if (common >= 0) {
        split(n, common, W, &lay.head, &lay.nvec, &lay.vec_ok);
        return lay;
    }
    int64_t h0 = head16(&addr[R], 1, esz);
    if (h0 < 0) {
        split(n, -1, W, &lay.head, &lay.nvec, &lay.vec_ok);
        return lay;
    }
    int64_t smax = 0;
    for (int r = 0; r < R; ++r) {
        const int64_t sr = (int64_t)((addr[r] + (uintptr_t)h0 * esz) & 15u) / esz;
        if (sr > smax) smax = sr;
    }
    if (smax > h0) h0 += W;
    lay.shift = 1;
    lay.vec_ok = 1;
    lay.head = h0 < n ? h0 : n;
    const int64_t whole = (n - lay.head) / W;
    lay.nvec = whole > 1 ? whole - 1 : 0;
    return lay;
}

}  // namespace zl
