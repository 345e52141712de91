// Index checks of the checked build.
//
// Device code cannot be built with the address sanitiser, and the orrery
// performance page ("A note on the sanitisers") asks instead that index
// conversions be checked rather than trusted. Built with ORR_CHECKED=1
// (liborr_checked.so), the kernels test every index they take from data that
// another kernel wrote (node escapes, leaf ranges, the sort's permutation,
// node slots and lists of the build) against the length of the array it
// addresses. A failed check sets kBadIndex in the build's status word
// (DevParams::bad_input) and the access is skipped; a walk that meets a bad
// escape ends. Nothing traps: the next call that synchronises reports the
// failure (ORR_ERR_HIP), and the results of that build are invalid.
//
// In the normal build checked_lt is the constant true and generates no code,
// and guarded_lt is the plain comparison the kernel makes anyway. A check
// that needs a statement of its own (an early exit from a walk loop) is
// written inside ORR_IF_CHECKED, which leaves the normal build's source, and
// so its code, as it is without the check: even a statement that folds away
// can change how the compiler lays out a loop.
#pragma once

#include "orr_internal.h"

#ifndef ORR_CHECKED
#define ORR_CHECKED 0
#endif

#if ORR_CHECKED
#define ORR_IF_CHECKED(...) __VA_ARGS__
#else
#define ORR_IF_CHECKED(...)
#endif

namespace orr {

constexpr bool kChecked = ORR_CHECKED != 0;

// Where a kernel reports, and the particle count its leaf ranges and
// permutation entries are checked against.
struct Check {
    uint32_t *word;
    uint32_t n_particles;
};

// Kernels that only read the parameter block take it as const (their loads
// of it may go through the scalar cache); the checked build still reports
// through it. That is sound because none of them reads the status word, and
// the atomic goes to memory, past the caches the const loads may use.
__device__ __forceinline__ Check make_check(const DevParams *prm) {
    if constexpr (kChecked)
        return Check{const_cast<uint32_t *>(&prm->bad_input), prm->n_particles};
    else
        return Check{nullptr, 0u};
}

__device__ __forceinline__ void report_bad_index(uint32_t *word) { atomicOr(word, kBadIndex); }

// i < limit, checked: true in the normal build; in the checked build the
// comparison, reported when false.
__device__ __forceinline__ bool checked_lt(uint64_t i, uint64_t limit, uint32_t *word) {
    if constexpr (kChecked) {
        if (i < limit) return true;
        report_bad_index(word);
        return false;
    } else {
        return true;
    }
}

// i < limit in both builds, for guards the kernel keeps anyway; the checked
// build also reports a false one.
__device__ __forceinline__ bool guarded_lt(uint64_t i, uint64_t limit, uint32_t *word) {
    const bool ok = i < limit;
    if constexpr (kChecked)
        if (!ok) report_bad_index(word);
    return ok;
}

// A node record's escape e, read at node c of a tree of n_nodes nodes:
// c < e <= n_nodes in every well-formed tree (a walk moves forward to it).
__device__ __forceinline__ bool escape_ok(uint32_t c, uint32_t e, uint32_t n_nodes, uint32_t *word) {
    return checked_lt(c, e, word) && checked_lt(e, (uint64_t)n_nodes + 1u, word);
}

// A leaf's particles [b, b + cnt) lie among the build's sorted particles.
__device__ __forceinline__ bool leaf_ok(uint32_t b, uint32_t cnt, const Check &ck) {
    return checked_lt((uint64_t)b + cnt, (uint64_t)ck.n_particles + 1u, ck.word);
}

}  // namespace orr
