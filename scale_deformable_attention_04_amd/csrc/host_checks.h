// host_checks.h -- the host-side part of libmsda.so that needs no GPU: the
// size checks every entry point makes before launching anything, the
// validation of a host copy of the level table, the backward workspace
// layouts and the status strings.  Plain C++ with no HIP dependency: the HIP
// translation units include it, and host_checks.cpp compiles it on its own
// (with g++) into the library and into the CPU sanitizer build.
#ifndef MSDA_CSRC_HOST_CHECKS_H
#define MSDA_CSRC_HOST_CHECKS_H

#include <stddef.h>
#include <stdint.h>

#include "msda.h"

namespace msda_host {

constexpr int kMaxLevels = 16;
constexpr int kChunk = 2048;        // grad_value records per work item, at most
constexpr int kRecQueryShift = 7;   // a record keeps the query index above 7 cell bits

inline bool supported_d(int64_t D) {
    return D == 4 || D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256;
}

// Sizes of a call, before anything is launched.  coords = 2 for the 2-D core,
// 3 for the volume variant (floats per location).
inline msda_status check_sizes_n(int value_dtype, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                                 int64_t D, int64_t L, int64_t K, int coords) {
    if (value_dtype != MSDA_F32 && value_dtype != MSDA_BF16) return MSDA_ERR_DTYPE;
    if (B < 0 || Nv < 0 || Nq < 0 || M < 1 || D < 1 || L < 1 || K < 1) return MSDA_ERR_SHAPE;
    if (L > kMaxLevels || !supported_d(D)) return MSDA_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t)1 << 31;
    // the rows of one workgroup's queries stay 31-bit addressable
    if (M > ((int64_t)1 << 20) / D) return MSDA_ERR_UNSUPPORTED;
    // one batch slice of grad_value (fp32) and of the point arrays must be 31-bit addressable
    if (Nv > lim / (M * D * 4) || Nv * M * D * 4 >= lim) return MSDA_ERR_UNSUPPORTED;
    if (K > lim / L || Nq > lim / (M * L * K * coords) || Nq * M * L * K * coords >= lim)
        return MSDA_ERR_UNSUPPORTED;
    // the 2-D backward stores point indices of the whole problem, four per
    // point, in 32 bits
    if (coords == 2 && B > 0 && Nq > 0 && B > (((int64_t)1 << 32) - 1) / (Nq * M * L * K * 4))
        return MSDA_ERR_UNSUPPORTED;
    // one launch covers Nq*M items with D/4 lanes each: keep the grid under 2^31 threads
    if (Nq * M > lim / (D / 4)) return MSDA_ERR_UNSUPPORTED;
    // whole tensors stay below 2^50 bytes, so that no size or workspace
    // offset computed from them overflows (the batch is otherwise unbounded)
    if (B > 0) {
        int64_t per_b = Nv * M * D * 4;                                   // value, grad_value
        per_b = Nq * M * L * K * coords * 4 > per_b ? Nq * M * L * K * coords * 4 : per_b;
        per_b = Nq * M * D * 4 > per_b ? Nq * M * D * 4 : per_b;         // out, grad_out
        if (per_b > 0 && B > ((int64_t)1 << 50) / per_b) return MSDA_ERR_UNSUPPORTED;
    }
    return MSDA_OK;
}

inline msda_status check_sizes(int value_dtype, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                               int64_t D, int64_t L, int64_t K) {
    return check_sizes_n(value_dtype, B, Nv, Nq, M, D, L, K, 2);
}

inline msda_status check_sizes3(int value_dtype, int64_t B, int64_t Nv, int64_t Nq, int64_t M,
                                int64_t D, int64_t L, int64_t K) {
    return check_sizes_n(value_dtype, B, Nv, Nq, M, D, L, K, 3);
}

// A host copy of the level table: rows of `dims` extents ((H, W) or
// (Z, H, W)), every extent >= 1 and < 2^24 (pixel coordinates are formed in
// fp32, and stay exact integers), level_start[l] the number of rows of the
// levels before l, and Nv the total.
inline msda_status validate_levels(const int64_t *shapes, const int64_t *starts, int64_t L,
                                   int64_t Nv, int dims) {
    if (!shapes || !starts) return MSDA_ERR_NULL;
    int64_t total = 0;
    for (int64_t l = 0; l < L; ++l) {
        const int64_t *e = shapes + dims * l;
        for (int a = 0; a < dims; ++a)
            if (e[a] < 1) return MSDA_ERR_SHAPE;
        for (int a = 0; a < dims; ++a)
            if (e[a] >= ((int64_t)1 << 24)) return MSDA_ERR_UNSUPPORTED;
        if (starts[l] != total) return MSDA_ERR_SHAPE;
        int64_t rows = 1;
        for (int a = 0; a < dims; ++a) {
            if (e[a] > Nv / rows) return MSDA_ERR_SHAPE;  // the product would pass Nv
            rows *= e[a];
        }
        total += rows;
        if (total > Nv) return MSDA_ERR_SHAPE;
    }
    return total == Nv ? MSDA_OK : MSDA_ERR_SHAPE;
}

// Upper bound of the number of 8x8 tiles over all levels, from Nv and L only:
// sum ceil(H/8)*ceil(W/8) <= sum (HW + 7(H+W) + 49)/64 <= (15 Nv + 49 L)/64.
inline int64_t bins_bound(int64_t Nv, int64_t L) { return (15 * Nv + 49 * L) / 64 + 1; }

// The workspace of the backward's grad_value pipeline: bin counters, starts
// and cursors [B][nb_max][M], the work list, its totals, the zero list, the
// list of split bins and the records.  2-D levels (vol = false): at most four records per point and
// bins_bound(Nv, L) bins per (batch, head).  Volumes: two planes of four
// tiles, so eight records per point, and at most one bin per voxel.
struct WorkLayout {
    int64_t nb_max, bm_bins, work_max, sorted_max;
    size_t off_counts, off_start, off_cursor, off_items, off_total, off_zero, off_split,
        off_sorted, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline WorkLayout work_layout(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L,
                              int64_t K, bool vol = false) {
    WorkLayout w;
    w.nb_max = vol ? Nv + 1 : bins_bound(Nv, L);
    w.bm_bins = B * M * w.nb_max;
    const int64_t pts = B * Nq * M * L * K;
    w.sorted_max = (vol ? 8 : 4) * pts;
    w.work_max = w.bm_bins + (w.sorted_max + kChunk - 1) / kChunk;
    size_t o = 0;
    w.off_counts = o;
    o = align256(o + 4 * (size_t)w.bm_bins);
    w.off_start = o;
    o = align256(o + 4 * (size_t)w.bm_bins);
    w.off_cursor = o;
    o = align256(o + 4 * (size_t)w.bm_bins);
    w.off_items = o;
    o = align256(o + 16 * (size_t)w.work_max);
    w.off_total = o;
    o = align256(o + 16);
    w.off_zero = o;
    o = align256(o + 4 * (size_t)w.bm_bins);
    w.off_split = o;
    o = align256(o + 4 * (size_t)w.bm_bins);
    w.off_sorted = o;
    o = align256(o + 16 * (size_t)w.sorted_max);
    w.bytes = o;
    return w;
}

// Fewest queries in a pass of the grad_value pipeline (see pass_plan): below
// this the passes' launches would cost more than their work.
constexpr int64_t kMinPassQueries = 1024;

// The passes of the grad_value pipeline in a workspace of `bytes`: boxes of
// nb batches x nm heads x nq queries, each run as a problem of its own in a
// layout `wl` for that box.  A pass costs its launches and their latency
// (about 60 us at the encoder shape), so the plan takes the fewest passes:
// the whole problem; else groups of whole batches; else one batch and
// ranges of nq queries with every head (the tensors' rows stay contiguous);
// only when not even min(Nq, kMinPassQueries) queries of every head fit,
// groups of nm heads and ranges of queries.  nb = 0: not even the smallest
// pass (one head, min(Nq, kMinPassQueries) queries) fits.  Layout sizes grow
// with the batches, heads and queries, so each largest fit is found by
// bisection.
struct PassPlan {
    int64_t nb, nm, nq;
    WorkLayout wl;
};

inline int64_t min_pass_queries(int64_t Nq) { return Nq < kMinPassQueries ? Nq : kMinPassQueries; }

// The smallest workspace any pass plan accepts (one batch, one head,
// min_pass_queries).
inline size_t min_workspace(int64_t Nv, int64_t Nq, int64_t L, int64_t K, bool vol) {
    return work_layout(1, Nv, min_pass_queries(Nq), 1, L, K, vol).bytes;
}

inline PassPlan pass_plan(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L, int64_t K,
                          bool vol, size_t bytes) {
    auto fits = [&](int64_t nb, int64_t nm, int64_t nq) {
        return work_layout(nb, Nv, nq, nm, L, K, vol).bytes <= bytes;
    };
    // the largest n in [lo, hi] with fit(n), given fit(lo)
    auto largest = [](int64_t lo, int64_t hi, auto fit) {
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo + 1) / 2;
            if (fit(mid))
                lo = mid;
            else
                hi = mid - 1;
        }
        return lo;
    };
    const int64_t q_min = min_pass_queries(Nq);
    PassPlan p{B, M, Nq, WorkLayout{}};
    if (!fits(B, M, Nq)) {
        if (fits(1, M, Nq)) {
            p.nb = largest(1, B - 1, [&](int64_t nb) { return fits(nb, M, Nq); });
        } else if (fits(1, M, q_min)) {
            p.nb = 1;
            p.nq = largest(q_min, Nq - 1, [&](int64_t nq) { return fits(1, M, nq); });
        } else if (fits(1, 1, q_min)) {
            p.nb = 1;
            p.nm = largest(1, M - 1, [&](int64_t nm) { return fits(1, nm, q_min); });
            p.nq = largest(q_min, Nq, [&](int64_t nq) { return fits(1, p.nm, nq); });
        } else {
            return PassPlan{0, 0, 0, WorkLayout{}};
        }
    }
    p.wl = work_layout(p.nb, Nv, p.nq, p.nm, L, K, vol);
    return p;
}

// Workspace of the fused backward: the locations [pts][2] and weights [pts]
// the prologue writes, the per-(item, level) location-gradient sums, then
// the core's (`core` bytes at off_core for the whole problem in one pass,
// at least core_min).
struct FusedLayout {
    size_t off_loc, off_attn, off_part, off_core, core, core_min, bytes;
};

inline FusedLayout fused_layout(int64_t B, int64_t Nv, int64_t Nq, int64_t M, int64_t L,
                                int64_t K) {
    const size_t pts = (size_t)(B * Nq * M * L * K);
    FusedLayout f;
    f.off_loc = 0;
    f.off_attn = align256(f.off_loc + 8 * pts);
    f.off_part = align256(f.off_attn + 4 * pts);
    f.off_core = align256(f.off_part + 8 * (size_t)(B * Nq * M * L));
    f.core = work_layout(B, Nv, Nq, M, L, K).bytes;
    f.core_min = min_workspace(Nv, Nq, L, K, false);
    f.bytes = f.off_core + f.core;
    return f;
}

inline const char *status_string(int status) {
    switch (status) {
    case MSDA_OK: return "ok";
    case MSDA_ERR_NULL: return "a required pointer is NULL";
    case MSDA_ERR_SHAPE: return "sizes are negative or inconsistent with the level table";
    case MSDA_ERR_DTYPE: return "unknown value dtype";
    case MSDA_ERR_UNSUPPORTED:
        return "outside the supported limits (D in {4,8,...,256}, 1 <= L <= 16, 31-bit slices)";
    case MSDA_ERR_HIP: return "the HIP runtime refused a launch";
    case MSDA_ERR_WORKSPACE:
        return "workspace smaller than the *_workspace_min size or not 256-byte aligned";
    case MSDA_ERR_SCRATCH:
        return "even the smallest pass needs more scratch than msda_backward_noalloc's "
               "static buffer (MSDA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown msda status";
    }
}

}  // namespace msda_host

#endif  // MSDA_CSRC_HOST_CHECKS_H
