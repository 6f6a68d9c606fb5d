// Tile-order schedules shared by the GEMM kernels, the trace kernel and the
// host-side trace.  Every function here is __host__ __device__ so that the
// schedule a kernel follows and the schedule the library reports are the same
// code.
//
// Orders
//   row-major ("(1/n) Triton matmul ... persistent kernel", naive tiled listing):
//     tile_m = t / num_n_tiles, tile_n = t % num_n_tiles.
//   grouped ("(2/n) ... grouped ordering (CTA swizzle)", section Implementation):
//     tiles are dealt in groups of G tile rows; group g covers rows
//     [g*G, g*G + gs) with gs = min(G, num_m_tiles - g*G) (the last group may be
//     short) and, inside a group, consecutive ids walk down the gs rows of one
//     tile column before moving to the next column.
// Modes
//   tiled: workgroup w computes tile id w.
//   persistent ("(1/n) ...", naive persistent listing): P workgroups; workgroup p
//     computes ids p, p+P, ... below num_tiles.
//   flattened cross-tile ("(3/n) ... cross tile pipelining"): the same ids and K
//     steps as persistent, walked as one loop whose counter k wraps to 0 after
//     the last K step of a tile.
//   stream-K (the follow-on the persistent page names; the split below is this
//     library's design): the tiles of the last, partial round of the persistent
//     grid are cut along K and spread evenly over all P programs (see StreamK).
// XCD remap (this library's addition; not on the pages): MI355X deals the
//   workgroups of a launch round-robin over its 8 XCDs, each with a private L2.
//   Renumbering w -> (w % X) * q + min(w % X, r) + w / X (q = n / X, r = n % X)
//   gives XCD x one contiguous run of logical ids, so that neighbouring tiles in
//   the chosen order share an L2.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define TS_HD __host__ __device__ __forceinline__
#else
#define TS_HD inline
#endif

namespace ts {

enum : int { ORDER_ROW_MAJOR = 0, ORDER_GROUPED = 1 };
enum : int { MODE_TILED = 0, MODE_PERSISTENT = 1, MODE_CROSSTILE = 2, MODE_STREAMK = 3 };
// Kernels of the cross-tile mode on direct-to-LDS tiles, the same (tile, k)
// sequence as MODE_CROSSTILE (not schedules of their own): the nested loop with the
// deferred wait (one tile per program, at least 8 K steps) and without it (programs
// of more than one tile, at least 2 K steps).
enum : int { MODE_XTILE = 4, MODE_XTILE_PLAIN = 5 };

// Division by an invariant divisor d >= 1 with one multiply-high, one add and one
// shift, after Granlund and Montgomery, "Division by invariant integers using
// multiplication" (PLDI 1994), with the round-up multiplier: for 0 <= n < 2^31,
//   n / d = (umulhi(n, m) + n) >> l,  l = ceil(log2 d),  m = floor(2^32 (2^l - d) / d) + 1.
// umulhi(n, m) <= n, so the sum stays below 2^32.  The multiplier is made on the
// host once per launch.
struct FastDiv {
    uint32_t m;   // multiplier
    uint32_t l;   // shift
};

TS_HD uint32_t umulhi32(uint32_t a, uint32_t b) { return (uint32_t)(((uint64_t)a * b) >> 32); }
TS_HD int fdiv(int n, const FastDiv& f) { return (int)((umulhi32((uint32_t)n, f.m) + (uint32_t)n) >> f.l); }
inline FastDiv make_fastdiv(int d) {
    uint32_t l = 0;
    while ((1ull << l) < (uint64_t)d) ++l;
    FastDiv f;
    f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - (uint64_t)d)) / (uint64_t)d + 1);
    f.l = l;
    return f;
}

// Everything a program needs to find its tiles.  Plain integers, passed by value
// to kernels.  `group_m` is already clamped to [1, nm] by the host (values above
// nm give the same map as nm and would only risk overflow in group_m * nn).
struct SchedArgs {
    int nm, nn;        // tile grid: cdiv(M, BM), cdiv(N, BN)
    int ks;            // K steps: cdiv(K, BK)
    int num_tiles;     // nm * nn
    int order;         // ORDER_*
    int group_m;       // G in [1, nm]
    int grid;          // programs launched (P, or num_tiles when tiled)
    int remap;         // XCD remap on/off
    int xcds;          // XCDs the dispatcher deals workgroups over
    int fastdiv;       // 1: tile_coords divides by the multipliers below
    FastDiv f_nn;      // by nn
    FastDiv f_group;   // by G * nn (tiles per band)
    FastDiv f_g;       // by G (rows of a full band)
    FastDiv f_glast;   // by the rows of the last band
};

TS_HD int cdiv_i(int a, int b) { return (a + b - 1) / b; }
TS_HD int min_i(int a, int b) { return a < b ? a : b; }

// Fills the multipliers of s (nm, nn and group_m set); used when s.fastdiv is on.
inline void set_fastdiv(SchedArgs& s) {
    const int G = s.group_m > 0 ? s.group_m : 1;
    s.f_nn = make_fastdiv(s.nn > 0 ? s.nn : 1);
    s.f_group = make_fastdiv(G * (s.nn > 0 ? s.nn : 1));
    s.f_g = make_fastdiv(G);
    const int last_rows = s.nm > 0 ? s.nm - ((s.nm - 1) / G) * G : 1;
    s.f_glast = make_fastdiv(last_rows);
}

TS_HD int xcd_remap(int w, int n, int X) {
    const int q = n / X, r = n % X, x = w % X;
    return x * q + min_i(x, r) + w / X;
}

// Ids at or past num_tiles (the cursors of the flattened loop run ahead of the
// last tile) map to (0, 0), so that no division by a band of zero rows occurs;
// nothing is loaded or stored for them.
TS_HD void tile_coords(const SchedArgs& s, int t, int& tm, int& tn) {
    if (t >= s.num_tiles) {
        tm = tn = 0;
    } else if (s.fastdiv) {   // the same map, divisions by multiply-high
        if (s.order == ORDER_GROUPED) {
            const int gid = fdiv(t, s.f_group);
            const int tig = t - gid * (s.group_m * s.nn);
            const int first_m = gid * s.group_m;
            const bool full = first_m + s.group_m <= s.nm;
            const int gs = full ? s.group_m : s.nm - first_m;
            const int q = fdiv(tig, full ? s.f_g : s.f_glast);
            tm = first_m + (tig - q * gs);
            tn = q;
        } else {
            tm = fdiv(t, s.f_nn);
            tn = t - tm * s.nn;
        }
    } else if (s.order == ORDER_GROUPED) {
        const int in_group = s.group_m * s.nn;            // tiles per full group
        const int gid = t / in_group;
        const int tig = t - gid * in_group;               // id inside the group
        const int first_m = gid * s.group_m;
        const int gs = min_i(s.group_m, s.nm - first_m);  // rows in this group
        tm = first_m + tig % gs;
        tn = tig / gs;
    } else {
        tm = t / s.nn;
        tn = t - tm * s.nn;
    }
}

// The work of one program: tile ids start, start + grid, ... below `limit`
// (num_tiles, or the whole-tile part of a stream-K launch), each with max(ks, 1)
// K steps.  ks == 0 (K == 0) keeps one step per tile so that the tile is still
// written (with zeros).
struct ProgramWork {
    int start;   // first logical tile id
    int step;    // distance between consecutive tile ids of this program
    int ntiles;  // tiles this program computes
    int ksp;     // K steps per tile, at least 1

    TS_HD ProgramWork(const SchedArgs& s, int program) : ProgramWork(s, program, s.num_tiles) {}
    TS_HD ProgramWork(const SchedArgs& s, int program, int limit) {
        start = s.remap ? xcd_remap(program, s.grid, s.xcds) : program;
        step = s.grid;
        ntiles = start < limit ? cdiv_i(limit - start, s.grid) : 0;
        ksp = s.ks > 0 ? s.ks : 1;
    }
    TS_HD int tile_id(int i) const { return start + i * step; }
    TS_HD int total_items() const { return ntiles * ksp; }
};

// Stream-K split of a launch of P = grid programs over T tiles of ks K steps.
// The first dp_tiles = T - (T mod P) tile ids (whole rounds of the persistent
// grid) are computed whole, persistent style.  The remaining T mod P tiles form
// sk_items = (T mod P) * ks (tile, K step) items, numbered tile-major from tile
// id dp_tiles, k ascending inside a tile; they are dealt as P contiguous ranges
// whose lengths differ by at most one (the first `rem` ranges one longer).
// Program p takes range r = P - 1 - p, so that a tile's ranges run from a higher
// program index (the range holding K step 0, which finishes the tile) down to
// lower ones.  No range is longer than a tile (the split tiles number fewer than
// P), so a range touches at most two tiles.  With ks == 0 nothing is split.
struct StreamK {
    int dp_tiles;   // tiles computed whole
    int sk_items;   // (tile, K step) items of the split tiles
    int q, rem;     // range r holds q + (r < rem) items

    TS_HD explicit StreamK(const SchedArgs& s) {
        const int sk_tiles = (s.ks > 0 && s.grid > 0) ? s.num_tiles % s.grid : 0;
        dp_tiles = s.num_tiles - sk_tiles;
        sk_items = sk_tiles * s.ks;
        q = s.grid > 0 ? sk_items / s.grid : 0;
        rem = s.grid > 0 ? sk_items - q * s.grid : 0;
    }
    TS_HD int range_begin(int r) const { return r * q + min_i(r, rem); }
    // range holding item i (0 <= i < sk_items)
    TS_HD int range_of(int i) const {
        const int big = rem * (q + 1);
        return i < big ? i / (q + 1) : rem + (i - big) / q;
    }
    TS_HD int range_of_program(const SchedArgs& s, int program) const { return s.grid - 1 - program; }
};

// Cursor of the flattened loop: (tile id, k) advanced one K step at a time;
// after the last K step of a tile, k wraps to 0 and the tile id moves on by P.
struct FlatCursor {
    int tile;
    int k;
    TS_HD FlatCursor(const ProgramWork& w) : tile(w.start), k(0) {}
    TS_HD bool last_k(const ProgramWork& w) const { return k == w.ksp - 1; }
    TS_HD void advance(const ProgramWork& w) {
        if (k == w.ksp - 1) {
            k = 0;
            tile += w.step;
        } else {
            ++k;
        }
    }
};

// One program's trace rows (p, it, tile_m, tile_n, k) into rows[0 .. max_items),
// padded with -1.  The nested walk is used for tiled and persistent modes, the
// flattened cursor for the cross-tile mode, exactly as the kernels do.
TS_HD void trace_program(const SchedArgs& s, int mode, int program, int max_items, int32_t* rows) {
    int it = 0;
    if (mode == MODE_STREAMK) {
        // the split items of this program's range first, then its whole tiles
        const StreamK sk(s);
        const int r = sk.range_of_program(s, program);
        for (int i = sk.range_begin(r), e = sk.range_begin(r + 1); i < e; ++i, ++it) {
            int tm, tn;
            tile_coords(s, sk.dp_tiles + i / s.ks, tm, tn);
            int32_t* row = rows + 5 * it;
            row[0] = program; row[1] = it; row[2] = tm; row[3] = tn; row[4] = i % s.ks;
        }
        const ProgramWork w(s, program, sk.dp_tiles);
        for (int i = 0; i < w.ntiles; ++i) {
            int tm, tn;
            tile_coords(s, w.tile_id(i), tm, tn);
            for (int k = 0; k < w.ksp; ++k, ++it) {
                int32_t* row = rows + 5 * it;
                row[0] = program; row[1] = it; row[2] = tm; row[3] = tn; row[4] = k;
            }
        }
        for (; it < max_items; ++it)
            for (int f = 0; f < 5; ++f) rows[5 * it + f] = -1;
        return;
    }
    const ProgramWork w(s, program);
    if (mode == MODE_CROSSTILE) {
        FlatCursor c(w);
        for (int n = w.total_items(); it < n; ++it) {
            int tm, tn;
            tile_coords(s, c.tile, tm, tn);
            int32_t* r = rows + 5 * it;
            r[0] = program; r[1] = it; r[2] = tm; r[3] = tn; r[4] = c.k;
            c.advance(w);
        }
    } else {
        for (int i = 0; i < w.ntiles; ++i) {
            int tm, tn;
            tile_coords(s, w.tile_id(i), tm, tn);
            for (int k = 0; k < w.ksp; ++k, ++it) {
                int32_t* r = rows + 5 * it;
                r[0] = program; r[1] = it; r[2] = tm; r[3] = tn; r[4] = k;
            }
        }
    }
    for (; it < max_items; ++it)
        for (int f = 0; f < 5; ++f) rows[5 * it + f] = -1;
}

}  // namespace ts
