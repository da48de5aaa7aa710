// lf_decode.h -- division by call constants and the band-task decode,
// shared by the host planner, the gfx950 tile kernel and a CPU unit test
// (the test compiles this header with g++, where the HIP qualifiers are
// empty).  Internal to liblfattn.so.
#ifndef LF_DECODE_H
#define LF_DECODE_H

#include <stdint.h>

#include "lf_kernels.h"

#if defined(__HIPCC__)
#define LF_HD __host__ __device__ __forceinline__
#else
#define LF_HD inline
#endif

namespace lfk {

// n / d for 0 <= n < 2^31 with the divisor's Magic (see lf_kernels.h)
LF_HD int mdiv(int n, Magic g) {
    return g.s == 0 ? n : (int)((uint32_t)(((uint64_t)(uint32_t)n * g.m) >> 32) >> (g.s - 1));
}

// The Magic of a divisor d >= 1: s = ceil(log2 d), m = ceil(2^(31+s) / d)
// (below 2^32), so that mulhi(n, m) >> (s - 1) = n / d for n < 2^31.
inline Magic magic_for(long long d) {
    Magic g;
    if (d <= 1) {
        g.m = 0;
        g.s = 0;
        return g;
    }
    int l = 0;
    while ((1LL << l) < d) l++;
    const unsigned __int128 num = (unsigned __int128)1 << (31 + l);
    const unsigned __int128 m = (num + (unsigned __int128)d - 1) / (unsigned __int128)d;
    g.m = (uint32_t)m;
    g.s = l;
    return g;
}

// The band-task part of a plan: per head its dilation, class lengths and
// tile counts (tiles of LFK_BM class positions), the task prefix over heads
// and the divisors' Magics.  Returns the band tasks of one batch entry.
inline long long fill_band_plan(Plan& P, int B, int H, int T, const int32_t* dilation) {
    const long long BMq = LFK_BM;
    P.B = B;
    P.H = H;
    P.T = T;
    long long start = 0;
    for (int h = 0; h < H; h++) {
        const int delta = dilation ? dilation[h] : 1;
        P.dil[h] = delta;
        P.mg_dil[h] = magic_for(delta);
        P.head_start[h] = (int)start;
        const long long qq = T / delta, rem = T % delta;
        P.hq[h] = (int)qq;
        P.hrem[h] = (int)rem;
        P.htb[h] = (int)((qq + 1 + BMq - 1) / BMq);
        P.hts[h] = (int)((qq + BMq - 1) / BMq);
        P.mg_tb[h] = magic_for(P.htb[h]);
        P.mg_ts[h] = magic_for(P.hts[h]);
        start += rem * P.htb[h] + (delta - rem) * P.hts[h];
    }
    P.head_start[H] = (int)start;
    P.uniform_head_tasks = (int)(start / H);
    for (int h = 0; h < H; h++)
        if (P.head_start[h + 1] - P.head_start[h] != P.uniform_head_tasks) P.uniform_head_tasks = 0;
    P.band_tasks_per_batch = (int)start;
    P.mg_tpb = magic_for(start);
    P.mg_uht = magic_for(P.uniform_head_tasks);
    P.mg_H = magic_for(H);
    return start;
}

// Heads with unequal radii make band tiles of unequal cost.  The band tasks
// (batch-major, then head, then class and tile) are cut into 8 contiguous
// runs of about equal cost, one per die: each die still streams neighbouring
// tiles (which share keys in its L2), and no die is left with the expensive
// heads alone.  A tile's cost is its key steps plus a fixed part (set-up,
// Q loads, output stores) worth about 14 steps of 32 keys.  The global-row
// tasks of a head go to the die that holds the middle of its band tiles, so
// that the keys they stream are the ones that die's L2 already holds.
inline void split_by_cost(Plan& P) {
    for (int x = 0; x < 9; x++) P.band_die[x] = P.glob_die[x] = 0;
    const long long n_band = P.n_band_tasks;
    bool equal = true;
    for (int h = 1; h < P.H; h++) equal &= P.rad[h] == P.rad[0];
    if (equal || n_band == 0) return;
    double head_cost[LF_MAX_HEADS];
    for (int h = 0; h < P.H; h++) {
        const double keys = (P.one_sided ? P.rad[h] : 2.0 * P.rad[h]) + LFK_BM;
        head_cost[h] = 14.0 + keys / 32.0;
    }
    double total = 0;
    for (int h = 0; h < P.H; h++) total += head_cost[h] * (P.head_start[h + 1] - P.head_start[h]);
    total *= P.B;
    const long long tpb = P.band_tasks_per_batch;
    double acc = 0;
    int die = 1;
    for (int b = 0; b < P.B && die < 8; b++)
        for (int h = 0; h < P.H && die < 8; h++)
            for (long long t = b * tpb + P.head_start[h]; t < b * tpb + P.head_start[h + 1]; t++) {
                // task t opens die `die` once the tasks before it hold that die's share
                while (die < 8 && acc >= total * die / 8.0) P.band_die[die++] = (int)t;
                acc += head_cost[h];
            }
    while (die < 8) P.band_die[die++] = (int)n_band;
    P.band_die[8] = (int)n_band;
    // global-row tasks: (b, h)-major, n_split * n_ggroups per head
    const long long per_bh = (long long)P.n_split * P.n_ggroups;
    int x = 0;
    for (int bh = 0; bh < P.B * P.H && P.n_tasks > P.n_band_tasks; bh++) {
        const long long mid = (long long)(bh / P.H) * tpb + (P.head_start[bh % P.H] + P.head_start[bh % P.H + 1]) / 2;
        while (x < 7 && mid >= P.band_die[x + 1]) P.glob_die[++x] = (int)(bh * per_bh);
    }
    while (x < 7) P.glob_die[++x] = P.n_tasks - P.n_band_tasks;
    P.glob_die[8] = P.n_tasks - P.n_band_tasks;
}

// Split of the T keys for the global-row tasks: `per` = B * H * (groups of
// 64 global queries).  About 144 tasks in all (a little over one per two
// compute units), no split longer than 4096 keys, at most 64 splits per head
// (which bounds the combine's reads), at least 64 keys a split; lengths are
// multiples of 32 keys.  A split shares its compute unit with band tiles and
// slows them, so fewer, longer splits disturb fewer units (B1 H12 T4096
// r256 with one global: 228 splits of 224 keys took 16.43 us a forward
// call, 144 of 352 keys 15.54 us; one-sided 13.96 -> 12.84 us).
inline void global_splits(long long per, int T, int* split_len, int* n_split) {
    const long long T32 = ((long long)T + 31) / 32 * 32;
    long long ns = 144 / per;
    const long long ns_len = ((long long)T + 4095) / 4096;
    if (ns < ns_len) ns = ns_len;
    if (ns < 1) ns = 1;
    if (ns > 64) ns = 64;
    long long sl = (((long long)T + ns - 1) / ns + 31) / 32 * 32;
    if (sl < 64) sl = 64;
    if (sl >= T) sl = T32;   // one split: the whole (32-rounded) sequence
    *split_len = (int)sl;
    *n_split = (int)(((long long)T + sl - 1) / sl);
}

// Workgroup slots per die: its global-row tasks, then its band tasks (an
// eighth of each, or the runs the plan cut by cost).
inline int slots_per_die(const Plan& P) {
    const int nb = P.n_band_tasks, ng = P.n_tasks - P.n_band_tasks;
    if (P.band_die[8] == 0) return (nb + 7) / 8 + (ng + 7) / 8;
    int m = 0;
    for (int x = 0; x < 8; x++) {
        const int n = P.band_die[x + 1] - P.band_die[x] + P.glob_die[x + 1] - P.glob_die[x];
        m = m > n ? m : n;
    }
    return m;
}

// The task of workgroup slot `slot` of die `xcd`, -1 past the die's tasks.
// globals_first: the die's global-row tasks take its first slots (they are
// short and end with a combine), else its last (they fill the tail of the
// band tiles' last round).
LF_HD int task_of_slot(const Plan& P, int xcd, int slot, bool globals_first) {
    const int nb = P.n_band_tasks, ng = P.n_tasks - P.n_band_tasks;
    int g_o, g_n, b_o, b_n;
    if (P.band_die[8] > 0) {
        g_o = P.glob_die[xcd];
        g_n = P.glob_die[xcd + 1] - g_o;
        b_o = P.band_die[xcd];
        b_n = P.band_die[xcd + 1] - b_o;
    } else {
        g_n = (ng >> 3) + (xcd < (ng & 7));
        g_o = xcd * (ng >> 3) + (xcd < (ng & 7) ? xcd : (ng & 7));
        b_n = (nb >> 3) + (xcd < (nb & 7));
        b_o = xcd * (nb >> 3) + (xcd < (nb & 7) ? xcd : (nb & 7));
    }
    if (globals_first) {
        if (slot < g_n) return nb + g_o + slot;
        slot -= g_n;
        return slot < b_n ? b_o + slot : -1;
    }
    if (slot < b_n) return b_o + slot;
    slot -= b_n;
    return slot < g_n ? nb + g_o + slot : -1;
}

// Band task t of the plan -> (b, h, residue class c, class length n, tile).
// Tasks run batch-major, then head, then class, then tile; classes
// 0 .. hrem-1 of a head hold hq + 1 positions (htb tiles each), the others
// hq (hts tiles).
struct BandTask {
    int b, h, c, n, tile;
};

LF_HD BandTask decode_band(const Plan& P, int t) {
    BandTask k;
    k.b = mdiv(t, P.mg_tpb);
    int x = t - k.b * P.band_tasks_per_batch;
    int h;
    if (P.uniform_head_tasks > 0) {
        h = mdiv(x, P.mg_uht);
        x -= h * P.uniform_head_tasks;
    } else {
        // heads are few (<= LF_MAX_HEADS): binary search on the band-task prefix
        int lo = 0, hi = P.H - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (P.head_start[mid] <= x) lo = mid; else hi = mid - 1;
        }
        h = lo;
        x -= P.head_start[h];
    }
    k.h = h;
    if (P.dil[h] == 1) {
        k.c = 0;
        k.tile = x;
        k.n = P.T;
    } else {
        const int rem = P.hrem[h], tb = P.htb[h], ts = P.hts[h];
        if (x < rem * tb) {
            k.c = mdiv(x, P.mg_tb[h]);
            k.tile = x - k.c * tb;
            k.n = P.hq[h] + 1;
        } else {
            const int y = x - rem * tb;
            const int cc = mdiv(y, P.mg_ts[h]);
            k.c = rem + cc;
            k.tile = y - cc * ts;
            k.n = P.hq[h];
        }
    }
    return k;
}

// Global-row task g (counted from the first global-row task) -> (b*H + h,
// group of global slots, key split).
struct RowTask {
    int bh, grp, split;
};

LF_HD RowTask decode_rows(const Plan& P, int g) {
    RowTask k;
    const int per_bh = P.n_split * P.n_ggroups;
    k.bh = mdiv(g, P.mg_per_bh);
    const int rem = g - k.bh * per_bh;
    k.grp = mdiv(rem, P.mg_nsplit);
    k.split = rem - k.grp * P.n_split;
    return k;
}

}  // namespace lfk

#endif
