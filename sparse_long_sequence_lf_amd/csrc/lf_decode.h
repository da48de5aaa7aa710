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
