// CPU check of the division by call constants and of the band-task and
// global-row-task decodes the tile kernel runs (lf_decode.h, compiled here
// with g++): every division exact, every task decoded to a distinct
// (b, h, class, tile) inside its ranges, in the order of a plain decode
// written with ordinary division.  Prints "OK <count>" or the first failure.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "lf_decode.h"

using namespace lfk;

static int fails = 0;
#define CHECK(c, ...)                         \
    do {                                      \
        if (!(c)) {                           \
            if (fails++ < 10) {               \
                std::printf("FAIL: " __VA_ARGS__); \
                std::printf("\n");            \
            }                                 \
        }                                     \
    } while (0)

int main() {
    long long checked = 0;
    // ---- n / d
    std::mt19937_64 rng(12345);
    std::vector<long long> ds = {1, 2, 3, 5, 7, 63, 64, 65, 96, 100, 255, 256, 257, 1000, 4095, 4096, 4097,
                                 65535, 65536, 65537, 1 << 20, (1 << 20) + 1, (1 << 24) - 1, 1 << 24,
                                 (1LL << 30) - 1, 1LL << 30, (1LL << 31) - 1};
    for (int i = 0; i < 2000; i++) ds.push_back(1 + (long long)(rng() % ((1ULL << 31) - 1)));
    for (int i = 0; i < 2000; i++) ds.push_back(1 + (long long)(rng() % 5000));
    for (long long d : ds) {
        const Magic g = magic_for(d);
        std::vector<long long> ns = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, (1LL << 31) - 1, (1LL << 31) - 2,
                                     ((1LL << 31) - 1) / d * d, ((1LL << 31) - 1) / d * d - 1};
        for (int i = 0; i < 300; i++) ns.push_back((long long)(rng() % (1ULL << 31)));
        for (long long n : ns) {
            if (n < 0 || n >= (1LL << 31)) continue;
            const int q = mdiv((int)n, g);
            CHECK(q == n / d, "mdiv(%lld, %lld) = %d, want %lld", n, d, q, n / d);
            checked++;
        }
    }
    // ---- band-task decode on shapes with uniform and unequal heads
    struct Shape { int B, H, T; std::vector<int32_t> dil; };
    std::vector<Shape> shapes = {
        {1, 12, 4096, {1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1}},
        {1, 12, 4096, {1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 4, 4}},
        {4, 16, 16384, {}},
        {2, 3, 1, {1, 2, 3}},
        {3, 5, 777, {1, 7, 64, 65, 1000}},
        {2, 4, 130, {3, 3, 3, 3}},
        {1, 2, 65, {65535, 1}},
    };
    for (int i = 0; i < 40; i++) {
        Shape s;
        s.B = 1 + (int)(rng() % 4);
        s.H = 1 + (int)(rng() % 9);
        s.T = 1 + (int)(rng() % 3000);
        for (int h = 0; h < s.H; h++) s.dil.push_back(1 + (int32_t)(rng() % 9));
        shapes.push_back(s);
    }
    for (const Shape& sh : shapes) {
        Plan P;
        std::memset(&P, 0, sizeof P);
        const int32_t* dil = sh.dil.empty() ? nullptr : sh.dil.data();
        const long long tpb = fill_band_plan(P, sh.B, sh.H, sh.T, dil);
        // the plain decode: ordinary division, in the same task order
        long long t = 0;
        std::set<std::tuple<int, int, int, int>> seen;
        for (int b = 0; b < sh.B; b++)
            for (int h = 0; h < sh.H; h++) {
                const int delta = dil ? dil[h] : 1;
                for (int c = 0; c < delta && c < sh.T; c++) {
                    const int n = (sh.T - c + delta - 1) / delta;
                    const int tiles = (n + LFK_BM - 1) / LFK_BM;
                    for (int tile = 0; tile < tiles; tile++, t++) {
                        const BandTask k = decode_band(P, (int)t);
                        CHECK(k.b == b && k.h == h && k.c == c && k.tile == tile && k.n == n,
                              "T=%d task %lld -> (%d,%d,%d,%d,n=%d), want (%d,%d,%d,%d,n=%d)", sh.T, t, k.b, k.h,
                              k.c, k.tile, k.n, b, h, c, tile, n);
                        CHECK(seen.insert(std::make_tuple(k.b, k.h, k.c, k.tile)).second, "task %lld repeats", t);
                        checked++;
                    }
                }
            }
        CHECK(t == tpb * sh.B, "T=%d: %lld tasks, plan says %lld", sh.T, t, tpb * sh.B);
        // global-row tasks: every (bh, group, split) once, in order
        for (int ng : {1, 3}) {
            for (int ns : {1, 7, 16}) {
                P.n_split = ns;
                P.n_ggroups = ng;
                P.mg_per_bh = magic_for((long long)ns * ng);
                P.mg_nsplit = magic_for(ns);
                long long g = 0;
                for (int bh = 0; bh < sh.B * sh.H; bh++)
                    for (int grp = 0; grp < ng; grp++)
                        for (int sp = 0; sp < ns; sp++, g++) {
                            const RowTask k = decode_rows(P, (int)g);
                            CHECK(k.bh == bh && k.grp == grp && k.split == sp, "row task %lld", g);
                            CHECK(mdiv(bh, P.mg_H) == bh / sh.H, "bh / H");
                            checked++;
                        }
            }
        }
        // workgroup slots -> tasks: with equal radii (an eighth per die) and
        // with unequal ones (runs cut by cost), every task exactly once
        for (int unequal = 0; unequal < 2; unequal++) {
            for (int h = 0; h < sh.H; h++) P.rad[h] = unequal ? (int32_t)(rng() % 600) : 256;
            P.one_sided = (int)(rng() % 2);
            P.n_split = 1 + (int)(rng() % 9);
            P.n_ggroups = 1 + (int)(rng() % 3);
            P.n_band_tasks = (int)(tpb * sh.B);
            P.n_tasks = P.n_band_tasks + (rng() % 2 ? sh.B * sh.H * P.n_split * P.n_ggroups : 0);
            split_by_cost(P);
            const bool cut = P.band_die[8] > 0;
            CHECK(cut == (unequal && sh.H > 1 && P.n_band_tasks > 0 && [&] {
                      for (int h = 1; h < sh.H; h++) if (P.rad[h] != P.rad[0]) return true;
                      return false; }()), "T=%d: cost cut %d", sh.T, (int)cut);
            const int spd = slots_per_die(P);
            for (int first = 0; first < 2; first++) {
                std::vector<int> hits(P.n_tasks, 0);
                for (int x = 0; x < 8; x++)
                    for (int sl = 0; sl < spd; sl++) {
                        const int t = task_of_slot(P, x, sl, first != 0);
                        CHECK(t >= -1 && t < P.n_tasks, "slot (%d,%d) -> %d", x, sl, t);
                        if (t >= 0 && t < P.n_tasks) hits[t]++;
                        // the global-row tasks of a die come first, or last
                        if (t >= 0 && sl > 0) {
                            const int tp = task_of_slot(P, x, sl - 1, first != 0);
                            const bool g = t >= P.n_band_tasks, gp = tp >= P.n_band_tasks;
                            CHECK(tp >= 0 && (first ? (!g || gp) : (g || !gp)), "die %d: task order", x);
                        }
                    }
                for (int t = 0; t < P.n_tasks; t++)
                    CHECK(hits[t] == 1, "T=%d: task %d taken %d times", sh.T, t, hits[t]);
                checked += P.n_tasks;
            }
            if (cut) {
                for (int x = 0; x < 8; x++)
                    CHECK(P.band_die[x] <= P.band_die[x + 1] && P.glob_die[x] <= P.glob_die[x + 1], "runs not ordered");
                // a head's global-row tasks sit on the die of the middle of its band tiles
                const int per_bh = P.n_split * P.n_ggroups;
                for (int x = 0; x < 8 && P.n_tasks > P.n_band_tasks; x++)
                    for (int g = P.glob_die[x]; g < P.glob_die[x + 1]; g++) {
                        const int bh = g / per_bh, b = bh / sh.H, h = bh % sh.H;
                        const long long mid = (long long)b * tpb + (P.head_start[h] + P.head_start[h + 1]) / 2;
                        CHECK(mid >= P.band_die[x] && (mid < P.band_die[x + 1] || x == 7), "head %d off its die", bh);
                    }
            }
        }
    }
    // ---- the global-row split plan: splits cover [0, T) exactly, lengths are
    // multiples of 32 of at least 64 keys (or the whole 32-rounded sequence),
    // at most 64 splits, no split over 4096 keys unless 64 splits cannot
    // cover T otherwise, and about 144 tasks when T is short enough (between
    // half and all of them: lengths rounded up to 32 keys make fewer splits)
    {
        std::vector<int> Ts = {1, 31, 32, 33, 63, 64, 65, 100, 128, 700, 1000, 1024, 4095, 4096, 4097, 8192,
                               16384, 65536, 262143, 262144, 262145, 1 << 20, (1 << 24) - 1};
        for (int i = 0; i < 300; i++) Ts.push_back(1 + (int)(rng() % (1 << 24)));
        std::vector<long long> pers = {1, 2, 3, 11, 12, 13, 47, 48, 64, 143, 144, 145, 1000, 1LL << 20};
        for (int T : Ts)
            for (long long per : pers) {
                int sl = 0, ns = 0;
                global_splits(per, T, &sl, &ns);
                const long long T32 = ((long long)T + 31) / 32 * 32;
                CHECK(sl % 32 == 0 && (sl >= 64 || sl == T32), "T %d per %lld: split %d", T, per, sl);
                CHECK(ns >= 1 && ns <= 64, "T %d per %lld: %d splits", T, per, ns);
                CHECK((long long)ns * sl >= T && (long long)(ns - 1) * sl < T, "T %d per %lld: %d x %d", T, per, ns, sl);
                CHECK(sl <= 4096 || (long long)T > 64LL * 4096 || sl == T32, "T %d per %lld: split %d", T, per, sl);
                if ((long long)T <= 4096 && per <= 144 && T >= 64LL * 144 / per)
                    CHECK(2 * per * ns >= 144 - per && per * ns <= 144 + per, "T %d per %lld: %lld tasks", T, per, per * ns);
                checked++;
            }
        // the headline shape: B1 H12, one global, T = 4096 -> 12 splits of 352 keys
        int sl = 0, ns = 0;
        global_splits(12, 4096, &sl, &ns);
        CHECK(sl == 352 && ns == 12, "headline split %d x %d", ns, sl);
    }
    if (fails) {
        std::printf("FAILED %d\n", fails);
        return 1;
    }
    std::printf("OK %lld\n", checked);
    return 0;
}
