// lf_host.cpp -- the C ABI of liblfattn.so: argument checks, the global-set
// normalisation, task planning, the per-stream workspace and the launches.
//
// Every argument check runs before the first HIP call, so a rejected call
// enqueues nothing and leaves `out` untouched (and works without a GPU).

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "lf_attn.h"
#include "lf_kernels.h"
#include "lf_decode.h"
#include "lf_bwd.h"

extern "C" hipError_t lfk_launch(const lfk::Args *A, const lfk::Plan *P, int dtype_bf16, void *stream);
extern "C" int lfk_supports_d(int d);
extern "C" hipError_t lfk_noalloc_scratch(void **ptr);
extern "C" hipError_t lfk_write_plan(const void *plan, size_t bytes, void *dst, int *zero, int n_zero, void *stream);
extern "C" hipError_t lfk_bwd_launch(const lfk::BwdArgs *A, const void *const *t, int d, int bf16, void *stream);
extern "C" hipError_t lfk_bwd_dq(const lfk::BwdBandArgs *A, const lfk::Plan *P, void *stream);
extern "C" hipError_t lfk_bwd_dkdv(const lfk::BwdBandArgs *A, const lfk::Plan *P, void *stream);

namespace {

thread_local std::string g_err;

lf_status_t fail(lf_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Device workspaces, one set per (device, stream): calls on one stream are
// ordered, so they can share it; calls on other streams get their own.
//
//  * counters: the global-row completion counters, one int per (b, h).  They
//    must read zero at the start of every call: the allocation is zeroed
//    and every call's kernel returns each counter it uses to zero.  Nothing
//    else is ever stored there.
//  * scratch: the global-row partials and, for fp32 input, the bf16 planes
//    of K and V; no contents carry over between calls.
//  * plan, aux, bwd: device copies of the call's lfk::Plan, random-block
//    table and backward tables, kSlots of each keyed by content (plus one
//    more for each slot a captured graph holds), so that calls alternating
//    between a few configurations reuse them.  A missing one is written
//    into the least recently used free slot by a small kernel
//    that carries the bytes in its arguments: the write is ordered on the
//    stream like the kernels that read it, the host never waits for it, and
//    a write recorded in a graph replays with its own bytes.
//
// No call waits for the device.  A buffer too small for a call is replaced;
// the old one is released once an event recorded after the work that used
// it has passed (checked at later calls).  During stream capture nothing
// is allocated or released: a call that needs a larger buffer is refused.
// Whatever a captured call used (buffers, slots) is pinned: never released
// or overwritten with other contents, so that the graph stays valid while
// later calls on the stream move on to other buffers and slots.  A slot
// written during capture holds its contents only once the graph has run,
// so other calls do not use it.
constexpr int kSlots = 4;

struct Buffer {
    void *ptr = nullptr;
    size_t bytes = 0;
    bool pinned = false;
};
struct Slot {
    Buffer buf;
    std::vector<uint32_t> shadow;   // what buf holds, if valid
    bool valid = false;
    uint64_t used = 0;              // call count at the last use (least recently used goes first)
};
struct Retired {
    void *ptr;
    hipEvent_t done;
};
struct Workspace {
    Buffer counters, scratch;
    std::vector<Slot> plan = std::vector<Slot>(kSlots), aux = std::vector<Slot>(kSlots),
                      bwd = std::vector<Slot>(kSlots);
    Buffer bwd_stats, bwd_gpart;   // backward: row statistics; global-split records
    Buffer bwd_count;              // backward (bf16): the global tasks' completion counters
    Buffer bwd_fwd;                // backward (bf16) without the forward's results: its output and lse
    std::vector<Retired> retired;
    uint64_t calls = 0;
    bool capturing = false;        // the current call is being captured
};
std::mutex g_ws_mu;
std::map<std::pair<int, void *>, Workspace> g_ws;

// release the retired buffers whose work has finished
void reap(Workspace &w) {
    size_t k = 0;
    for (size_t i = 0; i < w.retired.size(); i++) {
        if (hipEventQuery(w.retired[i].done) == hipSuccess) {
            (void)hipFree(w.retired[i].ptr);
            (void)hipEventDestroy(w.retired[i].done);
        } else {
            w.retired[k++] = w.retired[i];
        }
    }
    w.retired.resize(k);
}

// give up b: freed once the stream has passed the work enqueued so far, or
// kept for good when a captured graph refers to it
lf_status_t retire(Workspace &w, Buffer &b, void *stream) {
    if (b.ptr && !b.pinned) {
        hipEvent_t ev;
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventRecord(ev, (hipStream_t)stream);
        if (e != hipSuccess) return fail(LF_E_HIP, "retiring a workspace buffer: %s", hipGetErrorString(e));
        w.retired.push_back({b.ptr, ev});
    }
    b = Buffer();
    return LF_OK;
}

// b holds at least `bytes` bytes (zeroed when first allocated if `zero`);
// during capture it must already, and is pinned
lf_status_t grow(Workspace &w, Buffer &b, size_t bytes, bool zero, void *stream) {
    if (b.bytes >= bytes) {
        if (w.capturing) b.pinned = true;
        return LF_OK;
    }
    if (w.capturing)
        return fail(LF_E_UNSUPPORTED,
                    "this call needs a larger workspace than the stream has during stream capture; make one "
                    "call of this size on the stream outside capture first");
    lf_status_t st = retire(w, b, stream);
    if (st != LF_OK) return st;
    const size_t want = std::max(bytes, (size_t)1 << 16);
    hipError_t e = hipMalloc(&b.ptr, want);
    if (e != hipSuccess) {
        b.ptr = nullptr;
        (void)hipGetLastError();
        return fail(LF_E_NOMEM, "workspace of %zu bytes: %s", want, hipGetErrorString(e));
    }
    if (zero) {
        e = hipMemsetAsync(b.ptr, 0, want, (hipStream_t)stream);
        if (e != hipSuccess) {
            (void)hipFree(b.ptr);
            b.ptr = nullptr;
            return fail(LF_E_HIP, "hipMemsetAsync: %s", hipGetErrorString(e));
        }
    }
    b.bytes = want;
    return LF_OK;
}

// the workspace of the calling thread's device and `stream`, its retired
// buffers reaped and its capture state taken
Workspace *workspace_for(void *stream, lf_status_t *st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *st = fail(LF_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing((hipStream_t)stream, &cs);
    if (e != hipSuccess) {
        *st = fail(LF_E_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
        return nullptr;
    }
    Workspace *w = &g_ws[std::make_pair(dev, stream)];
    w->capturing = cs != hipStreamCaptureStatusNone;
    w->calls++;
    if (!w->capturing) reap(*w);
    *st = LF_OK;
    return w;
}

// A device copy of `words` among the slots: an existing one when a slot
// holds it, else written into the least recently used unpinned slot.  A
// slot held by a graph is replaced by a new one (outside capture), so that
// eager calls always keep kSlots free slots.
lf_status_t put_table(Workspace &w, std::vector<Slot> &slots, const uint32_t *words, size_t n, void *stream,
                      const void **dev, const char *what) {
    for (Slot &sl : slots)
        if (sl.valid && sl.shadow.size() == n && std::memcmp(sl.shadow.data(), words, n * 4) == 0) {
            sl.used = w.calls;
            if (w.capturing) sl.buf.pinned = true;
            *dev = sl.buf.ptr;
            return LF_OK;
        }
    int free_slots = 0;
    for (const Slot &sl : slots) free_slots += !sl.buf.pinned;
    if (free_slots < kSlots && !w.capturing) slots.emplace_back();
    Slot *victim = nullptr;
    for (Slot &sl : slots) {
        if (sl.buf.pinned) continue;
        if (!victim || !sl.valid || (victim->valid && sl.used < victim->used)) victim = &sl;
        if (!victim->valid) break;
    }
    if (!victim)
        return fail(LF_E_UNSUPPORTED,
                    "every %s slot of this stream is held by a captured graph; make one identical call on the "
                    "stream outside capture first", what);
    // a slot is never grown during capture: it is allocated large enough first
    if (victim->buf.bytes < n * 4) {
        if (w.capturing)
            return fail(LF_E_UNSUPPORTED,
                        "the %s of this call needs a new slot during stream capture; make one identical call on "
                        "the stream outside capture first", what);
        lf_status_t st = grow(w, victim->buf, n * 4, false, stream);
        if (st != LF_OK) return st;
    }
    hipError_t e = lfk_write_plan(words, n * 4, victim->buf.ptr, nullptr, 0, stream);
    if (e != hipSuccess) {
        victim->valid = false;
        return fail(LF_E_HIP, "%s upload: %s", what, hipGetErrorString(e));
    }
    victim->used = w.calls;
    if (w.capturing) {
        // holds the words only once the graph runs
        victim->buf.pinned = true;
        victim->valid = false;
        victim->shadow.clear();
    } else {
        victim->shadow.assign(words, words + n);
        victim->valid = true;
    }
    *dev = victim->buf.ptr;
    return LF_OK;
}

// device copy of *P on this stream's workspace
lf_status_t upload_plan(Workspace &w, const lfk::Plan &P, void *stream, const lfk::Plan **dev_plan) {
    const void *dev = nullptr;
    lf_status_t st = put_table(w, w.plan, (const uint32_t *)&P, sizeof P / 4, stream, &dev, "plan");
    *dev_plan = (const lfk::Plan *)dev;
    return st;
}

}  // namespace

extern "C" const char *lf_last_error(void) { return g_err.c_str(); }

#ifndef LF_SOURCE_HASH
#define LF_SOURCE_HASH "unset"
#endif
extern "C" const char *lf_build_hash(void) { return LF_SOURCE_HASH; }

namespace {

// Argument checks of a forward call (no HIP call): radius is NULL (r for
// every head) or one radius per head.
lf_status_t check_fwd(const void *q, const void *k, const void *v, int B, int H, int T, int d, int r,
                      const int32_t *radius, int one_sided, const int32_t *rand_blocks, int n_rand,
                      const int32_t *dilation, const int32_t *global_idx, int n_global, const void *out,
                      const float *lse, lf_dtype_t dtype) {
    if (!q || !k || !v || !out) return fail(LF_E_INVALID, "q, k, v and out must be non-null");
    if (dtype != LF_F32 && dtype != LF_BF16) return fail(LF_E_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (B < 1 || H < 1 || T < 1) return fail(LF_E_INVALID, "B, H, T must be >= 1 (got %d, %d, %d)", B, H, T);
    if (!lfk_supports_d(d)) return fail(LF_E_UNSUPPORTED, "head dimension %d: only 32, 64 and 128 are built", d);
    if (H > LF_MAX_HEADS) return fail(LF_E_UNSUPPORTED, "H = %d exceeds %d", H, LF_MAX_HEADS);
    if (T > LF_MAX_SEQ) return fail(LF_E_UNSUPPORTED, "T = %d exceeds %d", T, LF_MAX_SEQ);
    {
        // one head's rows as the kernels address them (the fp32 input, or its
        // three bf16 planes) must stay below 2^31 bytes
        const long long row = dtype == LF_BF16 ? 2LL * d : 6LL * d;
        if ((long long)T * row >= (1LL << 31))
            return fail(LF_E_UNSUPPORTED, "T = %d with d = %d: one head exceeds the 2 GiB a kernel addresses", T, d);
    }
    if (r < 0) return fail(LF_E_INVALID, "window radius r = %d must be >= 0", r);
    if (one_sided != 0 && one_sided != 1) return fail(LF_E_INVALID, "one_sided = %d must be 0 or 1", one_sided);
    if (radius)
        for (int h = 0; h < H; h++)
            if (radius[h] < 0) return fail(LF_E_INVALID, "radius[%d] = %d must be >= 0", h, radius[h]);
    if (n_global < 0) return fail(LF_E_INVALID, "n_global = %d must be >= 0", n_global);
    if (n_global > 0 && !global_idx) return fail(LF_E_INVALID, "global_idx is NULL with n_global = %d", n_global);
    if (dilation) {
        for (int h = 0; h < H; h++) {
            if (dilation[h] < 1) return fail(LF_E_INVALID, "dilation[%d] = %d must be >= 1", h, dilation[h]);
            if (dilation[h] > LF_MAX_DILATION)
                return fail(LF_E_UNSUPPORTED, "dilation[%d] = %d exceeds %d", h, dilation[h], LF_MAX_DILATION);
        }
    }
    for (int i = 0; i < n_global; i++)
        if (global_idx[i] < 0 || global_idx[i] >= T)
            return fail(LF_E_INVALID, "global_idx[%d] = %d outside [0, %d)", i, global_idx[i], T);
    const long long nqb = cdiv(T, 64);
    if (n_rand < 0) return fail(LF_E_INVALID, "n_rand = %d must be >= 0", n_rand);
    if (n_rand > 0) {
        if (!rand_blocks) return fail(LF_E_INVALID, "rand_blocks is NULL with n_rand = %d", n_rand);
        if (n_rand > LF_MAX_RAND_BLOCKS)
            return fail(LF_E_UNSUPPORTED, "n_rand = %d exceeds %d", n_rand, LF_MAX_RAND_BLOCKS);
        for (int h = 0; h < H; h++)
            if (dilation && dilation[h] != 1)
                return fail(LF_E_UNSUPPORTED, "random key blocks need undilated heads (dilation[%d] = %d)", h,
                            dilation[h]);
        for (long long e = 0; e < (long long)H * nqb * n_rand; e++)
            if (rand_blocks[e] < 0 || rand_blocks[e] >= nqb)
                return fail(LF_E_INVALID, "rand_blocks[%lld] = %d outside [0, %lld)", e, rand_blocks[e], nqb);
    }
    const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u;
    if (mis) return fail(LF_E_INVALID, "q, k, v and out must be 16-byte aligned");
    if (((uintptr_t)lse & 3u) != 0) return fail(LF_E_INVALID, "lse must be 4-byte aligned");
    const size_t esize = dtype == LF_BF16 ? 2 : 4;
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)T * (size_t)d * esize;
    if ((size_t)B * (size_t)H > (size_t)1 << 24)
        return fail(LF_E_UNSUPPORTED, "B*H = %lld too large", (long long)B * H);
    if (overlaps(out, nbytes, q, nbytes) || overlaps(out, nbytes, k, nbytes) || overlaps(out, nbytes, v, nbytes))
        return fail(LF_E_INVALID, "out overlaps q, k or v");
    const size_t lbytes = (size_t)B * (size_t)H * (size_t)T * sizeof(float);
    if (lse && (overlaps(lse, lbytes, q, nbytes) || overlaps(lse, lbytes, k, nbytes) ||
                overlaps(lse, lbytes, v, nbytes) || overlaps(lse, lbytes, out, nbytes)))
        return fail(LF_E_INVALID, "lse overlaps q, k, v or out");

    return LF_OK;
}

// What a forward call needs besides its tensors: the plan (workspace
// pointers still unset), the random-block table with the global bitmap, and
// the sizes of its workspace parts.
struct FwdPlan {
    lfk::Plan P;
    std::vector<uint32_t> aux;   // rtab [H][ceil(T/64)][n_rand], then the global bitmap [ceil(T/32)]
    size_t cnt_bytes = 0;        // global-row completion counters
    size_t scratch_bytes = 0;    // global-row partial records, then (fp32) the planes of K and V
    size_t planes_off = 0, plane_bytes = 0;
};

// The plan of a checked forward call (no HIP call).
lf_status_t plan_fwd(int B, int H, int T, int d, int r, const int32_t *radius, int one_sided,
                     const int32_t *rand_blocks, int n_rand, const int32_t *dilation, const int32_t *global_idx,
                     int n_global, lf_dtype_t dtype, FwdPlan &F) {
    const long long nqb = cdiv(T, 64);
    const size_t esize = dtype == LF_BF16 ? 2 : 4;
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)T * (size_t)d * esize;
    // ---- normalise G: a set of positions, ascending
    std::vector<int32_t> G(global_idx, global_idx + n_global);
    std::sort(G.begin(), G.end());
    G.erase(std::unique(G.begin(), G.end()), G.end());
    if ((int)G.size() > LF_MAX_GLOBALS)
        return fail(LF_E_UNSUPPORTED, "%zu distinct globals exceed %d", G.size(), LF_MAX_GLOBALS);

    // ---- plan
    constexpr int BM = LFK_BM;
    lfk::Plan &P = F.P;
    std::memset(&P, 0, sizeof P);
    P.B = B; P.H = H; P.T = T; P.d = d;
    // |i - j| < T always, so radii beyond T change nothing
    P.r = 0;
    for (int h = 0; h < H; h++) {
        const int rh = radius ? radius[h] : r;
        P.rad[h] = rh < T ? rh : T;
        P.r = std::max(P.r, P.rad[h]);
    }
    P.one_sided = one_sided;
    // random key blocks: each query block's list sorted, duplicates dropped
    // (-1 fills the rest), then a bitmap of the global positions (a random
    // block leaves the globals to their own path)
    std::vector<uint32_t> &aux = F.aux;
    aux.clear();
    if (n_rand > 0) {
        const size_t nt = (size_t)H * nqb * n_rand;
        aux.resize(nt + (size_t)cdiv(T, 32), 0u);
        std::vector<int32_t> row(n_rand);
        for (size_t base = 0; base < nt; base += n_rand) {
            std::copy(rand_blocks + base, rand_blocks + base + n_rand, row.begin());
            std::sort(row.begin(), row.end());
            const size_t u = std::unique(row.begin(), row.end()) - row.begin();
            for (int e = 0; e < n_rand; e++) aux[base + e] = (uint32_t)(e < (int)u ? row[e] : -1);
        }
        for (int g : G) aux[nt + (g >> 5)] |= 1u << (g & 31);
    }
    P.n_rand = n_rand;
    P.n_g = (int)G.size();
    for (int i = 0; i < P.n_g; i++) P.glob[i] = G[i];
    const long long start = lfk::fill_band_plan(P, B, H, T, dilation);
    const long long n_band = (long long)B * start;
    long long n_glob_tasks = 0;
    size_t &cnt_bytes = F.cnt_bytes, &scratch_bytes = F.scratch_bytes;
    cnt_bytes = scratch_bytes = 0;
    if (P.n_g > 0) {
        P.n_ggroups = (int)cdiv(P.n_g, BM);
        P.g_pad = P.n_ggroups * BM;
        lfk::global_splits((long long)B * H * P.n_ggroups, T, &P.split_len, &P.n_split);
        n_glob_tasks = (long long)B * H * P.n_split * P.n_ggroups;
        P.mg_per_bh = lfk::magic_for((long long)P.n_split * P.n_ggroups);
        P.mg_nsplit = lfk::magic_for(P.n_split);
        cnt_bytes = (size_t)B * H * sizeof(int);
        // partial records of d + 4 floats: O[d], m, l, 0, 0
        scratch_bytes = (size_t)B * H * P.n_split * P.g_pad * (size_t)(d + 4) * sizeof(float);
    }
    if (n_band + n_glob_tasks > (1LL << 30))
        return fail(LF_E_UNSUPPORTED, "problem needs %lld workgroups", n_band + n_glob_tasks);
    P.n_band_tasks = (int)n_band;
    P.n_tasks = (int)(n_band + n_glob_tasks);
    lfk::split_by_cost(P);
    // Backward: a die's global tasks go after its band tiles and fill the
    // tail of their last round, unless they are the longer kind (a split
    // longer than a band tile's key range), which then start first.
    P.bwd_globals_first = P.n_g > 0 && P.split_len > (one_sided ? P.r : 2 * P.r) + BM;
    // fp32: K and V are split into three bf16 planes per row (1.5 times the
    // fp32 tensors' bytes) ahead of the tile kernel
    F.planes_off = 0;
    F.plane_bytes = nbytes / 4 * 6;
    if (dtype == LF_F32) {
        if ((long long)B * H * T * (d / 8) / 256 >= (1LL << 31))
            return fail(LF_E_UNSUPPORTED, "fp32 problem too large for the plane split");
        F.planes_off = (scratch_bytes + 255) / 256 * 256;
        scratch_bytes = F.planes_off + 2 * F.plane_bytes;
    }

    return LF_OK;
}

// With g_ws_mu held: the stream's workspace for the plan (counters,
// partials, planes, random-block table) and the plan on the device.
lf_status_t bind_fwd(Workspace &w, FwdPlan &F, bool fp32, void *stream, const lfk::Plan **dev_plan) {
    if (F.scratch_bytes > 0) {
        lf_status_t st = grow(w, w.counters, F.cnt_bytes, true, stream);
        if (st != LF_OK) return st;
        st = grow(w, w.scratch, F.scratch_bytes, false, stream);
        if (st != LF_OK) return st;
        char *ws = (char *)w.scratch.ptr;
        if (F.P.n_g > 0) {
            F.P.counter = (int *)w.counters.ptr;
            F.P.part = (float *)ws;
        }
        if (fp32) {
            F.P.kp = ws + F.planes_off;
            F.P.vp = ws + F.planes_off + F.plane_bytes;
        }
    }
    if (F.P.n_rand > 0) {
        const void *dev = nullptr;
        lf_status_t st = put_table(w, w.aux, F.aux.data(), F.aux.size(), stream, &dev, "random-block table");
        if (st != LF_OK) return st;
        F.P.rtab = (const int32_t *)dev;
        F.P.gmap = (const uint32_t *)dev + (size_t)F.P.H * cdiv(F.P.T, 64) * F.P.n_rand;
    }
    return upload_plan(w, F.P, stream, dev_plan);
}

// The kernel argument's decode fields: set when every head has the same
// stride and radius (the plan's per-head tables are then not read to find
// a task), else off.
lfk::FastDecode fast_decode(const lfk::Plan &P) {
    lfk::FastDecode f;
    std::memset(&f, 0, sizeof f);
    for (int h = 1; h < P.H; h++)
        if (P.dil[h] != P.dil[0] || P.rad[h] != P.rad[0]) return f;
    f.on = 1;
    f.n_band = P.n_band_tasks;
    f.n_tasks = P.n_tasks;
    f.tph = P.head_start[1];
    f.mg_tph = lfk::magic_for(f.tph);
    f.mg_H = P.mg_H;
    f.H = P.H;
    f.T = P.T;
    f.delta = P.dil[0];
    f.r = P.rad[0];
    f.ra = P.one_sided ? 0 : P.rad[0];
    f.hq = P.hq[0];
    f.hrem = P.hrem[0];
    f.htb = P.htb[0];
    f.hts = P.hts[0];
    f.mg_htb = P.mg_tb[0];
    f.mg_hts = P.mg_ts[0];
    f.n_g = P.n_g;
    f.n_split = P.n_split;
    f.n_ggroups = P.n_ggroups;
    f.split_len = P.split_len;
    f.mg_per_bh = P.mg_per_bh;
    f.mg_nsplit = P.mg_nsplit;
    return f;
}

// The call behind the forward entry points: radius is NULL (r for every
// head) or one radius per head.
lf_status_t attn_fwd(const void *q, const void *k, const void *v, int B, int H, int T, int d, int r,
                     const int32_t *radius, int one_sided, const int32_t *rand_blocks, int n_rand,
                     const int32_t *dilation, const int32_t *global_idx, int n_global,
                     const uint8_t *key_padding_mask, void *out, float *lse, lf_dtype_t dtype, void *stream,
                     bool noalloc = false, bool global_rows_only = false) {
    g_err.clear();
    // no HIP call before every check has passed
    lf_status_t st = check_fwd(q, k, v, B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation,
                               global_idx, n_global, out, lse, dtype);
    if (st != LF_OK) return st;
    if (global_rows_only && n_global == 0) return LF_OK;
    FwdPlan F;
    st = plan_fwd(B, H, T, d, r, radius, one_sided, rand_blocks, n_rand, dilation, global_idx, n_global, dtype, F);
    if (st != LF_OK) return st;
    lfk::Plan &P = F.P;
    if (noalloc) {
        // the static scratch array: plan, counters, partial records, planes
        auto up = [](size_t x) { return (x + 255) / 256 * 256; };
        const size_t plan_bytes = up(sizeof(lfk::Plan));
        const size_t cnt_off = plan_bytes, part_off = cnt_off + up(F.cnt_bytes);
        const size_t total = part_off + F.scratch_bytes;
        if (n_rand > 0) return fail(LF_E_UNSUPPORTED, "random key blocks are not taken without allocation");
        if (total > (size_t)LF_NOALLOC_SCRATCH_BYTES)
            return fail(LF_E_UNSUPPORTED,
                        "this call needs a workspace of %zu bytes; the allocation-free entry point has %d",
                        total, (int)LF_NOALLOC_SCRATCH_BYTES);
        void *base = nullptr;
        hipError_t e = lfk_noalloc_scratch(&base);
        if (e != hipSuccess) return fail(LF_E_HIP, "scratch address: %s", hipGetErrorString(e));
        char *ws = (char *)base + part_off;
        if (P.n_g > 0) {
            P.counter = (int *)((char *)base + cnt_off);
            P.part = (float *)ws;
        }
        if (dtype == LF_F32) {
            P.kp = ws + F.planes_off;
            P.vp = ws + F.planes_off + F.plane_bytes;
        }
        e = lfk_write_plan(&P, sizeof P, base, P.n_g > 0 ? P.counter : nullptr, P.n_g > 0 ? B * H : 0, stream);
        if (e != hipSuccess) return fail(LF_E_HIP, "plan copy launch: %s", hipGetErrorString(e));
        lfk::Args A{};
        A.q = q; A.k = k; A.v = v; A.out = out;
        A.pad = key_padding_mask;
        A.lse = lse;
        A.plan = (const lfk::Plan *)base;
        A.fd = fast_decode(P);
        e = lfk_launch(&A, &P, dtype == LF_BF16, stream);
        if (e != hipSuccess) return fail(LF_E_HIP, "kernel launch: %s", hipGetErrorString(e));
        return LF_OK;
    }

    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace *w = workspace_for(stream, &st);
    if (!w) return st;
    lfk::Args A{};
    A.q = q; A.k = k; A.v = v; A.out = out;
    A.pad = key_padding_mask;
    A.lse = lse;
    A.global_rows_only = global_rows_only;
    st = bind_fwd(*w, F, dtype == LF_F32, stream, &A.plan);
    if (st != LF_OK) return st;
    A.fd = fast_decode(P);
    hipError_t e = lfk_launch(&A, &P, dtype == LF_BF16, stream);
    if (e != hipSuccess) return fail(LF_E_HIP, "kernel launch: %s", hipGetErrorString(e));
    return LF_OK;
}

// Gradients (lf_attn_bwd, lf_attn_bwd_ex): checks, the tables, the launches.
// bf16: the forward's output and lse (given, or computed here into the
// workspace), then the two matrix-core kernels: dq (it also writes the row
// statistics and takes the global rows as split tasks), then dk and dv (the
// global keys likewise).  fp32: the vector kernels, which find the
// statistics themselves (out and lse are not read).
lf_status_t attn_bwd(const void *q, const void *k, const void *v, const void *dy, const void *out,
                     const float *lse, int B, int H, int T, int d, const int32_t *radius, int one_sided,
                     const int32_t *rand_blocks, int n_rand, const int32_t *dilation, const int32_t *global_idx,
                     int n_global, const uint8_t *key_padding_mask, void *dq, void *dk, void *dv, lf_dtype_t dtype,
                     void *stream) {
    if (!q || !k || !v || !dy || !dq || !dk || !dv)
        return fail(LF_E_INVALID, "q, k, v, dy, dq, dk and dv must be non-null");
    if ((out == nullptr) != (lse == nullptr))
        return fail(LF_E_INVALID, "out and lse are given together or not at all");
    if (!radius) return fail(LF_E_INVALID, "radius must be a host array of H radii");
    if (dtype != LF_F32 && dtype != LF_BF16) return fail(LF_E_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (B < 1 || H < 1 || T < 1) return fail(LF_E_INVALID, "B, H, T must be >= 1 (got %d, %d, %d)", B, H, T);
    if (!lfk_supports_d(d)) return fail(LF_E_UNSUPPORTED, "head dimension %d: only 32, 64 and 128 are built", d);
    if (H > LF_MAX_HEADS) return fail(LF_E_UNSUPPORTED, "H = %d exceeds %d", H, LF_MAX_HEADS);
    if (T > LF_MAX_SEQ) return fail(LF_E_UNSUPPORTED, "T = %d exceeds %d", T, LF_MAX_SEQ);
    if (one_sided != 0 && one_sided != 1) return fail(LF_E_INVALID, "one_sided = %d must be 0 or 1", one_sided);
    for (int h = 0; h < H; h++)
        if (radius[h] < 0) return fail(LF_E_INVALID, "radius[%d] = %d must be >= 0", h, radius[h]);
    if (n_global < 0) return fail(LF_E_INVALID, "n_global = %d must be >= 0", n_global);
    if (n_global > 0 && !global_idx) return fail(LF_E_INVALID, "global_idx is NULL with n_global = %d", n_global);
    if (dilation)
        for (int h = 0; h < H; h++) {
            if (dilation[h] < 1) return fail(LF_E_INVALID, "dilation[%d] = %d must be >= 1", h, dilation[h]);
            if (dilation[h] > LF_MAX_DILATION)
                return fail(LF_E_UNSUPPORTED, "dilation[%d] = %d exceeds %d", h, dilation[h], LF_MAX_DILATION);
        }
    for (int i = 0; i < n_global; i++)
        if (global_idx[i] < 0 || global_idx[i] >= T)
            return fail(LF_E_INVALID, "global_idx[%d] = %d outside [0, %d)", i, global_idx[i], T);
    const long long nqb = cdiv(T, 64);
    if (n_rand < 0) return fail(LF_E_INVALID, "n_rand = %d must be >= 0", n_rand);
    if (n_rand > 0) {
        if (!rand_blocks) return fail(LF_E_INVALID, "rand_blocks is NULL with n_rand = %d", n_rand);
        if (n_rand > LF_MAX_RAND_BLOCKS)
            return fail(LF_E_UNSUPPORTED, "n_rand = %d exceeds %d", n_rand, LF_MAX_RAND_BLOCKS);
        for (int h = 0; h < H; h++)
            if (dilation && dilation[h] != 1)
                return fail(LF_E_UNSUPPORTED, "random key blocks need undilated heads (dilation[%d] = %d)", h,
                            dilation[h]);
        for (long long e = 0; e < (long long)H * nqb * n_rand; e++)
            if (rand_blocks[e] < 0 || rand_blocks[e] >= nqb)
                return fail(LF_E_INVALID, "rand_blocks[%lld] = %d outside [0, %lld)", e, rand_blocks[e], nqb);
    }
    const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)dy | (uintptr_t)dq |
                           (uintptr_t)dk | (uintptr_t)dv) & 15u;
    if (mis) return fail(LF_E_INVALID, "q, k, v, dy, dq, dk and dv must be 16-byte aligned");
    if ((size_t)B * (size_t)H > (size_t)1 << 24)
        return fail(LF_E_UNSUPPORTED, "B*H = %lld too large", (long long)B * H);
    const size_t esize = dtype == LF_BF16 ? 2 : 4;
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)T * (size_t)d * esize;
    const void *ins[4] = {q, k, v, dy};
    void *outs[3] = {dq, dk, dv};
    for (int o = 0; o < 3; o++) {
        for (int e = 0; e < 4; e++)
            if (overlaps(outs[o], nbytes, ins[e], nbytes)) return fail(LF_E_INVALID, "dq, dk, dv overlap an input");
        for (int e = o + 1; e < 3; e++)
            if (overlaps(outs[o], nbytes, outs[e], nbytes)) return fail(LF_E_INVALID, "dq, dk, dv overlap");
    }
    if (out) {
        if (((uintptr_t)out & 15u) != 0 || ((uintptr_t)lse & 3u) != 0)
            return fail(LF_E_INVALID, "out must be 16-byte and lse 4-byte aligned");
        const size_t lbytes = (size_t)B * (size_t)H * (size_t)T * sizeof(float);
        for (int o = 0; o < 3; o++)
            if (overlaps(outs[o], nbytes, out, nbytes) || overlaps(outs[o], nbytes, lse, lbytes))
                return fail(LF_E_INVALID, "dq, dk, dv overlap out or lse");
    }
    std::vector<int32_t> G(global_idx, global_idx + n_global);
    std::sort(G.begin(), G.end());
    G.erase(std::unique(G.begin(), G.end()), G.end());
    if ((int)G.size() > LF_MAX_GLOBALS)
        return fail(LF_E_UNSUPPORTED, "%zu distinct globals exceed %d", G.size(), LF_MAX_GLOBALS);
    if ((long long)B * H * G.size() >= (1LL << 31))
        return fail(LF_E_UNSUPPORTED, "too many global rows");

    // table: rad[H] | dil[H] | head_chunk[H+1] | hord[H] | glob[n_g] | gmap[ceil(T/32)]
    //        | rtab[H][nqb][n_rand] | inv_off[H][nqb+1] | inv_list
    const size_t o_dil = H, o_hc = 2 * (size_t)H, o_ord = o_hc + H + 1, o_glob = o_ord + H;
    const size_t o_gmap = o_glob + G.size();
    const size_t o_rtab = o_gmap + (size_t)cdiv(T, 32);
    const size_t n_rt = n_rand > 0 ? (size_t)H * nqb * n_rand : 0;
    const size_t o_off = o_rtab + n_rt, n_off = n_rand > 0 ? (size_t)H * (nqb + 1) : 0;
    const size_t o_inv = o_off + n_off;
    std::vector<uint32_t> tab(o_inv, 0u);
    if (n_rand > 0) {
        // each query block's draws sorted, duplicates dropped (-1 after the
        // last), and per key block the query blocks that drew it, ascending
        std::vector<int32_t> row(n_rand);
        std::vector<std::vector<int32_t>> inv((size_t)nqb);
        for (int h = 0; h < H; h++) {
            for (auto &x : inv) x.clear();
            for (long long qb = 0; qb < nqb; qb++) {
                const size_t base = ((size_t)h * nqb + qb) * n_rand;
                std::copy(rand_blocks + base, rand_blocks + base + n_rand, row.begin());
                std::sort(row.begin(), row.end());
                const size_t u = std::unique(row.begin(), row.end()) - row.begin();
                for (int e = 0; e < n_rand; e++) tab[o_rtab + base + e] = (uint32_t)(e < (int)u ? row[e] : -1);
                for (size_t e = 0; e < u; e++) inv[row[e]].push_back((int32_t)qb);
            }
            size_t at = tab.size() - o_inv;
            for (long long kb = 0; kb < nqb; kb++) {
                tab[o_off + (size_t)h * (nqb + 1) + kb] = (uint32_t)at;
                for (int32_t qb : inv[kb]) tab.push_back((uint32_t)qb);
                at += inv[kb].size();
            }
            tab[o_off + (size_t)h * (nqb + 1) + nqb] = (uint32_t)at;
        }
    }
    // lanes per row of the vector-unit band kernels (lf_bwd.h): as few as
    // leave a lane 8 fp32 channels or 16 bf16 channels (four at the least),
    // doubled while the problem would make fewer than LFB_MIN_WAVES waves
    const long long all_rows = (long long)B * H * T;
    int lpr = std::max(4, dtype == LF_BF16 ? d / 16 : d / 8);
    while (lpr < 16 && all_rows * lpr / 64 < LFB_MIN_WAVES) lpr *= 2;
    const int rows_per_wave = 64 / lpr;
    // waves are dealt out head by head, the heads of the largest radius first
    std::vector<int> hord(H);
    for (int h = 0; h < H; h++) hord[h] = h;
    std::stable_sort(hord.begin(), hord.end(), [&](int a, int b) { return radius[a] > radius[b]; });
    long long chunks = 0;
    for (int o = 0; o < H; o++) {
        const int h = hord[o];
        const int delta = dilation ? dilation[h] : 1;
        tab[h] = (uint32_t)std::min(radius[h], T);   // |i - j| < T: larger radii change nothing
        tab[o_dil + h] = (uint32_t)delta;
        tab[o_hc + o] = (uint32_t)chunks;
        tab[o_ord + o] = (uint32_t)h;
        const long long qq = T / delta, rm = T % delta;
        chunks += rm * cdiv(qq + 1, rows_per_wave) + (delta - rm) * cdiv(qq, rows_per_wave);
    }
    tab[o_hc + H] = (uint32_t)chunks;
    if ((long long)B * chunks >= (1LL << 31)) return fail(LF_E_UNSUPPORTED, "problem needs too many waves");
    // bf16 at d = 64: the matrix-core kernels on the forward's plan (its band
    // tiles are their tiles); fp32, and bf16 at other d: the vector units
    const bool mfma = dtype == LF_BF16 && d == LF_HEAD_DIM;
    FwdPlan F;
    if (mfma) {
        lf_status_t st = plan_fwd(B, H, T, d, 0, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
                                  n_global, dtype, F);
        if (st != LF_OK) return st;
    }
    for (size_t e = 0; e < G.size(); e++) {
        tab[o_glob + e] = (uint32_t)G[e];
        tab[o_gmap + (G[e] >> 5)] |= 1u << (G[e] & 31);
    }

    std::lock_guard<std::mutex> lock(g_ws_mu);
    lf_status_t st;
    Workspace *w = workspace_for(stream, &st);
    if (!w) return st;
    st = grow(*w, w->bwd_stats, (size_t)B * H * T * 2 * sizeof(float), false, stream);
    if (st != LF_OK) return st;
    // global rows and keys (vector path): splits of a multiple of 64
    // positions (a workgroup's 64 groups of four lanes take one position
    // each in turn), as many as bring the grid to about 2048 workgroups (at
    // most 64, at least 1)
    const long long recs = (long long)B * H * (long long)G.size();
    long long want = recs > 0 ? std::min(64LL, std::max(1LL, cdiv(2048, recs))) : 1;
    want = std::min(want, cdiv(T, 64));
    const long long per_group = cdiv(T, 64 * want);
    const int split_len = (int)(64 * per_group);
    const int n_split = (int)cdiv(T, split_len);
    const size_t n_rec = (size_t)recs * n_split;
    if (n_rec >= ((size_t)1 << 31)) return fail(LF_E_UNSUPPORTED, "too many global-row splits");
    const size_t gstat_bytes = (n_rec * 16 + 255) / 256 * 256;
    if (n_rec > 0 && !mfma) {
        st = grow(*w, w->bwd_gpart, gstat_bytes + n_rec * 3 * (size_t)d * sizeof(float), false, stream);
        if (st != LF_OK) return st;
    }
    const void *dtab = nullptr;
    st = put_table(*w, w->bwd, tab.data(), tab.size(), stream, &dtab, "backward table");
    if (st != LF_OK) return st;
    const uint32_t *dt = (const uint32_t *)dtab;
    lfk::BwdArgs A;
    A.pad = key_padding_mask;
    A.gmap = dt + o_gmap;
    A.glob = (const int32_t *)dt + o_glob;
    A.rad = (const int32_t *)dt;
    A.dil = (const int32_t *)dt + o_dil;
    A.head_chunk = (const int32_t *)dt + o_hc;
    A.n_chunks = (int)chunks;
    A.hord = (const int32_t *)dt + o_ord;
    A.stats = w->bwd_stats.ptr;
    A.B = B; A.H = H; A.T = T; A.n_g = (int)G.size(); A.one_sided = one_sided;
    A.n_split = n_split;
    A.split_len = split_len;
    A.gstat = n_rec > 0 ? (float4 *)w->bwd_gpart.ptr : nullptr;
    A.gpart = n_rec > 0 ? (float *)((char *)w->bwd_gpart.ptr + gstat_bytes) : nullptr;
    A.n_rand = n_rand;
    A.lpr = lpr;
    A.rtab = n_rand > 0 ? (const int32_t *)dt + o_rtab : nullptr;
    A.inv_off = n_rand > 0 ? (const int32_t *)dt + o_off : nullptr;
    A.inv_list = n_rand > 0 ? (const int32_t *)dt + o_inv : nullptr;
    const void *t[7] = {q, k, v, dy, dq, dk, dv};
    if (!mfma) {
        hipError_t e = lfk_bwd_launch(&A, t, d, dtype == LF_BF16, stream);
        if (e != hipSuccess) return fail(LF_E_HIP, "kernel launch: %s", hipGetErrorString(e));
        return LF_OK;
    }
    const lfk::Plan *dplan = nullptr;
    st = bind_fwd(*w, F, false, stream, &dplan);
    if (st != LF_OK) return st;
    const size_t rows = (size_t)B * H * T;
    hipError_t e;
    if (!out) {
        // the forward, into the workspace: output rows, then lse
        const size_t ybytes = (nbytes + 255) / 256 * 256;
        st = grow(*w, w->bwd_fwd, ybytes + rows * sizeof(float), false, stream);
        if (st != LF_OK) return st;
        lfk::Args FA{};
        FA.q = q; FA.k = k; FA.v = v;
        FA.out = w->bwd_fwd.ptr;
        FA.pad = key_padding_mask;
        FA.lse = (float *)((char *)w->bwd_fwd.ptr + ybytes);
        FA.plan = dplan;
        FA.fd = fast_decode(F.P);
        e = lfk_launch(&FA, &F.P, 1, stream);
        if (e != hipSuccess) return fail(LF_E_HIP, "forward launch: %s", hipGetErrorString(e));
        out = FA.out;
        lse = FA.lse;
    }
    lfk::BwdBandArgs BA;
    BA.q = q; BA.k = k; BA.v = v; BA.dy = dy;
    BA.y = out;
    BA.lse = lse;
    BA.dq = dq; BA.dk = dk; BA.dv = dv;
    BA.pad = key_padding_mask;
    BA.plan = dplan;
    BA.stats = (float *)A.stats;
    BA.gmap = A.gmap;
    BA.inv_off = A.inv_off;
    BA.inv_list = A.inv_list;
    BA.part_q = BA.part_kv = nullptr;
    BA.count_q = BA.count_kv = nullptr;
    if (F.P.n_g > 0) {
        // the global tasks' partial records (64 floats a split and slot for
        // dq, 128 for dk and dv) and their two sets of completion counters
        const size_t recs = (size_t)B * H * F.P.n_split * F.P.g_pad;
        const size_t q_bytes = (recs * 64 * sizeof(float) + 255) / 256 * 256;
        st = grow(*w, w->bwd_gpart, q_bytes + recs * 128 * sizeof(float), false, stream);
        if (st != LF_OK) return st;
        st = grow(*w, w->bwd_count, 2 * (size_t)B * H * sizeof(int), true, stream);
        if (st != LF_OK) return st;
        BA.part_q = (float *)w->bwd_gpart.ptr;
        BA.part_kv = (float *)((char *)w->bwd_gpart.ptr + q_bytes);
        BA.count_q = (int *)w->bwd_count.ptr;
        BA.count_kv = BA.count_q + (size_t)B * H;
    }
    // dq first: it writes every row's statistics; the global rows and keys
    // are tasks of the two kernels
    e = lfk_bwd_dq(&BA, &F.P, stream);
    if (e != hipSuccess) return fail(LF_E_HIP, "dq launch: %s", hipGetErrorString(e));
    e = lfk_bwd_dkdv(&BA, &F.P, stream);
    if (e != hipSuccess) return fail(LF_E_HIP, "dk/dv launch: %s", hipGetErrorString(e));
    return LF_OK;
}

}  // namespace

extern "C" lf_status_t lf_attn_bwd(const void *q, const void *k, const void *v, const void *dy, int B, int H,
                                   int T, int d, const int32_t *radius, int one_sided, const int32_t *rand_blocks,
                                   int n_rand, const int32_t *dilation, const int32_t *global_idx, int n_global,
                                   const uint8_t *key_padding_mask, void *dq, void *dk, void *dv, lf_dtype_t dtype,
                                   void *stream) {
    g_err.clear();
    return attn_bwd(q, k, v, dy, nullptr, nullptr, B, H, T, d, radius, one_sided, rand_blocks, n_rand, dilation,
                    global_idx, n_global, key_padding_mask, dq, dk, dv, dtype, stream);
}

extern "C" lf_status_t lf_attn_bwd_ex(const void *q, const void *k, const void *v, const void *dy, const void *out,
                                      const float *lse, int B, int H, int T, int d, const int32_t *radius,
                                      int one_sided, const int32_t *rand_blocks, int n_rand, const int32_t *dilation,
                                      const int32_t *global_idx, int n_global, const uint8_t *key_padding_mask,
                                      void *dq, void *dk, void *dv, lf_dtype_t dtype, void *stream) {
    g_err.clear();
    return attn_bwd(q, k, v, dy, out, lse, B, H, T, d, radius, one_sided, rand_blocks, n_rand, dilation,
                    global_idx, n_global, key_padding_mask, dq, dk, dv, dtype, stream);
}

extern "C" lf_status_t lf_attn_fwd(const void *q, const void *k, const void *v, int B, int H, int T,
                                   int d, int r, const int32_t *dilation, const int32_t *global_idx,
                                   int n_global, const uint8_t *key_padding_mask, void *out,
                                   lf_dtype_t dtype, void *stream) {
    return attn_fwd(q, k, v, B, H, T, d, r, nullptr, 0, nullptr, 0, dilation, global_idx, n_global,
                    key_padding_mask, out, nullptr, dtype, stream);
}

extern "C" lf_status_t lf_attn_fwd_noalloc(const void *q, const void *k, const void *v, int B, int H, int T,
                                           int d, int r, const int32_t *dilation, const int32_t *global_idx,
                                           int n_global, const uint8_t *key_padding_mask, void *out,
                                           lf_dtype_t dtype, void *stream) {
    return attn_fwd(q, k, v, B, H, T, d, r, nullptr, 0, nullptr, 0, dilation, global_idx, n_global,
                    key_padding_mask, out, nullptr, dtype, stream, true);
}

extern "C" lf_status_t lf_attn_fwd_global_rows(const void *q, const void *k, const void *v, int B, int H, int T,
                                               int d, const int32_t *global_idx, int n_global,
                                               const uint8_t *key_padding_mask, void *out, float *lse,
                                               lf_dtype_t dtype, void *stream) {
    // a global row sees every valid key: the window takes no part (radius 0)
    return attn_fwd(q, k, v, B, H, T, d, 0, nullptr, 0, nullptr, 0, nullptr, global_idx, n_global,
                    key_padding_mask, out, lse, dtype, stream, false, true);
}

extern "C" lf_status_t lf_attn_fwd_ex(const void *q, const void *k, const void *v, int B, int H, int T,
                                      int d, const int32_t *radius, int one_sided, const int32_t *rand_blocks,
                                      int n_rand, const int32_t *dilation, const int32_t *global_idx,
                                      int n_global, const uint8_t *key_padding_mask, void *out, float *lse,
                                      lf_dtype_t dtype, void *stream) {
    g_err.clear();
    if (!radius) return fail(LF_E_INVALID, "radius must be a host array of H radii");
    return attn_fwd(q, k, v, B, H, T, d, 0, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
                    n_global, key_padding_mask, out, lse, dtype, stream);
}
