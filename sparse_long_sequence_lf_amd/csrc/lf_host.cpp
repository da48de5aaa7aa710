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
#include "lf_bwd.h"

extern "C" hipError_t lfk_launch(const lfk::Args *A, const lfk::Plan *P, int dtype_bf16, void *stream);
extern "C" hipError_t lfk_bwd_launch(const lfk::BwdArgs *A, const void *const *t, int dtype_bf16, void *stream);

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
//  * scratch: the global-row partials and, for fp32 input, the bf16 hi/lo
//    planes of K and V; no contents carry over between calls.
//  * plan: the device copy of the call's lfk::Plan, with a host shadow of
//    what it holds; it is re-uploaded (in stream order) only when it changes.
//
// Buffers only grow; an old buffer is released after the stream has drained it.
struct Buffer {
    void *ptr = nullptr;
    size_t bytes = 0;
};
struct Workspace {
    Buffer counters, scratch, plan, aux;
    lfk::Plan shadow;
    bool shadow_valid = false;
    std::vector<uint32_t> aux_shadow;   // what aux holds: random-block table and global bitmap
    Buffer bwd_tab, bwd_stats, bwd_gpart;   // backward: tables; row statistics; global-split records
    std::vector<uint32_t> bwd_shadow;   // what bwd_tab holds
};
std::mutex g_ws_mu;
std::map<std::pair<int, void *>, Workspace> g_ws;

lf_status_t grow(Buffer &b, size_t bytes, bool zero, void *stream) {
    if (b.bytes >= bytes) return LF_OK;
    hipError_t e;
    if (b.ptr) {
        e = hipStreamSynchronize((hipStream_t)stream);
        if (e != hipSuccess) return fail(LF_E_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
        (void)hipFree(b.ptr);
        b.ptr = nullptr;
        b.bytes = 0;
    }
    const size_t want = std::max(bytes, (size_t)1 << 16);
    e = hipMalloc(&b.ptr, want);
    if (e != hipSuccess) {
        b.ptr = nullptr;
        (void)hipGetLastError();
        return fail(LF_E_NOMEM, "workspace of %zu bytes: %s", want, hipGetErrorString(e));
    }
    if (zero) {
        e = hipMemset(b.ptr, 0, want);
        if (e != hipSuccess) {
            (void)hipFree(b.ptr);
            b.ptr = nullptr;
            return fail(LF_E_HIP, "hipMemset: %s", hipGetErrorString(e));
        }
    }
    b.bytes = want;
    return LF_OK;
}

Workspace *workspace_for(void *stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    return &g_ws[std::make_pair(dev, stream)];
}

// Host-to-device copy of a table the next kernels on `stream` read, finished
// before returning: the copy is enqueued on the stream, then the stream is
// drained.  A small copy from pageable memory was seen to land after the
// following kernels had read the old table, so an upload does not rely on
// the copy's own ordering.  Uploads happen only when a table changes (never
// in steady state, and never during capture, which the callers refuse).
hipError_t upload(void *dst, const void *src, size_t bytes, void *stream) {
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize((hipStream_t)stream);
}

// Device copy of *P on this stream's workspace; uploads only when it differs
// from the last upload.  An upload cannot be recorded into a graph (its source
// is a host temporary), so a changed plan during stream capture is refused.
lf_status_t upload_plan(Workspace &w, const lfk::Plan &P, void *stream, const lfk::Plan **dev_plan) {
    lf_status_t st = grow(w.plan, sizeof(lfk::Plan), false, stream);
    if (st != LF_OK) return st;
    if (!w.shadow_valid || std::memcmp(&w.shadow, &P, sizeof P) != 0) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cs);
        if (e != hipSuccess) return fail(LF_E_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
        if (cs != hipStreamCaptureStatusNone)
            return fail(LF_E_UNSUPPORTED,
                        "the call's shape, dilation or global set differs from the previous call on this stream "
                        "during stream capture; make one identical call outside capture first");
        e = upload(w.plan.ptr, &P, sizeof P, stream);
        if (e != hipSuccess) {
            w.shadow_valid = false;
            return fail(LF_E_HIP, "plan upload: %s", hipGetErrorString(e));
        }
        std::memcpy(&w.shadow, &P, sizeof P);
        w.shadow_valid = true;
    }
    *dev_plan = (const lfk::Plan *)w.plan.ptr;
    return LF_OK;
}

}  // namespace

extern "C" const char *lf_last_error(void) { return g_err.c_str(); }

namespace {

// The call behind both entry points: radius is NULL (r for every head) or
// one radius per head.
lf_status_t attn_fwd(const void *q, const void *k, const void *v, int B, int H, int T, int d, int r,
                     const int32_t *radius, int one_sided, const int32_t *rand_blocks, int n_rand,
                     const int32_t *dilation, const int32_t *global_idx, int n_global,
                     const uint8_t *key_padding_mask, void *out, lf_dtype_t dtype, void *stream) {
    g_err.clear();
    // ---- argument checks: no HIP call before all of them pass
    if (!q || !k || !v || !out) return fail(LF_E_INVALID, "q, k, v and out must be non-null");
    if (dtype != LF_F32 && dtype != LF_BF16) return fail(LF_E_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (B < 1 || H < 1 || T < 1) return fail(LF_E_INVALID, "B, H, T must be >= 1 (got %d, %d, %d)", B, H, T);
    if (d != LF_HEAD_DIM) return fail(LF_E_UNSUPPORTED, "head dimension %d: only %d is built", d, LF_HEAD_DIM);
    if (H > LF_MAX_HEADS) return fail(LF_E_UNSUPPORTED, "H = %d exceeds %d", H, LF_MAX_HEADS);
    if (T > LF_MAX_SEQ) return fail(LF_E_UNSUPPORTED, "T = %d exceeds %d", T, LF_MAX_SEQ);
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
    const size_t esize = dtype == LF_BF16 ? 2 : 4;
    const size_t nbytes = (size_t)B * (size_t)H * (size_t)T * (size_t)d * esize;
    if ((size_t)B * (size_t)H > (size_t)1 << 24)
        return fail(LF_E_UNSUPPORTED, "B*H = %lld too large", (long long)B * H);
    if (overlaps(out, nbytes, q, nbytes) || overlaps(out, nbytes, k, nbytes) || overlaps(out, nbytes, v, nbytes))
        return fail(LF_E_INVALID, "out overlaps q, k or v");

    // ---- normalise G: a set of positions, ascending
    std::vector<int32_t> G(global_idx, global_idx + n_global);
    std::sort(G.begin(), G.end());
    G.erase(std::unique(G.begin(), G.end()), G.end());
    if ((int)G.size() > LF_MAX_GLOBALS)
        return fail(LF_E_UNSUPPORTED, "%zu distinct globals exceed %d", G.size(), LF_MAX_GLOBALS);

    // ---- plan
    constexpr int QB = LFK_QB;
    constexpr int BM = 32 * QB;
    lfk::Plan P;
    std::memset(&P, 0, sizeof P);
    P.B = B; P.H = H; P.T = T;
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
    std::vector<uint32_t> aux;
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
    // heads with unequal radii make tiles of unequal cost: deal runs of 8
    // tiles to the dies in turn instead of one contiguous eighth per die
    P.band_chunk = 0;
    for (int h = 1; h < H; h++)
        if (P.rad[h] != P.rad[0]) P.band_chunk = 8;
    P.n_g = (int)G.size();
    for (int i = 0; i < P.n_g; i++) P.glob[i] = G[i];
    long long start = 0;
    for (int h = 0; h < H; h++) {
        const int delta = dilation ? dilation[h] : 1;
        P.dil[h] = delta;
        P.head_start[h] = (int)start;
        const long long qq = T / delta, rem = T % delta;
        start += rem * cdiv(qq + 1, BM) + (delta - rem) * cdiv(qq, BM);
    }
    P.head_start[H] = (int)start;
    P.uniform_head_tasks = (int)(start / H);
    for (int h = 0; h < H; h++)
        if (P.head_start[h + 1] - P.head_start[h] != P.uniform_head_tasks) P.uniform_head_tasks = 0;
    P.band_tasks_per_batch = (int)start;
    const long long n_band = (long long)B * start;
    long long n_glob_tasks = 0;
    size_t cnt_bytes = 0, scratch_bytes = 0;
    if (P.n_g > 0) {
        P.n_ggroups = (int)cdiv(cdiv(P.n_g, 32), QB);
        P.g_pad = P.n_ggroups * BM;
        // a split about as long as a band tile's key range (64 + 2r keys),
        // so both kinds of task cost about the same (measured faster than
        // the shortest splits); at least 256 keys, and at most 16 splits
        // (bounds the partial records and the combine's reads)
        long long sl = cdiv((long long)BM + 2LL * P.r, 64) * 64;
        if (sl < 256) sl = 256;
        const long long sl16 = cdiv(cdiv(T, 16), 32) * 32;
        if (sl < sl16) sl = sl16;
        P.split_len = (int)(sl < T ? sl : cdiv(T, 32) * 32);
        P.n_split = (int)cdiv(T, P.split_len);
        n_glob_tasks = (long long)B * H * P.n_split * P.n_ggroups;
        cnt_bytes = (size_t)B * H * sizeof(int);
        scratch_bytes = (size_t)B * H * P.n_split * P.g_pad * 272;  // 272-byte partial records
    }
    if (n_band + n_glob_tasks > (1LL << 30))
        return fail(LF_E_UNSUPPORTED, "problem needs %lld workgroups", n_band + n_glob_tasks);
    P.n_band_tasks = (int)n_band;
    P.n_tasks = (int)(n_band + n_glob_tasks);
    // fp32: K and V are split into bf16 hi/lo planes (same byte size as the
    // fp32 tensors) ahead of the tile kernel
    size_t planes_off = 0;
    if (dtype == LF_F32) {
        if ((long long)B * H * T * 8 / 256 >= (1LL << 31))
            return fail(LF_E_UNSUPPORTED, "fp32 problem too large for the plane split");
        planes_off = (scratch_bytes + 255) / 256 * 256;
        scratch_bytes = planes_off + 2 * nbytes;
    }

    // ---- HIP work
    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace *w = workspace_for(stream);
    if (!w) return fail(LF_E_HIP, "hipGetDevice failed");
    if (scratch_bytes > 0) {
        lf_status_t st = grow(w->counters, cnt_bytes, true, stream);
        if (st != LF_OK) return st;
        st = grow(w->scratch, scratch_bytes, false, stream);
        if (st != LF_OK) return st;
        char *ws = (char *)w->scratch.ptr;
        if (P.n_g > 0) {
            P.counter = (int *)w->counters.ptr;
            P.part = (float *)ws;
        }
        if (dtype == LF_F32) {
            P.kp = ws + planes_off;
            P.vp = ws + planes_off + nbytes;
        }
    }
    if (n_rand > 0) {
        lf_status_t st = grow(w->aux, aux.size() * sizeof(uint32_t), false, stream);
        if (st != LF_OK) return st;
        if (w->aux_shadow != aux) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cs);
            if (e != hipSuccess) return fail(LF_E_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
            if (cs != hipStreamCaptureStatusNone)
                return fail(LF_E_UNSUPPORTED,
                            "the random key blocks differ from the previous call on this stream during stream "
                            "capture; make one identical call outside capture first");
            e = upload(w->aux.ptr, aux.data(), aux.size() * sizeof(uint32_t), stream);
            if (e != hipSuccess) {
                w->aux_shadow.clear();
                return fail(LF_E_HIP, "random-block upload: %s", hipGetErrorString(e));
            }
            w->aux_shadow = aux;
        }
        P.rtab = (const int32_t *)w->aux.ptr;
        P.gmap = (const uint32_t *)w->aux.ptr + (size_t)H * nqb * n_rand;
    }
    lfk::Args A;
    A.q = q; A.k = k; A.v = v; A.out = out;
    A.pad = key_padding_mask;
    lf_status_t st = upload_plan(*w, P, stream, &A.plan);
    if (st != LF_OK) return st;
    hipError_t e = lfk_launch(&A, &P, dtype == LF_BF16, stream);
    if (e != hipSuccess) return fail(LF_E_HIP, "kernel launch: %s", hipGetErrorString(e));
    return LF_OK;
}

// Gradients (lf_attn_bwd): checks, the per-head tables, four launches.
lf_status_t attn_bwd(const void *q, const void *k, const void *v, const void *dy, int B, int H, int T, int d,
                     const int32_t *radius, int one_sided, const int32_t *rand_blocks, int n_rand,
                     const int32_t *dilation, const int32_t *global_idx, int n_global,
                     const uint8_t *key_padding_mask, void *dq, void *dk, void *dv, lf_dtype_t dtype,
                     void *stream) {
    if (!q || !k || !v || !dy || !dq || !dk || !dv)
        return fail(LF_E_INVALID, "q, k, v, dy, dq, dk and dv must be non-null");
    if (!radius) return fail(LF_E_INVALID, "radius must be a host array of H radii");
    if (dtype != LF_F32 && dtype != LF_BF16) return fail(LF_E_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (B < 1 || H < 1 || T < 1) return fail(LF_E_INVALID, "B, H, T must be >= 1 (got %d, %d, %d)", B, H, T);
    if (d != LF_HEAD_DIM) return fail(LF_E_UNSUPPORTED, "head dimension %d: only %d is built", d, LF_HEAD_DIM);
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
        chunks += rm * cdiv(qq + 1, LFB_ROWS_PER_WAVE) + (delta - rm) * cdiv(qq, LFB_ROWS_PER_WAVE);
    }
    tab[o_hc + H] = (uint32_t)chunks;
    if ((long long)B * chunks >= (1LL << 31)) return fail(LF_E_UNSUPPORTED, "problem needs too many waves");
    for (size_t e = 0; e < G.size(); e++) {
        tab[o_glob + e] = (uint32_t)G[e];
        tab[o_gmap + (G[e] >> 5)] |= 1u << (G[e] & 31);
    }

    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace *w = workspace_for(stream);
    if (!w) return fail(LF_E_HIP, "hipGetDevice failed");
    lf_status_t st = grow(w->bwd_tab, tab.size() * sizeof(uint32_t), false, stream);
    if (st != LF_OK) return st;
    st = grow(w->bwd_stats, (size_t)B * H * T * 2 * sizeof(float), false, stream);
    if (st != LF_OK) return st;
    // global rows and keys: splits of a multiple of 256 positions, as many
    // as bring the grid to about 2048 workgroups (at most 64, at least 1)
    const long long recs = (long long)B * H * (long long)G.size();
    long long want = recs > 0 ? std::min(64LL, std::max(1LL, cdiv(2048, recs))) : 1;
    want = std::min(want, cdiv(T, 256));
    const long long per_thread = cdiv(T, 256 * want);
    const int split_len = (int)(256 * per_thread);
    const int n_split = (int)cdiv(T, split_len);
    const size_t n_rec = (size_t)recs * n_split;
    if (n_rec >= ((size_t)1 << 31)) return fail(LF_E_UNSUPPORTED, "too many global-row splits");
    const size_t gstat_bytes = (n_rec * 16 + 255) / 256 * 256;
    if (n_rec > 0) {
        st = grow(w->bwd_gpart, gstat_bytes + n_rec * 192 * sizeof(float), false, stream);
        if (st != LF_OK) return st;
    }
    if (w->bwd_shadow != tab) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cs);
        if (e != hipSuccess) return fail(LF_E_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
        if (cs != hipStreamCaptureStatusNone)
            return fail(LF_E_UNSUPPORTED,
                        "the call's shape, radii, dilation or global set differs from the previous backward call "
                        "on this stream during stream capture; make one identical call outside capture first");
        e = upload(w->bwd_tab.ptr, tab.data(), tab.size() * sizeof(uint32_t), stream);
        if (e != hipSuccess) {
            w->bwd_shadow.clear();
            return fail(LF_E_HIP, "backward table upload: %s", hipGetErrorString(e));
        }
        w->bwd_shadow = tab;
    }
    const uint32_t *dt = (const uint32_t *)w->bwd_tab.ptr;
    lfk::BwdArgs A;
    A.pad = key_padding_mask;
    A.gmap = dt + o_gmap;
    A.glob = (const int32_t *)dt + o_glob;
    A.rad = (const int32_t *)dt;
    A.dil = (const int32_t *)dt + o_dil;
    A.head_chunk = (const int32_t *)dt + o_hc;
    A.hord = (const int32_t *)dt + o_ord;
    A.stats = w->bwd_stats.ptr;
    A.B = B; A.H = H; A.T = T; A.n_g = (int)G.size(); A.one_sided = one_sided;
    A.n_split = n_split;
    A.split_len = split_len;
    A.gstat = n_rec > 0 ? (float4 *)w->bwd_gpart.ptr : nullptr;
    A.gpart = n_rec > 0 ? (float *)((char *)w->bwd_gpart.ptr + gstat_bytes) : nullptr;
    A.n_rand = n_rand;
    A.rtab = n_rand > 0 ? (const int32_t *)dt + o_rtab : nullptr;
    A.inv_off = n_rand > 0 ? (const int32_t *)dt + o_off : nullptr;
    A.inv_list = n_rand > 0 ? (const int32_t *)dt + o_inv : nullptr;
    const void *t[7] = {q, k, v, dy, dq, dk, dv};
    hipError_t e = lfk_bwd_launch(&A, t, dtype == LF_BF16, stream);
    if (e != hipSuccess) return fail(LF_E_HIP, "kernel launch: %s", hipGetErrorString(e));
    return LF_OK;
}

}  // namespace

extern "C" lf_status_t lf_attn_bwd(const void *q, const void *k, const void *v, const void *dy, int B, int H,
                                   int T, int d, const int32_t *radius, int one_sided, const int32_t *rand_blocks,
                                   int n_rand, const int32_t *dilation, const int32_t *global_idx, int n_global,
                                   const uint8_t *key_padding_mask, void *dq, void *dk, void *dv, lf_dtype_t dtype,
                                   void *stream) {
    g_err.clear();
    return attn_bwd(q, k, v, dy, B, H, T, d, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
                    n_global, key_padding_mask, dq, dk, dv, dtype, stream);
}

extern "C" lf_status_t lf_attn_fwd(const void *q, const void *k, const void *v, int B, int H, int T,
                                   int d, int r, const int32_t *dilation, const int32_t *global_idx,
                                   int n_global, const uint8_t *key_padding_mask, void *out,
                                   lf_dtype_t dtype, void *stream) {
    return attn_fwd(q, k, v, B, H, T, d, r, nullptr, 0, nullptr, 0, dilation, global_idx, n_global,
                    key_padding_mask, out, dtype, stream);
}

extern "C" lf_status_t lf_attn_fwd_ex(const void *q, const void *k, const void *v, int B, int H, int T,
                                      int d, const int32_t *radius, int one_sided, const int32_t *rand_blocks,
                                      int n_rand, const int32_t *dilation, const int32_t *global_idx,
                                      int n_global, const uint8_t *key_padding_mask, void *out,
                                      lf_dtype_t dtype, void *stream) {
    g_err.clear();
    if (!radius) return fail(LF_E_INVALID, "radius must be a host array of H radii");
    return attn_fwd(q, k, v, B, H, T, d, 0, radius, one_sided, rand_blocks, n_rand, dilation, global_idx,
                    n_global, key_padding_mask, out, dtype, stream);
}
