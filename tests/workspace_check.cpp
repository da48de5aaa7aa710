// CPU check of the library's per-stream workspace under stream capture
// (csrc/lf_host.cpp compiled with g++ against the stand-ins below for the
// HIP runtime calls and the kernel launchers it makes).  The stand-ins model
// a stream as an ordered queue: outside capture an operation runs when it is
// enqueued; during capture it is recorded into the stream's graph instead,
// and a replay runs the recorded operations again.  A recorded launch checks,
// each time it runs, that the plan it reads holds the bytes it was given and
// that no buffer it uses has been freed.
//
// What is checked (prints "OK <checks>" or the failures):
//   - a captured call allocates nothing, and a call that would have to grow
//     the workspace during capture is refused with LF_E_UNSUPPORTED;
//   - what a captured call uses (its plan slot, counters, partials) is never
//     overwritten or freed by later eager calls on the stream, with more
//     plans than slots and with a larger shape that grows the workspace, so
//     every replay still reads its own plan;
//   - a plan written during capture is not used by eager calls before a
//     replay has written it;
//   - slots held by graphs are replaced for eager calls, so any number of
//     graphs can each hold one; captures of new plans in a row take the free
//     slots and are refused once none is left, and eager calls keep working;
//   - retired buffers are freed only after the stream has passed their last
//     use, and buffers of other streams are their own.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <set>
#include <vector>

#include "lf_attn.h"
#include "lf_kernels.h"
#include "lf_bwd.h"

static int fails = 0;
static long checks = 0;
#define CHECK(c, ...)                              \
    do {                                           \
        checks++;                                  \
        if (!(c)) {                                \
            if (fails++ < 20) {                    \
                std::printf("FAIL line %d: ", __LINE__); \
                std::printf(__VA_ARGS__);          \
                std::printf("\n");                 \
            }                                      \
        }                                          \
    } while (0)

// ---- the simulated device
using Op = std::function<void()>;
static std::map<void*, bool> g_capturing;
static std::map<void*, std::vector<Op>> g_graph;      // ops recorded during the current capture
static std::map<void*, long> g_enqueued, g_done;       // per stream: ops enqueued, ops finished
static std::set<void*> g_live, g_freed;
static int g_mallocs_in_capture = 0, g_mallocs = 0;

static void enqueue(void* s, Op op) {
    if (g_capturing[s]) {
        g_graph[s].push_back(op);
        return;
    }
    op();
    g_enqueued[s]++;
}
static void drain(void* s) { g_done[s] = g_enqueued[s]; }

struct Event {
    void* stream;
    long seq;
};

extern "C" {
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stand-in error"; }
hipError_t hipStreamIsCapturing(hipStream_t s, hipStreamCaptureStatus* st) {
    *st = g_capturing[(void*)s] ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
    for (auto& kv : g_capturing)
        if (kv.second) g_mallocs_in_capture++;
    *p = std::malloc(n);
    std::memset(*p, 0xAB, n);   // what a fresh allocation holds is unknown
    g_live.insert(*p);
    g_freed.erase(*p);
    g_mallocs++;
    return hipSuccess;
}
hipError_t hipFree(void* p) {
    CHECK(g_live.count(p) == 1, "hipFree of a pointer that is not live");
    g_live.erase(p);
    g_freed.insert(p);
    std::free(p);
    return hipSuccess;
}
hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t s) {
    CHECK(!g_capturing[(void*)s], "hipMemsetAsync recorded into a graph");
    enqueue((void*)s, [=] { std::memset(p, v, n); });
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    *e = (hipEvent_t) new Event{nullptr, 0};
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
    Event* ev = (Event*)e;
    ev->stream = (void*)s;
    ev->seq = g_enqueued[(void*)s];
    return hipSuccess;
}
hipError_t hipEventQuery(hipEvent_t e) {
    const Event* ev = (const Event*)e;
    return g_done[ev->stream] >= ev->seq ? hipSuccess : hipErrorNotReady;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    delete (Event*)e;
    return hipSuccess;
}

// ---- the kernel launchers
int lfk_supports_d(int d) { return d == 32 || d == 64 || d == 128; }
static char g_noalloc[1 << 20];
hipError_t lfk_noalloc_scratch(void** p) {
    *p = g_noalloc;
    return hipSuccess;
}
hipError_t lfk_write_plan(const void* plan, size_t bytes, void* dst, int* zero, int n_zero, void* stream) {
    std::vector<char> copy((const char*)plan, (const char*)plan + bytes);   // the bytes travel in the launch
    enqueue(stream, [=] {
        CHECK(g_live.count(dst) == 1, "plan write into a freed buffer");
        if (g_live.count(dst)) std::memcpy(dst, copy.data(), copy.size());
        for (int i = 0; i < n_zero; i++) zero[i] = 0;
    });
    return hipSuccess;
}
static long g_launches = 0;
static std::vector<const void*> g_plan_ptrs;   // device plan of every launch, in order
hipError_t lfk_launch(const lfk::Args* A, const lfk::Plan* P, int, void* stream) {
    const lfk::Plan want = *P;   // what the kernel must find behind A->plan when it runs
    const void* dplan = A->plan;
    g_plan_ptrs.push_back(dplan);
    enqueue(stream, [=] {
        g_launches++;
        CHECK(g_live.count((void*)dplan) == 1, "a launch reads a freed plan buffer");
        if (g_live.count((void*)dplan)) {
            const lfk::Plan* got = (const lfk::Plan*)dplan;
            // the workspace pointers are filled in the device copy too; the
            // rest of the plan must be the call's own
            CHECK(got->B == want.B && got->H == want.H && got->T == want.T && got->r == want.r &&
                      got->n_g == want.n_g && got->n_tasks == want.n_tasks &&
                      std::memcmp(got->glob, want.glob, sizeof want.glob) == 0 &&
                      got->counter == want.counter && got->part == want.part,
                  "a launch finds another call's plan (T %d r %d n_g %d, want T %d r %d n_g %d)", got->T, got->r,
                  got->n_g, want.T, want.r, want.n_g);
        }
        if (want.counter) CHECK(!g_freed.count((void*)want.counter), "a launch uses freed counters");
        if (want.part) CHECK(!g_freed.count((void*)want.part), "a launch uses freed partials");
    });
    return hipSuccess;
}
hipError_t lfk_bwd_launch(const lfk::BwdArgs*, const void* const*, void*) { return hipSuccess; }
hipError_t lfk_bwd_dq(const lfk::BwdBandArgs*, const lfk::Plan*, void*) { return hipSuccess; }
hipError_t lfk_bwd_dkdv(const lfk::BwdBandArgs*, const lfk::Plan*, void*) { return hipSuccess; }
}

// ---- calls
static const uintptr_t kQ = 0x100000000ull, kK = 0x200000000ull, kV = 0x300000000ull, kOut = 0x400000000ull;

static lf_status_t fwd(void* s, int T, int r, std::vector<int32_t> G) {
    return lf_attn_fwd((const void*)kQ, (const void*)kK, (const void*)kV, 1, 2, T, 64, r, nullptr, G.data(),
                       (int)G.size(), nullptr, (void*)kOut, LF_BF16, s);
}

static void replay(void* s, const std::vector<Op>& graph) {
    for (const Op& op : graph) op();
    g_enqueued[s]++;
}

int main() {
    void* s = (void*)0x5000;
    void* s2 = (void*)0x6000;

    // 1. nothing sized yet: a captured call that needs a workspace is refused
    //    and allocates nothing
    g_capturing[s] = true;
    CHECK(fwd(s, 1000, 16, {0, 5}) == LF_E_UNSUPPORTED, "capture without a workspace: %s", lf_last_error());
    g_capturing[s] = false;
    g_graph[s].clear();
    CHECK(g_mallocs_in_capture == 0, "hipMalloc during capture");

    // 2. an eager call sizes the workspace; the same call captured uses it
    CHECK(fwd(s, 1000, 16, {0, 5}) == LF_OK, "eager call: %s", lf_last_error());
    const int mallocs_before = g_mallocs;
    g_capturing[s] = true;
    CHECK(fwd(s, 1000, 16, {0, 5}) == LF_OK, "captured call: %s", lf_last_error());
    g_capturing[s] = false;
    const std::vector<Op> graph_a = g_graph[s];
    g_graph[s].clear();
    CHECK(g_mallocs == mallocs_before, "the captured call allocated");
    CHECK(!graph_a.empty(), "nothing was recorded");

    // 3. more plans than slots, eagerly, then a larger shape that grows the
    //    counters and partials; the graph must still read its own plan and
    //    buffers, before and after the stream has drained and reaped
    for (int i = 0; i < 3; i++) {
        for (int r : {3, 7, 11, 40, 90, 3, 7}) CHECK(fwd(s, 1000, r, {1, 2, 3}) == LF_OK, "eager: %s", lf_last_error());
        replay(s, graph_a);
        CHECK(fwd(s, 5000 + 1000 * i, 20, {0, 7, 9, 4000}) == LF_OK, "grow: %s", lf_last_error());
        drain(s);
        CHECK(fwd(s, 1000, 5, {1}) == LF_OK, "after drain: %s", lf_last_error());   // reaps retired buffers
        replay(s, graph_a);
    }

    // 4. a capture whose workspace would have to grow is refused
    g_capturing[s] = true;
    const int m4 = g_mallocs;
    std::vector<int32_t> many;
    for (int g = 0; g < 300; g++) many.push_back(7 * g);
    CHECK(fwd(s, 60000, 20, many) == LF_E_UNSUPPORTED, "growth during capture was not refused");
    CHECK(g_mallocs == m4, "the refused capture allocated");
    g_capturing[s] = false;
    g_graph[s].clear();

    // 5. a plan not resident, written inside the graph: eager calls of the
    //    same configuration do not read that slot before a replay wrote it
    CHECK(fwd(s, 1000, 77, {0, 5}) == LF_OK, "eager: %s", lf_last_error());   // make sure a free slot exists
    g_capturing[s] = true;
    const size_t n0 = g_plan_ptrs.size();
    CHECK(fwd(s, 1000, 61, {2, 3}) == LF_OK, "capture of a new plan: %s", lf_last_error());
    g_capturing[s] = false;
    const std::vector<Op> graph_b = g_graph[s];
    g_graph[s].clear();
    const void* slot_b = g_plan_ptrs[n0];
    CHECK(fwd(s, 1000, 61, {2, 3}) == LF_OK, "eager after capture: %s", lf_last_error());
    CHECK(g_plan_ptrs.back() != slot_b, "an eager call reads a plan slot only a replay writes");
    for (int i = 0; i < 2; i++) {
        replay(s, graph_b);
        replay(s, graph_a);
        CHECK(fwd(s, 1000, 13 + i, {4}) == LF_OK, "eager: %s", lf_last_error());
    }

    // 6. many graphs, each holding a plan slot: eager calls keep getting
    //    free slots (a held slot is replaced), every replay reads its own plan
    std::vector<std::vector<Op>> graphs;
    for (int r = 100; r < 110; r++) {
        CHECK(fwd(s, 1000, r, {0}) == LF_OK, "eager: %s", lf_last_error());
        g_capturing[s] = true;
        CHECK(fwd(s, 1000, r, {0}) == LF_OK, "capture of a resident plan: %s", lf_last_error());
        g_capturing[s] = false;
        graphs.push_back(g_graph[s]);
        g_graph[s].clear();
        for (int e = 0; e < 6; e++) CHECK(fwd(s, 1000, 200 + e, {1}) == LF_OK, "eager: %s", lf_last_error());
    }
    for (const auto& g : graphs) replay(s, g);
    replay(s, graph_a);
    replay(s, graph_b);
    //    captures of new plans in a row, with no eager call between them to
    //    replace the slots they take: once the free slots are gone the next
    //    one is refused
    lf_status_t st = LF_OK;
    int taken = 0;
    for (int r = 300; r < 310 && st == LF_OK; r++) {
        g_capturing[s] = true;
        st = fwd(s, 1000, r, {0});
        g_capturing[s] = false;
        if (st == LF_OK) {
            graphs.push_back(g_graph[s]);
            taken++;
        }
        g_graph[s].clear();
    }
    CHECK(st == LF_E_UNSUPPORTED && taken == 4, "captures of new plans: %d taken, status %d", taken, (int)st);
    CHECK(fwd(s, 1000, 400, {0}) == LF_OK, "eager after the slots were taken: %s", lf_last_error());
    for (const auto& g : graphs) replay(s, g);

    // 7. another stream has its own workspace: its calls never touch this
    //    stream's buffers
    const size_t n1 = g_plan_ptrs.size();
    CHECK(fwd(s2, 1000, 16, {0, 5}) == LF_OK, "other stream: %s", lf_last_error());
    for (size_t i = 0; i < n1; i++) CHECK(g_plan_ptrs[i] != g_plan_ptrs.back(), "streams share a plan slot");
    drain(s);
    drain(s2);
    CHECK(fwd(s, 1000, 16, {0, 5}) == LF_OK, "eager: %s", lf_last_error());
    replay(s, graph_a);

    CHECK(g_launches > 40, "only %ld launches ran", g_launches);
    if (fails) {
        std::printf("FAILED %d of %ld checks\n", fails, checks);
        return 1;
    }
    std::printf("OK %ld\n", checks);
    return 0;
}
