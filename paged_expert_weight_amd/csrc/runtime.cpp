// Host runtime of the paged fused-MoE C ABI: argument validation, the layer's
// location table (page table), the double-buffer event protocol and the
// workspace layout.  All compute is in the HIP kernels (route_align.hip,
// moe_gemm.hip); this file only validates and enqueues.
#include "moe.h"
#include "internal.h"

#include <algorithm>
#include <array>
#include <iterator>
#include <cstring>
#include <string>
#include <vector>

using pmoe::DevLoc;

struct moe_pool {
    moe_pool_desc desc;
    int E_tot = 0, keff = 0;
    int device = 0;
    DevLoc *d_locs = nullptr;           // device copy of the location table
    moe_expert_loc *h_stage = nullptr;  // pinned staging of the last upload
    hipEvent_t upload_done = nullptr;   // staging may be rewritten once this fired
    bool upload_pending = false;
    bool locs_set = false;
    bool uses_loadbuf = false;          // the table names at least one load-buffer expert
    hipEvent_t filled[2] = {nullptr, nullptr};   // last fill of buffer b done (read-after-write)
    bool ever_filled[2] = {false, false};
    // write-after-read marks of buffer b since its last fill: per stream that
    // ran a forward reading it, an event recorded after that stream's last
    // such forward (one event per stream, so forwards on several streams are
    // all waited for by the next fill); events return to spare_events then
    struct ReadMark {
        hipStream_t stream;
        hipEvent_t done;
    };
    std::vector<ReadMark> read_marks[2];
    std::vector<hipEvent_t> spare_events;
    // streams of forwards that read buffer b with MOE_FLAG_DEFER_READ_DONE and
    // have not been marked yet (by the next fill of b or by destroy)
    std::vector<hipStream_t> deferred_readers[2];
    // stage timing (measurement only): one set of 4 events per recorded forward
    bool timing = false;
    std::vector<std::array<hipEvent_t, 4>> tev;
    size_t tev_used = 0;
};

constexpr size_t kMaxTimedForwards = 1024;

// Events that only mark "the readers of a buffer have finished" (before it is
// overwritten or handed out again) need no system-scope fence: nothing they
// order has to become visible to anyone, and the fence would write back and
// invalidate the caches after every forward.
constexpr unsigned kReadDoneEvent = hipEventDisableTiming | hipEventDisableSystemFence;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string &msg)
{
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define HIP_TRY(call)                                                                              \
    do {                                                                                           \
        hipError_t e_ = (call);                                                                    \
        if (e_ != hipSuccess)                                                                      \
            return hip_fail(e_, #call);                                                            \
    } while (0)

constexpr int64_t kMaxBuf = (int64_t)1 << 31; // every buffer read through a descriptor stays < 2 GiB

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

int check_desc(const moe_pool_desc *d)
{
    if (!d)
        return fail(MOE_ERR_INVALID_ARG, "desc is null");
    if (!d->pool_base)
        return fail(MOE_ERR_INVALID_ARG, "pool_base is null");
    if (!aligned(d->pool_base, 16))
        return fail(MOE_ERR_ALIGN, "pool_base not 16-byte aligned");
    if (d->num_pages < 1)
        return fail(MOE_ERR_INVALID_ARG, "num_pages < 1");
    if (d->d <= 0 || d->f <= 0)
        return fail(MOE_ERR_INVALID_ARG, "d and f must be positive");
    if (d->d % 64 || d->f % 64)
        return fail(MOE_ERR_UNSUPPORTED, "d and f must be multiples of 64");
    if ((int64_t)d->f * d->d * 2 >= kMaxBuf)
        return fail(MOE_ERR_UNSUPPORTED, "one page (f*d bf16) must be < 2 GiB");
    if (d->num_shared < 0 || d->num_shared > 1)
        return fail(MOE_ERR_INVALID_ARG, "num_shared must be 0 or 1");
    if (d->num_experts < 1 || d->num_experts + d->num_shared > pmoe::kMaxExpertsTotal)
        return fail(MOE_ERR_UNSUPPORTED, "num_experts + num_shared must be in [1, 1024]");
    if (d->top_k < 1 || d->top_k > d->num_experts || d->top_k > pmoe::kMaxTopK)
        return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, min(num_experts, 32)]");
    if (d->loadbuf_slots < 0)
        return fail(MOE_ERR_INVALID_ARG, "loadbuf_slots < 0");
    if (d->loadbuf_slots > 0) {
        for (int b = 0; b < 2; b++) {
            if (!d->loadbuf_base[b])
                return fail(MOE_ERR_INVALID_ARG, "loadbuf_base is null while loadbuf_slots > 0");
            if (!aligned(d->loadbuf_base[b], 16))
                return fail(MOE_ERR_ALIGN, "loadbuf_base not 16-byte aligned");
        }
    }
    return MOE_OK;
}

struct Sizes {
    int64_t n, sorted_cap, blocks_cap;
    size_t off_counts, off_h, off_comb, off_part, part, total;
};

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

Sizes sizes_for(const moe_pool *p, int64_t T, int bm, uint32_t flags)
{
    Sizes s{};
    s.n = T * p->keff;
    s.sorted_cap = s.n + (int64_t)p->E_tot * (bm - 1);
    s.blocks_cap = (s.sorted_cap + bm - 1) / bm;
    const size_t counts = (size_t)pmoe::route_workspace_bytes(T, p->keff, p->E_tot);
    const size_t h = (size_t)s.sorted_cap * p->desc.f * 2;
    const size_t comb = (flags & MOE_FLAG_ATOMIC_COMBINE) ? (size_t)T * p->desc.d * 4
                                                          : (size_t)s.n * p->desc.d * 2;
    // fp32 partial tiles of a split last wave (256-row tiles, one workgroup per CU: at most
    // one 256 x 256 tile per CU)
    s.part = 0;
    if (bm == 256) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
            s.part = (size_t)cus * 256 * 256 * 4;
        (void)hipGetLastError();
    }
    s.off_counts = 0;
    s.off_h = up256(counts);
    s.off_comb = s.off_h + up256(h);
    s.off_part = s.off_comb + up256(comb);
    s.total = s.off_part + up256(s.part);
    return s;
}

// Shared checks of moe_route / the forwards: T range and buffer-size limits.
int check_tokens(const moe_pool *p, int64_t T, int bm)
{
    if (T < 0)
        return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (!valid_block_m(bm))
        return fail(MOE_ERR_INVALID_ARG, "block_m must be 16, 32, 64, 128 or 256");
    const int64_t n = T * p->keff;
    if (n + (int64_t)p->E_tot * bm >= ((int64_t)1 << 31))
        return fail(MOE_ERR_UNSUPPORTED, "T*(k+S) too large for int32 indices");
    if (T * p->desc.d * 2 >= kMaxBuf)
        return fail(MOE_ERR_UNSUPPORTED, "x (T*d bf16) must be < 2 GiB");
    const int64_t sorted_cap = n + (int64_t)p->E_tot * (bm - 1);
    if (sorted_cap * p->desc.f * 2 >= kMaxBuf)
        return fail(MOE_ERR_UNSUPPORTED, "activation buffer (sorted_cap*f bf16) must be < 2 GiB");
    return MOE_OK;
}

int check_dev(const void *ptr, size_t align, const char *name)
{
    if (!ptr)
        return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is null");
    if (!aligned(ptr, align))
        return fail(MOE_ERR_ALIGN, std::string(name) + " misaligned");
    return MOE_OK;
}

#define CHECK(expr)                                                                                \
    do {                                                                                           \
        int rc_ = (expr);                                                                          \
        if (rc_ != MOE_OK)                                                                         \
            return rc_;                                                                            \
    } while (0)

pmoe::RouteArgs route_args(const moe_pool *p, const float *logits, int64_t T, int32_t bm, int32_t *ids, float *w,
                           int32_t *sorted, int32_t *blk, int32_t *npad, void *ws, const Sizes &sz)
{
    pmoe::RouteArgs a{};
    a.logits = logits;
    a.T = T;
    a.E = p->desc.num_experts;
    a.k = p->desc.top_k;
    a.S = p->desc.num_shared;
    a.keff = p->keff;
    a.E_tot = p->E_tot;
    a.BM = bm;
    a.topk_ids = ids;
    a.topk_w = w;
    a.sorted_ids = sorted;
    a.block_expert = blk;
    a.num_padded = npad;
    a.sorted_cap = sz.sorted_cap;
    a.blocks_cap = sz.blocks_cap;
    a.counts = (int32_t *)((char *)ws + sz.off_counts);
    return a;
}

// The forward on routing outputs (ids ... npad).  With logits (route + forward
// in one call) the routing is computed first: inside the decode form's gate/up
// launch when decode_routed_fits holds, else by the routing kernels.
int forward_common(const moe_pool *p, const void *w13, const void *w2, bool paged, const void *x,
                   int64_t T, int32_t bm, const int32_t *ids, const float *w, const int32_t *sorted,
                   const int32_t *blk, const int32_t *npad, int32_t active_buf, void *y, void *ws,
                   size_t ws_bytes, uint32_t flags, hipStream_t s, hipEvent_t *ev,
                   const float *logits = nullptr)
{
    if (flags & ~MOE_FLAG_ATOMIC_COMBINE)
        return fail(MOE_ERR_INVALID_ARG, "unknown flag bits");
    CHECK(check_tokens(p, T, bm));
    if (T == 0)
        return MOE_OK;
    CHECK(check_dev(x, 16, "x"));
    CHECK(check_dev(y, 16, "y"));
    CHECK(check_dev(ids, 4, "topk_ids"));
    CHECK(check_dev(w, 4, "topk_w"));
    CHECK(check_dev(sorted, 4, "sorted_ids"));
    CHECK(check_dev(blk, 4, "block_expert"));
    CHECK(check_dev(npad, 4, "num_padded"));
    CHECK(check_dev(ws, 256, "workspace"));
    const Sizes sz = sizes_for(p, T, bm, flags);
    if (ws_bytes < sz.total)
        return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(sz.total) + " bytes");
    pmoe::FwdArgs a{};
    if (paged) {
        a.locs = p->d_locs;
        a.pool = (const uint16_t *)p->desc.pool_base;
        a.loadbuf = p->desc.loadbuf_slots > 0 ? (const uint16_t *)p->desc.loadbuf_base[active_buf] : nullptr;
    } else {
        a.w13 = (const uint16_t *)w13;
        a.w2 = (const uint16_t *)w2;
    }
    a.x = (const uint16_t *)x;
    a.T = T;
    a.d = p->desc.d;
    a.f = p->desc.f;
    a.keff = p->keff;
    a.E_tot = p->E_tot;
    a.BM = bm;
    a.topk_ids = ids;
    a.topk_w = w;
    a.sorted_ids = sorted;
    a.block_expert = blk;
    a.num_padded = npad;
    a.sorted_cap = sz.sorted_cap;
    a.blocks_cap = sz.blocks_cap;
    a.y = (uint16_t *)y;
    a.h = (uint16_t *)((char *)ws + sz.off_h);
    a.comb = (char *)ws + sz.off_comb;
    a.part = (float *)((char *)ws + sz.off_part);
    a.part_bytes = (int64_t)sz.part;
    a.atomic = (flags & MOE_FLAG_ATOMIC_COMBINE) != 0;
    if (ev)
        for (int i = 0; i < 4; i++)
            a.ev[i] = ev[i];
    if (logits) {
        CHECK(check_dev(logits, 4, "logits"));
        pmoe::DecRouteArgs dr{};
        dr.logits = logits;
        dr.E = p->desc.num_experts;
        dr.k = p->desc.top_k;
        dr.S = p->desc.num_shared;
        dr.topk_ids = const_cast<int32_t *>(ids);
        dr.topk_w = const_cast<float *>(w);
        dr.sorted_ids = const_cast<int32_t *>(sorted);
        dr.block_expert = const_cast<int32_t *>(blk);
        dr.num_padded = const_cast<int32_t *>(npad);
        if (pmoe::decode_routed_fits(a, dr)) {
            HIP_TRY(pmoe::launch_decode_routed(a, dr, s));
            return MOE_OK;
        }
        const pmoe::RouteArgs ra = route_args(p, logits, T, bm, dr.topk_ids, dr.topk_w, dr.sorted_ids,
                                              dr.block_expert, dr.num_padded, ws, sz);
        HIP_TRY(pmoe::launch_route_align(ra, s));
    }
    if (pmoe::decode_fits(a))
        HIP_TRY(pmoe::launch_decode(a, s));
    else
        HIP_TRY(pmoe::launch_forward(a, s));
    return MOE_OK;
}

// Events for the next timed forward of p, or nullptr when timing is off or full.
hipEvent_t *next_timing_events(moe_pool *p)
{
    if (!p->timing || p->tev_used >= kMaxTimedForwards)
        return nullptr;
    if (p->tev_used == p->tev.size()) {
        std::array<hipEvent_t, 4> ev{};
        for (auto &e : ev)
            if (hipEventCreate(&e) != hipSuccess)
                return nullptr;
        p->tev.push_back(ev);
    }
    return p->tev[p->tev_used++].data();
}

} // namespace

namespace pmoe {
int set_error(int code, const char *msg) { return fail(code, msg); }
bool pool_shape(const moe_pool *p, int32_t *E_tot, int64_t *page_bytes)
{
    if (!p)
        return false;
    *E_tot = p->E_tot;
    *page_bytes = (int64_t)p->desc.f * p->desc.d * 2;
    return true;
}
void pool_loadbufs(const moe_pool *p, void *bases[2])
{
    const bool has = p->desc.loadbuf_slots > 0;
    bases[0] = has ? p->desc.loadbuf_base[0] : nullptr;
    bases[1] = has ? p->desc.loadbuf_base[1] : nullptr;
}

// A forward about to read load buffer buf on stream s waits for the buffer's
// last fill (read after write).  MOE_ERR_STATE if the buffer was never filled.
int loadbuf_read_begin(moe_pool *p, int32_t buf, hipStream_t s)
{
    if (!p->ever_filled[buf])
        return fail(MOE_ERR_STATE, "load buffer " + std::to_string(buf) +
                                       " was never filled but the table reads from it");
    // a fill that has already completed needs no wait on the stream (the
    // wait would still cost a queue round trip before the first kernel)
    const hipError_t q = hipEventQuery(p->filled[buf]);
    if (q == hipErrorNotReady) {
        (void)hipGetLastError();
        HIP_TRY(hipStreamWaitEvent(s, p->filled[buf], 0));
    } else if (q != hipSuccess) {
        return hip_fail(q, "hipEventQuery");
    }
    return MOE_OK;
}

// A spare write-after-read event of the pool, or a new one.
int take_read_event(moe_pool *p, hipEvent_t *ev)
{
    if (!p->spare_events.empty()) {
        *ev = p->spare_events.back();
        p->spare_events.pop_back();
        return MOE_OK;
    }
    // marks the end of reads only: no cache writeback is needed before a later overwrite
    const hipError_t e = hipEventCreateWithFlags(ev, kReadDoneEvent);
    if (e != hipSuccess)
        return hip_fail(e, "hipEventCreate");
    return MOE_OK;
}

// After a forward that read load buffer buf on stream s: mark the buffer read
// (write after read), now (the event of stream s, recorded again) or
// (MOE_FLAG_DEFER_READ_DONE) at its next fill.
int loadbuf_read_end(moe_pool *p, int32_t buf, uint32_t flags, hipStream_t s)
{
    if (flags & MOE_FLAG_DEFER_READ_DONE) {
        auto &rd = p->deferred_readers[buf];
        if (std::find(rd.begin(), rd.end(), s) == rd.end())
            rd.push_back(s);
        return MOE_OK;
    }
    auto &marks = p->read_marks[buf];
    hipEvent_t ev = nullptr;
    for (const auto &m : marks)
        if (m.stream == s)
            ev = m.done;
    if (!ev) {
        CHECK(take_read_event(p, &ev));
        marks.push_back({s, ev});
    }
    HIP_TRY(hipEventRecord(ev, s));
    return MOE_OK;
}

// The end of a forward whose launches may read load buffer buf, rc being the
// forward's result: the read mark is recorded even when the forward failed (a
// launch that failed may follow launches already enqueued that read the
// buffer), and the forward's own error, if any, is the one reported.
int loadbuf_read_end_after(moe_pool *p, int32_t buf, uint32_t flags, hipStream_t s, int rc)
{
    if (rc == MOE_OK)
        return loadbuf_read_end(p, buf, flags, s);
    const std::string first = g_err;
    (void)loadbuf_read_end(p, buf, flags, s);
    g_err = first;
    return rc;
}

} // namespace pmoe

extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }

int moe_version(void) { return 103; }

int moe_validate_locs(const moe_pool_desc *desc, const moe_expert_loc *locs, int32_t n)
{
    CHECK(check_desc(desc));
    const int E_tot = desc->num_experts + desc->num_shared;
    if (!locs)
        return fail(MOE_ERR_INVALID_ARG, "locs is null");
    if (n != E_tot)
        return fail(MOE_ERR_INVALID_ARG, "locs must have num_experts + num_shared entries");
    std::vector<int32_t> page_owner(desc->num_pages, -1);
    std::vector<int32_t> slot_owner(desc->loadbuf_slots > 0 ? desc->loadbuf_slots : 0, -1);
    for (int e = 0; e < n; e++) {
        const moe_expert_loc &L = locs[e];
        if (L.kind == MOE_LOC_POOL) {
            for (int m = 0; m < 3; m++) {
                const int64_t pg = L.idx[m];
                if (pg < 0 || pg >= desc->num_pages)
                    return fail(MOE_ERR_PAGE_RANGE, "expert " + std::to_string(e) + ": page " +
                                                        std::to_string(pg) + " out of range");
                if (page_owner[pg] >= 0)
                    return fail(MOE_ERR_PAGE_ALIAS, "page " + std::to_string(pg) + " used twice (experts " +
                                                        std::to_string(page_owner[pg]) + ", " +
                                                        std::to_string(e) + ")");
                page_owner[pg] = e;
            }
        } else if (L.kind == MOE_LOC_LOADBUF) {
            const int s = L.idx[0];
            if (s < 0 || s >= desc->loadbuf_slots)
                return fail(MOE_ERR_SLOT_RANGE, "expert " + std::to_string(e) + ": slot " +
                                                    std::to_string(s) + " out of range");
            if (slot_owner[s] >= 0)
                return fail(MOE_ERR_SLOT_RANGE, "slot " + std::to_string(s) + " given to two experts");
            slot_owner[s] = e;
        } else {
            return fail(MOE_ERR_INVALID_ARG, "expert " + std::to_string(e) + ": unknown kind");
        }
    }
    return MOE_OK;
}

int moe_pool_create(const moe_pool_desc *desc, moe_pool **out)
{
    if (!out)
        return fail(MOE_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    CHECK(check_desc(desc));
    moe_pool *p = new moe_pool();
    p->desc = *desc;
    p->E_tot = desc->num_experts + desc->num_shared;
    p->keff = desc->top_k + desc->num_shared;
    auto cleanup = [&](int rc) {
        moe_pool_destroy(p);
        return rc;
    };
    hipError_t e;
    if ((e = hipGetDevice(&p->device)) != hipSuccess)
        return cleanup(hip_fail(e, "hipGetDevice"));
    if ((e = hipMalloc((void **)&p->d_locs, sizeof(DevLoc) * p->E_tot)) != hipSuccess)
        return cleanup(hip_fail(e, "hipMalloc(location table)"));
    if ((e = hipHostMalloc((void **)&p->h_stage, sizeof(moe_expert_loc) * p->E_tot, hipHostMallocDefault)) !=
        hipSuccess)
        return cleanup(hip_fail(e, "hipHostMalloc(staging)"));
    if ((e = hipEventCreateWithFlags(&p->upload_done, hipEventDisableTiming)) != hipSuccess)
        return cleanup(hip_fail(e, "hipEventCreate"));
    for (int b = 0; b < 2; b++)
        if ((e = hipEventCreateWithFlags(&p->filled[b], hipEventDisableTiming)) != hipSuccess)
            return cleanup(hip_fail(e, "hipEventCreate"));
    *out = p;
    return MOE_OK;
}

int moe_pool_destroy(moe_pool *p)
{
    if (!p)
        return MOE_OK;
    if (p->upload_pending && p->upload_done)
        (void)hipEventSynchronize(p->upload_done);
    for (int b = 0; b < 2; b++) {
        if (p->filled[b]) {
            if (p->ever_filled[b])
                (void)hipEventSynchronize(p->filled[b]);
            (void)hipEventDestroy(p->filled[b]);
        }
        for (const auto &m : p->read_marks[b]) {
            (void)hipEventSynchronize(m.done);
            p->spare_events.push_back(m.done);
        }
        p->read_marks[b].clear();
        for (hipStream_t r : p->deferred_readers[b]) { // forwards whose reads were not marked yet
            hipEvent_t ev = nullptr;
            if (pmoe::take_read_event(p, &ev) == MOE_OK) {
                if (hipEventRecord(ev, r) == hipSuccess)
                    (void)hipEventSynchronize(ev);
                p->spare_events.push_back(ev);
            }
        }
    }
    for (hipEvent_t ev : p->spare_events)
        (void)hipEventDestroy(ev);
    if (p->upload_done)
        (void)hipEventDestroy(p->upload_done);
    for (auto &ev : p->tev)
        for (auto e : ev)
            if (e)
                (void)hipEventDestroy(e);
    if (p->d_locs)
        (void)hipFree(p->d_locs);
    if (p->h_stage)
        (void)hipHostFree(p->h_stage);
    delete p;
    return MOE_OK;
}

int moe_set_expert_locs(moe_pool *p, const moe_expert_loc *locs, int32_t n, void *stream)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    CHECK(moe_validate_locs(&p->desc, locs, n));
    if (p->upload_pending)
        HIP_TRY(hipEventSynchronize(p->upload_done));
    std::memcpy(p->h_stage, locs, sizeof(moe_expert_loc) * n);
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(hipMemcpyAsync(p->d_locs, p->h_stage, sizeof(moe_expert_loc) * n, hipMemcpyHostToDevice, s));
    HIP_TRY(hipEventRecord(p->upload_done, s));
    p->upload_pending = true;
    p->locs_set = true;
    p->uses_loadbuf = false;
    for (int e = 0; e < n; e++)
        p->uses_loadbuf |= locs[e].kind == MOE_LOC_LOADBUF;
    return MOE_OK;
}

int moe_route_capacity(const moe_pool *p, int64_t T, int32_t block_m, int64_t *sorted_cap, int64_t *blocks_cap)
{
    if (!p || !sorted_cap || !blocks_cap)
        return fail(MOE_ERR_INVALID_ARG, "null argument");
    CHECK(check_tokens(p, T, block_m));
    const Sizes s = sizes_for(p, T, block_m, 0);
    *sorted_cap = s.sorted_cap;
    *blocks_cap = s.blocks_cap;
    return MOE_OK;
}

int moe_workspace_bytes(const moe_pool *p, int64_t T, int32_t block_m, uint32_t flags, size_t *bytes)
{
    if (!p || !bytes)
        return fail(MOE_ERR_INVALID_ARG, "null argument");
    if (flags & ~(MOE_FLAG_ATOMIC_COMBINE | MOE_FLAG_DEFER_READ_DONE))
        return fail(MOE_ERR_INVALID_ARG, "unknown flag bits");
    CHECK(check_tokens(p, T, block_m));
    *bytes = sizes_for(p, T, block_m, flags).total;
    return MOE_OK;
}

int moe_route(moe_pool *p, const float *logits, int64_t T, int32_t block_m, int32_t *topk_ids, float *topk_w,
              int32_t *sorted_ids, int32_t *block_expert, int32_t *num_padded, void *ws, size_t ws_bytes,
              void *stream)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    CHECK(check_tokens(p, T, block_m));
    if (T == 0)
        return MOE_OK;
    CHECK(check_dev(logits, 4, "logits"));
    CHECK(check_dev(topk_ids, 4, "topk_ids"));
    CHECK(check_dev(topk_w, 4, "topk_w"));
    CHECK(check_dev(sorted_ids, 4, "sorted_ids"));
    CHECK(check_dev(block_expert, 4, "block_expert"));
    CHECK(check_dev(num_padded, 4, "num_padded"));
    const Sizes sz = sizes_for(p, T, block_m, 0);
    if (sz.off_h > 0) {
        CHECK(check_dev(ws, 256, "workspace"));
        if (ws_bytes < sz.off_h)
            return fail(MOE_ERR_WORKSPACE, "workspace too small for routing");
    }
    const pmoe::RouteArgs a =
        route_args(p, logits, T, block_m, topk_ids, topk_w, sorted_ids, block_expert, num_padded, ws, sz);
    HIP_TRY(pmoe::launch_route_align(a, (hipStream_t)stream));
    return MOE_OK;
}


namespace {

// Checks of a paged forward, and its wait for the last fill of the load
// buffer it reads (read after write).
int paged_begin(moe_pool *p, int64_t T, int32_t active_buf, uint32_t flags, hipStream_t s)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    if (active_buf < 0 || active_buf > 1)
        return fail(MOE_ERR_INVALID_ARG, "active_buf must be 0 or 1");
    if (!p->locs_set)
        return fail(MOE_ERR_STATE, "no location table: call moe_set_expert_locs first");
    if (flags & ~(MOE_FLAG_ATOMIC_COMBINE | MOE_FLAG_DEFER_READ_DONE))
        return fail(MOE_ERR_INVALID_ARG, "unknown flag bits");
    if (p->uses_loadbuf && !p->ever_filled[active_buf])
        return fail(MOE_ERR_STATE, "load buffer " + std::to_string(active_buf) +
                                       " was never filled but the table reads from it");
    if (T > 0 && p->uses_loadbuf)
        return pmoe::loadbuf_read_begin(p, active_buf, s);
    return MOE_OK;
}

// After a paged forward whose result is rc: mark its load buffer read (write
// after read), now or (MOE_FLAG_DEFER_READ_DONE) at the buffer's next fill,
// also when the forward failed part-way.
int paged_end(moe_pool *p, int64_t T, int32_t active_buf, uint32_t flags, hipStream_t s, int rc)
{
    if (T > 0 && p->uses_loadbuf)
        return pmoe::loadbuf_read_end_after(p, active_buf, flags, s, rc);
    return rc;
}

} // namespace

int moe_paged_forward(moe_pool *p, const void *x, int64_t T, int32_t block_m, const int32_t *topk_ids,
                      const float *topk_w, const int32_t *sorted_ids, const int32_t *block_expert,
                      const int32_t *num_padded, int32_t active_buf, void *y, void *ws, size_t ws_bytes,
                      uint32_t flags, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    CHECK(paged_begin(p, T, active_buf, flags, s));
    const int rc = forward_common(p, nullptr, nullptr, true, x, T, block_m, topk_ids, topk_w, sorted_ids,
                                  block_expert, num_padded, active_buf, y, ws, ws_bytes,
                                  flags & MOE_FLAG_ATOMIC_COMBINE, s, T > 0 ? next_timing_events(p) : nullptr);
    return paged_end(p, T, active_buf, flags, s, rc);
}

int moe_route_forward(moe_pool *p, const float *logits, const void *x, int64_t T, int32_t block_m,
                      int32_t *topk_ids, float *topk_w, int32_t *sorted_ids, int32_t *block_expert,
                      int32_t *num_padded, int32_t active_buf, void *y, void *ws, size_t ws_bytes,
                      uint32_t flags, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    CHECK(paged_begin(p, T, active_buf, flags, s));
    if (T > 0 && !logits)
        return fail(MOE_ERR_INVALID_ARG, "logits is null");
    const int rc = forward_common(p, nullptr, nullptr, true, x, T, block_m, topk_ids, topk_w, sorted_ids,
                                  block_expert, num_padded, active_buf, y, ws, ws_bytes,
                                  flags & MOE_FLAG_ATOMIC_COMBINE, s, T > 0 ? next_timing_events(p) : nullptr,
                                  logits);
    return paged_end(p, T, active_buf, flags, s, rc);
}

int moe_route_contiguous_forward(const moe_pool *p, const void *w13, const void *w2, const float *logits,
                                 const void *x, int64_t T, int32_t block_m, int32_t *topk_ids, float *topk_w,
                                 int32_t *sorted_ids, int32_t *block_expert, int32_t *num_padded, void *y,
                                 void *ws, size_t ws_bytes, uint32_t flags, void *stream)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    if (T > 0 && !logits)
        return fail(MOE_ERR_INVALID_ARG, "logits is null");
    CHECK(check_dev(w13, 16, "w13"));
    CHECK(check_dev(w2, 16, "w2"));
    return forward_common(p, w13, w2, false, x, T, block_m, topk_ids, topk_w, sorted_ids, block_expert,
                          num_padded, 0, y, ws, ws_bytes, flags, (hipStream_t)stream, nullptr, logits);
}

int moe_contiguous_forward(const moe_pool *p, const void *w13, const void *w2, const void *x, int64_t T,
                           int32_t block_m, const int32_t *topk_ids, const float *topk_w,
                           const int32_t *sorted_ids, const int32_t *block_expert, const int32_t *num_padded,
                           void *y, void *ws, size_t ws_bytes, uint32_t flags, void *stream)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    CHECK(check_dev(w13, 16, "w13"));
    CHECK(check_dev(w2, 16, "w2"));
    return forward_common(p, w13, w2, false, x, T, block_m, topk_ids, topk_w, sorted_ids, block_expert,
                          num_padded, 0, y, ws, ws_bytes, flags, (hipStream_t)stream, nullptr);
}

int moe_loadbuf_fill(moe_pool *p, int32_t buf, int32_t n, const int32_t *slots, const void *const *host_src,
                     void *copy_stream)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    if (buf < 0 || buf > 1)
        return fail(MOE_ERR_INVALID_ARG, "buf must be 0 or 1");
    if (p->desc.loadbuf_slots <= 0)
        return fail(MOE_ERR_STATE, "this layer has no load buffers");
    if (n < 0 || n > p->desc.loadbuf_slots)
        return fail(MOE_ERR_INVALID_ARG, "n out of range");
    if (n > 0 && (!slots || !host_src))
        return fail(MOE_ERR_INVALID_ARG, "slots / host_src is null");
    std::vector<char> seen(p->desc.loadbuf_slots, 0);
    for (int i = 0; i < n; i++) {
        if (slots[i] < 0 || slots[i] >= p->desc.loadbuf_slots)
            return fail(MOE_ERR_SLOT_RANGE, "slot " + std::to_string(slots[i]) + " out of range");
        if (seen[slots[i]])
            return fail(MOE_ERR_SLOT_RANGE, "slot " + std::to_string(slots[i]) + " listed twice");
        seen[slots[i]] = 1;
        if (!host_src[i])
            return fail(MOE_ERR_INVALID_ARG, "host_src entry is null");
        hipPointerAttribute_t attr;
        hipError_t e = hipPointerGetAttributes(&attr, host_src[i]);
        if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return fail(MOE_ERR_INVALID_ARG, "host_src must be pinned host memory");
        }
    }
    hipStream_t s = (hipStream_t)copy_stream;
    // write after read: every stream's last forward that read this buffer
    // (a forward on the copy stream itself is ordered already).  A wait takes
    // an event as recorded at the time of the call, so the events can be
    // reused at once.
    for (const auto &m : p->read_marks[buf]) {
        if (m.stream != s)
            HIP_TRY(hipStreamWaitEvent(s, m.done, 0));
        p->spare_events.push_back(m.done);
    }
    p->read_marks[buf].clear();
    // deferred readers: mark each stream now
    for (hipStream_t r : p->deferred_readers[buf]) {
        if (r == s)
            continue; // same stream: already ordered
        hipEvent_t ev = nullptr;
        CHECK(pmoe::take_read_event(p, &ev));
        p->spare_events.push_back(ev);
        HIP_TRY(hipEventRecord(ev, r));
        HIP_TRY(hipStreamWaitEvent(s, ev, 0));
    }
    p->deferred_readers[buf].clear();
    if (p->ever_filled[buf])
        HIP_TRY(hipStreamWaitEvent(s, p->filled[buf], 0));
    const size_t bytes = (size_t)3 * p->desc.f * p->desc.d * 2;
    char *dst0 = (char *)p->desc.loadbuf_base[buf];
    for (int i = 0; i < n; i++)
        HIP_TRY(hipMemcpyAsync(dst0 + (size_t)slots[i] * bytes, host_src[i], bytes, hipMemcpyHostToDevice, s));
    HIP_TRY(hipEventRecord(p->filled[buf], s));
    p->ever_filled[buf] = true;
    return MOE_OK;
}

int moe_resolve_addrs(moe_pool *p, int32_t active_buf, int64_t n, const int32_t *e, const int32_t *which,
                      const int64_t *row, const int64_t *col, int64_t *off, int32_t *base, void *stream)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    if (active_buf < 0 || active_buf > 1)
        return fail(MOE_ERR_INVALID_ARG, "active_buf must be 0 or 1");
    if (!p->locs_set)
        return fail(MOE_ERR_STATE, "no location table: call moe_set_expert_locs first");
    if (n < 0)
        return fail(MOE_ERR_INVALID_ARG, "n < 0");
    if (n == 0)
        return MOE_OK;
    CHECK(check_dev(e, 4, "e"));
    CHECK(check_dev(which, 4, "which"));
    CHECK(check_dev(row, 8, "row"));
    CHECK(check_dev(col, 8, "col"));
    CHECK(check_dev(off, 8, "off"));
    CHECK(check_dev(base, 4, "base"));
    pmoe::ResolveArgs r{};
    r.locs = p->d_locs;
    r.pool = (const uint16_t *)p->desc.pool_base;
    r.loadbuf0 = (const uint16_t *)p->desc.loadbuf_base[0];
    r.loadbuf1 = (const uint16_t *)p->desc.loadbuf_base[1];
    r.active_buf = active_buf;
    r.d = p->desc.d;
    r.f = p->desc.f;
    r.E_tot = p->E_tot;
    r.n = n;
    r.e = e;
    r.which = which;
    r.row = row;
    r.col = col;
    r.off = off;
    r.base = base;
    HIP_TRY(pmoe::launch_resolve(r, (hipStream_t)stream));
    return MOE_OK;
}

int moe_stage_timing(moe_pool *p, int32_t enable)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pool is null");
    p->timing = enable != 0;
    p->tev_used = 0;
    return MOE_OK;
}

int moe_stage_times(moe_pool *p, float *ms, int32_t *count)
{
    if (!p || !ms || !count)
        return fail(MOE_ERR_INVALID_ARG, "null argument");
    ms[0] = ms[1] = ms[2] = 0.f;
    for (size_t i = 0; i < p->tev_used; i++) {
        auto &ev = p->tev[i];
        HIP_TRY(hipEventSynchronize(ev[3]));
        for (int k = 0; k < 3; k++) {
            float t = 0.f;
            HIP_TRY(hipEventElapsedTime(&t, ev[k], ev[k + 1]));
            ms[k] += t;
        }
    }
    *count = (int32_t)p->tev_used;
    p->tev_used = 0;
    return MOE_OK;
}

int32_t moe_forward_form(const moe_pool *p, int64_t T)
{
    if (!p || T < 0)
        return fail(MOE_ERR_INVALID_ARG, "bad arguments");
    pmoe::FwdArgs a{};
    a.T = T;
    a.d = p->desc.d;
    a.f = p->desc.f;
    a.keff = p->keff;
    return pmoe::decode_fits(a) ? MOE_FORM_DECODE : MOE_FORM_TILES;
}

int32_t moe_route_forward_form(const moe_pool *p, int64_t T)
{
    const int32_t form = moe_forward_form(p, T);
    if (form != MOE_FORM_DECODE)
        return form;
    pmoe::FwdArgs a{};
    a.T = T;
    a.d = p->desc.d;
    a.f = p->desc.f;
    a.keff = p->keff;
    a.E_tot = p->E_tot;
    a.BM = 16; // the smallest block height; the routed form needs T <= block_m
    pmoe::DecRouteArgs r{};
    r.E = p->desc.num_experts;
    return pmoe::decode_routed_fits(a, r) ? MOE_FORM_DECODE_ROUTED : form;
}

int32_t moe_suggest_block_m(const moe_pool *p, int64_t T)
{
    if (!p || T <= 0)
        return 16;
    // expected rows per active expert; cover them with one block when that
    // costs no more MFMA work than two smaller blocks (the weights of an
    // expert's column tile are then streamed once)
    const int64_t n = T * p->keff;
    const int64_t active = n < p->E_tot ? n : p->E_tot;
    const int64_t per = n / active;
    if (per <= 16)
        return 16;
    if (per <= 32)
        return 32;
    if (per <= 64)
        return 64;
    // 256-row tiles (with 256-column down tiles) only pay off once an expert
    // fills several of them: they halve the operand traffic per MFMA but need
    // d to be a multiple of 256
    if (per >= 512 && p->desc.d % 256 == 0 && p->desc.f % 128 == 0)
        return 256;
    return 128;
}

} // extern "C"

// ---------------------------------------------------------------------------- multi-layer pipeline
// One forward pass over L MoE layers (the digest's pipeline section and its
// two alternating loading buffers; the ordering rules at the end of the
// adjuster section).  Layer l reads load buffer l mod 2, so the fill for layer
// l + 1 runs on the copy stream while layer l computes, and the fill for
// layer l + 2 waits until layer l has read the buffer.  A change of a layer's
// table (experts newly cached in reserved pages, experts evicted) is applied
// when the layer next runs, after the copies into the new pages have landed;
// pages the table stops naming stay readable until every forward enqueued
// before the switch (the pass that was running) has finished, and only then
// does moe_pipeline_reclaim report them.

struct moe_pipeline {
    int L = 0;
    std::vector<moe_pool *> layers;
    hipStream_t copy = nullptr;
    hipEvent_t filled[2] = {nullptr, nullptr}, consumed[2] = {nullptr, nullptr};
    bool filled_rec[2] = {false, false}, consumed_rec[2] = {false, false};
    int filled_for[2] = {-1, -1}; // layer the last fill of buffer b was for
    bool unread[2] = {false, false}; // that layer has not run since the fill
    struct Staged {
        bool pending = false;
        std::vector<moe_expert_loc> locs;
        std::vector<int32_t> dropped; // pages of the current table the new one does not name
        hipEvent_t copied = nullptr;  // table upload and page copies done (copy stream)
        bool copied_rec = false;
        // The layer's second device table: the staged table is uploaded into it
        // on the copy stream, and the switch swaps it with the handle's.
        DevLoc *alt = nullptr;
        moe_expert_loc *h_up = nullptr; // pinned source of that upload
        hipEvent_t switched = nullptr;  // forward stream at the last switch
        bool switched_rec = false;
    };
    std::vector<Staged> staged;
    std::vector<std::vector<moe_expert_loc>> current; // table each layer runs with
    hipStream_t fwd = nullptr;                        // the one stream all forwards run on
    bool fwd_set = false;
    struct Batch {
        hipEvent_t done; // recorded on the forward stream at the table switch
        std::vector<int32_t> pages;
    };
    std::vector<Batch> batches; // dropped pages whose last readers may still run
    std::vector<int32_t> ready;  // reclaimable, not yet reported
};

namespace {

std::vector<int32_t> table_pages(const std::vector<moe_expert_loc> &t)
{
    std::vector<int32_t> pg;
    for (const auto &L : t)
        if (L.kind == MOE_LOC_POOL)
            for (int m = 0; m < 3; m++)
                pg.push_back(L.idx[m]);
    std::sort(pg.begin(), pg.end());
    return pg;
}

bool is_pinned(const void *p)
{
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeHost;
}

} // namespace

extern "C" {

int moe_pipeline_create(int32_t L, moe_pool *const *layers, void *copy_stream, moe_pipeline **out)
{
    if (!out)
        return fail(MOE_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    if (L < 1 || !layers)
        return fail(MOE_ERR_INVALID_ARG, "need L >= 1 layer handles");
    const moe_pool_desc &d0 = layers[0] ? layers[0]->desc : moe_pool_desc{};
    for (int l = 0; l < L; l++) {
        if (!layers[l])
            return fail(MOE_ERR_INVALID_ARG, "layer handle " + std::to_string(l) + " is null");
        const moe_pool_desc &d = layers[l]->desc;
        if (d.pool_base != d0.pool_base || d.num_pages != d0.num_pages || d.d != d0.d || d.f != d0.f ||
            d.loadbuf_slots != d0.loadbuf_slots || d.loadbuf_base[0] != d0.loadbuf_base[0] ||
            d.loadbuf_base[1] != d0.loadbuf_base[1])
            return fail(MOE_ERR_INVALID_ARG, "layers must share the pool, d, f and the two load buffers");
        if (layers[l]->device != layers[0]->device)
            return fail(MOE_ERR_INVALID_ARG, "layers must live on one device");
        for (int m = 0; m < l; m++)
            if (layers[m] == layers[l])
                return fail(MOE_ERR_INVALID_ARG, "a layer handle is listed twice");
        if (!layers[l]->locs_set)
            return fail(MOE_ERR_STATE, "layer " + std::to_string(l) + " has no location table");
    }
    moe_pipeline *p = new moe_pipeline();
    p->L = L;
    p->layers.assign(layers, layers + L);
    p->copy = (hipStream_t)copy_stream;
    p->staged.resize(L);
    p->current.resize(L);
    for (int l = 0; l < L; l++) {
        const moe_pool *h = layers[l];
        p->current[l].assign(h->h_stage, h->h_stage + h->E_tot); // the table the handle holds
    }
    {
        std::vector<int32_t> all;
        for (int l = 0; l < L; l++) {
            const std::vector<int32_t> pg = table_pages(p->current[l]);
            all.insert(all.end(), pg.begin(), pg.end());
        }
        std::sort(all.begin(), all.end());
        if (std::adjacent_find(all.begin(), all.end()) != all.end()) {
            delete p;
            return fail(MOE_ERR_PAGE_ALIAS, "two layers' tables name the same page");
        }
    }
    hipError_t e = hipSuccess;
    for (int b = 0; b < 2 && e == hipSuccess; b++) {
        e = hipEventCreateWithFlags(&p->filled[b], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&p->consumed[b], kReadDoneEvent);
    }
    for (int l = 0; l < L && e == hipSuccess; l++) {
        moe_pipeline::Staged &st = p->staged[l];
        const size_t n = (size_t)layers[l]->E_tot;
        e = hipEventCreateWithFlags(&st.copied, hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&st.switched, kReadDoneEvent);
        if (e == hipSuccess)
            e = hipMalloc((void **)&st.alt, sizeof(DevLoc) * n);
        if (e == hipSuccess)
            e = hipHostMalloc((void **)&st.h_up, sizeof(moe_expert_loc) * n, hipHostMallocDefault);
    }
    if (e != hipSuccess) {
        moe_pipeline_destroy(p);
        return hip_fail(e, "pipeline set-up");
    }
    *out = p;
    return MOE_OK;
}

int moe_pipeline_destroy(moe_pipeline *p)
{
    if (!p)
        return MOE_OK;
    for (int b = 0; b < 2; b++) {
        if (p->filled[b]) {
            if (p->filled_rec[b])
                (void)hipEventSynchronize(p->filled[b]);
            (void)hipEventDestroy(p->filled[b]);
        }
        if (p->consumed[b]) {
            if (p->consumed_rec[b])
                (void)hipEventSynchronize(p->consumed[b]);
            (void)hipEventDestroy(p->consumed[b]);
        }
    }
    for (auto &s : p->staged) {
        if (s.copied) {
            if (s.copied_rec)
                (void)hipEventSynchronize(s.copied);
            (void)hipEventDestroy(s.copied);
        }
        if (s.switched) {
            if (s.switched_rec)
                (void)hipEventSynchronize(s.switched); // forwards that read the table in alt
            (void)hipEventDestroy(s.switched);
        }
        if (s.alt)
            (void)hipFree(s.alt);
        if (s.h_up)
            (void)hipHostFree(s.h_up);
    }
    for (auto &bt : p->batches) {
        (void)hipEventSynchronize(bt.done);
        (void)hipEventDestroy(bt.done);
    }
    delete p;
    return MOE_OK;
}

int moe_pipeline_stage_table(moe_pipeline *p, int32_t layer, const moe_expert_loc *locs, int32_t n, int32_t n_copy,
                             const int32_t *copy_expert, const void *const *copy_src)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pipeline is null");
    if (layer < 0 || layer >= p->L)
        return fail(MOE_ERR_INVALID_ARG, "layer out of range");
    moe_pipeline::Staged &st = p->staged[layer];
    if (st.pending)
        return fail(MOE_ERR_STATE, "layer " + std::to_string(layer) + " already has a change waiting to be applied");
    moe_pool *h = p->layers[layer];
    CHECK(moe_validate_locs(&h->desc, locs, n));
    if (n_copy < 0 || (n_copy > 0 && (!copy_expert || !copy_src)))
        return fail(MOE_ERR_INVALID_ARG, "copy list is null or negative");
    // pages this layer may not name: those of the other layers' tables (current
    // and staged) and dropped pages whose last reading pass has not ended
    std::vector<int32_t> busy;
    for (int l = 0; l < p->L; l++) {
        if (l == layer)
            continue;
        for (const auto *t : {&p->current[l], p->staged[l].pending ? &p->staged[l].locs : nullptr})
            if (t) {
                const std::vector<int32_t> pg = table_pages(*t);
                busy.insert(busy.end(), pg.begin(), pg.end());
            }
        if (p->staged[l].pending)
            busy.insert(busy.end(), p->staged[l].dropped.begin(), p->staged[l].dropped.end());
    }
    for (const auto &bt : p->batches)
        busy.insert(busy.end(), bt.pages.begin(), bt.pages.end());
    std::sort(busy.begin(), busy.end());
    const std::vector<moe_expert_loc> nt(locs, locs + n);
    for (int32_t pg : table_pages(nt))
        if (std::binary_search(busy.begin(), busy.end(), pg))
            return fail(MOE_ERR_PAGE_ALIAS, "page " + std::to_string(pg) +
                                                " belongs to another layer or awaits the end of a pass");
    const std::vector<int32_t> cur = table_pages(p->current[layer]);
    std::vector<char> copied(n, 0);
    for (int i = 0; i < n_copy; i++) {
        const int e = copy_expert[i];
        if (e < 0 || e >= n || locs[e].kind != MOE_LOC_POOL)
            return fail(MOE_ERR_INVALID_ARG, "copied expert " + std::to_string(e) + " must be a pool expert of the new table");
        if (copied[e])
            return fail(MOE_ERR_INVALID_ARG, "expert " + std::to_string(e) + " listed twice in the copy list");
        copied[e] = 1;
        for (int m = 0; m < 3; m++)
            if (std::binary_search(cur.begin(), cur.end(), locs[e].idx[m]))
                return fail(MOE_ERR_PAGE_ALIAS, "page " + std::to_string(locs[e].idx[m]) +
                                                    " is read by the current table and cannot receive a copy");
        if (!copy_src[i] || !is_pinned(copy_src[i]))
            return fail(MOE_ERR_INVALID_ARG, "copy sources must be pinned host memory");
    }
    if (st.copied_rec)
        HIP_TRY(hipEventSynchronize(st.copied)); // the last upload from h_up has finished
    std::memcpy(st.h_up, locs, sizeof(moe_expert_loc) * n);
    if (st.switched_rec)
        HIP_TRY(hipStreamWaitEvent(p->copy, st.switched, 0)); // no forward reads alt any more
    HIP_TRY(hipMemcpyAsync(st.alt, st.h_up, sizeof(moe_expert_loc) * n, hipMemcpyHostToDevice, p->copy));
    const int64_t fd = (int64_t)h->desc.f * h->desc.d;
    char *pool = (char *)h->desc.pool_base;
    for (int i = 0; i < n_copy; i++) {
        const moe_expert_loc &L = locs[copy_expert[i]];
        for (int m = 0; m < 3; m++)
            HIP_TRY(hipMemcpyAsync(pool + (int64_t)L.idx[m] * fd * 2, (const char *)copy_src[i] + m * fd * 2, fd * 2,
                                   hipMemcpyHostToDevice, p->copy));
    }
    HIP_TRY(hipEventRecord(st.copied, p->copy));
    st.copied_rec = true;
    st.locs.assign(locs, locs + n);
    const std::vector<int32_t> nxt = table_pages(st.locs);
    st.dropped.clear();
    std::set_difference(cur.begin(), cur.end(), nxt.begin(), nxt.end(), std::back_inserter(st.dropped));
    st.pending = true;
    return MOE_OK;
}

int moe_pipeline_prefetch(moe_pipeline *p, int32_t layer, int32_t n, const int32_t *slots, const void *const *host_src)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pipeline is null");
    if (layer < 0 || layer >= p->L)
        return fail(MOE_ERR_INVALID_ARG, "layer out of range");
    moe_pool *h = p->layers[layer];
    if (h->desc.loadbuf_slots <= 0)
        return fail(MOE_ERR_STATE, "the layers have no load buffers");
    if (n < 0 || n > h->desc.loadbuf_slots || (n > 0 && (!slots || !host_src)))
        return fail(MOE_ERR_INVALID_ARG, "bad slot list");
    std::vector<char> seen(h->desc.loadbuf_slots, 0);
    for (int i = 0; i < n; i++) {
        if (slots[i] < 0 || slots[i] >= h->desc.loadbuf_slots || seen[slots[i]])
            return fail(MOE_ERR_SLOT_RANGE, "slot " + std::to_string(slots[i]) + " out of range or listed twice");
        seen[slots[i]] = 1;
        if (!host_src[i] || !is_pinned(host_src[i]))
            return fail(MOE_ERR_INVALID_ARG, "host_src must be pinned host memory");
    }
    const int b = layer & 1;
    if (p->unread[b] && p->filled_for[b] != layer)
        return fail(MOE_ERR_STATE, "load buffer " + std::to_string(b) + " still holds the experts of layer " +
                                       std::to_string(p->filled_for[b]) + ", which has not run yet");
    if (p->consumed_rec[b])
        HIP_TRY(hipStreamWaitEvent(p->copy, p->consumed[b], 0)); // the previous reader of buffer b is done
    const size_t bytes = (size_t)3 * h->desc.f * h->desc.d * 2;
    char *dst0 = (char *)h->desc.loadbuf_base[b];
    for (int i = 0; i < n; i++)
        HIP_TRY(hipMemcpyAsync(dst0 + (size_t)slots[i] * bytes, host_src[i], bytes, hipMemcpyHostToDevice, p->copy));
    HIP_TRY(hipEventRecord(p->filled[b], p->copy));
    p->filled_rec[b] = true;
    p->filled_for[b] = layer;
    p->unread[b] = true;
    return MOE_OK;
}

int moe_pipeline_forward(moe_pipeline *p, int32_t layer, const void *x, int64_t T, int32_t block_m,
                         const int32_t *topk_ids, const float *topk_w, const int32_t *sorted_ids,
                         const int32_t *block_expert, const int32_t *num_padded, void *y, void *ws, size_t ws_bytes,
                         uint32_t flags, void *stream)
{
    if (!p)
        return fail(MOE_ERR_INVALID_ARG, "pipeline is null");
    if (layer < 0 || layer >= p->L)
        return fail(MOE_ERR_INVALID_ARG, "layer out of range");
    moe_pool *h = p->layers[layer];
    hipStream_t s = (hipStream_t)stream;
    moe_pipeline::Staged &st = p->staged[layer];
    const std::vector<moe_expert_loc> &tab = st.pending ? st.locs : p->current[layer];
    bool uses_lb = false;
    for (const auto &L : tab)
        uses_lb |= L.kind == MOE_LOC_LOADBUF;
    const int b = layer & 1;
    if (uses_lb && p->filled_for[b] != layer)
        return fail(MOE_ERR_STATE, "layer " + std::to_string(layer) + " reads load buffer " + std::to_string(b) +
                                       ", which was last filled for another layer");
    if (p->fwd_set && s != p->fwd)
        return fail(MOE_ERR_INVALID_ARG, "all forwards of a pipeline must run on one stream");
    p->fwd = s;
    p->fwd_set = true;
    if (st.pending) {
        // finish copying (pages and the table) before pointing the layer at the new table
        HIP_TRY(hipStreamWaitEvent(s, st.copied, 0));
        std::swap(h->d_locs, st.alt);
        HIP_TRY(hipEventRecord(st.switched, s));
        st.switched_rec = true;
        h->uses_loadbuf = uses_lb;
        if (h->upload_pending) {
            HIP_TRY(hipEventSynchronize(h->upload_done));
            h->upload_pending = false;
        }
        std::memcpy(h->h_stage, st.locs.data(), sizeof(moe_expert_loc) * st.locs.size());
        p->current[layer] = st.locs;
        st.pending = false;
        if (!st.dropped.empty()) {
            // every earlier forward that may read the dropped pages is on s already
            moe_pipeline::Batch bt;
            bt.pages.swap(st.dropped);
            HIP_TRY(hipEventCreateWithFlags(&bt.done, kReadDoneEvent));
            const hipError_t e = hipEventRecord(bt.done, s);
            if (e != hipSuccess) {
                (void)hipEventDestroy(bt.done);
                return hip_fail(e, "hipEventRecord");
            }
            p->batches.push_back(std::move(bt));
        }
    }
    if (T > 0 && uses_lb) {
        const hipError_t q = hipEventQuery(p->filled[b]);
        if (q == hipErrorNotReady) {
            (void)hipGetLastError();
            HIP_TRY(hipStreamWaitEvent(s, p->filled[b], 0));
        } else if (q != hipSuccess) {
            return hip_fail(q, "hipEventQuery");
        }
    }
    const int rc = forward_common(h, nullptr, nullptr, true, x, T, block_m, topk_ids, topk_w, sorted_ids,
                                  block_expert, num_padded, b, y, ws, ws_bytes, flags, s, nullptr);
    if (T > 0 && uses_lb) {
        // recorded also when the forward failed part-way: launches enqueued
        // before a failing one still read the buffer
        const hipError_t e = hipEventRecord(p->consumed[b], s);
        if (e == hipSuccess)
            p->consumed_rec[b] = true;
        else if (rc == MOE_OK)
            return hip_fail(e, "hipEventRecord");
        else
            (void)hipGetLastError();
    }
    if (rc != MOE_OK)
        return rc;
    if (p->filled_for[b] == layer)
        p->unread[b] = false;
    return MOE_OK;
}

int moe_pipeline_reclaim(moe_pipeline *p, int32_t *pages, int32_t cap, int32_t *n)
{
    if (!p || !n || cap < 0 || (cap > 0 && !pages))
        return fail(MOE_ERR_INVALID_ARG, "bad arguments");
    for (size_t i = 0; i < p->batches.size();) {
        const hipError_t q = hipEventQuery(p->batches[i].done);
        if (q == hipErrorNotReady) {
            (void)hipGetLastError();
            i++;
            continue;
        }
        if (q != hipSuccess)
            return hip_fail(q, "hipEventQuery");
        p->ready.insert(p->ready.end(), p->batches[i].pages.begin(), p->batches[i].pages.end());
        (void)hipEventDestroy(p->batches[i].done);
        p->batches.erase(p->batches.begin() + i);
    }
    const int32_t m = (int32_t)std::min<size_t>(p->ready.size(), (size_t)cap);
    for (int32_t i = 0; i < m; i++)
        pages[i] = p->ready[i];
    p->ready.erase(p->ready.begin(), p->ready.begin() + m);
    *n = m;
    return MOE_OK;
}

} // extern "C"
