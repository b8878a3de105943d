// Expert weights behind remapped virtual addresses: the PagedTensor design of
// the wiki page "FluxMoE: Decoupling Expert Residency for High-Performance MoE
// Serving" (core method), beside Rimuru's in-kernel page lookup.
//
// Every page (one expert matrix, f*d bf16) is its own physical allocation.
// Each is mapped twice: once into a contiguous pool view (page p at p*page,
// the pool the paged kernels read through the location table) or a load-buffer
// view (slot s, matrix m at (3s+m)*page), and once into the expert views that
// the contiguous kernels read unchanged: w13 [E+S][2f][d] (W1 then W3 of each
// expert) and w2 [E+S][d][f].  The page's invariants hold by construction: a
// view address never moves, a view page maps at most one physical page, a
// physical page is only re-pointed after the readers of the old mapping are
// done (the stream is synchronised first), and the physical pages form one
// fixed set that is reused.

#include "moe.h"
#include "internal.h"

#include <hip/hip_runtime.h>

#include <string>
#include <vector>

namespace pmoe {
// experts (E + S) and expert-page bytes (f*d*2) of a layer handle; false for NULL
bool pool_shape(const moe_pool *p, int32_t *E_tot, int64_t *page_bytes);
// the layer handle's load-buffer events around a forward that reads buffer buf
int loadbuf_read_begin(moe_pool *p, int32_t buf, hipStream_t s);
int loadbuf_read_end(moe_pool *p, int32_t buf, uint32_t flags, hipStream_t s);
// the same after a forward whose result is rc, also when it failed part-way
int loadbuf_read_end_after(moe_pool *p, int32_t buf, uint32_t flags, hipStream_t s, int rc);
// the layer handle's load-buffer base addresses
void pool_loadbufs(const moe_pool *p, void *bases[2]);
} // namespace pmoe

struct moe_vmm {
    int device = 0;
    int64_t page = 0, num_pages = 0;
    int32_t slots = 0, E_tot = 0;
    std::vector<hipMemGenericAllocationHandle_t> h; // pool pages, then [buf][slot][matrix]
    std::vector<char> h_ok;
    char *pool_va = nullptr, *lb_va[2] = {nullptr, nullptr}, *w13_va = nullptr, *w2_va = nullptr;
    std::vector<int64_t> src;    // per expert-view page (3e + m; m = W1, W3, W2): handle mapped there, -1 none
    std::vector<char> base_mapped; // per handle: mapped into its pool / load-buffer view
    int64_t gran = 0, align = 0; // minimum and recommended mapping granularity
    bool all_mapped = false, broken = false;
    // the mapped table places experts in load buffer active_buf (whose fills
    // and readers are ordered by the layer handle's events)
    bool uses_loadbuf = false;
    int32_t active_buf = 0;
};

namespace {

int err(int code, const std::string &msg) { return pmoe::set_error(code, msg.c_str()); }

int hip_err(hipError_t e, const char *what)
{
    return err(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define VTRY(call)                                                                                 \
    do {                                                                                           \
        hipError_t e_ = (call);                                                                    \
        if (e_ != hipSuccess)                                                                      \
            return hip_err(e_, #call);                                                             \
    } while (0)

hipMemAccessDesc access_desc(int device)
{
    hipMemAccessDesc a{};
    a.location.type = hipMemLocationTypeDevice;
    a.location.id = device;
    a.flags = hipMemAccessFlagsProtReadWrite;
    return a;
}

char *view_page(const moe_vmm *v, int64_t e, int m)
{
    return m < 2 ? v->w13_va + (2 * e + m) * v->page : v->w2_va + e * v->page;
}

char *base_page(const moe_vmm *v, int64_t hidx)
{
    if (hidx < v->num_pages)
        return v->pool_va + hidx * v->page;
    const int64_t r = hidx - v->num_pages, per_buf = (int64_t)v->slots * 3;
    return v->lb_va[r / per_buf] + (r % per_buf) * v->page;
}

void teardown(moe_vmm *v)
{
    (void)hipDeviceSynchronize();
    for (size_t i = 0; i < v->src.size(); i++)
        if (v->src[i] >= 0)
            (void)hipMemUnmap(view_page(v, (int64_t)i / 3, (int)(i % 3)), v->page);
    for (size_t i = 0; i < v->base_mapped.size(); i++)
        if (v->base_mapped[i])
            (void)hipMemUnmap(base_page(v, (int64_t)i), v->page);
    const int64_t lb = (int64_t)v->slots * 3 * v->page;
    if (v->pool_va)
        (void)hipMemAddressFree(v->pool_va, v->num_pages * v->page);
    for (int b = 0; b < 2; b++)
        if (v->lb_va[b])
            (void)hipMemAddressFree(v->lb_va[b], lb);
    if (v->w13_va)
        (void)hipMemAddressFree(v->w13_va, (int64_t)v->E_tot * 2 * v->page);
    if (v->w2_va)
        (void)hipMemAddressFree(v->w2_va, (int64_t)v->E_tot * v->page);
    for (size_t i = 0; i < v->h.size(); i++)
        if (v->h_ok[i])
            (void)hipMemRelease(v->h[i]);
}

int create_into(moe_vmm *v)
{
    VTRY(hipGetDevice(&v->device));
    int vmm = 0;
    VTRY(hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, v->device));
    if (!vmm)
        return err(MOE_ERR_UNSUPPORTED, "the device does not support virtual memory management");
    hipMemAllocationProp prop{};
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = v->device;
    size_t gran = 0, align = 0;
    VTRY(hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum));
    VTRY(hipMemGetAllocationGranularity(&align, &prop, hipMemAllocationGranularityRecommended));
    if (gran == 0 || v->page % (int64_t)gran)
        return err(MOE_ERR_UNSUPPORTED, "page of " + std::to_string(v->page) +
                                            " bytes is not a multiple of the mapping granularity " +
                                            std::to_string(gran));
    if (align < gran || align % gran)
        align = gran;
    v->gran = (int64_t)gran;
    v->align = (int64_t)align;
    const int64_t n_h = v->num_pages + 2 * (int64_t)v->slots * 3;
    v->h.assign(n_h, hipMemGenericAllocationHandle_t{});
    v->h_ok.assign(n_h, 0);
    v->base_mapped.assign(n_h, 0);
    v->src.assign((size_t)v->E_tot * 3, -1);
    for (int64_t i = 0; i < n_h; i++) {
        VTRY(hipMemCreate(&v->h[i], v->page, &prop, 0));
        v->h_ok[i] = 1;
    }
    VTRY(hipMemAddressReserve((void **)&v->pool_va, v->num_pages * v->page, align, nullptr, 0));
    if (v->slots > 0)
        for (int b = 0; b < 2; b++)
            VTRY(hipMemAddressReserve((void **)&v->lb_va[b], (int64_t)v->slots * 3 * v->page, align, nullptr, 0));
    VTRY(hipMemAddressReserve((void **)&v->w13_va, (int64_t)v->E_tot * 2 * v->page, align, nullptr, 0));
    VTRY(hipMemAddressReserve((void **)&v->w2_va, (int64_t)v->E_tot * v->page, align, nullptr, 0));
    const hipMemAccessDesc acc = access_desc(v->device);
    for (int64_t i = 0; i < n_h; i++) {
        VTRY(hipMemMap(base_page(v, i), v->page, 0, v->h[i], 0));
        v->base_mapped[i] = 1;
        VTRY(hipMemSetAccess(base_page(v, i), v->page, &acc, 1));
    }
    return MOE_OK;
}

} // namespace

extern "C" {

int moe_vmm_create(int64_t page_bytes, int64_t num_pages, int32_t loadbuf_slots, int32_t n_experts_total,
                   moe_vmm **out)
{
    if (!out)
        return err(MOE_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    if (page_bytes <= 0 || num_pages <= 0 || loadbuf_slots < 0 || n_experts_total <= 0 ||
        n_experts_total > 1024)
        return err(MOE_ERR_INVALID_ARG, "sizes out of range");
    moe_vmm *v = new moe_vmm();
    v->page = page_bytes;
    v->num_pages = num_pages;
    v->slots = loadbuf_slots;
    v->E_tot = n_experts_total;
    const int rc = create_into(v);
    if (rc != MOE_OK) {
        const std::string msg = moe_last_error();
        teardown(v);
        delete v;
        return err(rc, msg);
    }
    *out = v;
    return MOE_OK;
}

int moe_vmm_destroy(moe_vmm *v)
{
    if (!v)
        return MOE_OK;
    teardown(v);
    delete v;
    return MOE_OK;
}

int moe_vmm_views(const moe_vmm *v, void **pool_base, void **loadbuf0, void **loadbuf1, void **w13, void **w2)
{
    if (!v)
        return err(MOE_ERR_INVALID_ARG, "vmm is null");
    if (pool_base)
        *pool_base = v->pool_va;
    if (loadbuf0)
        *loadbuf0 = v->lb_va[0];
    if (loadbuf1)
        *loadbuf1 = v->lb_va[1];
    const bool ready = v->all_mapped && !v->broken;
    if (w13)
        *w13 = ready ? v->w13_va : nullptr;
    if (w2)
        *w2 = ready ? v->w2_va : nullptr;
    return MOE_OK;
}

int moe_vmm_granularity(const moe_vmm *v, int64_t *minimum, int64_t *recommended)
{
    if (!v || !minimum || !recommended)
        return err(MOE_ERR_INVALID_ARG, "null argument");
    *minimum = v->gran;
    *recommended = v->align;
    return MOE_OK;
}

int moe_vmm_map_experts(moe_vmm *v, const moe_expert_loc *locs, int32_t n, int32_t active_buf, void *stream,
                        int32_t *n_remapped)
{
    if (!v || !locs)
        return err(MOE_ERR_INVALID_ARG, "null argument");
    if (v->broken)
        return err(MOE_ERR_STATE, "an earlier mapping failed; destroy this object");
    if (n != v->E_tot)
        return err(MOE_ERR_INVALID_ARG, "the table must place all " + std::to_string(v->E_tot) + " experts");
    if (active_buf < 0 || active_buf > 1)
        return err(MOE_ERR_INVALID_ARG, "active_buf must be 0 or 1");
    // the handle behind every expert-view page, checked before anything changes
    std::vector<int64_t> want((size_t)n * 3);
    std::vector<char> seen_page(v->num_pages, 0), seen_slot(v->slots, 0);
    for (int32_t e = 0; e < n; e++) {
        const moe_expert_loc &L = locs[e];
        if (L.kind == MOE_LOC_POOL) {
            for (int m = 0; m < 3; m++) {
                const int64_t p = L.idx[m];
                if (p < 0 || p >= v->num_pages)
                    return err(MOE_ERR_PAGE_RANGE, "page " + std::to_string(p) + " out of range");
                if (seen_page[p]++)
                    return err(MOE_ERR_PAGE_ALIAS, "page " + std::to_string(p) + " used twice");
                want[(size_t)e * 3 + m] = p;
            }
        } else if (L.kind == MOE_LOC_LOADBUF) {
            const int32_t s = L.idx[0];
            if (s < 0 || s >= v->slots || seen_slot[s]++)
                return err(MOE_ERR_SLOT_RANGE, "slot " + std::to_string(s) + " out of range or used twice");
            for (int m = 0; m < 3; m++)
                want[(size_t)e * 3 + m] = v->num_pages + ((int64_t)active_buf * v->slots + s) * 3 + m;
        } else {
            return err(MOE_ERR_INVALID_ARG, "bad location kind for expert " + std::to_string(e));
        }
    }
    // readers of the current mappings are done before any page is re-pointed
    VTRY(hipStreamSynchronize((hipStream_t)stream));
    const hipMemAccessDesc acc = access_desc(v->device);
    int32_t changed = 0;
    for (size_t i = 0; i < want.size(); i++) {
        if (v->src[i] == want[i])
            continue;
        char *va = view_page(v, (int64_t)i / 3, (int)(i % 3));
        hipError_t e = hipSuccess;
        if (v->src[i] >= 0) {
            e = hipMemUnmap(va, v->page);
            if (e == hipSuccess)
                v->src[i] = -1;
        }
        if (e == hipSuccess)
            e = hipMemMap(va, v->page, 0, v->h[want[i]], 0);
        if (e == hipSuccess) {
            v->src[i] = want[i];
            e = hipMemSetAccess(va, v->page, &acc, 1);
        }
        if (e != hipSuccess) {
            v->broken = true;
            v->all_mapped = false;
            return hip_err(e, "remapping an expert view page");
        }
        changed++;
    }
    v->all_mapped = true;
    v->active_buf = active_buf;
    v->uses_loadbuf = false;
    for (int32_t e = 0; e < n; e++)
        v->uses_loadbuf |= locs[e].kind == MOE_LOC_LOADBUF;
    if (n_remapped)
        *n_remapped = changed;
    return MOE_OK;
}

int moe_vmm_forward(const moe_vmm *v, moe_pool *pool, const void *x, int64_t T, int32_t block_m,
                    const int32_t *topk_ids, const float *topk_w, const int32_t *sorted_ids,
                    const int32_t *block_expert, const int32_t *num_padded, void *y, void *ws, size_t ws_bytes,
                    uint32_t flags, void *stream)
{
    if (!v)
        return err(MOE_ERR_INVALID_ARG, "vmm is null");
    if (!v->all_mapped || v->broken)
        return err(MOE_ERR_STATE, "the expert views are not fully mapped");
    if (flags & ~(MOE_FLAG_ATOMIC_COMBINE | MOE_FLAG_DEFER_READ_DONE))
        return err(MOE_ERR_INVALID_ARG, "unknown flag bits");
    int32_t E_tot = 0;
    int64_t page = 0;
    if (!pmoe::pool_shape(pool, &E_tot, &page))
        return err(MOE_ERR_INVALID_ARG, "pool is null");
    if (E_tot != v->E_tot || page != v->page)
        return err(MOE_ERR_INVALID_ARG, "the layer handle's experts or page size differ from the views'");
    // expert views onto a load buffer: the forward waits for that buffer's last
    // fill and marks it read afterwards, through the layer handle whose fills
    // write it (the same events as a paged forward of that buffer)
    const bool lb = T > 0 && v->uses_loadbuf;
    hipStream_t s = (hipStream_t)stream;
    if (lb) {
        void *bases[2] = {nullptr, nullptr};
        pmoe::pool_loadbufs(pool, bases);
        if (bases[v->active_buf] != v->lb_va[v->active_buf])
            return err(MOE_ERR_INVALID_ARG, "the layer handle's load buffers are not these views'");
        const int rc = pmoe::loadbuf_read_begin(pool, v->active_buf, s);
        if (rc != MOE_OK)
            return rc;
    }
    const int rc = moe_contiguous_forward(pool, v->w13_va, v->w2_va, x, T, block_m, topk_ids, topk_w, sorted_ids,
                                          block_expert, num_padded, y, ws, ws_bytes,
                                          flags & MOE_FLAG_ATOMIC_COMBINE, stream);
    if (!lb)
        return rc;
    return pmoe::loadbuf_read_end_after(pool, v->active_buf, flags, s, rc);
}

} // extern "C"
