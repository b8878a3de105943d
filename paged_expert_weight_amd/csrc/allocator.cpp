// Three-tier page pool of the digest "Rimuru: Unified Memory Management for
// Modern LLM Serving via Elastic Expert Offloading", section "One pool for
// data whose sizes differ by orders of magnitude".
//
// One byte range, indexed through a view per page kind (page i of a kind of
// size B is bytes [i*B, (i+1)*B)).  Huge pages (lcm of the expert and SSM page
// sizes, or the expert page) split into expert or SSM pages on demand; an
// expert page splits into KV or convolution-state pages on demand.  A KV
// request takes a free small page already split off, then splits a free expert
// page, then a free huge page into expert pages; a huge page is never cut
// straight into small pages.  Freed pages merge back up as soon as all
// siblings are free.  Small pages of one expert page go to one request where
// possible, so that they are freed together.
//
// Host-only: no HIP calls.  The expert-page index it hands out is the page
// number the GEMM kernels take in the location table.

#include "moe.h"
#include "internal.h"

#include <algorithm>
#include <cstdint>
#include <map>
#include <numeric>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

namespace {

enum : int8_t { kAbsent = -1, kFree = 0, kUsed = 1, kSplitKV = 2, kSplitConv = 3 };
enum : int8_t { kHugeFree = 0, kHugeExpert = 1, kHugeSsm = 2 };

struct SmallKind {
    int64_t bytes = 0;
    int64_t per_mid = 0;             // small pages in one expert page
    int64_t words = 0;               // 64-bit words of one page's free-slot bitmap
    std::vector<uint64_t> freebits;  // [mid][words]: bit set = slot free (split pages only)
    std::vector<int64_t> owner;      // [mid * per_mid + slot]: request, -1 free
    std::vector<int32_t> nfree;      // [mid]: free slots of a split page
    std::set<int64_t> open;          // split pages of this kind with a free slot
    int64_t used = 0, free = 0, split = 0;
};

struct Req {
    std::map<int64_t, int32_t> mids[2]; // expert pages holding this request's small pages -> count
    std::set<int64_t> pages[2];
};

} // namespace

struct moe_alloc {
    int64_t pool_bytes = 0, huge_bytes = 0, expert_bytes = 0, ssm_bytes = 0;
    int64_t n_huge = 0, e_per_huge = 0, s_per_huge = 0;
    bool packing = true;
    std::vector<int8_t> huge;             // kHuge*
    std::set<int64_t> free_huge;
    std::vector<int8_t> mid;              // per expert page: kAbsent / kFree / kUsed / kSplit*
    std::vector<int32_t> mid_busy;        // per huge page: expert pages not free
    std::set<int64_t> free_mid;
    int64_t used_mid = 0;
    std::vector<int8_t> ssm;              // per SSM page: kAbsent / kFree / kUsed
    std::vector<int32_t> ssm_busy;        // per huge page: SSM pages used
    std::set<int64_t> free_ssm;
    int64_t used_ssm = 0;
    SmallKind small[2];
    std::unordered_map<int64_t, Req> reqs;
};

namespace {

int set_error(int code, const std::string &msg) { return pmoe::set_error(code, msg.c_str()); }

int64_t lcm64(int64_t a, int64_t b) { return a / std::gcd(a, b) * b; }

void split_huge_expert(moe_alloc *a, int64_t h)
{
    a->free_huge.erase(h);
    a->huge[h] = kHugeExpert;
    for (int64_t p = h * a->e_per_huge; p < (h + 1) * a->e_per_huge; p++) {
        a->mid[p] = kFree;
        a->free_mid.insert(p);
    }
    a->mid_busy[h] = 0;
}

void split_huge_ssm(moe_alloc *a, int64_t h)
{
    a->free_huge.erase(h);
    a->huge[h] = kHugeSsm;
    for (int64_t s = h * a->s_per_huge; s < (h + 1) * a->s_per_huge; s++) {
        a->ssm[s] = kFree;
        a->free_ssm.insert(s);
    }
    a->ssm_busy[h] = 0;
}

// a free expert page, splitting the lowest free huge page if none is left
int64_t take_free_mid(moe_alloc *a)
{
    if (a->free_mid.empty())
        split_huge_expert(a, *a->free_huge.begin());
    const int64_t p = *a->free_mid.begin();
    a->free_mid.erase(a->free_mid.begin());
    a->mid_busy[p / a->e_per_huge]++;
    return p;
}

void release_mid(moe_alloc *a, int64_t p)
{
    a->mid[p] = kFree;
    a->free_mid.insert(p);
    const int64_t h = p / a->e_per_huge;
    if (--a->mid_busy[h] == 0) { // every expert page under h is free: the huge page returns
        for (int64_t q = h * a->e_per_huge; q < (h + 1) * a->e_per_huge; q++) {
            a->free_mid.erase(q);
            a->mid[q] = kAbsent;
        }
        a->huge[h] = kHugeFree;
        a->free_huge.insert(h);
    }
}

int64_t first_free_slot(const SmallKind &k, int64_t m)
{
    const uint64_t *w = &k.freebits[m * k.words];
    for (int64_t i = 0; i < k.words; i++)
        if (w[i])
            return i * 64 + __builtin_ctzll(w[i]);
    return -1;
}

void take_slot(moe_alloc *a, int kind, int64_t m, int64_t slot, int64_t request)
{
    SmallKind &k = a->small[kind];
    k.freebits[m * k.words + slot / 64] &= ~(1ull << (slot % 64));
    k.owner[m * k.per_mid + slot] = request;
    if (--k.nfree[m] == 0)
        k.open.erase(m);
    k.used++;
    k.free--;
    Req &r = a->reqs[request];
    r.mids[kind][m]++;
    r.pages[kind].insert(m * k.per_mid + slot);
}

int64_t alloc_one_small(moe_alloc *a, int kind, int64_t request)
{
    SmallKind &k = a->small[kind];
    int64_t m = -1;
    if (a->packing) { // a page that already holds this request's pages
        auto it = a->reqs.find(request);
        if (it != a->reqs.end())
            for (const auto &mc : it->second.mids[kind])
                if (k.nfree[mc.first] > 0) {
                    m = mc.first;
                    break;
                }
    }
    if (m < 0 && !k.open.empty())
        m = *k.open.begin();
    if (m < 0) { // split a free expert page (a huge page first if need be)
        m = take_free_mid(a);
        a->mid[m] = kind == MOE_PAGE_KV ? kSplitKV : kSplitConv;
        uint64_t *w = &k.freebits[m * k.words];
        for (int64_t i = 0; i < k.words; i++) {
            const int64_t left = k.per_mid - i * 64;
            w[i] = left >= 64 ? ~0ull : ((1ull << left) - 1);
        }
        k.nfree[m] = (int32_t)k.per_mid;
        k.open.insert(m);
        k.split++;
        k.free += k.per_mid;
    }
    const int64_t slot = first_free_slot(k, m);
    take_slot(a, kind, m, slot, request);
    return m * k.per_mid + slot;
}

void free_one_small(moe_alloc *a, int kind, int64_t q)
{
    SmallKind &k = a->small[kind];
    const int64_t m = q / k.per_mid, slot = q % k.per_mid;
    const int64_t request = k.owner[q];
    k.owner[q] = -1;
    k.freebits[m * k.words + slot / 64] |= 1ull << (slot % 64);
    if (k.nfree[m]++ == 0)
        k.open.insert(m);
    k.used--;
    k.free++;
    auto it = a->reqs.find(request);
    Req &r = it->second;
    r.pages[kind].erase(q);
    auto mc = r.mids[kind].find(m);
    if (--mc->second == 0)
        r.mids[kind].erase(mc);
    if (r.pages[0].empty() && r.pages[1].empty())
        a->reqs.erase(it);
    if (k.nfree[m] == k.per_mid) { // all small pages free: an expert page again
        k.open.erase(m);
        k.split--;
        k.free -= k.per_mid;
        release_mid(a, m);
    }
}

bool distinct(int32_t n, const int64_t *v)
{
    std::vector<int64_t> s(v, v + n);
    std::sort(s.begin(), s.end());
    return std::adjacent_find(s.begin(), s.end()) == s.end();
}

int64_t expert_available(const moe_alloc *a)
{
    return (int64_t)a->free_mid.size() + (int64_t)a->free_huge.size() * a->e_per_huge;
}

} // namespace

extern "C" {

int moe_alloc_create(const moe_alloc_desc *d, moe_alloc **out)
{
    if (!out || !d)
        return set_error(MOE_ERR_INVALID_ARG, "null argument");
    *out = nullptr;
    if (d->pool_bytes <= 0 || d->expert_page_bytes <= 0 || d->kv_page_bytes <= 0 || d->ssm_page_bytes < 0 ||
        d->conv_page_bytes < 0)
        return set_error(MOE_ERR_INVALID_ARG, "page sizes must be positive (SSM and conv may be 0)");
    if (d->flags & ~MOE_ALLOC_NO_PACKING)
        return set_error(MOE_ERR_INVALID_ARG, "unknown flag bits");
    for (int64_t b : {d->kv_page_bytes, d->conv_page_bytes})
        if (b && d->expert_page_bytes % b)
            return set_error(MOE_ERR_INVALID_ARG, "small page sizes must divide the expert page");
    const int64_t H = d->ssm_page_bytes ? lcm64(d->expert_page_bytes, d->ssm_page_bytes) : d->expert_page_bytes;
    if (d->pool_bytes % H)
        return set_error(MOE_ERR_INVALID_ARG, "the pool must hold a whole number of huge pages (" +
                                                  std::to_string(H) + " bytes)");
    moe_alloc *a = new moe_alloc();
    a->pool_bytes = d->pool_bytes;
    a->huge_bytes = H;
    a->expert_bytes = d->expert_page_bytes;
    a->ssm_bytes = d->ssm_page_bytes;
    a->n_huge = d->pool_bytes / H;
    a->e_per_huge = H / d->expert_page_bytes;
    a->s_per_huge = d->ssm_page_bytes ? H / d->ssm_page_bytes : 0;
    a->packing = !(d->flags & MOE_ALLOC_NO_PACKING);
    a->huge.assign(a->n_huge, kHugeFree);
    for (int64_t h = 0; h < a->n_huge; h++)
        a->free_huge.insert(a->free_huge.end(), h);
    const int64_t n_mid = a->n_huge * a->e_per_huge;
    a->mid.assign(n_mid, kAbsent);
    a->mid_busy.assign(a->n_huge, 0);
    a->ssm.assign(a->n_huge * a->s_per_huge, kAbsent);
    a->ssm_busy.assign(a->n_huge, 0);
    const int64_t sb[2] = {d->kv_page_bytes, d->conv_page_bytes};
    for (int k = 0; k < 2; k++) {
        SmallKind &s = a->small[k];
        s.bytes = sb[k];
        if (!sb[k])
            continue;
        s.per_mid = d->expert_page_bytes / sb[k];
        s.words = (s.per_mid + 63) / 64;
        s.freebits.assign(n_mid * s.words, 0);
        s.owner.assign(n_mid * s.per_mid, -1);
        s.nfree.assign(n_mid, 0);
    }
    *out = a;
    return MOE_OK;
}

int moe_alloc_destroy(moe_alloc *a)
{
    delete a;
    return MOE_OK;
}

int moe_alloc_expert_pages(moe_alloc *a, int32_t n, int64_t *pages)
{
    if (!a || n < 0 || (n > 0 && !pages))
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    if (expert_available(a) < n)
        return set_error(MOE_ERR_NO_SPACE, "not enough free expert pages");
    for (int32_t i = 0; i < n; i++) {
        const int64_t p = take_free_mid(a);
        a->mid[p] = kUsed;
        a->used_mid++;
        pages[i] = p;
    }
    return MOE_OK;
}

int moe_free_expert_pages(moe_alloc *a, int32_t n, const int64_t *pages)
{
    if (!a || n < 0 || (n > 0 && !pages))
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    for (int32_t i = 0; i < n; i++)
        if (pages[i] < 0 || pages[i] >= (int64_t)a->mid.size() || a->mid[pages[i]] != kUsed)
            return set_error(MOE_ERR_INVALID_ARG, "page " + std::to_string(pages[i]) + " is not an allocated expert page");
    if (!distinct(n, pages))
        return set_error(MOE_ERR_INVALID_ARG, "a page is listed twice");
    for (int32_t i = 0; i < n; i++) {
        a->used_mid--;
        release_mid(a, pages[i]);
    }
    return MOE_OK;
}

int moe_alloc_ssm_pages(moe_alloc *a, int32_t n, int64_t *pages)
{
    if (!a || n < 0 || (n > 0 && !pages))
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    if (!a->ssm_bytes)
        return set_error(MOE_ERR_INVALID_ARG, "the pool has no SSM pages");
    if ((int64_t)a->free_ssm.size() + (int64_t)a->free_huge.size() * a->s_per_huge < n)
        return set_error(MOE_ERR_NO_SPACE, "not enough free SSM pages");
    for (int32_t i = 0; i < n; i++) {
        if (a->free_ssm.empty())
            split_huge_ssm(a, *a->free_huge.begin());
        const int64_t s = *a->free_ssm.begin();
        a->free_ssm.erase(a->free_ssm.begin());
        a->ssm[s] = kUsed;
        a->ssm_busy[s / a->s_per_huge]++;
        a->used_ssm++;
        pages[i] = s;
    }
    return MOE_OK;
}

int moe_free_ssm_pages(moe_alloc *a, int32_t n, const int64_t *pages)
{
    if (!a || n < 0 || (n > 0 && !pages))
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    for (int32_t i = 0; i < n; i++)
        if (pages[i] < 0 || pages[i] >= (int64_t)a->ssm.size() || a->ssm[pages[i]] != kUsed)
            return set_error(MOE_ERR_INVALID_ARG, "page " + std::to_string(pages[i]) + " is not an allocated SSM page");
    if (!distinct(n, pages))
        return set_error(MOE_ERR_INVALID_ARG, "a page is listed twice");
    for (int32_t i = 0; i < n; i++) {
        const int64_t s = pages[i], h = s / a->s_per_huge;
        a->ssm[s] = kFree;
        a->free_ssm.insert(s);
        a->used_ssm--;
        if (--a->ssm_busy[h] == 0) {
            for (int64_t q = h * a->s_per_huge; q < (h + 1) * a->s_per_huge; q++) {
                a->free_ssm.erase(q);
                a->ssm[q] = kAbsent;
            }
            a->huge[h] = kHugeFree;
            a->free_huge.insert(h);
        }
    }
    return MOE_OK;
}

int moe_alloc_small_pages(moe_alloc *a, int32_t kind, int64_t request, int32_t n, int64_t *pages)
{
    if (!a || n < 0 || (n > 0 && !pages) || request < 0)
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    if (kind != MOE_PAGE_KV && kind != MOE_PAGE_CONV)
        return set_error(MOE_ERR_INVALID_ARG, "kind must be MOE_PAGE_KV or MOE_PAGE_CONV");
    SmallKind &k = a->small[kind];
    if (!k.bytes)
        return set_error(MOE_ERR_INVALID_ARG, "the pool has no pages of this kind");
    if (k.free + expert_available(a) * k.per_mid < n)
        return set_error(MOE_ERR_NO_SPACE, "not enough free small pages");
    for (int32_t i = 0; i < n; i++)
        pages[i] = alloc_one_small(a, kind, request);
    return MOE_OK;
}

int moe_free_small_pages(moe_alloc *a, int32_t kind, int32_t n, const int64_t *pages)
{
    if (!a || n < 0 || (n > 0 && !pages))
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    if ((kind != MOE_PAGE_KV && kind != MOE_PAGE_CONV) || !a->small[kind].bytes)
        return set_error(MOE_ERR_INVALID_ARG, "bad kind");
    const SmallKind &k = a->small[kind];
    for (int32_t i = 0; i < n; i++)
        if (pages[i] < 0 || pages[i] >= (int64_t)k.owner.size() || k.owner[pages[i]] < 0)
            return set_error(MOE_ERR_INVALID_ARG, "page " + std::to_string(pages[i]) + " is not an allocated small page");
    if (!distinct(n, pages))
        return set_error(MOE_ERR_INVALID_ARG, "a page is listed twice");
    for (int32_t i = 0; i < n; i++)
        free_one_small(a, kind, pages[i]);
    return MOE_OK;
}

int moe_free_request(moe_alloc *a, int64_t request, int64_t *n_freed)
{
    if (!a || !n_freed)
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    *n_freed = 0;
    for (int kind = 0; kind < 2; kind++) {
        auto it = a->reqs.find(request);
        if (it == a->reqs.end())
            break;
        const std::vector<int64_t> qs(it->second.pages[kind].begin(), it->second.pages[kind].end());
        for (int64_t q : qs) // ascending; the request entry may vanish with its last page
            free_one_small(a, kind, q);
        *n_freed += (int64_t)qs.size();
    }
    return MOE_OK;
}

int moe_alloc_get_stats(const moe_alloc *a, moe_alloc_stats *s)
{
    if (!a || !s)
        return set_error(MOE_ERR_INVALID_ARG, "bad arguments");
    s->huge_bytes = a->huge_bytes;
    s->n_huge = a->n_huge;
    s->free_huge = (int64_t)a->free_huge.size();
    s->free_expert = (int64_t)a->free_mid.size();
    s->used_expert = a->used_mid;
    s->free_ssm = (int64_t)a->free_ssm.size();
    s->used_ssm = a->used_ssm;
    s->trapped_bytes = 0;
    for (int k = 0; k < 2; k++) {
        s->split[k] = a->small[k].split;
        s->used_small[k] = a->small[k].used;
        s->free_small[k] = a->small[k].free;
        s->trapped_bytes += a->small[k].free * a->small[k].bytes;
    }
    s->expert_available = expert_available(a);
    return MOE_OK;
}

} // extern "C"
