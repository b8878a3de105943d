// Top-k softmax routing and token alignment (gfx950, wave64).
//
// Routing: one wave per token (route_token.h: each lane sorts its logits into
// pick order, every pick is a wave max of the lanes' first entries with ties
// to the lower id; weights are the softmax renormalised over the k picks; a
// shared expert is appended with weight 1).  The pages do not print a routing
// rule; this is the top-k softmax router of the MoE layer whose fused kernel
// the Rimuru digest's kernel section rewrites.
//
// Alignment: a stable counting sort of the flat picks i = t*(k+S) + j by expert
// with each expert's run padded to the GEMM tile height BM, so that every
// BM-row block of the grouped GEMMs belongs to one expert:
//   histogram (per chunk of flat entries: counts are order free)
//   -> exclusive scan of the padded counts over experts, and of the raw counts
//      over chunks and waves (the start of every (chunk, wave, expert) run)
//   -> in-order scatter: inside a chunk each wave owns a contiguous range and
//      walks it 64 entries at a time.  The lanes that hold the same expert are
//      found in one pass by slicing the expert id into bits (one ballot per
//      bit: the lanes agreeing with mine on every bit hold my expert); a lane's
//      rank is the popcount of the matching lanes below it, and the lowest
//      matching lane advances the run's cursor by the match count.  Distinct
//      experts of a group update distinct cursors, so the 64 entries of a group
//      are placed at once, in flat order.
// Small batches run routing and alignment in one workgroup (one launch; the
// smallest with a leaner eight-wave form); larger ones route with one wave per token and align in one workgroup up to
// kChunkElems entries, or over chunks with two launches: the per-chunk histograms,
// then one workgroup per chunk that scans the counts and scatters its chunk.
#include "internal.h"
#include "route_token.h"

namespace pmoe {
namespace {

using namespace rt;

// Workgroup barrier that orders LDS only.  Nothing these kernels store to
// global memory is read back by another thread of the same launch, so the
// barriers need not wait for global stores to complete (a full __syncthreads
// would, costing a memory round trip at every phase).
__device__ __forceinline__ void lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kAlignWaves = 16;
constexpr int kAlignThreads = 64 * kAlignWaves;
constexpr int kChunkElems = 8192; // flat entries aligned by one workgroup (the one-workgroup forms)
constexpr int kMultiChunk = 2048;  // flat entries per histogram / scatter workgroup of larger batches
constexpr int kSmallTokens = 64;  // route + align in one workgroup when T <= this (and T*keff <= kChunkElems)

template <int NV>
__global__ __launch_bounds__(256) void k_route(const RouteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T)
        return;
    float v[NV];
    load_logits<NV>(a.logits + t * a.E, a.E, lane, v);
    route_token<NV>(v, a.E, a.k, a.S, lane, a.topk_ids + t * a.keff, a.topk_w + t * a.keff, nullptr);
}

// Route a wave's tokens (token r's outputs at flat offset off + r * step, its
// ids also at lds_ids + r * step): all R at once when all are live, so that
// their cross-lane steps overlap, else the live ones one after the other (an
// interleaved round of dead tokens costs issue slots and gains nothing).
template <int NV, int R>
__device__ __forceinline__ void route_wave_tokens(const float (&v)[R][NV], const bool (&live)[R], const RouteArgs &a,
                                                  int lane, int64_t off, int step, int32_t *lds_ids)
{
    if (live[R - 1]) {
        route_token_n<NV, R>(v, live, a.E, a.k, a.S, lane, a.topk_ids + off, a.topk_w + off, step, lds_ids);
        return;
    }
#pragma unroll
    for (int r = 0; r < R - 1; r++)
        if (live[r])
            route_token<NV>(v[r], a.E, a.k, a.S, lane, a.topk_ids + off + r * step, a.topk_w + off + r * step,
                            lds_ids + r * step);
}

// dst[i] = src[i] for i < n (n <= kChunkElems): all loads of a thread are
// issued before any of them is waited for.
__device__ __forceinline__ void stage_ids(int32_t *dst, const int32_t *src, int n)
{
    constexpr int R = kChunkElems / kAlignThreads;
    int32_t v[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int i = threadIdx.x + r * kAlignThreads;
        v[r] = i < n ? src[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int i = threadIdx.x + r * kAlignThreads;
        if (i < n)
            dst[i] = v[r];
    }
}

__device__ __forceinline__ void wave_range(int n, int w, int &lo, int &hi)
{
    int per = (n + kAlignWaves - 1) / kAlignWaves;
    per = (per + 63) & ~63;
    lo = min(n, w * per);
    hi = min(n, lo + per);
}

// Lanes of the wave whose id equals mine (valid lanes only), from one ballot per id bit.
__device__ __forceinline__ uint64_t same_id_lanes(int e, bool valid, int nbits)
{
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; b++) {
        const bool bit = (e >> b) & 1;
        const uint64_t on = __ballot(bit);
        m &= bit ? on : ~on;
    }
    return m;
}

__device__ __forceinline__ int id_bits(int E_tot)
{
    int b = 0;
    while ((1 << b) < E_tot)
        b++;
    return b;
}

__device__ __forceinline__ uint64_t lanes_below()
{
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Per-wave histogram of the chunk s_ids[0..n): s_cnt[w*E_tot + e] (must start
// at zero).  Counts do not depend on order, so each entry is one LDS atomic add
// (the id matching of the scatter costs a ballot per id bit).
__device__ void chunk_hist(const int32_t *s_ids, int n, int E_tot, int *s_cnt)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int lo, hi;
    wave_range(n, w, lo, hi);
    for (int i = lo + lane; i < hi; i += 64)
        atomicAdd(&s_cnt[w * E_tot + s_ids[i]], 1);
}

// In-order scatter of the chunk s_ids[0..n) whose first flat index is elem0.
// s_cur[w*E_tot + e] = position in sorted_ids of wave w's next entry of expert e.
__device__ void chunk_scatter(const int32_t *s_ids, int n, int elem0, int E_tot, int *s_cur,
                              int32_t *sorted_ids)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nbits = id_bits(E_tot);
    const uint64_t below = lanes_below();
    int lo, hi;
    wave_range(n, w, lo, hi);
    for (int g = lo; g < hi; g += 64) {
        const int i = g + lane;
        const bool valid = i < hi;
        const int e = valid ? s_ids[i] : 0;
        const uint64_t m = same_id_lanes(e, valid, nbits);
        if (valid) {
            const int base = s_cur[w * E_tot + e];
            sorted_ids[base + __popcll(m & below)] = elem0 + i;
        }
        // every lane has read its cursor before any leader moves one
        __builtin_amdgcn_wave_barrier();
        if (valid && (m & below) == 0)
            s_cur[w * E_tot + e] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

// Exclusive scan across the workgroup of one int per thread; *total gets the sum.
__device__ int wg_exclusive_scan(int v, int *s_tmp, int *total)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        s_tmp[w] = x;
    lds_sync();
    int before = 0, all = 0;
    for (int i = 0; i < kAlignWaves; i++) {
        const int s = s_tmp[i];
        before += i < w ? s : 0;
        all += s;
    }
    lds_sync();
    *total = all;
    return before + x - v;
}

// Given per-expert token counts cnt(e): each expert's padded segment start in
// seg_start[e] (and its count in seg_cnt[e]) and num_padded.  Thread t owns
// expert t (E_tot <= kAlignThreads).
template <class CountFn>
__device__ void scan_segments(CountFn cnt, int E_tot, int BM, int *seg_start, int *seg_cnt, int *s_tmp,
                              const RouteArgs &a)
{
    const int e = threadIdx.x;
    const int c = e < E_tot ? cnt(e) : 0;
    const int p = (c + BM - 1) / BM * BM;
    int total;
    const int o = wg_exclusive_scan(p, s_tmp, &total);
    if (e < E_tot) {
        seg_start[e] = o;
        seg_cnt[e] = c;
    }
    if (threadIdx.x == 0)
        *a.num_padded = total;
}

// The sentinel padding and block->expert map of experts [e0, e1), one wave per
// expert run with its lanes on consecutive positions.
template <class SegFn>
__device__ void pad_segments(SegFn seg, int e0, int e1, int BM, int n, const RouteArgs &a)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int x = e0 + w; x < e1; x += kAlignWaves) {
        int ox, cx;
        seg(x, ox, cx);
        const int px = (cx + BM - 1) / BM * BM;
        for (int i = lane; i < px - cx; i += 64)
            a.sorted_ids[ox + cx + i] = n;
        for (int i = lane; i < px / BM; i += 64)
            a.block_expert[ox / BM + i] = x;
    }
}

// Both, for a batch aligned by one workgroup.
template <class CountFn>
__device__ void scan_experts(CountFn cnt, int E_tot, int BM, int n, int *seg_start, int *seg_cnt, int *s_tmp,
                             const RouteArgs &a)
{
    scan_segments(cnt, E_tot, BM, seg_start, seg_cnt, s_tmp, a);
    lds_sync();
    pad_segments([&](int x, int &ox, int &cx) { ox = seg_start[x]; cx = seg_cnt[x]; }, 0, E_tot, BM, n, a);
}

// Turn per-wave counts s_cnt[w][e] into per-wave cursors starting at start(e).
template <class StartFn>
__device__ void wave_cursors(StartFn start, int E_tot, int *s_cnt)
{
    for (int e = threadIdx.x; e < E_tot; e += kAlignThreads) {
        int run = start(e);
        for (int w = 0; w < kAlignWaves; w++) {
            const int c = s_cnt[w * E_tot + e];
            s_cnt[w * E_tot + e] = run;
            run += c;
        }
    }
}

struct AlignSmem {
    int32_t ids[kChunkElems];
    int cnt[kAlignWaves * kMaxExpertsTotal];
    int seg[kMaxExpertsTotal];
    int segc[kMaxExpertsTotal];
    int tmp[kAlignWaves];
};

__device__ void zero_counts(AlignSmem &sm, int E_tot)
{
    for (int i = threadIdx.x; i < kAlignWaves * E_tot; i += kAlignThreads)
        sm.cnt[i] = 0;
}

// Alignment of a whole batch in one workgroup (n <= kChunkElems); sm.ids filled, sm.cnt zero.
__device__ void align_in_one_wg(AlignSmem &sm, int n, const RouteArgs &a)
{
    chunk_hist(sm.ids, n, a.E_tot, sm.cnt);
    lds_sync();
    auto count = [&](int e) {
        int c = 0;
        for (int w = 0; w < kAlignWaves; w++)
            c += sm.cnt[w * a.E_tot + e];
        return c;
    };
    scan_experts(count, a.E_tot, a.BM, n, sm.seg, sm.segc, sm.tmp, a);
    lds_sync();
    wave_cursors([&](int e) { return sm.seg[e]; }, a.E_tot, sm.cnt);
    lds_sync();
    chunk_scatter(sm.ids, n, 0, a.E_tot, sm.cnt, a.sorted_ids);
}

template <int NV>
__global__ __launch_bounds__(kAlignThreads) void k_route_align_small(const RouteArgs a)
{
    __shared__ AlignSmem sm;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    zero_counts(sm, a.E_tot);
    // this wave's tokens w, w+16, ... (at most kSmallTokens/kAlignWaves): load
    // all their logits first, then route them
    constexpr int TPW = kSmallTokens / kAlignWaves;
    float v[TPW][NV];
    bool live[TPW];
#pragma unroll
    for (int r = 0; r < TPW; r++) {
        const int t = w + r * kAlignWaves;
        live[r] = t < (int)a.T;
        if (live[r])
            load_logits<NV>(a.logits + (int64_t)t * a.E, a.E, lane, v[r]);
        else
#pragma unroll
            for (int i = 0; i < NV; i++)
                v[r][i] = 0.f;
    }
    route_wave_tokens<NV, TPW>(v, live, a, lane, (int64_t)w * a.keff, kAlignWaves * a.keff, sm.ids + w * a.keff);
    lds_sync();
    align_in_one_wg(sm, (int)a.T * a.keff, a);
}

// Tiny batches (T <= kTinyTokens, T*(k+S) <= kTinyPicks): routing and alignment
// in one workgroup of eight waves with four barriers.  Wave w routes tokens w,
// w+8, ...; then holds flat picks [64w, 64w+64) and counts them per expert with
// the bit-sliced lane match; thread t scans experts 2t and 2t+1 (padded counts,
// exclusive over experts, then per-wave cursors) and writes their padding and
// block map; finally every pick is placed at its wave's cursor plus its rank
// among the lanes below with the same expert.
constexpr int kTinyWaves = 8, kTinyThreads = 64 * kTinyWaves;
constexpr int kTinyTokens = 32, kTinyPicks = 64 * kTinyWaves;

template <int NV>
__global__ __launch_bounds__(kTinyThreads) void k_route_align_tiny(const RouteArgs a)
{
    __shared__ int32_t s_ids[kTinyPicks];
    __shared__ int s_cnt[kTinyWaves * kMaxExpertsTotal]; // per-wave counts, then per-wave cursors
    __shared__ int s_wsum[kTinyWaves];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int E_tot = a.E_tot, BM = a.BM;
    const int n = (int)a.T * a.keff;
    for (int i = threadIdx.x; i < kTinyWaves * E_tot; i += kTinyThreads)
        s_cnt[i] = 0;
    constexpr int TPW = kTinyTokens / kTinyWaves;
    float v[TPW][NV];
    bool live[TPW];
#pragma unroll
    for (int r = 0; r < TPW; r++) {
        const int t = w + r * kTinyWaves;
        live[r] = t < (int)a.T;
        if (live[r])
            load_logits<NV>(a.logits + (int64_t)t * a.E, a.E, lane, v[r]);
        else
#pragma unroll
            for (int i = 0; i < NV; i++)
                v[r][i] = 0.f;
    }
    route_wave_tokens<NV, TPW>(v, live, a, lane, (int64_t)w * a.keff, kTinyWaves * a.keff, s_ids + w * a.keff);
    lds_sync();

    // per-wave counts and each pick's rank within its wave
    const int p = 64 * w + lane;
    const bool valid = p < n;
    const int e = valid ? s_ids[p] : 0;
    const uint64_t m = same_id_lanes(e, valid, id_bits(E_tot));
    const int rank = __popcll(m & lanes_below());
    if (valid && rank == 0)
        s_cnt[w * E_tot + e] = __popcll(m);
    lds_sync();

    // experts 2t, 2t+1: totals, padded segment starts, cursors, padding, block map
    int tot[2], pad[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int x = 2 * (int)threadIdx.x + q;
        int c = 0;
        if (x < E_tot)
            for (int ww = 0; ww < kTinyWaves; ww++)
                c += s_cnt[ww * E_tot + x];
        tot[q] = c;
        pad[q] = (c + BM - 1) / BM * BM;
    }
    const int local = pad[0] + pad[1];
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off)
            incl += y;
    }
    if (lane == 63)
        s_wsum[w] = incl;
    lds_sync();
    int base = 0, all = 0;
    for (int ww = 0; ww < kTinyWaves; ww++) {
        const int sv = s_wsum[ww];
        base += ww < w ? sv : 0;
        all += sv;
    }
    if (threadIdx.x == 0)
        *a.num_padded = all;
    int seg = base + incl - local;
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int x = 2 * (int)threadIdx.x + q;
        if (x < E_tot && pad[q] > 0) {
            int run = seg;
            for (int ww = 0; ww < kTinyWaves; ww++) {
                const int c = s_cnt[ww * E_tot + x];
                s_cnt[ww * E_tot + x] = run;
                run += c;
            }
            for (int i = seg + tot[q]; i < seg + pad[q]; i++)
                a.sorted_ids[i] = n;
            for (int bb = seg / BM; bb < (seg + pad[q]) / BM; bb++)
                a.block_expert[bb] = x;
        }
        seg += pad[q];
    }
    lds_sync();
    if (valid)
        a.sorted_ids[s_cnt[w * E_tot + e] + rank] = p;
}

__global__ __launch_bounds__(kAlignThreads) void k_align_single(const RouteArgs a)
{
    __shared__ AlignSmem sm;
    const int n = (int)a.T * a.keff;
    zero_counts(sm, a.E_tot);
    stage_ids(sm.ids, a.topk_ids, n);
    lds_sync();
    align_in_one_wg(sm, n, a);
}

// Per-chunk counts are stored expert-major, counts[e][ch] with a row stride of
// the chunk count rounded up to 4, so one expert's column is contiguous.
__host__ __device__ __forceinline__ int count_stride(int64_t n)
{
    const int nch = (int)((n + kMultiChunk - 1) / kMultiChunk);
    return (nch + 3) & ~3;
}

__global__ __launch_bounds__(kAlignThreads) void k_align_hist(const RouteArgs a)
{
    __shared__ int hist[kMaxExpertsTotal];
    const int64_t n = a.T * a.keff;
    const int64_t lo = (int64_t)blockIdx.x * kMultiChunk;
    const int cn = (int)min((int64_t)kMultiChunk, n - lo);
    for (int e = threadIdx.x; e < a.E_tot; e += kAlignThreads)
        hist[e] = 0;
    constexpr int R = kMultiChunk / kAlignThreads;
    int32_t v[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int i = threadIdx.x + r * kAlignThreads;
        v[r] = i < cn ? a.topk_ids[lo + i] : -1;
    }
    lds_sync();
#pragma unroll
    for (int r = 0; r < R; r++)
        if (v[r] >= 0)
            atomicAdd(&hist[v[r]], 1);
    lds_sync();
    const int nchp = count_stride(n);
    for (int e = threadIdx.x; e < a.E_tot; e += kAlignThreads)
        a.counts[(int64_t)e * nchp + blockIdx.x] = hist[e];
}

// One workgroup per chunk of flat entries.  Every workgroup reads the whole
// count table (E_tot columns of nch chunks: 90 KB for 90112 picks over 513
// experts) for each expert's total and its count in the chunks before its own,
// scans the padded totals into segment starts (the same scan in every
// workgroup; workgroup 0 stores num_padded), then ranks and scatters its chunk
// and writes the padding and block map of its share of the experts.  Thread e
// holds expert e's column in registers, kScanRegs chunks at a time (16-byte
// loads, all issued before the first is used).  Doing the scan here instead of
// in a one-workgroup launch of its own takes a launch and its memory round
// trips off the step.
constexpr int kScanRegs = 48;

__global__ __launch_bounds__(kAlignThreads) void k_align_scatter(const RouteArgs a, int nch)
{
    __shared__ AlignSmem sm;
    const int64_t n = a.T * a.keff;
    const int ch = (int)blockIdx.x;
    const int64_t lo = (int64_t)ch * kMultiChunk;
    const int cn = (int)min((int64_t)kMultiChunk, n - lo);
    const int nchp = count_stride(n);
    const int e = threadIdx.x; // E_tot <= kAlignThreads
    const bool mine = e < a.E_tot;
    const int32_t *col = a.counts + (int64_t)(mine ? e : 0) * nchp;
    int tot = 0, before = 0;
    for (int ch0 = 0; ch0 < nch; ch0 += kScanRegs) {
        int4 v[kScanRegs / 4];
#pragma unroll
        for (int r = 0; r < kScanRegs / 4; r++)
            v[r] = (mine && ch0 + 4 * r < nchp) ? *(const int4 *)(col + ch0 + 4 * r) : make_int4(0, 0, 0, 0);
        if (ch0 == 0) { // this chunk's ids are staged while the first columns load
            zero_counts(sm, a.E_tot);
            stage_ids(sm.ids, a.topk_ids + lo, cn);
        }
        // entries past nch (row padding) are never written: count only chunks < nch
#pragma unroll
        for (int i = 0; i < kScanRegs; i++) {
            const int4 q = v[i / 4];
            const int x = (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
            const int c = ch0 + i;
            tot += c < nch ? x : 0;
            before += c < ch ? x : 0;
        }
    }
    int total;
    const int seg = wg_exclusive_scan(mine ? (tot + a.BM - 1) / a.BM * a.BM : 0, sm.tmp, &total);
    if (mine) {
        sm.seg[e] = seg;
        sm.segc[e] = tot;
    }
    if (ch == 0 && threadIdx.x == 0)
        *a.num_padded = total;
    chunk_hist(sm.ids, cn, a.E_tot, sm.cnt);
    lds_sync();
    wave_cursors([&](int) { return seg + before; }, a.E_tot, sm.cnt);
    lds_sync();
    chunk_scatter(sm.ids, cn, (int)lo, a.E_tot, sm.cnt, a.sorted_ids);
    // this workgroup's share of the experts: their padding and block map (one
    // workgroup would issue all of these stores alone, at one CU's store rate)
    const int e0 = (int)((int64_t)blockIdx.x * a.E_tot / gridDim.x);
    const int e1 = (int)((int64_t)(blockIdx.x + 1) * a.E_tot / gridDim.x);
    pad_segments([&](int x, int &ox, int &cx) { ox = sm.seg[x]; cx = sm.segc[x]; }, e0, e1, a.BM, (int)n, a);
}

template <int NV>
hipError_t launch_nv(const RouteArgs &a, hipStream_t s)
{
    const int64_t n = a.T * a.keff;
    if (a.T <= kTinyTokens && n <= kTinyPicks && a.E_tot <= 2 * kTinyThreads) {
        k_route_align_tiny<NV><<<1, kTinyThreads, 0, s>>>(a);
        return hipGetLastError();
    }
    if (a.T <= kSmallTokens && n <= kChunkElems) {
        k_route_align_small<NV><<<1, kAlignThreads, 0, s>>>(a);
        return hipGetLastError();
    }
    k_route<NV><<<(unsigned)((a.T + 3) / 4), 256, 0, s>>>(a);
    if (n <= kChunkElems) {
        k_align_single<<<1, kAlignThreads, 0, s>>>(a);
    } else {
        const int nch = (int)((n + kMultiChunk - 1) / kMultiChunk);
        k_align_hist<<<nch, kAlignThreads, 0, s>>>(a);
        k_align_scatter<<<nch, kAlignThreads, 0, s>>>(a, nch);
    }
    return hipGetLastError();
}

} // namespace

int64_t route_workspace_bytes(int64_t T, int keff, int E_tot)
{
    const int64_t n = T * keff;
    if (n <= kChunkElems)
        return 0;
    // counts [E_tot][stride]
    return (int64_t)count_stride(n) * E_tot * (int64_t)sizeof(int32_t);
}

hipError_t launch_route_align(const RouteArgs &a, hipStream_t s)
{
    if (a.T <= 0)
        return hipSuccess;
    if (a.E <= 64)
        return launch_nv<1>(a, s);
    if (a.E <= 128)
        return launch_nv<2>(a, s);
    if (a.E <= 256)
        return launch_nv<4>(a, s);
    if (a.E <= 512)
        return launch_nv<8>(a, s);
    return launch_nv<16>(a, s);
}

} // namespace pmoe
