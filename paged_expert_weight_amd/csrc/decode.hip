// Decode form of the layer's two GEMMs for a handful of tokens.
//
// With T <= 8 tokens every expert block holds at most T valid rows, so a
// 16-row MFMA tile would multiply mostly padding while the layer is bound by
// streaming the touched experts' weights once (the same page-addressed reads
// as the digest "Rimuru: Unified Memory Management for Modern LLM Serving via
// Elastic Expert Offloading", kernel section: page resolved once per expert,
// then fixed strides inside the page).  Here each weight row is read once and
// dotted on the vector ALUs with the x rows of all picks that chose the expert:
//
//   gate/up: for expert block b and rows r of the intermediate dimension,
//            h[pick][r] = bf16(silu(W1[r] . x_t) * (W3[r] . x_t)) for every
//            valid pick of the block (h in pick order t*keff + j);
//   down + combine: for token t and output columns c,
//            y[t][c] = bf16(sum_j  w_tj * (W2_{e_tj}[c] . h[t*keff + j])),
//            the picks added in slot order j, so the result is reproducible
//            and no per-pick partial rows or combine pass are needed.
//
// Dot products: each lane takes 8 consecutive elements of every 512-element
// chunk of the row, accumulates in fp32, and the wave adds its lanes with a
// fixed butterfly; the same order for paged and contiguous weights.

#include "internal.h"
#include "route_token.h"

#include <hip/hip_runtime.h>

namespace pmoe {
namespace {

constexpr int kDecWaves = 4;
// Granularity: intermediate rows per gate/up wave and output columns per down
// workgroup.  Batches of 2+ tokens run 2 rows / 4 columns; a one-token step runs
// 1 row / 2 columns (twice the workgroups, each with half the loads: 17.1
// against 17.8 us per Qwen1.5-shaped step; at 4 tokens it is 4 % slower).
constexpr int kDecRowsPerWave = 2;  // gate/up: intermediate rows per wave
constexpr int kDecColsPerGroup = 4; // down: output columns per workgroup
constexpr int kDecRowsPerWave1 = 1, kDecColsPerGroup1 = 2; // T = 1
constexpr int kDecMaxT = 8;         // tokens (hence valid rows of one expert block)
constexpr int kDecMaxD = 4096;
constexpr int kDecMaxKeff = 64;   // picks per token (top-k plus the shared expert)
// Routing inside the gate/up launch pays off up to this many tokens: every
// workgroup routes all of them before its first weight load, and the rows of
// workgroups past the chosen experts route too before they can exit.
// Measured one-step times (Qwen1.5-shaped layer, us, separate routing launch /
// routing inside): T=1 24.3 / 19.5, 2 34.5 / 30.9, 4 56.7 / 54.0,
// 6 73.5 / 74.7, 8 87.9 / 91.1.
constexpr int kDecRoutedMaxT = 4;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u); // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// 8 bf16 of a (weights) times 8 bf16 of b, added to acc with packed dot2
// instructions (the bf16 pairs are used as loaded, no unpacking)
__device__ __forceinline__ float dot8(uint4 a, uint4 b, float acc)
{
    acc = dot2(a.x, b.x, acc);
    acc = dot2(a.y, b.y, acc);
    acc = dot2(a.z, b.z, acc);
    acc = dot2(a.w, b.w, acc);
    return acc;
}

// A weight chunk: read once per step, so loaded non-temporally (a streaming
// read of HBM measured ~7.0 TB/s this way against ~6.2 TB/s with plain loads).
__device__ __forceinline__ uint4 load_stream(const uint16_t *p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// lanes' partial sums added with DPP row steps and lane swaps (route_token.h)
__device__ __forceinline__ float wave_sum(float v) { return rt::wave_sum(v, threadIdx.x & 63); }

// Base of matrix m (0 W1, 1 W3, 2 W2) of expert e: a pool page, a load-buffer
// slot (W1, W3, W2 back to back), or the contiguous arrays.
// Base of matrix m of the expert whose table entry is L (kind, idx[0..2]).
__device__ __forceinline__ const uint16_t *matrix_base_of(const FwdArgs &a, int4 L, int m)
{
    const int64_t fd = (int64_t)a.f * a.d;
    const bool in_pool = L.x == 0; // selects: no field is loaded late
    const int64_t o = in_pool ? (int64_t)(m == 0 ? L.y : m == 1 ? L.z : L.w) * fd : ((int64_t)L.y * 3 + m) * fd;
    return (in_pool ? a.pool : a.loadbuf) + o;
}

template <bool PAGED>
__device__ __forceinline__ const uint16_t *matrix_base(const FwdArgs &a, int e, int m)
{
    const int64_t fd = (int64_t)a.f * a.d;
    if constexpr (PAGED) {
        // the whole 16-byte entry in one load (the table is 16-byte aligned)
        return matrix_base_of(a, *(const int4 *)(a.locs + e), m);
    } else {
        if (m < 2)
            return a.w13 + (int64_t)e * 2 * fd + m * fd;
        return a.w2 + (int64_t)e * fd;
    }
}

// Gate/up rows of expert e for the picks pick(0 .. ncand) (flat index or -1,
// ascending): every wave works on its own (no LDS, no barrier): it issues its
// weight rows first, finds the valid picks with a ballot while those loads are
// in flight, then reads each pick's x row (shared by all waves, so mostly from
// L2) and writes that pick's h values.
template <int NCH, int RPW, class PickFn>
__device__ __forceinline__ void dec_gate_up_rows(const FwdArgs &a, const uint16_t *w1, const uint16_t *w3, int ncand,
                                                 PickFn pick)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = ((int)blockIdx.x * kDecWaves + wave) * RPW;
    uint4 g[RPW][NCH], u[RPW][NCH];
#pragma unroll
    for (int r = 0; r < RPW; r++)
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            const int o = c * 512 + lane * 8;
            if (o < a.d) {
                g[r][c] = load_stream(&w1[(int64_t)(r0 + r) * a.d + o]);
                u[r][c] = load_stream(&w3[(int64_t)(r0 + r) * a.d + o]);
            } else {
                g[r][c] = make_uint4(0, 0, 0, 0);
                u[r][c] = make_uint4(0, 0, 0, 0);
            }
        }
    for (int i0 = 0; i0 < ncand; i0 += 64) {
        const int cand = i0 + lane < ncand ? pick(i0 + lane) : -1;
        uint64_t m = __ballot(cand >= 0);
        while (m) {
            const int bit = __builtin_ctzll(m);
            m &= m - 1;
            const int flat = __shfl(cand, bit, 64);
            const int64_t t = flat / a.keff;
            float sg[RPW], su[RPW];
#pragma unroll
            for (int r = 0; r < RPW; r++)
                sg[r] = su[r] = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                const int o = c * 512 + lane * 8;
                const uint4 xv = o < a.d ? *(const uint4 *)&a.x[t * a.d + o] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < RPW; r++) {
                    sg[r] = dot8(g[r][c], xv, sg[r]);
                    su[r] = dot8(u[r][c], xv, su[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < RPW; r++) {
                const float gs = wave_sum(sg[r]), us = wave_sum(su[r]);
                if (lane == r)
                    a.h[(int64_t)flat * a.f + r0 + r] = f32_to_bf16_rne(silu_mul(gs, us));
            }
        }
    }
}

// grid: (f / (kDecWaves * RPW), expert blocks): the picks of block b are its BM
// entries of sorted_ids.
template <bool PAGED, int NCH, int RPW>
__global__ __launch_bounds__(64 * kDecWaves) void k_dec_gate_up(const FwdArgs a)
{
    const int b = (int)blockIdx.y;
    const int npad = *a.num_padded;
    if ((int64_t)b * a.BM >= npad)
        return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E_tot)
        return;
    const int64_t nflat = a.T * a.keff;
    const int32_t *sid = a.sorted_ids + (int64_t)b * a.BM;
    dec_gate_up_rows<NCH, RPW>(a, matrix_base<PAGED>(a, e, 0), matrix_base<PAGED>(a, e, 1), a.BM, [&](int i) {
        const int flat = sid[i];
        return (flat >= 0 && flat < nflat) ? flat : -1;
    });
}

// Routing and the gate/up rows in one launch.  Every workgroup routes the
// batch's T <= kDecMaxT tokens itself (route_token.h, the routing kernels'
// code), marks the chosen experts in an LDS bitmap, and takes as its expert
// the blockIdx.y-th chosen one in ascending id order -- the expert of aligned
// block blockIdx.y, since with at most T <= block_m picks per expert every
// expert fills one block.  Only the ids stand before the first weight load;
// workgroup (0, 0) computes the routing weights at its end and writes the
// routing outputs (topk ids and weights and the aligned order, the block map
// and num_padded, as the routing kernels would), and with them the W2 base of
// every pick, so that the down pass starts its W2 rows after one load.
// NL > 0: the expert table (E + S <= 64 NL entries, one per lane) is loaded
// beside the logits, so the chosen expert's page bases follow the routing
// without a table read in between.
template <bool PAGED, int NCH, int NV, int RPW, int NL>
__global__ __launch_bounds__(64 * kDecWaves) void k_dec_route_gate_up(const FwdArgs a, const DecRouteArgs ra)
{
    constexpr int kWords = kMaxExpertsTotal / 32;
    __shared__ int32_t s_ids[kDecMaxT * kDecMaxKeff];
    __shared__ uint32_t s_bits[kWords];
    __shared__ int s_pre[kWords + 1]; // exclusive prefix popcounts of s_bits, s_pre[nwords] = experts chosen
    __shared__ int s_e;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NT = 64 * kDecWaves;
    const int T = (int)a.T, keff = a.keff, n = T * keff;
    const int nwords = (a.E_tot + 31) / 32;
    for (int i = tid; i < nwords; i += NT)
        s_bits[i] = 0;
    if (tid == 0)
        s_e = -1;
    int4 tl[NL > 0 ? NL : 1];
    if constexpr (PAGED && NL > 0) {
#pragma unroll
        for (int q = 0; q < NL; q++) {
            const int i = lane + 64 * q;
            tl[q] = i < a.E_tot ? *(const int4 *)(a.locs + i) : make_int4(0, 0, 0, 0);
        }
    }
    // wave w routes tokens w and w + kDecWaves (T <= 2 * kDecWaves): both
    // tokens' logits are loaded before either is routed
    constexpr int TPW = kDecMaxT / kDecWaves;
    float v[TPW][NV];
#pragma unroll
    for (int q = 0; q < TPW; q++) {
        const int t = wave + q * kDecWaves;
        if (t < T)
            rt::load_logits<NV>(ra.logits + (int64_t)t * ra.E, ra.E, lane, v[q]);
        else
#pragma unroll
            for (int i = 0; i < NV; i++)
                v[q][i] = 0.f;
    }
    __syncthreads(); // the bitmap is cleared
    float pv[TPW]; // the logit of pick `lane` of each routed token (for the weights)
    bool live[TPW];
#pragma unroll
    for (int q = 0; q < TPW; q++)
        live[q] = wave + q * kDecWaves < T;
    // all of the wave's tokens at once when all are live (their cross-lane
    // steps overlap), else the live ones one after the other
    if (live[TPW - 1]) {
        rt::route_ids_n<NV, TPW>(v, live, ra.E, ra.k, ra.S, lane, s_ids + wave * keff, kDecWaves * keff, nullptr, pv);
    } else {
#pragma unroll
        for (int q = 0; q < TPW - 1; q++)
            if (live[q])
                pv[q] = rt::route_ids<NV>(v[q], ra.E, ra.k, ra.S, lane, s_ids + (wave + q * kDecWaves) * keff, nullptr);
    }
#pragma unroll
    for (int q = 0; q < TPW; q++) {
        const int t = wave + q * kDecWaves;
        // lane j < k+S wrote pick j: mark its expert
        if (t < T && lane < keff) {
            const int id = s_ids[t * keff + lane];
            atomicOr(&s_bits[id >> 5], 1u << (id & 31));
        }
    }
    __syncthreads();
    if (wave == 0) {
        const uint32_t word = lane < nwords ? s_bits[lane] : 0u;
        const int c = __popc(word);
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off)
                incl += y;
        }
        if (lane < nwords)
            s_pre[lane] = incl - c;
        if (lane == nwords - 1)
            s_pre[nwords] = incl;
        const int u = (int)blockIdx.y;
        if (lane < nwords && u >= incl - c && u < incl) {
            uint32_t wd = word;
            for (int q = u - (incl - c); q > 0; q--)
                wd &= wd - 1; // drop the lower set bits
            s_e = lane * 32 + __builtin_ctz(wd);
        }
    }
    __syncthreads();
    const int e = __builtin_amdgcn_readfirstlane(s_e); // uniform: the table entry and bases load as scalars
    if (e >= 0) {
        const uint16_t *w1, *w3;
        if constexpr (PAGED && NL > 0) {
            const int q = e >> 6, l = e & 63;
            int4 L = tl[0];
#pragma unroll
            for (int j = 1; j < NL; j++)
                if (q == j)
                    L = tl[j];
            L = make_int4(__builtin_amdgcn_readlane(L.x, l), __builtin_amdgcn_readlane(L.y, l),
                          __builtin_amdgcn_readlane(L.z, l), __builtin_amdgcn_readlane(L.w, l));
            w1 = matrix_base_of(a, L, 0);
            w3 = matrix_base_of(a, L, 1);
        } else {
            w1 = matrix_base<PAGED>(a, e, 0);
            w3 = matrix_base<PAGED>(a, e, 1);
        }
        dec_gate_up_rows<NCH, RPW>(a, w1, w3, n, [&](int i) { return s_ids[i] == e ? i : -1; });
    }
    if (blockIdx.x != 0 || blockIdx.y != 0)
        return;
    // the routing outputs, as the routing kernels write them, and the W2 base
    // of every pick (the down pass reads its W2 rows from there)
    const int U = s_pre[nwords], BM = a.BM;
    if (live[TPW - 1]) {
        rt::route_weights_n<TPW>(pv, live, ra.k, ra.S, lane, ra.topk_w + (int64_t)wave * keff, kDecWaves * keff);
    } else {
#pragma unroll
        for (int q = 0; q < TPW - 1; q++)
            if (live[q])
                rt::route_weights(pv[q], ra.k, ra.S, lane, ra.topk_w + (int64_t)(wave + q * kDecWaves) * keff);
    }
    const uint16_t **w2b = (const uint16_t **)a.comb;
    for (int i = tid; i < n; i += NT) {
        ra.topk_ids[i] = s_ids[i];
        w2b[i] = matrix_base<PAGED>(a, s_ids[i], 2);
    }
    for (int i = tid; i < U * BM; i += NT)
        ra.sorted_ids[i] = n;
    for (int q = tid; q < U; q += NT) {
        int wi = 0;
        while (s_pre[wi + 1] <= q)
            wi++;
        uint32_t wd = s_bits[wi];
        for (int r = q - s_pre[wi]; r > 0; r--)
            wd &= wd - 1;
        ra.block_expert[q] = wi * 32 + __builtin_ctz(wd);
    }
    if (tid == 0)
        *ra.num_padded = U * BM;
    __syncthreads(); // the sentinels are stored before the picks overwrite theirs
    for (int i = tid; i < n; i += NT) {
        const int ei = s_ids[i];
        const int seg = BM * (s_pre[ei >> 5] + __popc(s_bits[ei >> 5] & ((1u << (ei & 31)) - 1u)));
        int rank = 0;
        for (int j = 0; j < i; j++)
            rank += s_ids[j] == ei;
        ra.sorted_ids[seg + rank] = i;
    }
}

// grid: (d / CPG, T).  Wave w takes the token's picks w, w + 4,
// ...: it issues the W2 rows of its pick, reads the pick's h row (from L2),
// and leaves w_tj * dot per column in LDS; after the one barrier the sums over
// the picks are taken in slot order.  ROUTED: the routing ran in the gate/up
// launch, which left every pick's W2 base in the combine area of the
// workspace (no combine buffer in this form); else the base is resolved from
// the pick's expert id.
template <bool PAGED, int NCH, int CPG, bool ROUTED>
__global__ __launch_bounds__(64 * kDecWaves) void k_dec_down(const FwdArgs a)
{
    __shared__ float res[kDecMaxKeff * CPG];
    const int t = (int)blockIdx.y;
    const int c0 = (int)blockIdx.x * CPG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int j = wave; j < a.keff; j += kDecWaves) {
        const int64_t i = (int64_t)t * a.keff + j;
        const uint16_t *w2;
        if constexpr (ROUTED) {
            w2 = ((const uint16_t *const *)a.comb)[i];
        } else {
            const int e = a.topk_ids[i];
            w2 = (e >= 0 && e < a.E_tot) ? matrix_base<PAGED>(a, e, 2) : nullptr;
        }
        const float w = a.topk_w[i];
        float s[CPG];
#pragma unroll
        for (int c = 0; c < CPG; c++)
            s[c] = 0.f;
        if (w2) {
            uint4 wv[CPG][NCH];
#pragma unroll
            for (int c = 0; c < CPG; c++)
#pragma unroll
                for (int k = 0; k < NCH; k++) {
                    const int o = k * 512 + lane * 8;
                    wv[c][k] = o < a.f ? load_stream(&w2[(int64_t)(c0 + c) * a.f + o]) : make_uint4(0, 0, 0, 0);
                }
            const uint16_t *hrow = a.h + ((int64_t)t * a.keff + j) * a.f;
#pragma unroll
            for (int k = 0; k < NCH; k++) {
                const int o = k * 512 + lane * 8;
                const uint4 hv = o < a.f ? *(const uint4 *)&hrow[o] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int c = 0; c < CPG; c++)
                    s[c] = dot8(wv[c][k], hv, s[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < CPG; c++) {
            const float v = wave_sum(s[c]);
            if (lane == c)
                res[j * CPG + c] = w * v;
        }
    }
    __syncthreads();
    if (tid < CPG) {
        float acc = 0.f;
        for (int j = 0; j < a.keff; j++)
            acc += res[j * CPG + tid];
        a.y[(int64_t)t * a.d + c0 + tid] = f32_to_bf16_rne(acc);
    }
}

template <int NCH_D, int RPW>
struct RoutedGateUp {
    template <bool PAGED, int NV>
    static void go(const FwdArgs &a, const DecRouteArgs &r, dim3 g, hipStream_t s)
    {
        // the table beside the logits pays at one token only (the launches with
        // RPW = kDecRowsPerWave1; T=1 17.4 -> 17.2 us, 2 and 4 tokens measured
        // 0.1-0.4 us slower), with E + S <= 64 (NV = 1) or <= 128 (NV <= 2)
        constexpr bool kTable = PAGED && RPW == kDecRowsPerWave1 && NV <= 2;
        if constexpr (kTable && NV == 1) {
            if (a.E_tot <= 64) {
                k_dec_route_gate_up<PAGED, NCH_D, NV, RPW, 1><<<g, 64 * kDecWaves, 0, s>>>(a, r);
                return;
            }
        }
        if constexpr (kTable) {
            if (a.E_tot <= 128) {
                k_dec_route_gate_up<PAGED, NCH_D, NV, RPW, 2><<<g, 64 * kDecWaves, 0, s>>>(a, r);
                return;
            }
        }
        k_dec_route_gate_up<PAGED, NCH_D, NV, RPW, 0><<<g, 64 * kDecWaves, 0, s>>>(a, r);
    }
};

template <bool PAGED, int NCH_D, int RPW>
void launch_gate_up(const FwdArgs &a, const DecRouteArgs *ra, dim3 g1, hipStream_t s)
{
    if (!ra) {
        k_dec_gate_up<PAGED, NCH_D, RPW><<<g1, 64 * kDecWaves, 0, s>>>(a);
        return;
    }
    using R = RoutedGateUp<NCH_D, RPW>;
    if (ra->E <= 64)
        R::template go<PAGED, 1>(a, *ra, g1, s);
    else if (ra->E <= 128)
        R::template go<PAGED, 2>(a, *ra, g1, s);
    else if (ra->E <= 256)
        R::template go<PAGED, 4>(a, *ra, g1, s);
    else if (ra->E <= 512)
        R::template go<PAGED, 8>(a, *ra, g1, s);
    else
        R::template go<PAGED, 16>(a, *ra, g1, s);
}

template <bool PAGED, int NCH_D, int NCH_F, int RPW, int CPG>
hipError_t launch_g(const FwdArgs &a, const DecRouteArgs *ra, hipStream_t s)
{
    auto mark = [&](int i) {
        if (a.ev[i])
            (void)hipEventRecord(a.ev[i], s);
    };
    mark(0);
    // rows of workgroups: at most n / BM + min(n, E+S) blocks exist (the
    // capacity bound, which counts every expert's padding, is far larger for a
    // few tokens, and every surplus workgroup still has to start and exit)
    const int64_t n = a.T * a.keff;
    int64_t rows = n / a.BM + (n < a.E_tot ? n : a.E_tot);
    rows = rows < a.blocks_cap ? rows : a.blocks_cap;
    const dim3 g1((unsigned)(a.f / (kDecWaves * RPW)), (unsigned)rows);
    launch_gate_up<PAGED, NCH_D, RPW>(a, ra, g1, s);
    mark(1);
    const dim3 g2((unsigned)(a.d / CPG), (unsigned)a.T);
    if (ra)
        k_dec_down<PAGED, NCH_F, CPG, true><<<g2, 64 * kDecWaves, 0, s>>>(a);
    else
        k_dec_down<PAGED, NCH_F, CPG, false><<<g2, 64 * kDecWaves, 0, s>>>(a);
    mark(2);
    mark(3);
    return hipGetLastError();
}

template <bool PAGED, int NCH_D, int NCH_F>
hipError_t launch_t(const FwdArgs &a, const DecRouteArgs *ra, hipStream_t s)
{
    if (a.T == 1)
        return launch_g<PAGED, NCH_D, NCH_F, kDecRowsPerWave1, kDecColsPerGroup1>(a, ra, s);
    return launch_g<PAGED, NCH_D, NCH_F, kDecRowsPerWave, kDecColsPerGroup>(a, ra, s);
}

template <bool PAGED, int NCH_D>
hipError_t launch_f(const FwdArgs &a, const DecRouteArgs *ra, hipStream_t s)
{
    const int nf = (a.f + 511) / 512;
    if (nf <= 1)
        return launch_t<PAGED, NCH_D, 1>(a, ra, s);
    if (nf <= 2)
        return launch_t<PAGED, NCH_D, 2>(a, ra, s);
    if (nf <= 3)
        return launch_t<PAGED, NCH_D, 3>(a, ra, s);
    return launch_t<PAGED, NCH_D, 4>(a, ra, s);
}

template <bool PAGED>
hipError_t launch_d(const FwdArgs &a, const DecRouteArgs *ra, hipStream_t s)
{
    const int nd = (a.d + 511) / 512;
    if (nd <= 1)
        return launch_f<PAGED, 1>(a, ra, s);
    if (nd <= 2)
        return launch_f<PAGED, 2>(a, ra, s);
    if (nd <= 4)
        return launch_f<PAGED, 4>(a, ra, s);
    return launch_f<PAGED, 8>(a, ra, s);
}

} // namespace

// The decode form applies: few tokens and rows short enough for the register
// tiles (d <= 4096, f <= 2048).
bool decode_fits(const FwdArgs &a)
{
    return a.T >= 1 && a.T <= kDecMaxT && a.d <= kDecMaxD && a.f <= 2048 && a.d % kDecColsPerGroup == 0 &&
           a.f % (kDecWaves * kDecRowsPerWave) == 0 && a.keff <= kDecMaxKeff && a.BM <= 256;
}

hipError_t launch_decode(const FwdArgs &a, hipStream_t s)
{
    return a.locs ? launch_d<true>(a, nullptr, s) : launch_d<false>(a, nullptr, s);
}

bool decode_routed_fits(const FwdArgs &a, const DecRouteArgs &r)
{
    // every chosen expert fills one aligned block: at most T <= block_m picks each
    return decode_fits(a) && a.T <= kDecRoutedMaxT && a.T <= a.BM && r.E >= 1 && r.E <= 1024 &&
           a.E_tot <= kMaxExpertsTotal;
}

hipError_t launch_decode_routed(const FwdArgs &a, const DecRouteArgs &r, hipStream_t s)
{
    return a.locs ? launch_d<true>(a, &r, s) : launch_d<false>(a, &r, s);
}

} // namespace pmoe
