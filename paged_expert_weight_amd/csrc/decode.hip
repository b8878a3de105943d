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

#include <hip/hip_runtime.h>

namespace pmoe {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecRowsPerWave = 2;  // gate/up: intermediate rows per wave
constexpr int kDecColsPerGroup = 4; // down: output columns per workgroup
constexpr int kDecMaxT = 8;         // tokens (hence valid rows of one expert block)
constexpr int kDecMaxD = 4096;
constexpr int kDecMaxKeff = 64;   // picks per token (top-k plus the shared expert)

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

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

// Base of matrix m (0 W1, 1 W3, 2 W2) of expert e: a pool page, a load-buffer
// slot (W1, W3, W2 back to back), or the contiguous arrays.
template <bool PAGED>
__device__ __forceinline__ const uint16_t *matrix_base(const FwdArgs &a, int e, int m)
{
    const int64_t fd = (int64_t)a.f * a.d;
    if constexpr (PAGED) {
        const DevLoc L = a.locs[e];
        if (L.kind == 0)
            return a.pool + (int64_t)L.idx[m] * fd;
        return a.loadbuf + ((int64_t)L.idx[0] * 3 + m) * fd;
    } else {
        if (m < 2)
            return a.w13 + (int64_t)e * 2 * fd + m * fd;
        return a.w2 + (int64_t)e * fd;
    }
}

// grid: (f / (kDecWaves * kDecRowsPerWave), expert blocks).  Every wave works
// on its own (no LDS, no barrier): it issues its weight rows first, finds the
// block's valid picks with a ballot over sorted_ids while those loads are in
// flight, then reads each pick's x row (shared by all waves, so mostly from
// L2) and writes that pick's h values.
template <bool PAGED, int NCH>
__global__ __launch_bounds__(64 * kDecWaves) void k_dec_gate_up(const FwdArgs a)
{
    const int b = (int)blockIdx.y;
    const int npad = *a.num_padded;
    if ((int64_t)b * a.BM >= npad)
        return;
    const int e = a.block_expert[b];
    if (e < 0 || e >= a.E_tot)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nflat = a.T * a.keff;
    const int32_t *sid = a.sorted_ids + (int64_t)b * a.BM;
    // the block's slots: BM <= 256, so at most four per lane
    int s4[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        s4[i] = (i * 64 + lane < a.BM) ? sid[i * 64 + lane] : -1;
    const int r0 = ((int)blockIdx.x * kDecWaves + wave) * kDecRowsPerWave;
    const uint16_t *w1 = matrix_base<PAGED>(a, e, 0), *w3 = matrix_base<PAGED>(a, e, 1);
    uint4 g[kDecRowsPerWave][NCH], u[kDecRowsPerWave][NCH];
#pragma unroll
    for (int r = 0; r < kDecRowsPerWave; r++)
#pragma unroll
        for (int c = 0; c < NCH; c++) {
            const int o = c * 512 + lane * 8;
            if (o < a.d) {
                g[r][c] = *(const uint4 *)&w1[(int64_t)(r0 + r) * a.d + o];
                u[r][c] = *(const uint4 *)&w3[(int64_t)(r0 + r) * a.d + o];
            } else {
                g[r][c] = make_uint4(0, 0, 0, 0);
                u[r][c] = make_uint4(0, 0, 0, 0);
            }
        }
    for (int i = 0; i < 4; i++) {
        const bool ok = s4[i] >= 0 && s4[i] < nflat;
        uint64_t m = __ballot(ok);
        while (m) {
            const int bit = __builtin_ctzll(m);
            m &= m - 1;
            const int flat = __shfl(s4[i], bit, 64);
            const int64_t t = flat / a.keff;
            float sg[kDecRowsPerWave], su[kDecRowsPerWave];
#pragma unroll
            for (int r = 0; r < kDecRowsPerWave; r++)
                sg[r] = su[r] = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; c++) {
                const int o = c * 512 + lane * 8;
                const uint4 xv = o < a.d ? *(const uint4 *)&a.x[t * a.d + o] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < kDecRowsPerWave; r++) {
                    sg[r] = dot8(g[r][c], xv, sg[r]);
                    su[r] = dot8(u[r][c], xv, su[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < kDecRowsPerWave; r++) {
                const float gs = wave_sum(sg[r]), us = wave_sum(su[r]);
                if (lane == r)
                    a.h[(int64_t)flat * a.f + r0 + r] = f32_to_bf16_rne(gs / (1.f + __expf(-gs)) * us);
            }
        }
    }
}

// grid: (d / kDecColsPerGroup, T).  Wave w takes the token's picks w, w + 4,
// ...: it issues the four W2 rows of its pick, reads the pick's h row (from
// L2), and leaves w_tj * dot per column in LDS; after the one barrier the sums
// over the picks are taken in slot order.
template <bool PAGED, int NCH>
__global__ __launch_bounds__(64 * kDecWaves) void k_dec_down(const FwdArgs a)
{
    __shared__ float res[kDecMaxKeff * kDecColsPerGroup];
    const int t = (int)blockIdx.y;
    const int c0 = (int)blockIdx.x * kDecColsPerGroup;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int j = wave; j < a.keff; j += kDecWaves) {
        const int e = a.topk_ids[(int64_t)t * a.keff + j];
        const float w = a.topk_w[(int64_t)t * a.keff + j];
        float s[kDecColsPerGroup];
#pragma unroll
        for (int c = 0; c < kDecColsPerGroup; c++)
            s[c] = 0.f;
        if (e >= 0 && e < a.E_tot) {
            const uint16_t *w2 = matrix_base<PAGED>(a, e, 2);
            uint4 wv[kDecColsPerGroup][NCH];
#pragma unroll
            for (int c = 0; c < kDecColsPerGroup; c++)
#pragma unroll
                for (int k = 0; k < NCH; k++) {
                    const int o = k * 512 + lane * 8;
                    wv[c][k] = o < a.f ? *(const uint4 *)&w2[(int64_t)(c0 + c) * a.f + o] : make_uint4(0, 0, 0, 0);
                }
            const uint16_t *hrow = a.h + ((int64_t)t * a.keff + j) * a.f;
#pragma unroll
            for (int k = 0; k < NCH; k++) {
                const int o = k * 512 + lane * 8;
                const uint4 hv = o < a.f ? *(const uint4 *)&hrow[o] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int c = 0; c < kDecColsPerGroup; c++)
                    s[c] = dot8(wv[c][k], hv, s[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < kDecColsPerGroup; c++) {
            const float v = wave_sum(s[c]);
            if (lane == c)
                res[j * kDecColsPerGroup + c] = w * v;
        }
    }
    __syncthreads();
    if (tid < kDecColsPerGroup) {
        float acc = 0.f;
        for (int j = 0; j < a.keff; j++)
            acc += res[j * kDecColsPerGroup + tid];
        a.y[(int64_t)t * a.d + c0 + tid] = f32_to_bf16_rne(acc);
    }
}

template <bool PAGED, int NCH_D, int NCH_F>
hipError_t launch_t(const FwdArgs &a, hipStream_t s)
{
    auto mark = [&](int i) {
        if (a.ev[i])
            (void)hipEventRecord(a.ev[i], s);
    };
    mark(0);
    const dim3 g1((unsigned)(a.f / (kDecWaves * kDecRowsPerWave)), (unsigned)a.blocks_cap);
    k_dec_gate_up<PAGED, NCH_D><<<g1, 64 * kDecWaves, 0, s>>>(a);
    mark(1);
    const dim3 g2((unsigned)(a.d / kDecColsPerGroup), (unsigned)a.T);
    k_dec_down<PAGED, NCH_F><<<g2, 64 * kDecWaves, 0, s>>>(a);
    mark(2);
    mark(3);
    return hipGetLastError();
}

template <bool PAGED, int NCH_D>
hipError_t launch_f(const FwdArgs &a, hipStream_t s)
{
    const int nf = (a.f + 511) / 512;
    if (nf <= 1)
        return launch_t<PAGED, NCH_D, 1>(a, s);
    if (nf <= 2)
        return launch_t<PAGED, NCH_D, 2>(a, s);
    if (nf <= 3)
        return launch_t<PAGED, NCH_D, 3>(a, s);
    return launch_t<PAGED, NCH_D, 4>(a, s);
}

template <bool PAGED>
hipError_t launch_d(const FwdArgs &a, hipStream_t s)
{
    const int nd = (a.d + 511) / 512;
    if (nd <= 1)
        return launch_f<PAGED, 1>(a, s);
    if (nd <= 2)
        return launch_f<PAGED, 2>(a, s);
    if (nd <= 4)
        return launch_f<PAGED, 4>(a, s);
    return launch_f<PAGED, 8>(a, s);
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
    return a.locs ? launch_d<true>(a, s) : launch_d<false>(a, s);
}

} // namespace pmoe
