// Top-k softmax routing of one token by one wave (gfx950, wave64): the device
// functions shared by the routing kernels and the fused decode forward.
//
// Lane L holds logits L, L+64, ..., sorted once into pick order (larger logit
// first, equal logits by lower id); each of the k rounds takes a butterfly max
// of the lanes' first entries (DPP and lane-swap steps, no LDS), then the id of
// the lowest lane holding it when that is the lowest id (one entry per lane, or
// one such lane), else a butterfly min of those lanes' ids, so all lanes agree
// on the winner, whose lane then moves on to its next entry.  Lane j keeps pick
// j; the weights are the softmax of the k picks renormalised over them,
// exp(l_j - l_0) / sum_i exp(l_i - l_0), computed in fp64 and stored as fp32.
// A shared expert (id E, weight 1) is appended as pick k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmoe {
namespace rt {

// Cross-lane exchange without the LDS crossbar.  Within a row of 16 lanes:
// DPP quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i <-> 7-i of its 8) and row_mirror (i <-> 15-i).
// Across rows: v_permlane16_swap / v_permlane32_swap, which hand every lane the
// value of lane ^ 16 / lane ^ 32 in one of their two results.  Applied in this
// order, each step pairs every lane with a lane of the other half of the group
// the previous steps made uniform, so a commutative, associative combine ends
// with the same result in all 64 lanes.
template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ int xor16(int v, int lane)
{
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)(((lane >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ int xor32(int v, int lane)
{
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)(lane >= 32 ? r[0] : r[1]);
}
__device__ __forceinline__ float wave_sum(float x, int lane)
{
    const auto f = [](int v) { return __builtin_bit_cast(float, v); };
    const auto i = [](float v) { return __builtin_bit_cast(int, v); };
    x += f(dpp<kDppXor1>(i(x)));
    x += f(dpp<kDppXor2>(i(x)));
    x += f(dpp<kDppHalfMirror>(i(x)));
    x += f(dpp<kDppMirror>(i(x)));
    x += f(xor16(i(x), lane));
    x += f(xor32(i(x), lane));
    return x;
}

// Wave-wide fp64 sum, each exchange on the two 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double dpp(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = dpp<CTRL>((int)(uint32_t)u), hi = dpp<CTRL>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double xor16(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = xor16((int)(uint32_t)u, lane), hi = xor16((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double xor32(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = xor32((int)(uint32_t)u, lane), hi = xor32((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ double wave_sum(double x, int lane)
{
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    x += dpp<kDppMirror>(x);
    x += xor16(x, lane);
    x += xor32(x, lane);
    return x;
}

// Lane L's logits L, L+64, ... of one token row.
template <int NV>
__device__ __forceinline__ void load_logits(const float *row, int E, int lane, float (&v)[NV])
{
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = lane + 64 * i;
        v[i] = e < E ? row[e] : 0.f;
    }
}

// Wave-wide max / min of an int, returned as a wave-uniform value.  Each step
// combines with a DPP-permuted copy whose disabled lanes read the operation's
// identity, so the move folds into the max / min: two in-quad swaps, the
// half-row and row mirrors (every row of 16 then uniform), then lane 15 of a
// row into the next row and lane 31 into rows 2 and 3, which leaves the
// result in lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_or(int ident, int v)
{
    return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROWS, 0xF, false);
}
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

__device__ __forceinline__ int wave_max(int x)
{
    constexpr int I = (int)0x80000000;
    x = max(x, dpp_or<kDppXor1, 0xF>(I, x));
    x = max(x, dpp_or<kDppXor2, 0xF>(I, x));
    x = max(x, dpp_or<kDppHalfMirror, 0xF>(I, x));
    x = max(x, dpp_or<kDppMirror, 0xF>(I, x));
    x = max(x, dpp_or<kDppRowBcast15, 0xA>(I, x));
    x = max(x, dpp_or<kDppRowBcast31, 0xC>(I, x));
    return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ int wave_min(int x)
{
    constexpr int I = 0x7fffffff;
    x = min(x, dpp_or<kDppXor1, 0xF>(I, x));
    x = min(x, dpp_or<kDppXor2, 0xF>(I, x));
    x = min(x, dpp_or<kDppHalfMirror, 0xF>(I, x));
    x = min(x, dpp_or<kDppMirror, 0xF>(I, x));
    x = min(x, dpp_or<kDppRowBcast15, 0xA>(I, x));
    x = min(x, dpp_or<kDppRowBcast31, 0xC>(I, x));
    return __builtin_amdgcn_readlane(x, 63);
}

// A finite fp32 logit as an int whose order is the float order: -0 and +0
// both map to 0 (they compare equal as floats), negatives to -1 - |bits|.
__device__ __forceinline__ int order_key(float v)
{
    int b = __builtin_bit_cast(int, v);
    b = b == (int)0x80000000 ? 0 : b;
    return b < 0 ? b ^ 0x7fffffff : b;
}

__device__ __forceinline__ float key_value(int k)
{
    return __builtin_bit_cast(float, k < 0 ? k ^ 0x7fffffff : k);
}

// Compare-exchange of lane-local entries a, b so that a comes first in the
// pick order (larger logit first, equal logits by lower id).
__device__ __forceinline__ void order_pair(int &ka, int &ia, int &kb, int &ib)
{
    const bool sw = kb > ka || (kb == ka && ib < ia);
    const int tk = ka, ti = ia;
    ka = sw ? kb : ka;
    ia = sw ? ib : ia;
    kb = sw ? tk : kb;
    ib = sw ? ti : ib;
}

// Sort a lane's NV entries into pick order (odd-even transposition network).
template <int NV>
__device__ __forceinline__ void sort_lane(int (&sk)[NV], int (&si)[NV])
{
#pragma unroll
    for (int round = 0; round < NV; round++)
#pragma unroll
        for (int t = round & 1; t + 1 < NV; t += 2)
            order_pair(sk[t], si[t], sk[t + 1], si[t + 1]);
}

// The id of a pick whose key the lanes in `tied` hold as their first entry:
// the lowest of their ids.  With one entry per lane (NV = 1) lane L holds id L,
// and with a single such lane there is nothing to compare, so the id is read
// from the lowest lane of the ballot; otherwise a butterfly min of the ids.
template <int NV>
__device__ __forceinline__ int pick_id(bool tied, int id)
{
    constexpr int kNone = 0x7fffffff;
    const uint64_t b = __ballot(tied);
    if (NV == 1 || (b & (b - 1)) == 0)
        return __builtin_amdgcn_readlane(id, (int)__builtin_ctzll(b));
    return wave_min(tied ? id : kNone);
}

// The k picks of R tokens with one wave from their loaded logits (token r's
// in v[r]).  Writes token r's ids[0 .. k+S) at ids + r * step (and, when
// lds_ids is not null, at lds_ids + r * step) unless live[r] is false, and
// leaves in pv[r], in lane j < k, the logit of its pick j (for
// route_weights).  Each lane sorts its logits (lane, lane+64, ...) once into
// pick order; every pick is then the wave maximum of the lanes' first entries,
// and among the lanes whose first entry equals it the lowest expert id (the
// same order as comparing (logit, id) pairs); the lane that holds it moves on
// to its next entry.  The R tokens' cross-lane steps are independent, so a
// round issues them together and their latencies overlap.
template <int NV, int R>
__device__ void route_ids_n(const float (&v)[R][NV], const bool (&live)[R], int E, int k, int S, int lane,
                            int32_t *ids, int step, int32_t *lds_ids, float (&pv)[R])
{
    constexpr int kNone = 0x7fffffff, kEmpty = (int)0x80000000; // id / key of a lane's used-up entries
    int sk[R][NV], si[R][NV];
#pragma unroll
    for (int r = 0; r < R; r++) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int e = lane + 64 * i;
            sk[r][i] = e < E ? order_key(v[r][i]) : kEmpty;
            si[r][i] = e < E ? e : kNone;
        }
        sort_lane<NV>(sk[r], si[r]);
    }
    int my_k[R], my_id[R];
#pragma unroll
    for (int r = 0; r < R; r++)
        my_k[r] = my_id[r] = 0;
    for (int j = 0; j < k; j++) {
        int m[R], bi[R];
#pragma unroll
        for (int r = 0; r < R; r++)
            m[r] = wave_max(sk[r][0]);
#pragma unroll
        for (int r = 0; r < R; r++)
            bi[r] = pick_id<NV>(sk[r][0] == m[r], si[r][0]);
#pragma unroll
        for (int r = 0; r < R; r++) {
            if (lane == j) {
                my_k[r] = m[r];
                my_id[r] = bi[r];
            }
            // the lane holding the pick drops it: its entries move up by one.
            // A bitwise blend, not a select between neighbours (which the
            // compiler turns into an indexed access and then into compare chains)
            const int msk = -(int)(si[r][0] == bi[r]);
#pragma unroll
            for (int t = 0; t + 1 < NV; t++) {
                sk[r][t] ^= (sk[r][t] ^ sk[r][t + 1]) & msk;
                si[r][t] ^= (si[r][t] ^ si[r][t + 1]) & msk;
            }
            sk[r][NV - 1] ^= (sk[r][NV - 1] ^ kEmpty) & msk;
            si[r][NV - 1] ^= (si[r][NV - 1] ^ kNone) & msk;
        }
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
        pv[r] = key_value(my_k[r]);
        if (!live[r])
            continue;
        int32_t *o = ids + r * step;
        if (lane < k) {
            o[lane] = my_id[r];
            if (lds_ids)
                lds_ids[r * step + lane] = my_id[r];
        }
        if (S && lane == k) {
            o[k] = E;
            if (lds_ids)
                lds_ids[r * step + k] = E;
        }
    }
}

// One token: returns its pick logits.
template <int NV>
__device__ float route_ids(const float (&v)[NV], int E, int k, int S, int lane, int32_t *ids, int32_t *lds_ids)
{
    float vr[1][NV];
#pragma unroll
    for (int i = 0; i < NV; i++)
        vr[0][i] = v[i];
    const bool live[1] = {true};
    float pv[1];
    route_ids_n<NV, 1>(vr, live, E, k, S, lane, ids, 0, lds_ids, pv);
    return pv[0];
}

// The routing weights of R tokens from route_ids_n's per-lane pick logits
// (token r's at w + r * step unless live[r] is false):
// w[j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k picks, and 1 for
// the shared expert (pick k).  Computed in fp64, rounded once to fp32: the
// difference of two fp32 logits is exact in fp64, so exp of it keeps its
// relative accuracy at any logit gap (in fp32 the rounding of l_j - l_0 alone
// is |l_j - l_0| * 2^-24 relative after exp, 3e-6 at a gap of 50).
template <int R>
__device__ __forceinline__ void route_weights_n(const float (&pv)[R], const bool (&live)[R], int k, int S, int lane,
                                                float *w, int step)
{
    double ex[R], sum[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const float lmax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, pv[r])));
        ex[r] = lane < k ? exp((double)pv[r] - (double)lmax) : 0.0;
    }
#pragma unroll
    for (int r = 0; r < R; r++)
        sum[r] = wave_sum(ex[r], lane); // commutative pairs: every lane ends with the same sum
#pragma unroll
    for (int r = 0; r < R; r++) {
        if (!live[r])
            continue;
        if (lane < k)
            w[r * step + lane] = (float)(ex[r] / sum[r]);
        if (S && lane == k)
            w[r * step + k] = 1.f;
    }
}

__device__ __forceinline__ void route_weights(float my_v, int k, int S, int lane, float *w)
{
    const float pv[1] = {my_v};
    const bool live[1] = {true};
    route_weights_n<1>(pv, live, k, S, lane, w, 0);
}

// Route R tokens: ids and weights.
template <int NV, int R>
__device__ void route_token_n(const float (&v)[R][NV], const bool (&live)[R], int E, int k, int S, int lane,
                              int32_t *ids, float *w, int step, int32_t *lds_ids)
{
    float pv[R];
    route_ids_n<NV, R>(v, live, E, k, S, lane, ids, step, lds_ids, pv);
    route_weights_n<R>(pv, live, k, S, lane, w, step);
}

// Route one token: ids and weights.
template <int NV>
__device__ void route_token(const float (&v)[NV], int E, int k, int S, int lane, int32_t *ids, float *w,
                            int32_t *lds_ids)
{
    route_weights(route_ids<NV>(v, E, k, S, lane, ids, lds_ids), k, S, lane, w);
}

} // namespace rt
} // namespace pmoe
