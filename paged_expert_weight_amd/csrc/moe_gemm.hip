// Grouped GEMMs of the paged fused-MoE layer (gfx950, bf16 MFMA, wave64).
//
// Every BM-row block of the aligned token order belongs to one expert e.  A
// workgroup owns one (block, output-column tile) pair and resolves the base of
// the expert's weight pages once, at its start (the Rimuru digest's kernel
// section: the page lookup happens once per output tile, reads inside the page
// then use fixed strides).  The bases become buffer resource descriptors, one
// per page, so every weight read is a 32-bit in-page offset from a scalar base
// and a read past the page returns zero instead of touching a neighbour page.
//
//   gate/up:  h[i][j] = bf16( silu(sum_t x[tok(i)][t] W1_e[j][t]) * sum_t x[tok(i)][t] W3_e[j][t] )
//             The fused operand's column n in [0, 2f) lives on the W1 page for
//             n < f and on the W3 page for n >= f, row n mod f
//             (addr_e(n,t) = B_P + p_e(n) f d + (n mod f) d + t); a tile takes
//             the same columns j0..j0+BN of both halves, so gate and up of one
//             output land in the same lane and the SiLU*mul epilogue runs in
//             registers.
//   down:     o[i][r] = sum_c h[i][c] W2_e[r][c], W2 page [d][f]; scaled by the
//             routing weight of flat pick i and written to the combine buffer
//             row i (fixed order) or added into y32[token] (fp32 atomics).
//   combine:  y[t] = bf16( sum_j comb[t*(k+S)+j] ), j ascending.
//
// Operands are K-contiguous on both sides (x rows and weight rows run along d;
// h rows and W2 rows run along f), so each stage moves 128-byte row segments
// from HBM to LDS with 16-byte loads and feeds v_mfma_f32_16x16x32_bf16 from
// LDS with one 16-byte read per lane.  Two LDS stages: the global loads of
// stage k+1 are in flight while stage k is multiplied.
#include "internal.h"

namespace pmoe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;         // K elements per stage
constexpr int BKP = BK + 8;    // LDS row pitch in elements (144 bytes)
constexpr uint32_t kOOB = 0x80000000u; // byte offset past every buffer (all are < 2 GiB): loads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float v)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Page bases of expert e: the per-tile resolver shared by the GEMMs and moe_resolve_addrs.
template <bool PAGED>
__device__ __forceinline__ void gate_up_bases(const FwdArgs &a, int e, const uint16_t *&w1,
                                              const uint16_t *&w3)
{
    const int64_t fd = (int64_t)a.f * a.d;
    if constexpr (PAGED) {
        const DevLoc L = a.locs[e];
        if (L.kind == 0) {
            w1 = a.pool + L.idx[0] * fd;
            w3 = a.pool + L.idx[1] * fd;
        } else {
            w1 = a.loadbuf + (int64_t)L.idx[0] * 3 * fd;
            w3 = w1 + fd;
        }
    } else {
        w1 = a.w13 + (int64_t)e * 2 * fd;
        w3 = w1 + fd;
    }
}

template <bool PAGED>
__device__ __forceinline__ const uint16_t *down_base(const FwdArgs &a, int e)
{
    const int64_t fd = (int64_t)a.f * a.d;
    if constexpr (PAGED) {
        const DevLoc L = a.locs[e];
        return L.kind == 0 ? a.pool + L.idx[2] * fd : a.loadbuf + ((int64_t)L.idx[0] * 3 + 2) * fd;
    } else {
        return a.w2 + (int64_t)e * fd;
    }
}

// Validity of block b; returns its expert or -1.
__device__ __forceinline__ int block_owner(const FwdArgs &a, int BM, int b)
{
    const int npad = *a.num_padded;
    if ((int64_t)(b + 1) * BM > a.sorted_cap || b * BM >= npad)
        return -1;
    const int e = a.block_expert[b];
    return (e >= 0 && e < a.E_tot) ? e : -1;
}

// ---------------------------------------------------------------------------- gate/up + SiLU*mul
template <int BM, int BN, int WAVES_M, bool PAGED>
__global__ __launch_bounds__(256) void k_gemm1(const FwdArgs a)
{
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int FM = WM / 16, FN = WN / 16;
    static_assert(FM >= 1 && FN >= 1 && WM % 16 == 0 && WN % 16 == 0, "tile");
    constexpr int A_ROWS = BM, B_ROWS = 2 * BN;
    constexpr int A_LD = (A_ROWS * 8 + 255) / 256;
    constexpr int B_LD = B_ROWS * 8 / 256;
    constexpr int B_GATE_LD = BN * 8 / 256; // loads q < this fetch W1 rows
    static_assert(B_ROWS * 8 % 256 == 0 && BN * 8 % 256 == 0, "B tile");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][A_ROWS * BKP];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][B_ROWS * BKP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int b = blockIdx.y;
    const int e = block_owner(a, BM, b);
    if (e < 0)
        return;
    const uint16_t *w1, *w3;
    gate_up_bases<PAGED>(a, e, w1, w3);
    const int d = a.d, f = a.f, keff = a.keff;
    const int j0 = blockIdx.x * BN;
    const uint32_t page_bytes = (uint32_t)((int64_t)f * d * 2);
    const auto rx = make_rsrc(a.x, (uint32_t)(a.T * d * 2));
    const auto r1 = make_rsrc(w1, page_bytes);
    const auto r3 = make_rsrc(w3, page_bytes);
    const int64_t nflat = a.T * keff;

    uint32_t aoff[A_LD], boff[B_LD];
#pragma unroll
    for (int q = 0; q < A_LD; q++) {
        const int L = tid + 256 * q, row = L >> 3, ch = L & 7;
        aoff[q] = kOOB;
        if (L < A_ROWS * 8) {
            const int flat = a.sorted_ids[b * BM + row];
            if (flat >= 0 && flat < nflat)
                aoff[q] = (uint32_t)(flat / keff) * (uint32_t)d * 2u + ch * 16u;
        }
    }
#pragma unroll
    for (int q = 0; q < B_LD; q++) {
        const int L = tid + 256 * q, row = L >> 3, ch = L & 7;
        boff[q] = (uint32_t)(j0 + row % BN) * (uint32_t)d * 2u + ch * 16u;
    }

    i32x4 ra[A_LD], rb[B_LD];
    auto gload = [&](int kt) {
        const int soff = kt * BK * 2;
#pragma unroll
        for (int q = 0; q < A_LD; q++)
            ra[q] = bload(rx, aoff[q], soff);
#pragma unroll
        for (int q = 0; q < B_LD; q++)
            rb[q] = bload(q < B_GATE_LD ? r1 : r3, boff[q], soff);
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < A_LD; q++) {
            const int L = tid + 256 * q;
            if (L < A_ROWS * 8)
                *(i32x4 *)&As[buf][(L >> 3) * BKP + (L & 7) * 8] = ra[q];
        }
#pragma unroll
        for (int q = 0; q < B_LD; q++) {
            const int L = tid + 256 * q;
            *(i32x4 *)&Bs[buf][(L >> 3) * BKP + (L & 7) * 8] = rb[q];
        }
    };

    f32x4 accg[FM][FN], accu[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
            accg[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int KT = d / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int lrow = lane & 15, lk = 8 * (lane >> 4);
    for (int kt = 0; kt < KT; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            gload(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 af[FM], bg[FN], bu[FN];
#pragma unroll
            for (int i = 0; i < FM; i++)
                af[i] = *(const bf16x8 *)&As[cur][(wm * WM + i * 16 + lrow) * BKP + kk + lk];
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int r = wn * WN + j * 16 + lrow;
                bg[j] = *(const bf16x8 *)&Bs[cur][r * BKP + kk + lk];
                bu[j] = *(const bf16x8 *)&Bs[cur][(BN + r) * BKP + kk + lk];
            }
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    accg[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bg[j], accg[i][j], 0, 0, 0);
                    accu[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bu[j], accu[i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < KT)
            sstore(cur ^ 1);
        __syncthreads();
    }

    uint16_t *hb = a.h + (int64_t)b * BM * f + j0;
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = wm * WM + i * 16 + 4 * (lane >> 4) + r;
                const int col = wn * WN + j * 16 + lrow;
                const float g = accg[i][j][r], u = accu[i][j][r];
                hb[(int64_t)row * f + col] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
            }
}

// ---------------------------------------------------------------------------- down + weighted combine
template <int BM, int BN, int WAVES_M, bool PAGED, bool ATOMIC>
__global__ __launch_bounds__(256) void k_gemm2(const FwdArgs a)
{
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int FM = WM / 16, FN = WN / 16;
    static_assert(FM >= 1 && FN >= 1 && WM % 16 == 0 && WN % 16 == 0, "tile");
    constexpr int A_LD = (BM * 8 + 255) / 256;
    constexpr int B_LD = BN * 8 / 256;
    static_assert(BN * 8 % 256 == 0, "B tile");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BKP];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BKP];
    __shared__ int s_flat[BM];
    __shared__ float s_w[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int b = blockIdx.y;
    const int e = block_owner(a, BM, b);
    if (e < 0)
        return;
    const uint16_t *w2 = down_base<PAGED>(a, e);
    const int d = a.d, f = a.f;
    const int r0 = blockIdx.x * BN;
    const int64_t nflat = a.T * a.keff;
    const auto rh = make_rsrc(a.h, (uint32_t)(a.sorted_cap * f * 2));
    const auto rw = make_rsrc(w2, (uint32_t)((int64_t)f * d * 2));

    if (tid < BM) {
        const int flat = a.sorted_ids[b * BM + tid];
        const bool ok = flat >= 0 && flat < nflat;
        s_flat[tid] = ok ? flat : -1;
        s_w[tid] = ok ? a.topk_w[flat] : 0.f;
    }

    uint32_t aoff[A_LD], boff[B_LD];
#pragma unroll
    for (int q = 0; q < A_LD; q++) {
        const int L = tid + 256 * q, row = L >> 3, ch = L & 7;
        aoff[q] = L < BM * 8 ? (uint32_t)(b * BM + row) * (uint32_t)f * 2u + ch * 16u : kOOB;
    }
#pragma unroll
    for (int q = 0; q < B_LD; q++) {
        const int L = tid + 256 * q, row = L >> 3, ch = L & 7;
        boff[q] = (uint32_t)(r0 + row) * (uint32_t)f * 2u + ch * 16u;
    }

    i32x4 ra[A_LD], rb[B_LD];
    auto gload = [&](int kt) {
        const int soff = kt * BK * 2;
#pragma unroll
        for (int q = 0; q < A_LD; q++)
            ra[q] = bload(rh, aoff[q], soff);
#pragma unroll
        for (int q = 0; q < B_LD; q++)
            rb[q] = bload(rw, boff[q], soff);
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < A_LD; q++) {
            const int L = tid + 256 * q;
            if (L < BM * 8)
                *(i32x4 *)&As[buf][(L >> 3) * BKP + (L & 7) * 8] = ra[q];
        }
#pragma unroll
        for (int q = 0; q < B_LD; q++) {
            const int L = tid + 256 * q;
            *(i32x4 *)&Bs[buf][(L >> 3) * BKP + (L & 7) * 8] = rb[q];
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = f / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int lrow = lane & 15, lk = 8 * (lane >> 4);
    for (int kt = 0; kt < KT; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            gload(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; i++)
                af[i] = *(const bf16x8 *)&As[cur][(wm * WM + i * 16 + lrow) * BKP + kk + lk];
#pragma unroll
            for (int j = 0; j < FN; j++)
                bf[j] = *(const bf16x8 *)&Bs[cur][(wn * WN + j * 16 + lrow) * BKP + kk + lk];
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT)
            sstore(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int row = wm * WM + i * 16 + 4 * (lane >> 4) + r;
            const int flat = s_flat[row];
            if (flat < 0)
                continue;
            const float wt = s_w[row];
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int col = r0 + wn * WN + j * 16 + lrow;
                const float v = acc[i][j][r] * wt;
                if constexpr (ATOMIC)
                    unsafeAtomicAdd(&a.comb[(int64_t)(flat / a.keff) * d + col], v);
                else
                    a.comb[(int64_t)flat * d + col] = v;
            }
        }
}

// ---------------------------------------------------------------------------- combine / convert
// y[t][c] = bf16( sum_{j < rows} comb[t*rows + j][c] ), four columns per thread.
__global__ __launch_bounds__(256) void k_combine(const float *comb, int64_t T, int d, int rows, uint16_t *y)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int q = d / 4;
    if (idx >= T * q)
        return;
    const int64_t t = idx / q;
    const int c = (int)(idx % q) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < rows; j++) {
        const float4 v = *(const float4 *)&comb[(t * rows + j) * d + c];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
    o.y = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
    *(uint2 *)&y[t * d + c] = o;
}

__global__ __launch_bounds__(256) void k_zero(float4 *p, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------- address resolver
__global__ __launch_bounds__(256) void k_resolve(const ResolveArgs r, const FwdArgs a)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= r.n)
        return;
    const int e = r.e[q], which = r.which[q];
    const int64_t row = r.row[q], col = r.col[q];
    const int64_t f = r.f, d = r.d;
    const bool ok = e >= 0 && e < r.E_tot &&
                    ((which == 0 && row >= 0 && row < 2 * f && col >= 0 && col < d) ||
                     (which == 1 && row >= 0 && row < d && col >= 0 && col < f));
    if (!ok) {
        r.off[q] = -1;
        r.base[q] = -1;
        return;
    }
    const bool in_pool = r.locs[e].kind == 0;
    const uint16_t *origin = in_pool ? r.pool : a.loadbuf;
    int64_t off;
    if (which == 0) {
        const uint16_t *w1, *w3;
        gate_up_bases<true>(a, e, w1, w3);
        off = ((row < f ? w1 : w3) - origin) + (row % f) * d + col;
    } else {
        off = (down_base<true>(a, e) - origin) + row * f + col;
    }
    r.off[q] = off;
    r.base[q] = in_pool ? 0 : 1 + r.active_buf;
}

template <int BM, int BN1, int BN2, int WAVES_M, bool PAGED>
hipError_t launch_tiles(const FwdArgs &a, hipStream_t s)
{
    const int64_t n = a.T * a.keff;
    int64_t grid_m = n / BM + (n < a.E_tot ? n : a.E_tot);
    if (grid_m > a.blocks_cap)
        grid_m = a.blocks_cap;
    auto mark = [&](int i) {
        if (a.ev[i])
            (void)hipEventRecord(a.ev[i], s);
    };
    if (a.atomic) {
        const int64_t n4 = a.T * a.d / 4;
        k_zero<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>((float4 *)a.comb, n4);
    }
    mark(0);
    k_gemm1<BM, BN1, WAVES_M, PAGED><<<dim3(a.f / BN1, (unsigned)grid_m), 256, 0, s>>>(a);
    mark(1);
    if (a.atomic)
        k_gemm2<BM, BN2, WAVES_M, PAGED, true><<<dim3(a.d / BN2, (unsigned)grid_m), 256, 0, s>>>(a);
    else
        k_gemm2<BM, BN2, WAVES_M, PAGED, false><<<dim3(a.d / BN2, (unsigned)grid_m), 256, 0, s>>>(a);
    mark(2);
    const int rows = a.atomic ? 1 : a.keff;
    const int64_t nq = a.T * a.d / 4;
    k_combine<<<(unsigned)((nq + 255) / 256), 256, 0, s>>>(a.comb, a.T, a.d, rows, a.y);
    mark(3);
    return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_paged(const FwdArgs &a, hipStream_t s)
{
    switch (a.BM) {
    case 16: return launch_tiles<16, 64, 64, 1, PAGED>(a, s);
    case 32: return launch_tiles<32, 64, 64, 2, PAGED>(a, s);
    case 64: return launch_tiles<64, 64, 64, 2, PAGED>(a, s);
    case 128: return launch_tiles<128, 64, 64, 2, PAGED>(a, s);
    case 256: return launch_tiles<256, 64, 64, 4, PAGED>(a, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t s)
{
    if (a.T <= 0)
        return hipSuccess;
    return a.locs ? launch_paged<true>(a, s) : launch_paged<false>(a, s);
}

hipError_t launch_resolve(const ResolveArgs &r, hipStream_t s)
{
    if (r.n <= 0)
        return hipSuccess;
    FwdArgs a{};
    a.locs = r.locs;
    a.pool = r.pool;
    a.loadbuf = r.active_buf ? r.loadbuf1 : r.loadbuf0;
    a.d = r.d;
    a.f = r.f;
    a.E_tot = r.E_tot;
    k_resolve<<<(unsigned)((r.n + 255) / 256), 256, 0, s>>>(r, a);
    return hipGetLastError();
}

} // namespace pmoe
