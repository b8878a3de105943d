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
//   down:     o[i][r] = sum_c h[i][c] W2_e[r][c], W2 page [d][f]; row i is
//             rounded to bf16 into the combine buffer at its flat pick (ordered
//             mode), or scaled by the pick's routing weight and added into
//             y32[token] (fp32 atomics).
//   combine:  y[t] = bf16( sum_j w[t][j] * comb[t*(k+S)+j] ), in fp32, j ascending.
//
// Epilogues store each lane's adjacent output columns of a row with one 8- or
// 16-byte store (stage_col); in 128-row tiles a wave whose rows are all
// padding skips its MFMAs (kSkipPaddingWaves).
//
// Operands are K-contiguous on both sides (x rows and weight rows run along d;
// h rows and W2 rows run along f).  Each K-step (64 elements for most tiles)
// moves 128-byte row segments from HBM straight into LDS
// (buffer_load_dwordx4 ... lds, no VGPR round trip): the A rows into one of S
// stages of their ring and the B rows into one of SB >= S stages of theirs, so
// S-1 (SB-1) K-steps of A (B) rows are in flight while one is multiplied;
// v_mfma_f32_16x16x32_bf16 reads its operands from LDS with one 16-byte read
// per lane, XOR-swizzled so 8 rows never share a bank group.
#include "internal.h"

#include <mutex>
#include <type_traits>

namespace pmoe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOOB = 0x80000000u; // byte offset past every buffer (all are < 2 GiB): loads return 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Two fp32 values rounded to the nearest bf16 (ties to even; a NaN stays a
// NaN) by the hardware conversion v_cvt_pk_bf16_f32, packed with lo in bits
// 0-15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// N adjacent values rounded to bf16 and stored with one instruction (N = 1, 2,
// 4 or 8; p aligned to 2N bytes); NT: non-temporally.
template <int N, bool NT>
__device__ __forceinline__ void store_bf16(uint16_t *p, const float (&v)[N])
{
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "store width");
    auto put = [p](auto o) {
        using V = decltype(o);
        if constexpr (NT)
            __builtin_nontemporal_store(o, (V *)p);
        else
            *(V *)p = o;
    };
    if constexpr (N == 1)
        put((uint16_t)pack_bf16x2(v[0], 0.f));
    else if constexpr (N == 2)
        put(pack_bf16x2(v[0], v[1]));
    else if constexpr (N == 4)
        put((u32x2){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    else
        put((u32x4v){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])});
}

// Page bases of expert e: the per-tile resolver shared by the GEMMs and moe_resolve_addrs.
// The whole 16-byte entry in one load (the table is 16-byte aligned), so that
// the page bases follow one memory round trip after the expert is known.
__device__ __forceinline__ int4 load_loc(const DevLoc *locs, int e)
{
    const int4 L = *(const int4 *)(locs + e);
    // every field is needed here: the compiler would otherwise load the
    // second index only after testing the kind, one more round trip
    asm volatile("" ::"v"(L.x), "v"(L.y), "v"(L.z), "v"(L.w));
    return L;
}

template <bool PAGED>
__device__ __forceinline__ void gate_up_bases(const FwdArgs &a, int e, const uint16_t *&w1,
                                              const uint16_t *&w3)
{
    const int64_t fd = (int64_t)a.f * a.d;
    if constexpr (PAGED) {
        const int4 L = load_loc(a.locs, e); // kind, idx[0..2]
        // selects, not branches: every field is used, so none is loaded late
        const bool in_pool = L.x == 0;
        const int64_t o1 = in_pool ? (int64_t)L.y * fd : (int64_t)L.y * 3 * fd;
        const int64_t o3 = in_pool ? (int64_t)L.z * fd : o1 + fd;
        const uint16_t *base = in_pool ? a.pool : a.loadbuf;
        w1 = base + o1;
        w3 = base + o3;
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
        const int4 L = load_loc(a.locs, e);
        const bool in_pool = L.x == 0;
        const int64_t o2 = in_pool ? (int64_t)L.w * fd : ((int64_t)L.y * 3 + 2) * fd;
        return (in_pool ? a.pool : a.loadbuf) + o2;
    } else {
        return a.w2 + (int64_t)e * fd;
    }
}

// ---------------------------------------------------------------------------- tile order
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i mod 8, each XCD with its own L2), and inside an XCD to whichever CU
// frees first.  The grid is sized for the most blocks the routing can produce,
// but only num_padded / BM blocks exist, so the logical tiles u of the
// existing blocks are dealt out first and surplus workgroups exit.  Two ways
// of dealing them, chosen per launch:
// - contiguous eighths: XCD x walks the range u in [x*per_xcd, (x+1)*per_xcd);
// - chunks of C consecutive tiles to the XCDs in turn: the k-th workgroup of
//   XCD x takes tile u = ((k / C) * 8 + x) * C + k mod C (the grid is whole
//   rounds of 8C), so the tiles an XCD runs at one time are still neighbours
//   in u while every XCD works through the whole order.  With contiguous
//   eighths the XCD whose tiles ran slowest was left alone at the end of a
//   Mixtral-shaped launch (256-row tiles, chunks of 32: step 2642 -> 2598 us)
//   and of the gate/up launch of layers with many 128-row blocks (chunks of
//   64: Qwen3-Next-shaped gate/up 605 -> 578 us).  The other launches keep the
//   eighths: chunked, they ran 1-8 % slower (Qwen3-Next-shaped down, 128- and
//   64-row tiles of 1024- and 512-token layers).
// Tiles are grouped GM blocks at a time, column-tile major inside a group: the
// GM blocks of a group reuse each weight tile from L2, and each block's
// activation rows are reused across the group's column tiles.
constexpr int kXcdChunk = 32;     // 256-row tiles
constexpr int kXcdChunkWide = 64; // 128 x 256 gate/up tiles of layers with many blocks

template <int C>
__device__ __forceinline__ int chunk_tile(int i)
{
    const int x = i & 7, k = i >> 3;
    return ((k / C) * 8 + x) * C + k % C;
}

struct TileSpace {
    int blocks, total, per_xcd; // blocks of BM rows, (block, column tile) pairs, pairs per XCD range
};

__device__ __forceinline__ TileSpace tile_space(const FwdArgs &a, int BM, int ntiles)
{
    TileSpace t;
    t.blocks = *a.num_padded / BM;
    const int cap = (int)(a.sorted_cap / BM);
    t.blocks = t.blocks < cap ? t.blocks : cap;
    t.total = t.blocks * ntiles;
    t.per_xcd = (t.total + 7) / 8;
    return t;
}

// Logical tile u -> (block b, column tile nt): groups of GM blocks, column-tile
// major inside a group.
template <int GM>
__device__ __forceinline__ void tile_at(const TileSpace &t, int ntiles, int u, int &b, int &nt)
{
    const int g = u / (GM * ntiles), r = u % (GM * ntiles);
    const int gm = min(GM, t.blocks - g * GM);
    nt = r / gm;
    b = g * GM + r % gm;
}

// Expert-aligned groups: the blocks of one expert's segment are grouped GM at
// a time from the segment's first block, so a group never spans two experts
// (a group that did would stream two experts' weight tiles for the blocks of
// one L2).  Groups still partition the blocks in order, so the group of tile u
// is that of block u / ntiles: its segment is found with two 64-entry reads of
// block_expert around that block (more only for segments longer than 64
// blocks).  Used by the long tiles, where these reads are a negligible part
// of a tile.
__device__ __forceinline__ int expert_segment(const FwdArgs &a, int nblocks, int q, int &lo, int &hi)
{
    const int lane = threadIdx.x & 63;
    // the expert of block q and the 64 blocks on either side, loaded together
    const int il = q - 64 + lane, ih = q + 1 + lane;
    const int e = a.block_expert[q];
    const int vl = a.block_expert[il > 0 ? il : 0];
    const int vh = a.block_expert[ih < nblocks ? ih : nblocks - 1];
    uint64_t other = __ballot(il >= 0 && vl != e);
    lo = 0;
    for (int base = q - 64;; base -= 64) { // other: blocks base .. base+63 that are not e's
        if (other) {
            lo = base + (63 - __builtin_clzll(other)) + 1;
            break;
        }
        if (base <= 0)
            break;
        const int i = base - 64 + lane;
        other = __ballot(i >= 0 && a.block_expert[i] != e);
    }
    other = __ballot(ih < nblocks && vh != e);
    hi = nblocks;
    for (int base = q + 1;; base += 64) {
        if (other) {
            hi = base + __builtin_ctzll(other);
            break;
        }
        if (base + 64 >= nblocks)
            break;
        const int i = base + 64 + lane;
        other = __ballot(i < nblocks && a.block_expert[i] != e);
    }
    return e;
}

// What the tile mapping learnt about a tile's block: its expert (or
// kExpertUnknown) and whether that expert has no other block (-1: unknown).
constexpr int kExpertUnknown = -2;
struct BlockInfo {
    int e, single;
};

template <int GM>
__device__ __forceinline__ BlockInfo tile_at_aligned(const FwdArgs &a, const TileSpace &t, int ntiles, int u,
                                                     int &b, int &nt)
{
    const int q = u / ntiles;
    int lo, hi;
    const int e = expert_segment(a, t.blocks, q, lo, hi);
    const int s = lo + (q - lo) / GM * GM;
    const int m = min(GM, hi - s);
    const int r = u - s * ntiles;
    nt = r / m;
    b = s + r % m;
    return BlockInfo{e, hi - lo == 1 ? 1 : 0};
}

// Tile u -> (block, column tile), and what the mapping learnt of the block.
template <int GM, bool ALIGNED>
__device__ __forceinline__ BlockInfo tile_pick(const FwdArgs &a, const TileSpace &t, int ntiles, int u, int &b,
                                               int &nt)
{
    if constexpr (ALIGNED) {
        return tile_at_aligned<GM>(a, t, ntiles, u, b, nt);
    } else {
        tile_at<GM>(t, ntiles, u, b, nt);
        return BlockInfo{kExpertUnknown, -1};
    }
}

// One tile per workgroup: workgroup i takes tile (i mod 8) * per_xcd + i / 8
// (CHUNK = 0), or chunk_tile<CHUNK>(i).
template <int GM, bool ALIGNED, int CHUNK>
__device__ __forceinline__ bool tile_of(const FwdArgs &a, int BM, int ntiles, int &b, int &nt, BlockInfo &bi,
                                        int &nblocks)
{
    const TileSpace t = tile_space(a, BM, ntiles);
    nblocks = t.blocks;
    int u;
    if constexpr (CHUNK > 0) {
        u = chunk_tile<CHUNK>((int)blockIdx.x);
    } else {
        u = (int)(blockIdx.x % 8) * t.per_xcd + (int)(blockIdx.x / 8);
        if ((int)(blockIdx.x / 8) >= t.per_xcd)
            return false;
    }
    if (u >= t.total)
        return false;
    bi = tile_pick<GM, ALIGNED>(a, t, ntiles, u, b, nt);
    return true;
}

// Last-wave split.  With P resident workgroups, tiles [0, full) run as
// floor(total / P) whole waves; if the remaining tail <= P / 2 tiles, each is
// cut into ks contiguous K ranges (ks = min(4, P / tail)) so that the last
// wave fills the machine.  Every range writes its fp32 accumulators to a
// partial tile; a fix-up kernel adds the ks partials of a tile in range order
// and applies the epilogue.  Long-K, large tiles only (one workgroup per CU).
constexpr int kMaxSplit = 4;
struct TailPlan {
    int full, tail, ks;
};

__device__ __forceinline__ TailPlan tail_plan(const TileSpace &t, int P)
{
    TailPlan p{t.total, 0, 1};
    if (P > 0) {
        const int full = t.total / P * P, tail = t.total - full;
        if (tail > 0 && 2 * tail <= P) {
            p.full = full;
            p.tail = tail;
            p.ks = min(kMaxSplit, P / tail);
        }
    }
    return p;
}

// Expert of block b (b < num_padded / BM), or -1 for a corrupt map entry.
__device__ __forceinline__ int block_owner(const FwdArgs &a, int b)
{
    const int e = a.block_expert[b];
    return (e >= 0 && e < a.E_tot) ? e : -1;
}

// ---------------------------------------------------------------------------- LDS stages
// A stage holds the K-slice [k0, k0+BK) of the A rows (BM) and of the B rows
// (2*BN gate|up, or BN) as rows of BK bf16 (BK*2 bytes), filled by
// buffer_load_dwordx4 ... lds: one instruction moves 64 x 16 bytes into 1 KB of
// LDS, lane L at byte 16*L.  A lane therefore picks which global 16-byte chunk
// lands in its LDS slot; chunk c of row r is stored at position
// c ^ swz(r) of that row, so that the 16-byte MFMA operand reads of 8
// consecutive rows at one chunk index hit 8 different 16-byte bank groups
// (rows of 128 or 256 bytes: swz = r mod 8; rows of 64 bytes hold two rows
// per 128-byte bank line: swz = (r / 2) mod 4).
template <int BK>
struct StageGeom {
    static constexpr int ROWB = BK * 2;          // bytes per row
    static constexpr int CH = BK / 8;            // 16-byte chunks per row
    static constexpr int ROWS_PER_LD = 64 / CH;  // rows one DMA instruction covers
    __device__ static __forceinline__ int swz(int r) { return CH >= 8 ? (r & 7) : ((r >> 1) & 3); }
};

// Cache policy of the stage DMA (the instruction's aux bits).  A streaming
// read of HBM into LDS measured 7.2 TB/s with non-temporal loads against
// 5.7 TB/s with plain ones, but a non-temporal line is the first to leave L2:
// weight tiles go non-temporal only when no other tile reads them (the
// expert has one block); x and h rows, which other column tiles re-read,
// never do.
constexpr int kDmaPlain = 0;
constexpr int kDmaStream = 2;

template <int N>
struct Int {
    static constexpr int value = N;
};

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0(Int<N>)
{
    static_assert(N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// ---------------------------------------------------------------------------- grouped GEMM
// G1 (gate/up): A = x rows gathered by token, B = W1 rows n0..n0+BN and W3 rows
//     n0..n0+BN, K = d; epilogue h = bf16(silu(gate) * up).
// G2 (down):    A = h rows of the block, B = W2 rows n0..n0+BN, K = f;
//     epilogue: x routing weight -> combine buffer (ordered) or y32 (atomic).
// The K order of the accumulation (32-wide MFMA steps, lane group g holding k
// 8g..8g+7 of each step) is the same for every tile shape, so the result of an
// output element does not depend on BM, BN or the weight layout.
constexpr int gcd_(int a, int b) { return b ? gcd_(b, a % b) : a; }

// S stages of A rows and SB stages of B rows: each operand has its own ring of
// LDS buffers, so one operand may be loaded further ahead than the other (the
// B rows, weights whose misses go to HBM, or the A rows, x rows gathered by
// token).
template <int BM, int BN, int WAVES_M, int WAVES_N, int WK, int BK, int S, bool G1, int SB = S>
struct Gemm {
    using Geo = StageGeom<BK>;
    // WAVES_M x WAVES_N waves share one tile; with WK > 1 (one wave per tile)
    // WK waves split K into contiguous ranges, each with private LDS stages and
    // no barriers, and their partial sums are added in wave order at the end.
    static constexpr int NT = WAVES_M * WAVES_N;
    static constexpr int NW = NT * WK;
    static_assert(WK == 1 || NT == 1, "split-K tiles have one wave per K range");
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static_assert(FM >= 1 && FN >= 1 && WM % 16 == 0 && WN % 16 == 0, "wave tile");
    static constexpr int B_ROWS = G1 ? 2 * BN : BN;
    static constexpr int ROWS = BM + B_ROWS;
    static_assert(ROWS % (Geo::ROWS_PER_LD * NT) == 0, "DMA instructions must split evenly over the waves");
    static constexpr int IPW = ROWS / Geo::ROWS_PER_LD / NT; // DMA instructions per wave per K-step
    static constexpr int IA = BM / Geo::ROWS_PER_LD / NT;    // of which A rows (the first IA)
    static constexpr int IB = IPW - IA;
    static_assert(IA * Geo::ROWS_PER_LD * NT == BM, "A rows split evenly over the waves");
    static_assert(BM % Geo::ROWS_PER_LD == 0 && BN % Geo::ROWS_PER_LD == 0, "sections");
    // K-steps of lookahead of the two rings, the longer one, and the loop period
    // (both ring positions are compile-time constants inside one period)
    static constexpr int LA = S - 1, LB = SB - 1, LM = LA > LB ? LA : LB, P = S * SB / gcd_(S, SB);
    static constexpr int A_BYTES = BM * Geo::ROWB, B_BYTES = B_ROWS * Geo::ROWB;
    static constexpr int RING_BYTES = S * A_BYTES + SB * B_BYTES; // per K range
    static constexpr int LDS_BYTES = WK * RING_BYTES;
    // Each step issues the nearer operand's rows first, then the farther one's
    // (A first when the lookaheads are equal).  At a step's top the rows of the
    // step awaited last in the stream are the nearer operand's, issued Ln steps
    // before; after them come the farther operand's rows of that step and Ln - 1
    // whole steps, which may stay in flight.
    static constexpr bool B_FIRST = LA > LB;
    static constexpr int N_AFTER = LA == LB ? (LA - 1) * IPW
                                   : B_FIRST ? IA + (LB - 1) * IPW
                                             : IB + (LA - 1) * IPW;
    static_assert(S >= 2 && SB >= 2 && S <= 8 && SB <= 8 && N_AFTER < 64, "stages");
    static constexpr int BM_ = BM, BN_ = BN, WK_ = WK, WAVES_N_ = WAVES_N;
    // Waves whose rows are all padding skip their MFMAs in 128-row tiles, the height
    // of layers with many small experts, whose blocks are mostly padding (414 of the
    // 513 experts of a Qwen3-Next-shaped layer have one block of ~60 picks): a
    // 8192-token step 1008 -> 984 us.  Elsewhere it measured no gain (256-row
    // tiles: their weight rows stream at the same rate whatever the MFMA load;
    // 64-row tiles: +1 us at 512 tokens), and those kernels compile without it.
    static constexpr bool kSkipPaddingWaves = BM == 128;

    __amdgpu_buffer_rsrc_t ra, rb0, rb1;
    uint32_t voff[IPW];
    int wave, wt, kg, wm, wn, l16, lg;
    uint8_t *lds; // WK rings (S A stages, then SB B stages), one workgroup-scope array
    bool live;    // false: every output row of this wave is padding, so it multiplies nothing
    f32x4 acc0[FM][FN], acc1[FM][FN];

    // Stages at constant offsets: the waits on the DMA into one stage then
    // never cover the LDS reads of another.
    template <int J>
    __device__ __forceinline__ uint8_t *a_stage() const
    {
        static_assert(J < S, "stage");
        return lds + kg * RING_BYTES + J * A_BYTES;
    }
    template <int J>
    __device__ __forceinline__ uint8_t *b_stage() const
    {
        static_assert(J < SB, "stage");
        return lds + kg * RING_BYTES + S * A_BYTES + J * B_BYTES;
    }

    // DMA of the A rows of K-step kt into A stage J (this wave's instructions i < IA)
    template <int J>
    __device__ __forceinline__ void issue_a(int kt)
    {
        uint8_t *slot = a_stage<J>();
        const int soff = kt * BK * 2;
#pragma unroll
        for (int i = 0; i < IA; i++) {
            const int q = wt + NT * i;
            auto *dst = (__attribute__((address_space(3))) void *)(slot + q * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, voff[i], soff, 0, kDmaPlain);
        }
    }

    // DMA of the B rows of K-step kt into B stage J (instructions i >= IA): the
    // W1 / W2 rows, then the W3 rows; STREAM: non-temporally.
    template <int J, bool STREAM>
    __device__ __forceinline__ void issue_b(int kt)
    {
        uint8_t *slot = b_stage<J>();
        const int soff = kt * BK * 2;
#pragma unroll
        for (int i = IA; i < IPW; i++) {
            const int q = wt + NT * i - BM / Geo::ROWS_PER_LD; // instruction within the B rows
            auto *dst = (__attribute__((address_space(3))) void *)(slot + q * 1024);
            if (!G1 || q * Geo::ROWS_PER_LD < BN)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb0, dst, 16, voff[i], soff, 0, STREAM ? kDmaStream : kDmaPlain);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb1, dst, 16, voff[i], soff, 0, STREAM ? kDmaStream : kDmaPlain);
        }
    }

    template <int JA, int JB>
    __device__ __forceinline__ void compute()
    {
        if constexpr (kSkipPaddingWaves)
            if (!live) // its accumulators stay zero, as they would over the zero rows staged for padding
                return;
        const uint8_t *sa = a_stage<JA>(), *sb = b_stage<JB>();
#pragma unroll
        for (int sub = 0; sub < BK / 32; sub++) {
            const int chunk = 4 * sub + lg;
            bf16x8 af[FM], b0[FN], b1[FN];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int row = wm * WM + 16 * i + l16;
                af[i] = *(const bf16x8 *)(sa + row * Geo::ROWB + ((chunk ^ Geo::swz(row)) * 16));
            }
#pragma unroll
            for (int j = 0; j < FN; j++) {
                // B row r of the stage (row BM + r of the rows the swizzle counts)
                const int r = wn * WN + 16 * j + l16;
                b0[j] = *(const bf16x8 *)(sb + r * Geo::ROWB + ((chunk ^ Geo::swz(BM + r)) * 16));
                if constexpr (G1) {
                    const int r1 = r + BN;
                    b1[j] = *(const bf16x8 *)(sb + r1 * Geo::ROWB + ((chunk ^ Geo::swz(BM + r1)) * 16));
                }
            }
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    acc0[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b0[j], acc0[i][j], 0, 0, 0);
                    if constexpr (G1)
                        acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b1[j], acc1[i][j], 0, 0, 0);
                }
        }
    }

    // The loads before the first K-step, in the order the steady state issues
    // them (step s issues A(s + LA) and B(s + LB), the nearer one first), for
    // virtual steps s = kb - LM .. kb - 1: the waits count on that order.
    template <int V, bool STREAM>
    __device__ __forceinline__ void prologue(int kb, int ke)
    {
        if constexpr (V < LM) {
            constexpr int a = V - LM + LA, bq = V - LM + LB; // A(kb + a), B(kb + bq)
            auto pa = [&]() {
                if constexpr (a >= 0)
                    if (kb + a < ke)
                        this->template issue_a<a % S>(kb + a);
            };
            auto pb = [&]() {
                if constexpr (bq >= 0)
                    if (kb + bq < ke)
                        this->template issue_b<bq % SB, STREAM>(kb + bq);
            };
            if constexpr (B_FIRST) {
                pb();
                pa();
            } else {
                pa();
                pb();
            }
            this->template prologue<V + 1, STREAM>(kb, ke);
        }
    }

    // one loop period: K-steps kt0 .. kt0+P-1 (of the range ending at ke)
    template <int J, bool STREAM>
    __device__ __forceinline__ void steps(int kt0, int ke)
    {
        if constexpr (J < P) {
            const int kt = kt0 + J;
            // K-step kt has landed for this wave and this wave's reads of the
            // stages about to be refilled are done; then the same for every
            // wave that shares the stages.  Only steps inside [kb, ke) are
            // loaded, so near the end fewer later loads are in flight and the
            // wait drains them all.
            if (kt + LM - 1 < ke)
                wait_vm_lgkm0(Int<N_AFTER>{});
            else
                wait_vm_lgkm0(Int<0>{});
            if constexpr (NT > 1)
                __builtin_amdgcn_s_barrier();
            if constexpr (B_FIRST)
                if (kt + LB < ke)
                    this->template issue_b<(J + LB) % SB, STREAM>(kt + LB);
            if (kt + LA < ke)
                this->template issue_a<(J + LA) % S>(kt + LA);
            if constexpr (!B_FIRST)
                if (kt + LB < ke)
                    this->template issue_b<(J + LB) % SB, STREAM>(kt + LB);
            if (kt < ke)
                this->template compute<J % S, J % SB>();
            this->template steps<J + 1, STREAM>(kt0, ke);
        }
    }

    // K-steps [kb, ke): begin() issues the loads ahead of the first step, then
    // the caller may issue loads of its own, then run() does the rest.
    template <bool STREAM>
    __device__ __forceinline__ void begin(int kb, int ke)
    {
        this->template prologue<0, STREAM>(kb, ke);
    }

    template <bool STREAM>
    __device__ __forceinline__ void run(int kb, int ke)
    {
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++) {
                acc0[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc1[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        for (int kt0 = kb; kt0 < ke; kt0 += P)
            this->template steps<0, STREAM>(kt0, ke);
        wait_vm_lgkm0(Int<0>{}); // no DMA may still be writing this workgroup's LDS when it exits
    }

    // Split-K: add the partial sums of waves 1..WK-1 into wave 0's, in wave order.
    // Returns false for the waves that are done.
    __device__ __forceinline__ bool reduce_k()
    {
        if constexpr (WK == 1) {
            return true;
        } else {
            constexpr int PER = FM * FN * 8; // floats per lane
            __syncthreads();
            float *red = (float *)lds;
            const int lane = threadIdx.x & 63;
            if (kg > 0) {
                float *dst = red + ((kg - 1) * PER) * 64;
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            dst[((i * FN + j) * 8 + r) * 64 + lane] = acc0[i][j][r];
                            dst[((i * FN + j) * 8 + 4 + r) * 64 + lane] = acc1[i][j][r];
                        }
            }
            __syncthreads();
            if (kg > 0)
                return false;
            for (int w = 1; w < WK; w++) {
                const float *src = red + ((w - 1) * PER) * 64;
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            acc0[i][j][r] += src[((i * FN + j) * 8 + r) * 64 + lane];
                            acc1[i][j][r] += src[((i * FN + j) * 8 + 4 + r) * 64 + lane];
                        }
            }
            return true;
        }
    }
};

// The output column (within the tile) whose weight row B stage row r holds.
// compute() gives wave (wm, wn) the stage rows wn*WN + 16*j + l16 as fragment j
// of lane l16; they hold columns wn*WN + FN*l16 + j, so a lane's FN
// accumulators of one output row are FN adjacent columns and the epilogue
// stores them with one 2*FN-byte store (the K order of every output is
// unchanged: only which weight row a stage row is loaded from).
template <class G>
__device__ __forceinline__ int stage_col(int r)
{
    const int w = r / G::WN, q = r % G::WN;
    return w * G::WN + (q % 16) * G::FN + q / 16;
}

// One output tile (block b, column tile nt) of a grouped GEMM.  Its rows are
// rows b*RU .. b*RU + BM - 1 of the aligned order: RU = BM, or RU = 128 for a
// 256-row tile over a pair of 128-row blocks (k_gemm's paired blocks).
template <class G, bool G1, bool PAGED, bool ATOMIC, bool E_KNOWN, int RU = G::BM_>
__device__ __forceinline__ void gemm_tile(const FwdArgs &a, G &g, int b, int nt, BlockInfo bi, int nblocks,
                                          int ks = 0, int nks = 1, float *part = nullptr)
{
    constexpr int BM = G::BM_, BN = G::BN_, WK = G::WK_;
    constexpr int BK = G::Geo::ROWB / 2;
    using Geo = typename G::Geo;
    // DMA instructions i < IA of a wave stage A rows, the others B rows
    constexpr int IA = G::IA;
    const int lane = threadIdx.x & 63;
    const int lrow = lane / Geo::CH, lpos = lane % Geo::CH;
    // The tile's first loads are issued together so that their latencies
    // overlap: the flat picks of this wave's A rows, the block's expert unless
    // the tile mapping read it, then the page table entry.  A padding row (no
    // pick) is staged from an out-of-range offset: zeros, no memory traffic.
    int flat_a[IA];
#pragma unroll
    for (int i = 0; i < IA; i++)
        flat_a[i] = a.sorted_ids[b * RU + (g.wt + G::NT * i) * Geo::ROWS_PER_LD + lrow];
    int e, single;
    if constexpr (E_KNOWN) {
        e = bi.e >= 0 && bi.e < a.E_tot ? bi.e : -1;
        single = bi.single;
    } else { // the block's expert and its neighbours' (read together)
        e = block_owner(a, b);
        const int ep = b > 0 ? a.block_expert[b - 1] : -1;
        const int en = b + 1 < nblocks ? a.block_expert[b + 1] : -1;
        single = ep != e && en != e;
    }
    if (e < 0)
        return;
    const int d = a.d, f = a.f, K = G1 ? d : f;
    const int n0 = nt * BN;
    const int64_t nflat = a.T * a.keff;
    const uint32_t page_bytes = (uint32_t)((int64_t)f * d * 2);

    if constexpr (G1) {
        const uint16_t *w1, *w3;
        gate_up_bases<PAGED>(a, e, w1, w3);
        g.ra = make_rsrc(a.x, (uint32_t)(a.T * d * 2));
        g.rb0 = make_rsrc(w1, page_bytes);
        g.rb1 = make_rsrc(w3, page_bytes);
    } else {
        g.ra = make_rsrc(a.h, (uint32_t)(a.sorted_cap * f * 2));
        g.rb0 = g.rb1 = make_rsrc(down_base<PAGED>(a, e), page_bytes);
    }

    // per-lane source offset of each DMA instruction this wave issues
#pragma unroll
    for (int i = 0; i < G::IPW; i++) {
        const int q = g.wt + G::NT * i;                // instruction index within the stage
        const int row = q * Geo::ROWS_PER_LD + lrow;  // row within the stage
        const int chunk = lpos ^ Geo::swz(row);
        uint32_t off;
        if (i < IA) {
            const int flat = flat_a[i];
            const bool pick = flat >= 0 && flat < nflat;
            if constexpr (G1) // the token's x row
                off = pick ? (uint32_t)(flat / a.keff) * (uint32_t)d * 2u : kOOB;
            else // the block's h row
                off = pick ? (uint32_t)(b * RU + row) * (uint32_t)f * 2u : kOOB;
        } else {
            const int br = (row - BM) % BN; // B stage row (W1 / W2 rows, then W3 rows)
            off = (uint32_t)(n0 + stage_col<G>(br)) * (uint32_t)K * 2u;
        }
        g.voff[i] = off + chunk * 16u;
    }

    // The flat pick of every output row this lane stores (and, for the atomic
    // combine, its routing weight).  Small wave tiles fetch the picks
    // before the first stages are issued, so their latency overlaps the K
    // loop; large ones (whose accumulators fill the register file, and whose
    // K loop is long) fetch them after it.
    int eflat[G::FM][4];
    float ewt[G::FM][4];
    auto epilogue_picks = [&]() {
#pragma unroll
        for (int i = 0; i < G::FM; i++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = g.wm * G::WM + i * 16 + 4 * g.lg + r;
                const int flat = a.sorted_ids[b * RU + row];
                eflat[i][r] = (flat >= 0 && flat < nflat) ? flat : -1;
            }
    };
    auto epilogue_weights = [&]() {
#pragma unroll
        for (int i = 0; i < G::FM; i++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                ewt[i][r] = eflat[i][r] >= 0 ? a.topk_w[eflat[i][r]] : 0.f;
    };
    constexpr bool kPrefetchRows = G::FM <= 4;
    // the picks are read before the first stages are issued (nothing waits
    // for them until the epilogue); the ordered combine applies the routing
    // weights itself, the atomic one reads them after the K loop
    g.live = true;
    if constexpr (kPrefetchRows)
        epilogue_picks();
    if constexpr (kPrefetchRows && G::kSkipPaddingWaves) {
        // a wave whose rows (all WM of them, over its lanes) are padding skips its
        // MFMAs and operand reads; it still issues its share of the stage DMA
        bool any = false;
#pragma unroll
        for (int i = 0; i < G::FM; i++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                any |= eflat[i][r] >= 0;
        g.live = __ballot(any) != 0;
    }

    // K-steps [kb, ke): range ks of nks (the whole contraction unless the tile
    // is split), divided again over the WK waves of a split-K tile
    const int KT = K / BK;
    const int kb = ks * KT / nks, ke = (ks + 1) * KT / nks;
    const int wkb = kb + g.kg * (ke - kb) / WK, wke = kb + (g.kg + 1) * (ke - kb) / WK;
    // the weight rows go non-temporal when the expert has no other block
    // (one copy of the K loop per policy, chosen once per tile)
    auto pipeline = [&](auto stream) {
        constexpr bool ST = decltype(stream)::value;
        g.template begin<ST>(wkb, wke);
        g.template run<ST>(wkb, wke);
    };
    if (single)
        pipeline(std::true_type{});
    else
        pipeline(std::false_type{});
    if (!g.reduce_k())
        return;
    const int lg = g.lg, l16 = g.l16;
    const int col0 = g.wn * G::WN + G::FN * l16; // this lane's FN adjacent columns (stage_col)
    if (part) {
        // partial tile [BM][BNE] fp32 (gate/up: gate columns, then up columns)
        constexpr int BNE = G1 ? 2 * BN : BN;
#pragma unroll
        for (int i = 0; i < G::FM; i++)
#pragma unroll
            for (int j = 0; j < G::FN; j++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int row = g.wm * G::WM + i * 16 + 4 * lg + r;
                    const int col = col0 + j;
                    part[row * BNE + col] = g.acc0[i][j][r];
                    if constexpr (G1)
                        part[row * BNE + BN + col] = g.acc1[i][j][r];
                }
        return;
    }
    if constexpr (!kPrefetchRows)
        epilogue_picks();
    if constexpr (!G1 && ATOMIC)
        epilogue_weights();

    if constexpr (G1) { // rows without a pick (padding) are not stored: the down GEMM never reads them
        uint16_t *hb = a.h + (int64_t)b * RU * f + n0;
#pragma unroll
        for (int i = 0; i < G::FM; i++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                if (eflat[i][r] < 0)
                    continue;
                const int row = g.wm * G::WM + i * 16 + 4 * lg + r;
                float hv[G::FN];
#pragma unroll
                for (int j = 0; j < G::FN; j++) {
                    hv[j] = silu_mul(g.acc0[i][j][r], g.acc1[i][j][r]);
                }
                store_bf16<G::FN, false>(hb + (int64_t)row * f + col0, hv);
            }
    } else {
#pragma unroll
        for (int i = 0; i < G::FM; i++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int flat = eflat[i][r];
                if (flat < 0)
                    continue;
                if constexpr (ATOMIC) {
#pragma unroll
                    for (int j = 0; j < G::FN; j++)
                        unsafeAtomicAdd(&((float *)a.comb)[(int64_t)(flat / a.keff) * d + n0 + col0 + j],
                                        g.acc0[i][j][r] * ewt[i][r]);
                } else { // written once, read once by the combine: non-temporal
                    float ov[G::FN];
#pragma unroll
                    for (int j = 0; j < G::FN; j++)
                        ov[j] = g.acc0[i][j][r];
                    store_bf16<G::FN, true>((uint16_t *)a.comb + (int64_t)flat * d + n0 + col0, ov);
                }
            }
    }
}

// A tile's per-wave state: its LDS rings and the wave's place in the tile.
template <class T>
__device__ __forceinline__ void tile_state(T &g, uint8_t *lds)
{
    const int tid = threadIdx.x, lane = tid & 63;
    g.lds = lds;
    g.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    g.wt = g.wave % T::NT;  // wave within the tile
    g.kg = g.wave / T::NT;  // K range of this wave
    g.wm = g.wt / T::WAVES_N_;
    g.wn = g.wt % T::WAVES_N_;
    g.l16 = lane & 15;
    g.lg = lane >> 4;
}

template <class GP>
struct PairLds {
    static constexpr int bytes = GP::LDS_BYTES;
};
template <>
struct PairLds<void> {
    static constexpr int bytes = 0;
};

// GP (not void; 128-row blocks, block-major tiles): blocks 2i and 2i+1 of one
// expert run as one 256-row GP tile, GP::BN_ = BN / 2 columns wide, so the
// pair's weight rows are staged once per 256 rows instead of once per 128
// (the tile count per block is unchanged: block b's tile nt is the pair's
// column tile ntiles * (b mod 2) + nt).  Other blocks run G tiles.
template <class G, int GM, bool G1, bool PAGED, bool ATOMIC, bool TAIL, int CHUNK, class GP = void>
__global__ __launch_bounds__(64 * G::NW) void k_gemm(const FwdArgs a)
{
    // The host pass only needs this kernel's signature (for its launch stub);
    // the pipeline's gfx950 builtins are compiled in the device pass.
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int BM = G::BM_, BN = G::BN_;
    constexpr int LB = PairLds<GP>::bytes > G::LDS_BYTES ? PairLds<GP>::bytes : G::LDS_BYTES;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LB];
    G g;
    tile_state(g, lds);
    const int ntiles = (G1 ? a.f : a.d) / BN;
    int b, nt;
    if constexpr (TAIL) {
        const TileSpace ts = tile_space(a, BM, ntiles);
        const TailPlan tp = tail_plan(ts, a.slots[G1 ? 0 : 1]);
        if (tp.tail > 0) {
            const int i = (int)blockIdx.x;
            if (i < tp.full) { // whole tiles, dealt to the XCDs as in tile_of when full is whole rounds of
                               // chunks, else in contiguous eighths (full is a multiple of 8)
                static_assert(CHUNK > 0, "the split-tail launches deal their tiles in chunks");
                const int u = tp.full % (8 * CHUNK) == 0 ? chunk_tile<CHUNK>(i) : (i & 7) * (tp.full >> 3) + (i >> 3);
                const BlockInfo bi = tile_pick<GM, TAIL>(a, ts, ntiles, u, b, nt);
                gemm_tile<G, G1, PAGED, ATOMIC, TAIL>(a, g, b, nt, bi, ts.blocks);
            } else if (i - tp.full < tp.tail * tp.ks) {
                const int v = i - tp.full;
                const BlockInfo bi = tile_pick<GM, TAIL>(a, ts, ntiles, tp.full + v / tp.ks, b, nt);
                constexpr int BNE = G1 ? 2 * BN : BN;
                gemm_tile<G, G1, PAGED, ATOMIC, TAIL>(a, g, b, nt, bi, ts.blocks, v % tp.ks, tp.ks,
                                                      a.part + (int64_t)v * BM * BNE);
            }
            return;
        }
    }
    BlockInfo bi;
    int nblocks;
    if (!tile_of<GM, TAIL, CHUNK>(a, BM, ntiles, b, nt, bi, nblocks))
        return;
    if constexpr (!std::is_void<GP>::value) {
        static_assert(!TAIL && GM == 1 && BM == 128 && GP::BM_ == 256 && 2 * GP::BN_ == BN && GP::NW == G::NW,
                      "paired 128-row blocks");
        // the block's expert and its neighbours' (read here instead of in gemm_tile)
        const int ep = b > 0 ? a.block_expert[b - 1] : -1;
        const int e = block_owner(a, b);
        const int en = b + 1 < nblocks ? a.block_expert[b + 1] : -1;
        if (e >= 0 && ((b & 1) ? ep : en) == e) {
            GP gp;
            tile_state(gp, lds);
            gemm_tile<GP, G1, PAGED, ATOMIC, true, BM>(a, gp, b & ~1, ntiles * (b & 1) + nt, BlockInfo{e, 0},
                                                       nblocks);
        } else {
            gemm_tile<G, G1, PAGED, ATOMIC, true>(a, g, b, nt, BlockInfo{e, ep != e && en != e}, nblocks);
        }
        return;
    }
    gemm_tile<G, G1, PAGED, ATOMIC, TAIL>(a, g, b, nt, bi, nblocks);
#endif
}

// The epilogue of the split tail tiles: partials added in range order.  Tile
// t of the tail is handled by kFixupChunks(BM, BN) workgroups, each thread four
// consecutive columns of one row.
constexpr int fixup_chunks(int BM, int BN) { return BM * BN / 1024; }

template <int BM, int BN, int GM, bool G1, bool ATOMIC>
__global__ __launch_bounds__(256) void k_tail_fixup(const FwdArgs a)
{
    constexpr int CHUNKS = fixup_chunks(BM, BN);
    static_assert(CHUNKS * 1024 == BM * BN, "tile size");
    const int ntiles = (G1 ? a.f : a.d) / BN;
    const TileSpace ts = tile_space(a, BM, ntiles);
    const TailPlan tp = tail_plan(ts, a.slots[G1 ? 0 : 1]);
    const int t = (int)blockIdx.x / CHUNKS;
    if (t >= tp.tail)
        return;
    int b, nt;
    tile_pick<GM, true>(a, ts, ntiles, tp.full + t, b, nt); // the split tiles' (256-row) order
    if (block_owner(a, b) < 0)
        return;
    constexpr int BNE = G1 ? 2 * BN : BN;
    const int q = (((int)blockIdx.x % CHUNKS) * 256 + (int)threadIdx.x) * 4;
    const int row = q / BN, col = q % BN;
    const float *p = a.part + (int64_t)t * tp.ks * BM * BNE + (int64_t)row * BNE + col;
    float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
    for (int k = 0; k < tp.ks; k++) {
        const float4 v = *(const float4 *)(p + (int64_t)k * BM * BNE);
        s0.x += v.x, s0.y += v.y, s0.z += v.z, s0.w += v.w;
        if constexpr (G1) {
            const float4 u = *(const float4 *)(p + (int64_t)k * BM * BNE + BN);
            s1.x += u.x, s1.y += u.y, s1.z += u.z, s1.w += u.w;
        }
    }
    const int n0 = nt * BN;
    uint2 o;
    if constexpr (G1) {
        o.x = pack_bf16x2(silu_mul(s0.x, s1.x), silu_mul(s0.y, s1.y));
        o.y = pack_bf16x2(silu_mul(s0.z, s1.z), silu_mul(s0.w, s1.w));
        *(uint2 *)&a.h[((int64_t)b * BM + row) * a.f + n0 + col] = o;
    } else {
        const int flat = a.sorted_ids[b * BM + row];
        if (flat < 0 || flat >= a.T * a.keff)
            return;
        if constexpr (ATOMIC) {
            const float w = a.topk_w[flat];
            float *y32 = (float *)a.comb + (int64_t)(flat / a.keff) * a.d + n0 + col;
            unsafeAtomicAdd(y32 + 0, s0.x * w);
            unsafeAtomicAdd(y32 + 1, s0.y * w);
            unsafeAtomicAdd(y32 + 2, s0.z * w);
            unsafeAtomicAdd(y32 + 3, s0.w * w);
        } else {
            o.x = pack_bf16x2(s0.x, s0.y);
            o.y = pack_bf16x2(s0.z, s0.w);
            *(uint2 *)&((uint16_t *)a.comb)[(int64_t)flat * a.d + n0 + col] = o;
        }
    }
}

// ---------------------------------------------------------------------------- combine / convert
// Ordered: y[t][c] = bf16( sum_{j < keff} w[t][j] * part[t*keff + j][c] ), the
// bf16 expert output rows weighted and added in fp32 in slot order.  Atomic:
// y = bf16(y32).
// Eight columns per thread (combine), four (convert).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__global__ __launch_bounds__(256) void k_combine(const uint16_t *part, const float *w, int64_t T, int d, int keff,
                                                 uint16_t *y)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int q = d / 8;
    if (idx >= T * q)
        return;
    const int64_t t = idx / q;
    const int c = (int)(idx % q) * 8;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; k++)
        acc[k] = 0.f;
    for (int j0 = 0; j0 < keff; j0 += 4) {
        u32x4 v[4];
        float wj[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const bool in = j0 + r < keff;
            // each expert output row is read once: non-temporal
            v[r] = in ? __builtin_nontemporal_load((const u32x4 *)&part[(t * keff + j0 + r) * d + c])
                      : u32x4{0u, 0u, 0u, 0u};
            wj[r] = in ? w[t * keff + j0 + r] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; r++) // slot order; a missing slot adds +0
#pragma unroll
            for (int k = 0; k < 4; k++) {
                acc[2 * k] += wj[r] * bf16_to_f32(v[r][k] & 0xffffu);
                acc[2 * k + 1] += wj[r] * bf16_to_f32(v[r][k] >> 16);
            }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *(uint4 *)&y[t * d + c] = o;
}

__global__ __launch_bounds__(256) void k_convert(const float *y32, int64_t T, int d, uint16_t *y)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int q = d / 4;
    if (idx >= T * q)
        return;
    const float4 v = *(const float4 *)&y32[idx * 4];
    uint2 o;
    o.x = pack_bf16x2(v.x, v.y);
    o.y = pack_bf16x2(v.z, v.w);
    *(uint2 *)&y[idx * 4] = o;
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

// Tile shapes per block height: the gate/up and down GEMMs,
// Gemm<BM, BN, waves M, waves N, split-K waves, BK, stages, gate/up>.
template <int BM_, class G1T, class G2T, int CHUNK1_ = 0, int CHUNK2_ = 0, class P1T = void, class P2T = void>
struct Tiles {
    static constexpr int BM = BM_;
    using K1 = G1T;
    using K2 = G2T;
    // tiles of paired 128-row blocks (void: none)
    using P1 = P1T;
    using P2 = P2T;
    // tiles dealt to the XCDs in chunks of this many (0: contiguous eighths), per launch
    static constexpr int CHUNK1 = CHUNK1_, CHUNK2 = CHUNK2_;
    static_assert(G1T::BM_ == BM_ && G2T::BM_ == BM_, "block height");
};
// decode-sized blocks: one wave per 16-row tile, waves splitting K (many bytes in flight)
using Tiles16 = Tiles<16, Gemm<16, 16, 1, 1, 4, 64, 3, true>, Gemm<16, 32, 1, 1, 2, 64, 4, false>>;
using Tiles32 = Tiles<32, Gemm<32, 32, 1, 2, 1, 64, 2, true>, Gemm<32, 32, 1, 2, 1, 64, 2, false>>;
using Tiles64 = Tiles<64, Gemm<64, 64, 2, 2, 1, 64, 2, true>, Gemm<64, 64, 2, 2, 1, 64, 2, false>>;
// when d is a multiple of 256: 256-column down tiles, 8 waves of 32x64 (a
// block's h rows are re-read by 4x fewer column tiles; 63 against 77 us for the
// down GEMM of a 512-token Qwen1.5-shaped layer)
using Tiles64w = Tiles<64, Gemm<64, 64, 2, 2, 1, 64, 2, true>, Gemm<64, 256, 2, 4, 1, 64, 2, false>>;
// 128 x 64 gate/up tiles hold three stages of weight rows beside two of x rows
// (80 KB of LDS, two workgroups per CU): the weight rows are loaded two K-steps
// ahead (a 1024-token Qwen1.5-shaped gate/up GEMM 153 -> 149 us)
using Gate128 = Gemm<128, 64, 2, 2, 1, 64, 2, true, 3>;
using Tiles128 = Tiles<128, Gate128, Gemm<128, 128, 2, 2, 1, 64, 2, false>>;
// 128-row blocks of layers with many small experts (a block's x or h rows are
// re-read once per column tile): 256-column tiles, 8 waves of 64x64
// accumulators (gate/up: 64 x (64 gate + 64 up)); the gate/up stages fill all
// 160 KB of LDS, the down GEMM's short K loop (K = f) keeps three stages.
using Down128w = Gemm<128, 256, 2, 4, 1, 64, 3, false>;
using Tiles128w = Tiles<128, Gemm<128, 256, 2, 4, 1, 64, 2, true>, Down128w>;
using Tiles128d = Tiles<128, Gate128, Down128w>;
// batches of many 128-row blocks with d a multiple of 512: 512-column down
// tiles (8 waves of 64x128, two stages fill the 160 KB of LDS), so a block's h
// rows are re-read by half as many column tiles (Qwen3-Next-shaped down GEMM
// 400 -> 376 us); with few blocks the halved tile count leaves CUs idle (a
// 1024-token Qwen1.5-shaped layer: 69 -> 70 us), hence kWideDownTiles
using Down128x = Gemm<128, 512, 2, 4, 1, 64, 2, false>;
using Tiles128wx = Tiles<128, Gemm<128, 256, 2, 4, 1, 64, 2, true>, Down128x, kXcdChunkWide, 0,
                         Gemm<256, 128, 4, 2, 1, 64, 2, true>, Gemm<256, 256, 4, 2, 1, 64, 2, false>>;
using Tiles128dx = Tiles<128, Gate128, Down128x>;
constexpr int64_t kWideDownTiles = 1024; // 512-column down tiles from this many on (at most blocks x d / 512)
// when d is not a multiple of 128 (d and f are multiples of 64)
using Tiles128n = Tiles<128, Gate128, Gemm<128, 64, 2, 2, 1, 64, 2, false>>;
// large blocks (MFMA-bound shapes): 8 waves, two per SIMD, each with a 64x128
// accumulator tile (gate/up: 64 x (64 gate + 64 up)); 256x256 down tiles.  K
// steps of 64: every staged row is a 128-byte segment, which L2 feeds into LDS
// markedly faster than 64-byte ones; two stages fill 128 KB of LDS.
using Tiles256 = Tiles<256, Gemm<256, 128, 4, 2, 1, 64, 2, true>, Gemm<256, 256, 4, 2, 1, 64, 2, false>, kXcdChunk,
                       kXcdChunk>;
// when f or d is not a multiple of 128 / 256
using Tiles256n = Tiles<256, Gemm<256, 64, 4, 2, 1, 32, 4, true>, Gemm<256, 64, 4, 1, 1, 32, 4, false>>;

// Blocks per group.  Up to 128-row blocks, one: a block's column tiles run
// together, reading its x (or h) rows from L2 (these layers have few blocks
// per expert, so weight tiles are rarely shared; against groups of 4, a
// 1024-token Qwen1.5-shaped step took 223.8 against 231.6 us).  256-row tiles
// of experts with many blocks: up to 8, starting at each expert's first block.
constexpr int kGroupM = 1;
constexpr int kGroupMLong = 8; // 256-row tiles (expert-aligned groups)

// Workgroups of a kernel that fit on the current device at once (a multiple of
// 8), or 0 if the runtime cannot tell.  Cached per kernel and device.
int resident_slots(const void *kern, int threads)
{
    static std::mutex mu;
    struct Entry {
        const void *kern;
        int dev, slots;
    };
    static Entry cache[64];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; i++)
        if (cache[i].kern == kern && cache[i].dev == dev)
            return cache[i].slots;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        per_cu = cus = 0;
    }
    const int slots = per_cu * cus / 8 * 8;
    if (used < 64)
        cache[used++] = Entry{kern, dev, slots};
    return slots;
}

template <class C, bool PAGED, bool ATOMIC>
hipError_t launch_tiles_t(const FwdArgs &a_in, hipStream_t s)
{
    constexpr int BM = C::BM;
    using G1T = typename C::K1;
    using G2T = typename C::K2;
    constexpr int BN1 = G1T::BN_, BN2 = G2T::BN_;
    // the last-wave split is used by the 256-row tiles, whose K loops are long
    constexpr bool TAIL = BM == 256 && BN2 == 256;
    FwdArgs a = a_in;
    const int64_t n = a.T * a.keff;
    int64_t grid_m = n / BM + (n < a.E_tot ? n : a.E_tot);
    if (grid_m > a.blocks_cap)
        grid_m = a.blocks_cap;
    if (a.f % BN1 || a.d % BN2)
        return hipErrorInvalidValue;
    constexpr int T1 = 64 * G1T::NW, T2 = 64 * G2T::NW;
    constexpr int GM = TAIL ? kGroupMLong : kGroupM;
    // the split-tail launches deal their tiles in chunks (kXcdChunk unless the table says otherwise)
    constexpr int C1 = C::CHUNK1 ? C::CHUNK1 : (TAIL ? kXcdChunk : 0);
    constexpr int C2 = C::CHUNK2 ? C::CHUNK2 : (TAIL ? kXcdChunk : 0);
    auto k1 = k_gemm<G1T, GM, true, PAGED, false, TAIL, C1, typename C::P1>;
    auto k2 = k_gemm<G2T, GM, false, PAGED, ATOMIC, TAIL, C2, typename C::P2>;
    a.slots[0] = a.slots[1] = 0;
    if constexpr (TAIL) {
        const int p1 = resident_slots((const void *)k1, T1), p2 = resident_slots((const void *)k2, T2);
        if ((int64_t)p1 * BM * 2 * BN1 * 4 <= a.part_bytes)
            a.slots[0] = p1;
        if ((int64_t)p2 * BM * BN2 * 4 <= a.part_bytes)
            a.slots[1] = p2;
    }
    auto mark = [&](int i) {
        if (a.ev[i])
            (void)hipEventRecord(a.ev[i], s);
    };
    // whole rounds of chunks for chunk-dealt tiles, whole rounds of XCDs otherwise
    auto grid = [&](int ntiles, int slots, int chunk) {
        const int64_t round = 8 * (chunk > 0 ? chunk : 1);
        return (unsigned)((grid_m * ntiles + round - 1) / round * round + slots);
    };
    if (ATOMIC) {
        const int64_t n4 = a.T * a.d / 4;
        k_zero<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>((float4 *)a.comb, n4);
    }
    mark(0);
    k1<<<grid(a.f / BN1, a.slots[0], C1), T1, 0, s>>>(a);
    if constexpr (TAIL)
        if (a.slots[0])
            k_tail_fixup<BM, BN1, GM, true, false>
                <<<(unsigned)(a.slots[0] / 2 * fixup_chunks(BM, BN1)), 256, 0, s>>>(a);
    mark(1);
    k2<<<grid(a.d / BN2, a.slots[1], C2), T2, 0, s>>>(a);
    if constexpr (TAIL)
        if (a.slots[1])
            k_tail_fixup<BM, BN2, GM, false, ATOMIC>
                <<<(unsigned)(a.slots[1] / 2 * fixup_chunks(BM, BN2)), 256, 0, s>>>(a);
    mark(2);
    const int64_t nq = a.T * a.d / 4;
    if (ATOMIC)
        k_convert<<<(unsigned)((nq + 255) / 256), 256, 0, s>>>((const float *)a.comb, a.T, a.d, a.y);
    else
        k_combine<<<(unsigned)((nq / 2 + 255) / 256), 256, 0, s>>>((const uint16_t *)a.comb, a.topk_w, a.T, a.d, a.keff,
                                                               a.y);
    mark(3);
    return hipGetLastError();
}

template <class C, bool PAGED>
hipError_t launch_tiles(const FwdArgs &a, hipStream_t s)
{
    return a.atomic ? launch_tiles_t<C, PAGED, true>(a, s) : launch_tiles_t<C, PAGED, false>(a, s);
}

template <bool PAGED>
hipError_t launch_paged(const FwdArgs &a, hipStream_t s)
{
    switch (a.BM) {
    case 16: return launch_tiles<Tiles16, PAGED>(a, s);
    case 32: return launch_tiles<Tiles32, PAGED>(a, s);
    case 64: return a.d % 256 == 0 ? launch_tiles<Tiles64w, PAGED>(a, s) : launch_tiles<Tiles64, PAGED>(a, s);
    case 128:
        if (a.d % 512 == 0) {
            // the most blocks the batch can produce (as the launch grid counts them)
            const int64_t n = a.T * a.keff;
            int64_t blocks = n / 128 + (n < a.E_tot ? n : a.E_tot);
            blocks = blocks < a.blocks_cap ? blocks : a.blocks_cap;
            if (blocks * (a.d / 512) >= kWideDownTiles)
                return a.f % 256 == 0 ? launch_tiles<Tiles128wx, PAGED>(a, s) : launch_tiles<Tiles128dx, PAGED>(a, s);
        }
        if (a.d % 256 == 0)
            return a.f % 256 == 0 ? launch_tiles<Tiles128w, PAGED>(a, s) : launch_tiles<Tiles128d, PAGED>(a, s);
        return a.d % 128 == 0 ? launch_tiles<Tiles128, PAGED>(a, s) : launch_tiles<Tiles128n, PAGED>(a, s);
    case 256:
        if (a.f % Tiles256::K1::BN_ == 0 && a.d % Tiles256::K2::BN_ == 0)
            return launch_tiles<Tiles256, PAGED>(a, s);
        return launch_tiles<Tiles256n, PAGED>(a, s);
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
