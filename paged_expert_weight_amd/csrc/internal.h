// Internal declarations shared by the host runtime and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmoe {

// Device copy of one location-table entry; same 16-byte layout as moe_expert_loc.
struct DevLoc {
    int32_t kind;   // 0 pool page, 1 load-buffer slot
    int32_t idx[3]; // pool: W1, W3, W2 page; load buffer: slot in idx[0]
};

// The SwiGLU gate of one h element as every forward kernel computes it:
// silu(g) * u = g * (1 / (1 + e^-g)) * u in fp32, with the hardware's
// exponential (v_exp_f32) and reciprocal (v_rcp_f32, 1 ulp) instead of an
// IEEE division (about ten instructions); h is rounded to bf16 right after.
__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

constexpr int kMaxExpertsTotal = 1024; // E + S
constexpr int kMaxTopK = 32;

struct RouteArgs {
    const float *logits;
    int64_t T;
    int E, k, S, keff, E_tot, BM;
    int32_t *topk_ids;
    float *topk_w;
    int32_t *sorted_ids;
    int32_t *block_expert;
    int32_t *num_padded;
    int64_t sorted_cap, blocks_cap;
    int32_t *counts; // workspace: per-chunk counts [E_tot][chunks rounded up to 4] (large path only)
};

// Route + align.  Picks the fused one-workgroup path for small T, otherwise
// route, then per-chunk histograms and a scan + scatter per chunk.
hipError_t launch_route_align(const RouteArgs &a, hipStream_t s);
int64_t route_workspace_bytes(int64_t T, int keff, int E_tot);

struct FwdArgs {
    // weights: paged (locs != nullptr) or contiguous
    const DevLoc *locs;
    const uint16_t *pool;
    const uint16_t *loadbuf; // active load buffer (may be null)
    const uint16_t *w13;     // contiguous only
    const uint16_t *w2;      // contiguous only
    const uint16_t *x;
    int64_t T;
    int d, f, keff, E_tot, BM;
    const int32_t *topk_ids;
    const float *topk_w;
    const int32_t *sorted_ids;
    const int32_t *block_expert;
    const int32_t *num_padded;
    int64_t sorted_cap, blocks_cap;
    uint16_t *y;
    uint16_t *h;  // workspace [sorted_cap][f] bf16
    void *comb;   // workspace: bf16 [T*keff][d] expert output rows (ordered) or fp32 [T][d] (atomic)
    float *part;  // workspace: fp32 K-split partial tiles of the last partial wave (large tiles only)
    int64_t part_bytes;
    int slots[2]; // resident workgroups of the gate/up and down kernels when the last wave is split (0: never)
    bool atomic;
    hipEvent_t ev[4]; // optional: recorded before gate/up, after gate/up, after down, after combine
};

hipError_t launch_forward(const FwdArgs &a, hipStream_t s);

// Routing done inside the decode form's gate/up launch (route + forward in one
// call for a few tokens): the router's inputs and the routing outputs the
// launch writes (the same as the routing kernels').
struct DecRouteArgs {
    const float *logits; // [T][E] fp32
    int E, k, S;
    int32_t *topk_ids;
    float *topk_w;
    int32_t *sorted_ids;
    int32_t *block_expert;
    int32_t *num_padded;
};
bool decode_fits(const FwdArgs &a);
bool decode_routed_fits(const FwdArgs &a, const DecRouteArgs &r);
hipError_t launch_decode(const FwdArgs &a, hipStream_t s);
hipError_t launch_decode_routed(const FwdArgs &a, const DecRouteArgs &r, hipStream_t s);

struct ResolveArgs {
    const DevLoc *locs;
    const uint16_t *pool;
    const uint16_t *loadbuf0, *loadbuf1;
    int active_buf;
    int d, f, E_tot;
    int64_t n;
    const int32_t *e, *which;
    const int64_t *row, *col;
    int64_t *off;
    int32_t *base;
};
hipError_t launch_resolve(const ResolveArgs &a, hipStream_t s);

// Records msg for moe_last_error() and returns code.
int set_error(int code, const char *msg);

} // namespace pmoe
