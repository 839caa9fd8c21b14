// flint_internal.hpp -- private to libflint_moe.so: workspace layout, kernel
// parameter blocks, launcher declarations and small device helpers.
//
// Written for gfx950 (CDNA4): 64-lane wavefronts, 256 compute units in 8
// XCDs, 160 KiB LDS per CU.  Nothing here is portable on purpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_NVFP4 = 2 };

// ---------------------------------------------------------------------------
// Workspace: carved from one allocation made at create time, sized for
// max_tokens.  "Slots" number the rows of the expert outputs: routed pair
// positions 0..kT-1 in sorted (expert, pair id) order, then the shared
// expert's T rows kT..kT+T-1 in token order.
// ---------------------------------------------------------------------------
struct Workspace {
    float* logits;       // [Tm][E] fp32 router logits
    int* sel;            // [Tm][k] chosen experts, descending logit
    float* wts;          // [Tm][k] combine weights
    int* counts;         // [E] tokens per routed expert
    int* offsets;        // [E+1] exclusive scan of counts
    int* sorted_pair;    // [k*Tm] pair ids ordered by (expert, pair id)
    int* pair_pos;       // [k*Tm] inverse: slot of pair id
    int4* groups;        // [E+1] active groups {expert (E = shared), first sorted index, rows, first slot}
    int* n_groups;       // [1]
    int2* tiles;         // [max_tiles] prefill m-tiles {group, first row}
    int* n_tiles;        // [1]
    int* counter;        // [1] last-block ticket, zero between launches
    void* h;             // [(k+1)*Tm][fmax]: fp32 (decode) or bf16 (prefill)
    void* y;             // [(k+1)*Tm][d]:    fp32 (decode) or bf16 (prefill)
    int max_tiles;
};

struct Dims {
    int T, d, E, k, f, fs;
    int act;   // DT_F32 / DT_BF16
    int wdt;   // DT_F32 / DT_BF16 / DT_NVFP4
};

struct WeightPtrs {
    const void* gu;         // gate_up
    const void* dn;         // down
    const uint8_t* gus;     // NVFP4 gate_up block scales
    const uint8_t* dns;     // NVFP4 down block scales
    const float* ts;        // NVFP4 tensor scales [n][3]
};

struct LayerArgs {
    Dims dm;
    const void* x;
    const float* wr;
    const float* bias;
    WeightPtrs routed, shared;
    const float* residual;
    void* out;
};

// Launchers (each enqueues exactly one kernel on `s`).
hipError_t launch_route_decode(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_router_logits(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_topk(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_sort(const LayerArgs& a, const Workspace& w, int bm, hipStream_t s);
hipError_t launch_gateup_decode(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_down_decode(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_gateup_prefill(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_down_prefill(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_combine(const LayerArgs& a, const Workspace& w, bool y_bf16, hipStream_t s);
hipError_t launch_rmsnorm(int T, int d, const float* in, float eps, void* out, hipStream_t s);

// Prefill tile height (rows of A per MFMA tile); the sort builds its tile list with it.
constexpr int kPrefillBM = 64;

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

#endif

}  // namespace flint
