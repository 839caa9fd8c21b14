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
    float* rpart;        // [d/256][64][E] split-K router partial logits (decode, T <= 64)
    int* rcount;         // [4 ceil(E/16) + 8] router tickets, zero between launches
    uint16_t* w3;        // [3][E][d] router split into exact hi, mid, lo bf16 planes (prefill)
    float* sorted_wt;    // [k*Tm] combine weight of each sorted pair (wts[sorted_pair[i]])
    int4* groups;        // [E+1] active groups {expert (E = shared), first sorted index, rows, first slot}
    int* n_groups;       // [1]
    int2* tiles;         // [max_tiles] prefill m-tiles {group, first row}
    int* n_tiles;        // [1]
    int* counter;        // [1 + ceil(Tm/16)] last-block tickets, zero between launches
    int* dcount;         // [ceil(d/16)] decode down tickets (combine folded in), zero between launches
    float* part;         // [kchunks][kSplitRowsMax][d] split-K partial sums of the decode down (f > 1024)
    int* kcount;         // [(E+1) ceil(d/16)] split-K tickets, zero between launches
    void* h;             // [(k+1)*Tm][fmax] x 8 B: fp32 (decode VALU), three exact bf16 planes (decode
                         // MFMA), two f16 planes (NVFP4), or bf16 (prefill)
    void* y;             // [(k+1)*Tm][d]:    fp32 (decode) or bf16 (prefill)
    int max_tiles;
};

// The matrix-core decode down kernel holds at most 1024 of K in registers;
// wider experts split K into 1024-wide chunks whose partial sums meet in
// Workspace::part, which holds up to kSplitRowsMax (token, slot) rows.
constexpr int kDownKChunk = 1024;
constexpr int kSplitRowsMax = 576;

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
hipError_t launch_route_mfma(const LayerArgs& a, const Workspace& w, bool do_sort, hipStream_t s);
bool route_mfma_ok(const Dims& dm);
bool prefill_ok(const Dims& dm);
hipError_t launch_router_logits(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_topk(const LayerArgs& a, const Workspace& w, hipStream_t s);
bool router_gemm_ok(const Dims& dm);
hipError_t launch_router_gemm(const LayerArgs& a, const Workspace& w, hipStream_t s);
constexpr int kSortBlock = 1024;  // pairs per block of the prefill sort
hipError_t launch_sort(const LayerArgs& a, const Workspace& w, int bm, hipStream_t s);
hipError_t launch_gateup_decode(const LayerArgs& a, const Workspace& w, hipStream_t s);
hipError_t launch_down_decode(const LayerArgs& a, const Workspace& w, hipStream_t s);
// true when launch_down_decode also performs the combine (no launch_combine then)
bool down_decode_combines(const Dims& dm);
bool decode_fp4_ok(const Dims& dm);
hipError_t launch_gateup_prefill(const LayerArgs& a, const Workspace& w, int n_cu, hipStream_t s);
hipError_t launch_down_prefill(const LayerArgs& a, const Workspace& w, int n_cu, hipStream_t s);
hipError_t launch_combine(const LayerArgs& a, const Workspace& w, bool y_bf16, hipStream_t s);
hipError_t launch_rmsnorm(int T, int d, const float* in, float eps, void* out, hipStream_t s);

// Prefill tile height (rows of A per MFMA tile); the sort builds its tile list with it.
constexpr int kPrefillBM = 256;

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

// SiLU z * sigmoid(z) = z / (1 + e^-z) from the hardware base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32; about 1 ulp each): four instructions in
// place of the expf expansion and the IEEE divide sequence.  Every caller rounds
// the product to bf16 or scales it into an fp32 sum, far coarser than this error.
__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// fp32 -> bf16 with the hardware convert (v_cvt_pk_bf16_f32: round to nearest
// even, the result f32_to_bf16 gives for every non-NaN input).
__device__ __forceinline__ uint16_t f32_to_bf16_hw(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
// Two fp32 values to a packed bf16 pair (lo in bits 0-15) with one v_cvt_pk_bf16_f32.
typedef __attribute__((ext_vector_type(2))) float floatx2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2_t){lo, hi}, bf16x2_t));
}

// Cross-workgroup hand-off inside one kernel without full device fences.
// Data that another workgroup reads later in the same kernel is written and
// read with agent-scope relaxed atomics (device-coherent, so no L2 writeback
// or invalidate is needed for it); the writer waits for its stores to
// complete (vmcnt 0) before the workgroup barrier that precedes its ticket,
// and the reader issues its loads only after its ticket has returned.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

// Workgroup barrier that leaves pending global loads in flight.  A
// __syncthreads() carries a workgroup fence, for which the compiler waits for
// every outstanding vector-memory load (vmcnt 0) before the barrier, which
// would drain a prefetch pipeline at each step.  Callers wait explicitly
// (s_waitcnt) for the data they hand over; the memory clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

// All threads: finish this workgroup's hand-off stores, then thread 0 takes a
// ticket; returns true (in every thread) for the workgroup that arrives last.
__device__ __forceinline__ bool last_arrival(int* counter, int n_arrivals, int* s_flag) {
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int t = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = t == n_arrivals - 1;
        if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

// Raw buffer view of [base, base + bytes): a load whose offset lies at or past
// the end returns zeros without touching memory, which is how kernels skip the
// rows of a 16-row MFMA tile that hold no token.  Offsets are 32-bit; kOffNone
// is past the end of every view (views stay below 2 GiB).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
constexpr uint32_t kOffNone = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// MFMA operand types (gfx950 v_mfma_f32_16x16x32_bf16).  Lane l of a wave
// supplies A row (l & 15) and B column (l & 15), each with the 8 consecutive
// k values 8*(l >> 4) .. +7 of a 32-wide k step; the 16x16 fp32 result puts
// rows 4*(l >> 4) .. +3 of column (l & 15) in lane l.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float floatx4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ floatx4_t mfma16x16x32(uint4 a, uint4 b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// gfx950 v_mfma_f32_32x32x16_bf16: lane l supplies A row (l & 31) and B column
// (l & 31), each with the 8 consecutive k values 8*(l >> 5) .. +7 of a 16-wide
// k step; result value v of lane l is row 8*(v >> 2) + 4*(l >> 5) + (v & 3),
// column l & 31.
typedef __attribute__((ext_vector_type(16))) float floatx16_t;
__device__ __forceinline__ floatx16_t mfma32x32x16(uint4 a, uint4 b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Exact split of 8 fp32 values into hi + mid + lo bf16 parts (hi = RNE(v),
// mid = RNE(v - hi), lo = v - hi - mid, which fits bf16 exactly for normal
// inputs): a bf16 x bf16 MFMA over the three parts reproduces an fp32 operand.
__device__ __forceinline__ void split3_bf16(const float v[8], uint4& hi, uint4& mid, uint4& lo) {
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float a = v[2 * i], b = v[2 * i + 1];
        uint16_t ah = f32_to_bf16(a), bh = f32_to_bf16(b);
        float ar = a - bf16_to_f32(ah), br = b - bf16_to_f32(bh);
        uint16_t am = f32_to_bf16(ar), bm = f32_to_bf16(br);
        float ar2 = ar - bf16_to_f32(am), br2 = br - bf16_to_f32(bm);
        h[i] = (uint32_t)ah | ((uint32_t)bh << 16);
        m[i] = (uint32_t)am | ((uint32_t)bm << 16);
        l[i] = pack_bf16x2(ar2, br2);
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    mid = make_uint4(m[0], m[1], m[2], m[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Two-part split (hi + lo) of 8 fp32 values; relative error about 2^-17.
__device__ __forceinline__ void split2_bf16(const float v[8], uint4& hi, uint4& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float a = v[2 * i], b = v[2 * i + 1];
        uint16_t ah = f32_to_bf16(a), bh = f32_to_bf16(b);
        h[i] = (uint32_t)ah | ((uint32_t)bh << 16);
        l[i] = pack_bf16x2(a - bf16_to_f32(ah), b - bf16_to_f32(bh));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

#endif

}  // namespace flint
