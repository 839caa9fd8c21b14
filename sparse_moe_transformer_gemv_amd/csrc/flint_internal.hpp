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
    int* bhist;          // [ceil(Tm/16)][256] prefill: chosen experts per 16-token block (top-k kernel, read by the sort)
    int* n_tiles;        // [1]
    int* counter;        // [1 + ceil(Tm/16)] last-block tickets, zero between launches
    int* dcount;         // [ceil(d/16)] decode down tickets (combine folded in), zero between launches
    float* part;         // [kchunks][kSplitRowsMax][d] split-K partial sums of the decode down (f > 1024)
    int* kcount;         // [(E+1) ceil(d/16)] split-K tickets, zero between launches
    int* fbar;           // [kFusedBarrierInts] single-launch decode: grid-barrier counters and
                         // flags (zero between launches) and a sticky fault word
    void* h;             // [(k+1)*Tm][fmax] x 8 B: fp32 (decode VALU), three exact bf16 planes (decode
                         // MFMA), two f16 planes (NVFP4), or bf16 (prefill)
    void* y;             // [(k+1)*Tm][d] weighted expert outputs: fp32 rows (decode), or 2 bytes per
                         // element in 4-column blocks (prefill, pack_bfp4)
    int max_tiles;
    size_t ticket_bytes;  // the tickets occupy [0, ticket_bytes) of the allocation
    size_t float_off;     // floating-point data from here to the end
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
// Ints of the single-launch decode's barrier region: 2 barriers x 64 group slots
// + 4 slots (roots, generation, fault word) + 16 work counters, 256 ints each.
constexpr int kFusedBarrierInts = (2 * 64 + 20) * 256;
// Index of the fault word in that region (sticky: set when a wait gave up).
constexpr int kFusedFaultInt = (2 * 64 + 3) * 256;
// Single-launch decode: its grid size for this shape on n_cu compute units (every
// workgroup resident), or 0 where it does not apply; and its launch.
int fused_decode_grid(const Dims& dm, int n_cu);
hipError_t launch_decode_fused(const LayerArgs& a, const Workspace& w, int nblocks, hipStream_t s);
hipError_t launch_gateup_prefill(const LayerArgs& a, const Workspace& w, int n_cu, hipStream_t s);
hipError_t launch_down_prefill(const LayerArgs& a, const Workspace& w, int n_cu, hipStream_t s);
// packed: the y rows are in the prefill down kernels' block format (pack_bfp4), else fp32
hipError_t launch_combine(const LayerArgs& a, const Workspace& w, bool packed, hipStream_t s);
hipError_t launch_rmsnorm(int T, int d, const float* in, float eps, void* out, hipStream_t s);
constexpr int kCombineMaxK = 8;  // the largest top_k a configuration may ask for
// The combine and the next layer's pre-norm in one launch (out fp32, norm bf16);
// combine_norm_ok: the shapes it takes
bool combine_norm_ok(const Dims& dm);
hipError_t launch_combine_norm(const LayerArgs& a, const Workspace& w, bool packed, float eps, void* norm,
                               hipStream_t s);
// p[0 .. n) = v (a plain kernel, no memset node, so it is safe under graph capture)
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);

// Size of the static device scratch of the allocation-free forward, and its
// device address on the current device (set up on first use per device).
constexpr size_t kScratchBytes = 16u << 20;
hipError_t scratch_for_current_device(void** ptr);

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

__device__ __forceinline__ float wave_sum_dpp(float v);
// Sum over the 64 lanes, returned in every lane (the DPP reduction below).
__device__ __forceinline__ float wave_sum(float v) { return wave_sum_dpp(v); }

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

// 16 consecutive ints through the scalar cache, complete on return (the wait
// is in the same asm block and covers scalar and LDS operations only, not
// vector-memory loads in flight).  ptr 4-byte aligned; only for data written
// by an earlier launch (the scalar cache holds no stale copy).  pick16 gives
// each lane element i (a chain of selects, no memory).
typedef __attribute__((ext_vector_type(16))) int sint16_t;
__device__ __forceinline__ sint16_t sload_int16(const int* ptr) {
    sint16_t v;
    asm volatile("s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
    return v;
}
__device__ __forceinline__ int pick16(const sint16_t& v, int i) {
    int r = v[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) r = i == j ? v[j] : r;
    return r;
}

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

// Maximum over the 64 lanes: quad swaps, half-row and row mirrors reduce
// each row of 16 lanes, the row broadcasts carry the result to lane 63, and
// it is read back as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
// (lanes a step does not write read 0, the identity of the maximum, which
// lets the compiler fold each step into one v_max_u32 with a DPP operand)
#define FLINT_DPP_MAX(ctrl, rmask) \
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, rmask, 0xF, false))
    FLINT_DPP_MAX(0xB1, 0xF);   // quad_perm [1,0,3,2]
    FLINT_DPP_MAX(0x4E, 0xF);   // quad_perm [2,3,0,1]
    FLINT_DPP_MAX(0x141, 0xF);  // row_half_mirror
    FLINT_DPP_MAX(0x140, 0xF);  // row_mirror
    FLINT_DPP_MAX(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
    FLINT_DPP_MAX(0x143, 0xC);  // row_bcast:31 into rows 2 and 3
#undef FLINT_DPP_MAX
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Order-preserving map of a float to an unsigned key (-0 taken as +0); key 0
// marks an expert that can no longer be chosen.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key >> 31) ? (key & 0x7FFFFFFFu) : ~key);
}

// Sum over the 64 lanes, as wave_max_u32 reduces (DPP steps within rows, then
// row broadcasts; lanes a step does not write read 0), read from lane 63.
__device__ __forceinline__ float wave_sum_dpp(float v) {
#define FLINT_DPP_ADD(ctrl, rmask) \
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xF, false))
    FLINT_DPP_ADD(0xB1, 0xF);   // quad_perm [1,0,3,2]
    FLINT_DPP_ADD(0x4E, 0xF);   // quad_perm [2,3,0,1]
    FLINT_DPP_ADD(0x141, 0xF);  // row_half_mirror
    FLINT_DPP_ADD(0x140, 0xF);  // row_mirror
    FLINT_DPP_ADD(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
    FLINT_DPP_ADD(0x143, 0xC);  // row_bcast:31 into rows 2 and 3
#undef FLINT_DPP_ADD
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Inclusive sum over the 64 lanes: rows of 16 lanes (row_shr 1, 2, 4, 8;
// lanes shifted in from outside the row read 0), then row 15's total into
// rows 1 and 3 and row 31's into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
    return v;
}

// Top-k (k <= 8) of one token's E <= 256 logits held in LDS, by one
// wavefront: lane l takes the order-preserving keys of experts 4 l .. 4 l + 3
// and sorts them (equal keys keep the lower expert first); each round takes
// the wavefront maximum of the lanes' heads, the lowest lane holding it wins
// (which is the lowest expert index among equal logits) and pops its head.
// Weights: softmax of the chosen logits, hardware exp2 and reciprocal (about
// 1 ulp each).  Lane j < k returns slot j: *sel (expert) and *w (weight).
__device__ __forceinline__ void topk_token_lds(const float* lrow, int E, int k, int lane, int* sel, float* w) {
    uint32_t key[4];
    int eid[4];
    if ((E & 3) == 0 && (reinterpret_cast<uintptr_t>(lrow) & 15) == 0) {
        // one 16-byte read per lane (no read past the row: 4 lane < E covers it whole)
        const float4 v = 4 * lane < E ? *reinterpret_cast<const float4*>(lrow + 4 * lane)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            key[i] = 4 * lane < E ? order_key(vv[i]) : 0u;
            eid[i] = 4 * lane + i;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            key[i] = e < E ? order_key(lrow[e]) : 0u;
            eid[i] = e;
        }
    }
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b2 = 0; b2 < 3 - a; ++b2)
            if (key[b2 + 1] > key[b2]) {
                const uint32_t tk = key[b2];
                key[b2] = key[b2 + 1];
                key[b2 + 1] = tk;
                const int te = eid[b2];
                eid[b2] = eid[b2 + 1];
                eid[b2 + 1] = te;
            }
    float lsel = 0.f, l0 = 0.f;
    int esel = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j >= k) break;  // uniform
        const uint32_t M = wave_max_u32(key[0]);
        const int L = __builtin_ctzll(__ballot(key[0] == M));
        const int ej = __builtin_amdgcn_readlane(eid[0], L);
        if (lane == L) {
            key[0] = key[1]; key[1] = key[2]; key[2] = key[3]; key[3] = 0u;
            eid[0] = eid[1]; eid[1] = eid[2]; eid[2] = eid[3];
        }
        const float lj = key_value(M);
        if (j == 0) l0 = lj;
        if (lane == j) {
            lsel = lj;
            esel = ej;
        }
    }
    const float pj = lane < k ? __builtin_amdgcn_exp2f((lsel - l0) * 1.4426950408889634f) : 0.f;
    const float sum = wave_sum_dpp(pj);
    *sel = esel;
    *w = pj * __builtin_amdgcn_rcpf(sum);
}

// Raw buffer view of [base, base + bytes): a load whose offset lies at or past
// the end returns zeros without touching memory, which is how kernels skip the
// rows of a 16-row MFMA tile that hold no token.  Offsets are 32-bit; kOffNone
// is past the end of every view (views stay below 2 GiB).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
constexpr uint32_t kOffNone = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// The same load and a 16-byte store at agent scope (cache policy sc1, as the
// agent-scope atomics above): data handed between workgroups of one launch.
constexpr int kCpolAgent = 16;
__device__ __forceinline__ uint4 buffer_load16_agent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolAgent);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void buffer_store16_agent(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){v.x, v.y, v.z, v.w}, r, (int)off, 0, kCpolAgent);
}

// Packed y elements (the prefill path's weighted expert rows): block floating
// point over 4 consecutive columns in 8 bytes, one 8-bit exponent E shared by
// four 14-bit two's-complement mantissas q, value = q * 2^(E - 139).  E is the
// fp32 exponent field of the block's largest magnitude (at least 13), so every
// |q| <= 2^13 - 1 and each value's error is at most 2^-12 of that largest
// magnitude (half a step of 2^(E - 139), a whole step where the top is clamped);
// a block whose largest magnitude is below 2^-114 is stored with E = 13, its
// error under 2^-126.
// Bits: [0,8) E, [8,22) q0, [22,36) q1, [36,50) q2, [50,64) q3.  A block holding
// a NaN or an infinity is stored with E = 255 and reads back as four NaNs.
// Written without branches (the epilogue that calls it runs 32 blocks per lane
// back to back): each value is scaled by 2^(139 - E), which is exact, and
// rounded to an integer, ties to even, by adding 1.5 x 2^23, whose sum has a
// unit of 1 and so holds the integer in the low bits of its mantissa (two's
// complement there, the offset having 22 zero low bits); the clamp to +-8191
// acts on that sum.  A fused multiply-add of the two steps gives the same
// sum, the product being exact.  Also compiled for the host, where a test
// checks it bit for bit against the format's plain definition.
__host__ __device__ __forceinline__ uint2 pack_bfp4(float a, float b, float c, float d) {
    const uint32_t ma = __builtin_bit_cast(uint32_t, a) & 0x7FFFFFFFu, mb = __builtin_bit_cast(uint32_t, b) & 0x7FFFFFFFu;
    const uint32_t mc = __builtin_bit_cast(uint32_t, c) & 0x7FFFFFFFu, md = __builtin_bit_cast(uint32_t, d) & 0x7FFFFFFFu;
    const uint32_t mab = ma > mb ? ma : mb, mcd = mc > md ? mc : md;
    const uint32_t m = mab > mcd ? mab : mcd;
    const uint32_t e8 = m >> 23;  // 255 for a NaN or an infinity
    const uint32_t E = e8 > 13u ? e8 : 13u;
    const float s = __builtin_bit_cast(float, (266u - E) << 23);  // 2^(139 - E)
    constexpr float kM = 12582912.0f, kLo = kM - 8191.0f, kHi = kM + 8191.0f;
    const uint32_t q0 = __builtin_bit_cast(uint32_t, fminf(fmaxf(a * s + kM, kLo), kHi));
    const uint32_t q1 = __builtin_bit_cast(uint32_t, fminf(fmaxf(b * s + kM, kLo), kHi));
    const uint32_t q2 = __builtin_bit_cast(uint32_t, fminf(fmaxf(c * s + kM, kLo), kHi));
    const uint32_t q3 = __builtin_bit_cast(uint32_t, fminf(fmaxf(d * s + kM, kLo), kHi));
    const uint32_t w0 = E | ((q0 & 0x3FFFu) << 8) | (q1 << 22);
    const uint32_t w1 = ((q1 >> 10) & 0xFu) | ((q2 & 0x3FFFu) << 4) | (q3 << 18);
    const bool bad = E == 255u;
    return make_uint2(bad ? 255u : w0, bad ? 0u : w1);
}
__device__ __forceinline__ float4 unpack_bfp4(uint2 v) {
    const uint32_t E = v.x & 0xFFu;
    const float s = E == 255u ? __uint_as_float(0x7FC00000u) : __uint_as_float((E - 12u) << 23);  // 2^(E - 139)
    const int q0 = (int)(v.x << 10) >> 18;
    const int q1 = (int)(__builtin_amdgcn_alignbit(v.y, v.x, 22) << 18) >> 18;
    const int q2 = (int)(v.y << 14) >> 18;
    const int q3 = (int)v.y >> 18;
    return make_float4((float)q0 * s, (float)q1 * s, (float)q2 * s, (float)q3 * s);
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
