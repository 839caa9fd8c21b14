// expert_decode.hip -- bandwidth-bound expert kernels for decode-sized token
// counts (gfx950).
//
// Decoding reads each selected expert's weights once per step, so the time is
// set by weight bytes over HBM bandwidth [kongchang.com, "Recursive
// Open-Sources Flint: A 40B MoE Local Coding Model with 2.5B Active
// Parameters", section "125+ tokens/s: The Practical Threshold for Local
// Inference"; futurpulse.com, "Flint model: local coding with fewer active
// parameters", section "How does Flint use 39.8B parameters efficiently?":
// only the routed group and the shared expert are read per token].
//
// The kernels are weight-stationary: every active (group, row block) work
// item streams its weight rows from HBM exactly once with 16-byte-per-lane
// coalesced loads and applies them to all tokens routed to that group (token
// vectors come through L1/L2).  Groups are the experts with at least one token
// plus the shared expert, listed by the router's counting sort.
//
//   gate/up:  h[slot][j] = SiLU(G_j . x_t) * (U_j . x_t)      (fp32 out)
//   down:     y[slot][n] = w_slot * (D_n . h[slot])           (fp32 out)
//
// Weight formats: fp32, bf16, and NVFP4 (E2M1 codes with one E4M3 scale per
// 16 elements and an fp32 tensor scale [evermx.com, "Recursive Flint:
// Open-Weight MoE Coding Model, 2.5B Active", Feature Overview,
// "Quantization"]; decoded in registers).
#include "flint_internal.hpp"

namespace flint {

// ---------------------------------------------------------------------------
// Weight chunk loaders: VEC consecutive elements of one row starting at k0
// (k0 a multiple of VEC), returned as fp32.
// ---------------------------------------------------------------------------
template <int WT> struct WChunk;

template <> struct WChunk<DT_F32> {
    static constexpr int VEC = 4;
    uint4 raw;
    __device__ __forceinline__ void load(const void* row, const uint8_t*, int k0) {
        raw = *reinterpret_cast<const uint4*>(static_cast<const float*>(row) + k0);
    }
    __device__ __forceinline__ void decode(float v[VEC], float) const {
        v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
        v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
    }
};

template <> struct WChunk<DT_BF16> {
    static constexpr int VEC = 8;
    uint4 raw;
    __device__ __forceinline__ void load(const void* row, const uint8_t*, int k0) {
        raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + k0);
    }
    __device__ __forceinline__ void decode(float v[VEC], float) const {
        v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x); v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
        v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z); v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
    }
};

// E2M1 magnitude codes 0..7 -> 0, 0.5, 1, 1.5, 2, 3, 4, 6 (OCP MX): exponent
// field e (bias 1) and mantissa bit m; e == 0 is subnormal (0.5 * m).
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
    return (c & 8u) ? -mag : mag;
}

// E4M3 (OCP FP8 "E4M3FN") -> fp32: bias 7, subnormals 0.m * 2^-6, S.1111.111 = NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t s = c >> 7, e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
    else if (e == 0u) v = (float)m * 0.001953125f;  // m/8 * 2^-6
    else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return s ? -v : v;
}

template <> struct WChunk<DT_NVFP4> {
    static constexpr int VEC = 16;  // one block-scale group per chunk
    uint2 raw;                      // 16 E2M1 codes, even element in the low nibble
    uint32_t sc;                    // E4M3 block-scale code
    __device__ __forceinline__ void load(const void* row, const uint8_t* srow, int k0) {
        raw = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(row) + k0 / 2);
        sc = srow[k0 / 16];
    }
    __device__ __forceinline__ void decode(float v[VEC], float tscale) const {
        const float s = e4m3_to_f32(sc) * tscale;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = e2m1_to_f32(raw.x >> (4 * i)) * s;
            v[8 + i] = e2m1_to_f32(raw.y >> (4 * i)) * s;
        }
    }
};

// Row pointers of expert matrices.  Element offsets for fp32/bf16, byte
// offsets for NVFP4 codes (2 per byte) and scales (1 per 16 elements).
template <int WT>
__device__ __forceinline__ const void* row_ptr(const void* base, size_t row, int K) {
    if constexpr (WT == DT_F32) return static_cast<const float*>(base) + row * K;
    else if constexpr (WT == DT_BF16) return static_cast<const uint16_t*>(base) + row * K;
    else return static_cast<const uint8_t*>(base) + row * (K / 2);
}

template <typename ActT, int VEC>
__device__ __forceinline__ void load_act(const ActT* x, float v[VEC]) {
    if constexpr (sizeof(ActT) == 4) {
#pragma unroll
        for (int i = 0; i < VEC; i += 4) {
            float4 a = *reinterpret_cast<const float4*>(x + i);
            v[i] = a.x; v[i + 1] = a.y; v[i + 2] = a.z; v[i + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; i += 8) {
            uint4 a = *reinterpret_cast<const uint4*>(x + i);
            v[i] = bf16_lo(a.x); v[i + 1] = bf16_hi(a.x); v[i + 2] = bf16_lo(a.y);
            v[i + 3] = bf16_hi(a.y); v[i + 4] = bf16_lo(a.z); v[i + 5] = bf16_hi(a.z);
            v[i + 6] = bf16_lo(a.w); v[i + 7] = bf16_hi(a.w);
        }
    }
}

template <int VEC>
__device__ __forceinline__ void load_h(const float* h, float v[VEC]) {
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
        float4 a = *reinterpret_cast<const float4*>(h + i);
        v[i] = a.x; v[i + 1] = a.y; v[i + 2] = a.z; v[i + 3] = a.w;
    }
}

struct ExpertParams {
    Dims dm;
    const void* x;
    WeightPtrs routed, shared;
    Workspace ws;
    int hstride;  // row stride of h (max(f, fs))
    // down kernels that fold the combine in (see down_mfma_kernel)
    int combine;            // 1: this launch also writes out
    const float* residual;  // added first when not null
    void* out;              // [T][d] fp32 (out_f32) or bf16
    int out_f32;
    int kchunks;            // down kernels: K chunks of the widest group (1: no split)
};

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Block = 4 waves, each wave owns FPW features (FPW gate
// rows and the matching FPW up rows); work item = (group, block of 4*FPW
// features).  Tokens of the group are processed kTG at a time, each pass
// streaming the block's weight rows once: 4 for small batches, 16 from 16
// tokens on (fewer passes over the weights, more accumulators).
// ---------------------------------------------------------------------------
constexpr int kFPW = 2;
constexpr int kFPB = 4 * kFPW;
constexpr int kTGWide = 16;  // tokens per pass from this batch size on
__host__ __device__ constexpr int tokens_per_pass(int T) { return T >= kTGWide ? kTGWide : 4; }

template <typename ActT, int WT, int kTG>
__global__ __launch_bounds__(256) void gateup_decode_kernel(ExpertParams p) {
    using W = WChunk<WT>;
    constexpr int VEC = W::VEC;
    constexpr int NR = 2 * kFPW;  // rows per wave
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int fmax = max(p.dm.f, p.dm.fs);
    const int fblocks = (fmax + kFPB - 1) / kFPB;
    const int gi = blockIdx.x / fblocks, fb = blockIdx.x % fblocks;
    if (gi >= *p.ws.n_groups) return;
    const int4 g = p.ws.groups[gi];  // {expert, first sorted index, rows, first slot}
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int j0 = fb * kFPB + wave * kFPW;
    if (j0 >= F) return;
    const int d = p.dm.d;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const size_t row0 = e * 2 * F;  // first gate_up row of this expert
    float tsc[NR];
    const void* rows[NR];
    const uint8_t* srows[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        // rows 0..FPW-1: gate j0+r; rows FPW..: up j0+r-FPW
        const size_t rr = row0 + (r < kFPW ? (size_t)(j0 + r) : (size_t)(F + j0 + r - kFPW));
        rows[r] = row_ptr<WT>(wp.gu, rr, d);
        srows[r] = (WT == DT_NVFP4) ? wp.gus + rr * (d / 16) : nullptr;
        tsc[r] = (WT == DT_NVFP4) ? wp.ts[e * 3 + (r < kFPW ? 0 : 1)] : 1.f;
    }
    const ActT* x = static_cast<const ActT*>(p.x);
    const int kT = p.dm.k * p.dm.T;
    (void)kT;
    for (int r0 = 0; r0 < g.z; r0 += kTG) {
        int tok[kTG];
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt) {
            const int r = r0 + tt;
            tok[tt] = (r < g.z) ? (is_shared ? r : p.ws.sorted_pair[g.y + r] / p.dm.k) : -1;
        }
        float acc[kTG][NR];
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[tt][r] = 0.f;
        for (int k0 = lane * VEC; k0 < d; k0 += 64 * VEC) {
            W wc[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) wc[r].load(rows[r], srows[r], k0);
#pragma unroll
            for (int tt = 0; tt < kTG; ++tt) {
                if (tok[tt] < 0) continue;
                float xv[VEC];
                load_act<ActT, VEC>(x + (size_t)tok[tt] * d + k0, xv);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    float wv[VEC];
                    wc[r].decode(wv, tsc[r]);
                    float a = acc[tt][r];
#pragma unroll
                    for (int v = 0; v < VEC; ++v) a = fmaf(wv[v], xv[v], a);
                    acc[tt][r] = a;
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt) {
            if (tok[tt] < 0) continue;  // uniform across the wave
            float s[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) s[r] = wave_sum(acc[tt][r]);
            if (lane < kFPW) {
                float gv = s[0], uv = s[kFPW];
#pragma unroll
                for (int q = 1; q < kFPW; ++q)
                    if (lane == q) { gv = s[q]; uv = s[kFPW + q]; }
                float* hrow = static_cast<float*>(p.ws.h) + (size_t)(g.w + r0 + tt) * p.hstride;
                hrow[j0 + lane] = silu_f32(gv) * uv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down.  Block = 4 waves x kRPW output rows; work item = (group, block of
// 4*kRPW rows of d).  Each lane reads VEC elements of a row of D (K = F).
// ---------------------------------------------------------------------------
constexpr int kRPW = 4;
constexpr int kRPB = 4 * kRPW;

template <int WT, int kTG>
__global__ __launch_bounds__(256) void down_decode_kernel(ExpertParams p) {
    using W = WChunk<WT>;
    constexpr int VEC = W::VEC;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = p.dm.d;
    const int rblocks = (d + kRPB - 1) / kRPB;
    const int gi = blockIdx.x / rblocks, rb = blockIdx.x % rblocks;
    if (gi >= *p.ws.n_groups) return;
    const int4 g = p.ws.groups[gi];
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int n0 = rb * kRPB + wave * kRPW;
    if (n0 >= d) return;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const void* rows[kRPW];
    const uint8_t* srows[kRPW];
    const float tsc = (WT == DT_NVFP4) ? wp.ts[e * 3 + 2] : 1.f;
#pragma unroll
    for (int r = 0; r < kRPW; ++r) {
        const size_t rr = e * (size_t)d + (size_t)(n0 + r);
        rows[r] = row_ptr<WT>(wp.dn, rr, F);
        srows[r] = (WT == DT_NVFP4) ? wp.dns + rr * (F / 16) : nullptr;
    }
    const float* h = static_cast<const float*>(p.ws.h);
    float* y = static_cast<float*>(p.ws.y);
    for (int r0 = 0; r0 < g.z; r0 += kTG) {
        int slot[kTG];
        float wslot[kTG];
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt) {
            const int r = r0 + tt;
            slot[tt] = (r < g.z) ? g.w + r : -1;
            wslot[tt] = (r < g.z && !is_shared) ? p.ws.sorted_wt[g.y + r] : 1.f;
        }
        float acc[kTG][kRPW];
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt)
#pragma unroll
            for (int r = 0; r < kRPW; ++r) acc[tt][r] = 0.f;
        for (int k0 = lane * VEC; k0 < F; k0 += 64 * VEC) {
            W wc[kRPW];
#pragma unroll
            for (int r = 0; r < kRPW; ++r) wc[r].load(rows[r], srows[r], k0);
#pragma unroll
            for (int tt = 0; tt < kTG; ++tt) {
                if (slot[tt] < 0) continue;
                float hv[VEC];
                load_h<VEC>(h + (size_t)slot[tt] * p.hstride + k0, hv);
#pragma unroll
                for (int r = 0; r < kRPW; ++r) {
                    float wv[VEC];
                    wc[r].decode(wv, tsc);
                    float a = acc[tt][r];
#pragma unroll
                    for (int v = 0; v < VEC; ++v) a = fmaf(wv[v], hv[v], a);
                    acc[tt][r] = a;
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < kTG; ++tt) {
            if (slot[tt] < 0) continue;
            float s[kRPW];
#pragma unroll
            for (int r = 0; r < kRPW; ++r) s[r] = wave_sum(acc[tt][r]);
            if (lane < kRPW) {
                float v = s[0];
#pragma unroll
                for (int q = 1; q < kRPW; ++q)
                    if (lane == q) v = s[q];
                y[(size_t)slot[tt] * d + n0 + lane] = wslot[tt] * v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 x bf16 fast path on the matrix cores.  The MFMA is only the dot-product
// engine here (the kernels stay bound by weight bytes): a 16x16x32 step
// consumes 16 weight rows x 32 k (1 KiB) against up to 16 tokens, with no
// cross-lane reduction and no VALU conversion.  Weight fragments are loaded
// straight from HBM in the MFMA layout (each row contributes 64 contiguous
// bytes per load instruction) and stay in registers while every token tile of
// the group streams past.  K is split over the 4 waves of a block; the partial
// tiles are summed through LDS in a fixed order.
// ---------------------------------------------------------------------------

// One 16-token tile of a bf16 gate/up block; sp is the sorted pair of this
// lane's token row.  Padding rows read as zeros (buffer view past T).
// The lane's activation fragments of one 16-token tile (token row r0 + row).
// The sorted pair of token row `row` of a group's first tile, read after the
// weight loads are issued: 16 entries through the scalar cache (rows past the
// group read the entries after it, which are never used).  A vector load
// issued before direct-to-LDS weight loads is waited for with vmcnt(0) (the
// compiler does not order the two kinds), which would hold the activation
// loads back until every weight byte has arrived; the scalar path waits for
// scalar loads alone.  The sorted pairs are followed by more workspace, so the
// 16 entries stay inside the allocation.
__device__ __forceinline__ int gateup_row_pair(const ExpertParams& p, const int4& g, int row) {
    return pick16(sload_int16(p.ws.sorted_pair + g.y), row);
}

template <int NSTEP>
__device__ __forceinline__ void gateup_load_x(const ExpertParams& p, const int4& g, bool is_shared, int r0, int sp,
                                              __amdgpu_buffer_rsrc_t xv, int kl, uint4 (&a)[NSTEP]) {
    const int row = threadIdx.x & 15;
    const int m = r0 + row;
    const int tok = is_shared ? m : sp / p.dm.k;
    const uint32_t xo = m < g.z ? (uint32_t)(tok * p.dm.d + kl) * 2 : kOffNone;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) a[s] = buffer_load16(xv, xo + 64 * s);
}

// a: the tile's activation fragments (gateup_load_x).  COH: h is read by other
// workgroups of the same launch (single-launch decode), so it is stored at
// agent scope.
template <int NSTEP, bool COH = false>
__device__ __forceinline__ void gateup_mfma_tile(const ExpertParams& p, const int4& g, int r0,
                                                 const uint4 (&a)[NSTEP], const uint4 (&b)[NSTEP], int j0,
                                                 float (&s_part)[4][256], uint16_t (&s_h)[16][3][8]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first MFMA
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) acc = mfma16x16x32(a[s], b[s], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[wave][(4 * q + i) * 16 + row] = acc[i];
    __syncthreads();
    const int mm = tid >> 4, n = tid & 15;
    if (n < 8 && r0 + mm < g.z) {
        const int gi_ = mm * 16 + n, ui_ = gi_ + 8;
        const float gv = ((s_part[0][gi_] + s_part[1][gi_]) + s_part[2][gi_]) + s_part[3][gi_];
        const float uv = ((s_part[0][ui_] + s_part[1][ui_]) + s_part[2][ui_]) + s_part[3][ui_];
        // h goes out as its exact three-part bf16 split (hi + mid + lo), once,
        // instead of being split again by every down block that reads it
        const float hv = silu_f32(gv) * uv;
        const uint16_t hi = f32_to_bf16(hv);
        const float r1 = hv - bf16_to_f32(hi);
        const uint16_t mid = f32_to_bf16(r1);
        s_h[mm][0][n] = hi;
        s_h[mm][1][n] = mid;
        s_h[mm][2][n] = f32_to_bf16(r1 - bf16_to_f32(mid));
    }
    __syncthreads();
    // one 16-byte store per (token row, plane): the 8 features of this block
    if (tid < 48 && r0 + tid / 3 < g.z) {
        const int r = tid / 3, pl = tid % 3;
        const size_t plane = (size_t)(p.dm.k + 1) * p.dm.T * p.hstride;
        const size_t e_off = pl * plane + (size_t)(g.w + r0 + r) * p.hstride + j0;
        const uint4 v = *reinterpret_cast<const uint4*>(&s_h[r][pl][0]);
        if constexpr (COH)
            buffer_store16_agent(v, buffer_view(p.ws.h, (uint32_t)(3 * plane * 2)), (uint32_t)(e_off * 2));
        else
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.ws.h) + e_off) = v;
    }
}

// gate/up: block = (group, 8 features): B columns 0..7 are gate rows j0..j0+7,
// columns 8..15 the matching up rows.  NSTEP = k steps per wave = d / 128.
// The weights are requested first, then the token rows' sorted pairs (scalar
// loads, see gateup_row_pair), then the first token tile's activations, all
// before the first wait on the weights; that tile is peeled off the loop so no
// loop-carried register forces an earlier wait.
// With NSTEP >= 2 the weights travel through LDS: each wave fetches its 16
// rows x d / 4 k with direct-to-LDS loads of whole 128-byte lines (8 rows per
// load) carrying the non-temporal hint, then reads them back in the MFMA
// layout.  Loads of 64 bytes per row (the MFMA layout straight from memory)
// split every line over two instructions, and the hint then makes the second
// half fetch the line again; whole lines with the hint stream about 6% faster
// than the split form without it.  Each wave reads only what it loaded, so no
// barrier is needed; 16-byte chunks are XOR-swizzled by row so the reads are
// free of bank conflicts.  With d = 2048 the fourth wave loads its weights
// straight into registers instead: staging all four waves' 64 KiB leaves room
// for two workgroups per CU, staging three (48 KiB) for three, and the weight
// bytes a CU keeps in flight set the rate (as measured for down).
template <int NSTEP>
struct GateupWeightLds {
    static constexpr int kWaves = NSTEP >= 16 ? 3 : 4;  // waves that stage through LDS
    static constexpr int kBytes = NSTEP >= 2 ? kWaves * 16 * 64 * NSTEP : 16;  // kWaves x 16 rows x d / 2 bytes
    static constexpr int kAllBytes = 4 * 16 * 64 * NSTEP;  // all four waves (the single-launch kernel)
};

template <int NSTEP>
__global__ __launch_bounds__(256) void gateup_mfma_kernel(ExpertParams p) {
    __shared__ float s_part[4][256];
    __shared__ __attribute__((aligned(16))) uint16_t s_h[16][3][8];
    __shared__ __attribute__((aligned(16))) unsigned char s_w[GateupWeightLds<NSTEP>::kBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const int fblocks = p.hstride / 8;
    const int gi = blockIdx.x / fblocks, fb = blockIdx.x % fblocks;
    if (gi >= *p.ws.n_groups) return;
    const int4 g = p.ws.groups[gi];
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int j0 = fb * 8;
    if (j0 >= F) return;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const uint16_t* gu = static_cast<const uint16_t*>(is_shared ? p.shared.gu : p.routed.gu);
    const size_t wr = e * 2 * F + (row < 8 ? (size_t)(j0 + row) : (size_t)(F + j0 + row - 8));
    const int kl = wave * (d / 4) + 8 * q;
    const __amdgpu_buffer_rsrc_t xv = buffer_view(p.x, (uint32_t)p.dm.T * d * 2);
    uint4 b[NSTEP];
    if constexpr (NSTEP >= 2) {
        uint4 a0[NSTEP];
        if (wave < GateupWeightLds<NSTEP>::kWaves) {  // uniform per wave
            // load i: rows 8 (i & 1) + (lane >> 3) of this block, 128-byte segment i >> 1 of
            // the wave's k range; the lane fetches logical chunk (lane & 7) ^ (row & 7)
            unsigned char* sw = s_w + wave * (16 * 64 * NSTEP);
            const int kw = wave * (d / 4);
#pragma unroll
            for (int i = 0; i < NSTEP; ++i) {
                const int r = 8 * (i & 1) + (lane >> 3);
                const size_t wrr = e * 2 * F + (r < 8 ? (size_t)(j0 + r) : (size_t)(F + j0 + r - 8));
                const int c = (lane & 7) ^ (r & 7);
                __builtin_amdgcn_global_load_lds(gu + wrr * d + kw + 64 * (i >> 1) + 8 * c, sw + i * 1024, 16, 0,
                                                 2);
            }
            gateup_load_x<NSTEP>(p, g, is_shared, 0, gateup_row_pair(p, g, row), xv, kl, a0);
            // every load above has landed before the reads below (the compiler waits for
            // the direct-to-LDS loads before any LDS read)
            const uint32_t rbase = (uint32_t)((row >> 3) * 1024 + (row & 7) * 128);
#pragma unroll
            for (int s = 0; s < NSTEP; ++s) {
                const uint32_t off = (s >> 1) * 2048 + rbase + ((((4 * (s & 1)) + q) ^ (row & 7)) << 4);
                b[s] = *reinterpret_cast<const uint4*>(sw + off);
            }
        } else {
            const uint16_t* wrow = gu + wr * d + kl;
#pragma unroll
            for (int s = 0; s < NSTEP; ++s) b[s] = *reinterpret_cast<const uint4*>(wrow + 32 * s);
            gateup_load_x<NSTEP>(p, g, is_shared, 0, gateup_row_pair(p, g, row), xv, kl, a0);
        }
        gateup_mfma_tile<NSTEP>(p, g, 0, a0, b, j0, s_part, s_h);
    } else {
        const uint16_t* wrow = gu + wr * d + kl;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) b[s] = *reinterpret_cast<const uint4*>(wrow + 32 * s);
        uint4 a0[NSTEP];
        gateup_load_x<NSTEP>(p, g, is_shared, 0, gateup_row_pair(p, g, row), xv, kl, a0);
        gateup_mfma_tile<NSTEP>(p, g, 0, a0, b, j0, s_part, s_h);
    }
    for (int r0 = 16; r0 < g.z; r0 += 16) {
        const int m = r0 + row;
        const int spn = p.ws.sorted_pair[g.y + (m < g.z ? m : g.z - 1)];
        uint4 a[NSTEP];
        gateup_load_x<NSTEP>(p, g, is_shared, r0, spn, xv, kl, a);
        gateup_mfma_tile<NSTEP>(p, g, r0, a, b, j0, s_part, s_h);
    }
}

// One 16-token tile of a bf16 down block; ws is the routing weight of the
// token row this thread stores.  h arrives as its three bf16 planes; padding
// rows read as zeros.
// COH: h was written by other workgroups of the same launch (agent-scope loads).
template <int NSMAX, int NT, bool COH = false>
__device__ __forceinline__ void down_mfma_tile(const ExpertParams& p, const int4& g, int r0, int nsteps, int kl,
                                               int n0, const __amdgpu_buffer_rsrc_t (&hv)[3],
                                               const uint4 (&b)[NT][NSMAX], float ws, float (&s_part)[4][NT][256],
                                               float* ybase, bool handoff) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int m = r0 + row;
    const uint32_t ho = m < g.z ? (uint32_t)(m * p.hstride + kl) * 2 : kOffNone;
    uint4 ah[3][NSMAX];
#pragma unroll
    for (int s = 0; s < NSMAX; ++s)
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
            ah[pl][s] = COH ? buffer_load16_agent(hv[pl], ho + 64 * s) : buffer_load16(hv[pl], ho + 64 * s);
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first MFMA
    floatx4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSMAX; ++s) {
        if (s >= nsteps) break;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            acc[t] = mfma16x16x32(ah[0][s], b[t][s], acc[t]);
            acc[t] = mfma16x16x32(ah[1][s], b[t][s], acc[t]);
            acc[t] = mfma16x16x32(ah[2][s], b[t][s], acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_part[wave][t][(4 * q + i) * 16 + row] = acc[t][i];
    __syncthreads();
    const int mm = tid >> 4, n = tid & 15;
    if (r0 + mm < g.z) {
        float* yr = ybase + (size_t)(g.w + r0 + mm) * p.dm.d + n0 + n;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float v = ((s_part[0][t][tid] + s_part[1][t][tid]) + s_part[2][t][tid]) + s_part[3][t][tid];
            if (handoff)
                st_agent(yr + 16 * t, ws * v);  // read by another workgroup of this launch
            else
                yr[16 * t] = ws * v;
        }
    }
    __syncthreads();
}

// The combine of output columns n0 .. n0 + 16 NT - 1 for every token, by the
// last down workgroup of those columns (the y rows of every group are written
// through at agent scope and read the same way): out = residual + shared row +
// routed rows in pair order, the order of combine_kernel.  Every load of a
// thread is issued before the first add (addresses clamped to valid rows, the
// unused terms selected away), so the tail costs two memory round trips.
// kPer elements per thread cover T x 16 NT outputs.
constexpr int kDownCombineMaxT = 8;
template <int NT, int kPer>
__device__ __forceinline__ void combine_columns_n(const ExpertParams& p, int n0, const int* s_pos) {
    constexpr int nc = 16 * NT;
    const int T = p.dm.T, d = p.dm.d, k = p.dm.k;
    const float* y = static_cast<const float*>(p.ws.y);
    const size_t kT = (size_t)k * T;
    const bool has_shared = p.dm.fs > 0;
    float v[kPer][kCombineMaxK + 2];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = threadIdx.x + 256 * r;
        const int t = min(i / nc, T - 1), c = n0 + i % nc;
        v[r][0] = p.residual ? p.residual[(size_t)t * d + c] : 0.f;
        v[r][1] = has_shared ? ld_agent(y + (kT + t) * d + c) : 0.f;
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j)
            v[r][2 + j] = ld_agent(y + (size_t)s_pos[t * k + (j < k ? j : 0)] * d + c);
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int i = threadIdx.x + 256 * r;
        const int t = i / nc, c = n0 + i % nc;
        if (t >= T) continue;
        float acc = v[r][0];
        if (has_shared) acc += v[r][1];
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j)
            if (j < k) acc += v[r][2 + j];
        if (p.out_f32)
            static_cast<float*>(p.out)[(size_t)t * d + c] = acc;
        else
            static_cast<uint16_t*>(p.out)[(size_t)t * d + c] = f32_to_bf16(acc);
    }
}
template <int NT>
__device__ __forceinline__ void combine_columns(const ExpertParams& p, int n0) {
    static_assert(kDownCombineMaxT * 16 * NT <= 4 * 256, "at most four elements per thread");
    __shared__ int s_pos[kDownCombineMaxT * kCombineMaxK];
    for (int i = threadIdx.x; i < p.dm.T * p.dm.k; i += blockDim.x) s_pos[i] = p.ws.pair_pos[i];
    __syncthreads();
    const int n = p.dm.T * 16 * NT;  // uniform
    if (n <= 256) combine_columns_n<NT, 1>(p, n0, s_pos);
    else if (n <= 512) combine_columns_n<NT, 2>(p, n0, s_pos);
    else combine_columns_n<NT, 4>(p, n0, s_pos);
}

// down: block = (group, NT tiles of 16 output rows, K chunk); K = F (or its
// chunk) split over the waves, NSMAX >= chunk / 128 k steps per wave.  Groups
// wider than kDownKChunk split K into chunks of that width: each chunk writes
// its weighted partial rows to Workspace::part, and the last chunk of the
// (group, rows) pair to arrive sums them in chunk order into y.  h enters the MFMA exactly as the
// three bf16 planes (hi + mid + lo of the fp32 value) written by the gate/up
// kernel, the weights exactly, so the only rounding is the fp32 accumulation.  Load order and the peeled first
// token tile as in gateup_mfma_kernel.
constexpr int kDownMfmaTiles = 4;  // 64 output rows per block

// Down weights through LDS (groups 512 wide, 64 output rows: a wave's k slice
// is 128 wide, 256 bytes per row).  Waves 0..2 fetch their 64 rows x 256 bytes
// with direct-to-LDS loads of whole lines carrying the non-temporal hint (four
// rows per load; the 16 chunks of a row are XOR-swizzled by row, so the
// fragment reads are free of bank conflicts); wave 3 loads its own straight
// into registers (64 bytes per row and instruction).  A staging wave's partial
// sums then reuse its own region (its weights are in registers by then), so a
// workgroup holds 3 x 16 + 4 KiB of LDS and three fit in a CU, as with the
// registers-only form.
constexpr int kDownLdsWaves = 3;
constexpr int kDownLdsRegion = 64 * 256;  // bytes per staging wave
constexpr int kDownLdsBytes = kDownLdsWaves * kDownLdsRegion + 4 * 4 * 256;  // + wave 3's partial sums
__device__ __forceinline__ float* down_lds_part(unsigned char* s_lds, int w) {
    return reinterpret_cast<float*>(s_lds + (w < kDownLdsWaves ? w * kDownLdsRegion : kDownLdsWaves * kDownLdsRegion));
}

// One 16-token tile of the LDS form (NSMAX = 4, NT = 4); the first tile reads
// a staging wave's weights from LDS after its h loads are issued.
__device__ __forceinline__ void down_mfma_tile_lds(const ExpertParams& p, const int4& g, int r0, int kl, int n0,
                                                   const __amdgpu_buffer_rsrc_t (&hv)[3], uint4 (&b)[4][4], float ws,
                                                   unsigned char* s_lds, float* ybase, bool handoff, bool first) {
    constexpr int NT = 4, NSMAX = 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int m = r0 + row;
    const uint32_t ho = m < g.z ? (uint32_t)(m * p.hstride + kl) * 2 : kOffNone;
    uint4 ah[3][NSMAX];
#pragma unroll
    for (int s = 0; s < NSMAX; ++s)
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) ah[pl][s] = buffer_load16(hv[pl], ho + 64 * s);
    if (first && wave < kDownLdsWaves) {  // uniform per wave
        // the compiler waits for the direct-to-LDS loads before these reads
        const unsigned char* sw = s_lds + wave * kDownLdsRegion;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int s = 0; s < NSMAX; ++s)
                b[t][s] = *reinterpret_cast<const uint4*>(sw + (16 * t + row) * 256 + (((4 * s + q) ^ row) << 4));
    }
    __builtin_amdgcn_sched_barrier(0);
    floatx4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSMAX; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            acc[t] = mfma16x16x32(ah[0][s], b[t][s], acc[t]);
            acc[t] = mfma16x16x32(ah[1][s], b[t][s], acc[t]);
            acc[t] = mfma16x16x32(ah[2][s], b[t][s], acc[t]);
        }
    float* mine = down_lds_part(s_lds, wave);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[t * 256 + (4 * q + i) * 16 + row] = acc[t][i];
    __syncthreads();
    const int mm = tid >> 4, n = tid & 15;
    if (r0 + mm < g.z) {
        float* yr = ybase + (size_t)(g.w + r0 + mm) * p.dm.d + n0 + n;
        const float* p0 = down_lds_part(s_lds, 0);
        const float* p1 = down_lds_part(s_lds, 1);
        const float* p2 = down_lds_part(s_lds, 2);
        const float* p3 = down_lds_part(s_lds, 3);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int o = t * 256 + tid;
            const float v = ((p0[o] + p1[o]) + p2[o]) + p3[o];
            if (handoff)
                st_agent(yr + 16 * t, ws * v);  // read by another workgroup of this launch
            else
                yr[16 * t] = ws * v;
        }
    }
    __syncthreads();
}

// LDS: the routed and shared experts are both 128 NSMAX = 512 wide and NT = 4
// (the LDS form above); otherwise every wave loads its weights into registers.
template <int NSMAX, int NT, bool LDS = false>
__global__ __launch_bounds__(256) void down_mfma_kernel(ExpertParams p) {
    constexpr bool kLds = LDS;  // weights of waves 0..2 through LDS
    static_assert(!LDS || (NSMAX == 4 && NT == 4), "the LDS form holds 64 rows x 512");
    __shared__ __attribute__((aligned(16))) unsigned char s_lds[kLds ? kDownLdsBytes : 4 * NT * 256 * 4];
    float(&s_part)[4][NT][256] = *reinterpret_cast<float(*)[4][NT][256]>(s_lds);  // registers-only form
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const int rblocks = d / (16 * NT);
    const int per_g = rblocks * p.kchunks;
    const int gi = blockIdx.x / per_g, rb = blockIdx.x % rblocks, kc = (blockIdx.x % per_g) / rblocks;
    if (gi >= *p.ws.n_groups) return;
    const int4 g = p.ws.groups[gi];
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int kcg = F > kDownKChunk ? F / kDownKChunk : 1;  // this group's K chunks
    if (kc >= kcg) return;
    const int mm = tid >> 4;
    const float rw_load = p.ws.sorted_wt[g.y + (mm < g.z ? mm : g.z - 1)];
    __builtin_amdgcn_sched_barrier(0);
    const int Fc = F / kcg;
    const int nsteps = Fc / 128;
    const int kl = kc * Fc + wave * (Fc / 4) + 8 * q;
    const bool split = kcg > 1;
    float* ybase = split ? p.ws.part + (size_t)kc * kSplitRowsMax * d : static_cast<float*>(p.ws.y);
    const bool handoff = split || p.combine;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const uint16_t* dn = static_cast<const uint16_t*>(is_shared ? p.shared.dn : p.routed.dn);
    const int n0 = rb * 16 * NT;
    uint4 b[NT][NSMAX];
    const bool staged = kLds && wave < kDownLdsWaves;  // uniform per wave
    if (staged) {
        // load i: rows 4 i + (lane >> 4) of the block, 16-byte position lane & 15
        // of the row holding chunk (lane & 15) ^ (row & 15) of the wave's k slice
        unsigned char* sw = s_lds + wave * kDownLdsRegion;
        const int kw = kc * Fc + wave * (Fc / 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int c = (lane & 15) ^ (r & 15);
            __builtin_amdgcn_global_load_lds(dn + (e * d + (size_t)(n0 + r)) * F + kw + 8 * c, sw + i * 1024, 16, 0,
                                             2);
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint16_t* drow = dn + (e * d + (size_t)(n0 + 16 * t + row)) * F + kl;
#pragma unroll
            for (int s = 0; s < NSMAX; ++s) {
                const int sc = s < nsteps ? s : 0;  // clamped: steps past nsteps are loaded but unused
                b[t][s] = *reinterpret_cast<const uint4*>(drow + 32 * sc);
            }
        }
    }
    const uint16_t* h16 = static_cast<const uint16_t*>(p.ws.h);
    const size_t plane = (size_t)(p.dm.k + 1) * p.dm.T * p.hstride;
    const uint32_t vbytes = (uint32_t)g.z * p.hstride * 2;
    __amdgpu_buffer_rsrc_t hv[3];
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) hv[pl] = buffer_view(h16 + pl * plane + (size_t)g.w * p.hstride, vbytes);
    if constexpr (kLds) {
        down_mfma_tile_lds(p, g, 0, kl, n0, hv, b, is_shared ? 1.f : rw_load, s_lds, ybase, handoff, true);
        for (int r0 = 16; r0 < g.z; r0 += 16) {
            const int m = r0 + mm;
            const float rw = is_shared ? 1.f : p.ws.sorted_wt[g.y + (m < g.z ? m : g.z - 1)];
            down_mfma_tile_lds(p, g, r0, kl, n0, hv, b, rw, s_lds, ybase, handoff, false);
        }
    } else {
        down_mfma_tile<NSMAX, NT>(p, g, 0, nsteps, kl, n0, hv, b, is_shared ? 1.f : rw_load, s_part, ybase,
                                  handoff);
        for (int r0 = 16; r0 < g.z; r0 += 16) {
            const int m = r0 + mm;
            const float rw = is_shared ? 1.f : p.ws.sorted_wt[g.y + (m < g.z ? m : g.z - 1)];
            down_mfma_tile<NSMAX, NT>(p, g, r0, nsteps, kl, n0, hv, b, rw, s_part, ybase, handoff);
        }
    }
    if (split) {  // uniform: the last chunk of (group, rows) sums the partials in chunk order
        __shared__ int s_kflag;
        if (!last_arrival(&p.ws.kcount[gi * rblocks + rb], kcg, &s_kflag)) return;
        float* y = static_cast<float*>(p.ws.y);
        for (int i = tid; i < g.z * 16 * NT; i += blockDim.x) {
            const size_t o = (size_t)(g.w + i / (16 * NT)) * d + n0 + i % (16 * NT);
            float v = ld_agent(p.ws.part + o);
            for (int c = 1; c < kcg; ++c) v += ld_agent(p.ws.part + (size_t)c * kSplitRowsMax * d + o);
            if (p.combine)
                st_agent(y + o, v);
            else
                y[o] = v;
        }
    }
    if (p.combine) {  // uniform
        // one workgroup per active group arrives for these columns; the last one combines
        __shared__ int s_flag;
        if (last_arrival(&p.ws.dcount[rb], *p.ws.n_groups, &s_flag)) combine_columns<NT>(p, n0);
    }
}

// ---------------------------------------------------------------------------
// NVFP4 on the matrix cores, in f16.  A weight is E2M1 x E4M3 (at most 6
// significant bits, within 2^-10 .. 2688 in magnitude), so it is exact in f16:
// the hardware convert of a pair of codes applies the power-of-two part of the
// block scale exactly, and one packed f16 multiply applies its 3-bit mantissa
// (1 VALU per weight).  Activations enter as f16 scaled by a power of two per
// token and wave k range (see x_tile_to_f16; exact for every value above the
// f16 normal range's floor), the hidden state h as two f16 parts (hi + lo, 22
// significant bits).  The tensor scale and the power-of-two factors multiply
// the fp32 sums.
//
// Lane quarter q of a 128-wide k group holds elements 32 q .. 32 q + 31, eight
// per MFMA step: the same permutation of k for activations and weights, which
// leaves every dot product unchanged.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;

__device__ __forceinline__ floatx4_t mfma16x16x32_f16(uint4 a, uint4 b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
}
__device__ __forceinline__ uint32_t u4_word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// An E4M3 block scale split into its power-of-two part (fp32, for the
// convert's scale operand) and its mantissa in [1, 2) (f16 pair).
struct Fp4Scale {
    float p2;
    half2_t m;
};
__device__ __forceinline__ Fp4Scale fp4_scale(float s) {
    const uint32_t b = __float_as_uint(s);
    const float m = __uint_as_float((b & 0x007FFFFFu) | 0x3F800000u);
    const _Float16 mh = (_Float16)m;  // exact: at most 3 fraction bits
    return Fp4Scale{__uint_as_float(b & 0xFF800000u), half2_t{mh, mh}};
}

#define FLINT_FP4_F16_PAIR(w, B, sc)                                                               \
    ({                                                                                              \
        const half2_t v_ = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w), (sc).p2, B) * (sc).m;      \
        __builtin_bit_cast(uint32_t, v_);                                                           \
    })
// Eight E2M1 codes (one word, even element in the low nibble) times their
// block scale, as one f16 MFMA operand.
__device__ __forceinline__ uint4 fp4x8_to_f16(uint32_t w, Fp4Scale sc) {
    return make_uint4(FLINT_FP4_F16_PAIR(w, 0, sc), FLINT_FP4_F16_PAIR(w, 1, sc), FLINT_FP4_F16_PAIR(w, 2, sc),
                      FLINT_FP4_F16_PAIR(w, 3, sc));
}
#undef FLINT_FP4_F16_PAIR

constexpr int kGateupFp4FeatureTiles = 2;  // 16-feature tile pairs per gate/up block
// LDS row stride of a gate/up block's staged E4M3 scales: d / 16 bytes, plus
// 16 so that the 16 rows read by one instruction fall in different banks.
template <int NG, int NW>
constexpr int kFp4ScRow = 8 * NG * NW + 16;
// LDS row stride of a down block's staged scales: at most F / 16 = 32 NGMAX
// bytes, plus 16 (banks, as for gate/up)
template <int NGMAX>
constexpr int kFp4DownScRow = 32 * NGMAX + 16;
constexpr int kFp4DownKChunk = 2048;  // K held by one NVFP4 down block (NGMAX = 4)

// h of the NVFP4 path: two f16 planes (hi, lo) of (k+1) T rows each, holding
// h * 2^-8 (headroom above the f16 range for large activations).
constexpr float kHScale = 1.0f / 256.0f;

// Activations to f16 inside the NVFP4 gate/up kernel.  The four lanes of a
// token row in one wave (lanes row + 16 q) hold that token's whole k range of
// the wave (its d / NW activations); their largest magnitude sets a power of
// two 2^-e that brings it into [2^14, 2^15), the bf16 values are scaled by it
// (exact) and rounded to f16, and the wave's fp32 partial sums for that token
// are multiplied back by 2^e (exact) before the waves' sums are added.
template <int NG>
__device__ __forceinline__ float x_tile_to_f16(uint4 (&a)[NG][4]) {
    // largest |x| of this lane's values, as bf16 bits (two 16-bit lanes at a time)
    typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;
    u16x2_t m2 = {0, 0};
#pragma unroll
    for (int gg = 0; gg < NG; ++gg)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint32_t w[4] = {a[gg][st].x, a[gg][st].y, a[gg][st].z, a[gg][st].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
        }
    uint32_t mx = m2.x > m2.y ? m2.x : m2.y;
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
    // biased exponent E of the maximum: scale 2^(141 - E) puts it in [2^14, 2^15),
    // limited to 2^127 for tiny rows and to 1 for rows of zeros or past the group
    const int E = (int)(mx >> 7);
    int sb = mx == 0 ? 127 : 268 - E;  // biased exponent of the scale
    sb = sb < 1 ? 1 : (sb > 254 ? 254 : sb);
    const float sc = __uint_as_float((uint32_t)sb << 23);
#pragma unroll
    for (int gg = 0; gg < NG; ++gg)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint32_t w[4] = {a[gg][st].x, a[gg][st].y, a[gg][st].z, a[gg][st].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2_t h = {(_Float16)(__uint_as_float(w[i] << 16) * sc),
                                   (_Float16)(__uint_as_float(w[i] & 0xFFFF0000u) * sc)};
                w[i] = __builtin_bit_cast(uint32_t, h);
            }
            a[gg][st] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    return __uint_as_float((uint32_t)(254 - sb) << 23);  // 1 / sc, exact
}

// One 16-token tile of an NVFP4 gate/up block (see gateup_fp4_kernel).  sp is
// the sorted pair of this lane's token row.
template <int NG, int NW, int FT, bool COH = false>
__device__ __forceinline__ void gateup_fp4_tile(const ExpertParams& p, const int4& g, bool is_shared, int r0,
                                                int sp, __amdgpu_buffer_rsrc_t xv, int kl, uint4 (&cw)[2 * FT][NG],
                                                const uint8_t* s_sc, bool first, uint4* sc_dst, const uint4& sc_val,
                                                float tsg, float tsu, int j0, float (&s_part)[NW][2 * FT][256]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const int m = r0 + row;
    const int tok = is_shared ? m : sp / p.dm.k;
    const uint32_t xo = m < g.z ? (uint32_t)(tok * d + kl) * 2 : kOffNone;
    uint4 a[NG][4];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg)
#pragma unroll
        for (int st = 0; st < 4; ++st) a[gg][st] = buffer_load16(xv, xo + (128 * gg + 8 * st) * 2);
    __builtin_amdgcn_sched_barrier(0);
    // first tile (uniform): the block's scales, loaded before the codes, go to
    // LDS once every load of the tile is in flight (sc_dst is null for threads
    // past the last chunk)
    if (first) {
        if (sc_dst != nullptr) *sc_dst = sc_val;
        __syncthreads();
    }
    // Decode the weights here, after the activation loads are issued: an empty
    // asm that claims to change the codes keeps the decode from being hoisted
    // ahead of those loads or out of the token loop (where its f16 operands
    // would cost 32 NG more registers per tile than the packed codes).
#pragma unroll
    for (int t = 0; t < 2 * FT; ++t)
#pragma unroll
        for (int gg = 0; gg < NG; ++gg)
            asm volatile("" : "+v"(cw[t][gg].x), "+v"(cw[t][gg].y), "+v"(cw[t][gg].z), "+v"(cw[t][gg].w));
    // this lane's two block scales per k group: row (16 t + row), k = kl + 128 gg
    uint16_t sw[2 * FT][NG];
#pragma unroll
    for (int t = 0; t < 2 * FT; ++t)
#pragma unroll
        for (int gg = 0; gg < NG; ++gg)
            sw[t][gg] = *reinterpret_cast<const uint16_t*>(s_sc + (16 * t + row) * kFp4ScRow<NG, NW> +
                                                          kl / 16 + 8 * gg);
    const float xinv = x_tile_to_f16<NG>(a);  // 2^e of this lane's token row
    floatx4_t acc[2 * FT];
#pragma unroll
    for (int t = 0; t < 2 * FT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
#pragma unroll
        for (int t = 0; t < 2 * FT; ++t) {
            const Fp4Scale s0 = fp4_scale(__builtin_amdgcn_cvt_f32_fp8(sw[t][gg], 0));
            const Fp4Scale s1 = fp4_scale(__builtin_amdgcn_cvt_f32_fp8(sw[t][gg], 1));
#pragma unroll
            for (int st = 0; st < 4; ++st)
                acc[t] = mfma16x16x32_f16(a[gg][st], fp4x8_to_f16(u4_word(cw[t][gg], st), st < 2 ? s0 : s1), acc[t]);
        }
    }
    // acc[t][i] belongs to token row 4 q + i, whose scale lane 4 q + i holds
    float xr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = __shfl(xinv, 4 * q + i, 64);
#pragma unroll
    for (int t = 0; t < 2 * FT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_part[wave][t][(4 * q + i) * 16 + row] = acc[t][i] * xr[i];
    __syncthreads();
    // thread -> (feature tile ft, token row mm, feature n); tiles ft (gate) and FT + ft (up)
    for (int idx = tid; idx < 256 * FT; idx += 64 * NW) {
        const int ft = idx >> 8, mm = (idx >> 4) & 15, n = idx & 15, o = idx & 255;
        if (r0 + mm >= g.z) continue;
        float gs = s_part[0][ft][o], us = s_part[0][FT + ft][o];
#pragma unroll
        for (int w = 1; w < NW; ++w) {  // fixed order
            gs += s_part[w][ft][o];
            us += s_part[w][FT + ft][o];
        }
        const float hv = silu_f32(tsg * gs) * (tsu * us) * kHScale;
        const _Float16 hi = (_Float16)hv;
        const _Float16 lo = (_Float16)(hv - (float)hi);
        uint16_t* h16 = static_cast<uint16_t*>(p.ws.h);
        const size_t plane = (size_t)(p.dm.k + 1) * p.dm.T * p.hstride;
        const size_t off = (size_t)(g.w + r0 + mm) * p.hstride + j0 + 16 * ft + n;
        if (COH) {  // read by other workgroups of this launch: agent-scope stores
            const __amdgpu_buffer_rsrc_t hv2 = buffer_view(h16, (uint32_t)(2 * plane * 2));
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, hi), hv2, (int)(off * 2), 0, kCpolAgent);
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, lo), hv2, (int)((plane + off) * 2), 0,
                                                  kCpolAgent);
        } else {
            h16[off] = __builtin_bit_cast(uint16_t, hi);
            h16[plane + off] = __builtin_bit_cast(uint16_t, lo);
        }
    }
    __syncthreads();
}

// gate/up + SwiGLU, NVFP4 weights: block = (group, 16 FT features): MFMA tiles
// 0..FT-1 hold their gate rows and tiles FT..2FT-1 their up rows, so the two
// results of one feature land in the same lane.  K is split over the NW waves,
// NG groups of 128 per wave (d = 128 NG NW).  The first token tile is peeled
// off the loop so that the weights and its activations are all in flight
// before the first wait.
template <int NG, int NW, int FT>
__global__ __launch_bounds__(64 * NW) void gateup_fp4_kernel(ExpertParams p) {
    __shared__ float s_part[NW][2 * FT][256];
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[2 * FT * 16 * kFp4ScRow<NG, NW>];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const int fblocks = p.hstride / (16 * FT);
    const int gi = blockIdx.x / fblocks, fb = blockIdx.x % fblocks;
    if (gi >= *p.ws.n_groups) return;
    const int4 g = p.ws.groups[gi];
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int j0 = fb * 16 * FT;
    if (j0 >= F) return;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const int kl = wave * (d / NW) + 32 * q;  // this lane's first element in each group
    // The token index is requested before the weights: vector loads retire in
    // order, so the activation loads that need it wait for it alone.
    const int sp = p.ws.sorted_pair[g.y + (row < g.z ? row : g.z - 1)];
    __builtin_amdgcn_sched_barrier(0);
    // The block's scales (2 FT x 16 rows of d / 16 bytes) in 16-byte chunks,
    // one per thread, coalesced; threads past the last chunk repeat it.
    constexpr int kCpr = NG * NW / 2;  // chunks per row
    constexpr int kChunks = 2 * FT * 16 * kCpr;
    static_assert(kChunks <= 64 * NW, "one scale chunk per thread");
    const int sc_c = tid < kChunks ? tid : kChunks - 1;
    const int sc_r = sc_c / kCpr, sc_cc = sc_c % kCpr, sc_t = sc_r >> 4;
    const size_t sc_wr = e * 2 * F + (size_t)(sc_t >= FT ? F : 0) + j0 + 16 * (sc_t % FT) + (sc_r & 15);
    const uint4 sc_val = *reinterpret_cast<const uint4*>(wp.gus + sc_wr * (d / 16) + 16 * sc_cc);
    uint4* sc_dst = reinterpret_cast<uint4*>(s_sc + sc_r * kFp4ScRow<NG, NW> + 16 * sc_cc);
    uint4 cw[2 * FT][NG];
#pragma unroll
    for (int t = 0; t < 2 * FT; ++t) {
        const size_t wr = e * 2 * F + (size_t)(t >= FT ? F : 0) + j0 + 16 * (t % FT) + row;
        const uint8_t* crow = static_cast<const uint8_t*>(wp.gu) + wr * (d / 2) + kl / 2;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) cw[t][gg] = *reinterpret_cast<const uint4*>(crow + 64 * gg);
    }
    const float tsg = wp.ts[e * 3 + 0], tsu = wp.ts[e * 3 + 1];
    const __amdgpu_buffer_rsrc_t xv = buffer_view(p.x, (uint32_t)p.dm.T * d * 2);
    gateup_fp4_tile<NG, NW, FT>(p, g, is_shared, 0, sp, xv, kl, cw, s_sc, true, tid < kChunks ? sc_dst : nullptr,
                                sc_val, tsg, tsu, j0, s_part);
    for (int r0 = 16; r0 < g.z; r0 += 16) {
        const int m = r0 + row;
        const int spn = p.ws.sorted_pair[g.y + (m < g.z ? m : g.z - 1)];
        gateup_fp4_tile<NG, NW, FT>(p, g, is_shared, r0, spn, xv, kl, cw, s_sc, false, nullptr, sc_val, tsg, tsu, j0,
                                    s_part);
    }
}

// One 16-token tile of an NVFP4 down block (see down_fp4_kernel); ws is the
// routing weight of the token row this thread stores, times the tensor scale
// and the inverse of the h scale.
template <int NT, int NGMAX, bool COH = false>
__device__ __forceinline__ void down_fp4_tile(const ExpertParams& p, const int4& g, int r0, int ng, int kl, int kls,
                                              int n0,
                                              __amdgpu_buffer_rsrc_t hv_hi, __amdgpu_buffer_rsrc_t hv_lo,
                                              uint4 (&cw)[NT][NGMAX], uint8_t* s_sc, bool first, int sc_o0,
                                              int sc_o1, u32x4_t sc_v0, u32x4_t sc_v1, float ws,
                                              float (&s_part)[4][NT][256], float* ybase, bool handoff) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int m = r0 + row;
    const uint32_t ho = m < g.z ? (uint32_t)(m * p.hstride + kl) * 2 : kOffNone;
    floatx4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < NGMAX; ++gg) {
        if (gg >= ng) break;
        uint4 hhi[4], hlo[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            // (h written by other workgroups of this launch: agent-scope loads)
            hhi[st] = COH ? buffer_load16_agent(hv_hi, ho + (128 * gg + 8 * st) * 2)
                          : buffer_load16(hv_hi, ho + (128 * gg + 8 * st) * 2);
            hlo[st] = COH ? buffer_load16_agent(hv_lo, ho + (128 * gg + 8 * st) * 2)
                          : buffer_load16(hv_lo, ho + (128 * gg + 8 * st) * 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        // first tile (uniform): the block's scales go to LDS once the first h
        // loads are in flight (see gateup_fp4_tile)
        if (first && gg == 0) {
            if (sc_o0 >= 0) *reinterpret_cast<u32x4_t*>(s_sc + sc_o0) = sc_v0;
            if (sc_o1 >= 0) *reinterpret_cast<u32x4_t*>(s_sc + sc_o1) = sc_v1;
            __syncthreads();
        }
        // decode after the h loads are issued, and inside the token loop
        // (see gateup_fp4_tile)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            asm volatile("" : "+v"(cw[t][gg].x), "+v"(cw[t][gg].y), "+v"(cw[t][gg].z), "+v"(cw[t][gg].w));
        Fp4Scale sc[NT][2];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint16_t sw = *reinterpret_cast<const uint16_t*>(s_sc + (16 * t + row) * kFp4DownScRow<NGMAX> +
                                                                  kls / 16 + 8 * gg);
            sc[t][0] = fp4_scale(__builtin_amdgcn_cvt_f32_fp8(sw, 0));
            sc[t][1] = fp4_scale(__builtin_amdgcn_cvt_f32_fp8(sw, 1));
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint4 bw = fp4x8_to_f16(u4_word(cw[t][gg], st), sc[t][st >> 1]);
                acc[t] = mfma16x16x32_f16(hhi[st], bw, acc[t]);
                acc[t] = mfma16x16x32_f16(hlo[st], bw, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_part[wave][t][(4 * q + i) * 16 + row] = acc[t][i];
    __syncthreads();
    const int mm = tid >> 4, n = tid & 15;
    if (r0 + mm < g.z) {
        float* yr = ybase + (size_t)(g.w + r0 + mm) * p.dm.d + n0 + n;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float v = ((s_part[0][t][tid] + s_part[1][t][tid]) + s_part[2][t][tid]) + s_part[3][t][tid];
            if (handoff)
                st_agent(yr + 16 * t, ws * v);  // read by another workgroup of this launch
            else
                yr[16 * t] = ws * v;
        }
    }
    __syncthreads();
}

// down, NVFP4 weights: block = (group, 16 NT output rows), K = F split over
// the 4 waves in groups of 128; h enters as its two f16 parts (two MFMAs per
// step).  First token tile peeled as in gateup_fp4_kernel.
constexpr int kDownFp4Tiles = 4;  // 64 output rows per block

template <int NT, int NGMAX>
__global__ __launch_bounds__(256) void down_fp4_kernel(ExpertParams p) {
    __shared__ float s_part[4][NT][256];
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[16 * NT * kFp4DownScRow<NGMAX>];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const int rblocks = d / (16 * NT);
    const int per_g = rblocks * p.kchunks;
    const int gi = blockIdx.x / per_g, rb = blockIdx.x % rblocks, kc = (blockIdx.x % per_g) / rblocks;
    if (gi >= *p.ws.n_groups) return;
    const int4 g = p.ws.groups[gi];
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    // groups wider than kFp4DownKChunk split K as down_mfma_kernel does
    const int kcg = F > kFp4DownKChunk ? F / kFp4DownKChunk : 1;
    if (kc >= kcg) return;
    // routing weight of the row this thread stores in the first token tile
    const int mm = tid >> 4;
    const float rw_load = p.ws.sorted_wt[g.y + (mm < g.z ? mm : g.z - 1)];
    const int Fc = F / kcg;                            // this chunk's K
    const int ng = Fc / 512;
    const int kls = wave * (Fc / 4) + 32 * q;          // within the chunk (scales in LDS)
    const int kl = kc * Fc + kls;                      // within the row (codes, h)
    const bool split = kcg > 1;
    float* ybase = split ? p.ws.part + (size_t)kc * kSplitRowsMax * d : static_cast<float*>(p.ws.y);
    const bool handoff = split || p.combine;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const int n0 = rb * 16 * NT;
    // The block's scales (16 NT rows of F / 16 bytes) in 16-byte chunks, at
    // most two per thread, coalesced; chunks past the last repeat it.
    static_assert(16 * NT * 2 * NGMAX <= 2 * 256, "two scale chunks per thread");
    const int cpr = Fc / 256, nchunks = 16 * NT * cpr;
    auto sc_chunk = [&](int ci, u32x4_t& v) {  // LDS offset of chunk ci, or -1 past the last
        const int cc = ci < nchunks ? ci : nchunks - 1;
        const int r = cc / cpr, col = cc % cpr;
        const size_t wr = e * (size_t)d + (size_t)(n0 + r);
        v = *reinterpret_cast<const u32x4_t*>(wp.dns + wr * (F / 16) + kc * (Fc / 16) + 16 * col);
        return ci < nchunks ? r * kFp4DownScRow<NGMAX> + 16 * col : -1;
    };
    u32x4_t sc_v0, sc_v1;
    const int sc_o0 = sc_chunk(tid, sc_v0), sc_o1 = sc_chunk(tid + 256, sc_v1);
    uint4 cw[NT][NGMAX];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const size_t wr = e * (size_t)d + (size_t)(n0 + 16 * t + row);
        const uint8_t* crow = static_cast<const uint8_t*>(wp.dn) + wr * (F / 2) + kl / 2;
#pragma unroll
        for (int gg = 0; gg < NGMAX; ++gg) {
            const int gc = gg < ng ? gg : 0;  // clamped: groups past ng are loaded but unused
            cw[t][gg] = *reinterpret_cast<const uint4*>(crow + 64 * gc);
        }
    }
    const float tsd = wp.ts[e * 3 + 2] / kHScale;
    const float rw0 = is_shared ? 1.f : rw_load;
    const uint16_t* h16 = static_cast<const uint16_t*>(p.ws.h);
    const size_t plane = (size_t)(p.dm.k + 1) * p.dm.T * p.hstride;
    const uint32_t vbytes = (uint32_t)g.z * p.hstride * 2;
    const __amdgpu_buffer_rsrc_t hv_hi = buffer_view(h16 + (size_t)g.w * p.hstride, vbytes);
    const __amdgpu_buffer_rsrc_t hv_lo = buffer_view(h16 + plane + (size_t)g.w * p.hstride, vbytes);
    down_fp4_tile<NT, NGMAX>(p, g, 0, ng, kl, kls, n0, hv_hi, hv_lo, cw, s_sc, true, sc_o0, sc_o1, sc_v0, sc_v1,
                             tsd * rw0, s_part, ybase, handoff);
    for (int r0 = 16; r0 < g.z; r0 += 16) {
        const int m = r0 + mm;
        const float rw = is_shared ? 1.f : p.ws.sorted_wt[g.y + (m < g.z ? m : g.z - 1)];
        down_fp4_tile<NT, NGMAX>(p, g, r0, ng, kl, kls, n0, hv_hi, hv_lo, cw, s_sc, false, -1, -1, sc_v0,
                                 sc_v1, tsd * rw, s_part, ybase, handoff);
    }
    if (split) {  // uniform: the last chunk of (group, rows) sums the partials in chunk order
        __shared__ int s_kflag;
        if (!last_arrival(&p.ws.kcount[gi * rblocks + rb], kcg, &s_kflag)) return;
        float* y = static_cast<float*>(p.ws.y);
        for (int i = tid; i < g.z * 16 * NT; i += blockDim.x) {
            const size_t o = (size_t)(g.w + i / (16 * NT)) * d + n0 + i % (16 * NT);
            float v = ld_agent(p.ws.part + o);
            for (int c = 1; c < kcg; ++c) v += ld_agent(p.ws.part + (size_t)c * kSplitRowsMax * d + o);
            if (p.combine)
                st_agent(y + o, v);
            else
                y[o] = v;
        }
    }
    if (p.combine) {  // uniform; as in down_mfma_kernel
        __shared__ int s_flag;
        if (last_arrival(&p.ws.dcount[rb], *p.ws.n_groups, &s_flag)) combine_columns<NT>(p, n0);
    }
}

bool decode_fp4_ok(const Dims& dm) {
    const int fmax = dm.f > dm.fs ? dm.f : dm.fs;
    const int ng = dm.d / 512;
    auto width_ok = [&](int w) { return w <= kFp4DownKChunk || w % kFp4DownKChunk == 0; };
    const bool split_ok = fmax <= kFp4DownKChunk || (size_t)(dm.k + 1) * dm.T <= (size_t)kSplitRowsMax;
    return dm.act == DT_BF16 && dm.wdt == DT_NVFP4 && dm.d % 512 == 0 &&
           (ng == 1 || ng == 2 || ng == 4) && dm.f % 512 == 0 && dm.fs % 512 == 0 && width_ok(dm.f) &&
           width_ok(dm.fs) && split_ok &&
           (size_t)dm.T * dm.d * 2 < kOffNone && (size_t)dm.T * fmax * 4 < kOffNone;
}

bool decode_mfma_ok(const Dims& dm) {
    const int fmax = dm.f > dm.fs ? dm.f : dm.fs;
    const int ns = dm.d / 128;
    // widths above kDownKChunk split K in the down kernel: whole chunks, and a
    // partial-sum buffer that holds every (token, slot) row
    auto width_ok = [&](int w) { return w <= kDownKChunk || w % kDownKChunk == 0; };
    const bool split_ok = fmax <= kDownKChunk || (size_t)(dm.k + 1) * dm.T <= (size_t)kSplitRowsMax;
    return dm.act == DT_BF16 && dm.wdt == DT_BF16 && dm.d % 128 == 0 &&
           (ns == 1 || ns == 2 || ns == 4 || ns == 8 || ns == 16) && dm.f % 128 == 0 &&
           dm.fs % 128 == 0 && width_ok(dm.f) && width_ok(dm.fs) && split_ok && dm.d % 32 == 0 &&
           (size_t)dm.T * dm.d * 2 < kOffNone && (size_t)dm.T * fmax * 4 < kOffNone;
}

static int max_groups(const Dims& dm) {
    const int routed = dm.k * dm.T < dm.E ? dm.k * dm.T : dm.E;
    return routed + (dm.fs > 0 ? 1 : 0);
}

static ExpertParams make_params(const LayerArgs& a, const Workspace& w) {
    ExpertParams p;
    p.dm = a.dm;
    p.x = a.x;
    p.routed = a.routed;
    p.shared = a.shared;
    p.ws = w;
    p.hstride = a.dm.f > a.dm.fs ? a.dm.f : a.dm.fs;
    p.combine = 0;
    p.residual = a.residual;
    p.out = a.out;
    p.out_f32 = (a.residual != nullptr || a.dm.act == DT_F32) ? 1 : 0;
    p.kchunks = 1;
    return p;
}

template <int TG>
static void launch_gateup_generic(const LayerArgs& a, const ExpertParams& p, dim3 grid, hipStream_t s) {
    const bool f32 = a.dm.act == DT_F32;
    switch (a.dm.wdt) {
    case DT_F32:
        if (f32) hipLaunchKernelGGL((gateup_decode_kernel<float, DT_F32, TG>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gateup_decode_kernel<uint16_t, DT_F32, TG>), grid, dim3(256), 0, s, p);
        break;
    case DT_BF16:
        if (f32) hipLaunchKernelGGL((gateup_decode_kernel<float, DT_BF16, TG>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gateup_decode_kernel<uint16_t, DT_BF16, TG>), grid, dim3(256), 0, s, p);
        break;
    default:
        if (f32) hipLaunchKernelGGL((gateup_decode_kernel<float, DT_NVFP4, TG>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gateup_decode_kernel<uint16_t, DT_NVFP4, TG>), grid, dim3(256), 0, s, p);
        break;
    }
}

hipError_t launch_gateup_decode(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    ExpertParams p = make_params(a, w);
    if (decode_fp4_ok(a.dm)) {
        // 8 waves split K; 32 features (64 weight rows) per block
        constexpr int FT = kGateupFp4FeatureTiles;
        dim3 grid(max_groups(a.dm) * (p.hstride / (16 * FT)));
        switch (a.dm.d / 1024) {
        case 0: hipLaunchKernelGGL((gateup_fp4_kernel<1, 4, FT>), grid, dim3(256), 0, s, p); break;  // d = 512
        case 1: hipLaunchKernelGGL((gateup_fp4_kernel<1, 8, FT>), grid, dim3(512), 0, s, p); break;
        default: hipLaunchKernelGGL((gateup_fp4_kernel<2, 8, FT>), grid, dim3(512), 0, s, p); break;
        }
        return hipGetLastError();
    }
    if (decode_mfma_ok(a.dm)) {
        dim3 grid(max_groups(a.dm) * (p.hstride / 8));
        switch (a.dm.d / 128) {
        case 1: hipLaunchKernelGGL(gateup_mfma_kernel<1>, grid, dim3(256), 0, s, p); break;
        case 2: hipLaunchKernelGGL(gateup_mfma_kernel<2>, grid, dim3(256), 0, s, p); break;
        case 4: hipLaunchKernelGGL(gateup_mfma_kernel<4>, grid, dim3(256), 0, s, p); break;
        case 8: hipLaunchKernelGGL(gateup_mfma_kernel<8>, grid, dim3(256), 0, s, p); break;
        default: hipLaunchKernelGGL(gateup_mfma_kernel<16>, grid, dim3(256), 0, s, p); break;
        }
        return hipGetLastError();
    }
    const int fblocks = (p.hstride + kFPB - 1) / kFPB;
    dim3 grid(max_groups(a.dm) * fblocks);
    if (tokens_per_pass(a.dm.T) == kTGWide) launch_gateup_generic<kTGWide>(a, p, grid, s);
    else launch_gateup_generic<4>(a, p, grid, s);
    return hipGetLastError();
}

// The matrix-core down kernels fold the combine in (bf16 weights up to 8
// tokens, NVFP4 up to 4): the last workgroup of each block of output columns
// sums those columns, which saves the combine launch.  Every workgroup then
// waits for its write-through stores and takes a ticket; the short NVFP4
// workgroups pay more for that at 16 tokens than the combine launch costs, and
// at 16 tokens bf16 is faster with the LDS-staged down kernel and a separate
// combine (measured).  Above these sizes the combine kernel, which spreads the
// rows over the whole chip, is as fast.
constexpr int kDownCombineMaxTFp4 = 4;
bool down_decode_combines(const Dims& dm) {
    const bool fp4 = decode_fp4_ok(dm);
    return (fp4 || decode_mfma_ok(dm)) && dm.T <= (fp4 ? kDownCombineMaxTFp4 : kDownCombineMaxT) &&
           dm.k <= kCombineMaxK;
}

hipError_t launch_down_decode(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    ExpertParams p = make_params(a, w);
    if (decode_fp4_ok(a.dm)) {
        constexpr int NT = kDownFp4Tiles;
        if (a.dm.d % (16 * NT) != 0) return hipErrorInvalidValue;
        p.combine = down_decode_combines(a.dm) ? 1 : 0;
        p.kchunks = p.hstride > kFp4DownKChunk ? p.hstride / kFp4DownKChunk : 1;
        dim3 grid(max_groups(a.dm) * (a.dm.d / (16 * NT)) * p.kchunks);
        switch (p.hstride / 512) {
        case 1: hipLaunchKernelGGL((down_fp4_kernel<NT, 1>), grid, dim3(256), 0, s, p); break;
        case 2: hipLaunchKernelGGL((down_fp4_kernel<NT, 2>), grid, dim3(256), 0, s, p); break;
        default: hipLaunchKernelGGL((down_fp4_kernel<NT, 4>), grid, dim3(256), 0, s, p); break;
        }
        return hipGetLastError();
    }
    if (decode_mfma_ok(a.dm)) {
        constexpr int NT = kDownMfmaTiles;
        p.combine = down_decode_combines(a.dm) ? 1 : 0;
        p.kchunks = p.hstride > kDownKChunk ? p.hstride / kDownKChunk : 1;
        dim3 grid(max_groups(a.dm) * (a.dm.d / (16 * NT)) * p.kchunks);
        switch ((p.hstride + 127) / 128) {
        case 1: hipLaunchKernelGGL((down_mfma_kernel<1, NT>), grid, dim3(256), 0, s, p); break;
        case 2: hipLaunchKernelGGL((down_mfma_kernel<2, NT>), grid, dim3(256), 0, s, p); break;
        case 3:
        case 4:
            // the LDS form measured faster without the folded combine (3 us at
            // T = 64) and slower with it (2 us at T = 16)
            if (a.dm.f == 512 && (a.dm.fs == 512 || a.dm.fs == 0) && NT == 4 && !p.combine)
                hipLaunchKernelGGL((down_mfma_kernel<4, NT, true>), grid, dim3(256), 0, s, p);
            else
                hipLaunchKernelGGL((down_mfma_kernel<4, NT>), grid, dim3(256), 0, s, p);
            break;
        default: hipLaunchKernelGGL((down_mfma_kernel<8, NT>), grid, dim3(256), 0, s, p); break;
        }
        return hipGetLastError();
    }
    const int rblocks = (a.dm.d + kRPB - 1) / kRPB;
    dim3 grid(max_groups(a.dm) * rblocks);
    const bool wide = tokens_per_pass(a.dm.T) == kTGWide;
    switch (a.dm.wdt) {
    case DT_F32:
        if (wide) hipLaunchKernelGGL((down_decode_kernel<DT_F32, kTGWide>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((down_decode_kernel<DT_F32, 4>), grid, dim3(256), 0, s, p);
        break;
    case DT_BF16:
        if (wide) hipLaunchKernelGGL((down_decode_kernel<DT_BF16, kTGWide>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((down_decode_kernel<DT_BF16, 4>), grid, dim3(256), 0, s, p);
        break;
    default:
        if (wide) hipLaunchKernelGGL((down_decode_kernel<DT_NVFP4, kTGWide>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((down_decode_kernel<DT_NVFP4, 4>), grid, dim3(256), 0, s, p);
        break;
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Single-launch decode for small bf16 batches (T <= kFusedMaxT).
//
// A small decode batch is bound by latency, not bytes: with one kernel per
// step (route, gate/up, down) every step pays a launch, the first HBM round
// trip and the tail of its grid.  This kernel runs the whole layer in one
// launch over a grid that is resident at once (kFusedBlocksPerCU workgroups
// per CU), with two grid-wide barriers and the last-arrival combine:
//   phase 0  workgroup e < E computes router logit e for every token (fp32
//            FMA over exact bf16 x fp32 products, a fixed reduction order);
//            the next fs / 8 workgroups run the shared expert's gate/up items
//            meanwhile (the shared expert needs no routing);
//   barrier  every router workgroup has written its logits;
//   phase 1  every workgroup selects the top-k of every token and sorts the
//            pairs itself, in LDS (at most 8 x 8 pairs), so no further
//            hand-off is needed to learn the routing; it issues the weight
//            loads of its first gate/up item as soon as the group list is
//            known; workgroup 0 publishes the routing for
//            flint_moe_get_routing;
//   phase 2  the routed gate/up items (group, 8 features), spread round-robin;
//            h leaves as its exact three-plane bf16 split at agent scope;
//   barrier  every gate/up item is done; each workgroup issues the weight
//            loads of its first down item before it waits here;
//   phase 3  the down items (group, 64 output rows): y rows at agent scope,
//            and the last item of each 64-column block sums those columns of
//            every token (residual, shared row, routed rows in pair order);
// The barriers are trees of counters taken with agent-scope atomics after each
// writer has waited for its stores (vmcnt 0), with per-group release flags
// polled by one thread per workgroup (see tree_arrive); data crosses
// workgroups only through agent-scope (sc1) stores and loads, which are served
// coherently across the XCDs' separate L2 caches.  A poll gives up after
// kFusedPollCap tries and records a fault word, so the kernel always ends even
// if a workgroup were never scheduled (the host sizes the grid from the
// occupancy query, so all of it is resident).
// ---------------------------------------------------------------------------
// Largest batch it takes: measured against the separate launches on the full
// layer (d = 2048, 256 experts, f = 512), it is 13-14% faster at T = 1 and 2,
// 5% at T = 4, even at T = 8, and slower from T = 12 (the separate gate/up and
// down launches balance their work better than the persistent grid does).
constexpr int kFusedMaxT = 8;
constexpr int kFusedBlocksPerCU = 2;
constexpr int kFusedPollCap = 1 << 20;
constexpr int kFusedMaxPairs = kFusedMaxT * kCombineMaxK;

struct FusedParams {
    ExpertParams e;    // dims, activations, weights, workspace, residual, out
    const float* wr;   // router [E][d] fp32
    const float* bias; // [E] or null
    int nblocks;       // grid size (every workgroup resident)
};

// Grid barriers as trees: an arriving workgroup adds to its group's counter
// (kBarGroup workgroups per group), the last of a group adds to the root
// counter, and the last group releases every waiting group by writing the
// launch's generation number into the group's flag; a waiting workgroup polls
// its own group's flag.  Counters and flags sit kBarSlot ints apart, so no
// line takes more than kBarGroup atomics or polls (hundreds of atomics on one
// address serialise for microseconds, and hundreds of pollers on one line
// slow the memory channel that holds it).  Every counter is reset by its own
// last arrival, and flags are never cleared: a launch waits for its own
// generation, which the release of its last barrier advances (every
// workgroup has read it by then), so no exit barrier is needed.
// Barrier ids: 0 = router logits written, 1 = h written.
constexpr int kBarGroup = 16;
constexpr int kBarMaxGroups = 64;  // grids of up to 1024 workgroups
constexpr int kBarSlot = 256;      // ints between two group slots (1 KiB)
__device__ __forceinline__ int* bar_cnt(int* fbar, int b, int g) { return fbar + (b * kBarMaxGroups + g) * kBarSlot; }
__device__ __forceinline__ int* bar_flag(int* fbar, int b, int g) { return bar_cnt(fbar, b, g) + 32; }
__device__ __forceinline__ int* bar_root(int* fbar, int b) { return fbar + (2 * kBarMaxGroups + b) * kBarSlot; }
__device__ __forceinline__ int* bar_gen(int* fbar) { return fbar + (2 * kBarMaxGroups + 2) * kBarSlot; }
__device__ __forceinline__ int* bar_fault(int* fbar) { return fbar + (2 * kBarMaxGroups + 3) * kBarSlot; }
// work counter q of the gate/up (q = XCD 0..7) and down (q = 8 + XCD) phases,
// zero when the phase starts
__device__ __forceinline__ int* bar_queue(int* fbar, int q) { return fbar + (2 * kBarMaxGroups + 4 + q) * kBarSlot; }
static_assert((2 * kBarMaxGroups + 20) * kBarSlot == kFusedBarrierInts, "barrier region size");
static_assert((2 * kBarMaxGroups + 3) * kBarSlot == kFusedFaultInt, "fault word index");

// Workgroup `id` of the n that arrive at barrier b (all threads call it).  The
// writer's stores complete before its arrival; returns true in thread 0 of
// the workgroup that arrived last overall.
__device__ __forceinline__ bool tree_arrive(int* fbar, int b, int id, int n) {
    wait_stores();
    __syncthreads();
    bool last = false;
    if (threadIdx.x == 0) {
        const int g = id / kBarGroup;
        const int gsize = min(kBarGroup, n - g * kBarGroup);
        int* cnt = bar_cnt(fbar, b, g);
        if (__hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gsize - 1) {
            st_agent(cnt, 0);  // every arrival of this launch is in
            const int ngroups = (n + kBarGroup - 1) / kBarGroup;
            int* root = bar_root(fbar, b);
            last = __hip_atomic_fetch_add(root, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1;
            if (last) st_agent(root, 0);
        }
    }
    return last;
}

// The last arrival (thread 0) releases the nwait waiting groups of generation gen.
__device__ __forceinline__ void tree_release(int* fbar, int b, int nwait, int gen) {
    for (int g = 0; g < nwait; ++g) st_agent(bar_flag(fbar, b, g), gen);
}

// Wait (all threads) until barrier b releases generation gen for workgroup
// id's group.  A poll gives up after kFusedPollCap tries and records a fault
// word, so the kernel ends even if a workgroup never arrived.
__device__ __forceinline__ void tree_wait(int* fbar, int b, int id, int gen) {
    if (threadIdx.x == 0) {
        const int* f = bar_flag(fbar, b, id / kBarGroup);
        int n = 0;
        while (ld_agent(f) != gen) {
            __builtin_amdgcn_s_sleep(2);
            if (++n >= kFusedPollCap) {
                st_agent(bar_fault(fbar), 1);
                break;
            }
        }
    }
    __syncthreads();
}

// Router logits of expert e for every token: 8 consecutive k per thread and
// pass, fp32 FMA chains, then a wavefront sum and the four waves in order.
__device__ void fused_router_expert(const FusedParams& P, int e, float (&s_red)[4][kFusedMaxT]) {
    const ExpertParams& p = P.e;
    const int T = p.dm.T, d = p.dm.d, E = p.dm.E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const __amdgpu_buffer_rsrc_t xv = buffer_view(p.x, (uint32_t)T * d * 2);
    float acc[kFusedMaxT];
#pragma unroll
    for (int t = 0; t < kFusedMaxT; ++t) acc[t] = 0.f;
    for (int c = tid * 8; c < d; c += 2048) {
        const float4 w0 = *reinterpret_cast<const float4*>(P.wr + (size_t)e * d + c);
        const float4 w1 = *reinterpret_cast<const float4*>(P.wr + (size_t)e * d + c + 4);
        uint4 xa[kFusedMaxT];
#pragma unroll
        for (int t = 0; t < kFusedMaxT; ++t) xa[t] = buffer_load16(xv, t < T ? (uint32_t)(t * d + c) * 2 : kOffNone);
#pragma unroll
        for (int t = 0; t < kFusedMaxT; ++t) {
            float a = acc[t];
            a = fmaf(w0.x, bf16_lo(xa[t].x), a);
            a = fmaf(w0.y, bf16_hi(xa[t].x), a);
            a = fmaf(w0.z, bf16_lo(xa[t].y), a);
            a = fmaf(w0.w, bf16_hi(xa[t].y), a);
            a = fmaf(w1.x, bf16_lo(xa[t].z), a);
            a = fmaf(w1.y, bf16_hi(xa[t].z), a);
            a = fmaf(w1.z, bf16_lo(xa[t].w), a);
            a = fmaf(w1.w, bf16_hi(xa[t].w), a);
            acc[t] = a;
        }
    }
#pragma unroll
    for (int t = 0; t < kFusedMaxT; ++t) {
        if (t >= T) break;  // uniform
        const float v = wave_sum(acc[t]);
        if (lane == 0) s_red[wave][t] = v;
    }
    __syncthreads();
    if (tid < T) {
        const float v = ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
        st_agent(p.ws.logits + (size_t)tid * E + e, v + (P.bias ? P.bias[e] : 0.f));
    }
}

// Top-k of every token, one wavefront per token (tokens wave, wave + 4, ...,
// topk_token_lds).  The logits come into LDS first, with one round of 16-byte
// agent-scope loads by the whole workgroup.  Results in LDS.
__device__ void fused_topk(const ExpertParams& p, float* s_logit, int* s_sel, float* s_wt) {
    const int T = p.dm.T, E = p.dm.E, k = p.dm.k;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t bytes = (uint32_t)(T * E * 4 + 15) & ~15u;  // within the 256-byte padded region
    const __amdgpu_buffer_rsrc_t lv = buffer_view(p.ws.logits, bytes);
    // every load of the (at most 16 KiB) block is issued before the first
    // store; loads past the view return zeros and are not stored
    constexpr int kChunks = kFusedMaxT * 256 * 4 / (16 * 256);
    uint4 lg[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) lg[i] = buffer_load16_agent(lv, (threadIdx.x + 256 * i) * 16);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const uint32_t o = (threadIdx.x + 256 * i) * 16;
        if (o < bytes) *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(s_logit) + o) = lg[i];
    }
    __syncthreads();
    for (int t = wave; t < T; t += 4) {
        int e;
        float w;
        topk_token_lds(s_logit + t * E, E, k, lane, &e, &w);
        if (lane < k) {
            s_sel[t * k + lane] = e;
            s_wt[t * k + lane] = w;
        }
    }
}

// Stable counting sort of the k T pairs by expert, in LDS, in two parts so
// that a workgroup can start loading the weights of its first gate/up item
// between them.  A token picks an expert at most once, so a bitmask of the
// tokens that picked each expert (s_mask, T <= 32) gives both the count (its
// population) and each pair's rank among the earlier pairs of its expert (the
// tokens below its own).
//   fused_groups: the masks, the exclusive scan of the counts (s_off) and the
//     group list (the shared expert first, then every expert with tokens,
//     ascending), from one pass of wave 0 over 4 experts per lane;
//   fused_place: the sorted pair list, its inverse and the weight of each
//     sorted pair.
__device__ void fused_groups(const ExpertParams& p, const int* s_sel, unsigned* s_mask, int* s_off, int4* s_groups,
                             int* s_ng) {
    const int T = p.dm.T, k = p.dm.k, E = p.dm.E, P = k * T;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < E; i += blockDim.x) s_mask[i] = 0u;
    __syncthreads();
    if (tid < P) atomicOr(&s_mask[s_sel[tid]], 1u << (tid / k));
    __syncthreads();
    if (wave == 0) {
        int c[4], local = 0, nact = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            c[i] = e < E ? __popc(s_mask[e]) : 0;
            local += c[i];
            nact += c[i] > 0 ? 1 : 0;
        }
        // (count, active experts) of the lanes below, packed in one int: at most
        // 256 pairs and 256 experts, so 16 bits each
        const int inc = wave_incl_scan(local | (nact << 16));
        int run = (inc & 0xFFFF) - local;
        int gi = (p.dm.fs > 0 ? 1 : 0) + (inc >> 16) - nact;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) s_off[e] = run;
            if (c[i] > 0) s_groups[gi++] = make_int4(e, run, c[i], run);
            run += c[i];
        }
        if (lane == 63) {
            s_off[E] = inc & 0xFFFF;
            *s_ng = (p.dm.fs > 0 ? 1 : 0) + (inc >> 16);
        }
        if (lane == 0 && p.dm.fs > 0) s_groups[0] = make_int4(E, 0, T, P);
    }
    __syncthreads();
}
__device__ void fused_place(const ExpertParams& p, const int* s_sel, const float* s_wt, const unsigned* s_mask,
                            const int* s_off, int* s_sp, int* s_pos, float* s_swt) {
    const int k = p.dm.k, P = k * p.dm.T;
    const int tid = threadIdx.x;
    if (tid < P) {
        const int key = s_sel[tid];
        const int pos = s_off[key] + __popc(s_mask[key] & ((1u << (tid / k)) - 1u));
        s_sp[pos] = tid;
        s_pos[tid] = pos;
        s_swt[pos] = s_wt[tid];
    }
    // a workgroup barrier for the LDS writes alone: the gate/up weight loads
    // issued before it stay in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    barrier_keep_loads();
}

// One gate/up item (group g, features 8 fb .. 8 fb + 7): the body of
// gateup_mfma_kernel with the sorted pairs from LDS and h stored at agent scope.
// Its weight loads (16 rows x d into the wave's part of s_w), on their own so
// that they can be issued before the item runs.
template <int NSTEP>
__device__ __forceinline__ void fused_gateup_issue(const ExpertParams& p, const int4& g, int fb, unsigned char* s_w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = p.dm.d;
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int j0 = fb * 8;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const uint16_t* gu = static_cast<const uint16_t*>(is_shared ? p.shared.gu : p.routed.gu);
    unsigned char* sw = s_w + wave * (16 * 64 * NSTEP);
    const int kw = wave * (d / 4);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        const int r = 8 * (i & 1) + (lane >> 3);
        const size_t wrr = e * 2 * F + (r < 8 ? (size_t)(j0 + r) : (size_t)(F + j0 + r - 8));
        const int c = (lane & 7) ^ (r & 7);
        __builtin_amdgcn_global_load_lds(gu + wrr * d + kw + 64 * (i >> 1) + 8 * c, sw + i * 1024, 16, 0, 2);
    }
}
// issued: fused_gateup_issue has run for this item already
template <int NSTEP>
__device__ void fused_gateup_item(const ExpertParams& p, const int4& g, int fb, const int* s_sp, unsigned char* s_w,
                                  float (&s_part)[4][256], uint16_t (&s_h)[16][3][8], bool issued) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const bool is_shared = g.x == p.dm.E;
    const int j0 = fb * 8;
    const int sp = is_shared ? 0 : s_sp[g.y + (row < g.z ? row : g.z - 1)];
    const int kl = wave * (d / 4) + 8 * q;
    const __amdgpu_buffer_rsrc_t xv = buffer_view(p.x, (uint32_t)p.dm.T * d * 2);
    uint4 b[NSTEP];
    unsigned char* sw = s_w + wave * (16 * 64 * NSTEP);
    if (!issued) fused_gateup_issue<NSTEP>(p, g, fb, s_w);
    uint4 a0[NSTEP];
    gateup_load_x<NSTEP>(p, g, is_shared, 0, sp, xv, kl, a0);
    // the weights have landed once at most the NSTEP activation loads issued
    // after them are in flight (vector loads retire in order).  Stated here
    // because the weights may have been issued before this item's code: the
    // compiler does not wait for them by itself then.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NSTEP & 15) | ((NSTEP >> 4) << 14));  // vmcnt(NSTEP)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t rbase = (uint32_t)((row >> 3) * 1024 + (row & 7) * 128);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        const uint32_t off = (s >> 1) * 2048 + rbase + ((((4 * (s & 1)) + q) ^ (row & 7)) << 4);
        b[s] = *reinterpret_cast<const uint4*>(sw + off);
    }
    gateup_mfma_tile<NSTEP, true>(p, g, 0, a0, b, j0, s_part, s_h);
    for (int r0 = 16; r0 < g.z; r0 += 16) {
        const int m = r0 + row;
        const int spn = is_shared ? 0 : s_sp[g.y + (m < g.z ? m : g.z - 1)];
        uint4 a[NSTEP];
        gateup_load_x<NSTEP>(p, g, is_shared, r0, spn, xv, kl, a);
        gateup_mfma_tile<NSTEP, true>(p, g, r0, a, b, j0, s_part, s_h);
    }
}

// Weight fragments of one down item (group g, output rows 64 rb .. + 63).
template <int NSMAX>
__device__ __forceinline__ void fused_down_weights(const ExpertParams& p, const int4& g, int rb,
                                                   uint4 (&b)[kDownMfmaTiles][NSMAX]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int nsteps = F / 128;
    const int kl = wave * (F / 4) + 8 * q;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const uint16_t* dn = static_cast<const uint16_t*>(is_shared ? p.shared.dn : p.routed.dn);
    const int n0 = rb * 16 * kDownMfmaTiles;
#pragma unroll
    for (int t = 0; t < kDownMfmaTiles; ++t) {
        const uint16_t* drow = dn + (e * d + (size_t)(n0 + 16 * t + row)) * F + kl;
#pragma unroll
        for (int s = 0; s < NSMAX; ++s) b[t][s] = *reinterpret_cast<const uint4*>(drow + 32 * (s < nsteps ? s : 0));
    }
}

// One down item with its weights in b: y rows at agent scope, then the
// last-arrival combine of the item's 64 columns.
template <int NSMAX>
__device__ void fused_down_item(const ExpertParams& p, const int4& g, int rb, int ng,
                                const uint4 (&b)[kDownMfmaTiles][NSMAX], const float* s_swt, const int* s_pos,
                                float (&s_dpart)[4][kDownMfmaTiles][256], int* s_flag) {
    constexpr int NT = kDownMfmaTiles;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4;
    const int mm = tid >> 4;
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int nsteps = F / 128;
    const int kl = wave * (F / 4) + 8 * q;
    const int n0 = rb * 16 * NT;
    const uint16_t* h16 = static_cast<const uint16_t*>(p.ws.h);
    const size_t plane = (size_t)(p.dm.k + 1) * p.dm.T * p.hstride;
    const uint32_t vbytes = (uint32_t)g.z * p.hstride * 2;
    __amdgpu_buffer_rsrc_t hv[3];
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) hv[pl] = buffer_view(h16 + pl * plane + (size_t)g.w * p.hstride, vbytes);
    float* y = static_cast<float*>(p.ws.y);
    for (int r0 = 0; r0 < g.z; r0 += 16) {
        const int m = r0 + mm;
        const float rw = is_shared ? 1.f : s_swt[g.y + (m < g.z ? m : g.z - 1)];
        down_mfma_tile<NSMAX, NT, true>(p, g, r0, nsteps, kl, n0, hv, b, rw, s_dpart, y, true);
    }
    if (last_arrival(&p.ws.dcount[rb], ng, s_flag)) {
        const int n = p.dm.T * 16 * NT;  // uniform
        if (n <= 256) combine_columns_n<NT, 1>(p, n0, s_pos);
        else if (n <= 512) combine_columns_n<NT, 2>(p, n0, s_pos);
        else combine_columns_n<NT, 4>(p, n0, s_pos);
    }
}

template <int NSTEP, int NSMAX>
__global__ __launch_bounds__(256) void decode_fused_kernel(FusedParams P) {
    constexpr int kStage = GateupWeightLds<NSTEP>::kAllBytes > 16384 ? GateupWeightLds<NSTEP>::kAllBytes : 16384;
    __shared__ __attribute__((aligned(16))) unsigned char s_w[kStage];
    __shared__ float s_part[4][256];
    __shared__ __attribute__((aligned(16))) uint16_t s_h[16][3][8];
    __shared__ float s_red[4][kFusedMaxT];
    __shared__ int s_sel[kFusedMaxPairs];
    __shared__ float s_wt[kFusedMaxPairs];
    __shared__ int s_sp[kFusedMaxPairs];
    __shared__ int s_pos[kFusedMaxPairs];
    __shared__ float s_swt[kFusedMaxPairs];
    __shared__ unsigned s_mask[256];
    __shared__ int s_off[257];
    __shared__ int4 s_groups[257];
    __shared__ int s_ng, s_flag, s_next;
    // the down partial sums reuse the gate/up weight stage (free after phase 2)
    float(&s_dpart)[4][kDownMfmaTiles][256] = *reinterpret_cast<float(*)[4][kDownMfmaTiles][256]>(s_w);
    static_assert(sizeof(float) * 4 * kDownMfmaTiles * 256 <= kStage, "stage too small for the down partials");

    const ExpertParams& p = P.e;
    const int G = P.nblocks, bid = blockIdx.x;
    const int E = p.dm.E, T = p.dm.T, k = p.dm.k;
    int* fbar = p.ws.fbar;
    const int nwait = (G + kBarGroup - 1) / kBarGroup;  // groups of waiting workgroups
    // this launch's generation: flags of earlier launches hold smaller ones
    // (the count wraps after 2^32 launches, far apart in time)
    __shared__ int s_gen;
    if (threadIdx.x == 0) s_gen = ld_agent(bar_gen(fbar)) + 1;
    __syncthreads();
    const int gen = s_gen;
    const int fs_items = p.dm.fs / 8, f_items = p.dm.f / 8;

    // ---- phase 0: router logits; the shared expert's gate/up meanwhile ----
    if (bid < E) {
        fused_router_expert(P, bid, s_red);
        if (tree_arrive(fbar, 0, bid, E)) {
            // the previous launch has ended: its down work counters start over
            for (int x = 0; x < 8; ++x) st_agent(bar_queue(fbar, 8 + x), 0);
            tree_release(fbar, 0, nwait, gen);
        }
    } else if (bid - E < fs_items) {
        fused_gateup_item<NSTEP>(p, make_int4(E, 0, T, k * T), bid - E, s_sp, s_w, s_part, s_h, false);
    }
    tree_wait(fbar, 0, bid, gen);

    // ---- phase 1: routing, redundantly in every workgroup.  Once the group
    // list is known, the weight loads of the workgroup's first gate/up item
    // are issued; the rest of the sort runs while they fly. ----
    fused_topk(p, reinterpret_cast<float*>(s_w), s_sel, s_wt);
    __syncthreads();
    fused_groups(p, s_sel, s_mask, s_off, s_groups, &s_ng);
    const int ng = s_ng;
    const int g0 = p.dm.fs > 0 ? 1 : 0;
    const int n_up = (ng - g0) * f_items;
    const int first_up = (bid & 7) + 8 * (bid >> 3);
    if (first_up < n_up) fused_gateup_issue<NSTEP>(p, s_groups[g0 + first_up / f_items], first_up % f_items, s_w);
    fused_place(p, s_sel, s_wt, s_mask, s_off, s_sp, s_pos, s_swt);
    if (bid == 0) {  // the routing of this forward, for flint_moe_get_routing
        for (int i = threadIdx.x; i < k * T; i += blockDim.x) {
            p.ws.sel[i] = s_sel[i];
            p.ws.wts[i] = s_wt[i];
            p.ws.sorted_pair[i] = s_sp[i];
            p.ws.pair_pos[i] = s_pos[i];
            p.ws.sorted_wt[i] = s_swt[i];
        }
        for (int i = threadIdx.x; i < E; i += blockDim.x) {
            p.ws.counts[i] = __popc(s_mask[i]);
            p.ws.offsets[i] = s_off[i];
        }
    }

    // ---- phase 2: routed gate/up items.  Item j of XCD x is routed item
    // x + 8 j (workgroups are dispatched round-robin over the 8 XCDs): a
    // workgroup's first item is its rank in its XCD, the following ones come
    // from the XCD's counter, fetched while the current item runs, so the
    // workgroups that stream faster take more items. ----
    {
        const int x = bid & 7, per_xcd = G >> 3;
        int* ctr = bar_queue(fbar, x);
        // with no more items than workgroups every item is some workgroup's
        // first: no counter (its fetch would wait for everything in flight)
        const bool dyn = n_up > 8 * per_xcd;
        int i = bid >> 3;
        while (x + 8 * i < n_up) {  // uniform
            int next = per_xcd;
            if (dyn && threadIdx.x == 0)
                next = per_xcd + __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int j = x + 8 * i;
            fused_gateup_item<NSTEP>(p, s_groups[g0 + j / f_items], j % f_items, s_sp, s_w, s_part, s_h,
                                     j == first_up);
            if (threadIdx.x == 0) s_next = next;
            __syncthreads();
            i = s_next;
            __syncthreads();
        }
    }

    // ---- barrier: every h row is written.  Down items are scheduled like the
    // gate/up ones (item x + 8 i, first by rank, then from the XCD's counter);
    // a workgroup with a first down item issues its weight loads before it
    // waits, one without skips the wait. ----
    const int rblocks = p.dm.d / (16 * kDownMfmaTiles);
    const int n_down = ng * rblocks;
    const int xd = bid & 7, per_xcd = G >> 3;
    int id = bid >> 3;               // this workgroup's down item: xd + 8 id
    const int j0 = xd + 8 * id;
    uint4 bw[kDownMfmaTiles][NSMAX];
    if (tree_arrive(fbar, 1, bid, G)) {
        // every workgroup has arrived: each has read the generation and taken
        // its last gate/up work index
        st_agent(bar_gen(fbar), gen);
        for (int x = 0; x < 8; ++x) st_agent(bar_queue(fbar, x), 0);
        tree_release(fbar, 1, nwait, gen);
    }
    if (j0 < n_down) {
        fused_down_weights<NSMAX>(p, s_groups[j0 / rblocks], j0 % rblocks, bw);
        tree_wait(fbar, 1, bid, gen);
    }

    // ---- phase 3: down items and the combine ----
    const bool dyn_down = n_down > 8 * per_xcd;
    while (xd + 8 * id < n_down) {  // uniform
        const int j = xd + 8 * id;
        if (j != j0) fused_down_weights<NSMAX>(p, s_groups[j / rblocks], j % rblocks, bw);
        int next = per_xcd;
        if (dyn_down && threadIdx.x == 0)
            next = per_xcd + __hip_atomic_fetch_add(bar_queue(fbar, 8 + xd), 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        fused_down_item<NSMAX>(p, s_groups[j / rblocks], j % rblocks, ng, bw, s_swt, s_pos, s_dpart, &s_flag);
        if (threadIdx.x == 0) s_next = next;
        __syncthreads();
        id = s_next;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Single-launch decode with NVFP4 weights: the phases of decode_fused_kernel
// (router, routing in every workgroup, gate/up items, down items with the
// last-arrival combine, the same tree barriers) with the NVFP4 tiles of the
// separate kernels.  A gate/up item is (group, 16 features): 16 gate and 16
// up rows, K split over the 4 waves, NG groups of 128 per wave (d = 512 NG),
// h written as its two f16 planes at agent scope.  A down item is (group, 64
// output rows) with the whole K (F <= kFp4DownKChunk) in one workgroup.
// ---------------------------------------------------------------------------
constexpr int kFusedFp4Features = 16;  // features per gate/up item

template <int NG>
__device__ void fused_fp4_gateup_item(const ExpertParams& p, const int4& g, int fb, const int* s_sp, uint8_t* s_sc,
                                      float (&s_part)[4][2][256]) {
    constexpr int NW = 4, FT = 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int j0 = fb * 16 * FT;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const int kl = wave * (d / NW) + 32 * q;  // this lane's first element in each group
    const int sp = is_shared ? 0 : s_sp[g.y + (row < g.z ? row : g.z - 1)];
    // the item's scales (2 FT x 16 rows of d / 16 bytes), one 16-byte chunk per thread
    constexpr int kCpr = NG * NW / 2;
    constexpr int kChunks = 2 * FT * 16 * kCpr;
    static_assert(kChunks <= 64 * NW, "one scale chunk per thread");
    const int sc_c = tid < kChunks ? tid : kChunks - 1;
    const int sc_r = sc_c / kCpr, sc_cc = sc_c % kCpr, sc_t = sc_r >> 4;
    const size_t sc_wr = e * 2 * F + (size_t)(sc_t >= FT ? F : 0) + j0 + 16 * (sc_t % FT) + (sc_r & 15);
    const uint4 sc_val = *reinterpret_cast<const uint4*>(wp.gus + sc_wr * (d / 16) + 16 * sc_cc);
    uint4* sc_dst = reinterpret_cast<uint4*>(s_sc + sc_r * kFp4ScRow<NG, NW> + 16 * sc_cc);
    uint4 cw[2 * FT][NG];
#pragma unroll
    for (int t = 0; t < 2 * FT; ++t) {
        const size_t wr = e * 2 * F + (size_t)(t >= FT ? F : 0) + j0 + 16 * (t % FT) + row;
        const uint8_t* crow = static_cast<const uint8_t*>(wp.gu) + wr * (d / 2) + kl / 2;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) cw[t][gg] = *reinterpret_cast<const uint4*>(crow + 64 * gg);
    }
    const float tsg = wp.ts[e * 3 + 0], tsu = wp.ts[e * 3 + 1];
    const __amdgpu_buffer_rsrc_t xv = buffer_view(p.x, (uint32_t)p.dm.T * d * 2);
    gateup_fp4_tile<NG, NW, FT, true>(p, g, is_shared, 0, sp, xv, kl, cw, s_sc, true, tid < kChunks ? sc_dst : nullptr,
                                      sc_val, tsg, tsu, j0, s_part);
    for (int r0 = 16; r0 < g.z; r0 += 16) {
        const int m = r0 + row;
        const int spn = is_shared ? 0 : s_sp[g.y + (m < g.z ? m : g.z - 1)];
        gateup_fp4_tile<NG, NW, FT, true>(p, g, is_shared, r0, spn, xv, kl, cw, s_sc, false, nullptr, sc_val, tsg,
                                          tsu, j0, s_part);
    }
}

// The weights of one NVFP4 down item (group g, output rows 64 rb .. + 63):
// the lane's codes, and up to two 16-byte chunks of the item's block scales
// with their LDS offsets (-1: none), written to LDS by the item's first tile.
template <int NGMAX>
struct Fp4DownRegs {
    uint4 cw[kDownFp4Tiles][NGMAX];
    u32x4_t sc_v0, sc_v1;
    int sc_o0, sc_o1;
};
template <int NGMAX>
__device__ __forceinline__ void fused_fp4_down_weights(const ExpertParams& p, const int4& g, int rb,
                                                       Fp4DownRegs<NGMAX>& w) {
    constexpr int NT = kDownFp4Tiles;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int ng = F / 512;
    const int kl = wave * (F / 4) + 32 * q;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const int n0 = rb * 16 * NT;
    const int cpr = F / 256, nchunks = 16 * NT * cpr;
    auto sc_chunk = [&](int ci, u32x4_t& v) {  // LDS offset of chunk ci, or -1 past the last
        const int cc = ci < nchunks ? ci : nchunks - 1;
        const int r = cc / cpr, col = cc % cpr;
        const size_t wr = e * (size_t)d + (size_t)(n0 + r);
        v = *reinterpret_cast<const u32x4_t*>(wp.dns + wr * (F / 16) + 16 * col);
        return ci < nchunks ? r * kFp4DownScRow<NGMAX> + 16 * col : -1;
    };
    w.sc_o0 = sc_chunk(tid, w.sc_v0);
    w.sc_o1 = sc_chunk(tid + 256, w.sc_v1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const size_t wr = e * (size_t)d + (size_t)(n0 + 16 * t + row);
        const uint8_t* crow = static_cast<const uint8_t*>(wp.dn) + wr * (F / 2) + kl / 2;
#pragma unroll
        for (int gg = 0; gg < NGMAX; ++gg) w.cw[t][gg] = *reinterpret_cast<const uint4*>(crow + 64 * (gg < ng ? gg : 0));
    }
}

// One NVFP4 down item with its weights in w: y rows at agent scope, then the
// last-arrival combine of the item's 64 columns.
template <int NGMAX>
__device__ void fused_fp4_down_item(const ExpertParams& p, const int4& g, int rb, int ngroups, Fp4DownRegs<NGMAX>& w,
                                    const float* s_swt, const int* s_pos, uint8_t* s_sc,
                                    float (&s_part)[4][kDownFp4Tiles][256], int* s_flag) {
    constexpr int NT = kDownFp4Tiles;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4;
    const int mm = tid >> 4;
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int ng = F / 512;
    const int kl = wave * (F / 4) + 32 * q;
    const int n0 = rb * 16 * NT;
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const float tsd = wp.ts[e * 3 + 2] / kHScale;
    const uint16_t* h16 = static_cast<const uint16_t*>(p.ws.h);
    const size_t plane = (size_t)(p.dm.k + 1) * p.dm.T * p.hstride;
    const uint32_t vbytes = (uint32_t)g.z * p.hstride * 2;
    const __amdgpu_buffer_rsrc_t hv_hi = buffer_view(h16 + (size_t)g.w * p.hstride, vbytes);
    const __amdgpu_buffer_rsrc_t hv_lo = buffer_view(h16 + plane + (size_t)g.w * p.hstride, vbytes);
    float* y = static_cast<float*>(p.ws.y);
    for (int r0 = 0; r0 < g.z; r0 += 16) {
        const int m = r0 + mm;
        const float rw = is_shared ? 1.f : s_swt[g.y + (m < g.z ? m : g.z - 1)];
        down_fp4_tile<NT, NGMAX, true>(p, g, r0, ng, kl, kl, n0, hv_hi, hv_lo, w.cw, s_sc, r0 == 0, w.sc_o0, w.sc_o1,
                                       w.sc_v0, w.sc_v1, tsd * rw, s_part, y, true);
    }
    if (last_arrival(&p.ws.dcount[rb], ngroups, s_flag)) {
        const int n = p.dm.T * 16 * NT;  // uniform
        if (n <= 256) combine_columns_n<NT, 1>(p, n0, s_pos);
        else if (n <= 512) combine_columns_n<NT, 2>(p, n0, s_pos);
        else combine_columns_n<NT, 4>(p, n0, s_pos);
    }
}

template <int NG, int NGMAX>
__global__ __launch_bounds__(256) void decode_fused_fp4_kernel(FusedParams P) {
    constexpr int kScUp = 2 * 16 * kFp4ScRow<NG, 4>, kScDown = 16 * kDownFp4Tiles * kFp4DownScRow<NGMAX>;
    __shared__ __attribute__((aligned(16))) float s_logit[kFusedMaxT * 256];
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[kScUp > kScDown ? kScUp : kScDown];
    __shared__ float s_upart[4][2][256];
    __shared__ float s_dpart[4][kDownFp4Tiles][256];
    __shared__ float s_red[4][kFusedMaxT];
    __shared__ int s_sel[kFusedMaxPairs];
    __shared__ float s_wt[kFusedMaxPairs];
    __shared__ int s_sp[kFusedMaxPairs];
    __shared__ int s_pos[kFusedMaxPairs];
    __shared__ float s_swt[kFusedMaxPairs];
    __shared__ unsigned s_mask[256];
    __shared__ int s_off[257];
    __shared__ int4 s_groups[257];
    __shared__ int s_ng, s_flag, s_next, s_gen;

    const ExpertParams& p = P.e;
    const int G = P.nblocks, bid = blockIdx.x;
    const int E = p.dm.E, T = p.dm.T, k = p.dm.k;
    int* fbar = p.ws.fbar;
    const int nwait = (G + kBarGroup - 1) / kBarGroup;
    if (threadIdx.x == 0) s_gen = ld_agent(bar_gen(fbar)) + 1;
    __syncthreads();
    const int gen = s_gen;
    const int fs_items = p.dm.fs / kFusedFp4Features, f_items = p.dm.f / kFusedFp4Features;

    // ---- phase 0: router logits; the shared expert's gate/up meanwhile ----
    if (bid < E) {
        fused_router_expert(P, bid, s_red);
        if (tree_arrive(fbar, 0, bid, E)) {
            for (int x = 0; x < 8; ++x) st_agent(bar_queue(fbar, 8 + x), 0);
            tree_release(fbar, 0, nwait, gen);
        }
    } else if (bid - E < fs_items) {
        fused_fp4_gateup_item<NG>(p, make_int4(E, 0, T, k * T), bid - E, s_sp, s_sc, s_upart);
    }
    tree_wait(fbar, 0, bid, gen);

    // ---- phase 1: routing, redundantly in every workgroup ----
    fused_topk(p, s_logit, s_sel, s_wt);
    __syncthreads();
    fused_groups(p, s_sel, s_mask, s_off, s_groups, &s_ng);
    const int ng = s_ng;
    const int g0 = p.dm.fs > 0 ? 1 : 0;
    const int n_up = (ng - g0) * f_items;
    fused_place(p, s_sel, s_wt, s_mask, s_off, s_sp, s_pos, s_swt);
    if (bid == 0) {  // the routing of this forward, for flint_moe_get_routing
        for (int i = threadIdx.x; i < k * T; i += blockDim.x) {
            p.ws.sel[i] = s_sel[i];
            p.ws.wts[i] = s_wt[i];
            p.ws.sorted_pair[i] = s_sp[i];
            p.ws.pair_pos[i] = s_pos[i];
            p.ws.sorted_wt[i] = s_swt[i];
        }
        for (int i = threadIdx.x; i < E; i += blockDim.x) {
            p.ws.counts[i] = __popc(s_mask[i]);
            p.ws.offsets[i] = s_off[i];
        }
    }

    // ---- phase 2: routed gate/up items (item x + 8 j of XCD x first by rank,
    // then from the XCD's counter when there are more items than workgroups) ----
    const int per_xcd = G >> 3;
    {
        const int x = bid & 7;
        int* ctr = bar_queue(fbar, x);
        const bool dyn = n_up > 8 * per_xcd;
        int i = bid >> 3;
        while (x + 8 * i < n_up) {  // uniform
            int next = per_xcd;
            if (dyn && threadIdx.x == 0)
                next = per_xcd + __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int j = x + 8 * i;
            fused_fp4_gateup_item<NG>(p, s_groups[g0 + j / f_items], j % f_items, s_sp, s_sc, s_upart);
            if (threadIdx.x == 0) s_next = next;
            __syncthreads();
            i = s_next;
            __syncthreads();
        }
    }

    // ---- barrier: every h row is written; a workgroup with a first down item
    // loads its weights before it waits ----
    const int rblocks = p.dm.d / (16 * kDownFp4Tiles);
    const int n_down = ng * rblocks;
    const int xd = bid & 7;
    int id = bid >> 3;
    const int j0 = xd + 8 * id;
    Fp4DownRegs<NGMAX> w;
    if (tree_arrive(fbar, 1, bid, G)) {
        st_agent(bar_gen(fbar), gen);
        for (int x = 0; x < 8; ++x) st_agent(bar_queue(fbar, x), 0);
        tree_release(fbar, 1, nwait, gen);
    }
    if (j0 < n_down) {
        fused_fp4_down_weights<NGMAX>(p, s_groups[j0 / rblocks], j0 % rblocks, w);
        tree_wait(fbar, 1, bid, gen);
    }

    // ---- phase 3: down items and the combine ----
    const bool dyn_down = n_down > 8 * per_xcd;
    while (xd + 8 * id < n_down) {  // uniform
        const int j = xd + 8 * id;
        if (j != j0) fused_fp4_down_weights<NGMAX>(p, s_groups[j / rblocks], j % rblocks, w);
        int next = per_xcd;
        if (dyn_down && threadIdx.x == 0)
            next = per_xcd + __hip_atomic_fetch_add(bar_queue(fbar, 8 + xd), 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        fused_fp4_down_item<NGMAX>(p, s_groups[j / rblocks], j % rblocks, ng, w, s_swt, s_pos, s_sc, s_dpart,
                                   &s_flag);
        if (threadIdx.x == 0) s_next = next;
        __syncthreads();
        id = s_next;
        __syncthreads();
    }
}

template <int NSTEP, int NSMAX>
static const void* fused_kernel_ptr() {
    return reinterpret_cast<const void*>(&decode_fused_kernel<NSTEP, NSMAX>);
}

// The kernel instance for the shape, or null: NSTEP = d / 128 k steps per wave,
// NSMAX = the widest expert / 128.
static const void* fused_kernel_for(const Dims& dm) {
    const int fmax = dm.f > dm.fs ? dm.f : dm.fs;
    if (dm.wdt == DT_NVFP4) {  // NG = d / 512, NGMAX = the widest expert / 512
        const int ng = dm.d / 512, nm = fmax / 512;
#define FLINT_FUSED_FP4_CASE(S)                                                                   \
        if (ng == S) {                                                                            \
            if (nm <= 1) return reinterpret_cast<const void*>(&decode_fused_fp4_kernel<S, 1>);    \
            if (nm <= 2) return reinterpret_cast<const void*>(&decode_fused_fp4_kernel<S, 2>);    \
            return reinterpret_cast<const void*>(&decode_fused_fp4_kernel<S, 4>);                 \
        }
        FLINT_FUSED_FP4_CASE(1)
        FLINT_FUSED_FP4_CASE(2)
        FLINT_FUSED_FP4_CASE(4)
#undef FLINT_FUSED_FP4_CASE
        return nullptr;
    }
    const int ns = dm.d / 128, nm = (fmax + 127) / 128;
#define FLINT_FUSED_CASE(S)                                  \
    if (ns == S) {                                           \
        if (nm <= 1) return fused_kernel_ptr<S, 1>();        \
        if (nm <= 2) return fused_kernel_ptr<S, 2>();        \
        if (nm <= 4) return fused_kernel_ptr<S, 4>();        \
        return fused_kernel_ptr<S, 8>();                     \
    }
    FLINT_FUSED_CASE(2)
    FLINT_FUSED_CASE(4)
    FLINT_FUSED_CASE(8)
    FLINT_FUSED_CASE(16)
#undef FLINT_FUSED_CASE
    return nullptr;
}

int fused_decode_grid(const Dims& dm, int n_cu) {
    const int fmax = dm.f > dm.fs ? dm.f : dm.fs;
    const int ns = dm.d / 128;
    const bool common = dm.act == DT_BF16 && dm.T >= 1 && dm.T <= kFusedMaxT && dm.k <= kCombineMaxK && dm.E <= 256;
    const bool bf16 = dm.wdt == DT_BF16 && dm.d % 256 == 0 && (ns == 2 || ns == 4 || ns == 8 || ns == 16) &&
                      dm.f % 128 == 0 && dm.fs % 128 == 0 && fmax <= kDownKChunk;
    const int ng = dm.d / 512, nm = fmax / 512;
    const bool fp4 = dm.wdt == DT_NVFP4 && dm.d % 512 == 0 && (ng == 1 || ng == 2 || ng == 4) && dm.f % 512 == 0 &&
                     dm.fs % 512 == 0 && nm >= 1 && nm <= 4 && fmax <= kFp4DownKChunk;
    if (!common || !(bf16 || fp4)) return 0;
    const void* kp = fused_kernel_for(dm);
    if (!kp) return 0;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kp, 256, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    per_cu = per_cu < kFusedBlocksPerCU ? per_cu : kFusedBlocksPerCU;
    const int G = (per_cu * n_cu) & ~7;  // the gate/up work is split over the 8 XCDs
    // the router takes one workgroup per expert and the shared gate/up items the next ones
    const int fs_items = dm.fs / (dm.wdt == DT_NVFP4 ? kFusedFp4Features : 8);
    if (per_cu < 1 || dm.E + fs_items > G || G > kBarGroup * kBarMaxGroups) return 0;
    return G;
}

hipError_t launch_decode_fused(const LayerArgs& a, const Workspace& w, int nblocks, hipStream_t s) {
    FusedParams P;
    P.e = make_params(a, w);
    P.wr = a.wr;
    P.bias = a.bias;
    P.nblocks = nblocks;
    const void* kp = fused_kernel_for(a.dm);
    if (!kp) return hipErrorInvalidValue;
    void* args[] = {&P};
    return hipLaunchKernel(kp, dim3(nblocks), dim3(256), args, 0, s);
}

}  // namespace flint
