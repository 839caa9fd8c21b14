// expert_prefill.hip -- grouped expert GEMMs on the matrix cores for
// prefill-sized token counts (gfx950).
//
// After the counting sort, the tokens routed to one expert (a "group") are
// contiguous; the shared expert is a group holding every token [evermx.com,
// "Recursive Flint: Open-Weight MoE Coding Model, 2.5B Active", Feature
// Overview, "Sparse architecture": 256 routed experts, 6 per token, plus an
// always-active shared expert].  Each group is a dense GEMM with its own
// weights, so one launch walks a device-built list of 256-row tiles of all
// groups.  The pages name kernels for prompt processing and MoE operations
// written for Apple silicon [same page, "Kernels and inference"]; this is a
// design for CDNA4 matrix cores, not a port of those.
//
//   gate/up:  H[r][j] = SiLU(X_r . G_j) * (X_r . U_j)   (bf16 out, fp32 math)
//   down:     Y[r][n] = w_r * (H_r . D_n)                (bf16 out, fp32 math)
//
// Tile 256 rows x 256 B rows, 8 waves as 2 (M) x 4 (N), each wave 128 x 64 =
// 8 x 4 MFMA 16x16x32 tiles (128 fp32 accumulators per lane), two waves per
// SIMD.  For gate/up the 256 B rows of a tile are, per 64-row quarter q, 32
// gate rows then the matching 32 up rows of features 32q..32q+31, so each wave
// holds matching gate and up columns and applies SwiGLU in registers.
//
// K advances in stages of 32 through four 32 KiB LDS buffers, filled straight
// from global memory (direct-to-LDS 16-byte loads) three stages ahead; 16-byte
// chunks of each 64-byte LDS row are XOR-swizzled by row so fragment reads are
// free of bank conflicts.  The two waves of a SIMD run a ping-pong schedule:
// waves 0-3 and 4-7 are kept one phase apart by workgroup barriers, so while
// one group issues its 32 MFMAs of a stage the other reads its fragments of
// that stage from LDS and issues the loads of a later one, and the matrix
// pipe never waits for LDS.
//
// Scheduling: a persistent grid (one workgroup per CU) walks the tiles; the
// tile range is cut into 8 contiguous chunks, one per XCD (workgroups are
// dispatched round-robin over the 8 XCDs), so the workgroups of one XCD work
// at the same time on neighbouring tiles that share A rows or B panels, and
// those shared K slices are served by that XCD's L2.
#include "flint_internal.hpp"

namespace flint {

constexpr int PBM = 256;  // rows per tile (the sort's tile height)
constexpr int PBN = 256;  // B rows per tile
constexpr int PBK = 32;   // k per stage
constexpr int kNStage = 4;
constexpr int kStageBytes = (PBM + PBN) * PBK * 2;  // 32 KiB
constexpr int kLdsBytes = kNStage * kStageBytes;     // 128 KiB
static_assert(PBM == kPrefillBM, "tile height must match the sort's tile list");

struct PrefillParams {
    Dims dm;
    const uint16_t* x;
    WeightPtrs routed, shared;
    Workspace ws;
    int hstride;
    int nblk;  // B-row blocks per m-tile
};

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

// byte offset of 16-byte chunk `chunk` (k = 8 chunk .. +7) of LDS row `row`
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
    return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4);
}

constexpr int kThreads = 512;

// Fragments of one stage: 8 A and NI B 16-byte LDS reads, 16 rows (1 KiB)
// apart, from two per-lane base addresses, issued together and waited for
// inside the same asm block.  Written as asm because the compiler cannot tell
// these reads from the direct-to-LDS loads still in flight into other stages
// and would otherwise wait for all of them (vmcnt 0) first.
typedef __attribute__((ext_vector_type(4))) uint32_t frag_t;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int NI>
__device__ __forceinline__ void read_frags(uint32_t a_base, uint32_t b_base, uint4 (&fa)[8], uint4 (&fb)[NI]);
template <>
__device__ __forceinline__ void read_frags<4>(uint32_t a_base, uint32_t b_base, uint4 (&fa)[8], uint4 (&fb)[4]) {
    frag_t a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3;
    asm volatile(
        "ds_read_b128 %0, %12 offset:0\n\t"
        "ds_read_b128 %1, %12 offset:1024\n\t"
        "ds_read_b128 %2, %12 offset:2048\n\t"
        "ds_read_b128 %3, %12 offset:3072\n\t"
        "ds_read_b128 %4, %12 offset:4096\n\t"
        "ds_read_b128 %5, %12 offset:5120\n\t"
        "ds_read_b128 %6, %12 offset:6144\n\t"
        "ds_read_b128 %7, %12 offset:7168\n\t"
        "ds_read_b128 %8, %13 offset:0\n\t"
        "ds_read_b128 %9, %13 offset:1024\n\t"
        "ds_read_b128 %10, %13 offset:2048\n\t"
        "ds_read_b128 %11, %13 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(a4), "=&v"(a5), "=&v"(a6), "=&v"(a7), "=&v"(b0),
          "=&v"(b1), "=&v"(b2), "=&v"(b3)
        : "v"(a_base), "v"(b_base));
    fa[0] = make_uint4(a0.x, a0.y, a0.z, a0.w);
    fa[1] = make_uint4(a1.x, a1.y, a1.z, a1.w);
    fa[2] = make_uint4(a2.x, a2.y, a2.z, a2.w);
    fa[3] = make_uint4(a3.x, a3.y, a3.z, a3.w);
    fa[4] = make_uint4(a4.x, a4.y, a4.z, a4.w);
    fa[5] = make_uint4(a5.x, a5.y, a5.z, a5.w);
    fa[6] = make_uint4(a6.x, a6.y, a6.z, a6.w);
    fa[7] = make_uint4(a7.x, a7.y, a7.z, a7.w);
    fb[0] = make_uint4(b0.x, b0.y, b0.z, b0.w);
    fb[1] = make_uint4(b1.x, b1.y, b1.z, b1.w);
    fb[2] = make_uint4(b2.x, b2.y, b2.z, b2.w);
    fb[3] = make_uint4(b3.x, b3.y, b3.z, b3.w);
}
template <>
__device__ __forceinline__ void read_frags<2>(uint32_t a_base, uint32_t b_base, uint4 (&fa)[8], uint4 (&fb)[2]) {
    frag_t a0, a1, a2, a3, a4, a5, a6, a7, b0, b1;
    asm volatile(
        "ds_read_b128 %0, %10 offset:0\n\t"
        "ds_read_b128 %1, %10 offset:1024\n\t"
        "ds_read_b128 %2, %10 offset:2048\n\t"
        "ds_read_b128 %3, %10 offset:3072\n\t"
        "ds_read_b128 %4, %10 offset:4096\n\t"
        "ds_read_b128 %5, %10 offset:5120\n\t"
        "ds_read_b128 %6, %10 offset:6144\n\t"
        "ds_read_b128 %7, %10 offset:7168\n\t"
        "ds_read_b128 %8, %11 offset:0\n\t"
        "ds_read_b128 %9, %11 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(a4), "=&v"(a5), "=&v"(a6), "=&v"(a7), "=&v"(b0),
          "=&v"(b1)
        : "v"(a_base), "v"(b_base));
    fa[0] = make_uint4(a0.x, a0.y, a0.z, a0.w);
    fa[1] = make_uint4(a1.x, a1.y, a1.z, a1.w);
    fa[2] = make_uint4(a2.x, a2.y, a2.z, a2.w);
    fa[3] = make_uint4(a3.x, a3.y, a3.z, a3.w);
    fa[4] = make_uint4(a4.x, a4.y, a4.z, a4.w);
    fa[5] = make_uint4(a5.x, a5.y, a5.z, a5.w);
    fa[6] = make_uint4(a6.x, a6.y, a6.z, a6.w);
    fa[7] = make_uint4(a7.x, a7.y, a7.z, a7.w);
    fb[0] = make_uint4(b0.x, b0.y, b0.z, b0.w);
    fb[1] = make_uint4(b1.x, b1.y, b1.z, b1.w);
}

// A barrier that no instruction is scheduled across (the MFMAs of a compute
// phase must stay between its two barriers for the ping-pong to hold).
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    barrier_keep_loads();
    __builtin_amdgcn_sched_barrier(0);
}

// One tile: 256 rows of one group (from m0) times 64 NI B rows (NI = 4: a
// full tile; NI = 2: a half tile, see prefill_gemm_kernel) from B row nb0 of
// the weights (gate/up: feature nb0 / 1 ... see below; down: output row nb0).
// For gate/up the B rows are taken in quarters of 16 NI rows: 8 NI gate rows,
// then the 8 NI up rows of the same features, so wave wn's NI column tiles
// hold matching gate (ni < NI / 2) and up (ni >= NI / 2) columns.
template <int MODE, int NI>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, unsigned char* lds, const int4& g, int m0,
                                             int nb0) {
    constexpr int BN = 64 * NI;  // B rows of the tile
    constexpr int HS = 8 * NI;   // gate/up: features per wave (gate rows, then as many up rows)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;  // wm is also the ping-pong group
    const int row16 = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const uint32_t lds0 = lds_addr(lds);
    // this lane's fragment base addresses within a stage
    const uint32_t a_rd = swz(128 * wm + row16, q);
    const uint32_t b_rd = PBM * PBK * 2 + swz(BN / 4 * wn + row16, q);
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int rows = min(PBM, g.z - m0);
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const int K = MODE == MODE_GATEUP ? d : F;

    // Load slots: A slot j (0, 1) of this wave fills LDS rows 32 wave + 16 j ..
    // +15 of the A half of a stage, B slot j (< NI / 2) rows BN / 8 wave + 16 j
    // .. +15 of the B half; lane l fills row (l >> 2) of a slot, physical chunk
    // l & 3.  Per-lane global sources (logical chunk of the lane's slot):
    const uint16_t* asrc[2];
    const uint16_t* bsrc[NI / 2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 32 * wave + 16 * j + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 1) & 3);
        const int m = r < rows ? r : 0;  // padding rows repeat row 0; never stored
        if (MODE == MODE_GATEUP) {
            const int mm = m0 + m;
            const int tok = is_shared ? mm : p.ws.sorted_pair[g.y + mm] / p.dm.k;
            asrc[j] = p.x + (size_t)tok * d + 8 * c;
        } else {
            asrc[j] = static_cast<const uint16_t*>(p.ws.h) + (size_t)(g.w + m0 + m) * p.hstride + 8 * c;
        }
    }
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
        const int r = BN / 8 * wave + 16 * j + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 1) & 3);
        if (MODE == MODE_GATEUP) {
            const int seg = r / HS, rr = r % HS;  // even: gate rows, odd: the matching up rows
            const size_t wrow = e * 2 * F + (size_t)((seg & 1) ? F : 0) + nb0 + HS * (seg >> 1) + rr;
            bsrc[j] = static_cast<const uint16_t*>(wp.gu) + wrow * K + 8 * c;
        } else {
            bsrc[j] = static_cast<const uint16_t*>(wp.dn) + (e * (size_t)d + nb0 + r) * K + 8 * c;
        }
    }

    floatx4_t acc[8][NI];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // loads per wave and stage: 2 A + NI / 2 B
    constexpr int LPS = 2 + NI / 2;
    auto issue = [&](int s_) {
        unsigned char* st_ = lds + (s_ & (kNStage - 1)) * kStageBytes;
        const int k0_ = s_ * PBK;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + k0_, st_ + (32 * wave + 16 * j) * 64, 16, 0, 0);
#pragma unroll
        for (int j = 0; j < NI / 2; ++j)
            __builtin_amdgcn_global_load_lds(bsrc[j] + k0_, st_ + PBM * PBK * 2 + (BN / 8 * wave + 16 * j) * 64,
                                             16, 0, 0);
    };
    // s_waitcnt vmcnt(n) for n own loads still in flight (n = 0, LPS, 2 LPS)
    auto wait_loads = [&](int stages_ahead) {
        if (stages_ahead >= 2) {
            if (LPS == 4) __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
            else __builtin_amdgcn_s_waitcnt(0x0F76);           // vmcnt(6)
        } else if (stages_ahead == 1) {
            if (LPS == 4) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
            else __builtin_amdgcn_s_waitcnt(0x0F73);           // vmcnt(3)
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
    };

    const int nk = K / PBK;
    __syncthreads();  // the previous tile's epilogue is done with LDS (and its stores retired)
    // prologue: stages 0..2 in flight, then every wave's stage 0 landed
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 2) issue(2);
    wait_loads(min(nk, 3) - 1);
    phase_barrier();
    if (wm == 1) phase_barrier();  // group 1 runs one phase behind
    for (int s = 0; s < nk; ++s) {
        // ---- memory phase of stage s: refill the buffer of stage s - 1 (read by both
        // groups by now) with stage s + 3, make sure this wave's part of stage s + 1
        // has landed (the other group reads it right after the next barrier), read
        // this stage's fragments ----
        if (s + 3 < nk) issue(s + 3);
        wait_loads(min(s + 3, nk - 1) - s - 1);
        const uint32_t st = lds0 + (s & (kNStage - 1)) * kStageBytes;
        uint4 fa[8], fb[NI];
        read_frags<NI>(st + a_rd, st + b_rd, fa, fb);
        phase_barrier();
        // ---- compute phase of stage s ----
#pragma unroll
        for (int mi = 0; mi < 8; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma16x16x32(fa[mi], fb[ni], acc[mi][ni]);
        phase_barrier();
    }
    if (wm == 0) phase_barrier();  // matches group 1's extra barrier

    // ---- epilogue: results go through LDS (free after the K loop) so that
    // global stores are whole 16-byte chunks of output rows ----
    __syncthreads();  // all waves are done with the stages
    float wrow[8][4];  // routing weight of each of this lane's output rows (down)
    if (MODE == MODE_DOWN) {
        float* s_w = reinterpret_cast<float*>(lds);
        if (tid < PBM) {  // one row per thread
            const int m = tid;
            s_w[m] = (is_shared || m >= rows) ? 1.f : p.ws.sorted_wt[g.y + m0 + m];
        }
        __syncthreads();
#pragma unroll
        for (int mi = 0; mi < 8; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) wrow[mi][i] = s_w[128 * wm + 16 * mi + 4 * q + i];
        __syncthreads();  // s_w is overwritten below
    }
    // this wave's output sub-tile in LDS: 128 rows x OC bf16, row stride OC*2 bytes
    constexpr int OC = (MODE == MODE_GATEUP) ? HS : 16 * NI;
    static_assert(8 * 128 * OC * 2 <= kLdsBytes, "epilogue staging fits the stages");
    uint16_t* so = reinterpret_cast<uint16_t*>(lds + wave * (128 * OC * 2));
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ml = 16 * mi + 4 * q + i;  // row within the wave's 128
            if (MODE == MODE_GATEUP) {
#pragma unroll
                for (int ni = 0; ni < NI / 2; ++ni) {
                    const float gv = acc[mi][ni][i], uv = acc[mi][ni + NI / 2][i];
                    so[ml * OC + 16 * ni + row16] = f32_to_bf16(silu_f32(gv) * uv);
                }
            } else {
                const float ws = wrow[mi][i];
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) so[ml * OC + 16 * ni + row16] = f32_to_bf16(ws * acc[mi][ni][i]);
            }
        }
    }
    __syncthreads();
    // copy out: each lane moves 16-byte chunks of the wave's rows
    {
        constexpr int CPR = OC * 2 / 16;  // chunks per row
        uint16_t* dst_base;
        size_t dst_stride;
        if (MODE == MODE_GATEUP) {
            dst_base = static_cast<uint16_t*>(p.ws.h) + (size_t)(g.w + m0 + 128 * wm) * p.hstride + nb0 + OC * wn;
            dst_stride = p.hstride;
        } else {
            dst_base = static_cast<uint16_t*>(p.ws.y) + (size_t)(g.w + m0 + 128 * wm) * d + nb0 + OC * wn;
            dst_stride = d;
        }
        const int wrows = min(128, rows - 128 * wm);
        for (int idx = lane; idx < 128 * CPR; idx += 64) {
            const int r = idx / CPR, cc = idx % CPR;
            if (r < wrows)
                *reinterpret_cast<uint4*>(dst_base + (size_t)r * dst_stride + cc * 8) =
                    *reinterpret_cast<const uint4*>(so + r * OC + cc * 8);
        }
    }
}

// Persistent grid: the work items (m-tile, B-row block) are cut into 8
// contiguous chunks, one per XCD, walked by that XCD's workgroups in rounds.
// When the last round of a chunk would leave at least half of the XCD's
// workgroups idle, its items are split into two half tiles (half the B rows
// each), so that round takes about half as long.
template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_gemm_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    const int total = *p.ws.n_tiles * p.nblk;
    const int per_xcd = (total + 7) / 8;
    const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, j = blockIdx.x >> 3;
    const int t0 = xcd * per_xcd;
    const int cnt = max(0, min(total, t0 + per_xcd) - t0);  // items of this XCD
    const int rem = cnt % nper;
    const bool split = rem > 0 && 2 * rem <= nper;
    const int nfull = split ? cnt - rem : cnt;
    auto coords = [&](int t, int4& g, int& m0, int& jb) {
        const int2 tile = p.ws.tiles[t / p.nblk];
        jb = t % p.nblk;
        g = p.ws.groups[tile.x];
        m0 = tile.y;
    };
    for (int i = j; i < nfull; i += nper) {
        int4 g;
        int m0, jb;
        coords(t0 + i, g, m0, jb);
        if (MODE == MODE_GATEUP) {
            const int F = g.x == p.dm.E ? p.dm.fs : p.dm.f;
            const int nb0 = jb * (PBN / 2);  // first h feature of this tile
            if (nb0 >= F) continue;
            prefill_tile<MODE, 4>(p, lds, g, m0, nb0);
        } else {
            prefill_tile<MODE, 4>(p, lds, g, m0, jb * PBN);
        }
    }
    if (split && j < 2 * rem) {
        int4 g;
        int m0, jb;
        coords(t0 + nfull + (j >> 1), g, m0, jb);
        const int h = j & 1;  // which half of the item's B rows
        if (MODE == MODE_GATEUP) {
            const int F = g.x == p.dm.E ? p.dm.fs : p.dm.f;
            const int nb0 = jb * (PBN / 2) + h * (PBN / 4);  // first h feature of this half
            if (nb0 < F) prefill_tile<MODE, 2>(p, lds, g, m0, nb0);
        } else {
            prefill_tile<MODE, 2>(p, lds, g, m0, jb * PBN + h * (PBN / 2));
        }
    }
}

static PrefillParams make_prefill_params(const LayerArgs& a, const Workspace& w, int nblk) {
    PrefillParams p;
    p.dm = a.dm;
    p.x = static_cast<const uint16_t*>(a.x);
    p.routed = a.routed;
    p.shared = a.shared;
    p.ws = w;
    p.hstride = a.dm.f > a.dm.fs ? a.dm.f : a.dm.fs;
    p.nblk = nblk;
    return p;
}

bool prefill_ok(const Dims& dm) {
    return dm.act == DT_BF16 && dm.wdt == DT_BF16 && dm.d % PBN == 0 && dm.f % (PBN / 2) == 0 &&
           dm.fs % (PBN / 2) == 0 && dm.d % PBK == 0 && dm.f % PBK == 0;
}

template <int MODE>
static hipError_t launch_prefill(const PrefillParams& p, int n_cu, hipStream_t s) {
    const int grid = ((n_cu > 0 ? n_cu : 256) + 7) / 8 * 8;
    hipLaunchKernelGGL(prefill_gemm_kernel<MODE>, dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gateup_prefill(const LayerArgs& a, const Workspace& w, int n_cu, hipStream_t s) {
    const int hs = a.dm.f > a.dm.fs ? a.dm.f : a.dm.fs;
    return launch_prefill<MODE_GATEUP>(make_prefill_params(a, w, hs / (PBN / 2)), n_cu, s);
}

hipError_t launch_down_prefill(const LayerArgs& a, const Workspace& w, int n_cu, hipStream_t s) {
    return launch_prefill<MODE_DOWN>(make_prefill_params(a, w, a.dm.d / PBN), n_cu, s);
}

}  // namespace flint
