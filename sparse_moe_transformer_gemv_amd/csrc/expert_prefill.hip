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
// Tile 256 rows x 256 B rows, K step 64, 8 waves as 2 (M) x 4 (N), each wave
// 128 x 64 = 8 x 4 MFMA 16x16x32 tiles (128 fp32 accumulators per lane), two
// waves per SIMD so that one wave's LDS reads overlap the other's MFMAs.  For
// gate/up the 256 B rows of a tile are, per 64-row quarter q, 32 gate rows then
// the matching 32 up rows of features 32q..32q+31, so each wave holds matching
// gate and up columns and applies SwiGLU in registers.  Two LDS stages of 64 KiB are
// filled straight from global memory (direct-to-LDS 16-byte loads, two K steps
// in flight); 16-byte chunks of each 128-byte LDS row are XOR-swizzled by row
// so fragment reads are free of bank conflicts.
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
constexpr int PBK = 64;   // k per stage
constexpr int kStageBytes = (PBM + PBN) * PBK * 2;  // 64 KiB
constexpr int kLdsBytes = 2 * kStageBytes;           // 128 KiB
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

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

template <int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_gemm_kernel(PrefillParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int row16 = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    // load-slot geometry: instruction i of this wave fills LDS rows 64 i + 8 wave .. +7;
    // lane l fills row (l >> 3) of those with global chunk (l & 7) ^ (l >> 3)
    const int lrow = 8 * wave + (lane >> 3);
    const int lchunk = (lane & 7) ^ (lane >> 3);

    const int total = *p.ws.n_tiles * p.nblk;
    const int per_xcd = (total + 7) / 8;
    const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3;
    const int t_end = min(total, (xcd + 1) * per_xcd);
    for (int t = xcd * per_xcd + (int)(blockIdx.x >> 3); t < t_end; t += nper) {
        const int2 tile = p.ws.tiles[t / p.nblk];
        const int jb = t % p.nblk;
        const int4 g = p.ws.groups[tile.x];
        const bool is_shared = g.x == p.dm.E;
        const int F = is_shared ? p.dm.fs : p.dm.f;
        const int m0 = tile.y;
        const int rows = min(PBM, g.z - m0);
        const size_t e = is_shared ? 0 : (size_t)g.x;
        const WeightPtrs& wp = is_shared ? p.shared : p.routed;
        int K, nb0;
        if (MODE == MODE_GATEUP) {
            K = d;
            nb0 = jb * (PBN / 2);  // first h feature of this tile
            if (nb0 >= F) continue;
        } else {
            K = F;
            nb0 = jb * PBN;  // first output row
        }

        // per-lane global pointers of the 4 A and 4 B load instructions
        const uint16_t* asrc[4];
        const uint16_t* bsrc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 64 * i + lrow;
            const int m = r < rows ? r : 0;  // padding rows repeat row 0; never stored
            if (MODE == MODE_GATEUP) {
                const int mm = m0 + m;
                const int tok = is_shared ? mm : p.ws.sorted_pair[g.y + mm] / p.dm.k;
                asrc[i] = p.x + (size_t)tok * d + 8 * lchunk;
                const int seg = r >> 5, rr = r & 31;  // per 64 rows: 32 gate, then 32 up
                const size_t wrow = e * 2 * F + (size_t)((seg & 1) ? F : 0) + nb0 + 32 * (seg >> 1) + rr;
                bsrc[i] = static_cast<const uint16_t*>(wp.gu) + wrow * K + 8 * lchunk;
            } else {
                asrc[i] = static_cast<const uint16_t*>(p.ws.h) + (size_t)(g.w + m0 + m) * p.hstride +
                          8 * lchunk;
                bsrc[i] = static_cast<const uint16_t*>(wp.dn) + (e * (size_t)d + nb0 + r) * K +
                          8 * lchunk;
            }
        }

        floatx4_t acc[8][4];
#pragma unroll
        for (int mi = 0; mi < 8; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx4_t{0.f, 0.f, 0.f, 0.f};

#define FLINT_ISSUE(kt_, stage_)                                                        \
    do {                                                                                \
        unsigned char* sa_ = smem + (stage_) * kStageBytes;                             \
        unsigned char* sb_ = sa_ + PBM * PBK * 2;                                       \
        const int k0_ = (kt_) * PBK;                                                    \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                \
            __builtin_amdgcn_global_load_lds(asrc[i_] + k0_, sa_ + (64 * i_ + 8 * wave) * 128, \
                                             16, 0, 0);                                 \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_)                                \
            __builtin_amdgcn_global_load_lds(bsrc[i_] + k0_, sb_ + (64 * i_ + 8 * wave) * 128, \
                                             16, 0, 0);                                 \
    } while (0)

        const int nk = K / PBK;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // previous tile's stores retired (vmcnt 0)
        __syncthreads();  // the previous tile's readers are done with both stages
        FLINT_ISSUE(0, 0);
        if (nk > 1) FLINT_ISSUE(1, 1);
        for (int kt = 0; kt < nk; ++kt) {
            // stage kt % 2 has landed once at most the next stage's 8 loads are pending
            // (gfx9 s_waitcnt: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
            if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F78 /* vmcnt(8) */);
            else __builtin_amdgcn_s_waitcnt(0x0F70 /* vmcnt(0) */);
            __syncthreads();
            const unsigned char* sa = smem + (kt & 1) * kStageBytes;
            const unsigned char* sb = sa + PBM * PBK * 2;
            // fragments of both k steps first, then 128 MFMAs (rows past the
            // tile's end hold a copy of its first row and are never stored)
            uint4 fa[2][8], fb[2][4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int c = ks * 4 + q;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fb[ks][i] = *reinterpret_cast<const uint4*>(sb + swz(64 * wn + 16 * i + row16, c));
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    fa[ks][i] = *reinterpret_cast<const uint4*>(sa + swz(128 * wm + 16 * i + row16, c));
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mi = 0; mi < 8; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = mfma16x16x32(fa[ks][mi], fb[ks][ni], acc[mi][ni]);
            if (kt + 2 < nk) {
                __syncthreads();  // everyone has read stage kt % 2
                FLINT_ISSUE(kt + 2, kt & 1);
            }
        }
#undef FLINT_ISSUE

        // ---- epilogue: results go through LDS (free after the K loop) so that
        // global stores are whole 16-byte chunks of output rows ----
        __syncthreads();  // all waves are done reading the last stage
        float wrow[8][4];  // routing weight of each of this lane's output rows (down)
        if (MODE == MODE_DOWN) {
            float* s_w = reinterpret_cast<float*>(smem);
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
        constexpr int OC = (MODE == MODE_GATEUP) ? 32 : 64;
        uint16_t* so = reinterpret_cast<uint16_t*>(smem + wave * (128 * OC * 2));
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ml = 16 * mi + 4 * q + i;  // row within the wave's 128
                if (MODE == MODE_GATEUP) {
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        const float gv = acc[mi][ni][i], uv = acc[mi][ni + 2][i];
                        so[ml * OC + 16 * ni + row16] = f32_to_bf16(silu_f32(gv) * uv);
                    }
                } else {
                    const float ws = wrow[mi][i];
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) so[ml * OC + 16 * ni + row16] = f32_to_bf16(ws * acc[mi][ni][i]);
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
                dst_base = static_cast<uint16_t*>(p.ws.h) + (size_t)(g.w + m0 + 128 * wm) * p.hstride +
                           nb0 + 32 * wn;
                dst_stride = p.hstride;
            } else {
                dst_base = static_cast<uint16_t*>(p.ws.y) + (size_t)(g.w + m0 + 128 * wm) * d + nb0 +
                           64 * wn;
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
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_gemm_kernel<MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int grid = ((n_cu > 0 ? n_cu : 256) + 7) / 8 * 8;
    hipLaunchKernelGGL(prefill_gemm_kernel<MODE>, dim3(grid), dim3(kThreads), kLdsBytes, s, p);
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
