// expert_prefill.hip -- grouped expert GEMMs on the matrix cores for
// prefill-sized token counts (gfx950).
//
// After the counting sort, the tokens routed to one expert (a "group") are
// contiguous; the shared expert is a group holding every token [evermx.com,
// "Recursive Flint: Open-Weight MoE Coding Model, 2.5B Active", Feature
// Overview, "Sparse architecture": 256 routed experts, 6 per token, plus an
// always-active shared expert].  Each group is a dense GEMM with its own
// weights, so one launch walks a device-built list of 64-row tiles of all
// groups.  The pages name kernels for prompt processing and MoE operations
// written for Apple silicon [same page, "Kernels and inference"]; this is a
// design for CDNA4 matrix cores, not a port of those.
//
//   gate/up:  H[r][j] = SiLU(X_r . G_j) * (X_r . U_j)   (bf16 out, fp32 math)
//   down:     Y[r][n] = w_r * (H_r . D_n)                (bf16 out, fp32 math)
//
// Block tile 64 (rows) x 256 (B rows), K step 64, 4 waves side by side along
// N (each 64 x 64 = 4 x 4 MFMA 16x16x32 tiles).  For gate/up the 256 B rows of
// a block are 128 gate rows followed by the matching 128 up rows, and each
// wave owns 32 of each, so SwiGLU is applied in registers.  Global tiles are
// prefetched into registers one K step ahead; LDS rows of 64 bf16 (128 B) keep
// their 16-byte chunks XOR-swizzled by row so that fragment reads are free of
// bank conflicts.
#include "flint_internal.hpp"

namespace flint {

constexpr int PBM = 64;   // rows per tile (the sort's tile height)
constexpr int PBN = 256;  // B rows per tile
constexpr int PBK = 64;   // k per step
static_assert(PBM == kPrefillBM, "tile height must match the sort's tile list");

struct PrefillParams {
    Dims dm;
    const uint16_t* x;
    WeightPtrs routed, shared;
    Workspace ws;
    int hstride;
};

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void prefill_gemm_kernel(PrefillParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char sA[PBM * PBK * 2];
    __shared__ __attribute__((aligned(16))) unsigned char sB[PBN * PBK * 2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row16 = lane & 15, q = lane >> 4;
    if ((int)blockIdx.x >= *p.ws.n_tiles) return;
    const int2 tile = p.ws.tiles[blockIdx.x];
    const int4 g = p.ws.groups[tile.x];
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int d = p.dm.d;
    const int m0 = tile.y;
    const int rows = min(PBM, g.z - m0);
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;

    int K, nb0;
    if (MODE == MODE_GATEUP) {
        K = d;
        nb0 = blockIdx.y * (PBN / 2);  // first h feature of this block
        if (nb0 >= F) return;
    } else {
        K = F;
        nb0 = blockIdx.y * PBN;  // first output row of this block
        if (nb0 >= d) return;
    }

    // ---- global source rows for this thread's load slots ----
    // A: 64 rows x 8 chunks = 512 slots, 2 per thread; B: 256 x 8, 8 per thread.
    const uint16_t* a_src[2];
    bool a_ok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int id = tid + 256 * i, r = id >> 3, c = id & 7;
        const int m = r < rows ? r : 0;  // padding rows read row 0, zeroed below
        a_ok[i] = r < rows;
        if (MODE == MODE_GATEUP) {
            const int mm = m0 + m;
            const int tok = is_shared ? mm : p.ws.sorted_pair[g.y + mm] / p.dm.k;
            a_src[i] = p.x + (size_t)tok * d + 8 * c;
        } else {
            a_src[i] = static_cast<const uint16_t*>(p.ws.h) + (size_t)(g.w + m0 + m) * p.hstride + 8 * c;
        }
    }
    // B slot i of this thread is tile row tid/8 + 32 i: two base pointers (for
    // gate/up: the gate half and the up half) plus a uniform row stride
    const uint16_t* bbase = static_cast<const uint16_t*>(MODE == MODE_GATEUP ? wp.gu : wp.dn);
    const int r0 = tid >> 3, c0 = tid & 7;
    const uint16_t *b_lo, *b_hi;
    if (MODE == MODE_GATEUP) {
        b_lo = bbase + (e * 2 * F + (size_t)(nb0 + r0)) * K + 8 * c0;
        b_hi = bbase + (e * 2 * F + (size_t)(F + nb0 + r0)) * K + 8 * c0;
    } else {
        b_lo = bbase + (e * (size_t)d + (size_t)(nb0 + r0)) * K + 8 * c0;
        b_hi = b_lo + (size_t)(PBN / 2) * K;
    }
    const size_t bstep = (size_t)32 * K;  // 32 tile rows

    // B rows (in the LDS tile) of this wave's four 16-column MFMA tiles
    int brow[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        if (MODE == MODE_GATEUP)
            brow[ni] = (ni < 2 ? 0 : PBN / 2) + 32 * wave + 16 * (ni & 1) + row16;
        else
            brow[ni] = 64 * wave + 16 * ni + row16;
    }
    // LDS byte offsets of this thread's store slots
    int a_dst[2], b_dst[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int id = tid + 256 * i;
        a_dst[i] = swz(id >> 3, id & 7);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int id = tid + 256 * i;
        b_dst[i] = swz(id >> 3, id & 7);
    }
    const uint32_t keep0 = a_ok[0] ? 0xFFFFFFFFu : 0u, keep1 = a_ok[1] ? 0xFFFFFFFFu : 0u;

    floatx4_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra0, ra1, rb[8];
#define FLINT_GLOAD(k0)                                                            \
    do {                                                                           \
        ra0 = *reinterpret_cast<const uint4*>(a_src[0] + (k0));                    \
        ra1 = *reinterpret_cast<const uint4*>(a_src[1] + (k0));                    \
        _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                         \
            rb[i_] = *reinterpret_cast<const uint4*>(b_lo + i_ * bstep + (k0));    \
            rb[4 + i_] = *reinterpret_cast<const uint4*>(b_hi + i_ * bstep + (k0)); \
        }                                                                          \
    } while (0)
#define FLINT_LSTORE()                                                             \
    do {                                                                           \
        *reinterpret_cast<uint4*>(sA + a_dst[0]) =                                 \
            make_uint4(ra0.x & keep0, ra0.y & keep0, ra0.z & keep0, ra0.w & keep0); \
        *reinterpret_cast<uint4*>(sA + a_dst[1]) =                                 \
            make_uint4(ra1.x & keep1, ra1.y & keep1, ra1.z & keep1, ra1.w & keep1); \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_)                           \
            *reinterpret_cast<uint4*>(sB + b_dst[i_]) = rb[i_];                    \
    } while (0)
#define FLINT_COMPUTE()                                                            \
    do {                                                                           \
        _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                         \
            const int c_ = ks * 4 + q;                                             \
            uint4 fa[4], fb[4];                                                    \
            _Pragma("unroll") for (int mi = 0; mi < 4; ++mi)                       \
                fa[mi] = *reinterpret_cast<const uint4*>(sA + swz(16 * mi + row16, c_)); \
            _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                       \
                fb[ni] = *reinterpret_cast<const uint4*>(sB + swz(brow[ni], c_));  \
            _Pragma("unroll") for (int mi = 0; mi < 4; ++mi)                       \
                _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                   \
                    acc[mi][ni] = mfma16x16x32(fa[mi], fb[ni], acc[mi][ni]);       \
        }                                                                          \
    } while (0)

    const int nk = K / PBK;
    FLINT_GLOAD(0);
    FLINT_LSTORE();
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) {
        FLINT_GLOAD((kt + 1) * PBK);  // next tile in flight during this tile's MFMAs
        FLINT_COMPUTE();
        __syncthreads();
        FLINT_LSTORE();
        __syncthreads();
    }
    FLINT_COMPUTE();
#undef FLINT_GLOAD
#undef FLINT_LSTORE
#undef FLINT_COMPUTE

    // ---- epilogue ----
    if (MODE == MODE_GATEUP) {
        uint16_t* h = static_cast<uint16_t*>(p.ws.h);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int j = nb0 + 32 * wave + 16 * ni + row16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 16 * mi + 4 * q + i;
                    if (m < rows) {
                        const float gv = acc[mi][ni][i], uv = acc[mi][ni + 2][i];
                        h[(size_t)(g.w + m0 + m) * p.hstride + j] = f32_to_bf16(silu_f32(gv) * uv);
                    }
                }
            }
    } else {
        uint16_t* y = static_cast<uint16_t*>(p.ws.y);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * mi + 4 * q + i;
                if (m >= rows) continue;
                const float ws = is_shared ? 1.f : p.ws.wts[p.ws.sorted_pair[g.y + m0 + m]];
                uint16_t* yr = y + (size_t)(g.w + m0 + m) * d + nb0 + 64 * wave + row16;
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) yr[16 * ni] = f32_to_bf16(ws * acc[mi][ni][i]);
            }
    }
}

static PrefillParams make_prefill_params(const LayerArgs& a, const Workspace& w) {
    PrefillParams p;
    p.dm = a.dm;
    p.x = static_cast<const uint16_t*>(a.x);
    p.routed = a.routed;
    p.shared = a.shared;
    p.ws = w;
    p.hstride = a.dm.f > a.dm.fs ? a.dm.f : a.dm.fs;
    return p;
}

bool prefill_ok(const Dims& dm) {
    return dm.act == DT_BF16 && dm.wdt == DT_BF16 && dm.d % PBN == 0 && dm.f % (PBN / 2) == 0 &&
           dm.fs % (PBN / 2) == 0 && dm.d % PBK == 0 && dm.f % PBK == 0;
}

hipError_t launch_gateup_prefill(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    PrefillParams p = make_prefill_params(a, w);
    dim3 grid(w.max_tiles, (p.hstride + PBN / 2 - 1) / (PBN / 2));
    hipLaunchKernelGGL(prefill_gemm_kernel<MODE_GATEUP>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_down_prefill(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    PrefillParams p = make_prefill_params(a, w);
    dim3 grid(w.max_tiles, a.dm.d / PBN);
    hipLaunchKernelGGL(prefill_gemm_kernel<MODE_DOWN>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace flint
