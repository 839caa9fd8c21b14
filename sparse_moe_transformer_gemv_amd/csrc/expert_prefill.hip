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
//   down:     Y[r][n] = w_r * (H_r . D_n)                (fp32 out, fp32 math)
//
// Tile 256 rows x 256 B rows, 8 waves as 2 (M) x 4 (N), each wave 128 x 64 =
// 8 x 4 MFMA 16x16x32 tiles (128 fp32 accumulators per lane), two waves per
// SIMD.  For gate/up the 256 B rows of a tile are, per 64-row quarter q, 32
// gate rows then the matching 32 up rows of features 32q..32q+31, so each wave
// holds matching gate and up columns and applies SwiGLU in registers.  The
// MFMAs take the weights as their first operand, which leaves 4 consecutive
// output columns of one row in each lane.  For gate/up (bf16 h) the weight
// rows of each pair of column tiles are interleaved so that a lane holds 8;
// down (fp32 y) keeps each tile's order, so the 4 lanes of a row store 64
// contiguous bytes; either way the results leave as 16-byte stores straight
// from registers.
//
// K advances in pairs of 32-wide sub-stages through two 64 KiB LDS buffers,
// filled straight from global memory with direct-to-LDS 16-byte loads of whole
// 128-byte lines (8 rows x 128 bytes per load: on this part that moves about a
// third more bytes per clock than 16 rows x 64 bytes); 16-byte chunks of each
// 128-byte LDS row are XOR-swizzled by row so fragment reads are free of bank
// conflicts.  One barrier per pair: after it a pair's data is visible to every
// wave and the other buffer is free for the next pair, whose loads fly while
// the two sub-stages run.  The two waves of a SIMD interleave on their own
// (one issues MFMAs while the other reads fragments); keeping them one phase
// apart with a barrier per phase measured slower.
//
// Rows of a tile past its group's end are neither loaded (their lanes get
// out-of-range buffer offsets) nor multiplied (their 16-row MFMA blocks are
// skipped); they are not stored.
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
constexpr int PBK = 32;   // k per MFMA step (one sub-stage)
constexpr int kRowBytes = 128;                    // an LDS row holds k = 64 (two sub-stages)
constexpr int kPairBytes = (PBM + PBN) * kRowBytes;  // 64 KiB: A rows, then B rows
constexpr int kLdsBytes = 2 * kPairBytes;            // 128 KiB
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

// Byte offset of 16-byte chunk `chunk` (k = 8 chunk .. +7 of the pair's 64) of
// LDS row `row`: the 8 chunks of a 128-byte row are XOR-swizzled by row & 7, so
// the fragment reads (one chunk column of 16 consecutive rows per 16 lanes)
// are free of LDS bank conflicts (measured).
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

constexpr int kThreads = 512;

// Fragments of one sub-stage: 8 A and NI B 16-byte LDS reads, 16 rows (2 KiB)
// apart, from two per-lane base addresses, issued together and waited for
// inside the same asm block.  Written as asm because the compiler cannot tell
// these reads from the direct-to-LDS loads still in flight into the other buffer
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
        "ds_read_b128 %1, %12 offset:2048\n\t"
        "ds_read_b128 %2, %12 offset:4096\n\t"
        "ds_read_b128 %3, %12 offset:6144\n\t"
        "ds_read_b128 %4, %12 offset:8192\n\t"
        "ds_read_b128 %5, %12 offset:10240\n\t"
        "ds_read_b128 %6, %12 offset:12288\n\t"
        "ds_read_b128 %7, %12 offset:14336\n\t"
        "ds_read_b128 %8, %13 offset:0\n\t"
        "ds_read_b128 %9, %13 offset:2048\n\t"
        "ds_read_b128 %10, %13 offset:4096\n\t"
        "ds_read_b128 %11, %13 offset:6144\n\t"
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
        "ds_read_b128 %1, %10 offset:2048\n\t"
        "ds_read_b128 %2, %10 offset:4096\n\t"
        "ds_read_b128 %3, %10 offset:6144\n\t"
        "ds_read_b128 %4, %10 offset:8192\n\t"
        "ds_read_b128 %5, %10 offset:10240\n\t"
        "ds_read_b128 %6, %10 offset:12288\n\t"
        "ds_read_b128 %7, %10 offset:14336\n\t"
        "ds_read_b128 %8, %11 offset:0\n\t"
        "ds_read_b128 %9, %11 offset:2048\n\t"
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

// A workgroup barrier that keeps this wave's loads in flight (no vmcnt wait)
// and that no instruction is scheduled across.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    barrier_keep_loads();
    __builtin_amdgcn_sched_barrier(0);
}

// Output column (within a wave's block of 16 NT columns) produced by row jr of
// MFMA column tile tn.  The MFMA result puts rows 4 q .. 4 q + 3 of a tile in
// lane group q, so tiles 2 t and 2 t + 1 are interleaved in steps of 4: lane
// group q then holds 8 consecutive output columns 32 t + 8 q .. +7 of the two
// tiles, written with one 16-byte store.  A single tile (NT = 1) keeps its order.
template <int NT>
__device__ __forceinline__ int out_col(int tn, int jr) {
    if (NT == 1) return jr;
    return 32 * (tn >> 1) + 8 * (jr >> 2) + 4 * (tn & 1) + (jr & 3);
}

// One tile: 256 rows of one group (from m0) times 64 NI B rows (NI = 4: a
// full tile; NI = 2: a half tile, see prefill_gemm_kernel) from B row nb0 of
// the weights (gate/up: first feature nb0; down: first output row nb0).  For
// gate/up the B rows are taken in quarters of 16 NI rows: 8 NI gate rows, then
// the 8 NI up rows of the same features (in out_col order), so wave wn's NI
// column tiles hold matching gate (ni < NI / 2) and up (ni >= NI / 2) columns.
template <int MODE, int NI, int WF>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, unsigned char* lds, const int4& g, int m0,
                                             int nb0) {
    constexpr int BN = 64 * NI;  // B rows of the tile
    constexpr int HS = 8 * NI;   // gate/up: features per wave (gate rows, then as many up rows)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int row16 = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const uint32_t lds0 = lds_addr(lds);
    // this lane's fragment base addresses within a pair buffer, sub-stage 0
    // (sub-stage 1 reads logical chunk q + 4: address bit 6 flipped)
    const uint32_t a_rd = swz(128 * wm + row16, q);
    const uint32_t b_rd = PBM * kRowBytes + swz(BN / 4 * wn + row16, q);
    const bool is_shared = g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const int rows = min(PBM, g.z - m0);
    const size_t e = is_shared ? 0 : (size_t)g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const int K = MODE == MODE_GATEUP ? d : F;
    // 16-row MFMA blocks of this wave's 128 rows that hold rows of the group
    const int nmi = (min(max(rows - 128 * wm, 0), 128) + 15) >> 4;

    // Load slots: A slot j (< 4) of this wave fills LDS rows 32 wave + 8 j .. +7
    // of the A part of a pair buffer, B slot j (< NI) rows BN / 8 wave + 8 j ..
    // +7 of the B part; lane l fills row (l >> 3) of a slot, physical chunk l & 7,
    // so each load moves whole 128-byte lines of 8 rows.  Both operands go through
    // buffer views: the lanes of A padding rows (past the group's end) fetch
    // nothing, and every offset fits 32 bits.
    __amdgpu_buffer_rsrc_t aview, bview;
    uint32_t aoff[4];   // byte offset of the lane's A chunk at k = 0 (kOffNone: padding)
    uint32_t boff[NI];  // byte offset of the lane's B chunk at k = 0
    if (MODE == MODE_GATEUP) {
        aview = buffer_view(p.x, (uint32_t)((size_t)p.dm.T * d * 2));
        bview = buffer_view(static_cast<const uint16_t*>(wp.gu) + e * 2 * F * (size_t)K,
                            (uint32_t)((size_t)2 * F * K * 2));
    } else {
        // the tile's rows of h are contiguous: view exactly those
        aview = buffer_view(static_cast<const uint16_t*>(p.ws.h) + (size_t)(g.w + m0) * p.hstride,
                            (uint32_t)((size_t)rows * p.hstride * 2));
        bview = buffer_view(static_cast<const uint16_t*>(wp.dn) + e * (size_t)d * K, (uint32_t)((size_t)d * K * 2));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);  // logical chunk landing in physical chunk lane & 7
        if (r >= rows) {
            aoff[j] = kOffNone;
        } else if (MODE == MODE_GATEUP) {
            const int mm = m0 + r;
            const int tok = is_shared ? mm : p.ws.sorted_pair[g.y + mm] / p.dm.k;
            aoff[j] = (uint32_t)(((size_t)tok * d + 8 * c) * 2);
        } else {
            aoff[j] = (uint32_t)(((size_t)r * p.hstride + 8 * c) * 2);
        }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int r = BN / 8 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        // B row r is row jr of column tile tn of the wave block wb that reads it;
        // out_col() gives the output column (gate/up: feature) it produces
        const int wb = r / (16 * NI), tn = (r >> 4) % NI, jr = r & 15;
        if (MODE == MODE_GATEUP) {
            // tiles < NI / 2 gate, the rest the matching up rows
            const bool up = tn >= NI / 2;
            const int wrow = (up ? F : 0) + nb0 + HS * wb + out_col<NI / 2>(tn % (NI / 2), jr);
            boff[j] = (uint32_t)(((size_t)wrow * K + 8 * c) * 2);
        } else {
            // down writes fp32: tiles keep their own order (column 16 tn + jr),
            // so each store instruction covers 64 contiguous bytes of a row
            boff[j] = (uint32_t)(((size_t)(nb0 + 16 * NI * wb + 16 * tn + jr) * K + 8 * c) * 2);
        }
    }

    // NVFP4 weights (WF): the B rows are dequantised in registers and written to
    // LDS as bf16 in the layout the direct-to-LDS loads give them.  FL = 512 / BN
    // lanes share a B row (fr), each covering FW words of 8 E2M1 codes (8 FW
    // consecutive k of the 64 of a pair, part fh) and their E4M3 block scales.
    constexpr int FL = kThreads / BN, FW = 8 / FL;
    const int fr = tid / FL, fh = tid % FL;
    __amdgpu_buffer_rsrc_t cview, sview;
    uint32_t coff = 0, soff = 0;  // byte offsets of the lane's codes / the row's scales at k = 0
    float ts_a = 1.f, ts_b = 1.f;  // tensor scales: gate and up (gate/up), down twice (down)
    if constexpr (WF == DT_NVFP4) {
        const int wb = fr / (16 * NI), tn = (fr >> 4) % NI, jr = fr & 15;
        int wrow;
        if (MODE == MODE_GATEUP)
            wrow = (tn >= NI / 2 ? F : 0) + nb0 + HS * wb + out_col<NI / 2>(tn % (NI / 2), jr);
        else
            wrow = nb0 + 16 * NI * wb + 16 * tn + jr;
        const size_t erows = MODE == MODE_GATEUP ? (size_t)2 * F : (size_t)d;
        const uint8_t* codes = static_cast<const uint8_t*>(MODE == MODE_GATEUP ? wp.gu : wp.dn) + e * erows * (K / 2);
        const uint8_t* scales = (MODE == MODE_GATEUP ? wp.gus : wp.dns) + e * erows * (K / 16);
        cview = buffer_view(codes, (uint32_t)(erows * (K / 2)));
        sview = buffer_view(scales, (uint32_t)(erows * (K / 16)));
        coff = (uint32_t)(wrow * (K / 2) + 4 * FW * fh);
        soff = (uint32_t)(wrow * (K / 16));
        if (MODE == MODE_GATEUP) {
            ts_a = wp.ts[e * 3 + 0];
            ts_b = wp.ts[e * 3 + 1];
        } else {
            ts_a = ts_b = wp.ts[e * 3 + 2];
        }
    }
    // the lane's codes (FW words) and its row's 4 scales of pair pp
    auto fp4_load = [&](int pp, uint32_t (&cw)[FW], uint32_t& sw) {
        if constexpr (FW == 4) {
            const uint4 v = buffer_load16(cview, coff + 32 * pp);
            cw[0] = v.x; cw[1] = v.y; cw[2] = v.z; cw[3] = v.w;
        } else {
            const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(cview, (int)(coff + 32 * pp), 0, 0));
            cw[0] = v.x; cw[1] = v.y;
        }
        sw = __builtin_amdgcn_raw_buffer_load_b32(sview, (int)(soff + 4 * pp), 0, 0);
    };
    // E2M1 x E4M3 is exact in bf16 (at most 6 significant bits): the hardware
    // convert applies the scale's power of two, an fp32 multiply its 3-bit
    // significand, and the pack to bf16 rounds nothing
    auto fp4_store = [&](int pp, const uint32_t (&cw)[FW], uint32_t sw) {
        unsigned char* bb = lds + (pp & 1) * kPairBytes + PBM * kRowBytes;
#pragma unroll
        for (int i = 0; i < FW; ++i) {
            // word i holds k = 8 (FW fh + i) .. + 7 of the pair: scale (FW fh + i) / 2
            const int kw = FW * fh + i;
            const float sv = __builtin_amdgcn_cvt_f32_fp8(sw >> (8 * (kw >> 1)), 0);
            const uint32_t sb = __float_as_uint(sv);
            const float p2 = __uint_as_float(sb & 0xFF800000u);
            const float mt = __uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u);
            uint32_t pk[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                floatx2_t v;
                if (b == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], p2, 0);
                else if (b == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], p2, 1);
                else if (b == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], p2, 2);
                else v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], p2, 3);
                pk[b] = pack_bf16x2_hw(v.x * mt, v.y * mt);
            }
            *reinterpret_cast<uint4*>(bb + swz(fr, kw)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        }
    };

    floatx4_t acc[8][NI];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // k advances in pairs of sub-stages (k = 64 per pair); pair pp lands in buffer pp & 1
    auto issue = [&](int pp) {
        unsigned char* st_ = lds + (pp & 1) * kPairBytes;
        const uint32_t kb = (uint32_t)pp * kRowBytes;  // byte offset of k = 64 pp in a row
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(aview, st_ + (32 * wave + 8 * j) * kRowBytes, 16, aoff[j] + kb,
                                                     0, 0, 0);
        if constexpr (WF != DT_NVFP4) {
#pragma unroll
            for (int j = 0; j < NI; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(bview,
                                                         st_ + PBM * kRowBytes + (BN / 8 * wave + 8 * j) * kRowBytes,
                                                         16, boff[j] + kb, 0, 0, 0);
        }
    };

    const int np = K / (2 * PBK);  // pairs (K is a multiple of 64)
    // Buffer 0 is free: the previous tile's last pair (np is even) was in buffer 1,
    // and every wave read its pair np - 2 before that pair's barrier.
    uint32_t cw[FW], sw = 0;
    if constexpr (WF == DT_NVFP4) {
        fp4_load(0, cw, sw);
        fp4_store(0, cw, sw);
    }
    issue(0);
    if constexpr (WF == DT_NVFP4) {
        if (np > 1) fp4_load(1, cw, sw);  // in flight behind pair 0's A loads
    }
    for (int pp = 0; pp < np; ++pp) {
        // this wave's part of pair pp has landed; after the barrier every wave's has,
        // and every wave is done reading pair pp - 1, whose buffer pair pp + 1 refills
        // while the two sub-stages of pair pp run.  NVFP4: the two code / scale loads
        // of pair pp + 1 may stay in flight, and the LDS writes of pair pp's weights
        // must be done
        if (WF == DT_NVFP4 && pp + 1 < np)
            __builtin_amdgcn_s_waitcnt(0x0072);  // vmcnt(2) lgkmcnt(0)
        else if (WF == DT_NVFP4)
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        phase_barrier();
        if (pp + 1 < np) issue(pp + 1);
        const uint32_t st = lds0 + (pp & 1) * kPairBytes;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t hx = (uint32_t)h << 6;
            uint4 fa[8], fb[NI];
            if (WF == DT_NVFP4 && h == 1 && pp + 1 < np) {
                // pair pp + 1's weights into the free buffer, then its successor's loads
                fp4_store(pp + 1, cw, sw);
                if (pp + 2 < np) fp4_load(pp + 2, cw, sw);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (nmi > 0) read_frags<NI>(st + (a_rd ^ hx), st + (b_rd ^ hx), fa, fb);
            // 16-row blocks past the group's end are skipped
            if (nmi == 8) {
#pragma unroll
                for (int mi = 0; mi < 8; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma16x16x32(fb[ni], fa[mi], acc[mi][ni]);
            } else {
#pragma unroll
                for (int mi = 0; mi < 8; ++mi)
                    if (mi < nmi) {
#pragma unroll
                        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma16x16x32(fb[ni], fa[mi], acc[mi][ni]);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- epilogue, straight from registers.  The MFMAs take the B rows (weights)
    // as their first operand, so lane (row16, q) holds, for each (mi, ni), rows
    // 4 q .. 4 q + 3 of B tile ni for output row 16 mi + row16.  Gate/up: out_col()
    // made the two tiles of a pair 8 consecutive features, one 16-byte bf16 store
    // (8 bytes for a lone tile).  Down: columns 16 ni + 4 q .. + 3, one 16-byte
    // fp32 store per tile.  Either way 64 contiguous bytes per row and
    // instruction. ----
    const int wrows = min(max(rows - 128 * wm, 0), 128);
    if (MODE == MODE_GATEUP) {
        // gate tile t and up tile t + NI / 2 hold the same features
        uint16_t* dst = static_cast<uint16_t*>(p.ws.h) + (size_t)(g.w + m0 + 128 * wm + row16) * p.hstride + nb0 +
                        HS * wn + (NI == 4 ? 8 : 4) * q;
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            if (16 * mi + row16 < wrows) {
                uint16_t* o = dst + (size_t)16 * mi * p.hstride;
                if (NI == 4) {
                    float hv[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        hv[i] = silu_f32(ts_a * acc[mi][0][i]) * (ts_b * acc[mi][2][i]);
                        hv[4 + i] = silu_f32(ts_a * acc[mi][1][i]) * (ts_b * acc[mi][3][i]);
                    }
                    *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2_hw(hv[0], hv[1]), pack_bf16x2_hw(hv[2], hv[3]),
                                                              pack_bf16x2_hw(hv[4], hv[5]), pack_bf16x2_hw(hv[6], hv[7]));
                } else {
                    float hv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) hv[i] = silu_f32(ts_a * acc[mi][0][i]) * (ts_b * acc[mi][1][i]);
                    *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2_hw(hv[0], hv[1]), pack_bf16x2_hw(hv[2], hv[3]));
                }
            }
        }
    } else {
        float* dst = static_cast<float*>(p.ws.y) + (size_t)(g.w + m0 + 128 * wm + row16) * d + nb0 +
                     16 * NI * wn + 4 * q;
        // routing weights of the lane's 8 rows, loaded before any store (loads and
        // stores share one in-order counter, so a load after a store waits for it)
        // (unconditional buffer loads: a load behind a branch makes every later use
        // wait for all of this wave's memory operations)
        const __amdgpu_buffer_rsrc_t wview = buffer_view(p.ws.sorted_wt + g.y + m0, (uint32_t)(rows * 4));
        float wv[8];
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            const int m = 128 * wm + 16 * mi + row16;
            const uint32_t off = (is_shared || m >= rows) ? kOffNone : (uint32_t)(m * 4);
            const float w = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wview, (int)off, 0, 0));
            wv[mi] = (is_shared ? 1.f : w) * ts_a;  // ts_a: the down tensor scale (1 for bf16)
        }
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            if (16 * mi + row16 < wrows) {
                const float ws = wv[mi];
                float* o = dst + (size_t)16 * mi * d;
#pragma unroll
                for (int t = 0; t < NI; ++t) {
                    const floatx4_t& a = acc[mi][t];
                    *reinterpret_cast<float4*>(o + 16 * t) = make_float4(ws * a[0], ws * a[1], ws * a[2], ws * a[3]);
                }
            }
        }
    }
}

constexpr int kNMajorBlocks = 64;  // B-row blocks per m-tile from which items run B-block-major

// Persistent grid: the work items (m-tile, B-row block) are cut into 8
// contiguous chunks, one per XCD, walked by that XCD's workgroups in rounds.
// When the last round of a chunk would leave at least half of the XCD's
// workgroups idle, its items are split into two half tiles (half the B rows
// each), so that round takes about half as long.
template <int MODE, int WF>
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
    // Items run m-tile-major (the B-row blocks of one m-tile in a row, sharing its
    // A rows), except with many B-row blocks per tile (a wide dense layer): then
    // B-row-block-major, so each XCD's chunk reads its own slice of the weights
    // once, rather than every XCD reading all of them.
    const int ntl = *p.ws.n_tiles;
    const bool nmajor = p.nblk >= kNMajorBlocks;
    auto coords = [&](int t, int4& g, int& m0, int& jb) {
        const int2 tile = p.ws.tiles[nmajor ? t % ntl : t / p.nblk];
        jb = nmajor ? t / ntl : t % p.nblk;
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
            prefill_tile<MODE, 4, WF>(p, lds, g, m0, nb0);
        } else {
            prefill_tile<MODE, 4, WF>(p, lds, g, m0, jb * PBN);
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
            if (nb0 < F) prefill_tile<MODE, 2, WF>(p, lds, g, m0, nb0);
        } else {
            prefill_tile<MODE, 2, WF>(p, lds, g, m0, jb * PBN + h * (PBN / 2));
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
    // the activation rows are read through one buffer view, whose offsets are 32-bit
    // and must stay below kOffNone
    return dm.act == DT_BF16 && (dm.wdt == DT_BF16 || dm.wdt == DT_NVFP4) && dm.d % PBN == 0 &&
           dm.f % (PBN / 2) == 0 &&
           dm.fs % (PBN / 2) == 0 && dm.d % PBK == 0 && dm.f % PBK == 0 &&
           (size_t)dm.T * dm.d * 2 < (size_t)kOffNone;
}

template <int MODE>
static hipError_t launch_prefill(const PrefillParams& p, int n_cu, hipStream_t s) {
    const int grid = ((n_cu > 0 ? n_cu : 256) + 7) / 8 * 8;
    if (p.dm.wdt == DT_NVFP4)
        hipLaunchKernelGGL((prefill_gemm_kernel<MODE, DT_NVFP4>), dim3(grid), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_gemm_kernel<MODE, DT_BF16>), dim3(grid), dim3(kThreads), 0, s, p);
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
