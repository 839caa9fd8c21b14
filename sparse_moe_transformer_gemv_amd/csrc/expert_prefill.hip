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
//   down:     Y[r][n] = w_r * (H_r . D_n)                (packed out, fp32 math)
//
// Tile 256 rows x 256 B rows, 8 waves as 2 (M) x 4 (N), each wave 128 x 64 =
// 8 x 4 MFMA 16x16x32 tiles (128 fp32 accumulators per lane), two waves per
// SIMD.  For gate/up the 256 B rows of a tile are, per 64-row quarter q, 32
// gate rows then the matching 32 up rows of features 32q..32q+31, so each wave
// holds matching gate and up columns and applies SwiGLU in registers.  The
// MFMAs take the weights as their first operand, which leaves 4 consecutive
// output columns of one row in each lane.  The weight rows of each pair of
// column tiles are interleaved so that a lane holds 8 consecutive columns, and
// the results leave as 16-byte stores straight from registers (8 bf16 h
// values, or two packed y blocks), 64 contiguous bytes of a row per
// instruction.  y is stored 2 bytes per element as block floating point over 4
// columns (pack_bfp4: a shared exponent and 14-bit mantissas, error at most
// 2^-12 of the block's largest magnitude), which keeps the combine's sum of
// seven rows well inside the layer's tolerance while moving half the bytes of
// fp32 rows through the down stores and the combine loads.
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

// A tile: 256 rows of group g (from row m0 of the group) times the B rows from
// nb0 (gate/up: first feature; down: first output row).
struct TileRef {
    int4 g;
    int m0, nb0;
};

// Operand views of a tile (bf16 weights).  Both operands go through buffer
// views: the lanes of A padding rows (past the group's end) fetch nothing, and
// every offset fits 32 bits.
template <int MODE>
__device__ __forceinline__ void tile_views(const PrefillParams& p, const TileRef& t, __amdgpu_buffer_rsrc_t& aview,
                                           __amdgpu_buffer_rsrc_t& bview) {
    const bool is_shared = t.g.x == p.dm.E;
    const int F = is_shared ? p.dm.fs : p.dm.f;
    const size_t e = is_shared ? 0 : (size_t)t.g.x;
    const WeightPtrs& wp = is_shared ? p.shared : p.routed;
    const int d = p.dm.d;
    if (MODE == MODE_GATEUP) {
        aview = buffer_view(p.x, (uint32_t)((size_t)p.dm.T * d * 2));
        bview = buffer_view(static_cast<const uint16_t*>(wp.gu) + e * 2 * F * (size_t)d, (uint32_t)((size_t)2 * F * d * 2));
    } else {
        // the tile's rows of h are contiguous: view exactly those
        const int rows = min(PBM, t.g.z - t.m0);
        aview = buffer_view(static_cast<const uint16_t*>(p.ws.h) + (size_t)(t.g.w + t.m0) * p.hstride,
                            (uint32_t)((size_t)rows * p.hstride * 2));
        bview = buffer_view(static_cast<const uint16_t*>(wp.dn) + e * (size_t)d * F, (uint32_t)((size_t)d * F * 2));
    }
}

// Load slots: A slot j (< 4) of wave w fills LDS rows 32 w + 8 j .. +7 of the
// A part of a pair buffer, B slot j (< NI) rows BN / 8 w + 8 j .. +7 of the B
// part; lane l fills row (l >> 3) of a slot, physical chunk l & 7, so each load
// moves whole 128-byte lines of 8 rows.
//
// Gate/up A rows are gathered through the sorted pair list: a_rows_load issues
// the lane's 4 list loads (unconditional, through a view; padding rows and the
// shared group, whose rows are the tokens themselves, load nothing), and
// a_offsets turns them into the byte offsets of the lane's A chunks at k = 0
// (kOffNone: padding).  Down A rows are the tile's h rows.
template <int MODE>
__device__ __forceinline__ void a_rows_load(const PrefillParams& p, const TileRef& t, uint32_t (&raw)[4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (MODE != MODE_GATEUP) return;
    const int rows = min(PBM, t.g.z - t.m0);
    const bool is_shared = t.g.x == p.dm.E;
    const __amdgpu_buffer_rsrc_t sview = buffer_view(p.ws.sorted_pair, (uint32_t)((size_t)p.dm.k * p.dm.T * 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        const uint32_t off = (is_shared || r >= rows) ? kOffNone : (uint32_t)((t.g.y + t.m0 + r) * 4);
        raw[j] = __builtin_amdgcn_raw_buffer_load_b32(sview, (int)off, 0, 0);
    }
}
template <int MODE>
__device__ __forceinline__ void a_offsets(const PrefillParams& p, const TileRef& t, const uint32_t (&raw)[4],
                                          uint32_t (&aoff)[4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rows = min(PBM, t.g.z - t.m0);
    const bool is_shared = t.g.x == p.dm.E;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);  // logical chunk landing in physical chunk lane & 7
        if (r >= rows) {
            aoff[j] = kOffNone;
        } else if (MODE == MODE_GATEUP) {
            const int tok = is_shared ? t.m0 + r : (int)raw[j] / p.dm.k;
            aoff[j] = (uint32_t)(((size_t)tok * p.dm.d + 8 * c) * 2);
        } else {
            aoff[j] = (uint32_t)(((size_t)r * p.hstride + 8 * c) * 2);
        }
    }
}
// Byte offsets of the lane's B chunks at k = 0.  B row r is row jr of column
// tile tn of the wave block wb that reads it; out_col() gives the output
// column (gate/up: feature) it produces.
template <int MODE, int NI>
__device__ __forceinline__ int b_row(const PrefillParams& p, const TileRef& t, int r) {
    constexpr int HS = 8 * NI;
    const int wb = r / (16 * NI), tn = (r >> 4) % NI, jr = r & 15;
    if (MODE == MODE_GATEUP) {
        // tiles < NI / 2 gate, the rest the matching up rows
        const int F = t.g.x == p.dm.E ? p.dm.fs : p.dm.f;
        return (tn >= NI / 2 ? F : 0) + t.nb0 + HS * wb + out_col<NI / 2>(tn % (NI / 2), jr);
    }
    // down: B rows interleaved as for gate/up, so that lane q of a wave holds
    // columns 8 q .. 8 q + 7 of each 32-column half of its block (tiles 2 h and
    // 2 h + 1 give half h): the packed y blocks of two tiles leave as one
    // 16-byte store, 64 contiguous bytes of a row per instruction (8-byte
    // stores of one tile each, 32 bytes per row, cost the down GEMM 12 us more)
    return t.nb0 + 16 * NI * wb + 32 * (tn >> 1) + 8 * (jr >> 2) + 4 * (tn & 1) + (jr & 3);
}
template <int MODE, int NI>
__device__ __forceinline__ void b_offsets(const PrefillParams& p, const TileRef& t, uint32_t (&boff)[NI]) {
    constexpr int BN = 64 * NI;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = MODE == MODE_GATEUP ? p.dm.d : (t.g.x == p.dm.E ? p.dm.fs : p.dm.f);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int r = BN / 8 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        boff[j] = (uint32_t)(((size_t)b_row<MODE, NI>(p, t, r) * K + 8 * c) * 2);
    }
}

// Vector memory operations a full bf16 tile's epilogue issues per wave, all of
// them stores (the down kernel's weight loads come before the next tile's
// loads): the next tile's first wait lets exactly these stay in flight.
template <int MODE>
constexpr int epilogue_stores() { return MODE == MODE_GATEUP ? 8 : 16; }
// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding: vmcnt in bits 3..0
// and 15..14, expcnt and lgkmcnt at their no-wait values)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// One tile: 256 rows of one group (from m0) times 64 NI B rows (NI = 4: a
// full tile; NI = 2: a half tile, see prefill_gemm_kernel) from B row nb0 of
// the weights (gate/up: first feature nb0; down: first output row nb0).  For
// gate/up the B rows are taken in quarters of 16 NI rows: 8 NI gate rows, then
// the 8 NI up rows of the same features (in out_col order), so wave wn's NI
// column tiles hold matching gate (ni < NI / 2) and up (ni >= NI / 2) columns.
//
// aoff / boff hold the tile's operand offsets on entry.  `prefetched`: pair 0
// is already in flight into buffer 0 (issued by the previous tile before its
// epilogue, whose stores may still be in flight behind it).  HAS_NEXT
// (bf16 weights, full tiles only; a separate instance, so that the waits the
// compiler places in the epilogue count the next tile's loads): after the last pair's barrier the tile
// issues the next tile's row-list loads, after its MFMAs the next tile's pair
// 0, then runs its epilogue; aoff / boff then hold the next tile's offsets.
// The pipeline thus runs across tiles: the next tile's first loads fly while
// this one computes its last pair and writes its results.
template <int MODE, int NI, int WF, bool HAS_NEXT>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, unsigned char* lds, const TileRef& t,
                                             uint32_t (&aoff)[4], uint32_t (&boff)[NI], bool prefetched,
                                             const TileRef& nxt) {
    constexpr int BN = 64 * NI;  // B rows of the tile
    constexpr int HS = 8 * NI;   // gate/up: features per wave (gate rows, then as many up rows)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int row16 = lane & 15, q = lane >> 4;
    const int d = p.dm.d;
    const int4 g = t.g;
    const int m0 = t.m0, nb0 = t.nb0;
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
    __amdgpu_buffer_rsrc_t aview, bview;
    tile_views<MODE>(p, t, aview, bview);

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
        const int wrow = b_row<MODE, NI>(p, t, fr);
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

    // pair pp (k = 64 pp .. + 63) of a tile into LDS buffer pp & 1: this wave's 4 A
    // and (bf16 weights) NI B direct-to-LDS loads, through views av / bv
#define FLINT_ISSUE_PAIR(av, bv, load_b, pp_)                                                                    \
    do {                                                                                                         \
        unsigned char* st_ = lds + ((pp_) & 1) * kPairBytes;                                                     \
        const uint32_t kb = (uint32_t)(pp_) * kRowBytes; /* byte offset of k = 64 pp in a row */                \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                            \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(av, st_ + (32 * wave + 8 * j) * kRowBytes, 16, aoff[j] + kb, \
                                                     0, 0, 0);                                                   \
        if (load_b) {                                                                                            \
            _Pragma("unroll") for (int j = 0; j < NI; ++j)                                                       \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(bv, st_ + PBM * kRowBytes + (BN / 8 * wave + 8 * j) * kRowBytes, \
                                                         16, boff[j] + kb, 0, 0, 0);                             \
        }                                                                                                        \
    } while (0)
    constexpr bool kLoadB = WF != DT_NVFP4;
    const int np = K / (2 * PBK);  // pairs (K is a multiple of 64)
    // Buffer 0 is free: the previous tile's last pair (np is even) was in buffer 1,
    // and every wave read its pair np - 2 before that pair's barrier.
    uint32_t cw[FW], sw = 0;
    if (!prefetched) {
        if constexpr (WF == DT_NVFP4) {
            fp4_load(0, cw, sw);
            fp4_store(0, cw, sw);
        }
        FLINT_ISSUE_PAIR(aview, bview, kLoadB, 0);
        if constexpr (WF == DT_NVFP4) {
            if (np > 1) fp4_load(1, cw, sw);  // in flight behind pair 0's A loads
        }
    }
    uint32_t nraw[4];  // the next tile's row-list entries (gate/up)
    for (int pp = 0; pp < np; ++pp) {
        // this wave's part of pair pp has landed; after the barrier every wave's has,
        // and every wave is done reading pair pp - 1, whose buffer pair pp + 1 refills
        // while the two sub-stages of pair pp run.  A prefetched pair 0 may have the
        // previous tile's epilogue stores in flight behind it.  NVFP4: the two code /
        // scale loads of pair pp + 1 may stay in flight, and the LDS writes of pair
        // pp's weights must be done
        if (WF == DT_NVFP4 && pp + 1 < np)
            __builtin_amdgcn_s_waitcnt(0x0072);  // vmcnt(2) lgkmcnt(0)
        else if (WF == DT_NVFP4)
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        else if (pp == 0 && prefetched)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(epilogue_stores<MODE>()));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        phase_barrier();
        if (pp + 1 < np) FLINT_ISSUE_PAIR(aview, bview, kLoadB, pp + 1);
        else if (HAS_NEXT) a_rows_load<MODE>(p, nxt, nraw);
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
    // (8 bytes for a lone tile), 64 contiguous bytes per row and instruction.
    // Down: tiles 2 h and 2 h + 1 give columns 32 h + 8 q .. + 7 (b_row), two
    // packed blocks, one 16-byte store, 64 contiguous bytes per row and
    // instruction.  Every store is issued (rows past the group's end get an
    // offset past the view), so a wave always issues the same number. ----
    float wv[8];
    if (MODE == MODE_DOWN) {
        // routing weights of the lane's 8 rows, loaded before any store and before
        // the next tile's loads (loads and stores share one in-order counter, so a
        // load waits for every memory operation issued before it)
        const __amdgpu_buffer_rsrc_t wview = buffer_view(p.ws.sorted_wt + g.y + m0, (uint32_t)(rows * 4));
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            const int m = 128 * wm + 16 * mi + row16;
            const uint32_t off = (is_shared || m >= rows) ? kOffNone : (uint32_t)(m * 4);
            wv[mi] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wview, (int)off, 0, 0));
        }
    }
    if constexpr (HAS_NEXT) {
        // the next tile's offsets (its row-list loads have landed by now) and pair 0
        __amdgpu_buffer_rsrc_t nav, nbv;
        tile_views<MODE>(p, nxt, nav, nbv);
        a_offsets<MODE>(p, nxt, nraw, aoff);
        b_offsets<MODE, NI>(p, nxt, boff);
        FLINT_ISSUE_PAIR(nav, nbv, true, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (MODE == MODE_GATEUP) {
        // gate tile t and up tile t + NI / 2 hold the same features
        const __amdgpu_buffer_rsrc_t hview = buffer_view(static_cast<uint16_t*>(p.ws.h) + (size_t)(g.w + m0) * p.hstride,
                                                         (uint32_t)((size_t)rows * p.hstride * 2));
        const int col = nb0 + HS * wn + (NI == 4 ? 8 : 4) * q;
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            const int m = 128 * wm + 16 * mi + row16;
            const uint32_t off = m < rows ? (uint32_t)(((size_t)m * p.hstride + col) * 2) : kOffNone;
            if (NI == 4) {
                float hv[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hv[i] = silu_f32(ts_a * acc[mi][0][i]) * (ts_b * acc[mi][2][i]);
                    hv[4 + i] = silu_f32(ts_a * acc[mi][1][i]) * (ts_b * acc[mi][3][i]);
                }
                __builtin_amdgcn_raw_buffer_store_b128(
                    (u32x4_t){pack_bf16x2_hw(hv[0], hv[1]), pack_bf16x2_hw(hv[2], hv[3]),
                              pack_bf16x2_hw(hv[4], hv[5]), pack_bf16x2_hw(hv[6], hv[7])},
                    hview, (int)off, 0, 0);
            } else {
                float hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) hv[i] = silu_f32(ts_a * acc[mi][0][i]) * (ts_b * acc[mi][1][i]);
                __builtin_amdgcn_raw_buffer_store_b64(
                    (u32x2_t){pack_bf16x2_hw(hv[0], hv[1]), pack_bf16x2_hw(hv[2], hv[3])}, hview, (int)off, 0, 0);
            }
        }
    } else {
        const __amdgpu_buffer_rsrc_t yview = buffer_view(static_cast<uint16_t*>(p.ws.y) + (size_t)(g.w + m0) * d,
                                                         (uint32_t)((size_t)rows * d * 2));
        const int col = nb0 + 16 * NI * wn + 8 * q;  // this lane's first run of 8 columns (b_row)
        // (the run of tiles t4, t4 + 1 starts 32 t4 / 2 columns further: 32 t4 bytes)
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) {
            const int m = 128 * wm + 16 * mi + row16;
            const float ws = (is_shared ? 1.f : wv[mi]) * ts_a;  // ts_a: the down tensor scale (1 for bf16)
            const uint32_t off = m < rows ? (uint32_t)(((size_t)m * d + col) * 2) : kOffNone;
#pragma unroll
            for (int t4 = 0; t4 < NI; t4 += 2) {
                const floatx4_t& a = acc[mi][t4];
                const floatx4_t& c = acc[mi][t4 + 1];
                const uint2 b0 = pack_bfp4(ws * a[0], ws * a[1], ws * a[2], ws * a[3]);
                const uint2 b1 = pack_bfp4(ws * c[0], ws * c[1], ws * c[2], ws * c[3]);
                // (a row past the group's end stays past the view with the column offset added).  No
                // non-temporal hint: with it the combine, which reads y next, found it in HBM rather
                // than in the caches (4 us slower)
                __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){b0.x, b0.y, b1.x, b1.y}, yview, (int)(off + 32 * t4), 0,
                                                       0);
            }
        }
    }
    // keeps the two instances' epilogues apart: merged into one block, the
    // compiler's waits before the stores would have to allow for both and would
    // then wait for the next tile's loads as well
    if constexpr (HAS_NEXT) asm volatile("; next tile in flight" ::: "memory");
}

#undef FLINT_ISSUE_PAIR

// Wave-uniform loads of the tile and group lists through the scalar cache,
// complete on return (the wait is in the same asm block).  As vector loads
// they would share the in-order vector-memory counter with the stores of the
// previous tile's epilogue, and waiting for them would wait for those stores.
// The lists are written by an earlier launch, so the scalar cache holds no
// stale copy of them.
typedef __attribute__((ext_vector_type(2))) int sint2_t;
typedef __attribute__((ext_vector_type(4))) int sint4_t;
__device__ __forceinline__ int2 sload_int2(const int2* ptr) {
    sint2_t v;
    asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
    return make_int2(v.x, v.y);
}
__device__ __forceinline__ int4 sload_int4(const int4* ptr) {
    sint4_t v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
    return make_int4(v.x, v.y, v.z, v.w);
}

constexpr int kNMajorBlocks = 64;  // B-row blocks per m-tile from which items run B-block-major

// Persistent grid: the work items (m-tile, B-row block) are cut into 8
// contiguous chunks, one per XCD, walked by that XCD's workgroups in rounds.
// When the last round of a chunk would leave at least half of the XCD's
// workgroups idle, its items are split into two half tiles (half the B rows
// each), so that round takes about half as long.  With bf16 weights each full
// item issues the first loads of the workgroup's next full item before its
// epilogue (see prefill_tile).
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
    // item i of this XCD as a full tile; false when it holds no work (gate/up
    // blocks past a narrower group's width)
    // (every field is loaded into scalar registers: the operand views built from
    // them then live there too, and each buffer load is one instruction rather
    // than a loop over possibly distinct descriptors)
    auto item = [&](int i, TileRef& t) -> bool {
        const int it = __builtin_amdgcn_readfirstlane(t0 + i);
        const int2 tile = sload_int2(p.ws.tiles + (nmajor ? it % ntl : it / p.nblk));
        const int jb = nmajor ? it / ntl : it % p.nblk;
        t.g = sload_int4(p.ws.groups + tile.x);
        t.m0 = tile.y;
        if (MODE == MODE_GATEUP) {
            const int F = t.g.x == p.dm.E ? p.dm.fs : p.dm.f;
            t.nb0 = jb * (PBN / 2);  // first h feature of this tile
            return t.nb0 < F;
        }
        t.nb0 = jb * PBN;
        return true;
    };
    auto next_item = [&](int i, TileRef& t) -> int {  // first item from i with work, or nfull
        for (; i < nfull; i += nper)
            if (item(i, t)) return i;
        return nfull;
    };
    TileRef cur, nxt;
    int i = next_item(j, cur);
    if (i < nfull) {
        uint32_t aoff[4], boff[4], raw[4];
        a_rows_load<MODE>(p, cur, raw);
        a_offsets<MODE>(p, cur, raw, aoff);
        b_offsets<MODE, 4>(p, cur, boff);
        bool prefetched = false;
        while (i < nfull) {
            const int inext = next_item(i + nper, nxt);
            const bool chain = WF != DT_NVFP4 && inext < nfull;
            if constexpr (WF != DT_NVFP4) {
                if (chain) prefill_tile<MODE, 4, WF, true>(p, lds, cur, aoff, boff, prefetched, nxt);
                else prefill_tile<MODE, 4, WF, false>(p, lds, cur, aoff, boff, prefetched, nxt);
            } else {
                prefill_tile<MODE, 4, WF, false>(p, lds, cur, aoff, boff, false, nxt);
            }
            if (!chain && inext < nfull) {
                a_rows_load<MODE>(p, nxt, raw);
                a_offsets<MODE>(p, nxt, raw, aoff);
                b_offsets<MODE, 4>(p, nxt, boff);
            }
            prefetched = chain;
            cur = nxt;
            i = inext;
        }
    }
    if (split && j < 2 * rem) {
        TileRef t;
        item(nfull + (j >> 1), t);
        const int h = j & 1;  // which half of the item's B rows
        bool work = true;
        if (MODE == MODE_GATEUP) {
            const int F = t.g.x == p.dm.E ? p.dm.fs : p.dm.f;
            t.nb0 += h * (PBN / 4);  // first h feature of this half
            work = t.nb0 < F;
        } else {
            t.nb0 += h * (PBN / 2);
        }
        if (work) {
            uint32_t aoff[4], boff[2], raw[4];
            a_rows_load<MODE>(p, t, raw);
            a_offsets<MODE>(p, t, raw, aoff);
            b_offsets<MODE, 2>(p, t, boff);
            prefill_tile<MODE, 2, WF, false>(p, lds, t, aoff, boff, false, t);
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
