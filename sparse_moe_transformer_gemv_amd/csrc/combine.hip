// combine.hip -- weighted unpermute + shared expert (+ residual), and the
// RMSNorm pre-norm of the stacked-layer workload (gfx950).
//
// Every token always gets the shared expert on top of its routed experts
// [evermx.com, "Recursive Flint: Open-Weight MoE Coding Model, 2.5B Active",
// Feature Overview, "Sparse architecture"; swarmz.net, "Recursive Flint: 40B
// Open Model, 2.5B Active", section "The architecture, in plain terms"]:
//     out[t] = (residual[t]) + y[shared slot t] + sum_j y[slot of pair (t, j)]
// where the routed rows of y already carry their combine weight (a layer built
// without a shared expert skips that term).  The sum runs
// in a fixed order (residual, shared, slot 0..k-1), so results are
// deterministic; no atomics.  The y rows are fp32 (decode) or 2 bytes per
// element in 4-column blocks (prefill, see pack_bfp4); the kernels take the
// format as a template parameter and sum in fp32 either way.
#include "flint_internal.hpp"

namespace flint {

struct CombineParams {
    int T, d, k;
    const void* y;        // [(k+1)T][d] fp32 or packed rows
    const int* pair_pos;  // [T][k]
    const float* residual;
    void* out;
    int out_f32;     // 1: fp32 out (act fp32, or residual given); 0: bf16 out
    int has_shared;  // 0: no shared expert (f_s = 0); its slots are never written
};

// the 4 y values from column c (a multiple of 4) of slot row `row`
template <bool PACKED>
__device__ __forceinline__ float4 y_row4(const void* y, size_t row, int d, int c) {
    if constexpr (PACKED) {
        return unpack_bfp4(*reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(y) + row * d + c));
    } else {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(y) + row * d + c);
    }
}
// the same through a buffer view of the y rows (element offset e, or kOffNone: zeros)
template <bool PACKED>
__device__ __forceinline__ float4 y_view4(__amdgpu_buffer_rsrc_t v, uint32_t e) {
    if constexpr (PACKED) {
        const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(v, (int)(e == kOffNone ? kOffNone : e * 2), 0, 0);
        return unpack_bfp4(make_uint2(w.x, w.y));
    } else
        return __builtin_bit_cast(float4, buffer_load16(v, e == kOffNone ? kOffNone : e * 4));
}

// One block of 256 threads per (token, 256 CPT columns); CPT = 8 columns per
// thread for packed rows (two 8-byte blocks in one 16-byte load), 4 for fp32
// rows.  Every load of the thread's columns (residual, shared row, the K
// routed rows) is issued before the first add.
template <bool PACKED, int K>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    constexpr int CPT = PACKED ? 8 : 4;
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * CPT;
    if (c >= p.d) return;
    const size_t kT = (size_t)K * p.T;
    int slot[K];
#pragma unroll
    for (int j = 0; j < K; ++j) slot[j] = p.pair_pos[(size_t)t * K + j];
    // rows of a layer without a shared expert are never written: that load reads
    // the first routed row instead and its values are dropped
    const size_t srow = p.has_shared ? kT + t : (size_t)slot[0];
    const float* rrow = p.residual ? p.residual + (size_t)t * p.d : static_cast<const float*>(p.y);
    float4 r[CPT / 4], sh[CPT / 4], yv[K][CPT / 4];
#pragma unroll
    for (int i = 0; i < CPT / 4; ++i) r[i] = *reinterpret_cast<const float4*>(rrow + c + 4 * i);
    if constexpr (PACKED) {
        const uint16_t* y = static_cast<const uint16_t*>(p.y);
        const uint4 s4 = *reinterpret_cast<const uint4*>(y + srow * p.d + c);
        uint4 v4[K];
#pragma unroll
        for (int j = 0; j < K; ++j) v4[j] = *reinterpret_cast<const uint4*>(y + (size_t)slot[j] * p.d + c);
        sh[0] = unpack_bfp4(make_uint2(s4.x, s4.y));
        sh[1] = unpack_bfp4(make_uint2(s4.z, s4.w));
#pragma unroll
        for (int j = 0; j < K; ++j) {
            yv[j][0] = unpack_bfp4(make_uint2(v4[j].x, v4[j].y));
            yv[j][1] = unpack_bfp4(make_uint2(v4[j].z, v4[j].w));
        }
    } else {
        const float* y = static_cast<const float*>(p.y);
        sh[0] = *reinterpret_cast<const float4*>(y + srow * p.d + c);
#pragma unroll
        for (int j = 0; j < K; ++j) yv[j][0] = *reinterpret_cast<const float4*>(y + (size_t)slot[j] * p.d + c);
    }
    // residual, shared row, routed rows in pair order
    float acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT / 4; ++i) {
        float* a = acc + 4 * i;
        if (p.residual) {
            a[0] = r[i].x; a[1] = r[i].y; a[2] = r[i].z; a[3] = r[i].w;
        } else {
            a[0] = a[1] = a[2] = a[3] = 0.f;
        }
        if (p.has_shared) {
            a[0] += sh[i].x; a[1] += sh[i].y; a[2] += sh[i].z; a[3] += sh[i].w;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
            a[0] += yv[j][i].x; a[1] += yv[j][i].y; a[2] += yv[j][i].z; a[3] += yv[j][i].w;
        }
    }
    if (p.out_f32) {
        float* o = static_cast<float*>(p.out) + (size_t)t * p.d + c;
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i)
            *reinterpret_cast<float4*>(o + 4 * i) = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    } else {
        uint16_t* o = static_cast<uint16_t*>(p.out) + (size_t)t * p.d + c;
        if constexpr (CPT == 8) {
            *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                      pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        } else {
            *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        }
    }
}

template <bool PACKED>
static void launch_combine_k(const CombineParams& p, hipStream_t s) {
    constexpr int CPT = PACKED ? 8 : 4;
    const dim3 grid((p.d + 256 * CPT - 1) / (256 * CPT), p.T);
    switch (p.k) {
    case 1: hipLaunchKernelGGL((combine_kernel<PACKED, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((combine_kernel<PACKED, 2>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((combine_kernel<PACKED, 3>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((combine_kernel<PACKED, 4>), grid, dim3(256), 0, s, p); break;
    case 5: hipLaunchKernelGGL((combine_kernel<PACKED, 5>), grid, dim3(256), 0, s, p); break;
    case 6: hipLaunchKernelGGL((combine_kernel<PACKED, 6>), grid, dim3(256), 0, s, p); break;
    case 7: hipLaunchKernelGGL((combine_kernel<PACKED, 7>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((combine_kernel<PACKED, 8>), grid, dim3(256), 0, s, p); break;
    }
}

hipError_t launch_combine(const LayerArgs& a, const Workspace& w, bool packed, hipStream_t s) {
    CombineParams p;
    p.T = a.dm.T;
    p.d = a.dm.d;
    p.k = a.dm.k;
    p.y = w.y;
    p.pair_pos = w.pair_pos;
    p.residual = a.residual;
    p.out = a.out;
    p.out_f32 = (a.residual != nullptr || a.dm.act == DT_F32) ? 1 : 0;
    p.has_shared = a.dm.fs > 0 ? 1 : 0;
    if (packed) launch_combine_k<true>(p, s);
    else launch_combine_k<false>(p, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The combine followed by the next layer's pre-norm, one block per token:
// out[t] as combine_kernel computes it (fp32 output), then
// norm[t] = bf16(out[t] / sqrt(mean(out[t]^2) + eps)) as rmsnorm_kernel
// computes it from out[t]: the same thread owns the same columns and sums
// their squares in the same order, so both give the same bits as the two
// separate launches.  d <= 4 * 1024 (the row stays in registers).
// ---------------------------------------------------------------------------
constexpr int kNormChunks = 4;
__device__ __forceinline__ float rms_scale(float ss, int d, float eps, float* s_part);

template <bool PACKED>
__global__ __launch_bounds__(256) void combine_norm_kernel(CombineParams p, float eps, uint16_t* __restrict__ norm) {
    __shared__ float s_part[4];
    const int t = blockIdx.x;
    const size_t kT = (size_t)p.k * p.T;
    int slot[kCombineMaxK];
#pragma unroll
    for (int j = 0; j < kCombineMaxK; ++j) slot[j] = j < p.k ? p.pair_pos[(size_t)t * p.k + j] : 0;
    // every load of the row is issued before the first store (a load issued
    // after a store would wait for it: they share one in-order counter); loads
    // of absent terms get an offset past their view and return zeros
    const __amdgpu_buffer_rsrc_t rview =
        buffer_view(p.residual ? p.residual + (size_t)t * p.d : p.y, p.residual ? (uint32_t)p.d * 4 : 0u);
    const __amdgpu_buffer_rsrc_t yview = buffer_view(p.y, (uint32_t)((kT + p.T) * p.d * (PACKED ? 2 : 4)));
    float4 r[kNormChunks], sh[kNormChunks], yv[kNormChunks][kCombineMaxK];
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
        const int c = threadIdx.x * 4 + 1024 * i;
        const bool in = c < p.d;
        r[i] = __builtin_bit_cast(float4, buffer_load16(rview, in ? (uint32_t)c * 4 : kOffNone));
        sh[i] = y_view4<PACKED>(yview, in && p.has_shared ? (uint32_t)((kT + t) * p.d + c) : kOffNone);
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j)
            yv[i][j] = y_view4<PACKED>(yview, in && j < p.k ? (uint32_t)((size_t)slot[j] * p.d + c) : kOffNone);
    }
    float4 v[kNormChunks];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
        const int c = threadIdx.x * 4 + 1024 * i;
        if (c >= p.d) continue;
        // residual, shared row, routed rows in pair order, as combine_kernel
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.residual) {
            acc[0] = r[i].x; acc[1] = r[i].y; acc[2] = r[i].z; acc[3] = r[i].w;
        }
        if (p.has_shared) {
            acc[0] += sh[i].x; acc[1] += sh[i].y; acc[2] += sh[i].z; acc[3] += sh[i].w;
        }
#pragma unroll
        for (int j = 0; j < kCombineMaxK; ++j) {
            if (j < p.k) {
                acc[0] += yv[i][j].x; acc[1] += yv[i][j].y; acc[2] += yv[i][j].z; acc[3] += yv[i][j].w;
            }
        }
        v[i] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        ss = fmaf(v[i].x, v[i].x, ss);
        ss = fmaf(v[i].y, v[i].y, ss);
        ss = fmaf(v[i].z, v[i].z, ss);
        ss = fmaf(v[i].w, v[i].w, ss);
    }
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
        const int c = threadIdx.x * 4 + 1024 * i;
        if (c >= p.d) break;
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (size_t)t * p.d + c) = v[i];
    }
    const float rs = rms_scale(ss, p.d, eps, s_part);
    uint16_t* orow = norm + (size_t)t * p.d;
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
        const int c = threadIdx.x * 4 + 1024 * i;
        if (c >= p.d) break;
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(v[i].x * rs) | ((uint32_t)f32_to_bf16(v[i].y * rs) << 16);
        o.y = (uint32_t)f32_to_bf16(v[i].z * rs) | ((uint32_t)f32_to_bf16(v[i].w * rs) << 16);
        *reinterpret_cast<uint2*>(orow + c) = o;
    }
}

bool combine_norm_ok(const Dims& dm) {
    // the y rows are read through one buffer view, whose offsets are 32-bit
    return dm.d % 4 == 0 && dm.d <= 1024 * kNormChunks &&
           (size_t)(dm.k + 1) * dm.T * dm.d * 4 < (size_t)kOffNone;
}

hipError_t launch_combine_norm(const LayerArgs& a, const Workspace& w, bool packed, float eps, void* norm,
                               hipStream_t s) {
    CombineParams p;
    p.T = a.dm.T;
    p.d = a.dm.d;
    p.k = a.dm.k;
    p.y = w.y;
    p.pair_pos = w.pair_pos;
    p.residual = a.residual;
    p.out = a.out;
    p.out_f32 = 1;
    p.has_shared = a.dm.fs > 0 ? 1 : 0;
    if (packed)
        hipLaunchKernelGGL(combine_norm_kernel<true>, dim3(a.dm.T), dim3(256), 0, s, p, eps,
                           static_cast<uint16_t*>(norm));
    else
        hipLaunchKernelGGL(combine_norm_kernel<false>, dim3(a.dm.T), dim3(256), 0, s, p, eps,
                           static_cast<uint16_t*>(norm));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm, unit gain: out = bf16(v / sqrt(mean(v^2) + eps)); one block per row.
// ---------------------------------------------------------------------------
// 1 / sqrt(mean + eps) from each thread's sum of squares: wave sums, then the
// four waves' sums in wave order
__device__ __forceinline__ float rms_scale(float ss, int d, float eps, float* s_part) {
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    return 1.0f / sqrtf(tot / (float)d + eps);
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(int d, const float* __restrict__ in,
                                                      float eps, uint16_t* __restrict__ out) {
    __shared__ float s_part[4];
    const float* row = in + (size_t)blockIdx.x * d;
    float ss = 0.f;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        float4 v = *reinterpret_cast<const float4*>(row + c);
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    const float r = rms_scale(ss, d, eps, s_part);
    uint16_t* orow = out + (size_t)blockIdx.x * d;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        float4 v = *reinterpret_cast<const float4*>(row + c);
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(v.x * r) | ((uint32_t)f32_to_bf16(v.y * r) << 16);
        o.y = (uint32_t)f32_to_bf16(v.z * r) | ((uint32_t)f32_to_bf16(v.w * r) << 16);
        *reinterpret_cast<uint2*>(orow + c) = o;
    }
}

hipError_t launch_rmsnorm(int T, int d, const float* in, float eps, void* out, hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, s, d, in, eps,
                       static_cast<uint16_t*>(out));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fill of n 32-bit words (workspace clearing and the debug poison).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p, n,
                       v);
    return hipGetLastError();
}

}  // namespace flint
