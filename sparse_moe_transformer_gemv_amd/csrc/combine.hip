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
// deterministic; no atomics.
#include "flint_internal.hpp"

namespace flint {

struct CombineParams {
    int T, d, k;
    const void* y;        // fp32 or bf16 rows, see y_bf16
    const int* pair_pos;  // [T][k]
    const float* residual;
    void* out;
    int out_f32;     // 1: fp32 out (act fp32, or residual given); 0: bf16 out
    int has_shared;  // 0: no shared expert (f_s = 0); its slots are never written
};

template <bool YBF16>
__device__ __forceinline__ void load_y4(const void* y, size_t row, int d, int c, float v[4]) {
    if constexpr (YBF16) {
        uint2 a = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(y) + row * d + c);
        v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    } else {
        float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(y) + row * d + c);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    }
}

template <bool YBF16>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= p.d) return;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.residual) {
        float4 r = *reinterpret_cast<const float4*>(p.residual + (size_t)t * p.d + c);
        acc[0] = r.x; acc[1] = r.y; acc[2] = r.z; acc[3] = r.w;
    }
    float v[4];
    const size_t kT = (size_t)p.k * p.T;
    if (p.has_shared) {
        load_y4<YBF16>(p.y, kT + t, p.d, c, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += v[i];
    }
    for (int j = 0; j < p.k; ++j) {
        const int slot = p.pair_pos[(size_t)t * p.k + j];
        load_y4<YBF16>(p.y, (size_t)slot, p.d, c, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += v[i];
    }
    if (p.out_f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (size_t)t * p.d + c) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + (size_t)t * p.d + c) = o;
    }
}

hipError_t launch_combine(const LayerArgs& a, const Workspace& w, bool y_bf16, hipStream_t s) {
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
    dim3 grid((a.dm.d + 1023) / 1024, a.dm.T);
    if (y_bf16) hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm, unit gain: out = bf16(v / sqrt(mean(v^2) + eps)); one block per row.
// ---------------------------------------------------------------------------
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
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
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

}  // namespace flint
