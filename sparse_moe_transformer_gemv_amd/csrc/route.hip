// route.hip -- router logits, top-k selection and the counting-sort token
// permutation of the MoE layer (gfx950).
//
// Selection: per token, the k largest of the E router logits, ties to the
// lower expert index; weights are the softmax of the chosen logits, i.e. the
// full softmax renormalised over the chosen k.  The pages fix 256 experts with
// 6 chosen per token [evermx.com, "Recursive Flint: Open-Weight MoE Coding
// Model, 2.5B Active", Feature Overview, "Sparse architecture"]; the softmax,
// renormalisation and tie rule are the readings this library takes where the
// pages are silent.
//
// Permutation: the k*T (token, slot) pairs are stably sorted by expert, so the
// tokens of one expert are contiguous and in token order; per-expert counts,
// offsets and the inverse map feed the expert kernels and the combine.  Ranks
// come from ballot-based matching inside each wavefront plus per-wave LDS
// histograms, so the order never depends on atomic timing.
#include "flint_internal.hpp"

namespace flint {

// ---------------------------------------------------------------------------
// Router logits for one expert row and a run of tokens: one wavefront per
// expert, lanes stride K with float4 loads, token groups of 8 accumulators.
// ---------------------------------------------------------------------------
template <typename ActT>
__device__ __forceinline__ void load_act4(const ActT* x, float v[4]);

template <>
__device__ __forceinline__ void load_act4<float>(const float* x, float v[4]) {
    float4 a = *reinterpret_cast<const float4*>(x);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

template <>
__device__ __forceinline__ void load_act4<uint16_t>(const uint16_t* x, float v[4]) {
    uint2 a = *reinterpret_cast<const uint2*>(x);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
}

template <typename ActT>
__device__ void router_row_logits(const ActT* __restrict__ x, const float* __restrict__ wrow,
                                  float b, int t_begin, int t_end, int d, int E, int e,
                                  float* __restrict__ logits, int lane) {
    constexpr int TG = 8;
    for (int t0 = t_begin; t0 < t_end; t0 += TG) {
        float acc[TG];
#pragma unroll
        for (int i = 0; i < TG; ++i) acc[i] = 0.f;
        for (int k0 = lane * 4; k0 < d; k0 += 256) {
            float4 w = *reinterpret_cast<const float4*>(wrow + k0);
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) {
                if (t0 + tt < t_end) {
                    float xv[4];
                    load_act4<ActT>(x + (size_t)(t0 + tt) * d + k0, xv);
                    float a = acc[tt];
                    a = fmaf(w.x, xv[0], a);
                    a = fmaf(w.y, xv[1], a);
                    a = fmaf(w.z, xv[2], a);
                    a = fmaf(w.w, xv[3], a);
                    acc[tt] = a;
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
            float v = wave_sum(acc[tt]);
            if (lane == 0 && t0 + tt < t_end) st_agent(logits + (size_t)(t0 + tt) * E + e, v + b);
        }
    }
}

// ---------------------------------------------------------------------------
// Top-k of one token by one wavefront.  Lane l holds logits e = l + 64 i.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float ov = __shfl_xor(v, off, 64);
        int oi = __shfl_xor(i, off, 64);
        if (ov > v || (ov == v && oi < i)) {
            v = ov;
            i = oi;
        }
    }
}

template <bool COHERENT = true>
__device__ void wave_topk_token(const float* __restrict__ lrow, int E, int k, int lane,
                                int* __restrict__ sel_out, float* __restrict__ w_out) {
    constexpr int NONE = 0x7FFFFFFF;
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        const int ec = e < E ? e : 0;  // unconditional; lanes past E never compete
        lv[i] = COHERENT ? ld_agent(lrow + ec) : lrow[ec];
    }
    unsigned taken = 0;
    float my_v = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = NONE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u)) {
                // strictly greater keeps the lower index on equal logits
                if (bi == NONE || lv[i] > bv) {
                    bv = lv[i];
                    bi = e;
                }
            }
        }
        wave_argmax(bv, bi);
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) {
            my_v = bv;
            my_e = bi;
        }
    }
    // weights: softmax over the chosen logits; slot 0 holds the largest
    float l0 = __shfl(my_v, 0, 64);
    float p = (lane < k) ? expf(my_v - l0) : 0.f;
    float s = wave_sum(p);
    if (lane < k) {
        st_agent(sel_out + lane, my_e);
        st_agent(w_out + lane, p / s);
    }
}

// Active groups from the expert offsets s_off[0..E] (LDS), written by one
// wavefront: the shared expert first (its work items are the longest, so they
// start first), then the experts with tokens in ascending order; with bm > 0
// also the prefill tile list, ceil(rows / bm) tiles per group.
__device__ void write_groups(const int* s_off, int E, int T, int k, bool has_shared, int bm, const Workspace& ws,
                             int lane) {
    const unsigned long long lt = (1ull << lane) - 1ull;
    int n = 0, ntile = 0;
    if (has_shared) {
        if (lane == 0) ws.groups[0] = make_int4(E, 0, T, k * T);
        if (bm > 0) {
            const int nt = (T + bm - 1) / bm;
            for (int t = lane; t < nt; t += 64) ws.tiles[t] = make_int2(0, t * bm);
            ntile = nt;
        }
        n = 1;
    }
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int c = (e < E) ? s_off[e + 1] - s_off[e] : 0;
        const unsigned long long act = __ballot(c > 0);
        const int gidx = n + __popcll(act & lt);
        if (c > 0) ws.groups[gidx] = make_int4(e, s_off[e], c, s_off[e]);
        if (bm > 0) {
            const int nt = (c + bm - 1) / bm;
            int inc = nt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(inc, off, 64);
                if (lane >= off) inc += v;
            }
            const int pos = ntile + inc - nt;
            for (int t = 0; t < nt; ++t) ws.tiles[pos + t] = make_int2(gidx, t * bm);
            ntile += __shfl(inc, 63, 64);
        }
        n += __popcll(act);
    }
    if (lane == 0) {
        *ws.n_groups = n;
        if (bm > 0) *ws.n_tiles = ntile;
    }
}

// ---------------------------------------------------------------------------
// Stable counting sort of P pair keys (expert ids < E <= 256) by one block.
// Writes counts[E], offsets[E+1], sorted_pair[P], pair_pos[P], sorted_wt[P]
// (from the pair weights wts), the active group list and (if bm > 0) the
// prefill tile list.
// s_hist: LDS [NW*E]; s_off: LDS [E+1].
// ---------------------------------------------------------------------------
template <int NT, bool COHERENT = true>
__device__ void block_sort_and_groups(const int* __restrict__ keys, const float* __restrict__ wts, int P, int E,
                                      int T, int k,
                                      bool has_shared, int bm, const Workspace& ws, int* s_hist,
                                      int* s_off) {
    // keys written earlier in the same kernel by other workgroups need
    // device-coherent loads; keys from an earlier kernel are read plainly
    auto key_at = [&](int i) { return COHERENT ? ld_agent(keys + i) : keys[i]; };
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const unsigned long long lt = (1ull << lane) - 1ull;

    for (int i = tid; i < NW * E; i += NT) s_hist[i] = 0;
    __syncthreads();
    const int S = (((P + NW - 1) / NW) + 63) & ~63;
    const int b0 = min(P, w * S), b1 = min(P, b0 + S);
    // keys are read KU chunks of 64 at a time so that their loads overlap
    constexpr int KU = 8;
    for (int c0 = b0; c0 < b1; c0 += 64 * KU) {
        int kv[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int i = c0 + 64 * u + lane;
            kv[u] = i < b1 ? key_at(i) : -1;
        }
#pragma unroll
        for (int u = 0; u < KU; ++u)
            if (kv[u] >= 0) atomicAdd(&s_hist[w * E + kv[u]], 1);
    }
    __syncthreads();

    // per-expert totals and their exclusive scan (wave 0; 4 experts per lane)
    if (w == 0) {
        int c[4];
        int local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = lane * 4 + i, s = 0;
            if (e < E)
                for (int ww = 0; ww < NW; ++ww) s += s_hist[ww * E + e];
            c[i] = s;
            local += s;
        }
        int inc = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int v = __shfl_up(inc, off, 64);
            if (lane >= off) inc += v;
        }
        int run = inc - local;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = lane * 4 + i;
            if (e < E) {
                s_off[e] = run;
                ws.offsets[e] = run;
                ws.counts[e] = c[i];
            }
            run += c[i];
        }
        if (lane == 63) {
            s_off[E] = inc;
            ws.offsets[E] = inc;
        }
    }
    __syncthreads();
    // turn per-wave counts into per-wave base positions
    for (int e = tid; e < E; e += NT) {
        int run = s_off[e];
        for (int ww = 0; ww < NW; ++ww) {
            int c = s_hist[ww * E + e];
            s_hist[ww * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    // ordered scatter: rank inside each 64-pair chunk by ballot matching
    for (int c0 = b0; c0 < b1; c0 += 64 * KU) {
        int kv[KU];
        float wv[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int i = c0 + 64 * u + lane;
            const int ic = i < b1 ? i : b0;
            kv[u] = i < b1 ? key_at(ic) : -1;
            wv[u] = COHERENT ? ld_agent(wts + ic) : wts[ic];
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            if (c0 + 64 * u >= b1) break;  // uniform
            const int i = c0 + 64 * u + lane;
            const bool valid = kv[u] >= 0;
            const int key = valid ? kv[u] : 0;
            unsigned long long m = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const bool bit = (key >> b) & 1;
                const unsigned long long bb = __ballot(valid && bit);
                m &= bit ? bb : ~bb;
            }
            if (valid) {
                const int pos = s_hist[w * E + key] + __popcll(m & lt);
                ws.sorted_pair[pos] = i;
                ws.pair_pos[i] = pos;
                ws.sorted_wt[pos] = wv[u];
            }
            // the highest lane of each key group advances that key's base
            if (valid && (m >> lane) == 1ull) s_hist[w * E + key] += __popcll(m);
        }
    }
    __syncthreads();

    if (w == 0) write_groups(s_off, E, T, k, has_shared, bm, ws, lane);
}


// ---------------------------------------------------------------------------
// Router on the matrix cores (bf16 activations): logits of a 16-token x
// 16-expert tile, K split over the 4 waves and summed in a fixed order.  The
// fp32 router rows are split exactly into three bf16 parts, so the bf16 MFMA
// reproduces the fp32 products (x is bf16); accumulation is fp32.  The last
// expert block of each token tile then selects the top-k of its 16 tokens, and
// (decode path) the last token tile sorts all pairs.
// Tickets: counter[0] for the sort, counter[1 + token tile] per tile.
// ---------------------------------------------------------------------------
struct RouteMfmaParams {
    const uint16_t* x;
    const float* wr;
    const float* bias;
    int T, d, E, k;
    int has_shared;
    int do_sort;  // 0: logits only (prefill: top-k and sort run as their own kernels)
    Workspace ws;
};

// 8 waves per block; wave w covers k in [w*d/8, (w+1)*d/8) in NSTEP steps of
// 32, with every load of its range issued before the first MFMA.  A block
// covers TT 16-token row tiles (the router rows are loaded once for all of
// them) and one 16-expert column tile.
template <int NSTEP, int TT>
__global__ __launch_bounds__(512) void route_mfma_kernel(RouteMfmaParams p) {
    constexpr int NW = 8;
    constexpr int TOK = 16 * TT;
    __shared__ float s_part[NW][TT * 256];
    __shared__ int s_hist[NW * 256];
    __shared__ int s_off[257];
    __shared__ int s_flag;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int t0 = blockIdx.x * TOK, e0 = blockIdx.y * 16;
    const int kbeg = wave * (32 * NSTEP);
    const int ex = e0 + row;
    const bool ex_ok = ex < p.E;
    const float* wrow = p.wr + (size_t)(ex_ok ? ex : 0) * p.d + kbeg + 8 * q;
    // unconditional loads from clamped rows, so they issue back to back;
    // rows past T or E are zeroed afterwards
    uint4 a[TT][NSTEP];
    float4 w0[NSTEP], w1[NSTEP];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int tok = t0 + 16 * tt + row;
        const uint16_t* xr = p.x + (size_t)(tok < p.T ? tok : 0) * p.d + kbeg + 8 * q;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) a[tt][s] = *reinterpret_cast<const uint4*>(xr + 32 * s);
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        w0[s] = *reinterpret_cast<const float4*>(wrow + 32 * s);
        w1[s] = *reinterpret_cast<const float4*>(wrow + 32 * s + 4);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first MFMA
    const float keep_w = ex_ok ? 1.f : 0.f;
    floatx4_t acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const uint32_t keep_a = (t0 + 16 * tt + row < p.T) ? 0xFFFFFFFFu : 0u;
        acc[tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
            a[tt][s] = make_uint4(a[tt][s].x & keep_a, a[tt][s].y & keep_a, a[tt][s].z & keep_a,
                                  a[tt][s].w & keep_a);
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        const float wv[8] = {w0[s].x * keep_w, w0[s].y * keep_w, w0[s].z * keep_w, w0[s].w * keep_w,
                             w1[s].x * keep_w, w1[s].y * keep_w, w1[s].z * keep_w, w1[s].w * keep_w};
        uint4 hi, mid, lo;
        split3_bf16(wv, hi, mid, lo);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            acc[tt] = mfma16x16x32(a[tt][s], hi, acc[tt]);
            acc[tt] = mfma16x16x32(a[tt][s], mid, acc[tt]);
            acc[tt] = mfma16x16x32(a[tt][s], lo, acc[tt]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_part[wave][tt * 256 + (4 * q + i) * 16 + row] = acc[tt][i];
    __syncthreads();
    for (int idx = tid; idx < TT * 256; idx += 512) {
        const int m = idx >> 4, n = idx & 15;  // token m of the block, expert n
        float v = s_part[0][idx];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += s_part[w][idx];
        if (t0 + m < p.T && e0 + n < p.E)
            st_agent(p.ws.logits + (size_t)(t0 + m) * p.E + e0 + n,
                     v + (p.bias ? p.bias[e0 + n] : 0.f));
    }
    if (!p.do_sort) return;
    // top-k of this token tile by the last of its expert blocks
    if (!last_arrival(&p.ws.counter[1 + blockIdx.x], (int)gridDim.y, &s_flag)) return;
    for (int m = wave; m < TOK; m += NW) {
        const int t = t0 + m;
        if (t < p.T)
            wave_topk_token(p.ws.logits + (size_t)t * p.E, p.E, p.k, lane,
                            p.ws.sel + (size_t)t * p.k, p.ws.wts + (size_t)t * p.k);
    }
    // counting sort of every pair by the last token tile
    if (!last_arrival(&p.ws.counter[0], (int)gridDim.x, &s_flag)) return;
    block_sort_and_groups<512>(p.ws.sel, p.ws.wts, p.k * p.T, p.E, p.T, p.k, p.has_shared != 0, 0, p.ws,
                               s_hist, s_off);
}

// ---------------------------------------------------------------------------
// Decode path without the matrix cores (fp32 activations, or shapes the
// matrix-core router does not take), one launch of (E / 4) x (T / 16) blocks:
// wave w of block (bx, by) computes router logit 4 bx + w of the 16 tokens of
// tile by; the last expert block of each token tile to finish stages the
// tile's logits in LDS and selects the top-k of its tokens, one wavefront per
// token, and the last token tile to finish runs the counting sort.
// ---------------------------------------------------------------------------
struct RouteDecodeParams {
    const void* x;
    const float* wr;
    const float* bias;
    int T, d, E, k;
    int has_shared;
    Workspace ws;
};

template <typename ActT>
__global__ __launch_bounds__(256) void route_decode_kernel(RouteDecodeParams p) {
    __shared__ int s_hist[4 * 256];
    __shared__ int s_off[257];
    __shared__ int s_last;
    __shared__ __attribute__((aligned(16))) float s_logit[16 * 256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = blockIdx.x * 4 + wave;
    const int t0 = blockIdx.y * 16, t1 = min(p.T, t0 + 16);
    if (e < p.E)
        router_row_logits<ActT>(static_cast<const ActT*>(p.x), p.wr + (size_t)e * p.d,
                                p.bias ? p.bias[e] : 0.f, t0, t1, p.d, p.E, e, p.ws.logits, lane);
    if (!last_arrival(p.ws.counter + 1 + blockIdx.y, (int)gridDim.x, &s_last)) return;
    {
        // the tile's logits into LDS (16-byte agent-scope loads: other blocks of
        // this launch wrote them), then one wavefront per token
        const int nt = t1 - t0;
        const uint32_t bytes = (uint32_t)(nt * p.E * 4 + 15) & ~15u;  // within the 256-byte padding
        const __amdgpu_buffer_rsrc_t lv = buffer_view(p.ws.logits + (size_t)t0 * p.E, bytes);
        uint4 lg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lg[i] = buffer_load16_agent(lv, (uint32_t)(tid + 256 * i) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = (uint32_t)(tid + 256 * i) * 16;
            if (o < bytes) *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(s_logit) + o) = lg[i];
        }
        __syncthreads();
        for (int m = wave; m < nt; m += 4) {
            const int t = t0 + m;
            int se;
            float w;
            topk_token_lds(s_logit + m * p.E, p.E, p.k, lane, &se, &w);
            if (lane < p.k) {
                st_agent(p.ws.sel + t * p.k + lane, se);
                st_agent(p.ws.wts + t * p.k + lane, w);
            }
        }
    }
    if (!last_arrival(p.ws.counter, (int)gridDim.y, &s_last)) return;
    block_sort_and_groups<256>(p.ws.sel, p.ws.wts, p.k * p.T, p.E, p.T, p.k, p.has_shared != 0, 0, p.ws,
                               s_hist, s_off);
}

hipError_t launch_route_decode(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    RouteDecodeParams p{a.x, a.wr, a.bias, a.dm.T, a.dm.d, a.dm.E, a.dm.k, a.dm.fs > 0, w};
    dim3 grid((a.dm.E + 3) / 4, (a.dm.T + 15) / 16);
    if (a.dm.act == DT_F32)
        hipLaunchKernelGGL(route_decode_kernel<float>, grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(route_decode_kernel<uint16_t>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// Stable counting sort of the P = k T pairs (T <= 64) by one block of 512
// threads, from their experts and weights in LDS, with the decode lists of
// block_sort_and_groups as results.  A token picks an expert at most once, so
// a 64-bit mask of the tokens that picked each expert gives its count (the
// population) and each pair's rank among that expert's pairs (the tokens
// below its own): one LDS OR per pair, one scan by wave 0 over four experts
// per lane (offsets and the group list together), one placement per pair.
__device__ void mask_sort_small(const int* s_key, const float* s_w, int P, int E, int T, int k, bool has_shared,
                                const Workspace& ws, unsigned long long* s_mask, int* s_off) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < E; i += 512) s_mask[i] = 0ull;
    __syncthreads();
    if (tid < P) atomicOr(&s_mask[s_key[tid]], 1ull << (tid / k));
    __syncthreads();
    if (wave == 0) {
        int c[4], local = 0, nact = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            c[i] = e < E ? __popcll(s_mask[e]) : 0;
            local += c[i];
            nact += c[i] > 0 ? 1 : 0;
        }
        // (pairs, active experts) up to this lane, packed: at most 512 and 256
        const int inc = wave_incl_scan(local | (nact << 16));
        int run = (inc & 0xFFFF) - local;
        int gi = (has_shared ? 1 : 0) + (inc >> 16) - nact;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) {
                s_off[e] = run;
                ws.offsets[e] = run;
                ws.counts[e] = c[i];
            }
            if (c[i] > 0) ws.groups[gi++] = make_int4(e, run, c[i], run);
            run += c[i];
        }
        if (lane == 63) {
            ws.offsets[E] = inc & 0xFFFF;
            *ws.n_groups = (has_shared ? 1 : 0) + (inc >> 16);
        }
        if (lane == 0 && has_shared) ws.groups[0] = make_int4(E, 0, T, P);
    }
    __syncthreads();
    if (tid < P) {
        const int e = s_key[tid];
        const int pos = s_off[e] + __popcll(s_mask[e] & ((1ull << (tid / k)) - 1ull));
        ws.sorted_pair[pos] = tid;
        ws.pair_pos[tid] = pos;
        ws.sorted_wt[pos] = s_w[tid];
    }
}

constexpr int kRouteSplitMaxT = 64;

// ---------------------------------------------------------------------------
// Decode router for T <= 64, in one launch of (d/256) x (E/16) x (T/16)
// blocks and four stages handed on by tickets:
//   1. block (kc, et, tt) computes the partial logits of the 16 tokens of
//      tile tt and the 16 experts of tile et over k in [256 kc, 256 kc + 256)
//      (8 waves, one 32-wide MFMA step each) into rpart[kc];
//   2. the last k-chunk block of (et, tt) sums the d/256 partials in kc order
//      (so the result does not depend on timing) and adds the bias;
//   3. the last expert tile of token tile tt stages the tile's logits in LDS
//      and selects the top-k of its tokens, one wavefront per token;
//   4. the last token tile sorts every pair (mask_sort_small).
// Spreading the 2 MB of fp32 router rows over >= 128 blocks keeps enough loads
// in flight (a block per 16 experts would be bound by one CU's miss queue),
// and spreading the selection over token tiles keeps it off one CU.
// ---------------------------------------------------------------------------
template <int NS>  // NS = d / 256 k-chunks
__global__ __launch_bounds__(512) void route_splitk_kernel(RouteMfmaParams p) {
    constexpr int NW = 8;
    __shared__ float s_part[NW][256];
    __shared__ __attribute__((aligned(16))) float s_logit[16 * 256];
    __shared__ unsigned long long s_mask[256];
    __shared__ int s_off[257];
    __shared__ int s_sel[kRouteSplitMaxT * 8];
    __shared__ float s_wt[kRouteSplitMaxT * 8];
    __shared__ int s_flag;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, q = lane >> 4;
    const int E = p.E, d = p.d, T = p.T;
    const int NE = (E + 15) / 16, ntt = (T + 15) / 16, npairs = NS * NE;
    // block -> (k-chunk, expert tile) pair and token tile; when the pairs
    // divide into the 8 XCDs, the token tiles of one pair get ids equal mod 8
    // (one XCD, so its router rows are fetched into one L2)
    int pair, tt;
    if (npairs % 8 == 0) {
        const int slot = blockIdx.x >> 3;
        pair = (slot / ntt) * 8 + (blockIdx.x & 7);
        tt = slot % ntt;
    } else {
        pair = blockIdx.x / ntt;
        tt = blockIdx.x % ntt;
    }
    const int kc = pair % NS, et = pair / NS, e0 = et * 16, t0 = tt * 16;
    const int kl = kc * 256 + wave * 32 + 8 * q;
    // 1. partial logits; router rows past E and tokens past T read as zeros
    const __amdgpu_buffer_rsrc_t wv = buffer_view(p.wr, (uint32_t)E * d * 4);
    const uint32_t wo = e0 + row < E ? (uint32_t)((e0 + row) * d + kl) * 4 : kOffNone;
    const uint4 w0 = buffer_load16(wv, wo), w1 = buffer_load16(wv, wo + 16);
    const __amdgpu_buffer_rsrc_t xv = buffer_view(p.x, (uint32_t)T * d * 2);
    const int tok = t0 + row;
    const uint4 a = buffer_load16(xv, tok < T ? (uint32_t)(tok * d + kl) * 2 : kOffNone);
    const float wf[8] = {__uint_as_float(w0.x), __uint_as_float(w0.y), __uint_as_float(w0.z),
                         __uint_as_float(w0.w), __uint_as_float(w1.x), __uint_as_float(w1.y),
                         __uint_as_float(w1.z), __uint_as_float(w1.w)};
    uint4 hi, mid, lo;
    split3_bf16(wf, hi, mid, lo);
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma16x16x32(a, hi, acc);
    acc = mfma16x16x32(a, mid, acc);
    acc = mfma16x16x32(a, lo, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[wave][(4 * q + i) * 16 + row] = acc[i];
    __syncthreads();
    const int m = tid >> 4, n = tid & 15;  // token t0 + m, expert e0 + n (first 256 threads)
    const bool mine = tid < 256 && t0 + m < T && e0 + n < E;
    const size_t o = (size_t)(t0 + m) * E + e0 + n;
    if (mine) {
        float v = s_part[0][tid];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += s_part[w][tid];
        st_agent(p.ws.rpart + (size_t)kc * kRouteSplitMaxT * E + o, v);
    }
    // 2. the last k-chunk block of (et, tt) finishes these logits
    if (!last_arrival(&p.ws.rcount[tt * NE + et], NS, &s_flag)) return;
    if (mine) {
        float pv[NS];
#pragma unroll
        for (int c = 0; c < NS; ++c) pv[c] = ld_agent(p.ws.rpart + (size_t)c * kRouteSplitMaxT * E + o);
        float v = pv[0];
#pragma unroll
        for (int c = 1; c < NS; ++c) v += pv[c];
        st_agent(p.ws.logits + o, v + (p.bias ? p.bias[e0 + n] : 0.f));
    }
    // 3. the last expert tile of token tile tt selects its tokens' experts:
    //    the tile's logits into LDS (16-byte agent-scope loads, all issued
    //    before the first LDS store), then one wavefront per token
    if (!last_arrival(&p.ws.rcount[ntt * NE + tt], NE, &s_flag)) return;
    {
        const int nt = min(16, T - t0);
        // rounded up within the logits buffer's 256-byte padding
        const uint32_t bytes = (uint32_t)(nt * E * 4 + 15) & ~15u;
        const __amdgpu_buffer_rsrc_t lv = buffer_view(p.ws.logits + (size_t)t0 * E, bytes);
        uint4 lg[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) lg[i] = buffer_load16_agent(lv, (uint32_t)(tid + 512 * i) * 16);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t o = (uint32_t)(tid + 512 * i) * 16;
            if (o < bytes) *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(s_logit) + o) = lg[i];
        }
        __syncthreads();
        for (int m = wave; m < nt; m += NW) {
            const int t = t0 + m;
            int e;
            float w;
            topk_token_lds(s_logit + m * E, E, p.k, lane, &e, &w);
            if (lane < p.k) {
                st_agent(p.ws.sel + t * p.k + lane, e);
                st_agent(p.ws.wts + t * p.k + lane, w);
                s_sel[t * p.k + lane] = e;
                s_wt[t * p.k + lane] = w;
            }
        }
    }
    // 4. the last token tile sorts every pair (its own tile's from LDS; with
    //    several tiles the others' selections are read back first)
    const int P = p.k * T;
    if (ntt > 1) {
        if (!last_arrival(&p.ws.rcount[ntt * NE + ntt], ntt, &s_flag)) return;
        for (int i = tid; i < P; i += 512) {
            const int t = i / p.k;
            if (t < t0 || t >= t0 + 16) {
                s_sel[i] = ld_agent(p.ws.sel + i);
                s_wt[i] = ld_agent(p.ws.wts + i);
            }
        }
    }
    __syncthreads();
    mask_sort_small(s_sel, s_wt, P, E, T, p.k, p.has_shared != 0, p.ws, s_mask, s_off);
}

bool route_mfma_ok(const Dims& dm) {
    const int ns = dm.d / 256;
    return dm.act == DT_BF16 && dm.d % 256 == 0 && (ns == 1 || ns == 2 || ns == 4 || ns == 8);
}

hipError_t launch_route_mfma(const LayerArgs& a, const Workspace& w, bool do_sort, hipStream_t s) {
    RouteMfmaParams p{static_cast<const uint16_t*>(a.x), a.wr, a.bias, a.dm.T, a.dm.d, a.dm.E,
                      a.dm.k, a.dm.fs > 0, do_sort ? 1 : 0, w};
    if (do_sort && a.dm.T <= kRouteSplitMaxT && a.dm.E <= 256 && a.dm.k <= 8) {
        dim3 grid((a.dm.d / 256) * ((a.dm.E + 15) / 16) * ((a.dm.T + 15) / 16));
        switch (a.dm.d / 256) {
        case 1: hipLaunchKernelGGL((route_splitk_kernel<1>), grid, dim3(512), 0, s, p); break;
        case 2: hipLaunchKernelGGL((route_splitk_kernel<2>), grid, dim3(512), 0, s, p); break;
        case 4: hipLaunchKernelGGL((route_splitk_kernel<4>), grid, dim3(512), 0, s, p); break;
        default: hipLaunchKernelGGL((route_splitk_kernel<8>), grid, dim3(512), 0, s, p); break;
        }
        return hipGetLastError();
    }
    const bool wide = a.dm.T > 64;  // prefill-sized: 64-token blocks share router loads
    const int tok = wide ? 64 : 16;
    dim3 grid((a.dm.T + tok - 1) / tok, (a.dm.E + 15) / 16);
#define FLINT_ROUTE_LAUNCH(NS)                                                                \
    if (wide) hipLaunchKernelGGL((route_mfma_kernel<NS, 4>), grid, dim3(512), 0, s, p);        \
    else hipLaunchKernelGGL((route_mfma_kernel<NS, 1>), grid, dim3(512), 0, s, p);
    switch (a.dm.d / 256) {
    case 1: FLINT_ROUTE_LAUNCH(1) break;
    case 2: FLINT_ROUTE_LAUNCH(2) break;
    case 4: FLINT_ROUTE_LAUNCH(4) break;
    default: FLINT_ROUTE_LAUNCH(8) break;
    }
#undef FLINT_ROUTE_LAUNCH
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill path: logits (token blocks x expert blocks), top-k (a wave per
// token), then one block sorts.
// ---------------------------------------------------------------------------
constexpr int kLogitTokensPerBlock = 64;

template <typename ActT>
__global__ __launch_bounds__(256) void router_logits_kernel(RouteDecodeParams p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wave;
    const int t0 = blockIdx.y * kLogitTokensPerBlock;
    const int t1 = min(p.T, t0 + kLogitTokensPerBlock);
    if (e < p.E)
        router_row_logits<ActT>(static_cast<const ActT*>(p.x), p.wr + (size_t)e * p.d,
                                p.bias ? p.bias[e] : 0.f, t0, t1, p.d, p.E, e, p.ws.logits, lane);
}

hipError_t launch_router_logits(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    RouteDecodeParams p{a.x, a.wr, a.bias, a.dm.T, a.dm.d, a.dm.E, a.dm.k, a.dm.fs > 0, w};
    dim3 grid((a.dm.E + 3) / 4, (a.dm.T + kLogitTokensPerBlock - 1) / kLogitTokensPerBlock);
    if (a.dm.act == DT_F32)
        hipLaunchKernelGGL(router_logits_kernel<float>, grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(router_logits_kernel<uint16_t>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill router logits as a tiled GEMM.  The fp32 router is first split
// exactly into three bf16 planes (hi + mid + lo, once per forward), so bf16
// MFMAs against the bf16 activations reproduce the fp32 products; the three
// planes are accumulated in fp32 in the same k order.  Tiles of 64 tokens x
// 64 experts are staged through LDS with coalesced row loads (an MFMA operand
// loaded straight from global memory would put 16 different rows in each
// load instruction, which the vector L1 serves one lane at a time).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr, uint16_t* __restrict__ w3,
                                                           size_t n) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= n) return;
    const float4 a = *reinterpret_cast<const float4*>(wr + i);
    const float4 b = *reinterpret_cast<const float4*>(wr + i + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint4 hi, mid, lo;
    split3_bf16(v, hi, mid, lo);
    *reinterpret_cast<uint4*>(w3 + i) = hi;
    *reinterpret_cast<uint4*>(w3 + n + i) = mid;
    *reinterpret_cast<uint4*>(w3 + 2 * n + i) = lo;
}

struct RouterGemmParams {
    const uint16_t* x;
    const uint16_t* w3;
    const float* bias;
    float* logits;
    int T, d, E;
};

constexpr int kRgBN = 64, kRgBK = 64;
constexpr int kRgPlaneBytes = kRgBN * kRgBK * 2;  // 8 KiB per router plane per stage
constexpr int kRgThreads = 512;                   // 8 waves: 2 (tokens) x 4 (16 experts each)
template <int BM>
struct RgTile {
    static constexpr int ABytes = BM * kRgBK * 2;
    static constexpr int StageBytes = ABytes + 3 * kRgPlaneBytes;
    static constexpr int AChunks = BM * 8 / kRgThreads;  // 16-byte A chunks per thread per stage
    static constexpr int BChunks = 3 * kRgBN * 8 / kRgThreads;
    static constexpr int Chunks = AChunks + BChunks;
    static constexpr int MI = BM / 32;  // 16-row A fragments per wave (2 waves along M)
};

// byte offset of 16-byte chunk c of 128-byte LDS row r (chunks XOR-swizzled by row)
__device__ __forceinline__ int rg_swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// One K step: refill rega with stage s + 2 (clamped: unconditional loads keep
// the staging registers in registers), multiply LDS stage s, move regb (stage
// s + 1) into the other LDS buffer, which nobody reads until after the barrier.
template <int BM>
__device__ __forceinline__ void router_gemm_step(int s, int nk, const uint16_t* const (&src)[RgTile<BM>::Chunks],
                                                 const int (&dst)[RgTile<BM>::Chunks], unsigned char* lds, int wm,
                                                 int wn, int row16, int q, u32x4_t (&rega)[RgTile<BM>::Chunks],
                                                 const u32x4_t (&regb)[RgTile<BM>::Chunks],
                                                 floatx4_t (&acc)[RgTile<BM>::MI]) {
    using TL = RgTile<BM>;
    const int s2 = s + 2 < nk ? s + 2 : nk - 1;
#pragma unroll
    for (int i = 0; i < TL::Chunks; ++i) rega[i] = *reinterpret_cast<const u32x4_t*>(src[i] + s2 * kRgBK);
    __builtin_amdgcn_sched_barrier(0);  // these loads go out before anything else in the step
    const unsigned char* buf = lds + (s & 1) * TL::StageBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int c = 4 * ks + q;
        uint4 a[TL::MI], b[3];
#pragma unroll
        for (int i = 0; i < TL::MI; ++i)
            a[i] = *reinterpret_cast<const uint4*>(buf + rg_swz((BM / 2) * wm + 16 * i + row16, c));
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
            b[pl] = *reinterpret_cast<const uint4*>(buf + TL::ABytes + pl * kRgPlaneBytes + rg_swz(16 * wn + row16, c));
#pragma unroll
        for (int i = 0; i < TL::MI; ++i)
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) acc[i] = mfma16x16x32(a[i], b[pl], acc[i]);
    }
    unsigned char* nbuf = lds + ((s + 1) & 1) * TL::StageBytes;
#pragma unroll
    for (int i = 0; i < TL::Chunks; ++i) *reinterpret_cast<u32x4_t*>(nbuf + dst[i]) = regb[i];
    // a barrier for the LDS alone: __syncthreads() would also wait for the
    // loads of stage s + 2 issued above (vmcnt 0), which defeats the prefetch
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's LDS reads and writes are done
    barrier_keep_loads();
}

// Block = BM tokens x 64 experts, 8 waves as 2 (tokens) x 4 (16 experts).
template <int BM>
__global__ __launch_bounds__(kRgThreads) void router_gemm_kernel(RouterGemmParams p) {
    using TL = RgTile<BM>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * TL::StageBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int row16 = lane & 15, q = lane >> 4;
    const int t0 = blockIdx.x * BM, e0 = blockIdx.y * kRgBN;
    const int d = p.d;
    const size_t plane = (size_t)p.E * d;
    // this thread's chunks of a stage: AChunks of A (x rows), then BChunks of
    // the router planes; chunk id c -> row c >> 3, 16-byte column c & 7 (8
    // threads per row)
    const uint16_t* src[TL::Chunks];
    int dst[TL::Chunks];
#pragma unroll
    for (int i = 0; i < TL::Chunks; ++i) {
        if (i < TL::AChunks) {
            const int c = tid + kRgThreads * i;
            const int r = c >> 3, col = c & 7;
            const int t = t0 + r < p.T ? t0 + r : p.T - 1;  // rows past T repeat a valid row; never stored
            src[i] = p.x + (size_t)t * d + 8 * col;
            dst[i] = rg_swz(r, col);
        } else {
            const int c = tid + kRgThreads * (i - TL::AChunks);  // over the 3 planes' 3 x 64 rows
            const int pr = c >> 3, col = c & 7;
            const int pl = pr / kRgBN, r = pr % kRgBN;
            const int e = e0 + r < p.E ? e0 + r : p.E - 1;
            src[i] = p.w3 + pl * plane + (size_t)e * d + 8 * col;
            dst[i] = TL::ABytes + pl * kRgPlaneBytes + rg_swz(r, col);
        }
    }
    // two register stages in flight ahead of the LDS stage being multiplied
    const int nk = d / kRgBK;
    u32x4_t st0[TL::Chunks], st1[TL::Chunks];
#pragma unroll
    for (int i = 0; i < TL::Chunks; ++i) st0[i] = *reinterpret_cast<const u32x4_t*>(src[i]);
#pragma unroll
    for (int i = 0; i < TL::Chunks; ++i) st1[i] = *reinterpret_cast<const u32x4_t*>(src[i] + (nk > 1 ? kRgBK : 0));
#pragma unroll
    for (int i = 0; i < TL::Chunks; ++i) *reinterpret_cast<u32x4_t*>(lds + dst[i]) = st0[i];
    __syncthreads();
    floatx4_t acc[TL::MI];
#pragma unroll
    for (int i = 0; i < TL::MI; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nk; s += 2) {  // nk is even
        router_gemm_step<BM>(s, nk, src, dst, lds, wm, wn, row16, q, st0, st1, acc);
        router_gemm_step<BM>(s + 1, nk, src, dst, lds, wm, wn, row16, q, st1, st0, acc);
    }
    const int e = e0 + 16 * wn + row16;
    if (e < p.E) {
        const float b = p.bias ? p.bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < TL::MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + (BM / 2) * wm + 16 * i + 4 * q + r;
                if (t < p.T) p.logits[(size_t)t * p.E + e] = acc[i][r] + b;
            }
    }
}

constexpr int kRgBM = 64;  // tokens per block (32 doubles the router bytes per token and is slower)

bool router_gemm_ok(const Dims& dm) {
    return dm.act == DT_BF16 && dm.d % (2 * kRgBK) == 0 && (size_t)3 * dm.E * dm.d < ((size_t)1 << 31);
}

hipError_t launch_router_gemm(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    const size_t n = (size_t)a.dm.E * a.dm.d;  // d % 64 == 0, so n % 8 == 0
    hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s, a.wr, w.w3, n);
    RouterGemmParams p{static_cast<const uint16_t*>(a.x), w.w3, a.bias, w.logits, a.dm.T, a.dm.d, a.dm.E};
    dim3 grid((a.dm.T + kRgBM - 1) / kRgBM, (a.dm.E + kRgBN - 1) / kRgBN);
    hipLaunchKernelGGL(router_gemm_kernel<kRgBM>, grid, dim3(kRgThreads), 0, s, p);
    return hipGetLastError();
}

// Prefill top-k: 8 waves per block, two tokens per wave (16 per block).  The
// block also counts its chosen experts (Workspace::bhist row blockIdx.x), so
// the sort reads 16-token block counts instead of counting every pair again.
__global__ __launch_bounds__(512) void topk_kernel(RouteDecodeParams p) {
    // the block's 16 logit rows into LDS (16-byte loads, all issued before the
    // first LDS store), then one wavefront per token (topk_token_lds)
    __shared__ __attribute__((aligned(16))) float s_logit[16 * 256];
    __shared__ int s_hist[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * 16, nt = min(16, p.T - t0);
    // rounded up within the logits buffer's 256-byte padding
    const uint32_t bytes = (uint32_t)(nt * p.E * 4 + 15) & ~15u;
    const __amdgpu_buffer_rsrc_t lv = buffer_view(p.ws.logits + (size_t)t0 * p.E, bytes);
    uint4 lg[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) lg[i] = buffer_load16(lv, (uint32_t)(tid + 512 * i) * 16);
    if (tid < 256) s_hist[tid] = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t o = (uint32_t)(tid + 512 * i) * 16;
        if (o < bytes) *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(s_logit) + o) = lg[i];
    }
    __syncthreads();
    for (int m = wave; m < nt; m += 8) {
        const int t = t0 + m;
        int e;
        float w;
        topk_token_lds(s_logit + m * p.E, p.E, p.k, lane, &e, &w);
        if (lane < p.k) {
            p.ws.sel[t * p.k + lane] = e;
            p.ws.wts[t * p.k + lane] = w;
            atomicAdd(&s_hist[e], 1);
        }
    }
    __syncthreads();
    if (tid < 256) p.ws.bhist[(size_t)blockIdx.x * 256 + tid] = s_hist[tid];
}

hipError_t launch_topk(const LayerArgs& a, const Workspace& w, hipStream_t s) {
    RouteDecodeParams p{a.x, a.wr, a.bias, a.dm.T, a.dm.d, a.dm.E, a.dm.k, a.dm.fs > 0, w};
    hipLaunchKernelGGL(topk_kernel, dim3((a.dm.T + 15) / 16), dim3(512), 0, s, p);
    return hipGetLastError();
}

struct SortParams {
    int T, E, k, has_shared, bm;
    int cb;  // 16-token top-k blocks per sort block
    Workspace ws;
};

// ---------------------------------------------------------------------------
// Prefill counting sort, one launch.  Sort block b places the pairs of the
// top-k blocks [cb b, cb (b + 1)) (cb 16-token blocks, 16 k cb <= kSortBlock
// pairs, one per thread).  The per-expert counts come from the top-k blocks'
// own counts (Workspace::bhist, rows of 256): the pairs in earlier blocks give each
// expert's start for this block, all of them the totals, so no pair key is
// read twice and no hand-off between blocks is needed.  The block's own pairs
// are ranked among equal keys by ballots over the 8 key bits, then placed in
// wave order.  The order is stable (pairs of one expert keep pair order), so
// the result does not depend on timing.  Block 0 also writes the counts,
// offsets, group list and tile list.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSortBlock) void sort_kernel(SortParams p) {
    constexpr int NW = kSortBlock / 64, U = 16;
    __shared__ int s_cnt[NW][2][256];  // per wave's rows of the block counts: pairs before this block, all pairs
    __shared__ int s_base[NW][256];    // per wave: this block's pairs per expert, then their first positions
    __shared__ int s_tot[256];
    __shared__ int s_before[256];
    __shared__ int s_off[257];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int E = p.E, P = p.k * p.T, b = (int)blockIdx.x;
    const int nblk = (p.T + 15) / 16, first_blk = b * p.cb, pb = p.cb * 16 * p.k;
    for (int j = tid; j < NW * 256; j += kSortBlock) (&s_base[0][0])[j] = 0;
    // this block's own pair, requested before the block counts
    const int i = b * pb + tid;
    const bool valid = tid < pb && i < P;
    const int key = valid ? p.ws.sel[i] : 0;
    const float wt = valid ? p.ws.wts[i] : 0.f;
    {
        // wave w sums the count rows w, w + NW, ...; lane: experts 4 lane .. + 3
        // (16-byte loads of rows 256 entries long, U in flight)
        int4 before = make_int4(0, 0, 0, 0), tot = make_int4(0, 0, 0, 0);
        for (int c0 = w; c0 < nblk; c0 += NW * U) {
            int4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + NW * u;
                v[u] = c < nblk ? *reinterpret_cast<const int4*>(p.ws.bhist + (size_t)c * 256 + 4 * lane)
                                : make_int4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                tot.x += v[u].x;
                tot.y += v[u].y;
                tot.z += v[u].z;
                tot.w += v[u].w;
                if (c0 + NW * u < first_blk) {
                    before.x += v[u].x;
                    before.y += v[u].y;
                    before.z += v[u].z;
                    before.w += v[u].w;
                }
            }
        }
        *reinterpret_cast<int4*>(&s_cnt[w][0][4 * lane]) = before;
        *reinterpret_cast<int4*>(&s_cnt[w][1][4 * lane]) = tot;
    }
    __syncthreads();
    // lanes of this wave holding the same expert as this lane
    unsigned long long m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool set = (key >> bit) & 1;
        const unsigned long long bb = __ballot(valid && set);
        m &= set ? bb : ~bb;
    }
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    // the highest lane of each group of equal keys records its size
    if (valid && (m >> lane) == 1ull) s_base[w][key] = __popcll(m);
    if (tid < E) {
        int before = 0, tot = 0;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            before += s_cnt[q][0][tid];
            tot += s_cnt[q][1][tid];
        }
        s_before[tid] = before;
        s_tot[tid] = tot;
    }
    __syncthreads();
    // exclusive scan of the totals (wave 0, 4 experts per lane)
    if (w == 0) {
        int c[4], local = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * lane + q;
            c[q] = e < E ? s_tot[e] : 0;
            local += c[q];
        }
        int inc = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(inc, off, 64);
            if (lane >= off) inc += v;
        }
        int run = inc - local;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * lane + q;
            if (e < E) {
                s_off[e] = run;
                if (b == 0) {
                    p.ws.offsets[e] = run;
                    p.ws.counts[e] = c[q];
                }
            }
            run += c[q];
        }
        if (lane == 63) {
            s_off[E] = inc;
            if (b == 0) p.ws.offsets[E] = inc;
        }
    }
    __syncthreads();
    // first position of each (wave, expert) of this block, in wave order
    if (tid < E) {
        int run = s_off[tid] + s_before[tid];
        for (int ww = 0; ww < NW; ++ww) {
            const int c = s_base[ww][tid];
            s_base[ww][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    if (valid) {
        const int pos = s_base[w][key] + rank;
        p.ws.sorted_pair[pos] = i;
        p.ws.pair_pos[i] = pos;
        p.ws.sorted_wt[pos] = wt;
    }
    if (b == 0 && w == 0) write_groups(s_off, E, p.T, p.k, p.has_shared != 0, p.bm, p.ws, lane);
}

// Needs the top-k kernel's block counts (launch_topk) of the same batch.
hipError_t launch_sort(const LayerArgs& a, const Workspace& w, int bm, hipStream_t s) {
    const int cb = kSortBlock / (16 * a.dm.k);  // k <= 8, so cb >= 8
    SortParams p{a.dm.T, a.dm.E, a.dm.k, a.dm.fs > 0, bm, cb, w};
    const int nblk = (a.dm.T + 15) / 16;
    const dim3 grid((nblk + cb - 1) / cb);
    hipLaunchKernelGGL(sort_kernel, grid, dim3(kSortBlock), 0, s, p);
    return hipGetLastError();
}

}  // namespace flint
