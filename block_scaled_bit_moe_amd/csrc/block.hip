// block.hip -- the steps either side of the MoE layer, which make the call a
// whole MoE block: the RMSNorm in front (nextsycl README, dense 27B engine: a
// norm that emits the next kernel's input; knivesysl README, "how it works":
// RMS fused into the quantisation), the router scores with top-k fused into
// the same launch (Strata docs/INTEL.md, "Decode round 2" and "Planned":
// scores + top-k as one graph node), and the residual add, which the layer's
// combine does before its single rounding.
//
// router_kernel: workgroup b computes the scores of router rows 4b .. 4b+3,
// one row per wave, for every token.  The tokens' activations are staged in
// LDS in batches; with NORM each workgroup normalises them itself (the same
// arithmetic in every workgroup, so every copy is bitwise the same) and
// workgroup 0 writes them out for the layer.  A row's 64 lanes take 16-byte
// pieces of it, 4 bf16 pairs per token each (dot2, fp32), reduced in a fixed
// order.  For up to 16 tokens the last workgroup to finish (an agent-scope
// counter in the workspace header, reset by that workgroup) ranks the scores:
// one wave per token, the routing of the decode kernels.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moeq {

constexpr int BK_THREADS = 256;
constexpr int BK_MAX_TB = 16;                    // tokens per staged batch
constexpr size_t BK_LDS = 64 * 1024;             // staged activations (bf16)

// Sum over the 256 threads in a fixed order: each wave's DPP sum (valid in
// every lane), then the four wave sums in order.
__device__ inline float bk_block_sum(float v, float *s_tmp) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    v = group_sum_dpp(v, 64);
    if (lane == 0) s_tmp[wv] = v;
    __syncthreads();
    const float r = ((s_tmp[0] + s_tmp[1]) + s_tmp[2]) + s_tmp[3];
    __syncthreads();
    return r;
}

// 1 / sqrt(mean of the squares of row x + eps), the mean in fp32 over the
// 256 threads' partial sums (thread i sums elements i, i + 256, ... in order)
__device__ inline float bk_inv_rms(const uint16_t *x, int H, float eps, float *s_tmp) {
    float ss = 0.f;
    for (int j = threadIdx.x; j < H; j += BK_THREADS) {
        const float v = bf16_to_f32(x[j]);
        ss = __builtin_fmaf(v, v, ss);
    }
    const float tot = bk_block_sum(ss, s_tmp);
    return 1.0f / __builtin_sqrtf(tot / (float)H + eps);
}

// y = x * g * r for one row (bf16 out, or fp32)
__global__ __launch_bounds__(BK_THREADS) void rmsnorm_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ g, int H, float eps,
                                                            void *__restrict__ y, int out_f32) {
    __shared__ float s_tmp[4];
    const uint16_t *xt = x + (int64_t)blockIdx.x * H;
    const float r = bk_inv_rms(xt, H, eps, s_tmp);
    for (int j = threadIdx.x; j < H; j += BK_THREADS) {
        const float v = (bf16_to_f32(xt[j]) * bf16_to_f32(g[j])) * r;
        const int64_t o = (int64_t)blockIdx.x * H + j;
        if (out_f32) reinterpret_cast<float *>(y)[o] = v;
        else reinterpret_cast<uint16_t *>(y)[o] = f32_to_bf16_rne(v);
    }
}

struct RouterArgs {
    const uint16_t *x;        // bf16 [T][H]: the activation (NORM: the residual stream)
    const uint16_t *gamma;    // bf16 [H] (NORM)
    const uint16_t *wr;       // bf16 [E][H]
    float eps;
    int T, H, E, k;
    int tb;                   // tokens per staged batch
    uint16_t *xn_out;         // bf16 [T][H] normalised activation (NORM; written by workgroup 0)
    float *logits;            // fp32 [T][E]
    int32_t *idx;             // [T][k] (fused top-k; nullable)
    float *w;                 // [T][k]
    u32 *counter;             // arrival counter (fused top-k), zero between calls
    int fused;
};

template <int PER_LANE>
__device__ inline void bk_route_tokens(const RouterArgs &a) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int t = wv; t < a.T; t += BK_THREADS / 64) {
        int e;
        float wt;
        route_one_token_wave<PER_LANE>(a.logits + (int64_t)t * a.E, a.E, a.k, lane, e, wt);
        if (lane < a.k) {
            if (a.idx) a.idx[(int64_t)t * a.k + lane] = e;
            if (a.w) a.w[(int64_t)t * a.k + lane] = wt;
        }
    }
}

template <bool NORM>
__global__ __launch_bounds__(BK_THREADS) void router_kernel(RouterArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t s_x[];   // [tb][H]
    __shared__ float s_tmp[4];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, E = a.E;
    const int e = blockIdx.x * 4 + wv;
    const uint16_t *wrow = a.wr + (int64_t)min(e, E - 1) * H;
    for (int t0 = 0; t0 < a.T; t0 += a.tb) {
        const int tb = min(a.tb, a.T - t0);
        // stage the batch (16-byte pieces; H is a multiple of 32)
        for (int q = tid; q < tb * (H / 8); q += BK_THREADS) {
            const int t = q / (H / 8), c = q - t * (H / 8);
            *reinterpret_cast<uint4 *>(s_x + t * H + 8 * c) =
                *reinterpret_cast<const uint4 *>(a.x + (int64_t)(t0 + t) * H + 8 * c);
        }
        __syncthreads();
        if (NORM) {
            for (int t = 0; t < tb; ++t) {
                uint16_t *row = s_x + t * H;
                const float r = bk_inv_rms(row, H, a.eps, s_tmp);
                for (int j = tid; j < H; j += BK_THREADS) {
                    const uint16_t v = f32_to_bf16_rne((bf16_to_f32(row[j]) * bf16_to_f32(a.gamma[j])) * r);
                    row[j] = v;
                    if (blockIdx.x == 0 && a.xn_out) a.xn_out[(int64_t)(t0 + t) * H + j] = v;
                }
            }
            __syncthreads();
        }
        // scores of row e for the batch: lane l takes the 16-byte pieces l, l + 64, ...
        float acc[BK_MAX_TB];
#pragma unroll
        for (int t = 0; t < BK_MAX_TB; ++t) acc[t] = 0.f;
        for (int c = lane; c < H / 8; c += 64) {
            const uint4 wq = *reinterpret_cast<const uint4 *>(wrow + 8 * c);
            const u32 wv4[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
            for (int t = 0; t < BK_MAX_TB; ++t) {
                if (t < tb) {
                    const uint4 xq = *reinterpret_cast<const uint4 *>(s_x + t * H + 8 * c);
                    const u32 xv4[4] = {xq.x, xq.y, xq.z, xq.w};
                    float s = acc[t];
#pragma unroll
                    for (int i = 0; i < 4; ++i) s = dot2(wv4[i], xv4[i], s);
                    acc[t] = s;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < BK_MAX_TB; ++t) {
            if (t < tb) {
                const float v = group_sum_dpp(acc[t], 64);
                if (lane == 0 && e < E) a.logits[(int64_t)(t0 + t) * E + e] = v;
            }
        }
        __syncthreads();   // the batch's LDS is free
    }
    if (!a.fused) return;
    // the last workgroup to finish ranks every token's scores
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const u32 old = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (E <= 64) bk_route_tokens<1>(a);
    else if (E <= 128) bk_route_tokens<2>(a);
    else if (E <= 256) bk_route_tokens<4>(a);
    else if (E <= 512) bk_route_tokens<8>(a);
    else bk_route_tokens<16>(a);
    if (tid == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_rmsnorm(const uint16_t *x, const uint16_t *g, int T, int H, float eps, void *y, int out_f32,
                          hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(BK_THREADS), 0, s, x, g, H, eps, y, out_f32);
    return hipGetLastError();
}

hipError_t launch_router(const uint16_t *x, const uint16_t *gamma, float eps, const uint16_t *wr, int T, int H, int E,
                         int k, uint16_t *xn_out, float *logits, int32_t *idx, float *w, uint32_t *counter,
                         hipStream_t s) {
    RouterArgs a;
    a.x = x;
    a.gamma = gamma;
    a.wr = wr;
    a.eps = eps;
    a.T = T;
    a.H = H;
    a.E = E;
    a.k = k;
    a.tb = (int)std::min<size_t>(BK_MAX_TB, BK_LDS / ((size_t)H * 2));
    a.xn_out = xn_out;
    a.logits = logits;
    a.idx = idx;
    a.w = w;
    a.counter = counter;
    a.fused = (T <= BK_MAX_TB && (idx || w)) ? 1 : 0;
    if (a.tb < 1) return hipErrorInvalidValue;
    const size_t dyn = (size_t)a.tb * H * 2;
    auto kern = gamma ? router_kernel<true> : router_kernel<false>;
    const hipError_t le = ensure_dyn_lds(reinterpret_cast<const void *>(kern), dyn);
    if (le != hipSuccess) return le;
    hipLaunchKernelGGL(kern, dim3((E + 3) / 4), dim3(BK_THREADS), dyn, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.fused || !(idx || w)) return e;
    // more tokens than one batch: rank in a launch of its own
    return launch_route(logits, T, E, k, idx, w, s);
}

}  // namespace moeq
