// block.hip -- the steps either side of the MoE layer, which make the call a
// whole MoE block: the RMSNorm in front (nextsycl README, dense 27B engine: a
// norm that emits the next kernel's input; knivesysl README, "how it works":
// RMS fused into the quantisation), the router scores with top-k fused into
// the same launch (Strata docs/INTEL.md, "Decode round 2" and "Planned":
// scores + top-k as one graph node), and the residual add, which the layer's
// combine does before its single rounding.
//
// rmsnorm_kernel: one workgroup per token, its sum of squares in a fixed
// order.  router_kernel: one workgroup per router row, the row's quarters on
// the four waves, every token's score reduced in a fixed order; for up to 16
// tokens the last workgroup to finish (an agent-scope counter in the
// workspace header, reset by that workgroup) ranks the scores in the same
// launch, one wave per token, with the routing of the decode kernels.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "memops.h"

namespace moeq {

constexpr int BK_THREADS = 256;

// One normalised bf16 pair: (x * g) * r, each product in fp32, one rounding.
__device__ inline u32 bk_norm_pair(u32 x2, u32 g2, float r) {
    const float x0 = __builtin_bit_cast(float, x2 << 16), x1 = __builtin_bit_cast(float, x2 & 0xFFFF0000u);
    const float g0 = __builtin_bit_cast(float, g2 << 16), g1 = __builtin_bit_cast(float, g2 & 0xFFFF0000u);
    return (u32)f32_to_bf16_rne((x0 * g0) * r) | ((u32)f32_to_bf16_rne((x1 * g1) * r) << 16);
}

// y = x * g * r for one row per workgroup (bf16 out, or fp32).  A thread's
// pieces of the row and of the gains are loaded together first (one round
// trip), summed, then normalised from registers.
constexpr int BK_NORM_MAXC = 16;   // pieces per thread: H <= 16 * 8 * 256
template <int MC>
__global__ __launch_bounds__(BK_THREADS) void rmsnorm_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ g, int H, float eps,
                                                            void *__restrict__ y, int out_f32) {
    __shared__ float s_tmp[1][4];
    const int tid = threadIdx.x, nc = H / 8;
    const uint16_t *xt = x + (int64_t)blockIdx.x * H;
    uint4 xq[MC], gq[MC];
#pragma unroll
    for (int i = 0; i < MC; ++i) {
        const int c = min(tid + BK_THREADS * i, nc - 1);
        xq[i] = *reinterpret_cast<const uint4 *>(xt + 8 * c);
        gq[i] = *reinterpret_cast<const uint4 *>(g + 8 * c);
    }
    // sum of squares: each thread its pieces in order, then DPP, then the four waves in order
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MC; ++i) {
        if (tid + BK_THREADS * i < nc) {
            const u32 v4[4] = {xq[i].x, xq[i].y, xq[i].z, xq[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = __builtin_bit_cast(float, v4[j] << 16), hi = __builtin_bit_cast(float, v4[j] & 0xFFFF0000u);
                ss = __builtin_fmaf(lo, lo, ss);
                ss = __builtin_fmaf(hi, hi, ss);
            }
        }
    }
    const int lane = tid & 63, wv = tid >> 6;
    const float wsum = group_sum_dpp(ss, 64);
    if (lane == 0) s_tmp[0][wv] = wsum;
    __syncthreads();
    const float r = 1.0f / __builtin_sqrtf((((s_tmp[0][0] + s_tmp[0][1]) + s_tmp[0][2]) + s_tmp[0][3]) / (float)H + eps);
#pragma unroll
    for (int i = 0; i < MC; ++i) {
        const int c = tid + BK_THREADS * i;
        if (c >= nc) continue;
        const u32 xv[4] = {xq[i].x, xq[i].y, xq[i].z, xq[i].w}, gv[4] = {gq[i].x, gq[i].y, gq[i].z, gq[i].w};
        const int64_t o = (int64_t)blockIdx.x * H + 8 * c;
        if (out_f32) {
            float *yo = reinterpret_cast<float *>(y) + o;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x0 = __builtin_bit_cast(float, xv[j] << 16), x1 = __builtin_bit_cast(float, xv[j] & 0xFFFF0000u);
                const float g0 = __builtin_bit_cast(float, gv[j] << 16), g1 = __builtin_bit_cast(float, gv[j] & 0xFFFF0000u);
                yo[2 * j] = (x0 * g0) * r;
                yo[2 * j + 1] = (x1 * g1) * r;
            }
        } else {
            uint4 q;
            q.x = bk_norm_pair(xv[0], gv[0], r);
            q.y = bk_norm_pair(xv[1], gv[1], r);
            q.z = bk_norm_pair(xv[2], gv[2], r);
            q.w = bk_norm_pair(xv[3], gv[3], r);
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(y) + o) = q;
        }
    }
}

struct RouterArgs {
    const uint16_t *x;        // bf16 [T][H]
    const uint16_t *wr;       // bf16 [E][H]
    int T, H, E, k;
    float *logits;            // fp32 [T][E]
    int32_t *idx;             // [T][k] (fused top-k; nullable)
    float *w;                 // [T][k]
    u32 *counter;             // arrival counter (fused top-k), zero between calls
    int fused;
};

template <int PER_LANE>
__device__ inline void bk_route_tokens(const RouterArgs &a) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t lr = rsrc_of(a.logits, (uint64_t)a.T * a.E * 4);
    for (int t = wv; t < a.T; t += BK_THREADS / 64) {
        int e;
        float wt;
        float lg[PER_LANE];
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j)   // device-coherent loads (sc1) of the token's scores
            lg[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  lr, (int)((t * a.E + min(lane * PER_LANE + j, a.E - 1)) * 4), 0, 16));
        route_from_logits<PER_LANE>(lg, a.E, a.k, lane, e, wt);
        if (lane < a.k) {
            if (a.idx) a.idx[(int64_t)t * a.k + lane] = e;
            if (a.w) a.w[(int64_t)t * a.k + lane] = wt;
        }
    }
}

constexpr int BK_TG = 4;      // tokens per group: their activation pieces are loaded together

// Workgroup e computes router row e for every token: wave q takes the q-th
// quarter of the row, each lane its 16-byte pieces there (all loaded at
// once); tokens go in groups of four whose activation pieces are loaded
// together; per token the lane sums are reduced by DPP within the wave and the
// four quarter sums added in order.
template <int BK_MAXC>   // 16-byte pieces of the row per lane (H <= 8 * 64 * 4 * BK_MAXC)
__global__ __launch_bounds__(BK_THREADS) void router_kernel(RouterArgs a) {
    __shared__ float s_part[4][BK_TG];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, E = a.E, e = blockIdx.x;
    const int nc = H / 8, nq = (nc + 3) / 4, c0 = wv * nq, c1 = min(nc, c0 + nq);
    const uint16_t *wrow = a.wr + (int64_t)e * H;
    const __amdgpu_buffer_rsrc_t lr = rsrc_of(a.logits, (uint64_t)a.T * E * 4);
    uint4 wq[BK_MAXC];
#pragma unroll
    for (int i = 0; i < BK_MAXC; ++i) {
        const int c = c0 + lane + 64 * i;
        wq[i] = *reinterpret_cast<const uint4 *>(wrow + 8 * min(c, nc - 1));
    }
    for (int t0 = 0; t0 < a.T; t0 += BK_TG) {
        const int tg = min(BK_TG, a.T - t0);
        uint4 xq[BK_TG][BK_MAXC];
#pragma unroll
        for (int t = 0; t < BK_TG; ++t)
#pragma unroll
            for (int i = 0; i < BK_MAXC; ++i) {
                const int c = c0 + lane + 64 * i;
                xq[t][i] = *reinterpret_cast<const uint4 *>(a.x + (int64_t)min(t0 + t, a.T - 1) * H + 8 * min(c, nc - 1));
            }
        float acc[BK_TG];
#pragma unroll
        for (int t = 0; t < BK_TG; ++t) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < BK_MAXC; ++i) {
                if (c0 + lane + 64 * i < c1) {
                    s = dot2(wq[i].x, xq[t][i].x, s);
                    s = dot2(wq[i].y, xq[t][i].y, s);
                    s = dot2(wq[i].z, xq[t][i].z, s);
                    s = dot2(wq[i].w, xq[t][i].w, s);
                }
            }
            acc[t] = group_sum_dpp(s, 64);
        }
        if (lane == 0)
#pragma unroll
            for (int t = 0; t < BK_TG; ++t) s_part[wv][t] = acc[t];
        __syncthreads();
        if (tid < tg) {
            const float v = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
            // device-coherent store (sc1): the last workgroup may run on another XCD
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, v), lr, (int)(((t0 + tid) * E + e) * 4), 0, 16);
        }
        __syncthreads();
    }
    if (!a.fused) return;
    // the last workgroup to finish ranks every token's scores: each workgroup's
    // stores complete before its arrival is counted, and the last one reads
    // the scores device-coherently
    wait_vm<0>();
    __syncthreads();
    if (tid == 0) {
        const u32 old = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last) return;
    if (E <= 64) bk_route_tokens<1>(a);
    else if (E <= 128) bk_route_tokens<2>(a);
    else if (E <= 256) bk_route_tokens<4>(a);
    else if (E <= 512) bk_route_tokens<8>(a);
    else bk_route_tokens<16>(a);
    if (tid == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_rmsnorm(const uint16_t *x, const uint16_t *g, int T, int H, float eps, void *y, int out_f32,
                          hipStream_t s) {
    const int mc = (H / 8 + BK_THREADS - 1) / BK_THREADS;
    if (mc <= 1) hipLaunchKernelGGL(rmsnorm_kernel<1>, dim3(T), dim3(BK_THREADS), 0, s, x, g, H, eps, y, out_f32);
    else if (mc <= 2) hipLaunchKernelGGL(rmsnorm_kernel<2>, dim3(T), dim3(BK_THREADS), 0, s, x, g, H, eps, y, out_f32);
    else if (mc <= 4) hipLaunchKernelGGL(rmsnorm_kernel<4>, dim3(T), dim3(BK_THREADS), 0, s, x, g, H, eps, y, out_f32);
    else if (mc <= 8) hipLaunchKernelGGL(rmsnorm_kernel<8>, dim3(T), dim3(BK_THREADS), 0, s, x, g, H, eps, y, out_f32);
    else hipLaunchKernelGGL(rmsnorm_kernel<BK_NORM_MAXC>, dim3(T), dim3(BK_THREADS), 0, s, x, g, H, eps, y, out_f32);
    return hipGetLastError();
}

hipError_t launch_router(const uint16_t *x, const uint16_t *wr, int T, int H, int E, int k, float *logits,
                         int32_t *idx, float *w, uint32_t *counter, hipStream_t s) {
    if (H > ROUTER_MAX_H) return hipErrorInvalidValue;
    RouterArgs a;
    a.x = x;
    a.wr = wr;
    a.T = T;
    a.H = H;
    a.E = E;
    a.k = k;
    a.logits = logits;
    a.idx = idx;
    a.w = w;
    a.counter = counter;
    a.fused = (T <= 16 && (idx || w)) ? 1 : 0;
    const int per_lane = (H / 8 + 255) / 256;
    if (per_lane <= 1) hipLaunchKernelGGL(router_kernel<1>, dim3(E), dim3(BK_THREADS), 0, s, a);
    else if (per_lane <= 2) hipLaunchKernelGGL(router_kernel<2>, dim3(E), dim3(BK_THREADS), 0, s, a);
    else if (per_lane <= 4) hipLaunchKernelGGL(router_kernel<4>, dim3(E), dim3(BK_THREADS), 0, s, a);
    else hipLaunchKernelGGL(router_kernel<8>, dim3(E), dim3(BK_THREADS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.fused || !(idx || w)) return e;
    // more than 16 tokens: rank in a launch of its own
    return launch_route(logits, T, E, k, idx, w, s);
}

}  // namespace moeq
