// route.hip -- moe_route_topk: one wave per token, top-k by exact comparison of
// the fp32 logits (ties to the lower expert index), softmax over the k picks.
// Strata docs/INTEL.md, "The engine itself on Intel" names the router_top10
// kernel; colibri README, "DeepSeek V4" uses top-6 of 256 plus a shared expert.
#include "common.h"
#include "kernels.h"

namespace moeq {

template <int PER_LANE>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                   int32_t *__restrict__ idx, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int e;
    float wt;
    route_one_token_wave<PER_LANE>(logits + (int64_t)t * E, E, k, lane, e, wt);
    if (lane < k) {
        idx[(int64_t)t * k + lane] = e;
        w[(int64_t)t * k + lane] = wt;
    }
}

hipError_t launch_route(const float *logits, int T, int E, int k, int32_t *idx, float *w, hipStream_t s) {
    dim3 grid((T + 3) / 4), block(256);
    if (E <= 64) hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, T, E, k, idx, w);
    else if (E <= 128) hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, T, E, k, idx, w);
    else if (E <= 256) hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, T, E, k, idx, w);
    else if (E <= 512) hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, T, E, k, idx, w);
    else hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, logits, T, E, k, idx, w);
    return hipGetLastError();
}

}  // namespace moeq
