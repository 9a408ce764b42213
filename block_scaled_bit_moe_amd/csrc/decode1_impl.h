// decode1_impl.h -- the MoE layer for ONE token in one launch, shaped for
// latency (the decode step of nextsycl README, "What it does"; Strata
// docs/INTEL.md, "The engine itself on Intel": router_top10, shared_expert).
//
// With one token every selected expert serves exactly one row, so the work is
// static once the token is routed:
//   gate | up : workgroup w < G_gu computes PP consecutive (gate row, up row)
//               pairs of ONE expert (the shared expert's workgroups first, so
//               they need not wait for the routing);
//   down      : workgroup w computes RW consecutive output rows for EVERY
//               selected expert and combines them itself, in rank order, so no
//               partial sums leave the CU.
// Each workgroup routes the token itself, then issues all of its weight loads
// at once (gate/up rows and down rows, into registers), so the whole layer is
// in flight after one routing delay.
//
// The down rows need every expert's h.  Instead of a device-wide barrier, h is
// published as 64-bit words (fp32 value, call tag) with atomic device-coherent
// stores, and each consumer polls the words it needs until every tag is the
// current one (bounded).  The tag is the workspace's call counter + 1: every
// workgroup reads the counter on entry and raises it to counter + 1 on exit.
// That is safe because every workgroup publishes some h (the grid has no
// down-only workgroups), so none can finish before all have read the counter;
// and it stays correct when the launch is replayed from a captured graph.
#pragma once

#include "kernels.h"
#include "rowdot.h"

namespace moeq {

__device__ inline u32 d1_ld_relaxed(const u32 *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void d1_st_relaxed(u32 *p, u32 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void d1_st64_relaxed(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct D1Plan {
    int pp;            // gate/up pairs per workgroup (divides I and the shared I)
    int g_gu;          // workgroups with gate/up work
    int rw;            // output rows per workgroup
    u32 magic_rw;      // floor((2^32-1) / rw) + 1: d / rw == umulhi(d, magic_rw) for the small d used here
    int lpr_d;         // lanes per row of the down projection (down_lanes_per_row)
};

constexpr int D1_MAX_GROUPS = 33;           // k <= 32 routed + shared
constexpr int D1_H_LDS_WORDS = 16384;       // all of h as bf16 hi/lo words (64 KiB)
constexpr int D1_MAX_RW = 64;

struct D1Shared {
    int sel[D1_MAX_GROUPS];         // expert of group g (-1: shared)
    float wsel[D1_MAX_GROUPS];      // its gate weight (1 for the shared expert)
    u32 tag;
    float gu[2 * 64];               // gate/up dot results of this workgroup (pp <= 64)
    float y[D1_MAX_GROUPS * D1_MAX_RW];   // down results: [group][local row]
};

// Region of the workspace holding h for this kernel: [group][Imax] 64-bit words.
__host__ __device__ inline size_t d1_h_offset(int H, int I, int Ish) {
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    return WS_HEADER + (size_t)DEC_MAX_PAIRS * Imax * 4 + (size_t)DEC_MAX_PAIRS * H * 4;
}

template <int FMT, int DEC, int QG, int QD, int MG, int MD>
__global__ __launch_bounds__(256) void decode1_kernel(DecodeArgs a, D1Plan plan) {
    constexpr int PAIR = (DEC == DEC_LUT) ? (FMT == FMT_E2M1 ? LUT_E2M1_PAIR : LUT_E2M3_PAIR) : 1;
    __shared__ u32 s_pair[PAIR];
    __shared__ float s_scale[LUT_SCALE];
    __shared__ D1Shared S;
    extern __shared__ __attribute__((aligned(16))) u32 s_h[];   // NG * Imax words
    const Luts Lt{s_pair, s_scale};
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const LayerArgs &ly = a.L;
    const int H = ly.H, I = ly.I, k = ly.k, Ish = ly.Ish, E = ly.E;
    const int NG = k + (Ish > 0 ? 1 : 0);
    const int Imax = I > Ish ? I : Ish;
    u32 *hdr = reinterpret_cast<u32 *>(a.ws);
    uint64_t *hw = reinterpret_cast<uint64_t *>(a.ws + d1_h_offset(H, I, Ish));
    const int64_t crbH = Fmt<FMT>::code_row_bytes(H), srbH = Fmt<FMT>::scale_row_bytes(H);

    // call tag, activation units and the routing logits are all fetched at once;
    // the routing wave issues its logit loads first of all
    float lgt[16];
    if (wv == 0) {
        if (E <= 64) route_load_logits<1>(a.logits, E, lane, reinterpret_cast<float(&)[1]>(lgt));
        else if (E <= 128) route_load_logits<2>(a.logits, E, lane, reinterpret_cast<float(&)[2]>(lgt));
        else if (E <= 256) route_load_logits<4>(a.logits, E, lane, reinterpret_cast<float(&)[4]>(lgt));
        else if (E <= 512) route_load_logits<8>(a.logits, E, lane, reinterpret_cast<float(&)[8]>(lgt));
        else route_load_logits<16>(a.logits, E, lane, lgt);
    }
    // the routing wave does nothing else until it has routed: the call tag and
    // the tables come from the other three waves (first used after the
    // barrier that follows routing)
    if (tid == 64) S.tag = d1_ld_relaxed(&hdr[WS_EPOCH]) + 1u;
    if (wv > 0) build_luts<FMT>(Lt, tid - 64, 192, DEC == DEC_LUT);
    const int UH = H / 32, LPRg = lanes_per_row(UH), RPWg = WAVE / LPRg;
    const int lrg = lane & (LPRg - 1), rsg = lane / LPRg;
    u32 xr[QG][1][16];
    {
        const uint16_t *xp[1] = {a.x};
        load_x_units<QG, 1>(xr, xp, UH, lrg, LPRg);
    }

    // ------------------------------------------------ gate/up share: group, first pair
    const int w = blockIdx.x;
    const int sh_wgs = Ish / plan.pp;                 // shared expert's workgroups come first
    const bool has_gu = w < plan.g_gu;
    const bool gu_shared = has_gu && w < sh_wgs;
    const int gu_group = !has_gu ? 0 : (gu_shared ? k : (w - sh_wgs) / (I / plan.pp));
    const int gu_i0 = !has_gu ? 0 : (gu_shared ? w * plan.pp : ((w - sh_wgs) % (I / plan.pp)) * plan.pp);
    const int Igu = gu_shared ? Ish : I;

    Unit<FMT> gu_un[MG][QG];
    int gu_task[MG];
#pragma unroll
    for (int s = 0; s < MG; ++s) gu_task[s] = -1;
    auto issue_gu = [&](const uint8_t *c13, const uint8_t *s13) {
#pragma unroll
        for (int s = 0; s < MG; ++s) {
            const int t = (wv + 4 * s) * RPWg + rsg;          // t < pp: gate row, else up row
            gu_task[s] = (has_gu && t < 2 * plan.pp) ? t : -1;
            if (gu_task[s] >= 0) {
                const int row = (t < plan.pp) ? gu_i0 + t : Igu + gu_i0 + (t - plan.pp);
                const uint8_t *c = c13 + (int64_t)row * crbH;
                const uint8_t *sc = s13 + (int64_t)row * srbH;
#pragma unroll
                for (int q = 0; q < QG; ++q) {
                    const int u = lrg + LPRg * q;
                    if (u < UH) load_unit<FMT>(gu_un[s][q], c, sc, u);
                }
            }
        }
    };
    if (gu_shared) issue_gu(ly.sh13c, ly.sh13s);      // before routing: nothing to wait for

    // ------------------------------------------------ route (every workgroup, wave 0)
    if (wv == 0) {
        int e;
        float wt;
        if (E <= 64) route_from_logits<1>(reinterpret_cast<const float(&)[1]>(lgt), E, k, lane, e, wt);
        else if (E <= 128) route_from_logits<2>(reinterpret_cast<const float(&)[2]>(lgt), E, k, lane, e, wt);
        else if (E <= 256) route_from_logits<4>(reinterpret_cast<const float(&)[4]>(lgt), E, k, lane, e, wt);
        else if (E <= 512) route_from_logits<8>(reinterpret_cast<const float(&)[8]>(lgt), E, k, lane, e, wt);
        else route_from_logits<16>(lgt, E, k, lane, e, wt);
        if (lane < k) {
            S.sel[lane] = e;
            S.wsel[lane] = wt;
            if (blockIdx.x == 0) {
                if (a.idx_out) a.idx_out[lane] = e;
                if (a.w_out) a.w_out[lane] = wt;
            }
        }
        if (lane == 0 && Ish > 0) {
            S.sel[k] = -1;
            S.wsel[k] = 1.0f;
        }
    }
    __syncthreads();

    // ------------------------------------------------ issue the remaining weight loads
    // Every expert id needed is read from LDS first, then the gate/up and the
    // down loads are issued back to back (nothing in between that would make
    // the compiler wait for the first batch before issuing the second).
    const int o0 = w * plan.rw;
    const int nr = max(0, min(H, o0 + plan.rw) - o0);
    const int LPRd = plan.lpr_d, RPWd = WAVE / LPRd;
    const int lrd = lane & (LPRd - 1), rsd = lane / LPRd;
    int dn_g[MD], dn_r[MD], dn_e[MD];
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        // down task d in [0, NG*nr): group d / rw, local row d % rw
        const int d = (wv + 4 * s) * RPWd + rsd;
        const int g = (int)__umulhi((u32)d, plan.magic_rw);
        const int r = d - g * plan.rw;
        const bool ok = (nr > 0) && (g < NG) && (r < nr);
        dn_g[s] = ok ? g : -1;
        dn_r[s] = r;
        dn_e[s] = ok ? S.sel[g] : 0;
    }
    const int gu_e = (has_gu && !gu_shared) ? S.sel[gu_group] : 0;
    if (has_gu && !gu_shared) issue_gu(ly.w13c + (int64_t)gu_e * 2 * I * crbH, ly.w13s + (int64_t)gu_e * 2 * I * srbH);
    Unit<FMT> dn_un[MD][QD];
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        if (dn_g[s] >= 0) {
            const int e = dn_e[s], r = dn_r[s];
            const int Ig = (e >= 0) ? I : Ish;
            const int64_t crbI = Fmt<FMT>::code_row_bytes(Ig), srbI = Fmt<FMT>::scale_row_bytes(Ig);
            const uint8_t *c = (e >= 0) ? ly.w2c + ((int64_t)e * H + o0 + r) * crbI : ly.sh2c + (int64_t)(o0 + r) * crbI;
            const uint8_t *sc = (e >= 0) ? ly.w2s + ((int64_t)e * H + o0 + r) * srbI : ly.sh2s + (int64_t)(o0 + r) * srbI;
            const int Ug = Ig / 32;
#pragma unroll
            for (int q = 0; q < QD; ++q) {
                const int u = lrd + LPRd * q;
                if (u < Ug) load_unit<FMT>(dn_un[s][q], c, sc, u);
            }
        }
    }

    // ------------------------------------------------ gate | up dots, h published with the call tag
    const u32 tag = S.tag;
#pragma unroll
    for (int s = 0; s < MG; ++s) {
        float acc = 0.f;
        if (gu_task[s] >= 0) {
#pragma unroll
            for (int q = 0; q < QG; ++q) {
                const int u = lrg + LPRg * q;
                if (u < UH) {
                    u32 wd[16];
                    decode_unit<FMT, DEC>(gu_un[s][q], Lt, wd);
                    float s0, s1;
                    unit_scales<FMT>(gu_un[s][q], Lt, s0, s1);
                    acc = unit_dot<FMT>(wd, xr[q][0], s0, s1, acc);
                }
            }
        }
        acc = group_sum_dpp(acc, LPRg);
        if (gu_task[s] >= 0 && lrg == 0) S.gu[gu_task[s]] = acc;
    }
    __syncthreads();
    if (has_gu && tid < plan.pp) {
        const float h = silu_f32(S.gu[tid]) * S.gu[plan.pp + tid];
        d1_st64_relaxed(hw + (size_t)gu_group * Imax + gu_i0 + tid,
                        ((uint64_t)tag << 32) | __builtin_bit_cast(u32, h));
    }

    // ------------------------------------------------ gather all of h (poll until every tag is current)
    // into LDS as bf16 hi/lo words: per group, unit u = 16 words of hi pairs then 16 words of lo pairs.
    // Batches of NB 16-byte pieces (2 elements each) per thread, every batch loaded at once (each
    // batch costs a device-coherent round trip, so a batch covers a whole layer of the common sizes).
    {
        constexpr int NB = 12;   // 3,072 pieces per batch: one round trip for 11 groups of 512
        const int total2 = NG * Imax / 2;
        const __amdgpu_buffer_rsrc_t hr =
            __builtin_amdgcn_make_buffer_rsrc(hw, (short)0, (int)(NG * Imax * 8), 0x00020000);
        typedef __attribute__((ext_vector_type(4))) u32 v4u;
        u32 spins = 0;
        for (int base = 0; base < total2; base += 256 * NB) {
            // pieces of this batch: piece j holds elements e0, e0 + 1 of group g (e0 < Ig: needed)
            u32 val[NB][2];
            bool need[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int q = base + tid + 256 * j;
                need[j] = false;
                if (q < total2) {
                    const int g = (2 * q) / Imax, e0 = (2 * q) % Imax;
                    need[j] = e0 < ((S.sel[g] >= 0) ? I : Ish);
                }
                val[j][0] = val[j][1] = 0u;
            }
            // poll: reload every needed piece until both of its tags are current
            for (;;) {
                bool all = true;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const u32 off = (u32)(base + tid + 256 * j) * 16u;
                    const v4u p = need[j] ? __builtin_amdgcn_raw_buffer_load_b128(hr, (int)off, 0, 16)   // sc1
                                          : v4u{0u, tag, 0u, tag};
                    val[j][0] = p.x;
                    val[j][1] = p.z;
                    all = all && (p.y == tag) && (p.w == tag);
                }
                if (all) break;
                if (spins++ >= a.spin_limit) { d1_st_relaxed(&hdr[WS_ERR], 1u); break; }
                __builtin_amdgcn_s_sleep(1);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int q = base + tid + 256 * j;
                if (q < total2) {
                    const int g = (2 * q) / Imax, e0 = (2 * q) % Imax;   // elements e0, e0+1 of group g
                    const float h0 = __builtin_bit_cast(float, val[j][0]), h1 = __builtin_bit_cast(float, val[j][1]);
                    const u32 hi0 = f32_to_bf16_rne(h0), hi1 = f32_to_bf16_rne(h1);
                    const u32 lo0 = f32_to_bf16_rne(h0 - __builtin_bit_cast(float, hi0 << 16));
                    const u32 lo1 = f32_to_bf16_rne(h1 - __builtin_bit_cast(float, hi1 << 16));
                    const int pe = e0 >> 1;
                    u32 *dst = s_h + g * Imax + 32 * (pe >> 4);
                    dst[pe & 15] = hi0 | (hi1 << 16);
                    dst[16 + (pe & 15)] = lo0 | (lo1 << 16);
                }
            }
        }
    }
    __syncthreads();

    // ------------------------------------------------ down dots, then the combine
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        float acc = 0.f;
        if (dn_g[s] >= 0) {
            const int g = dn_g[s];
            const int Ug = ((S.sel[g] >= 0) ? I : Ish) / 32;
#pragma unroll
            for (int q = 0; q < QD; ++q) {
                const int u = lrd + LPRd * q;
                if (u < Ug) {
                    const uint4 *hp = reinterpret_cast<const uint4 *>(s_h + g * Imax + 32 * u);
                    u32 xh[16], xl[16];
#pragma unroll
                    for (int vv = 0; vv < 4; ++vv) {
                        const uint4 A = hp[vv], B = hp[4 + vv];
                        xh[4 * vv] = A.x; xh[4 * vv + 1] = A.y; xh[4 * vv + 2] = A.z; xh[4 * vv + 3] = A.w;
                        xl[4 * vv] = B.x; xl[4 * vv + 1] = B.y; xl[4 * vv + 2] = B.z; xl[4 * vv + 3] = B.w;
                    }
                    u32 wd[16];
                    decode_unit<FMT, DEC>(dn_un[s][q], Lt, wd);
                    float s0, s1;
                    unit_scales<FMT>(dn_un[s][q], Lt, s0, s1);
                    acc = unit_dot_split<FMT>(wd, xh, xl, s0, s1, acc);
                }
            }
        }
        acc = group_sum_dpp(acc, LPRd);
        if (dn_g[s] >= 0 && lrd == 0) S.y[dn_g[s] * D1_MAX_RW + dn_r[s]] = acc;
    }
    __syncthreads();
    for (int r = tid; r < nr; r += 256) {
        float acc = 0.f;
        for (int g = 0; g < k; ++g) acc = __builtin_fmaf(S.wsel[g], S.y[g * D1_MAX_RW + r], acc);
        if (Ish > 0) acc += S.y[k * D1_MAX_RW + r];
        if (a.out_f32) reinterpret_cast<float *>(a.out)[o0 + r] = acc;
        else reinterpret_cast<uint16_t *>(a.out)[o0 + r] = f32_to_bf16_rne(acc);
    }
    // every workgroup leaves its tag as the call counter (a max, so the counter
    // never moves back even after an expired wait)
    if (tid == 0) __hip_atomic_fetch_max(&hdr[WS_EPOCH], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moeq

namespace moeq {

template <typename K>
static int d1_coresident(K kernel, size_t dyn_lds) {
    int dev = 0, cus = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (cus <= 0) cus = 1;
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void *>(kernel), 256, dyn_lds) !=
            hipSuccess ||
        per <= 0)
        per = 1;
    return per * cus;
}

// Try a launch with MG gate/up slots and MD down slots per wave; returns
// hipErrorNotSupported when the shape does not fit (the caller falls back).
template <int FMT, int DEC, int QG, int QD, int MG, int MD>
static hipError_t decode1_try(const DecodeArgs &a, hipStream_t s) {
    auto kern = decode1_kernel<FMT, DEC, QG, QD, MG, MD>;
    const LayerArgs &L = a.L;
    const int NG = L.k + (L.Ish > 0 ? 1 : 0);
    const int Imax = L.I > L.Ish ? L.I : L.Ish;
    const size_t dyn = (size_t)NG * Imax * 4;
    const int cap = d1_coresident(kern, dyn);
    const int RPWg = WAVE / lanes_per_row(L.H / 32);
    const int RPWd = WAVE / down_lanes_per_row(L.I, L.Ish);
    // pairs per workgroup: a power of two dividing I and the shared I, at most 64
    // and what the gate/up slots hold; the smallest that fits the grid
    for (int pp = 16; pp <= 64; pp *= 2) {
        if (L.I % pp || (L.Ish > 0 && L.Ish % pp)) break;
        if (2 * pp > 4 * MG * RPWg) break;
        const int g_gu = (L.k * L.I + L.Ish) / pp;
        if (g_gu > cap) continue;
        int G = g_gu > 0 ? g_gu : 1;
        const int rw = (L.H + G - 1) / G;
        if (rw > D1_MAX_RW) continue;
        if (NG * rw > 4 * MD * RPWd) continue;
        // every workgroup must publish h (see the tag argument above): no down-only workgroups
        if ((L.H + rw - 1) / rw > g_gu) continue;
        D1Plan plan{pp, g_gu, rw, (u32)(0xFFFFFFFFull / (u32)rw + 1u), down_lanes_per_row(L.I, L.Ish)};
        hipLaunchKernelGGL(kern, dim3(G), dim3(256), dyn, s, a, plan);
        return hipGetLastError();
    }
    return hipErrorNotSupported;
}

template <int FMT, int DEC, int QG, int QD>
static hipError_t decode1_q(const DecodeArgs &a, hipStream_t s) {
    hipError_t e = decode1_try<FMT, DEC, QG, QD, 2, 4>(a, s);
    if (e != hipErrorNotSupported) return e;
    e = decode1_try<FMT, DEC, QG, QD, 8, 8>(a, s);
    if (e != hipErrorNotSupported) return e;
    return decode1_try<FMT, DEC, QG, QD, 16, 12>(a, s);
}

template <int FMT, int DEC>
hipError_t decode1_fd(const DecodeArgs &a, hipStream_t s) {
    const LayerArgs &L = a.L;
    if (a.T != 1 || a.mode != MODE_ROUTE) return hipErrorNotSupported;
    const int NG = L.k + (L.Ish > 0 ? 1 : 0);
    const int Imax = L.I > L.Ish ? L.I : L.Ish;
    if (NG > D1_MAX_GROUPS || NG * Imax > D1_H_LDS_WORDS) return hipErrorNotSupported;
    const int UH = L.H / 32, LPRg = lanes_per_row(UH), QG = (UH + LPRg - 1) / LPRg;
    const int LPRd = down_lanes_per_row(L.I, L.Ish), QD = (Imax / 32 + LPRd - 1) / LPRd;
    if (QG == 1 && QD == 1) return decode1_q<FMT, DEC, 1, 1>(a, s);
    if (QG == 1 && QD == 2) return decode1_q<FMT, DEC, 1, 2>(a, s);
    if (QG == 2 && QD == 1) return decode1_q<FMT, DEC, 2, 1>(a, s);
    if (QG == 2 && QD == 2) return decode1_q<FMT, DEC, 2, 2>(a, s);
    return hipErrorNotSupported;
}

}  // namespace moeq
