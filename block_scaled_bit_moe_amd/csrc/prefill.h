// prefill.h -- the MoE layer for many tokens at once, on the matrix cores.
//
// With a prompt chunk of 2,048 tokens and top-10 of 512 experts each expert
// sees about 40 tokens, enough rows for the bf16 matrix instructions to pay
// (knivesysl "Prompt processing" notes; Strata SYCL port, "MoE prefill").
// A chunk runs as five launches on one stream:
//
//   route    top-k per token (the decode path's routing kernel)
//   group    per expert slot, the tokens that selected it in ascending token
//            order; the last workgroup to finish turns the counts into pair
//            offsets and a list of blocks of up to 64 tokens of one slot
//   gate/up  per (block, tile of 64 intermediate rows): g = Wg x, u = Wu x
//            on MFMA 16x16x32 bf16 with fp32 accumulation, then
//            h = silu(g) * u, stored as a bf16 hi + lo pair
//   down     per (block, tile of 128 hidden rows): y = Wd (h_hi + h_lo)
//            into fp32 partials, one row per (token, expert) pair
//   combine  per token: sum of w_r * y_r in rank order, plus the shared
//            expert, rounded once to bf16
//
// Weights.  Each wave owns 16-row groups of the weight tile for the whole K
// range, so no other wave needs its decoded weights: a lane loads one unit
// (32 consecutive weights of one row) per 128-wide K step, decodes it with
// the hardware conversion and multiplies in the block scale (exact: every
// product of a code value and a scale has at most 5 significant bits and
// stays in bf16's range), which gives the B operand of four MFMAs directly.
// Lane l covers row l%16 and the K sub-range 32*(l/16) .. +32 of each step;
// MFMA step s takes weights 8s..8s+7 of that sub-range, so within one
// instruction the four lane groups contribute K offsets {8s, 32+8s, 64+8s,
// 96+8s} + 0..7.  The A operand (token activations) is read with the same
// mapping, so every product pairs a weight with its own activation.
//
// Activations.  The 64 x 128 bf16 activation tile of a K step is staged in
// LDS (row stride 272 bytes, so the 16 rows a quarter-wave reads fall on
// distinct banks), double-buffered, and read by all four waves.
#pragma once

#include "common.h"

namespace moeq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) u32 u32x4_t;

constexpr int PF_THREADS = 256;
constexpr int PF_MB = 64;                   // tokens per block (four 16-row sub-tiles)
constexpr int PF_KS = 128;                  // K per step
constexpr int PF_ROW = PF_KS * 2 + 16;      // bytes per staged activation row
constexpr int PF_STAGE = PF_MB * PF_ROW;    // bytes per staged plane
constexpr int PF_RG_GU = 1;                 // 16-row groups per wave: gate/up (each of gate and up)
constexpr int PF_RG_DN = 2;                 // down
constexpr int PF_PD = 3;                    // weight units in flight per row group (K steps ahead)
constexpr int PF_MAX_K = 32;                // top-k limit of the layer

struct PfArgs {
    LayerArgs L;
    const uint16_t *x;        // bf16 [T][H] of the chunk
    int T;                    // tokens in the chunk
    int NS;                   // expert slots: E routed, +1 shared (slot E)
    int mode, fixed_e;
    const int32_t *idx;       // [T][k] (route mode)
    const float *w;           // [T][k]
    int32_t *rank;            // [T][k]: position of the token in its expert's list
    int32_t *cnt;             // [NS]
    int32_t *off;             // [NS + 1]: first pair of each slot
    int32_t *nblk;            // [1]
    int32_t *blk;             // [nblk_max]: slot << 16 | first token of the block
    int32_t *tok;             // [NS][T]: token ids of each slot, ascending
    uint16_t *h_hi, *h_lo;    // [pairs][Imax] bf16
    float *y;                 // [pairs][H] fp32
    void *out;                // [T][H] bf16 or fp32
    int out_f32;
    uint32_t *hdr;            // workspace header (arrival counter)
    int Imax;
};

constexpr int WS_PF_ARRIVE = 4;   // header word: group workgroups finished

__device__ inline void pf_st_relaxed(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int32_t pf_ld_relaxed(const int32_t *p) {
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Which slot receives which tokens.  In route mode slot e < E gets the tokens
// whose top-k holds e and slot E (the shared expert) every token; with a
// fixed expert only that slot is active and it gets every token.
__device__ inline bool pf_slot_identity(const PfArgs &a, int slot) {
    if (a.mode == MODE_ROUTE) return slot == a.L.E;
    return a.mode == MODE_FIXED_ROUTED ? slot == a.fixed_e : slot == a.L.E;
}

// Exclusive scan over the 256 threads of a block (values in v, total returned).
__device__ inline int pf_block_scan(int v, int *s_tmp, int tid, int &total) {
    const int lane = tid & 63, wv = tid >> 6;
    // inclusive scan within the wave
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_tmp[wv] = x;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wv; ++i) base += s_tmp[i];
    total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    __syncthreads();
    return base + x - v;
}

__global__ __launch_bounds__(PF_THREADS) void pf_group_kernel(PfArgs a) {
    const int slot = blockIdx.x, tid = threadIdx.x;
    const int T = a.T, k = a.L.k;
    __shared__ int s_tmp[4];
    __shared__ int s_last;
    int count = 0;
    int32_t *list = a.tok + (size_t)slot * T;
    if (pf_slot_identity(a, slot)) {
        for (int t = tid; t < T; t += PF_THREADS) list[t] = t;
        count = T;
    } else if (a.mode == MODE_ROUTE) {
        for (int t0 = 0; t0 < T; t0 += PF_THREADS) {
            const int t = t0 + tid;
            int r = -1;
            if (t < T) {
                const int32_t *row = a.idx + (size_t)t * k;
                for (int j = 0; j < k; ++j)
                    if (row[j] == slot) r = j;
            }
            int total;
            const int pos = count + pf_block_scan(r >= 0 ? 1 : 0, s_tmp, tid, total);
            if (r >= 0) {
                list[pos] = t;
                a.rank[(size_t)t * k + r] = pos;
            }
            count += total;
        }
    }
    // publish the count; the last workgroup to arrive builds the plan
    if (tid == 0) {
        pf_st_relaxed(&a.cnt[slot], count);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const u32 prev = __hip_atomic_fetch_add(&a.hdr[WS_PF_ARRIVE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (u32)(a.NS - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    // plan: pair offsets and the block list, slot by slot in ascending order
    const int NS = a.NS;
    const int per = (NS + PF_THREADS - 1) / PF_THREADS;
    const int s0 = tid * per;
    int c_sum = 0, b_sum = 0;
    for (int s = s0; s < s0 + per && s < NS; ++s) {
        const int c = pf_ld_relaxed(&a.cnt[s]);
        c_sum += c;
        b_sum += (c + PF_MB - 1) / PF_MB;
    }
    int c_tot, b_tot;
    int c_base = pf_block_scan(c_sum, s_tmp, tid, c_tot);
    int b_base = pf_block_scan(b_sum, s_tmp, tid, b_tot);
    for (int s = s0; s < s0 + per && s < NS; ++s) {
        const int c = pf_ld_relaxed(&a.cnt[s]);
        a.off[s] = c_base;
        const int nb = (c + PF_MB - 1) / PF_MB;
        for (int j = 0; j < nb; ++j) a.blk[b_base + j] = (s << 16) | (j * PF_MB);
        c_base += c;
        b_base += nb;
    }
    if (tid == 0) {
        a.off[NS] = c_tot;
        a.nblk[0] = b_tot;
        __hip_atomic_store(&a.hdr[WS_PF_ARRIVE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// bf16 pair times a block scale; exact because the products fit in bf16.
__device__ inline u32 pf_scale_pair(u32 p, float s) {
    const float lo = __builtin_bit_cast(float, p << 16) * s;
    const float hi = __builtin_bit_cast(float, p & 0xFFFF0000u) * s;
    return (__builtin_bit_cast(u32, hi) & 0xFFFF0000u) | (__builtin_bit_cast(u32, lo) >> 16);
}

// Decode one unit into the B operands of the four MFMA steps of a K step.
template <int FMT>
__device__ inline void pf_unit_to_b(const Unit<FMT> &U, const Luts &Lt, bool valid, bf16x8_t (&b)[4]) {
    u32 w[16];
    decode_unit<FMT, DEC_HW>(U, Lt, w);
    float s0, s1;
    unit_scales<FMT>(U, Lt, s0, s1);
    if constexpr (FMT == FMT_E2M3) s1 = s0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float sc = s < 2 ? s0 : s1;
        u32x4_t v;
        v[0] = valid ? pf_scale_pair(w[4 * s + 0], sc) : 0u;
        v[1] = valid ? pf_scale_pair(w[4 * s + 1], sc) : 0u;
        v[2] = valid ? pf_scale_pair(w[4 * s + 2], sc) : 0u;
        v[3] = valid ? pf_scale_pair(w[4 * s + 3], sc) : 0u;
        b[s] = __builtin_bit_cast(bf16x8_t, v);
    }
}

// Grouped GEMM over the block list.  DOWN = false: gate/up with the SiLU
// epilogue (NB = 2 * RG weight row groups per wave: RG of gate, RG of up);
// DOWN = true: down projection from the h pair (NB = RG).
template <int FMT, bool DOWN>
__global__ __launch_bounds__(PF_THREADS, 2) void pf_gemm_kernel(PfArgs a, int NT) {
    constexpr int RG = DOWN ? PF_RG_DN : PF_RG_GU;
    constexpr int NB = DOWN ? RG : 2 * RG;
    constexpr int NPL = DOWN ? 2 : 1;        // staged activation planes (hi, lo)
    __shared__ __attribute__((aligned(16))) uint8_t pf_smem[2 * NPL * PF_STAGE];
    __shared__ float s_scale[LUT_SCALE];
    __shared__ int s_tok[PF_MB];

    // block and tile of this workgroup; the NT tiles of a block share an XCD
    const int wid = blockIdx.x;
    const int win = wid / (8 * NT), q = wid - win * 8 * NT;
    const int b = win * 8 + (q & 7), nt = q >> 3;
    if (b >= a.nblk[0]) return;
    const int packed = a.blk[b];
    const int slot = packed >> 16, m0 = packed & 0xFFFF;
    const int E = a.L.E, H = a.L.H;
    const bool shared = slot == E;
    const int Is = shared ? a.L.Ish : a.L.I;
    const int N = DOWN ? H : Is;
    const int K = DOWN ? Is : H;
    const int n0 = nt * 64 * RG;
    if (n0 >= N) return;
    const int M = min(PF_MB, a.cnt[slot] - m0);
    const int nsub = (M + 15) >> 4;
    const int p0 = a.off[slot] + m0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lg = lane >> 4, lr = lane & 15;

    Luts Lt;
    Lt.pair = nullptr;
    Lt.scale = s_scale;
    build_luts<FMT>(Lt, tid, PF_THREADS, false);
    if (tid < PF_MB) s_tok[tid] = a.tok[(size_t)slot * a.T + m0 + min(tid, M - 1)];

    // weight rows of this wave
    using F = Fmt<FMT>;
    const int64_t crb = F::code_row_bytes(K), srb = F::scale_row_bytes(K);
    const uint8_t *wc, *ws;
    if (DOWN) {
        wc = shared ? a.L.sh2c : a.L.w2c + (size_t)slot * H * crb;
        ws = shared ? a.L.sh2s : a.L.w2s + (size_t)slot * H * srb;
    } else {
        wc = shared ? a.L.sh13c : a.L.w13c + (size_t)slot * 2 * Is * crb;
        ws = shared ? a.L.sh13s : a.L.w13s + (size_t)slot * 2 * Is * srb;
    }
    const uint8_t *rc[NB];
    const uint8_t *rs[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int g = DOWN ? j : (j % RG);
        int n = n0 + wv * 16 * RG + g * 16 + lr;
        n = min(n, N - 1);                      // rows past N: a valid row, result dropped
        const int row = (!DOWN && j >= RG) ? Is + n : n;
        rc[j] = wc + (size_t)row * crb;
        rs[j] = ws + (size_t)row * srb;
    }
    const int nK = (K + PF_KS - 1) / PF_KS;
    const int UK = K / 32;                      // units per row

    // activation staging: thread t moves 16-byte pieces c = t + 256 i of the tile
    // (row c / 16, piece c % 16 = k offset 8 * (c % 16)); rows >= 16 * nsub are skipped
    auto stage_src = [&](int c, int pl) -> const uint16_t * {
        const int row = c >> 4;
        if (DOWN) {
            const int p = p0 + min(row, M - 1);
            return (pl == 0 ? a.h_hi : a.h_lo) + (size_t)p * a.Imax;
        }
        return a.x + (size_t)s_tok[row] * H;
    };
    uint4 st[NPL][4];
    auto stage_load = [&](int kb) {
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + PF_THREADS * i;
                const int row = c >> 4, kk = kb + (c & 15) * 8;
                if (row < nsub * 16 && kk < K) st[pl][i] = *reinterpret_cast<const uint4 *>(stage_src(c, pl) + kk);
                else st[pl][i] = make_uint4(0u, 0u, 0u, 0u);
            }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + PF_THREADS * i;
                uint8_t *d = pf_smem + (size_t)(buf * NPL + pl) * PF_STAGE + (c >> 4) * PF_ROW + (c & 15) * 16;
                *reinterpret_cast<uint4 *>(d) = st[pl][i];
            }
    };

    // weight units in flight: wq[d][j] holds K step (it + d) for row group j
    Unit<FMT> wq[PF_PD][NB];
    auto load_w = [&](Unit<FMT> (&U)[NB], int it) {
        const int u = it * 4 + lg;
        if (it < nK && u < UK) {
#pragma unroll
            for (int j = 0; j < NB; ++j) load_unit<FMT>(U[j], rc[j], rs[j], u);
        }
    };

    __syncthreads();   // s_tok, LUT
#pragma unroll
    for (int d = 0; d < PF_PD; ++d) load_w(wq[d], d);
    stage_load(0);
    stage_store(0);
    __syncthreads();

    f32x4_t acc[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int it0 = 0; it0 < nK; it0 += PF_PD) {
#pragma unroll
        for (int d = 0; d < PF_PD; ++d) {
            const int it = it0 + d;
            if (it >= nK) break;
            if (it + 1 < nK) stage_load((it + 1) * PF_KS);
            const bool uvalid = it * 4 + lg < UK;
            bf16x8_t bw[NB][4];
#pragma unroll
            for (int j = 0; j < NB; ++j) pf_unit_to_b<FMT>(wq[d][j], Lt, uvalid, bw[j]);
            load_w(wq[d], it + PF_PD);
            const uint8_t *abase = pf_smem + (size_t)((it & 1) * NPL) * PF_STAGE + lr * PF_ROW + lg * 64;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (m < nsub) {
                        const uint8_t *ap = abase + m * 16 * PF_ROW + s * 16;
                        const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap));
                        if (DOWN) {
                            const bf16x8_t a1 =
                                __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + PF_STAGE));
#pragma unroll
                            for (int j = 0; j < NB; ++j) {
                                acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bw[j][s], acc[j][m], 0, 0, 0);
                                acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bw[j][s], acc[j][m], 0, 0, 0);
                            }
                        } else {
#pragma unroll
                            for (int j = 0; j < NB; ++j)
                                acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bw[j][s], acc[j][m], 0, 0, 0);
                        }
                    }
                }
            }
            if (it + 1 < nK) stage_store((it + 1) & 1);
            __syncthreads();
        }
    }

    // epilogue: lane holds rows (tokens) 16m + 4 lg + i, column (weight row) lr
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int n = n0 + wv * 16 * RG + g * 16 + lr;
        if (n >= N) continue;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m >= nsub) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * m + 4 * lg + i;
                if (t >= M) continue;
                const size_t p = (size_t)(p0 + t);
                if (DOWN) {
                    a.y[p * H + n] = acc[g][m][i];
                } else {
                    const float h = silu_f32(acc[g][m][i]) * acc[RG + g][m][i];
                    const uint16_t hi = f32_to_bf16_rne(h);
                    const uint16_t lo = f32_to_bf16_rne(h - __builtin_bit_cast(float, (u32)hi << 16));
                    a.h_hi[p * a.Imax + n] = hi;
                    a.h_lo[p * a.Imax + n] = lo;
                }
            }
        }
    }
}

// out[t] = sum_r w[t][r] * y[pair(t, r)] (rank order) + y[shared pair of t];
// with a fixed expert, out[t] = y[pair of t].
__global__ __launch_bounds__(PF_THREADS) void pf_combine_kernel(PfArgs a) {
    const int t = blockIdx.x, tid = threadIdx.x;
    const int H = a.L.H, k = a.L.k, E = a.L.E;
    __shared__ int s_p[PF_MAX_K + 1];
    __shared__ float s_w[PF_MAX_K];
    int np = 0;
    bool add_shared = false;
    if (a.mode == MODE_ROUTE) {
        if (tid < k) {
            const int e = a.idx[(size_t)t * k + tid];
            s_p[tid] = a.off[e] + a.rank[(size_t)t * k + tid];
            s_w[tid] = a.w[(size_t)t * k + tid];
        }
        if (tid == 0 && a.L.Ish > 0) s_p[k] = a.off[E] + t;
        np = k;
        add_shared = a.L.Ish > 0;
    } else {
        const int slot = a.mode == MODE_FIXED_ROUTED ? a.fixed_e : E;
        if (tid == 0) s_p[0] = a.off[slot] + t;
    }
    __syncthreads();
    for (int c = tid * 4; c < H; c += PF_THREADS * 4) {
        float4 acc;
        if (a.mode == MODE_ROUTE) {
            acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int r = 0; r < np; ++r) {
                const float4 v = *reinterpret_cast<const float4 *>(a.y + (size_t)s_p[r] * H + c);
                const float wr = s_w[r];
                acc.x = __builtin_fmaf(wr, v.x, acc.x);
                acc.y = __builtin_fmaf(wr, v.y, acc.y);
                acc.z = __builtin_fmaf(wr, v.z, acc.z);
                acc.w = __builtin_fmaf(wr, v.w, acc.w);
            }
            if (add_shared) {
                const float4 v = *reinterpret_cast<const float4 *>(a.y + (size_t)s_p[k] * H + c);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
        } else {
            acc = *reinterpret_cast<const float4 *>(a.y + (size_t)s_p[0] * H + c);
        }
        const size_t o = (size_t)t * H + c;
        if (a.out_f32) {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + o) = acc;
        } else {
            const u32 lo = (u32)f32_to_bf16_rne(acc.x) | ((u32)f32_to_bf16_rne(acc.y) << 16);
            const u32 hi = (u32)f32_to_bf16_rne(acc.z) | ((u32)f32_to_bf16_rne(acc.w) << 16);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + o) = make_uint2(lo, hi);
        }
    }
}

}  // namespace moeq
