// prefill.hip -- host side of the many-token MoE layer: workspace layout,
// chunking of the tokens and the launches per chunk.
#include <algorithm>

#include "prefill.h"

namespace moeq {

// Workspace of one chunk of Tc tokens, after the shared header.
struct PfLayout {
    size_t idx, w, rank, cnt, off, nblk, blk, tok, h_hi, h_lo, y, xq, xs, xd, total;
    int Tc, NS, pairs, nblk_max;
};

static size_t align256(size_t v) { return (v + 255u) & ~(size_t)255u; }

static PfLayout pf_layout(int T, int H, int I, int Ish, int k, int E) {
    PfLayout l;
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    // chunk: at most PF_CHUNK tokens, and small enough that the h pair of
    // every (token, expert) pair stays below 2 GiB (32-bit buffer offsets)
    size_t cap = ((size_t)1 << 31) / ((size_t)(k + 1) * Imax * 2);
    cap = cap < 16 ? 16 : (cap & ~(size_t)15);
    const int chunk = (int)(cap < (size_t)PF_CHUNK ? cap : (size_t)PF_CHUNK);
    l.Tc = T < chunk ? T : chunk;
    l.NS = E + (Ish > 0 ? 1 : 0);
    l.pairs = l.Tc * (k + 1);
    l.nblk_max = ((l.pairs + (PF_MB - 1) * l.NS) / PF_MB + 8) & ~7;
    // after everything the decode kernels use, so one workspace serves both
    // paths and nothing written here can pass for a tagged word of the
    // single-token kernel
    size_t o = align256(decode_workspace_bytes(DEC_MAX_T, H, I, Ish, k));
    auto take = [&](size_t bytes) {
        const size_t r = o;
        o = align256(o + bytes);
        return r;
    };
    l.idx = take((size_t)l.Tc * k * 4);
    l.w = take((size_t)l.Tc * k * 4);
    l.rank = take((size_t)l.Tc * k * 4);
    l.cnt = take((size_t)(l.NS + 1) * 4);
    l.off = take((size_t)(l.NS + 1) * 4);
    l.nblk = take(4);
    l.blk = take((size_t)l.nblk_max * 4);
    l.tok = take((size_t)l.NS * l.Tc * 4);
    l.h_hi = take((size_t)l.pairs * Imax * 2);
    l.h_lo = take((size_t)l.pairs * Imax * 2);
    l.y = take((size_t)l.pairs * H * 4);
    l.xq = take((size_t)l.Tc * H);          // MX activations of the chunk (MOE_ACT_MXFP8)
    l.xs = take((size_t)l.Tc * H / 32);
    l.xd = take((size_t)l.Tc * H * 2);
    l.total = o;
    return l;
}

size_t prefill_workspace_bytes(int T, int H, int I, int Ish, int k, int E) {
    return pf_layout(T, H, I, Ish, k, E).total;
}

template <int FMT>
static hipError_t pf_chunk(const PfArgs &p, const PfLayout &l, hipStream_t s) {
    const int Imax = p.L.I > p.L.Ish ? p.L.I : p.L.Ish;
    const int rows_gu = 4 * 16 * PF_RG_GU, rows_dn = 8 * 16 * pf_rg_dn<FMT>();   // weight rows per workgroup
    const int nt_gu = (Imax + rows_gu - 1) / rows_gu;
    const int nt_dn = (p.L.H + rows_dn - 1) / rows_dn;
    if (p.mode == MODE_ROUTE) {
        // route and group: one wave per token, the last workgroup builds the plan
        constexpr int tpw = PF_RG_THREADS / 64;   // tokens per workgroup
        const dim3 grid((p.T + tpw - 1) / tpw), block(PF_RG_THREADS);
        const int E = p.L.E;
        if (E <= 64) hipLaunchKernelGGL(pf_route_group_kernel<1>, grid, block, 0, s, p);
        else if (E <= 128) hipLaunchKernelGGL(pf_route_group_kernel<2>, grid, block, 0, s, p);
        else if (E <= 256) hipLaunchKernelGGL(pf_route_group_kernel<4>, grid, block, 0, s, p);
        else if (E <= 512) hipLaunchKernelGGL(pf_route_group_kernel<8>, grid, block, 0, s, p);
        else hipLaunchKernelGGL(pf_route_group_kernel<16>, grid, block, 0, s, p);
    } else {
        hipLaunchKernelGGL(pf_group_kernel, dim3(p.NS), dim3(PF_THREADS), 0, s, p);
    }
    // gate | up: MX activations on MX weights take the scaled matrix cores;
    // otherwise 256-wide K steps where H allows, else 128-wide
    const int nt_g2 = (Imax + PF_G2_NW * 16 - 1) / (PF_G2_NW * 16);
    bool mx = false;
    if constexpr (Fmt<FMT>::SCALE == SC_UE8M0) mx = p.xq != nullptr;
    if (mx) {
        if constexpr (Fmt<FMT>::SCALE == SC_UE8M0)
            hipLaunchKernelGGL((pf_gateup_mx_kernel<FMT>), dim3(l.nblk_max * nt_gu), dim3(256), 0, s, p, nt_gu);
    } else if (Fmt<FMT>::SCALE == SC_UE8M0 && p.L.H % PF_G2_KS == 0) {
        // the UE8M0 formats, whose conversion applies the scale itself (measured on
        // the 2,048-token layer: 0.455 / 0.366 ms against 0.477 / 0.394 with 128-wide
        // steps; the formats that multiply every weight by its scale, e2m1 + e4m3 and
        // int4 + fp16, were slower with it: 0.445 / 0.649 against 0.428 / 0.599 ms)
        if constexpr (Fmt<FMT>::SCALE == SC_UE8M0)
            hipLaunchKernelGGL((pf_gu256_kernel<FMT>), dim3(l.nblk_max * nt_g2), dim3(64 * PF_G2_NW), 0, s, p, nt_g2);
    } else {
        hipLaunchKernelGGL((pf_gemm_kernel<FMT, false>), dim3(l.nblk_max * nt_gu), dim3(256), 0, s, p, nt_gu);
    }
    // down: the h-resident kernel when every expert's K fits its LDS tile
    const bool res = p.L.I % PF_KS == 0 && p.L.I >= 2 * PF_KS && p.L.I <= PF_DR_KMAX &&
                     (p.L.Ish == 0 || (p.L.Ish % PF_KS == 0 && p.L.Ish >= 2 * PF_KS && p.L.Ish <= PF_DR_KMAX));
    if (res) {
        // persistent: one workgroup per CU, the passes of all blocks shared out evenly
        const int npass = (p.L.H + 8 * PF_DR_RG * 16 - 1) / (8 * PF_DR_RG * 16);
        const int64_t most = (int64_t)l.nblk_max * npass;
        const int G = (int)std::min<int64_t>(most, cached_cus());
        hipLaunchKernelGGL((pf_down_res_kernel<FMT>), dim3(G), dim3(512), 0, s, p);
    }
    else
        hipLaunchKernelGGL((pf_gemm_kernel<FMT, true>), dim3(l.nblk_max * nt_dn), dim3(512), 0, s, p, nt_dn);
    hipLaunchKernelGGL(pf_combine_kernel, dim3(p.T), dim3(PF_THREADS), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_prefill(const DecodeArgs &a, hipStream_t s) {
    const LayerArgs &L = a.L;
    const PfLayout l = pf_layout(a.T, L.H, L.I, L.Ish, L.k, L.E);
    uint8_t *ws = a.ws;
    const size_t out_elt = a.out_f32 ? 4 : 2;
    for (int c0 = 0; c0 < a.T; c0 += l.Tc) {
        const int Tc = (a.T - c0) < l.Tc ? (a.T - c0) : l.Tc;
        PfArgs p;
        p.L = L;
        p.x = a.x + (size_t)c0 * L.H;
        p.T = Tc;
        p.NS = l.NS;
        p.mode = a.mode;
        p.fixed_e = a.fixed_e;
        int32_t *idx = a.idx_out ? a.idx_out + (size_t)c0 * L.k : (int32_t *)(ws + l.idx);
        float *w = a.w_out ? a.w_out + (size_t)c0 * L.k : (float *)(ws + l.w);
        p.idx = idx;
        p.w = w;
        p.rank = (int32_t *)(ws + l.rank);
        p.cnt = (int32_t *)(ws + l.cnt);
        p.off = (int32_t *)(ws + l.off);
        p.nblk = (int32_t *)(ws + l.nblk);
        p.blk = (int32_t *)(ws + l.blk);
        p.tok = (int32_t *)(ws + l.tok);
        p.h_hi = (uint16_t *)(ws + l.h_hi);
        p.h_lo = (uint16_t *)(ws + l.h_lo);
        p.y = (float *)(ws + l.y);
        p.out = (uint8_t *)a.out + (size_t)c0 * L.H * out_elt;
        p.out_f32 = a.out_f32;
        p.residual = a.residual ? a.residual + (size_t)c0 * L.H : nullptr;
        p.hdr = (uint32_t *)ws;
        p.Imax = L.I > L.Ish ? L.I : L.Ish;
        p.xq = nullptr;
        p.xs = nullptr;
        if (a.act_mx) {
            // the chunk's activations to MX e4m3; MX weights take the codes on the
            // scaled matrix cores (H a multiple of 256), the rest the dequantised bf16 rows
            const bool mx = (L.fmt == FMT_E2M3 || L.fmt == FMT_MXFP4) && L.H % PF_MX_KS == 0;
            uint16_t *xd = (uint16_t *)(ws + l.xd);
            hipError_t e = launch_mx_quant(p.x, Tc, L.H, ws + l.xq, ws + l.xs, mx ? nullptr : xd, s);
            if (e != hipSuccess) return e;
            if (mx) {
                p.xq = ws + l.xq;
                p.xs = ws + l.xs;
            } else {
                p.x = xd;
            }
        }
        p.logits = a.mode == MODE_ROUTE ? a.logits + (size_t)c0 * L.E : nullptr;
        hipError_t e;
        switch (L.fmt) {
            case FMT_E2M1: e = pf_chunk<FMT_E2M1>(p, l, s); break;
            case FMT_E2M3: e = pf_chunk<FMT_E2M3>(p, l, s); break;
            case FMT_MXFP4: e = pf_chunk<FMT_MXFP4>(p, l, s); break;
            case FMT_INT4: e = pf_chunk<FMT_INT4>(p, l, s); break;
            default: e = pf_chunk<FMT_E2M3S>(p, l, s); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moeq
