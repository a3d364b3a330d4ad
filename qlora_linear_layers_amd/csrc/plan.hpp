// Workspace layout and launch plan shared by the host entry points and the
// launchers.  Everything is a pure function of (T, K, N, r), so the size that
// qlora_workspace_bytes() reports is exactly what the launchers carve up.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ql {

constexpr int kTileSmall = 64;   // LoRA rank padding

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Token split of an adapter-gradient product over C columns: at most 256
// workgroups (128 columns x 64 ranks each, one per CU at a time) so that the
// grid runs in one round, each wave taking `cpw` chunks of 32 tokens; returns
// the number of splits (fp32 partials).
inline int grad_splits(int64_t T, int64_t C, int64_t r_pad, int& cpw) {
    const int64_t groups = ceil_div(C, 128) * (r_pad / 64);
    int64_t target = 256 / (groups > 0 ? groups : 1);
    if (target < 1) target = 1;
    cpw = (int)ceil_div(T, 128 * target);
    return (int)ceil_div(T, 128 * (int64_t)cpw);
}

// Reduction splits of a down projection with 64-row tiles: about 256
// workgroups, at most 8 splits and one 64-wide round per split at least.
inline int down_splits(int64_t T, int64_t L) {
    const int64_t tiles = ceil_div(T, 64);
    int64_t s = 256 / tiles;
    if (s > 8) s = 8;
    if (s > L / 64) s = L / 64;
    return (int)(s < 1 ? 1 : s);
}

// Split of the reduction of a 256 x 256-tile GEMM (out [T][C], reduction L)
// over several workgroups when its tiles fill too little of the chip: S
// workgroups per tile each take L/S of the reduction and leave an fp32
// partial tile [S][C][T] that one small launch adds.  S minimises a time
// model fitted to kernel timings of the LLaMA-7B shapes at T = 256 .. 2048:
// rounds of ceil(L / 64 / S) k tiles at 1.2 + 0.5 W / 256 us each (W
// workgroups in flight of 256), plus 0.2 us per MB of partials (written and
// read back) and 10 us for the partial tile stores and the summing launch;
// at least 4 k tiles per split, at most 16 splits, and partials of at most
// `max_bytes` (aligned to 256).  Partial rows hold T rounded up to 4 floats.
inline int64_t split_row(int64_t T) { return (T + 3) & ~int64_t(3); }
inline int gemm_splits(int64_t T, int64_t L, int64_t C, size_t max_bytes) {
    const int64_t tiles = ceil_div(C, 256) * ceil_div(T, 256);
    const int64_t kt = L / 64;
    auto cost = [&](int64_t S) {
        const int64_t wgs = tiles * S;
        const double w = (double)(wgs < 256 ? wgs : 256) / 256.0;
        double t = (double)ceil_div(wgs, 256) * (double)ceil_div(kt, S) * (1.2 + 0.5 * w);
        if (S > 1) t += 0.2e-6 * (double)S * (double)C * (double)split_row(T) * 4.0 + 10.0;
        return t;
    };
    double best = cost(1);
    int bs = 1;
    for (int S = 2; S <= 16; ++S) {
        if (kt / S < 4) break;
        if (align256((size_t)S * C * split_row(T) * 4) > max_bytes) break;
        const double t = cost(S);
        if (t < best) { best = t; bs = S; }
    }
    return bs;
}

constexpr size_t kSplitPartialMax = size_t(64) << 20;

struct LoraPlan {
    int64_t T, K, N, r, r_pad, T8;
    int s_down_x, s_down_dy;   // reduction splits of s X A and s dY B^T
    int64_t ld_at, ld_t;   // row strides of A^T and of the transposed intermediates (padded by 64)
    int s_da, cpw_da;    // dA = X^T G: token splits, chunks per wave
    int s_db, cpw_db;    // dB = P^T dY

    // byte offsets inside the workspace
    size_t off_at;                      // A^T, bf16 [r_pad][ld_at] (rows >= r zero)
    size_t off_ps_hi, off_ps_lo;        // P = s X A as bf16 hi/lo, [T][r_pad] each
    size_t off_gs_hi, off_gs_lo;        // G = s dY B^T as bf16 hi/lo, [T][r_pad] each
    size_t off_scl;                     // block scales c1', fp32 transposed [K/64][N] (dX)
    size_t off_pst_hi, off_pst_lo;      // P^T hi/lo, [r_pad][ld_t] each
    size_t off_gst_hi, off_gst_lo;      // G^T hi/lo, [r_pad][ld_t] each
    size_t off_pda, off_pdb;            // fp32 partials [s_da][K][r_pad], [s_db][N][r_pad]
    size_t off_dpart;                   // fp32 partials of a down projection [splits][T][r_pad]
    // fused backward (QLORA_BWD_FUSED_GRADS): the gradient partials of k_dx's
    // epilogue, one per group of fz_tpg 256-token tiles, in place of the
    // k_grad partials
    int s_fz, fz_tpg;
    size_t off_fza, off_fzb;            // fp32 [s_fz][K][r_pad], [s_fz][N][r_pad]
    // split-k forward (s_fwd > 1): fp32 partial tiles [s_fwd][N][T rounded up to 4] after the
    // forward's state; the backward's regions start at the end of that state
    int s_fwd;
    size_t off_fsp;
    // split-k dX (s_dx > 1): fp32 partial tiles [s_dx][K][T rounded up to 4],
    // over the k_grad partials (written only after dX is summed), or after
    // the fused backward's partials (written while dX runs)
    int s_dx;
    size_t off_dxp, off_dxp_fused;
    size_t fwd_bytes, bwd_bytes, bwd_grad_bytes, bwd_fused_bytes;

    // fwd_cap: the most workspace the forward may take; the split-k partials
    // get at most what the forward's state leaves of it (and at most 64 MiB)
    LoraPlan(int64_t T_, int64_t K_, int64_t N_, int64_t r_, size_t fwd_cap = SIZE_MAX)
        : T(T_), K(K_), N(N_), r(r_) {
        r_pad = r > 0 ? ceil_div(r, kTileSmall) * kTileSmall : 0;
        T8 = ceil_div(T, 8) * 8;
        // a 128-byte shift per row keeps the same column of consecutive rows off
        // one memory channel
        ld_at = K + 64;
        ld_t = T8 + 64;
        cpw_da = cpw_db = 1;
        s_down_x = down_splits(T, K);
        s_down_dy = down_splits(T, N);
        s_da = r > 0 ? grad_splits(T, K, r_pad, cpw_da) : 0;
        s_db = r > 0 ? grad_splits(T, N, r_pad, cpw_db) : 0;
        const size_t scl = align256((size_t)(K / 64) * N * 4);
        auto splits_within = [&](size_t state) {
            const size_t room = fwd_cap > state ? fwd_cap - state : 0;
            s_fwd = gemm_splits(T, K, N, room < kSplitPartialMax ? room : kSplitPartialMax);
            return s_fwd > 1 ? align256((size_t)s_fwd * N * split_row(T) * 4) : 0;
        };
        s_dx = gemm_splits(T, N, K, kSplitPartialMax);
        const size_t dxp = s_dx > 1 ? align256((size_t)s_dx * K * split_row(T) * 4) : 0;
        if (r == 0) {
            const size_t fsp = splits_within(0);
            off_at = off_ps_hi = off_ps_lo = off_gs_hi = off_gs_lo = 0;
            off_pst_hi = off_pst_lo = off_gst_hi = off_gst_lo = off_pda = off_pdb = 0;
            off_dpart = 0;
            off_scl = 0;
            s_fz = fz_tpg = 0;
            off_fza = off_fzb = 0;
            off_fsp = 0;
            fwd_bytes = fsp;
            off_dxp = off_dxp_fused = scl;
            bwd_bytes = bwd_grad_bytes = bwd_fused_bytes = scl + dxp;
            return;
        }
        const size_t tr2 = (size_t)T * r_pad * 2, rt2 = (size_t)r_pad * ld_t * 2;
        size_t o = 0;
        // forward: A^T, s X A (both layouts, kept for the backward), split partials
        off_at = o;     o = align256(o + (size_t)r_pad * ld_at * 2);
        off_ps_hi = o;  o = align256(o + tr2);
        off_ps_lo = o;  o = align256(o + tr2);
        off_pst_hi = o; o = align256(o + rt2);
        off_pst_lo = o; o = align256(o + rt2);
        off_dpart = o;
        {
            const int sd = s_down_x > s_down_dy ? s_down_x : s_down_dy;
            o = align256(o + (sd > 1 ? (size_t)sd * T * r_pad * 4 : 0));
        }
        off_fsp = o;
        fwd_bytes = o + splits_within(o);
        // backward (dX): s dY B^T, block scales (over the forward's split
        // partials, which are dead once the forward has finished)
        off_gs_hi = o;  o = align256(o + tr2);
        off_gs_lo = o;  o = align256(o + tr2);
        off_scl = o;    o = align256(o + scl);
        bwd_bytes = o;
        // adapter gradients
        off_gst_hi = o; o = align256(o + rt2);
        off_gst_lo = o; o = align256(o + rt2);
        const size_t grad_start = o;
        off_pda = o;    o = align256(o + (size_t)s_da * K * r_pad * 4);
        off_pdb = o;    o = align256(o + (size_t)s_db * N * r_pad * 4);
        bwd_grad_bytes = o;
        off_dxp = grad_start;
        if (grad_start + dxp > bwd_grad_bytes) bwd_grad_bytes = grad_start + dxp;
        if (grad_start + dxp > bwd_bytes) bwd_bytes = grad_start + dxp;
        {
            const int64_t tiles = ceil_div(T, 256);
            fz_tpg = tiles >= 4 ? 2 : 1;      // two tiles per partial halve the partials' bytes
            s_fz = (int)ceil_div(tiles, fz_tpg);
        }
        o = grad_start;
        off_fza = o;    o = align256(o + (size_t)s_fz * K * r_pad * 4);
        off_fzb = o;    o = align256(o + (size_t)s_fz * N * r_pad * 4);
        off_dxp_fused = o;
        bwd_fused_bytes = o + dxp;
    }
};

}  // namespace ql
