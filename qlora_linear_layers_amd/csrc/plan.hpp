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
    size_t fwd_bytes, bwd_bytes, bwd_grad_bytes;

    LoraPlan(int64_t T_, int64_t K_, int64_t N_, int64_t r_) : T(T_), K(K_), N(N_), r(r_) {
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
        if (r == 0) {
            off_at = off_ps_hi = off_ps_lo = off_gs_hi = off_gs_lo = 0;
            off_pst_hi = off_pst_lo = off_gst_hi = off_gst_lo = off_pda = off_pdb = 0;
            off_dpart = 0;
            off_scl = 0;
            fwd_bytes = 0;
            bwd_bytes = bwd_grad_bytes = scl;
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
        fwd_bytes = o;
        // backward (dX): s dY B^T, block scales
        off_gs_hi = o;  o = align256(o + tr2);
        off_gs_lo = o;  o = align256(o + tr2);
        off_scl = o;    o = align256(o + scl);
        bwd_bytes = o;
        // adapter gradients
        off_gst_hi = o; o = align256(o + rt2);
        off_gst_lo = o; o = align256(o + rt2);
        off_pda = o;    o = align256(o + (size_t)s_da * K * r_pad * 4);
        off_pdb = o;    o = align256(o + (size_t)s_db * N * r_pad * 4);
        bwd_grad_bytes = o;
    }
};

}  // namespace ql
