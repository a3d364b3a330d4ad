// Workspace layout and split-K plan shared by the host entry points and the
// GEMM launchers.  Everything is a pure function of (T, K, N, r), so the size
// that qlora_workspace_bytes() reports is exactly what the launchers carve up.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ql {

constexpr int kTileA = 256;   // rows of the big operand tiles
constexpr int kTileSmall = 64;
constexpr int kBK = 64;       // reduction elements per LDS tile

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Number of reduction splits for a small GEMM with `tiles` output tiles and
// `ktiles` 64-wide reduction tiles: about one workgroup per compute unit
// (256), at least four reduction tiles per split, and fp32 partials kept
// under `part_cap` elements so that the finalize pass stays cheap.
inline int plan_splits(int64_t tiles, int64_t ktiles, int64_t part_elems, int64_t part_cap = 4 << 20) {
    int64_t s = ceil_div(256, tiles > 0 ? tiles : 1);
    const int64_t cap = ktiles / 4 > 1 ? ktiles / 4 : 1;
    if (s > cap) s = cap;
    while (s > 1 && s * part_elems > part_cap) --s;
    if (s > 64) s = 64;
    return (int)(s < 1 ? 1 : s);
}

struct LoraPlan {
    int64_t T, K, N, r, r_pad;
    // X A  (and s X A as bf16 hi/lo): reduction over K
    int s_xa;
    // dY B^T (and s dY B^T as bf16 hi/lo): reduction over N
    int s_g;
    // dA = X^T G_s: reduction over 2T (hi and lo halves of G_s)
    int s_da;
    // dB = (P_s)^T dY: reduction over 2T
    int s_db;

    // byte offsets inside the workspace
    size_t off_pxa, off_ps_hi, off_ps_lo;     // fp32 partials [s_xa][T][r_pad], bf16 [T][r_pad] x 2
    size_t off_pg, off_gs_hi, off_gs_lo;      // fp32 partials [s_g][T][r_pad], bf16 [T][r_pad] x 2
    size_t off_pda, off_pdb;                  // fp32 partials [s_da][K][r_pad], [s_db][r_pad][N]
    size_t off_scl;                           // fp32 block scales c1', transposed [K/64][N] (backward)
    size_t fwd_bytes, bwd_bytes, bwd_grad_bytes;

    LoraPlan(int64_t T_, int64_t K_, int64_t N_, int64_t r_) : T(T_), K(K_), N(N_), r(r_) {
        r_pad = r > 0 ? ceil_div(r, kTileSmall) * kTileSmall : 0;
        const int64_t ttiles = ceil_div(T, kTileA);
        s_xa = plan_splits(ttiles * (r_pad / kTileSmall), K / kBK, T * r_pad);
        s_g = plan_splits(ttiles * (r_pad / kTileSmall), N / kBK, T * r_pad);
        s_da = plan_splits(ceil_div(K, kTileA) * (r_pad / kTileSmall), ceil_div(2 * T, kBK), K * r_pad);
        s_db = plan_splits(ceil_div(N, kTileA) * (r_pad / kTileSmall), ceil_div(2 * T, kBK), N * r_pad);
        const size_t tr4 = (size_t)T * r_pad * 4, tr2 = (size_t)T * r_pad * 2;
        const size_t scl = align256((size_t)(K / 64) * N * 4);
        size_t o = 0;
        if (r == 0) {
            off_pxa = off_ps_hi = off_ps_lo = off_pg = off_gs_hi = off_gs_lo = off_pda = off_pdb = 0;
            off_scl = 0;
            fwd_bytes = 0;
            bwd_bytes = bwd_grad_bytes = scl;
            return;
        }
        off_scl = o;   o = align256(o + scl);
        off_pxa = o;   o = align256(o + tr4 * s_xa);
        off_ps_hi = o; o = align256(o + tr2);
        off_ps_lo = o; o = align256(o + tr2);
        fwd_bytes = o;
        off_pg = o;    o = align256(o + tr4 * s_g);
        off_gs_hi = o; o = align256(o + tr2);
        off_gs_lo = o; o = align256(o + tr2);
        bwd_bytes = o;
        off_pda = o;   o = align256(o + (size_t)s_da * K * r_pad * 4);
        off_pdb = o;   o = align256(o + (size_t)s_db * r_pad * N * 4);
        bwd_grad_bytes = o;
    }
};

}  // namespace ql
