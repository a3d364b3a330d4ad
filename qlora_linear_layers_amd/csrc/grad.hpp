// The adapter-gradient block product, shared by k_grad (lora.hip) and the
// gradient epilogue of the fused backward in k_dx (gemm.hip).  The gradients
// follow from the layer by differentiation, and only the adapters receive
// them ("从LoRA到QLoRA" section 3.1):
//   dA = X^T G   (S = X,  V = G = s dY B^T)
//   dB = P^T dY  (S = dY, V = P = s X A)
// both as part[split][c][j] = sum over the split's tokens t of
// S[t][c] (V_hi + V_lo)[t][j], fp32.
//
// The reduction runs over tokens, which index the rows of S, so a lane loads
// an 8 (t) x 8 (c) bf16 block with eight 16-byte loads and transposes it with
// 32 byte permutes into eight v_mfma_f32_16x16x32_bf16 operands, one per
// column c.  A wave covers 128 columns x 32 tokens per chunk; the four waves
// take consecutive token ranges of 32 cpw tokens and are added in LDS in a
// fixed order, so the result is deterministic.
#pragma once

#include "common.hpp"

namespace ql {

struct GradArgs {
    const uint16_t* s;       // [T][C] bf16 (X or dY)
    const uint16_t* vt_hi;   // [r_pad][ldt] bf16 (G^T or P^T, hi and lo; tokens [0, T8))
    const uint16_t* vt_lo;
    float* part;             // [splits][C][r_pad] fp32
    int64_t T, T8, ldt, C, r_pad;
    int cblocks;             // ceil(C / 128)
    int cpw;                 // 32-token chunks per wave
};

// The adapter gradients computed by the fused backward's k_dx after its dX
// tile (a problem with part == nullptr is not asked for).  The work is split
// into blocks of 128 columns x 64 ranks x `tpg` 256-token tiles (one fp32
// partial per tile group); block q goes to wave q mod waves of the grid (wave
// w of workgroup b is 4 b + w).  Blocks are numbered token group first, then
// column block, then rank block, dA's before dB's, so that the neighbouring
// waves of a group read the same rows of V.
struct FusedGrads {
    GradArgs ga, gb;
    int tpg;             // 256-token tiles per token group (= per partial)
    int groups;          // token groups: ceil(ceil(T / 256) / tpg)
    int waves;           // waves of the k_dx grid
};

constexpr int kGradThreads = 256;
constexpr size_t kGradSmem = (size_t)4 * 8 * 4 * 64 * 4 * 4;   // the wave sums, 128 KB

// One wave's sums acc[i][jt] over the tokens [tw, tw + 32 nch) for the 128
// columns of block cb and the ranks j0 .. j0 + 63 (lane l: operand i is
// column cb 128 + 8 (l % 16) + i; acc[i][jt][v] is column
// cb 128 + 8 (4 (l / 16) + v) + i, rank j0 + 16 jt + l % 16).  The chunks are
// walked from chunk `rot` on, in a fixed order.
template <bool F16>
QL_DEV void grad_accumulate(const GradArgs& a, int cb, int64_t tw, int nch, int rot, int64_t j0,
                            f32x4_t (&acc)[8][4]) {
    const int l = threadIdx.x & 63;
    const int64_t c0 = (int64_t)cb * 128 + 8 * (l & 15);          // this lane's 8 columns
    const int tl8 = 8 * (l >> 4);                                 // lane's token group in a chunk

    const rsrc_t rs = make_rsrc(a.s, a.T * a.C * 2);
    const rsrc_t rh = make_rsrc(a.vt_hi, a.r_pad * a.ldt * 2);
    const rsrc_t rl = make_rsrc(a.vt_lo, a.r_pad * a.ldt * 2);
    const bool cok = c0 < a.C;

#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[i][jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    u32x4_t xr[2][8], vh[2][4], vl[2][4];
    auto load = [&](int ch, int slot) {
        const bool live = ch < nch;
        int cr = live ? ch + rot : 0;
        cr = cr >= nch ? cr - nch : cr;
        const int64_t tc = tw + (int64_t)cr * 32 + tl8;           // first of the lane's 8 tokens
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int64_t t = tc + s;
            xr[slot][s] = bload16(rs, (live && cok && t < a.T) ? (uint32_t)((t * a.C + c0) * 2) : kOOB, 0);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const int64_t j = j0 + jt * 16 + (l & 15);
            const uint32_t vo = (live && tc < a.T8) ? (uint32_t)((j * a.ldt + tc) * 2) : kOOB;
            vh[slot][jt] = bload16(rh, vo, 0);
            vl[slot][jt] = bload16(rl, vo, 0);
        }
    };
    auto compute = [&](int slot) {
        // transpose the 8 x 8 block: operand i holds column c0 + i over the 8 tokens
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
            u32x4_t o;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                o[p] = __builtin_amdgcn_perm(xr[slot][2 * p + 1][i >> 1], xr[slot][2 * p][i >> 1], sel);
            const bf16x8_t xi = __builtin_bit_cast(bf16x8_t, o);
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                acc[i][jt] = mfma16x16x32<F16>(xi, __builtin_bit_cast(bf16x8_t, vh[slot][jt]), acc[i][jt]);
                acc[i][jt] = mfma16x16x32<F16>(xi, __builtin_bit_cast(bf16x8_t, vl[slot][jt]), acc[i][jt]);
            }
        }
    };
    load(0, 0);
    load(1, 1);
    for (int ch = 0; ch < nch; ch += 2) {
        compute(0);
        load(ch + 2, 0);
        if (ch + 1 < nch) compute(1);
        load(ch + 3, 1);
    }
}

// part[split][c][j] for the 128 columns of column block cb and the 64 ranks
// j0 .. j0 + 63, over the tokens of `split` (wave w takes the 32 cpw tokens
// from (4 split + w) 32 cpw).  Every thread of a 256-thread workgroup calls
// it with the same arguments; `red` is kGradSmem bytes of LDS.  It ends with
// a barrier, so calls can follow one another on the same LDS.
template <bool F16>
QL_DEV void grad_block(const GradArgs& a, int cb, int split, int64_t j0, float* red) {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    f32x4_t acc[8][4];
    // workgroups of one split read the same V columns; each column block walks
    // its chunks from its own starting point
    grad_accumulate<F16>(a, cb, ((int64_t)split * 4 + w) * 32 * a.cpw, a.cpw, (int)(cb % a.cpw), j0, acc);

    // fixed-order sum of the four waves, then one fp32 partial per split
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            *reinterpret_cast<f32x4_t*>(red + (((w * 8 + i) * 4 + jt) * 64 + l) * 4) = acc[i][jt];
    __syncthreads();
    // thread: one (operand i, rank tile jt, lane) slot, the four waves' float4s
    // added in wave order; the float4 holds rows c = 8 (4 (lane / 16) + v) + i
    float* out = a.part + (int64_t)split * a.C * a.r_pad;
    const f32x4_t* red4 = reinterpret_cast<const f32x4_t*>(red);
    for (int e = threadIdx.x; e < 8 * 4 * 64; e += kGradThreads) {
        const int ll = e & 63, jt = (e >> 6) & 3, i = e >> 8;
        f32x4_t s4 = red4[(i * 4 + jt) * 64 + ll];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) s4 += red4[((ww * 8 + i) * 4 + jt) * 64 + ll];
        const int64_t j = j0 + jt * 16 + (ll & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t c = (int64_t)cb * 128 + 8 * (4 * (ll >> 4) + v) + i;
            if (c < a.C) out[c * a.r_pad + j] = s4[v];
        }
    }
    __syncthreads();                          // `red` may be written again by the next call
}

// One wave alone: part[split][c][j] for column block cb and ranks j0 .. j0 + 63
// over the 256 tpg tokens of token group `split` (8 tpg chunks), written
// straight from the wave's sums: no partner waves, no LDS, no barrier, so the
// waves of a workgroup can each take their own blocks.
template <bool F16>
QL_DEV void grad_wave(const GradArgs& a, int cb, int split, int tpg, int64_t j0) {
    const int l = threadIdx.x & 63;
    f32x4_t acc[8][4];
    grad_accumulate<F16>(a, cb, (int64_t)split * 256 * tpg, 8 * tpg, 0, j0, acc);
    float* out = a.part + (int64_t)split * a.C * a.r_pad;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const int64_t j = j0 + jt * 16 + (l & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t c = (int64_t)cb * 128 + 8 * (4 * (l >> 4) + v) + i;
                if (c < a.C) out[c * a.r_pad + j] = acc[i][jt][v];
            }
        }
}

}  // namespace ql
