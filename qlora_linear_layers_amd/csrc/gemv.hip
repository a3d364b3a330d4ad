// Decode-size forward (T <= 16 tokens): fused NF4 double dequantization and
// a small-M MFMA product, then one small kernel for the split sums and the
// LoRA up projection.  The weight stream is the only large operand (0.516
// bytes per weight), so the kernel is organised around issuing all of it at
// once, with enough waves in flight to cover the memory latency.
//
// Layer: Y = X W'^T + s (X A) B with W' = RNE_bf16(fl32(q[code] * c1')) and
// c1' = fl32(e4m3(f) * s2) ("QLoRA 原理精讲" section 2.2; the layer equation of
// the Volcengine article section 3.4, read as above).
//
// Product: v_mfma_f32_16x16x32_bf16 with X as the 16-row A operand (tokens,
// rows past T read as zeros) and the dequantized W as the B operand (16 rows
// of W per MFMA).  The contraction order inside a 128-wide k step is free, so
// lane group g (lanes 16g .. 16g+15) takes the 32 consecutive k at 32g for
// both operands: one 16-byte code load per W row and four 16-byte X loads
// per lane, and sub-step j of the step uses k 32g + 8j .. +7.  The codes of
// one byte (two weights) are looked up in the 16-way replicated pair table
// (32 KB; a bit-field extract and a shift-or build the LDS address), scaled
// by the block constant, rounded to bf16 and packed: the per-weight work does
// not grow with T.
//
// Workgroup (kKW, kRG below): eight waves, two groups of 64 W rows (four
// 16-row MFMA tiles per wave) times four 128-wide k steps, so 128 rows x 512 k;
// the k waves of a row group are added in LDS in wave order and one fp32 partial per
// (k split, token, row) is written.  The LoRA down projection runs as extra
// workgroups of the same launch over 256-wide k slices (VALU).  With the
// 32 KB table and at most 80 registers, at least three workgroups share a CU:
// the kernel's time is set by how many units' latencies overlap, not by any
// one unit's work, and the third workgroup per CU (over the 64 KB table's
// two) pays for the extra address instruction per code byte.
#include <type_traits>

#include "common.hpp"
#include "plan.hpp"

namespace ql {

struct GemvArgs {
    const uint16_t* x;        // [T][K]
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    const float* absmax;      // single quantization: fp32 block absmax (fp8/sup unused)
    const uint16_t* lora_a;   // [K][r]
    const uint16_t* lora_b;   // [r][N]
    float* part;              // [KS][T][N] fp32 base partials
    float* lpart;             // [KL][T][r_pad] fp32 LoRA down-projection partials
    uint16_t* y;              // [T][N]
    int64_t T, K, N, r, r_pad;
    int KS, KL, gemv_blocks;
    float scaling;
    int skip;                 // leading token rows not written (see GemvProblem)
};

// Up to kMaxGroup independent problems (same T, same rank) in one launch.
// Launch 1 lays out the LoRA down-projection blocks of every problem first
// (they are short and latency-bound, so they start while the weight stream
// ramps up), then the base blocks; `lora_end`, `base_end` and `fin_end` hold
// the cumulative block ends (absolute block ids) of each problem.
struct GemvGroup {
    GemvArgs p[kMaxGroup];
    int lora_end[kMaxGroup];
    int base_end[kMaxGroup];
    int fin_end[kMaxGroup];
    int count;
};

// Problem that owns block `bid`, given ascending cumulative ends (uniform).
__device__ __forceinline__ int group_find(const int* ends, int count, int bid) {
    int i = 0;
#pragma unroll
    for (int j = 0; j < kMaxGroup - 1; ++j) i += (j < count - 1 && bid >= ends[j]) ? 1 : 0;
    return i;
}

constexpr int kKW = 4;            // k waves per row group, 128 k each
constexpr int kRG = 2;            // row groups of 64 W rows
constexpr int kDecThreads = 64 * kKW * kRG;
constexpr int kDecRows = 64 * kRG;  // W rows per workgroup
constexpr int kDecK = 128 * kKW;    // k per workgroup
static_assert(kRG * kKW * 4 * 64 * 16 <= (int)kNarrowTableBytes, "wave sums must fit over the pair table");
static_assert(4 * 2 * kGemvMaxT * 64 * 4 <= (int)kNarrowTableBytes, "LoRA block sums must fit in the table's space");
static_assert(kRG * kKW * 4 * 8 * 64 * 4 <= (int)kWideTableBytes, "VALU wave sums (8 tokens) must fit too");
constexpr int kLoraSlice = 256;   // k per LoRA down-projection workgroup (one 64-k chunk per wave)
constexpr size_t kDecLds = kWideTableBytes;   // VALU form: pair table; later reused for the wave sums

// LoRA down-projection partials of one 256-wide k slice and 64 ranks:
// lpart[kl][t][j] = sum_{k in slice} X[t][k] A[k][j].  X[0:TT][slice] is
// staged in LDS; waves 0-3 take a quarter of the slice (64 rows of A) each.
// Lane (h, q) of a wave holds ranks 2q, 2q + 1 of rows 32h .. 32h + 31 of its
// quarter, one 4-byte load per row issued in one burst (32 registers), and
// reads X as LDS broadcasts; the eight (wave, half) sums of every output are
// then added in LDS in that order.  Every thread of the workgroup reaches
// every barrier.
template <int TT, bool F16>
__device__ __forceinline__ void lora_down_block(const GemvArgs& p, uint8_t* dyn, int lb) {
    typedef __attribute__((address_space(3))) float g_lds_f32_t;
    lds8_t* xl = (lds8_t*)dyn;                                         // [TT][kLoraSlice] bf16
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jc = lb % (int)(p.r_pad / 64), kl = lb / (int)(p.r_pad / 64);
    const int h = lane >> 5, q = lane & 31;
    const int64_t j0 = (int64_t)jc * 64 + 2 * q;                       // this lane's two ranks
    const int64_t k0 = (int64_t)kl * kLoraSlice;
    const rsrc_t rx = make_rsrc(p.x, p.T * p.K * 2);
    for (int ch = threadIdx.x; ch < TT * (kLoraSlice / 8); ch += kDecThreads) {
        const int t = ch / (kLoraSlice / 8);
        const int64_t kk = k0 + (ch % (kLoraSlice / 8)) * 8;
        const u32x4_t v = bload16(rx, (t < p.T && kk < p.K) ? (uint32_t)((t * p.K + kk) * 2) : kOOB, 0);
        *reinterpret_cast<lds_u32x4_t*>(xl + (t * kLoraSlice + (ch % (kLoraSlice / 8)) * 8) * 2) = v;
    }
    __syncthreads();
    float acc[TT][2];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t][0] = acc[t][1] = 0.0f;
    if (wave < 4) {
        // A[k][j0], A[k][j0 + 1] as one dword (r is a multiple of 8, so both
        // ranks exist or neither): ranks j0 >= r get an offset past the end,
        // and so do rows k >= K (their offset is at least K r 2 bytes), both
        // read 0
        const rsrc_t ra = make_rsrc(p.lora_a, p.K * p.r * 2);
        const int kw = (kLoraSlice / 4) * wave + 32 * h;               // first row of this lane's 32
        const uint32_t vo = j0 < p.r ? (uint32_t)(((k0 + kw) * p.r + j0) * 2) : kOOB;
        const uint32_t row = (uint32_t)(p.r * 2);
        uint32_t av[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) av[i] = bload4(ra, vo + i * row, 0);
        // rows in order for every token (8 rows per step, every token per step)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const u32x4_t xv = *reinterpret_cast<const lds_u32x4_t*>(xl + (t * kLoraSlice + kw + 8 * c) * 2);
                float v0 = acc[t][0], v1 = acc[t][1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float xa = lo16<F16>(xv[e]), xb = hi16<F16>(xv[e]);
                    const uint32_t ra0 = av[8 * c + 2 * e], ra1 = av[8 * c + 2 * e + 1];
                    v0 = fmaf(xa, lo16<F16>(ra0), v0);
                    v1 = fmaf(xa, hi16<F16>(ra0), v1);
                    v0 = fmaf(xb, lo16<F16>(ra1), v0);
                    v1 = fmaf(xb, hi16<F16>(ra1), v1);
                }
                acc[t][0] = v0;
                acc[t][1] = v1;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    g_lds_f32_t* red = (g_lds_f32_t*)dyn;                              // [4 waves][2 halves][TT][64]
    if (wave < 4) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            red[((wave * 2 + h) * TT + t) * 64 + 2 * q] = acc[t][0];
            red[((wave * 2 + h) * TT + t) * 64 + 2 * q + 1] = acc[t][1];
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < TT * 64; i += kDecThreads) {
        const int t = i >> 6, jj = i & 63;
        if (t < p.T) {
            float v = red[t * 64 + jj];
#pragma unroll
            for (int u = 1; u < 8; ++u) v += red[(u * TT + t) * 64 + jj];
            p.lpart[((int64_t)kl * p.T + t) * p.r_pad + jc * 64 + jj] = v;
        }
    }
}

// Launch 1.  Blocks [0, gemv_blocks) are base blocks: rows [n0, n0 + 128) over
// the k split ks (512 k); the rest are LoRA down-projection blocks.  SQ: the
// block constant is the stored fp32 absmax (single quantization).
//
// DOT: the same blocks, loads and dequantization with the product on the VALU
// instead of the matrix cores (TT <= 8).  Per code byte and token one
// v_dot2c_f32_bf16 adds the two dequantized weights times the two X values to
// an fp32 sum per (W row, token); the four lane groups of a row (k 32g .. +31)
// and the k waves are added in LDS, lane group inside wave, in that order.
// Up to 4 tokens a lane holds the X of every token for its 32 k in registers
// (TT x 16); above that the workgroup's X [TT][512] is staged in LDS behind
// the pair table and read per 8-k sub-step (TT x 4 registers), which keeps the
// occupancy of the MFMA form.  Per weight this adds T/2 VALU instructions to
// the two of the dequantization, where the MFMA form adds a quarter of an
// MFMA whatever T is.
template <int TT, bool SQ, bool F16, bool DOT>
__global__ __launch_bounds__(kDecThreads, (DOT || (F16 && TT > 8)) ? 4 : 6) void k_gemv(GemvGroup grp, Codebook cb) {
    static_assert(!DOT || TT <= kGemvValuMaxT, "VALU product: up to 8 tokens");
    constexpr bool LX = DOT && TT > 4;                                 // X staged in LDS
    extern __shared__ __align__(16) uint8_t dyn[];
    const int bid = (int)blockIdx.x;
    const int lora_total = grp.lora_end[grp.count - 1];
    if (bid < lora_total) {
        const int i = group_find(grp.lora_end, grp.count, bid);
        const GemvArgs p = grp.p[i];
        lora_down_block<TT, F16>(p, dyn, bid - (i ? grp.lora_end[i - 1] : 0));
        return;
    }
    const int gi = group_find(grp.base_end, grp.count, bid);
    const GemvArgs p = grp.p[gi];
    const int bx = bid - (gi ? grp.base_end[gi - 1] : lora_total);     // block within the problem
    lds8_t* tbl = (lds8_t*)dyn;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = wv % kKW, rg = wv / kKW;                          // k step, row group
    const int nl = lane & 15, g = lane >> 4;
    const int nb = (int)ceil_div(p.N, kDecRows);
    const int rb = bx % nb, ks = bx / nb;
    const int64_t n0 = (int64_t)rb * kDecRows + 64 * rg;
    const int64_t kk = (int64_t)ks * kDecK + 128 * wave + 32 * g;      // this lane's 32 k
    const bool kok = kk < p.K;                                         // K % 64 == 0: all 32 or none
    const rsrc_t rc = make_rsrc(p.codes, p.N * p.K / 2);
    const rsrc_t rf = SQ ? make_rsrc(p.absmax, p.N * p.K / 64 * 4) : make_rsrc(p.fp8, p.N * p.K / 64);
    const rsrc_t rs = SQ ? rf : make_rsrc(p.sup, ceil_div(p.N * p.K / 64, 256) * 4);
    const rsrc_t rx = make_rsrc(p.x, p.T * p.K * 2);

    // every load of the wave first: 16 code bytes, the FP8 constant and the
    // super-scale of four rows, and the lane's 32 k of X (MFMA: token nl;
    // VALU: every token)
    constexpr int XT = DOT && !LX ? TT : 1;
    u32x4_t cw[4], xv[XT][4];
    uint32_t f8[4], s2[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t n = n0 + 16 * c + nl;
        const bool ok = kok && n < p.N;
        const int64_t blk = n * (p.K / 64) + kk / 64;
        cw[c] = bload16(rc, ok ? (uint32_t)(n * (p.K / 2) + kk / 2) : kOOB, 0);
        if constexpr (SQ) {
            f8[c] = 0;
            s2[c] = bload4(rf, ok ? (uint32_t)blk * 4u : kOOB, 0);
        } else {
            f8[c] = bload1(rf, ok ? (uint32_t)blk : kOOB, 0);
            s2[c] = bload4(rs, ok ? (uint32_t)(blk >> 8) * 4u : kOOB, 0);
        }
    }
    lds8_t* xl = tbl + kWideTableBytes;                                // LX: X [TT][kDecK] bf16
    if constexpr (LX) {
        // one 16-byte piece of X [TT][512] per thread (TT * 64 pieces <= 512 threads)
        const int t = (int)threadIdx.x / (kDecK / 8), pc = (int)threadIdx.x % (kDecK / 8);
        const int64_t kx = (int64_t)ks * kDecK + 8 * pc;
        if (t < TT) {
            const u32x4_t v = bload16(rx, (t < p.T && kx < p.K) ? (uint32_t)((t * p.K + kx) * 2) : kOOB, 0);
            *reinterpret_cast<lds_u32x4_t*>(xl + (t * kDecK + 8 * pc) * 2) = v;
        }
    } else {
#pragma unroll
        for (int t = 0; t < XT; ++t) {
            const int tx = DOT ? t : nl;
            const bool xok = kok && tx < p.T;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xv[t][j] = bload16(rx, xok ? (uint32_t)((tx * p.K + kk + 8 * j) * 2) : kOOB, 0);
        }
    }
    if (threadIdx.x < 256) {
        if constexpr (DOT) build_wide_pair_table(tbl, cb);
        else build_pair_table16(tbl, cb);
    }
    __syncthreads();

    const uint32_t lane8 = lds_addr(tbl) + (uint32_t)(lane & (DOT ? 31 : 15)) * 8u;   // table at LDS address 0
    // address bytes of a pair lookup: [0] lane copy, [1] code byte b, [2..3] table base
    auto dequant4 = [&](uint32_t codes4, float c1p) {
        u32x4_t w;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t addr = DOT ? __builtin_amdgcn_perm(codes4, lane8, 0x03020000u | ((4u + b) << 8))
                                      : ((__builtin_amdgcn_ubfe(codes4, 8 * b, 8) << 7) | lane8);
            const f32x2_t q = *lds_at<f32x2_t>(addr);
            w[b] = pack16x2<F16>(__fmul_rn(q[0], c1p), __fmul_rn(q[1], c1p));
        }
        return w;
    };
    f32x4_t acc[4];
    float dacc[4][DOT ? TT : 1];
    if constexpr (DOT) {
        float c1p[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            c1p[c] = SQ ? __uint_as_float(s2[c]) : block_scale(f8[c], __uint_as_float(s2[c]));
#pragma unroll
            for (int t = 0; t < TT; ++t) dacc[c][t] = 0.0f;
        }
        // sub-step j (k kk + 8j .. +7) of every row tile: X of every token, then
        // per tile the four code bytes' weights and their dot products
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4_t xj[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if constexpr (LX)
                    xj[t] = *reinterpret_cast<const lds_u32x4_t*>(xl + (t * kDecK + 128 * wave + 32 * g + 8 * j) * 2);
                else
                    xj[t] = xv[t < XT ? t : 0][j];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4_t w = dequant4(cw[c][j], c1p[c]);
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int t = 0; t < TT; ++t) dacc[c][t] = dot16x2<F16>(w[b], xj[t][b], dacc[c][t]);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            const float c1p = SQ ? __uint_as_float(s2[c]) : block_scale(f8[c], __uint_as_float(s2[c]));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[c] = mfma16x16x32<F16>(__builtin_bit_cast(bf16x8_t, xv[0][j]),
                                           __builtin_bit_cast(bf16x8_t, dequant4(cw[c][j], c1p)), acc[c]);
        }
    }

    // the k waves of a row group meet in LDS (over the table), in wave order
    __syncthreads();
    if constexpr (DOT) {
        // [kRG][kKW waves][4 tiles][TT tokens][64 lanes]; lane 16g + i holds
        // row 16c + i over k 32g .. 32g + 31
        float* redf = reinterpret_cast<float*>(dyn) + rg * (kKW * 4 * TT * 64);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int t = 0; t < TT; ++t) redf[((wave * 4 + c) * TT + t) * 64 + lane] = dacc[c][t];
        __syncthreads();
        if (wave < 4) {
            // thread (rg, c, l): row 16c + (l & 15) of tile c, tokens l / 16, l / 16 + 4
            const int c = wave, i = lane & 15;
            const int64_t n = n0 + 16 * c + i;
#pragma unroll
            for (int t = lane >> 4; t < TT; t += 4) {
                float v = redf[(c * TT + t) * 64 + i];
#pragma unroll
                for (int w = 0; w < kKW; ++w)
#pragma unroll
                    for (int g2 = (w == 0 ? 1 : 0); g2 < 4; ++g2) v += redf[((w * 4 + c) * TT + t) * 64 + 16 * g2 + i];
                if (t < p.T && n < p.N) p.part[((int64_t)ks * p.T + t) * p.N + n] = v;
            }
        }
        return;
    }
    f32x4_t* red = reinterpret_cast<f32x4_t*>(dyn) + rg * (kKW * 4 * 64);   // [kKW waves][4 tiles][64 lanes]
#pragma unroll
    for (int c = 0; c < 4; ++c) red[(wave * 4 + c) * 64 + lane] = acc[c];
    __syncthreads();
    if (wave < 4) {
        // thread (rg, c, l): tile c of its row group, accumulator lane l =
        // row 16c + (l & 15), tokens 4 (l >> 4) .. +3
        const int c = wave, l = lane;
        f32x4_t v = red[c * 64 + l];
#pragma unroll
        for (int w = 1; w < kKW; ++w) v += red[(w * 4 + c) * 64 + l];
        const int64_t n = n0 + 16 * c + (l & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * (l >> 4) + e;
            if (t < p.T && n < p.N) p.part[((int64_t)ks * p.T + t) * p.N + n] = v[e];
        }
    }
}

// Launch 2.  Y[t][n] = sum_ks part[ks][t][n] + sum_j u[t][j] B[j][n] with
// u = s X A rebuilt from its slice partials, rounded to the 16-bit type.  A
// workgroup owns 128 columns up to T = 8 (two adjacent ones per lane: N is a
// multiple of 64, so B is read as dwords, the base partials as float2s and Y
// written as dwords) and 64 above, and has W waves (T of them up to
// T = 4, then 4, and 8 for T > 8) that work alone: wave w takes the tokens
// t = w and, for T > 4, t = w + W (TW of them), adds their base partials in ks
// order, rebuilds each 64-rank chunk of u from the slice
// partials (lane (g, i) adds ranks 4i .. 4i + 3 over the slices g, g + 4, ...
// in order, then the four lane groups are added pairwise), and forms the rank
// dot with u read lane by lane (v_readlane) against the columns of B it holds
// in registers.  No LDS and no barrier: the B column, the base partials and
// the first slice partials are all issued before the first sum, so for the
// decode shapes the kernel waits for one round of loads.
// CPL columns per lane: 2 up to T = 8, 1 above (more workgroups for the
// 8-wave, 16-token case)
constexpr int fin_cols(int64_t T) { return T <= 8 ? 128 : 64; }
template <int TW, int CPL, bool LORA, bool F16>
__global__ __launch_bounds__(512) void k_gemv_finalize(GemvGroup grp) {
    const int gi = group_find(grp.fin_end, grp.count, (int)blockIdx.x);
    const GemvArgs p = grp.p[gi];
    const int bx = (int)blockIdx.x - (gi ? grp.fin_end[gi - 1] : 0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int T = (int)p.T;
    const int W = (int)(blockDim.x >> 6);                              // waves (tokens w, w + W)
    if (wave >= T) return;                                             // no token for this wave
    const int64_t n = (int64_t)bx * (64 * CPL) + CPL * lane;           // columns n .. n + CPL - 1 (N is even)
    const bool nok = n < p.N;
    constexpr int kC = 16 / TW;                                        // loads per token and round
    const int KS = p.KS, KL = p.KL, RP = (int)(p.r_pad / 64);

    // Every load takes its lane part as the vector offset and the uniform
    // part (row of the partials, rank of B) as the scalar offset; a lane past
    // N, or a partial past KS / KL or a token past T, gets an offset past the
    // buffer's end and reads 0.
    const uint32_t vn = nok ? (uint32_t)n : 0u;
    const uint32_t v4 = nok ? vn * 4u : kOOB;
    const rsrc_t rp = make_rsrc(p.part, (int64_t)KS * T * p.N * 4);
    auto part_at = [&](int ks, int tw, uint32_t& soff) -> uint32_t {
        const int t = wave + W * tw;
        soff = (uint32_t)(((int64_t)ks * T + t) * p.N * 4);
        return (ks < KS && t < T) ? v4 : kOOB;
    };
    [[maybe_unused]] const rsrc_t rl = make_rsrc(p.lpart, (int64_t)KL * T * p.r_pad * 4);
    // slice partials as float4s: lane (g, i) = (lane / 16, lane % 16) takes
    // ranks 4i .. 4i + 3 of the chunk from the slices kl = g mod 4
    const int sg = lane >> 4, si = lane & 15;
    [[maybe_unused]] auto lpart_at = [&](int kl0, int tw, int c, uint32_t& soff) -> uint32_t {
        const int t = wave + W * tw;
        soff = (uint32_t)((((int64_t)kl0 * T + t) * p.r_pad + 64 * c) * 4);
        return (kl0 + sg < KL && t < T) ? (uint32_t)(sg * T * p.r_pad * 4 + si * 16) : kOOB;
    };
    // ranks past r (padding up to the 64-rank chunk) read row r - 1: their
    // slice partials are exact zeros, so they add nothing
    [[maybe_unused]] const rsrc_t rb = make_rsrc(p.lora_b, p.r * p.N * 2);
    [[maybe_unused]] const uint32_t v2 = nok ? vn * 2u : kOOB;
    [[maybe_unused]] auto load_b = [&](uint32_t (&bv)[64], int c) {
        const uint32_t row = (uint32_t)(p.N * 2);
        const int jv = (int)(p.r - 64 * c);                            // ranks of this chunk below r
        const uint32_t last = v2 + (uint32_t)(jv - 1) * row;
        uint32_t vo = v2 + (uint32_t)(64 * c) * row;
#pragma unroll
        for (int j = 0; j < 64; ++j, vo += row)                        // B[j][n] (and B[j][n + 1])
            bv[j] = CPL == 2 ? bload4(rb, j < jv ? vo : last, 0) : bload2(rb, j < jv ? vo : last, 0);
    };

    // Partials are added kC per token and round (a load past KS or KL reads
    // 0 and adds nothing); the next round is issued before the current one
    // is added.  The first round of base partials and slice partials and the
    // B column of rank chunk 0 are all issued before the first addition.
    typedef u32x2_t round_t[TW][kC];                                   // .y unused with one column
    auto load_base = [&](round_t& v, int ks0) {
#pragma unroll
        for (int c = 0; c < kC; ++c)
#pragma unroll
            for (int tw = 0; tw < TW; ++tw) {
                uint32_t so;
                const uint32_t vo = part_at(ks0 + c, tw, so);
                if constexpr (CPL == 2) v[tw][c] = bload8(rp, vo, so);
                else v[tw][c][0] = bload4(rp, vo, so);
            }
    };
    constexpr int kCU = 8 / TW;                                        // float4 slice loads per token and round
    typedef u32x4_t uround_t[TW][kCU];
    [[maybe_unused]] auto load_slices = [&](uround_t& v, int kl0, int c) {
#pragma unroll
        for (int cc = 0; cc < kCU; ++cc)
#pragma unroll
            for (int tw = 0; tw < TW; ++tw) {
                uint32_t so;
                const uint32_t vo = lpart_at(kl0 + 4 * cc, tw, c, so);
                v[tw][cc] = bload16(rl, vo, so);
            }
    };
    auto add = [&](f32x2_t (&acc)[TW], const round_t& v) {
#pragma unroll
        for (int c = 0; c < kC; ++c)
#pragma unroll
            for (int tw = 0; tw < TW; ++tw) {
                acc[tw][0] += __uint_as_float(v[tw][c][0]);
                if constexpr (CPL == 2) acc[tw][1] += __uint_as_float(v[tw][c][1]);
            }
    };
    // sum of `count` partials in order, the first round already in `r0`
    auto add_rounds = [&](f32x2_t (&acc)[TW], round_t& r0, round_t& r1, int count, auto load) {
        for (int i = 0;; i += 2 * kC) {
            if (i + kC < count) load(r1, i + kC);
            add(acc, r0);
            if (i + kC >= count) break;
            if (i + 2 * kC < count) load(r0, i + 2 * kC);
            add(acc, r1);
            if (i + 2 * kC >= count) break;
        }
    };

    uint32_t bv[LORA ? 64 : 1];
    round_t pb0, pb1;
    [[maybe_unused]] uround_t pu0, pu1;
    if constexpr (LORA) load_b(bv, 0);
    load_base(pb0, 0);
    if constexpr (LORA) load_slices(pu0, 0, 0);

    // base partials in ks order (-0 is the identity of fp32 addition)
    f32x2_t y[TW];
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) y[tw] = f32x2_t{-0.0f, -0.0f};
    add_rounds(y, pb0, pb1, KS, load_base);

    if constexpr (LORA) {
#pragma unroll 1
        for (int c = 0; c < RP; ++c) {
            if (c > 0) {
                load_b(bv, c);
                load_slices(pu0, 0, c);
            }
            // u of this rank chunk: each lane adds its slices in kl order, the
            // four slice groups are then added pairwise across lanes
            f32x4_t u[TW];
#pragma unroll
            for (int tw = 0; tw < TW; ++tw) u[tw] = f32x4_t{-0.0f, -0.0f, -0.0f, -0.0f};
            auto addu = [&](const uround_t& v) {
#pragma unroll
                for (int cc = 0; cc < kCU; ++cc)
#pragma unroll
                    for (int tw = 0; tw < TW; ++tw) u[tw] += __builtin_bit_cast(f32x4_t, v[tw][cc]);
            };
            constexpr int kR = 4 * kCU;                                // slices per round
            for (int i = 0;; i += 2 * kR) {
                if (i + kR < KL) load_slices(pu1, i + kR, c);
                addu(pu0);
                if (i + kR >= KL) break;
                if (i + 2 * kR < KL) load_slices(pu0, i + 2 * kR, c);
                addu(pu1);
                if (i + 2 * kR >= KL) break;
            }
#pragma unroll
            for (int tw = 0; tw < TW; ++tw) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = u[tw][e];
                    v += __shfl_xor(v, 16);
                    v += __shfl_xor(v, 32);
                    u[tw][e] = v * p.scaling;
                }
            }
            // rank dot in rank order: u[t][64c + j] sits in lane j / 4, component j % 4
#pragma unroll
            for (int j = 0; j < 64; ++j) {
                const float b0 = lo16<F16>(bv[j]), b1 = hi16<F16>(bv[j]);
#pragma unroll
                for (int tw = 0; tw < TW; ++tw) {
                    const float uj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u[tw][j & 3]), j >> 2));
                    y[tw][0] = fmaf(uj, b0, y[tw][0]);
                    if constexpr (CPL == 2) y[tw][1] = fmaf(uj, b1, y[tw][1]);
                }
                if (j % 16 == 15) __builtin_amdgcn_sched_barrier(0);       // bounds the live scalar registers
            }
        }
    }

#pragma unroll
    for (int tw = 0; tw < TW; ++tw) {
        const int t = wave + W * tw;
        if (nok && t < T && t >= p.skip) {
            if constexpr (CPL == 2)
                *reinterpret_cast<uint32_t*>(p.y + (int64_t)t * p.N + n) = pack16x2<F16>(y[tw][0], y[tw][1]);
            else
                p.y[(int64_t)t * p.N + n] = (uint16_t)(pack16x2<F16>(y[tw][0], 0.0f) & 0xFFFFu);
        }
    }
}

int gemv_ks(int64_t K) { return (int)ceil_div(K, kDecK); }
int gemv_kl(int64_t K) { return (int)ceil_div(K, kLoraSlice); }
size_t gemv_workspace(int64_t T, int64_t K, int64_t N, int64_t r_pad) {
    // base partials [KS][T][N], LoRA partials [KL][T][r_pad] (none without an adapter)
    return align256((size_t)gemv_ks(K) * T * N * 4) + align256((size_t)gemv_kl(K) * T * r_pad * 4);
}

size_t gemv_group_workspace(const GemvProblem* probs, int count, int64_t T, int64_t r_pad) {
    size_t n = 0;
    for (int i = 0; i < count; ++i) n += gemv_workspace(T, probs[i].K, probs[i].N, r_pad);
    return n;
}

hipError_t launch_gemv_group(const GemvProblem* probs, int count, int64_t T, int64_t r, uint8_t* ws, hipStream_t s,
                             bool f16, DecodeProduct prod) {
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
    if (prod == DecodeProduct::Valu && T > kGemvValuMaxT) return hipErrorInvalidValue;
    const bool dot = prod == DecodeProduct::Valu;
    const int64_t r_pad = r > 0 ? ceil_div(r, 64) * 64 : 0;
    GemvGroup g{};
    g.count = count;
    int nl = 0, nbase = 0, nfin = 0;
    for (int i = 0; i < count; ++i) {
        const GemvProblem& q = probs[i];
        GemvArgs& a = g.p[i];
        a = GemvArgs{q.x, q.codes, q.sc.fp8, q.sc.sup, q.sc.absmax, q.lora_a, q.lora_b, nullptr, nullptr, q.y,
                     T, q.K, q.N, r, r_pad, gemv_ks(q.K), r ? gemv_kl(q.K) : 0, 0, q.scaling, (int)q.skip};
        a.part = reinterpret_cast<float*>(ws);
        a.lpart = reinterpret_cast<float*>(ws + align256((size_t)a.KS * T * q.N * 4));
        ws += gemv_workspace(T, q.K, q.N, r_pad);
        a.gemv_blocks = (int)ceil_div(q.N, kDecRows) * a.KS;
        nl += r ? (int)(r_pad / 64) * a.KL : 0;
        g.lora_end[i] = nl;
        nbase += a.gemv_blocks;
        nfin += (int)ceil_div(q.N, fin_cols(T));
        g.fin_end[i] = nfin;
    }
    for (int i = 0; i < count; ++i) g.base_end[i] = (i ? g.base_end[i - 1] : nl) + g.p[i].gemv_blocks;
    for (int i = count; i < kMaxGroup; ++i) g.lora_end[i] = g.base_end[i] = g.fin_end[i] = 0x7FFFFFFF;
    const bool sq = probs[0].sc.single();
    if (dot && (sq || f16)) return hipErrorInvalidValue;             // the VALU form serves the bf16 DQ path
    const Codebook& cb = host_codebook();
    const dim3 grid((unsigned)(nl + nbase));
    hipError_t ae = hipSuccess;
    size_t lds = dot ? kDecLds : (size_t)kNarrowTableBytes;
    auto go = [&](auto kern) {
        // 64 KB (and more) of dynamic LDS: above the default limit
        ae = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds);
        if (ae == hipSuccess) hipLaunchKernelGGL(kern, grid, dim3(kDecThreads), lds, s, g, cb);
    };
    auto pick = [&](auto tt) {
        constexpr int TT = decltype(tt)::value;
        if constexpr (TT <= kGemvValuMaxT) {
            if (dot) {                                                 // double quantization, bf16 only
                if (TT > 4) lds += (size_t)TT * kDecK * 2;             // X staged behind the table
                go(k_gemv<TT, false, false, true>);
                return;
            }
        }
        if (sq) f16 ? go(k_gemv<TT, true, true, false>) : go(k_gemv<TT, true, false, false>);
        else f16 ? go(k_gemv<TT, false, true, false>) : go(k_gemv<TT, false, false, false>);
    };
    if (T <= 1) pick(std::integral_constant<int, 1>{});
    else if (T <= 2) pick(std::integral_constant<int, 2>{});
    else if (T <= 4) pick(std::integral_constant<int, 4>{});
    else if (T <= 8) pick(std::integral_constant<int, 8>{});
    else pick(std::integral_constant<int, 16>{});
    if (ae != hipSuccess) return ae;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // waves: one per token up to 4, four for T <= 8 (two tokens each), eight
    // for T > 8 (two tokens each); every wave loads the B column itself
    const int fw = T <= 4 ? (int)T : T <= 8 ? 4 : 8;
    const dim3 fg((unsigned)nfin), fb((unsigned)(64 * fw));
    auto fin = [&](auto kern) { hipLaunchKernelGGL(kern, fg, fb, 0, s, g); };
    auto fin_tw = [&](auto tw, auto cpl) {
        constexpr int TW = decltype(tw)::value, CPL = decltype(cpl)::value;
        if (r_pad > 0) f16 ? fin(k_gemv_finalize<TW, CPL, true, true>) : fin(k_gemv_finalize<TW, CPL, true, false>);
        else f16 ? fin(k_gemv_finalize<TW, CPL, false, true>) : fin(k_gemv_finalize<TW, CPL, false, false>);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (T <= 4) fin_tw(I1{}, I2{});
    else if (T <= 8) fin_tw(I2{}, I2{});
    else fin_tw(I2{}, I1{});
    return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* x, const uint8_t* codes, BlockScales sc, const uint16_t* lora_a,
                       const uint16_t* lora_b, float scaling, const LoraPlan& pl, uint8_t* ws, uint16_t* y,
                       hipStream_t s, bool f16) {
    const GemvProblem q{x, codes, sc, lora_a, lora_b, scaling, pl.K, pl.N, y};
    return launch_gemv_group(&q, 1, pl.T, pl.r, ws, s, f16);
}

}  // namespace ql
