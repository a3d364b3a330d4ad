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
// one byte (two weights) are looked up in the 32-way replicated pair table
// (one byte permute builds the LDS address), scaled by the block constant,
// rounded to bf16 and packed: the per-weight work does not grow with T.
//
// Workgroup (kKW, kRG below): eight waves, two groups of 64 W rows (four
// 16-row MFMA tiles per wave) times four 128-wide k steps, so 128 rows x 512 k;
// the k waves of a row group are added in LDS in wave order and one fp32 partial per
// (k split, token, row) is written.  The LoRA down projection runs as extra
// workgroups of the same launch over 256-wide k slices (VALU, lane = rank).
#include <type_traits>

#include "common.hpp"
#include "plan.hpp"

namespace ql {

namespace {


}  // namespace

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
static_assert(kRG * kKW * 4 * 64 * 16 <= (int)kWideTableBytes, "wave sums must fit over the pair table");
constexpr int kLoraSlice = 256;   // k per LoRA down-projection workgroup (one 64-k chunk per wave)
constexpr size_t kDecLds = kWideTableBytes;   // pair table; later reused for the wave sums

// LoRA down-projection partials of one 256-wide k slice and 64 ranks:
// lpart[kl][t][j] = sum_{k in slice} X[t][k] A[k][j].  X[0:TT][slice] is
// staged in LDS; waves 0-3 take a quarter of the slice each: lane j loads
// its 64 A values in one burst and reads X as LDS broadcasts.  Every thread
// of the workgroup reaches every barrier.
template <int TT, bool F16>
__device__ __forceinline__ void lora_down_block(const GemvArgs& p, uint8_t* dyn, int lb) {
    typedef __attribute__((address_space(3))) float g_lds_f32_t;
    lds8_t* xl = (lds8_t*)dyn;                                         // [TT][kLoraSlice] bf16
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int jc = lb % (int)(p.r_pad / 64), kl = lb / (int)(p.r_pad / 64);
    const int64_t j = (int64_t)jc * 64 + lane;
    const int64_t k0 = (int64_t)kl * kLoraSlice;
    const rsrc_t rx = make_rsrc(p.x, p.T * p.K * 2);
    for (int ch = threadIdx.x; ch < TT * (kLoraSlice / 8); ch += kDecThreads) {
        const int t = ch / (kLoraSlice / 8);
        const int64_t kk = k0 + (ch % (kLoraSlice / 8)) * 8;
        const u32x4_t v = bload16(rx, (t < p.T && kk < p.K) ? (uint32_t)((t * p.K + kk) * 2) : kOOB, 0);
        *reinterpret_cast<lds_u32x4_t*>(xl + (t * kLoraSlice + (ch % (kLoraSlice / 8)) * 8) * 2) = v;
    }
    __syncthreads();
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
    if (wave < 4) {
        // A[k][j] by buffer loads: ranks j >= r get an offset past the end, and
        // so do rows k >= K (their offset is at least K r 2 bytes), both read 0
        const rsrc_t ra = make_rsrc(p.lora_a, p.K * p.r * 2);
        const int kw = (kLoraSlice / 4) * wave;                         // chunk start inside the slice
        const uint32_t vo = j < p.r ? (uint32_t)(((k0 + kw) * p.r + j) * 2) : kOOB;
        const uint32_t row = (uint32_t)(p.r * 2);
        float av[64];
#pragma unroll
        for (int i = 0; i < 64; ++i) av[i] = lo16<F16>(bload2(ra, vo + i * row, 0));
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float v = acc[t];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const u32x4_t xv = *reinterpret_cast<const lds_u32x4_t*>(xl + (t * kLoraSlice + kw + 8 * c) * 2);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v = fmaf(lo16<F16>(xv[e]), av[8 * c + 2 * e], v);
                    v = fmaf(hi16<F16>(xv[e]), av[8 * c + 2 * e + 1], v);
                }
            }
            acc[t] = v;
        }
    }
    __syncthreads();
    g_lds_f32_t* red = (g_lds_f32_t*)dyn;                              // [4][TT][64]
    if (wave < 4) {
#pragma unroll
        for (int t = 0; t < TT; ++t) red[(wave * TT + t) * 64 + lane] = acc[t];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < TT * 64; i += kDecThreads) {
        const int t = i >> 6, jj = i & 63;
        if (t < p.T) {
            const float v = red[(0 * TT + t) * 64 + jj] + red[(1 * TT + t) * 64 + jj] +
                            red[(2 * TT + t) * 64 + jj] + red[(3 * TT + t) * 64 + jj];
            p.lpart[((int64_t)kl * p.T + t) * p.r_pad + jc * 64 + jj] = v;
        }
    }
}

// Launch 1.  Blocks [0, gemv_blocks) are base blocks: rows [n0, n0 + 128) over
// the k split ks (512 k); the rest are LoRA down-projection blocks.  SQ: the
// block constant is the stored fp32 absmax (single quantization).
template <int TT, bool SQ, bool F16>
__global__ __launch_bounds__(kDecThreads) void k_gemv(GemvGroup grp, Codebook cb) {
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
    // super-scale of four rows, and the lane's 32 k of X (token nl)
    u32x4_t cw[4], xv[4];
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
    const bool xok = kok && nl < p.T;
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = bload16(rx, xok ? (uint32_t)((nl * p.K + kk + 8 * j) * 2) : kOOB, 0);
    if (threadIdx.x < 256) build_wide_pair_table(tbl, cb);
    __syncthreads();

    const uint32_t lane8 = lds_addr(tbl) + (uint32_t)(lane & 31) * 8u;   // table at LDS address 0
    f32x4_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const float c1p = SQ ? __uint_as_float(s2[c]) : block_scale(f8[c], __uint_as_float(s2[c]));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4_t w;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                // address bytes: [0] lane copy, [1] code byte b, [2..3] table base
                const uint32_t addr = __builtin_amdgcn_perm(cw[c][j], lane8, 0x03020000u | ((4u + b) << 8));
                const f32x2_t q = *lds_at<f32x2_t>(addr);
                w[b] = pack16x2<F16>(__fmul_rn(q[0], c1p), __fmul_rn(q[1], c1p));
            }
            acc[c] = mfma16x16x32<F16>(__builtin_bit_cast(bf16x8_t, xv[j]), __builtin_bit_cast(bf16x8_t, w), acc[c]);
        }
    }

    // the k waves of a row group meet in LDS (over the table), in wave order
    __syncthreads();
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

// Launch 2.  Y[t][n] = sum_ks part[ks][t][n] + sum_j (s X A)[t][j] B[j][n],
// rounded to bf16.  A workgroup owns 64 columns n (one per lane); wave w takes
// ranks [w r_pad/4, (w+1) r_pad/4) of B and the base partials of the tokens
// t = w mod 4, and issues those loads first.  Meanwhile the whole workgroup
// rebuilds s X A from its slice partials: thread (e, g) adds slices
// g, g + G, g + 2G, ... of the float4 entry e, all loads independent, and the
// G group sums are added in g order.  The four wave sums of each output are
// added in wave order, so the result does not depend on timing.
constexpr int kFinCols = 64;
template <int RP, bool F16>
__global__ __launch_bounds__(256) void k_gemv_finalize(GemvGroup grp) {
    const int gi = group_find(grp.fin_end, grp.count, (int)blockIdx.x);
    const GemvArgs p = grp.p[gi];
    const int bx = (int)blockIdx.x - (gi ? grp.fin_end[gi - 1] : 0);
    constexpr int RQ = 16 * RP;                                        // ranks of B per wave
    __shared__ __align__(16) float pr[4 * 256];                        // group sums [G][W] float4
    __shared__ __align__(16) float ps[16 * 256];                       // s X A [T][r_pad]
    __shared__ __align__(16) float red[4 * 16 * kFinCols];             // wave sums [4][T][64]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n = (int64_t)bx * kFinCols + lane;
    const bool nok = n < p.N;

    // B column n over this wave's ranks, and the first 8 base partials of its tokens
    uint32_t bv[RQ > 0 ? RQ : 1];
    if constexpr (RP > 0) {
        const rsrc_t rb = make_rsrc(p.lora_b, p.r * p.N * 2);
#pragma unroll
        for (int u = 0; u < RQ; ++u) {
            const int64_t j = (int64_t)wave * RQ + u;
            bv[u] = bload2(rb, (nok && j < p.r) ? (uint32_t)((j * p.N + n) * 2) : kOOB, 0);
        }
    }
    const rsrc_t rp = make_rsrc(p.part, (int64_t)p.KS * p.T * p.N * 4);
    const uint32_t n4 = (uint32_t)n * 4u;
    auto part_at = [&](int ks, int t) -> uint32_t {
        const uint32_t row = (uint32_t)(((int64_t)ks * p.T + t) * p.N * 4);   // wave-uniform
        return (nok && t < p.T && ks < p.KS) ? row + n4 : kOOB;
    };
    uint32_t pv[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[c][i] = bload4(rp, part_at(c, wave + 4 * i), 0);

    if constexpr (RP > 0) {
        const int E4 = (int)(p.T * p.r_pad / 4);                       // float4 entries of s X A
        const int W = E4 < 256 ? E4 : 256;
        const int G = 256 / W;                                         // slice groups
        const int eb = (int)threadIdx.x % W, g = (int)threadIdx.x / W;
        const rsrc_t rl = make_rsrc(p.lpart, (int64_t)p.KL * p.T * p.r_pad * 4);
        const uint32_t slice = (uint32_t)(p.T * p.r_pad * 4);
        // threads past G groups of W (when W does not divide 256) take no part
        for (int e = eb; g < G && e < E4; e += W) {
            f32x4_t a = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int kb = g; kb < p.KL; kb += 16 * G) {
                u32x4_t v[16];
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const int kl = kb + c * G;
                    v[c] = bload16(rl, kl < p.KL ? kl * slice + (uint32_t)e * 16u : kOOB, 0);
                }
#pragma unroll
                for (int c = 0; c < 16; ++c) a += __builtin_bit_cast(f32x4_t, v[c]);
            }
            if (G == 1) {
                *reinterpret_cast<f32x4_t*>(ps + 4 * e) = a * p.scaling;
            } else {
                *reinterpret_cast<f32x4_t*>(pr + 4 * (g * W + e)) = a;
            }
        }
        if (G > 1) {
            __syncthreads();
            if ((int)threadIdx.x < E4) {
                f32x4_t a = *reinterpret_cast<const f32x4_t*>(pr + 4 * threadIdx.x);
                for (int gg = 1; gg < G; ++gg)
                    a += *reinterpret_cast<const f32x4_t*>(pr + 4 * (gg * W + threadIdx.x));
                *reinterpret_cast<f32x4_t*>(ps + 4 * threadIdx.x) = a * p.scaling;
            }
        }
        __syncthreads();
    }

    // base partials of this wave's tokens, in ks order
    float yb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = __uint_as_float(pv[0][i]);
#pragma unroll
        for (int c = 1; c < 8; ++c) v += __uint_as_float(pv[c][i]);
        yb[i] = v;
    }
    for (int ks0 = 8; ks0 < p.KS; ks0 += 8) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[c][i] = bload4(rp, part_at(ks0 + c, wave + 4 * i), 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 8; ++c) yb[i] += __uint_as_float(pv[c][i]);
    }

    // this wave's share of every output column: base partials (own tokens) + its ranks of B
    const int T = (int)p.T;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        if (t < T) {
            float v = (t & 3) == wave ? yb[t >> 2] : 0.0f;
            if constexpr (RP > 0) {
#pragma unroll
                for (int q = 0; q < RQ / 4; ++q) {
                    const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(ps + t * p.r_pad + wave * RQ + 4 * q);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v = fmaf(sv[e], lo16<F16>(bv[4 * q + e]), v);
                }
            }
            red[(wave * 16 + t) * kFinCols + lane] = v;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * kFinCols; i += 256) {
        const int t = i / kFinCols, l = i % kFinCols;
        const int64_t nn = (int64_t)bx * kFinCols + l;
        if (nn < p.N && t >= p.skip) {
            const float v = red[(0 * 16 + t) * kFinCols + l] + red[(1 * 16 + t) * kFinCols + l] +
                            red[(2 * 16 + t) * kFinCols + l] + red[(3 * 16 + t) * kFinCols + l];
            p.y[t * p.N + nn] = (uint16_t)(pack16x2<F16>(v, 0.0f) & 0xFFFFu);
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
                             bool f16) {
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
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
        nfin += (int)ceil_div(q.N, kFinCols);
        g.fin_end[i] = nfin;
    }
    for (int i = 0; i < count; ++i) g.base_end[i] = (i ? g.base_end[i - 1] : nl) + g.p[i].gemv_blocks;
    for (int i = count; i < kMaxGroup; ++i) g.lora_end[i] = g.base_end[i] = g.fin_end[i] = 0x7FFFFFFF;
    const bool sq = probs[0].sc.single();
    const Codebook& cb = host_codebook();
    const dim3 grid((unsigned)(nl + nbase));
    hipError_t ae = hipSuccess;
    auto go = [&](auto kern) {
        // 64 KB of dynamic LDS: above the default limit
        ae = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)kDecLds);
        if (ae == hipSuccess) hipLaunchKernelGGL(kern, grid, dim3(kDecThreads), kDecLds, s, g, cb);
    };
    auto pick = [&](auto tt) {
        constexpr int TT = decltype(tt)::value;
        if (sq) f16 ? go(k_gemv<TT, true, true>) : go(k_gemv<TT, true, false>);
        else f16 ? go(k_gemv<TT, false, true>) : go(k_gemv<TT, false, false>);
    };
    if (T <= 1) pick(std::integral_constant<int, 1>{});
    else if (T <= 2) pick(std::integral_constant<int, 2>{});
    else if (T <= 4) pick(std::integral_constant<int, 4>{});
    else if (T <= 8) pick(std::integral_constant<int, 8>{});
    else pick(std::integral_constant<int, 16>{});
    if (ae != hipSuccess) return ae;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 fg((unsigned)nfin), fb(256);
    auto fin = [&](auto kern) { hipLaunchKernelGGL(kern, fg, fb, 0, s, g); };
    switch (r_pad / 64) {
        case 0: f16 ? fin(k_gemv_finalize<0, true>) : fin(k_gemv_finalize<0, false>); break;
        case 1: f16 ? fin(k_gemv_finalize<1, true>) : fin(k_gemv_finalize<1, false>); break;
        case 2: f16 ? fin(k_gemv_finalize<2, true>) : fin(k_gemv_finalize<2, false>); break;
        case 3: f16 ? fin(k_gemv_finalize<3, true>) : fin(k_gemv_finalize<3, false>); break;
        default: f16 ? fin(k_gemv_finalize<4, true>) : fin(k_gemv_finalize<4, false>); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* x, const uint8_t* codes, BlockScales sc, const uint16_t* lora_a,
                       const uint16_t* lora_b, float scaling, const LoraPlan& pl, uint8_t* ws, uint16_t* y,
                       hipStream_t s, bool f16) {
    const GemvProblem q{x, codes, sc, lora_a, lora_b, scaling, pl.K, pl.N, y};
    return launch_gemv_group(&q, 1, pl.T, pl.r, ws, s, f16);
}

}  // namespace ql
