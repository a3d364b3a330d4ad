// Decode-size forward (T <= 16 tokens): fused NF4 double dequantization +
// GEMV on the vector ALUs, no MFMA.  The weight stream is the only large
// operand (0.516 bytes per weight), so the kernel is organised around reading
// it once with wide coalesced loads and reusing every dequantized weight for
// all T tokens.
//
// Layer: Y = X W'^T + s (X A) B with W' = RNE_bf16(fl32(q[code] * c1')) and
// c1' = fl32(e4m3(f) * s2) ("QLoRA 原理精讲" section 2.2; the layer equation of
// the Volcengine article section 3.4, read as above).  s X A arrives as the
// bf16 hi/lo pair the LoRA down-projection writes.
//
// Mapping: a workgroup of four wave64s owns R consecutive rows of W (R = 16,
// 8 or 4 as T grows) and one round of the reduction (4096 k, or 2048 at
// T > 8).  The round of X (T x round bf16) is staged in LDS once; each lane
// takes 16 consecutive k (8 code bytes per row, one block scale per row),
// dequantizes them once and multiplies them with all T tokens using
// v_dot2_f32_bf16 (two products per instruction, fp32 accumulation).  The 64
// lanes of a wave are summed with DPP row swaps and four lane reads, the four
// waves in LDS.  The LoRA down projection runs as extra workgroups of the
// same launch over 256-wide slices; a second small kernel adds all partial
// sums in a fixed order and applies the LoRA up projection.
#include "common.hpp"
#include "plan.hpp"

namespace ql {

namespace {

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t g_lds8_t;
typedef __attribute__((address_space(3))) u32x4_t g_lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x2_t g_lds_f32x2_t;


// Sum over the 64 lanes of a wave, returned in every lane (deterministic
// order): DPP swaps give every lane its 16-lane row's sum (quad_perm
// [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror), then the four row sums
// are read out and added.
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
    return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, a), __builtin_bit_cast(bf16x2v_t, b), c,
                                           false);
}

}  // namespace

struct GemvArgs {
    const uint16_t* x;        // [T][K]
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    const uint16_t* lora_a;   // [K][r]
    const uint16_t* lora_b;   // [r][N]
    float* part;              // [KS][T][N] fp32 base-GEMV partials
    float* lpart;             // [KL][T][r_pad] fp32 LoRA down-projection partials
    uint16_t* y;              // [T][N]
    int64_t T, K, N, r, r_pad;
    int KS, KL, gemv_blocks;
    float scaling;
};

// Rows per workgroup for a token count: the X reuse (R rows per X read) grows
// with T while the accumulators (R x TT registers) stay within budget.
template <int TT>
constexpr int gemv_rows() { return TT <= 4 ? 16 : (TT <= 8 ? 8 : 4); }
// k per workgroup (one LDS-staged round of X; four 1024-wide wave chunks)
template <int TT>
constexpr int gemv_round() { return TT <= 8 ? 4096 : 2048; }
constexpr int kLoraSlice = 256;   // k per LoRA down-projection workgroup (one 64-k chunk per wave)

// Launch 1.  Blocks [0, gemv_blocks) are GEMV blocks: rows [n0, n0 + R) over
// the k round ks; the round of X (T x 4096 bf16) is staged in LDS once and
// each wave takes one 1024-wide chunk of it (16 k per lane), so every load a
// wave needs (8 code bytes, one FP8 constant and one super-scale per row) is
// issued up front.  Weights are dequantized once and multiplied with all T
// tokens by v_dot2_f32_bf16; the four wave sums meet in LDS and one fp32
// partial per (ks, t, n) is written.  The remaining blocks compute partial
// sums of X A over 256-wide k slices (lane j, wave-uniform k, so the X values
// are scalar loads).
template <int TT>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs p, Codebook cb) {
    constexpr int R = gemv_rows<TT>();
    constexpr int KR = gemv_round<TT>();
    typedef __attribute__((address_space(3))) float g_lds_f32_t;
    extern __shared__ __align__(16) uint8_t dyn[];
    g_lds8_t* base = (g_lds8_t*)dyn;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    if ((int)blockIdx.x >= p.gemv_blocks) {
        // ---- LoRA down-projection partials: lpart[kl][t][j] = sum_{k in slice} X[t][k] A[k][j]
        // X[0:TT][slice] is staged in LDS; wave g takes its quarter of the slice
        // in chunks of 64: lane j loads its 64 A values of a chunk in one burst
        // and reads X as LDS broadcasts.
        const int lb = (int)blockIdx.x - p.gemv_blocks;
        const int jc = lb % (int)(p.r_pad / 64), kl = lb / (int)(p.r_pad / 64);
        const int64_t j = (int64_t)jc * 64 + lane;
        const int64_t k0 = (int64_t)kl * kLoraSlice;
        g_lds8_t* xl = base;                                           // [TT][kLoraSlice] bf16
        for (int ch = threadIdx.x; ch < TT * (kLoraSlice / 8); ch += 256) {
            const int t = ch / (kLoraSlice / 8);
            const int64_t kk = k0 + (ch % (kLoraSlice / 8)) * 8;
            u32x4_t v = {0, 0, 0, 0};
            if (t < p.T && kk < p.K) v = *reinterpret_cast<const u32x4_t*>(p.x + t * p.K + kk);
            *reinterpret_cast<g_lds_u32x4_t*>(xl + (t * kLoraSlice + (ch % (kLoraSlice / 8)) * 8) * 2) = v;
        }
        __syncthreads();
        float acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
        // A[k][j] by buffer loads: ranks j >= r get an offset past the end, and
        // so do rows k >= K (their offset is at least K r 2 bytes), both read 0
        const rsrc_t ra = make_rsrc(p.lora_a, p.K * p.r * 2);
        for (int sub = 0; sub < kLoraSlice / 256; ++sub) {
            const int kw = (kLoraSlice / 4) * wave + 64 * sub;         // chunk start inside the slice
            const uint32_t vo = j < p.r ? (uint32_t)(((k0 + kw) * p.r + j) * 2) : kOOB;
            const uint32_t row = (uint32_t)(p.r * 2);
            float av[64];
#pragma unroll
            for (int i = 0; i < 64; ++i) av[i] = bf16lo(bload2(ra, vo + i * row, 0));
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                float v = acc[t];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const u32x4_t xv = *reinterpret_cast<const g_lds_u32x4_t*>(xl + (t * kLoraSlice + kw + 8 * c) * 2);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v = fmaf(bf16lo(xv[e]), av[8 * c + 2 * e], v);
                        v = fmaf(bf16hi(xv[e]), av[8 * c + 2 * e + 1], v);
                    }
                }
                acc[t] = v;
            }
        }
        __syncthreads();
        g_lds_f32_t* red = (g_lds_f32_t*)base;                         // [4][TT][64]
#pragma unroll
        for (int t = 0; t < TT; ++t) red[(wave * TT + t) * 64 + lane] = acc[t];
        __syncthreads();
        for (int i = threadIdx.x; i < TT * 64; i += 256) {
            const int t = i >> 6, jj = i & 63;
            if (t < p.T) {
                const float v = red[(0 * TT + t) * 64 + jj] + red[(1 * TT + t) * 64 + jj] +
                                red[(2 * TT + t) * 64 + jj] + red[(3 * TT + t) * 64 + jj];
                p.lpart[((int64_t)kl * p.T + t) * p.r_pad + jc * 64 + jj] = v;
            }
        }
        return;
    }

    // ---- base GEMV partials
    g_lds8_t* tbl = base;                                              // 2 KB byte-pair table
    g_lds8_t* xs = base + 2048;                                        // [TT][KR] bf16
    {
        const f32x2_t v = {cb.q[threadIdx.x >> 4], cb.q[threadIdx.x & 15]};
        *reinterpret_cast<g_lds_f32x2_t*>(tbl + threadIdx.x * 8) = v;
    }
    const int nb = (int)ceil_div(p.N, R);
    const int rb = (int)blockIdx.x % nb, ks = (int)blockIdx.x / nb;
    const int64_t n0 = (int64_t)rb * R;
    const int64_t kr0 = (int64_t)ks * KR;
    const rsrc_t rc = make_rsrc(p.codes, p.N * p.K / 2);
    const rsrc_t rf = make_rsrc(p.fp8, p.N * p.K / 64);
    const rsrc_t rs = make_rsrc(p.sup, ceil_div(p.N * p.K / 64, 256) * 4);
    const rsrc_t rx = make_rsrc(p.x, p.T * p.K * 2);

    // this wave's loads first: codes, FP8 constants and super-scales of R rows
    const int64_t k = kr0 + wave * 1024 + lane * 16;
    const bool kok = k < p.K && k < kr0 + KR;
    u32x2_t cw[R];
    uint32_t f8[R];
    float s2[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t n = n0 + i;
        const bool ok = kok && n < p.N;
        const int64_t blk = n * (p.K / 64) + k / 64;
        cw[i] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                rc, ok ? (uint32_t)(n * (p.K / 2) + k / 2) : kOOB, 0, 0));
        f8[i] = __builtin_amdgcn_raw_buffer_load_b8(rf, ok ? (uint32_t)blk : kOOB, 0, 0);
        s2[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ok ? (uint32_t)(blk >> 8) * 4u : kOOB, 0, 0));
    }
    // stage X[0:TT][kr0 : kr0 + KR] (zeros past T and K)
#pragma unroll
    for (int c = 0; c < TT * KR / 8 / 256; ++c) {
        const int ch = threadIdx.x + c * 256;
        const int t = ch / (KR / 8);
        const int64_t kk = kr0 + (ch % (KR / 8)) * 8;
        const uint32_t vo = (t < p.T && kk < p.K) ? (uint32_t)((t * p.K + kk) * 2) : kOOB;
        const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, vo, 0, 0));
        *reinterpret_cast<g_lds_u32x4_t*>(xs + (int64_t)t * (KR * 2) + (ch % (KR / 8)) * 16) = v;
    }
    __syncthreads();

    float acc[R][TT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[i][t] = 0.0f;
    // A round narrower than the four wave chunks (KR = 2048) leaves waves 2, 3
    // without k: they read no X (their chunk lies outside the staged rows).
    if (wave * 1024 < KR) {
        u32x4_t xv[TT][2];
        const int xo = (wave * 1024 + lane * 16) * 2;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            xv[t][0] = *reinterpret_cast<const g_lds_u32x4_t*>(xs + t * (KR * 2) + xo);
            xv[t][1] = *reinterpret_cast<const g_lds_u32x4_t*>(xs + t * (KR * 2) + xo + 16);
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float c1p = block_scale(f8[i], s2[i]);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t byte = __builtin_amdgcn_ubfe(cw[i][d], 8 * b, 8);
                    const f32x2_t qq = *reinterpret_cast<const g_lds_f32x2_t*>(tbl + byte * 8);
                    const uint32_t wp = pack_bf16x2(__fmul_rn(qq[0], c1p), __fmul_rn(qq[1], c1p));
                    const int e = d * 4 + b;
#pragma unroll
                    for (int t = 0; t < TT; ++t) acc[i][t] = dot2(wp, xv[t][e >> 2][e & 3], acc[i][t]);
                }
            }
        }
    }
    // wave sums, then the four waves meet in LDS (reusing the X area)
    __syncthreads();
    g_lds_f32_t* red = (g_lds_f32_t*)xs;                               // [4][R][TT]
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float v = wave_sum(acc[i][t]);
            if (lane == 0) red[(wave * R + i) * TT + t] = v;
        }
    __syncthreads();
    if (threadIdx.x < R * TT) {
        const int i = threadIdx.x / TT, t = threadIdx.x % TT;
        const int64_t n = n0 + i;
        if (t < p.T && n < p.N) {
            const float v = red[(0 * R + i) * TT + t] + red[(1 * R + i) * TT + t] + red[(2 * R + i) * TT + t] +
                            red[(3 * R + i) * TT + t];
            p.part[((int64_t)ks * p.T + t) * p.N + n] = v;
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
template <int RP>
__global__ __launch_bounds__(256) void k_gemv_finalize(GemvArgs p) {
    constexpr int RQ = 16 * RP;                                        // ranks of B per wave
    __shared__ __align__(16) float pr[4 * 256];                        // group sums [G][W] float4
    __shared__ __align__(16) float ps[16 * 256];                       // s X A [T][r_pad]
    __shared__ __align__(16) float red[4 * 16 * kFinCols];             // wave sums [4][T][64]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n = (int64_t)blockIdx.x * kFinCols + lane;
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
        for (int e = eb; e < E4; e += W) {
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
            } else if (g < G) {
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
                    for (int e = 0; e < 4; ++e) v = fmaf(sv[e], bf16lo(bv[4 * q + e]), v);
                }
            }
            red[(wave * 16 + t) * kFinCols + lane] = v;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * kFinCols; i += 256) {
        const int t = i / kFinCols, l = i % kFinCols;
        const int64_t nn = (int64_t)blockIdx.x * kFinCols + l;
        if (nn < p.N) {
            const float v = red[(0 * 16 + t) * kFinCols + l] + red[(1 * 16 + t) * kFinCols + l] +
                            red[(2 * 16 + t) * kFinCols + l] + red[(3 * 16 + t) * kFinCols + l];
            p.y[t * p.N + nn] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
        }
    }
}

int gemv_ks(int64_t T, int64_t K) { return (int)ceil_div(K, T <= 8 ? 4096 : 2048); }
int gemv_kl(int64_t K) { return (int)ceil_div(K, kLoraSlice); }
size_t gemv_workspace(int64_t T, int64_t K, int64_t N, int64_t r_pad) {
    return align256((size_t)gemv_ks(T, K) * T * N * 4) + align256((size_t)gemv_kl(K) * T * (r_pad ? r_pad : 64) * 4);
}

hipError_t launch_gemv(const uint16_t* x, const uint8_t* codes, const uint8_t* fp8, const float* sup,
                       const uint16_t* lora_a, const uint16_t* lora_b, float scaling, const LoraPlan& pl,
                       uint8_t* ws, uint16_t* y, hipStream_t s) {
    GemvArgs a{x, codes, fp8, sup, lora_a, lora_b, nullptr, nullptr, y, pl.T, pl.K, pl.N, pl.r, pl.r_pad,
               gemv_ks(pl.T, pl.K), pl.r ? gemv_kl(pl.K) : 0, 0, scaling};
    a.part = reinterpret_cast<float*>(ws);
    a.lpart = reinterpret_cast<float*>(ws + align256((size_t)a.KS * pl.T * pl.N * 4));
    const Codebook& cb = host_codebook();
    const dim3 block(256);
    const int lora_blocks = pl.r ? (int)(pl.r_pad / 64) * a.KL : 0;
    hipError_t ae = hipSuccess;
    auto go = [&](auto kern, int R, int KR, int TT) {
        a.gemv_blocks = (int)ceil_div(pl.N, R) * a.KS;
        const size_t lds = 2048 + (size_t)TT * KR * 2;           // up to 66 KB: above the default limit
        ae = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds);
        if (ae == hipSuccess)
            hipLaunchKernelGGL(kern, dim3((unsigned)(a.gemv_blocks + lora_blocks)), block, lds, s, a, cb);
    };
    if (pl.T <= 1) go(k_gemv<1>, gemv_rows<1>(), gemv_round<1>(), 1);
    else if (pl.T <= 2) go(k_gemv<2>, gemv_rows<2>(), gemv_round<2>(), 2);
    else if (pl.T <= 4) go(k_gemv<4>, gemv_rows<4>(), gemv_round<4>(), 4);
    else if (pl.T <= 8) go(k_gemv<8>, gemv_rows<8>(), gemv_round<8>(), 8);
    else go(k_gemv<16>, gemv_rows<16>(), gemv_round<16>(), 16);
    if (ae != hipSuccess) return ae;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 fg((unsigned)ceil_div(pl.N, kFinCols));
    switch (pl.r_pad / 64) {
        case 0: hipLaunchKernelGGL(k_gemv_finalize<0>, fg, block, 0, s, a); break;
        case 1: hipLaunchKernelGGL(k_gemv_finalize<1>, fg, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(k_gemv_finalize<2>, fg, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL(k_gemv_finalize<3>, fg, block, 0, s, a); break;
        default: hipLaunchKernelGGL(k_gemv_finalize<4>, fg, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace ql
