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
// Mapping: a workgroup of four wave64s owns 16 consecutive rows of W (four
// per wave).  The reduction over K runs in slices of 1024: the slice of X
// (T x 1024 bf16) is staged in LDS once per workgroup, each lane takes 16
// consecutive k of the slice (8 code bytes per row, one block scale per row),
// dequantizes them once and multiplies them with all T tokens using
// v_dot2_f32_bf16 (two products per instruction, fp32 accumulation).  At the
// end the LoRA up-projection is added lane-parallel over the rank and a
// butterfly reduction over the wave gives each (row, token) sum.
#include "common.hpp"
#include "plan.hpp"

namespace ql {

namespace {

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t g_lds8_t;
typedef __attribute__((address_space(3))) u32x4_t g_lds_u32x4_t;
typedef __attribute__((address_space(3))) f32x2_t g_lds_f32x2_t;
typedef __amdgpu_buffer_rsrc_t g_rsrc_t;
constexpr uint32_t kGOOB = 0x80000000u;

__device__ __forceinline__ g_rsrc_t g_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
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
constexpr int kLoraSlice = 256;   // k per LoRA down-projection workgroup

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
        // X[0:TT][slice] is staged in LDS; lane j of wave g loads its 64 A values
        // (rows k0 + 64g .. +63) in one burst, then reads X as LDS broadcasts.
        const int lb = (int)blockIdx.x - p.gemv_blocks;
        const int jc = lb % (int)(p.r_pad / 64), kl = lb / (int)(p.r_pad / 64);
        const int64_t j = (int64_t)jc * 64 + lane;
        const int64_t k0 = (int64_t)kl * kLoraSlice;
        g_lds8_t* xl = base;                                           // [TT][256] bf16
        for (int ch = threadIdx.x; ch < TT * (kLoraSlice / 8); ch += 256) {
            const int t = ch / (kLoraSlice / 8);
            const int64_t kk = k0 + (ch % (kLoraSlice / 8)) * 8;
            u32x4_t v = {0, 0, 0, 0};
            if (t < p.T && kk < p.K) v = *reinterpret_cast<const u32x4_t*>(p.x + t * p.K + kk);
            *reinterpret_cast<g_lds_u32x4_t*>(xl + (t * kLoraSlice + (ch % (kLoraSlice / 8)) * 8) * 2) = v;
        }
        float av[64];
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const int64_t k = k0 + 64 * wave + i;
            av[i] = (j < p.r && k < p.K) ? bf16lo(p.lora_a[k * p.r + j]) : 0.0f;
        }
        __syncthreads();
        float acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float v = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const u32x4_t xv = *reinterpret_cast<const g_lds_u32x4_t*>(xl + (t * kLoraSlice + 64 * wave + 8 * c) * 2);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v = fmaf(bf16lo(xv[e]), av[8 * c + 2 * e], v);
                    v = fmaf(bf16hi(xv[e]), av[8 * c + 2 * e + 1], v);
                }
            }
            acc[t] = v;
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
    const g_rsrc_t rc = g_rsrc(p.codes, p.N * p.K / 2);
    const g_rsrc_t rf = g_rsrc(p.fp8, p.N * p.K / 64);
    const g_rsrc_t rs = g_rsrc(p.sup, ceil_div(p.N * p.K / 64, 256) * 4);
    const g_rsrc_t rx = g_rsrc(p.x, p.T * p.K * 2);

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
                                                rc, ok ? (uint32_t)(n * (p.K / 2) + k / 2) : kGOOB, 0, 0));
        f8[i] = __builtin_amdgcn_raw_buffer_load_b8(rf, ok ? (uint32_t)blk : kGOOB, 0, 0);
        s2[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, ok ? (uint32_t)(blk >> 8) * 4u : kGOOB, 0, 0));
    }
    // stage X[0:TT][kr0 : kr0 + KR] (zeros past T and K)
#pragma unroll
    for (int c = 0; c < TT * KR / 8 / 256; ++c) {
        const int ch = threadIdx.x + c * 256;
        const int t = ch / (KR / 8);
        const int64_t kk = kr0 + (ch % (KR / 8)) * 8;
        const uint32_t vo = (t < p.T && kk < p.K) ? (uint32_t)((t * p.K + kk) * 2) : kGOOB;
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
    // wave butterfly, then the four waves meet in LDS (reusing the X area)
    __syncthreads();
    g_lds_f32_t* red = (g_lds_f32_t*)xs;                               // [4][R][TT]
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float v = acc[i][t];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
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

// Launch 2.  s X A from its slice partials (fixed order, loads issued in
// batches of 8), then Y[t][n] = sum_ks part[ks][t][n] + sum_j (s X A)[t][j] B[j][n]
// rounded to bf16.  Thread n loads its column of B 64 ranks at a time before
// using it.
__global__ __launch_bounds__(256) void k_gemv_finalize(GemvArgs p) {
    __shared__ float ps[16 * 256];                                     // [T][r] (T <= 16, r <= 256)
    for (int64_t i = threadIdx.x; i < p.T * p.r; i += 256) {
        const int64_t t = i / p.r, j = i % p.r;
        const float* src = p.lpart + t * p.r_pad + j;
        const int64_t stride = p.T * p.r_pad;
        float v = 0.0f;
        int kl = 0;
        for (; kl + 8 <= p.KL; kl += 8) {
            float b[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) b[u] = src[(kl + u) * stride];
#pragma unroll
            for (int u = 0; u < 8; ++u) v += b[u];
        }
        for (; kl < p.KL; ++kl) v += src[kl * stride];
        ps[i] = v * p.scaling;
    }
    __syncthreads();
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= p.N) return;
    float y[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) y[t] = 0.0f;
    for (int ks = 0; ks < p.KS; ++ks) {
        float v[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) v[t] = t < p.T ? p.part[((int64_t)ks * p.T + t) * p.N + n] : 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) y[t] += v[t];
    }
    for (int64_t j0 = 0; j0 < p.r; j0 += 64) {
        float bv[64];
#pragma unroll
        for (int u = 0; u < 64; ++u) bv[u] = (j0 + u < p.r) ? bf16lo(p.lora_b[(j0 + u) * p.N + n]) : 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            if (t >= p.T) continue;
            float v = y[t];
#pragma unroll
            for (int u = 0; u < 64; ++u)
                if (j0 + u < p.r) v = fmaf(ps[t * p.r + j0 + u], bv[u], v);
            y[t] = v;
        }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t)
        if (t < p.T) p.y[t * p.N + n] = (uint16_t)(pack_bf16x2(y[t], 0.0f) & 0xFFFFu);
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
    hipLaunchKernelGGL(k_gemv_finalize, dim3((unsigned)ceil_div(pl.N, 256)), block, 0, s, a);
    return hipGetLastError();
}

}  // namespace ql
