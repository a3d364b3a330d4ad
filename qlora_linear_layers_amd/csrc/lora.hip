// The rank-r products of the LoRA branch on gfx950 (Volcengine article
// section 3.4 for the layer; the gradients follow by differentiation, and
// only the adapters receive them, "从LoRA到QLoRA" section 3.1):
//
//   down projections   P = s X A      [T, r]   (forward and backward)
//                      G = s dY B^T   [T, r]   (backward)
//   adapter gradients  dA = X^T G     [K, r]
//                      dB = P^T dY    [r, N]
//
// All four are bound by reading the big operand (X or dY) once from HBM; the
// r-wide operands are small and stay in L2.  They use v_mfma_f32_16x16x32_bf16
// (lane l holds 8 consecutive reduction elements of row / column l % 16, group
// l / 16; the 4 results of lane l are column l % 16, rows 4 (l / 16) .. +3).
//
// k_down: a workgroup owns 64 rows of X (or dY) and a range of the reduction,
// staged through LDS in whole cache lines; the ranges of one row tile are
// added in a fixed order by k_down_fin.  P and G leave as bf16 hi +
// lo pairs (hi = RNE(v), lo = RNE(v - hi)), row-major for the GEMM kernels and
// transposed for k_grad.  A is transposed once per call by k_transpose so that
// both down projections read the r-wide operand as rows.
//
// k_grad: the adapter-gradient block product of grad.hpp, one 128-column x
// 64-rank block per workgroup; token ranges of different workgroups produce
// fp32 partials that k_grad_finalize sums in split order.  Every result is
// deterministic.
#include "common.hpp"
#include "grad.hpp"
#include "plan.hpp"

namespace ql {

namespace {

constexpr int kThreads = 256;

template <bool F16>
QL_DEV f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return mfma16x16x32<F16>(a, b, c);
}

QL_DEV bf16x8_t as_bf16x8(const u32x4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// hi = RNE_16(v), lo = RNE_16(v - hi) as 16-bit patterns (bf16, or fp16 when F16)
template <bool F16>
QL_DEV void split_hi_lo(float v, uint16_t& hi, uint16_t& lo) {
    const uint32_t hb = pack16x2<F16>(v, 0.0f) & 0xFFFFu;
    hi = (uint16_t)hb;
    lo = (uint16_t)(pack16x2<F16>(v - lo16<F16>(hb), 0.0f) & 0xFFFFu);
}

}  // namespace

// ------------------------------------------------------------------ transpose

// dst[j][k] (row stride ldd) = src[k][j] for j < r, 0 for r <= j < r_pad
// (src [K][r] bf16, r a multiple of 8).  One workgroup per 64 k x 64 j tile:
// 16-byte loads of 8 j, an LDS tile, 16-byte stores of 8 k.
__global__ __launch_bounds__(kThreads) void k_transpose(const uint16_t* __restrict__ src, int64_t K, int64_t r,
                                                        int64_t r_pad, int64_t ldd, uint16_t* __restrict__ dst) {
    __shared__ uint16_t tile[64][64 + 8];
    const int64_t k0 = (int64_t)blockIdx.x * 64, j0 = (int64_t)blockIdx.y * 64;
    const int row = threadIdx.x >> 3, c8 = (threadIdx.x & 7) * 8;     // 32 rows x 8 chunks per pass
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kk = row + 32 * h;
        const int64_t k = k0 + kk, j = j0 + c8;
        u32x4_t v = {0, 0, 0, 0};
        if (k < K && j < r) v = *reinterpret_cast<const u32x4_t*>(src + k * r + j);
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[kk][c8 + e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int jj = row + 32 * h;
        const int64_t j = j0 + jj, k = k0 + c8;
        if (j >= r_pad || k >= K) continue;
        u32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (uint32_t)tile[c8 + 2 * e][jj] | ((uint32_t)tile[c8 + 2 * e + 1][jj] << 16);
        *reinterpret_cast<u32x4_t*>(dst + j * ldd + k) = v;
    }
}

// ------------------------------------------------------------------ down projections

struct DownArgs {
    const uint16_t* s;    // [T][L] bf16 (X or dY)
    const uint16_t* m;    // [m_rows][ldm] bf16 (A^T or B); rows m_rows .. r_pad-1 read as zero
    int64_t T, L, ldm, m_rows, r_pad;
    float scale;
    uint16_t* hi;         // [T][r_pad]
    uint16_t* lo;
    uint16_t* hit;        // [r_pad][ldt] (tokens [0, T8), T8 = T rounded up to 8) or null
    uint16_t* lot;
    int64_t T8, ldt;
    float* part;          // [splits][T][r_pad] fp32 partial sums (splits > 1)
    int splits;
    ScalesJob sj;         // the dX kernel's transposed block scales, as extra workgroups (sj.blocks may be 0)
};

// v (already scaled) -> hi/lo at row t, column j of both layouts
template <bool F16>
QL_DEV void down_out(const DownArgs& a, int64_t t, int j, float v, bool rowmajor) {
    uint16_t h, lw;
    split_hi_lo<F16>(v, h, lw);
    if (rowmajor) {
        if (t < a.T) {
            a.hi[t * a.r_pad + j] = h;
            a.lo[t * a.r_pad + j] = lw;
        }
    } else if (t < a.T8) {          // tokens [T, T8) are zeros (their S rows read as zero)
        a.hit[j * a.ldt + t] = h;
        a.lot[j * a.ldt + t] = lw;
    }
}

// sum[ROWS][R] (row stride R + 4) of rows t0 .. t0+ROWS-1 -> both output layouts
template <int R, int ROWS, bool F16>
QL_DEV void down_emit(const DownArgs& a, const float* sum, int64_t t0) {
    for (int e = threadIdx.x; e < ROWS * R; e += kThreads) {      // [T][r_pad], j fastest
        const int tl = e / R, j = e % R;
        down_out<F16>(a, t0 + tl, j, sum[tl * (R + 4) + j] * a.scale, true);
    }
    if (a.hit)
        for (int e = threadIdx.x; e < ROWS * R; e += kThreads) {  // [r_pad][ldt], t fastest
            const int j = e / ROWS, tl = e % ROWS;
            down_out<F16>(a, t0 + tl, j, sum[tl * (R + 4) + j] * a.scale, false);
        }
}

// out[t][j] = scale * sum_l S[t][l] M[j][l].  A workgroup owns 64 rows t
// (wave w: rows 16w .. 16w+15, all r_pad columns) and one of `splits` ranges
// of the reduction, walked in rounds of 64: each round's 64 rows of S and
// r_pad rows of M (128 contiguous bytes per row) are loaded PD rounds ahead
// into registers, written to a swizzled LDS buffer and read back as MFMA
// fragments, so every global load fetches whole cache lines and M is read
// once per 64 rows.  With several splits each workgroup stores an fp32
// partial (whole rows, through LDS) and k_down_fin adds them in split order.
template <int RT, bool F16>
__global__ __launch_bounds__(kThreads, 2) void k_down(DownArgs a) {
    constexpr int PD = RT <= 4 ? 4 : 2;
    constexpr int NX = 2;            // 16-byte chunks of the 64 x 64 S tile per thread
    constexpr int NM = RT / 2;       // 16-byte chunks of the r_pad x 64 M tile per thread
    constexpr int R = RT * 16;
    extern __shared__ __align__(16) uint8_t smem_raw[];
    lds8_t* smem = (lds8_t*)(smem_raw);
    constexpr uint32_t kXT = 64 * 128, kMT = R * 128, kBuf = kXT + kMT;
    const int tiles = (int)ceil_div(a.T, 64);
    const int bid = (int)blockIdx.x;
    if (bid >= tiles * a.splits) {              // block-scale workgroups of the same launch, dispatched
        scales_job(a.sj, bid - tiles * a.splits, smem);   // after the longer projection workgroups
        return;
    }
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tile = bid % tiles, split = bid / tiles;
    const int64_t t0 = (int64_t)tile * 64;
    const int nr_all = (int)(a.L / 64);
    const int r0 = split * nr_all / a.splits, r1 = (split + 1) * nr_all / a.splits;
    const int nr = r1 - r0;

    const rsrc_t rx = make_rsrc(a.s, a.T * a.L * 2);
    const rsrc_t rm = make_rsrc(a.m, a.m_rows * a.ldm * 2);
    uint32_t xo[NX], mo[NM];
#pragma unroll
    for (int u = 0; u < NX; ++u) {
        const int q = threadIdx.x + u * kThreads;
        const int64_t t = t0 + (q >> 3);
        xo[u] = t < a.T ? (uint32_t)((t * a.L + (int64_t)r0 * 64 + (q & 7) * 8) * 2) : kOOB;
    }
#pragma unroll
    for (int u = 0; u < NM; ++u) {
        const int q = threadIdx.x + u * kThreads;
        const int64_t j = q >> 3;
        mo[u] = j < a.m_rows ? (uint32_t)((j * a.ldm + (int64_t)r0 * 64 + (q & 7) * 8) * 2) : kOOB;
    }
    u32x4_t xr[PD][NX], mr[PD][NM];
    auto load = [&](int i, int slot) {           // round i of this split (zeros past nr)
        const bool ok = i < nr;
        const uint32_t so = ok ? (uint32_t)i * 128u : 0u;
#pragma unroll
        for (int u = 0; u < NX; ++u) xr[slot][u] = bload16(rx, ok ? xo[u] : kOOB, so);
#pragma unroll
        for (int u = 0; u < NM; ++u) mr[slot][u] = bload16(rm, ok ? mo[u] : kOOB, so);
    };
    auto store = [&](int slot, lds8_t* buf) {
#pragma unroll
        for (int u = 0; u < NX; ++u) {
            const int q = threadIdx.x + u * kThreads;
            *reinterpret_cast<lds_u32x4_t*>(buf + lds_off(q >> 3, q & 7)) = xr[slot][u];
        }
#pragma unroll
        for (int u = 0; u < NM; ++u) {
            const int q = threadIdx.x + u * kThreads;
            *reinterpret_cast<lds_u32x4_t*>(buf + kXT + lds_off(q >> 3, q & 7)) = mr[slot][u];
        }
    };

    f32x4_t acc[RT];
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) acc[jt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const lds8_t* buf) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int ch = 4 * st + (l >> 4);
            const bf16x8_t xv = *reinterpret_cast<const lds_bf16x8_t*>(buf + lds_off(16 * w + (l & 15), ch));
#pragma unroll
            for (int jt = 0; jt < RT; ++jt) {
                const bf16x8_t mv = *reinterpret_cast<const lds_bf16x8_t*>(buf + kXT + lds_off(16 * jt + (l & 15), ch));
                acc[jt] = mfma16<F16>(xv, mv, acc[jt]);
            }
        }
    };
    // the loop runs whole groups of PD rounds (rounds past nr load zeros), so
    // it has no branches and the loads stay in flight across it
#pragma unroll
    for (int p = 0; p < PD; ++p) load(p, p);
    for (int i = 0; i < nr; i += PD) {
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            lds8_t* buf = smem + ((i + p) & 1) * kBuf;
            store(p, buf);
            load(i + p + PD, p);
            __syncthreads();
            compute(buf);
        }
    }

    // the tile's sums [64][R] in LDS (the round buffers are free after a barrier)
    __syncthreads();
    float* sum = reinterpret_cast<float*>(smem_raw);
#pragma unroll
    for (int jt = 0; jt < RT; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sum[(16 * w + 4 * (l >> 4) + v) * (R + 4) + 16 * jt + (l & 15)] = acc[jt][v];
    __syncthreads();
    if (a.splits == 1) {
        down_emit<R, 64, F16>(a, sum, t0);
        return;
    }
    float* out = a.part + (int64_t)split * a.T * a.r_pad;     // whole rows, 16 bytes per lane
    for (int e = threadIdx.x; e < 16 * R; e += kThreads) {
        const int tl = e / (R / 4), j = 4 * (e % (R / 4));
        const int64_t t = t0 + tl;
        if (t < a.T) {
            const float* src = sum + tl * (R + 4) + j;
            *reinterpret_cast<f32x4_t*>(out + t * a.r_pad + j) = f32x4_t{src[0], src[1], src[2], src[3]};
        }
    }
}

// Split-ordered sum of the k_down partials of 16 rows, then both layouts.
template <int RT, bool F16>
__global__ __launch_bounds__(kThreads) void k_down_fin(DownArgs a) {
    constexpr int R = RT * 16;
    extern __shared__ __align__(16) uint8_t smem_raw[];
    float* sum = reinterpret_cast<float*>(smem_raw);           // [16][R + 4]
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    for (int e = threadIdx.x; e < 4 * R; e += kThreads) {
        const int tl = e / (R / 4), j = 4 * (e % (R / 4));
        const int64_t t = t0 + tl;
        f32x4_t v[8];
#pragma unroll
        for (int sp = 0; sp < 8; ++sp)                            // splits <= 8: loads issued together
            v[sp] = (sp < a.splits && t < a.T)
                        ? *reinterpret_cast<const f32x4_t*>(a.part + ((int64_t)sp * a.T + t) * a.r_pad + j)
                        : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        f32x4_t s4 = v[0];
#pragma unroll
        for (int sp = 1; sp < 8; ++sp) s4 += v[sp];
#pragma unroll
        for (int c = 0; c < 4; ++c) sum[tl * (R + 4) + j + c] = s4[c];
    }
    __syncthreads();
    down_emit<R, 16, F16>(a, sum, t0);
}

// ------------------------------------------------------------------ adapter gradients

// One launch serves both adapter gradients: workgroups [0, blocks0) take
// problem a0 (dA = X^T G), the rest problem a1 (dB = P^T dY); blockIdx.y
// picks the 64 ranks.
template <bool F16>
__global__ __launch_bounds__(kThreads, 1) void k_grad(GradArgs a0, GradArgs a1, int blocks0) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    const bool second = (int)blockIdx.x >= blocks0;
    const GradArgs& a = second ? a1 : a0;
    const int bx = second ? (int)blockIdx.x - blocks0 : (int)blockIdx.x;
    grad_block<F16>(a, bx % a.cblocks, bx / a.cblocks, (int64_t)blockIdx.y * 64, reinterpret_cast<float*>(smem_raw));
}

// dA[k][j] (transpose = 0) or dB[j][n] (transpose = 1): RNE_bf16 of the
// split-ordered sum of part[s][c][j], j < r.  One workgroup per 16 columns c;
// a thread sums four consecutive j with its split loads issued in batches of
// eight.  The transposed output goes through an LDS tile so that its stores
// run along c.  Workgroups [0, blocks0) serve the first problem, the rest the
// second.
struct GradFin {
    const float* part;
    int splits;
    int64_t C, r_pad, r;
    uint16_t* out;
    int transpose;
};

template <bool F16>
__global__ __launch_bounds__(256) void k_grad_finalize(GradFin f0, GradFin f1, int blocks0) {
    __shared__ uint16_t tile[256][16 + 2];              // [j][c] for the transposed output
    const bool second = (int)blockIdx.x >= blocks0;
    const GradFin& f = second ? f1 : f0;
    const int64_t c0 = (int64_t)(second ? (int)blockIdx.x - blocks0 : (int)blockIdx.x) * 16;
    const int64_t stride = f.C * f.r_pad;
    const int q = (int)(f.r_pad / 4);
    for (int e = threadIdx.x; e < 16 * q; e += 256) {
        const int cl = e / q, j = 4 * (e % q);
        const int64_t c = c0 + cl;
        f32x4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
        if (c < f.C) {
            const float* src = f.part + c * f.r_pad + j;
            int s = 0;
            for (; s + 8 <= f.splits; s += 8) {
                f32x4_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4_t*>(src + (int64_t)(s + u) * stride);
#pragma unroll
                for (int u = 0; u < 8; ++u) sum += v[u];
            }
            for (; s < f.splits; ++s) sum += *reinterpret_cast<const f32x4_t*>(src + (int64_t)s * stride);
        }
        const uint32_t p01 = pack16x2<F16>(sum[0], sum[1]), p23 = pack16x2<F16>(sum[2], sum[3]);
        if (!f.transpose) {
            if (c < f.C && j < f.r) *reinterpret_cast<u32x2_t*>(f.out + c * f.r + j) = u32x2_t{p01, p23};
        } else {
            tile[j][cl] = (uint16_t)p01;
            tile[j + 1][cl] = (uint16_t)(p01 >> 16);
            tile[j + 2][cl] = (uint16_t)p23;
            tile[j + 3][cl] = (uint16_t)(p23 >> 16);
        }
    }
    if (!f.transpose) return;
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * f.r; e += 256) {
        const int j = e / 16, cl = e % 16;
        const int64_t c = c0 + cl;
        if (c < f.C) f.out[j * f.C + c] = tile[j][cl];
    }
}

// ------------------------------------------------------------------ launchers

namespace {

template <class F>
hipError_t set_smem(F* f, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int RT, bool F16>
hipError_t down_rt(const DownArgs& a, hipStream_t s) {
    constexpr int R = RT * 16;
    const size_t bufs = (size_t)2 * (64 + R) * 128, sums = (size_t)64 * (R + 4) * 4;
    const size_t lds = bufs > sums ? bufs : sums;
    hipError_t e = set_smem(k_down<RT, F16>, lds);
    if (e != hipSuccess) return e;
    const unsigned tiles = (unsigned)ceil_div(a.T, 64);
    hipLaunchKernelGGL((k_down<RT, F16>), dim3(tiles * (unsigned)a.splits + (unsigned)a.sj.blocks), dim3(kThreads),
                       lds, s, a);
    if (a.splits > 1) {
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const size_t fl = (size_t)16 * (R + 4) * 4;
        hipLaunchKernelGGL((k_down_fin<RT, F16>), dim3((unsigned)ceil_div(a.T, 16)), dim3(kThreads), fl, s, a);
    }
    return hipGetLastError();
}

template <bool F16>
hipError_t down_t(const DownArgs& a, hipStream_t s) {
    switch (a.r_pad / 16) {
        case 4: return down_rt<4, F16>(a, s);
        case 8: return down_rt<8, F16>(a, s);
        case 12: return down_rt<12, F16>(a, s);
        case 16: return down_rt<16, F16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t down(const DownArgs& a, hipStream_t s, bool f16) { return f16 ? down_t<true>(a, s) : down_t<false>(a, s); }

// One k_grad launch over up to two problems (`n1` = 0: a0 alone).
hipError_t grad(const GradArgs& a0, int n0, const GradArgs& a1, int n1, int64_t r_pad, hipStream_t s, bool f16) {
    auto go = [&](auto kern) {
        hipError_t e = set_smem(kern, kGradSmem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)(n0 + n1), (unsigned)(r_pad / 64)), dim3(kThreads), kGradSmem, s,
                           a0, a1, n0);
        return hipGetLastError();
    };
    return f16 ? go(k_grad<true>) : go(k_grad<false>);
}

// One k_grad_finalize launch for dA (fa, when has_a) and dB (fb, when has_b).
hipError_t grad_finalize(GradFin fa, bool has_a, const GradFin& fb, bool has_b, const LoraPlan& pl, hipStream_t s,
                         bool f16) {
    const int ba = has_a ? (int)ceil_div(pl.K, 16) : 0;
    const int bb = has_b ? (int)ceil_div(pl.N, 16) : 0;
    if (!has_a) fa = fb;                   // a single problem runs as the first one
    if (f16)
        hipLaunchKernelGGL(k_grad_finalize<true>, dim3((unsigned)(ba + bb)), dim3(256), 0, s, fa, fb,
                           has_a ? ba : bb);
    else
        hipLaunchKernelGGL(k_grad_finalize<false>, dim3((unsigned)(ba + bb)), dim3(256), 0, s, fa, fb,
                           has_a ? ba : bb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose_a(const uint16_t* lora_a, const LoraPlan& pl, uint8_t* ws, hipStream_t s) {
    uint16_t* at = reinterpret_cast<uint16_t*>(ws + pl.off_at);
    hipLaunchKernelGGL(k_transpose, dim3((unsigned)ceil_div(pl.K, 64), (unsigned)(pl.r_pad / 64)), dim3(kThreads),
                       0, s, lora_a, pl.K, pl.r, pl.r_pad, pl.ld_at, at);
    return hipGetLastError();
}

// s X A -> P (hi/lo [T][r_pad]; also transposed when `transposed`).  Needs A^T in ws.
hipError_t launch_lora_down_x(const uint16_t* x, float scaling, const LoraPlan& pl, uint8_t* ws, bool transposed,
                              hipStream_t s, bool f16) {
    DownArgs a{x, reinterpret_cast<const uint16_t*>(ws + pl.off_at), pl.T, pl.K, pl.ld_at, pl.r_pad, pl.r_pad,
               scaling,
               reinterpret_cast<uint16_t*>(ws + pl.off_ps_hi), reinterpret_cast<uint16_t*>(ws + pl.off_ps_lo),
               transposed ? reinterpret_cast<uint16_t*>(ws + pl.off_pst_hi) : nullptr,
               transposed ? reinterpret_cast<uint16_t*>(ws + pl.off_pst_lo) : nullptr, pl.T8, pl.ld_t,
               reinterpret_cast<float*>(ws + pl.off_dpart), pl.s_down_x, ScalesJob{}};
    return down(a, s, f16);
}

// s dY B^T -> G (hi/lo [T][r_pad] and transposed); `scales` (if not NULL) runs
// as extra workgroups of the same launch.
hipError_t launch_lora_down_dy(const uint16_t* dy, const uint16_t* lora_b, float scaling, const LoraPlan& pl,
                               uint8_t* ws, bool transposed, hipStream_t s, bool f16, const ScalesJob* scales) {
    DownArgs a{dy, lora_b, pl.T, pl.N, pl.N, pl.r, pl.r_pad, scaling,
               reinterpret_cast<uint16_t*>(ws + pl.off_gs_hi), reinterpret_cast<uint16_t*>(ws + pl.off_gs_lo),
               transposed ? reinterpret_cast<uint16_t*>(ws + pl.off_gst_hi) : nullptr,
               transposed ? reinterpret_cast<uint16_t*>(ws + pl.off_gst_lo) : nullptr, pl.T8, pl.ld_t,
               reinterpret_cast<float*>(ws + pl.off_dpart), pl.s_down_dy, scales ? *scales : ScalesJob{}};
    return down(a, s, f16);
}

// dA = X^T G and dB = P^T dY from the transposed intermediates in ws.
hipError_t launch_lora_grads(const uint16_t* x, const uint16_t* dy, const LoraPlan& pl, uint8_t* ws,
                             uint16_t* d_lora_a, uint16_t* d_lora_b, hipStream_t s, bool f16) {
    float* pda = reinterpret_cast<float*>(ws + pl.off_pda);
    float* pdb = reinterpret_cast<float*>(ws + pl.off_pdb);
    GradFin fa{pda, pl.s_da, pl.K, pl.r_pad, pl.r, d_lora_a, 0};
    GradFin fb{pdb, pl.s_db, pl.N, pl.r_pad, pl.r, d_lora_b, 1};
    // dA and dB in one launch (either may be absent)
    const GradArgs ga{x, reinterpret_cast<const uint16_t*>(ws + pl.off_gst_hi),
                      reinterpret_cast<const uint16_t*>(ws + pl.off_gst_lo), pda, pl.T, pl.T8, pl.ld_t, pl.K,
                      pl.r_pad, (int)ceil_div(pl.K, 128), pl.cpw_da};
    const GradArgs gb{dy, reinterpret_cast<const uint16_t*>(ws + pl.off_pst_hi),
                      reinterpret_cast<const uint16_t*>(ws + pl.off_pst_lo), pdb, pl.T, pl.T8, pl.ld_t, pl.N,
                      pl.r_pad, (int)ceil_div(pl.N, 128), pl.cpw_db};
    const int na = d_lora_a ? ga.cblocks * pl.s_da : 0, nb = d_lora_b ? gb.cblocks * pl.s_db : 0;
    {
        hipError_t e = na ? grad(ga, na, gb, nb, pl.r_pad, s, f16) : grad(gb, nb, gb, 0, pl.r_pad, s, f16);
        if (e != hipSuccess) return e;
    }
    return grad_finalize(fa, d_lora_a != nullptr, fb, d_lora_b != nullptr, pl, s, f16);
}

// The fused backward's gradient problems: S = X against G^T for dA and S = dY
// against P^T for dB, one group of fz_tpg 256-token tiles per split, partials
// in the fused region of ws.
FusedGrads fused_grads_for(const uint16_t* x, const uint16_t* dy, const LoraPlan& pl, uint8_t* ws, bool da,
                           bool db) {
    FusedGrads f{};
    f.tpg = pl.fz_tpg;
    f.groups = pl.s_fz;
    f.waves = 0;                                   // set by the dX launcher from its grid
    if (da)
        f.ga = GradArgs{x, reinterpret_cast<const uint16_t*>(ws + pl.off_gst_hi),
                        reinterpret_cast<const uint16_t*>(ws + pl.off_gst_lo), reinterpret_cast<float*>(ws + pl.off_fza),
                        pl.T, pl.T8, pl.ld_t, pl.K, pl.r_pad, (int)ceil_div(pl.K, 128), 8};
    if (db)
        f.gb = GradArgs{dy, reinterpret_cast<const uint16_t*>(ws + pl.off_pst_hi),
                        reinterpret_cast<const uint16_t*>(ws + pl.off_pst_lo), reinterpret_cast<float*>(ws + pl.off_fzb),
                        pl.T, pl.T8, pl.ld_t, pl.N, pl.r_pad, (int)ceil_div(pl.N, 128), 8};
    return f;
}

// dA and dB from the fused backward's partials (one per 256-token tile).
hipError_t launch_fused_grads_finalize(const LoraPlan& pl, uint8_t* ws, uint16_t* d_lora_a, uint16_t* d_lora_b,
                                       hipStream_t s, bool f16) {
    const GradFin fa{reinterpret_cast<const float*>(ws + pl.off_fza), pl.s_fz, pl.K, pl.r_pad, pl.r, d_lora_a, 0};
    const GradFin fb{reinterpret_cast<const float*>(ws + pl.off_fzb), pl.s_fz, pl.N, pl.r_pad, pl.r, d_lora_b, 1};
    return grad_finalize(fa, d_lora_a != nullptr, fb, d_lora_b != nullptr, pl, s, f16);
}

}  // namespace ql
