// MFMA GEMMs of the QLoRA linear layer on gfx950, with NF4 double
// dequantization fused into the LDS tile producers.
//
// Layer (Volcengine article section 3.4, equation lost; reading used):
//   Y  = X W'^T + s (X A) B
//   dX = dY W'  + s (dY B^T) A^T,   dA = s X^T (dY B^T),   dB = s (X A)^T dY
// with W' the double-dequantized bf16 weight ("QLoRA 原理精讲" section 2.2:
// super-scale, then block constant, then weight) that is never written to HBM.
//
// Structure.  Every product here is C[a][b] = sum_k Pa(a, k) * Pb(b, k) with
// both operands staged in LDS as [rows][64] bf16 tiles (reduction contiguous),
// consumed by v_mfma_f32_32x32x16_bf16 from four wave64s arranged 2 x 2.
// What differs between the products is only how a tile is produced:
//   PlainRows  - bf16 rows already contiguous along the reduction (X, dY, ...)
//   NF4Rows    - W rows: 64 codes + one block scale per row -> bf16 in LDS
//   NF4Cols    - W read transposed for dX: an 8 x 8 code patch per thread,
//                dequantized and paired across rows by the bf16 pack itself
//   TransRows  - bf16 stored with the reduction as the row index (A, B, X, dY
//                in the LoRA products): pairs of rows packed into dwords
// and how C leaves the kernel (bf16 rows of the output, or fp32 split-K
// partials reduced in a fixed order by a finalize kernel, so results are
// deterministic).
#include "common.hpp"
#include "plan.hpp"

namespace ql {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// LDS tile of [rows][64] bf16: 128 bytes per row in 16-byte chunks, the chunk
// index XOR-swizzled with bits of the row so that the 32-row fragment reads
// (fixed chunk) and every producer's writes spread over all banks.
QL_DEV uint32_t lds_off(int row, int chunk) {
    return (uint32_t)row * 128u + ((uint32_t)(chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// ------------------------------------------------------------------ producers

template <int ROWS>
struct PlainRows {
    static constexpr int kChunks = ROWS * 8 / kThreads;     // 16-byte chunks per thread
    const uint16_t* src;
    int64_t ld;          // elements between consecutive rows
    int64_t nrows;       // valid rows (global)
    int64_t red_len;     // valid reduction length (multiple of 8)
    int64_t row0;
    // Reduction tiles kt >= split_kt read src2 at tile kt - split_kt (the
    // second half of a concatenated reduction, e.g. the lo part of hi/lo).
    const uint16_t* src2 = nullptr;
    int split_kt = 1 << 30;
    u32x4_t reg[kChunks];

    QL_DEV void load(int kt) {
        const uint16_t* base = kt < split_kt ? src : src2;
        const int ktl = kt < split_kt ? kt : kt - split_kt;
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int64_t gr = row0 + (c >> 3);
            const int64_t k = (int64_t)ktl * 64 + (c & 7) * 8;
            if (gr < nrows && k < red_len)
                reg[i] = *reinterpret_cast<const u32x4_t*>(base + gr * ld + k);
            else
                reg[i] = u32x4_t{0, 0, 0, 0};
        }
    }
    QL_DEV void store(uint8_t* lds, const float*) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = threadIdx.x + i * kThreads;
            *reinterpret_cast<u32x4_t*>(lds + lds_off(c >> 3, c & 7)) = reg[i];
        }
    }
};

// Dequantize 8 codes of one packed dword (element 2i in the high nibble of
// byte i) with block scale c1': w' = RNE_bf16(fl32(q[code] * c1')), packed in
// element order.
QL_DEV u32x4_t dequant8(uint32_t d, float c1p, const float* q) {
    u32x4_t o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (d >> (8 * b)) & 0xFFu;
        o[b] = pack_bf16x2(__fmul_rn(q[byte >> 4], c1p), __fmul_rn(q[byte & 15u], c1p));
    }
    return o;
}

// W [N, K] rows n0 .. n0+255 for reduction tile kt: thread t owns row n0 + t and
// its NF4 block kt (64 codes = 32 bytes, one FP8 constant, one super-scale).
struct NF4Rows {
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    int64_t K, N, row0;
    u32x4_t c0, c1;
    uint32_t f8;
    float s2;

    QL_DEV void load(int kt) {
        const int64_t n = row0 + threadIdx.x;
        if (n < N) {
            const uint8_t* p = codes + n * (K / 2) + (int64_t)kt * 32;
            c0 = *reinterpret_cast<const u32x4_t*>(p);
            c1 = *reinterpret_cast<const u32x4_t*>(p + 16);
            const int64_t b = n * (K / 64) + kt;
            f8 = fp8[b];
            s2 = sup[b >> 8];
        } else {
            c0 = c1 = u32x4_t{0, 0, 0, 0};
            f8 = 0;
            s2 = 0.0f;
        }
    }
    QL_DEV void store(uint8_t* lds, const float* q) {
        const float c1p = __fmul_rn(e4m3_decode(f8), s2);
        const int row = threadIdx.x;
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
            const uint32_t d = ch < 4 ? c0[ch] : c1[ch - 4];
            *reinterpret_cast<u32x4_t*>(lds + lds_off(row, ch)) = dequant8(d, c1p, q);
        }
    }
};

// W read transposed for dX: tile rows are k (256 of them), the reduction runs
// over n (64 per tile).  Thread t owns k = k0 + (t % 32) * 8 .. +7 and
// n = kt*64 + (t / 32) * 8 .. +7: eight 4-byte code words, eight scales.
struct NF4Cols {
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    int64_t K, N, col0;
    uint32_t cw[8], f8[8];
    float s2[8];

    QL_DEV void load(int kt) {
        const int64_t k = col0 + (threadIdx.x & 31) * 8;
        const int64_t n0 = (int64_t)kt * 64 + (threadIdx.x >> 5) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t n = n0 + i;
            if (k < K) {
                cw[i] = *reinterpret_cast<const uint32_t*>(codes + n * (K / 2) + k / 2);
                const int64_t b = n * (K / 64) + k / 64;
                f8[i] = fp8[b];
                s2[i] = sup[b >> 8];
            } else {
                cw[i] = 0;
                f8[i] = 0;
                s2[i] = 0.0f;
            }
        }
    }
    QL_DEV void store(uint8_t* lds, const float* q) {
        float c1p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c1p[i] = __fmul_rn(e4m3_decode(f8[i]), s2[i]);
        const int kc = threadIdx.x & 31, ng = threadIdx.x >> 5;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            // element kk of each row: byte kk/2, high nibble when kk is even
            const int sh = (kk >> 1) * 8 + ((kk & 1) ? 0 : 4);
            u32x4_t o;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float v0 = __fmul_rn(q[(cw[2 * p] >> sh) & 15u], c1p[2 * p]);
                const float v1 = __fmul_rn(q[(cw[2 * p + 1] >> sh) & 15u], c1p[2 * p + 1]);
                o[p] = pack_bf16x2(v0, v1);
            }
            *reinterpret_cast<u32x4_t*>(lds + lds_off(kc * 8 + kk, ng)) = o;
        }
    }
};

// bf16 source laid out [red][cols]; the tile rows are columns col0 .. col0+ROWS-1
// and the reduction runs down the source rows.  The reduction index space can
// be the concatenation of two sources: index i < red_split reads row i of
// src1, red_split <= i < 2 red_split reads row i - red_split of src2 (this is
// how hi/lo bf16 pairs enter one accumulation); rows at or beyond red_valid
// within a half read as zero.
template <int ROWS>
struct TransRows {
    static constexpr int kCC = ROWS / 8;                       // 8-column chunks
    static constexpr int kUnits = 32 * kCC / kThreads;         // row-pair x chunk units per thread
    const uint16_t* src1;
    const uint16_t* src2;
    int64_t ld, ncols, red_split, red_valid, col0;
    u32x4_t ra[kUnits], rb[kUnits];

    QL_DEV u32x4_t row_chunk(int64_t i, int64_t c) const {
        const bool second = i >= red_split;
        const int64_t li = second ? i - red_split : i;
        if (i >= 2 * red_split || li >= red_valid || c >= ncols) return u32x4_t{0, 0, 0, 0};
        return *reinterpret_cast<const u32x4_t*>((second ? src2 : src1) + li * ld + c);
    }
    QL_DEV void load(int kt) {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int unit = threadIdx.x + u * kThreads;
            const int pair = unit / kCC, cc = unit % kCC;
            const int64_t i = (int64_t)kt * 64 + 2 * pair;
            const int64_t c = col0 + cc * 8;
            ra[u] = row_chunk(i, c);
            rb[u] = row_chunk(i + 1, c);
        }
    }
    QL_DEV void store(uint8_t* lds, const float*) {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int unit = threadIdx.x + u * kThreads;
            const int pair = unit / kCC, cc = unit % kCC;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t lo = (ra[u][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                const uint32_t hi = (rb[u][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                *reinterpret_cast<uint32_t*>(lds + lds_off(cc * 8 + i, pair >> 2) + (pair & 3) * 4) = lo | (hi << 16);
            }
        }
    }
};

// ------------------------------------------------------------------ MFMA core

template <int TA, int TB>
struct Acc {
    static constexpr int MA = TA / 64, MB = TB / 64;   // 32x32 MFMA tiles per wave and dimension
    f32x16_t v[MA][MB];
    QL_DEV void zero() {
#pragma unroll
        for (int i = 0; i < MA; ++i)
#pragma unroll
            for (int j = 0; j < MB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) v[i][j][e] = 0.0f;
    }
};

template <int TA, int TB>
QL_DEV void mma_tile(const uint8_t* lA, const uint8_t* lB, Acc<TA, TB>& acc) {
    constexpr int MA = TA / 64, MB = TB / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wa = wave >> 1, wb = wave & 1;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8_t a[MA], b[MB];
#pragma unroll
        for (int i = 0; i < MA; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t*>(lA + lds_off(wa * (TA / 2) + i * 32 + r, 2 * s + h));
#pragma unroll
        for (int j = 0; j < MB; ++j)
            b[j] = *reinterpret_cast<const bf16x8_t*>(lB + lds_off(wb * (TB / 2) + j * 32 + r, 2 * s + h));
#pragma unroll
        for (int i = 0; i < MA; ++i)
#pragma unroll
            for (int j = 0; j < MB; ++j)
                acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
    }
}

// Double-buffered main loop over reduction tiles [kt0, kt1).  Global loads for
// tile kt+1 are issued before the MFMAs of tile kt and written to the other
// LDS buffer after them; one barrier per tile.
template <int TA, int TB, class PA, class PB>
QL_DEV void mainloop(PA& pa, PB& pb, int kt0, int kt1, Acc<TA, TB>& acc, uint8_t* smem, const float* q) {
    if (kt0 >= kt1) return;
    uint8_t* lA[2] = {smem, smem + TA * 128};
    uint8_t* lB[2] = {smem + 2 * TA * 128, smem + 2 * TA * 128 + TB * 128};
    pa.load(kt0);
    pb.load(kt0);
    pa.store(lA[0], q);
    pb.store(lB[0], q);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
        const int cur = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        if (more) {
            pa.load(kt + 1);
            pb.load(kt + 1);
        }
        mma_tile<TA, TB>(lA[cur], lB[cur], acc);
        if (more) {
            pa.store(lA[cur ^ 1], q);
            pb.store(lB[cur ^ 1], q);
        }
        __syncthreads();
    }
}

template <int TA, int TB>
constexpr size_t smem_bytes() { return (size_t)2 * (TA + TB) * 128 + 64; }

// Output C[a][b] to out[b][a] (a contiguous): each lane holds four consecutive
// a for one b per MFMA row group.  bf16 (8-byte stores) or fp32 (16-byte).
template <int TA, int TB, bool kBF16>
QL_DEV void store_out(const Acc<TA, TB>& acc, void* out, int64_t ldo, int64_t a0, int64_t b0, int64_t a_len,
                      int64_t b_len) {
    constexpr int MA = TA / 64, MB = TB / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wa = wave >> 1, wb = wave & 1;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < MA; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            const int64_t b = b0 + wb * (TB / 2) + j * 32 + r;
            if (b >= b_len) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t a = a0 + wa * (TA / 2) + i * 32 + g * 8 + h * 4;
                if (a >= a_len) continue;
                const f32x16_t& v = acc.v[i][j];
                if constexpr (kBF16) {
                    u32x2_t o = {pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3])};
                    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(out) + b * ldo + a) = o;
                } else {
                    f32x4_t o = {v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
                    *reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + b * ldo + a) = o;
                }
            }
        }
}

QL_DEV float* codebook_to_lds(uint8_t* smem, size_t off, const Codebook& cb) {
    float* q = reinterpret_cast<float*>(smem + off);
    if (threadIdx.x < 16) q[threadIdx.x] = cb.q[threadIdx.x];
    __syncthreads();
    return q;
}

// Map a linear workgroup id to an (a-tile, b-tile) pair.  Workgroups are
// dealt round-robin to the 8 XCDs, so ids are first regrouped to make each
// XCD own a contiguous range; that range is walked in bands of kBand b-tiles
// so that the workgroups sharing an L2 also share operand tiles.
QL_DEV void tile_of(int pid, int ga, int gb, int& ta, int& tb) {
    const int g = ga * gb;
    int l = pid;
    if ((g & 7) == 0) l = (pid & 7) * (g >> 3) + (pid >> 3);
    constexpr int kBand = 4;
    const int band = l / (kBand * ga);
    const int within = l % (kBand * ga);
    const int bw = (gb - band * kBand) < kBand ? (gb - band * kBand) : kBand;
    ta = within / bw;
    tb = band * kBand + within % bw;
}

// ------------------------------------------------------------------ kernels

struct FwdArgs {
    const uint16_t* x;
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    const uint16_t* lora_b;   // [r][N]
    const uint16_t* ps_hi;    // [T][r_pad] bf16: s X A = hi + lo
    const uint16_t* ps_lo;
    uint16_t* y;
    int64_t T, K, N, r, r_pad;
};

// Y = X W'^T (+ (s X A) B): a = n over W rows, b = t over tokens.
__global__ __launch_bounds__(kThreads, 1) void k_fwd(FwdArgs p, Codebook cb) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int TA = 256, TB = 256;
    const float* q = codebook_to_lds(smem, smem_bytes<TA, TB>() - 64, cb);
    const int ga = (int)ceil_div(p.N, TA), gb = (int)ceil_div(p.T, TB);
    int ta, tb;
    tile_of(blockIdx.x, ga, gb, ta, tb);
    const int64_t n0 = (int64_t)ta * TA, t0 = (int64_t)tb * TB;

    Acc<TA, TB> acc;
    acc.zero();
    {
        NF4Rows pa{p.codes, p.fp8, p.sup, p.K, p.N, n0};
        PlainRows<TB> pb{p.x, p.K, p.T, p.K, t0};
        mainloop<TA, TB>(pa, pb, 0, (int)(p.K / 64), acc, smem, q);
    }
    if (p.r > 0) {
        // reduction over [hi | lo] of s X A against B stacked twice
        TransRows<TA> pa{p.lora_b, p.lora_b, p.N, p.N, p.r_pad, p.r, n0};
        PlainRows<TB> pb{p.ps_hi, p.r_pad, p.T, p.r_pad, t0, p.ps_lo, (int)(p.r_pad / 64)};
        mainloop<TA, TB>(pa, pb, 0, (int)(2 * p.r_pad / 64), acc, smem, q);
    }
    store_out<TA, TB, true>(acc, p.y, p.N, n0, t0, p.N, p.T);
}

struct DxArgs {
    const uint16_t* dy;
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    const uint16_t* lora_a;   // [K][r]
    const uint16_t* gs_hi;    // [T][r_pad] bf16: s dY B^T = hi + lo
    const uint16_t* gs_lo;
    uint16_t* dx;
    int64_t T, K, N, r, r_pad;
};

// dX = dY W' (+ (s dY B^T) A^T): a = k over W columns, b = t.
__global__ __launch_bounds__(kThreads, 1) void k_dx(DxArgs p, Codebook cb) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int TA = 256, TB = 256;
    const float* q = codebook_to_lds(smem, smem_bytes<TA, TB>() - 64, cb);
    const int ga = (int)ceil_div(p.K, TA), gb = (int)ceil_div(p.T, TB);
    int ta, tb;
    tile_of(blockIdx.x, ga, gb, ta, tb);
    const int64_t k0 = (int64_t)ta * TA, t0 = (int64_t)tb * TB;

    Acc<TA, TB> acc;
    acc.zero();
    {
        NF4Cols pa{p.codes, p.fp8, p.sup, p.K, p.N, k0};
        PlainRows<TB> pb{p.dy, p.N, p.T, p.N, t0};
        mainloop<TA, TB>(pa, pb, 0, (int)(p.N / 64), acc, smem, q);
    }
    if (p.r > 0) {
        const int half = (int)(p.r_pad / 64);
        PlainRows<TA> pa{p.lora_a, p.r, p.K, p.r, k0, p.lora_a, half};
        PlainRows<TB> pb{p.gs_hi, p.r_pad, p.T, p.r_pad, t0, p.gs_lo, half};
        mainloop<TA, TB>(pa, pb, 0, 2 * half, acc, smem, q);
    }
    store_out<TA, TB, true>(acc, p.dx, p.K, k0, t0, p.K, p.T);
}

// Small LoRA products with split reduction; fp32 partials out[split][b][a].
enum SmallKind { kXA = 0, kG = 1, kDA = 2, kDB = 3 };

struct SmallArgs {
    const uint16_t* s0;   // see the instantiations below
    const uint16_t* s1;
    const uint16_t* s2;
    float* part;
    int64_t T, K, N, r, r_pad;
    int ktiles, splits;
};

template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void k_small(SmallArgs p) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int TA = (KIND == kDB) ? 256 : 64;
    constexpr int TB = (KIND == kDB) ? 64 : 256;
    const int split = blockIdx.y;
    const int per = (p.ktiles + p.splits - 1) / p.splits;
    const int kt0 = split * per;
    const int kt1 = (kt0 + per) < p.ktiles ? (kt0 + per) : p.ktiles;
    Acc<TA, TB> acc;
    acc.zero();
    int64_t a_len, b_len;
    int ga;
    if constexpr (KIND == kXA || KIND == kG || KIND == kDA) ga = (int)(p.r_pad / 64);
    else ga = (int)ceil_div(p.N, TA);
    const int ta = blockIdx.x % ga, tb = blockIdx.x / ga;
    const int64_t a0 = (int64_t)ta * TA, b0 = (int64_t)tb * TB;

    if constexpr (KIND == kXA) {
        // P[t][j] = sum_k X[t][k] A[k][j]: a = j (A transposed), b = t.  s0 = A, s1 = X.
        TransRows<TA> pa{p.s0, p.s0, p.r, p.r, p.K, p.K, a0};
        PlainRows<TB> pb{p.s1, p.K, p.T, p.K, b0};
        mainloop<TA, TB>(pa, pb, kt0, kt1, acc, smem, nullptr);
        a_len = p.r_pad; b_len = p.T;
    } else if constexpr (KIND == kG) {
        // G[t][j] = sum_n dY[t][n] B[j][n]: a = j, b = t.  s0 = B, s1 = dY.
        PlainRows<TA> pa{p.s0, p.N, p.r, p.N, a0};
        PlainRows<TB> pb{p.s1, p.N, p.T, p.N, b0};
        mainloop<TA, TB>(pa, pb, kt0, kt1, acc, smem, nullptr);
        a_len = p.r_pad; b_len = p.T;
    } else if constexpr (KIND == kDA) {
        // dA[k][j] = sum over 2T of X[t][k] (G_hi | G_lo)[t][j]: a = j, b = k.  s0 = G_hi, s1 = G_lo, s2 = X.
        TransRows<TA> pa{p.s0, p.s1, p.r_pad, p.r_pad, p.T, p.T, a0};
        TransRows<TB> pb{p.s2, p.s2, p.K, p.K, p.T, p.T, b0};
        mainloop<TA, TB>(pa, pb, kt0, kt1, acc, smem, nullptr);
        a_len = p.r_pad; b_len = p.K;
    } else {
        // dB[j][n] = sum over 2T of (P_hi | P_lo)[t][j] dY[t][n]: a = n, b = j.  s0 = P_hi, s1 = P_lo, s2 = dY.
        TransRows<TA> pa{p.s2, p.s2, p.N, p.N, p.T, p.T, a0};
        TransRows<TB> pb{p.s0, p.s1, p.r_pad, p.r_pad, p.T, p.T, b0};
        mainloop<TA, TB>(pa, pb, kt0, kt1, acc, smem, nullptr);
        a_len = p.N; b_len = p.r_pad;
    }
    float* out = p.part + (int64_t)split * a_len * b_len;
    store_out<TA, TB, false>(acc, out, a_len, a0, b0, a_len, b_len);
}

// Sum split partials [S][rows][cols] in split order; v = scale * sum.
// mode 0: bf16 hi = RNE(v), lo = RNE(v - hi) into two [rows][cols] arrays.
// mode 1: bf16 RNE(v) into out [rows][out_cols] for cols < out_cols.
__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ part, int splits, int64_t sstride,
                                                  int64_t rows, int64_t cols, float scale, int mode,
                                                  uint16_t* __restrict__ hi, uint16_t* __restrict__ lo,
                                                  int64_t out_cols) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * cols) return;
    float acc = 0.0f;
    for (int s = 0; s < splits; ++s) acc += part[(int64_t)s * sstride + i];
    const float v = acc * scale;
    const uint32_t hb = pack_bf16x2(v, 0.0f) & 0xFFFFu;
    if (mode == 0) {
        hi[i] = (uint16_t)hb;
        lo[i] = (uint16_t)(pack_bf16x2(v - bf16lo(hb), 0.0f) & 0xFFFFu);
    } else {
        const int64_t rr = i / cols, cc = i % cols;
        if (cc < out_cols) hi[rr * out_cols + cc] = (uint16_t)hb;
    }
}

// ------------------------------------------------------------------ launchers

namespace {
template <class F>
hipError_t set_smem(F* f, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

hipError_t finalize(const float* part, int splits, int64_t sstride, int64_t rows, int64_t cols, float scale,
                    int mode, uint16_t* hi, uint16_t* lo, int64_t out_cols, hipStream_t s) {
    const int64_t n = rows * cols;
    hipLaunchKernelGGL(k_finalize, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, part, splits, sstride, rows,
                       cols, scale, mode, hi, lo, out_cols);
    return hipGetLastError();
}

template <int KIND>
hipError_t small(const SmallArgs& a, int64_t tiles, hipStream_t s) {
    constexpr int TA = (KIND == kDB) ? 256 : 64;
    constexpr int TB = (KIND == kDB) ? 64 : 256;
    const size_t lds = smem_bytes<TA, TB>();
    hipError_t e = set_smem(k_small<KIND>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_small<KIND>, dim3((unsigned)tiles, (unsigned)a.splits), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}
}  // namespace

// s X A -> ws (hi/lo bf16 [T][r_pad])
hipError_t launch_lora_down_x(const uint16_t* x, const uint16_t* lora_a, float scaling, const LoraPlan& pl,
                              uint8_t* ws, hipStream_t s) {
    SmallArgs a{lora_a, x, nullptr, reinterpret_cast<float*>(ws + pl.off_pxa), pl.T, pl.K, pl.N, pl.r, pl.r_pad,
                (int)(pl.K / 64), pl.s_xa};
    const int64_t tiles = (pl.r_pad / 64) * ceil_div(pl.T, 256);
    hipError_t e = small<kXA>(a, tiles, s);
    if (e != hipSuccess) return e;
    return finalize(a.part, pl.s_xa, pl.T * pl.r_pad, pl.T, pl.r_pad, scaling, 0, reinterpret_cast<uint16_t*>(ws + pl.off_ps_hi),
                    reinterpret_cast<uint16_t*>(ws + pl.off_ps_lo), pl.r_pad, s);
}

// s dY B^T -> ws (hi/lo bf16 [T][r_pad])
hipError_t launch_lora_down_dy(const uint16_t* dy, const uint16_t* lora_b, float scaling, const LoraPlan& pl,
                               uint8_t* ws, hipStream_t s) {
    SmallArgs a{lora_b, dy, nullptr, reinterpret_cast<float*>(ws + pl.off_pg), pl.T, pl.K, pl.N, pl.r, pl.r_pad,
                (int)(pl.N / 64), pl.s_g};
    const int64_t tiles = (pl.r_pad / 64) * ceil_div(pl.T, 256);
    hipError_t e = small<kG>(a, tiles, s);
    if (e != hipSuccess) return e;
    return finalize(a.part, pl.s_g, pl.T * pl.r_pad, pl.T, pl.r_pad, scaling, 0, reinterpret_cast<uint16_t*>(ws + pl.off_gs_hi),
                    reinterpret_cast<uint16_t*>(ws + pl.off_gs_lo), pl.r_pad, s);
}

hipError_t launch_fwd(const uint16_t* x, const uint8_t* codes, const uint8_t* fp8, const float* sup,
                      const uint16_t* lora_b, const LoraPlan& pl, const uint8_t* ws, uint16_t* y, hipStream_t s) {
    FwdArgs a{x, codes, fp8, sup, lora_b, reinterpret_cast<const uint16_t*>(ws + pl.off_ps_hi),
              reinterpret_cast<const uint16_t*>(ws + pl.off_ps_lo), y,
              pl.T, pl.K, pl.N, pl.r, pl.r_pad};
    const size_t lds = smem_bytes<256, 256>();
    hipError_t e = set_smem(k_fwd, lds);
    if (e != hipSuccess) return e;
    const int64_t tiles = ceil_div(pl.N, 256) * ceil_div(pl.T, 256);
    hipLaunchKernelGGL(k_fwd, dim3((unsigned)tiles), dim3(kThreads), lds, s, a, host_codebook());
    return hipGetLastError();
}

hipError_t launch_dx(const uint16_t* dy, const uint8_t* codes, const uint8_t* fp8, const float* sup,
                     const uint16_t* lora_a, const LoraPlan& pl, const uint8_t* ws, uint16_t* dx, hipStream_t s) {
    DxArgs a{dy, codes, fp8, sup, lora_a, reinterpret_cast<const uint16_t*>(ws + pl.off_gs_hi),
             reinterpret_cast<const uint16_t*>(ws + pl.off_gs_lo), dx,
             pl.T, pl.K, pl.N, pl.r, pl.r_pad};
    const size_t lds = smem_bytes<256, 256>();
    hipError_t e = set_smem(k_dx, lds);
    if (e != hipSuccess) return e;
    const int64_t tiles = ceil_div(pl.K, 256) * ceil_div(pl.T, 256);
    hipLaunchKernelGGL(k_dx, dim3((unsigned)tiles), dim3(kThreads), lds, s, a, host_codebook());
    return hipGetLastError();
}

// dA and dB from the hi/lo intermediates already in ws.
hipError_t launch_lora_grads(const uint16_t* x, const uint16_t* dy, const LoraPlan& pl, uint8_t* ws,
                             uint16_t* d_lora_a, uint16_t* d_lora_b, hipStream_t s) {
    const int ktiles = (int)ceil_div(2 * pl.T, 64);
    if (d_lora_a) {
        SmallArgs a{reinterpret_cast<const uint16_t*>(ws + pl.off_gs_hi),
                    reinterpret_cast<const uint16_t*>(ws + pl.off_gs_lo), x,
                    reinterpret_cast<float*>(ws + pl.off_pda), pl.T, pl.K, pl.N, pl.r, pl.r_pad, ktiles, pl.s_da};
        hipError_t e = small<kDA>(a, (pl.r_pad / 64) * ceil_div(pl.K, 256), s);
        if (e != hipSuccess) return e;
        e = finalize(a.part, pl.s_da, pl.K * pl.r_pad, pl.K, pl.r_pad, 1.0f, 1, d_lora_a, nullptr, pl.r, s);
        if (e != hipSuccess) return e;
    }
    if (d_lora_b) {
        SmallArgs a{reinterpret_cast<const uint16_t*>(ws + pl.off_ps_hi),
                    reinterpret_cast<const uint16_t*>(ws + pl.off_ps_lo), dy,
                    reinterpret_cast<float*>(ws + pl.off_pdb), pl.T, pl.K, pl.N, pl.r, pl.r_pad, ktiles, pl.s_db};
        hipError_t e = small<kDB>(a, ceil_div(pl.N, 256) * (pl.r_pad / 64), s);
        if (e != hipSuccess) return e;
        // partials are [S][r_pad][N]; output rows j < r
        e = finalize(a.part, pl.s_db, pl.r_pad * pl.N, pl.r, pl.N, 1.0f, 1, d_lora_b, nullptr, pl.N, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ql
