// MFMA GEMMs of the QLoRA linear layer on gfx950, with NF4 double
// dequantization fused into the LDS tile producers.
//
// Layer (Volcengine article section 3.4, equation lost; reading used):
//   Y  = X W'^T + s (X A) B
//   dX = dY W'  + s (dY B^T) A^T,   dA = s X^T (dY B^T),   dB = s (X A)^T dY
// with W' the double-dequantized bf16 weight ("QLoRA 原理精讲" section 2.2:
// super-scale, then block constant, then weight) that is never written to HBM.
//
// Structure.  Both products are sums over 64-wide reduction tiles of
// v_mfma_f32_32x32x16_bf16 steps, with both operands fed as 8 consecutive
// reduction elements per lane:
//   k_fwd - W rows dequantized straight into A-operand registers, X through
//           swizzled LDS (reduction over k is contiguous in both);
//   k_dx  - W dequantized and transposed into LDS ([k][n] tiles), dY through
//           LDS (reduction over n).
// NF4 codes are decoded with byte-pair tables in LDS: one 8-byte read returns
// the two fp32 codewords of a packed byte.  The LoRA up-projection (rank r) is
// a short extra reduction at the end of each tile, from operands staged by
// PlainRows (bf16 rows contiguous along the reduction) or TransRows (bf16
// stored with the reduction as the row index).  Outputs leave as bf16 rows.
#include "common.hpp"
#include "grad.hpp"
#include "plan.hpp"

namespace ql {


constexpr int kThreads = 256;

// ------------------------------------------------------------------ LDS tile producers

// bf16 rows contiguous along the reduction (X, dY, ...), via buffer loads.
// Reduction tiles kt >= split_kt read src2 at tile kt - split_kt (the second
// half of a concatenated reduction, e.g. the lo part of a hi/lo pair).  With
// kCheckK, chunks at or beyond red_len within a tile read as zero (needed when
// the reduction length is not a multiple of 64).
template <int ROWS, bool kCheckK = false>
struct PlainRows {
    static constexpr int kChunks = ROWS * 8 / kThreads;     // 16-byte chunks per thread
    const uint16_t* src1;
    const uint16_t* src2;
    int64_t bytes;
    int split_kt;
    int64_t red_len;
    uint32_t voff[kChunks];
    u32x4_t reg[kChunks];

    QL_DEV void init(const uint16_t* s1, const uint16_t* s2, int64_t ld, int64_t nrows, int64_t row0, int64_t rl,
                     int split) {
        src1 = s1;
        src2 = s2 ? s2 : s1;
        bytes = nrows * ld * 2;
        split_kt = split;
        red_len = rl;
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int64_t row = row0 + (c >> 3);
            voff[i] = row < nrows ? (uint32_t)((row * ld + (c & 7) * 8) * 2) : kOOB;
        }
    }
    QL_DEV void load(int kt) {
        const bool first = kt < split_kt;
        const int ktl = first ? kt : kt - split_kt;
        const rsrc_t rs = make_rsrc(first ? src1 : src2, bytes);
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            u32x4_t v = bload16(rs, voff[i], (uint32_t)ktl * 128u);
            if constexpr (kCheckK) {
                const int c = threadIdx.x + i * kThreads;
                v = ((int64_t)ktl * 64 + (c & 7) * 8 < red_len) ? v : u32x4_t{0, 0, 0, 0};
            }
            reg[i] = v;
        }
    }
    QL_DEV void store(lds8_t* lds, const lds8_t*) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = threadIdx.x + i * kThreads;
            *reinterpret_cast<lds_u32x4_t*>(lds + lds_off(c >> 3, c & 7)) = reg[i];
        }
    }
};

// bf16 source laid out [red][cols]; the tile rows are columns col0 .. col0+ROWS-1
// and the reduction runs down the source rows.  The reduction index space can
// be the concatenation of two sources: index i < red_split reads row i of
// src1, red_split <= i < 2 red_split reads row i - red_split of src2 (this is
// how hi/lo bf16 pairs enter one accumulation); rows at or beyond red_valid
// within a half read as zero.  Two source rows are paired into dwords.
template <int ROWS>
struct TransRows {
    static constexpr int kCC = ROWS / 8;                       // 8-column chunks
    static constexpr int kUnits = 32 * kCC / kThreads;         // row-pair x chunk units per thread
    const uint16_t* src1;
    const uint16_t* src2;
    int64_t ld, ncols, red_split, red_valid, col0;
    u32x4_t ra[kUnits], rb[kUnits];

    QL_DEV void init(const uint16_t* s1, const uint16_t* s2, int64_t ld_, int64_t nc, int64_t rs, int64_t rv,
                     int64_t c0) {
        src1 = s1; src2 = s2; ld = ld_; ncols = nc; red_split = rs; red_valid = rv; col0 = c0;
    }
    QL_DEV u32x4_t row_chunk(int64_t i, int64_t c) const {
        const bool second = i >= red_split;
        const int64_t li = second ? i - red_split : i;
        const bool ok = i < 2 * red_split && li < red_valid && c < ncols;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>((second ? src2 : src1) + (ok ? li * ld + c : 0));
        return ok ? v : u32x4_t{0, 0, 0, 0};
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
    QL_DEV void store(lds8_t* lds, const lds8_t*) {
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int unit = threadIdx.x + u * kThreads;
            const int pair = unit / kCC, cc = unit % kCC;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t lo = (ra[u][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                const uint32_t hi = (rb[u][i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                *reinterpret_cast<lds_u32_t*>(lds + lds_off(cc * 8 + i, pair >> 2) + (pair & 3) * 4) = lo | (hi << 16);
            }
        }
    }
};

// ------------------------------------------------------------------ MFMA core

QL_DEV bf16x8_t lds_frag(const lds8_t* base, int row, int chunk) {
    return *reinterpret_cast<const lds_bf16x8_t*>(base + lds_off(row, chunk));
}

// Output tiles [256 (t)][256 (c)] of 16-bit values staged in LDS (128 KB) so
// that the global stores are whole rows.  Row t is 512 bytes; its 16-byte
// chunk c sits at chunk position c ^ (t & 31), which keeps both the
// accumulator writes (32 rows at one chunk) and the row reads conflict-free.
QL_DEV uint32_t otile_off(int t, int c) { return (uint32_t)t * 512u + ((uint32_t)(c ^ (t & 31)) << 4); }

// Columns col .. col+3 (col % 4 == 0) of tile row t: the four consecutive
// accumulator rows of MFMA row group g.
template <bool F16>
QL_DEV void otile_put4(lds8_t* lo, const f32x16_t& v, int g, int t, int col) {
    const u32x2_t o = {pack16x2<F16>(v[4 * g], v[4 * g + 1]), pack16x2<F16>(v[4 * g + 2], v[4 * g + 3])};
    *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(lo + otile_off(t, col >> 3) + (col & 7) * 2) = o;
}

// out[t0 + t][c0 + c] = tile[t][c] for t0 + t < T and c0 + c < C (C % 8 == 0):
// each wave store covers two rows of 512 contiguous bytes.
QL_DEV void otile_store(const lds8_t* lo, uint16_t* out, int64_t ldo, int64_t t0, int64_t c0, int64_t T, int64_t C) {
#pragma unroll 8
    for (int it = 0; it < 256 * 32 / kThreads; ++it) {
        const int u = threadIdx.x + it * kThreads;
        const int t = u >> 5, c = u & 31;
        const int64_t tg = t0 + t, cg = c0 + c * 8;
        if (tg < T && cg < C)
            *reinterpret_cast<u32x4_t*>(out + tg * ldo + cg) =
                *reinterpret_cast<const lds_u32x4_t*>(lo + otile_off(t, c));
    }
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

// ------------------------------------------------------------------ forward

struct FwdArgs {
    const uint16_t* x;
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    const float* absmax;      // single quantization: fp32 block absmax (fp8/sup unused)
    const uint16_t* lora_b;   // [r][N]
    const uint16_t* ps_hi;    // [T][r_pad] bf16: s X A = hi + lo
    const uint16_t* ps_lo;
    uint16_t* y;
    int64_t T, K, N, r, r_pad;
    float* part;              // split-k: fp32 partial tiles [splits][N][T rounded up to 4]
    int splits;
};

// Y = X W'^T (+ (s X A) B), tile 256 (n) x 256 (t), waves stacked along n.
//
// Wave w owns W rows n0 + 64w .. +63 (two 32-row MFMA A-fragments) against all
// 256 tokens (eight B-fragments).  Its W rows are private to it, so they are
// dequantized straight into A-operand registers: per 64-wide k tile a lane
// loads 16 code bytes of one row (32 k values), one FP8 constant and one
// super-scale.  The k order inside a tile is permuted consistently on both
// operands (MFMA step s, lane half h, slot j <-> k = 32h + 8s + j), which makes
// each lane's codes contiguous.
//
// Pipeline.  Global loads run two k tiles ahead (X and W codes into
// registers, alternating register sets by tile parity); X is written to the
// idle LDS buffer one tile ahead, in the middle of the last step of a tile;
// one barrier per tile.  Within the tile, see fwd_tile.
//
// SQ: single quantization, the block constant is the stored fp32 absmax (one
// 4-byte load per row and tile instead of the FP8 code and the super-scale).
template <bool SQ>
struct FwdPipe {
    static constexpr int TT = 256;
    static constexpr uint32_t kTile = TT * 128;   // one [256][64] bf16 LDS tile
    rsrc_t rc, rf, rs, rx;
    uint32_t cvo[2], fvo[2], blk[2], xvo[8];
    bool wok[2];
    uint32_t lane8;
    int KT;
    // global-load register sets, indexed by tile parity
    u32x4_t xr[2][8];
    u32x4_t wc[2][2];
    uint32_t wf[2][2];
    float ws[2][2];

    QL_DEV void load_w(int kt, int par) {
        kt = kt < KT ? kt : KT - 1;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            wc[par][i] = bload16(rc, cvo[i], (uint32_t)kt * 32u);
            if constexpr (SQ) {
                wf[par][i] = 0;
                ws[par][i] = __uint_as_float(bload4(rf, wok[i] ? (blk[i] + kt) * 4u : kOOB, 0));
            } else {
                wf[par][i] = bload1(rf, fvo[i], (uint32_t)kt);
                ws[par][i] = __uint_as_float(bload4(rs, wok[i] ? ((blk[i] + kt) >> 8) * 4u : kOOB, 0));
            }
        }
    }
    // block constant c1' of row i from register set par
    QL_DEV float c1(int par, int i) const { return SQ ? ws[par][i] : block_scale(wf[par][i], ws[par][i]); }
    QL_DEV void load_x(int kt, int par) {
        kt = kt < KT ? kt : KT - 1;
#pragma unroll
        for (int c = 0; c < 8; ++c) xr[par][c] = bload16(rx, xvo[c], (uint32_t)kt * 128u);
    }
    QL_DEV void store_x(int par, lds8_t* lx) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ch = threadIdx.x + c * kThreads;
            *reinterpret_cast<lds_u32x4_t*>(lx + lds_off(ch >> 3, ch & 7)) = xr[par][c];
        }
    }
};

// Pieces of one MFMA step s (16 k): eight X fragments from LDS, the eight
// codebook pairs of the two A fragments (codes dword s of each W row), the
// A fragments themselves, and the sixteen MFMAs.
typedef bf16x8_t XFr[8];
typedef f32x2_t QPr[2][4];
typedef bf16x8_t AFr[2];

QL_DEV void read_x(XFr& x, const lds8_t* xb, int s, int r, int h) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = lds_frag(xb, 32 * j + r, 4 * h + s);
}

QL_DEV void read_q(QPr& q, const u32x4_t (&wc)[2], int s, uint32_t lane8) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // address bytes: [0] lane copy, [1] code byte b, [2..3] from the table base
            const uint32_t addr = __builtin_amdgcn_perm(wc[i][s], lane8, 0x03020000u | ((4u + b) << 8));
            q[i][b] = *lds_at<f32x2_t>(addr);
        }
}

template <bool F16>
QL_DEV void make_a(AFr& a, const QPr& q, const float (&c1p)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        u32x4_t o;
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = pack16x2<F16>(__fmul_rn(q[i][b][0], c1p[i]), __fmul_rn(q[i][b][1], c1p[i]));
        a[i] = __builtin_bit_cast(bf16x8_t, o);
    }
}

template <bool F16>
QL_DEV void mfma16(f32x16_t (&acc)[2][8], const AFr& a, const XFr& x) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        acc[0][j] = mfma32x32x16<F16>(a[0], x[j], acc[0][j]);
        acc[1][j] = mfma32x32x16<F16>(a[1], x[j], acc[1][j]);
    }
}

// Scheduling hint for one step: each MFMA followed by one LDS read, two VALU
// instructions and (for the first kWrites) one LDS write, so the reads and
// the dequantization of later steps issue in the shadow of the 32-cycle MFMAs
// instead of in front of them.
template <int kMfma, int kReads, int kValu, int kWrites = 0, int kValuPer = 2>
QL_DEV void interleave() {
#pragma unroll
    for (int j = 0; j < kMfma; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
        if (j < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        if (j < kValu) __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);   // VALU
        if (j < kWrites) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
    }
}

// One k tile (parity P: LDS buffer and register sets).  Software pipeline over
// the steps: while the MFMAs of step s run, the X fragments of step s+1 and
// the codebook pairs of step s+2 are read, and the A fragments of step s+1
// are built from pairs read during step s-1.  On entry xa / aa hold step 0 of
// tile kt and qa the pairs of step 1; on exit the same for tile kt+1.
template <int P, bool SQ, bool F16>
QL_DEV void fwd_tile(FwdPipe<SQ>& pp, int kt, f32x16_t (&acc)[2][8], lds8_t* lX, int r, int h, XFr& xa, AFr& aa,
                     QPr& qa, float (&c1p)[2]) {
    constexpr int Q = P ^ 1;
    const lds8_t* xb = lX + P * FwdPipe<SQ>::kTile;
    XFr xb_;
    AFr ab;
    QPr qb;
    pp.load_x(kt + 2, P);                     // staging set P held tile kt, stored during tile kt-1
    __builtin_amdgcn_sched_barrier(0);
    // step 0
    read_x(xb_, xb, 1, r, h);
    read_q(qb, pp.wc[P], 2, pp.lane8);
    make_a<F16>(ab, qa, c1p);
    mfma16<F16>(acc, aa, xa);
    interleave<16, 16, 16>();
    __builtin_amdgcn_sched_barrier(0);
    // step 1
    read_x(xa, xb, 2, r, h);
    read_q(qa, pp.wc[P], 3, pp.lane8);
    make_a<F16>(aa, qb, c1p);
    mfma16<F16>(acc, ab, xb_);
    interleave<16, 16, 16>();
    __builtin_amdgcn_sched_barrier(0);
    // step 2: the pairs of the next tile's step 0 come from code set Q
    read_x(xb_, xb, 3, r, h);
    read_q(qb, pp.wc[Q], 0, pp.lane8);
    make_a<F16>(ab, qa, c1p);
    mfma16<F16>(acc, aa, xa);
    interleave<16, 16, 16>();
    __builtin_amdgcn_sched_barrier(0);
    pp.load_w(kt + 2, P);                     // code set P is no longer read
    const float n1p[2] = {pp.c1(Q, 0), pp.c1(Q, 1)};
    // step 3: the first half of its MFMAs cover the X store and the barrier
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[0][j] = mfma32x32x16<F16>(ab[0], xb_[j], acc[0][j]);
        acc[1][j] = mfma32x32x16<F16>(ab[1], xb_[j], acc[1][j]);
    }
    pp.store_x(Q, lX + Q * FwdPipe<SQ>::kTile);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_x(xa, lX + Q * FwdPipe<SQ>::kTile, 0, r, h);
    read_q(qa, pp.wc[Q], 1, pp.lane8);
    make_a<F16>(aa, qb, n1p);
#pragma unroll
    for (int j = 4; j < 8; ++j) {
        acc[0][j] = mfma32x32x16<F16>(ab[0], xb_[j], acc[0][j]);
        acc[1][j] = mfma32x32x16<F16>(ab[1], xb_[j], acc[1][j]);
    }
    interleave<8, 8, 8>();
    __builtin_amdgcn_sched_barrier(0);
    c1p[0] = n1p[0];
    c1p[1] = n1p[1];
}

// SPLIT: the grid holds `splits` workgroups per tile; workgroup (tile,
// split) takes k tiles [split KT / splits, (split + 1) KT / splits) (split 0
// also the LoRA term) and stores its fp32 tile in part[split][n][t], which
// k_split_sum adds in split order.  Partial rows are padded to a multiple of
// four tokens (ldp), so every row starts 16-byte aligned and both kernels
// move whole float4s; the padding holds the tile's zero columns.
template <bool SQ, bool F16, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void k_fwd(FwdArgs p, Codebook cb) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    lds8_t* smem = (lds8_t*)(smem_raw);
    constexpr int TT = FwdPipe<SQ>::TT;
    constexpr uint32_t kTile = FwdPipe<SQ>::kTile;
    lds8_t* const lX = smem;                  // 2 tiles (the LoRA phase reuses them)
    lds8_t* const lL = smem + kTile;
    lds8_t* const tbl = smem + 2 * kTile;     // wide pair table
    build_wide_pair_table(tbl, cb);

    const int ga = (int)ceil_div(p.N, 256), gb = (int)ceil_div(p.T, TT);
    const int KT_all = (int)(p.K / 64);
    int ta, tb, split = 0, kt0 = 0, kt1 = KT_all;
    if constexpr (SPLIT) {
        split = (int)blockIdx.x / (ga * gb);
        tile_of((int)blockIdx.x % (ga * gb), ga, gb, ta, tb);
        kt0 = split * KT_all / p.splits;
        kt1 = (split + 1) * KT_all / p.splits;
    } else {
        tile_of(blockIdx.x, ga, gb, ta, tb);
    }
    const int64_t n0 = (int64_t)ta * 256, t0 = (int64_t)tb * TT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 31, h = lane >> 5;

    FwdPipe<SQ> pp;
    pp.rc = make_rsrc(p.codes, p.N * p.K / 2);
    if constexpr (SQ) {
        pp.rf = make_rsrc(p.absmax, p.N * p.K / 64 * 4);
        pp.rs = pp.rf;
    } else {
        pp.rf = make_rsrc(p.fp8, p.N * p.K / 64);
        pp.rs = make_rsrc(p.sup, ceil_div(p.N * p.K / 64, 256) * 4);
    }
    pp.rx = make_rsrc(p.x, p.T * p.K * 2);
    pp.KT = kt1 - kt0;                        // k tiles of this workgroup, counted from kt0
    pp.lane8 = lds_addr(tbl) + (uint32_t)(lane & 31) * 8u;   // table is 64 KB aligned
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t n = n0 + 64 * w + 32 * i + r;
        pp.wok[i] = n < p.N;
        pp.cvo[i] = pp.wok[i] ? (uint32_t)(n * (p.K / 2) + 16 * h + 32 * kt0) : kOOB;
        pp.fvo[i] = pp.wok[i] ? (uint32_t)(n * (p.K / 64) + kt0) : kOOB;
        pp.blk[i] = pp.wok[i] ? (uint32_t)(n * (p.K / 64) + kt0) : 0u;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int ch = threadIdx.x + c * kThreads;
        const int64_t t = t0 + (ch >> 3);
        pp.xvo[c] = t < p.T ? (uint32_t)((t * p.K + (int64_t)kt0 * 64 + (ch & 7) * 8) * 2) : kOOB;
    }

    f32x16_t acc[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // prologue: tiles 0 and 1 in flight; tile 0's X in LDS and its step 0 ready
    pp.load_w(0, 0);
    pp.load_x(0, 0);
    pp.load_w(1, 1);
    pp.load_x(1, 1);
    pp.store_x(0, lX);
    __syncthreads();                          // pair table and X tile 0 visible
    XFr xa;
    AFr aa;
    QPr qa;
    float c1p[2] = {pp.c1(0, 0), pp.c1(0, 1)};
    {
        QPr q0;
        read_q(q0, pp.wc[0], 0, pp.lane8);
        make_a<F16>(aa, q0, c1p);
        read_q(qa, pp.wc[0], 1, pp.lane8);
        read_x(xa, lX, 0, r, h);
    }
    const int KT = pp.KT;
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        fwd_tile<0, SQ, F16>(pp, kt, acc, lX, r, h, xa, aa, qa, c1p);
        fwd_tile<1, SQ, F16>(pp, kt + 1, acc, lX, r, h, xa, aa, qa, c1p);
    }
    if (kt < KT) fwd_tile<0, SQ, F16>(pp, kt, acc, lX, r, h, xa, aa, qa, c1p);

    if (p.r > 0 && split == 0) {
        // reduction over [hi | lo] of s X A (tokens) against B^T stacked twice (rows n)
        TransRows<256> pl;
        pl.init(p.lora_b, p.lora_b, p.N, p.N, p.r_pad, p.r, n0);
        PlainRows<TT> ps;
        ps.init(p.ps_hi, p.ps_lo, p.r_pad, p.T, t0, p.r_pad, (int)(p.r_pad / 64));
        const int LT = (int)(2 * p.r_pad / 64);
        for (int lt = 0; lt < LT; ++lt) {
            pl.load(lt);
            ps.load(lt);
            __syncthreads();                  // previous readers of both buffers are done
            pl.store(lL, tbl);
            ps.store(lX, tbl);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8_t a0 = lds_frag(lL, 64 * w + r, 4 * h + s);
                const bf16x8_t a1 = lds_frag(lL, 64 * w + 32 + r, 4 * h + s);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bf16x8_t b = lds_frag(lX, 32 * j + r, 4 * h + s);
                    acc[0][j] = mfma32x32x16<F16>(a0, b, acc[0][j]);
                    acc[1][j] = mfma32x32x16<F16>(a1, b, acc[1][j]);
                }
            }
            __syncthreads();
        }
    }

    if constexpr (SPLIT) {
        // fp32 partial tile part[split][n][t], through LDS in two halves of 128
        // rows (A fragment i of every wave): LDS row 32 w + q holds tile row
        // 64 w + 32 i + q; the 16-byte chunks of rows with bit 2 set sit 128
        // bytes over, so the two rows of one accumulator store use distinct
        // banks; whole 1 KB rows then go out with 16-byte stores
        const int64_t ldp = (p.T + 3) & ~int64_t(3);
        float* out = p.part + (int64_t)split * p.N * ldp;
        float* lt = reinterpret_cast<float*>(smem_raw);                  // [128][256] fp32
        auto loff = [](int row, int t) { return row * 256 + (t ^ (((row >> 2) & 1) << 5)); };
#pragma unroll
        for (int i = 0; i < 2; ++i) {                                    // unrolled: acc indices stay static
            __syncthreads();                                             // LDS readers are done
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        lt[loff(32 * w + 8 * g + 4 * h + v, 32 * j + r)] = acc[i][j][4 * g + v];
            __syncthreads();
#pragma unroll 4
            for (int e = threadIdx.x; e < 128 * 64; e += kThreads) {     // 64 float4 per row
                const int row = e >> 6, c4 = e & 63;
                const int64_t n = n0 + 64 * (row >> 5) + 32 * i + (row & 31);
                const int64_t t = t0 + 4 * c4;
                if (n < p.N && t < p.T) {                                 // t + 3 < ldp
                    const float* src = lt + loff(row, 4 * c4);
                    *reinterpret_cast<f32x4_t*>(out + n * ldp + t) = f32x4_t{src[0], src[1], src[2], src[3]};
                }
            }
        }
        return;
    }
    // C[n][t] -> Y[t][n] through an LDS tile over the X buffers and the table
    __syncthreads();                          // every wave is done reading them
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) otile_put4<F16>(smem, acc[i][j], g, 32 * j + r, 64 * w + 32 * i + 8 * g + 4 * h);
    __syncthreads();
    otile_store(smem, p.y, p.N, t0, n0, p.T, p.N);
}

// out[t][c] = RNE_16(sum_s part[s][c][t]) for the split-k GEMMs: a workgroup
// adds a 64 (c) x 64 (t) block over the splits in split order (a thread four
// consecutive t, its split loads issued four at a time), turns it in LDS and
// stores whole 128-byte rows of out.
template <bool F16>
__global__ __launch_bounds__(256) void k_split_sum(const float* part, int splits, int64_t C, int64_t T,
                                                  uint16_t* out) {
    __shared__ uint16_t tile[64][64 + 8];             // [t][c]
    const int64_t c0 = (int64_t)blockIdx.x * 64, t0 = (int64_t)blockIdx.y * 64;
    const int64_t ldp = (T + 3) & ~int64_t(3);       // partial row stride (see k_fwd)
    const int64_t plane = C * ldp;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = (int)threadIdx.x + 256 * k;     // 64 rows c x 16 float4 of t
        const int cl = e >> 4, tl = 4 * (e & 15);
        const int64_t c = c0 + cl, t = t0 + tl;
        f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (c < C && t < T) {                         // t + 3 < ldp: whole float4s
            const float* src = part + c * ldp + t;
            v = *reinterpret_cast<const f32x4_t*>(src);
            for (int sp = 1; sp < splits; sp += 4) {
                f32x4_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = sp + q < splits ? *reinterpret_cast<const f32x4_t*>(src + (sp + q) * plane)
                                           : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (sp + q < splits) v += w[q];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) tile[tl + u][cl] = (uint16_t)(pack16x2<F16>(v[u], 0.0f) & 0xFFFFu);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 8; e += 256) {
        const int tl = e >> 3, ch = e & 7;
        const int64_t t = t0 + tl, c = c0 + ch * 8;
        if (t < T && c < C) {
            u32x4_t v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = (uint32_t)tile[tl][ch * 8 + 2 * q] | ((uint32_t)tile[tl][ch * 8 + 2 * q + 1] << 16);
            *reinterpret_cast<u32x4_t*>(out + t * C + c) = v;
        }
    }
}

constexpr size_t kFwdSmem = 2 * 256 * 128 + kWideTableBytes;

// ------------------------------------------------------------------ dX

struct DxArgs {
    const uint16_t* dy;
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    const uint16_t* lora_a;   // [K][r]
    const uint16_t* gs_hi;    // [T][r_pad] bf16: s dY B^T = hi + lo
    const uint16_t* gs_lo;
    const float* sclt;        // [K/64][N] block scales c1'
    uint16_t* dx;
    int64_t T, K, N, r, r_pad;
    float* part;              // split-k: fp32 partial tiles [splits][K][T rounded up to 4]
    int splits;
};

// The transposed block scales alone (when no other launch of the backward
// carries them).
__global__ __launch_bounds__(256) void k_scales_t(ScalesJob j) {
    __shared__ __align__(16) uint8_t lds[kScalesLds];
    scales_job(j, (int)blockIdx.x, (lds8_t*)lds);
}

// dX = dY W' (+ (s dY B^T) A^T): tile 256 (k) x 256 (t), reduction over n in
// tiles of 64, waves 2 x 2 (wave (wa, wb) owns k rows wa*128.. and t rows
// wb*128..; four A and four B fragments per MFMA step, both from LDS).
//
// The W tile is written to LDS already transposed ([k][n]): each thread owns
// an 8 (n) x 8 (k) patch, i.e. one code dword of each of 8 rows.  The patch
// is done in quarters of two k columns (code byte j of every row); for each
// k the eight n values form one whole 16-byte chunk of the [k][n] tile.  W
// tile rows are stored permuted (bit 0 of the row flipped when bit 6 is set),
// which makes those 16-byte writes bank-conflict-free: the 16 lanes of a
// write phase hold k groups 0..15, so their rows cover both parities and all
// eight swizzled chunk positions.  The 32-row fragment reads only see a
// permutation inside their 32 rows and stay conflict-free.  The codebook
// lookups use a 16-copy byte-pair table (entry e of copy c at e*128 + c*8,
// lane l uses copy l & 15).
//
// Pipeline (per reduction tile kt, LDS buffers and register sets by parity):
// step j of tile kt runs its sixteen MFMAs while it reads the fragments of
// step j+1, looks up the codebook pairs of quarter j+1 of tile kt+1's W patch
// and dequantizes quarter j into the idle W buffer.  Step 3 is split around
// the barrier: half its MFMAs, the last quarter and tile kt+1's dY rows
// written, barrier, then the fragments of tile kt+1's step 0 and the lookups
// of quarter 0 of tile kt+2 are read during the other half.  W codes and
// block scales are loaded about a tile and a half ahead, dY one tile ahead.
// LDS offset inside a W^T tile: rows permuted as described above.
QL_DEV uint32_t lds_off_w(int row, int chunk) { return lds_off(row ^ ((row >> 6) & 1), chunk); }

typedef f32x2_t DqPairs[8];   // codebook pairs of one quarter patch: code byte j of rows 0..7

struct DxPipe {
    static constexpr uint32_t kTile = 256 * 128;
    rsrc_t rc, rs, rd;
    uint32_t cvo, svo, dvo[8];
    uint32_t lane8;
    int64_t K, N;
    int NT;
    u32x4_t dr[8];                 // dY rows of the next tile to store
    uint32_t cw[2][8];             // W codes of the tiles being staged, by parity
    u32x4_t sc[2][2];              // their eight block scales (rows n..n+7)

    QL_DEV void load_w(int kt, int par) {
        kt = kt < NT ? kt : NT - 1;
        const uint32_t soc = (uint32_t)(kt * 64 * (K / 2));
#pragma unroll
        for (int i = 0; i < 8; ++i) cw[par][i] = bload4(rc, cvo + i * (uint32_t)(K / 2), soc);
        sc[par][0] = bload16(rs, svo, (uint32_t)kt * 256u);
        sc[par][1] = bload16(rs, svo + 16, (uint32_t)kt * 256u);
    }
    QL_DEV void load_dy(int kt) {
        kt = kt < NT ? kt : NT - 1;
#pragma unroll
        for (int c = 0; c < 8; ++c) dr[c] = bload16(rd, dvo[c], (uint32_t)kt * 128u);
    }
    QL_DEV void store_dy(lds8_t* l) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ch = threadIdx.x + c * kThreads;
            *reinterpret_cast<lds_u32x4_t*>(l + lds_off(ch >> 3, ch & 7)) = dr[c];
        }
    }
    // codebook pairs of code byte j of the eight code dwords of set par
    QL_DEV void lookup(DqPairs& qv, int par, int j) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t addr = (__builtin_amdgcn_ubfe(cw[par][i], 8 * j, 8) << 7) | lane8;
            qv[i] = *lds_at<f32x2_t>(addr);
        }
    }
    // k columns 2j, 2j+1 of the patch: w' = RNE_16(fl32(q * c1')), eight n
    // values per column packed into one 16-byte chunk
    template <bool F16>
    QL_DEV void finish(const DqPairs& qv, int par, int j, lds8_t* l) const {
        const int kc = threadIdx.x & 31, ng = threadIdx.x >> 5;
        float v[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float c1p = __uint_as_float(sc[par][i >> 2][i & 3]);
            v[i][0] = __fmul_rn(qv[i][0], c1p);
            v[i][1] = __fmul_rn(qv[i][1], c1p);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4_t o;
#pragma unroll
            for (int p = 0; p < 4; ++p) o[p] = pack16x2<F16>(v[2 * p][c], v[2 * p + 1][c]);
            *reinterpret_cast<lds_u32x4_t*>(l + lds_off_w(kc * 8 + 2 * j + c, ng)) = o;
        }
    }
};

struct DxFrags {
    bf16x8_t a[4], b[4];
};

template <bool kMapW>
QL_DEV void dx_reads(DxFrags& f, const lds8_t* lw, const lds8_t* ld, int s, int wa, int wb, int r, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wa * 128 + i * 32 + r;
        f.a[i] = *reinterpret_cast<const lds_bf16x8_t*>(lw + (kMapW ? lds_off_w(row, 2 * s + h) : lds_off(row, 2 * s + h)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = lds_frag(ld, wb * 128 + j * 32 + r, 2 * s + h);
}

template <bool F16>
QL_DEV void dx_mfma(f32x16_t (&acc)[4][4], const DxFrags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = mfma32x32x16<F16>(f.a[i], f.b[j], acc[i][j]);
}

// MFMAs of output rows i in [i0, i1) only (used to split a step around the barrier)
template <int i0, int i1, bool F16>
QL_DEV void dx_mfma_rows(f32x16_t (&acc)[4][4], const DxFrags& f) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = mfma32x32x16<F16>(f.a[i], f.b[j], acc[i][j]);
}

template <int P, bool F16>
QL_DEV void dx_tile(DxPipe& pp, int kt, f32x16_t (&acc)[4][4], lds8_t* lW, lds8_t* lD, int wa, int wb, int r,
                    int h, DxFrags& f0, DqPairs& qa) {
    constexpr int Q = P ^ 1;
    const lds8_t* cw = lW + P * DxPipe::kTile;
    const lds8_t* cd = lD + P * DxPipe::kTile;
    lds8_t* nw = lW + Q * DxPipe::kTile;
    lds8_t* nd = lD + Q * DxPipe::kTile;
    DxFrags f1;
    DqPairs qb;
    // step 0
    dx_reads<true>(f1, cw, cd, 1, wa, wb, r, h);
    pp.lookup(qb, Q, 1);
    pp.template finish<F16>(qa, Q, 0, nw);
    dx_mfma<F16>(acc, f0);
    interleave<16, 16, 16>();
    __builtin_amdgcn_sched_barrier(0);
    // step 1
    dx_reads<true>(f0, cw, cd, 2, wa, wb, r, h);
    pp.lookup(qa, Q, 2);
    pp.template finish<F16>(qb, Q, 1, nw);
    dx_mfma<F16>(acc, f1);
    interleave<16, 16, 16>();
    __builtin_amdgcn_sched_barrier(0);
    // step 2
    dx_reads<true>(f1, cw, cd, 3, wa, wb, r, h);
    pp.lookup(qb, Q, 3);
    pp.template finish<F16>(qa, Q, 2, nw);
    dx_mfma<F16>(acc, f0);
    interleave<16, 16, 16>();
    __builtin_amdgcn_sched_barrier(0);
    // step 3
    dx_mfma_rows<0, 2, F16>(acc, f1);
    pp.template finish<F16>(qb, Q, 3, nw);
    pp.store_dy(nd);
    interleave<8, 0, 8, 8, 4>();
    __builtin_amdgcn_sched_barrier(0);
    pp.load_dy(kt + 2);                       // dY registers are free again
    __syncthreads();
    dx_reads<true>(f0, nw, nd, 0, wa, wb, r, h);
    pp.lookup(qa, P, 0);                      // tile kt+2's codes (set P, loaded during tile kt-1)
    dx_mfma_rows<2, 4, F16>(acc, f1);
    interleave<8, 16, 0>();
    __builtin_amdgcn_sched_barrier(0);
    pp.load_w(kt + 3, Q);                     // set Q (tile kt+1) is no longer read
}

// SPLIT: as in k_fwd, `splits` workgroups per tile, each over a range of the
// reduction's n tiles (split 0 also adds the LoRA term), writing fp32
// partial tiles that k_split_sum adds in split order.
template <bool F16, bool FUSED, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void k_dx(DxArgs p, Codebook cb, FusedGrads fz) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    lds8_t* smem = (lds8_t*)(smem_raw);
    constexpr uint32_t kTile = DxPipe::kTile;
    lds8_t* const lW = smem;                  // 2 tiles [256 k][64 n] (rows permuted)
    lds8_t* const lD = smem + 2 * kTile;      // 2 tiles [256 t][64 n]
    lds8_t* const tbl = smem + 4 * kTile;     // 16-copy pair table
    build_pair_table16(tbl, cb);
    const int ga = (int)ceil_div(p.K, 256), gb = (int)ceil_div(p.T, 256);
    int ta, tb, split = 0;
    const int NT_all = (int)(p.N / 64);
    int nt0 = 0, nt1 = NT_all;
    if constexpr (SPLIT) {
        split = (int)blockIdx.x / (ga * gb);
        tile_of((int)blockIdx.x % (ga * gb), ga, gb, ta, tb);
        nt0 = split * NT_all / p.splits;
        nt1 = (split + 1) * NT_all / p.splits;
    } else {
        tile_of(blockIdx.x, ga, gb, ta, tb);
    }
    const int64_t k0 = (int64_t)ta * 256, t0 = (int64_t)tb * 256;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wa = wave >> 1, wb = wave & 1;
    const int r = lane & 31, h = lane >> 5;

    DxPipe pp;
    pp.K = p.K;
    pp.N = p.N;
    pp.NT = nt1 - nt0;
    pp.rc = make_rsrc(p.codes, p.N * p.K / 2);
    pp.rs = make_rsrc(p.sclt, (p.K / 64) * p.N * 4);
    pp.rd = make_rsrc(p.dy, p.T * p.N * 2);
    pp.lane8 = lds_addr(tbl) + (uint32_t)(lane & 15) * 8u;   // table is 32 KB aligned
    {
        const int64_t k = k0 + (threadIdx.x & 31) * 8;
        const int64_t n = (threadIdx.x >> 5) * 8;
        const bool ok = k < p.K;
        const int64_t nb = n + (int64_t)nt0 * 64;                    // first n of this split
        pp.cvo = ok ? (uint32_t)(nb * (p.K / 2) + k / 2) : kOOB;
        pp.svo = ok ? (uint32_t)(((k / 64) * p.N + nb) * 4) : kOOB;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int ch = threadIdx.x + c * kThreads;
        const int64_t t = t0 + (ch >> 3);
        pp.dvo[c] = t < p.T ? (uint32_t)((t * p.N + (int64_t)nt0 * 64 + (ch & 7) * 8) * 2) : kOOB;
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // prologue: tile 0 staged in LDS buffer 0; tile 1's codes and dY rows and
    // tile 2's codes in registers; tile 0's step-0 fragments and the pairs of
    // quarter 0 of tile 1 read
    pp.load_w(0, 0);
    pp.load_w(1, 1);
    pp.load_dy(0);
    __syncthreads();                          // pair table visible
    DqPairs qa;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pp.lookup(qa, 0, j);
        pp.template finish<F16>(qa, 0, j, lW);
    }
    pp.store_dy(lD);
    pp.load_dy(1);
    pp.load_w(2, 0);
    pp.lookup(qa, 1, 0);
    __syncthreads();
    DxFrags f0;
    dx_reads<true>(f0, lW, lD, 0, wa, wb, r, h);
    const int NT = pp.NT;
    int kt = 0;
    for (; kt + 1 < NT; kt += 2) {
        dx_tile<0, F16>(pp, kt, acc, lW, lD, wa, wb, r, h, f0, qa);
        dx_tile<1, F16>(pp, kt + 1, acc, lW, lD, wa, wb, r, h, f0, qa);
    }
    if (kt < NT) dx_tile<0, F16>(pp, kt, acc, lW, lD, wa, wb, r, h, f0, qa);

    if (p.r > 0 && split == 0) {
        // LoRA term (s dY B^T) A^T: reduction over [hi | lo] of s dY B^T against A stacked twice
        const int half = (int)(p.r_pad / 64);
        PlainRows<256, true> pa;
        pa.init(p.lora_a, p.lora_a, p.r, p.K, k0, p.r, half);
        PlainRows<256> pb;
        pb.init(p.gs_hi, p.gs_lo, p.r_pad, p.T, t0, p.r_pad, half);
        for (int lt = 0; lt < 2 * half; ++lt) {
            pa.load(lt);
            pb.load(lt);
            __syncthreads();
            pa.store(lW, tbl);
            pb.store(lD, tbl);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                DxFrags f;
                dx_reads<false>(f, lW, lD, s, wa, wb, r, h);
                dx_mfma<F16>(acc, f);
            }
        }
    }
    if constexpr (SPLIT) {
        // fp32 partial tile part[split][k][t] through LDS in two halves: half hf
        // holds accumulators i = 2 hf, 2 hf + 1 of every wave, LDS row
        // 64 wa + 32 (i & 1) + q = tile row 128 wa + 32 i + q (q = 8 g + 4 h + v);
        // the chunks of rows with bit 2 set sit 128 bytes over (distinct banks
        // for the two halves of a wave's store); whole 1 KB rows go out as float4s
        const int64_t ldp = (p.T + 3) & ~int64_t(3);
        float* out = p.part + (int64_t)split * p.K * ldp;
        float* lt = reinterpret_cast<float*>(smem_raw);                  // [128][256] fp32
        auto loff = [](int row, int t) { return row * 256 + (t ^ (((row >> 2) & 1) << 5)); };
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {                                 // unrolled: acc indices stay static
            __syncthreads();                                             // LDS readers are done
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            lt[loff(64 * wa + 32 * ii + 8 * g + 4 * h + v, wb * 128 + 32 * j + r)] =
                                acc[2 * hf + ii][j][4 * g + v];
            __syncthreads();
#pragma unroll 4
            for (int e = threadIdx.x; e < 128 * 64; e += kThreads) {     // 64 float4 per row
                const int row = e >> 6, c4 = e & 63;
                const int64_t k = k0 + 128 * (row >> 6) + 64 * hf + (row & 63);
                const int64_t t = t0 + 4 * c4;
                if (k < p.K && t < p.T) {                                 // t + 3 < ldp
                    const float* src = lt + loff(row, 4 * c4);
                    *reinterpret_cast<f32x4_t*>(out + k * ldp + t) = f32x4_t{src[0], src[1], src[2], src[3]};
                }
            }
        }
    } else {
        // C[k][t] -> dX[t][k] through an LDS tile over the W and dY tiles
        __syncthreads();                          // every wave is done reading them
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    otile_put4<F16>(smem, acc[i][j], g, wb * 128 + j * 32 + r, wa * 128 + i * 32 + g * 8 + h * 4);
        __syncthreads();
        otile_store(smem, p.dx, p.K, t0, k0, p.T, p.K);
    }

    if constexpr (FUSED) {
        // this wave's blocks of the adapter gradients (see FusedGrads): every
        // wave of the grid takes every waves-th block and writes its partial
        const int RB = (int)(p.r_pad / 64);
        const int na = fz.ga.part ? fz.groups * fz.ga.cblocks * RB : 0;
        const int nb = fz.gb.part ? fz.groups * fz.gb.cblocks * RB : 0;
#pragma unroll 1
        for (int q = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6); q < na + nb; q += fz.waves) {
            const bool first = q < na;
            const GradArgs g = first ? fz.ga : fz.gb;
            const int qq = first ? q : q - na;
            const int jb = qq % RB, cbx = (qq / RB) % g.cblocks, grp = qq / (RB * g.cblocks);
            grad_wave<F16>(g, cbx, grp, fz.tpg, (int64_t)jb * 64);
        }
    }
}

constexpr size_t kDxSmem = 4 * 256 * 128 + kNarrowTableBytes;

// ------------------------------------------------------------------ launchers

namespace {
template <class F>
hipError_t set_smem(F* f, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

}  // namespace

hipError_t launch_fwd(const uint16_t* x, const uint8_t* codes, BlockScales sc, const uint16_t* lora_b,
                      const LoraPlan& pl, const uint8_t* ws, uint16_t* y, hipStream_t s, bool f16) {
    const bool split = pl.s_fwd > 1;
    FwdArgs a{x, codes, sc.fp8, sc.sup, sc.absmax, lora_b, reinterpret_cast<const uint16_t*>(ws + pl.off_ps_hi),
              reinterpret_cast<const uint16_t*>(ws + pl.off_ps_lo), y,
              pl.T, pl.K, pl.N, pl.r, pl.r_pad,
              split ? reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + pl.off_fsp) : nullptr, pl.s_fwd};
    const size_t lds = kFwdSmem;
    const int64_t tiles = ceil_div(pl.N, 256) * ceil_div(pl.T, 256) * (split ? pl.s_fwd : 1);
    auto go = [&](auto kern) {
        hipError_t e = set_smem(kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kThreads), lds, s, a, host_codebook());
        return hipGetLastError();
    };
    if (split) {
        hipError_t e;
        if (sc.single()) e = f16 ? go(k_fwd<true, true, true>) : go(k_fwd<true, false, true>);
        else e = f16 ? go(k_fwd<false, true, true>) : go(k_fwd<false, false, true>);
        if (e != hipSuccess) return e;
        const dim3 g((unsigned)ceil_div(pl.N, 64), (unsigned)ceil_div(pl.T, 64));
        if (f16) hipLaunchKernelGGL(k_split_sum<true>, g, dim3(256), 0, s, a.part, pl.s_fwd, pl.N, pl.T, y);
        else hipLaunchKernelGGL(k_split_sum<false>, g, dim3(256), 0, s, a.part, pl.s_fwd, pl.N, pl.T, y);
        return hipGetLastError();
    }
    if (f16) return sc.single() ? go(k_fwd<true, true, false>) : go(k_fwd<false, true, false>);
    return sc.single() ? go(k_fwd<true, false, false>) : go(k_fwd<false, false, false>);
}

ScalesJob scales_job_for(BlockScales sc, const LoraPlan& pl, uint8_t* ws) {
    return ScalesJob{sc.fp8, sc.sup, sc.absmax, pl.N, pl.K / 64, reinterpret_cast<float*>(ws + pl.off_scl),
                     scales_job_blocks(pl.N, pl.K / 64)};
}

hipError_t launch_dx(const uint16_t* dy, const uint8_t* codes, BlockScales sc, const uint16_t* lora_a,
                     const LoraPlan& pl, const uint8_t* ws, uint16_t* dx, hipStream_t s, bool f16,
                     bool scales_ready, const FusedGrads* fused) {
    const float* sclt = reinterpret_cast<const float*>(ws + pl.off_scl);
    if (!scales_ready) {
        const ScalesJob j = scales_job_for(sc, pl, const_cast<uint8_t*>(ws));
        hipLaunchKernelGGL(k_scales_t, dim3((unsigned)j.blocks), dim3(256), 0, s, j);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
    }
    const bool split = pl.s_dx > 1;
    float* part = split ? reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + (fused ? pl.off_dxp_fused : pl.off_dxp))
                        : nullptr;
    DxArgs a{dy, codes, sc.fp8, sc.sup, lora_a, reinterpret_cast<const uint16_t*>(ws + pl.off_gs_hi),
             reinterpret_cast<const uint16_t*>(ws + pl.off_gs_lo), sclt, dx,
             pl.T, pl.K, pl.N, pl.r, pl.r_pad, part, pl.s_dx};
    const size_t lds = kDxSmem;
    const int64_t tiles = ceil_div(pl.K, 256) * ceil_div(pl.T, 256) * (split ? pl.s_dx : 1);
    FusedGrads f = fused ? *fused : FusedGrads{};
    f.waves = (int)tiles * 4;                         // the grid's waves share the gradient blocks
    auto go = [&](auto kern) {
        hipError_t e = set_smem(kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kThreads), lds, s, a, host_codebook(), f);
        return hipGetLastError();
    };
    hipError_t e;
    if (split) {
        if (fused) e = f16 ? go(k_dx<true, true, true>) : go(k_dx<false, true, true>);
        else e = f16 ? go(k_dx<true, false, true>) : go(k_dx<false, false, true>);
        if (e != hipSuccess) return e;
        const dim3 g((unsigned)ceil_div(pl.K, 64), (unsigned)ceil_div(pl.T, 64));
        if (f16) hipLaunchKernelGGL(k_split_sum<true>, g, dim3(256), 0, s, part, pl.s_dx, pl.K, pl.T, dx);
        else hipLaunchKernelGGL(k_split_sum<false>, g, dim3(256), 0, s, part, pl.s_dx, pl.K, pl.T, dx);
        return hipGetLastError();
    }
    if (fused) return f16 ? go(k_dx<true, true, false>) : go(k_dx<false, true, false>);
    return f16 ? go(k_dx<true, false, false>) : go(k_dx<false, false, false>);
}

}  // namespace ql
