// LoRA merge: W_m[n][k] = RNE_bf16(W'[n][k] + s sum_j A[k][j] B[j][n]), the
// adapted layer's weight in bf16 (fp16 with the F16 compute type) ("QLoRA 原理精讲" section 2.5 and section 3,
// pitfall 3: after training the adapter can be merged back into BF16 weights).
// W' = RNE_bf16(fl32(q[code] * c1')) with c1' = fl32(e4m3(f) * s2), the same
// values nf4_dequantize_dq writes.  The rank-r product is accumulated in fp32
// on MFMA and added to W' with one fused multiply-add before the rounding.
//
// HBM-bound: 0.516 bytes of codes and constants in and 2 bytes out per
// weight; A and B are small and re-read from L2.
//
// Workgroup: 64 rows n x 256 k, four waves of 64 k.  Everything the tile
// reads is staged through LDS with whole-line loads: the codes (64 rows of
// 128 bytes, each row read by eight lanes), the block constants c1' (decoded
// once per block by one thread), and per 64-rank chunk the A rows (256 rows of
// 128 bytes) and B's 64 columns transposed ([n][j], an 8 x 8 register
// transpose per lane, so that staging is 16-byte LDS writes).  Lanes then take
// their operands from LDS instead of gathering 4- and 16-byte pieces from 16
// rows per load.  Each wave runs v_mfma_f32_16x16x32_bf16 with the A operand =
// rows of A (index k) and the B operand = columns of B^T's transpose (index
// n), 4 x 4 tiles of 16 k x 16 n.  The k of MFMA row m in row tile t is
// 32 (t / 2) + 8 (m / 4) + 4 (t % 2) + (m % 4): the accumulator rows a lane
// holds (m = 4 (lane / 16) + v in every tile) then cover k 8q .. 8q+7 in
// tiles 0-1 and 32 + 8q .. +7 in tiles 2-3 (q = lane / 16), so the epilogue is
// two 4-byte code reads, 16 dequantized weights and two 16-byte LDS writes per
// (lane, n tile), straight from the accumulators; the [64][256] output tile
// (over the A rows' LDS, free by then) leaves as whole 512-byte rows with
// non-temporal stores.
#include <type_traits>

#include "common.hpp"
#include "plan.hpp"

namespace ql {

namespace {

struct MergeArgs {
    const uint8_t* codes;
    const uint8_t* fp8;
    const float* sup;
    const float* absmax;  // single quantization: fp32 block absmax (fp8/sup unused)
    const uint16_t* a;    // [K][r]
    const uint16_t* b;    // [r][N]
    uint16_t* w;          // [N][K]
    int64_t K, N, r;
    float s;
};

constexpr int kMergeRows = 64;    // n per workgroup
constexpr int kMergeK = 256;      // k per workgroup (64 per wave)

// LDS: the A rows of one 64-rank chunk [256][128 bytes] (reused for the output
// tile [64][256] of 16-bit values, 512-byte rows), B^T of the chunk [64][128
// bytes], the codes [64][128 bytes], c1' [64][4] and the codebook.
constexpr int kMergeLdsA = kMergeK * 128, kMergeLdsBt = kMergeRows * 128, kMergeLdsCodes = kMergeRows * 128;
constexpr int kMergeLds = kMergeLdsA + kMergeLdsBt + kMergeLdsCodes + kMergeRows * 4 * 4 + 16 * 4;

// Output tile [64 rows][256 k]: row t is 512 bytes and its 16-byte chunk c
// sits at chunk position c ^ (t & 31), so the epilogue's writes (16 rows at one
// chunk) and the row reads of the stores are bank-conflict-free.
QL_DEV uint32_t mtile_off(int t, int c) { return (uint32_t)t * 512u + ((uint32_t)(c ^ (t & 31)) << 4); }

// RP = r_pad / 64 (1..4) rank chunks.  SQ: the block constant is the stored
// fp32 absmax (single quantization).
template <int RP, bool SQ, bool F16>
__global__ __launch_bounds__(256, RP == 1 ? 3 : 2) void k_merge(MergeArgs p, Codebook cb) {
    typedef __attribute__((address_space(3))) float lds_f32_t;
    typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
    extern __shared__ __align__(16) uint8_t smem_raw[];
    lds8_t* const s_a = (lds8_t*)smem_raw;                             // A rows, later the output tile
    lds8_t* const s_out = s_a;
    lds8_t* const s_bt = s_a + kMergeLdsA;
    lds8_t* const s_codes = s_bt + kMergeLdsBt;
    lds_f32_t* const s_c1 = reinterpret_cast<lds_f32_t*>(s_codes + kMergeLdsCodes);   // [64][4]
    lds_f32_t* const s_q = s_c1 + kMergeRows * 4;                                       // [16]
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nl = lane & 15, q = lane >> 4;
    const int nb = (int)ceil_div(p.N, kMergeRows);
    const int rb = (int)blockIdx.x % nb, kb = (int)blockIdx.x / nb;
    const int64_t n0 = (int64_t)rb * kMergeRows;
    const int64_t kt0 = (int64_t)kb * kMergeK;                         // the workgroup's first k
    const int64_t KB = p.K / 64;
    const rsrc_t rc = make_rsrc(p.codes, p.N * p.K / 2);
    const rsrc_t rf = SQ ? make_rsrc(p.absmax, p.N * KB * 4) : make_rsrc(p.fp8, p.N * KB);
    const rsrc_t rs = SQ ? rf : make_rsrc(p.sup, ceil_div(p.N * KB, 256) * 4);
    const rsrc_t ra = make_rsrc(p.a, p.K * p.r * 2);
    const rsrc_t rbm = make_rsrc(p.b, p.r * p.N * 2);

    // global loads of one rank chunk: A rows kt0 .. kt0+255, ranks 64 cc .. +63
    // (piece e = tid + 256 i: row e / 8, ranks 8 (e % 8) .. +7; r % 8 == 0 keeps
    // a piece inside or outside the rank range as a whole), and B's ranks
    // 64 cc + 8 jb .. +7 of columns n0 + 8 nc .. +7 for the first 64 threads
    const int jb = tid >> 3, nc = tid & 7;
    auto load_chunk = [&](int cc, u32x4_t (&av)[8], u32x4_t (&bv)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            const int64_t k = kt0 + (e >> 3);
            const int64_t j = 64 * cc + 8 * (e & 7);
            av[i] = bload16(ra, (k < p.K && j < p.r) ? (uint32_t)((k * p.r + j) * 2) : kOOB, 0);
        }
        const int64_t nb8 = n0 + 8 * nc;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t j = 64 * cc + 8 * jb + e;
            bv[e] = bload16(rbm, (tid < 64 && j < p.r && nb8 < p.N) ? (uint32_t)((j * p.N + nb8) * 2) : kOOB, 0);
        }
    };
    // A pieces into [256][128] rows; B^T: thread (jb, nc) transposes its 8 x 8
    // block with 32 byte permutes and writes column n's 8 ranks as one 16-byte
    // chunk of the [n][j] rows (ranks >= r and columns >= N are zeros)
    auto store_chunk = [&](const u32x4_t (&av)[8], const u32x4_t (&bv)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = tid + 256 * i;
            *reinterpret_cast<lds_u32x4_t*>(s_a + lds_off(e >> 3, e & 7)) = av[i];
        }
        if (tid < 64) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high or low halves: column 8 nc + i
                u32x4_t o;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) o[pp] = __builtin_amdgcn_perm(bv[2 * pp + 1][i >> 1], bv[2 * pp][i >> 1], sel);
                *reinterpret_cast<lds_u32x4_t*>(s_bt + lds_off(8 * nc + i, jb)) = o;
            }
        }
    };

    // the codes: 64 rows x 128 bytes, eight 16-byte pieces per row (piece e =
    // tid + 256 i: row e / 8, k kt0 + 32 (e % 8) .. +31)
    u32x4_t cv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = tid + 256 * i;
        const int64_t n = n0 + (e >> 3), k = kt0 + 32 * (e & 7);
        cv[i] = bload16(rc, (n < p.N && k < p.K) ? (uint32_t)(n * (p.K / 2) + k / 2) : kOOB, 0);
    }
    // the block constants: thread (row tid / 4, block tid % 4)
    uint32_t f8v, s2v;
    {
        const int64_t n = n0 + (tid >> 2), kbl = kt0 / 64 + (tid & 3);
        const bool ok = n < p.N && kbl < KB;
        const int64_t blk = n * KB + kbl;
        if constexpr (SQ) {
            f8v = 0;
            s2v = bload4(rf, ok ? (uint32_t)blk * 4u : kOOB, 0);
        } else {
            f8v = bload1(rf, ok ? (uint32_t)blk : kOOB, 0);
            s2v = bload4(rs, ok ? (uint32_t)(blk >> 8) * 4u : kOOB, 0);
        }
    }
    u32x4_t av[8], bv[8];
    load_chunk(0, av, bv);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = tid + 256 * i;
        *reinterpret_cast<lds_u32x4_t*>(s_codes + lds_off(e >> 3, e & 7)) = cv[i];
    }
    s_c1[tid] = SQ ? __uint_as_float(s2v) : block_scale(f8v, __uint_as_float(s2v));
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (tid == j) s_q[j] = cb_value(cb, j);
    store_chunk(av, bv);
    __syncthreads();

    // rank-r product: acc[t][c] = 16 k x 16 n tile, 32 ranks per MFMA; A
    // operand row of this lane in tile t: m = nl -> k = 64 wave + 32 (t / 2) +
    // 8 (m / 4) + 4 (t % 2) + m % 4 of the staged rows
    f32x4_t acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[t][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < RP; ++cc) {
        if (cc > 0) {
            load_chunk(cc, av, bv);
            __syncthreads();                                           // the previous chunk is read
            store_chunk(av, bv);
            __syncthreads();
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {                                  // 32 ranks each
            u32x4_t af[4], bf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int row = 64 * wave + 32 * (t >> 1) + 8 * (nl >> 2) + 4 * (t & 1) + (nl & 3);
                af[t] = *reinterpret_cast<const lds_u32x4_t*>(s_a + lds_off(row, 4 * h + q));
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                bf[c] = *reinterpret_cast<const lds_u32x4_t*>(s_bt + lds_off(16 * c + nl, 4 * h + q));
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc[t][c] = mfma16x16x32<F16>(__builtin_bit_cast(bf16x8_t, af[t]),
                                                  __builtin_bit_cast(bf16x8_t, bf[c]), acc[t][c]);
        }
    }
    __syncthreads();                                                   // A rows read: the output tile may follow

    // epilogue: lane holds k 64 wave + 32 (t / 2) + 8q + 4 (t % 2) + v of row 16c + nl in acc[t][c][v]
    const float sc = p.s;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int row = 16 * c + nl;
        const float c1p = s_c1[row * 4 + wave];
        // code bytes of k 64 wave + 8q .. +7 and 64 wave + 32 + 8q .. +7: bytes 32 wave + 4q and + 16
        const uint32_t cw0 = *reinterpret_cast<const lds_u32_t*>(s_codes + lds_off(row, 2 * wave) + 4 * q);
        const uint32_t cw1 = *reinterpret_cast<const lds_u32_t*>(s_codes + lds_off(row, 2 * wave + 1) + 4 * q);
        u32x4_t o[2];
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            // code byte bb of half hf = bb / 4: k 8q + 2 (bb % 4) (high nibble) and the next,
            // plus 32 in half 1; they sit in tile t = 2 hf + (bb % 4) / 2, rows v = 2 (bb % 2) .. +1
            const uint32_t byte = (((bb >> 2) ? cw1 : cw0) >> (8 * (bb & 3))) & 0xFFu;
            const uint32_t wq = pack16x2<F16>(__fmul_rn(s_q[byte >> 4], c1p), __fmul_rn(s_q[byte & 15u], c1p));
            const int t = 2 * (bb >> 2) + ((bb & 3) >> 1), v = 2 * (bb & 1);
            const float m0 = fmaf(sc, acc[t][c][v], lo16<F16>(wq));
            const float m1 = fmaf(sc, acc[t][c][v + 1], hi16<F16>(wq));
            o[bb >> 2][bb & 3] = pack16x2<F16>(m0, m1);
        }
        // tile row 16c + nl, chunks (64 wave + 8 q) / 8 and 4 further
        *reinterpret_cast<lds_u32x4_t*>(s_out + mtile_off(row, 8 * wave + q)) = o[0];
        *reinterpret_cast<lds_u32x4_t*>(s_out + mtile_off(row, 8 * wave + q + 4)) = o[1];
    }
    __syncthreads();
    // whole rows out: each wave store writes two rows of 512 contiguous bytes,
    // streamed once (non-temporal, so it does not displace A and B in the caches)
#pragma unroll
    for (int it = 0; it < kMergeRows * 32 / 256; ++it) {
        const int u = tid + 256 * it;
        const int row = u >> 5, ch = u & 31;
        const int64_t n = n0 + row, k = kt0 + 8 * ch;
        if (n < p.N && k < p.K) {
            const u32x4_t v = *reinterpret_cast<const lds_u32x4_t*>(s_out + mtile_off(row, ch));
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p.w + n * p.K + k));
        }
    }
}

}  // namespace

hipError_t launch_merge(const uint8_t* codes, BlockScales sc, const uint16_t* lora_a, const uint16_t* lora_b,
                        int64_t K, int64_t N, int64_t r, float scaling, uint16_t* w_out, hipStream_t s, bool f16) {
    if (r == 0) return launch_dequantize(codes, sc, N * K, w_out, s, false, f16);
    const MergeArgs a{codes, sc.fp8, sc.sup, sc.absmax, lora_a, lora_b, w_out, K, N, r, scaling};
    const dim3 grid((unsigned)(ceil_div(N, kMergeRows) * ceil_div(K, kMergeK))), block(256);
    const Codebook& cb = host_codebook();
    hipError_t ae = hipSuccess;
    auto go = [&](auto kern) {
        // more than the default dynamic LDS limit
        ae = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kMergeLds);
        if (ae == hipSuccess) hipLaunchKernelGGL(kern, grid, block, kMergeLds, s, a, cb);
    };
    const bool sq = sc.single();
    auto pick = [&](auto rp) {
        constexpr int RP = decltype(rp)::value;
        if (sq) f16 ? go(k_merge<RP, true, true>) : go(k_merge<RP, true, false>);
        else f16 ? go(k_merge<RP, false, true>) : go(k_merge<RP, false, false>);
    };
    switch ((int)ceil_div(r, 64)) {
        case 1: pick(std::integral_constant<int, 1>{}); break;
        case 2: pick(std::integral_constant<int, 2>{}); break;
        case 3: pick(std::integral_constant<int, 3>{}); break;
        default: pick(std::integral_constant<int, 4>{}); break;
    }
    if (ae != hipSuccess) return ae;
    return hipGetLastError();
}

}  // namespace ql
