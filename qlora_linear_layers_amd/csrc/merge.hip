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
// Workgroup: 64 rows n x 256 k, four waves of 64 k.  B's 64 columns of the
// workgroup are staged transposed in LDS ([n][j], XOR-swizzled 64-wide j
// blocks; an 8 x 8 register transpose per lane, so the staging is 16-byte LDS
// writes), and both MFMA operands are 16-byte fragment reads.  Each wave runs
// v_mfma_f32_16x16x32_bf16 with the A operand = rows of A (index k) and the B
// operand = columns of B^T's transpose (index n), 4 x 4 tiles of 16 k x 16 n.
// The k of MFMA row m in row tile t is 32 (t / 2) + 8 (m / 4) + 4 (t % 2) +
// (m % 4): the accumulator rows a lane holds (m = 4 (lane / 16) + v in every
// tile) then cover k 8q .. 8q+7 in tiles 0-1 and 32 + 8q .. +7 in tiles 2-3
// (q = lane / 16), so the epilogue is two 4-byte code loads, 16 dequantized
// weights and two 16-byte LDS writes per (lane, n tile), straight from the
// accumulators; the workgroup's [64][256] output tile then leaves as whole
// 512-byte rows (measured +12% over storing the lanes' 64-byte row pieces
// directly).
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

// RP = r_pad / 64 (1..4): B^T is RP swizzled [64 n][64 j] tiles of 8 KB.
// SQ: the block constant is the stored fp32 absmax (single quantization).
// Output tile [64 rows][256 k] of 16-bit values in LDS: row t is 512 bytes and
// its 16-byte chunk c sits at chunk position c ^ (t & 31), so the epilogue's
// writes (16 rows at one chunk) and the row reads of the stores are
// bank-conflict-free.
QL_DEV uint32_t mtile_off(int t, int c) { return (uint32_t)t * 512u + ((uint32_t)(c ^ (t & 31)) << 4); }

template <int RP, bool SQ, bool F16>
__global__ __launch_bounds__(256) void k_merge(MergeArgs p, Codebook cb) {
    __shared__ float s_q[16];
    __shared__ __align__(16) uint8_t s_bt[RP * 8192];
    __shared__ __align__(16) uint8_t s_out[kMergeRows * kMergeK * 2];
    lds8_t* bt = (lds8_t*)s_bt;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nl = lane & 15, q = lane >> 4;
    const int nb = (int)ceil_div(p.N, kMergeRows);
    const int rb = (int)blockIdx.x % nb, kb = (int)blockIdx.x / nb;
    const int64_t n0 = (int64_t)rb * kMergeRows;
    const int64_t k0 = (int64_t)kb * kMergeK + 64 * wave;             // this wave's 64 k (one block per row)
    const bool kok = k0 < p.K;                                         // K % 64 == 0: all 64 or none
    const rsrc_t rc = make_rsrc(p.codes, p.N * p.K / 2);
    const rsrc_t rf = SQ ? make_rsrc(p.absmax, p.N * p.K / 64 * 4) : make_rsrc(p.fp8, p.N * p.K / 64);
    const rsrc_t rs = SQ ? rf : make_rsrc(p.sup, ceil_div(p.N * p.K / 64, 256) * 4);
    const rsrc_t ra = make_rsrc(p.a, p.K * p.r * 2);
    const rsrc_t rbm = make_rsrc(p.b, p.r * p.N * 2);

    // epilogue loads first: for n tile c, row n0 + 16c + nl, k0 + 8q .. +7 and k0 + 32 + 8q .. +7
    u32x2_t cw[4];
    uint32_t f8[4], s2[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t n = n0 + 16 * c + nl;
        const bool ok = kok && n < p.N;
        const int64_t blk = n * (p.K / 64) + k0 / 64;
        const uint32_t cb0 = ok ? (uint32_t)(n * (p.K / 2) + (k0 + 8 * q) / 2) : kOOB;
        cw[c][0] = bload4(rc, cb0, 0);
        cw[c][1] = bload4(rc, ok ? cb0 + 16u : kOOB, 0);
        if constexpr (SQ) {
            f8[c] = 0;
            s2[c] = bload4(rf, ok ? (uint32_t)blk * 4u : kOOB, 0);
        } else {
            f8[c] = bload1(rf, ok ? (uint32_t)blk : kOOB, 0);
            s2[c] = bload4(rs, ok ? (uint32_t)(blk >> 8) * 4u : kOOB, 0);
        }
    }

    // A fragments of the first kPre rank steps, before the barrier (A operand
    // row of this lane in tile t: m = nl -> k = 32 (t / 2) + 8 (m / 4) + 4 (t % 2) + m % 4)
    constexpr int kSteps = RP * 2, kPre = kSteps < 4 ? kSteps : 4;
    auto a_frag = [&](int js, int t) -> u32x4_t {
        const int j = 32 * js + 8 * q;                                 // this lane's 8 ranks
        const int64_t k = k0 + 32 * (t >> 1) + 8 * (nl >> 2) + 4 * (t & 1) + (nl & 3);
        return bload16(ra, (kok && j < p.r) ? (uint32_t)((k * p.r + j) * 2) : kOOB, 0);
    };
    u32x4_t apre[kPre][4];
#pragma unroll
    for (int js = 0; js < kPre; ++js)
#pragma unroll
        for (int t = 0; t < 4; ++t) apre[js][t] = a_frag(js, t);

    // stage B^T: thread (jb, nc) of the first RP * 64 loads the 8 x 8 block of
    // ranks 8 jb .. +7 and columns n0 + 8 nc .. +7 (16 bytes per rank row; N % 8
    // == 0 keeps them inside the row and 16-byte aligned), transposes it with 32
    // byte permutes and writes column n's 8 ranks as one 16-byte chunk of the
    // [n][j] tile; ranks j >= r and columns n >= N are zeros
    if ((int)threadIdx.x < RP * 64) {
        const int jb = (int)threadIdx.x >> 3, nc = (int)threadIdx.x & 7;
        const int64_t nb8 = n0 + 8 * nc;
        u32x4_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 8 * jb + e;
            v[e] = bload16(rbm, (j < p.r && nb8 < p.N) ? (uint32_t)((j * p.N + nb8) * 2) : kOOB, 0);
        }
        lds8_t* tile = bt + (jb >> 3) * 8192;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high or low halves: column 8 nc + i
            u32x4_t o;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) o[pp] = __builtin_amdgcn_perm(v[2 * pp + 1][i >> 1], v[2 * pp][i >> 1], sel);
            *reinterpret_cast<lds_u32x4_t*>(tile + lds_off(8 * nc + i, jb & 7)) = o;
        }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (threadIdx.x == j) s_q[j] = cb_value(cb, j);
    __syncthreads();

    // rank-r product: acc[t][c] = 16 k x 16 n tile, 32 ranks per MFMA
    f32x4_t acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[t][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int js = 0; js < kSteps; ++js) {
        u32x4_t af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) af[t] = js < kPre ? apre[js < kPre ? js : 0][t] : a_frag(js, t);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            bf[c] = *reinterpret_cast<const lds_u32x4_t*>(bt + (js >> 1) * 8192 +
                                                          lds_off(16 * c + nl, ((js & 1) << 2) + q));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[t][c] = mfma16x16x32<F16>(__builtin_bit_cast(bf16x8_t, af[t]), __builtin_bit_cast(bf16x8_t, bf[c]),
                                              acc[t][c]);
    }

    // epilogue: lane holds k0 + 32 (t / 2) + 8q + 4 (t % 2) + v of row n0 + 16c + nl in acc[t][c][v]
    const float sc = p.s;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t n = n0 + 16 * c + nl;
        const float c1p = SQ ? __uint_as_float(s2[c]) : block_scale(f8[c], __uint_as_float(s2[c]));
        u32x4_t o[2];
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            // code byte bb of half hf = bb / 4: k 8q + 2 (bb % 4) (high nibble) and the next,
            // plus 32 in half 1; they sit in tile t = 2 hf + (bb % 4) / 2, rows v = 2 (bb % 2) .. +1
            const uint32_t byte = (cw[c][bb >> 2] >> (8 * (bb & 3))) & 0xFFu;
            const uint32_t wq = pack16x2<F16>(__fmul_rn(s_q[byte >> 4], c1p), __fmul_rn(s_q[byte & 15u], c1p));
            const int t = 2 * (bb >> 2) + ((bb & 3) >> 1), v = 2 * (bb & 1);
            const float m0 = fmaf(sc, acc[t][c][v], lo16<F16>(wq));
            const float m1 = fmaf(sc, acc[t][c][v + 1], hi16<F16>(wq));
            o[bb >> 2][bb & 3] = pack16x2<F16>(m0, m1);
        }
        // tile row 16c + nl, chunks (64 wave + 8 q) / 8 and 4 further
        const int row = 16 * c + nl;
        *reinterpret_cast<lds_u32x4_t*>((lds8_t*)s_out + mtile_off(row, 8 * wave + q)) = o[0];
        *reinterpret_cast<lds_u32x4_t*>((lds8_t*)s_out + mtile_off(row, 8 * wave + q + 4)) = o[1];
    }
    __syncthreads();
    // whole rows out: each wave store writes two rows of 512 contiguous bytes,
    // streamed once (non-temporal, so it does not displace A and B in the caches)
    const int64_t kt0 = (int64_t)kb * kMergeK;
#pragma unroll
    for (int it = 0; it < kMergeRows * 32 / 256; ++it) {
        const int u = (int)threadIdx.x + 256 * it;
        const int row = u >> 5, ch = u & 31;
        const int64_t n = n0 + row, k = kt0 + 8 * ch;
        if (n < p.N && k < p.K) {
            const u32x4_t v = *reinterpret_cast<const lds_u32x4_t*>((lds8_t*)s_out + mtile_off(row, ch));
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
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, s, a, cb); };
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
    return hipGetLastError();
}

}  // namespace ql
