// NF4 quantization with double quantization, and double dequantization, for
// gfx950.  Both kernels are HBM-bound streams; they are written for 128-bit
// coalesced loads and stores and keep the codebook / encoder table in LDS.
//
// Method: "QLoRA 原理精讲" section 2.1 (absmax per block of 64, nearest of the 16
// NF4 codewords) and section 2.2 with its storage figure (the block constants
// quantized to FP8 in groups of 256 under one fp32 super-scale; dequantization
// in reverse order).
#include "common.hpp"
#include "plan.hpp"

namespace ql {

// -------------------------------------------------------------------- quantize
//
// One workgroup (4 wave64) per group of 256 blocks = 16384 bf16 (32 KB).  Thread
// t handles 16-byte chunk j*256 + t for j = 0..7, so the eight lanes of each
// 8-lane cluster hold one 64-element block; block absmax is an integer max of
// |bf16| bit patterns (order-preserving for non-negative values) across the
// cluster.  Encoding avoids a division: n = w * rcp(c1) has a relative error
// below 2^-22, while no ratio of two bf16 values lies closer than 2^-19.4
// (relative) to a decision midpoint, so comparing n with the round-down fp32
// midpoint gives the same code as the exact ratio.  Blocks whose c1 is outside
// [2^-64, 2^64] (where rcp could over/underflow) take correctly rounded
// division instead, which is the definition itself.
//
// SQ: single quantization (the first level alone): each block's fp32 absmax
// c1 is stored as it is and there is no second level.  EXACT: every ratio by
// correctly rounded division (the INT4 levels have exact midpoints such as
// 1/14 that ratios of bf16 values can reach, so the reciprocal shortcut does
// not hold for them).  F16: the weights are fp16 (11-bit significands, for
// which that argument does not hold either, so they take exact division too).
//
// A launch covers a group of tensors (one for the single-tensor entry points):
// workgroup ids are dealt to the tensors in order, `end` holding the
// cumulative workgroup ends.
template <bool SQ, bool EXACT, bool F16>
__global__ __launch_bounds__(256) void k_quantize(QuantGroup grp, EncodeTable tab) {
    __shared__ uint2 s_tab[34];
    __shared__ float s_c1[kGroup];
    __shared__ float s_wmax[4];

    const int ti = tensor_of(grp.end, grp.count, (int)blockIdx.x);
    const int gl = (int)blockIdx.x - (ti ? grp.end[ti - 1] : 0);        // group of 256 blocks within the tensor
    const uint16_t* __restrict__ w = grp.t[ti].w;
    const int64_t nblocks = grp.t[ti].numel / kBlock;
    uint8_t* __restrict__ codes = grp.t[ti].codes;
    uint8_t* __restrict__ fp8 = grp.t[ti].fp8;
    float* __restrict__ superscale = grp.t[ti].sup;
    float* __restrict__ absmax = grp.t[ti].absmax;

    const int tid = threadIdx.x;
    const int64_t blk0 = (int64_t)gl * kGroup;
    const int nb = (int)((nblocks - blk0) < kGroup ? (nblocks - blk0) : kGroup);
    if (tid < 34) s_tab[tid] = make_uint2(__float_as_uint(tab.thr[tid]), tab.base[tid]);
    const uint32_t tab_adj = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint2*)s_tab - 0x4B400000u * 8u;

    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w + blk0 * kBlock);
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int chunk = j * 256 + tid;
        v[j] = (chunk >> 3) < nb ? __builtin_nontemporal_load(src + chunk) : u32x4_t{0, 0, 0, 0};
    }
    __syncthreads();

    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + blk0 * (kBlock / 2));
    float gmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int chunk = j * 256 + tid;
        const int lb = chunk >> 3;
        const uint32_t d[4] = {v[j][0], v[j][1], v[j][2], v[j][3]};
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max(d[k] & 0x7FFFu, (d[k] >> 16) & 0x7FFFu));
        // max over the 8-lane cluster with DPP lane swaps (quad_perm [1,0,3,2],
        // [2,3,0,1], then row_half_mirror pairs each quad with the other)
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x141, 0xF, 0xF, false));
        // |w| bit patterns order like the values in both formats (sign-magnitude)
        const float c1 = F16 ? lo16<true>(m) : __uint_as_float(m << 16);
        const float r = c1 > 0.0f ? __builtin_amdgcn_rcpf(c1) : 0.0f;
        const bool exact = c1 != 0.0f && (EXACT || F16 || c1 < 0x1p-64f || c1 > 0x1p64f);

        float n[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = (e & 1) ? hi16<F16>(d[e >> 1]) : lo16<F16>(d[e >> 1]);
            n[e] = __fmul_rn(x, r);
        }
        if (__any(exact)) {
            if (exact) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (e & 1) ? hi16<F16>(d[e >> 1]) : lo16<F16>(d[e >> 1]);
                    n[e] = __fdiv_rn(x, c1);
                }
            }
        }
        uint32_t out = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // cell = round(16 n + 16): one fma against 1.5 * 2^23, whose ulp is 1,
            // leaves the rounded integer in the low mantissa bits; the table
            // entry's LDS address is 8 * (bits - bits(1.5 * 2^23)) + the table's
            // (|n| <= 1 + 2^-22 keeps the cell in [0, 32])
            const uint32_t vb = __float_as_uint(fmaf(n[e], 16.0f, 12582928.0f));
            const u32x2_t t = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(
                (uintptr_t)(vb * 8u + tab_adj));
            const uint32_t code = t[1] + (n[e] > __uint_as_float(t[0]) ? 1u : 0u);
            out |= code << ((e >> 1) * 8 + ((e & 1) ? 0 : 4));   // even element -> high nibble
        }
        if (lb < nb) {
            dst[chunk] = out;
            if ((tid & 7) == 0) {
                if constexpr (SQ) absmax[blk0 + lb] = c1;
                else s_c1[lb] = c1;
            }
        }
        gmax = fmaxf(gmax, c1);
    }
    if constexpr (SQ) return;                                 // uniform: no second level

    // Second level: group max -> fp32 super-scale, then one FP8 code per block.
    gmax = fmaxf(gmax, __shfl_xor(gmax, 8));
    gmax = fmaxf(gmax, __shfl_xor(gmax, 16));
    gmax = fmaxf(gmax, __shfl_xor(gmax, 32));
    if ((tid & 63) == 0) s_wmax[tid >> 6] = gmax;
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
    const float s2 = __fdiv_rn(amax, 448.0f);
    if (tid == 0) superscale[gl] = s2;
    if (tid < nb) {
        uint32_t code = 0;
        if (s2 > 0.0f) code = e4m3_encode_tie_low(fminf(__fdiv_rn(s_c1[tid], s2), 448.0f));
        fp8[blk0 + tid] = (uint8_t)code;
    }
}

hipError_t launch_quantize_group(const QuantTensor* ts, int count, hipStream_t s, bool f16) {
    if (count < 1 || count > kMaxTensors) return hipErrorInvalidValue;
    QuantGroup g{};
    int64_t wgs = 0;
    for (int i = 0; i < count; ++i) {
        g.t[i] = ts[i];
        wgs += ceil_div(ts[i].numel / kBlock, kGroup);
        if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
        g.end[i] = (int)wgs;
    }
    g.count = count;
    if (f16)
        hipLaunchKernelGGL((k_quantize<false, false, true>), dim3((unsigned)wgs), dim3(256), 0, s, g,
                           host_encode_table());
    else
        hipLaunchKernelGGL((k_quantize<false, false, false>), dim3((unsigned)wgs), dim3(256), 0, s, g,
                           host_encode_table());
    return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* w, int64_t numel, uint8_t* codes, uint8_t* fp8,
                           float* superscale, hipStream_t s, bool f16) {
    const QuantTensor t{w, numel, codes, fp8, superscale, nullptr, nullptr};
    return launch_quantize_group(&t, 1, s, f16);
}

hipError_t launch_quantize_sq(const uint16_t* w, int64_t numel, uint8_t* codes, float* absmax, hipStream_t s,
                              bool int4) {
    QuantGroup g{};
    g.t[0] = QuantTensor{w, numel, codes, nullptr, nullptr, absmax, nullptr};
    const int64_t wgs = ceil_div(numel / kBlock, kGroup);
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    g.end[0] = (int)wgs;
    g.count = 1;
    if (int4)
        hipLaunchKernelGGL((k_quantize<true, true, false>), dim3((unsigned)wgs), dim3(256), 0, s, g,
                           host_int4_encode_table());
    else
        hipLaunchKernelGGL((k_quantize<true, false, false>), dim3((unsigned)wgs), dim3(256), 0, s, g,
                           host_encode_table());
    return hipGetLastError();
}

// ------------------------------------------------------------------ dequantize
//
// Lane-contiguous streaming: each thread expands 4 packed bytes (8 codes) into
// one 16-byte bf16 store, so every wave-wide load and store instruction covers
// one contiguous span (256 B of codes in, 1 KB of bf16 out).  A thread handles
// kDeqUnits such units, 256 units apart, to keep several loads in flight.
// c1' = fl32(e4m3(f) * s2) per unit (single quantization: c1' = the stored
// fp32 absmax); w' = RNE_bf16(fl32(q[code] * c1')) per element with the
// codebook in LDS (16 floats: every lookup hits one of 16 distinct banks, so
// lookups never conflict).
constexpr int kDeqUnits = 4;
constexpr unsigned kDeqEarlyTableWgs = 4096;   // two rounds of 8 workgroups on each of 256 CUs

template <bool SQ, bool F16>
__global__ __launch_bounds__(256) void k_dequantize(QuantGroup grp, Codebook cb) {
    __shared__ float s_q[16];
    const int ti = tensor_of(grp.end, grp.count, (int)blockIdx.x);
    const int64_t gl = (int)blockIdx.x - (ti ? grp.end[ti - 1] : 0);    // workgroup within the tensor
    const uint32_t* __restrict__ codes = reinterpret_cast<const uint32_t*>(grp.t[ti].codes);
    const uint8_t* __restrict__ fp8 = grp.t[ti].fp8;
    const float* __restrict__ superscale = grp.t[ti].sup;
    const float* __restrict__ absmax = grp.t[ti].absmax;
    const int64_t nunits = grp.t[ti].numel / 8;
    u32x4_t* __restrict__ out = reinterpret_cast<u32x4_t*>(grp.t[ti].out);
    auto fill_table = [&] {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (threadIdx.x == j) s_q[j] = cb_value(cb, j);  // constant indexes: no memory round trip
    };
    // The barrier's fence waits for the loads issued before it.  A launch of
    // several rounds of workgroups fills the table and passes the barrier
    // first, so that unit 0 is expanded while the other loads are in flight;
    // a one-round launch issues its loads first, since there the barrier would
    // delay every load of the launch (uniform over the grid).
    const bool early = gridDim.x >= kDeqEarlyTableWgs;
    if (early) {
        fill_table();
        __syncthreads();
    }

    const int64_t u0 = gl * (256 * kDeqUnits) + threadIdx.x;
    uint32_t cv[kDeqUnits];
    uint32_t f8[kDeqUnits];
    float s2[kDeqUnits];
#pragma unroll
    for (int u = 0; u < kDeqUnits; ++u) {
        const int64_t i = u0 + u * 256;
        const int64_t ii = i < nunits ? i : 0;
        cv[u] = __builtin_nontemporal_load(codes + ii);
        const int64_t blk = ii >> 3;                      // 8 units of 8 codes per block
        if constexpr (SQ) {
            f8[u] = 0;
            s2[u] = absmax[blk];
        } else {
            f8[u] = fp8[blk];
            s2[u] = superscale[blk >> 8];
        }
    }
    if (!early) {
        fill_table();
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < kDeqUnits; ++u) {
        const int64_t i = u0 + u * 256;
        if (i >= nunits) continue;
        const float c1p = SQ ? s2[u] : __fmul_rn(e4m3_decode(f8[u]), s2[u]);
        u32x4_t o;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t byte = (cv[u] >> (8 * b)) & 0xFFu;
            o[b] = pack16x2<F16>(__fmul_rn(s_q[byte >> 4], c1p), __fmul_rn(s_q[byte & 15u], c1p));
        }
        __builtin_nontemporal_store(o, out + i);
    }
}

hipError_t launch_dequantize_group(const QuantTensor* ts, int count, hipStream_t s, bool int4, bool f16) {
    if (count < 1 || count > kMaxTensors) return hipErrorInvalidValue;
    const Codebook& cb = int4 ? host_int4_codebook() : host_codebook();
    QuantGroup g{};
    int64_t wgs = 0;
    const int64_t per_wg = 256 * kDeqUnits;
    for (int i = 0; i < count; ++i) {
        g.t[i] = ts[i];
        wgs += ceil_div(ts[i].numel / 8, per_wg);
        if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
        g.end[i] = (int)wgs;
    }
    g.count = count;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(256), 0, s, g, cb); };
    const bool sq = ts[0].absmax != nullptr;
    if (sq) f16 ? go(k_dequantize<true, true>) : go(k_dequantize<true, false>);
    else f16 ? go(k_dequantize<false, true>) : go(k_dequantize<false, false>);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, BlockScales sc, int64_t numel, uint16_t* out, hipStream_t s,
                             bool int4, bool f16) {
    const QuantTensor t{nullptr, numel, const_cast<uint8_t*>(codes), const_cast<uint8_t*>(sc.fp8),
                        const_cast<float*>(sc.sup), const_cast<float*>(sc.absmax), out};
    return launch_dequantize_group(&t, 1, s, int4, f16);
}

}  // namespace ql
