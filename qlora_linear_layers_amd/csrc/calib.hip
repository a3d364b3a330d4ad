// Calibration kernels: the achievable HBM bandwidth and bf16 MFMA rate of the
// device, measured beside the layer's kernels so that their roofline
// fractions can be read against what the part delivers as well as against
// its published peaks.  Neither is part of the QLoRA path.
#include "qlora_calib.h"
#include "common.hpp"

namespace ql {
namespace {

// dst = src in 16-byte pieces.  Each workgroup copies one contiguous 16 KB
// span (every thread four 16-byte pieces 4 KB apart, all loads issued before
// the stores, nontemporal): measured on MI355X against grid-stride variants
// with 1-8 pieces per thread and 1024-16384 workgroups, whose scattered
// DRAM pages cost 15-30% of the rate.
constexpr int kCopyPieces = 4;
__global__ __launch_bounds__(256) void k_stream_copy(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                     int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * 256 * kCopyPieces + threadIdx.x;
    u32x4_t v[kCopyPieces];
#pragma unroll
    for (int u = 0; u < kCopyPieces; ++u) {
        const int64_t j = base + u * 256;
        v[u] = j < n16 ? __builtin_nontemporal_load(src + j) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kCopyPieces; ++u) {
        const int64_t j = base + u * 256;
        if (j < n16) __builtin_nontemporal_store(v[u], dst + j);
    }
}

// One wave per SIMD, each running 16 independent chains of
// v_mfma_f32_32x32x16_bf16 (32768 flops each) for `iters` rounds; the operands
// come from memory and the accumulators are summed into `out`, so nothing can
// be folded away.
constexpr int kChains = 16;
__global__ __launch_bounds__(256, 1) void k_mfma_loop(const uint32_t* __restrict__ seed, float* __restrict__ out,
                                                      int iters) {
    const int lane = threadIdx.x & 63;
    u32x4_t av, bv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        av[e] = seed[(lane + e) & 63];
        bv[e] = seed[64 + ((lane + 3 * e) & 63)];
    }
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av), b = __builtin_bit_cast(bf16x8_t, bv);
    f32x16_t acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace ql

extern "C" {

int qlora_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst) return QLORA_CALIB_ERR;
    if (bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return QLORA_CALIB_ERR;
    if (bytes > (size_t(1) << 44)) return QLORA_CALIB_ERR;   // the grid stays below 2^31 workgroups
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t grid = (n16 + 256 * ql::kCopyPieces - 1) / (256 * ql::kCopyPieces);
    hipLaunchKernelGGL(ql::k_stream_copy, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const ql::u32x4_t*>(src), static_cast<ql::u32x4_t*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : QLORA_CALIB_ERR;
}

double qlora_calib_mfma_flops(int workgroups, int iters) {
    return (double)workgroups * 4.0 * iters * ql::kChains * 32.0 * 32.0 * 16.0 * 2.0;
}

int qlora_calib_mfma(const uint32_t* seed, float* out, int workgroups, int iters, void* stream) {
    if (!seed || !out || workgroups < 1 || iters < 1) return QLORA_CALIB_ERR;
    hipLaunchKernelGGL(ql::k_mfma_loop, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       seed, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : QLORA_CALIB_ERR;
}

}  // extern "C"
