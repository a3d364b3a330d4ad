// extern "C" entry points declared in include/qlora.h: host-side validation,
// workspace carving and kernel sequencing.  No device memory is allocated
// here; every buffer comes from the caller.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "qlora.h"
#include "common.hpp"
#include "grad.hpp"
#include "plan.hpp"

namespace ql {
hipError_t launch_transpose_a(const uint16_t* lora_a, const LoraPlan& pl, uint8_t* ws, hipStream_t s);
hipError_t launch_lora_down_x(const uint16_t* x, float scaling, const LoraPlan& pl, uint8_t* ws, bool transposed,
                              hipStream_t s, bool f16);
hipError_t launch_lora_down_dy(const uint16_t* dy, const uint16_t* lora_b, float scaling, const LoraPlan& pl,
                               uint8_t* ws, bool transposed, hipStream_t s, bool f16, const ScalesJob* scales);
hipError_t launch_fwd(const uint16_t* x, const uint8_t* codes, BlockScales sc, const uint16_t* lora_b,
                      const LoraPlan& pl, const uint8_t* ws, uint16_t* y, hipStream_t s, bool f16);
hipError_t launch_dx(const uint16_t* dy, const uint8_t* codes, BlockScales sc, const uint16_t* lora_a,
                     const LoraPlan& pl, const uint8_t* ws, uint16_t* dx, hipStream_t s, bool f16,
                     bool scales_ready, const FusedGrads* fused);
hipError_t launch_lora_grads(const uint16_t* x, const uint16_t* dy, const LoraPlan& pl, uint8_t* ws,
                             uint16_t* d_lora_a, uint16_t* d_lora_b, hipStream_t s, bool f16);
FusedGrads fused_grads_for(const uint16_t* x, const uint16_t* dy, const LoraPlan& pl, uint8_t* ws, bool da,
                           bool db);
hipError_t launch_fused_grads_finalize(const LoraPlan& pl, uint8_t* ws, uint16_t* d_lora_a, uint16_t* d_lora_b,
                                       hipStream_t s, bool f16);
}  // namespace ql

static_assert(QLORA_MAX_GROUP == ql::kMaxGroup, "group size of the header and the kernels");
static_assert(QLORA_GROUPED_MAX_T == ql::kGemvMaxT, "decode token limit of the header and the kernels");
static_assert(QLORA_MAX_TENSORS == ql::kMaxTensors, "tensor group size of the header and the kernels");

namespace {

// Largest element count of one quantized tensor: the dequantizer's grid
// (one workgroup per 8192 weights) then stays below 2^31 workgroups.
constexpr int64_t kMaxNumel = int64_t(1) << 43;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dev(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_DEVICE; }

// Workspace of a chunked forward (kGemvMaxT < T <= kChunkMaxT): one decode
// workspace per kGemvMaxT-token window of the grouped launch.
static_assert(ql::kChunkMaxT / ql::kGemvMaxT <= ql::kMaxGroup, "the windows fit one grouped launch");
size_t chunked_workspace(int64_t T, int64_t K, int64_t N, int64_t r_pad) {
    const int64_t windows = (T + ql::kGemvMaxT - 1) / ql::kGemvMaxT;
    return (size_t)windows * ql::gemv_workspace(ql::kGemvMaxT, K, N, r_pad);
}

// Shape rules shared by the linear entry points.  The GEMM kernels address
// each operand with 32-bit buffer offsets, so every operand stays below 2 GiB.
int check_linear_shape(int64_t T, int64_t K, int64_t N, int64_t r) {
    if (T < 1 || K < 64 || N < 64 || K % 64 || N % 64) return QLORA_ERR_SHAPE;
    if (r < 0 || r > QLORA_MAX_RANK || (r > 0 && r % 8)) return QLORA_ERR_SHAPE;
    if (T > (int64_t(1) << 22) || K > (int64_t(1) << 20) || N > (int64_t(1) << 20)) return QLORA_ERR_SHAPE;
    if (T * K > (int64_t(1) << 30) || T * N > (int64_t(1) << 30) || N * K >= (int64_t(1) << 32))
        return QLORA_ERR_SHAPE;
    return QLORA_OK;
}

// Block constants as the entry points receive them: the double-quantized pair
// or (for the _sq entry points) one fp32 absmax per block.  A missing array is
// a NULL error; a present one must be 16-byte aligned like every pointer.
ql::BlockScales dq_scales(const uint8_t* fp8, const float* sup) { return {fp8, sup, nullptr}; }
ql::BlockScales sq_scales(const float* absmax) { return {nullptr, nullptr, absmax}; }
bool scales_present(const ql::BlockScales& sc) { return sc.absmax || (sc.fp8 && sc.sup); }
bool scales_aligned(const ql::BlockScales& sc) {
    return (!sc.fp8 || aligned16(sc.fp8)) && (!sc.sup || aligned16(sc.sup)) && (!sc.absmax || aligned16(sc.absmax));
}

int dequantize_impl(const uint8_t* codes, ql::BlockScales sc, int64_t numel, uint16_t* w_out, void* stream,
                    bool int4 = false, bool f16 = false) {
    if (!codes || !scales_present(sc) || !w_out) return QLORA_ERR_NULL;
    if (numel <= 0 || numel % 64 || numel > kMaxNumel) return QLORA_ERR_SHAPE;
    if (!aligned16(w_out) || !aligned16(codes) || !scales_aligned(sc)) return QLORA_ERR_ALIGN;
    return dev(ql::launch_dequantize(codes, sc, numel, w_out, static_cast<hipStream_t>(stream), int4, f16));
}

int quantize_sq_impl(const uint16_t* w, int64_t numel, uint8_t* codes, float* absmax, void* stream, bool int4) {
    if (!w || !codes || !absmax) return QLORA_ERR_NULL;
    if (numel <= 0 || numel % 64 || numel > kMaxNumel) return QLORA_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax)) return QLORA_ERR_ALIGN;
    return dev(ql::launch_quantize_sq(w, numel, codes, absmax, static_cast<hipStream_t>(stream), int4));
}

// Argument checks of the forward (everything but the workspace).
int fwd_check(const uint16_t* x, int64_t T, int64_t K, int64_t N, const uint8_t* codes, ql::BlockScales sc,
              const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling, const uint16_t* y) {
    if (!x || !codes || !scales_present(sc) || !y) return QLORA_ERR_NULL;
    if (r > 0 && (!lora_a || !lora_b)) return QLORA_ERR_NULL;
    if (int st = check_linear_shape(T, K, N, r)) return st;
    if (r == 0 && (lora_a || lora_b)) return QLORA_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(codes) || !scales_aligned(sc) || !aligned16(y) ||
        (lora_a && !aligned16(lora_a)) || (lora_b && !aligned16(lora_b)))
        return QLORA_ERR_ALIGN;
    if (!std::isfinite(scaling)) return QLORA_ERR_VALUE;
    return QLORA_OK;
}

// Workspace bytes of one forward call (sizes already checked); `cap` limits
// the split-k partials of the tile GEMM as in LoraPlan.
size_t fwd_workspace(int64_t T, int64_t K, int64_t N, int64_t r, size_t cap = SIZE_MAX) {
    const ql::LoraPlan pl(T, K, N, r, cap);
    if (T <= ql::kGemvMaxT) return ql::gemv_workspace(T, K, N, pl.r_pad);
    if (T <= ql::kChunkMaxT) return chunked_workspace(T, K, N, pl.r_pad);
    return pl.fwd_bytes;
}

int fwd_impl(const uint16_t* x, int64_t T, int64_t K, int64_t N, const uint8_t* codes, ql::BlockScales sc,
             const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling, uint16_t* y, void* workspace,
             size_t workspace_bytes, void* stream, bool f16 = false, size_t cap = SIZE_MAX) {
    if (int st = fwd_check(x, T, K, N, codes, sc, lora_a, lora_b, r, scaling, y)) return st;
    if (workspace && !aligned16(workspace)) return QLORA_ERR_ALIGN;
    const ql::LoraPlan pl(T, K, N, r, cap);
    const bool chunked = T > ql::kGemvMaxT && T <= ql::kChunkMaxT;
    const size_t need = fwd_workspace(T, K, N, r, cap);
    if (need && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (T <= ql::kGemvMaxT)      // decode sizes: small-M MFMA, split-k partials
        return dev(ql::launch_gemv(x, codes, sc, lora_a, lora_b, scaling, pl, ws, y, s, f16));
    if (chunked) {
        // small prefill: kGemvMaxT-token windows as the problems of one grouped
        // decode launch pair (they share the weight).  Window c starts at token
        // min(16 c, T - 16), so every window is full; the last one overlaps its
        // predecessor, computes those rows identically and skips writing them.
        const int64_t windows = (T + ql::kGemvMaxT - 1) / ql::kGemvMaxT;
        ql::GemvProblem g[ql::kMaxGroup];
        for (int64_t c = 0; c < windows; ++c) {
            const int64_t t0 = std::min<int64_t>(c * ql::kGemvMaxT, T - ql::kGemvMaxT);
            g[c] = ql::GemvProblem{x + t0 * K, codes, sc, lora_a, lora_b, scaling, K, N, y + t0 * N,
                                   c * ql::kGemvMaxT - t0};
        }
        return dev(ql::launch_gemv_group(g, (int)windows, ql::kGemvMaxT, r, ws, s, f16));
    }
    if (r > 0) {
        if (int st = dev(ql::launch_transpose_a(lora_a, pl, ws, s))) return st;
        // s X A in both layouts: the transposed copy lets a backward with
        // QLORA_BWD_REUSE_FORWARD take the adapter gradients without recomputing it
        if (int st = dev(ql::launch_lora_down_x(x, scaling, pl, ws, true, s, f16))) return st;
    }
    return dev(ql::launch_fwd(x, codes, sc, lora_b, pl, ws, y, s, f16));
}

int bwd_impl(const uint16_t* dy, int64_t T, int64_t K, int64_t N, const uint8_t* codes, ql::BlockScales sc,
             const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling, uint16_t* dx, const uint16_t* x,
             uint16_t* d_lora_a, uint16_t* d_lora_b, void* workspace, size_t workspace_bytes, unsigned flags,
             void* stream, bool f16 = false) {
    if (!dy || !codes || !scales_present(sc) || !dx) return QLORA_ERR_NULL;
    if (r > 0 && (!lora_a || !lora_b)) return QLORA_ERR_NULL;
    const bool grads = d_lora_a || d_lora_b;
    if (grads && !x) return QLORA_ERR_NULL;
    if (int st = check_linear_shape(T, K, N, r)) return st;
    if (r == 0 && (lora_a || lora_b || grads)) return QLORA_ERR_SHAPE;
    if (!scales_aligned(sc)) return QLORA_ERR_ALIGN;
    const void* ptrs[] = {dy, codes, dx, x, lora_a, lora_b, d_lora_a, d_lora_b, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return QLORA_ERR_ALIGN;
    if (!std::isfinite(scaling)) return QLORA_ERR_VALUE;
    if (flags & ~(unsigned)(QLORA_BWD_REUSE_FORWARD | QLORA_BWD_FUSED_GRADS)) return QLORA_ERR_VALUE;
    const ql::LoraPlan pl(T, K, N, r);
    const bool fused = grads && (flags & QLORA_BWD_FUSED_GRADS);
    // > 0 in every case: the scale pre-pass needs room
    const size_t need = grads ? (fused ? pl.bwd_fused_bytes : pl.bwd_grad_bytes) : pl.bwd_bytes;
    // s X A from the forward's workspace (only the MFMA forward, T > kChunkMaxT, leaves it there)
    const bool reuse = (flags & QLORA_BWD_REUSE_FORWARD) && T > ql::kChunkMaxT;
    if (need && (!workspace || workspace_bytes < need)) return QLORA_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (r > 0) {
        // s dY B^T, with the dX kernel's block scales as extra workgroups of the same launch
        const ql::ScalesJob sj = ql::scales_job_for(sc, pl, ws);
        if (int st = dev(ql::launch_lora_down_dy(dy, lora_b, scaling, pl, ws, grads, s, f16, &sj))) return st;
    }
    // s X A (both layouts) for dB when the forward's is not reused
    auto recompute_p = [&]() -> int {
        if (int st = dev(ql::launch_transpose_a(lora_a, pl, ws, s))) return st;
        return dev(ql::launch_lora_down_x(x, scaling, pl, ws, true, s, f16));
    };
    if (fused) {
        // dX, and the gradient partials of each 256-token tile, from one k_dx launch
        if (!reuse)
            if (int st = recompute_p()) return st;
        const ql::FusedGrads fz = ql::fused_grads_for(x, dy, pl, ws, d_lora_a != nullptr, d_lora_b != nullptr);
        if (int st = dev(ql::launch_dx(dy, codes, sc, lora_a, pl, ws, dx, s, f16, true, &fz))) return st;
        return dev(ql::launch_fused_grads_finalize(pl, ws, d_lora_a, d_lora_b, s, f16));
    }
    if (int st = dev(ql::launch_dx(dy, codes, sc, lora_a, pl, ws, dx, s, f16, r > 0, nullptr))) return st;
    if (grads) {
        if (!reuse)
            if (int st = recompute_p()) return st;
        if (int st = dev(ql::launch_lora_grads(x, dy, pl, ws, d_lora_a, d_lora_b, s, f16))) return st;
    }
    return QLORA_OK;
}

int merge_impl(const uint8_t* codes, ql::BlockScales sc, int64_t K, int64_t N, const uint16_t* lora_a,
               const uint16_t* lora_b, int64_t r, float scaling, uint16_t* w_out, void* stream, bool f16 = false) {
    if (!codes || !scales_present(sc) || !w_out) return QLORA_ERR_NULL;
    if (r > 0 && (!lora_a || !lora_b)) return QLORA_ERR_NULL;
    if (K < 64 || K % 64 || N < 8 || N % 8 || K > (int64_t(1) << 20) || N > (int64_t(1) << 20) || N * K >= (int64_t(1) << 32))
        return QLORA_ERR_SHAPE;
    if (r < 0 || r > QLORA_MAX_RANK || r % 8 || (r == 0 && (lora_a || lora_b))) return QLORA_ERR_SHAPE;
    if (!scales_aligned(sc)) return QLORA_ERR_ALIGN;
    const void* ptrs[] = {codes, lora_a, lora_b, w_out};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return QLORA_ERR_ALIGN;
    if (!std::isfinite(scaling)) return QLORA_ERR_VALUE;
    return dev(ql::launch_merge(codes, sc, lora_a, lora_b, K, N, r, scaling, w_out, static_cast<hipStream_t>(stream),
                                f16));
}

// Host checks of one grouped decode problem (the rules of fwd_impl).
int check_problem(const qlora_linear_problem& q, int64_t T, int64_t r) {
    if (!q.x || !q.codes || !q.absmax_fp8 || !q.superscale || !q.y) return QLORA_ERR_NULL;
    if (r > 0 && (!q.lora_a || !q.lora_b)) return QLORA_ERR_NULL;
    if (int st = check_linear_shape(T, q.K, q.N, r)) return st;
    if (r == 0 && (q.lora_a || q.lora_b)) return QLORA_ERR_SHAPE;
    const void* ptrs[] = {q.x, q.codes, q.absmax_fp8, q.superscale, q.lora_a, q.lora_b, q.y};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return QLORA_ERR_ALIGN;
    if (!std::isfinite(q.scaling)) return QLORA_ERR_VALUE;
    return QLORA_OK;
}

int grouped_problems(int count, const qlora_linear_problem* problems, int64_t T, int64_t r,
                     ql::GemvProblem* out) {
    if (!problems) return QLORA_ERR_NULL;
    if (count < 1 || count > QLORA_MAX_GROUP || T < 1 || T > QLORA_GROUPED_MAX_T) return QLORA_ERR_SHAPE;
    for (int i = 0; i < count; ++i) {
        const qlora_linear_problem& q = problems[i];
        if (int st = check_problem(q, T, r)) return st;
        out[i] = ql::GemvProblem{q.x, q.codes, dq_scales(q.absmax_fp8, q.superscale), q.lora_a, q.lora_b, q.scaling,
                                 q.K, q.N, q.y};
    }
    return QLORA_OK;
}

// Host checks of a grouped quantize / dequantize (the rules of the single
// calls, per tensor), filling the kernel descriptors.
int grouped_tensors(int count, const nf4_tensor* tensors, ql::QuantTensor* out) {
    if (!tensors) return QLORA_ERR_NULL;
    if (count < 1 || count > QLORA_MAX_TENSORS) return QLORA_ERR_SHAPE;
    int64_t wgs = 0;
    for (int i = 0; i < count; ++i) {
        const nf4_tensor& t = tensors[i];
        if (!t.w || !t.codes || !t.absmax_fp8 || !t.superscale) return QLORA_ERR_NULL;
        if (t.numel <= 0 || t.numel % 64 || t.numel > kMaxNumel) return QLORA_ERR_SHAPE;
        if (!aligned16(t.w) || !aligned16(t.codes) || !aligned16(t.absmax_fp8) || !aligned16(t.superscale))
            return QLORA_ERR_ALIGN;
        // the larger of the two launches' workgroup counts (groups of 256 blocks; 8192 weights)
        wgs += ql::ceil_div(t.numel, 8192);
        if (wgs > 0x7FFFFFFF) return QLORA_ERR_SHAPE;
        out[i] = ql::QuantTensor{t.w, t.numel, t.codes, t.absmax_fp8, t.superscale, nullptr, t.w};
    }
    return QLORA_OK;
}

int quantize_dq_impl(const uint16_t* w, int64_t numel, uint8_t* codes, uint8_t* absmax_fp8, float* superscale,
                     void* stream, bool f16) {
    if (!w || !codes || !absmax_fp8 || !superscale) return QLORA_ERR_NULL;
    if (numel <= 0 || numel % 64 || numel > kMaxNumel) return QLORA_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(absmax_fp8) || !aligned16(superscale))
        return QLORA_ERR_ALIGN;
    return dev(ql::launch_quantize(w, numel, codes, absmax_fp8, superscale, static_cast<hipStream_t>(stream), f16));
}

// ------------------------------------------------------------ no-allocation forward
//
// qlora_linear_fwd_noalloc takes its workspace from this file-scope device
// array instead of the caller.  Host code never passes the array's name to a
// kernel or a copy (on the host it is only a stand-in for the symbol): the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept below.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_of_current_device(void** out) {
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kMaxDevices) return QLORA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[d]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_ERR_DEVICE;
        g_scratch[d] = p;
    }
    *out = g_scratch[d];
    return QLORA_OK;
}

}  // namespace

extern "C" {

size_t qlora_noalloc_scratch_bytes(void) { return kScratchBytes; }

int qlora_linear_fwd_noalloc(const uint16_t* x, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                             const uint8_t* absmax_fp8, const float* superscale, const uint16_t* lora_a,
                             const uint16_t* lora_b, int64_t r, float scaling, uint16_t* y, void* stream) {
    const ql::BlockScales sc = dq_scales(absmax_fp8, superscale);
    if (int st = fwd_check(x, T, K, N, codes, sc, lora_a, lora_b, r, scaling, y)) return st;
    // the tile GEMM's split-k partials are held to what the scratch leaves
    const size_t need = fwd_workspace(T, K, N, r, kScratchBytes);
    if (need > kScratchBytes) return QLORA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need)
        if (int st = scratch_of_current_device(&ws)) return st;
    return fwd_impl(x, T, K, N, codes, sc, lora_a, lora_b, r, scaling, y, ws, kScratchBytes, stream, false,
                    kScratchBytes);
}

const char* qlora_status_string(int status) {
    switch (status) {
        case QLORA_OK: return "ok";
        case QLORA_ERR_NULL: return "a required pointer is NULL";
        case QLORA_ERR_SHAPE: return "a size is out of range";
        case QLORA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case QLORA_ERR_VALUE: return "a scalar argument is not finite";
        case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
        case QLORA_ERR_DEVICE: return "HIP runtime error";
        default: return "unknown status";
    }
}

int nf4_build_codebook(float codebook_out[16]) {
    if (!codebook_out) return QLORA_ERR_NULL;
    const ql::Codebook& cb = ql::host_codebook();
    for (int i = 0; i < 16; ++i) codebook_out[i] = cb.q[i];
    return QLORA_OK;
}

int nf4_quantize_dq(const uint16_t* w, int64_t numel, uint8_t* codes, uint8_t* absmax_fp8, float* superscale,
                    void* stream) {
    return quantize_dq_impl(w, numel, codes, absmax_fp8, superscale, stream, false);
}

int nf4_quantize_dq_f16(const uint16_t* w, int64_t numel, uint8_t* codes, uint8_t* absmax_fp8, float* superscale,
                        void* stream) {
    return quantize_dq_impl(w, numel, codes, absmax_fp8, superscale, stream, true);
}

int nf4_dequantize_dq(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale, int64_t numel,
                      uint16_t* w_out, void* stream) {
    return dequantize_impl(codes, dq_scales(absmax_fp8, superscale), numel, w_out, stream);
}

int nf4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes, float* absmax, void* stream) {
    return quantize_sq_impl(w, numel, codes, absmax, stream, false);
}

int int4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes, float* absmax, void* stream) {
    return quantize_sq_impl(w, numel, codes, absmax, stream, true);
}

int int4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, uint16_t* w_out, void* stream) {
    return dequantize_impl(codes, sq_scales(absmax), numel, w_out, stream, true);
}

int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t numel, uint16_t* w_out, void* stream) {
    return dequantize_impl(codes, sq_scales(absmax), numel, w_out, stream);
}

size_t qlora_workspace_bytes(int64_t T, int64_t K, int64_t N, int64_t r) {
    if (check_linear_shape(T, K, N, r) != QLORA_OK) return 0;
    const ql::LoraPlan pl(T, K, N, r);
    const size_t f = fwd_workspace(T, K, N, r);
    return f > pl.bwd_grad_bytes ? f : pl.bwd_grad_bytes;
}

size_t qlora_workspace_bytes_bwd(int64_t T, int64_t K, int64_t N, int64_t r, unsigned flags) {
    if (check_linear_shape(T, K, N, r) != QLORA_OK) return 0;
    if (flags & ~(unsigned)(QLORA_BWD_REUSE_FORWARD | QLORA_BWD_FUSED_GRADS)) return 0;
    const ql::LoraPlan pl(T, K, N, r);
    const size_t b = (flags & QLORA_BWD_FUSED_GRADS) ? pl.bwd_fused_bytes : pl.bwd_grad_bytes;
    const size_t f = fwd_workspace(T, K, N, r);
    return b > f ? b : f;
}

size_t qlora_workspace_bytes_upto(int64_t T_max, int64_t K, int64_t N, int64_t r) {
    if (check_linear_shape(T_max, K, N, r) != QLORA_OK) return 0;
    // the size peaks in the decode and window range (T <= kChunkMaxT) and
    // wherever a split-k forward keeps partial tiles (a grid of fewer than
    // 256 tiles: T < 65536); beyond that it grows with T
    size_t n = qlora_workspace_bytes(T_max, K, N, r);
    for (int64_t T = 1; T <= std::min<int64_t>(T_max, 65536); ++T) {
        const size_t m = qlora_workspace_bytes(T, K, N, r);
        if (m > n) n = m;
    }
    return n;
}

int qlora_linear_fwd(const uint16_t* x, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                     const uint8_t* absmax_fp8, const float* superscale, const uint16_t* lora_a,
                     const uint16_t* lora_b, int64_t r, float scaling, uint16_t* y, void* workspace,
                     size_t workspace_bytes, void* stream) {
    return fwd_impl(x, T, K, N, codes, dq_scales(absmax_fp8, superscale), lora_a, lora_b, r, scaling, y, workspace,
                    workspace_bytes, stream);
}

int qlora_linear_fwd_sq(const uint16_t* x, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                        const float* absmax, const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                        float scaling, uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_impl(x, T, K, N, codes, sq_scales(absmax), lora_a, lora_b, r, scaling, y, workspace,
                    workspace_bytes, stream);
}

int qlora_linear_bwd_input(const uint16_t* dy, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                           const uint8_t* absmax_fp8, const float* superscale, const uint16_t* lora_a,
                           const uint16_t* lora_b, int64_t r, float scaling, uint16_t* dx, const uint16_t* x,
                           uint16_t* d_lora_a, uint16_t* d_lora_b, void* workspace, size_t workspace_bytes,
                           unsigned flags, void* stream) {
    return bwd_impl(dy, T, K, N, codes, dq_scales(absmax_fp8, superscale), lora_a, lora_b, r, scaling, dx, x,
                    d_lora_a, d_lora_b, workspace, workspace_bytes, flags, stream);
}

int qlora_linear_bwd_input_sq(const uint16_t* dy, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                              const float* absmax, const uint16_t* lora_a, const uint16_t* lora_b, int64_t r,
                              float scaling, uint16_t* dx, const uint16_t* x, uint16_t* d_lora_a,
                              uint16_t* d_lora_b, void* workspace, size_t workspace_bytes, unsigned flags,
                              void* stream) {
    return bwd_impl(dy, T, K, N, codes, sq_scales(absmax), lora_a, lora_b, r, scaling, dx, x, d_lora_a, d_lora_b,
                    workspace, workspace_bytes, flags, stream);
}

int qlora_merge_lora(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale, int64_t K, int64_t N,
                     const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling, uint16_t* w_out,
                     void* stream) {
    return merge_impl(codes, dq_scales(absmax_fp8, superscale), K, N, lora_a, lora_b, r, scaling, w_out, stream);
}

int qlora_merge_lora_sq(const uint8_t* codes, const float* absmax, int64_t K, int64_t N, const uint16_t* lora_a,
                        const uint16_t* lora_b, int64_t r, float scaling, uint16_t* w_out, void* stream) {
    return merge_impl(codes, sq_scales(absmax), K, N, lora_a, lora_b, r, scaling, w_out, stream);
}

int nf4_dequantize_dq_f16(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale, int64_t numel,
                          uint16_t* w_out, void* stream) {
    return dequantize_impl(codes, dq_scales(absmax_fp8, superscale), numel, w_out, stream, false, true);
}

int qlora_linear_fwd_f16(const uint16_t* x, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                         const uint8_t* absmax_fp8, const float* superscale, const uint16_t* lora_a,
                         const uint16_t* lora_b, int64_t r, float scaling, uint16_t* y, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return fwd_impl(x, T, K, N, codes, dq_scales(absmax_fp8, superscale), lora_a, lora_b, r, scaling, y, workspace,
                    workspace_bytes, stream, true);
}

int qlora_linear_bwd_input_f16(const uint16_t* dy, int64_t T, int64_t K, int64_t N, const uint8_t* codes,
                               const uint8_t* absmax_fp8, const float* superscale, const uint16_t* lora_a,
                               const uint16_t* lora_b, int64_t r, float scaling, uint16_t* dx, const uint16_t* x,
                               uint16_t* d_lora_a, uint16_t* d_lora_b, void* workspace, size_t workspace_bytes,
                               unsigned flags, void* stream) {
    return bwd_impl(dy, T, K, N, codes, dq_scales(absmax_fp8, superscale), lora_a, lora_b, r, scaling, dx, x,
                    d_lora_a, d_lora_b, workspace, workspace_bytes, flags, stream, true);
}

int qlora_merge_lora_f16(const uint8_t* codes, const uint8_t* absmax_fp8, const float* superscale, int64_t K,
                         int64_t N, const uint16_t* lora_a, const uint16_t* lora_b, int64_t r, float scaling,
                         uint16_t* w_out, void* stream) {
    return merge_impl(codes, dq_scales(absmax_fp8, superscale), K, N, lora_a, lora_b, r, scaling, w_out, stream,
                      true);
}

int nf4_quantize_dq_grouped(int count, const nf4_tensor* tensors, void* stream) {
    ql::QuantTensor t[ql::kMaxTensors];
    if (int st = grouped_tensors(count, tensors, t)) return st;
    return dev(ql::launch_quantize_group(t, count, static_cast<hipStream_t>(stream), false));
}

int nf4_dequantize_dq_grouped(int count, const nf4_tensor* tensors, void* stream) {
    ql::QuantTensor t[ql::kMaxTensors];
    if (int st = grouped_tensors(count, tensors, t)) return st;
    return dev(ql::launch_dequantize_group(t, count, static_cast<hipStream_t>(stream), false, false));
}

size_t qlora_grouped_workspace_bytes(int count, const qlora_linear_problem* problems, int64_t T, int64_t r) {
    ql::GemvProblem g[ql::kMaxGroup];
    if (grouped_problems(count, problems, T, r, g) != QLORA_OK) return 0;
    return ql::gemv_group_workspace(g, count, T, r > 0 ? ql::ceil_div(r, 64) * 64 : 0);
}

int qlora_linear_fwd_grouped_ex(int count, const qlora_linear_problem* problems, int64_t T, int64_t r,
                                unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
    ql::GemvProblem g[ql::kMaxGroup];
    if (int st = grouped_problems(count, problems, T, r, g)) return st;
    ql::DecodeProduct prod = ql::DecodeProduct::Auto;
    if (flags == QLORA_DECODE_MFMA) prod = ql::DecodeProduct::Mfma;
    else if (flags == QLORA_DECODE_VALU) prod = ql::DecodeProduct::Valu;
    else if (flags != 0) return QLORA_ERR_VALUE;
    if (prod == ql::DecodeProduct::Valu && T > ql::kGemvValuMaxT) return QLORA_ERR_VALUE;
    if (workspace && !aligned16(workspace)) return QLORA_ERR_ALIGN;
    const size_t need = ql::gemv_group_workspace(g, count, T, r > 0 ? ql::ceil_div(r, 64) * 64 : 0);
    if (!workspace || workspace_bytes < need) return QLORA_ERR_WORKSPACE;
    return dev(ql::launch_gemv_group(g, count, T, r, static_cast<uint8_t*>(workspace),
                                     static_cast<hipStream_t>(stream), false, prod));
}

int qlora_linear_fwd_grouped(int count, const qlora_linear_problem* problems, int64_t T, int64_t r,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return qlora_linear_fwd_grouped_ex(count, problems, T, r, 0u, workspace, workspace_bytes, stream);
}

}  // extern "C"
