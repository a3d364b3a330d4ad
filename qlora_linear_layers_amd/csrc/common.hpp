// Shared device helpers and host-side launch declarations for the gfx950
// QLoRA library.  Everything here is written for CDNA4 (wave64, MFMA, 160 KB
// LDS); there is no other target.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define QL_DEV __device__ __forceinline__

namespace ql {

constexpr int kBlock = 64;    // weights per NF4 block
constexpr int kGroup = 256;   // blocks per fp32 super-scale

// The 16 NF4 codewords (fp32, ascending; index = code).  Passed to kernels by
// value as a kernel argument and copied to LDS at kernel start.
struct Codebook {
    float q[16];
};

// Encoder lookup over n in [-1, 1]: cell = round(16 n + 16) in [0, 32]; the
// code is base[cell] + (n > thr[cell]), base[cell] counting the midpoints
// below the cell.  Each cell of width 1/16 holds at most one decision midpoint
// (neighbouring midpoints are >= 0.08 apart), whose round-down fp32 value is
// thr[cell] (cells without one carry thr = 2).  A value exactly on a cell's
// lower edge may be sent to the cell below (ties to even); the lookup there
// gives the same code.
struct EncodeTable {
    float thr[34];
    uint32_t base[34];
};

// Host: the library's codebook and encoder table (computed once, thread-safe).
const Codebook& host_codebook();
const EncodeTable& host_encode_table();
// INT4 absmax levels (i - 8) / 7 and their encoder table (data-type ablation)
const Codebook& host_int4_codebook();
const EncodeTable& host_int4_encode_table();

// ------------------------------------------------------------------ bf16

QL_DEV float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
QL_DEV float bf16hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Round-to-nearest-even of two fp32 values into one packed dword: `a` in the
// low half (lower address), `b` in the high half (v_cvt_pk_bf16_f32).
QL_DEV uint32_t pack_bf16x2(float a, float b) {
    f32x2_t v = {a, b};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------------------ 16-bit compute type
//
// The layer computes in bf16, or in fp16 when F16 (the compute dtype the pages
// tell users to switch to on GPUs without bf16, "QLoRA 原理精讲" section 3,
// pitfall 4).  Only packing, unpacking and the MFMA and dot opcodes depend on it; a
// 16-byte fragment travels as bf16x8_t bits either way.
template <bool F16>
QL_DEV uint32_t pack16x2(float a, float b) {     // RNE, `a` in the low half
    if constexpr (F16) {
        f32x2_t v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));   // v_cvt_pk_f16_f32
    } else {
        return pack_bf16x2(a, b);
    }
}
template <bool F16>
QL_DEV float lo16(uint32_t v) {
    if constexpr (F16) return (float)__builtin_bit_cast(f16x2_t, v)[0];
    else return bf16lo(v);
}
template <bool F16>
QL_DEV float hi16(uint32_t v) {
    if constexpr (F16) return (float)__builtin_bit_cast(f16x2_t, v)[1];
    else return bf16hi(v);
}
// c + a.lo * b.lo + a.hi * b.hi on the VALU (v_dot2c_f32_bf16 / _f16), fp32 accumulate
template <bool F16>
QL_DEV float dot16x2(uint32_t a, uint32_t b, float c) {
    if constexpr (F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                               false);
}
template <bool F16>
QL_DEV f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
QL_DEV f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ FP8 E4M3FN

// Exact value of a non-negative E4M3FN code (0x00..0x7E): bias 7, 3 fraction
// bits, subnormal spacing 2^-9.  The code's exponent and fraction fields moved
// into an fp32's (bits 23.. and 20..) read as 2^(e-127) (1 + m/8) for e > 0
// and as the fp32 subnormal m 2^-129 for e = 0; one exact multiply by 2^120
// turns both into the E4M3 value (fp32 subnormals are kept, not flushed, in
// these kernels).
QL_DEV float e4m3_decode(uint32_t code) {
    return __uint_as_float((code & 0x7Fu) << 20) * 0x1p120f;
}

// Nearest E4M3FN code to y in [0, 448]; an exact tie goes to the lower code.
QL_DEV uint32_t e4m3_encode_tie_low(float y) {
    if (y < 0.015625f) {                                         // below 2^-6: fixed spacing 2^-9
        const float s = y * 512.0f;                              // exact
        const float f = floorf(s);
        return (uint32_t)f + ((s - f) > 0.5f ? 1u : 0u);         // 8 -> code 0x08 = 2^-6
    }
    const uint32_t b = __float_as_uint(y);
    const uint32_t code = ((((b >> 23) & 0xFF) - 120u) << 3) | ((b >> 20) & 7u);
    return code + ((b & 0xFFFFFu) > 0x80000u ? 1u : 0u);        // strictly above half -> up
}

// Block scale c1' = fl32(e4m3(f) * s2) (first step of the reverse-order
// dequantization).
QL_DEV float block_scale(uint32_t f8, float s2) { return __fmul_rn(e4m3_decode(f8), s2); }

// ------------------------------------------------------------------ LDS and buffer access

// LDS pointers carry address space 3 explicitly so that every tile access is a
// ds_read / ds_write (a generic pointer would fall back to flat instructions).
typedef __attribute__((address_space(3))) uint8_t lds8_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
typedef __attribute__((address_space(3))) float lds_f32_t;
typedef __attribute__((address_space(3))) f32x2_t lds_f32x2_t;

// LDS byte address of a pointer, and a pointer from an LDS byte address.  The
// codebook tables are aligned to their own size (64 KB / 32 KB) inside LDS, so
// a lookup address is the table's address OR-ed with the entry offset, built
// by one permute or shift-or with no add (dynamic LDS starts at address 0 in
// these kernels, which declare no static LDS).
QL_DEV uint32_t lds_addr(const lds8_t* p) { return (uint32_t)(uintptr_t)p; }
template <class T>
QL_DEV const __attribute__((address_space(3))) T* lds_at(uint32_t a) {
    return reinterpret_cast<const __attribute__((address_space(3))) T*>((uintptr_t)a);
}

// Byte-pair codebook tables in LDS: the entry of code byte e holds the fp32
// pair (q[e >> 4], q[e & 15]), i.e. the values of its high (even element) and
// low (odd element) nibbles.  The table is replicated so that the lanes one
// LDS cycle serves read distinct banks:
//   wide:   32 copies, entry e of copy c at e*256 + c*8 (64 KB), copy = lane & 31;
//   narrow: 16 copies, entry e of copy c at e*128 + c*8 (32 KB), copy = lane & 15.
// Both builders take a 256-thread workgroup.  Each thread writes entries whose
// high nibble is a compile-time constant of the unrolled loop and whose low
// nibble is fixed per thread, so every codebook value is read from the kernel
// arguments with a constant index (scalar loads once, no per-entry memory
// round trip).
constexpr uint32_t kWideTableBytes = 256 * 256;
constexpr uint32_t kNarrowTableBytes = 256 * 128;

// Codebook value j as a wave-uniform register (keeps selects between values
// from being folded into a per-lane indexed load)
QL_DEV float cb_value(const Codebook& cb, int j) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cb.q[j])));
}

QL_DEV void build_wide_pair_table(lds8_t* tbl, const Codebook& cb) {
    // thread: copy (tid & 31), entries e = (tid >> 5) + 8 i, i < 32, so
    // e >> 4 = i >> 1 and e & 15 = (tid >> 5) + 8 (i & 1)
    const int sub = (int)threadIdx.x >> 5;
    float lo0 = cb_value(cb, 0), lo1 = cb_value(cb, 8);
#pragma unroll
    for (int j = 1; j < 8; ++j)
        if (sub == j) {
            lo0 = cb_value(cb, j);
            lo1 = cb_value(cb, j + 8);
        }
    lds8_t* dst = tbl + sub * 256 + (threadIdx.x & 31) * 8;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const f32x2_t v = {cb_value(cb, i >> 1), (i & 1) ? lo1 : lo0};
        *reinterpret_cast<lds_f32x2_t*>(dst + i * 2048) = v;
    }
}

QL_DEV void build_pair_table16(lds8_t* tbl, const Codebook& cb) {
    // thread: copy (tid & 15), entries e = (tid >> 4) + 16 i, i < 16, so
    // e >> 4 = i and e & 15 = tid >> 4
    const int sub = (int)threadIdx.x >> 4;
    float lo = cb_value(cb, 0);
#pragma unroll
    for (int j = 1; j < 16; ++j)
        if (sub == j) lo = cb_value(cb, j);
    lds8_t* dst = tbl + sub * 128 + (threadIdx.x & 15) * 8;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const f32x2_t v = {cb_value(cb, i), lo};
        *reinterpret_cast<lds_f32x2_t*>(dst + i * 2048) = v;
    }
}

// LDS tile of [rows][64] bf16: 128 bytes per row in 16-byte chunks, the chunk
// index XOR-swizzled with bits of the row so that fragment reads (16 or 32
// consecutive rows at a fixed chunk) and row-wise writes spread over all banks.
QL_DEV uint32_t lds_off(int row, int chunk) {
    return (uint32_t)row * 128u + ((uint32_t)(chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// Raw buffer loads: a per-thread 32-bit byte offset (constant over the k loop)
// plus a scalar per-tile offset, no 64-bit address arithmetic per load.  A
// thread whose row lies outside the operand gets an offset past the buffer's
// end, for which the hardware returns zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

QL_DEV rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
QL_DEV u32x4_t bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
QL_DEV u32x2_t bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
QL_DEV uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
QL_DEV uint32_t bload2(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
QL_DEV uint32_t bload1(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// ------------------------------------------------------------------ launchers

// Block constants of a quantized weight: the double-quantized pair (one FP8
// code per block, one fp32 super-scale per 256 blocks), or with `absmax` set
// the fp32 absmax of every block (single quantization, no second level).
struct BlockScales {
    const uint8_t* fp8;
    const float* sup;
    const float* absmax;
    bool single() const { return absmax != nullptr; }
};

// The transposed block scales c1' of a quantized W [N, K] that the dX kernel
// reads: out[kb][n] = c1' of block kb of row n, i.e. fl32(e4m3(f) * s2) (the
// stored fp32 absmax with single quantization), [K/64][N] so that eight
// consecutive rows of one block column are contiguous.  It runs as extra
// workgroups of another launch (or alone), 2,048 constants per workgroup so
// that it adds few workgroups to the launch it rides on.
struct ScalesJob {
    const uint8_t* fp8;
    const float* sup;
    const float* absmax;      // single quantization (fp8, sup unused)
    int64_t N, KB;
    float* out;
    int blocks;               // scales_job_blocks(N, KB), 0 = no job
};
// A workgroup takes a tile of 32 rows n x 64 blocks kb: it reads the
// FP8 codes (or fp32 absmax) of each row as 64 consecutive elements, decodes
// them into an LDS tile, and writes each kb row's 32 values as 128 contiguous
// bytes.  Workgroup b takes n tile b % ceil(N / 32) of kb tile b / ceil(N / 32).
// `lds` holds kScalesLds bytes; every thread of the workgroup calls this.
constexpr int kScalesTileN = 32, kScalesTileKB = 64;
constexpr int kScalesLds = kScalesTileN * (kScalesTileKB + 1) * 4;
inline int scales_job_blocks(int64_t N, int64_t KB) {
    return (int)(((N + kScalesTileN - 1) / kScalesTileN) * ((KB + kScalesTileKB - 1) / kScalesTileKB));
}
QL_DEV void scales_job(const ScalesJob& j, int b, lds8_t* lds) {
    typedef __attribute__((address_space(3))) float lds_f32_t;
    lds_f32_t* tile = reinterpret_cast<lds_f32_t*>(lds);                 // [32][65]
    const int ntn = (int)((j.N + kScalesTileN - 1) / kScalesTileN);
    const int64_t n0 = (int64_t)(b % ntn) * kScalesTileN, kb0 = (int64_t)(b / ntn) * kScalesTileKB;
#pragma unroll
    for (int u = 0; u < kScalesTileN * kScalesTileKB / 256; ++u) {
        const int e = (int)threadIdx.x + 256 * u;
        const int nl = e >> 6, kl = e & 63;                             // a wave reads 64 kb of one row
        const int64_t n = n0 + nl, kb = kb0 + kl;
        if (n < j.N && kb < j.KB) {
            const int64_t blk = n * j.KB + kb;
            tile[nl * (kScalesTileKB + 1) + kl] = j.absmax ? j.absmax[blk] : block_scale(j.fp8[blk], j.sup[blk >> 8]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kScalesTileN * kScalesTileKB / 256; ++u) {
        const int e = (int)threadIdx.x + 256 * u;
        const int nl = e & 31, kl = e >> 5;                             // 32 n of one kb row per half-wave
        const int64_t n = n0 + nl, kb = kb0 + kl;
        if (n < j.N && kb < j.KB) j.out[kb * j.N + n] = tile[nl * (kScalesTileKB + 1) + kl];
    }
}

// One tensor of a grouped quantize or dequantize launch: `w` is read by the
// quantizer, `out` written by the dequantizer; `absmax` set selects single
// quantization (fp8/sup unused).
constexpr int kMaxTensors = 16;
struct QuantTensor {
    const uint16_t* w;
    int64_t numel;
    uint8_t* codes;
    uint8_t* fp8;
    float* sup;
    float* absmax;
    uint16_t* out;
};
struct QuantGroup {
    QuantTensor t[kMaxTensors];
    int end[kMaxTensors];     // cumulative workgroup ends
    int count;
};

// Tensor that owns workgroup `bid`, given ascending cumulative ends (uniform).
template <int MAXG>
QL_DEV int group_index(const int* ends, int count, int bid) {
    int i = 0;
#pragma unroll
    for (int j = 0; j < MAXG - 1; ++j) i += (j < count - 1 && bid >= ends[j]) ? 1 : 0;
    return i;
}
QL_DEV int tensor_of(const int* ends, int count, int bid) { return group_index<kMaxTensors>(ends, count, bid); }

hipError_t launch_quantize_group(const QuantTensor* ts, int count, hipStream_t s, bool f16);
hipError_t launch_dequantize_group(const QuantTensor* ts, int count, hipStream_t s, bool int4, bool f16);

// f16: the weights (quantize) / the output (dequantize, merge) are fp16
hipError_t launch_quantize(const uint16_t* w, int64_t numel, uint8_t* codes, uint8_t* fp8,
                           float* superscale, hipStream_t s, bool f16 = false);
// int4: the INT4 absmax levels instead of NF4 (single quantization only)
hipError_t launch_quantize_sq(const uint16_t* w, int64_t numel, uint8_t* codes, float* absmax, hipStream_t s,
                              bool int4 = false);
hipError_t launch_dequantize(const uint8_t* codes, BlockScales sc, int64_t numel, uint16_t* out, hipStream_t s,
                             bool int4 = false, bool f16 = false);

// Forward calls with at most this many tokens take the decode (small-M MFMA) path.
constexpr int64_t kGemvMaxT = 16;
// Forward sizes T (kGemvMaxT < T <= kChunkMaxT) that run as kGemvMaxT-token
// windows through one grouped decode launch: each window streams the weight.
// Up to 96 tokens that beats the split-k MFMA tiles (the LLaMA-7B projections:
// 371 against 397 us at T = 96); from about 100 tokens the tiles win (395
// against 456 us at T = 128).
constexpr int64_t kChunkMaxT = 96;
struct LoraPlan;
ScalesJob scales_job_for(BlockScales sc, const LoraPlan& pl, uint8_t* ws);
size_t gemv_workspace(int64_t T, int64_t K, int64_t N, int64_t r_pad);
hipError_t launch_merge(const uint8_t* codes, BlockScales sc, const uint16_t* lora_a, const uint16_t* lora_b,
                        int64_t K, int64_t N, int64_t r, float scaling, uint16_t* w_out, hipStream_t s, bool f16);
hipError_t launch_gemv(const uint16_t* x, const uint8_t* codes, BlockScales sc, const uint16_t* lora_a,
                       const uint16_t* lora_b, float scaling, const LoraPlan& pl, uint8_t* ws, uint16_t* y,
                       hipStream_t s, bool f16);

// Decode forward of up to kMaxGroup independent problems in one launch pair
// (same token count T and rank r, same storage format).
constexpr int kMaxGroup = 8;
struct GemvProblem {
    const uint16_t* x;
    const uint8_t* codes;
    BlockScales sc;
    const uint16_t* lora_a;
    const uint16_t* lora_b;
    float scaling;
    int64_t K, N;
    uint16_t* y;
    int64_t skip = 0;     // leading token rows computed but not written (another problem writes them)
};
size_t gemv_group_workspace(const GemvProblem* probs, int count, int64_t T, int64_t r_pad);
// The decode product: on the matrix cores (16 token rows, padded) or as VALU
// dot products (T <= kGemvValuMaxT; bf16 with double quantization); Auto is the
// library's choice per T.
enum class DecodeProduct { Auto, Mfma, Valu };
constexpr int64_t kGemvValuMaxT = 8;
hipError_t launch_gemv_group(const GemvProblem* probs, int count, int64_t T, int64_t r, uint8_t* ws, hipStream_t s,
                             bool f16, DecodeProduct prod = DecodeProduct::Auto);

}  // namespace ql
