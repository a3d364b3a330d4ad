// Host-side NF4 codebook and encoder table.
//
// Codebook: "QLoRA 原理精讲" section 2.1 and "从LoRA到QLoRA" section 2.3 build the
// 4-bit NormalFloat values from quantiles of the standard normal at evenly
// spaced probabilities and rescale them to [-1, 1].  With 16 values and an exact
// zero the set is asymmetric: 8 positive values at probabilities
// 1/2 + j (d - 1/2) / 8, j = 1..8, 7 negative values mirrored at
// 1/2 + j (d - 1/2) / 7, j = 1..7, with the tail offset d = ((1 - 1/30) +
// (1 - 1/32)) / 2 (half a bin short of 1, averaged over the two halves), all
// divided by z = Phi^-1(d) so that the ends are exactly -1 and +1.
//
// The inverse normal CDF here is our own: bisection on Phi(x) = erfc(-x/sqrt2)/2
// (C library erfc), polished by Newton steps, all in fp64.  Each codeword is
// rounded once to fp32.
#include <cmath>
#include <mutex>

#include "common.hpp"

namespace ql {
namespace {

double phi(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }
double phi_density(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

double inverse_phi(double p) {
    double lo = -12.0, hi = 12.0;
    for (int i = 0; i < 80; ++i) {              // bracket to below fp64 resolution
        const double mid = 0.5 * (lo + hi);
        if (phi(mid) < p) lo = mid; else hi = mid;
    }
    double x = 0.5 * (lo + hi);
    for (int i = 0; i < 3; ++i) x -= (phi(x) - p) / phi_density(x);
    return x;
}

Codebook g_codebook, g_int4_codebook;
EncodeTable g_table, g_int4_table;
std::once_flag g_once;

// Decision midpoints of neighbouring fp32 codewords (exact in fp64), then the
// per-cell (base, threshold) lookup used by the encoder kernels.  Cell c is
// [(c - 1/2)/16 - 1, (c + 1/2)/16 - 1), the values that round(16 n + 16)
// sends to c.  Valid for any ascending codebook on [-1, 1] whose neighbouring
// midpoints are more than 1/16 apart (NF4: at least 0.08; INT4: 1/7).
void build_table(const Codebook& cb, EncodeTable& tab) {
    double mid[15];
    for (int i = 0; i < 15; ++i) mid[i] = 0.5 * ((double)cb.q[i] + (double)cb.q[i + 1]);
    for (int c = 0; c < 34; ++c) {
        const double lo = (c - 0.5) / 16.0 - 1.0, hi = (c + 0.5) / 16.0 - 1.0;
        uint32_t base = 0;
        float thr = 2.0f;
        for (int i = 0; i < 15; ++i) {
            if (mid[i] < lo) ++base;
            else if (mid[i] < hi) {
                float t = (float)mid[i];                       // round to nearest ...
                if ((double)t > mid[i]) t = std::nextafter(t, -INFINITY);   // ... then down
                thr = t;
            }
        }
        tab.base[c] = base;
        tab.thr[c] = thr;
    }
}

void build_all() {
    const double d = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
    const double z = inverse_phi(d);
    double v[16];
    for (int j = 1; j <= 7; ++j) v[7 - j] = -inverse_phi(0.5 + j * (d - 0.5) / 7.0) / z;
    v[7] = 0.0;
    for (int j = 1; j <= 8; ++j) v[7 + j] = inverse_phi(0.5 + j * (d - 0.5) / 8.0) / z;
    for (int i = 0; i < 16; ++i) g_codebook.q[i] = (float)v[i];

    build_table(g_codebook, g_table);

    // INT4 absmax levels (i - 8) / 7 ("QLoRA 原理精讲" section 2.1: 16 uniform
    // integers [-8, 7]; +absmax lands on 7), the baseline of the data-type ablation
    for (int i = 0; i < 16; ++i) g_int4_codebook.q[i] = (float)((i - 8) / 7.0);
    build_table(g_int4_codebook, g_int4_table);
}

}  // namespace

const Codebook& host_codebook() {
    std::call_once(g_once, build_all);
    return g_codebook;
}

const EncodeTable& host_encode_table() {
    std::call_once(g_once, build_all);
    return g_table;
}

const Codebook& host_int4_codebook() {
    std::call_once(g_once, build_all);
    return g_int4_codebook;
}

const EncodeTable& host_int4_encode_table() {
    std::call_once(g_once, build_all);
    return g_int4_table;
}

}  // namespace ql
