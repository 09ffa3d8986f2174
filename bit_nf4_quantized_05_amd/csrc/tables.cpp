// Host-side construction of the NF4 constant tables.
//
// Code book: the NF4 data type of the QLoRA pages - quantiles of N(0,1) taken at
// equal probability steps, with a separate negative half (7 values) and positive
// half (8 values) that share one exact zero, normalised so the ends are -1 and +1
// (learn.ifs.name QLoRA deck, cards 2-3; whoami-wesleyyou.top "1. NF4"; the printed
// quant book of jjjymmm.cn "4-bit NormalFloat(NF4)"). The outermost probability,
// which keeps the infinite quantile at p = 1 out, is 0.967704: the printed 4-decimal
// book holds for offsets in [0.9677024, 0.9677083] only, and this value keeps each
// of the 16 entries farthest inside the rounding interval of its printed digits.
//
// Quantiles are found by bisection on the normal CDF written with erfc, in double;
// the float32 rounding of each value has a wide margin to that error.
//
// Code search: "nearest code, lower index on an exact tie" is the same as counting
// the thresholds T_k that x exceeds, where T_k is the exact midpoint of codes k and
// k+1 rounded down to float32. [-1, 1] is cut into 32 equal cells; no cell holds
// more than one threshold and no threshold lies near a cell edge (both checked
// here), so code(x) = base[cell] + (x > thr[cell]).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <mutex>

#include "internal.h"

namespace qn {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_quantile(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 2000; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (normal_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

float round_down_f32(double v) {
    float f = static_cast<float>(v);
    if (static_cast<double>(f) > v) f = std::nextafter(f, -std::numeric_limits<float>::infinity());
    return f;
}

NF4Tables build() {
    NF4Tables t{};
    const double top = 0.967704;
    const double norm = normal_quantile(top);
    double v[16];
    // negative half, most negative first: probabilities 1-top ... stepping to 1/2
    for (int i = 0; i < 7; ++i) v[i] = -normal_quantile(top - i * (top - 0.5) / 7.0) / norm;
    v[7] = 0.0;
    for (int i = 0; i < 8; ++i) v[15 - i] = normal_quantile(top - i * (top - 0.5) / 8.0) / norm;
    for (int i = 0; i < 16; ++i) t.code[i] = static_cast<float>(v[i]);
    t.code[0] = -1.0f;
    t.code[15] = 1.0f;

    float thr[15];
    for (int k = 0; k < 15; ++k)
        thr[k] = round_down_f32((static_cast<double>(t.code[k]) + static_cast<double>(t.code[k + 1])) * 0.5);

    for (int c = 0; c < kCells; ++c) {
        const double lo = -1.0 + c / 16.0, hi = lo + 1.0 / 16.0;
        uint32_t base = 0;
        int inside = 0;
        float th = std::numeric_limits<float>::infinity();
        for (int k = 0; k < 15; ++k) {
            const double tk = thr[k];
            if (tk < lo) ++base;
            else if (tk < hi) { ++inside; th = thr[k]; }
            if (std::fabs(tk - lo) < 1e-5 || std::fabs(tk - hi) < 1e-5) {
                std::fprintf(stderr, "qlora_nf4: threshold too close to a cell edge\n");
                std::abort();
            }
        }
        if (inside > 1) {
            std::fprintf(stderr, "qlora_nf4: two thresholds in one cell\n");
            std::abort();
        }
        t.cell_base[c] = base;
        t.cell_thr[c] = th;
    }
    return t;
}

}  // namespace

const NF4Tables& tables() {
    static std::once_flag once;
    static NF4Tables t;
    std::call_once(once, [] { t = build(); });
    return t;
}

}  // namespace qn
