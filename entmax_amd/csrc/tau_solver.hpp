// Per-row threshold solve for 1.5-entmax by bisection.
//
// "ADASPLASH -- ROBERTA Benchmark Result", section 2.3 Theorem 2: g(t) =
// sum_j [(s_j - t)/2]_+^2 is strictly decreasing where positive, so
// bisection on g(t) = 1 converges.  Bracket ("DistilBERT SST-2 with AdaSplash
// Attention" model card, Mathematical Formulation 2) in the max-shifted
// domain x = s - max: [-2, -2/sqrt(n)], n = allowed entries of the row.
// Each of the 25 steps evaluates g at the midpoint; g > 1 moves the lower end
// up, otherwise the upper end down; the result is the final midpoint.
//
// Every step evaluates the full sum g(mid); the work per step is kept
// proportional to the entries that can still change the decision:
//   * entries x <= lo contribute 0 at every remaining midpoint (mid > lo);
//   * entries x > hi contribute (x - mid)^2 at every remaining midpoint and
//     are folded into three running numbers kept relative to hi,
//       cnt = #{x > hi}, a1 = sum (x - hi), a2 = sum (x - hi)^2,
//     so sum (x - mid)^2 = a2 + 2 (hi - mid) a1 + cnt (hi - mid)^2, a sum of
//     non-negative terms (no cancellation);
//   * only the "band" lo < x <= hi is visited.
// The band is held three ways, switching when it has shrunk (all switches
// are uniform over the wave):
//   A. a bitmask over the lane's (read-only) entries, while some lane of the
//      wave has more than kSlots band entries;
//   B. kSlots registers per lane (-inf when empty);
//   C. nothing, once no lane of the wave has a band entry: g(mid) is then the
//      closed form above, evaluated from the row totals of (cnt, a1, a2).
#pragma once

#include "common.hpp"

namespace ea {

// Row-wide (N consecutive lanes, N in {1, 2, 4, 8, 16}) all-reduce through
// DPP lane moves (no LDS traffic).  Every lane of the group ends with a
// bitwise-identical result (operands are combined commutatively in pairs).
template <int N, typename Op>
__device__ __forceinline__ float dpp_allreduce(float v, Op op) {
    if constexpr (N >= 2) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    if constexpr (N >= 4) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    if constexpr (N >= 8) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
    if constexpr (N >= 16) v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
    static_assert(N <= 16, "row groups of at most 16 lanes");
    return v;
}
template <int N>
__device__ __forceinline__ float row_sum(float v) {
    return dpp_allreduce<N>(v, [](float a, float b) { return a + b; });
}
template <int N>
__device__ __forceinline__ float row_max(float v) {
    return dpp_allreduce<N>(v, [](float a, float b) { return fmaxf(a, b); });
}

constexpr int kSlots = 4;

// TPR: lanes sharing one row (consecutive, aligned).  get(i), i < nel <= 64:
// this lane's i-th entry in the shifted domain (-inf when excluded).
// n >= 1: allowed entries of the row; all TPR lanes pass the same n.
// Every lane of the wave must call this (mode switches are wave-uniform).
// Returns tau in the shifted domain.
template <int TPR, typename Get>
__device__ __forceinline__ float solve_tau_shifted(Get get, int nel, int n) {
    float lo = -2.f;
    float hi = -2.f / sqrtf(static_cast<float>(n));
    float cnt = 0.f, a1 = 0.f, a2 = 0.f;
    unsigned long long band = 0ull;
    {
        int i = 0;
        for (; i + 4 <= nel; i += 4) {
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = get(i + j);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y = x[j] - hi;
                const bool up = y > 0.f;
                cnt += up ? 1.f : 0.f;
                a1 += up ? y : 0.f;
                a2 = up ? fmaf(y, y, a2) : a2;
                band |= (!up && x[j] > lo) ? (1ull << (i + j)) : 0ull;
            }
        }
        for (; i < nel; ++i) {
            const float x = get(i);
            const float y = x - hi;
            const bool up = y > 0.f;
            cnt += up ? 1.f : 0.f;
            a1 += up ? y : 0.f;
            a2 = up ? fmaf(y, y, a2) : a2;
            band |= (!up && x > lo) ? (1ull << i) : 0ull;
        }
    }

    int it = 0;
    // ---- A: band as a bitmask over the LDS entries ----------------------------
    for (; it < kIters && __any(__popcll(band) > kSlots); ++it) {
        const float mid = 0.5f * (lo + hi);
        const float dh = hi - mid;
        const float gu = fmaf(cnt * dh, dh, fmaf(2.f * dh, a1, a2));
        float c1 = 0.f, b1 = 0.f, b2 = 0.f;
        unsigned long long upper = 0ull;
        unsigned long long rest = band;
        while (rest) {
            // two entries per trip so that their LDS reads overlap
            const int i0 = __ffsll(static_cast<long long>(rest)) - 1;
            rest &= rest - 1ull;
            const int i1 = rest ? __ffsll(static_cast<long long>(rest)) - 1 : -1;
            if (rest) rest &= rest - 1ull;
            const float x0 = get(i0);
            const float x1 = i1 >= 0 ? get(i1) : -kInf;
            const float y0 = x0 - mid, y1 = x1 - mid;
            if (y0 > 0.f) { c1 += 1.f; b1 += y0; b2 = fmaf(y0, y0, b2); upper |= 1ull << i0; }
            if (y1 > 0.f) { c1 += 1.f; b1 += y1; b2 = fmaf(y1, y1, b2); upper |= 1ull << i1; }
        }
        // 4 g(mid) = sum over the row of (x - mid)^2 for x > mid
        const float g4 = row_sum<TPR>(gu + b2);
        if (g4 > 4.f) {
            lo = mid;
            band = upper;
        } else {
            a1 = fmaf(cnt, dh, a1) + b1;
            a2 = gu + b2;
            cnt += c1;
            hi = mid;
            band &= ~upper;
        }
    }

    // ---- B: band in registers -------------------------------------------------
    float sl[kSlots];
    {
        unsigned long long rest = band;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            const int i0 = rest ? __ffsll(static_cast<long long>(rest)) - 1 : -1;
            if (rest) rest &= rest - 1ull;
            sl[j] = i0 >= 0 ? get(i0) : -kInf;
        }
    }
    for (; it < kIters; ++it) {
        bool live = false;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) live |= sl[j] > -kInf;
        if (!__any(live)) break;
        const float mid = 0.5f * (lo + hi);
        const float dh = hi - mid;
        const float gu = fmaf(cnt * dh, dh, fmaf(2.f * dh, a1, a2));
        float b2 = 0.f;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            const float yp = fmaxf(sl[j] - mid, 0.f);
            b2 = fmaf(yp, yp, b2);
        }
        const float g4 = row_sum<TPR>(gu + b2);
        if (g4 > 4.f) {
            lo = mid;
#pragma unroll
            for (int j = 0; j < kSlots; ++j) sl[j] = sl[j] > mid ? sl[j] : -kInf;
        } else {
            float c1 = 0.f, b1 = 0.f;
#pragma unroll
            for (int j = 0; j < kSlots; ++j) {
                const float y = sl[j] - mid;
                const bool up = y > 0.f;
                c1 += up ? 1.f : 0.f;
                b1 += up ? y : 0.f;
                sl[j] = up ? -kInf : sl[j];
            }
            a1 = fmaf(cnt, dh, a1) + b1;
            a2 = gu + b2;
            cnt += c1;
            hi = mid;
        }
    }

    // ---- C: closed form from the row totals ------------------------------------
    if (it < kIters) {
        cnt = row_sum<TPR>(cnt);
        a1 = row_sum<TPR>(a1);
        a2 = row_sum<TPR>(a2);
        for (; it < kIters; ++it) {
            const float mid = 0.5f * (lo + hi);
            const float dh = hi - mid;
            const float g4 = fmaf(cnt * dh, dh, fmaf(2.f * dh, a1, a2));
            if (g4 > 4.f) {
                lo = mid;
            } else {
                a1 = fmaf(cnt, dh, a1);
                a2 = g4;
                hi = mid;
            }
        }
    }
    return 0.5f * (lo + hi);
}

}  // namespace ea
