// Threshold solve with one lane per row (rows whose scores sit in LDS).
//
// Same bisection as tau_solver.hpp ("ADASPLASH -- ROBERTA Benchmark Result",
// section 2.3 Theorem 2; bracket [max - 2, max - 2/sqrt(n)] of the
// "DistilBERT SST-2 with AdaSplash Attention" model card, Mathematical
// Formulation 2; 25 steps, g(mid) > 1 moves the lower end, final midpoint),
// organised for a lane that owns a whole row.
//
// Every step evaluates g(mid) = sum_j [(x_j - mid)/2]_+^2 exactly (x = s - max)
// from two parts:
//   * U, the entries above a reference point hc (>= every later midpoint),
//     kept as cnt = #U, a1 = sum (x - hc), a2 = sum (x - hc)^2, so that
//     sum_U (x - mid)^2 = a2 + 2 (hc - mid) a1 + cnt (hc - mid)^2 -- a sum of
//     non-negative terms, no cancellation;
//   * the band, entries in (lo_c, hc] at the last compaction, each adding
//     max(x - mid, 0)^2 (entries that have since fallen below lo add 0).
// Entries at or below max - 2 never count (tau >= max - 2).  A step costs
// three operations per band slot (plus one lane exchange when two lanes
// share a row); the band is only rebuilt at compactions
// (hc := hi, entries above hi folded into U, entries at or below lo
// dropped), which shrink the register slots 32 -> 8 -> 2 -> 0.  Stage
// switches are uniform over the wave.
#pragma once

#include "common.hpp"

namespace ea {

// Sum over the TPR (1 or 2) lanes of a row; bitwise identical in both lanes.
template <int TPR>
__device__ __forceinline__ float row_sum_lanes(float v) {
    if constexpr (TPR == 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    static_assert(TPR == 1 || TPR == 2, "one or two lanes per row");
    return v;
}

struct BandU {
    float hc, cnt, a1, a2;
};

template <int TPR, int K>
__device__ __forceinline__ void band_steps(const float (&sl)[K], int steps, int& it, float& lo, float& hi,
                                           const BandU& u) {
    for (int s = 0; s < steps && it < kIters; ++s, ++it) {
        const float mid = 0.5f * (lo + hi);
        const float dh = u.hc - mid;
        float acc[4] = {fmaf(u.cnt * dh, dh, fmaf(2.f * dh, u.a1, u.a2)), 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float yp = fmaxf(sl[j] - mid, 0.f);
            acc[j % 4] = fmaf(yp, yp, acc[j % 4]);
        }
        const float g4 = row_sum_lanes<TPR>((acc[0] + acc[1]) + (acc[2] + acc[3]));
        if (g4 > 4.f) lo = mid;
        else hi = mid;
    }
}

// Fold slots above hi into U (rebased to hc = hi), drop slots at or below
// lo; returns the number of slots left in (lo, hi], compacted into e[0..).
// Only e[0 .. len) is written (slots from len on hold -inf).
template <int K>
__device__ __forceinline__ int band_compact(const float (&sl)[K], int len, float lo, float hi, BandU& u, float* e) {
    const float d = u.hc - hi;   // >= 0
    u.a2 = fmaf(u.cnt * d, d, fmaf(2.f * d, u.a1, u.a2));
    u.a1 = fmaf(u.cnt, d, u.a1);
    u.hc = hi;
    int w = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const float y = sl[j] - hi;
        const bool up = y > 0.f;
        u.cnt += up ? 1.f : 0.f;
        u.a1 += up ? y : 0.f;
        u.a2 = up ? fmaf(y, y, u.a2) : u.a2;
        if (j < len) e[w] = sl[j];   // w <= j: stays inside e[0 .. len)
        w += (!up && sl[j] > lo) ? 1 : 0;
    }
    return w;
}

template <int K>
__device__ __forceinline__ void band_load(float (&sl)[K], const float* e, int len) {
#pragma unroll
    for (int k = 0; k < K; k += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(e + k);
#pragma unroll
        for (int j = 0; j < 4; ++j) sl[k + j] = k + j < len ? v[j] : -kInf;
    }
}

// TPR (1 or 2) consecutive lanes share a row; lane `sub` scans entries
// [j0, j1) = [i0 + sub * h, min(i1, i0 + (sub + 1) * h)) with
// h = ceil((i1 - i0) / TPR) rounded up to 4, in batches of 32, and compacts
// its candidates in place to the start of its own range (erow + j0).
// erow: the row in LDS (unshifted scores, -inf when excluded), 16-byte
// aligned; reads may run up to 32 floats past j0 (masked, so any LDS
// contents there are harmless); writes stay inside [j0, j1), so lanes that
// share a row never touch each other's entries.  i0, i1 are
// multiples of 4, entries outside [i0, i1) count as excluded.  m: row max,
// n >= 1 allowed entries.  The row is overwritten.  Every lane of the wave
// must call this.  Returns tau in the shifted domain (tau_unshifted =
// m + result), equal in the TPR lanes.
template <int TPR>
__device__ __forceinline__ float solve_row_lane(float* erow, int i0, int i1, float m, int n, int sub) {
    float lo = -2.f;
    float hi = -2.f / sqrtf(static_cast<float>(n));
    BandU u = {hi, 0.f, 0.f, 0.f};

    // scan: entries above lo (x > -2 in the shifted domain) are compacted in
    // place; all reads of a batch come before its stores, which only touch
    // positions already read
    const int h = (((i1 - i0) + 4 * TPR - 1) / (4 * TPR)) * 4;
    const int j0 = i0 + sub * h;
    const int j1 = j0 + h < i1 ? j0 + h : i1;
    float* e = erow + j0;
    int len = 0;
    for (int i = j0; i < j1; i += 32) {
        float xs[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const bool in = i + 4 * q < j1;
            const f32x4 v = *reinterpret_cast<const f32x4*>(erow + (in ? i + 4 * q : j0));
#pragma unroll
            for (int j = 0; j < 4; ++j) xs[4 * q + j] = in ? v[j] - m : -kInf;
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            // len <= i + k - j0: the store stays inside the lane's own range
            // (a non-candidate is overwritten or left past the end)
            if (i + k < j1) e[len] = xs[k];
            len += xs[k] > -2.f ? 1 : 0;
        }
    }

    int it = 0;
    // ---- rows with more than 32 candidates: band kept in LDS ---------------------
    while (it < kIters && __any(len > 32)) {
        const float mid = 0.5f * (lo + hi);
        const float dh = u.hc - mid;
        float g4 = fmaf(u.cnt * dh, dh, fmaf(2.f * dh, u.a1, u.a2));
        for (int k = 0; k < len; k += 16) {
            f32x4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(e + k + 4 * q);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float yp = k + 4 * q + j < len ? fmaxf(v[q][j] - mid, 0.f) : 0.f;
                    g4 = fmaf(yp, yp, g4);
                }
        }
        g4 = row_sum_lanes<TPR>(g4);
        if (g4 > 4.f) lo = mid;
        else hi = mid;
        ++it;
        // compact the list in place (fold above hi into U, drop at or below lo)
        const float d = u.hc - hi;
        u.a2 = fmaf(u.cnt * d, d, fmaf(2.f * d, u.a1, u.a2));
        u.a1 = fmaf(u.cnt, d, u.a1);
        u.hc = hi;
        int w = 0;
        for (int k = 0; k < len; k += 16) {
            f32x4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(e + k + 4 * q);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = v[q][j];
                    const bool in = k + 4 * q + j < len;
                    const float y = x - hi;
                    const bool up = in && y > 0.f;
                    u.cnt += up ? 1.f : 0.f;
                    u.a1 += up ? y : 0.f;
                    u.a2 = up ? fmaf(y, y, u.a2) : u.a2;
                    if (in) e[w] = x;
                    w += (in && !up && x > lo) ? 1 : 0;
                }
        }
        len = w;
    }

    // ---- register slots: 32, 8, 2, then none --------------------------------------
    {
        float s32[32];
        band_load<32>(s32, e, len);
        band_steps<TPR, 32>(s32, 3, it, lo, hi, u);
        len = band_compact<32>(s32, len, lo, hi, u, e);
    }
    while (it < kIters && __any(len > 8)) {   // rare: slow shrink
        float s32[32];
        band_load<32>(s32, e, len);
        band_steps<TPR, 32>(s32, 2, it, lo, hi, u);
        len = band_compact<32>(s32, len, lo, hi, u, e);
    }
    {
        float s8[8];
        band_load<8>(s8, e, len);
        band_steps<TPR, 8>(s8, 3, it, lo, hi, u);
        len = band_compact<8>(s8, len, lo, hi, u, e);
    }
    while (it < kIters && __any(len > 2)) {
        float s8[8];
        band_load<8>(s8, e, len);
        band_steps<TPR, 8>(s8, 2, it, lo, hi, u);
        len = band_compact<8>(s8, len, lo, hi, u, e);
    }
    while (it < kIters && __any(len > 0)) {
        float s2[2];
        s2[0] = 0 < len ? e[0] : -kInf;
        s2[1] = 1 < len ? e[1] : -kInf;
        band_steps<TPR, 2>(s2, 4, it, lo, hi, u);
        len = band_compact<2>(s2, len, lo, hi, u, e);
    }

    // ---- closed form: no band left ------------------------------------------------
    u.cnt = row_sum_lanes<TPR>(u.cnt);
    u.a1 = row_sum_lanes<TPR>(u.a1);
    u.a2 = row_sum_lanes<TPR>(u.a2);
    for (; it < kIters; ++it) {
        const float mid = 0.5f * (lo + hi);
        const float dh = u.hc - mid;
        const float g4 = fmaf(u.cnt * dh, dh, fmaf(2.f * dh, u.a1, u.a2));
        if (g4 > 4.f) lo = mid;
        else hi = mid;
    }
    return 0.5f * (lo + hi);
}

}  // namespace ea
