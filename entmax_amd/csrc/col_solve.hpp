// Threshold solve for a query row whose scores sit in registers, spread over
// the four lanes c, c + 16, c + 32, c + 48 of a wave (one column of an
// S^T = K Q^T MFMA tile: lane (g, c) holds keys 4g .. 4g + 3 of every
// 16-key tile for query c).
//
// The bisection is the one of "ADASPLASH -- ROBERTA Benchmark Result",
// section 2.3 Theorem 2, on the bracket of the "DistilBERT SST-2 with
// AdaSplash Attention" model card, Mathematical Formulation 2
// ([max - 2, max - 2/sqrt(n)]), 25 steps, g(mid) > 1 moves the lower end,
// final midpoint.  It runs in the half-scaled, max-shifted domain
// x = (s - max)/2, where p = [x - t]_+^2 with t = (tau - max)/2, the bracket
// is [-1, -1/sqrt(n)] and x <= 0, so every [x - mid]_+ is at most 1 and is a
// single clamped subtraction.
//
// g(mid) is evaluated exactly (up to rounding order) from two parts:
//   * U, the entries above a reference point hc (>= every later midpoint):
//     count, sum (x - hc) and sum (x - hc)^2, so that
//     sum_U (x - mid)^2 = a2 + 2 (hc - mid) a1 + cnt (hc - mid)^2;
//   * the band, entries between the bracket ends at the last compaction,
//     held in register slots (2 VALU operations per slot and step).
// Entries at or below the lower end never count again and are dropped.
// Before any step, the exact root over the row's four lane maxima (a
// subset, hence a lower bound of the root) prunes the candidates: entries at
// or below it never count, and steps whose midpoint lies below it are
// decided without evaluation.
// A first stage of bisection steps runs on the band, then a compaction
// (hc := hi, band entries above hi folded into U, entries at or below lo
// dropped) leaves a few band entries per lane.
//
// The remaining steps are not stepped through one by one.  Their outcome is
// fixed by the exact root t* of g(t) = 1 inside the current bracket: g is
// continuous and strictly decreasing there, so each step moves the lower
// end exactly when mid < t*, and the final midpoint is the centre of the
// dyadic cell of the bracket that holds t* (the cell (lo, hi] with t* in
// it, g(t*) = 1 itself moving the upper end).  t* comes from Newton steps
// from the left (g is convex, so every Newton iterate is a lower bound)
// and, at each iterate, the closed form of Theorem 1 on the entries above
// the iterate; the closed form is accepted once every entry of that support
// lies above it (the KKT conditions of the same theorem), which identifies
// the exact support.  All stage switches are uniform over the wave; the four
// lanes of a row always take the same decisions because the cross-lane sums
// are bitwise identical in all four.
#pragma once

#include "common.hpp"

namespace ea {

typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Sum / max over lanes c, c + 16, c + 32, c + 48; the result is bitwise
// identical in the four lanes.  v_permlane16_swap(v, v) yields the even
// 16-lane rows in its first and the odd rows in its second result;
// v_permlane32_swap(v, v) the lower and the upper halves.
__device__ __forceinline__ float col4_sum(float v) {
    const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float t = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ int col4_sum_int(int v) {
    const u32x2 a = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
    const unsigned t = a[0] + a[1];
    const u32x2 b = __builtin_amdgcn_permlane32_swap(t, t, false, false);
    return static_cast<int>(b[0] + b[1]);
}
__device__ __forceinline__ float col4_max(float v) {
    const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float t = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// max(x, 0) for x <= 1, as one clamp (folds into the producing instruction)
__device__ __forceinline__ float relu1(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 1.f); }

struct ColState {
    float lo, hi;       // bracket (half-scaled, shifted domain)
    float lb;           // certified lower bound of the root (lb <= t*)
    int it;             // steps taken (uniform over the wave)
    float hc, cnt, a1, a2;   // U statistics of this lane
};

template <int K>
__device__ __forceinline__ void col_steps(const float (&sl)[K], int steps, ColState& s) {
    for (int k = 0; k < steps; ++k) {
        if (s.it >= kIters) break;
        const float mid = 0.5f * (s.lo + s.hi);
        const float dh = s.hc - mid;
        float acc[4] = {fmaf(s.cnt * dh, dh, fmaf(2.f * dh, s.a1, s.a2)), 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float y = relu1(sl[j] - mid);
            acc[j % 4] = fmaf(y, y, acc[j % 4]);
        }
        const float gs = col4_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
        // below lb the outcome is known (entries at or below lb were never
        // loaded, so gs would be short there)
        if (gs > 1.f || mid < s.lb) s.lo = mid;
        else s.hi = mid;
        ++s.it;
    }
}

// Rebase U on hc := hi, fold slots above hi into it, keep slots in (lo, hi]
// at col[0], col[kWave], ... (this lane's column of the scratch area).
template <int K>
__device__ __forceinline__ int col_compact(const float (&sl)[K], ColState& s, float* col) {
    const float d = s.hc - s.hi;
    s.a2 = fmaf(s.cnt * d, d, fmaf(2.f * d, s.a1, s.a2));
    s.a1 = fmaf(s.cnt, d, s.a1);
    s.hc = s.hi;
    int w = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const float x = sl[j];
        const float y = relu1(x - s.hi);
        const bool up = x > s.hi;
        s.cnt += up ? 1.f : 0.f;
        s.a1 += y;
        s.a2 = fmaf(y, y, s.a2);
        col[w * kWave] = x;          // w <= j: the slot was already read
        w += (!up && x > s.lo) ? 1 : 0;
    }
    return w;
}

__device__ __forceinline__ float col4_min(float v) {
    const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float t = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Exact root of g(t) = 1 in (s.lo, s.hi] from U and the band slots sl (this
// lane's share; -inf marks an empty slot).  Starts from t = s.lo, where
// g >= 1.  Uniform loop: at most `cap` rounds, then the last Newton iterate.
template <int K>
__device__ __forceinline__ float col_exact(const float (&sl)[K], const ColState& s, int cap) {
    float tt = fmaxf(s.lo, s.lb);   // g(tt) >= 1; nothing at or below tt is held
    float res = tt;
    bool done = false;
    for (int r = 0; r < cap; ++r) {
        const float d = s.hc - tt;            // >= 0
        float s1 = fmaf(s.cnt, d, s.a1);
        float s2 = fmaf(s.cnt * d, d, fmaf(2.f * d, s.a1, s.a2));
        int ci = static_cast<int>(s.cnt);   // an integer count: one add-with-carry per slot
        float mn = kInf;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float x = sl[j];
            const float y = relu1(x - tt);
            const bool in = x > tt;
            s1 += y;
            s2 = fmaf(y, y, s2);
            ci += in ? 1 : 0;
            mn = fminf(mn, in ? x : kInf);
        }
        s1 = col4_sum(s1);
        s2 = col4_sum(s2);
        const float cn = static_cast<float>(col4_sum_int(ci));
        mn = col4_min(mn);
        // closed form on the support {x > tt}: sum (x - tt - e)^2 = 1, the
        // smaller root e = (s1 - sqrt(D)) / cn = (s2 - 1) / (s1 + sqrt(D)),
        // D = s1^2 - cn (s2 - 1) (a real root exists whenever the support is
        // exact).  Hardware reciprocal and square root (1 ulp) suffice here.
        const float q = s2 - 1.f;
        const float disc = fmaf(s1, s1, -cn * q);
        const float tc = fmaf(q, __builtin_amdgcn_rcpf(s1 + __builtin_amdgcn_sqrtf(fmaxf(disc, 0.f))), tt);
        // (a row without entries -- only rows with no allowed key -- is done)
        const bool ok = (disc >= 0.f && tc < mn && tc <= s.hc) || cn == 0.f;
        if (!done) res = ok ? tc : res;
        done = done | ok;
        if (!__any(!done)) break;
        // Newton step from the left (g(tt) = s2 >= 1, g'(tt) = -2 s1)
        const float tn = fmaf(0.5f * q, __builtin_amdgcn_rcpf(s1), tt);
        tt = fmaxf(tt, fminf(tn, s.hi));
        if (!done) res = tt;
    }
    return res;
}

// Midpoint of the cell, after the remaining bisection steps, that holds ts.
__device__ __forceinline__ float col_dyadic(const ColState& s, float ts) {
    const int r = kIters - s.it;
    if (r <= 0) return 0.5f * (s.lo + s.hi);
    const float cells = ldexpf(1.f, r);
    const float w = (s.hi - s.lo) * ldexpf(1.f, -r);        // exact: power-of-two scaling
    // ts in (lo + j w, lo + (j + 1) w]; an error of one cell here is far
    // below the rounding of g itself
    float j = ceilf((ts - s.lo) * (cells * __builtin_amdgcn_rcpf(s.hi - s.lo))) - 1.f;
    j = fminf(fmaxf(j, 0.f), cells - 1.f);
    return fmaf(j + 0.5f, w, s.lo);
}

template <int K, int STEPS>
__device__ __forceinline__ void col_stage(float* col, int& len, ColState& s) {
    float sl[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const float v = col[j * kWave];
        sl[j] = j < len ? v : -kInf;
    }
    col_steps<K>(sl, STEPS, s);
    len = col_compact<K>(sl, s, col);
}

template <int K>
__device__ __forceinline__ float col_exact_from(const float* col, int len, const ColState& s) {
    float sl[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const float v = col[j * kWave];
        sl[j] = j < len ? v : -kInf;
    }
    return col_exact<K>(sl, s, K * 4 + 3);
}

template <int KMAX>
__device__ __forceinline__ float col_finish(float* col, int len, ColState& s);

// Exact root over the row's four lane maxima (xl: this lane's maximum in
// the half-scaled shifted domain): a subset of the row, so by Theorem 1 its
// root is at most the row's.  Sort and support search as for the full row,
// on four values; a margin of 2^-20 covers rounding.
__device__ __forceinline__ float col_lower_bound(float xl) {
    xl = fmaxf(xl, -2.f);   // lanes without entries: below every root
    const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(xl), __float_as_uint(xl), false, false);
    const u32x2 b0 = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
    const u32x2 b1 = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
    float z0 = __uint_as_float(b0[0]), z1 = __uint_as_float(b1[0]), z2 = __uint_as_float(b0[1]), z3 = __uint_as_float(b1[1]);
    // sort descending (5 compare-exchanges)
    auto cx = [](float& u, float& v) { const float hi = fmaxf(u, v), lo = fminf(u, v); u = hi; v = lo; };
    cx(z0, z1); cx(z2, z3); cx(z0, z2); cx(z1, z3); cx(z1, z2);
    // support search: t_k = mean_k - sqrt(1/k - var_k), largest valid k
    float s1 = 0.f, s2 = 0.f, best = -1.f;
    const float zs[4] = {z0, z1, z2, z3};
#pragma unroll
    for (int k = 1; k <= 4; ++k) {
        const float z = zs[k - 1] - z0;   // relative to the top entry
        s1 += z;
        s2 = fmaf(z, z, s2);
        const float ik = 1.f / k, mu = s1 * ik;
        const float dl = ik - fmaf(s2, ik, -mu * mu);
        const float tk = mu - __builtin_amdgcn_sqrtf(fmaxf(dl, 0.f));
        best = (dl >= 0.f && z > tk) ? tk : best;
    }
    return z0 + best - 0x1p-20f;
}

// sv: this lane's raw scores (unscaled accumulators, -inf where excluded)
// of tiles [t0, t1); x = fma(acc, c2, -mc2) is the half-scaled shifted
// score (c2 = scale / 2, mc2 = row max of acc times c2).  n >= 1: allowed
// keys of the row.  xlmax: this lane's largest x (-inf if none).  col: this
// lane's scratch column (KMAX floats at stride kWave; KMAX exceeds the
// number of this lane's allowed keys).  Must be called by every lane of the
// wave.  Returns t in
// the half-scaled shifted domain (tau = 2 (mc2 + t)), equal in the four
// lanes of the row.
template <int NT, int KMAX>
__device__ __forceinline__ float col_solve(const f32x4 (&sv)[NT], int t0, int t1, float c2, float mc2, float n,
                                           float xlmax, float* col) {
    ColState s;
    s.lb = fmaxf(col_lower_bound(xlmax), -1.f);
    s.lo = -1.f;
    s.hi = -__builtin_amdgcn_rsqf(n);
    s.it = 0;
    s.hc = s.hi;
    s.cnt = 0.f;
    s.a1 = 0.f;
    s.a2 = 0.f;
    // candidates (x > lb) into the scratch column
    int len = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < t0 || t >= t1) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = fmaf(sv[t][i], c2, -mc2);
            col[len * kWave] = x;
            len += x > s.lb ? 1 : 0;
        }
    }
    return col_finish<KMAX>(col, len, s);
}

// Threshold of a row whose scores all sit in registers of its four lanes
// (tiles [t0, t1) of sv; -inf where excluded), by Newton steps on
// sqrt(g(t)) - 1 from the exact root over the four lane maxima (a lower
// bound).  sqrt(g) is the Euclidean norm of [x - t]_+, convex and
// decreasing in t, so every iterate stays at or below the root t*; a row
// stops once its step is below 1e-5, the error then being of the order of
// the step squared over the mean excess.  Returns the centre of the 25-step
// bisection's dyadic cell of [-1, -1/sqrt(n)] that holds t* (half-scaled,
// shifted domain; tau = 2 (mc2 + t)), equal in the four lanes of the row.
// Must be called by every lane of the wave.
template <int NT>
__device__ __forceinline__ float col_newton(const f32x4 (&sv)[NT], int t0, int t1, float c2, float mc2, float n,
                                           float xlmax) {
    const bool empty = n == 0.f;
    const float hi = -__builtin_amdgcn_rsqf(empty ? 1.f : n);
    float t = fminf(fmaxf(col_lower_bound(xlmax), -1.f), hi);
    bool done = empty || n <= 1.f;   // n = 1: the root is the lower end -1
    for (int r = 0; r < 16 && __any(!done); ++r) {
        const float bias = -(mc2 + t);
        float s1 = 0.f, s2 = 0.f, u1 = 0.f, u2 = 0.f;   // two chains each
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            if (k < t0 || k >= t1) continue;   // uniform: -inf there
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float y = relu1(fmaf(sv[k][i], c2, bias));
                if (i & 1) {
                    u1 += y;
                    u2 = fmaf(y, y, u2);
                } else {
                    s1 += y;
                    s2 = fmaf(y, y, s2);
                }
            }
        }
        s1 = col4_sum(s1 + u1);
        s2 = col4_sum(s2 + u2);
        if (!done) {
            const float rg = __builtin_amdgcn_sqrtf(s2);
            const float step = (rg - 1.f) * rg * __builtin_amdgcn_rcpf(s1);
            t = fminf(t + fmaxf(step, 0.f), hi);
            done = step < 1e-5f;
        }
    }
    if (empty || n <= 1.f) return -1.f;
    ColState st;
    st.lo = -1.f;
    st.hi = hi;
    st.it = 0;
    return col_dyadic(st, t);
}

// From a state whose band (entries in (lo, hi] above lb, at most KMAX per
// lane) sits in the scratch column: one stage of bisection steps, then the
// exact finish on what is left of the band.  Returns t (half-scaled,
// shifted), equal in the four lanes of a row.
template <int KMAX>
__device__ __forceinline__ float col_finish(float* col, int len, ColState& s) {
    if (s.it >= kIters) return 0.5f * (s.lo + s.hi);
    if (KMAX > 16 && __any(len > 16)) {
        col_stage<(KMAX > 16 ? 32 : 16), 3>(col, len, s);
        // a dense row can keep more than 16 band entries in a lane after
        // three steps; the exact finish below holds 16, so step on
        while (__any(len > 16)) {
            if (s.it >= kIters) return 0.5f * (s.lo + s.hi);
            col_stage<(KMAX > 16 ? 32 : 16), 3>(col, len, s);
        }
    }
    else if (__any(len > 8)) col_stage<16, 3>(col, len, s);
    else if (__any(len > 4)) col_stage<8, 3>(col, len, s);
    else if (__any(len > 2)) col_stage<4, 2>(col, len, s);
    else if (__any(len > 0)) col_stage<2, 2>(col, len, s);
    float ts;
    if (__any(len > 8)) ts = col_exact_from<16>(col, len, s);
    else if (__any(len > 4)) ts = col_exact_from<8>(col, len, s);
    else if (__any(len > 2)) ts = col_exact_from<4>(col, len, s);
    else if (__any(len > 0)) ts = col_exact_from<2>(col, len, s);
    else {
        float sl[1] = {-kInf};
        ts = col_exact<1>(sl, s, 2);
    }
    return col_dyadic(s, ts);
}

}  // namespace ea
