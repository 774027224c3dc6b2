// Row-wise alpha-entmax on a score matrix [R, L] (row-major), forward and
// backward: the per-row threshold solve of the attention kernels as an op of
// its own (the pages' entmax_bisect and entmax15_bisect exports, "ADASPLASH --
// ROBERTA Benchmark Result", section 4), for alpha in (1, 2].
//
// Forward at alpha = 1.5: p_j = [(s_j - tau)/2]_+^2 over the allowed entries
// of the row (section 2.2 Theorem 1), tau from 25 bisection steps (section
// 2.3 Theorem 2) on the bracket [max - 2, max - 2/sqrt(n)] ("DistilBERT
// SST-2 with AdaSplash Attention" model card, Mathematical Formulation 2),
// run in the half-scaled shifted domain x = (s - max)/2 where the bracket is
// [-1, -1/sqrt(n)].  Other alphas use the same steps with the powers below.
// One wave per row (a workgroup per row when there are few long rows); lane
// l holds entries 256 c + 4 l .. + 3 of chunk c (1024 c + 4 l with a
// workgroup), so every load and store is one contiguous block per wave.
// Rows of at most 16 chunks stay in registers for all 25 steps; longer rows
// are re-read for every step (the pages' algorithm as printed; HBM-bound).
//
// Backward (section 2.4 Jacobian): with w = sqrt(p) at alpha = 1.5,
// ds_j = w_j (dp_j - sum_k w_k dp_k / sum_k w_k).
#pragma once

#include "col_solve.hpp"
#include "common.hpp"
#include "dpp.hpp"

namespace ea {

struct RowsArgs {
    const void* s;            // [R, L] scores (fp32 or bf16)
    const uint8_t* mask;      // [R, L], nonzero = allowed; or null
    float* p;                 // [R, L] or null (tau only)
    float* tau;               // [R] (score units) or null
    int R, L;                 // rows; row pitch (elements, a multiple of 4)
    float alpha;              // in (1, 2]; 1.5 unless GEN
    // [R] or null: row r takes part in the row only in its first
    // min(row_len[r], L) entries (the rest count as not allowed); entries
    // of -inf never count
    const int* row_len = nullptr;
};

// General alpha ("ADASPLASH -- ROBERTA Benchmark Result", section 2.1, and
// the entmax_bisect routine of section 4): p_j = [(alpha - 1)(s_j - max) - t]_+
// ^ (1/(alpha - 1)), t with sum p = 1, in the domain x = (alpha - 1)(s - max)
// <= 0 where the bracket [-1, -n^(1 - alpha)] holds (at -1 the maximum alone
// gives 1; at -n^(1-alpha) each of the n terms is at most 1/n).  Powers of y
// in [0, 1] by the hardware base-2 exponential and logarithm (about 1 ulp).
__device__ __forceinline__ float pow01(float y, float e) {
    return y > 0.f ? __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(y)) : 0.f;
}

// Sum over the 64 lanes of the wave, bitwise identical in every lane.  The
// empty asm keeps the compiler from fusing a product that forms v into the
// first cross-lane addition: each lane would then round its own product
// differently from its neighbour's, and the lanes would disagree.
__device__ __forceinline__ float wave_sum(float v) {
    asm volatile("" : "+v"(v));
    return col4_sum(row_sum<16>(v));
}
__device__ __forceinline__ float wave_max(float v) { return col4_max(row_max<16>(v)); }

// 4 consecutive entries of row `row` starting at column j (j % 4 == 0, may
// run past L: those read column 0 and are marked invalid by the caller)
template <int DT>
__device__ __forceinline__ f32x4 load4(const void* s, size_t row_off, int j, int L) {
    const int jj = j < L ? j : 0;   // whole quads: L % 4 == 0 is required
    if constexpr (DT == DT_BF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(s) + row_off + jj);
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
    } else {
        return *reinterpret_cast<const f32x4*>(static_cast<const float*>(s) + row_off + jj);
    }
}

// Allowed bits of entries j .. j + 3 (j % 4 == 0): below the row's length
// n and, with a mask, nonzero there (the mask has the row pitch, so whole
// quads below n are in bounds)
__device__ __forceinline__ unsigned valid4(const uint8_t* mask, size_t row_off, int j, int n) {
    unsigned v = 0u;
    if (j < n) {
        const unsigned mb = mask ? *reinterpret_cast<const unsigned*>(mask + row_off + j) : 0x01010101u;
#pragma unroll
        for (int i = 0; i < 4; ++i) v |= (((mb >> (8 * i)) & 0xFFu) != 0u && j + i < n) ? (1u << i) : 0u;
    }
    return v;
}

// Upper end of the bracket in the scaled shifted domain: -n^(1 - alpha)
// (-1/sqrt(n) at alpha = 1.5).
template <bool GEN>
__device__ __forceinline__ float bracket_hi(float n, float am1) {
    return GEN ? -__builtin_amdgcn_exp2f(-am1 * __builtin_amdgcn_logf(n)) : -__builtin_amdgcn_rsqf(n);
}

// Exact root t* of g(t) = sum [x - t]_+^2 = 1 (alpha = 1.5) from the
// candidates cs of this thread (every entry of the row above lo, where
// g(lo) >= 1 and t* lies in (lo, hi]).  Newton steps from the left (g is
// convex and decreasing there, so the iterates stay at or below t*) and, at
// each iterate t, the closed form of "ADASPLASH -- ROBERTA Benchmark
// Result", section 2.2 Theorem 1, on the entries above t: the smaller root
// tc of sum (x - t - e)^2 = 1, accepted when no entry lies in (t, tc] (then
// every entry above tc is in the support and tc = t*).  Returns whether
// every row of the wave was accepted within the round cap (uniform).
template <int K, class RSum>
__device__ __forceinline__ bool exact_root(const float (&cs)[K], float lo, float hi, RSum rsum, float& ts) {
    float t = lo, res = lo;
    bool done = false;
    for (int r = 0; r < 8; ++r) {
        float s1 = 0.f, s2 = 0.f, c = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float y = relu1(cs[k] - t);
            s1 += y;
            s2 = fmaf(y, y, s2);
            c += cs[k] > t ? 1.f : 0.f;
        }
        s1 = rsum(s1);
        s2 = rsum(s2);
        c = rsum(c);
        // e = (s1 - sqrt(D)) / c = (s2 - 1) / (s1 + sqrt(D)), D = s1^2 - c (s2 - 1);
        // s1 > 0: the row maximum (x = 0) lies above every t <= hi < 0
        const float q = s2 - 1.f;
        const float disc = fmaf(s1, s1, -c * q);
        const float tc = fmaf(q, __builtin_amdgcn_rcpf(s1 + __builtin_amdgcn_sqrtf(fmaxf(disc, 0.f))), t);
        float inb = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) inb += (cs[k] > t && cs[k] <= tc) ? 1.f : 0.f;
        inb = rsum(inb);
        const bool ok = disc >= 0.f && inb == 0.f && tc <= hi;
        res = (!done && ok) ? tc : res;
        done = done || ok;
        if (!__any(!done)) break;
        // Newton step from the left: g(t) = s2, g'(t) = -2 s1
        const float tn = fmaf(0.5f * q, __builtin_amdgcn_rcpf(s1), t);
        t = fmaxf(t, fminf(tn, hi));
    }
    ts = res;
    return !__any(!done);
}

// The midpoint that the remaining kIters - it bisection steps on [lo, hi]
// end at when the root is ts: the centre of the dyadic cell (lo + j w,
// lo + (j + 1) w] holding ts (g(mid) = 1 moves the upper end).  An error of
// one cell (2^-25 of the bracket) is below the rounding of g itself.
__device__ __forceinline__ float dyadic_mid(float lo, float hi, int it, float ts) {
    const int r = kIters - it;
    if (r <= 0 || !(hi > lo)) return 0.5f * (lo + hi);
    const float cells = ldexpf(1.f, r);
    const float w = (hi - lo) * ldexpf(1.f, -r);   // exact: power-of-two scaling
    float j = ceilf((ts - lo) * (cells / (hi - lo))) - 1.f;
    j = fminf(fmaxf(j, 0.f), cells - 1.f);
    return fmaf(j + 0.5f, w, lo);
}

// 25 bisection steps on t for a row held in registers, NV quads per thread:
// x = (alpha - 1)(s - max), -inf where not allowed, n >= 1 allowed entries.
// g(mid) = sum [x - mid]_+^(1/(alpha-1)) (each term at most 1: x <= 0 and
// mid >= -1), g > 1 moves the lower end; returns the final midpoint.
// Entries at or below the lower end never count again (every later midpoint
// lies above it): after the first kFirst steps, when no thread holds more
// than kCand entries above the lower end, the remaining steps run over those
// slots (with a wave or less per row, two more steps and a second
// compaction when no thread holds more than 2 kCand).  At alpha = 1.5 with
// a wave or less per row the remaining steps are not taken one by one:
// their end point follows from the exact root (exact_root, dyadic_mid), with
// the steps as the fallback.  pw: y -> y^(1/(alpha-1)); rsum: sum over the row's TPR threads,
// bitwise identical in all of them.  TPR <= 64: the threads of a wave take
// the same path (several rows per wave with TPR < 64).
template <int NV, bool GEN, int TPR, class PW, class RSum>
__device__ __forceinline__ float bisect_regs(const f32x4 (&xs)[NV], float n, float am1, PW pw, RSum rsum) {
    constexpr int kFirst = 4, kCand = 4;
    float lo = -1.f, hi = bracket_hi<GEN>(n, am1);
    auto step = [&](auto&& partial) {
        const float mid = 0.5f * (lo + hi);
        if (rsum(partial(mid)) > 1.f) lo = mid;
        else hi = mid;
    };
    auto full = [&](float mid) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NV; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc += pw(relu1(xs[q][i] - mid));
        return acc;
    };
    int it = 0;
    for (; it < kFirst; ++it) step(full);
    float cs[kCand];
    int nc = 0;
    auto compact = [&]() {
        nc = 0;
#pragma unroll
        for (int k = 0; k < kCand; ++k) cs[k] = -kInf;
#pragma unroll
        for (int q = 0; q < NV; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = xs[q][i];
                const bool cand = x > lo;
#pragma unroll
                for (int k = 0; k < kCand; ++k) cs[k] = (cand & (nc == k)) ? x : cs[k];
                nc += cand ? 1 : 0;
            }
    };
    compact();
    bool few;
    if constexpr (TPR <= kWave) {
        few = !__any(nc > kCand);   // over the wave (all its rows)
        // a thread with a few more candidates: two more steps over every
        // entry (about a quarter of the band is left), then compact again
        if (!few && !__any(nc > 2 * kCand)) {
            step(full);
            step(full);
            it += 2;
            compact();
            few = !__any(nc > kCand);
        }
        if constexpr (!GEN) {
            // alpha = 1.5: the remaining steps follow from the exact root,
            // found over the candidates or, for a dense row, over every entry
            float ts;
            bool ok;
            if (few) {
                ok = exact_root(cs, lo, hi, rsum, ts);
            } else {
                float xa[4 * NV];
#pragma unroll
                for (int q = 0; q < NV; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xa[4 * q + i] = xs[q][i];
                ok = exact_root(xa, lo, hi, rsum, ts);
            }
            if (ok) return dyadic_mid(lo, hi, it, ts);
        }
    } else {
        few = !__syncthreads_or(nc > kCand);
    }
    if constexpr (TPR == kThreads) {
        // a workgroup per row: when the whole row holds at most 64
        // candidates, wave 0 takes the remaining steps alone, without a
        // barrier per step.  The candidates are gathered in thread order (a
        // prefix sum of the counts), so the result does not depend on timing.
        __shared__ float gath[kWave];
        __shared__ int wtot[kThreads / kWave];
        __shared__ float fin[2];
        const int wv = threadIdx.x / kWave, ln = threadIdx.x % kWave;
        int inc = nc;   // inclusive prefix over the wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(inc, o, kWave);
            inc += ln >= o ? y : 0;
        }
        if (ln == kWave - 1) wtot[wv] = inc;
        __syncthreads();
        int base = 0, tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kThreads / kWave; ++w2) {
            base += w2 < wv ? wtot[w2] : 0;
            tot += wtot[w2];
        }
        if (few && tot <= kWave) {   // uniform over the workgroup
            const int off = base + inc - nc;
#pragma unroll
            for (int k = 0; k < kCand; ++k)
                if (k < nc) gath[off + k] = cs[k];
            __syncthreads();
            if (wv == 0) {
                const float x = ln < tot ? gath[ln] : -kInf;
                for (; it < kIters; ++it) {
                    const float mid = 0.5f * (lo + hi);
                    if (wave_sum(pw(relu1(x - mid))) > 1.f) lo = mid;
                    else hi = mid;
                }
                if (ln == 0) {
                    fin[0] = lo;
                    fin[1] = hi;
                }
            }
            __syncthreads();
            return 0.5f * (fin[0] + fin[1]);
        }
    }
    if (few) {
        for (; it < kIters; ++it)
            step([&](float mid) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < kCand; ++k) acc += pw(relu1(cs[k] - mid));
                return acc;
            });
    } else {
        for (; it < kIters; ++it) step(full);
    }
    return 0.5f * (lo + hi);
}

// TPR threads per row: a wave (many rows), or the whole workgroup (few long
// rows, as at decode time: sums then go through LDS, one barrier each).
// NV chunks of 4 TPR entries per row in registers (L <= 4 TPR NV); NV = 0:
// any L, streamed from memory at every step.
template <int DT, int NV, bool GEN, int TPR = kWave>
__global__ __launch_bounds__(kThreads) void rows_fwd_kernel(RowsArgs a) {
    static_assert(TPR == kWave || TPR == kThreads, "a wave or a workgroup per row");
    constexpr int CH = 4 * TPR;   // entries per chunk
    const float am1 = GEN ? a.alpha - 1.f : 0.5f;        // alpha - 1
    const float beta = GEN ? 1.f / (a.alpha - 1.f) : 2.f;   // 1 / (alpha - 1)
    // [y]^beta: a square for alpha = 1.5
    auto pw = [&](float y) { return GEN ? pow01(y, beta) : y * y; };
    const int lane = threadIdx.x % TPR;   // position within the row's threads
    const int row = TPR == kWave ? blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave)
                                 : static_cast<int>(blockIdx.x);
    if (row >= a.R) return;   // uniform over the row's threads
    const int L = a.L;
    const int Lr = a.row_len != nullptr ? min(max(a.row_len[row], 0), L) : L;   // entries of this row
    const size_t off = static_cast<size_t>(row) * L;
    const int nch = NV > 0 ? NV : (Lr + CH - 1) / CH;   // chunks the solve reads
    // reductions over the row's threads, bitwise identical in all of them
    __shared__ float xch[2][kThreads / kWave];
    int par = 0;
    auto across = [&](float w, bool is_max) {
        if (threadIdx.x % kWave == 0) xch[par][threadIdx.x / kWave] = w;
        __syncthreads();
        const float* s = xch[par];
        par ^= 1;   // the next reduction writes the other slot set
        return is_max ? fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) : (s[0] + s[1]) + (s[2] + s[3]);
    };
    auto rsum = [&](float v) {
        const float w = wave_sum(v);
        if constexpr (TPR == kWave) return w;
        else return across(w, false);
    };
    auto rmax = [&](float v) {
        const float w = wave_max(v);
        if constexpr (TPR == kWave) return w;
        else return across(w, true);
    };

    // pass 1: row max and allowed count
    float mraw = -kInf, cnt = 0.f;
    f32x4 xs[NV > 0 ? NV : 1];
    unsigned vb[NV > 0 ? NV : 1];
    for (int c = 0; c < nch; ++c) {
        const int j = CH * c + 4 * lane;
        const f32x4 v = load4<DT>(a.s, off, j, L);
        const unsigned ok = valid4(a.mask, off, j, Lr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool on = ((ok >> i) & 1u) && v[i] > -kInf;   // -inf: not allowed
            mraw = fmaxf(mraw, on ? v[i] : -kInf);
            cnt += on ? 1.f : 0.f;
        }
        if constexpr (NV > 0) {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q == c) { xs[q] = v; vb[q] = ok; }
        }
    }
    const float m = rmax(mraw);
    const float n = rsum(cnt);
    const int ncw = NV > 0 ? NV : (L + CH - 1) / CH;    // chunks of p written
    if (n == 0.f) {
        // no allowed entry: p = 0, tau = +inf
        for (int c = 0; c < ncw; ++c) {
            const int j = CH * c + 4 * lane;
            if (a.p != nullptr && j < L) *reinterpret_cast<f32x4*>(a.p + off + j) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (a.tau != nullptr && lane == 0) a.tau[row] = kInf;
        return;
    }
    // x = (s - m)/2 on allowed entries, -inf elsewhere
    auto shifted = [&](const f32x4& v, unsigned ok) {
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = ((ok >> i) & 1u) ? am1 * (v[i] - m) : -kInf;
        return x;
    };
    if constexpr (NV > 0) {
#pragma unroll
        for (int q = 0; q < NV; ++q) xs[q] = shifted(xs[q], vb[q]);
    }
    float t;
    if constexpr (NV > 0) {
        t = bisect_regs<NV, GEN, TPR>(xs, n, am1, pw, rsum);
    } else {
        // rows longer than the registers hold: every step re-reads the row
        float lo = -1.f, hi = bracket_hi<GEN>(n, am1);
        for (int it = 0; it < kIters; ++it) {
            const float mid = 0.5f * (lo + hi);
            float acc = 0.f;
            for (int c = 0; c < nch; ++c) {
                const int j = CH * c + 4 * lane;
                const f32x4 x = shifted(load4<DT>(a.s, off, j, L), valid4(a.mask, off, j, Lr));
#pragma unroll
                for (int i = 0; i < 4; ++i) acc += pw(relu1(x[i] - mid));
            }
            if (rsum(acc) > 1.f) lo = mid;
            else hi = mid;
        }
        t = 0.5f * (lo + hi);
    }
    if (a.tau != nullptr && lane == 0) a.tau[row] = m + t * beta;   // score units: p = [(alpha-1)(s - tau)]_+^beta
    if (a.p == nullptr) return;
    for (int c = 0; c < ncw; ++c) {
        const int j = CH * c + 4 * lane;
        f32x4 x;
        if constexpr (NV > 0) {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q == c) x = xs[q];
        } else {
            x = shifted(load4<DT>(a.s, off, j, L), valid4(a.mask, off, j, Lr));
        }
        f32x4 p;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = pw(relu1(x[i] - t));
        if (j < L) *reinterpret_cast<f32x4*>(a.p + off + j) = p;
    }
}

struct RowsBwdArgs {
    const float* p;    // [R, L]
    const float* dp;   // [R, L]
    float* ds;         // [R, L]
    int R, L;
    float alpha;       // in (1, 2]; 1.5 unless GEN
};

// One wave per row: sum w and sum w dp, then ds = w (dp - c).  Rows of at
// most 256 NV entries are read once and kept in registers; NV = 0 reads p
// and dp twice.
// General alpha: dp_i/ds_j = w_i (delta_ij - w_j / sum w) with w = p^(2 - alpha)
// on the support (differentiating p = [(alpha-1)(s - tau)]_+^(1/(alpha-1))
// under sum p = 1); w = sqrt(p) for alpha = 1.5.
template <int NV, bool GEN>
__global__ __launch_bounds__(kThreads) void rows_bwd_kernel(RowsBwdArgs a) {
    const float e = 2.f - a.alpha;
    auto wt = [&](float p) { return GEN ? pow01(p, e) : __builtin_sqrtf(p); };
    const int lane = threadIdx.x % kWave;
    const int row = blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (row >= a.R) return;
    const int L = a.L;
    const size_t off = static_cast<size_t>(row) * L;
    constexpr int NR = NV > 0 ? NV : 1;
    f32x4 ws[NR], ds_[NR];
    float sw = 0.f, swd = 0.f;
    const int nch = NV > 0 ? NV : (L + 255) / 256;
    for (int c = 0; c < nch; ++c) {
        const int j = 256 * c + 4 * lane;
        const int jj = j < L ? j : 0;   // past L: read column 0, weight 0
        // every element is read and written once: non-temporal (streaming)
        // accesses keep the caches out of the way (1208 MB at 6.4 TB/s
        // instead of 5.3 on the rows workload)
        const f32x4 p = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.p + off + jj));
        const f32x4 d = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.dp + off + jj));
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = j < L ? wt(p[i]) : 0.f;
            sw += w[i];
            swd = fmaf(w[i], d[i], swd);
        }
        if constexpr (NV > 0) {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q == c) { ws[q] = w; ds_[q] = d; }
        }
    }
    sw = wave_sum(sw);
    swd = wave_sum(swd);
    const float cc = sw > 0.f ? swd / sw : 0.f;
    for (int c = 0; c < nch; ++c) {
        const int j = 256 * c + 4 * lane;
        f32x4 w, d;
        if constexpr (NV > 0) {
#pragma unroll
            for (int q = 0; q < NV; ++q)
                if (q == c) { w = ws[q]; d = ds_[q]; }
        } else {
            const int jj = j < L ? j : 0;
            const f32x4 p = *reinterpret_cast<const f32x4*>(a.p + off + jj);
            d = *reinterpret_cast<const f32x4*>(a.dp + off + jj);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = wt(p[i]);
        }
        f32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = w[i] * (d[i] - cc);
        if (j < L) __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(a.ds + off + j));
    }
}

}  // namespace ea
