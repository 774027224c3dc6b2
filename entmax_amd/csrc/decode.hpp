// Decode-time forward: the newest Lq queries of each sequence against a
// key/value cache (the causal decoders of "ADASPLASH -- ROBERTA Benchmark
// Result", section 3, with the splash window of the decoder configuration in
// section 7.1); Lq = 1 is one decode step, Lq > 1 a chunk of new tokens.
//
// Sequence b holds n_b cached positions, the queries' own included: query i
// sits at position n_b - Lq + i and may attend keys j <= that position (and
// j > position - W with a window W > 0); without the causal mask every one
// of the n_b keys.  The rows of a workgroup are the
// (query head, query) pairs that share one key/value head, 16 at a time.
// The keys any of them may attend, [lo_b, n_b), are split into chunks of 256
// so that a long cache spreads over many workgroups (a decode step has few
// query rows: the work is the HBM read of K and V).  Scores of keys a row
// may not attend are -inf, which the row solver counts as not allowed.
//   1. dec_scores: per (chunk, b, key/value head, row group): S = q K^T /
//      sqrt(d) on MFMA, written to a float32 row per query row, plus each
//      row's maximum over the chunk.
//   2. tau per row by the row-wise solver (rows.hpp).
//   3. dec_pv: per chunk, skipped whole (no V read) when no row of the group
//      has a score above its tau in the chunk; else the chunk's partial
//      O = P V on float32 MFMA.
//   4. dec_reduce: O = sum of the partials of the chunks that hold a score
//      above tau (the same test as step 3), one wave per row.
// Spans of at most 256 keys (the splash window, short caches) take one
// launch instead: dec_short_kernel keeps the scores of its group in LDS,
// solves each row with one wave (or 16 lanes) and forms O directly.
#pragma once

#include <type_traits>
#include <utility>

#include "col_solve.hpp"
#include "common.hpp"
#include "rows.hpp"

namespace ea {

constexpr int kDecChunk = 256;   // keys per workgroup, 64 per wave

struct DecArgs {
    const void* q;        // [B, H, Lq, d]
    const void* k;        // [B, Hkv, S, d]
    const void* v;        // [B, Hkv, S, d]
    const int* seqlens;   // [B]
    float* out;           // [B, H, Lq, d]
    float* tau_out;       // [B, H, Lq] or null
    // workspace (rows: the B H Lq query rows in the order of out)
    float* sbuf;          // [rows, P] scores, P = nch * 256
    float* cmax;          // [rows, nch] chunk maxima
    float* part;          // [rows, nch, d] partial outputs
    float* tau;           // [rows]
    int* row_len;         // [rows] span length of the row's sequence
    int B, H, Hkv, Lq, S, window;
    int causal;           // 0: every one of the n_b keys for every query (window 0)
    int nch, P;           // chunks of the longest possible span; row pitch of sbuf
    float scale;
};

// Keys [lo, n) of sequence b's cache that any of its queries may attend.
__device__ __forceinline__ void dec_span(const DecArgs& a, int b, int* lo, int* n) {
    int len = a.seqlens[b];
    len = len < 0 ? 0 : (len > a.S ? a.S : len);
    *n = len;
    const int first = len - a.Lq;   // position of query 0
    *lo = (a.causal && a.window > 0 && first - a.window + 1 > 0) ? first - a.window + 1 : 0;
}

// Group z of the rows served by one key/value head: local rows [j0, j1) of
// its G Lq (query head, query) pairs; the key/value head's rows start at
// global row bk G Lq.
__device__ __forceinline__ void dec_rows(const DecArgs& a, int z, int* j0, int* j1) {
    const int GL = (a.H / a.Hkv) * a.Lq;
    *j0 = 16 * z;
    *j1 = *j0 + 16 < GL ? *j0 + 16 : GL;
}

// Key k (< n) may be attended by local row j (query j % Lq) of a sequence
// of n: causal, query i at n - Lq + i; otherwise every key.
__device__ __forceinline__ bool dec_allowed(const DecArgs& a, int n, int j, int k) {
    if (!a.causal) return true;
    const int pos = n - a.Lq + j % a.Lq;
    return k <= pos && (a.window <= 0 || k > pos - a.window);
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void dec_scores_kernel(DecArgs a) {
    using T = typename InT<DT>::type;
    const int chunk = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.Hkv;
    const int rb = bk * (a.H / a.Hkv) * a.Lq;   // first global row of this key/value head
    int j0, j1, lo, n;
    dec_rows(a, blockIdx.z, &j0, &j1);
    dec_span(a, b, &lo, &n);
    const int span = n - lo;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave, g = lane / 16, c = lane % 16;
    if (chunk == 0 && tid < j1 - j0) a.row_len[rb + j0 + tid] = span;
    if (kDecChunk * chunk >= span) return;   // uniform over the workgroup

    // A operand: rows j0 + c (zero rows past j1)
    QFrag<DT, D> qf;
    qf.load(static_cast<const T*>(a.q) + static_cast<size_t>(rb) * D, j0 + c, j1, g);
    const T* kh = static_cast<const T*>(a.k) + static_cast<size_t>(bk) * a.S * D;

    float mx[4] = {-kInf, -kInf, -kInf, -kInf};
    const int r0 = kDecChunk * chunk + 64 * wv;   // first key of this wave, relative to lo
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = r0 + 16 * t + c;            // this lane's key (column c of the tile)
        const bool ok = r < span;
        // keys past the span read key n - 1 (valid: span > 0) and are masked
        const f32x4 acc = qf.tile(kh, ok ? lo + r : n - 1, n, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + 4 * g + i;
            const float s = ok && dec_allowed(a, n, j, lo + r) ? acc[i] * a.scale : -kInf;
            if (j < j1) a.sbuf[static_cast<size_t>(rb + j) * a.P + r] = s;
            mx[i] = fmaxf(mx[i], s);
        }
    }
    __shared__ float red[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float m = group_max<16>(mx[i]);
        if (c == 0) red[wv][4 * g + i] = m;
    }
    __syncthreads();
    if (tid < j1 - j0) {
        const float m = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
        a.cmax[static_cast<size_t>(rb + j0 + tid) * a.nch + chunk] = m;
    }
}

// Feature f of the output tile: lane c of feature tile ct serves feature
// c (D/16) + ct, so that each lane reads D/16 consecutive features of a V row
// (kept raw; f(ct) converts).
template <int DT, int D> struct VRow;
template <int D> struct VRow<DT_BF16, D> {
    static constexpr int N = D / 16;
    unsigned w[N / 2];
    __device__ __forceinline__ void load(const uint16_t* row, int c) {
        const uint16_t* p = row + N * c;
        if constexpr (N == 8) {
            const u32x4 u = *reinterpret_cast<const u32x4*>(p);
            w[0] = u[0]; w[1] = u[1]; w[2] = u[2]; w[3] = u[3];
        } else {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            w[0] = u.x; w[1] = u.y;
        }
    }
    __device__ __forceinline__ float f(int e) const {
        return __uint_as_float((e & 1) ? (w[e / 2] & 0xFFFF0000u) : (w[e / 2] << 16));
    }
};
template <int D> struct VRow<DT_F32, D> {
    static constexpr int N = D / 16;
    f32x4 w[N / 4];
    __device__ __forceinline__ void load(const float* row, int c) {
        const float* p = row + N * c;
#pragma unroll
        for (int e = 0; e < N / 4; ++e) w[e] = *reinterpret_cast<const f32x4*>(p + 4 * e);
    }
    __device__ __forceinline__ float f(int e) const { return w[e / 4][e % 4]; }
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void dec_pv_kernel(DecArgs a) {
    using T = typename InT<DT>::type;
    constexpr int NF = D / 16;
    const int chunk = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.Hkv;
    const int rb = bk * (a.H / a.Hkv) * a.Lq;
    int j0, j1, lo, n;
    dec_rows(a, blockIdx.z, &j0, &j1);
    dec_span(a, b, &lo, &n);
    const int span = n - lo;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave, g = lane / 16, c = lane % 16;
    if (kDecChunk * chunk >= span) return;   // uniform
    // skip the chunk when every row's scores in it lie at or below its tau
    bool act = false;
    if (tid < j1 - j0) {
        const int row = rb + j0 + tid;
        act = a.cmax[static_cast<size_t>(row) * a.nch + chunk] > a.tau[row];
    }
    if (!__syncthreads_or(act)) return;

    // lane (g, c): A[c][g] = p of row j0 + c at key r0 + 16 g + s (step s);
    // B[g][c] = V at that key, features c NF .. c NF + NF - 1
    const int r0 = kDecChunk * chunk + 64 * wv;
    float p[16];
    {
        const bool rok = j0 + c < j1;
        const int row = rb + (rok ? j0 + c : j0);
        const float tq = a.tau[row];
        const float* sp = a.sbuf + static_cast<size_t>(row) * a.P + r0 + 16 * g;
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(sp + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float y = relu1(0.5f * (s4[i] - tq));
                p[e + i] = rok ? y * y : 0.f;   // keys not attended hold -inf: p = 0
            }
        }
    }
    const T* vh = static_cast<const T*>(a.v) + static_cast<size_t>(bk) * a.S * D;
    f32x4 o[NF];
#pragma unroll
    for (int ct = 0; ct < NF; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        // a step whose four keys have p = 0 in every row of the group adds
        // nothing: its V rows are not read (sparse rows leave most steps so)
        if (!__any(p[s] > 0.f)) continue;   // uniform
        const int r = r0 + 16 * g + s;
        VRow<DT, D> vr;
        vr.load(vh + static_cast<size_t>(r < span ? lo + r : n - 1) * D, c);   // past the span: p = 0
#pragma unroll
        for (int ct = 0; ct < NF; ++ct) o[ct] = mfma_f32(p[s], vr.f(ct), o[ct]);
    }
    // lane (g, c) holds O[row 4 g + i][feature c NF + ct]; sum the four waves
    __shared__ float red[4][16][D];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < NF; ++ct) red[wv][4 * g + i][c * NF + ct] = o[ct][i];
    __syncthreads();
    const int ng = j1 - j0;
    for (int e = tid; e < ng * D; e += kThreads) {
        const int jr = e / D, f = e - jr * D;
        const float sum = (red[0][jr][f] + red[1][jr][f]) + (red[2][jr][f] + red[3][jr][f]);
        a.part[(static_cast<size_t>(rb + j0 + jr) * a.nch + chunk) * D + f] = sum;
    }
}

// One wave per row: O = sum over the chunks holding a score above tau, in
// chunk order.  Lane l tests chunk c0 + l; the partials of the active chunks
// are then loaded four at a time, so that their loads are in flight together.
template <int D>
__global__ __launch_bounds__(kThreads) void dec_reduce_kernel(DecArgs a) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x % kWave;
    const int row = blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (row >= a.B * a.H * a.Lq) return;
    const int span = a.row_len[row];
    const float t = a.tau[row];
    const int nc = (span + kDecChunk - 1) / kDecChunk;
    const float* pr = a.part + static_cast<size_t>(row) * a.nch * D;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    for (int c0 = 0; c0 < nc; c0 += kWave) {
        const int ch = c0 + lane;
        const bool act = ch < nc && a.cmax[static_cast<size_t>(row) * a.nch + ch] > t;
        unsigned long long m = __ballot(act);
        while (m != 0ull) {
            int idx[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ok[u] = m != 0ull;
                idx[u] = ok[u] ? c0 + __builtin_ctzll(m) : c0;
                m = ok[u] ? m & (m - 1ull) : m;
            }
            float v[4][E];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e) v[u][e] = pr[static_cast<size_t>(idx[u]) * D + 64 * e + lane];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[e] += ok[u] ? v[u][e] : 0.f;   // unused slots: discarded
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) a.out[static_cast<size_t>(row) * D + 64 * e + lane] = acc[e];
    if (a.tau_out != nullptr && lane == 0) a.tau_out[row] = t;
}

// Whole decode step for spans of at most 256 keys: one workgroup per
// (b, key/value head, group of up to 16 rows).  Scores into LDS as in
// dec_scores; each row is solved by the register bisection of the row-wise
// op (one f32x4 per lane: 16 lanes per row when the span is at most 64
// keys, four rows per wave at once, else a wave per row) and overwritten
// with p; then P V as in dec_pv, summed over the four waves.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void dec_short_kernel(DecArgs a) {
    using T = typename InT<DT>::type;
    constexpr int NF = D / 16;
    constexpr int SP = kDecChunk + 4;             // LDS row pitch of the scores
    const int bk = blockIdx.x;
    const int b = bk / a.Hkv;
    const int rb = bk * (a.H / a.Hkv) * a.Lq;
    int j0, j1, lo, n;
    dec_rows(a, blockIdx.y, &j0, &j1);
    dec_span(a, b, &lo, &n);
    const int span = n - lo;                      // <= 256 (checked by the host)
    const int ng = j1 - j0;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave, g = lane / 16, c = lane % 16;
    if (span == 0) {   // uniform: nothing to attend
        for (int e = tid; e < ng * D; e += kThreads) a.out[static_cast<size_t>(rb + j0) * D + e] = 0.f;
        if (a.tau_out != nullptr && tid < ng) a.tau_out[rb + j0 + tid] = kInf;
        return;
    }
    __shared__ float Ss[16][SP];
    __shared__ float red[4][16][D];

    // 1. scores of keys 64 w .. 64 w + 63 of the span (-inf where not attended)
    {
        QFrag<DT, D> qf;
        qf.load(static_cast<const T*>(a.q) + static_cast<size_t>(rb) * D, j0 + c, j1, g);
        const T* kh = static_cast<const T*>(a.k) + static_cast<size_t>(bk) * a.S * D;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 64 * wv + 16 * t + c;
            const bool live = 64 * wv + 16 * t < span;   // uniform: the tile holds a key of the span
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (live) acc = qf.tile(kh, r < span ? lo + r : n - 1, n, g);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Ss[4 * g + i][r] = r < span && dec_allowed(a, n, j0 + 4 * g + i, lo + r) ? acc[i] * a.scale : -kInf;
        }
    }
    __syncthreads();

    // V rows of this wave's keys, in flight during the solve
    const bool pv_live = 64 * wv < span;   // uniform
    VRow<DT, D> vr[16];
    if (pv_live) {
        const T* vh = static_cast<const T*>(a.v) + static_cast<size_t>(bk) * a.S * D;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int r = 64 * wv + 16 * g + s;
            vr[s].load(vh + static_cast<size_t>(r < span ? lo + r : n - 1) * D, c);   // past the span: p = 0
        }
    }

    // 2. tau per row; p = [(s - tau)/2]_+^2 replaces the scores.  Entries of
    // -inf are keys the row may not attend: they do not count in n.
    auto sq = [](float y) { return y * y; };
    auto solve_row = [&](f32x4 (&xs)[1], auto&& rmax, auto&& rsum, auto tpr) {
        constexpr int TPR = decltype(tpr)::value;
        float cnt = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt += xs[0][i] > -kInf ? 1.f : 0.f;
        const float nr = rsum(cnt);
        const float m = rmax(fmaxf(fmaxf(xs[0][0], xs[0][1]), fmaxf(xs[0][2], xs[0][3])));
        if (nr == 0.f)   // no key: p = 0, tau = +inf (uniform over the row's lanes)
            return std::pair<f32x4, float>(f32x4{0.f, 0.f, 0.f, 0.f}, kInf);
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[0][i] = xs[0][i] > -kInf ? 0.5f * (xs[0][i] - m) : -kInf;
        const float tt = bisect_regs<1, false, TPR>(xs, nr, 0.5f, sq, rsum);
        f32x4 p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y = relu1(xs[0][i] - tt);
            p[i] = y * y;
        }
        return std::pair<f32x4, float>(p, m + 2.f * tt);
    };
    if (span <= 64) {
        // one row per 16 lanes: wave w solves rows 4 w .. 4 w + 3 at once
        const int jr = 4 * wv + g, l = lane % 16;
        if (4 * wv < ng) {   // uniform
            f32x4 xs[1];
            xs[0] = *reinterpret_cast<const f32x4*>(&Ss[jr][4 * l]);
            const auto r = solve_row(xs, [](float v) { return row_max<16>(v); },
                                     [](float v) { return row_sum<16>(v); }, std::integral_constant<int, 16>());
            if (jr < ng) {
                *reinterpret_cast<f32x4*>(&Ss[jr][4 * l]) = r.first;
                if (l == 0 && a.tau_out != nullptr) a.tau_out[rb + j0 + jr] = r.second;
            }
        }
    } else {
        // one row per wave: wave w solves rows w, w + 4, ...
        for (int jr = wv; jr < ng; jr += 4) {
            f32x4 xs[1];
            xs[0] = *reinterpret_cast<const f32x4*>(&Ss[jr][4 * lane]);
            const auto r = solve_row(xs, [](float v) { return wave_max(v); },
                                     [](float v) { return wave_sum(v); }, std::integral_constant<int, kWave>());
            *reinterpret_cast<f32x4*>(&Ss[jr][4 * lane]) = r.first;
            if (lane == 0 && a.tau_out != nullptr) a.tau_out[rb + j0 + jr] = r.second;
        }
    }
    __syncthreads();

    // 3. O = P V: lane (g, c) holds p of row j0 + c at key 64 w + 16 g + s
    f32x4 o[NF];
#pragma unroll
    for (int ct = 0; ct < NF; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (pv_live) {
        const float* pr = &Ss[c < ng ? c : 0][64 * wv + 16 * g];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const float ps = c < ng ? pr[s] : 0.f;   // keys not attended hold p = 0
#pragma unroll
            for (int ct = 0; ct < NF; ++ct) o[ct] = mfma_f32(ps, vr[s].f(ct), o[ct]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < NF; ++ct) red[wv][4 * g + i][c * NF + ct] = o[ct][i];
    __syncthreads();
    for (int e = tid; e < ng * D; e += kThreads) {
        const int jr = e / D, f = e - jr * D;
        a.out[static_cast<size_t>(rb + j0 + jr) * D + f] = (red[0][jr][f] + red[1][jr][f]) + (red[2][jr][f] + red[3][jr][f]);
    }
}

}  // namespace ea
