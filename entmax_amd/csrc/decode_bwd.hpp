// Backward of the decode-time forward (query length Lq at or below the key
// length: the newest Lq queries of each sequence against its key/value
// cache), from the forward's tau.  Jacobian of "ADASPLASH -- ROBERTA
// Benchmark Result", section 2.4: per query row, w_j = sqrt(p_j) =
// [(s_j - tau)/2]_+, dp_j = dO . v_j, c = sum w dp / sum w and
// dS_j = w_j (dp_j - c); dq = scale sum_j dS_j k_j, and each key j of the
// row's key/value head gets scale dS_j q (dk) and p_j dO (dv).
//
//   1. dec_scores_kernel (decode.hpp) writes every row's scores of its span
//      [lo_b, n_b) to the workspace (scaled; -inf where not allowed).
//   2. dec_bwd_rows_kernel: one wave per query row.  The support (w > 0)
//      is found 64 keys at a time by ballot; its keys are taken four at a
//      time, their V rows (then K rows) read by the whole wave, lane l on
//      features l, l + 64.  A first pass forms c, a second forms dS (written
//      to the workspace next to the scores) and dq.
//   3. dec_bwd_keys_kernel: one wave per key of a key/value head: dk and dv
//      sum the rows of the head's group (its query heads times Lq) in row
//      order, reading q and dO only for rows whose p at the key is nonzero;
//      keys outside every row's span get zero.
// Every output row is summed by one wave in a fixed order: no atomics, and
// repeated calls give identical bits.
#pragma once

#include "common.hpp"
#include "decode.hpp"

namespace ea {

struct DecBwdArgs {
    DecArgs f;            // q, k, v, seqlens, sbuf (scores), row_len, shapes
    const float* tau;     // [B, H, Lq] from the forward
    const void* dout;     // [B, H, Lq, d]
    float* dq;            // [B, H, Lq, d]
    float* dk;            // [B, Hkv, S, d]
    float* dv;            // [B, Hkv, S, d]
    float* dsbuf;         // [rows, P] dS of every (row, key of its span) with w > 0
};

// Features f = lane + 64 e of a row (D / 64 per lane), as float.
template <int DT, int D> struct WRow;
template <int D> struct WRow<DT_BF16, D> {
    static constexpr int E = D / 64;
    float x[E];
    __device__ __forceinline__ void load(const uint16_t* row, int lane) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = bf16_bits_to_f32(row[lane + 64 * e]);
    }
};
template <int D> struct WRow<DT_F32, D> {
    static constexpr int E = D / 64;
    float x[E];
    __device__ __forceinline__ void load(const float* row, int lane) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = row[lane + 64 * e];
    }
};

// Row r (global: (b H + h) Lq + i) of the decode form: its batch, key/value
// head and the span [lo, n) of its sequence.
__device__ __forceinline__ void dec_row_span(const DecArgs& a, int r, int* bk, int* lo, int* n) {
    const int b = r / (a.H * a.Lq);
    const int h = (r / a.Lq) % a.H;
    *bk = b * a.Hkv + h / (a.H / a.Hkv);
    dec_span(a, b, lo, n);
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void dec_bwd_rows_kernel(DecBwdArgs a) {
    using T = typename InT<DT>::type;
    constexpr int E = D / 64;
    const DecArgs& f = a.f;
    const int lane = threadIdx.x % kWave;
    const int row = blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (row >= f.B * f.H * f.Lq) return;   // uniform over the wave
    int bk, lo, n;
    dec_row_span(f, row, &bk, &lo, &n);
    const int span = n - lo;
    const float tq = a.tau[row];
    const float* sr = f.sbuf + static_cast<size_t>(row) * f.P;
    float* dsr = a.dsbuf + static_cast<size_t>(row) * f.P;
    const T* kh = static_cast<const T*>(f.k) + static_cast<size_t>(bk) * f.S * D;
    const T* vh = static_cast<const T*>(f.v) + static_cast<size_t>(bk) * f.S * D;
    WRow<DT, D> dor;
    dor.load(static_cast<const T*>(a.dout) + static_cast<size_t>(row) * D, lane);

    // w of key lo + r (0 off the support and past the span)
    auto wkey = [&](int r) { return r < span ? fmaxf(0.5f * (sr[r] - tq), 0.f) : 0.f; };
    // fn(keys[4], w[4], dp[4]) for the support of every 64-key chunk, four
    // keys at a time (unused slots: key 0, w = 0, dp = 0), in key order
    auto support = [&](auto&& fn) {
        for (int c0 = 0; c0 < span; c0 += kWave) {
            const float wl = wkey(c0 + lane);
            unsigned long long m = __ballot(wl > 0.f);
            while (m != 0ull) {
                int key[4];
                float w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool ok = m != 0ull;
                    const int l = ok ? __builtin_ctzll(m) : 0;
                    key[u] = ok ? c0 + l : 0;
                    w[u] = __shfl(wl, l, kWave);
                    w[u] = ok ? w[u] : 0.f;
                    m = ok ? m & (m - 1ull) : m;
                }
                WRow<DT, D> vr[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) vr[u].load(vh + static_cast<size_t>(lo + key[u]) * D, lane);
                float dp[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) part = fmaf(dor.x[e], vr[u].x[e], part);
                    dp[u] = wave_sum(part);
                }
                fn(key, w, dp);
            }
        }
    };

    // pass 1: sum w and sum w dp
    float sw = 0.f, swdp = 0.f;
    support([&](const int (&)[4], const float (&w)[4], const float (&dp)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sw += w[u];
            swdp = fmaf(w[u], dp[u], swdp);
        }
    });
    const float cc = sw > 0.f ? swdp / sw : 0.f;

    // pass 2: dS (to the workspace) and dq = scale sum dS k
    float dq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) dq[e] = 0.f;
    support([&](const int (&key)[4], const float (&w)[4], const float (&dp)[4]) {
        WRow<DT, D> kr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kr[u].load(kh + static_cast<size_t>(lo + key[u]) * D, lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float ds = w[u] * (dp[u] - cc);   // 0 for unused slots (w = 0)
            if (w[u] > 0.f && lane == 0) dsr[key[u]] = ds;
#pragma unroll
            for (int e = 0; e < E; ++e) dq[e] = fmaf(ds, kr[u].x[e], dq[e]);
        }
    });
    float* dqr = a.dq + static_cast<size_t>(row) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) dqr[lane + 64 * e] = f.scale * dq[e];
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void dec_bwd_keys_kernel(DecBwdArgs a) {
    using T = typename InT<DT>::type;
    constexpr int E = D / 64;
    const DecArgs& f = a.f;
    const int lane = threadIdx.x % kWave;
    const int bk = blockIdx.y;
    const int j = blockIdx.x * (kThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (j >= f.S) return;   // uniform over the wave
    const int b = bk / f.Hkv;
    int lo, n;
    dec_span(f, b, &lo, &n);
    const int GL = (f.H / f.Hkv) * f.Lq;
    const int rb = bk * GL;   // first global row of the group
    float dk[E], dv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { dk[e] = 0.f; dv[e] = 0.f; }
    if (j >= lo && j < n) {   // uniform
        const int r = j - lo;
        for (int jl = 0; jl < GL; ++jl) {
            const int row = rb + jl;
            const float w = fmaxf(0.5f * (f.sbuf[static_cast<size_t>(row) * f.P + r] - a.tau[row]), 0.f);
            if (w > 0.f) {   // uniform: one key, one row
                const float ds = a.dsbuf[static_cast<size_t>(row) * f.P + r];
                WRow<DT, D> qr, dr;
                qr.load(static_cast<const T*>(f.q) + static_cast<size_t>(row) * D, lane);
                dr.load(static_cast<const T*>(a.dout) + static_cast<size_t>(row) * D, lane);
                const float p = w * w;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    dk[e] = fmaf(ds, qr.x[e], dk[e]);
                    dv[e] = fmaf(p, dr.x[e], dv[e]);
                }
            }
        }
    }
    const size_t o = (static_cast<size_t>(bk) * f.S + j) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        a.dk[o + lane + 64 * e] = f.scale * dk[e];
        a.dv[o + lane + 64 * e] = dv[e];
    }
}

}  // namespace ea
