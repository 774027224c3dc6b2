// Backward pass of 1.5-entmax attention, driven by the forward's tau.
//
// Jacobian ("ADASPLASH -- ROBERTA Benchmark Result", section 2.4; "RoBERTa
// Base with AdaSplash Attention" model card, Mathematical Formulation 2): with
// w_ij = sqrt(p_ij) = (s_ij - tau_i)/2 on the support and dp_ij = dO_i . V_j,
//   c_i = sum_j w_ij dp_ij / sum_j w_ij,   dS_ij = w_ij (dp_ij - c_i),
//   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i,
//   dV_j = sum_i p_ij dO_i.
// Everything off the support is exactly zero, so only the scores need a
// dense pass: one workgroup = 4 independent waves of 16 query rows; each
// wave recomputes S tile by tile on MFMA (same tile code as the forward),
// and handles every support entry as it appears:
//   dp_ij by a gather of V_j and a 16-lane dot product with dO_i,
//   sum w, sum w dp, X_i = sum w dp K_j and Y_i = sum w K_j,
// so that dQ_i = scale (X_i - c_i Y_i) needs no second pass.  The entries
// (key, w, dp) are kept in an LDS list; after c_i is known each entry adds
// scale dS_ij Q_i to dK_j and p_ij dO_i to dV_j with fp32 atomics.  A row
// whose support outgrows its list redoes the score pass for that step.
#pragma once

#include "common.hpp"
#include "fwd_stream.hpp"
#include "tau_solver.hpp"

namespace ea {

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const uint8_t* key_mask;
    const float* tau;
    const void* dout;
    float* dq;
    float* dk;
    float* dv;
    int B, H, L;
    int causal, window;
    float scale;
    int nqt;
};

template <int CAP>
struct BwdCfg {
    static constexpr int BM = 64;
    static constexpr size_t lds_bytes = static_cast<size_t>(BM) * CAP * (2 * sizeof(float) + sizeof(uint16_t));
};

template <int DT, int DPL>
__device__ __forceinline__ void load_row_slice(const typename InT<DT>::type* p, float (&x)[DPL]) {
    if constexpr (DT == DT_BF16) {
#pragma unroll
        for (int j = 0; j < DPL; j += 4) {
            const uint2 u = *reinterpret_cast<const uint2*>(p + j);
            x[j + 0] = __uint_as_float(u.x << 16);
            x[j + 1] = __uint_as_float(u.x & 0xFFFF0000u);
            x[j + 2] = __uint_as_float(u.y << 16);
            x[j + 3] = __uint_as_float(u.y & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int j = 0; j < DPL; j += 4) {
            const f32x4 u = *reinterpret_cast<const f32x4*>(p + j);
#pragma unroll
            for (int q = 0; q < 4; ++q) x[j + q] = u[q];
        }
    }
}

__global__ void zero_fill_kernel(float* p, size_t n) {
    const size_t i = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
    if (i + 3 < n) {
        *reinterpret_cast<f32x4*>(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        for (size_t j = i; j < n; ++j) p[j] = 0.f;
    }
}

template <int DT, int D, int CAP>
__global__ __launch_bounds__(kThreads) void bwd_kernel(BwdArgs a) {
    typedef typename InT<DT>::type T;
    constexpr int DPL = D / 16;
    constexpr int BM = BwdCfg<CAP>::BM;
    extern __shared__ float lds[];
    float* lw = lds;                       // [BM][CAP] w
    float* ldp = lw + BM * CAP;            // [BM][CAP] dp
    uint16_t* lk = reinterpret_cast<uint16_t*>(ldp + BM * CAP);   // [BM][CAP] key

    const int total = a.B * a.H * a.nqt;
    const int wi = xcd_swizzle(blockIdx.x, total);
    const int bh = wi / a.nqt;
    const int qt = wi - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * BM;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const T* kh = static_cast<const T*>(a.k) + head_off;
    const T* vh = static_cast<const T*>(a.v) + head_off;
    const T* doh = static_cast<const T*>(a.dout) + head_off;
    float* dqh = a.dq + head_off;
    float* dkh = a.dk + head_off;
    float* dvh = a.dv + head_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wv = tid / kWave;
    const int g = lane / 16, c = lane % 16;
    const int r0 = 16 * wv;

    int klo, khi;
    key_range(q0 + r0, 16, L, a.causal, a.window, &klo, &khi);
    const int kt0 = klo / kBN;
    const int ntile = khi > klo ? (khi + kBN - 1) / kBN - kt0 : 0;

    QFrag<DT, D> qf;
    qf.load(qh, q0 + r0 + c, L, g);

    float tau[4], dor[4][DPL], qr[4][DPL], X[4][DPL], Y[4][DPL], sw[4], swdp[4];
    int cnt[4];
    bool ovf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = q0 + r0 + 4 * g + i;
        const bool in = row < L;
        tau[i] = in ? a.tau[static_cast<size_t>(bh) * L + row] : kInf;
#pragma unroll
        for (int j = 0; j < DPL; ++j) { dor[i][j] = 0.f; qr[i][j] = 0.f; X[i][j] = 0.f; Y[i][j] = 0.f; }
        if (in) {
            load_row_slice<DT, DPL>(doh + static_cast<size_t>(row) * D + DPL * c, dor[i]);
            load_row_slice<DT, DPL>(qh + static_cast<size_t>(row) * D + DPL * c, qr[i]);
        }
        sw[i] = 0.f;
        swdp[i] = 0.f;
        cnt[i] = 0;
        ovf[i] = false;
    }

    // key validity without a branch around the mask load (see common.hpp)
    auto key_ok = [&](int key) {
        const bool in = key < L;
        if (km == nullptr) return in;
        const uint8_t mb = km[clamp_row(key, L)];   // unconditional load
        return in && mb != 0;
    };
    auto score = [&](int key, bool kv, const f32x4& acc, int i) {
        const int row = q0 + r0 + 4 * g + i;
        const bool ok = kv && row < L && allowed_ij(row, key, a.causal, a.window);
        return ok ? acc[i] * a.scale : -kInf;
    };
    auto dot_dp = [&](int i, int key) {
        float vr[DPL];
        load_row_slice<DT, DPL>(vh + static_cast<size_t>(key) * D + DPL * c, vr);
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) part = fmaf(dor[i][j], vr[j], part);
        return row_sum<16>(part);
    };
    // Insert this tile's support entries of row i at positions [base, ...).
    auto insert = [&](int i, int base, const float (&s)[4][4], int kbase, bool active) {
        const int rl = r0 + 4 * g + i;
        int added = 0;
#pragma unroll
        for (int c16 = 0; c16 < 4; ++c16) {
            const float x = s[c16][i] - tau[i];
            const bool pred = active && x > 0.f;
            int rank, tot;
            group_rank(__ballot(pred), g, c, &rank, &tot);
            if (pred) {
                lk[rl * CAP + base + added + rank] = static_cast<uint16_t>(kbase + 16 * c16 + c);
                lw[rl * CAP + base + added + rank] = 0.5f * x;
            }
            added += tot;
        }
        return added;
    };

    // ---- pass 1: support, dp, row sums, X and Y ------------------------------
    for (int t = 0; t < ntile; ++t) {
        const int kbase = (kt0 + t) * kBN;
        float s[4][4];
#pragma unroll
        for (int c16 = 0; c16 < 4; ++c16) {
            const int key = kbase + 16 * c16 + c;
            const bool kv = key_ok(key);
            const f32x4 acc = qf.tile(kh, key, L, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) s[c16][i] = score(key, kv, acc, i);
        }
        int from[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (cnt[i] + kBN > CAP) {   // no room for a full tile: keep only a staging window
                ovf[i] = true;
                cnt[i] = 0;
            }
            from[i] = cnt[i];
            cnt[i] += insert(i, cnt[i], s, kbase, true);
        }
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = r0 + 4 * g + i;
            for (int e = from[i]; e < cnt[i]; ++e) {
                const int key = lk[rl * CAP + e];
                const float w = lw[rl * CAP + e];
                const float dp = dot_dp(i, key);
                if (c == 0) ldp[rl * CAP + e] = dp;
                sw[i] += w;
                swdp[i] = fmaf(w, dp, swdp[i]);
                float kr[DPL];
                load_row_slice<DT, DPL>(kh + static_cast<size_t>(key) * D + DPL * c, kr);
                const float wdp = w * dp;
#pragma unroll
                for (int j = 0; j < DPL; ++j) {
                    X[i][j] = fmaf(wdp, kr[j], X[i][j]);
                    Y[i][j] = fmaf(w, kr[j], Y[i][j]);
                }
            }
        }
        wave_sync();
    }

    // ---- dQ ------------------------------------------------------------------
    float cc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cc[i] = sw[i] > 0.f ? swdp[i] / sw[i] : 0.f;
        const int row = q0 + r0 + 4 * g + i;
        if (row < L) {
            float* dst = dqh + static_cast<size_t>(row) * D + DPL * c;
#pragma unroll
            for (int j = 0; j < DPL; j += 4)
                *reinterpret_cast<f32x4*>(dst + j) =
                    f32x4{a.scale * fmaf(-cc[i], Y[i][j], X[i][j]), a.scale * fmaf(-cc[i], Y[i][j + 1], X[i][j + 1]),
                          a.scale * fmaf(-cc[i], Y[i][j + 2], X[i][j + 2]), a.scale * fmaf(-cc[i], Y[i][j + 3], X[i][j + 3])};
        }
    }

    // ---- pass 2: scatter dK, dV -----------------------------------------------
    auto scatter = [&](int i, int key, float w, float dp) {
        const float ds = a.scale * w * (dp - cc[i]);
        const float p = w * w;
        float* dkr = dkh + static_cast<size_t>(key) * D + DPL * c;
        float* dvr = dvh + static_cast<size_t>(key) * D + DPL * c;
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
            unsafeAtomicAdd(dkr + j, ds * qr[i][j]);
            unsafeAtomicAdd(dvr + j, p * dor[i][j]);
        }
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (ovf[i]) continue;
        const int rl = r0 + 4 * g + i;
        for (int e = 0; e < cnt[i]; ++e) scatter(i, lk[rl * CAP + e], lw[rl * CAP + e], ldp[rl * CAP + e]);
    }
    const bool my_ovf = ovf[0] || ovf[1] || ovf[2] || ovf[3];
    if (__any(my_ovf)) {
        wave_sync();
        for (int t = 0; t < ntile; ++t) {
            const int kbase = (kt0 + t) * kBN;
            float s[4][4];
#pragma unroll
            for (int c16 = 0; c16 < 4; ++c16) {
                const int key = kbase + 16 * c16 + c;
                const bool kv = key_ok(key);
                const f32x4 acc = qf.tile(kh, key, L, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) s[c16][i] = score(key, kv, acc, i);
            }
            int n_in[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) n_in[i] = insert(i, 0, s, kbase, ovf[i]);
            wave_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = r0 + 4 * g + i;
                for (int e = 0; e < n_in[i]; ++e) {
                    const int key = lk[rl * CAP + e];
                    const float w = lw[rl * CAP + e];
                    scatter(i, key, w, dot_dp(i, key));
                }
            }
            wave_sync();
        }
    }
}

}  // namespace ea
