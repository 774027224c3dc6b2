// Backward pass of 1.5-entmax attention, driven by the forward's tau: the
// query side (dQ and the per-row constant c_i).
//
// Jacobian ("ADASPLASH -- ROBERTA Benchmark Result", section 2.4; "RoBERTa
// Base with AdaSplash Attention" model card, Mathematical Formulation 2): with
// w_ij = sqrt(p_ij) = (s_ij - tau_i)/2 on the support and dp_ij = dO_i . V_j,
//   c_i = sum_j w_ij dp_ij / sum_j w_ij,   dS_ij = w_ij (dp_ij - c_i),
//   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i,
//   dV_j = sum_i p_ij dO_i.
// Everything off the support is exactly zero, so only the scores need a
// dense pass.  This kernel owns query rows: it writes dQ_i and c_i (to the
// caller's workspace); dK and dV are formed by key-owning workgroups in
// bwd_wide.hpp from the same c_i, so no two workgroups ever add into one
// gradient row and the result does not depend on timing.
// One workgroup = 4 waves of 16 query rows of one (batch, head); lane (g, c)
// of a wave holds rows 4g .. 4g + 3 of each 16 x 16 score tile (key c) and
// the d-slice [c D/16, (c + 1) D/16) of those rows' dO.
//   1. S is recomputed on MFMA from K chunks staged in LDS (chunk_stream.hpp,
//      one buffer, loads one chunk ahead) and every support entry (key, w)
//      goes to its row's list in LDS.
//   2. Per row, the entries are processed in batches of NB = 2 (V and K row
//      gathers of a batch are issued before any is used): dp by a 16-lane
//      dot product, then sum w, sum w dp, X = sum w dp K_j, Y = sum w K_j,
//      and dQ_i = scale (X - c_i Y) without another pass.
// A row whose support outgrows its list is finished by two more passes over
// the keys (all waves take part, only those rows do work): one for dp and the
// sums, one for dQ_i = scale sum_j dS_ij K_j once c_i is known (for a long
// support the difference X - c_i Y would cost digits).
// In fix-up mode (args.fixup) a workgroup only runs when one of its rows
// carries the overflow marker (kCMarker in c_i) left by the wide query-side kernel,
// and then recomputes dQ and c for its whole tile.
#pragma once

#include "chunk_stream.hpp"
#include "common.hpp"
#include "fwd_short.hpp"
#include "dpp.hpp"

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
    float* cbuf;   // [B, H, L] c_i (workspace)
    // support buckets of the key side (long spans; null otherwise):
    // kcnt [B, H_kv, L] entries appended per key (zero before the query
    // side), kflag: set when some query row could not append its entries
    int* kcnt;
    int* kflag;
    int B, H, L;
    int Hkv;   // key/value heads (H % Hkv == 0)
    int causal, window;
    float scale;
    int nqt;
    int fixup;     // run only for tiles holding an overflow marker in c_i
    // the support saved by the forward (long spans; see FwdArgs), read by
    // the query side instead of recomputing the scores
    const int* scount;
    const float* sent;
};

template <int DT, int D>
struct BwdCfg : ChunkCfg<DT, D> {
    typedef ChunkCfg<DT, D> S;
    static constexpr int BM = 64;
    // support entries per row; with one K chunk buffer (ChunkStream<.., 1>)
    // a bf16 d = 128 workgroup takes under a third of the LDS
    static constexpr int CAP = 48;
    static constexpr int NB = 2;     // entries per gather batch
    static constexpr size_t list_bytes = static_cast<size_t>(BM) * CAP * (sizeof(float) + sizeof(uint16_t));
    static constexpr size_t lds_bytes = S::k_bytes + list_bytes + 64;
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

// Rank of this lane among the set lanes of its 16-lane group in `mask`.
__device__ __forceinline__ void group_rank16(unsigned long long mask, int g, int c, int* rank, int* total) {
    const unsigned gm = static_cast<unsigned>((mask >> (16 * g)) & 0xFFFFull);
    *rank = __popc(gm & ((1u << c) - 1u));
    *total = __popc(gm);
}

// Overflow marker left in c_i by the wide query-side kernel for rows it
// could not finish (a quiet-NaN bit pattern, compared as an integer: the
// library is built without NaN semantics, and no computed c_i has these bits).
constexpr unsigned kCMarker = 0x7FC0DEADu;

// True (in every thread) when one of rows [q0, q0 + n) of head bh carries
// the overflow marker.  Called by the whole workgroup.
__device__ __forceinline__ bool tile_marked(const float* cbuf, size_t bh, int L, int q0, int n, int* flag) {
    const int t = threadIdx.x;
    if (t == 0) *flag = 0;
    __syncthreads();
    if (t < n && q0 + t < L) {
        if (reinterpret_cast<const unsigned*>(cbuf)[bh * L + q0 + t] == kCMarker) atomicOr(flag, 1);
    }
    __syncthreads();
    const bool r = *flag != 0;
    __syncthreads();
    return r;
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads, (DT == DT_BF16 ? 3 : 2)) void bwd_kernel(BwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef BwdCfg<DT, D> C;
    constexpr int DPL = D / 16, BM = C::BM, CAP = C::CAP, NB = C::NB, CK = C::S::CK;
    // the overflow passes stage one chunk's entries of four rows (one per
    // lane group) in the four lists of that lane group's rows
    static_assert(4 * CAP >= CK, "a chunk's entries of one row fit the staging window");
    extern __shared__ float lds[];
    char* Kb = reinterpret_cast<char*>(lds);
    float* lw = reinterpret_cast<float*>(Kb + C::S::k_bytes);        // [BM][CAP] w
    uint16_t* lk = reinterpret_cast<uint16_t*>(lw + BM * CAP);        // [BM][CAP] key
    int* flag = reinterpret_cast<int*>(lk + BM * CAP);                // workgroup vote

    const int total = a.B * a.H * a.nqt;
    const int wi = xcd_swizzle(blockIdx.x, total);
    const int bh = wi / a.nqt;
    const int qt = wi - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * BM;
    const int L = a.L;
    if (a.fixup && !tile_marked(a.cbuf, static_cast<size_t>(bh), L, q0, BM, flag)) return;   // uniform
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const T* vh = static_cast<const T*>(a.v) + kv_off;
    const T* doh = static_cast<const T*>(a.dout) + head_off;
    float* dqh = a.dq + head_off;
    float* ch = a.cbuf + static_cast<size_t>(bh) * L;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;
    const bool hasm = km != nullptr;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane / 16, c = lane % 16;
    const int r0 = 16 * wv;

    int klo, khi;
    key_range(q0, BM, L, a.causal, a.window, &klo, &khi);
    const int ch0 = klo / CK, ch1 = (khi + CK - 1) / CK;
    int wlo, whi;
    key_range(q0 + r0, 16, L, a.causal, a.window, &wlo, &whi);

    ChunkStream<DT, D, 1, 1> cs;
    cs.Kb = Kb;
    cs.Vb = nullptr;
    cs.kh = kh;
    cs.vh = vh;
    cs.kmp = hasm ? km : reinterpret_cast<const uint8_t*>(qh);
    cs.hasm = hasm;
    cs.L = L;
    cs.tid = tid;
    cs.lane = lane;

    QFrag<DT, D> qf;
    qf.load(qh, q0 + r0 + c, L, g);

    float tau[4];
    int cnt[4];
    bool ovf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = q0 + r0 + 4 * g + i;
        tau[i] = row < L ? a.tau[static_cast<size_t>(bh) * L + clamp_row(row, L)] : kInf;
        cnt[i] = 0;
        ovf[i] = false;
    }
    // this lane's d-slice of dO for row 4g + i (loaded when the row is processed)
    float dor[DPL];
    auto load_row = [&](int i) {
        const int row = clamp_row(q0 + r0 + 4 * g + i, L);
        load_row_slice<DT, DPL>(doh + static_cast<size_t>(row) * D + DPL * c, dor);
    };

    // Support entries of one chunk for this wave: calls put(i, e, key, w)
    // for each (row 4g + i, key) with s > tau, e = its rank among this
    // chunk's entries of that row (uniform count per 16-lane group via tot).
    auto chunk_entries = [&](int ch, const char* kb, unsigned long long M, auto&& put) {
        const int cb = ch * CK;
#pragma unroll
        for (int t = 0; t < CK / 16; ++t) {
            const unsigned mb = static_cast<unsigned>((M >> (16 * t)) & 0xFFFFull);
            if (mb == 0u || cb + 16 * t >= whi || cb + 16 * t + 16 <= wlo) continue;   // uniform
            KFrag<DT, D> kf;
            kf.load_lds(kb + (16 * t + c) * C::S::KSTR, g);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (DT == DT_BF16) {
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) acc = mfma_bf16(qf.a[ks], kf.a[ks], acc);
            } else {
#pragma unroll
                for (int u = 0; u < D / 16; ++u)
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = mfma_f32(qf.a[u][s], kf.a[u][s], acc);
            }
            float xs[4];
            bool anyc = false;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[i] = fmaf(acc[i], a.scale, -tau[i]);
                anyc |= xs[i] > 0.f;
            }
            // most tiles of a long row hold no support entry at all: the
            // masks and the list appends run only where one may be
            if (!__any(anyc)) continue;   // uniform
            const int key = cb + 16 * t + c;
            const bool kv = ((mb >> c) & 1u) != 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = q0 + r0 + 4 * g + i;
                const bool ok = kv & (row < L) & allowed_ij(row, key, a.causal, a.window);
                const float x = xs[i];
                const bool pred = ok & (x > 0.f);
                int rank, tot;
                group_rank16(__ballot(pred), g, c, &rank, &tot);
                put(i, pred, rank, tot, key, 0.5f * x);
            }
        }
    };

    // ---- 1. lists --------------------------------------------------------------------
    cs.run(ch0, ch1, false, [&](int ch, const char* kb, const char*, unsigned long long M) {
        chunk_entries(ch, kb, M, [&](int i, bool pred, int rank, int tot, int key, float w) {
            const int rl = r0 + 4 * g + i;
            const bool fits = !ovf[i] && cnt[i] + tot <= CAP;
            if (pred && fits) {
                lk[rl * CAP + cnt[i] + rank] = static_cast<uint16_t>(key);
                lw[rl * CAP + cnt[i] + rank] = w;
            }
            ovf[i] = ovf[i] || !fits;
            cnt[i] += fits ? tot : 0;
        });
    });
    wave_sync();

    // dp of a batch of entries at list offset base (entries e0 .. e0 + NB - 1
    // of n): V and K row slices are all gathered first
    auto batch = [&](int base, int e0, int n, int (&key)[NB], float (&w)[NB], float (&dp)[NB], float (&kr)[NB][DPL]) {
        float vr[NB][DPL];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int e = e0 + j;
            const bool in = e < n;
            key[j] = in ? static_cast<int>(lk[base + (in ? e : 0)]) : 0;
            w[j] = in ? lw[base + (in ? e : 0)] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            load_row_slice<DT, DPL>(vh + static_cast<size_t>(key[j]) * D + DPL * c, vr[j]);
            load_row_slice<DT, DPL>(kh + static_cast<size_t>(key[j]) * D + DPL * c, kr[j]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float part = 0.f;
#pragma unroll
            for (int d = 0; d < DPL; ++d) part = fmaf(dor[d], vr[j][d], part);
            dp[j] = row_sum<16>(part);
        }
    };
    // dQ_i = scale (X - cc Y) and the row's c_i = crow
    auto store_dq = [&](int i, float cc, const float (&X)[DPL], const float (&Y)[DPL], float crow) {
        const int row = q0 + r0 + 4 * g + i;
        if (row < L) {
            float* dst = dqh + static_cast<size_t>(row) * D + DPL * c;
#pragma unroll
            for (int d = 0; d < DPL; d += 4)
                *reinterpret_cast<f32x4*>(dst + d) =
                    f32x4{a.scale * fmaf(-cc, Y[d], X[d]), a.scale * fmaf(-cc, Y[d + 1], X[d + 1]),
                          a.scale * fmaf(-cc, Y[d + 2], X[d + 2]), a.scale * fmaf(-cc, Y[d + 3], X[d + 3])};
            if (c == 0) ch[row] = crow;
        }
    };

    // ---- 2. rows whose lists hold the whole support -------------------------------------
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = r0 + 4 * g + i;
        const int n = ovf[i] ? 0 : cnt[i];   // uniform in the 16-lane group
        // (rows without entries still store dQ = 0 and c = 0; the gathers are skipped)
        if (__any(n > 0)) load_row(i);
        float X[DPL], Y[DPL], sw = 0.f, swdp = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) { X[d] = 0.f; Y[d] = 0.f; }
        for (int e0 = 0; __any(e0 < n); e0 += NB) {
            int key[NB];
            float w[NB], dp[NB], kr[NB][DPL];
            batch(rl * CAP, e0, n, key, w, dp, kr);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                sw += w[j];
                swdp = fmaf(w[j], dp[j], swdp);
                const float wdp = w[j] * dp[j];
#pragma unroll
                for (int d = 0; d < DPL; ++d) {
                    X[d] = fmaf(wdp, kr[j][d], X[d]);
                    Y[d] = fmaf(w[j], kr[j][d], Y[d]);
                }
            }
        }
        const float cc = sw > 0.f ? swdp / sw : 0.f;
        if (!ovf[i]) store_dq(i, cc, X, Y, cc);
    }

    // ---- 3. rows with more support than their list --------------------------------------
    // workgroup-wide vote (the passes below stream keys for every wave)
    wave_sync();
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (__any(ovf[0] || ovf[1] || ovf[2] || ovf[3]) && lane == 0) atomicOr(flag, 1);
    __syncthreads();
    if (*flag == 0) return;   // uniform

    // One row index i at a time (two passes each: sums, then dQ); per chunk,
    // the overflowed rows' entries of that chunk are staged in the lists of
    // the lane group's four rows (at most CK <= 4 CAP entries per chunk), all
    // free once section 2 is done.
    const int stage_base = (r0 + 4 * g) * CAP;
    for (int i = 0; i < 4; ++i) {
        load_row(i);
        float X[DPL], Y[DPL], sw = 0.f, swdp = 0.f, cc = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) { X[d] = 0.f; Y[d] = 0.f; }
        for (int pass = 0; pass < 2; ++pass) {
            cs.run(ch0, ch1, false, [&](int ch, const char* kb, const char*, unsigned long long M) {
                int n = 0;
                chunk_entries(ch, kb, M, [&](int ii, bool pred, int rank, int tot, int key, float w) {
                    if (ii != i) return;
                    if (pred && ovf[i]) {
                        lk[stage_base + n + rank] = static_cast<uint16_t>(key);
                        lw[stage_base + n + rank] = w;
                    }
                    n += ovf[i] ? tot : 0;
                });
                wave_sync();
                for (int e0 = 0; __any(e0 < n); e0 += NB) {
                    int key[NB];
                    float w[NB], dp[NB], kr[NB][DPL];
                    batch(stage_base, e0, n, key, w, dp, kr);
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        if (pass == 0) {
                            sw += w[j];
                            swdp = fmaf(w[j], dp[j], swdp);
                        } else if (e0 + j < n) {
                            // dQ directly from dS: a long support would lose
                            // digits in the difference X - c Y
                            const float ds = w[j] * (dp[j] - cc);
#pragma unroll
                            for (int d = 0; d < DPL; ++d) X[d] = fmaf(ds, kr[j][d], X[d]);
                        }
                    }
                }
                wave_sync();
            });
            if (pass == 0) {
                cc = sw > 0.f ? swdp / sw : 0.f;
            } else if (ovf[i]) {
                store_dq(i, 0.f, X, Y, cc);   // Y stays zero: dQ = scale X
            }
        }
    }
}

}  // namespace ea
