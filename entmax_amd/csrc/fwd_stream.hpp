// Forward kernel for rows whose key span does not fit in LDS (> 1024 keys).
//
// One workgroup = 4 independent waves, each owning 16 query rows of one
// (batch, head).  The score row is never stored whole:
//   1. one pass over the KV tiles computes S = Q K^T / sqrt(d) on MFMA with
//      the masks folded in, keeps the running row max m and the allowed count
//      n, and appends every score above m - 2 (with its key) to the row's
//      candidate list in LDS.  tau >= max - 2 ("DistilBERT SST-2 with
//      AdaSplash Attention" model card, Mathematical Formulation 2), so every
//      key of the final support is in the list; lists that would fill up are
//      compacted with the current threshold.
//   2. tau by 25 bisection steps over the list (tau_solver.hpp), 4 lanes/row.
//   3. O_i = sum over list entries with s > tau of p * V_key, gathering V rows
//      (sparse aggregation, "RoBERTa Base with AdaSplash Attention" model
//      card, Architecture Overview).
// A row whose candidates still overflow its list falls back to bisection with
// S recomputed from the K tiles at every step, then a recompute pass that
// streams its support into the list and flushes it into O when full.
#pragma once

#include <type_traits>

#include "chunk_stream.hpp"
#include "common.hpp"
#include "fwd_short.hpp"
#include "tau_solver.hpp"

namespace ea {

template <int D, int CAP>
struct StreamCfg {
    static constexpr int BM = 64;
    static constexpr int TPR = kThreads / BM;   // 4 lanes per row in the solve
    // list row stride: CAP + 4 words puts rows 4 apart (the rows of one lane
    // group) and consecutive rows (the solve's lanes) on different LDS banks
    static constexpr int LST = CAP + 4;
    static constexpr size_t lds_bytes =
        static_cast<size_t>(BM) * LST * (sizeof(float) + sizeof(uint16_t)) +
        sizeof(float) * 3 * BM + sizeof(int) * 2 * BM;
    // one K chunk buffer (ChunkStream<.., 1>): with CAP = 80 a bf16 workgroup
    // takes under a third of the LDS
    template <int DT>
    static constexpr size_t total_bytes() { return lds_bytes + ChunkCfg<DT, D>::k_bytes; }
    static_assert(CAP / TPR <= 64, "at most 64 list entries per lane in the solve");
};

// Rank of this lane among the set lanes of its 16-lane group in `mask`.
__device__ __forceinline__ void group_rank(unsigned long long mask, int g, int c, int* rank, int* total) {
    const unsigned gm = static_cast<unsigned>((mask >> (16 * g)) & 0xFFFFull);
    *rank = __popc(gm & ((1u << c) - 1u));
    *total = __popc(gm);
}

template <int DT, int D, int CAP>
__global__ __launch_bounds__(kThreads, (DT == DT_BF16 ? 3 : 1)) void fwd_stream_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef StreamCfg<D, CAP> C;
    constexpr int BM = C::BM, TPR = C::TPR, LST = C::LST;
    extern __shared__ float lds[];
    float* lv = lds;                                   // [BM][LST] candidate scores (CAP used per row)
    float* rowm = lv + BM * LST;                       // [BM] row max
    float* rowts = rowm + BM;                          // [BM] shifted tau
    int* rown = reinterpret_cast<int*>(rowts + BM + BM);            // [BM] allowed count
    int* rowc = rown + BM;                             // [BM] list length, -1 = overflow
    uint16_t* lk = reinterpret_cast<uint16_t*>(rowc + BM);         // [BM][LST] keys
    float* kbufs = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + C::lds_bytes);   // K chunk buffers

    const int total = a.B * a.H * a.nqt;
    const int w = xcd_swizzle(blockIdx.x, total);
    const int bh = w / a.nqt;
    const int qt = w - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * BM;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const T* vh = static_cast<const T*>(a.v) + kv_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane / 16, c = lane % 16;
    const int r0 = 16 * wv;            // this wave's first row (tile-local)

    // key span of this wave's rows
    int klo, khi;
    key_range(q0 + r0, 16, L, a.causal, a.window, &klo, &khi);
    const int kt0 = klo / kBN;
    const int ntile = khi > klo ? (khi + kBN - 1) / kBN - kt0 : 0;

    QFrag<DT, D> qf;
    qf.load(qh, q0 + r0 + c, L, g);

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

    // ---- 1. scores, row max, candidate lists --------------------------------
    // K streams through LDS in 64-key chunks shared by the four waves
    // (chunk_stream.hpp); the row max is reduced once per chunk, the allowed
    // count once at the end, and chunks without a candidate for the wave
    // cost only the products and a comparison.
    float m[4];
    int n[4], cnt[4];
    bool ovf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m[i] = -kInf; n[i] = 0; cnt[i] = 0; ovf[i] = false; }
    float nl[4] = {0.f, 0.f, 0.f, 0.f};
    {
        int wlo_k, whi_k;
        key_range(q0, BM, L, a.causal, a.window, &wlo_k, &whi_k);
        const int ch0 = wlo_k / kBN, ch1 = (whi_k + kBN - 1) / kBN;
        ChunkStream<DT, D, 1> cs;
        cs.Kb = reinterpret_cast<char*>(kbufs);
        cs.Vb = nullptr;
        cs.kh = kh;
        cs.vh = vh;
        cs.kmp = km != nullptr ? km : reinterpret_cast<const uint8_t*>(qh);
        cs.hasm = km != nullptr;
        cs.L = L;
        cs.tid = tid;
        cs.lane = lane;
        const float inv_scale = 1.f / a.scale;
        cs.run(ch0, ch1, false, [&](int ch, const char* kb, const char*, unsigned long long M) {
            const int kbase = ch * kBN;
            if (kbase >= khi || kbase + kBN <= klo) return;   // uniform: none of this wave's keys
            float s[4][4];
            float thr_s[4];   // each row's current threshold m - 2, in the units of s
            bool any = false;
            auto products = [&](auto causal_tag, auto full_tag) {
                constexpr bool CAUSAL = decltype(causal_tag)::value;
                constexpr bool FULL = decltype(full_tag)::value;   // every key of the chunk valid
                float tm[4] = {-kInf, -kInf, -kInf, -kInf};
#pragma unroll
                for (int c16 = 0; c16 < 4; ++c16) {
                    KFrag<DT, D> kf;
                    kf.load_lds(kb + (16 * c16 + c) * ChunkCfg<DT, D>::KSTR, g);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (DT == DT_BF16) {
#pragma unroll
                        for (int ks = 0; ks < D / 32; ++ks) acc = mfma_bf16(qf.a[ks], kf.a[ks], acc);
                    } else {
#pragma unroll
                        for (int u = 0; u < D / 16; ++u)
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc = mfma_f32(qf.a[u][q], kf.a[u][q], acc);
                    }
                    const int key = kbase + 16 * c16 + c;
                    const bool kv = ((M >> (16 * c16 + c)) & 1ull) != 0ull;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (CAUSAL) {
                            // scaled scores, masks per element, count per element
                            s[c16][i] = score(key, kv, acc, i);
                            nl[i] += s[c16][i] > -kInf ? 1.f : 0.f;
                        } else if constexpr (FULL) {
                            s[c16][i] = acc[i];   // raw accumulator (scaled where kept)
                        } else {
                            // raw accumulators (scaled only where they are kept);
                            // rows past L are never written out
                            s[c16][i] = kv ? acc[i] : -kInf;
                        }
                        tm[i] = fmaxf(tm[i], s[c16][i]);
                    }
                }
                if constexpr (!CAUSAL) {
                    const float nv = static_cast<float>(__popcll(M));   // uniform
#pragma unroll
                    for (int i = 0; i < 4; ++i) nl[i] += c == 0 ? nv : 0.f;   // summed over the 16 lanes below
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float rm = row_max<16>(tm[i]);
                    m[i] = fmaxf(m[i], CAUSAL ? rm : rm * a.scale);
                    // threshold m - 2, in the units of s (a slightly lower raw
                    // threshold only keeps more candidates)
                    const float thr = CAUSAL ? m[i] - 2.f : (m[i] - 2.f) * inv_scale - 1e-6f * fabsf(m[i] * inv_scale);
                    thr_s[i] = thr;
                    any |= tm[i] > thr;   // this lane's largest entry of the row decides
                }
            };
            const bool raw = !(a.causal || a.window > 0);   // s holds unscaled accumulators
            if (a.causal || a.window > 0) products(std::true_type{}, std::false_type{});
            else if (M == ~0ull) products(std::false_type{}, std::true_type{});
            else products(std::false_type{}, std::false_type{});
            if (!__any(any)) return;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = r0 + 4 * g + i;
                const float thr = m[i] - 2.f;
                // this chunk's candidates of the row (a ballot per 16-key tile)
                unsigned long long bal[4];
#pragma unroll
                for (int c16 = 0; c16 < 4; ++c16) bal[c16] = __ballot(!ovf[i] && s[c16][i] > thr_s[i]);
                // no candidate for these four rows in this chunk (uniform): the
                // lists stay as they are
                if ((bal[0] | bal[1] | bal[2] | bal[3]) == 0ull) continue;
                int add = 0;
#pragma unroll
                for (int c16 = 0; c16 < 4; ++c16) add += __popc(static_cast<unsigned>((bal[c16] >> (16 * g)) & 0xFFFFull));
                // make room: drop entries that fell below the current threshold
                const bool need = !ovf[i] && cnt[i] + add > CAP;
                if (__any(need)) {
                    int wr = 0;
                    const int tot = need ? cnt[i] : 0;
                    int nch = (tot + 15) / 16;
                    int maxch = nch;
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) maxch = max(maxch, __shfl_xor(maxch, o, kWave));
                    for (int chh = 0; chh < maxch; ++chh) {
                        const int idx = 16 * chh + c;
                        const bool in = idx < tot;
                        const float v = in ? lv[rl * LST + idx] : -kInf;
                        const uint16_t kk = in ? lk[rl * LST + idx] : static_cast<uint16_t>(0);
                        const bool keep = in && v > thr;
                        int rank, tot2;
                        group_rank(__ballot(keep), g, c, &rank, &tot2);
                        wave_sync();
                        if (keep) {
                            lv[rl * LST + wr + rank] = v;
                            lk[rl * LST + wr + rank] = kk;
                        }
                        wave_sync();
                        wr += tot2;
                    }
                    if (need) cnt[i] = wr;
                }
                // appends: most (row, tile) pairs of a chunk have none, and
                // skip the ranking (uniform test)
#pragma unroll
                for (int c16 = 0; c16 < 4; ++c16) {
                    if (bal[c16] == 0ull) continue;
                    const bool pred = ((bal[c16] >> lane) & 1ull) != 0ull;
                    int rank, tot2;
                    group_rank(bal[c16], g, c, &rank, &tot2);
                    const int slot = cnt[i] + rank;
                    if (pred && slot < CAP) {
                        lv[rl * LST + slot] = raw ? s[c16][i] * a.scale : s[c16][i];
                        lk[rl * LST + slot] = static_cast<uint16_t>(kbase + 16 * c16 + c);
                    }
                    cnt[i] += tot2;
                }
                if (cnt[i] > CAP) ovf[i] = true;
            }
        });
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = static_cast<int>(row_sum<16>(nl[i]));
    if (c == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = r0 + 4 * g + i;
            rowm[rl] = n[i] > 0 ? m[i] : 0.f;
            rown[rl] = n[i];
            rowc[rl] = ovf[i] ? -1 : cnt[i];
        }
    }
    __syncthreads();

    // ---- 2. tau over the candidate lists (4 lanes per row) -------------------
    {
        const int r = tid / TPR, sub = tid % TPR;
        const int nr = rown[r];
        const int len = rowc[r];
        const float mm = rowm[r];
        const float* vrow = lv + r * LST;
        const int nel = len > 0 ? (len + TPR - 1) / TPR : 0;
        auto get = [&](int i) {
            const int idx = sub + TPR * i;
            return idx < len ? vrow[idx] - mm : -kInf;
        };
        float ts = solve_tau_shifted<TPR>(get, nel, nr > 0 ? nr : 1);
        if (nr == 0) ts = kInf;
        if (sub == 0) rowts[r] = ts;
    }
    __syncthreads();

    // ---- 3. O = sum p V over the support -------------------------------------
    constexpr int DPL = D / 16;        // output columns per lane
    float o[4][DPL];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[i][j] = 0.f;

    auto flush = [&](int i, int len, float mm, float ts) {
        const int rl = r0 + 4 * g + i;
        for (int e = 0; e < len; ++e) {
            const float x = (lv[rl * LST + e] - mm) - ts;
            if (x > 0.f) {
                const float p = 0.25f * x * x;
                const int key = lk[rl * LST + e];
                const T* vr = vh + static_cast<size_t>(key) * D + DPL * c;
                if constexpr (DT == DT_BF16) {
#pragma unroll
                    for (int j = 0; j < DPL; j += 4) {
                        const uint2 u = *reinterpret_cast<const uint2*>(vr + j);
                        o[i][j + 0] = fmaf(p, __uint_as_float(u.x << 16), o[i][j + 0]);
                        o[i][j + 1] = fmaf(p, __uint_as_float(u.x & 0xFFFF0000u), o[i][j + 1]);
                        o[i][j + 2] = fmaf(p, __uint_as_float(u.y << 16), o[i][j + 2]);
                        o[i][j + 3] = fmaf(p, __uint_as_float(u.y & 0xFFFF0000u), o[i][j + 3]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < DPL; j += 4) {
                        const f32x4 u = *reinterpret_cast<const f32x4*>(vr + j);
#pragma unroll
                        for (int q = 0; q < 4; ++q) o[i][j + q] = fmaf(p, u[q], o[i][j + q]);
                    }
                }
            }
        }
    };

    float mrow[4], tsrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = r0 + 4 * g + i;
        mrow[i] = rowm[rl];
        tsrow[i] = rowts[rl];
        if (!ovf[i]) flush(i, cnt[i], mrow[i], tsrow[i]);
    }

    // ---- overflow fallback (this wave only) ----------------------------------
    bool my_ovf = ovf[0] || ovf[1] || ovf[2] || ovf[3];
    if (__any(my_ovf)) {
        float lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo[i] = -2.f;
            hi[i] = -2.f / sqrtf(static_cast<float>(n[i] > 0 ? n[i] : 1));
        }
        for (int it = 0; it < kIters; ++it) {
            float mid[4], acc4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { mid[i] = 0.5f * (lo[i] + hi[i]); acc4[i] = 0.f; }
            for (int t = 0; t < ntile; ++t) {
                const int kbase = (kt0 + t) * kBN;
#pragma unroll
                for (int c16 = 0; c16 < 4; ++c16) {
                    const int key = kbase + 16 * c16 + c;
                    const bool kv = key_ok(key);
                    const f32x4 acc = qf.tile(kh, key, L, g);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float dx = (score(key, kv, acc, i) - mrow[i]) - mid[i];
                        acc4[i] = dx > 0.f ? fmaf(dx, dx, acc4[i]) : acc4[i];
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float g4 = row_sum<16>(acc4[i]);
                if (g4 > 4.f) lo[i] = mid[i];
                else hi[i] = mid[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (ovf[i]) {
                tsrow[i] = n[i] > 0 ? 0.5f * (lo[i] + hi[i]) : kInf;
                cnt[i] = 0;
            }
        }
        // stream the support of overflowing rows through their lists
        for (int t = 0; t < ntile; ++t) {
            const int kbase = (kt0 + t) * kBN;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool full = ovf[i] && cnt[i] + kBN > CAP;
                if (full) {
                    wave_sync();
                    flush(i, cnt[i], mrow[i], tsrow[i]);
                    cnt[i] = 0;
                }
            }
            wave_sync();
#pragma unroll
            for (int c16 = 0; c16 < 4; ++c16) {
                const int key = kbase + 16 * c16 + c;
                const bool kv = key_ok(key);
                const f32x4 acc = qf.tile(kh, key, L, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rl = r0 + 4 * g + i;
                    const float sc = score(key, kv, acc, i);
                    const bool pred = ovf[i] && (sc - mrow[i]) - tsrow[i] > 0.f;
                    int rank, tot2;
                    group_rank(__ballot(pred), g, c, &rank, &tot2);
                    if (pred) {
                        lv[rl * LST + cnt[i] + rank] = sc;
                        lk[rl * LST + cnt[i] + rank] = static_cast<uint16_t>(key);
                    }
                    cnt[i] += tot2;
                }
            }
        }
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (ovf[i]) flush(i, cnt[i], mrow[i], tsrow[i]);
    }

    // ---- write O and tau -------------------------------------------------------
    float* outh = a.out + head_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = q0 + r0 + 4 * g + i;
        if (row < L) {
            float* orow = outh + static_cast<size_t>(row) * D + DPL * c;
#pragma unroll
            for (int j = 0; j < DPL; j += 4)
                *reinterpret_cast<f32x4*>(orow + j) = f32x4{o[i][j], o[i][j + 1], o[i][j + 2], o[i][j + 3]};
            if (a.tau != nullptr && c == 0)
                a.tau[static_cast<size_t>(bh) * L + row] = n[i] > 0 ? mrow[i] + tsrow[i] : kInf;
        }
    }
}

}  // namespace ea
