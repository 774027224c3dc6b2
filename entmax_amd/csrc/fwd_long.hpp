// Forward kernel for query tiles whose key span exceeds 128 keys.
//
// One workgroup (4 waves) per (batch, head, 64 query rows); wave w owns rows
// 16w .. 16w+15 and lane (g, c) serves query row c, as in the short-span
// kernel: the 16-key S^T tiles give lane (g, c) keys 4g .. 4g + 3 of each
// tile for query c, so the four lanes c, c + 16, c + 32, c + 48 hold a row.
//
// The key span is streamed in chunks of 64 keys, each staged once per
// workgroup in LDS (two buffers; a chunk's loads are issued two chunks ahead)
// and shared by the four waves; S is recomputed on MFMA in every pass
// instead of being stored.
//   A. row max and allowed count;
//   C. (when a row allows more keys than its lists hold, until every lane's
//      band fits) three bisection levels at once ("ADASPLASH -- ROBERTA
//      Benchmark Result", section 2.3 Theorem 2; bracket of the "DistilBERT
//      SST-2 with AdaSplash Attention" model card, Mathematical Formulation
//      2): a per-lane histogram of the bracket's eight cells three steps
//      down, with the count and the first two moments per cell, gives g at
//      all seven midpoints and the exact band size of every cell;
//   B. the band: scores in the current bracket (lo, hi] go to a per-lane
//      list in LDS, those above hi are folded into exact sums (U); if a
//      list overflows, C runs again and B is repeated;
//   then tau from the list and U as in the short-span kernel
//      (col_solve.hpp);
//   D. P = [(S - tau)/2]_+^2 and O = P V on MFMA, V staged per chunk
//      (bf16: row-major, read back with transpose loads), chunks where a
//      wave has no nonzero P skipped for that wave.  O is written in fp32.
// Every pass decision is uniform over the workgroup (the chunk loop and its
// barriers are shared).  In fix-up mode (args.fixup) a workgroup runs only
// when one of its rows carries the wide forward's overflow marker.
#pragma once

#include <type_traits>

#include "chunk_stream.hpp"
#include "col_solve.hpp"
#include "common.hpp"
#include "fwd_short.hpp"
#include "fwd_wide.hpp"

namespace ea {

template <int DT, int D>
struct LongCfg : ChunkCfg<DT, D> {
    typedef ChunkCfg<DT, D> S;
    static constexpr int BM = 64;
    static constexpr int NTC = S::CK / 16;            // 16-key tiles per chunk
    static constexpr int CAP = 32;                    // band entries per lane
    // one more row: where the branch-free appends land once a list is full
    static constexpr int list_bytes = 4 * (CAP + 1) * kWave * 4;
    // the band lists (passes B, solve) and the V buffers (pass D) share a region
    static constexpr int vl_bytes = 2 * S::v_bytes > list_bytes ? 2 * S::v_bytes : list_bytes;
    static constexpr size_t lds_bytes = static_cast<size_t>(2 * S::k_bytes) + vl_bytes + 64;
    static constexpr int kOcc = (DT == DT_BF16 && D == 64) ? 3 : (DT == DT_F32 && D == 128) ? 1 : 2;
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads, (LongCfg<DT, D>::kOcc)) void fwd_long_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef LongCfg<DT, D> C;
    constexpr int BM = C::BM, CK = C::CK, NTC = C::NTC;
    constexpr int CAP = C::CAP;
    extern __shared__ float lds[];
    char* Kb = reinterpret_cast<char*>(lds);                           // 2 K buffers
    char* Vb = Kb + 2 * C::S::k_bytes;                                    // 2 V buffers (pass D)
    float* lists = reinterpret_cast<float*>(Vb);                       // band lists (B, solve)
    int* flag = reinterpret_cast<int*>(Vb + C::vl_bytes);              // workgroup-wide vote

    const int total = a.B * a.H * a.nqt;
    const int w = xcd_swizzle(blockIdx.x, total);
    const int bh = w / a.nqt;
    const int qt = w - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * BM;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    if (a.fixup) {
        // fix-up mode: run only for a tile holding a row the wide kernel
        // could not finish (kOMarker in its tau word when tau is written,
        // else in O[row][0]), and then for all its rows
        const int t = threadIdx.x;
        if (t == 0) *flag = 0;
        __syncthreads();
        if (t < BM && q0 + t < L) {
            const unsigned mk = a.tau != nullptr
                                    ? reinterpret_cast<const unsigned*>(a.tau)[static_cast<size_t>(bh) * L + q0 + t]
                                    : reinterpret_cast<const unsigned*>(a.out)[head_off + static_cast<size_t>(q0 + t) * D];
            if (mk == kOMarker) atomicOr(flag, 1);
        }
        __syncthreads();
        const bool marked = *flag != 0;
        __syncthreads();
        if (!marked) return;   // uniform
    }
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const T* vh = static_cast<const T*>(a.v) + kv_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;
    const bool hasm = km != nullptr;
    const uint8_t* kmp = hasm ? km : reinterpret_cast<const uint8_t*>(qh);

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane / 16, c = lane % 16;
    const int qrow = q0 + 16 * wv + c;
    const bool rowok = qrow < L;

    // chunks of the workgroup's key span, and the keys this wave's rows may attend
    int klo, khi;
    key_range(q0, BM, L, a.causal, a.window, &klo, &khi);
    const int ch0 = klo / CK, ch1 = (khi + CK - 1) / CK;
    int wlo, whi;
    key_range(q0 + 16 * wv, 16, L, a.causal, a.window, &wlo, &whi);
    const int khi_i = qrow;                                   // causal: key <= query
    const int klo_i = a.window > 0 ? qrow - a.window : -1;    // window: key > query - W

    QFrag<DT, D> qf;
    qf.load(qh, qrow, L, g);

    // ---- chunk streaming (chunk_stream.hpp) ---------------------------------------
    ChunkStream<DT, D> cs;
    cs.Kb = Kb;
    cs.Vb = Vb;
    cs.kh = kh;
    cs.vh = vh;
    cs.kmp = kmp;
    cs.hasm = hasm;
    cs.L = L;
    cs.tid = tid;
    cs.lane = lane;
    auto stream = [&](bool withv, auto&& fn) { cs.run(ch0, ch1, withv, fn); };
    // S^T tiles of one chunk for this wave (raw accumulators, masked keys
    // -1e30 through the bias step, causal / window entries -inf), or -inf
    // for tiles outside the wave's keys.  ok(t): tile computed.
    constexpr unsigned kMaskedBits = DT == DT_BF16 ? 0xF149u : 0xF149F2CAu;   // -1e30
    const int klane = c * C::KSTR + 16 * g;   // this lane's K piece within a staged chunk
    // every row of the wave is a query row (uniform)
    const bool allrows = q0 + 16 * wv + 15 < L;
    auto tiles = [&](int ch, const char* kb, unsigned long long M, f32x4 (&sv)[NTC], bool (&ok)[NTC]) {
        const int cb = ch * CK;
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            const unsigned mb = static_cast<unsigned>((M >> (16 * t)) & 0xFFFFull);
            ok[t] = mb != 0u && cb + 16 * t < whi && cb + 16 * t + 16 > wlo;   // uniform
            if (!ok[t]) {
                sv[t] = f32x4{-kInf, -kInf, -kInf, -kInf};
                continue;
            }
            KFrag<DT, D> kf;
            kf.load_lds_at(kb + klane + 16 * t * C::KSTR);
            sv[t] = mb == 0xFFFFu ? kf.st(qf) : kf.st_bias(qf, ((mb >> c) & 1u) ? 0u : kMaskedBits, g);
            if (a.causal) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = cb + 16 * t + 4 * g + i;
                    sv[t][i] = ((key <= khi_i) & (key > klo_i)) ? sv[t][i] : -kInf;
                }
            }
            if (!allrows) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[t][i] = rowok ? sv[t][i] : -kInf;
            }
        }
    };

    const float c2 = 0.5f * a.scale;

    // ---- A. row max and allowed count -----------------------------------------------
    // Without a causal mask every row of the tile allows the same keys: the
    // count comes from the chunks' key bits.
    float mlane = -kInf, nl = 0.f, npop = 0.f;
    stream(false, [&](int ch, const char* kb, const char*, unsigned long long M) {
        f32x4 sv[NTC];
        bool ok[NTC];
        tiles(ch, kb, M, sv, ok);
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            if (!ok[t]) continue;
            mlane = fmaxf(mlane, fmaxf(fmaxf(sv[t][0], sv[t][1]), fmaxf(sv[t][2], sv[t][3])));
            if (a.causal) {
#pragma unroll
                for (int i = 0; i < 4; ++i) nl += sv[t][i] > -1e29f ? 1.f : 0.f;
            }
        }
        if (!a.causal) npop += static_cast<float>(__popcll(M));
    });
    if (!a.causal) nl = (g == 0 && rowok) ? npop : 0.f;
    const float mrow = col4_max(mlane);
    const float n = col4_sum(nl);
    const bool empty = n == 0.f;
    const float mc2 = empty ? 0.f : mrow * c2;

    ColState s;
    s.lb = fmaxf(col_lower_bound(fmaf(mlane, c2, -mc2)), -1.f);
    s.lo = -1.f;
    s.hi = -__builtin_amdgcn_rsqf(empty ? 1.f : n);
    s.it = 0;

    // workgroup-wide vote (uniform result)
    auto vote_any = [&](bool v) {
        if (tid == 0) *flag = 0;
        __syncthreads();
        if (__any(v) && lane == 0) atomicOr(flag, 1);
        __syncthreads();
        const int r = *flag;
        __syncthreads();
        return r != 0;
    };

    // ---- C. three bisection levels per pass, from a histogram -------------------
    // The bracket [lo, hi] is cut into the 8 cells three steps down; every
    // entry above max(lo, lb) goes to its cell (cell 8: above hi), where this
    // lane accumulates the count and the first two moments of its offset r
    // from the cell's lower edge e (cells 0-7: r in cell widths, cell 8:
    // r = x - hi), in 22-bit fixed point through integer LDS adds (one
    // private slot per lane: no two lanes touch one address; integer adds are
    // full rate, float adds are not).  After the pass, g at each of the seven
    // inner edges follows from the cell sums above it
    //   sum_{x > e_k} (x - e_k)^2 = sum over cells j >= k of
    //     S2_j + 2 (e_j - e_k) S1_j + (e_j - e_k)^2 N_j,
    // and the three steps walk the tree of these midpoints.  Entries at or
    // below max(lo, lb) go to a dump cell (9).  The fixed-point rounding
    // (to nearest, 2^-23 of a cell width, or absolute for cell 8) is of the
    // order of the float rounding of the sums themselves.
    constexpr int kCells = 10;
    unsigned* hist = reinterpret_cast<unsigned*>(lists) + wv * (kCells * 3 * kWave) + lane;   // [cell][N, S1, S2] at stride kWave
    static_assert(4 * kCells * 3 * kWave * 4 <= C::vl_bytes, "histograms fit the list region");
    // steps whose midpoint lies below lb move the lower end without an
    // evaluation: take them before a pass, so that its levels all count
    auto forced = [&]() {
        for (;;) {
            const float mid = 0.5f * (s.lo + s.hi);
            const bool f = s.it < kIters && mid < s.lb;
            if (!__any(f)) break;
            if (f) {
                s.lo = mid;
                ++s.it;
            }
        }
    };
    auto pass_c = [&]() -> int {
        forced();
        const float lo = s.lo, hi = s.hi;
        const float w = (hi - lo) * 0.125f;          // cell width (power-of-two scaling)
        const float iw = 8.f / (hi - lo);
        const float lo_eff = fmaxf(lo, s.lb);
        // u = (x - lo) / w straight from the raw accumulator (x = sv c2 - mc2);
        // entries with u at or below u_eff (x at or below lo_eff) are dumped
        const float ua = c2 * iw, ub = -(mc2 + lo) * iw;
        const float u_eff = (lo_eff - lo) * iw;
        constexpr float kFix = 4194304.f;            // 2^22
#pragma unroll
        for (int k = 0; k < kCells * 3; ++k) hist[k * kWave] = 0u;
        stream(false, [&](int ch, const char* kb, const char*, unsigned long long M) {
            f32x4 sv[NTC];
            bool ok[NTC];
            tiles(ch, kb, M, sv, ok);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                if (!ok[t]) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float u = fmaf(sv[t][i], ua, ub);
                    int ci = static_cast<int>(u);   // the cell, for u > u_eff >= 0
                    ci = ci < 8 ? ci : 8;
                    ci = u > u_eff ? ci : 9;
                    // offset in [0, 1]: the fraction of u in cells 0-7, x - hi
                    // = (u - 8) w in [0, 1] in cell 8; the dump cell's lies
                    // in [0, 1) and is never read
                    const float r = ci == 8 ? (u - 8.f) * w : __builtin_amdgcn_fractf(u);
                    // rounded to nearest: truncation would bias every term
                    // the same way, and over hundreds of entries per cell the
                    // bias would move g at the edges by more than the float
                    // rounding of the sums
                    const float rk = r * kFix;
                    unsigned* h = hist + ci * (3 * kWave);
                    lds_add(h, 1u);
                    lds_add(h + kWave, static_cast<unsigned>(rk + 0.5f));
                    lds_add(h + 2 * kWave, static_cast<unsigned>(fmaf(r, rk, 0.5f)));
                }
            }
        });
        // row sums per cell; this lane's counts are kept for the band size
        constexpr float kUnfix = 1.f / kFix;
        float nl_cell[8];
        float N = 0.f, A1 = 0.f, A2 = 0.f;   // cells above the current edge, relative to it
        float gk[8];                          // g at the edges e_0 .. e_7
        N = col4_sum(static_cast<float>(hist[(8 * 3) * kWave]));
        A1 = col4_sum(static_cast<float>(hist[(8 * 3 + 1) * kWave])) * kUnfix;
        A2 = col4_sum(static_cast<float>(hist[(8 * 3 + 2) * kWave])) * kUnfix;
#pragma unroll
        for (int k = 7; k >= 0; --k) {
            // reference from e_(k+1) down to e_k
            A2 = fmaf(w * N, w, fmaf(2.f * w, A1, A2));
            A1 = fmaf(w, N, A1);
            const float nk = static_cast<float>(hist[(k * 3) * kWave]);
            nl_cell[k] = nk;
            N += col4_sum(nk);
            A1 = fmaf(col4_sum(static_cast<float>(hist[(k * 3 + 1) * kWave])), w * kUnfix, A1);
            A2 = fmaf(col4_sum(static_cast<float>(hist[(k * 3 + 2) * kWave])), w * w * kUnfix, A2);
            gk[k] = A2;
        }
        // the seven midpoints of the next three levels, as the steps would form them
        const float p4 = 0.5f * (lo + hi);
        const float p2 = 0.5f * (lo + p4), p6 = 0.5f * (p4 + hi);
        const float p1 = 0.5f * (lo + p2), p3 = 0.5f * (p2 + p4), p5 = 0.5f * (p4 + p6), p7 = 0.5f * (p6 + hi);
        const float pts[8] = {lo, p1, p2, p3, p4, p5, p6, p7};
        // walk the tree: g > 1 (or a midpoint below lb) moves the lower end
        int node = 4, cell = 0;
#pragma unroll
        for (int lev = 0; lev < 3; ++lev) {
            if (s.it >= kIters) break;
            const int step = 4 >> (lev + 1);
            const float mid = pts[node];
            const bool up = gk[node] > 1.f || mid < s.lb;
            if (up) {
                s.lo = mid;
                cell = node;
            } else {
                s.hi = mid;
            }
            ++s.it;
            node = up ? node + step : node - step;
        }
        // this lane's entries in the final cell (lo, hi]; none for rows
        // that have taken all their steps
        float band = nl_cell[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) band = cell == k ? nl_cell[k] : band;
        return s.it >= kIters ? 0 : static_cast<int>(band);
    };

    // ---- B. band lists and U ---------------------------------------------------------
    float* col = lists + wv * ((CAP + 1) * kWave) + lane;
    int len = 0;
    auto pass_b = [&]() {
        s.hc = s.hi;
        s.cnt = 0.f;
        s.a1 = 0.f;
        s.a2 = 0.f;
        len = 0;
        const float lo_eff = fmaxf(s.lo, s.lb);
        stream(false, [&](int ch, const char* kb, const char*, unsigned long long M) {
            f32x4 sv[NTC];
            bool ok[NTC];
            tiles(ch, kb, M, sv, ok);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                if (!ok[t]) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = fmaf(sv[t][i], c2, -mc2);
                    const float y = relu1(x - s.hi);
                    s.cnt += x > s.hi ? 1.f : 0.f;
                    s.a1 += y;
                    s.a2 = fmaf(y, y, s.a2);
                    col[(len < CAP ? len : CAP) * kWave] = x;   // row CAP: overflow dump
                    len += ((x > lo_eff) & (x <= s.hi)) ? 1 : 0;
                }
            }
        });
    };

    // ---- tau -----------------------------------------------------------------------------
    // lists alias the V buffers, which pass D rewrites only after this
    {
        // pass C until the band of every lane fits its list (known exactly
        // from the cell counts), then pass B.  Rows allowing more keys than
        // four full lists start with pass C; a list that overflows anyway
        // sends the workgroup back to pass C.  Rows take different numbers
        // of steps (forced ones), so every loop decision is a vote.
        bool need_c = vote_any(n > static_cast<float>(4 * CAP));
        for (;;) {
            while (need_c) need_c = vote_any(pass_c() > CAP);
            pass_b();
            if (!vote_any(len > CAP && s.it < kIters)) break;
            need_c = true;
        }
    }
    // rows that have taken all 25 steps return the midpoint
    const float tr = col_finish<CAP>(col, len, s);
    if (a.tau != nullptr && g == 0 && rowok) a.tau[static_cast<size_t>(bh) * L + qrow] = empty ? kInf : 2.f * (mc2 + tr);
    const float sh = empty ? 0.f : mc2 + tr;
    __syncthreads();   // lists done: the region holds V from now on

    // ---- D. O = P V ----------------------------------------------------------------------
    f32x4 o[D / 16];
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream(true, [&](int ch, const char* kb, const char* vb, unsigned long long M) {
        f32x4 sv[NTC];
        bool ok[NTC];
        tiles(ch, kb, M, sv, ok);
        f32x4 yv[NTC];   // p = y^2
        bool nz = false;
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float y = relu1(fmaf(sv[t][i], c2, -sh));
                yv[t][i] = y;
                nz |= y > 0.f;
            }
        }
        if (!__any(nz)) return;   // uniform: nothing of this chunk reaches the wave's rows
        if constexpr (DT == DT_BF16) {
#pragma unroll
            for (int h = 0; h < NTC / 2; ++h) {
                float y8[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y8[i] = yv[2 * h][i];
                    y8[4 + i] = yv[2 * h + 1][i];
                }
                bf16x8 phi, plo;
                split_sq_bf16(y8, phi, plo);
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    // B operand through transpose loads (see the short-span kernel)
                    const char* src = vb + (32 * h + 4 * g + (c >> 2)) * C::VRS + (16 * ct + 4 * (c & 3)) * 2;
                    const s16x4 r0 = ds_read_tr16(src);
                    const s16x4 r1 = ds_read_tr16(src + 16 * C::VRS);
                    const bf16x8 bv = __builtin_bit_cast(bf16x8, s16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]});
                    o[ct] = mfma_bf16(phi, bv, o[ct]);
                    o[ct] = mfma_bf16(plo, bv, o[ct]);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    const f32x4 bv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(vb) + (16 * ct + c) * C::VSTR + 16 * t + 4 * g);
#pragma unroll
                    for (int q = 0; q < 4; ++q) o[ct] = mfma_f32(yv[t][q] * yv[t][q], bv[q], o[ct]);
                }
            }
        }
    });

    float* outh = a.out + head_off;
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = q0 + 16 * wv + 4 * g + i;
            if (row < L) outh[static_cast<size_t>(row) * D + 16 * ct + c] = o[ct][i];
        }
}

}  // namespace ea
