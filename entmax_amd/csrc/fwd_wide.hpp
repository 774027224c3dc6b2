// Forward kernel for query tiles whose key span exceeds 2048 keys.
//
// One workgroup = 4 waves of NF fragments of 16 query rows (64 rows per wave
// in bf16) of one (batch, head); lane (g, c) holds query row 16 f + c of
// each fragment f and keys 4g .. 4g + 3 of every 16-key tile of the S^T
// products, so the four lanes c, c + 16, c + 32, c + 48 hold a row.  K
// streams through LDS in chunks of 64 keys shared by the four waves
// (wide.hpp); each LDS read of K feeds NF products.  The score row is never
// stored whole; K is streamed one and a half times:
//   1. every other chunk: scores and the running maximum of each lane's
//      share of that sample of the row;
//   2. a certified lower bound of tau per row from the sample: the larger
//      of ms - 2, ms the sample's maximum ("DistilBERT SST-2 with AdaSplash
//      Attention" model card, Mathematical Formulation 2: tau >= m - 2 >=
//      ms - 2), and the root of sum_j ((s_j - t)/2)^2 = 1 over the four
//      lanes' sampled maxima ("ADASPLASH -- ROBERTA Benchmark Result",
//      section 2.2 Theorem 1: the root over a subset of a row is at most
//      the row's);
//   3. every chunk: the scores again, the row maximum m, the allowed count,
//      and every score above that bound into the row's candidate list: the
//      lane keeps its first PL candidates (score, key) in LDS and the next
//      D/8 - PL in the row's own O row in memory, still unwritten (slot
//      4 k + g for the lane's k-th entry there): no counter is shared
//      between lanes, and few stores to memory hold up the chunk loads;
//   4. tau is the 25-step bisection result on [m - 2, m - 2/sqrt(n)], found
//      as in the short-span kernel (exact root by Newton steps from the left
//      and the closed form of Theorem 1 on the list entries above the bound
//      from all of m and the lanes' maxima, then the centre of the dyadic
//      cell that holds it; col_solve.hpp); the entries with s > tau go to
//      a per-row list in LDS (the row's four lanes in order), and O_i =
//      sum_j p_ij V_j over it, gathering V rows (sparse aggregation,
//      "RoBERTa Base with AdaSplash Attention" model card, Architecture
//      Overview).
// Not a single pass: a pass must bound tau from the keys seen so far, and a
// prefix of a row can have a far larger support than the whole row (a flat
// top that a later, larger score dwarfs), so its lists would have to be much
// longer; the sample of every other chunk bounds tau nearly as tightly as
// the whole row.  A row with more than D/8 scores above its bound in one
// lane is marked (kOMarker in O[row][0], and in its tau word when tau is
// written, so that the check reads tau rather than one O row per row); the long-span kernel
// (fwd_long.hpp) then recomputes the marked 64-row tiles in fix-up mode,
// with S recomputed from the K tiles pass by pass.
#pragma once

#include <type_traits>

#include "chunk_stream.hpp"
#include "col_solve.hpp"
#include "common.hpp"
#include "fwd_short.hpp"
#include "wide.hpp"

namespace ea {

// Marker left in O[row][0] for rows the wide forward could not finish (a
// quiet-NaN bit pattern, compared as an integer; finite inputs never give a
// NaN output).
constexpr unsigned kOMarker = 0x7FC0BEEFu;

// MASKED = false: an instance for calls without a key mask or causal mask
// whose length is a multiple of the workgroup's rows, so that every chunk
// is clean; the masked chunk path is not compiled into it (a smaller loop
// for the instruction cache: 2 % on the long-context forward).
template <int DT, int D, bool MASKED = true>
__global__ __launch_bounds__(kThreads, (WideCfg<DT, D>::kOcc)) void fwd_wide_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef WideCfg<DT, D> C;
    constexpr int NF = C::NF, CK = C::CK, DQ = C::DQ;
    constexpr int SUB = D / 8;     // list slots per lane: D/2 per row (8 bytes each in the row's O)
    constexpr int kSampleStep = 2; // the first pass reads every other chunk
    constexpr int NBO = 4;         // list entries gathered per batch
    constexpr int PL = C::PL;      // candidates per lane in LDS
    static_assert(PL < SUB, "the lists in memory take the rest");
    extern __shared__ float lds[];
    char* Kb = reinterpret_cast<char*>(lds);
    // the LDS candidates: entry k of lane group g of the workgroup's row r at [(4 k + g) BR + r]
    f32x2* const cand = reinterpret_cast<f32x2*>(Kb + 2 * C::k_bytes);

    const int total = a.B * a.H * a.nqt;
    const int wi = xcd_swizzle(blockIdx.x, total);
    const int bh = wi / a.nqt;
    const int qt = wi - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * C::BR;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const T* vh = static_cast<const T*>(a.v) + kv_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;
    const bool hasm = km != nullptr;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane / 16, c = lane % 16;
    const int rbase = q0 + wv * NF * 16;   // the wave's first row

    int klo, khi;
    key_range(q0, C::BR, L, a.causal, a.window, &klo, &khi);
    const int ch0 = klo / CK, ch1 = (khi + CK - 1) / CK;
    int wlo, whi;   // keys the wave's rows may attend
    key_range(rbase, NF * 16, L, a.causal, a.window, &wlo, &whi);

    const float scale = a.scale;
    QFrag<DT, D> qf[NF];
    float LM[NF];      // running maximum of this lane's share of the row (raw accumulator units)
    float thrr[NF];    // the row's candidate threshold (raw)
    float lbs[NF];     // its certified lower bound of tau (scaled units)
    float m[NF];       // row maximum (raw)
    bool ovf[NF];
    float nl[NF];      // allowed keys seen by this lane (causal rows)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        qf[f].load(qh, rbase + 16 * f + c, L, g);
        LM[f] = -kInf;
        ovf[f] = false;
        nl[f] = 0.f;
    }
    float npop = 0.f;   // valid keys of the span (rows without a causal mask; uniform)
    const bool allrows = rbase + NF * 16 <= L;
    // the list of row f in memory: entries (score scaled, key bits) in the
    // row's O; lane g of the row owns the slots g, g + 4, ..., its k-th
    // entry there at [4 k]
    float* outh = a.out + head_off;
    auto lst = [&](int f, int lane_g) {
        return reinterpret_cast<f32x2*>(outh + static_cast<size_t>(clamp_row(rbase + 16 * f + c, L)) * D) + lane_g;
    };
    int pc[NF];   // this lane's candidates of row f so far

    // pass 1 (every other chunk) fetches one chunk ahead; pass 2 (every
    // chunk) two ahead, in two register sets
    ChunkStream<DT, D, 2, 1> cs;
    ChunkStream<DT, D, 2, 2> cs2;
    auto init_stream = [&](auto& st) {
        st.Kb = Kb;
        st.Vb = nullptr;
        st.kh = kh;
        st.vh = vh;
        st.kmp = hasm ? km : reinterpret_cast<const uint8_t*>(qh);
        st.hasm = hasm;
        st.L = L;
        st.tid = tid;
        st.lane = lane;
    };
    init_stream(cs);
    init_stream(cs2);
    constexpr unsigned kMaskedBits = DT == DT_BF16 ? 0xF149u : 0xF149F2CAu;   // -1e30
    const int klane = c * C::KSTR + 16 * g;

    // Score tiles of one chunk.  A chunk of valid keys that no causal /
    // window bound crosses and whose rows are all query rows ("clean",
    // uniform) takes plain products and no masking.
    auto scores = [&](auto clean_tag, int cb, const char* kb, unsigned long long M, f32x4 (&s)[NF][4]) {
        constexpr bool CLEAN = decltype(clean_tag)::value;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 o[NF];
            if constexpr (CLEAN) {
                tile_products<DT, D, NF>(kb + klane + 16 * t * C::KSTR, qf, o);
            } else {
                const unsigned mb = static_cast<unsigned>((M >> (16 * t)) & 0xFFFFull);
                const bool ok = mb != 0u && cb + 16 * t < whi && cb + 16 * t + 16 > wlo;   // uniform
                if (!ok) {
#pragma unroll
                    for (int f = 0; f < NF; ++f) s[f][t] = f32x4{-kInf, -kInf, -kInf, -kInf};
                    continue;
                }
                const unsigned bias = ((mb >> c) & 1u) ? 0u : kMaskedBits;
                tile_products<DT, D, NF, true>(kb + klane + 16 * t * C::KSTR, qf, o, bias, g);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int row = rbase + 16 * f + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = cb + 16 * t + 4 * g + i;
                        const bool okk = row < L && (!a.causal || allowed_ij(row, key, 1, a.window));
                        o[f][i] = okk ? o[f][i] : -kInf;
                    }
                }
            }
#pragma unroll
            for (int f = 0; f < NF; ++f) s[f][t] = o[f];
        }
    };
    auto clean_chunk = [&](int cb, unsigned long long M) {
        const bool cross = a.causal && (cb + CK - 1 > rbase || (a.window > 0 && cb <= rbase + NF * 16 - 1 - a.window));
        return M == ~0ull && !cross && allrows;
    };

    // ---- 1. a lower bound of each row's maximum from every other chunk -----------------------
    cs.template run<kSampleStep>(ch0, ch1, false, [&](int chn, const char* kb, const char*, unsigned long long M) {
        const int cb = chn * CK;
        if (cb >= whi || cb + CK <= wlo) return;   // uniform: none of the wave's keys
        f32x4 s[NF][4];
        if (!MASKED || clean_chunk(cb, M)) scores(std::true_type{}, cb, kb, M, s);
        else scores(std::false_type{}, cb, kb, M, s);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            float mx = LM[f];
#pragma unroll
            for (int t = 0; t < 4; ++t) mx = fmaxf(fmaxf(mx, s[f][t][0]), fmaxf(fmaxf(s[f][t][1], s[f][t][2]), s[f][t][3]));
            LM[f] = mx;
        }
    });

    // ---- 2. candidate thresholds: a certified lower bound of tau from the sampled maxima ----
    // The larger of ms - 2 and the root of sum_j ((s_j - t)/2)^2 = 1 over the
    // four lanes' sampled maxima, ms their maximum: the root over a subset of
    // a row is at most the row's, and ms - 2 <= m - 2 <= tau.  A row with no
    // allowed key among the sampled chunks keeps every allowed score.
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const float msr = col4_max(LM[f]);
        const bool none = !(msr > -1e29f);
        const float ms = none ? 0.f : msr * scale;
        const float xl = LM[f] > -1e29f ? fmaf(LM[f], 0.5f * scale, -0.5f * ms) : -2.f;
        const float lbx = fmaxf(col_lower_bound(xl), -1.f);
        const float tr = fmaf(2.f, lbx, ms) / scale;
        thrr[f] = none ? -1e29f : tr - 1e-6f * fabsf(tr) - 1e-30f;   // a little low: rounding keeps more
        LM[f] = -kInf;   // the exact maxima come from the second pass
    }

    // ---- 3. every chunk: scores, maxima, allowed counts and the candidate lists ------------
#pragma unroll
    for (int f = 0; f < NF; ++f) pc[f] = 0;
    cs2.run(ch0, ch1, false, [&](int chn, const char* kb, const char*, unsigned long long M) {
        const int cb = chn * CK;
        npop += static_cast<float>(__popcll(M));
        if (cb >= whi || cb + CK <= wlo) return;   // uniform: none of the wave's keys
        f32x4 s[NF][4];
        if (!MASKED || clean_chunk(cb, M)) {
            scores(std::true_type{}, cb, kb, M, s);
            if (a.causal) {
                const float nc = g == 0 ? static_cast<float>(kWave) : 0.f;   // every key of the chunk allowed
#pragma unroll
                for (int f = 0; f < NF; ++f) nl[f] += nc;
            }
        } else {
            scores(std::false_type{}, cb, kb, M, s);
            if (a.causal) {
                // allowed count of causal rows: this lane's allowed, valid keys
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) nl[f] += s[f][t][i] > -1e29f ? 1.f : 0.f;
            }
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            float tm[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) tm[t] = fmaxf(fmaxf(s[f][t][0], s[f][t][1]), fmaxf(s[f][t][2], s[f][t][3]));
            const float cm = fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3]));
            LM[f] = fmaxf(LM[f], cm);
            if (!__any(cm > thrr[f])) continue;   // uniform
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (!__any(tm[t] > thrr[f])) continue;   // uniform: no candidate in this tile
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (s[f][t][i] > thrr[f]) {
                        const f32x2 en = {s[f][t][i] * scale, __uint_as_float(static_cast<unsigned>(cb + 16 * t + 4 * g + i))};
                        if (pc[f] < PL) {
                            cand[(4 * pc[f] + g) * C::BR + wv * NF * 16 + 16 * f + c] = en;
                        } else if (pc[f] < SUB) {
                            // slot 4 (pc - PL) + g; a 32-bit byte offset from the head's O (a head holds at most 2^32 bytes)
                            const unsigned off = (static_cast<unsigned>(clamp_row(rbase + 16 * f + c, L)) * D +
                                                  2u * static_cast<unsigned>(4 * (pc[f] - PL) + g)) * 4u;
                            *reinterpret_cast<f32x2*>(reinterpret_cast<char*>(outh) + off) = en;
                        } else {
                            ovf[f] = true;
                        }
                        ++pc[f];
                    }
                }
            }
        }
        // every 16 chunks: the bound from the lane maxima seen so far in this
        // pass (again a subset of the row) may exceed the sampled one
        if (((chn - ch0) & 15) == 15) {   // uniform
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const float mr = col4_max(LM[f]);
                if (mr > -1e29f) {
                    const float ms = mr * scale;
                    const float xl = LM[f] > -1e29f ? fmaf(LM[f], 0.5f * scale, -0.5f * ms) : -2.f;
                    const float tr = fmaf(2.f, fmaxf(col_lower_bound(xl), -1.f), ms) / scale;
                    thrr[f] = fmaxf(thrr[f], tr - 1e-6f * fabsf(tr) - 1e-30f);
                }
            }
        }
    });
    // the row maximum m and the lower bound of tau from all lanes' maxima
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        m[f] = col4_max(LM[f]);
        const bool none = !(m[f] > -kInf);   // a row without an allowed key
        const float ms = none ? 0.f : m[f] * scale;
        const float xl = LM[f] > -kInf ? fmaf(LM[f], 0.5f * scale, -0.5f * ms) : -2.f;
        const float lbx = fmaxf(col_lower_bound(xl), -1.f);
        lbs[f] = none ? -kInf : fmaf(2.f, lbx, ms);
    }
    // the lists written by the row's four lanes are visible to all of them,
    // and every wave is done with the K buffers, which take the support lists
    __syncthreads();
    // the support of the wave's row c of the fragment in hand: (y, key)
    // entries, the row's four lanes in lane-group order, each in its list
    // order
    f32x2* const sup = reinterpret_cast<f32x2*>(Kb) + (wv * 16 + c) * (4 * SUB);
    static_assert(4 * 16 * 4 * SUB * sizeof(f32x2) <= 2 * static_cast<size_t>(C::k_bytes), "support lists fit the K buffers");

    // ---- 4. tau, then O over the support, row by row ---------------------------------------
#pragma unroll 1
    for (int f = 0; f < NF; ++f) {
        const int row = rbase + 16 * f + c;
        const float n = row < L ? (a.causal ? col4_sum(nl[f]) : npop) : 0.f;
        const bool empty = n == 0.f;
        const float ms = empty ? 0.f : m[f] * scale;
        const float hs = 0.5f * ms;
        ColState st;
        st.lo = -1.f;
        st.hi = -__builtin_amdgcn_rsqf(empty ? 1.f : n);
        st.lb = fmaxf(-1.f, fmaf(lbs[f], 0.5f, -hs));
        st.it = 0;
        st.hc = 0.f;
        st.cnt = 0.f;
        st.a1 = 0.f;
        st.a2 = 0.f;
        const bool rovf = col4_sum_int(ovf[f] ? 1 : 0) != 0;   // a lane of the row ran out of slots
        const int len = rovf ? 0 : min(pc[f], SUB);             // this lane's entries: PL in LDS, then memory
        const f32x2* mine = lst(f, g);
        const f32x2* minel = cand + g * C::BR + wv * NF * 16 + 16 * f + c;
        float sl[SUB];
        unsigned kl[SUB];
#pragma unroll
        for (int k = 0; k < SUB; ++k) {
            const f32x2 v = k < PL ? minel[4 * k * C::BR] : mine[4 * (k < len ? k - PL : 0)];
            sl[k] = k < len ? fmaf(v[0], 0.5f, -hs) : -kInf;
            kl[k] = __float_as_uint(v[1]);
        }
        const float ts = col_exact<SUB>(sl, st, SUB * 4 + 3);
        const float t = col_dyadic(st, ts);
        // the support (p > 0) into the row's list in LDS: this lane's entries
        // after those of the row's lane groups below g
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < SUB; ++k) cnt += (!empty && sl[k] - t > 0.f) ? 1 : 0;
        int nsup;
        int at = col4_scan_int(cnt, g, &nsup);
#pragma unroll
        for (int k = 0; k < SUB; ++k) {
            const float y = sl[k] - t;
            if (!empty && y > 0.f) sup[at++] = f32x2{y, __uint_as_float(kl[k])};
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // O = sum p V over the support, NBO entries per batch of gathers
        float o[DQ];
#pragma unroll
        for (int d = 0; d < DQ; ++d) o[d] = 0.f;
        const int nmax = wave_max_int<kWave>(nsup);
        // the support, kept for the backward when asked, in the same order
        const size_t srow = static_cast<size_t>(bh) * L + clamp_row(row, L);
        f32x2* se = a.sent != nullptr ? reinterpret_cast<f32x2*>(a.sent) + srow * (D / 2) : nullptr;
#pragma unroll 1
        for (int e0 = 0; e0 < nmax; e0 += NBO) {
            int key[NBO];
            float p[NBO];
            RowSlice<DT, DQ> vr[NBO];
#pragma unroll
            for (int j = 0; j < NBO; ++j) {
                const bool in = e0 + j < nsup;
                const f32x2 en = sup[in ? e0 + j : 0];
                p[j] = in ? en[0] * en[0] : 0.f;
                key[j] = in ? static_cast<int>(__float_as_uint(en[1])) : 0;
                // lane group j % 4 keeps entry e0 + j
                if (se != nullptr && in && g == (j & 3) && row < L) se[e0 + j] = en;
            }
#pragma unroll
            for (int j = 0; j < NBO; ++j) vr[j].load(vh + static_cast<size_t>(key[j]) * D + g * DQ);
#pragma unroll
            for (int j = 0; j < NBO; ++j)
#pragma unroll
                for (int d = 0; d < DQ; ++d) o[d] = fmaf(p[j], vr[j].at(d), o[d]);
        }
        if (a.scount != nullptr && g == 0 && row < L) a.scount[srow] = rovf ? -1 : nsup;   // -1: recomputed, not saved
        // every lane of the wave has read the row's lists (in its O row and
        // in LDS) before any is overwritten
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (row < L) {
            float* orow = outh + static_cast<size_t>(row) * D + g * DQ;
#pragma unroll
            for (int d = 0; d < DQ; d += 4) *reinterpret_cast<f32x4*>(orow + d) = f32x4{o[d], o[d + 1], o[d + 2], o[d + 3]};
            if (rovf && g == 0) reinterpret_cast<unsigned*>(orow)[0] = kOMarker;   // recomputed by the fix-up
            // tau of a row left to the fix-up holds the marker too (bits, not a
            // float value), so that the fix-up reads one word per row from tau
            if (a.tau != nullptr && g == 0)
                reinterpret_cast<unsigned*>(a.tau)[static_cast<size_t>(bh) * L + row] =
                    rovf ? kOMarker : __float_as_uint(empty ? kInf : fmaf(2.f, t, ms));
        }
    }
}

}  // namespace ea
