// Forward kernel for key spans of 129 .. 1024 keys with the scores held in
// registers: S is computed once on MFMA and every later pass (threshold
// search, P, O = P V) reads it from registers instead of recomputing it.
//
// Workgroup: 4 waves, 32 query rows.  Wave w serves row group r = w & 1
// (rows 16 r .. 16 r + 15 of the tile) and key half h = w >> 1.  Keys are
// staged in pairs of 64-key chunks (128 keys, one LDS buffer per pair,
// two buffers): the wave of half h takes the chunk 2 j + h of pair j, so a
// row's keys are split over the two waves of its row group, 16-key S^T
// tiles as in the other kernels (lane (g, c) holds keys 4g .. 4g + 3 of each
// tile for query c).  A wave holds up to 8 pairs x 4 tiles x 4 scores per
// lane in registers.
//
// Threshold ("ADASPLASH -- ROBERTA Benchmark Result", section 2.3; bracket
// of the "DistilBERT SST-2 with AdaSplash Attention" model card,
// Mathematical Formulation 2), in the half-scaled shifted domain
// x = (s - max)/2, p = [x - t]_+^2:
//   * Newton steps on sqrt(g(t)) - 1, where sqrt(g) is the Euclidean norm
//     of the vector [x - t]_+: a convex, decreasing function of t, so every
//     iterate from the left stays at or below the root t* (and unlike g
//     itself it is nearly linear far from the root: one entry is solved in
//     one step);
//   * the start is a lower bound from subsets of the row (the root of a
//     subset is at most the row's): the larger of the exact roots over each
//     wave's four lane maxima, raised by two Newton steps over the row's 64
//     pair maxima (each lane's maximum of every 128-key pair, both halves);
//   * a row stops once its step is below 1e-5 (the error then is of the
//     order of the step squared over the mean excess);
//   * the 25-step bisection's final midpoint is the centre of the dyadic
//     cell of the bracket that holds t* (col_dyadic).
// The two halves of a row meet in LDS once per round; every round decision
// is uniform over the workgroup.  O = P V on MFMA, bf16 P split into a high
// and a low part so that P keeps about 16 bits; pairs whose P is zero for a
// wave's rows are skipped by that wave.  The first V pair is fetched before
// the rounds.
#pragma once

#include <type_traits>

#include "col_solve.hpp"
#include "common.hpp"
#include "fwd_short.hpp"

namespace ea {

template <int DT, int D>
struct RegCfg {
    static constexpr int PK = 128;                       // keys per staged pair of chunks
    static constexpr int NP = 8;                         // pairs held: spans of up to 1024 keys
    static constexpr int NT = NP * 4;                    // 16-key tiles per wave
    static constexpr int BM = 32;                        // query rows per workgroup
    static constexpr int ESZ = DT == DT_BF16 ? 2 : 4;
    static constexpr int EPC = 16 / ESZ;                 // elements per 16-byte piece
    static constexpr int CPR = D / EPC;                  // pieces per row
    static constexpr int NPC = PK * CPR / kThreads;      // pieces per thread per pair
    static constexpr int KSTR = D * ESZ + 32;            // K row stride in LDS (bytes): conflict-free tile reads
    static constexpr int k_bytes = PK * KSTR;
    static constexpr int VRS = D * 2 + 32;               // bf16: V row stride (bytes)
    static constexpr int VSTR = PK + EPC;                // fp32: V^T row stride (elements)
    static constexpr int v_bytes = DT == DT_BF16 ? PK * VRS : D * VSTR * 4;
    static constexpr int buf_bytes = k_bytes > v_bytes ? k_bytes : v_bytes;
    // row exchange: [parity 2][wave 4][row 16] x f32x4, then [parity 2][wave 4] votes
    static constexpr int xch_bytes = 2 * 4 * 16 * 16 + 2 * 4 * 4;
    static constexpr size_t lds_bytes = static_cast<size_t>(2) * buf_bytes + xch_bytes;
    static constexpr int RB = D * ESZ;                   // bytes per K / V row in HBM
    static constexpr int RS = RB == 128 ? 7 : RB == 256 ? 8 : 9;
    static constexpr int kRounds = 16;                   // threshold rounds at most
    static constexpr float kStop = 1e-5f;                // a step below this ends a row's rounds
    static_assert(NPC >= 1 && (1 << RS) == RB, "whole pieces per thread; row bytes a power of two");
    static_assert(BM * D * 4 <= 2 * buf_bytes, "the halves' partial O fit the staging buffers");
};

template <int DT, int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_reg_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef RegCfg<DT, D> C;
    constexpr int PK = C::PK, NP = C::NP, NT = C::NT;
    // register sets for K and V pairs in flight: two at d = 64 (the loads run
    // two pairs ahead of the products); at d = 128 a second set would spill
    constexpr int NS = D == 64 ? (DT == DT_BF16 ? 3 : 2) : 1;
    extern __shared__ float lds[];
    char* buf = reinterpret_cast<char*>(lds);                                // 2 staging buffers
    f32x4* xch = reinterpret_cast<f32x4*>(buf + 2 * C::buf_bytes);          // row exchange
    int* votes = reinterpret_cast<int*>(xch + 2 * 4 * 16);

    const int total = a.B * a.H * a.nqt;
    const int wi = xcd_swizzle(blockIdx.x, total);
    const int bh = wi / a.nqt;
    const int qt = wi - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * C::BM;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const char* kc = reinterpret_cast<const char*>(static_cast<const T*>(a.k) + kv_off);
    const char* vc = reinterpret_cast<const char*>(static_cast<const T*>(a.v) + kv_off);
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int rg = wv & 1, hf = wv >> 1;
    const int g = lane / 16, c = lane % 16;
    const int rbase = q0 + 16 * rg;
    const int qrow = rbase + c;
    const bool rowok = qrow < L;
    const bool allrows = rbase + 16 <= L;   // uniform

    int klo, khi;   // keys of the workgroup's rows
    key_range(q0, C::BM, L, a.causal, a.window, &klo, &khi);
    const int j0 = klo / PK, j1 = (khi + PK - 1) / PK;   // pairs; j1 - j0 <= NP (host check)
    int wlo, whi;   // keys of this wave's rows
    key_range(rbase, 16, L, a.causal, a.window, &wlo, &whi);

    QFrag<DT, D> qf;
    qf.load(qh, qrow, L, g);

    // ---- staging of one pair (K or V) -----------------------------------------------------
    struct Pre {
        u32x4 p[C::NPC];
        uint8_t m0, m1;
    };
    auto prefetch = [&](int jp, const char* src, Pre& pr) {
        const int cb = jp * PK;
        pr.m0 = km != nullptr ? km[clamp_row(cb + lane, L)] : uint8_t(1);
        pr.m1 = km != nullptr ? km[clamp_row(cb + 64 + lane, L)] : uint8_t(1);
#pragma unroll
        for (int j = 0; j < C::NPC; ++j) {
            const int pc = tid + kThreads * j;
            const unsigned off = (static_cast<unsigned>(clamp_row(cb + pc / C::CPR, L)) << C::RS) + (pc % C::CPR) * 16u;
            pr.p[j] = *reinterpret_cast<const u32x4*>(src + off);
        }
    };
    auto stage_k = [&](int bi, const Pre& pr) {
        char* kb = buf + bi * C::buf_bytes;
#pragma unroll
        for (int j = 0; j < C::NPC; ++j) {
            const int pc = tid + kThreads * j;
            *reinterpret_cast<u32x4*>(kb + (pc / C::CPR) * C::KSTR + (pc % C::CPR) * 16) = pr.p[j];
        }
    };
    auto stage_v = [&](int bi, const Pre& pr) {
        char* vb = buf + bi * C::buf_bytes;
#pragma unroll
        for (int j = 0; j < C::NPC; ++j) {
            const int pc = tid + kThreads * j;
            const int key = pc / C::CPR, d0 = (pc % C::CPR) * C::EPC;
            if constexpr (DT == DT_BF16) {
                *reinterpret_cast<u32x4*>(vb + key * C::VRS + d0 * 2) = pr.p[j];
            } else {
#pragma unroll
                for (int e = 0; e < C::EPC; ++e)
                    reinterpret_cast<float*>(vb)[(d0 + e) * C::VSTR + key] = __uint_as_float(pr.p[j][e]);
            }
        }
    };
    // valid-key bits of this wave's chunk of pair jp (key < L and key mask)
    auto bits = [&](int jp, const Pre& pr) {
        const int key = jp * PK + 64 * hf + lane;
        return __ballot(key < L && (hf ? pr.m1 : pr.m0) != 0);
    };

    // ---- 1. S = Q K^T into registers, row maxima and allowed counts --------------------------
    constexpr unsigned kMaskedBits = DT == DT_BF16 ? 0xF149u : 0xF149F2CAu;   // -1e30
    const int khi_i = qrow;                                  // causal: key <= query
    const int klo_i = a.window > 0 ? qrow - a.window : -1;   // window: key > query - W
    f32x4 S[NT];
    float mlane = -kInf, nl = 0.f;
    float mpair[NP];   // this lane's maximum of each pair
    {
        // NS register sets: pairs are fetched NS ahead of the products
        Pre pr[NS];
        prefetch(j0, kc, pr[0]);
        if (NS >= 2 && j0 + 1 < j1) prefetch(j0 + 1, kc, pr[1 % NS]);
        if (NS >= 3 && j0 + 2 < j1) prefetch(j0 + 2, kc, pr[2 % NS]);
        stage_k(0, pr[0]);
        unsigned long long M = bits(j0, pr[0]);
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < NP; ++jj) {
            const int jp = j0 + jj;
            if (jp >= j1) {   // uniform
#pragma unroll
                for (int t = 0; t < 4; ++t) S[4 * jj + t] = f32x4{-kInf, -kInf, -kInf, -kInf};
                mpair[jj] = -kInf;
                continue;
            }
            if (jp + NS < j1) prefetch(jp + NS, kc, pr[jj % NS]);   // this set was staged last step
            const char* kb = buf + (jj & 1) * C::buf_bytes + (64 * hf + c) * C::KSTR + 16 * g;
            const int cb = jp * PK + 64 * hf;
            // a clean chunk (every key valid, no causal / window bound
            // crossing the wave's rows, every row a query row: uniform) takes
            // plain products and no masking
            const bool cross = a.causal && (cb + 63 > rbase || (a.window > 0 && cb <= rbase + 15 - a.window));
            float mpr = -kInf;   // this lane's maximum over the pair
            auto tiles = [&](auto clean_tag) {
                constexpr bool CLEAN = decltype(clean_tag)::value;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f32x4 sv = {-kInf, -kInf, -kInf, -kInf};
                    if constexpr (CLEAN) {
                        KFrag<DT, D> kf;
                        kf.load_lds_at(kb + 16 * t * C::KSTR);
                        sv = kf.st(qf);
                        mpr = fmaxf(mpr, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
                    } else {
                        const unsigned mb = static_cast<unsigned>((M >> (16 * t)) & 0xFFFFull);
                        const bool ok = mb != 0u && cb + 16 * t < whi && cb + 16 * t + 16 > wlo;   // uniform
                        if (ok) {
                            KFrag<DT, D> kf;
                            kf.load_lds_at(kb + 16 * t * C::KSTR);
                            sv = kf.st_bias(qf, ((mb >> c) & 1u) ? 0u : kMaskedBits, g);
                            if (a.causal) {
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int key = cb + 16 * t + 4 * g + i;
                                    sv[i] = ((key <= khi_i) & (key > klo_i)) ? sv[i] : -kInf;
                                }
                            }
#pragma unroll
                            for (int i = 0; i < 4; ++i) sv[i] = rowok ? sv[i] : -kInf;
                            mpr = fmaxf(mpr, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
                            if (a.causal) {
#pragma unroll
                                for (int i = 0; i < 4; ++i) nl += sv[i] > -1e29f ? 1.f : 0.f;
                            }
                        }
                    }
                    S[4 * jj + t] = sv;
                }
            };
            if (M == ~0ull && !cross && allrows) tiles(std::true_type{});
            else tiles(std::false_type{});
            mpair[jj] = mpr;
            mlane = fmaxf(mlane, mpr);
            if (a.causal && M == ~0ull && !cross && allrows) nl += 16.f;   // four clean tiles: 16 keys of this lane
            if (!a.causal) nl += static_cast<float>(__popcll(M));
            if (jp + 1 < j1) {
                stage_k((jj + 1) & 1, pr[(jj + 1) % NS]);
                M = bits(jp + 1, pr[(jj + 1) % NS]);
            }
            __syncthreads();
        }
    }
    if (!a.causal) nl = (g == 0 && rowok) ? nl : 0.f;

    // one value per row and wave to the partner wave (same rows, other half);
    // the exchanges alternate between two slots, so that one barrier per
    // call suffices.  With a vote: every wave also tells whether its flag
    // was set, and all four waves learn whether any flag was.
    int xp = 0;
    auto exchange_vote = [&](f32x4 v, bool flag, bool* any) -> f32x4 {
        if (g == 0) xch[(xp * 4 + wv) * 16 + c] = v;
        if (lane == 0) votes[xp * 4 + wv] = flag ? 1 : 0;
        __syncthreads();
        const f32x4 o = xch[(xp * 4 + (wv ^ 2)) * 16 + c];
        *any = (votes[xp * 4] | votes[xp * 4 + 1] | votes[xp * 4 + 2] | votes[xp * 4 + 3]) != 0;
        xp ^= 1;
        return o;
    };
    auto exchange = [&](f32x4 v) -> f32x4 {
        bool unused;
        return exchange_vote(v, false, &unused);
    };

    // ---- 2. the threshold ------------------------------------------------------------------
    // V of the first pair is fetched now; its latency passes under the rounds
    Pre prv[NS];   // as for K, NS pairs ahead
    prefetch(j0, vc, prv[0]);
    if (NS >= 2 && j0 + 1 < j1) prefetch(j0 + 1, vc, prv[1 % NS]);
    if (NS >= 3 && j0 + 2 < j1) prefetch(j0 + 2, vc, prv[2 % NS]);
    const float c2 = 0.5f * a.scale;
    const f32x4 mw = {col4_max(mlane), col4_sum(nl), 0.f, 0.f};
    const f32x4 mp = exchange(mw);
    const float mrow = fmaxf(mw[0], mp[0]);
    const float n = mw[1] + mp[1];   // allowed keys of the row, both halves
    const bool empty = n == 0.f;
    const float mc2 = empty ? 0.f : mrow * c2;
    const float hi = -__builtin_amdgcn_rsqf(empty ? 1.f : n);
    // A lower bound of the root from a subset of the row: the larger of the
    // two halves' roots over their four lane maxima (each at or below the
    // root over the row's eight), then two Newton steps (as below, from the
    // left) over the row's 64 pair maxima, the halves adding their sums
    // through LDS; the iterates stay at or below that subset's root.  (Each
    // half stepping on its own 32 maxima left one round more per row group
    // in a float64 simulation of the long workload: 4.0 against 3.3.)
    const float lbw = fmaxf(col_lower_bound(fmaf(mlane, c2, -mc2)), -1.f);
    const f32x4 lp = exchange(f32x4{lbw, 0.f, 0.f, 0.f});
    float t = fmaxf(lbw, lp[0]);   // the same in both halves
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int jj = 0; jj < NP; ++jj) {
            const float y = relu1(fmaf(mpair[jj], c2, -(mc2 + t)));
            s1 += y;
            s2 = fmaf(y, y, s2);
        }
        s1 = col4_sum(s1);
        s2 = col4_sum(s2);
        const f32x4 pq = exchange(f32x4{s1, s2, 0.f, 0.f});
        const float S1 = s1 + pq[0], S2 = s2 + pq[1];   // addition commutes: both halves agree
        const float rg = __builtin_amdgcn_sqrtf(S2);
        // S1 = 0 where the row holds nothing above the bound
        t += S1 > 0.f ? fmaxf((rg - 1.f) * rg * __builtin_amdgcn_rcpf(S1), 0.f) : 0.f;
    }
    t = fminf(t, hi);
    const bool trivial = empty || n <= 1.f;   // n = 1: the root is the lower end -1
    const int nt = 4 * (j1 - j0);             // tiles holding keys (uniform)

    // Newton step on sqrt(g) - 1 from the sums over both halves; the same
    // value in both waves of the row group (addition commutes)
    auto newton_step = [&](float s1, float s2, f32x4 pp) {
        const float S1 = s1 + pp[0], S2 = s2 + pp[1];
        const float rg = __builtin_amdgcn_sqrtf(S2);   // (sqrt(g))' = -S1 / sqrt(g)
        return (rg - 1.f) * rg * __builtin_amdgcn_rcpf(S1);
    };

    // A round whose vote finds no wave with an open row ends the loop (every
    // wave skipped its pass in it): one barrier per round.
    bool done = trivial;
#pragma unroll 1
    for (int r = 0; r <= C::kRounds; ++r) {
        const bool open = __any(!done);
        float s1 = 0.f, s2 = 0.f;
        if (open && r < C::kRounds) {   // a wave whose rows are all done skips the pass (so does its partner)
            const float bias = -(mc2 + t);
            float u1 = 0.f, u2 = 0.f;   // two chains each
            auto tile = [&](int k) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float y = relu1(fmaf(S[k][i], c2, bias));
                    if (i & 1) {
                        u1 += y;
                        u2 = fmaf(y, y, u2);
                    } else {
                        s1 += y;
                        s2 = fmaf(y, y, s2);
                    }
                }
            };
            if (nt == NT) {   // uniform: every tile holds keys, one straight block
#pragma unroll
                for (int k = 0; k < NT; ++k) tile(k);
            } else {
                // tiles past the span hold -inf (y = 0): skipped, a pair at a time
#pragma unroll
                for (int k = 0; k < NT; k += 4)
                    if (k < nt) {   // uniform
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) tile(k + kk);
                    }
            }
            s1 = col4_sum(s1 + u1);
            s2 = col4_sum(s2 + u2);
        }
        bool any_open;
        const f32x4 pp = exchange_vote(f32x4{s1, s2, 0.f, 0.f}, open, &any_open);
        if (!any_open || r == C::kRounds) break;   // uniform
        if (!done) {
            const float step = newton_step(s1, s2, pp);
            t = fminf(t + fmaxf(step, 0.f), hi);
            done = step < C::kStop;
        }
    }
    const float tx = t;
    float tf = -1.f;
    if (!trivial) {
        ColState st;
        st.lo = -1.f;
        st.hi = hi;
        st.it = 0;
        tf = col_dyadic(st, tx);
    }
    if (a.tau != nullptr && g == 0 && hf == 0 && rowok)
        a.tau[static_cast<size_t>(bh) * L + qrow] = empty ? kInf : 2.f * (mc2 + tf);
    // p = relu(s c2 + pb)^2; an empty row has no finite score and gets pb = -inf
    const float pb = empty ? -kInf : -(mc2 + tf);

    // ---- 3. O = P V --------------------------------------------------------------------------
    f32x4 o[D / 16];
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        stage_v(0, prv[0]);
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < NP; ++jj) {
            const int jp = j0 + jj;
            if (jp >= j1) continue;   // uniform
            if (jp + NS < j1) prefetch(jp + NS, vc, prv[jj % NS]);   // this set was staged last step
            // the lane's largest score of the pair decides whether any of its
            // p is nonzero (fma with c2 > 0 is monotone in the score)
            const bool nz = fmaf(mpair[jj], c2, pb) > 0.f;
            if (__any(nz)) {   // uniform over the wave
                float y[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[t][i] = relu1(fmaf(S[4 * jj + t][i], c2, pb));
                const char* vb = buf + (jj & 1) * C::buf_bytes;
                if constexpr (DT == DT_BF16) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        float y8[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            y8[i] = y[2 * h2][i];
                            y8[4 + i] = y[2 * h2 + 1][i];
                        }
                        bf16x8 phi, plo;
                        split_sq_bf16(y8, phi, plo);
#pragma unroll
                        for (int ct = 0; ct < D / 16; ++ct) {
                            // B operand through transpose loads: keys 64 hf + 32 h2 + slot
                            const char* src = vb + (64 * hf + 32 * h2 + 4 * g + (c >> 2)) * C::VRS + (16 * ct + 4 * (c & 3)) * 2;
                            const s16x4 r0 = ds_read_tr16(src);
                            const s16x4 r1 = ds_read_tr16(src + 16 * C::VRS);
                            const bf16x8 bv = __builtin_bit_cast(bf16x8, s16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]});
                            o[ct] = mfma_bf16(phi, bv, o[ct]);
                            o[ct] = mfma_bf16(plo, bv, o[ct]);
                        }
                    }
                } else {
                    const float* vt = reinterpret_cast<const float*>(vb);
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int ct = 0; ct < D / 16; ++ct) {
                            const f32x4 bv = *reinterpret_cast<const f32x4*>(vt + (16 * ct + c) * C::VSTR + 64 * hf + 16 * t + 4 * g);
#pragma unroll
                            for (int q = 0; q < 4; ++q) o[ct] = mfma_f32(y[t][q] * y[t][q], bv[q], o[ct]);
                        }
                }
            }
            if (jp + 1 < j1) stage_v((jj + 1) & 1, prv[(jj + 1) % NS]);
            __syncthreads();
        }
    }

    // ---- 4. the halves' partial O: half 1 through LDS, half 0 adds and stores -------------
    float* po = reinterpret_cast<float*>(buf) + rg * 16 * D;   // [row group][16 rows][D]
    if (hf == 1) {
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) po[(4 * g + i) * D + 16 * ct + c] = o[ct][i];
    }
    __syncthreads();
    if (hf == 0) {
        float* outh = a.out + head_off;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = rbase + 4 * g + i;
                if (row < L) outh[static_cast<size_t>(row) * D + 16 * ct + c] = o[ct][i] + po[(4 * g + i) * D + 16 * ct + c];
            }
    }
}

}  // namespace ea
