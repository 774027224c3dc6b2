// Backward pass of 1.5-entmax attention for long key spans, with 64 rows of
// the stationary operand per wave, and the key side (dK, dV) for every span.
//
// Jacobian ("ADASPLASH -- ROBERTA Benchmark Result", section 2.4; "RoBERTa
// Base with AdaSplash Attention" model card, Mathematical Formulation 2):
// with w_ij = sqrt(p_ij) = (s_ij - tau_i)/2 on the support, dp_ij = dO_i . V_j
// and c_i = sum_j w_ij dp_ij / sum_j w_ij,
//   dS_ij = w_ij (dp_ij - c_i),  dQ_i = scale sum_j dS_ij K_j,
//   dK_j = scale sum_i dS_ij Q_i,  dV_j = sum_i p_ij dO_i.
//
// Both kernels keep NF fragments of 16 rows of one operand in registers
// (the stationary rows: 64 per wave in bf16) and stream the other operand
// through LDS in chunks of 64 rows shared by the four waves
// (chunk_stream.hpp).  Holding 64 rows per wave lets every LDS read of the
// streamed operand feed NF products, which keeps the score recompute near
// the MFMA rate instead of the LDS rate.
//
//  * bwd_q_kernel (query rows stationary, keys streamed): the support
//    entries of each row (s_ij > tau_i) go to the row's list, kept in the
//    row's own dQ row (still unwritten: D/2 entries of (w, key), D/8 per
//    lane, lane-private so that an append is one store, entry e of lane
//    group g at slot 4 e + g so that a row's first entries share one
//    32-byte sector); afterwards each row
//    gathers V_j and K_j of its entries and forms c_i and
//    dQ_i = scale (sum w dp K - c_i sum w K).  A row whose support outgrows
//    its lists gets the overflow marker in c_i, and the tile-wise kernel of
//    bwd.hpp finishes it in fix-up mode.
//    With support buckets (kcnt non-null), every entry (i, j) with w > 0
//    also goes to key j's bucket: (query, w, w dp), 16 bytes, at a slot
//    taken with an integer atomic on kcnt_j, stored in j's dK and dV rows
//    (still unwritten: KCAP = D/2 slots).
//  * bwd_q_saved_kernel: the same per-row work on the support the wide
//    forward kept (entries with p > 0 as (w, key) in a caller's buffer), so
//    no score is formed: D/8 lanes per row, 8 columns each; a row the
//    forward did not keep goes to the fix-up as an overflowing row does.
//  * bwd_kv_gather_kernel: per key, the bucket is put in query order and
//    summed: dK_j = scale sum (w dp - w c_i) Q_i, dV_j = sum w^2 dO_i.  The
//    order is fixed by the entries themselves, not by the atomics, so
//    repeated calls give identical bits.  A key whose bucket overflowed is
//    left to bwd_kv_kernel in fix-up mode (all keys when some query row
//    overflowed its list and emitted nothing).
//  * bwd_kv_kernel (keys stationary, query rows streamed): the same scores
//    transposed; the support entries of each key (query index, w) go to the
//    key's list.  A list that cannot take a tile's entries is flushed (the
//    chunk's tiles from that one on are then redone), and every list is
//    flushed at the end of each query head: gather dO_i, Q_i and c_i,
//    dp = dO_i . V_j, then dK_j += scale w (dp - c_i) Q_i and
//    dV_j += w^2 dO_i.  Each key row of dK and dV belongs to one lane group
//    of one workgroup, so the accumulation is a plain read-modify-write in a
//    fixed order: no atomics, and repeated calls give identical bits.
#pragma once

#include <type_traits>

#include "bwd.hpp"
#include "chunk_stream.hpp"
#include "col_solve.hpp"
#include "common.hpp"
#include "fwd_short.hpp"
#include "wide.hpp"

namespace ea {

// ============================================================================
// Query side: dQ and c for rows of long key spans
// ============================================================================
template <int DT, int D>
__global__ __launch_bounds__(kThreads, (WideCfg<DT, D>::kOcc)) void bwd_q_kernel(BwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef WideCfg<DT, D> C;
    constexpr int NF = C::NF, CK = C::CK, DQ = C::DQ, NB = C::NB;
    constexpr int SUB = D / 8;     // list entries per lane (8 bytes each in the row's dQ)
    constexpr int NBQ = DT == DT_BF16 ? (D == 128 ? 3 : 4) : 2;   // support entries gathered per batch (registers)
    extern __shared__ float lds[];
    char* Kb = reinterpret_cast<char*>(lds);

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
    const T* doh = static_cast<const T*>(a.dout) + head_off;
    float* dqh = a.dq + head_off;
    float* ch = a.cbuf + static_cast<size_t>(bh) * L;
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

    QFrag<DT, D> qf[NF];
    float tau[NF], traw[NF];
    int cnt[NF];        // entries in this lane's list of the row
    bool ovf[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int row = rbase + 16 * f + c;
        qf[f].load(qh, row, L, g);
        tau[f] = row < L ? a.tau[static_cast<size_t>(bh) * L + clamp_row(row, L)] : kInf;
        // raw-accumulator threshold, a little low (the exact test is the fma
        // below); +inf for rows without an allowed key
        const float tr = tau[f] / a.scale;
        traw[f] = tau[f] < kInf ? tr - 1e-6f * fabsf(tr) - 1e-30f : kInf;
        cnt[f] = 0;
        ovf[f] = false;
    }
    const bool allrows = rbase + NF * 16 <= L;
    // support buckets of the key side: query head within its group, and the
    // key/value head's dK, dV rows and counters
    const unsigned hq16 = static_cast<unsigned>((bh - b * a.H) % (a.H / a.Hkv)) << 16;
    int* kch = a.kcnt != nullptr ? a.kcnt + static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L : nullptr;
    float* dkb = a.dk + kv_off;
    float* dvb = a.dv + kv_off;
    // this lane's list of row f: entries (w, key bits) in the row's dQ,
    // entry e at [4 e]
    auto lst = [&](int f, int lane_g) {
        return reinterpret_cast<f32x2*>(dqh + static_cast<size_t>(clamp_row(rbase + 16 * f + c, L)) * D) + lane_g;
    };

    ChunkStream<DT, D, 2, 1> cs;
    cs.Kb = Kb;
    cs.Vb = nullptr;
    cs.kh = kh;
    cs.vh = vh;
    cs.kmp = hasm ? km : reinterpret_cast<const uint8_t*>(qh);
    cs.hasm = hasm;
    cs.L = L;
    cs.tid = tid;
    cs.lane = lane;
    constexpr unsigned kMaskedBits = DT == DT_BF16 ? 0xF149u : 0xF149F2CAu;   // -1e30
    const int klane = c * C::KSTR + 16 * g;

    // ---- support lists ----------------------------------------------------------------
    // A chunk of valid keys that no causal / window bound crosses and whose
    // rows are all query rows ("clean", uniform) takes plain products and no
    // masking; the support test itself only runs for a fragment whose
    // running maximum clears one of its rows' thresholds.
    auto body = [&](auto clean_tag, int cb, const char* kb, unsigned long long M) {
        constexpr bool CLEAN = decltype(clean_tag)::value;
        f32x4 s[NF][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (CLEAN) {
                f32x4 o[NF];
                tile_products<DT, D, NF>(kb + klane + 16 * t * C::KSTR, qf, o);
#pragma unroll
                for (int f = 0; f < NF; ++f) s[f][t] = o[f];
            } else {
                const unsigned mb = static_cast<unsigned>((M >> (16 * t)) & 0xFFFFull);
                const bool ok = mb != 0u && cb + 16 * t < whi && cb + 16 * t + 16 > wlo;   // uniform
                if (!ok) {
#pragma unroll
                    for (int f = 0; f < NF; ++f) s[f][t] = f32x4{-kInf, -kInf, -kInf, -kInf};
                    continue;
                }
                const unsigned bias = ((mb >> c) & 1u) ? 0u : kMaskedBits;
                f32x4 o[NF];
                tile_products<DT, D, NF, true>(kb + klane + 16 * t * C::KSTR, qf, o, bias, g);
#pragma unroll
                for (int f = 0; f < NF; ++f) s[f][t] = o[f];
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int row = rbase + 16 * f + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = cb + 16 * t + 4 * g + i;
                        const bool okk = row < L && (!a.causal || allowed_ij(row, key, 1, a.window));
                        s[f][t][i] = okk ? s[f][t][i] : -kInf;
                    }
                }
            }
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            float tm[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) tm[t] = fmaxf(fmaxf(s[f][t][0], s[f][t][1]), fmaxf(s[f][t][2], s[f][t][3]));
            if (!__any(fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3])) > traw[f])) continue;   // uniform: no support entry here
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (!__any(tm[t] > traw[f])) continue;   // uniform: none in this tile
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (s[f][t][i] > traw[f]) {
                        // w = (s - tau)/2; an entry the low raw threshold let in
                        // by rounding gets w = 0 and contributes nothing
                        if (cnt[f] < SUB)
                            lst(f, g)[4 * cnt[f]] = f32x2{fmaxf(0.5f * fmaf(s[f][t][i], a.scale, -tau[f]), 0.f),
                                                      __uint_as_float(static_cast<unsigned>(cb + 16 * t + 4 * g + i))};
                        else
                            ovf[f] = true;
                        ++cnt[f];
                    }
                }
            }
        }
    };
    cs.run(ch0, ch1, false, [&](int chn, const char* kb, const char*, unsigned long long M) {
        const int cb = chn * CK;
        if (cb >= whi || cb + CK <= wlo) return;   // uniform: none of the wave's keys
        const bool cross = a.causal && (cb + CK - 1 > rbase || (a.window > 0 && cb <= rbase + NF * 16 - 1 - a.window));
        if (M == ~0ull && !cross && allrows) body(std::true_type{}, cb, kb, M);
        else body(std::false_type{}, cb, kb, M);
    });
    // the lists written by the row's four lanes are visible to all of them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    // ---- c and dQ per row ---------------------------------------------------------------
#pragma unroll 1
    for (int f = 0; f < NF; ++f) {
        const int row = rbase + 16 * f + c;
        const bool rovf = col4_sum_int(ovf[f] ? 1 : 0) != 0;   // some lane's list overflowed
        const int len = rovf ? 0 : min(cnt[f], SUB);
        float dor[DQ];
        load_cols<DT, DQ>(doh + static_cast<size_t>(clamp_row(row, L)) * D + g * DQ, dor);
        float X[DQ], Y[DQ], sw = 0.f, swdp = 0.f;
#pragma unroll
        for (int d = 0; d < DQ; ++d) { X[d] = 0.f; Y[d] = 0.f; }
        // the four lanes' lists in one index space, in lane-group order: lane
        // group g2's k-th entry is number P[g2] + k of the row, so that one
        // batch of gathers spans the lists (the summation order is the
        // lists' order)
        int P[4];
        P[0] = 0;
#pragma unroll
        for (int g2 = 0; g2 < 3; ++g2) P[g2 + 1] = P[g2] + __shfl(len, 16 * g2 + c, kWave);
        const int T = P[3] + __shfl(len, 48 + c, kWave);
        const int Tmax = wave_max_int<kWave>(T);
#pragma unroll 1
        for (int e0 = 0; e0 < Tmax; e0 += NBQ) {
            int key[NBQ], own[NBQ];
            float w[NBQ];
            RowSlice<DT, DQ> vr[NBQ], kr[NBQ];
#pragma unroll
            for (int j = 0; j < NBQ; ++j) {
                const int e = e0 + j;
                const bool in = e < T;
                const int g2 = (e >= P[1] ? 1 : 0) + (e >= P[2] ? 1 : 0) + (e >= P[3] ? 1 : 0);
                const int k = e - (g2 == 0 ? 0 : g2 == 1 ? P[1] : g2 == 2 ? P[2] : P[3]);
                const f32x2 en = lst(f, in ? g2 : 0)[4 * (in ? k : 0)];
                key[j] = in ? static_cast<int>(__float_as_uint(en[1])) : 0;
                w[j] = in ? en[0] : 0.f;
                own[j] = in ? g2 : -1;   // the lane group whose list holds the entry
            }
#pragma unroll
            for (int j = 0; j < NBQ; ++j) {
                vr[j].load(vh + static_cast<size_t>(key[j]) * D + g * DQ);
                kr[j].load(kh + static_cast<size_t>(key[j]) * D + g * DQ);
            }
#pragma unroll
            for (int j = 0; j < NBQ; ++j) {
                float part = 0.f;
#pragma unroll
                for (int d = 0; d < DQ; ++d) part = fmaf(dor[d], vr[j].at(d), part);
                const float dp = col4_sum(part);
                sw += w[j];
                swdp = fmaf(w[j], dp, swdp);
                const float wdp = w[j] * dp;
#pragma unroll
                for (int d = 0; d < DQ; ++d) {
                    X[d] = fmaf(wdp, kr[j].at(d), X[d]);
                    Y[d] = fmaf(w[j], kr[j].at(d), Y[d]);
                }
                // the list's own lane hands the entry to key j's bucket
                if (kch != nullptr && g == own[j] && w[j] > 0.f) {
                    const int slot = atomicAdd(kch + key[j], 1);
                    if (slot < D / 2) {
                        float* dst = (slot < D / 4 ? dkb : dvb) + static_cast<size_t>(key[j]) * D + 4 * (slot % (D / 4));
                        *reinterpret_cast<u32x4*>(dst) =
                            u32x4{hq16 | static_cast<unsigned>(row), __float_as_uint(w[j]), __float_as_uint(wdp), 0u};
                    }
                }
            }
        }
        // every lane of the wave has read the row's lists before dQ overwrites them
        __builtin_amdgcn_wave_barrier();
        if (row < L) {
            if (rovf) {
                if (g == 0) {
                    reinterpret_cast<unsigned*>(ch)[row] = kCMarker;   // finished by the fix-up pass
                    if (a.kflag != nullptr) *a.kflag = 1;             // its entries are in no bucket
                }
            } else {
                const float cc = sw > 0.f ? swdp / sw : 0.f;
                float* dst = dqh + static_cast<size_t>(row) * D + g * DQ;
#pragma unroll
                for (int d = 0; d < DQ; d += 4)
                    *reinterpret_cast<f32x4*>(dst + d) =
                        f32x4{a.scale * fmaf(-cc, Y[d], X[d]), a.scale * fmaf(-cc, Y[d + 1], X[d + 1]),
                              a.scale * fmaf(-cc, Y[d + 2], X[d + 2]), a.scale * fmaf(-cc, Y[d + 3], X[d + 3])};
                if (g == 0) ch[row] = cc;
            }
        }
    }
}

// ============================================================================
// Query side on the forward's saved support
// ============================================================================
// D/8 lanes per query row (8 columns each), 256/(D/8) rows per workgroup;
// grid: ceil(B H L / rows per workgroup).  Entries are taken in the order
// the forward kept them; per entry the row's lanes gather V_j and K_j.
// bf16: five waves per SIMD (96 registers, a few bytes spilled) hide more
// of the gather latency than four (110 registers): 424 -> 413 us on the
// long-context backward; six spill heavily.
template <int DT, int D>
__global__ __launch_bounds__(kThreads, (DT == DT_BF16 ? 5 : 1)) void bwd_q_saved_kernel(BwdArgs a) {
    typedef typename InT<DT>::type T;
    constexpr int LPR = D / 8;          // lanes per row
    constexpr int CPL = 8;              // columns per lane
    constexpr int NBS = 2;              // entries gathered per batch (long-context backward: 404 us at 2, 413 at 4; 8 spills)
    const int tid = threadIdx.x;
    const int l = tid % LPR;            // the lane's column group
    const long long rows = static_cast<long long>(a.B) * a.H * a.L;
    const long long gr = static_cast<long long>(blockIdx.x) * (kThreads / LPR) + tid / LPR;
    const bool valid = gr < rows;       // the same in a row's lanes
    const long long r = valid ? gr : 0;
    const int bh = static_cast<int>(r / a.L);
    const int row = static_cast<int>(r - static_cast<long long>(bh) * a.L);
    const int b = bh / a.H;
    const int L = a.L;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const T* vh = static_cast<const T*>(a.v) + kv_off;
    // support buckets of the key side (query head within its group, row)
    const unsigned code = (static_cast<unsigned>((bh - b * a.H) % (a.H / a.Hkv)) << 16) | static_cast<unsigned>(row);
    int* kch = a.kcnt + static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L;
    float* dkb = a.dk + kv_off;
    float* dvb = a.dv + kv_off;

    const int ns = valid ? a.scount[r] : 0;
    const bool rovf = ns < 0;           // not kept by the forward: the fix-up finishes the row
    const int tn = rovf ? 0 : ns;
    const f32x2* se = reinterpret_cast<const f32x2*>(a.sent) + static_cast<size_t>(r) * (D / 2);
    float dor[CPL];
    load_cols<DT, CPL>(static_cast<const T*>(a.dout) + static_cast<size_t>(r) * D + l * CPL, dor);
    float X[CPL], Y[CPL], sw = 0.f, swdp = 0.f;
#pragma unroll
    for (int d = 0; d < CPL; ++d) { X[d] = 0.f; Y[d] = 0.f; }
    const int tmax = wave_max_int<kWave>(tn);
#pragma unroll 1
    for (int e0 = 0; e0 < tmax; e0 += NBS) {
        int key[NBS];
        float w[NBS];
        RowSlice<DT, CPL> vr[NBS], kr[NBS];
#pragma unroll
        for (int j = 0; j < NBS; ++j) {
            const bool in = e0 + j < tn;
            const f32x2 en = se[in ? e0 + j : 0];
            key[j] = in ? static_cast<int>(__float_as_uint(en[1])) : 0;
            w[j] = in ? en[0] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < NBS; ++j) {
            vr[j].load(vh + static_cast<size_t>(key[j]) * D + l * CPL);
            kr[j].load(kh + static_cast<size_t>(key[j]) * D + l * CPL);
        }
#pragma unroll
        for (int j = 0; j < NBS; ++j) {
            float part = 0.f;
#pragma unroll
            for (int d = 0; d < CPL; ++d) part = fmaf(dor[d], vr[j].at(d), part);
            const float dp = group_sum<LPR>(part);
            sw += w[j];
            swdp = fmaf(w[j], dp, swdp);
            const float wdp = w[j] * dp;
#pragma unroll
            for (int d = 0; d < CPL; ++d) {
                X[d] = fmaf(wdp, kr[j].at(d), X[d]);
                Y[d] = fmaf(w[j], kr[j].at(d), Y[d]);
            }
            // one lane of the row hands the entry to key j's bucket
            if (l == (e0 + j) % LPR && w[j] > 0.f) {
                const int slot = atomicAdd(kch + key[j], 1);
                if (slot < D / 2) {
                    float* dst = (slot < D / 4 ? dkb : dvb) + static_cast<size_t>(key[j]) * D + 4 * (slot % (D / 4));
                    *reinterpret_cast<u32x4*>(dst) = u32x4{code, __float_as_uint(w[j]), __float_as_uint(wdp), 0u};
                }
            }
        }
    }
    if (!valid) return;
    float* ch = a.cbuf + static_cast<size_t>(bh) * L;
    if (rovf) {
        if (l == 0) {
            reinterpret_cast<unsigned*>(ch)[row] = kCMarker;   // finished by the fix-up pass
            *a.kflag = 1;                                     // its entries are in no bucket
        }
        return;
    }
    const float cc = sw > 0.f ? swdp / sw : 0.f;
    float* dst = a.dq + static_cast<size_t>(r) * D + l * CPL;
#pragma unroll
    for (int d = 0; d < CPL; d += 4)
        *reinterpret_cast<f32x4*>(dst + d) =
            f32x4{a.scale * fmaf(-cc, Y[d], X[d]), a.scale * fmaf(-cc, Y[d + 1], X[d + 1]),
                  a.scale * fmaf(-cc, Y[d + 2], X[d + 2]), a.scale * fmaf(-cc, Y[d + 3], X[d + 3])};
    if (l == 0) ch[row] = cc;
}

// ============================================================================
// Key side from the support buckets
// ============================================================================
// D/8 lanes per key (8 features each), 256/(D/8) keys per workgroup.  grid:
// B H_kv ceil(L / keys per workgroup).
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void bwd_kv_gather_kernel(BwdArgs a) {
    typedef typename InT<DT>::type T;
    constexpr int KCAP = D / 2;      // bucket slots per key
    constexpr int LPK = D / 8;       // lanes per key
    constexpr int FPL = 8;           // features per lane
    constexpr int EPL = KCAP / LPK;  // bucket slots per lane while ordering
    constexpr int KPB = kThreads / LPK;
    constexpr int UB = 2;            // entries gathered per batch (59 registers at 2; 82 at 4, 32 us slower)
    __shared__ u32x4 srt[KPB][KCAP];
    if (*a.kflag != 0) return;       // uniform: the recompute kernel does every key

    const int L = a.L;
    const int nkg = (L + KPB - 1) / KPB;
    const int total = a.B * a.Hkv * nkg;
    const int wi = xcd_swizzle(blockIdx.x, total);
    const int bkv = wi / nkg;
    const int b = bkv / a.Hkv;
    const int hk = bkv - b * a.Hkv;
    const int rep = a.H / a.Hkv;
    const int tid = threadIdx.x;
    const int ks = tid / LPK;        // key slot in the workgroup
    const int l = tid % LPK;
    const int key = (wi - bkv * nkg) * KPB + ks;
    const bool kin = key < L;
    const size_t kv_off = static_cast<size_t>(bkv) * L * D;
    float* dkr = a.dk + kv_off + static_cast<size_t>(kin ? key : 0) * D;
    float* dvr = a.dv + kv_off + static_cast<size_t>(kin ? key : 0) * D;
    const int n = kin ? a.kcnt[static_cast<size_t>(bkv) * L + key] : 0;
    const bool mine = kin && n <= KCAP;   // else the recompute kernel writes this key
    const int ne = mine ? n : 0;

    // bucket slots l, l + 16, ...; rank of each = entries with a smaller
    // (query head, query) code, all codes of one bucket being distinct
    u32x4 e[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const int s = l + LPK * r;
        const float* src = (s < D / 4 ? dkr : dvr) + 4 * (s % (D / 4));
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        e[r] = s < ne ? v : u32x4{0xFFFFFFFFu, 0u, 0u, 0u};
    }
    int rank[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) rank[r] = 0;
    const int nw = wave_max_int<kWave>(ne);
    const int gb = (tid % kWave) & ~(LPK - 1);   // first lane of this key's group
#pragma unroll
    for (int r2 = 0; r2 < EPL; ++r2) {
        if (LPK * r2 >= nw) break;   // uniform
#pragma unroll 4
        for (int l2 = 0; l2 < LPK; ++l2) {
            const unsigned o = static_cast<unsigned>(__shfl(static_cast<int>(e[r2][0]), gb + l2, kWave));
#pragma unroll
            for (int r = 0; r < EPL; ++r) rank[r] += o < e[r][0] ? 1 : 0;
        }
    }
#pragma unroll
    for (int r = 0; r < EPL; ++r)
        if (l + LPK * r < ne) srt[ks][rank[r]] = e[r];
    wave_sync();   // a key's lanes share one wave

    float dk[FPL], dv[FPL];
#pragma unroll
    for (int d = 0; d < FPL; ++d) { dk[d] = 0.f; dv[d] = 0.f; }
    const size_t hstride = static_cast<size_t>(L) * D;
    const T* q0 = static_cast<const T*>(a.q) + static_cast<size_t>(b * a.H + hk * rep) * hstride + l * FPL;
    const T* o0 = static_cast<const T*>(a.dout) + static_cast<size_t>(b * a.H + hk * rep) * hstride + l * FPL;
    const float* c0 = a.cbuf + static_cast<size_t>(b * a.H + hk * rep) * L;
    for (int e0 = 0; e0 < nw; e0 += UB) {
        float w[UB], wdp[UB], ci[UB];
        RowSlice<DT, FPL> qr[UB], orr[UB];
#pragma unroll
        for (int j = 0; j < UB; ++j) {
            const bool in = e0 + j < ne;
            const u32x4 en = srt[ks][in ? e0 + j : 0];
            const unsigned code = in ? en[0] : 0u;
            const size_t qrow = static_cast<size_t>(code >> 16) * L + (code & 0xFFFFu);
            w[j] = in ? __uint_as_float(en[1]) : 0.f;
            wdp[j] = in ? __uint_as_float(en[2]) : 0.f;
            qr[j].load(q0 + qrow * D);
            orr[j].load(o0 + qrow * D);
            ci[j] = c0[qrow];
        }
#pragma unroll
        for (int j = 0; j < UB; ++j) {
            const float ds = a.scale * fmaf(-w[j], ci[j], wdp[j]);
            const float p = w[j] * w[j];
#pragma unroll
            for (int d = 0; d < FPL; ++d) {
                dk[d] = fmaf(ds, qr[j].at(d), dk[d]);
                dv[d] = fmaf(p, orr[j].at(d), dv[d]);
            }
        }
    }
    if (mine) {
#pragma unroll
        for (int d = 0; d < FPL; d += 4) {
            *reinterpret_cast<f32x4*>(dkr + l * FPL + d) = f32x4{dk[d], dk[d + 1], dk[d + 2], dk[d + 3]};
            *reinterpret_cast<f32x4*>(dvr + l * FPL + d) = f32x4{dv[d], dv[d + 1], dv[d + 2], dv[d + 3]};
        }
    }
}

// ============================================================================
// Key side: dK and dV, by key ownership
// ============================================================================
template <int DT, int D>
__global__ __launch_bounds__(kThreads, (WideCfg<DT, D>::kOcc)) void bwd_kv_kernel(BwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef WideCfg<DT, D> C;
    constexpr int NF = C::NF, CK = C::CK, CAP = C::CAP, DQ = C::DQ;
    constexpr int NB = 1;   // flush gathers per batch: the flush runs beside the live chunk state
    extern __shared__ float lds[];
    char* Qb = reinterpret_cast<char*>(lds);
    float* lw = reinterpret_cast<float*>(Qb + 2 * C::k_bytes);
    uint16_t* lq = reinterpret_cast<uint16_t*>(lw + C::list_elems);
    float* tq_lds = reinterpret_cast<float*>(lq + C::list_elems);   // tau of the staged query chunks [2][64]

    const int nkt = a.nqt;   // key tiles per key/value head
    const int total = a.B * a.Hkv * nkt;
    const int wi = xcd_swizzle(blockIdx.x, total);
    const int bkv = wi / nkt;
    const int kt = wi - bkv * nkt;
    const int b = bkv / a.Hkv;
    const int hk = bkv - b * a.Hkv;
    const int rep = a.H / a.Hkv;
    const int k0 = kt * C::BR;
    const int L = a.L;
    const size_t kv_off = static_cast<size_t>(bkv) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const T* vh = static_cast<const T*>(a.v) + kv_off;
    float* dkh = a.dk + kv_off;
    float* dvh = a.dv + kv_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane / 16, c = lane % 16;
    const int kbase = k0 + wv * NF * 16;   // the wave's first key

    // query rows that may attend the workgroup's keys, and the wave's keys
    int qlo = 0, qhi = L, wqlo = 0, wqhi = L;
    if (a.causal) {
        qlo = k0;
        wqlo = kbase;
        if (a.window > 0) {
            qhi = min(L, k0 + C::BR - 1 + a.window);
            wqhi = min(L, kbase + NF * 16 - 1 + a.window);
        }
    }
    const int ch0 = qlo / CK, ch1 = qlo < qhi ? (qhi + CK - 1) / CK : ch0;

    // fix-up mode (after the bucket gather): only keys whose bucket
    // overflowed, or every key when some query row emitted no entries
    const bool every = !a.fixup || *a.kflag != 0;   // uniform
    const int* kcb = a.kcnt != nullptr ? a.kcnt + static_cast<size_t>(bkv) * L : nullptr;
    if (!every) {
        const int kt0 = k0 + tid;
        const bool over = tid < C::BR && kt0 < L && kcb[kt0] > D / 2;
        if (!__syncthreads_or(over)) return;
    }

    QFrag<DT, D> kf[NF];   // stationary keys in the B-operand layout
    bool kok[NF];
    bool kwr[NF];          // this call writes the key's rows
    int cnt[NF];           // entries in the key's list (the same in its four lanes)
    bool written[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int key = kbase + 16 * f + c;
        kf[f].load(kh, key, L, g);
        const uint8_t mb = km != nullptr ? km[clamp_row(key, L)] : uint8_t(1);
        kok[f] = key < L && mb != 0;
        kwr[f] = key < L && (every || kcb[key] > D / 2);
        cnt[f] = 0;
        written[f] = false;
    }
    bool kall_l = true;
#pragma unroll
    for (int f = 0; f < NF; ++f) kall_l = kall_l && kok[f];
    const bool kall = __all(kall_l);   // every key of the wave valid (uniform)
    auto slot_index = [&](int f, int s) { return ((wv * NF + f) * CAP + s) * 16 + c; };
    const int qlane = c * C::KSTR + 16 * g;
    const float inv_scale = 1.f / a.scale;

#pragma unroll 1
    for (int hh = 0; hh < rep; ++hh) {
        const int bh = b * a.H + hk * rep + hh;
        const size_t head_off = static_cast<size_t>(bh) * L * D;
        const T* qh = static_cast<const T*>(a.q) + head_off;
        const T* doh = static_cast<const T*>(a.dout) + head_off;
        const float* tauh = a.tau + static_cast<size_t>(bh) * L;
        const float* chh = a.cbuf + static_cast<size_t>(bh) * L;
        const bool last = hh == rep - 1;

        // Flush the list of fragment f into dK, dV (lane group g owns columns
        // [g DQ, (g + 1) DQ) of key kbase + 16 f + c).  Called by the whole
        // wave.  final_write: also write the rows of keys never written (zero
        // gradients).
        auto flush = [&](int f, bool final_write) {
            wave_sync();   // the other lanes' list writes are visible
            const int key = kbase + 16 * f + c;
            RowSlice<DT, DQ> vj;
            vj.load(vh + static_cast<size_t>(clamp_row(key, L)) * D + g * DQ);
            float dk[DQ], dv[DQ];
#pragma unroll
            for (int d = 0; d < DQ; ++d) { dk[d] = 0.f; dv[d] = 0.f; }
            const int n = cnt[f];
            const int nmax = wave_max_int<kWave>(n);
            for (int e0 = 0; e0 < nmax; e0 += NB) {
                int qi[NB];
                float w[NB], ci[NB];
                RowSlice<DT, DQ> dor[NB], qr[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const bool in = e0 + j < n;
                    const int idx = slot_index(f, in ? e0 + j : 0);
                    qi[j] = in ? static_cast<int>(lq[idx]) : 0;
                    w[j] = in ? lw[idx] : 0.f;
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    dor[j].load(doh + static_cast<size_t>(qi[j]) * D + g * DQ);
                    qr[j].load(qh + static_cast<size_t>(qi[j]) * D + g * DQ);
                    ci[j] = chh[qi[j]];
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    float part = 0.f;
#pragma unroll
                    for (int d = 0; d < DQ; ++d) part = fmaf(dor[j].at(d), vj.at(d), part);
                    const float dp = col4_sum(part);
                    const float ds = a.scale * w[j] * (dp - ci[j]);   // 0 for empty slots (w = 0)
                    const float p = w[j] * w[j];
#pragma unroll
                    for (int d = 0; d < DQ; ++d) {
                        dk[d] = fmaf(ds, qr[j].at(d), dk[d]);
                        dv[d] = fmaf(p, dor[j].at(d), dv[d]);
                    }
                }
            }
            if (kwr[f] && (n > 0 || (final_write && !written[f]))) {
                float* dkr = dkh + static_cast<size_t>(key) * D + g * DQ;
                float* dvr = dvh + static_cast<size_t>(key) * D + g * DQ;
#pragma unroll
                for (int d = 0; d < DQ; d += 4) {
                    f32x4 k4 = {dk[d], dk[d + 1], dk[d + 2], dk[d + 3]};
                    f32x4 v4 = {dv[d], dv[d + 1], dv[d + 2], dv[d + 3]};
                    if (written[f]) {
                        k4 += *reinterpret_cast<const f32x4*>(dkr + d);
                        v4 += *reinterpret_cast<const f32x4*>(dvr + d);
                    }
                    *reinterpret_cast<f32x4*>(dkr + d) = k4;
                    *reinterpret_cast<f32x4*>(dvr + d) = v4;
                }
                written[f] = true;
            }
            cnt[f] = 0;
            wave_sync();   // every lane is done reading the list before it refills
        };

        ChunkStream<DT, D, 2, 1> cs;
        cs.Kb = Qb;
        cs.Vb = nullptr;
        cs.kh = qh;
        cs.vh = qh;
        cs.kmp = reinterpret_cast<const uint8_t*>(qh);
        cs.hasm = false;
        cs.L = L;
        cs.tid = tid;
        cs.lane = lane;
        cs.side = tauh;     // tau of the streamed queries (+inf past L) comes with each chunk
        cs.sideb = tq_lds;
        // One attempt at a chunk's entries for every key of the wave, from
        // tile tn[f] on; returns (in tn) the first tile that did not fit.
        // A clean chunk (no causal / window bound crosses the wave's keys,
        // which are all valid: uniform) takes no masking.
        // tqb: the staged tau of the chunk's queries (LDS); tr: the same in raw
        // accumulator units, a little low
        auto attempt = [&](auto clean_tag, int cb, const char* qb, const float* tqb, const float (&tr)[4][4],
                           int (&tn)[NF]) {
            constexpr bool CLEAN = decltype(clean_tag)::value;
            f32x4 s[NF][4];   // [query 16t + 4g + i][key 16f + c]
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f32x4 o[NF];
                tile_products<DT, D, NF>(qb + qlane + 16 * t * C::KSTR, kf, o);
#pragma unroll
                for (int f = 0; f < NF; ++f) s[f][t] = o[f];
            }
            bool pend = false;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int key = kbase + 16 * f + c;
                // d > 0: the pair is in the support; -inf where the pair is
                // not allowed or its tile already listed
                auto dval = [&](int t, int i) {
                    float dv = s[f][t][i] - tr[t][i];
                    if constexpr (!CLEAN) {
                        const int qrow = cb + 16 * t + 4 * g + i;
                        const bool ok = kok[f] && t >= tn[f] && (!a.causal || allowed_ij(qrow, key, 1, a.window));
                        dv = ok ? dv : -kInf;
                    }
                    return dv;
                };
                float tm[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) tm[t] = fmaxf(fmaxf(dval(t, 0), dval(t, 1)), fmaxf(dval(t, 2), dval(t, 3)));
                int tb = 4;   // first tile that did not fit
                if (__any(fmaxf(fmaxf(tm[0], tm[1]), fmaxf(tm[2], tm[3])) > 0.f)) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if (!__any(tm[t] > 0.f)) continue;   // uniform: none in this tile
                        float d[4];
                        int np = 0;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            d[i] = dval(t, i);
                            np += d[i] > 0.f ? 1 : 0;
                        }
                        int tot;
                        int pos = cnt[f] + col4_scan_int(np, g, &tot);
                        const bool fits = tb == 4 && cnt[f] + tot <= CAP;
                        const f32x4 tq4 = *reinterpret_cast<const f32x4*>(tqb + 16 * t + 4 * g);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if (fits && d[i] > 0.f) {
                                // w = (s - tau)/2; an entry the low threshold let in
                                // by rounding gets w = 0 and contributes nothing
                                const int idx = slot_index(f, pos);
                                lw[idx] = fmaxf(0.5f * fmaf(s[f][t][i], a.scale, -tq4[i]), 0.f);
                                lq[idx] = static_cast<uint16_t>(cb + 16 * t + 4 * g + i);
                                ++pos;
                            }
                        }
                        cnt[f] += fits ? tot : 0;
                        tb = (tb == 4 && tot > 0 && !fits) ? t : tb;
                    }
                }
                tn[f] = tb;
                pend |= tb < 4;
            }
            return pend;
        };
        cs.run(ch0, ch1, false, [&](int chn, const char* qb, const char*, unsigned long long) {
            const int cb = chn * CK;
            if (cb >= wqhi || cb + CK <= wqlo) return;   // uniform: no query of the wave's keys
            // tau of this lane's queries: rows cb + 16 t + 4 g + i (past L: +inf)
            const float* tqb = tq_lds + ((qb - Qb) / C::k_bytes) * CK;
            float tr[4][4];   // tau in raw accumulator units (a little low; +inf stays +inf)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(tqb + 16 * t + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float r = v4[i] * inv_scale;
                    tr[t][i] = r - 1e-6f * fabsf(r) - 1e-30f;
                }
            }
            const bool cross = a.causal && (cb < kbase + NF * 16 - 1 ||
                                            (a.window > 0 && cb + CK - 1 >= kbase + a.window));
            int tn[NF];
#pragma unroll
            for (int f = 0; f < NF; ++f) tn[f] = 0;
            bool pend = (!cross && kall) ? attempt(std::true_type{}, cb, qb, tqb, tr, tn)
                                         : attempt(std::false_type{}, cb, qb, tqb, tr, tn);
            while (__any(pend)) {   // uniform
                // some list is full: flush those and redo the chunk from the
                // first tile left out.  The score tiles are dead here, and the
                // stationary fragments are read again afterwards (from L2), so
                // that the flush has their registers.
#pragma unroll 1
                for (int f = 0; f < NF; ++f)
                    if (__any(tn[f] < 4)) flush(f, false);
#pragma unroll
                for (int f = 0; f < NF; ++f) kf[f].load(kh, kbase + 16 * f + c, L, g);
                pend = attempt(std::false_type{}, cb, qb, tqb, tr, tn);
            }
        });
        wave_sync();
#pragma unroll 1
        for (int f = 0; f < NF; ++f) flush(f, last);
        wave_sync();
    }
}

}  // namespace ea
