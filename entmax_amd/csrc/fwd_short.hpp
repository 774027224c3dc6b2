// Forward kernel for query tiles whose key span is at most 128 keys
// (encoder-length sequences; causal decoders with a short splash window).
//
// One workgroup (4 waves) per (batch, head, 64 query rows); wave w owns rows
// 16w .. 16w+15.  The whole key span is resident:
//   0. every global load is issued at once: the wave's Q fragments, the K
//      rows of the span (into LDS, row-major) and the V rows (held in
//      registers until the K region is free).  Key rows that are masked out
//      or past L are not read (zero-filled).
//   1. S = Q K^T / sqrt(d) on MFMA, B operand from LDS; padding / causal /
//      window masks folded in as -inf; 16x16 tiles that the causal / window
//      mask removes entirely are skipped.  S stays in LDS.
//   2. V is written transposed into the freed K region; the row max and
//      allowed count come from step 1 (16-lane DPP reductions of the MFMA
//      output); waves 0 and 1 find tau by 25 bisection steps
//      (tau_solver.hpp), 2 lanes per row, 64 contiguous entries each.
//   3. O = P V on MFMA with P = [(S - tau)/2]_+^2 read from LDS and V^T
//      fragments from LDS; key chunks where P vanishes for all 16 rows of a
//      wave are skipped.  O is written in fp32.
#pragma once

#include "common.hpp"
#include "fwd_dense.hpp"
#include "pv_tile.hpp"
#include "tau_solver.hpp"

namespace ea {

template <int DT, int D, int NKT>
struct ShortCfg {
    static constexpr int BM = 64;
    static constexpr int SPAN = NKT * kBN;
    static constexpr int ESZ = DT == DT_BF16 ? 2 : 4;
    static constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;               // chunks per row
    static constexpr int NCH = SPAN * CPR / kThreads; // chunks per thread (K and V each)
    static constexpr int SSTR = SPAN + 4;             // S row stride (floats)
    static constexpr int KSTR = D + EPC;              // K row stride (elements), 16-byte padded
    static constexpr int VSTR = SPAN + EPC;           // V^T row stride (elements)
    static constexpr int s_bytes = BM * SSTR * 4;
    static constexpr int k_bytes = SPAN * KSTR * ESZ;
    static constexpr int v_bytes = D * VSTR * ESZ;
    static constexpr int kv_bytes = k_bytes > v_bytes ? k_bytes : v_bytes;
    static constexpr size_t lds_bytes = static_cast<size_t>(s_bytes) + kv_bytes + 2 * BM * 4 + SPAN;
    static constexpr int TPR = 2;                     // lanes per row in the solve
    static constexpr int NEL = SPAN / TPR;            // entries per solve lane
    static_assert(NCH >= 2 && NCH % 2 == 0, "whole chunk pairs per thread");
    static_assert(NEL <= 64, "solve entries per lane");
};

template <int DT, int D, int NKT>
__global__ __launch_bounds__(kThreads) void fwd_short_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef ShortCfg<DT, D, NKT> C;
    constexpr int BM = C::BM, SPAN = C::SPAN, EPC = C::EPC, CPR = C::CPR, NCH = C::NCH;
    constexpr int SSTR = C::SSTR, KSTR = C::KSTR, VSTR = C::VSTR, TPR = C::TPR, NEL = C::NEL;
    extern __shared__ float lds[];
    float* S = lds;
    T* KV = reinterpret_cast<T*>(reinterpret_cast<char*>(lds) + C::s_bytes);
    float* rowm = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + C::s_bytes + C::kv_bytes);
    float* rowtau = rowm + BM;
    uint8_t* kvalid = reinterpret_cast<uint8_t*>(rowtau + BM);   // [SPAN] key may be attended

    const int total = a.B * a.H * a.nqt;
    const int w = xcd_swizzle(blockIdx.x, total);
    const int bh = w / a.nqt;
    const int qt = w - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * BM;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const T* kh = static_cast<const T*>(a.k) + head_off;
    const T* vh = static_cast<const T*>(a.v) + head_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;

    int klo, khi;
    key_range(q0, BM, L, a.causal, a.window, &klo, &khi);
    const int kbase = (klo / kBN) * kBN;   // first key of the span

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wv = tid / kWave;
    const int g = lane / 16, c = lane % 16;

    // ---- 0. issue every global load ------------------------------------------
    // K item j of this thread -> (key, chunk); V item j -> (key pair, chunk)
    // with keys 2p and 2p + 1.  Mask bytes first (K/V loads depend on them),
    // then Q, so that waiting for the mask leaves Q in flight.
    int keyk[NCH], keyv[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int itk = tid + kThreads * j;
        keyk[j] = kbase + itk / CPR;
        const int itv = tid + kThreads * (j / 2);
        keyv[j] = kbase + 2 * (itv / CPR) + (j % 2);
    }
    bool okk[NCH], okv[NCH];
    bool ok_own = tid < SPAN && kbase + tid < L;
    if (km != nullptr) {
        uint8_t mk[NCH], mv[NCH], mown = 0;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            mk[j] = keyk[j] < L ? km[keyk[j]] : static_cast<uint8_t>(0);
            mv[j] = keyv[j] < L ? km[keyv[j]] : static_cast<uint8_t>(0);
        }
        if (ok_own) mown = km[kbase + tid];
#pragma unroll
        for (int j = 0; j < NCH; ++j) { okk[j] = mk[j] != 0; okv[j] = mv[j] != 0; }
        ok_own = mown != 0;
    } else {
#pragma unroll
        for (int j = 0; j < NCH; ++j) { okk[j] = keyk[j] < L; okv[j] = keyv[j] < L; }
    }
    QFrag<DT, D> qf;
    qf.load(qh, q0 + 16 * wv + c, L, g);
    u32x4 kreg[NCH], vreg[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const int chk = (tid + kThreads * j) % CPR;
        const int chv = (tid + kThreads * (j / 2)) % CPR;
        kreg[j] = okk[j] ? *reinterpret_cast<const u32x4*>(kh + static_cast<size_t>(keyk[j]) * D + chk * EPC) : z;
        vreg[j] = okv[j] ? *reinterpret_cast<const u32x4*>(vh + static_cast<size_t>(keyv[j]) * D + chv * EPC) : z;
    }
    if (tid < SPAN) kvalid[tid] = ok_own ? 1 : 0;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int itk = tid + kThreads * j;
        *reinterpret_cast<u32x4*>(KV + (itk / CPR) * KSTR + (itk % CPR) * EPC) = kreg[j];
    }
    __syncthreads();

    // ---- 1. S = Q K^T / sqrt(d) into LDS -------------------------------------
    float rmax[4] = {-kInf, -kInf, -kInf, -kInf}, rcnt[4] = {0.f, 0.f, 0.f, 0.f};
    {
        const int rlo = q0 + 16 * wv, rhi = rlo + 15;
#pragma unroll
        for (int t16 = 0; t16 < SPAN / 16; ++t16) {
            const int k0 = kbase + 16 * t16;
            const bool dead = (a.causal && k0 > rhi) || (a.window > 0 && k0 + 15 <= rlo - a.window);
            if (dead) {   // uniform over the wave
#pragma unroll
                for (int i = 0; i < 4; ++i) S[(16 * wv + 4 * g + i) * SSTR + 16 * t16 + c] = -kInf;
                continue;
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const T* krow = KV + (16 * t16 + c) * KSTR;
            if constexpr (DT == DT_BF16) {
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    const bf16x8 bfr = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 32 * ks + 8 * g));
                    acc = mfma_bf16(qf.a[ks], bfr, acc);
                }
            } else {
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const f32x4 bfr = *reinterpret_cast<const f32x4*>(krow + 16 * u + 4 * g);
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = mfma_f32(qf.a[u][s], bfr[s], acc);
                }
            }
            const int key = k0 + c;
            const bool kv = kvalid[16 * t16 + c] != 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = rlo + 4 * g + i;
                const bool ok = kv && row < L && allowed_ij(row, key, a.causal, a.window);
                const float sv = ok ? acc[i] * a.scale : -kInf;
                S[(16 * wv + 4 * g + i) * SSTR + 16 * t16 + c] = sv;
                rmax[i] = fmaxf(rmax[i], sv);
                rcnt[i] += ok ? 1.f : 0.f;
            }
        }
        // row max and allowed count over the 16 lanes holding each row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m = row_max<16>(rmax[i]);
            const float n = row_sum<16>(rcnt[i]);
            if (c == 0) {
                rowm[16 * wv + 4 * g + i] = m;
                rowtau[16 * wv + 4 * g + i] = n;
            }
        }
    }
    __syncthreads();

    // ---- 2. V^T into LDS; per-row threshold -----------------------------------
#pragma unroll
    for (int j = 0; j < NCH; j += 2) {
        const int itv = tid + kThreads * (j / 2);
        const int key0 = 2 * (itv / CPR);
        const int d0 = (itv % CPR) * EPC;
        if constexpr (DT == DT_BF16) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const unsigned w0 = vreg[j][e / 2], w1 = vreg[j + 1][e / 2];
                const unsigned lo16 = (e & 1) ? (w0 >> 16) : (w0 & 0xFFFFu);
                const unsigned hi16 = (e & 1) ? (w1 & 0xFFFF0000u) : (w1 << 16);
                *reinterpret_cast<unsigned*>(KV + (d0 + e) * VSTR + key0) = lo16 | hi16;
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                uint2 pr;
                pr.x = vreg[j][e];
                pr.y = vreg[j + 1][e];
                *reinterpret_cast<uint2*>(KV + (d0 + e) * VSTR + key0) = pr;
            }
        }
    }
    // waves 0 and 1: 32 rows each, TPR lanes per row (rowm / rowtau hold the
    // row max and allowed count from step 1 on entry)
    if (wv < BM * TPR / kWave) {
        const int r = tid / TPR, sub = tid % TPR;
        const float* srow = S + r * SSTR + sub * NEL;
        const float m = rowm[r];
        const int n = static_cast<int>(rowtau[r]);
        const bool empty = n == 0;
        const float mm = empty ? 0.f : m;
        auto get = [&](int i) { return srow[i] - mm; };
        float ts = solve_tau_shifted<TPR>(get, NEL, empty ? 1 : n);
        if (empty) ts = kInf;
        if (sub == 0) {
            rowm[r] = mm;
            rowtau[r] = ts;
            const int row = q0 + r;
            if (a.tau != nullptr && row < L) a.tau[static_cast<size_t>(bh) * L + row] = empty ? kInf : mm + ts;
        }
    }
    __syncthreads();

    // ---- 3. O = P V ---------------------------------------------------------------
    typedef PVTile<DT, D> PV;
    f32x4 o[D / 16];
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const int rl = 16 * wv + c;
        const float mr = rowm[rl], tr = rowtau[rl];
        const float* srow = S + rl * SSTR;
#pragma unroll
        for (int ch = 0; ch < SPAN / PV::kChunk; ++ch) {
            const int col = ch * PV::kChunk + PV::kPer * g;
            float p[PV::kPer];
            bool nz = false;
#pragma unroll
            for (int i4 = 0; i4 < PV::kPer / 4; ++i4) {
                const f32x4 sv = *reinterpret_cast<const f32x4*>(srow + col + 4 * i4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = (sv[j] - mr) - tr;
                    const bool pos = x > 0.f;
                    p[4 * i4 + j] = pos ? 0.25f * x * x : 0.f;
                    nz |= pos;
                }
            }
            if (!__any(nz)) continue;
            PV::acc_lds(o, p, KV, VSTR, col, c);
        }
    }

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
