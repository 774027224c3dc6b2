// Forward kernel for query tiles whose key span is at most 128 keys
// (encoder-length sequences; causal decoders with a short splash window).
//
// One workgroup (4 waves) per (batch, head, 64 query rows); wave w owns rows
// 16w .. 16w+15 and lane (g, c) = (lane / 16, lane % 16) serves query row c.
//   0. All global loads are issued at once, none behind a branch: key-mask
//      bytes first, then the Q fragments, the K fragments of every 16-key
//      tile of the span (kept in registers for both products if they fit)
//      and the V rows,
//      which are stored transposed into LDS.  Key rows that are masked out or
//      past L are redirected to an already-fetched row and zeroed.
//   1. S^T = K Q^T on MFMA (operands swapped, so each lane holds 4
//      consecutive keys of one query), scaled by 1/sqrt(d), masked
//      (padding / causal / window as -inf), written row-major to LDS with one
//      128-bit store per tile; row max and allowed count reduced across the 4
//      lanes of each query.  16-key tiles past the last valid key are
//      skipped by the later steps.
//   2. Two lanes per row (waves 0 and 1) find tau (25 bisection steps,
//      solve_lane.hpp); the row of S in LDS is their workspace.
//   3. S^T is recomputed on MFMA from the register fragments, P =
//      [(S - tau)/2]_+^2 formed in registers directly in the A-operand layout,
//      and O = P V on MFMA with V^T from LDS; 32-key chunks where P vanishes
//      for the whole wave are skipped.  O is written in fp32.
#pragma once

#include "common.hpp"
#include "fwd_dense.hpp"
#include "solve_lane.hpp"

namespace ea {

template <int DT, int D, int NKT>
struct ShortCfg {
    static constexpr int BM = 64;
    static constexpr int SPAN = NKT * kBN;
    static constexpr int NT = SPAN / 16;              // 16-key tiles
    static constexpr int ESZ = DT == DT_BF16 ? 2 : 4;
    static constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;               // chunks per V row
    static constexpr int NCH = SPAN * CPR / kThreads; // V chunks per thread
    static constexpr int SSTR = SPAN + 4;             // S row stride (floats)
    static constexpr int VSTR = SPAN + EPC;           // V^T row stride (elements)
    static constexpr int s_bytes = BM * SSTR * 4;
    static constexpr int v_bytes = D * VSTR * ESZ;
    static constexpr size_t lds_bytes = static_cast<size_t>(s_bytes) + v_bytes + 3 * BM * 4;
    static_assert(NCH >= 2 && NCH % 2 == 0, "whole chunk pairs per thread");
    // waves per SIMD to aim for: 3 workgroups per CU where the register
    // budget allows it (168 registers), else whatever fits
    static constexpr int kOcc = (DT == DT_BF16 && D == 64) ? 3 : 1;
};

// K fragments of one 16-key tile, in the same lane layout as QFrag::a.
template <int DT, int D> struct KFrag;
template <int D> struct KFrag<DT_BF16, D> {
    bf16x8 a[D / 32];
    // key must be a valid row index; ok = false loads it but yields zeros
    __device__ __forceinline__ void load(const uint16_t* kh, int key, bool ok, int g) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) a[ks] = ld_bf16x8_or_zero(kh + static_cast<size_t>(key) * D + 32 * ks + 8 * g, ok);
    }
    // S^T tile: lane (g, c) gets keys 4g + i of query c
    __device__ __forceinline__ f32x4 st(const QFrag<DT_BF16, D>& q) const {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) acc = mfma_bf16(a[ks], q.a[ks], acc);
        return acc;
    }
};
template <int D> struct KFrag<DT_F32, D> {
    f32x4 a[D / 16];
    __device__ __forceinline__ void load(const float* kh, int key, bool ok, int g) {
#pragma unroll
        for (int u = 0; u < D / 16; ++u) a[u] = ld_f32x4_or_zero(kh + static_cast<size_t>(key) * D + 16 * u + 4 * g, ok);
    }
    __device__ __forceinline__ f32x4 st(const QFrag<DT_F32, D>& q) const {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < D / 16; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_f32(a[u][s], q.a[u][s], acc);
        return acc;
    }
};

template <int DT, int D, int NKT>
__global__ __launch_bounds__(kThreads, (ShortCfg<DT, D, NKT>::kOcc)) void fwd_short_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef ShortCfg<DT, D, NKT> C;
    constexpr int BM = C::BM, SPAN = C::SPAN, NT = C::NT, EPC = C::EPC, CPR = C::CPR, NCH = C::NCH;
    constexpr int SSTR = C::SSTR, VSTR = C::VSTR;
    extern __shared__ float lds[];
    float* S = lds;
    T* VT = reinterpret_cast<T*>(reinterpret_cast<char*>(lds) + C::s_bytes);
    float* rowm = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + C::s_bytes + C::v_bytes);
    float* rown = rowm + BM;
    float* rowts = rown + BM;

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
    const int qrow = q0 + 16 * wv + c;        // this lane's query (as S^T column)

    // ---- 0. loads ----------------------------------------------------------------
    // Mask bytes first: the K and V loads depend on them.  Every load is
    // unconditional (clamped address) so that none waits for another.
    // Lane (g, c) owns S^T keys kbase + 16t + 4g + i (t < NT, i < 4): their
    // validity becomes the bitmask kbits (bit 4t + i).
    bool okv[NCH], okk[NT];
    int keyv[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int itv = tid + kThreads * (j / 2);
        keyv[j] = kbase + 2 * (itv / CPR) + (j % 2);
    }
    if (km != nullptr) {
        uint8_t mv[NCH], mk[NT];
#pragma unroll
        for (int j = 0; j < NCH; ++j) mv[j] = km[clamp_row(keyv[j], L)];
#pragma unroll
        for (int t = 0; t < NT; ++t) mk[t] = km[clamp_row(kbase + 16 * t + c, L)];
#pragma unroll
        for (int j = 0; j < NCH; ++j) okv[j] = keyv[j] < L && mv[j] != 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) okk[t] = kbase + 16 * t + c < L && mk[t] != 0;
    } else {
#pragma unroll
        for (int j = 0; j < NCH; ++j) okv[j] = keyv[j] < L;
#pragma unroll
        for (int t = 0; t < NT; ++t) okk[t] = kbase + 16 * t + c < L;
    }
    // okk[t] of lanes c = 0..15 (g = 0) covers the 16 keys of tile t: a
    // ballot hands lane (g, c) the validity of its S^T keys 4g .. 4g + 3
    unsigned kbits = 0u;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const unsigned long long bal = __ballot(okk[t]);
        kbits |= static_cast<unsigned>((bal >> (4 * g)) & 0xFull) << (4 * t);
    }
    QFrag<DT, D> qf;
    qf.load(qh, qrow, L, g);
    // K fragments: kept in registers for both products when they fit in 64
    // registers per lane, else fetched again for step 3 (from L2).  Rows that
    // are masked out or past L are read from the span's first key row
    // instead (valid, and fetched anyway), then zeroed: no branch, no extra
    // HBM traffic.
    constexpr bool kKeepK = NT * D * C::ESZ / 16 <= 64;
    KFrag<DT, D> kf[kKeepK ? NT : 1];
    auto ktile = [&](int t) {
        KFrag<DT, D> f;
        f.load(kh, okk[t] ? kbase + 16 * t + c : kbase, okk[t], g);
        return f;
    };
    if constexpr (kKeepK) {
#pragma unroll
        for (int t = 0; t < NT; ++t) kf[t] = ktile(t);
    }
    auto kfrag = [&](int t) -> KFrag<DT, D> {
        if constexpr (kKeepK) return kf[t];
        else return ktile(t);
    };
    u32x4 vreg[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const int chv = (tid + kThreads * (j / 2)) % CPR;
        const u32x4 u = *reinterpret_cast<const u32x4*>(vh + static_cast<size_t>(okv[j] ? keyv[j] : kbase) * D + chv * EPC);
        vreg[j] = okv[j] ? u : z;
    }
    // live 16-key tiles: up to the last tile holding a valid key (the same
    // keys are seen by every wave, so a wave-wide vote suffices)
    int ntl = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) ntl = __any(((kbits >> (4 * t)) & 0xFu) != 0u) ? t + 1 : ntl;
    // V^T: pairs of keys (2p, 2p + 1) packed per element; read only after
    // the barrier that ends step 1
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
                *reinterpret_cast<unsigned*>(VT + (d0 + e) * VSTR + key0) = lo16 | hi16;
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                uint2 pr;
                pr.x = vreg[j][e];
                pr.y = vreg[j + 1][e];
                *reinterpret_cast<uint2*>(VT + (d0 + e) * VSTR + key0) = pr;
            }
        }
    }

    // ---- 1. S^T tiles, row max and count ----------------------------------------------
    // (no branches per tile, so that tiles overlap; masked entries are -inf)
    auto masked = [&](const f32x4& acc, int t, f32x4& sv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kbase + 16 * t + 4 * g + i;
            const bool ok = ((kbits >> (4 * t + i)) & 1u) != 0u && qrow < L && allowed_ij(qrow, key, a.causal, a.window);
            sv[i] = ok ? acc[i] * a.scale : -kInf;
        }
    };
    {
        float mx = -kInf, nf = 0.f;
        float* srow = S + (16 * wv + c) * SSTR;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 sv;
            masked(kfrag(t).st(qf), t, sv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mx = fmaxf(mx, sv[i]);
                nf += sv[i] > -kInf ? 1.f : 0.f;
            }
            *reinterpret_cast<f32x4*>(srow + 16 * t + 4 * g) = sv;
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        nf += __shfl_xor(nf, 16, kWave);
        nf += __shfl_xor(nf, 32, kWave);
        if (g == 0) {
            rowm[16 * wv + c] = mx;
            rown[16 * wv + c] = nf;
        }
    }
    __syncthreads();

    // ---- 2. tau, two lanes per row (waves 0 and 1) ---------------------------------------
    if (wv < 2) {
        const int r = tid / 2, sub = tid % 2;
        const int n = static_cast<int>(rown[r]);
        const bool empty = n == 0;
        const float mm = empty ? 0.f : rowm[r];
        // this row's own key range inside the span, widened to 4-entry groups
        int rlo_k, rhi_k;
        key_range(q0 + r, 1, L, a.causal, a.window, &rlo_k, &rhi_k);
        const int e0 = ((rlo_k > kbase ? rlo_k - kbase : 0) / 4) * 4;
        int e1 = rhi_k - kbase;
        e1 = e1 < 16 * ntl ? e1 : 16 * ntl;
        e1 = e1 > e0 ? ((e1 + 3) / 4) * 4 : e0;
        float ts = solve_row_lane<2>(S + r * SSTR, e0, e1, mm, empty ? 1 : n, sub);
        if (empty) ts = kInf;
        if (sub == 0) {
            rowm[r] = mm;
            rowts[r] = ts;
            const int row = q0 + r;
            if (a.tau != nullptr && row < L) a.tau[static_cast<size_t>(bh) * L + row] = empty ? kInf : mm + ts;
        }
    }
    __syncthreads();

    // ---- 3. O = P V --------------------------------------------------------------------------
    f32x4 o[D / 16];
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const float mr = rowm[16 * wv + c], tr = rowts[16 * wv + c];
        auto probs = [&](int t, f32x4& p) {
            f32x4 sv;
            masked(kfrag(t).st(qf), t, sv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = (sv[i] - mr) - tr;
                p[i] = x > 0.f ? 0.25f * x * x : 0.f;
            }
        };
        if constexpr (DT == DT_BF16) {
            // chunks of 32 keys = tiles (2h, 2h + 1): slot (g, i) holds key
            // 32h + 4g + i for i < 4 and 32h + 16 + 4g + i - 4 for i >= 4
#pragma unroll
            for (int h = 0; h < NT / 2; ++h) {
                if (2 * h >= ntl) break;   // uniform: no valid key from here on
                f32x4 p0, p1;
                probs(2 * h, p0);
                probs(2 * h + 1, p1);
                bf16x8 phi, plo;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float pv = i < 4 ? p0[i] : p1[i - 4];
                    const __bf16 hb = static_cast<__bf16>(pv);
                    phi[i] = hb;
                    plo[i] = static_cast<__bf16>(pv - static_cast<float>(hb));
                }
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    const T* vrow = VT + (16 * ct + c) * VSTR + 32 * h + 4 * g;
                    const uint2 u0 = *reinterpret_cast<const uint2*>(vrow);
                    const uint2 u1 = *reinterpret_cast<const uint2*>(vrow + 16);
                    const u32x4 u = {u0.x, u0.y, u1.x, u1.y};
                    const bf16x8 bv = __builtin_bit_cast(bf16x8, u);
                    o[ct] = mfma_bf16(phi, bv, o[ct]);
                    o[ct] = mfma_bf16(plo, bv, o[ct]);
                }
            }
        } else {
            // fp32: step s of tile t gives slot g the key 16t + 4g + s
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (t >= ntl) break;       // uniform: no valid key from here on
                f32x4 p;
                probs(t, p);
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
                    const f32x4 bv = *reinterpret_cast<const f32x4*>(VT + (16 * ct + c) * VSTR + 16 * t + 4 * g);
#pragma unroll
                    for (int s = 0; s < 4; ++s) o[ct] = mfma_f32(p[s], bv[s], o[ct]);
                }
            }
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
