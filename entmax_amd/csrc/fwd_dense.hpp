// Forward kernel for rows whose allowed key span fits in LDS (<= 1024 keys).
//
// One workgroup (4 waves) per (batch, head, tile of BM query rows):
//   1. S = Q K^T / sqrt(d) for every KV tile of the tile's key span, on MFMA,
//      with padding / causal / window masks folded in as -inf; kept in LDS.
//   2. per row: max, allowed count n, then tau by 25 bisection steps on
//      [max - 2, max - 2/sqrt(n)] (tau_solver.hpp); TPR lanes per row.
//   3. P = [(S - tau)/2]_+^2 straight from LDS into the MFMA A operand,
//      O = P V; 32-key chunks whose P is zero for all 16 rows of a wave are
//      skipped; O written in fp32.
// Waves split the tile as RG = BM/16 row groups x KG = 4/RG key groups;
// with KG > 1 the partial O of the key groups are summed through LDS.
#pragma once

#include "common.hpp"
#include "pv_tile.hpp"
#include "tau_solver.hpp"

namespace ea {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const uint8_t* key_mask;
    float* out;
    float* tau;
    int B, H, L;
    int causal, window;
    float scale;
    int nqt;   // query tiles per head
};

template <int D, int BM, int LSPAN>
struct DenseCfg {
    static constexpr int RG = BM / 16;
    static constexpr int KG = 4 / RG;
    static constexpr int TPR = kThreads / BM;
    static constexpr int SSTR = LSPAN + 4;   // row stride (floats): 16 B aligned, bank-skewed
    static constexpr int s_floats = BM * SSTR > KG * BM * D ? BM * SSTR : KG * BM * D;
    static constexpr size_t lds_bytes = sizeof(float) * (static_cast<size_t>(s_floats) + 2 * BM);
    static_assert(LSPAN / TPR <= 64, "at most 64 entries per lane in the solve");
};

template <int DT, int D, int BM, int LSPAN>
__global__ __launch_bounds__(kThreads) void fwd_dense_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef DenseCfg<D, BM, LSPAN> C;
    constexpr int RG = C::RG, KG = C::KG, TPR = C::TPR, SSTR = C::SSTR;
    extern __shared__ float lds[];
    float* S = lds;
    float* rowm = S + C::s_floats;
    float* rowtau = rowm + BM;

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
    const int kt0 = klo / kBN;
    const int ntile = (khi + kBN - 1) / kBN - kt0;
    const int span = ntile * kBN;

    const int tid = threadIdx.x;
    const int lane = tid % kWave, wv = tid / kWave;
    const int g = lane / 16, c = lane % 16;
    const int rg = wv % RG, kg = wv / RG;

    // ---- 1. score tiles into LDS ------------------------------------------
    {
        QFrag<DT, D> qf;
        qf.load(qh, q0 + 16 * rg + c, L, g);
        for (int t = kg; t < ntile; t += KG) {
#pragma unroll
            for (int c16 = 0; c16 < kBN / 16; ++c16) {
                const int key = (kt0 + t) * kBN + 16 * c16 + c;
                const uint8_t mb = km == nullptr ? static_cast<uint8_t>(1) : km[clamp_row(key, L)];
                const bool kv = key < L && mb != 0;
                const f32x4 acc = qf.tile(kh, key, L, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rl = 16 * rg + 4 * g + i;
                    const int row = q0 + rl;
                    const bool ok = kv && row < L && allowed_ij(row, key, a.causal, a.window);
                    S[rl * SSTR + t * kBN + 16 * c16 + c] = ok ? acc[i] * a.scale : -kInf;
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. per-row threshold ---------------------------------------------
    {
        const int r = tid / TPR, sub = tid % TPR;
        const float* srow = S + r * SSTR;
        const int nel = span / TPR;
        float m = -kInf, nf = 0.f;
        for (int i = 0; i < nel; ++i) {
            const float x = srow[sub + TPR * i];
            m = fmaxf(m, x);
            nf += x > -kInf ? 1.f : 0.f;
        }
        m = row_max<TPR>(m);
        const int n = static_cast<int>(row_sum<TPR>(nf));
        const bool empty = n == 0;
        const float mm = empty ? 0.f : m;
        auto get = [&](int i) { return srow[sub + TPR * i] - mm; };
        float ts = solve_tau_shifted<TPR>(get, nel, empty ? 1 : n);
        if (empty) ts = kInf;
        if (sub == 0) {
            rowm[r] = mm;
            rowtau[r] = ts;
            const int row = q0 + r;
            if (a.tau != nullptr && row < L) a.tau[static_cast<size_t>(bh) * L + row] = empty ? kInf : mm + ts;
        }
    }
    __syncthreads();

    // ---- 3. O = P V ---------------------------------------------------------
    typedef PVTile<DT, D> PV;
    f32x4 o[D / 16];
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const int rl = 16 * rg + c;
        const float mr = rowm[rl], tr = rowtau[rl];
        const float* srow = S + rl * SSTR;
        for (int t = kg; t < ntile; t += KG) {
#pragma unroll
            for (int ch = 0; ch < kBN / PV::kChunk; ++ch) {
                const int col = t * kBN + ch * PV::kChunk + PV::kPer * g;
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
                PV::acc(o, p, vh, (kt0 + t) * kBN + ch * PV::kChunk + PV::kPer * g, L, c);
            }
        }
    }

    float* outh = a.out + head_off;
    if constexpr (KG == 1) {
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = q0 + 16 * rg + 4 * g + i;
                if (row < L) outh[static_cast<size_t>(row) * D + 16 * ct + c] = o[ct][i];
            }
    } else {
        __syncthreads();   // S no longer read: reuse it for the partial sums
        float* red = S;
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[(kg * BM + 16 * rg + 4 * g + i) * D + 16 * ct + c] = o[ct][i];
        __syncthreads();
        for (int e = tid; e < BM * D; e += kThreads) {
            const int rl = e / D;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < KG; ++j) s += red[j * BM * D + e];
            if (q0 + rl < L) outh[static_cast<size_t>(q0) * D + e] = s;
        }
    }
}

}  // namespace ea
