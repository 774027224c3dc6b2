// Shared pieces of the wide kernels (fwd_wide.hpp, bwd_wide.hpp): waves that
// hold NF fragments of 16 rows of one operand in registers (64 rows per
// wave in bf16) while the other operand streams through LDS in chunks of 64
// rows (chunk_stream.hpp, two buffers, loads one chunk ahead), and per-row
// lists in LDS shared by the four lanes of a row.
#pragma once

#include "chunk_stream.hpp"
#include "col_solve.hpp"
#include "common.hpp"
#include "fwd_short.hpp"

namespace ea {

template <int DT, int D>
struct WideCfg : ChunkCfg<DT, D> {
    typedef ChunkCfg<DT, D> S;
    static constexpr int NF = DT == DT_BF16 ? 4 : 2;   // stationary 16-row fragments per wave
    static constexpr int BR = 4 * NF * 16;              // stationary rows per workgroup
    static constexpr int CAP = 24;                      // list entries per stationary row (key side)
    static constexpr int DQ = D / 4;                    // columns of a row per lane (lane group g)
    static constexpr int NB = 2;                        // entries per gather batch
    // lists: [wave][fragment][slot][row c] of a float (score or w) and the
    // other operand's row index (u16)
    static constexpr int list_elems = 4 * NF * CAP * 16;
    // two buffers of the streamed operand, the lists, and two chunks' worth
    // of one float per streamed row (tau of the staged queries, key side)
    static constexpr size_t lds_bytes = 2 * static_cast<size_t>(S::k_bytes) + list_elems * (sizeof(float) + sizeof(uint16_t)) +
                                        2 * S::CK * sizeof(float);
    // the kernels whose lists live in their output rows need the two
    // buffers only
    static constexpr size_t stream_lds_bytes = 2 * static_cast<size_t>(S::k_bytes);
    // the forward keeps each lane's first PL candidates in LDS (8 bytes
    // each) and the rest in the row's output row: stores to memory share the
    // wait counter of the chunk loads, so every chunk would wait for them
    static constexpr int PL = 5;
    static constexpr size_t fwd_lds_bytes = stream_lds_bytes + static_cast<size_t>(BR) * 4 * PL * 8;
    // two bf16 workgroups per CU (the registers allow two waves per SIMD)
    static constexpr int kOcc = DT == DT_BF16 ? 2 : 1;
};

// S^T products of one 16-row tile of the streamed operand (this lane's piece
// p of its row in LDS) against the NF stationary fragments:
// out[f] = tile . st[f]^T, lane (g, c) holding streamed rows 4g .. 4g + 3
// for stationary row 16 f + c.  The k-steps run outermost, so the NF
// accumulation chains advance side by side and no MFMA waits on the one
// just issued.  With a bias (bf16 / fp32 bits of the value added to
// streamed row c, from slot g = 0; 1 on the stationary side) one more step
// folds a mask into the products.
template <int DT, int D, int NF, bool BIAS = false>
__device__ __forceinline__ void tile_products(const char* p, const QFrag<DT, D> (&st)[NF], f32x4 (&out)[NF],
                                              unsigned bias_bits = 0u, int g = 0) {
    KFrag<DT, D> kf;
    kf.load_lds_at(p);
#pragma unroll
    for (int f = 0; f < NF; ++f) out[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == DT_BF16) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int f = 0; f < NF; ++f) out[f] = mfma_bf16(kf.a[ks], st[f].a[ks], out[f]);
        if constexpr (BIAS) {
            const u32x4 ub = {g == 0 ? bias_bits : 0u, 0u, 0u, 0u};
            const u32x4 uq = {g == 0 ? 0x3F80u : 0u, 0u, 0u, 0u};   // bf16 1.0
#pragma unroll
            for (int f = 0; f < NF; ++f)
                out[f] = mfma_bf16(__builtin_bit_cast(bf16x8, ub), __builtin_bit_cast(bf16x8, uq), out[f]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < D / 16; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int f = 0; f < NF; ++f) out[f] = mfma_f32(kf.a[u][q], st[f].a[u][q], out[f]);
        if constexpr (BIAS) {
#pragma unroll
            for (int f = 0; f < NF; ++f)
                out[f] = mfma_f32(g == 0 ? __uint_as_float(bias_bits) : 0.f, g == 0 ? 1.f : 0.f, out[f]);
        }
    }
}

// DQ consecutive elements of a row, widened to float.
template <int DT, int N>
__device__ __forceinline__ void load_cols(const typename InT<DT>::type* p, float (&x)[N]) {
    if constexpr (DT == DT_BF16) {
#pragma unroll
        for (int j = 0; j < N; j += 8) {
            const u32x4 u = *reinterpret_cast<const u32x4*>(p + j);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[j + 2 * k] = __uint_as_float(u[k] << 16);
                x[j + 2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            const f32x4 u = *reinterpret_cast<const f32x4*>(p + j);
#pragma unroll
            for (int k = 0; k < 4; ++k) x[j + k] = u[k];
        }
    }
}

// N consecutive elements of a row kept as loaded (bf16 pairs or floats);
// at(d) widens element d (d a compile-time index after unrolling).
template <int DT, int N> struct RowSlice;
template <int N> struct RowSlice<DT_BF16, N> {
    u32x4 u[N / 8];
    __device__ __forceinline__ void load(const uint16_t* p) {
#pragma unroll
        for (int j = 0; j < N / 8; ++j) u[j] = *reinterpret_cast<const u32x4*>(p + 8 * j);
    }
    __device__ __forceinline__ float at(int d) const {
        const unsigned w = u[d / 8][(d % 8) / 2];
        return __uint_as_float((d & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};
template <int N> struct RowSlice<DT_F32, N> {
    f32x4 u[N / 4];
    __device__ __forceinline__ void load(const float* p) {
#pragma unroll
        for (int j = 0; j < N / 4; ++j) u[j] = *reinterpret_cast<const f32x4*>(p + 4 * j);
    }
    __device__ __forceinline__ float at(int d) const { return u[d / 4][d % 4]; }
};

// Exclusive prefix over the four lanes c, c + 16, c + 32, c + 48 of a row
// (lane group g = lane / 16): the sum of v over the lane groups below g; the
// sum over all four goes to *total.  v_permlane16_swap(v, v) hands every
// lane the values of the even and the odd row of its pair of 16-lane rows,
// v_permlane32_swap(t, t) those of the lower and the upper half.
__device__ __forceinline__ int col4_scan_int(int v, int g, int* total) {
    const u32x2 a = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
    const unsigned t = a[0] + a[1];
    const u32x2 b = __builtin_amdgcn_permlane32_swap(t, t, false, false);
    *total = static_cast<int>(b[0] + b[1]);
    return static_cast<int>(((g & 1) ? a[0] : 0u) + ((g & 2) ? b[0] : 0u));
}

template <int N>
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int o = N / 2; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

}  // namespace ea
