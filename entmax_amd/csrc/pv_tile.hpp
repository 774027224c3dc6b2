// O += P V on MFMA, for one wave's 16 query rows and one chunk of keys.
//
// "RoBERTa Base with AdaSplash Attention" model card, Architecture Overview:
// O_i = sum over keys with A_ij > 0 of A_ij V_j.
//
// bf16 inputs: P (float32 in [0, 1]) is split into two bf16 terms
// p = hi + lo (hi = bf16(p), lo = bf16(p - hi)), each multiplied with the
// bf16 V on the 16x16x32 MFMA and accumulated in fp32: the split keeps 16
// significant bits of p (relative error about 2^-17), while a single bf16 p
// would carry up to 2^-9 relative error into O.
// f32 inputs: P and V stay fp32 on the 16x16x4 fp32 MFMA.
#pragma once

#include "common.hpp"

namespace ea {

template <int DT, int D> struct PVTile;

template <int D> struct PVTile<DT_BF16, D> {
    static constexpr int kChunk = 32;   // keys per chunk
    static constexpr int kPer = 8;      // P values per lane: keys kb + 8g + i
    // lane (g, c): p[i] = P[row c][kb + 8g + i]; V rows kb + 8g + i, columns 16 ct + c.
    __device__ static __forceinline__ void acc(f32x4 (&o)[D / 16], const float (&p)[kPer],
                                               const uint16_t* vh, int key_lane, int L, int c) {
        bf16x8 phi, plo;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const __bf16 h = static_cast<__bf16>(p[i]);
            phi[i] = h;
            plo[i] = static_cast<__bf16>(p[i] - static_cast<float>(h));
        }
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) {
            bf16x8 b;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int key = key_lane + i;
                const uint16_t raw = vh[static_cast<size_t>(clamp_row(key, L)) * D + 16 * ct + c];
                b[i] = __builtin_bit_cast(__bf16, key < L ? raw : static_cast<uint16_t>(0));
            }
            o[ct] = mfma_bf16(phi, b, o[ct]);
            o[ct] = mfma_bf16(plo, b, o[ct]);
        }
    }
    // Same product with V^T staged in LDS: vt[col * vstr + key], key = kcol + 8g + i.
    __device__ static __forceinline__ void acc_lds(f32x4 (&o)[D / 16], const float (&p)[kPer],
                                                   const uint16_t* vt, int vstr, int kcol, int c) {
        bf16x8 phi, plo;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const __bf16 h = static_cast<__bf16>(p[i]);
            phi[i] = h;
            plo[i] = static_cast<__bf16>(p[i] - static_cast<float>(h));
        }
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) {
            const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vt + (16 * ct + c) * vstr + kcol));
            o[ct] = mfma_bf16(phi, b, o[ct]);
            o[ct] = mfma_bf16(plo, b, o[ct]);
        }
    }
};

template <int D> struct PVTile<DT_F32, D> {
    static constexpr int kChunk = 16;
    static constexpr int kPer = 4;      // keys kb + 4g + s, s = 0..3
    __device__ static __forceinline__ void acc(f32x4 (&o)[D / 16], const float (&p)[kPer],
                                               const float* vh, int key_lane, int L, int c) {
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) {
#pragma unroll
            for (int s = 0; s < kPer; ++s) {
                const int key = key_lane + s;
                const float raw = vh[static_cast<size_t>(clamp_row(key, L)) * D + 16 * ct + c];
                const float b = key < L ? raw : 0.f;
                o[ct] = mfma_f32(p[s], b, o[ct]);
            }
        }
    }
    // V^T staged in LDS: vt[col * vstr + key], key = kcol + 4g + s.
    __device__ static __forceinline__ void acc_lds(f32x4 (&o)[D / 16], const float (&p)[kPer],
                                                   const float* vt, int vstr, int kcol, int c) {
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(vt + (16 * ct + c) * vstr + kcol);
#pragma unroll
            for (int s = 0; s < kPer; ++s) o[ct] = mfma_f32(p[s], b[s], o[ct]);
        }
    }
};

}  // namespace ea
