// Device helpers shared by the gfx950 1.5-entmax attention kernels.
//
// MFMA lane layouts used throughout (wave of 64 lanes, g = lane / 16,
// c = lane % 16):
//   v_mfma_f32_16x16x32_bf16: lane (g, c) supplies A[c][8g .. 8g+7] and
//     B[8g .. 8g+7][c]; the result D[4g + i][c] sits in element i.
//   v_mfma_f32_16x16x4_f32:   lane (g, c) supplies A[c][g] and B[g][c];
//     the result layout is the same as above.
// Only the pairing of A and B slots matters for the contraction, so each
// helper picks the contraction index of slot (g, i) to make its loads
// contiguous, and uses the same choice for both operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kWave = 64;
constexpr int kThreads = 256;     // threads per workgroup (4 waves)
constexpr int kBN = 64;           // keys per KV tile
constexpr int kIters = 25;        // bisection steps
constexpr float kInf = __builtin_huge_valf();

enum { DT_F32 = 0, DT_BF16 = 1 };

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
    u32x4 u = *reinterpret_cast<const u32x4*>(p);
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    u32x4 u = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two floats rounded to nearest-even bf16, the first in the low half
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// p = y^2 of 8 entries as two bf16 operands: hi the nearest bf16 of p, lo
// the nearest bf16 of the remainder p - hi (formed exactly by one fma), so
// that hi + lo carries about 16 significant bits of p.
__device__ __forceinline__ void split_sq_bf16(const float (&y)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float a = y[2 * m], b = y[2 * m + 1];
        h[m] = pack_bf16(a * a, b * b);
        const float ha = __uint_as_float(h[m] << 16), hb = __uint_as_float(h[m] & 0xffff0000u);
        l[m] = pack_bf16(fmaf(a, a, -ha), fmaf(b, b, -hb));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Sums / maxima over groups of N consecutive lanes (N a power of two <= 64).
// Butterfly order: every lane of the group ends with a bitwise-identical
// value (floating-point addition is commutative).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = N / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = N / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
template <int N>
__device__ __forceinline__ int group_sum_int(int v) {
#pragma unroll
    for (int o = N / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// Score tiles: S[16 queries x 16 keys] = Q K^T (unscaled), fp32 accumulate.
// ---------------------------------------------------------------------------

template <int DT, int D> struct QFrag;

// bf16: slot (g, i) of k-step ks holds feature 32*ks + 8*g + i.
// Loads below never branch on their predicate: a branch around a load makes
// the compiler wait for that load before the branches join, which
// serialises independent loads.  Out-of-range rows are read from a clamped
// (valid, usually cache-resident) address and replaced by zero afterwards.
__device__ __forceinline__ bf16x8 ld_bf16x8_or_zero(const uint16_t* p, bool ok) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
    const u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, ok ? u : z);
}
__device__ __forceinline__ f32x4 ld_f32x4_or_zero(const float* p, bool ok) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return ok ? u : z;
}
__device__ __forceinline__ int clamp_row(int r, int L) { return r < L ? r : L - 1; }

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives
// element k (k < 4) of the 4 x 16-bit row that lane 4k + j/4 points at, so
// a 16 x 4 block is read transposed.  p: LDS address, 8-byte aligned.
__device__ __forceinline__ s16x4 ds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(reinterpret_cast<uintptr_t>(p)));
}

template <int D> struct QFrag<DT_BF16, D> {
    bf16x8 a[D / 32];
    __device__ __forceinline__ void load(const uint16_t* qh, int row, int L, int g) {
        const uint16_t* p = qh + static_cast<size_t>(clamp_row(row, L)) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) a[ks] = ld_bf16x8_or_zero(p + 32 * ks, row < L);
    }
    // key: this lane's key (column c); the lane's K row is read 16 B at a time
    __device__ __forceinline__ f32x4 tile(const uint16_t* kh, int key, int L, int g) const {
        bf16x8 b[D / 32];
        const uint16_t* p = kh + static_cast<size_t>(clamp_row(key, L)) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) b[ks] = ld_bf16x8_or_zero(p + 32 * ks, key < L);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) acc = mfma_bf16(a[ks], b[ks], acc);
        return acc;
    }
};

// f32: step (u, s) gives slot g the feature 16*u + 4*g + s.
template <int D> struct QFrag<DT_F32, D> {
    f32x4 a[D / 16];
    __device__ __forceinline__ void load(const float* qh, int row, int L, int g) {
        const float* p = qh + static_cast<size_t>(clamp_row(row, L)) * D + 4 * g;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) a[u] = ld_f32x4_or_zero(p + 16 * u, row < L);
    }
    __device__ __forceinline__ f32x4 tile(const float* kh, int key, int L, int g) const {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const float* p = kh + static_cast<size_t>(clamp_row(key, L)) * D + 4 * g;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const f32x4 b = ld_f32x4_or_zero(p + 16 * u, key < L);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_f32(a[u][s], b[s], acc);
        }
        return acc;
    }
};

// Orders this wave's LDS writes before its later reads by other lanes.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Forward launch arguments (device pointers; see the C header for layouts).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const uint8_t* key_mask;
    float* out;
    float* tau;
    int B, H, L;
    int Hkv;   // key/value heads (H % Hkv == 0)
    int causal, window;
    float scale;
    int nqt;   // query tiles per head
    int fixup; // long-span kernel: only tiles with a row marked by the wide kernel
    // the support of every query row for the backward (the wide kernel; null
    // otherwise): scount [B, H, L] its size (-1: not saved), sent [B, H, L,
    // D/2] its entries (w = sqrt(p), key bits)
    int* scount;
    float* sent;
};

// Key/value head serving query head bh = b H + h when Hkv heads serve the H
// query heads in consecutive groups of H / Hkv (the grouped-query repeat of
// K and V in "ADASPLASH -- ROBERTA Benchmark Result", section 3, Step-by-Step
// Tensor Execution Trace): b Hkv + h / (H / Hkv).  Uniform.
__device__ __forceinline__ int kv_head(int bh, int H, int Hkv) {
    const int b = bh / H;
    return b * Hkv + (bh - b * H) / (H / Hkv);
}

template <int DT> struct InT;
template <> struct InT<DT_F32> { typedef float type; };
template <> struct InT<DT_BF16> { typedef uint16_t type; };

// ---------------------------------------------------------------------------
// Masking: key j allowed for query i (both already known to be < L).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool allowed_ij(int i, int j, int causal, int window) {
    return (!causal || j <= i) && (window <= 0 || j > i - window);
}

// Key range [lo, hi) that rows [q0, q0 + bm) may attend.
__host__ __device__ __forceinline__ void key_range(int q0, int bm, int L, int causal, int window,
                                                   int* lo, int* hi) {
    int h = L;
    if (causal) h = q0 + bm < L ? q0 + bm : L;
    int l = 0;
    if (window > 0) l = q0 - window + 1 > 0 ? q0 - window + 1 : 0;
    *lo = l;
    *hi = h;
}

// *p += v on an LDS address, as one LDS read-modify-write without return
// (ds_add_u32); relaxed, for slots that only the calling lane updates
__device__ __forceinline__ void lds_add(unsigned* p, unsigned v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Workgroup -> work item: consecutive work items (the Q tiles of one head)
// land on the same XCD, whose L2 then serves the head's K and V.
// Workgroups are dealt round-robin to the 8 XCDs.
__device__ __forceinline__ int xcd_swizzle(int bid, int total) {
    const int nx = 8;
    const int per = total / nx;
    if (bid < per * nx) return (bid % nx) * per + bid / nx;
    return bid;
}

}  // namespace ea
