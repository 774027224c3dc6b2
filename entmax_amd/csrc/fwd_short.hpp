// Forward kernel for query tiles whose key span is at most 128 keys
// (encoder-length sequences; causal decoders with a short splash window).
//
// One workgroup (4 waves) per (batch, head, 64 query rows); wave w owns rows
// 16w .. 16w+15 and lane (g, c) = (lane / 16, lane % 16) serves query row c.
// Apart from the V^T staging area every step is private to a wave: one
// barrier in total.
//   0. Global loads, none behind a branch: the key-mask bytes and the Q
//      fragments, then the K and V rows of the span (rows of keys that may
//      not be attended are redirected to an already-fetched row; their
//      scores are masked).  K is staged in LDS; V waits in registers and is
//      stored into LDS only after step 2, so that steps 1 and 2 run while it
//      arrives.
//   1. S^T = K Q^T on MFMA (operands swapped, so each lane holds 4
//      consecutive keys of one query in each 16-key tile), masked (padding /
//      causal / window as -inf) and kept in registers: the four lanes
//      c, c + 16, c + 32, c + 48 hold the whole row.  Tiles outside the
//      wave's key range are skipped.  Row max and allowed count by
//      cross-lane swaps.
//   2. tau by 25 bisection steps on the registers (col_solve.hpp), with a
//      per-lane scratch column in LDS for the shrinking band.
//   3. P = [(S - tau)/2]_+^2 formed from the same registers directly in the
//      A-operand layout of the P V MFMA (keys 4g + i of tiles 2h, 2h + 1
//      give 32-key chunk h), V^T from LDS; O is written in fp32.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "col_solve.hpp"

namespace ea {

// KC: scratch slots per lane for the solve's candidates, at least the
// largest number of allowed keys one lane can hold (4 per 16-key tile)
template <int DT, int D, int NKT, int KC = NKT * kBN / 4>
struct ShortCfg {
    static constexpr int BM = 64;
    static constexpr int SPAN = NKT * kBN;
    static constexpr int NT = SPAN / 16;              // 16-key tiles
    static constexpr int ESZ = DT == DT_BF16 ? 2 : 4;
    static constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;               // chunks per V row
    static constexpr int NCH = SPAN * CPR / kThreads; // V chunks per thread
    static constexpr int VSTR = SPAN + EPC;           // fp32: V^T row stride (elements)
    // bf16: V row-major, row stride D*2 + 32 bytes (conflict-free transpose
    // reads); fp32: V^T
    static constexpr int VRS = D * 2 + 32;
    static constexpr int v_bytes = DT == DT_BF16 ? SPAN * VRS : D * VSTR * ESZ;
    static constexpr int scr_bytes = 4 * KC * kWave * 4;       // per wave: KC rows x 64 lanes
    static constexpr int KSTR = D * ESZ + 32;                   // K row stride in LDS (bytes): conflict-free tile reads
    static constexpr int k_bytes = SPAN * KSTR;
    static constexpr int NKC = SPAN * CPR / kThreads;           // K chunks per thread
    // K staging (step 0-1) and the solve's scratch (step 2) share one region;
    // with a reduced scratch (KC below the span's 4 keys per tile and lane)
    // V takes the same region after the solve as well, at the cost of one
    // more barrier, so that more workgroups fit a CU
    static constexpr bool kAlias = KC < NT * 4;
    static constexpr int ks_bytes = k_bytes > scr_bytes ? k_bytes : scr_bytes;
    static constexpr int ksv_bytes = ks_bytes > v_bytes ? ks_bytes : v_bytes;
    static constexpr size_t lds_bytes = kAlias ? static_cast<size_t>(ksv_bytes) : static_cast<size_t>(ks_bytes) + v_bytes;
    static_assert(NCH >= 1 && SPAN <= 2 * kWave, "whole chunks per thread; mask bits in two ballots");
    // waves per SIMD to aim for (bf16, d = 64): five workgroups per CU with
    // the reduced scratch (KC = 16, 96 registers; the causal 32-key window:
    // 35.5 -> 34.3 us on the decoder workload), else four when their LDS
    // fits (128 registers), else three (168 registers)
    static constexpr int kOcc = (DT == DT_BF16 && D == 64)
                                    ? (KC == 16 && lds_bytes * 5 <= 160 * 1024 ? 5 : lds_bytes * 4 <= 160 * 1024 ? 4 : 3)
                                    : 1;
    static_assert(KC <= NT * 4 && KC >= 16, "scratch slots");
};

// K fragments of one 16-key tile, in the same lane layout as QFrag::a.
template <int DT, int D> struct KFrag;
template <int D> struct KFrag<DT_BF16, D> {
    bf16x8 a[D / 32];
    // from a row-major LDS copy (row = this lane's key)
    __device__ __forceinline__ void load_lds(const char* row, int g) { load_lds_at(row + 16 * g); }
    // p: this lane's first piece (row + 16 g)
    __device__ __forceinline__ void load_lds_at(const char* p) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) a[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + 64 * ks));
    }
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
    // Same, plus bias(key) for every query: one more k-step whose only
    // nonzero entries are bias(key c) (slot g = 0, i = 0 on the K side) and
    // 1 (the same slot on the Q side).  bias_bits: bf16 bits in the low half.
    __device__ __forceinline__ f32x4 st_bias(const QFrag<DT_BF16, D>& q, unsigned bias_bits, int g) const {
        const u32x4 ub = {g == 0 ? bias_bits : 0u, 0u, 0u, 0u};
        const u32x4 uq = {g == 0 ? 0x3F80u : 0u, 0u, 0u, 0u};   // bf16 1.0
        return mfma_bf16(__builtin_bit_cast(bf16x8, ub), __builtin_bit_cast(bf16x8, uq), st(q));
    }
};
template <int D> struct KFrag<DT_F32, D> {
    f32x4 a[D / 16];
    __device__ __forceinline__ void load_lds(const char* row, int g) { load_lds_at(row + 16 * g); }
    __device__ __forceinline__ void load_lds_at(const char* p) {
#pragma unroll
        for (int u = 0; u < D / 16; ++u) a[u] = *reinterpret_cast<const f32x4*>(p + 64 * u);
    }
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
    // bias_bits: fp32 bits of bias(key c)
    __device__ __forceinline__ f32x4 st_bias(const QFrag<DT_F32, D>& q, unsigned bias_bits, int g) const {
        return mfma_f32(g == 0 ? __uint_as_float(bias_bits) : 0.f, g == 0 ? 1.f : 0.f, st(q));
    }
};

template <int DT, int D, int NKT, int KC>
__global__ __launch_bounds__(kThreads, (ShortCfg<DT, D, NKT, KC>::kOcc)) void fwd_short_kernel(FwdArgs a) {
    typedef typename InT<DT>::type T;
    typedef ShortCfg<DT, D, NKT, KC> C;
    constexpr int BM = C::BM, NT = C::NT, EPC = C::EPC, CPR = C::CPR, NCH = C::NCH, VSTR = C::VSTR;
    extern __shared__ float lds[];
    char* Ks = reinterpret_cast<char*>(lds);              // K rows (steps 0-1)
    float* scratch = lds;                                  // the solve's scratch (step 2), same region
    char* Vs = reinterpret_cast<char*>(lds) + (C::kAlias ? 0 : C::ks_bytes);   // V (bf16: row-major; fp32: V^T)

    const int total = a.B * a.H * a.nqt;
    const int w = xcd_swizzle(blockIdx.x, total);
    const int bh = w / a.nqt;
    const int qt = w - bh * a.nqt;
    const int b = bh / a.H;
    const int q0 = qt * BM;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const T* vh = static_cast<const T*>(a.v) + kv_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;

    int klo, khi;
    key_range(q0, BM, L, a.causal, a.window, &klo, &khi);
    const int kbase = (klo / kBN) * kBN;   // first key of the span

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: scalar branches below
    const int g = lane / 16, c = lane % 16;
    const int qrow = q0 + 16 * wv + c;        // this lane's query (S^T column)

    // ---- 0. loads ----------------------------------------------------------------
    // Issue order matters: a wait on a load also waits for every load issued
    // before it.  The key-mask bytes go first (two per lane: keys kbase + lane
    // and kbase + 64 + lane), then Q, which does not depend on the mask; K
    // and V rows follow the mask.  No branch around any load: without a mask
    // the byte loads read a byte of Q and ignore it.
    const bool hasm = km != nullptr;
    const uint8_t* kmp = hasm ? km : reinterpret_cast<const uint8_t*>(qh);
    const int mkey0 = kbase + lane, mkey1 = kbase + kWave + lane;
    const uint8_t mb0 = kmp[hasm ? clamp_row(mkey0, L) : 0];
    const uint8_t mb1 = C::SPAN > kWave ? kmp[hasm ? clamp_row(mkey1, L) : 0] : uint8_t(0);
    // compiler-only fence: the mask loads are issued here, ahead of the
    // rest (no wait is implied; it only stops the compiler from moving them)
    asm volatile("" ::: "memory");
    QFrag<DT, D> qf;
    qf.load(qh, qrow, L, g);
    // K and V rows of the span, once per workgroup: 16-byte chunks,
    // consecutive threads on consecutive chunks
    // valid keys of the span as two 64-bit masks (bit k <-> key kbase + k,
    // resp. kbase + 64 + k), uniform over the wave.  K rows of keys that may
    // not be attended read the span's first row instead (fetched anyway), so
    // padded keys cost no HBM traffic; their scores are masked below.
    const unsigned long long M0 = __ballot((mkey0 < L) & (!hasm | (mb0 != 0)));
    const unsigned long long M1 = C::SPAN > kWave ? __ballot((mkey1 < L) & (!hasm | (mb1 != 0))) : 0ull;
    auto key_ok = [&](int kl) { return (((kl < kWave ? M0 : M1) >> (kl & (kWave - 1))) & 1ull) != 0ull; };
    u32x4 kreg[C::NKC], vreg[NCH];
#pragma unroll
    for (int j = 0; j < C::NKC; ++j) {
        const int ch = tid + kThreads * j;
        const int kl = ch / CPR;   // key within the span
        kreg[j] = *reinterpret_cast<const u32x4*>(kh + static_cast<size_t>(key_ok(kl) ? kbase + kl : kbase) * D + (ch % CPR) * EPC);
    }
#pragma unroll
    for (int j = 0; j < C::NKC; ++j) {
        const int ch = tid + kThreads * j;
        *reinterpret_cast<u32x4*>(Ks + (ch / CPR) * C::KSTR + (ch % CPR) * 16) = kreg[j];
    }
    __syncthreads();   // K staged

    auto mbits16 = [&](int t) -> unsigned {   // the 16 key bits of tile t
        return static_cast<unsigned>(((t < 4 ? M0 : M1) >> (16 * (t & 3))) & 0xFFFFull);
    };
    // V rows only now that the mask is known: a row that may not be attended
    // reads the span's first row instead (fetched anyway; its p is 0), so
    // padded keys cost no HBM traffic.  V is needed in step 3 only.
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int ch = tid + kThreads * j;
        const int kl = ch / CPR;   // key within the span
        vreg[j] = *reinterpret_cast<const u32x4*>(vh + static_cast<size_t>(key_ok(kl) ? kbase + kl : kbase) * D + (ch % CPR) * EPC);
    }

    // tiles this wave's 16 rows may attend (causal / window; the mask is
    // applied below): [t0, tc1), uniform over the wave
    int t0, tc1;
    {
        int wlo, whi;
        key_range(q0 + 16 * wv, 16, L, a.causal, a.window, &wlo, &whi);
        t0 = wlo > kbase ? (wlo - kbase) / 16 : 0;
        tc1 = (whi - kbase + 15) / 16;
        tc1 = tc1 < NT ? tc1 : NT;
    }

    // ---- 1. S^T tiles in registers ----------------------------------------------------
    // lane (g, c) owns S^T keys kbase + 16t + 4g + i: their validity is bit
    // 4t + i of kbits; okk(t): validity of this lane's K row (key 16t + c)
    unsigned kbits = 0u;
    unsigned full = 0u;   // bit t: every key of tile t valid (uniform)
    int ntl = 0;          // tiles up to the last one holding a valid key (uniform)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const unsigned mb = mbits16(t);
        kbits |= ((mb >> (4 * g)) & 0xFu) << (4 * t);
        ntl = mb != 0u ? t + 1 : ntl;
        full |= mb == 0xFFFFu ? (1u << t) : 0u;
    }
    const int t1 = tc1 < ntl ? tc1 : ntl;

    // Products for the wave's tiles [t0, t1) only (uniform).  In a tile with
    // keys that may not be attended (masked, or past L) the mask is folded
    // into the product: such a key gets a bias of -1e30 (finite, so no NaN
    // can arise), far below every candidate threshold.
    constexpr unsigned kMaskedBits = DT == DT_BF16 ? 0xF149u : 0xF149F2CAu;   // -1e30 (bf16 / fp32)
    f32x4 sv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        sv[t] = f32x4{-kInf, -kInf, -kInf, -kInf};
        if (t < t0 || t >= t1) continue;
        KFrag<DT, D> kf;
        kf.load_lds(Ks + (16 * t + c) * C::KSTR, g);
        sv[t] = ((full >> t) & 1u) ? kf.st(qf) : kf.st_bias(qf, ((mbits16(t) >> c) & 1u) ? 0u : kMaskedBits, g);
    }

    // causal / window masks, row max and count
    float mraw = -kInf, nl = 0.f;
    const bool rowok = qrow < L;
    // allowed keys of this lane's query: (klo_i, khi_i] for causal / window
    const int khi_i = qrow;
    const int klo_i = a.window > 0 ? qrow - a.window : -1;
    auto tiles = [&](auto causal_tag) {
        constexpr bool CAUSAL = decltype(causal_tag)::value;
        unsigned cm = kbits;
        if constexpr (CAUSAL) {
            // this lane's keys increase with the slot 4t + i, so the keys in
            // (klo_i, khi_i] are one run of slots: [slots with key <= klo_i,
            // slots with key <= khi_i)
            auto cnt_le = [&](int bound) {
                const int r = bound - kbase - 4 * g;
                const int c = r < 0 ? 0 : 4 * (r >> 4) + min((r & 15) + 1, 4);
                return c < 32 ? c : 32;
            };
            const int chi = cnt_le(khi_i), clo = a.window > 0 ? cnt_le(klo_i) : 0;
            const unsigned mhi = chi >= 32 ? 0xFFFFFFFFu : (1u << chi) - 1u;
            const unsigned mlo = clo >= 32 ? 0xFFFFFFFFu : (1u << clo) - 1u;
            cm = kbits & mhi & ~mlo;
            nl = static_cast<float>(__popc(cm));   // every allowed slot lies in [t0, t1)
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < t0 || t >= t1) continue;    // uniform: outside the wave's keys (-inf)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (CAUSAL) sv[t][i] = ((cm >> (4 * t + i)) & 1u) != 0u ? sv[t][i] : -kInf;
                mraw = fmaxf(mraw, sv[t][i]);
            }
        }
        if constexpr (!CAUSAL) {
            // every key of tiles [t0, t1) with its bit set
            const unsigned long long lo = (1ull << (4 * t0)) - 1ull, hi = (1ull << (4 * t1)) - 1ull;
            nl = static_cast<float>(__popc(kbits & static_cast<unsigned>(hi & ~lo)));
        }
    };
    if (a.causal) tiles(std::true_type{});
    else tiles(std::false_type{});
    if (!rowok) {
        // query rows past L: nothing allowed
        nl = 0.f;
        mraw = -kInf;
#pragma unroll
        for (int t = 0; t < NT; ++t) sv[t] = f32x4{-kInf, -kInf, -kInf, -kInf};
    }
    const float mlane = mraw;   // this lane's maximum
    mraw = col4_max(mraw);
    const float n = col4_sum(nl);
    const bool empty = n == 0.f;

    __syncthreads();   // every wave has its K fragments: the region becomes scratch

    // ---- 2. tau ----------------------------------------------------------------------------
    const float c2 = 0.5f * a.scale;
    const float mc2 = empty ? 0.f : mraw * c2;
    float tr = col_newton<NT>(sv, t0, t1, c2, mc2, n, fmaf(mlane, c2, -mc2));
    if (a.tau != nullptr && g == 0 && rowok) a.tau[static_cast<size_t>(bh) * L + qrow] = empty ? kInf : 2.f * (mc2 + tr);
    const float sh = empty ? 0.f : mc2 + tr;   // p = clamp(acc c2 - sh)^2; empty rows have acc = -inf

    // V into LDS, only now, so that steps 1 and 2 ran while it arrived.
    // bf16: row-major (the P V operand is read back with transpose loads);
    // fp32: transposed, one element at a time.
    if constexpr (C::kAlias) __syncthreads();   // every wave is done with its scratch: the region takes V
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int ch = tid + kThreads * j;
        const int key = ch / CPR, d0 = (ch % CPR) * EPC;
        if constexpr (DT == DT_BF16) {
            *reinterpret_cast<u32x4*>(Vs + key * C::VRS + d0 * 2) = vreg[j];
        } else {
#pragma unroll
            for (int e = 0; e < EPC; ++e) reinterpret_cast<float*>(Vs)[(d0 + e) * VSTR + key] = __uint_as_float(vreg[j][e]);
        }
    }
    __syncthreads();   // V staged

    // ---- 3. O = P V --------------------------------------------------------------------------
    f32x4 o[D / 16];
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto probs = [&](int t, f32x4& p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y = relu1(fmaf(sv[t][i], c2, -sh));
            p[i] = y * y;
        }
    };
    if constexpr (DT == DT_BF16) {
        // chunks of 32 keys = tiles (2h, 2h + 1): slot (g, i) holds key
        // 32h + 4g + i for i < 4 and 32h + 16 + 4g + i - 4 for i >= 4
#pragma unroll
        for (int h = 0; h < NT / 2; ++h) {
            if (2 * h + 1 < t0 || 2 * h >= t1) continue;   // uniform
            float y8[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y8[i] = relu1(fmaf(sv[2 * h][i], c2, -sh));
                y8[4 + i] = relu1(fmaf(sv[2 * h + 1][i], c2, -sh));
            }
            bf16x8 phi, plo;
            split_sq_bf16(y8, phi, plo);
#pragma unroll
            for (int ct = 0; ct < D / 16; ++ct) {
                // B operand: lane (g, c) needs V[key 32h + 4g + k][16ct + c]
                // (k < 4) and the same 16 keys on.  A transpose load hands
                // lane j of a 16-lane group element k of the 4 x b16 row read
                // by lane 4k + j/4, so lane (g, c) points at row
                // 32h + 4g + c/4, columns 16ct + 4(c%4) .. + 3.
                const char* src = Vs + (32 * h + 4 * g + (c >> 2)) * C::VRS + (16 * ct + 4 * (c & 3)) * 2;
                const s16x4 r0 = ds_read_tr16(src);
                const s16x4 r1 = ds_read_tr16(src + 16 * C::VRS);
                const bf16x8 bv = __builtin_bit_cast(bf16x8, s16x8{r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]});
                o[ct] = mfma_bf16(phi, bv, o[ct]);
                o[ct] = mfma_bf16(plo, bv, o[ct]);
            }
        }
    } else {
        // fp32: step s of tile t gives slot g the key 16t + 4g + s
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < t0 || t >= t1) continue;   // uniform
            f32x4 p;
            probs(t, p);
#pragma unroll
            for (int ct = 0; ct < D / 16; ++ct) {
                const f32x4 bv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(Vs) + (16 * ct + c) * VSTR + 16 * t + 4 * g);
#pragma unroll
                for (int s = 0; s < 4; ++s) o[ct] = mfma_f32(p[s], bv[s], o[ct]);
            }
        }
    }

    // O is written once and never read back here: non-temporal stores stream
    // it out instead of leaving dirty lines in L2 for the end of the kernel
    // (the encoder workload, one generation of workgroups: 14.4 -> 12.3 us).
    // Without L2 to merge them, stores of 64-byte row pieces (a lane group's
    // 16 columns) would reach HBM as partial lines, so each 64-column half
    // of the wave's 16 rows is restaged through LDS (row pitch 68 floats:
    // the two lane groups of a half-wave write disjoint banks) and every
    // store covers four whole 256-byte row pieces.
    __syncthreads();   // every wave is done with V and the scratch: LDS is free
    constexpr int OP = 68;
    static_assert(C::lds_bytes >= sizeof(float) * 4 * 16 * OP, "O staging fits");
    float* os = lds + wv * (16 * OP);
    float* outh = a.out + head_off;
#pragma unroll
    for (int h = 0; h < D / 64; ++h) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int i = 0; i < 4; ++i) os[(4 * g + i) * OP + 16 * cc + c] = o[4 * h + cc][i];
        wave_sync();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int rl = 4 * k + lane / 16, col = 4 * (lane % 16);   // row of the wave, first column
            const f32x4 v = *reinterpret_cast<const f32x4*>(os + rl * OP + col);
            const int row = q0 + 16 * wv + rl;
            if (row < L) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(outh + static_cast<size_t>(row) * D + 64 * h + col));
        }
        wave_sync();   // reads done before the next half overwrites the rows
    }
}

}  // namespace ea
