// Streaming a head's keys through LDS in chunks of 64, for kernels whose key
// span is too long to hold at once.
//
// Every chunk of K (and, on request, V) is loaded once per workgroup with
// 16-byte pieces (consecutive threads on consecutive pieces), staged in one
// of two LDS buffers and shared by the four waves.  A chunk's loads are
// issued two chunks ahead (register sets used alternately), so two chunks of
// work cover their latency; the workgroup advances in step, one barrier per
// chunk.  Rows past L are clamped to valid ones (their scores are masked by
// the caller); the valid-key bits of a chunk (key < L and key mask) come
// with it as a 64-bit ballot, one key per lane.
#pragma once

#include "common.hpp"

namespace ea {

template <int DT, int D>
struct ChunkCfg {
    static constexpr int CK = 64;                     // keys per chunk
    static constexpr int ESZ = DT == DT_BF16 ? 2 : 4;
    static constexpr int EPC = 16 / ESZ;              // elements per 16-byte piece
    static constexpr int CPR = D / EPC;               // pieces per row
    static constexpr int NPC = CK * CPR / kThreads;   // pieces per thread per chunk
    static constexpr int KSTR = D * ESZ + 32;         // K row stride in LDS (bytes): +32 keeps the 16-byte row reads of a tile free of bank conflicts (+16 and +64 conflict)
    static constexpr int k_bytes = CK * KSTR;         // one K buffer
    static constexpr int VRS = D * 2 + 32;            // bf16: V row stride (bytes), row-major
    static constexpr int VSTR = CK + EPC;             // fp32: V^T row stride (elements)
    static constexpr int v_bytes = DT == DT_BF16 ? CK * VRS : D * VSTR * 4;
    static constexpr int RB = D * ESZ;                // bytes per K / V row in HBM
    static constexpr int RS = RB == 128 ? 7 : RB == 256 ? 8 : 9;
    static_assert(NPC >= 1 && CK == kWave, "whole pieces per thread; one key per lane");
    static_assert((1 << RS) == RB, "row bytes a power of two");
};

// NBUF: LDS buffers per stream.  Two let a chunk be staged while the
// previous one is in use (one barrier per chunk); one halves the LDS at the
// cost of a second barrier per chunk.  NPRE: chunks in flight in registers,
// 2 (loads issued two chunks ahead) or 1 (one chunk ahead, half the
// registers).
template <int DT, int D, int NBUF = 2, int NPRE = 2>
struct ChunkStream {
    typedef typename InT<DT>::type T;
    typedef ChunkCfg<DT, D> C;
    char* Kb;              // 2 K buffers (row-major, stride KSTR)
    char* Vb;              // 2 V buffers (bf16 row-major, fp32 transposed)
    const T* kh;
    const T* vh;
    const uint8_t* kmp;    // key mask of the batch (or any readable byte when !hasm)
    bool hasm;
    int L, tid, lane;
    // optional per-row float staged with each chunk (side[row], +inf past L)
    // into sideb[64 b .. 64 b + 63] for the chunk's buffer b; null: none
    const float* side = nullptr;
    float* sideb = nullptr;

    struct Pre {
        u32x4 k[C::NPC];
        u32x4 v[C::NPC];
        uint8_t mb;
        float sv;
    };

    // 32-bit byte offsets from the head's base (a head holds at most
    // 65536 rows of at most 512 bytes), so that the address is one scalar
    // base plus one vector offset
    __device__ __forceinline__ void prefetch(int ch, bool withv, Pre& p) const {
        const int cb = ch * C::CK;
        p.mb = kmp[hasm ? clamp_row(cb + lane, L) : 0];   // no branch around the load
        if (side != nullptr) {
            const float sv = side[clamp_row(cb + lane, L)];
            p.sv = cb + lane < L ? sv : kInf;
        }
        const char* kc = reinterpret_cast<const char*>(kh);
        const char* vc = reinterpret_cast<const char*>(vh);
#pragma unroll
        for (int j = 0; j < C::NPC; ++j) {
            const int pc = tid + kThreads * j;
            const unsigned off = (static_cast<unsigned>(clamp_row(cb + pc / C::CPR, L)) << C::RS) + (pc % C::CPR) * 16u;
            p.k[j] = *reinterpret_cast<const u32x4*>(kc + off);
            if (withv) p.v[j] = *reinterpret_cast<const u32x4*>(vc + off);
        }
    }
    __device__ __forceinline__ void stage(int buf, bool withv, const Pre& p) const {
        if (sideb != nullptr && tid < C::CK) sideb[buf * C::CK + tid] = p.sv;
        char* kb = Kb + buf * C::k_bytes;
#pragma unroll
        for (int j = 0; j < C::NPC; ++j) {
            const int pc = tid + kThreads * j;
            *reinterpret_cast<u32x4*>(kb + (pc / C::CPR) * C::KSTR + (pc % C::CPR) * 16) = p.k[j];
        }
        if (withv) {
            char* vb = Vb + buf * C::v_bytes;
#pragma unroll
            for (int j = 0; j < C::NPC; ++j) {
                const int pc = tid + kThreads * j;
                const int key = pc / C::CPR, d0 = (pc % C::CPR) * C::EPC;
                if constexpr (DT == DT_BF16) {
                    *reinterpret_cast<u32x4*>(vb + key * C::VRS + d0 * 2) = p.v[j];
                } else {
#pragma unroll
                    for (int e = 0; e < C::EPC; ++e)
                        reinterpret_cast<float*>(vb)[(d0 + e) * C::VSTR + key] = __uint_as_float(p.v[j][e]);
                }
            }
        }
    }
    __device__ __forceinline__ unsigned long long valid_bits(int ch, const Pre& p) const {
        return __ballot((ch * C::CK + lane < L) & (!hasm | (p.mb != 0)));
    }
    // fn(ch, kbuf, vbuf, M) for the chunks ch0, ch0 + STEP, ... below ch1,
    // in order.  Every thread of the workgroup must call this with the same
    // arguments.  With a side array the staged values of a chunk sit at
    // sideb + (kbuf - Kb) / k_bytes * 64 (the buffer index times 64).
    template <int STEP = 1, typename F>
    __device__ __forceinline__ void run(int ch0, int ch1, bool withv, F&& fn) const {
        static_assert(STEP == 1 || (NBUF == 2 && NPRE == 1), "strided runs: two buffers, one chunk ahead");
        if (ch0 >= ch1) return;
        if constexpr (NBUF == 1 && NPRE == 1) {
            Pre pa;
            prefetch(ch0, withv, pa);
            for (int ch = ch0; ch < ch1; ++ch) {
                stage(0, withv, pa);
                const unsigned long long Ma = valid_bits(ch, pa);
                __syncthreads();
                if (ch + 1 < ch1) prefetch(ch + 1, withv, pa);
                fn(ch, Kb, Vb, Ma);
                __syncthreads();
            }
            return;
        }
        if constexpr (NBUF == 1) {
            Pre pa, pb;
            prefetch(ch0, withv, pa);
            if (ch0 + 1 < ch1) prefetch(ch0 + 1, withv, pb);
            for (int ch = ch0; ch < ch1; ch += 2) {
                // chunk ch is in flight in pa, chunk ch + 1 in pb
                stage(0, withv, pa);
                const unsigned long long Ma = valid_bits(ch, pa);
                __syncthreads();
                if (ch + 2 < ch1) prefetch(ch + 2, withv, pa);
                fn(ch, Kb, Vb, Ma);
                __syncthreads();
                if (ch + 1 >= ch1) break;
                stage(0, withv, pb);
                const unsigned long long Mb = valid_bits(ch + 1, pb);
                __syncthreads();
                if (ch + 3 < ch1) prefetch(ch + 3, withv, pb);
                fn(ch + 1, Kb, Vb, Mb);
                __syncthreads();
            }
            return;
        }
        if constexpr (NPRE == 1) {
            // two buffers, loads one chunk ahead: chunk ch is in buffer
            // (ch - ch0) & 1 while chunk ch + 1 arrives in registers and is
            // staged into the other buffer, which nobody reads since the
            // previous barrier
            Pre pa;
            prefetch(ch0, withv, pa);
            stage(0, withv, pa);
            unsigned long long Mc = valid_bits(ch0, pa);
            __syncthreads();
            int buf = 0;
            for (int ch = ch0; ch < ch1; ch += STEP) {
                if (ch + STEP < ch1) prefetch(ch + STEP, withv, pa);
                fn(ch, Kb + buf * C::k_bytes, Vb + buf * C::v_bytes, Mc);
                if (ch + STEP < ch1) {
                    stage(buf ^ 1, withv, pa);
                    Mc = valid_bits(ch + STEP, pa);
                }
                __syncthreads();
                buf ^= 1;
            }
            return;
        }
        Pre pa, pb;
        prefetch(ch0, withv, pa);
        if (ch0 + 1 < ch1) prefetch(ch0 + 1, withv, pb);
        stage(0, withv, pa);
        unsigned long long Ma = valid_bits(ch0, pa), Mb = 0ull;
        __syncthreads();
        for (int ch = ch0; ch < ch1; ch += 2) {
            // chunk ch sits in buffer 0; chunk ch + 1 is in flight in pb
            if (ch + 2 < ch1) prefetch(ch + 2, withv, pa);
            fn(ch, Kb, Vb, Ma);
            if (ch + 1 < ch1) {
                stage(1, withv, pb);
                Mb = valid_bits(ch + 1, pb);
            }
            __syncthreads();
            if (ch + 1 >= ch1) break;
            // chunk ch + 1 sits in buffer 1; chunk ch + 2 is in flight in pa
            if (ch + 3 < ch1) prefetch(ch + 3, withv, pb);
            fn(ch + 1, Kb + C::k_bytes, Vb + C::v_bytes, Mb);
            if (ch + 2 < ch1) {
                stage(0, withv, pa);
                Ma = valid_bits(ch + 2, pa);
            }
            __syncthreads();
        }
    }
};

}  // namespace ea
