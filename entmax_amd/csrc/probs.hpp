// Dense attention weights from tau, for inspection and tests:
// A_ij = [(s_ij - tau_i)/2]_+^2 on allowed (i, j), 0 elsewhere
// ("ADASPLASH -- ROBERTA Benchmark Result", section 2.2 Theorem 1;
// "DistilBERT SST-2 with AdaSplash Attention" model card, Mathematical
// Formulation 3: entries with s_ij <= tau_i are exactly zero).
// Scores are recomputed with the same MFMA tile code as the forward.
#pragma once

#include "common.hpp"

namespace ea {

struct ProbsArgs {
    const void* q;
    const void* k;
    const uint8_t* key_mask;
    const float* tau;
    float* probs;
    int B, H, L;
    int Hkv;   // key/value heads (H % Hkv == 0)
    int causal, window;
    float scale;
    int nrt, nkt;   // 16-row tiles, 64-key tiles per head
};

// One wave per (head, 16 rows, 64 keys); 4 waves per workgroup.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void probs_kernel(ProbsArgs a) {
    typedef typename InT<DT>::type T;
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wv = tid / kWave;
    const int g = lane / 16, c = lane % 16;
    const long long item = static_cast<long long>(blockIdx.x) * 4 + wv;
    const long long per_head = static_cast<long long>(a.nrt) * a.nkt;
    if (item >= per_head * a.B * a.H) return;
    const int bh = static_cast<int>(item / per_head);
    const int rem = static_cast<int>(item - bh * per_head);
    const int rt = rem / a.nkt, kt = rem % a.nkt;
    const int b = bh / a.H;
    const int L = a.L;
    const size_t head_off = static_cast<size_t>(bh) * L * D;
    const T* qh = static_cast<const T*>(a.q) + head_off;
    const size_t kv_off = static_cast<size_t>(kv_head(bh, a.H, a.Hkv)) * L * D;
    const T* kh = static_cast<const T*>(a.k) + kv_off;
    const uint8_t* km = a.key_mask ? a.key_mask + static_cast<size_t>(b) * L : nullptr;

    QFrag<DT, D> qf;
    qf.load(qh, 16 * rt + c, L, g);
#pragma unroll
    for (int c16 = 0; c16 < 4; ++c16) {
        const int key = kt * kBN + 16 * c16 + c;
        const f32x4 acc = qf.tile(kh, key, L, g);
        const uint8_t mb = km == nullptr ? static_cast<uint8_t>(1) : km[clamp_row(key, L)];
                const bool kv = key < L && mb != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * g + i;
            if (key < L && row < L) {
                const bool ok = kv && allowed_ij(row, key, a.causal, a.window);
                const float x = acc[i] * a.scale - a.tau[static_cast<size_t>(bh) * L + row];
                a.probs[(static_cast<size_t>(bh) * L + row) * L + key] = ok && x > 0.f ? 0.25f * x * x : 0.f;
            }
        }
    }
}

}  // namespace ea
