// C ABI of the gfx950 1.5-entmax attention library: argument validation,
// kernel selection and launch on the caller's stream.  See
// include/entmax_attn.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "entmax_attn.h"
#include "fwd_long.hpp"
#include "fwd_reg.hpp"
#include "fwd_short.hpp"
#include "fwd_wide.hpp"
#include "probs.hpp"
#include "rows.hpp"
#include "bwd.hpp"
#include "bwd_wide.hpp"
#include "decode.hpp"
#include "decode_bwd.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ENTMAX_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    g_err[0] = '\0';
    return ENTMAX_OK;
}

// Common argument checks; returns ENTMAX_OK or an error code.
int check_common(int B, int H, int Hkv, int L, int d, int dtype, int causal, int window) {
    if (B <= 0 || H <= 0 || L <= 0) return fail(ENTMAX_ERR_INVALID_ARG, "B, H, L must be positive (got %d, %d, %d)", B, H, L);
    if (Hkv <= 0 || H % Hkv != 0) return fail(ENTMAX_ERR_INVALID_ARG, "H_kv = %d must divide H = %d", Hkv, H);
    if (window < 0) return fail(ENTMAX_ERR_INVALID_ARG, "window must be >= 0 (got %d)", window);
    if (window > 0 && !causal) return fail(ENTMAX_ERR_INVALID_ARG, "window > 0 requires causal attention");
    if (d != 64 && d != 128) return fail(ENTMAX_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
    if (dtype != ENTMAX_F32 && dtype != ENTMAX_BF16) return fail(ENTMAX_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    if (L > 65536) return fail(ENTMAX_ERR_UNSUPPORTED, "L = %d exceeds 65536", L);
    if (static_cast<long long>(B) * H * ((L + 15) / 16) > (1LL << 30))
        return fail(ENTMAX_ERR_UNSUPPORTED, "B*H*L too large for one launch");
    return ENTMAX_OK;
}

// Largest key span (in 64-key tiles x 64) over the query tiles of height bm.
int max_span(int L, int bm, int causal, int window) {
    int best = 0;
    for (int q0 = 0; q0 < L; q0 += bm) {
        int lo, hi;
        ea::key_range(q0, bm, L, causal, window, &lo, &hi);
        const int span = (hi > lo) ? ((hi + ea::kBN - 1) / ea::kBN - lo / ea::kBN) * ea::kBN : 0;
        if (span > best) best = span;
    }
    return best;
}

template <typename K>
int set_lds(K kernel, size_t bytes) {
    if (bytes <= 65536) return ENTMAX_OK;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
    if (e != hipSuccess) return fail(ENTMAX_ERR_HIP, "hipFuncSetAttribute(%zu B LDS): %s", bytes, hipGetErrorString(e));
    return ENTMAX_OK;
}

template <int DT, int D, int NKT, int KC = NKT * ea::kBN / 4>
int launch_short(const ea::FwdArgs& a, hipStream_t st) {
    typedef ea::ShortCfg<DT, D, NKT, KC> C;
    auto kern = ea::fwd_short_kernel<DT, D, NKT, KC>;
    int rc = set_lds(kern, C::lds_bytes);
    if (rc) return rc;
    const int grid = a.B * a.H * a.nqt;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(ea::kThreads), C::lds_bytes, st, a);
    return check_launch("fwd_short");
}

// Spans beyond 2048 keys: the wide kernel (one pass over K, candidate
// lists, a gather over the support), then the long-span kernel in fix-up
// mode for the 64-row tiles holding a row whose candidates outgrew its list.
template <int DT, int D>
int launch_wide(ea::FwdArgs a, hipStream_t st) {
    typedef ea::WideCfg<DT, D> W;
    typedef ea::LongCfg<DT, D> C;
    // every chunk clean (no mask, no causal crossing, every row a query row):
    // the instance without the masked chunk path
    const bool clean = a.key_mask == nullptr && !a.causal && a.L % W::BR == 0;
    auto kw = clean ? ea::fwd_wide_kernel<DT, D, false> : ea::fwd_wide_kernel<DT, D, true>;
    auto kl = ea::fwd_long_kernel<DT, D>;
    int rc = set_lds(kw, W::fwd_lds_bytes);
    if (!rc) rc = set_lds(kl, C::lds_bytes);
    if (rc) return rc;
    a.nqt = (a.L + W::BR - 1) / W::BR;
    a.fixup = 0;
    hipLaunchKernelGGL(kw, dim3(a.B * a.H * a.nqt), dim3(ea::kThreads), W::fwd_lds_bytes, st, a);
    a.nqt = (a.L + C::BM - 1) / C::BM;
    a.fixup = 1;
    hipLaunchKernelGGL(kl, dim3(a.B * a.H * a.nqt), dim3(ea::kThreads), C::lds_bytes, st, a);
    return check_launch("fwd_wide");
}

template <int DT, int D>
int launch_long(ea::FwdArgs a, hipStream_t st) {
    typedef ea::LongCfg<DT, D> C;
    auto kern = ea::fwd_long_kernel<DT, D>;
    int rc = set_lds(kern, C::lds_bytes);
    if (rc) return rc;
    a.nqt = (a.L + C::BM - 1) / C::BM;
    const long long grid = static_cast<long long>(a.B) * a.H * a.nqt;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(ea::kThreads), C::lds_bytes, st, a);
    return check_launch("fwd_long");
}

template <int DT, int D>
int launch_reg(ea::FwdArgs a, hipStream_t st) {
    typedef ea::RegCfg<DT, D> C;
    auto kern = ea::fwd_reg_kernel<DT, D>;
    int rc = set_lds(kern, C::lds_bytes);
    if (rc) return rc;
    a.nqt = (a.L + C::BM - 1) / C::BM;
    const long long grid = static_cast<long long>(a.B) * a.H * a.nqt;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(ea::kThreads), C::lds_bytes, st, a);
    return check_launch("fwd_reg");
}

// The register-held kernel takes a tile of 32 rows when the 128-key pairs
// its rows may attend number at most 8.
bool reg_fits(int L, int causal, int window) {
    const int bm = 32, pk = 128;
    if (!causal || window <= 0) return (L + pk - 1) / pk <= 8;
    int worst = 0;
    for (int q0 = 0; q0 < L; q0 += bm) {
        int lo, hi;
        ea::key_range(q0, bm, L, causal, window, &lo, &hi);
        const int n = lo < hi ? (hi + pk - 1) / pk - lo / pk : 0;
        worst = n > worst ? n : worst;
    }
    return worst <= 8;
}

template <int DT, int D>
int dispatch_fwd(ea::FwdArgs a, hipStream_t st) {
    const int L = a.L;
    const int s64 = max_span(L, 64, a.causal, a.window);
    if (s64 <= 64) {
        a.nqt = (L + 63) / 64;
        return launch_short<DT, D, 1>(a, st);
    }
    if (s64 <= 128) {
        a.nqt = (L + 63) / 64;
        // a causal window of at most 32 keys leaves a lane at most 12 allowed
        // keys (three 16-key tiles): a smaller scratch, more workgroups per CU
        if (a.causal && a.window > 0 && a.window <= 32) return launch_short<DT, D, 2, 16>(a, st);
        return launch_short<DT, D, 2>(a, st);
    }
    // spans beyond 2048 keys: a sampled pass and a pass over K with
    // candidate lists, then a gather over the support (the multi-pass
    // long-span kernel re-reads K and V more than it saves there)
    if (s64 > 2048) return launch_wide<DT, D>(a, st);
    // (float32 at d = 128 would not keep its scores in registers)
    if constexpr (!(DT == ea::DT_F32 && D == 128))
        if (reg_fits(L, a.causal, a.window)) return launch_reg<DT, D>(a, st);
    return launch_long<DT, D>(a, st);
}

// Backward: query side (dQ, c) then key side (dK, dV), all on one stream.
// Spans beyond 2048 keys take the wide query-side kernel (on the forward's
// saved support when given, else with a pass over the keys), which also
// fills the support buckets of the key side; its rows with an overflowing support
// are finished by the tile kernel in fix-up mode, and keys whose bucket
// overflowed by the key-side recompute kernel in fix-up mode.  Shorter spans
// take the tile kernel and the key-side recompute kernel.
template <int DT, int D>
int launch_bwd(ea::BwdArgs a, hipStream_t st) {
    typedef ea::WideCfg<DT, D> W;
    auto kq = ea::bwd_kernel<DT, D>;
    auto kw = ea::bwd_q_kernel<DT, D>;

    auto kv = ea::bwd_kv_kernel<DT, D>;
    constexpr size_t lds_q = ea::BwdCfg<DT, D>::lds_bytes;
    int rc = set_lds(kq, lds_q);
    if (!rc) rc = set_lds(kw, W::stream_lds_bytes);
    if (!rc) rc = set_lds(kv, W::lds_bytes);
    if (rc) return rc;
    const int L = a.L;
    const int nt64 = (L + 63) / 64;
    const bool wide = max_span(L, 64, a.causal, a.window) > 2048;
    if (wide) {
        // bucket counters and the flag start at zero (a fill kernel, so that
        // the sequence can be captured in a graph)
        const size_t nz = static_cast<size_t>(reinterpret_cast<char*>(a.kflag) - reinterpret_cast<char*>(a.kcnt)) / 4 + 64;
        hipLaunchKernelGGL(ea::zero_fill_kernel, dim3(static_cast<unsigned>((nz / 4 + ea::kThreads) / ea::kThreads)),
                           dim3(ea::kThreads), 0, st, reinterpret_cast<float*>(a.kcnt), nz);
        a.nqt = (L + W::BR - 1) / W::BR;
        a.fixup = 0;
        if (a.scount != nullptr) {   // the forward's saved support: no pass over the keys
            constexpr int rpb = ea::kThreads / (D / 8);   // rows per workgroup
            const long long rows = static_cast<long long>(a.B) * a.H * L;
            hipLaunchKernelGGL((ea::bwd_q_saved_kernel<DT, D>), dim3(static_cast<unsigned>((rows + rpb - 1) / rpb)),
                               dim3(ea::kThreads), 0, st, a);
        } else {
            hipLaunchKernelGGL(kw, dim3(a.B * a.H * a.nqt), dim3(ea::kThreads), W::stream_lds_bytes, st, a);
        }
        a.fixup = 1;
    } else {
        a.kcnt = nullptr;
        a.kflag = nullptr;
        a.fixup = 0;
    }
    a.nqt = nt64;
    hipLaunchKernelGGL(kq, dim3(a.B * a.H * a.nqt), dim3(ea::kThreads), lds_q, st, a);
    if (wide) {
        constexpr int kpb = ea::kThreads / (D / 8);   // keys per gather workgroup
        const unsigned ng = static_cast<unsigned>(a.B * a.Hkv * ((L + kpb - 1) / kpb));
        hipLaunchKernelGGL((ea::bwd_kv_gather_kernel<DT, D>), dim3(ng), dim3(ea::kThreads), 0, st, a);
    }
    a.nqt = (L + W::BR - 1) / W::BR;   // key tiles per key/value head
    hipLaunchKernelGGL(kv, dim3(a.B * a.Hkv * a.nqt), dim3(ea::kThreads), W::lds_bytes, st, a);
    return check_launch("bwd");
}

// Workspace of the backward: c_i per query row, then a bucket counter per
// key (sized by the query heads, which bound the key/value heads), then the
// overflow flag; each part 256-byte aligned.
size_t bwd_ws_part(int B, int H, int L) {
    const size_t n = static_cast<size_t>(B) * H * L * sizeof(float);
    return (n + 255) & ~static_cast<size_t>(255);
}
size_t bwd_ws_bytes(int B, int H, int L) { return 2 * bwd_ws_part(B, H, L) + 256; }

// Scratch of the allocation-free backward (entmax_attn_bwd_noalloc): the
// backward's workspace for up to kScratchRows query rows (B H L): c_i and a
// bucket counter per row, and a flag, 8 MiB + 256 bytes.  Every GPU the
// library runs on holds one copy until the process ends.  In host code the
// name stands for a host-side stand-in: the device address comes from
// hipGetSymbolAddress, once per device (scratch_addr).
constexpr size_t kScratchRows = static_cast<size_t>(1) << 20;
static __device__ __align__(256) float scratch[2 * kScratchRows + 64];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first
// call on that device.
int scratch_addr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ENTMAX_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ENTMAX_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(ENTMAX_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ENTMAX_OK;
}

// Forward after the argument checks.
int fwd_run(ea::FwdArgs a, int d, int dtype, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == ENTMAX_BF16)
        return d == 64 ? dispatch_fwd<ea::DT_BF16, 64>(a, st) : dispatch_fwd<ea::DT_BF16, 128>(a, st);
    return d == 64 ? dispatch_fwd<ea::DT_F32, 64>(a, st) : dispatch_fwd<ea::DT_F32, 128>(a, st);
}

// The saved support of the forward (spans beyond 2048 keys, where the wide
// kernels run): a count per query row, then d/2 entries of 8 bytes per row;
// the count part 256-byte aligned.
bool saves_support(int L, int causal, int window) { return max_span(L, 64, causal, window) > 2048; }
size_t saved_part(int B, int H, int L) {
    const size_t n = static_cast<size_t>(B) * H * L * sizeof(int);
    return (n + 255) & ~static_cast<size_t>(255);
}
size_t saved_bytes(int B, int H, int L, int d) {
    return saved_part(B, H, L) + static_cast<size_t>(B) * H * L * (d / 2) * 8;
}

}  // namespace

template <int DT, bool GEN>
void launch_rows_fwd_g(const ea::RowsArgs& a, hipStream_t st) {
    const dim3 block(ea::kThreads);
    if (a.R < 1024 && a.L > 1024) {
        // few long rows (fewer than one wave per SIMD): a workgroup per row
        constexpr int T = ea::kThreads;
        const dim3 grid(a.R);
        if (a.L <= 2048) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 2, GEN, T>), grid, block, 0, st, a);
        else if (a.L <= 4096) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 4, GEN, T>), grid, block, 0, st, a);
        else if (a.L <= 8192) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 8, GEN, T>), grid, block, 0, st, a);
        else if (a.L <= 16384) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 16, GEN, T>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 0, GEN, T>), grid, block, 0, st, a);
        return;
    }
    const dim3 grid((a.R + 3) / 4);
    if (a.L <= 256) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 1, GEN>), grid, block, 0, st, a);
    else if (a.L <= 512) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 2, GEN>), grid, block, 0, st, a);
    else if (a.L <= 1024) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 4, GEN>), grid, block, 0, st, a);
    else if (a.L <= 2048) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 8, GEN>), grid, block, 0, st, a);
    else if (a.L <= 4096) hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 16, GEN>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((ea::rows_fwd_kernel<DT, 0, GEN>), grid, block, 0, st, a);
}

// alpha = 1.5 takes the instantiation that squares instead of calling powers
template <int DT>
void launch_rows_fwd(const ea::RowsArgs& a, hipStream_t st) {
    if (a.alpha == 1.5f) launch_rows_fwd_g<DT, false>(a, st);
    else launch_rows_fwd_g<DT, true>(a, st);
}

template <bool GEN>
void launch_rows_bwd_g(const ea::RowsBwdArgs& a, hipStream_t st) {
    const dim3 grid((a.R + 3) / 4), block(ea::kThreads);
    if (a.L <= 256) hipLaunchKernelGGL((ea::rows_bwd_kernel<1, GEN>), grid, block, 0, st, a);
    else if (a.L <= 1024) hipLaunchKernelGGL((ea::rows_bwd_kernel<4, GEN>), grid, block, 0, st, a);
    else if (a.L <= 4096) hipLaunchKernelGGL((ea::rows_bwd_kernel<16, GEN>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((ea::rows_bwd_kernel<0, GEN>), grid, block, 0, st, a);
}

void launch_rows_bwd(const ea::RowsBwdArgs& a, hipStream_t st) {
    if (a.alpha == 1.5f) launch_rows_bwd_g<false>(a, st);
    else launch_rows_bwd_g<true>(a, st);
}

// Workspace of the decode path: byte offsets of its arrays (each 256-byte
// aligned) for the longest span the arguments allow.
struct DecLayout {
    int nch, P;
    size_t sbuf, cmax, part, tau, rlen, total;
};

DecLayout dec_layout(int B, int H, int Lq, int S, int d, int window) {  // any H_kv
    auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    DecLayout l;
    // keys any of the Lq queries may attend: the window of the first query
    // widened by the Lq - 1 later ones
    const long long wide = static_cast<long long>(window) + Lq - 1;
    const int span = (window > 0 && wide < S) ? static_cast<int>(wide) : S;
    l.nch = (span + ea::kDecChunk - 1) / ea::kDecChunk;
    l.P = l.nch * ea::kDecChunk;
    const size_t rows = static_cast<size_t>(B) * H * Lq;
    l.sbuf = 0;
    l.cmax = l.sbuf + al(rows * l.P * sizeof(float));
    l.part = l.cmax + al(rows * l.nch * sizeof(float));
    l.tau = l.part + al(rows * l.nch * d * sizeof(float));
    l.rlen = l.tau + al(rows * sizeof(float));
    l.total = l.rlen + al(rows * sizeof(int));
    return l;
}

// Workspace of the decode backward: the scores and dS of every row's span,
// the chunk maxima and the span lengths (written by the scores kernel).
struct DecBwdLayout {
    int nch, P;
    size_t sbuf, dsbuf, cmax, rlen, total;
};

DecBwdLayout dec_bwd_layout(int B, int H, int Lq, int S, int d, int window) {
    auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    const DecLayout f = dec_layout(B, H, Lq, S, d, window);
    DecBwdLayout l;
    l.nch = f.nch;
    l.P = f.P;
    const size_t rows = static_cast<size_t>(B) * H * Lq;
    l.sbuf = 0;
    l.dsbuf = l.sbuf + al(rows * l.P * sizeof(float));
    l.cmax = l.dsbuf + al(rows * l.P * sizeof(float));
    l.rlen = l.cmax + al(rows * l.nch * sizeof(float));
    l.total = l.rlen + al(rows * sizeof(int));
    return l;
}

int check_decode(int B, int H, int Hkv, int Lq, int S, int d, int dtype, int causal, int window) {
    if (B <= 0 || H <= 0 || S <= 0) return fail(ENTMAX_ERR_INVALID_ARG, "B, H, S must be positive (got %d, %d, %d)", B, H, S);
    if (Lq <= 0 || Lq > S) return fail(ENTMAX_ERR_INVALID_ARG, "Lq = %d outside [1, S = %d]", Lq, S);
    if (Hkv <= 0 || H % Hkv != 0) return fail(ENTMAX_ERR_INVALID_ARG, "H_kv = %d must divide H = %d", Hkv, H);
    if (window < 0) return fail(ENTMAX_ERR_INVALID_ARG, "window must be >= 0 (got %d)", window);
    if (window > 0 && !causal) return fail(ENTMAX_ERR_INVALID_ARG, "window > 0 requires causal attention");
    if (d != 64 && d != 128) return fail(ENTMAX_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
    if (dtype != ENTMAX_F32 && dtype != ENTMAX_BF16) return fail(ENTMAX_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    if (S > (1 << 24)) return fail(ENTMAX_ERR_UNSUPPORTED, "S = %d exceeds 2^24", S);
    if (static_cast<long long>(B) * Hkv > 65535) return fail(ENTMAX_ERR_UNSUPPORTED, "B * H_kv exceeds 65535");
    if (static_cast<long long>(B) * H * Lq * (S + 255) > (1LL << 36)) return fail(ENTMAX_ERR_UNSUPPORTED, "B * H * Lq * S too large");
    if ((static_cast<long long>(H / Hkv) * Lq + 15) / 16 > 65535) return fail(ENTMAX_ERR_UNSUPPORTED, "H / H_kv * Lq too large");
    return ENTMAX_OK;
}

// Decode backward: scores of every row's span, then dq and dS per row, then
// dk and dv per key.
template <int DT, int D>
void launch_decode_bwd(const ea::DecBwdArgs& a, hipStream_t st) {
    const ea::DecArgs& f = a.f;
    const int nz = ((f.H / f.Hkv) * f.Lq + 15) / 16;
    const dim3 block(ea::kThreads);
    hipLaunchKernelGGL((ea::dec_scores_kernel<DT, D>), dim3(f.nch, f.B * f.Hkv, nz), block, 0, st, f);
    const int rows = f.B * f.H * f.Lq;
    const int wpb = ea::kThreads / ea::kWave;
    hipLaunchKernelGGL((ea::dec_bwd_rows_kernel<DT, D>), dim3((rows + wpb - 1) / wpb), block, 0, st, a);
    hipLaunchKernelGGL((ea::dec_bwd_keys_kernel<DT, D>), dim3((f.S + wpb - 1) / wpb, f.B * f.Hkv), block, 0, st, a);
}

template <int DT, int D>
void launch_decode(const ea::DecArgs& a, hipStream_t st) {
    const int nz = ((a.H / a.Hkv) * a.Lq + 15) / 16;   // groups of 16 query rows per key/value head
    const dim3 block(ea::kThreads);
    if (a.nch == 1) {   // every span fits one chunk: one launch
        hipLaunchKernelGGL((ea::dec_short_kernel<DT, D>), dim3(a.B * a.Hkv, nz), block, 0, st, a);
        return;
    }
    const dim3 grid(a.nch, a.B * a.Hkv, nz);
    hipLaunchKernelGGL((ea::dec_scores_kernel<DT, D>), grid, block, 0, st, a);
    ea::RowsArgs r;
    r.s = a.sbuf; r.mask = nullptr; r.p = nullptr; r.tau = a.tau; r.R = a.B * a.H * a.Lq; r.L = a.P; r.alpha = 1.5f;
    r.row_len = a.row_len;
    launch_rows_fwd<ea::DT_F32>(r, st);
    hipLaunchKernelGGL((ea::dec_pv_kernel<DT, D>), grid, block, 0, st, a);
    hipLaunchKernelGGL((ea::dec_reduce_kernel<D>), dim3((a.B * a.H * a.Lq + 3) / 4), block, 0, st, a);
}

int check_rows(int R, int L) {
    if (R <= 0 || L <= 0) return fail(ENTMAX_ERR_INVALID_ARG, "rows and L must be positive (got %d, %d)", R, L);
    if (L % 4 != 0) return fail(ENTMAX_ERR_UNSUPPORTED, "L = %d is not a multiple of 4", L);
    if (static_cast<long long>(R) * L > (1LL << 40)) return fail(ENTMAX_ERR_UNSUPPORTED, "R * L too large");
    if ((R + 3) / 4 > (1 << 30)) return fail(ENTMAX_ERR_UNSUPPORTED, "too many rows for one launch");
    return ENTMAX_OK;
}

// True when a non-null pointer of the list is not a multiple of `al` bytes:
// the kernels read and write rows with 16-byte vector accesses, and floats
// (tau, probs) and int32 lengths with 4-byte ones.
static bool misaligned(std::initializer_list<const void*> ps, uintptr_t al) {
    for (const void* p : ps)
        if (p != nullptr && reinterpret_cast<uintptr_t>(p) % al != 0) return true;
    return false;
}

extern "C" {

int entmax_attn_fwd_gqa(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal, int window,
                        float* out, float* tau_out, int B, int H, int Hkv, int L, int d, int dtype, void* stream) {
    if (!q || !k || !v || !out) return fail(ENTMAX_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
    if (misaligned({q, k, v, out}, 16) || misaligned({tau_out}, 4))
        return fail(ENTMAX_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned, tau_out 4-byte aligned");
    int rc = check_common(B, H, Hkv, L, d, dtype, causal, window);
    if (rc) return rc;
    ea::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.key_mask = key_mask;
    a.out = out; a.tau = tau_out;
    a.B = B; a.H = H; a.L = L; a.Hkv = Hkv;
    a.causal = causal ? 1 : 0; a.window = window;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
    a.nqt = 0;
    a.fixup = 0;
    a.scount = nullptr;
    a.sent = nullptr;
    return fwd_run(a, d, dtype, stream);
}

int entmax_attn_probs_gqa(const void* q, const void* k, const uint8_t* key_mask, int causal, int window,
                          const float* tau, float* probs, int B, int H, int Hkv, int L, int d, int dtype, void* stream) {
    if (!q || !k || !tau || !probs) return fail(ENTMAX_ERR_INVALID_ARG, "q, k, tau and probs must not be NULL");
    if (misaligned({q, k}, 16) || misaligned({tau, probs}, 4))
        return fail(ENTMAX_ERR_INVALID_ARG, "q and k must be 16-byte aligned, tau and probs 4-byte aligned");
    int rc = check_common(B, H, Hkv, L, d, dtype, causal, window);
    if (rc) return rc;
    ea::ProbsArgs a;
    a.q = q; a.k = k; a.key_mask = key_mask; a.tau = tau; a.probs = probs;
    a.B = B; a.H = H; a.L = L; a.Hkv = Hkv; a.causal = causal ? 1 : 0; a.window = window;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
    a.nrt = (L + 15) / 16;
    a.nkt = (L + ea::kBN - 1) / ea::kBN;
    const long long items = static_cast<long long>(B) * H * a.nrt * a.nkt;
    if ((items + 3) / 4 > (1LL << 31) - 1) return fail(ENTMAX_ERR_UNSUPPORTED, "probs grid too large");
    const dim3 grid(static_cast<unsigned>((items + 3) / 4));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == ENTMAX_BF16) {
        if (d == 64) hipLaunchKernelGGL((ea::probs_kernel<ea::DT_BF16, 64>), grid, dim3(ea::kThreads), 0, st, a);
        else hipLaunchKernelGGL((ea::probs_kernel<ea::DT_BF16, 128>), grid, dim3(ea::kThreads), 0, st, a);
    } else {
        if (d == 64) hipLaunchKernelGGL((ea::probs_kernel<ea::DT_F32, 64>), grid, dim3(ea::kThreads), 0, st, a);
        else hipLaunchKernelGGL((ea::probs_kernel<ea::DT_F32, 128>), grid, dim3(ea::kThreads), 0, st, a);
    }
    return check_launch("probs");
}

size_t entmax_attn_bwd_workspace_bytes(int B, int H, int L, int d) {
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0) return 0;
    return bwd_ws_bytes(B, H, L);
}

}  // extern "C"

namespace {

// Backward after the workspace checks: ws is a workspace of bwd_ws_bytes.
int bwd_run(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal, int window,
            const float* tau, const void* dout, float* dq, float* dk, float* dv,
            int B, int H, int Hkv, int L, int d, int dtype, void* ws, void* stream,
            const void* saved = nullptr) {
    ea::BwdArgs a;
    a.scount = nullptr;
    a.sent = nullptr;
    if (saved != nullptr) {
        a.scount = static_cast<const int*>(saved);
        a.sent = reinterpret_cast<const float*>(static_cast<const char*>(saved) + saved_part(B, H, L));
    }
    a.q = q; a.k = k; a.v = v; a.key_mask = key_mask; a.tau = tau; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv;
    char* w = static_cast<char*>(ws);
    const size_t part = bwd_ws_part(B, H, L);
    a.cbuf = reinterpret_cast<float*>(w);
    a.kcnt = reinterpret_cast<int*>(w + part);
    a.kflag = reinterpret_cast<int*>(w + 2 * part);
    a.B = B; a.H = H; a.L = L; a.Hkv = Hkv; a.causal = causal ? 1 : 0; a.window = window;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
    a.nqt = 0;
    a.fixup = 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == ENTMAX_BF16) return d == 64 ? launch_bwd<ea::DT_BF16, 64>(a, st) : launch_bwd<ea::DT_BF16, 128>(a, st);
    return d == 64 ? launch_bwd<ea::DT_F32, 64>(a, st) : launch_bwd<ea::DT_F32, 128>(a, st);
}

int bwd_check(const void* q, const void* k, const void* v, const void* tau, const void* dout,
              const void* dq, const void* dk, const void* dv, int causal, int window,
              int B, int H, int Hkv, int L, int d, int dtype) {
    if (!q || !k || !v || !tau || !dout || !dq || !dk || !dv)
        return fail(ENTMAX_ERR_INVALID_ARG, "q, k, v, tau, dout, dq, dk and dv must not be NULL");
    if (misaligned({q, k, v, dout, dq, dk, dv}, 16) || misaligned({tau}, 4))
        return fail(ENTMAX_ERR_INVALID_ARG, "q, k, v, dout, dq, dk and dv must be 16-byte aligned, tau 4-byte aligned");
    return check_common(B, H, Hkv, L, d, dtype, causal, window);
}

}  // namespace

extern "C" {

int entmax_attn_bwd_gqa(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal, int window,
                        const float* tau, const void* dout, float* dq, float* dk, float* dv,
                        int B, int H, int Hkv, int L, int d, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
    int rc = bwd_check(q, k, v, tau, dout, dq, dk, dv, causal, window, B, H, Hkv, L, d, dtype);
    if (rc) return rc;
    if (!workspace) return fail(ENTMAX_ERR_INVALID_ARG, "workspace must not be NULL");
    if (misaligned({workspace}, 256)) return fail(ENTMAX_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    const size_t need = bwd_ws_bytes(B, H, L);
    if (workspace_bytes < need)
        return fail(ENTMAX_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    return bwd_run(q, k, v, key_mask, causal, window, tau, dout, dq, dk, dv, B, H, Hkv, L, d, dtype, workspace,
                   stream);
}

int entmax_attn_bwd_noalloc(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal,
                            int window, const float* tau, const void* dout, float* dq, float* dk, float* dv,
                            int B, int H, int Hkv, int L, int d, int dtype, void* stream) {
    int rc = bwd_check(q, k, v, tau, dout, dq, dk, dv, causal, window, B, H, Hkv, L, d, dtype);
    if (rc) return rc;
    const size_t rows = static_cast<size_t>(B) * H * L;
    if (rows > kScratchRows)
        return fail(ENTMAX_ERR_INVALID_ARG, "B*H*L = %zu query rows exceeds the %zu of the built-in scratch",
                    rows, kScratchRows);
    void* ws = nullptr;
    rc = scratch_addr(&ws);
    if (rc) return rc;
    // c_i of every query row is written before it is read, and the bucket
    // counters are cleared by the call itself (a fill kernel)
    return bwd_run(q, k, v, key_mask, causal, window, tau, dout, dq, dk, dv, B, H, Hkv, L, d, dtype, ws, stream);
}

size_t entmax_attn_saved_bytes(int B, int H, int L, int d) {
    if (B <= 0 || H <= 0 || L <= 0 || d <= 0) return 0;
    return saved_bytes(B, H, L, d);
}

int entmax_attn_fwd_save(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal,
                         int window, float* out, float* tau_out, void* saved, size_t saved_bytes_given,
                         int B, int H, int Hkv, int L, int d, int dtype, void* stream) {
    if (!q || !k || !v || !out || !tau_out || !saved)
        return fail(ENTMAX_ERR_INVALID_ARG, "q, k, v, out, tau_out and saved must not be NULL");
    if (misaligned({q, k, v, out}, 16) || misaligned({tau_out}, 4) || misaligned({saved}, 256))
        return fail(ENTMAX_ERR_INVALID_ARG,
                    "q, k, v and out must be 16-byte aligned, tau_out 4-byte aligned, saved 256-byte aligned");
    int rc = check_common(B, H, Hkv, L, d, dtype, causal, window);
    if (rc) return rc;
    const size_t need = saved_bytes(B, H, L, d);
    if (saved_bytes_given < need)
        return fail(ENTMAX_ERR_INVALID_ARG, "saved buffer of %zu bytes, %zu needed", saved_bytes_given, need);
    ea::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.key_mask = key_mask;
    a.out = out; a.tau = tau_out;
    a.B = B; a.H = H; a.L = L; a.Hkv = Hkv;
    a.causal = causal ? 1 : 0; a.window = window;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
    a.nqt = 0;
    a.fixup = 0;
    a.scount = nullptr;
    a.sent = nullptr;
    if (saves_support(L, causal, window)) {
        a.scount = static_cast<int*>(saved);
        a.sent = reinterpret_cast<float*>(static_cast<char*>(saved) + saved_part(B, H, L));
    }
    return fwd_run(a, d, dtype, stream);
}

int entmax_attn_bwd_saved(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal,
                          int window, const float* tau, const void* dout, const void* saved,
                          size_t saved_bytes_given, float* dq, float* dk, float* dv, int B, int H, int Hkv, int L,
                          int d, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = bwd_check(q, k, v, tau, dout, dq, dk, dv, causal, window, B, H, Hkv, L, d, dtype);
    if (rc) return rc;
    if (!workspace || !saved) return fail(ENTMAX_ERR_INVALID_ARG, "workspace and saved must not be NULL");
    if (misaligned({workspace, saved}, 256))
        return fail(ENTMAX_ERR_INVALID_ARG, "workspace and saved must be 256-byte aligned");
    const size_t need = bwd_ws_bytes(B, H, L);
    if (workspace_bytes < need)
        return fail(ENTMAX_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    const size_t sneed = saved_bytes(B, H, L, d);
    if (saved_bytes_given < sneed)
        return fail(ENTMAX_ERR_INVALID_ARG, "saved buffer of %zu bytes, %zu needed", saved_bytes_given, sneed);
    return bwd_run(q, k, v, key_mask, causal, window, tau, dout, dq, dk, dv, B, H, Hkv, L, d, dtype, workspace,
                   stream, saves_support(L, causal, window) ? saved : nullptr);
}

int entmax_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal, int window,
                    float* out, float* tau_out, int B, int H, int L, int d, int dtype, void* stream) {
    return entmax_attn_fwd_gqa(q, k, v, key_mask, causal, window, out, tau_out, B, H, H, L, d, dtype, stream);
}

int entmax_attn_bwd(const void* q, const void* k, const void* v, const uint8_t* key_mask, int causal, int window,
                    const float* tau, const void* dout, float* dq, float* dk, float* dv,
                    int B, int H, int L, int d, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return entmax_attn_bwd_gqa(q, k, v, key_mask, causal, window, tau, dout, dq, dk, dv, B, H, H, L, d, dtype,
                               workspace, workspace_bytes, stream);
}

int entmax_attn_probs(const void* q, const void* k, const uint8_t* key_mask, int causal, int window,
                      const float* tau, float* probs, int B, int H, int L, int d, int dtype, void* stream) {
    return entmax_attn_probs_gqa(q, k, key_mask, causal, window, tau, probs, B, H, H, L, d, dtype, stream);
}

int entmax_bisect_rows_fwd(const void* scores, const uint8_t* mask, float* p, float* tau, int R, int L, float alpha,
                           int dtype, void* stream) {
    if (!scores || !p) return fail(ENTMAX_ERR_INVALID_ARG, "scores and p must not be NULL");
    if (misaligned({scores, mask, p}, 16) || misaligned({tau}, 4))
        return fail(ENTMAX_ERR_INVALID_ARG, "scores, mask and p must be 16-byte aligned, tau 4-byte aligned");
    if (!(alpha > 1.f && alpha <= 2.f)) return fail(ENTMAX_ERR_INVALID_ARG, "alpha = %g outside (1, 2]", alpha);
    int rc = check_rows(R, L);
    if (rc) return rc;
    if (dtype != ENTMAX_F32 && dtype != ENTMAX_BF16) return fail(ENTMAX_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    ea::RowsArgs a;
    a.s = scores; a.mask = mask; a.p = p; a.tau = tau; a.R = R; a.L = L; a.alpha = alpha;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == ENTMAX_BF16) launch_rows_fwd<ea::DT_BF16>(a, st);
    else launch_rows_fwd<ea::DT_F32>(a, st);
    return check_launch("rows_fwd");
}

int entmax_bisect_rows_bwd(const float* p, const float* dp, float* ds, int R, int L, float alpha, void* stream) {
    if (!p || !dp || !ds) return fail(ENTMAX_ERR_INVALID_ARG, "p, dp and ds must not be NULL");
    if (misaligned({p, dp, ds}, 16)) return fail(ENTMAX_ERR_INVALID_ARG, "p, dp and ds must be 16-byte aligned");
    if (!(alpha > 1.f && alpha <= 2.f)) return fail(ENTMAX_ERR_INVALID_ARG, "alpha = %g outside (1, 2]", alpha);
    int rc = check_rows(R, L);
    if (rc) return rc;
    ea::RowsBwdArgs a;
    a.p = p; a.dp = dp; a.ds = ds; a.R = R; a.L = L; a.alpha = alpha;
    launch_rows_bwd(a, static_cast<hipStream_t>(stream));
    return check_launch("rows_bwd");
}

int entmax15_rows_fwd(const void* scores, const uint8_t* mask, float* p, float* tau, int R, int L, int dtype,
                      void* stream) {
    return entmax_bisect_rows_fwd(scores, mask, p, tau, R, L, 1.5f, dtype, stream);
}

int entmax15_rows_bwd(const float* p, const float* dp, float* ds, int R, int L, void* stream) {
    return entmax_bisect_rows_bwd(p, dp, ds, R, L, 1.5f, stream);
}

size_t entmax_attn_decode_workspace_size(int B, int H, int H_kv, int Lq, int S, int d, int window) {
    if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || Lq <= 0 || S <= 0 || d <= 0 || window < 0) return 0;
    return dec_layout(B, H, Lq, S, d, window).total;
}

int entmax_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens, int causal,
                       int window, float* out, float* tau_out, void* workspace, size_t workspace_bytes, int B, int H,
                       int Hkv, int Lq, int S, int d, int dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !seqlens || !out || !workspace)
        return fail(ENTMAX_ERR_INVALID_ARG, "q, k_cache, v_cache, seqlens, out and workspace must not be NULL");
    if (misaligned({q, k_cache, v_cache, out}, 16) || misaligned({seqlens, tau_out}, 4))
        return fail(ENTMAX_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned, seqlens and tau_out 4-byte aligned");
    int rc = check_decode(B, H, Hkv, Lq, S, d, dtype, causal, window);
    if (rc) return rc;
    const DecLayout l = dec_layout(B, H, Lq, S, d, window);
    if (workspace_bytes < l.total)
        return fail(ENTMAX_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, l.total);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(ENTMAX_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    char* ws = static_cast<char*>(workspace);
    ea::DecArgs a;
    a.q = q; a.k = k_cache; a.v = v_cache; a.seqlens = seqlens; a.out = out; a.tau_out = tau_out;
    a.sbuf = reinterpret_cast<float*>(ws + l.sbuf);
    a.cmax = reinterpret_cast<float*>(ws + l.cmax);
    a.part = reinterpret_cast<float*>(ws + l.part);
    a.tau = reinterpret_cast<float*>(ws + l.tau);
    a.row_len = reinterpret_cast<int*>(ws + l.rlen);
    a.B = B; a.H = H; a.Hkv = Hkv; a.Lq = Lq; a.S = S; a.window = window; a.causal = causal != 0;
    a.nch = l.nch; a.P = l.P;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == ENTMAX_BF16) {
        if (d == 64) launch_decode<ea::DT_BF16, 64>(a, st);
        else launch_decode<ea::DT_BF16, 128>(a, st);
    } else {
        if (d == 64) launch_decode<ea::DT_F32, 64>(a, st);
        else launch_decode<ea::DT_F32, 128>(a, st);
    }
    return check_launch("decode");
}

size_t entmax_attn_decode_bwd_workspace_size(int B, int H, int H_kv, int Lq, int S, int d, int window) {
    if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || Lq <= 0 || S <= 0 || d <= 0 || window < 0) return 0;
    return dec_bwd_layout(B, H, Lq, S, d, window).total;
}

int entmax_attn_decode_bwd(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens, int causal,
                           int window, const float* tau, const void* dout, float* dq, float* dk, float* dv,
                           void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int Lq, int S, int d,
                           int dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !seqlens || !tau || !dout || !dq || !dk || !dv || !workspace)
        return fail(ENTMAX_ERR_INVALID_ARG,
                    "q, k_cache, v_cache, seqlens, tau, dout, dq, dk, dv and workspace must not be NULL");
    if (misaligned({q, k_cache, v_cache, dout, dq, dk, dv}, 16) || misaligned({seqlens, tau}, 4))
        return fail(ENTMAX_ERR_INVALID_ARG,
                    "q, k_cache, v_cache, dout, dq, dk and dv must be 16-byte aligned, seqlens and tau 4-byte aligned");
    int rc = check_decode(B, H, Hkv, Lq, S, d, dtype, causal, window);
    if (rc) return rc;
    const DecBwdLayout l = dec_bwd_layout(B, H, Lq, S, d, window);
    if (workspace_bytes < l.total)
        return fail(ENTMAX_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, l.total);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(ENTMAX_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    char* ws = static_cast<char*>(workspace);
    ea::DecBwdArgs a;
    ea::DecArgs& f = a.f;
    f.q = q; f.k = k_cache; f.v = v_cache; f.seqlens = seqlens; f.out = nullptr; f.tau_out = nullptr;
    f.sbuf = reinterpret_cast<float*>(ws + l.sbuf);
    f.cmax = reinterpret_cast<float*>(ws + l.cmax);
    f.part = nullptr;
    f.tau = nullptr;
    f.row_len = reinterpret_cast<int*>(ws + l.rlen);
    f.B = B; f.H = H; f.Hkv = Hkv; f.Lq = Lq; f.S = S; f.window = window; f.causal = causal != 0;
    f.nch = l.nch; f.P = l.P;
    f.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
    a.tau = tau; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
    a.dsbuf = reinterpret_cast<float*>(ws + l.dsbuf);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == ENTMAX_BF16) {
        if (d == 64) launch_decode_bwd<ea::DT_BF16, 64>(a, st);
        else launch_decode_bwd<ea::DT_BF16, 128>(a, st);
    } else {
        if (d == 64) launch_decode_bwd<ea::DT_F32, 64>(a, st);
        else launch_decode_bwd<ea::DT_F32, 128>(a, st);
    }
    return check_launch("decode_bwd");
}

const char* entmax_attn_status_string(int status) {
    switch (status) {
        case ENTMAX_OK: return "ok";
        case ENTMAX_ERR_INVALID_ARG: return "invalid argument";
        case ENTMAX_ERR_UNSUPPORTED: return "unsupported configuration";
        case ENTMAX_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* entmax_attn_last_error(void) { return g_err; }

int entmax_attn_version(void) { return 2; }

}  // extern "C"
