// C-ABI entry points of libfa355: argument checks, workspace layout and
// dispatch to the kernels.  Declared in include/fa355.h.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "fa355.h"
#include "fa_launch.h"

namespace {

constexpr float kLog2eHost = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

bool sizes_ok(int B, int Hq, int Hkv, int N) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return false;
    if (Hq % Hkv != 0) return false;
    // Block counts must fit a grid, and one head's rows (at 4 bytes per
    // element, d <= 128) must be addressable with 32-bit byte offsets.
    const long long rows = (long long)B * Hq * ((N + 31) / 32);
    return rows < (1LL << 31) && (long long)N * 128 * 4 < (1LL << 31);
}

bool dtype_ok(fa_dtype t) { return t == FA_DTYPE_FP32 || t == FA_DTYPE_FP16 || t == FA_DTYPE_BF16; }

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H_q,
                 int H_kv, int N, int d, int causal, float scale, fa_dtype dtype,
                 hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H_q, H_kv, N)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;

    fa355::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = H_q; a.Hkv = H_kv; a.N = N; a.d = d;
    a.causal = causal;
    a.cl2 = scale * kLog2eHost;
    a.dtype = (int)dtype;
    a.drop = 0;
    a.dp = fa355::DropParams{0, 0, 256, 1.f};
    a.sparse = 0;
    a.sp = fa355::SparseParams{nullptr, 1, 0, nullptr};
    a.stream = stream;
    return fa355::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// Keep threshold t8 = round((1 - p) 256) of a dropout probability; 0 when p
// is outside [0, 1) or leaves no byte below the threshold.
int drop_threshold(float p) {
    if (!(p >= 0.f) || !(p < 1.f)) return 0;
    const int t = (int)floor((1.0 - (double)p) * 256.0 + 0.5);
    return t >= 1 ? t : 0;
}

}  // namespace

fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H_q, int H_kv, int N, int d, int causal, float scale, float dropout_p,
                         unsigned long long seed, unsigned long long offset, fa_dtype dtype,
                         hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H_q, H_kv, N)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
    const int t8 = drop_threshold(dropout_p);
    if (t8 == 0) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;

    fa355::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = H_q; a.Hkv = H_kv; a.N = N; a.d = d;
    a.causal = causal;
    a.cl2 = scale * kLog2eHost;
    a.dtype = (int)dtype;
    a.drop = 1;
    a.dp = fa355::DropParams{seed, offset, t8, 256.f / (float)t8};
    a.sparse = 0;
    a.sp = fa355::SparseParams{nullptr, 1, 0, nullptr};
    a.stream = stream;
    return fa355::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             const unsigned char* block_mask, int mask_heads, int B, int H_q,
                             int H_kv, int N, int d, int causal, float scale, fa_dtype dtype,
                             hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !block_mask) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H_q, H_kv, N)) return FA_ERR_INVALID_ARG;
    if (mask_heads != 1 && mask_heads != H_q) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;

    fa355::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = H_q; a.Hkv = H_kv; a.N = N; a.d = d;
    a.causal = causal;
    a.cl2 = scale * kLog2eHost;
    a.dtype = (int)dtype;
    a.drop = 0;
    a.dp = fa355::DropParams{0, 0, 256, 1.f};
    a.sparse = 1;
    a.sp = fa355::SparseParams{block_mask, mask_heads, (N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK, nullptr};
    a.stream = stream;
    return fa355::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H_q, int H_kv, int N, int d, fa_dtype dtype) {
    if (!sizes_ok(B, H_q, H_kv, N) || !dtype_ok(dtype) || (d != 64 && d != 128)) return 0;
    const size_t rows = (size_t)B * H_q * N;
    return round256(rows * sizeof(float));
}

namespace {

fa_status check_common(int B, int H_q, int H_kv, int N, int d, int causal, float scale,
                       fa_dtype dtype) {
    if (!sizes_ok(B, H_q, H_kv, N)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

bool ptrs_ok(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p || !aligned16(p)) return false;
    return true;
}

fa355::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* delta, int B, int H_q, int H_kv, int N, int d, int causal,
                        float scale, fa_dtype dtype, hipStream_t stream) {
    fa355::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.delta = delta;
    a.B = B; a.Hq = H_q; a.Hkv = H_kv; a.N = N; a.d = d;
    a.causal = causal;
    a.scale = scale;
    a.cl2 = scale * kLog2eHost;
    a.dtype = (int)dtype;
    a.drop = 0;
    a.dp = fa355::DropParams{0, 0, 256, 1.f};
    a.sparse = 0;
    a.sp = fa355::SparseParams{nullptr, 1, 0, nullptr};
    a.stream = stream;
    return a;
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

}  // extern "C"

namespace {

bool split_sizes_ok(int B, int H_q, int H_kv, int N_q, int N_kv) {
    if (B < 1 || H_q < 1 || H_kv < 1 || N_q < 1 || N_kv < 1) return false;
    if (H_q % H_kv != 0) return false;
    const long long G = H_q / H_kv;
    // one K/V head and one group of stacked query rows must be addressable with
    // 32-bit byte offsets, and the grid must fit
    return (long long)N_kv * 128 * 2 < (1LL << 31) && G * N_q * 128 * 2 < (1LL << 31) &&
           (long long)B * H_kv < (1LL << 31) && (long long)B * H_q * N_q < (1LL << 31);
}

size_t split_parts_bytes(int B, int H_q, int N_q, int d, int num_splits) {
    const size_t rows = (size_t)B * H_q * N_q;
    return round256((size_t)num_splits * rows * d * sizeof(float));
}

}  // namespace

extern "C" {

int fa_fwd_splitkv_default_splits(int B, int H_q, int H_kv, int N_q, int N_kv, int d) {
    if (!split_sizes_ok(B, H_q, H_kv, N_q, N_kv) || (d != 64 && d != 128)) return 0;
    const long long G = H_q / H_kv;
    const long long groups = (long long)B * H_kv * ((G * N_q + 31) / 32);
    // about two one-wave workgroups per compute unit of a 256-unit device
    // (the rate of the decoding shapes peaks there: more, smaller chunks only
    // add partials for the merge to read), chunks of at least four key tiles
    const long long want = (512 + groups - 1) / groups;
    const long long tile = fa355::split_tile_keys(d);
    const long long most = (N_kv + 4 * tile - 1) / (4 * tile);
    long long n = want < most ? want : most;
    if (n < 1) n = 1;
    if (n > 1024) n = 1024;
    return (int)n;
}

size_t fa_fwd_splitkv_workspace_size(int B, int H_q, int N_q, int d, int num_splits) {
    if (B < 1 || H_q < 1 || N_q < 1 || num_splits < 1 || num_splits > 1024 || (d != 64 && d != 128))
        return 0;
    const size_t rows = (size_t)B * H_q * N_q;
    return split_parts_bytes(B, H_q, N_q, d, num_splits) + round256((size_t)num_splits * rows * sizeof(float));
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, int B, int H_q, int H_kv,
                         int N_q, int N_kv, int d, int causal, float scale, int num_splits,
                         fa_dtype dtype, hipStream_t stream) {
    if (!ptrs_ok({q, k, v, o, lse, workspace})) return FA_ERR_INVALID_ARG;
    if (!split_sizes_ok(B, H_q, H_kv, N_q, N_kv)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (causal && N_q > N_kv) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > 1024) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
    const size_t need = fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits);
    if (workspace_bytes < need) return FA_ERR_INVALID_ARG;

    fa355::SplitArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.opart = static_cast<float*>(workspace);
    a.lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       split_parts_bytes(B, H_q, N_q, d, num_splits));
    a.B = B; a.Hq = H_q; a.Hkv = H_kv; a.Nq = N_q; a.Nkv = N_kv; a.d = d;
    a.causal = causal;
    a.nsplit = num_splits;
    const int tile = fa355::split_tile_keys(d);
    const int per = (N_kv + num_splits - 1) / num_splits;
    a.chunk = (per + tile - 1) / tile * tile;
    a.cl2 = scale * kLog2eHost;
    a.dtype = (int)dtype;
    a.stream = stream;
    return hip_status(fa355::launch_fwd_split(a));
}

fa_status fa_bwd_prepare(const void* o, const void* dout, float* delta, int B, int H_q, int N,
                         int d, fa_dtype dtype, hipStream_t stream) {
    if (!ptrs_ok({o, dout, delta})) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_q, N, d, 0, 1.f, dtype);
    if (st != FA_OK) return st;
    const auto a = bwd_args(nullptr, nullptr, nullptr, o, nullptr, dout, nullptr, nullptr, nullptr,
                            delta, B, H_q, H_q, N, d, 0, 1.f, dtype, stream);
    return hip_status(fa355::launch_bwd_prepare(a));
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                      const void* dout, const float* delta, void* dk, void* dv, int B, int H_q,
                      int H_kv, int N, int d, int causal, float scale, fa_dtype dtype,
                      hipStream_t stream) {
    if (!ptrs_ok({q, k, v, lse, dout, delta, dk, dv})) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    const auto a = bwd_args(q, k, v, nullptr, lse, dout, nullptr, dk, dv, const_cast<float*>(delta),
                            B, H_q, H_kv, N, d, causal, scale, dtype, stream);
    return hip_status(fa355::launch_bwd_dkdv(a));
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                    const void* dout, const float* delta, void* dq, int B, int H_q, int H_kv,
                    int N, int d, int causal, float scale, fa_dtype dtype, hipStream_t stream) {
    if (!ptrs_ok({q, k, v, lse, dout, delta, dq})) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    const auto a = bwd_args(q, k, v, nullptr, lse, dout, dq, nullptr, nullptr,
                            const_cast<float*>(delta), B, H_q, H_kv, N, d, causal, scale, dtype,
                            stream);
    return hip_status(fa355::launch_bwd_dq(a));
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int H_q, int H_kv, int N, int d, int causal,
                 float scale, fa_dtype dtype, hipStream_t stream) {
    if (!ptrs_ok({q, k, v, o, lse, dout, dq, dk, dv, workspace})) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    if (workspace_bytes < fa_bwd_workspace_size(B, H_q, H_kv, N, d, dtype)) return FA_ERR_INVALID_ARG;
    const auto a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B,
                            H_q, H_kv, N, d, causal, scale, dtype, stream);
    hipError_t e = fa355::launch_bwd_prepare(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dkdv(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dq(a);
    return hip_status(e);
}
}  // extern "C"

namespace {

// Scratch of fa_bwd_noalloc: the D row terms that fa_bwd keeps in its
// workspace.  One copy per device, held until the process ends.  In host code
// the name stands for a host-side shadow, not a device address: kernels and
// copies take the address scratch_ptr() returns.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

// Device address of the scratch array on the current device, looked up once
// per device with that device current (null if the lookup fails).
void* scratch_ptr() {
    static std::atomic<void*> ptrs[64];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = ptrs[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = ptrs[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptrs[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                         int H_q, int H_kv, int N, int d, int causal, float scale, fa_dtype dtype,
                         hipStream_t stream) {
    if (!ptrs_ok({q, k, v, o, lse, dout, dq, dk, dv})) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    if (fa_bwd_workspace_size(B, H_q, H_kv, N, d, dtype) > FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_TOO_LARGE;
    void* ws = scratch_ptr();
    if (!ws) return FA_ERR_HIP;
    const auto a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(ws), B, H_q,
                            H_kv, N, d, causal, scale, dtype, stream);
    hipError_t e = fa355::launch_bwd_prepare(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dkdv(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dq(a);
    return hip_status(e);
}


fa_status fa_fp8_quantize(const void* x, const float* signs, unsigned char* codes, float* scales,
                          int B, int H, int N, int d, fa_dtype dtype, hipStream_t stream) {
    if (!ptrs_ok({x, codes}) || !scales || (reinterpret_cast<uintptr_t>(scales) & 3u)) return FA_ERR_INVALID_ARG;
    if (signs && !aligned16(signs)) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, H, N) || !dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
    fa355::Fp8QuantArgs a;
    a.x = x; a.signs = signs; a.codes = codes; a.scales = scales;
    a.B = B; a.H = H; a.N = N; a.d = d;
    a.rs = (float)(1.0 / sqrt((double)d));
    a.dtype = (int)dtype;
    a.stream = stream;
    return hip_status(fa355::launch_fp8_quantize(a));
}

fa_status fa_fwd_fp8(const unsigned char* q, const unsigned char* k, const unsigned char* v, const float* q_scale,
                     const float* k_scale, const float* v_scale, void* o, float* lse, int B,
                     int H_q, int H_kv, int N, int d, int causal, float scale, fa_dtype out_dtype,
                     hipStream_t stream) {
    if (!ptrs_ok({q, k, v, o, lse})) return FA_ERR_INVALID_ARG;
    for (const float* p : {q_scale, k_scale, v_scale})
        if (!p || (reinterpret_cast<uintptr_t>(p) & 3u)) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, out_dtype);
    if (st != FA_OK) return st;
    if (out_dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
    fa355::Fp8FwdArgs a;
    a.q = q; a.k = k; a.v = v;
    a.sq = q_scale; a.sk = k_scale; a.sv = v_scale;
    a.o = o; a.lse = lse;
    a.B = B; a.Hq = H_q; a.Hkv = H_kv; a.N = N; a.d = d;
    a.causal = causal;
    a.cl2 = scale * kLog2eHost;
    a.out_dtype = (int)out_dtype;
    a.stream = stream;
    return hip_status(fa355::launch_fwd_fp8(a));
}

fa_status fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, int B, int H_q, int H_kv, int N,
                         int d, int causal, float scale, float dropout_p, unsigned long long seed,
                         unsigned long long offset, fa_dtype dtype, hipStream_t stream) {
    if (!ptrs_ok({q, k, v, o, lse, dout, dq, dk, dv, workspace})) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    const int t8 = drop_threshold(dropout_p);
    if (t8 == 0) return FA_ERR_INVALID_ARG;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
    if (workspace_bytes < fa_bwd_workspace_size(B, H_q, H_kv, N, d, dtype)) return FA_ERR_INVALID_ARG;
    auto a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, H_q,
                      H_kv, N, d, causal, scale, dtype, stream);
    a.drop = 1;
    a.dp = fa355::DropParams{seed, offset, t8, 256.f / (float)t8};
    hipError_t e = fa355::launch_bwd_prepare(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dkdv(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dq(a);
    return hip_status(e);
}

fa_status fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             const unsigned char* block_mask, int mask_heads, int B, int H_q,
                             int H_kv, int N, int d, int causal, float scale, fa_dtype dtype,
                             hipStream_t stream) {
    if (!ptrs_ok({q, k, v, o, lse, dout, dq, dk, dv, workspace}) || !block_mask)
        return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    if (mask_heads != 1 && mask_heads != H_q) return FA_ERR_INVALID_ARG;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
    if (workspace_bytes < fa_bwd_workspace_size(B, H_q, H_kv, N, d, dtype)) return FA_ERR_INVALID_ARG;
    auto a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, H_q,
                      H_kv, N, d, causal, scale, dtype, stream);
    a.sparse = 1;
    a.sp = fa355::SparseParams{block_mask, mask_heads, (N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK, nullptr};
    hipError_t e = fa355::launch_bwd_prepare(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dkdv(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dq(a);
    return hip_status(e);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* seqlens, int B, int H_q, int H_kv, int N, int d, int causal,
                        float scale, fa_dtype dtype, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !seqlens) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(seqlens) & 3u) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H_q, H_kv, N)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;

    fa355::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.Hq = H_q; a.Hkv = H_kv; a.N = N; a.d = d;
    a.causal = causal;
    a.cl2 = scale * kLog2eHost;
    a.dtype = (int)dtype;
    a.drop = 0;
    a.dp = fa355::DropParams{0, 0, 256, 1.f};
    a.sparse = 1;
    a.sp = fa355::SparseParams{nullptr, 1, 0, seqlens};
    a.stream = stream;
    return fa355::launch_fwd(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, const int* seqlens, int B,
                        int H_q, int H_kv, int N, int d, int causal, float scale, fa_dtype dtype,
                        hipStream_t stream) {
    if (!ptrs_ok({q, k, v, o, lse, dout, dq, dk, dv, workspace}) || !seqlens) return FA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(seqlens) & 3u) return FA_ERR_INVALID_ARG;
    const fa_status st = check_common(B, H_q, H_kv, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
    if (workspace_bytes < fa_bwd_workspace_size(B, H_q, H_kv, N, d, dtype)) return FA_ERR_INVALID_ARG;
    auto a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, H_q,
                      H_kv, N, d, causal, scale, dtype, stream);
    a.sparse = 1;
    a.sp = fa355::SparseParams{nullptr, 1, 0, seqlens};
    hipError_t e = fa355::launch_bwd_prepare(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dkdv(a);
    if (e == hipSuccess) e = fa355::launch_bwd_dq(a);
    return hip_status(e);
}

const char* fa_status_string(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK: success";
        case FA_ERR_INVALID_ARG:
            return "FA_ERR_INVALID_ARG: null or misaligned pointer, bad size, flag or scale, "
                   "or workspace too small";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim or dtype not built";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime refused a kernel launch";
        case FA_ERR_TOO_LARGE:
            return "FA_ERR_TOO_LARGE: the problem needs more than the fixed scratch of "
                   "fa_bwd_noalloc (FA_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown fa_status";
}

int fa_version(void) { return 100; }

}  // extern "C"
