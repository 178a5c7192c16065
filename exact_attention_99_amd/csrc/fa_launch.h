// Internal launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa355 {

// Attention dropout: keep iff the element's Philox byte < t8; kept values
// scaled by 256 / t8 (see the device helpers in fa_common.h).
struct DropParams {
    uint64_t seed;
    uint64_t offset;
    int t8;        // 1..256
    float scale;   // 256 / t8
};

// General masked path (block-sparse and variable-length attention).  When
// mask is set, query i sees key j only if mask[h_m][i / 128][j / 128] != 0,
// h_m = 0 when heads == 1, else the query head; nb = ceil(N / 128).  When
// seqlens is set, batch element b has seqlens[b] valid positions (clamped to
// [0, N]); later queries and keys are padding (zero output, lse -inf, no
// gradient).
struct SparseParams {
    const unsigned char* mask;
    int heads;
    int nb;
    const int* seqlens;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, N, d;
    int causal;
    float cl2;       // scale * log2(e)
    int dtype;       // fa_dtype value
    int drop;        // 1: apply dropout with dp
    DropParams dp;
    int sparse;      // 1: apply the block mask sp
    SparseParams sp;
    hipStream_t stream;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;    // [B, Hq, N] float32 workspace: D_i = sum_k dO_ik O_ik
    int B, Hq, Hkv, N, d;
    int causal;
    float scale;
    float cl2;
    int dtype;
    int drop;        // 1: apply dropout with dp
    DropParams dp;
    int sparse;      // 1: apply the block mask sp
    SparseParams sp;
    hipStream_t stream;
};

struct SplitArgs {
    const void* q;   // [B, Hq, Nq, d]
    const void* k;   // [B, Hkv, Nkv, d]
    const void* v;
    void* o;         // [B, Hq, Nq, d]
    float* lse;      // [B, Hq, Nq]
    float* opart;    // [nsplit, B*Hq*Nq, d] float32 partial outputs (workspace)
    float* lpart;    // [nsplit, B*Hq*Nq] float32 partial logsumexps (workspace)
    int B, Hq, Hkv, Nq, Nkv, d;
    int causal;
    int nsplit;      // key chunks
    int chunk;       // keys per chunk (a multiple of the kernel's key tile)
    float cl2;
    int dtype;
    hipStream_t stream;
};

struct Fp8QuantArgs {
    const void* x;       // [B, H, N, d] bf16 / fp16
    const float* signs;  // [d] rotation signs, or null for no rotation
    uint8_t* codes;      // [B, H, N, d] e4m3
    float* scales;       // [B, H, ceil(N / 64)]
    int B, H, N, d;
    float rs;            // fp32(1 / sqrt(d))
    int dtype;
    hipStream_t stream;
};

struct Fp8FwdArgs {
    const uint8_t* q;    // [B, Hq, N, d] e4m3
    const uint8_t* k;    // [B, Hkv, N, d]
    const uint8_t* v;
    const float* sq;     // [B, Hq, ceil(N / 64)] block scales
    const float* sk;     // [B, Hkv, ceil(N / 64)]
    const float* sv;
    void* o;             // [B, Hq, N, d] out_dtype
    float* lse;          // [B, Hq, N]
    int B, Hq, Hkv, N, d;
    int causal;
    float cl2;
    int out_dtype;
    hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
// FP8 path: block quantizer and the e4m3 forward.
hipError_t launch_fp8_quantize(const Fp8QuantArgs& a);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a);
// Split-KV forward: partials per key chunk, then the merge.
hipError_t launch_fwd_split(const SplitArgs& a);
// Keys per tile of the split-KV kernel at head dimension d.
int split_tile_keys(int d);
// Backward phases; each reads only the BwdArgs fields it needs.
hipError_t launch_bwd_prepare(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace fa355
