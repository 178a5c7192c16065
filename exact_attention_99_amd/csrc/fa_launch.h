// Internal launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa355 {

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
    int fwd_variant; // tile variant of the 16-bit kernel (0 = default)
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
    int variant;     // kernel generation of the 16-bit passes (0 = default)
    hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
// Backward phases; each reads only the BwdArgs fields it needs.
hipError_t launch_bwd_prepare(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);

}  // namespace fa355
