// gdn_launch.h -- internal host-side launchers behind the C ABI (include/gdn.h).
// Arguments have been validated by the caller (gdn_api.cpp) when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

// With gated = false g_log and beta are the per-token decay and write
// strength and q, k arrive L2-normalised; with gated = true g_log and beta
// carry the raw gate inputs a and b, q and k are raw, and the kernels apply
// the prologue with A_log, dt_bias [Hv] and l2_eps (unused otherwise).
struct PrefillArgs {
    const void* q; const void* k; const void* v;
    const float* g_log; const float* beta; float scale;
    float* state; void* out;
    int B, Hk, Hv, S, Dk, Dv;
    bool gated;
    const float* A_log; const float* dt_bias; float l2_eps;
    int inverse = 0;   // 0: blocked substitution, 1: Neumann product (ungated only)
};

struct DecodeArgs {
    const void* q; const void* k; const void* v;
    const float* g_log; const float* beta; float scale;
    float* state; void* out;
    int B, Hk, Hv, Dk, Dv;
    bool gated;
    const float* A_log; const float* dt_bias; float l2_eps;
};

// Depthwise conv1d: x [B, C, T] (decode: [B, C]), w [C, K] fp32, out like x,
// state [B, C, K] (prefill: written; decode: in and out); 1 <= K <= 8.
struct ConvArgs {
    const void* x; const float* w; void* out; void* state;
    int B, C, T, K;
};

// Decode block extras: mixed [B, C] raw token (C = 2 Hk Dk + Hv Dv), z
// [B, Hv Dv], conv windows [B, C, K] in and out, conv_w [C, K], norm_w [Dv].
struct BlockArgs {
    const void* mixed; const void* z; const void* conv_in; void* conv_out;
    const float* conv_w; const float* norm_w; float norm_eps; int K;
};

// RMSNormGated over rows of Dv: o [B, Hv, S, Dv] (head-major), z and out
// [B, S, Hv, Dv] (token-major), w [Dv].
struct NormArgs {
    const void* o; const void* z; const float* w; float eps; void* out;
    int B, Hv, S, Dv;
};

// dtype: 0 = fp32 operands, 1 = bf16 operands (gdn_dtype).
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int dtype, hipStream_t stream);
hipError_t launch_conv1d(const ConvArgs& a, int dtype, bool decode, hipStream_t stream);
hipError_t launch_decode_block(const DecodeArgs& a, const BlockArgs& blk, int dtype,
                               hipStream_t stream);
hipError_t launch_rmsnorm_gated(const NormArgs& a, int dtype, hipStream_t stream);

}  // namespace gdn
