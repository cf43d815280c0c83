// gdn_conv1d.hip -- depthwise causal conv1d + SiLU and its window state.
//
// The step ahead of the gated delta rule on the "GDN Conv1D Kernel API
// Reference" page: every channel of the raw mixed q|k|v tensor is an
// independent K-tap FIR (Notes: depthwise, groups == C), the output is
// silu(conv) and the state is the last K raw tokens (introduction).
//
//   prefill: y[b,c,t] = sum_j w[c,j] x[b,c,t-(K-1)+j]  (x = 0 before t = 0)
//            out = silu(y) = y / (1 + e^{-y});  state[b,c,j] = x[b,c,T-K+j]
//   decode:  window = (state[b,c,1..K-1], x[b,c]);  out = silu(sum_j w[c,j] window_j);
//            state <- window (in place)
//
// Both are streams over HBM with a handful of flops per byte. Prefill: one
// workgroup of 256 threads covers 2048 consecutive tokens of one channel row
// ([B, C, T] rows are contiguous in T); each thread owns 8 consecutive
// tokens, read and written as 16-byte vectors (two on the fp32 path). The
// K-1 tokens of history a thread needs are the last ones of the previous
// lane's 8, passed by a lane shuffle; lane 0 of each wave reads them from
// memory (they belong to the previous wave's range and are cache hits, except
// at the first wave of a workgroup). The taps are a template parameter so the
// filter window stays in registers.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kConvThreads = 256;
constexpr int kConvNE = 8;                         // tokens per thread
constexpr int kConvTile = kConvThreads * kConvNE;  // tokens per workgroup

__device__ __forceinline__ float silu_f(float y) {
    return y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
}

// 8 consecutive elements as floats; ALIGNED: p is 16-byte aligned and all 8
// are in range, else element loads of those with index < n (others 0).
template <typename E, bool ALIGNED>
__device__ __forceinline__ void load8(const E* p, int n, float (&v)[kConvNE]) {
    if constexpr (ALIGNED) {
        if constexpr (sizeof(E) == 2) {
            const bf16x8 a = *(const bf16x8*)p;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
        } else {
            const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
        }
    } else {
#pragma unroll
        for (int e = 0; e < kConvNE; ++e) v[e] = e < n ? to_f32(p[e]) : 0.f;
    }
}

template <typename E, bool ALIGNED>
__device__ __forceinline__ void store8(E* p, int n, const float (&v)[kConvNE]) {
    if constexpr (ALIGNED) {
        if constexpr (sizeof(E) == 2) {
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (bf16)v[e];
            *(bf16x8*)p = a;
        } else {
            *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
            *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
    } else {
#pragma unroll
        for (int e = 0; e < kConvNE; ++e)
            if (e < n) p[e] = from_f32<E>(v[e]);
    }
}

// ALIGNED: T % 8 == 0 (every thread's 8 tokens are in range or all out of it,
// and rows start 16-byte aligned).
template <typename E, int K, bool ALIGNED>
__global__ __launch_bounds__(kConvThreads) void gdn_conv1d_prefill_kernel(
    const E* __restrict__ x, const float* __restrict__ w, E* __restrict__ out,
    E* __restrict__ state, int C, int T, int tiles)
{
    static_assert(K >= 1 && K <= kConvNE, "taps");
    const int row = blockIdx.x / tiles;                 // b * C + c
    const int tile = blockIdx.x - row * tiles;
    const int c = row % C;
    const int lane = threadIdx.x & 63;
    float wk[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wk[j] = w[(size_t)c * K + j];

    const E* xr = x + (size_t)row * T;
    const int t0 = tile * kConvTile + kConvNE * (int)threadIdx.x;
    const int n = min(kConvNE, T - t0);                 // tokens of this thread in range
    float cur[kConvNE];
    if (n > 0) load8<E, ALIGNED>(xr + t0, n, cur);
    else {
#pragma unroll
        for (int e = 0; e < kConvNE; ++e) cur[e] = 0.f;
    }
    // history: the previous 8 tokens (only the last K-1 are used)
    float prev[kConvNE];
#pragma unroll
    for (int e = 0; e < kConvNE; ++e) prev[e] = __shfl_up(cur[e], 1);
    if (lane == 0) {
        if (t0 >= kConvNE) load8<E, ALIGNED>(xr + t0 - kConvNE, kConvNE, prev);
        else {
#pragma unroll
            for (int e = 0; e < kConvNE; ++e) prev[e] = 0.f;
        }
    }
    if (n <= 0) return;

    float o[kConvNE];
#pragma unroll
    for (int e = 0; e < kConvNE; ++e) {
        float y = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int i = e - (K - 1) + j;              // token t0 + i
            y += wk[j] * (i < 0 ? prev[kConvNE + i] : cur[i]);
        }
        o[e] = silu_f(y);
    }
    store8<E, ALIGNED>(out + (size_t)row * T + t0, n, o);

    // state: the thread holding token T-1 writes the last K raw tokens
    if (t0 <= T - 1 && T - 1 < t0 + kConvNE) {
        E* st = state + (size_t)row * K;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int i = T - K + j - t0;               // in [-8, 8)
            const int t = T - K + j;
            float vj = 0.f;
#pragma unroll
            for (int e = 0; e < kConvNE; ++e) {
                if (i == e) vj = cur[e];
                if (i == e - kConvNE) vj = prev[e];
            }
            st[j] = from_f32<E>(t >= 0 ? vj : 0.f);
        }
    }
}

template <typename E, int K>
__global__ __launch_bounds__(kConvThreads) void gdn_conv1d_decode_kernel(
    const E* __restrict__ x, const float* __restrict__ w, E* __restrict__ state,
    E* __restrict__ out, int C, long long total)
{
    const long long i = (long long)blockIdx.x * kConvThreads + threadIdx.x;   // b * C + c
    if (i >= total) return;
    const int c = (int)(i % C);
    E* st = state + i * K;
    float win[K];
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) win[j] = to_f32(st[j + 1]);
    win[K - 1] = to_f32(x[i]);
    float y = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) y += w[(size_t)c * K + j] * win[j];
    out[i] = from_f32<E>(silu_f(y));
#pragma unroll
    for (int j = 0; j < K; ++j) st[j] = from_f32<E>(win[j]);   // exact: values are E
}

// ---------------------------------------------------------------- launch

template <typename E, int K>
static hipError_t conv_prefill_k(const ConvArgs& a, hipStream_t s)
{
    const int tiles = (a.T + kConvTile - 1) / kConvTile;
    const long long blocks = (long long)a.B * a.C * tiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.T % kConvNE == 0)
        hipLaunchKernelGGL((gdn_conv1d_prefill_kernel<E, K, true>), dim3((unsigned)blocks),
                           dim3(kConvThreads), 0, s, (const E*)a.x, a.w, (E*)a.out,
                           (E*)a.state, a.C, a.T, tiles);
    else
        hipLaunchKernelGGL((gdn_conv1d_prefill_kernel<E, K, false>), dim3((unsigned)blocks),
                           dim3(kConvThreads), 0, s, (const E*)a.x, a.w, (E*)a.out,
                           (E*)a.state, a.C, a.T, tiles);
    return hipGetLastError();
}

template <typename E, int K>
static hipError_t conv_decode_k(const ConvArgs& a, hipStream_t s)
{
    const long long total = (long long)a.B * a.C;
    const long long blocks = (total + kConvThreads - 1) / kConvThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_conv1d_decode_kernel<E, K>), dim3((unsigned)blocks),
                       dim3(kConvThreads), 0, s, (const E*)a.x, a.w, (E*)a.state, (E*)a.out,
                       a.C, total);
    return hipGetLastError();
}

template <typename E>
static hipError_t conv_dispatch(const ConvArgs& a, bool decode, hipStream_t s)
{
#define GDN_CONV_CASE(KK) \
    case KK: return decode ? conv_decode_k<E, KK>(a, s) : conv_prefill_k<E, KK>(a, s);
    switch (a.K) {
        GDN_CONV_CASE(1) GDN_CONV_CASE(2) GDN_CONV_CASE(3) GDN_CONV_CASE(4)
        GDN_CONV_CASE(5) GDN_CONV_CASE(6) GDN_CONV_CASE(7) GDN_CONV_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef GDN_CONV_CASE
}

hipError_t launch_conv1d(const ConvArgs& a, int dtype, bool decode, hipStream_t stream)
{
    return dtype == 1 ? conv_dispatch<bf16>(a, decode, stream)
                      : conv_dispatch<float>(a, decode, stream);
}

}  // namespace gdn
