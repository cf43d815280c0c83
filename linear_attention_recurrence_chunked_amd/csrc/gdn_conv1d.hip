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
// workgroup of 256 threads covers 8192 consecutive tokens of one channel row
// ([B, C, T] rows are contiguous in T) as four groups of 2048; in each group
// a thread owns 8 consecutive tokens, read and written as one 16-byte vector
// (two on the fp32 path), so a wave's load covers 1 KiB contiguously; all
// four loads are issued before any use (64 bytes per thread in flight). The
// K-1 tokens of history a thread needs are the last ones of the previous
// lane's 8, passed by a DPP whole-wave shift; lane 0 of each wave reads them from
// memory (the previous wave's range: cache hits, except at the first wave of
// a group). The taps are a template parameter so the filter window stays in
// registers. Measured on MI355X at B=4, C=8192, T=8192, bf16: 5.7 TB/s
// (5.4 TB/s for this layout before the DPP shift and the 2-D grid, against
// 5.0 TB/s with each thread's 16 or 32 tokens contiguous); non-temporal
// loads or stores, and two vectors per thread, were slower.
// Decode: one thread per (batch, channel); the window row is read and written
// as one vector where its size allows.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kConvThreads = 256;
constexpr int kConvNE = 8;                         // tokens per vector
constexpr int kConvNV = 4;                         // vectors per thread
constexpr int kConvTile = kConvThreads * kConvNE * kConvNV;  // tokens per workgroup

// x of the previous lane of the wave (0 in lane 0): a DPP whole-wave shift,
// in registers rather than through the LDS crossbar.
__device__ __forceinline__ float lane_shr1(float x) {
    constexpr int kDppWaveShr1 = 0x138;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), kDppWaveShr1, 0xf, 0xf, false));
}

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

// ALIGNED: T % 8 == 0 (every 8-token vector is wholly in range or wholly out
// of it, and rows start 16-byte aligned).
template <typename E, int K, bool ALIGNED>
__global__ __launch_bounds__(kConvThreads) void gdn_conv1d_prefill_kernel(
    const E* __restrict__ x, const float* __restrict__ w, E* __restrict__ out,
    E* __restrict__ state, int C, int T, int tiles, int tile0)
{
    static_assert(K >= 1 && K <= kConvNE, "taps");
    const int row = blockIdx.x;                         // b * C + c
    const int tile = tile0 + (int)blockIdx.y;
    const int c = row % C;
    const int lane = threadIdx.x & 63;
    float wk[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wk[j] = w[(size_t)c * K + j];
    const E* xr = x + (size_t)row * T;
    // vector group v holds tokens tile * kConvTile + 8 (256 v + tid) .. +7: the
    // 64 lanes of a wave cover 1 KiB (bf16) contiguously per load instruction.
    // All groups are loaded before any is used.
    float cur[kConvNV][kConvNE];
#pragma unroll
    for (int v = 0; v < kConvNV; ++v) {
        const int tv = tile * kConvTile + kConvNE * (kConvThreads * v + (int)threadIdx.x);
        const int n = min(kConvNE, T - tv);
        if (n > 0) load8<E, ALIGNED>(xr + tv, n, cur[v]);
        else {
#pragma unroll
            for (int e = 0; e < kConvNE; ++e) cur[v][e] = 0.f;
        }
    }
#pragma unroll
    for (int v = 0; v < kConvNV; ++v) {
        const int tv = tile * kConvTile + kConvNE * (kConvThreads * v + (int)threadIdx.x);
        float prev[kConvNE];
#pragma unroll
        for (int e = 0; e < kConvNE; ++e) prev[e] = lane_shr1(cur[v][e]);
        // lane 0 reads the 8 tokens before its vector from memory, only when
        // that vector is in the row (tv < T, so those 8 are too; a wave past
        // the end of the row must not read beyond it)
        if (lane == 0 && tv < T) {
            if (tv >= kConvNE) load8<E, ALIGNED>(xr + tv - kConvNE, kConvNE, prev);
            else {
#pragma unroll
                for (int e = 0; e < kConvNE; ++e) prev[e] = 0.f;
            }
        }
        const int n = min(kConvNE, T - tv);
        if (n <= 0) continue;                           // (after the shuffle: all lanes take part)
        float o[kConvNE];
#pragma unroll
        for (int e = 0; e < kConvNE; ++e) {
            float y = 0.f;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const int i = e - (K - 1) + j;
                y += wk[j] * (i < 0 ? prev[kConvNE + i] : cur[v][i]);
            }
            o[e] = silu_f(y);
        }
        store8<E, ALIGNED>(out + (size_t)row * T + tv, n, o);
    }
    // Window state: the last K raw tokens of the row (0 before t = 0), copied
    // from x by the first K threads of the workgroup whose tile holds token
    // T - 1 (this workgroup has just read them: cache hits). Picking them out
    // of the registers above would take a runtime index into register arrays,
    // which compiles to compare-and-select chains over every element.
    if (tile == tiles - 1 && (int)threadIdx.x < K) {
        const int j = threadIdx.x, t = T - K + j;
        state[(size_t)row * K + j] = t >= 0 ? xr[t] : from_f32<E>(0.f);
    }
}

// The window row of K elements of E as one vector load/store when it is 4, 8
// or 16 bytes (rows are then naturally aligned), else element by element.
template <typename E, int K>
__device__ __forceinline__ void load_row(const E* p, float (&v)[K]) {
    constexpr int NB = K * (int)sizeof(E);
    if constexpr (NB == 4 || NB == 8 || NB == 16) {
        typedef uint32_t W __attribute__((ext_vector_type(NB / 4)));
        union { W w; E e[K]; } u;
        u.w = *(const W*)p;
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = to_f32(u.e[j]);
    } else {
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = to_f32(p[j]);
    }
}

template <typename E, int K>
__device__ __forceinline__ void store_row(E* p, const float (&v)[K]) {
    constexpr int NB = K * (int)sizeof(E);
    if constexpr (NB == 4 || NB == 8 || NB == 16) {
        typedef uint32_t W __attribute__((ext_vector_type(NB / 4)));
        union { W w; E e[K]; } u;
#pragma unroll
        for (int j = 0; j < K; ++j) u.e[j] = from_f32<E>(v[j]);
        *(W*)p = u.w;
    } else {
#pragma unroll
        for (int j = 0; j < K; ++j) p[j] = from_f32<E>(v[j]);
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
    float old[K], win[K];
    load_row<E, K>(st, old);
#pragma unroll
    for (int j = 0; j + 1 < K; ++j) win[j] = old[j + 1];
    win[K - 1] = to_f32(x[i]);
    float y = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) y += w[(size_t)c * K + j] * win[j];
    out[i] = from_f32<E>(silu_f(y));
    store_row<E, K>(st, win);                          // exact: the values are E
}

// ---------------------------------------------------------------- launch

template <typename E, int K>
static hipError_t conv_prefill_k(const ConvArgs& a, hipStream_t s)
{
    // grid: x = channel row (b * C + c), y = token tile (from tile0)
    constexpr int kMaxGridY = 65535;
    const int tiles = (a.T + kConvTile - 1) / kConvTile;
    const long long rows = (long long)a.B * a.C;
    if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    for (int tile0 = 0; tile0 < tiles; tile0 += kMaxGridY) {   // one launch unless T is huge
        const dim3 grid((unsigned)rows, (unsigned)(tiles - tile0 < kMaxGridY ? tiles - tile0 : kMaxGridY));
        if (a.T % kConvNE == 0)
            hipLaunchKernelGGL((gdn_conv1d_prefill_kernel<E, K, true>), grid, dim3(kConvThreads), 0, s,
                               (const E*)a.x, a.w, (E*)a.out, (E*)a.state, a.C, a.T, tiles, tile0);
        else
            hipLaunchKernelGGL((gdn_conv1d_prefill_kernel<E, K, false>), grid, dim3(kConvThreads), 0, s,
                               (const E*)a.x, a.w, (E*)a.out, (E*)a.state, a.C, a.T, tiles, tile0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
