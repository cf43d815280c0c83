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
// workgroup of 512 threads covers 8192 consecutive tokens of one channel row
// ([B, C, T] rows are contiguous in T) as two groups of 4096; in each group
// a thread owns 8 consecutive tokens, read and written as one 16-byte vector
// (two on the fp32 path), so a wave's load covers 1 KiB contiguously. The
// K-1 tokens of history a thread needs are the last ones of the previous
// lane's 8, passed by a DPP whole-wave shift; lane 0 of each wave reads them
// from memory (the previous wave's range: cache hits). The taps are a
// template parameter so the filter window stays in registers.
// When T % 8 == 0 (every vector wholly in the row or wholly past it) the
// tile kernel does all of this through range-checked buffer loads and stores
// with no branch, so every load of a thread, the history included, is in
// flight before the first use; the row's loads and the output stores carry
// the non-temporal hint. (The general kernel's guarded loads compile to one
// branch per load with a wait inside it.)
// Decode: one thread per (batch, channel); the window row is read and written
// as one vector where its size allows.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kConvThreads = 512;
constexpr int kConvNE = 8;                         // tokens per vector
constexpr int kConvNV = 2;                         // vectors per thread
constexpr int kConvTile = kConvThreads * kConvNE * kConvNV;  // tokens per workgroup

// x of the previous lane of the wave (0 in lane 0): a DPP whole-wave shift,
// in registers rather than through the LDS crossbar.
__device__ __forceinline__ float lane_shr1(float x) {
    constexpr int kDppWaveShr1 = 0x138;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), kDppWaveShr1, 0xf, 0xf, false));
}

// SiLU of y from z = -log2(e) y (the prefill kernels scale their taps by
// -log2(e) once and accumulate z directly), so that the exponential is the
// hardware's base-2 one with no multiply in front of it:
//   silu(y) = y / (1 + e^{-y}) = z / ((1 + 2^z) (-log2(e))),  as -1/ln 2 = -log2(e).
constexpr float kNegLog2e = -1.4426950408889634f;
__device__ __forceinline__ float silu_z(float z) {
    return z * __builtin_amdgcn_rcpf(__builtin_fmaf(__builtin_amdgcn_exp2f(z), kNegLog2e, kNegLog2e));
}

// The elements p[0 .. n-1] of 8 consecutive ones as floats (the others 0),
// and the matching store: element accesses, as p need not be 16-byte aligned
// when T % 8 != 0.
template <typename E>
__device__ __forceinline__ void load8(const E* p, int n, float (&v)[kConvNE]) {
#pragma unroll
    for (int e = 0; e < kConvNE; ++e) v[e] = e < n ? to_f32(p[e]) : 0.f;
}

template <typename E>
__device__ __forceinline__ void store8(E* p, int n, const float (&v)[kConvNE]) {
#pragma unroll
    for (int e = 0; e < kConvNE; ++e)
        if (e < n) p[e] = from_f32<E>(v[e]);
}

// The prefill for any T (the launch uses it when T % 8 != 0; the tile kernel
// below takes T % 8 == 0).
template <typename E, int K>
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
    for (int j = 0; j < K; ++j) wk[j] = kNegLog2e * w[(size_t)c * K + j];
    const E* xr = x + (size_t)row * T;
    // vector group v holds tokens tile * kConvTile + 8 (512 v + tid) .. +7: the
    // 64 lanes of a wave cover 1 KiB (bf16) contiguously per load instruction.
    // All groups are loaded before any is used.
    float cur[kConvNV][kConvNE];
#pragma unroll
    for (int v = 0; v < kConvNV; ++v) {
        const int tv = tile * kConvTile + kConvNE * (kConvThreads * v + (int)threadIdx.x);
        const int n = min(kConvNE, T - tv);
        if (n > 0) load8<E>(xr + tv, n, cur[v]);
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
            if (tv >= kConvNE) load8<E>(xr + tv - kConvNE, kConvNE, prev);
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
            float z = 0.f;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const int i = e - (K - 1) + j;
                z += wk[j] * (i < 0 ? prev[kConvNE + i] : cur[v][i]);
            }
            o[e] = silu_z(z);
        }
        store8<E>(out + (size_t)row * T + tv, n, o);
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

// Fourth word of a raw buffer resource (32-bit data format; no swizzle).
constexpr int kConvBufDword3 = 0x00020000;
// Cache-policy operand of a buffer load or store: non-temporal. The row
// tokens and outputs are each touched once; with the hint on both the tile
// kernel measured 0.165 ms against 0.179-0.181 ms without it on the bench
// workload (B=4, C=8192, T=8192: 82 % against 75 % of the 8 TB/s peak), on
// the stores alone 0.176-0.178 ms, on the loads alone 0.185 ms, and on the
// history loads as well 0.169 ms.
constexpr int kConvNT = 2;
typedef uint32_t cu32x4 __attribute__((ext_vector_type(4)));

// x of the previous lane of the wave, and `old` in lane 0 (a DPP whole-wave
// shift whose lane without a source keeps the old value).
__device__ __forceinline__ float lane_shr1_or(float x, float old) {
    constexpr int kDppWaveShr1 = 0x138;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, old), __builtin_bit_cast(int, x), kDppWaveShr1, 0xf, 0xf, false));
}

// 8 elements of E from NQ = 1 (bf16) or 2 (fp32) 16-byte words.
template <typename E, int NQ>
__device__ __forceinline__ void unpack8(const cu32x4 (&q)[NQ], float (&v)[kConvNE]) {
    if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            v[2 * d] = __builtin_bit_cast(float, q[0][d] << 16);
            v[2 * d + 1] = __builtin_bit_cast(float, q[0][d] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kConvNE; ++e) {
            // (a copy first: the compiler mistranslates a bit cast applied
            // directly to a vector element, reading element 0 instead)
            const uint32_t u = q[e / 4][e % 4];
            v[e] = __builtin_bit_cast(float, u);
        }
    }
}

// The prefill when T % 8 == 0, so that every 8-token vector is wholly inside
// the row or wholly past its end. All loads and stores go through buffer
// resources covering this workgroup's tile (plus the 8 tokens before it), so
// the hardware range check replaces every branch: vectors past the end of
// the row read as zeros and their stores are dropped. Each thread issues its
// four vector loads and the history loads of its wave's first lane (the 8
// tokens before the lane's vector; every other lane gets an offset past the
// range and reads zeros without touching memory) before it uses any of them.
// The history then enters lane 0 as the old value of the DPP shift.
template <typename E, int K>
__global__ __launch_bounds__(kConvThreads) void gdn_conv1d_prefill_tile_kernel(
    const E* __restrict__ x, const float* __restrict__ w, E* __restrict__ out,
    E* __restrict__ state, int C, int T, int tiles, int tile0)
{
    static_assert(K >= 1 && K <= kConvNE, "taps");
    constexpr int ES = (int)sizeof(E);
    constexpr int NQ = kConvNE * ES / 16;               // 16-byte words per vector
    const int row = blockIdx.x;                         // b * C + c
    const int tile = tile0 + (int)blockIdx.y;
    const int c = row % C;
    const int lane = threadIdx.x & 63;
    float wk[K];
#pragma unroll
    for (int j = 0; j < K; ++j) wk[j] = kNegLog2e * w[(size_t)c * K + j];
    const int t0 = tile * kConvTile;
    const int len = min(kConvTile, T - t0);             // tokens of this tile
    const int sh = tile > 0 ? kConvNE : 0;              // tokens of history before it
    const E* xr = x + (size_t)row * T;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(xr + t0 - sh), (short)0, (len + sh) * ES, kConvBufDword3);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(out + (size_t)row * T + t0), (short)0, len * ES, kConvBufDword3);
    cu32x4 raw[kConvNV][NQ], hraw[kConvNV][NQ];
#pragma unroll
    for (int v = 0; v < kConvNV; ++v) {
        const uint32_t off = (uint32_t)((kConvNE * (kConvThreads * v + (int)threadIdx.x) + sh) * ES);
        const uint32_t hoff = lane == 0 ? off - (uint32_t)(kConvNE * ES) : 0x80000000u;
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd) {
            raw[v][qd] = __builtin_bit_cast(cu32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16 * qd, 0, kConvNT));
            hraw[v][qd] = __builtin_bit_cast(cu32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, hoff + 16 * qd, 0, 0));
        }
    }
#pragma unroll
    for (int v = 0; v < kConvNV; ++v) {
        float cur[kConvNE], hist[kConvNE], prev[kConvNE];
        unpack8<E, NQ>(raw[v], cur);
        unpack8<E, NQ>(hraw[v], hist);
#pragma unroll
        for (int e = 0; e < kConvNE; ++e) prev[e] = lane_shr1_or(cur[e], hist[e]);
        float o[kConvNE];
#pragma unroll
        for (int e = 0; e < kConvNE; ++e) {
            float z = 0.f;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const int i = e - (K - 1) + j;
                z += wk[j] * (i < 0 ? prev[kConvNE + i] : cur[i]);
            }
            o[e] = silu_z(z);
        }
        const uint32_t off = (uint32_t)(kConvNE * (kConvThreads * v + (int)threadIdx.x) * ES);
        if constexpr (sizeof(E) == 2) {
            cu32x4 pk;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                typedef float f2 __attribute__((ext_vector_type(2)));
                pk[d] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{o[2 * d], o[2 * d + 1]}, bf2));
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(cu32x4, pk), ro, off, 0, kConvNT);
        } else {
#pragma unroll
            for (int qd = 0; qd < NQ; ++qd)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(cu32x4, f32x4{o[4 * qd], o[4 * qd + 1], o[4 * qd + 2], o[4 * qd + 3]}),
                    ro, off + 16 * qd, 0, kConvNT);
        }
    }
    // Window state, as in the general kernel below.
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
    out[i] = from_f32<E>(silu_z(kNegLog2e * y));
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
            hipLaunchKernelGGL((gdn_conv1d_prefill_tile_kernel<E, K>), grid, dim3(kConvThreads), 0, s,
                               (const E*)a.x, a.w, (E*)a.out, (E*)a.state, a.C, a.T, tiles, tile0);
        else
            hipLaunchKernelGGL((gdn_conv1d_prefill_kernel<E, K>), grid, dim3(kConvThreads), 0, s,
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
