// gdn_norm.hip -- RMSNormGated output epilogue for the prefill output.
//
// The gated RMS norm that the "GDN Block TKG Kernel API Reference" page puts
// after the recurrence (introduction: "RMSNormGated"; Parameters norm_weight,
// the gamma over head_v_dim, and W_in_z, whose projection z is the gate):
//   y = o / sqrt(mean_d(o_d^2) + eps) * gamma_d * silu(z_d),  per (token, head)
// over the head's Dv outputs. The prefill writes o head-major [B, Hv, S, Dv]
// (the "GDN CTE Kernel API Reference" output, un-normalised); z and y are
// token-major [B, S, Hv, Dv], the layout of the block's output and of z's
// projection, so this pass also moves each Dv row to its token-major place.
//
// A stream over HBM (o and z read once, y written once). P lanes own one row
// (P = the power of two covering its 16-byte vectors), the row's sum of
// squares is a butterfly over those lanes, and each row moves as P
// contiguous 16-byte vectors (kNormNR rows per thread, all loaded before any
// is used). A workgroup's rows form a tile of HT heads x consecutive tokens
// (HT = 4 when Hv allows): the head-major
// reads of o then cover runs of consecutive tokens and the token-major z
// and y runs of consecutive heads, rather than one of the two jumping by a
// whole [S, Dv] head plane from row to row.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kNormThreads = 256;

// DPP permutation of x within rows of 16 lanes (GFX9 controls).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum of x over each aligned group of P lanes, in every lane of the group.
// Within a row of 16 lanes the partners come from DPP moves in registers:
// swap neighbours, swap pairs (quad permutations), then mirror the halves of
// 8 and the row of 16, each pairing two partial sums of equal size. Groups of
// 32 add the other row by a lane shuffle.
template <int P>
__device__ __forceinline__ float row_sum(float x) {
    constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
    if constexpr (P >= 2) x += dpp_f32<kQuadSwap1>(x);
    if constexpr (P >= 4) x += dpp_f32<kQuadSwap2>(x);
    if constexpr (P >= 8) x += dpp_f32<kRowHalfMirror>(x);
    if constexpr (P >= 16) x += dpp_f32<kRowMirror>(x);
    if constexpr (P >= 32) x += __shfl_xor(x, 16);
    static_assert(P <= 32, "row width");
    return x;
}
constexpr int kNormNR = 4;          // rows per thread (1, 2 and 8 measured slower)

template <typename E, int P, int HT>
__global__ __launch_bounds__(kNormThreads) void gdn_rmsnorm_gated_kernel(
    const E* __restrict__ o, const E* __restrict__ z, const float* __restrict__ w, float eps,
    E* __restrict__ out, int Hv, int S, int Dv, int b0)
{
    constexpr int VE = 16 / (int)sizeof(E);
    constexpr int RW = kNormThreads / P;               // rows per pass of the workgroup
    constexpr int TT = kNormNR * RW / HT;              // tokens per tile
    typedef typename std::conditional<sizeof(E) == 2, bf16x8, f32x4>::type V;
    const float inv_dv = 1.f / (float)Dv;
    const int li = threadIdx.x % P;
    const int c0 = li * VE;
    // grid: x = token tile, y = head tile, z = batch (from b0)
    const long long st = blockIdx.x, hb = blockIdx.y, b = b0 + (long long)blockIdx.z;
    // kNormNR rows per thread, all loaded before any is used
    V a[kNormNR], g[kNormNR];
    long long row[kNormNR];
    bool act[kNormNR];
#pragma unroll
    for (int n = 0; n < kNormNR; ++n) {
        const int rr = threadIdx.x / P + RW * n;       // row within the tile
        const long long h = hb * HT + rr / TT, s = st * TT + rr % TT;
        act[n] = s < S && c0 < Dv;
        row[n] = (b * S + s) * Hv + h;                 // token-major z / y row
        const long long orow = (b * Hv + h) * S + s;   // head-major o row
        if (act[n]) {
            // o is read by this pass only: a non-temporal load (0.139 -> 0.119 ms
            // with four rows per thread; the same hint on z measured slower)
            a[n] = __builtin_nontemporal_load((const V*)(o + orow * Dv + c0));
            g[n] = *(const V*)(z + row[n] * Dv + c0);
        }
    }
#pragma unroll
    for (int n = 0; n < kNormNR; ++n) {
        float ov[VE], ss = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            ov[e] = act[n] ? to_f32(a[n][e]) : 0.f;
            ss += ov[e] * ov[e];
        }
        ss = row_sum<P>(ss);
        if (!act[n]) continue;
        // 1/sqrt(mean + eps): mean by the reciprocal of Dv (exact for powers of
        // two), hardware reciprocal square root (about 1 ulp)
        const float r = __builtin_amdgcn_rsqf(ss * inv_dv + eps);
        V y;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const float zz = to_f32(g[n][e]);
            // silu(z) with the hardware exponential and reciprocal (relative
            // error ~1e-7, far below the bf16 output rounding and the fp32 checks)
            y[e] = from_f32<E>(ov[e] * r * w[c0 + e] * (zz * __builtin_amdgcn_rcpf(1.f + __expf(-zz))));
        }
        // y is not read again by this pass: a non-temporal store keeps it out
        // of the caches the o and z streams use
        __builtin_nontemporal_store(y, (V*)(out + row[n] * Dv + c0));
    }
}

template <typename E, int P, int HT>
static hipError_t norm_ph(const NormArgs& a, hipStream_t st)
{
    constexpr int TT = kNormNR * kNormThreads / P / HT;
    constexpr int kMaxGridYZ = 65535;
    const int stiles = (a.S + TT - 1) / TT;
    if (a.Hv / HT > kMaxGridYZ) return hipErrorInvalidConfiguration;
    for (int b0 = 0; b0 < a.B; b0 += kMaxGridYZ) {   // one launch unless B > 65535
        const int nb = a.B - b0 < kMaxGridYZ ? a.B - b0 : kMaxGridYZ;
        hipLaunchKernelGGL((gdn_rmsnorm_gated_kernel<E, P, HT>),
                           dim3((unsigned)stiles, (unsigned)(a.Hv / HT), (unsigned)nb),
                           dim3(kNormThreads), 0, st, (const E*)a.o, (const E*)a.z, a.w, a.eps,
                           (E*)a.out, a.Hv, a.S, a.Dv, b0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename E, int P>
static hipError_t norm_p(const NormArgs& a, hipStream_t st)
{
    return a.Hv % 4 == 0 ? norm_ph<E, P, 4>(a, st) : norm_ph<E, P, 1>(a, st);
}

template <typename E>
static hipError_t norm_e(const NormArgs& a, hipStream_t st)
{
    constexpr int VE = 16 / (int)sizeof(E);
    const int nv = a.Dv / VE;                          // vectors per row (Dv % 16 == 0)
    if (nv <= 2) return norm_p<E, 2>(a, st);
    if (nv <= 4) return norm_p<E, 4>(a, st);
    if (nv <= 8) return norm_p<E, 8>(a, st);
    if (nv <= 16) return norm_p<E, 16>(a, st);
    return norm_p<E, 32>(a, st);
}

hipError_t launch_rmsnorm_gated(const NormArgs& a, int dtype, hipStream_t stream)
{
    return dtype == 1 ? norm_e<bf16>(a, stream) : norm_e<float>(a, stream);
}

}  // namespace gdn
