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
// contiguous 16-byte vectors.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kNormThreads = 256;

template <typename E, int P>
__global__ __launch_bounds__(kNormThreads) void gdn_rmsnorm_gated_kernel(
    const E* __restrict__ o, const E* __restrict__ z, const float* __restrict__ w, float eps,
    E* __restrict__ out, int Hv, int S, int Dv, long long rows)
{
    constexpr int VE = 16 / (int)sizeof(E);
    typedef typename std::conditional<sizeof(E) == 2, bf16x8, f32x4>::type V;
    const long long row = (long long)blockIdx.x * (kNormThreads / P) + threadIdx.x / P;
    const int li = threadIdx.x % P;
    const int c0 = li * VE;
    const bool act = row < rows && c0 < Dv;
    // token-major output row (b, s, h) <- head-major input row (b, h, s)
    const long long hs = row % ((long long)S * Hv), b = row / ((long long)S * Hv);
    const long long s = hs / Hv, h = hs % Hv;
    const long long orow = (b * Hv + h) * S + s;
    float ov[VE], zv[VE];
    float ss = 0.f;
    if (act) {
        const V a = *(const V*)(o + orow * Dv + c0);
        const V g = *(const V*)(z + row * Dv + c0);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            ov[e] = to_f32(a[e]);
            zv[e] = to_f32(g[e]);
            ss += ov[e] * ov[e];
        }
    }
#pragma unroll
    for (int m = 1; m < P; m <<= 1) ss += __shfl_xor(ss, m);
    if (!act) return;
    const float r = 1.f / sqrtf(ss / (float)Dv + eps);
    V y;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const float gate = zv[e] / (1.f + expf(-zv[e]));
        y[e] = from_f32<E>(ov[e] * r * w[c0 + e] * gate);
    }
    *(V*)(out + row * Dv + c0) = y;
}

template <typename E, int P>
static hipError_t norm_p(const NormArgs& a, hipStream_t st)
{
    const long long rows = (long long)a.B * a.S * a.Hv;
    const long long blocks = (rows + kNormThreads / P - 1) / (kNormThreads / P);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_rmsnorm_gated_kernel<E, P>), dim3((unsigned)blocks),
                       dim3(kNormThreads), 0, st, (const E*)a.o, (const E*)a.z, a.w, a.eps,
                       (E*)a.out, a.Hv, a.S, a.Dv, rows);
    return hipGetLastError();
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
