// gdn_decode.hip -- single-token (S = 1) gated delta-rule step, in place.
//
// The single-token recurrence of the "GDN Block TKG Kernel API Reference"
// page (introduction: the decode layer's "single-token recurrence"):
//   x = S^T k,  y = S^T q                       (contractions over Dk)
//   u = beta (v - e^g x)
//   S' = e^g S + k u^T
//   o = scale S'^T q = scale (e^g y + (k . q) u)
//
// Memory-bound: the fp32 state (Dk x Dv, 64 KiB at 128 x 128) is read once and
// written once per step; everything else is a few hundred bytes. One
// workgroup of 512 threads owns one (b, h). Thread t holds columns
// 4*(t%32) .. +3 of rows (t/32) + 16i, i = 0..7: every row of 128 floats is
// read by 32 consecutive lanes as 16-byte vectors (fully coalesced), and the
// 32 state values stay in registers between the read and the write. The Dk
// reductions are per-thread partial sums followed by a 16-way LDS reduction
// in a fixed order (deterministic). The state is read with ordinary loads and
// written with non-temporal stores (the written state is not re-read by this
// step). In a sweep of layouts on MI355X at B = 256 this one streamed
// 6.9 TB/s, against 5.6 TB/s with non-temporal loads and 256 threads; over
// the 64 chained steps of a decode pass it moves 6.5 TB/s.
//
// GATED variant: the prologue the same page lists ahead of the recurrence
// ("l2norm/beta/g"; Parameters A_log, dt_bias) runs here too. g_log and beta
// then carry the raw a and b, g = -e^{A_log[h]} softplus(a + dt_bias[h]),
// beta = sigmoid(b), and q, k are raw: every wave forms rk = 1/sqrt(|k|^2 +
// eps) and rq from the staged vectors (same butterfly in every wave, so the
// values agree) and the norms scale the reductions: x = rk S^T k,
// y = rq S^T q, k.q = rk rq (k.q)_raw, and the write uses rk k.
//
// BLOCK variant (KB > 0 conv taps, implies GATED): the page's decode layer
// between its projections in one kernel. The workgroup of (b, h) first runs
// the conv1d decode step ("GDN Conv1D Kernel API Reference",
// gdn_conv1d_decode) for the channels it reads -- q and k of key head j and v
// of value head h in the raw mixed token (q|k|v channel order) -- keeping the
// silu outputs in LDS, then the gated step above, then RMSNormGated over its
// Dv outputs: y = o / sqrt(mean(o^2) + eps) gamma silu(z). The shifted conv
// windows go to a separate buffer: the Hv/Hk workgroups of a GQA group all
// read the q/k windows, and only the group's first head writes them.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int kDecThreads = 512;
constexpr int kDecRowPhases = kDecThreads / 32;   // 16
constexpr int kDecRowsPerThread = 128 / kDecRowPhases;

__device__ __forceinline__ float dec_silu(float y) { return y / (1.f + expf(-y)); }

template <typename E, bool GATED, int KB>
__global__ __launch_bounds__(kDecThreads) void gdn_decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ g_log, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, float l2_eps,
    float scale, float* __restrict__ state, E* __restrict__ out, int Hk, int Hv, int Dk, int Dv,
    const E* __restrict__ mixed, const E* __restrict__ zg, const E* __restrict__ conv_in,
    E* __restrict__ conv_out, const float* __restrict__ conv_w,
    const float* __restrict__ norm_w, float norm_eps)
{
    static_assert(KB == 0 || GATED, "the block variant includes the prologue");
    const int bh = blockIdx.x;                 // b * Hv + h
    const int b = bh / Hv;
    const int h = bh - b * Hv;
    const int j = h / (Hv / Hk);               // GQA: contiguous groups of Hv/Hk
    const int t = threadIdx.x;
    const int cg = t & 31;                     // columns 4cg .. 4cg+3
    const int r0 = t >> 5;                     // rows r0 + 16i

    __shared__ float sk[128], sq[128], su[128], sv[128];
    __shared__ float red[2][kDecRowPhases][128];
    __shared__ float skq;

    float* S = state + (size_t)bh * Dk * Dv;
    const bool colok = 4 * cg < Dv;
    // Loads are unconditional from clamped (in-bounds) addresses and
    // out-of-range values are zeroed by selection: per-load branches would
    // serialise the loads and inflate the register count.
    const int cl = colok ? 4 * cg : Dv - 4;
    f32x4 s[kDecRowsPerThread];
#pragma unroll
    for (int i = 0; i < kDecRowsPerThread; ++i) {
        const int r = r0 + kDecRowPhases * i;
        const f32x4 w = *(const f32x4*)(S + (size_t)min(r, Dk - 1) * Dv + cl);
        s[i] = (colok && r < Dk) ? w : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if constexpr (KB > 0) {
        // conv1d decode step for this head's channels, while the state loads fly
        const int C = 2 * Hk * Dk + Hv * Dv;
        const int nch = 2 * Dk + Dv;
        if (t < nch) {
            const int ch = t < Dk ? j * Dk + t
                         : t < 2 * Dk ? Hk * Dk + j * Dk + (t - Dk)
                                      : 2 * Hk * Dk + h * Dv + (t - 2 * Dk);
            const size_t row = (size_t)b * C + ch;
            float win[KB];
#pragma unroll
            for (int i = 0; i + 1 < KB; ++i) win[i] = to_f32(conv_in[row * KB + i + 1]);
            win[KB - 1] = to_f32(mixed[row]);
            float y = 0.f;
#pragma unroll
            for (int i = 0; i < KB; ++i) y += conv_w[(size_t)ch * KB + i] * win[i];
            const float val = dec_silu(y);
            if (t < Dk) sq[t] = val;
            else if (t < 2 * Dk) sk[t - Dk] = val;
            else sv[t - 2 * Dk] = val;
            // the q/k windows are shared by the group's heads: its first head writes them
            if (t >= 2 * Dk || h % (Hv / Hk) == 0) {
#pragma unroll
                for (int i = 0; i < KB; ++i) conv_out[row * KB + i] = from_f32<E>(win[i]);
            }
        }
        // zero the unused tails of sq and sk (rows Dk .. 127)
        if (t >= 384 && t - 384 + Dk < 128) sq[t - 384 + Dk] = 0.f;
        if (t >= 384 && t - 384 + Dk < 128) sk[t - 384 + Dk] = 0.f;
    } else {
        const size_t qk_off = ((size_t)b * Hk + j) * Dk;
        if (t < 128) sk[t] = (t < Dk) ? to_f32(k[qk_off + t]) : 0.0f;
        else if (t < 256) sq[t - 128] = (t - 128 < Dk) ? to_f32(q[qk_off + t - 128]) : 0.0f;
    }
    float a, be;
    if constexpr (GATED) {
        const float xg = g_log[bh] + dt_bias[h];
        const float sp = xg > 0.f ? xg + log1pf(expf(-xg)) : log1pf(expf(xg));
        a = __expf(-expf(A_log[h]) * sp);
        be = 1.f / (1.f + expf(-beta[bh]));
    } else {
        a = __expf(g_log[bh]);
        be = beta[bh];
    }
    __syncthreads();                           // sk, sq (and sv) visible
    float rk = 1.f, rq = 1.f;
    if constexpr (GATED) {
        const int ln = t & 63;
        float pk = sk[ln] * sk[ln] + sk[ln + 64] * sk[ln + 64];
        float pq = sq[ln] * sq[ln] + sq[ln + 64] * sq[ln + 64];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            pk += __shfl_xor(pk, off);
            pq += __shfl_xor(pq, off);
        }
        rk = 1.f / sqrtf(pk + l2_eps);
        rq = 1.f / sqrtf(pq + l2_eps);
    }

    f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kDecRowsPerThread; ++i) {
        const int r = r0 + kDecRowPhases * i;  // rows >= Dk hold zeros in s, sk, sq
        x += s[i] * sk[r];
        y += s[i] * sq[r];
    }
    *(f32x4*)&red[0][r0][4 * cg] = x;
    *(f32x4*)&red[1][r0][4 * cg] = y;
    if (t < 64) {
        float p = sk[t] * sq[t] + sk[t + 64] * sq[t + 64];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
        if (t == 0) skq = p;
    }
    __syncthreads();

    float o = 0.f;
    if (t < Dv) {
        float xs = 0.f, ys = 0.f;
#pragma unroll
        for (int p = 0; p < kDecRowPhases; ++p) { xs += red[0][p][t]; ys += red[1][p][t]; }
        const float vv = KB > 0 ? sv[t] : to_f32(v[(size_t)bh * Dv + t]);
        const float u = be * (vv - a * (rk * xs));
        su[t] = u;
        o = scale * (a * (rq * ys) + (rk * rq * skq) * u);
        if constexpr (KB == 0) out[(size_t)bh * Dv + t] = from_f32<E>(o);
    }
    __shared__ float sms[2];
    if constexpr (KB > 0) {
        // RMSNormGated over the Dv outputs (threads t < Dv <= 128: waves 0, 1)
        if (t < 128) {
            float p = o * o;                   // 0 for t >= Dv
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
            if ((t & 63) == 0) sms[t >> 6] = p;
        }
    }
    __syncthreads();

    if constexpr (KB > 0) {
        if (t < Dv) {
            const float ms = (sms[0] + sms[1]) / (float)Dv;
            const float zz = to_f32(zg[(size_t)bh * Dv + t]);
            out[(size_t)bh * Dv + t] =
                from_f32<E>(o * (1.f / sqrtf(ms + norm_eps)) * norm_w[t] * dec_silu(zz));
        }
    }
    if (colok) {
        const f32x4 uu = rk * *(const f32x4*)&su[4 * cg];   // the write uses rk k
#pragma unroll
        for (int i = 0; i < kDecRowsPerThread; ++i) {
            const int r = r0 + kDecRowPhases * i;
            if (r < Dk) {
                const f32x4 ns = a * s[i] + sk[r] * uu;
                __builtin_nontemporal_store(ns, (f32x4*)(S + (size_t)r * Dv + 4 * cg));
            }
        }
    }
}

template <typename E, bool GATED, int KB>
static hipError_t launch_decode_t(const DecodeArgs& a, const BlockArgs* blk, hipStream_t stream)
{
    const unsigned grid = (unsigned)a.B * (unsigned)a.Hv;
    hipLaunchKernelGGL((gdn_decode_kernel<E, GATED, KB>), dim3(grid), dim3(kDecThreads), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, a.g_log, a.beta,
                       a.A_log, a.dt_bias, a.l2_eps, a.scale,
                       a.state, (E*)a.out, a.Hk, a.Hv, a.Dk, a.Dv,
                       blk ? (const E*)blk->mixed : nullptr, blk ? (const E*)blk->z : nullptr,
                       blk ? (const E*)blk->conv_in : nullptr, blk ? (E*)blk->conv_out : nullptr,
                       blk ? blk->conv_w : nullptr, blk ? blk->norm_w : nullptr,
                       blk ? blk->norm_eps : 0.f);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream)
{
    if (a.gated)
        return dtype == 1 ? launch_decode_t<bf16, true, 0>(a, nullptr, stream)
                          : launch_decode_t<float, true, 0>(a, nullptr, stream);
    return dtype == 1 ? launch_decode_t<bf16, false, 0>(a, nullptr, stream)
                      : launch_decode_t<float, false, 0>(a, nullptr, stream);
}

template <typename E>
static hipError_t launch_block_e(const DecodeArgs& a, const BlockArgs& blk, hipStream_t s)
{
#define GDN_BLOCK_CASE(KK) case KK: return launch_decode_t<E, true, KK>(a, &blk, s);
    switch (blk.K) {
        GDN_BLOCK_CASE(1) GDN_BLOCK_CASE(2) GDN_BLOCK_CASE(3) GDN_BLOCK_CASE(4)
        GDN_BLOCK_CASE(5) GDN_BLOCK_CASE(6) GDN_BLOCK_CASE(7) GDN_BLOCK_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef GDN_BLOCK_CASE
}

hipError_t launch_decode_block(const DecodeArgs& a, const BlockArgs& blk, int dtype,
                               hipStream_t stream)
{
    return dtype == 1 ? launch_block_e<bf16>(a, blk, stream) : launch_block_e<float>(a, blk, stream);
}

}  // namespace gdn
