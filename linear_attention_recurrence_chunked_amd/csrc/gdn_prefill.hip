// gdn_prefill.hip -- chunk-parallel gated delta-rule prefill on gfx950.
//
// The chunked form that the "GDN CTE Kernel API Reference" page describes in
// its introduction (work inside a chunk is parallel and goes through a
// unit-lower-triangular inverse; a recurrence carries the state across
// chunks). For one head and a chunk of C tokens with start state S0,
// gamma = within-chunk inclusive cumulative sum of g_log:
//
//   A  = diag(beta) (K K^T) (.) Mstrict     Mstrict[r,s] = e^{gamma_r-gamma_s}, s < r
//   T  = (I + A)^{-1}                       unit lower triangular, fp32
//   W  = T diag(beta e^gamma) K             U~ = T diag(beta) V
//   U  = U~ - W S0                          the per-token updates u_t
//   O  = scale (diag(e^gamma) Q S0 + (Q K^T (.) Mincl) U)     Mincl: s <= r
//   S1 = e^{gamma_C} S0 + K^T diag(e^{gamma_C - gamma}) U
//
// (derived from the token recurrence S_t = e^{g_t} S_{t-1} + beta_t k_t
// (v_t - e^{g_t} S_{t-1}^T k_t)^T, o_t = scale S_t^T q_t).
//
// Design (one fused kernel, no HBM intermediates): one workgroup of NW waves
// owns one (batch, value head, BV-wide slice of Dv) and walks the chunks of
// that sequence in order, holding its [Dk x BV] slice of the fp32 state in
// MFMA accumulator registers the whole time. Per chunk only q, k, v, g, beta
// are read and out is written, so HBM traffic is the algorithmic minimum. The
// state-independent work of a chunk (gamma, A, T, W, U~, the masked Q K^T) is
// recomputed by each Dv slice; BV is chosen per launch so the grid fills the
// 256 compute units. Every product is a 16x16-tile MFMA from LDS (bf16
// operands, fp32 accumulation; fp32 operands on the fp32 path). The
// triangular inverse is computed in fp32: 16x16 diagonal blocks by forward
// substitution (one lane per column), then doubling merges
// T21 = -T22 A21 T11 on fp32 MFMA.
#include "gdn_common.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename E> struct Vec16;  // one 16-byte vector of E
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

__device__ __forceinline__ void store4(bf16* p, f32x4 x) {
    bf16x4 y = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    *(bf16x4*)p = y;
}
__device__ __forceinline__ void store4(float* p, f32x4 x) { *(f32x4*)p = x; }

// Linear index of a lower-triangular 16x16 tile (row-major over i >= j) -> (i, j).
__device__ __forceinline__ void tri_index(int lt, int& i, int& j) {
    i = 0;
    while (lt > i) { lt -= i + 1; ++i; }
    j = lt;
}

template <typename E, int C, int DK, int BV, int NW>
struct PrefillCfg {
    using M = Mfma<E>;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int VE = Vec16<E>::N;
    static constexpr int LDK = DK + M::PAD;   // rows of [t][dk] (K, Q, -W) and [v][dk] (St)
    static constexpr int LDC = C + M::PAD;    // rows of [x][t] (Kt, Vt, P, TK, TV, Ut, Ud)
    static constexpr int LDF = C + 4;         // rows of fp32 [t][s] (A, Tf)
    static constexpr int NT = C / 16;
    static constexpr int NKT = DK / 16;
    static constexpr int NVT = BV / 16;
    static constexpr int NLT = NT * (NT + 1) / 2;
    static constexpr int NO = NT * NVT;       // out / U tiles
    static constexpr int NS = NKT * NVT;      // state tiles
    static constexpr int NWT = NT * NKT;      // W tiles
    static constexpr int THREADS = NW * 64;
    static constexpr int OPW = (NO + NW - 1) / NW;
    static constexpr int SPW = (NS + NW - 1) / NW;
    static constexpr int WPW = (NWT + NW - 1) / NW;
    static constexpr int JPW = (2 * NLT + NW - 1) / NW;
    // LDS regions; buffers sharing a region have disjoint lifetimes in a chunk.
    static constexpr int SZ_TD = C * LDK * ES;                         // K -> -W
    static constexpr int SZ_Q = cmax(C * LDK * ES, C * LDF * 4);       // Q -> Tf
    static constexpr int SZ_KT = DK * LDC * ES;                        // Kt
    static constexpr int SZ_VT = BV * LDC * ES;                        // Vt
    static constexpr int SZ_ST = BV * LDK * ES;                        // St (bf16/fp32 copy of S^T)
    static constexpr int SZ_P = C * LDC * ES;                          // P = QK^T (.) Mincl
    static constexpr int SZ_T = 2 * C * LDC * ES;                      // TK, TV
    static constexpr int SZ_U = cmax(C * LDF * 4, 2 * BV * LDC * ES);  // A -> Ut, Ud
    static constexpr int SZ_X = (C / 2) * (C / 2 + 4) * 4;             // merge scratch
    static constexpr int SZ_SC = 8 * C * 4;                            // per-token scalars
    static constexpr int OFF_TD = 0;
    static constexpr int OFF_Q = OFF_TD + SZ_TD;
    static constexpr int OFF_KT = OFF_Q + SZ_Q;
    static constexpr int OFF_VT = OFF_KT + SZ_KT;
    static constexpr int OFF_ST = OFF_VT + SZ_VT;
    static constexpr int OFF_P = OFF_ST + SZ_ST;
    static constexpr int OFF_T = OFF_P + SZ_P;
    static constexpr int OFF_U = OFF_T + SZ_T;
    static constexpr int OFF_X = OFF_U + SZ_U;
    static constexpr int OFF_SC = OFF_X + SZ_X;
    static constexpr int LDS_BYTES = OFF_SC + SZ_SC;
    static_assert(LDS_BYTES <= 160 * 1024, "chunk tiles exceed the 160 KiB LDS of a CU");
    static_assert(C % M::KS == 0 && DK % M::KS == 0, "tile sizes must match the MFMA depth");
    static_assert(C >= 32 && (C & (C - 1)) == 0 && C <= 64, "chunk must be 32 or 64");
};

template <typename E, int C, int DK, int BV, int NW>
__global__ __launch_bounds__(NW * 64) void gdn_prefill_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ g_log, const float* __restrict__ beta, float scale,
    float* __restrict__ state, E* __restrict__ out,
    int Hk, int Hv, int S, int Dk, int Dv, int nvt)
{
    using Cf = PrefillCfg<E, C, DK, BV, NW>;
    using M = Mfma<E>;
    using VecE = typename Vec16<E>::type;
    constexpr int VE = Cf::VE, LDK = Cf::LDK, LDC = Cf::LDC, LDF = Cf::LDF, NW_ = NW;
    constexpr int THREADS = Cf::THREADS, KS = M::KS;

    __shared__ __attribute__((aligned(16))) char smem[Cf::LDS_BYTES];
    E* sK = (E*)(smem + Cf::OFF_TD);
    E* sW = sK;                                  // holds -W after the K^T products
    E* sQ = (E*)(smem + Cf::OFF_Q);
    float* sTf = (float*)(smem + Cf::OFF_Q);     // fp32 T after the Q products
    E* sKt = (E*)(smem + Cf::OFF_KT);
    E* sVt = (E*)(smem + Cf::OFF_VT);
    E* sSt = (E*)(smem + Cf::OFF_ST);
    E* sP = (E*)(smem + Cf::OFF_P);
    E* sTK = (E*)(smem + Cf::OFF_T);
    E* sTV = sTK + C * LDC;
    float* sA = (float*)(smem + Cf::OFF_U);
    E* sUt = (E*)(smem + Cf::OFF_U);
    E* sUd = sUt + BV * LDC;
    float* sX = (float*)(smem + Cf::OFF_X);
    float* sc = (float*)(smem + Cf::OFF_SC);
    float* sc_g = sc;              // raw g_log
    float* sc_b = sc + C;          // beta
    float* sc_gam = sc + 2 * C;    // gamma
    float* sc_eg = sc + 3 * C;     // e^gamma
    float* sc_bk = sc + 4 * C;     // beta e^gamma
    float* sc_dl = sc + 5 * C;     // e^{gamma_C - gamma}
    float* sc_misc = sc + 6 * C;   // [0] = e^{gamma_C}

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int l = tid & 63;
    const int lc = l & 15;          // column of this lane in a 16x16 C tile
    const int lr = 4 * (l >> 4);    // first of its 4 rows

    // blockIdx -> (v slice, value head, batch)
    int bid = blockIdx.x;
    const int vt = bid % nvt; bid /= nvt;
    const int h = bid % Hv;
    const int b = bid / Hv;
    const int j = h / (Hv / Hk);
    const int v0 = vt * BV;
    const int vcols = min(BV, Dv - v0);
    const size_t bh = (size_t)b * Hv + h;
    const E* kb = k + ((size_t)b * Hk + j) * (size_t)S * Dk;
    const E* qb = q + ((size_t)b * Hk + j) * (size_t)S * Dk;
    const E* vb = v + bh * (size_t)S * Dv + v0;
    const float* gb = g_log + bh * (size_t)S;
    const float* bb = beta + bh * (size_t)S;
    E* ob = out + bh * (size_t)S * Dv + v0;
    float* sb = state + bh * (size_t)Dk * Dv + v0;

    // ---- initial state: fp32 accumulators + LDS copy St[v][dk]
    f32x4 accS[Cf::SPW];
#pragma unroll
    for (int m = 0; m < Cf::SPW; ++m) {
        const int id = wave + NW_ * m;
        accS[m] = zero4();
        if (id < Cf::NS) {
            const int tk = id / Cf::NVT, vj = id % Cf::NVT;
            const int col = 16 * vj + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dk = 16 * tk + lr + e;
                accS[m][e] = (dk < Dk && col < vcols) ? sb[(size_t)dk * Dv + col] : 0.f;
            }
            store4(sSt + col * LDK + 16 * tk + lr, accS[m]);
        }
    }

    for (int c0 = 0; c0 < S; c0 += C) {
        __syncthreads();  // previous chunk (or the initial St) complete

        // ---- P0: stage K (row-major and transposed), Q, V^T, g, beta
        for (int id = tid; id < C * DK / VE; id += THREADS) {
            const int t = id % C, d0 = (id / C) * VE;
            VecE x = {};
            if (d0 < Dk) x = *(const VecE*)(kb + (size_t)(c0 + t) * Dk + d0);
            *(VecE*)(sK + t * LDK + d0) = x;
#pragma unroll
            for (int e = 0; e < VE; ++e) sKt[(d0 + e) * LDC + t] = x[e];
        }
        for (int id = tid; id < C * DK / VE; id += THREADS) {
            const int d0 = (id % (DK / VE)) * VE, t = id / (DK / VE);
            VecE x = {};
            if (d0 < Dk) x = *(const VecE*)(qb + (size_t)(c0 + t) * Dk + d0);
            *(VecE*)(sQ + t * LDK + d0) = x;
        }
        for (int id = tid; id < C * BV / VE; id += THREADS) {
            const int t = id % C, d0 = (id / C) * VE;
            VecE x = {};
            if (d0 < vcols) x = *(const VecE*)(vb + (size_t)(c0 + t) * Dv + d0);
#pragma unroll
            for (int e = 0; e < VE; ++e) sVt[(d0 + e) * LDC + t] = x[e];
        }
        if (tid < C) sc_g[tid] = gb[c0 + tid];
        else if (tid < 2 * C) sc_b[tid - C] = bb[c0 + tid - C];
        __syncthreads();

        // ---- P1: gamma = inclusive cumsum of g over the chunk (one wave)
        if (wave == 0) {
            float x = (l < C) ? sc_g[l] : 0.f;
#pragma unroll
            for (int off = 1; off < C; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (l >= off) x += y;
            }
            const float gC = __shfl(x, C - 1);
            if (l < C) {
                const float eg = __expf(x);
                sc_gam[l] = x;
                sc_eg[l] = eg;
                sc_bk[l] = sc_b[l] * eg;
                sc_dl[l] = __expf(gC - x);   // gC <= x: never overflows
            }
            if (l == 0) sc_misc[0] = __expf(gC);
        }
        __syncthreads();

        // ---- P2: A = masked beta K K^T (fp32), P = masked Q K^T, and Q S0
        //      Decay factors are formed as e^{gamma_r - gamma_s} only where
        //      s <= r (a select, never a product with a masked value).
#pragma unroll
        for (int m = 0; m < Cf::JPW; ++m) {
            const int job = wave + NW_ * m;
            if (job < 2 * Cf::NLT) {
                const bool isQ = job >= Cf::NLT;
                int ti, tj;
                tri_index(isQ ? job - Cf::NLT : job, ti, tj);
                const E* Ab = isQ ? sQ : sK;
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < DK; kk += KS)
                    acc = M::mma(M::ld(Ab, LDK, 16 * ti, kk), M::ld(sK, LDK, 16 * tj, kk), acc);
                const int s = 16 * tj + lc;
                const float gs = sc_gam[s];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * ti + lr + e;
                    const float dec = __expf(sc_gam[r] - gs);
                    if (!isQ) sA[r * LDF + s] = (s < r) ? sc_b[r] * dec * acc[e] : 0.f;
                    else sP[r * LDC + s] = from_f32<E>((s <= r) ? dec * acc[e] : 0.f);
                }
            }
        }
        for (int id = tid; id < C * C; id += THREADS) {   // zero the strictly-upper tiles of P
            const int r = id / C, s = id % C;
            if ((s >> 4) > (r >> 4)) sP[r * LDC + s] = from_f32<E>(0.f);
        }
        f32x4 accO[Cf::OPW];
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            accO[m] = zero4();
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
#pragma unroll
                for (int kk = 0; kk < DK; kk += KS)
                    accO[m] = M::mma(M::ld(sQ, LDK, 16 * ti, kk), M::ld(sSt, LDK, 16 * vj, kk),
                                     accO[m]);
            }
        }
        __syncthreads();

        // ---- P3a: 16x16 diagonal blocks of T by forward substitution (fp32)
        if (wave == 0) {
            const int d = l >> 4, jc = l & 15;
            if (d < Cf::NT) {
                const float* Ad = sA + (16 * d) * LDF + 16 * d;
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = (r == jc) ? 1.f : 0.f;
#pragma unroll
                    for (int s = 0; s < r; ++s) acc -= Ad[r * LDF + s] * x[s];
                    x[r] = acc;
                }
                float* Td = sTf + (16 * d) * LDF + 16 * d;
#pragma unroll
                for (int r = 0; r < 16; ++r) Td[r * LDF + jc] = x[r];
            }
        }
        __syncthreads();

        // ---- P3b: doubling merges, T21 = -T22 (A21 T11), fp32 MFMA
#pragma unroll
        for (int mb = 16; mb < C; mb *= 2) {
            const int nblk = C / (2 * mb);
            const int tpr = mb / 16;
            const int tpb = tpr * tpr;
            const int LDX = mb + 4;
            for (int job = wave; job < nblk * tpb; job += NW_) {     // X = A21 T11
                const int bk = job / tpb, tt = job % tpb, ti = tt / tpr, tj = tt % tpr;
                const int base = 2 * mb * bk;
                f32x4 acc = zero4();
                for (int kk = 16 * tj; kk < mb; kk += 4)
                    acc = Mfma<float>::mma(Mfma<float>::ld(sA, LDF, base + mb + 16 * ti, base + kk),
                                           ld_b_rowmajor(sTf, LDF, base + kk, base + 16 * tj), acc);
                float* Xb = sX + bk * mb * LDX;
#pragma unroll
                for (int e = 0; e < 4; ++e) Xb[(16 * ti + lr + e) * LDX + 16 * tj + lc] = acc[e];
            }
            __syncthreads();
            for (int job = wave; job < nblk * tpb; job += NW_) {     // T21 = -T22 X
                const int bk = job / tpb, tt = job % tpb, ti = tt / tpr, tj = tt % tpr;
                const int base = 2 * mb * bk;
                const float* Xb = sX + bk * mb * LDX;
                f32x4 acc = zero4();
                for (int kk = 0; kk < 16 * (ti + 1); kk += 4)
                    acc = Mfma<float>::mma(Mfma<float>::ld(sTf, LDF, base + mb + 16 * ti, base + mb + kk),
                                           ld_b_rowmajor(Xb, LDX, kk, 16 * tj), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sTf[(base + mb + 16 * ti + lr + e) * LDF + base + 16 * tj + lc] = -acc[e];
            }
            __syncthreads();
        }

        // ---- P3c: TK = T diag(beta e^gamma), TV = T diag(beta) in the operand type
        for (int id = tid; id < C * C; id += THREADS) {
            const int r = id / C, s = id % C;
            const float tv = (s <= r) ? sTf[r * LDF + s] : 0.f;
            sTK[r * LDC + s] = from_f32<E>(tv * sc_bk[s]);
            sTV[r * LDC + s] = from_f32<E>(tv * sc_b[s]);
        }
        __syncthreads();

        // ---- P4: -W = -(TK K) into LDS; U~ = TV V in registers
#pragma unroll
        for (int m = 0; m < Cf::WPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NWT) {
                const int ti = id / Cf::NKT, tk = id % Cf::NKT;
                const int kend = ((16 * (ti + 1) + KS - 1) / KS) * KS;
                f32x4 acc = zero4();
                for (int s = 0; s < kend; s += KS)
                    acc = M::mma(M::ld(sTK, LDC, 16 * ti, s), M::ld(sKt, LDC, 16 * tk, s), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sW[(16 * ti + lr + e) * LDK + 16 * tk + lc] = from_f32<E>(-acc[e]);
            }
        }
        f32x4 accU[Cf::OPW];
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            accU[m] = zero4();
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
                const int kend = ((16 * (ti + 1) + KS - 1) / KS) * KS;
                for (int s = 0; s < kend; s += KS)
                    accU[m] = M::mma(M::ld(sTV, LDC, 16 * ti, s), M::ld(sVt, LDC, 16 * vj, s),
                                     accU[m]);
            }
        }
        __syncthreads();

        // ---- P5: U = U~ - W S0; store U^T and (diag(e^{gamma_C-gamma}) U)^T
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
#pragma unroll
                for (int kk = 0; kk < DK; kk += KS)
                    accU[m] = M::mma(M::ld(sW, LDK, 16 * ti, kk), M::ld(sSt, LDK, 16 * vj, kk),
                                     accU[m]);
                const int vl = 16 * vj + lc, t0 = 16 * ti + lr;
                store4(sUt + vl * LDC + t0, accU[m]);
                f32x4 ud;
#pragma unroll
                for (int e = 0; e < 4; ++e) ud[e] = accU[m][e] * sc_dl[t0 + e];
                store4(sUd + vl * LDC + t0, ud);
            }
        }
        __syncthreads();

        // ---- P6: O = scale (e^gamma Q S0 + P U) -> out; S = e^{gamma_C} S0 + K^T Ud
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
#pragma unroll
                for (int e = 0; e < 4; ++e) accO[m][e] *= sc_eg[16 * ti + lr + e];
                const int kend = ((16 * (ti + 1) + KS - 1) / KS) * KS;
                for (int s = 0; s < kend; s += KS)
                    accO[m] = M::mma(M::ld(sP, LDC, 16 * ti, s), M::ld(sUt, LDC, 16 * vj, s),
                                     accO[m]);
                const int col = 16 * vj + lc;
                if (col < vcols) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ob[(size_t)(c0 + 16 * ti + lr + e) * Dv + col] =
                            from_f32<E>(scale * accO[m][e]);
                }
            }
        }
        const float egC = sc_misc[0];
#pragma unroll
        for (int m = 0; m < Cf::SPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NS) {
                const int tk = id / Cf::NVT, vj = id % Cf::NVT;
#pragma unroll
                for (int e = 0; e < 4; ++e) accS[m][e] *= egC;
#pragma unroll
                for (int t = 0; t < C; t += KS)
                    accS[m] = M::mma(M::ld(sKt, LDC, 16 * tk, t), M::ld(sUd, LDC, 16 * vj, t),
                                     accS[m]);
                store4(sSt + (16 * vj + lc) * LDK + 16 * tk + lr, accS[m]);
            }
        }
    }

    // ---- final state
#pragma unroll
    for (int m = 0; m < Cf::SPW; ++m) {
        const int id = wave + NW_ * m;
        if (id < Cf::NS) {
            const int tk = id / Cf::NVT, vj = id % Cf::NVT;
            const int col = 16 * vj + lc;
            if (col < vcols) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int dk = 16 * tk + lr + e;
                    if (dk < Dk) sb[(size_t)dk * Dv + col] = accS[m][e];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launch

template <typename E, int C, int DK, int BV>
static hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream)
{
    constexpr int NW = 8;
    const int nvt = (a.Dv + BV - 1) / BV;
    const long long blocks = (long long)nvt * a.Hv * a.B;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_prefill_kernel<E, C, DK, BV, NW>), dim3((unsigned)blocks),
                       dim3(NW * 64), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, a.g_log, a.beta, a.scale,
                       a.state, (E*)a.out, a.Hk, a.Hv, a.S, a.Dk, a.Dv, nvt);
    return hipGetLastError();
}

// Value-slice width: the widest of {max_bv, .., 16} that still gives at least
// one workgroup per compute unit (256 on MI355X); narrower slices repeat the
// state-independent chunk work, so wider is better once the chip is full.
static int pick_bv(const PrefillArgs& a, int max_bv)
{
    const long long units = (long long)a.B * a.Hv;
    for (int bv = max_bv; bv > 16; bv /= 2)
        if (a.Dv > bv / 2 && units * ((a.Dv + bv - 1) / bv) >= 256) return bv;
    return 16;
}

template <typename E, int C, int DK>
static hipError_t launch_dk(const PrefillArgs& a, int max_bv, hipStream_t stream)
{
    switch (pick_bv(a, max_bv)) {
        case 64: if constexpr (sizeof(E) == 2) return launch_cfg<E, C, DK, 64>(a, stream);
                 [[fallthrough]];
        case 32: return launch_cfg<E, C, DK, 32>(a, stream);
        default: return launch_cfg<E, C, DK, 16>(a, stream);
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, hipStream_t stream)
{
    if (dtype == 1) {   // bf16 operands: 64-token chunks
        return a.Dk <= 64 ? launch_dk<bf16, 64, 64>(a, 64, stream)
                          : launch_dk<bf16, 64, 128>(a, 64, stream);
    }
    // fp32 operands: 32-token chunks keep the fp32 tiles inside LDS
    return a.Dk <= 64 ? launch_dk<float, 32, 64>(a, 32, stream)
                      : launch_dk<float, 32, 128>(a, 32, stream);
}

}  // namespace gdn
