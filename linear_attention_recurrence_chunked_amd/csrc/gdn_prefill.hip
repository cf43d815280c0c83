// gdn_prefill.hip -- chunk-parallel gated delta-rule prefill on gfx950.
//
// The chunked form that the "GDN CTE Kernel API Reference" page describes in
// its introduction (work inside a chunk is parallel and goes through a
// unit-lower-triangular inverse; a recurrence carries the state across
// chunks). For one head and a chunk of C tokens with start state S0 and
// gamma = within-chunk inclusive cumulative sum of g_log:
//
//   A  = diag(beta) (K K^T) (.) Mstrict     Mstrict[r,s] = e^{gamma_r-gamma_s}, s < r
//   T  = (I + A)^{-1}                       unit lower triangular, fp32
//   R  = diag(beta) V - diag(beta e^gamma) K S0
//   U  = T R                                the per-token updates u_t
//   O  = scale (diag(e^gamma) Q S0 + P U),  P = Q K^T (.) Mincl  (s <= r)
//   S1 = e^{gamma_C} S0 + K^T diag(e^{gamma_C - gamma}) U
//
// derived from the token recurrence S_t = e^{g_t} S_{t-1} + beta_t k_t
// (v_t - e^{g_t} S_{t-1}^T k_t)^T, o_t = scale S_t^T q_t: unrolling a chunk
// gives (I + A) U = diag(beta) V - diag(beta e^gamma) K S0. R is formed in
// fp32 before any rounding, so the cancellation between new values and the
// state's prediction happens at full precision.
//
// One workgroup owns one (batch, value head, BV-wide slice of Dv) and walks
// the C = 32 token chunks of its sequence. Its waves have fixed roles and
// meet at one barrier per chunk:
//
//  * consumer waves, one per 16-column strip of the slice, keep their
//    [Dk x 16] slice of the fp32 state in MFMA accumulator registers for the
//    whole sequence. For chunk i they compute K S0 and Q S0 (state fed from
//    registers as the B operand), R, U = T R, O = e^gamma Q S0 + P U and the
//    state update K^T (dl U) -- every intermediate stays in registers; LDS is
//    only read for K, Q, V, T and P of the chunk (the first K/Q slice and
//    the row scalars of chunk i+1 already during chunk i's output phase).
//    With a single strip (PAIR) two waves share it, each holding half of
//    the key rows, and exchange their partial K S0 / Q S0 through LDS;
//  * two inverse waves build T = (I + A)^{-1}, taking alternate chunks and
//    spreading a chunk over two steps: fp32 substitution of the two 16x16
//    diagonal blocks for chunk i+2 (four lanes per column, the finished
//    unknown passed by a DPP quad broadcast), then the merge
//    T21 = -T22 (A21 T11) on fp32 MFMA and the stores for chunk i+1;
//  * the A wave builds A = diag(beta) (K K^T) (.) Mstrict for chunk i+3;
//  * the P wave builds P = Q K^T (.) Mincl for chunk i+1;
//  * two stager waves (K with g and beta; Q with V) issue the loads of chunk
//    i+LEAD+1 and store chunk i+LEAD (loaded a step earlier) into LDS, with
//    gamma and the per-token decay scalars; the HBM latency passes during
//    the rest of the step, off the sequential path.
// On the fp32 path (tiles twice as large) one inverse wave builds A and T of
// chunk i+1 in one step and the stagers run LEAD = 2 ahead.
//
// LDS holds the input slots of chunks i .. i+LEAD (5 on the bf16 path, 3 on
// the fp32 path), three T, two P and three A buffers (two T, two P, one A on
// the fp32 path), and with PAIR the consumers' exchange blocks.
// The state-independent work of a chunk therefore never sits on the
// sequential path. HBM traffic is the algorithmic minimum: q, k, v, g, beta
// read once per slice, out written once, the state read and written once.
// On the bf16 path every computed operand (S, T, R, P, U) is carried as a
// hi/lo bf16 pair (see gdn_mfma.h), so products keep about 16 bits.
//
// GATED variant: the decode block's prologue ("GDN Block TKG Kernel API
// Reference": introduction, "l2norm/beta/g"; Parameters A_log, dt_bias) is
// fused in. The g_log/beta streams then carry the raw a and b; the K stager
// forms g = -e^{A_log[h]} softplus(a + dt_bias[h]) and beta = sigmoid(b) per
// token. The raw q and k tiles go to the matrix cores unchanged and the
// norms rk = 1/sqrt(|k|^2 + eps), rq likewise, ride on per-token factors:
// |k_t|^2 is the diagonal of the K K^T tiles the A builder computes anyway,
// so it forms rk and folds it into A[r][s] (rk_r rk_s), into beta e^gamma
// (the K S0 term of R) and into e^{gamma_C - gamma} (the state update);
// the P wave adds the two diagonal Q Q^T tiles for rq and folds rq rk_s into
// P and rq into scale e^gamma (the Q S0 term). The consumers' code is the
// same for both variants, and no normalised copy of q or k is rounded.
//
// INV selects the intra-chunk inverse (the choice the "GDN CTE Kernel API
// Reference" page offers as its `algorithm` argument, Parameters): 0 =
// blocked forward substitution (below), 1 = a Neumann product on each 16x16
// diagonal block, (I + X)^{-1} = (I - X)(I + X^2)(I + X^4)(I + X^8) exactly
// for the nilpotent X, on fp32 MFMA; both then merge the off-diagonal block
// the same way.
#include "gdn_common.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

// Scheduling-barrier mask that lets ALU, VALU, SALU and MFMA instructions
// move across it while memory instructions stay on their side.
constexpr int kComputeMayCross = 0x000F;

// Fourth word of a raw buffer resource (32-bit data format; no swizzle).
constexpr int kBufDword3 = 0x00020000;

template <typename E> struct Vec16;  // one 16-byte vector of E
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

// Stores x (and, on the bf16 path, its low part x - bf16(x) at p + lo_off).
template <bool SPLIT>
__device__ __forceinline__ void store_pair(bf16* p, int lo_off, float x) {
    const bf16 hi = (bf16)x;
    p[0] = hi;
    if constexpr (SPLIT) p[lo_off] = (bf16)(x - (float)hi);
}
template <bool SPLIT>
__device__ __forceinline__ void store_pair(float* p, int, float x) { p[0] = x; }

template <typename E, int C, int DK, int BV>
struct PipeCfg {
    using O = Op<E>;
    static constexpr bool SP = O::SPLIT;
    static constexpr int ES = (int)sizeof(E);
    static constexpr int VE = Vec16<E>::N;
    static constexpr int NCW = BV / 16;            // 16-column strips of the state
    // SPREAD (bf16 path): two inverse waves take alternate chunks and spread
    // the inverse of a chunk over two steps (substitution, then merge and
    // stores), and an A wave builds A three chunks ahead. Without SPREAD
    // (fp32 path, whose tiles are twice as large) one inverse wave builds A
    // and T of a chunk in one step.
    static constexpr bool SPREAD = SP;
    // PAIR (a single strip on the bf16 path, Dk = 128: the instance that runs
    // when batch x heads cannot fill the chip with wider slices): two
    // consumer waves share the strip, each holding half of its key rows, and
    // exchange their partial K S0 and Q S0 products through LDS within the
    // step. Consumer wave w works on strip w / 2 and key half w % 2. (With two
    // strips the pairs measured 9 % slower: four consumer waves then share
    // SIMDs with the helpers, and R and U run twice per strip.)
    static constexpr bool PAIR = SPREAD && NCW == 1 && DK == 128;
    static constexpr int NCWW = PAIR ? 2 * NCW : NCW;    // consumer waves
    static constexpr int NKTW = (DK / 16) / (PAIR ? 2 : 1);   // state tiles per consumer wave
    // Wave w runs on SIMD w % 4 (waves are placed round-robin). With four
    // consumers, P and A share SIMDs 0 and 1 with the two stagers, and the
    // inverse waves (the heaviest helpers) get SIMDs 2 and 3 to themselves
    // (besides a consumer); the K stager (gamma scan, decay scalars, gates)
    // sits with the A wave and the lighter QV stager with the P wave, which
    // has more VALU work. With one or two consumers the consumers share their
    // SIMDs only with the stagers (the lightest roles) and the inverse waves
    // go with P and A; with one consumer the K stager has SIMD 3 alone.
    static constexpr int NTW = SPREAD ? 2 : 1;     // inverse waves
    static constexpr bool FEW = SPREAD && NCWW < 4;
    static constexpr int W_P = NCWW;               // P wave
    static constexpr int W_A = SPREAD ? NCWW + 1 : -1;   // A wave
    static constexpr int W_T0 = FEW ? NCWW + 4 : (SPREAD ? NCWW + 2 : NCWW + 1);   // inverse waves
    static constexpr int W_T1 = W_T0 + NTW - 1;
    static constexpr int W_SQ = FEW ? (NCWW == 1 ? NCWW + 3 : NCWW + 2) : W_T1 + 1;   // QV stager
    static constexpr int W_SK = FEW ? (NCWW == 1 ? NCWW + 2 : NCWW + 3) : W_T1 + 2;   // K stager
    static constexpr int NW = NCWW + (SPREAD ? 6 : 4);
    static constexpr int THREADS = 64 * NW;
    static constexpr int NSLOT = SPREAD ? 5 : 3;   // chunks i .. i+NSLOT-1 resident
    static constexpr int LEAD = NSLOT - 1;         // the stagers write chunk i+LEAD (even)
    static constexpr int NABUF = SPREAD ? 3 : 1;   // A of chunks i+1 .. i+3
    // Row strides (elements), chosen so that the 16-byte fragment reads and
    // the transpose reads of each buffer spread over the LDS banks (on the
    // bf16 path: K/Q rows of 72 dwords, T/P rows of 40 dwords).
    static constexpr int PADE = SP ? 8 : 4;
    static constexpr int LDK = DK + (SP ? 16 : 4); // K, Q rows [t][dk]
    static constexpr int LDV = BV + PADE;          // V rows [t][v]
    static constexpr int LDP = SP ? 2 * C + 16 : C + 4;  // T, P rows [t][hi tpos(s) | lo tpos(s)]
    static constexpr int ALD = 16 + 4;             // rows of the fp32 16x16 A blocks
    static constexpr int NT = C / 16;
    static constexpr int NKT = DK / 16;
    static constexpr int NKS = DK / 32;
    static constexpr int NVK = C * DK / VE / 64;   // 16-byte vectors per stager lane: K (and Q)
    static constexpr int NVV = C * BV / VE / 64;   //                                  V
    // LDS layout (bytes)
    static constexpr int SZ_K = C * LDK * ES;
    static constexpr int SZ_V = C * LDV * ES;
    static constexpr int SZ_SC = (7 * C + 4) * 4;
    static constexpr int OFF_SK = 0, OFF_SQ = SZ_K, OFF_SV = 2 * SZ_K, OFF_SSC = 2 * SZ_K + SZ_V;
    static constexpr int SZ_SLOT = 2 * SZ_K + SZ_V + SZ_SC;
    static constexpr int SZ_TP = C * LDP * ES;
    // A buffer: three 16 x ALD fp32 blocks, each in the layout its reader
    // wants: A11 transposed, A22 and A21 row-major.
    static constexpr int SZ_F = 3 * 16 * ALD * 4;
    static constexpr int AB_11T = 0, AB_22 = 16 * ALD, AB_21 = 32 * ALD;   // (floats)
    // The small T/P/A buffers sit at the bottom of LDS and the input slots
    // above them, so that their fixed offsets fit the 16-bit immediate offset
    // of LDS instructions (an address above 64 KiB costs an extra address
    // register per access).
    static constexpr int OFF_A = 0;
    static constexpr int OFF_T = OFF_A + NABUF * SZ_F;
    static constexpr int NTBUF = SPREAD ? 3 : 2;   // T of chunks i .. i+NTBUF-1
    static constexpr int OFF_P = OFF_T + NTBUF * SZ_TP;
    static constexpr int OFF_SLOTS = OFF_P + 2 * SZ_TP;
    // PAIR exchange: per consumer wave three 1 KiB blocks (its partial K S0
    // tiles 0 and 1, and its partial Q S0 tile of the other wave's output
    // rows: one f32x4 per lane each) and a step counter.
    static constexpr int OFF_X = OFF_SLOTS + NSLOT * SZ_SLOT;
    static constexpr int SZ_XW = 3 * 64 * 16;
    static constexpr int OFF_XF = OFF_X + NCWW * SZ_XW;
    static constexpr int LDS_BYTES = PAIR ? OFF_XF + 4 * NCWW : OFF_X;
    // scalar arrays inside a slot (floats): gamma (its fp32 value and, in SC_GAML,
    // the rest gamma - fp32(gamma)), scale e^gamma, beta, beta e^gamma,
    // e^{gamma_C - gamma}, [0] = e^{gamma_C}; on the GATED path rk (from the A
    // builder, for the P wave), and the second, fourth and fifth arrays carry the
    // factors rq, rk, rk once the P wave and the A builder have folded them in.
    static constexpr int SC_GAM = 0, SC_EG = C, SC_B = 2 * C, SC_BK = 3 * C, SC_DL = 4 * C,
                         SC_RK = 5 * C, SC_GAML = 6 * C, SC_EGC = 7 * C;

    static_assert(C == 32, "the pipeline is laid out for 32-token chunks");
    static_assert(LEAD % 2 == 0, "the stagers' prologue stores chunks in pairs");
    static_assert((1 << W_P | (SPREAD ? 1 << W_A : 0) | 1 << W_T0 | 1 << W_T1 | 1 << W_SQ | 1 << W_SK) ==
                      (((1 << NW) - 1) & ~((1 << NCWW) - 1)),
                  "every helper role has its own wave after the consumers");
    static_assert(DK % 32 == 0 && BV % 16 == 0 && BV <= 64, "tile sizes");
    static_assert((C * DK / VE) % 64 == 0 && (C * BV / VE) % 64 == 0, "stager vector split");
    static_assert((SZ_K | SZ_V | SZ_SC | SZ_TP | SZ_F) % 16 == 0, "16-byte LDS alignment");
    static_assert(LDS_BYTES <= 160 * 1024, "exceeds the 160 KiB LDS of a CU");
};

// ln(1 + e^x) = max(x, 0) + log1p(e^{-|x|}), with log1p(t) = ln(u) t / (u - 1),
// u = 1 + t, which cancels the rounding of u (accurate also for tiny t).
__device__ __forceinline__ float softplus_f(float x) {
    const float t = __expf(-fabsf(x));
    const float u = 1.f + t;
    const float lp = u == 1.f ? t : __logf(u) * (t * __builtin_amdgcn_rcpf(u - 1.f));
    return fmaxf(x, 0.f) + lp;
}

// DPP controls (GFX9 encoding): row shift right by n = kDppRowShr + n, and
// lane 15 of each row broadcast to the next row.
constexpr int kDppRowShr = 0x110, kDppRowBcast15 = 0x142;

// x of the lane that DPP control CTRL selects, in the rows of ROW_MASK; 0 in
// lanes without a source or outside ROW_MASK.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// x of lane k (0..3, a constant once unrolled) of this lane's quad: a DPP
// quad_perm broadcast.
__device__ __forceinline__ float quad_bcast(float x, int k) {
    const int xi = __builtin_bit_cast(int, x);
    int r;
    switch (k) {
        case 0: r = __builtin_amdgcn_mov_dpp(xi, 0x00, 0xf, 0xf, false); break;
        case 1: r = __builtin_amdgcn_mov_dpp(xi, 0x55, 0xf, 0xf, false); break;
        case 2: r = __builtin_amdgcn_mov_dpp(xi, 0xaa, 0xf, 0xf, false); break;
        default: r = __builtin_amdgcn_mov_dpp(xi, 0xff, 0xf, 0xf, false); break;
    }
    return __builtin_bit_cast(float, r);
}

// x of lane `lane` (uniform), through scalar registers.
__device__ __forceinline__ double readlane_f64(double x, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Element e (0..3, lane-dependent) of v, by selection (no indexed register access).
__device__ __forceinline__ float pick4(f32x4 v, int e) {
    return e == 0 ? v[0] : e == 1 ? v[1] : e == 2 ? v[2] : v[3];
}

// g_log, beta and the q/k streams: without GATED g_log and beta are the
// per-token decay and write strength and q, k are L2-normalised by the
// caller; with GATED g_log and beta carry the raw a and b of the prologue
// and q, k are raw (A_log, dt_bias [Hv] and l2_eps are used only then).
template <typename E, int C, int DK, int BV, bool GATED, int INV>
__global__ __launch_bounds__((PipeCfg<E, C, DK, BV>::THREADS)) void gdn_prefill_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ g_log, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, float l2_eps,
    float scale, float* __restrict__ state, E* __restrict__ out,
    int Hk, int Hv, int S, int Dk, int Dv, int nvt)
{
    using Cf = PipeCfg<E, C, DK, BV>;
    using O = typename Cf::O;
    using F = typename O::F;
    using VecE = typename Vec16<E>::type;
    constexpr bool SP = Cf::SP;
    constexpr int VE = Cf::VE, LDK = Cf::LDK, LDV = Cf::LDV, LDP = Cf::LDP, ALD = Cf::ALD;
    constexpr int NT = Cf::NT, NKT = Cf::NKT, NKS = Cf::NKS;

    __shared__ __attribute__((aligned(16))) char smem[Cf::LDS_BYTES];

    // The wave index is uniform across a wave; readfirstlane makes that
    // visible to the compiler so the role branches below are scalar branches
    // (otherwise every wave would step through every role under exec masks).
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int lc = l & 15;          // column of this lane in a 16x16 accumulator tile
    const int lr = 4 * (l >> 4);    // first of its 4 rows

    // blockIdx -> (value slice, value head, batch). The workgroups that read
    // the same key/query head (the Hv/Hk value heads of a GQA group times the
    // nvt value slices) are placed on one XCD: consecutive workgroup ids go
    // round-robin over the 8 XCDs, so id L runs on XCD L % 8, and the members
    // of a group get ids L, L+8, L+16, ... That keeps q/k re-reads in one L2.
    int bid = blockIdx.x;
    const int gu = (Hv / Hk) * nvt;             // workgroups per key-head group
    if (gridDim.x % (8 * gu) == 0) {
        const int slot = bid >> 3, grp = (bid & 7) + 8 * (slot / gu);
        bid = grp * gu + slot % gu;
    }
    const int vt = bid % nvt; bid /= nvt;
    const int h = bid % Hv;
    const int b = bid / Hv;
    const int j = h / (Hv / Hk);               // GQA: contiguous groups of Hv/Hk
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
    // Any S >= 1: the last chunk may be partial. Its missing tokens read as
    // zeros (k = q = v = 0, g = beta = 0: the range check of the buffer loads
    // below), which leave the state unchanged and touch no real token's
    // output; their outputs are not stored.
    const int NC = (S + C - 1) / C;

    auto slot_ptr = [&](int c) { return smem + Cf::OFF_SLOTS + (c % Cf::NSLOT) * Cf::SZ_SLOT; };

    // ------------------------------------------------------------ stagers
    // Two stager waves split each chunk: the K stager (wave W_SK) moves K, g
    // and beta and computes gamma and the decay scalars; the QV stager (wave
    // W_SQ) moves Q and V. Loads and stores of a chunk happen in the same
    // step, so no staging registers stay live across the barrier (the
    // register file is shared by all roles).
    // Global loads are buffer loads: a buffer resource per stream (scalar
    // registers) whose size is the stream's extent, and a 32-bit lane offset
    // (the lane's column plus the row). The row goes into the lane offset, not
    // the scalar offset, so the hardware range check covers it: rows past the
    // end of the sequence read as zero without touching memory. Lanes whose
    // vector lies past a ragged Dk or Dv edge get a column offset of 2^31,
    // beyond every stream's extent (row offsets stay below 2^31), so they read
    // zeros the same way, with no select in the stores. No branches: the
    // store that follows a step later waits only for its own loads.
    constexpr int KPR = DK / VE;                 // 16-byte vectors per K/Q row
    constexpr int KRI = 64 / KPR;                // rows per load instruction
    constexpr uint32_t kOutOfRange = 0x80000000u;
    const int kd0 = (l % KPR) * VE;
    const uint32_t koff = kd0 < Dk ? (uint32_t)(((l / KPR) * Dk + kd0) * Cf::ES) : kOutOfRange;
    const int nrec_k = S * Dk * Cf::ES;
    const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, nrec_k, kBufDword3);
    const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc((void*)qb, (short)0, nrec_k, kBufDword3);
    auto load_rows = [&](VecE (&r)[Cf::NVK], __amdgpu_buffer_rsrc_t rs, int c0) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < Cf::NVK; ++n)
            r[n] = __builtin_bit_cast(VecE, __builtin_amdgcn_raw_buffer_load_b128(
                                                rs, koff + (uint32_t)((c0 + KRI * n) * Dk * Cf::ES), 0, 0));
    };
    auto store_rows = [&](VecE (&r)[Cf::NVK], E* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < Cf::NVK; ++n) {
            const int id = l + 64 * n, t = id / (DK / VE), d0 = (id % (DK / VE)) * VE;
            *(VecE*)(dst + t * LDK + d0) = r[n];
        }
    };
    struct KRegs { VecE k[Cf::NVK]; float g, b; };
    float expA = 1.f, dtb = 0.f;                 // GATED: e^{A_log[h]}, dt_bias[h] (K stager)
    const uint32_t goff = (uint32_t)min(l, C - 1) * 4;
    const __amdgpu_buffer_rsrc_t rs_g = __builtin_amdgcn_make_buffer_rsrc((void*)gb, (short)0, S * 4, kBufDword3);
    const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)bb, (short)0, S * 4, kBufDword3);
    auto stage_k_load = [&](int c, KRegs& R) __attribute__((always_inline)) {
        load_rows(R.k, rs_k, c * C);
        R.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_g, goff + (uint32_t)(c * C * 4), 0, 0));
        R.b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_b, goff + (uint32_t)(c * C * 4), 0, 0));
    };
    auto stage_k_store = [&](int c, KRegs& R) __attribute__((always_inline)) {
        char* slot = slot_ptr(c);
        store_rows(R.k, (E*)(slot + Cf::OFF_SK));
        // gamma = inclusive cumulative sum of g over the chunk, and the scalars
        float* sc = (float*)(slot + Cf::OFF_SSC);
        float gl = R.g, be = R.b;
        if constexpr (GATED) {
            // the gates of missing tokens past the end of the sequence are 0
            const bool real = c * C + l < S;
            gl = real ? -expA * softplus_f(R.g + dtb) : 0.f;
            be = real ? __builtin_amdgcn_rcpf(1.f + __expf(-R.b)) : 0.f;
        }
        // The prefix sum runs in fp64: with strong decay gamma reaches thousands
        // within a chunk, where an fp32 sum would lose ~1e-4 absolute, and the
        // decay between close tokens is a difference of two such sums. gamma
        // is kept as an fp32 pair (value, rest); e^{gamma_C - gamma} comes from
        // the fp64 difference.
        // The scan runs in registers with DPP moves: shifts by 1, 2, 4, 8 within
        // each row of 16 lanes, then row 0's total added to row 1 (lanes past
        // the chunk hold 0), instead of lane shuffles through the LDS crossbar.
        double xd = l < C ? (double)gl : 0.0;
        xd += dpp_f64<kDppRowShr + 1, 0xf>(xd);
        xd += dpp_f64<kDppRowShr + 2, 0xf>(xd);
        xd += dpp_f64<kDppRowShr + 4, 0xf>(xd);
        xd += dpp_f64<kDppRowShr + 8, 0xf>(xd);
        xd += dpp_f64<kDppRowBcast15, 0xa>(xd);
        const double gCd = readlane_f64(xd, C - 1);
        const float x = (float)xd;
        if (l < C) {
            const float eg = __expf(x);
            sc[Cf::SC_GAM + l] = x;
            sc[Cf::SC_GAML + l] = (float)(xd - (double)x);
            sc[Cf::SC_EG + l] = scale * eg;
            sc[Cf::SC_B + l] = be;
            sc[Cf::SC_BK + l] = be * eg;
            sc[Cf::SC_DL + l] = __expf((float)(gCd - xd));   // gamma_C <= gamma: never overflows
        }
        if (l == 0) sc[Cf::SC_EGC] = __expf((float)gCd);
    };
    constexpr int VPR = BV / VE;                 // 16-byte vectors per V row of the slice
    constexpr int VRI = 64 / VPR;
    const int vd0 = (l % VPR) * VE;
    const uint32_t voff = vd0 < vcols ? (uint32_t)(((l / VPR) * Dv + vd0) * Cf::ES) : kOutOfRange;
    const __amdgpu_buffer_rsrc_t rs_v =
        __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, (S * Dv - v0) * Cf::ES, kBufDword3);
    struct QVRegs { VecE q[Cf::NVK], v[Cf::NVV]; };
    auto stage_qv_load = [&](int c, QVRegs& R) __attribute__((always_inline)) {
        const int c0 = c * C;
        load_rows(R.q, rs_q, c0);
#pragma unroll
        for (int n = 0; n < Cf::NVV; ++n)
            R.v[n] = __builtin_bit_cast(VecE, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs_v, voff + (uint32_t)((c0 + VRI * n) * Dv * Cf::ES), 0, 0));
    };
    auto stage_qv_store = [&](int c, QVRegs& R) __attribute__((always_inline)) {
        char* slot = slot_ptr(c);
        store_rows(R.q, (E*)(slot + Cf::OFF_SQ));
        E* sV = (E*)(slot + Cf::OFF_SV);
#pragma unroll
        for (int n = 0; n < Cf::NVV; ++n) {
            const int id = l + 64 * n, t = id / (BV / VE), d0 = (id % (BV / VE)) * VE;
            *(VecE*)(sV + t * LDV + d0) = R.v[n];
        }
    };

    // ------------------------------------------------------------ producers
    // Per-lane gamma and factors for the rows (16 ti + lr + e) and columns
    // (16 tj + lc) of the three lower 16x16 tiles of a chunk, read once: the
    // row factor is the product of scalar arrays `rowf` and `rowf2`, the
    // column factor scalar array `colf` (each omitted when < 0).
    // gamma_r - gamma_s = (gr - gs) + (grl - gsl): the fp32 values' difference
    // (exact when close, else rounded relative to itself) plus the rests.
    struct TileScalars { float gr[2][4], grl[2][4], br[2][4], gs[2], gsl[2], cs[2]; };
    auto tile_scalars = [&](const float* sc, int rowf, int rowf2, int colf)
        __attribute__((always_inline)) {
        TileScalars ts;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            ts.gs[ti] = sc[Cf::SC_GAM + 16 * ti + lc];
            ts.gsl[ti] = sc[Cf::SC_GAML + 16 * ti + lc];
            ts.cs[ti] = colf >= 0 ? sc[colf + 16 * ti + lc] : 1.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * ti + lr + e;
                ts.gr[ti][e] = sc[Cf::SC_GAM + t];
                ts.grl[ti][e] = sc[Cf::SC_GAML + t];
                ts.br[ti][e] = (rowf >= 0 ? sc[rowf + t] : 1.f) * (rowf2 >= 0 ? sc[rowf2 + t] : 1.f);
            }
        }
        return ts;
    };
    // GATED: norm factors 1/sqrt(|x_t|^2 + eps) of the 32 tokens of a chunk
    // from the two diagonal 16x16 tiles d[0], d[1] of X X^T (X = K or Q).
    // Lane (lr/4, lc) holds rows lr + e, column lc of a tile, so the lanes
    // with lc / 4 == lr / 4 hold the diagonal, in element lc % 4: those lanes
    // form the factor of token 16 ti + lc (0 for tokens t >= nreal past the
    // end of the sequence, whose rows are zero). Other lanes fetch it by a
    // lane shuffle, never through LDS:
    //   row factors  (token 16 ti + lr + e): lane 20 (lr / 4) + e = 5 lr + e
    //   column factor (token 16 ti + lc):   lane 16 (lc / 4) + lc
    struct NormF { float row[2][4], col[2]; };
    auto norm_factors = [&](const f32x4 (&d)[2], int nreal, bool rows) __attribute__((always_inline)) {
        NormF f;
        const int src_col = 16 * (lc >> 2) + lc;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const float own = 16 * ti + lc < nreal
                                  ? __builtin_amdgcn_rsqf(pick4(d[ti], lc & 3) + l2_eps) : 0.f;
            f.col[ti] = __shfl(own, src_col);
            if (rows) {
#pragma unroll
                for (int e = 0; e < 4; ++e) f.row[ti][e] = __shfl(own, 5 * lr + e);
            }
        }
        return f;
    };

    // A = diag(beta) (K K^T) (.) Mstrict of chunk c, into A buffer c % NABUF.
    // GATED: rk from the diagonal of K K^T first, then A = diag(beta rk)
    // (K K^T) diag(rk) (.) Mstrict, and rk folded into the chunk's beta
    // e^gamma and e^{gamma_C - gamma}.
    auto build_A = [&](int c) __attribute__((always_inline)) {
        char* slot = slot_ptr(c);
        const E* __restrict__ sK = (const E*)(slot + Cf::OFF_SK);
        float* sc = (float*)(slot + Cf::OFF_SSC);
        float* __restrict__ sA = (float*)(smem + Cf::OFF_A + (c % Cf::NABUF) * Cf::SZ_F);
        // K K^T on the three lower tiles; per 32-deep step the K fragments of
        // both row tiles are loaded once and serve as both operands. Decay
        // factors e^{gamma_r - gamma_s} are only used where s < r.
        // (one base address per buffer and lane, the tile offsets as immediates)
        const uint32_t kbase = opaque_base(lds_addr(sK) + O::ldc_lane(LDK));
        f32x4 acc3[3] = {zero4(), zero4(), zero4()};
#pragma unroll
        for (int m = 0; m < NKS; ++m) {
            const F k0 = O::ldc_at(kbase, LDK, 0, 32 * m);
            const F k1 = O::ldc_at(kbase, LDK, 16, 32 * m);
            acc3[0] = O::mma(k0, k0, acc3[0]);
            acc3[1] = O::mma(k1, k0, acc3[1]);
            acc3[2] = O::mma(k1, k1, acc3[2]);
        }
        const TileScalars ts = tile_scalars(sc, Cf::SC_B, -1, -1);
        // decay factors first (they do not depend on the norms), then on the
        // GATED path rk from the diagonal tiles: the wave does not stall on
        // that chain before the exponentials are issued.
        // lane (lr/4, lc) holds rows r = lr + e, column s = lc of each tile
        f32x4 d11, d21, d22;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            d11[e] = ts.br[0][e] * __expf((ts.gr[0][e] - ts.gs[0]) + (ts.grl[0][e] - ts.gsl[0])) * ts.cs[0];
            d21[e] = ts.br[1][e] * __expf((ts.gr[1][e] - ts.gs[0]) + (ts.grl[1][e] - ts.gsl[0])) * ts.cs[0];
            d22[e] = ts.br[1][e] * __expf((ts.gr[1][e] - ts.gs[1]) + (ts.grl[1][e] - ts.gsl[1])) * ts.cs[1];
        }
        if constexpr (GATED) {
            // A[r][s] carries rk_r rk_s; rk is folded into the chunk's beta
            // e^gamma and e^{gamma_C - gamma} (lane l < C: token l, whose
            // factor is this lane's column factor of tile l / 16) and kept for
            // the P wave
            const f32x4 dg[2] = {acc3[0], acc3[2]};
            const NormF rk = norm_factors(dg, S - c * C, true);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d11[e] *= rk.row[0][e] * rk.col[0];
                d21[e] *= rk.row[1][e] * rk.col[0];
                d22[e] *= rk.row[1][e] * rk.col[1];
            }
            if (l < C) {
                const float rkl = l < 16 ? rk.col[0] : rk.col[1];
                sc[Cf::SC_RK + l] = rkl;
                sc[Cf::SC_BK + l] *= rkl;
                sc[Cf::SC_DL + l] *= rkl;
            }
        }
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)     // A11, stored transposed: [s][r], one vector per lane
            w[e] = (lc < lr + e) ? d11[e] * acc3[0][e] : 0.f;
        *(f32x4*)(sA + Cf::AB_11T + lc * ALD + lr) = w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // A21 and A22 row-major: [r][s]
            sA[Cf::AB_21 + (lr + e) * ALD + lc] = d21[e] * acc3[1][e];
            sA[Cf::AB_22 + (lr + e) * ALD + lc] = (lc < lr + e) ? d22[e] * acc3[2][e] : 0.f;
        }
    };

    // Inverse wave: T = (I + A)^{-1} of chunk c from A buffer c % NABUF.
    //
    // Diagonal blocks by substitution in fp32, four lanes per column: lane
    // (j, q) = (l / 4, l % 4) holds rows 4q .. 4q+3 of column j. Step s needs
    // the finished unknown s of every column, which lives in quarter s / 4 of
    // the column's quad: a DPP quad broadcast hands it to the four lanes, and
    // each lane updates its four rows with the coefficients of step s (zero
    // where the triangle has none, so every lane runs the same instructions).
    //  * T11 = (I + A11)^{-1} column j, forward (s = 0 .. 14):
    //      x_r -= A11[r][s] x_s,  coefficients A11[4q..4q+3][s] = row s of
    //      the transposed A11 block;
    //  * T22^T = (I + A22^T)^{-1} column j, i.e. row j of T22, backward
    //      (s = 15 .. 1): y_r -= A22[s][r] y_s, coefficients A22[s][4q..4q+3]
    //      = row s of the row-major A22 block.
    // The two chains run in the same loop, and their 16-byte coefficient rows
    // are read LA steps ahead.
    //
    // Merge: T21 = -T22 (A21 T11) on fp32 MFMA (16x16x4, four steps). The
    // contraction index of step s for lane group g is 4g + s, so the B operand
    // of X = A21 T11 is T11[4g+s][n] (column n) and the A operand of T22 X is
    // T22[i][4g+s] = T22^T[4g+s][i]: both are element s of the substitution
    // results after one lane permutation (lane 16g + n takes lane 4n + g).
    const int jq = l >> 2, qq = l & 3;            // substitution lane roles: column, quarter
    auto t_solve = [&](int c, f32x4 (&x)[2]) __attribute__((always_inline)) {
        const float* __restrict__ sA = (const float*)(smem + Cf::OFF_A + (c % Cf::NABUF) * Cf::SZ_F);
        constexpr int LA = 4;
        const uint32_t ab = opaque_base(lds_addr(sA) + (uint32_t)(4 * qq * 4));
        f32x4 ca[LA + 1], cb[LA + 1];
        auto coef = [&](int t, f32x4& a, f32x4& b) {
            a = *lds_ptr<const f32x4>(ab + (uint32_t)((Cf::AB_11T + t * ALD) * 4));
            b = *lds_ptr<const f32x4>(ab + (uint32_t)((Cf::AB_22 + (15 - t) * ALD) * 4));
        };
#pragma unroll
        for (int t = 0; t < LA; ++t) coef(t, ca[t], cb[t]);
        f32x4 xa, yb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xa[e] = 4 * qq + e == jq ? 1.f : 0.f;
            yb[e] = xa[e];
        }
#pragma unroll
        for (int t = 0; t < 15; ++t) {
            if (t + LA < 15) coef(t + LA, ca[(t + LA) % (LA + 1)], cb[(t + LA) % (LA + 1)]);
            const int sa = t, sb = 15 - t;
            const float xs = quad_bcast(xa[sa & 3], sa >> 2);
            const float ys = quad_bcast(yb[sb & 3], sb >> 2);
            const f32x4 a = ca[t % (LA + 1)], b = cb[t % (LA + 1)];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xa[e] -= a[e] * xs;
                yb[e] -= b[e] * ys;
            }
        }
        x[0] = xa;
        x[1] = yb;
        // Diagonal blocks into the T buffer, rows [t][hi tpos(s) | lo tpos(s)]
        // (fp32: [t][tpos(s)]): T11[4q+e][j] at row 4q + e, column tpos(j);
        // row j of T22, columns 16 + 4q .. 16 + 4q + 3, at row 16 + j, columns
        // tpos(16 + 4q + e) = 8q + 4 + e.
        E* __restrict__ Tp = (E*)(smem + Cf::OFF_T + (c % Cf::NTBUF) * Cf::SZ_TP);
#pragma unroll
        for (int e = 0; e < 4; ++e) store_pair<SP>(Tp + (4 * qq + e) * LDP + tpos(jq), C, xa[e]);
        E* p22 = Tp + (16 + jq) * LDP + 8 * qq + 4;
        if constexpr (SP) {
            uint32_t h0, l0, h1, l1;
            split2(yb[0], yb[1], h0, l0);
            split2(yb[2], yb[3], h1, l1);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            *(u32x2*)p22 = u32x2{h0, h1};
            *(u32x2*)(p22 + C) = u32x2{l0, l1};
        } else {
            *(f32x4*)p22 = yb;
        }
    };

    auto t_merge = [&](int c, const f32x4 (&x)[2]) __attribute__((always_inline)) {
        const float* __restrict__ sA = (const float*)(smem + Cf::OFF_A + (c % Cf::NABUF) * Cf::SZ_F);
        E* __restrict__ Tp = (E*)(smem + Cf::OFF_T + (c % Cf::NTBUF) * Cf::SZ_TP);
        const f32x4 a21 = *(const f32x4*)(sA + Cf::AB_21 + lc * ALD + lr);   // A21[lc][lr..lr+3]
        // lane 16g + n takes element s of lane 4n + g
        const int src = 4 * (4 * lc + (lr >> 2));
        float b11[4], a22[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            b11[s2] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, (float)x[0][s2])));
            a22[s2] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, (float)x[1][s2])));
        }
        f32x4 X = zero4();
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) X = __builtin_amdgcn_mfma_f32_16x16x4f32(a21[s2], b11[s2], X, 0, 0, 0);
        f32x4 Y = zero4();
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a22[s2], X[s2], Y, 0, 0, 0);
        // T21 rows 16 + 4g + e, column n
#pragma unroll
        for (int e = 0; e < 4; ++e) store_pair<SP>(Tp + (16 + lr + e) * LDP + tpos(lc), C, -Y[e]);
    };

    // Neumann inverse (INV == 1). 16x16 matrices live in the accumulator
    // layout: lane (j, g) = (l % 16, l / 16) holds rows 4g .. 4g+3 of column j.
    // A product L R takes L^T and R in that layout: step s pairs lane group
    // g's k = 4g + s on both sides, so the A operand is element s of L^T's
    // vector and the B operand element s of R's. Keeping every factor and
    // its transpose in registers, all products chain without any exchange.
    auto mm4 = [&](f32x4 Lt, f32x4 R, f32x4 acc) __attribute__((always_inline)) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Lt[s2], R[s2], acc, 0, 0, 0);
        return acc;
    };
    // (I + P)^{-1} for nilpotent P, from P and P^T: with X = -P,
    // T = (I + X)(I + X^2)(I + X^4)(I + X^8), accumulated as T <- T + T X^(2^m).
    auto neumann16 = [&](f32x4 P, f32x4 Pt) __attribute__((always_inline)) {
        f32x4 id;
#pragma unroll
        for (int e = 0; e < 4; ++e) id[e] = (lc == lr + e) ? 1.f : 0.f;
        const f32x4 X = -P, Xt = -Pt;
        const f32x4 X2 = mm4(Xt, X, zero4()), X2t = mm4(X, Xt, zero4());
        const f32x4 T1 = id + X, T1t = id + Xt;
        const f32x4 T2 = mm4(T1t, X2, T1), T2t = mm4(X2, T1t, T1t);
        const f32x4 X4 = mm4(X2t, X2, zero4()), X4t = mm4(X2, X2t, zero4());
        const f32x4 T4 = mm4(T2t, X4, T2), T4t = mm4(X4, T2t, T2t);
        const f32x4 X8 = mm4(X4t, X4, zero4());
        return mm4(T4t, X8, T4);
    };
    // T11 and T22^T of chunk c (both in the accumulator layout) into tl, and
    // the diagonal blocks into the T buffer.
    auto n_solve = [&](int c, f32x4 (&tl)[2]) __attribute__((always_inline)) {
        const float* __restrict__ sA = (const float*)(smem + Cf::OFF_A + (c % Cf::NABUF) * Cf::SZ_F);
        const float* A11t = sA + Cf::AB_11T;   // [s][r] = A11[r][s]
        const float* A22 = sA + Cf::AB_22;     // row-major
        const f32x4 a11 = *(const f32x4*)(A11t + lc * ALD + lr);          // A11[lr+e][lc]
        f32x4 a11t, a22;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a11t[e] = A11t[(lr + e) * ALD + lc];                           // A11[lc][lr+e]
            a22[e] = A22[(lr + e) * ALD + lc];                              // A22[lr+e][lc]
        }
        const f32x4 a22t = *(const f32x4*)(A22 + lc * ALD + lr);          // A22[lc][lr+e]
        tl[0] = neumann16(a11, a11t);                                       // T11
        tl[1] = neumann16(a22t, a22);                                       // (I + A22^T)^{-1} = T22^T
        E* __restrict__ Tp = (E*)(smem + Cf::OFF_T + (c % Cf::NTBUF) * Cf::SZ_TP);
        // T11[lr+e][lc]: row lr+e, column tpos(lc); T22[lc][lr+e]: row 16+lc, columns 8g+4 ..
#pragma unroll
        for (int e = 0; e < 4; ++e) store_pair<SP>(Tp + (lr + e) * LDP + tpos(lc), C, tl[0][e]);
        if constexpr (SP) {
            uint32_t h0, l0, h1, l1;
            split2(tl[1][0], tl[1][1], h0, l0);
            split2(tl[1][2], tl[1][3], h1, l1);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            E* p = Tp + (16 + lc) * LDP + 2 * lr + 4;
            *(u32x2*)p = u32x2{h0, h1};
            *(u32x2*)(p + C) = u32x2{l0, l1};
        } else {
            *(f32x4*)(Tp + (16 + lc) * LDP + 2 * lr + 4) = tl[1];
        }
    };
    // T21 = -T22 (A21 T11) of chunk c from the registers n_solve left.
    auto n_merge = [&](int c, const f32x4 (&tl)[2]) __attribute__((always_inline)) {
        const float* __restrict__ sA = (const float*)(smem + Cf::OFF_A + (c % Cf::NABUF) * Cf::SZ_F);
        E* __restrict__ Tp = (E*)(smem + Cf::OFF_T + (c % Cf::NTBUF) * Cf::SZ_TP);
        const f32x4 a21 = *(const f32x4*)(sA + Cf::AB_21 + lc * ALD + lr);  // A21[lc][lr+e]
        const f32x4 Xm = mm4(a21, tl[0], zero4());                          // A21 T11
        const f32x4 Y = mm4(tl[1], Xm, zero4());                            // T22 (A21 T11)
        // T21 rows 16 + lr + e, column lc
#pragma unroll
        for (int e = 0; e < 4; ++e) store_pair<SP>(Tp + (16 + lr + e) * LDP + tpos(lc), C, -Y[e]);
    };

    // P wave: P = scale (Q K^T (.) Mincl). GATED: rq from the diagonal of
    // Q Q^T, P = scale diag(rq) (Q K^T) diag(rk) (.) Mincl, and rq folded into
    // the chunk's scale e^gamma. rk comes from the A builder, which finished
    // this chunk at least one step earlier on the bf16 path; on the fp32 path
    // it runs in the same step, so the P wave forms its own copy.
    auto build_P = [&](int c) __attribute__((always_inline)) {
        char* slot = slot_ptr(c);
        const E* __restrict__ sK = (const E*)(slot + Cf::OFF_SK);
        const E* __restrict__ sQ = (const E*)(slot + Cf::OFF_SQ);
        float* sc = (float*)(slot + Cf::OFF_SSC);
        E* __restrict__ Pp = (E*)(smem + Cf::OFF_P + (c & 1) * Cf::SZ_TP);
        F kf[2][NKS], qf[2][NKS];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
                kf[t2][m] = O::ldc(sK, LDK, 16 * t2, 32 * m);
                qf[t2][m] = O::ldc(sQ, LDK, 16 * t2, 32 * m);
            }
        // The scalars' "row" arrays index keys and "column" arrays queries
        // (tiles of K Q^T below): rk for the rows, rq for the columns.
        const TileScalars ts = tile_scalars(sc, (GATED && Cf::SPREAD) ? Cf::SC_RK : -1, -1, -1);
        // GATED: the diagonal Q Q^T tiles for rq (and, on the fp32 path, K K^T
        // for rk) are issued first; their factors are formed after the tile
        // products and the decays, which do not depend on them, so the wave
        // does not stall on that chain before issuing independent work.
        f32x4 dq[2] = {zero4(), zero4()}, dk[2] = {zero4(), zero4()};
        if constexpr (GATED) {
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int m = 0; m < NKS; ++m) {
                    dq[ti] = O::mma(qf[ti][m], qf[ti][m], dq[ti]);
                    if constexpr (!Cf::SPREAD) dk[ti] = O::mma(kf[ti][m], kf[ti][m], dk[ti]);
                }
        }
        // Tiles of (Q K^T)^T = K Q^T: lane (lr/4, lc) holds keys s = 16 tj + lr + e
        // of query row r = 16 ti + lc, which are adjacent in P's row layout
        // (tpos(s) = 8 (lr/4) + 4 tj + e), so each tile is stored as one
        // 8-byte vector per lane (hi and, on the bf16 path, lo).
        f32x4 acc[3], dec[3];
#pragma unroll
        for (int tt = 0; tt < 3; ++tt) {
            const int ti = tt == 0 ? 0 : 1, tj = tt == 2 ? 1 : 0;
            acc[tt] = zero4();
#pragma unroll
            for (int m = 0; m < NKS; ++m) acc[tt] = O::mma(kf[tj][m], qf[ti][m], acc[tt]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dec[tt][e] = scale * ts.br[tj][e] * ts.cs[ti] *
                             __expf((ts.gs[ti] - ts.gr[tj][e]) + (ts.gsl[ti] - ts.grl[tj][e]));
        }
        float colf[2] = {1.f, 1.f}, rowf[2][4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
        if constexpr (GATED) {
            const NormF rq = norm_factors(dq, S - c * C, false);
            colf[0] = rq.col[0];
            colf[1] = rq.col[1];
            if constexpr (!Cf::SPREAD) {
                const NormF rk = norm_factors(dk, S - c * C, true);
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int e = 0; e < 4; ++e) rowf[ti][e] = rk.row[ti][e];
            }
            if (l < C) sc[Cf::SC_EG + l] *= l < 16 ? rq.col[0] : rq.col[1];
        }
#pragma unroll
        for (int tt = 0; tt < 3; ++tt) {
            const int ti = tt == 0 ? 0 : 1, tj = tt == 2 ? 1 : 0;
            const int r = 16 * ti + lc;
            f32x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s2 = 16 * tj + lr + e;
                pv[e] = (s2 <= r) ? dec[tt][e] * (colf[ti] * rowf[tj][e]) * acc[tt][e] : 0.f;
            }
            E* dst = Pp + r * LDP + 8 * (lr >> 2) + 4 * tj;
            if constexpr (SP) {
                uint32_t h0, l0, h1, l1;
                split2(pv[0], pv[1], h0, l0);
                split2(pv[2], pv[3], h1, l1);
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                *(u32x2*)dst = u32x2{h0, h1};
                *(u32x2*)(dst + C) = u32x2{l0, l1};
            } else {
                *(f32x4*)dst = pv;
            }
        }
    };

    // ------------------------------------------------------------ consumers
    const int strip = Cf::PAIR ? wave >> 1 : wave;   // 16-column strip of a consumer wave
    const int vl = 16 * strip + lc;            // column of this lane within the slice
    const bool vok = wave < Cf::NCWW && vl < vcols;
    const bool wok = wave < Cf::NCWW && 16 * strip < vcols;   // this wave's 16 output columns exist
    // accS[kt]: state rows spos(kt, lr/4, e), column vl, held for the whole sequence
    // Operands of chunk i that a consumer reads ahead, during the output phase
    // of chunk i - 1 (before the barrier between them): the first 32-deep K
    // and Q fragments and, on the bf16 path, V, beta and beta e^gamma of this
    // lane's rows t = 16 ti + lr + e. The slot of chunk i was stored several
    // steps earlier and is not written again until step i + 1; beta e^gamma
    // (folded with rk on the GATED path) was final when the A wave finished
    // chunk i, three steps ahead. On the fp32 path the A wave builds chunk i
    // during step i - 1, so those scalars are read at the start of step i.
    // kb, sb: this lane's K/Q fragment and row-scalar addresses in the slot.
    struct ConsPre { F kf[NT], qf[NT]; float vv[NT][4], bt[NT][4], bk[NT][4]; uint32_t kb, sb; };
    // A consumer's reads of a chunk follow a few per-lane patterns. Each gets
    // one address register per chunk (the slot's offset plus the lane's
    // loop-invariant offset, opaque to the optimiser), and every tile of the
    // pattern is an immediate offset from it.
    const uint32_t smem_a = lds_addr(smem);
    const uint32_t c_kq = O::ldc_lane(LDK);                       // K/Q fragments
    const uint32_t c_kt = O::ldt_lane(LDK, 0);                    // transposed K
    const uint32_t c_tp = O::ldc_lane(LDP);                       // T and P fragments
    const uint32_t c_v = (uint32_t)((lr * LDV + vl) * Cf::ES);     // V rows lr.., column vl
    // PAIR: consumer wave h holds key rows 64h .. 64h+63, i.e. the 32-deep
    // steps m = 2h, 2h+1 of K S0 and Q S0 and state tiles kt = 4h .. 4h+3.
    const uint32_t kq0 = Cf::PAIR ? (uint32_t)(64 * (wave & 1) * Cf::ES) : 0u;
    auto slot_a = [&](int c) { return smem_a + (uint32_t)(Cf::OFF_SLOTS + (c % Cf::NSLOT) * Cf::SZ_SLOT); };
    auto cons_scalars = [&](int i, ConsPre& p) __attribute__((always_inline)) {
        const uint32_t sa = slot_a(i);
        const uint32_t vb = opaque_base(sa + Cf::OFF_SV + c_v);
        p.sb = opaque_base(sa + Cf::OFF_SSC + (uint32_t)(lr * 4));
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            const f32x4 bt4 = *lds_ptr<const f32x4>(p.sb + (uint32_t)((Cf::SC_B + 16 * ti) * 4));
            const f32x4 bk4 = *lds_ptr<const f32x4>(p.sb + (uint32_t)((Cf::SC_BK + 16 * ti) * 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p.vv[ti][e] = to_f32(*lds_ptr<const E>(vb + (uint32_t)((16 * ti + e) * LDV * Cf::ES)));
                p.bt[ti][e] = bt4[e];
                p.bk[ti][e] = bk4[e];
            }
        }
    };
    auto cons_prefetch = [&](int i, ConsPre& p) __attribute__((always_inline)) {
        p.kb = opaque_base(slot_a(i) + Cf::OFF_SK + c_kq + kq0);
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            p.kf[ti] = O::ldc_at(p.kb, LDK, 16 * ti, 0);
            p.qf[ti] = O::ldc_at(p.kb + Cf::SZ_K, LDK, 16 * ti, 0);
        }
        if constexpr (Cf::SPREAD) cons_scalars(i, p);
    };
    // the packed dot-product factors of split2_last, in scalar registers
    uint32_t dm0 = kDotNegLo, dm1 = kDotNegHi;
    asm volatile("" : "+s"(dm0), "+s"(dm1));
    auto consume = [&](int i, f32x4 (&accS)[NKT], ConsPre& pre) __attribute__((always_inline)) {
        const uint32_t sa = slot_a(i);
        const uint32_t tb = opaque_base(smem_a + (uint32_t)(Cf::OFF_T + (i % Cf::NTBUF) * Cf::SZ_TP) + c_tp);
        const uint32_t pb = opaque_base(smem_a + (uint32_t)(Cf::OFF_P + (i & 1) * Cf::SZ_TP) + c_tp);
        const int c0 = i * C;
        if constexpr (!Cf::SPREAD) cons_scalars(i, pre);
        const uint32_t kqb = pre.kb, srb = pre.sb;
        // scale e^gamma of token 16 ti + lc (folded with rq by the P wave during
        // step i - 1 on the GATED path) and e^{gamma_C}
        const uint32_t eb = opaque_base(sa + Cf::OFF_SSC + (uint32_t)(lc * 4));
        float egt[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) egt[ti] = *lds_ptr<const float>(eb + (uint32_t)((Cf::SC_EG + 16 * ti) * 4));
        const float egC = *lds_ptr<const float>(sa + (uint32_t)((Cf::OFF_SSC / 4 + Cf::SC_EGC) * 4));
        // LDS operands are read ahead of the products that use them: the
        // first 32-deep K and Q slice and the row scalars during the previous
        // chunk's output phase, each further slice one stage ahead, then T;
        // the transposed K tiles and e^{gamma_C - gamma} right after K S0;
        // P before the state update. A scheduling barrier after each batch of
        // reads keeps the compiler from sinking them back next to their use,
        // while arithmetic is still free to move across it.
        // K S0 ([token][value column] tiles) and (Q S0)^T ([value column][token]
        // tiles: the same fragments with the operands swapped), S0 from registers
        f32x4 ks[NT], qs[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) { ks[ti] = zero4(); qs[ti] = zero4(); }
        F kf[2][NT], qf[2][NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            kf[0][ti] = pre.kf[ti];
            qf[0][ti] = pre.qf[ti];
        }
        F tf[NT][2];
#pragma unroll
        for (int m = 0; m < NKS; ++m) {
            const int cb = m & 1, nb = cb ^ 1;
            if (m + 1 < NKS) {
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) {
                    kf[nb][ti] = O::ldc_at(kqb, LDK, 16 * ti, 32 * (m + 1));
                    qf[nb][ti] = O::ldc_at(kqb + Cf::SZ_K, LDK, 16 * ti, 32 * (m + 1));
                }
            } else {
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) {
                    tf[ti][0] = O::ldc_at(tb, LDP, 16 * ti, 0);
                    if constexpr (SP) tf[ti][1] = O::ldc_at(tb, LDP, 16 * ti, C);
                }
            }
            __builtin_amdgcn_sched_barrier(kComputeMayCross);
            F sh, sl;
            O::split(accS[2 * m], accS[2 * m + 1], sh, sl);
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
                if constexpr (SP) {
                    ks[ti] = O::mma(kf[cb][ti], sl, ks[ti]);
                    qs[ti] = O::mma(sl, qf[cb][ti], qs[ti]);
                }
                ks[ti] = O::mma(kf[cb][ti], sh, ks[ti]);
                qs[ti] = O::mma(sh, qf[cb][ti], qs[ti]);
            }
        }
        // All transposed K tiles of the state update, issued now (into the
        // registers the K and Q fragments held) so that they arrive during R
        // and U; one base address for all tiles, the offsets as immediates.
        const uint32_t ktb = opaque_base(sa + Cf::OFF_SK + c_kt);
        F kt_f[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) kt_f[kt] = O::ldt_at(ktb, LDK, kt);
        float dl[NT][4];                               // e^{gamma_C - gamma} of this lane's rows
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            const f32x4 d4 = *lds_ptr<const f32x4>(srb + (uint32_t)((Cf::SC_DL + 16 * ti) * 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) dl[ti][e] = d4[e];
        }
        __builtin_amdgcn_sched_barrier(kComputeMayCross);
        // R = beta V - beta e^gamma (K S0)
        f32x4 r[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti)
#pragma unroll
            for (int e = 0; e < 4; ++e) r[ti][e] = pre.bt[ti][e] * pre.vv[ti][e] - pre.bk[ti][e] * ks[ti][e];
        F rh, rl;
        O::template split<true>(r[0], r[1], rh, rl, dm0, dm1);
        // U = T R
        f32x4 u[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            u[ti] = zero4();
            if constexpr (SP) {
                u[ti] = O::mma(tf[ti][1], rh, u[ti]);
                u[ti] = O::mma(tf[ti][0], rl, u[ti]);
            }
            u[ti] = O::mma(tf[ti][0], rh, u[ti]);
        }
        // S = e^{gamma_C} S0 + K^T diag(e^{gamma_C - gamma}) U
        f32x4 ud[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti)
#pragma unroll
            for (int e = 0; e < 4; ++e) ud[ti][e] = u[ti][e] * dl[ti][e];
        F dh, dlo;
        O::template split<true>(ud[0], ud[1], dh, dlo, dm0, dm1);
        // P of the output, read while the state update runs
        F pf[NT][2];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            pf[ti][0] = O::ldc_at(pb, LDP, 16 * ti, 0);
            if constexpr (SP) pf[ti][1] = O::ldc_at(pb, LDP, 16 * ti, C);
        }
        __builtin_amdgcn_sched_barrier(kComputeMayCross);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) accS[kt][e] *= egC;
            if constexpr (SP) accS[kt] = O::mma(kt_f[kt], dlo, accS[kt]);
            accS[kt] = O::mma(kt_f[kt], dh, accS[kt]);
        }
        // the next chunk's first operands, read during the output phase
        cons_prefetch(i + 1, pre);
        // O^T = (Q S0)^T diag(scale e^gamma) + U^T P^T (P carries the scale):
        // lane (g, n) holds 4 consecutive value columns 4g.. of token 16 ti + n,
        // stored as one vector.
        F uh, ul;
        O::template split<true>(u[0], u[1], uh, ul, dm0, dm1);
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = qs[ti][e] * egt[ti];
            if constexpr (SP) {
                o = O::mma(uh, pf[ti][1], o);
                o = O::mma(ul, pf[ti][0], o);
            }
            o = O::mma(uh, pf[ti][0], o);
            if (wok && c0 + 16 * ti + lc < S) {         // tokens past the end are not stored
                E* dst = ob + (size_t)(c0 + 16 * ti + lc) * Dv + 16 * wave + lr;
                if constexpr (SP) {
                    *(bf16x4*)dst = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
                } else {
                    *(f32x4*)dst = o;
                }
            }
        }
    };

    // PAIR consumer wave h (0 or 1) of chunk i: the same steps as consume()
    // on key rows 64h .. 64h+63 (accS holds state tiles 4h .. 4h+3). Its
    // partial K S0 (both token tiles) and Q S0 (the other wave's output tile)
    // go to LDS, a step counter is released, and the other wave's partials are
    // added once its counter shows this step; both waves then hold the same
    // K S0 (a + b = b + a), form the same R and U, update their own rows and
    // store output token tile h.
    auto consume_pair = [&](int i, f32x4 (&accS)[Cf::NKTW], ConsPre& pre, int h) __attribute__((always_inline)) {
        const uint32_t sa = slot_a(i);
        const uint32_t tb = opaque_base(smem_a + (uint32_t)(Cf::OFF_T + (i % Cf::NTBUF) * Cf::SZ_TP) + c_tp);
        const uint32_t pb = opaque_base(smem_a + (uint32_t)(Cf::OFF_P + (i & 1) * Cf::SZ_TP) + c_tp +
                                        (uint32_t)(16 * h * LDP * Cf::ES));
        const int c0 = i * C;
        const uint32_t kqb = pre.kb, srb = pre.sb;
        const uint32_t eb = opaque_base(sa + Cf::OFF_SSC + (uint32_t)((16 * h + lc) * 4));
        const float egh = *lds_ptr<const float>(eb + (uint32_t)(Cf::SC_EG * 4));
        const float egC = *lds_ptr<const float>(sa + (uint32_t)((Cf::OFF_SSC / 4 + Cf::SC_EGC) * 4));
        f32x4 ks[NT], qs[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) { ks[ti] = zero4(); qs[ti] = zero4(); }
        F kf[2][NT], qf[2][NT], tf[NT][2];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            kf[0][ti] = pre.kf[ti];
            qf[0][ti] = pre.qf[ti];
            kf[1][ti] = O::ldc_at(kqb, LDK, 16 * ti, 32);
            qf[1][ti] = O::ldc_at(kqb + Cf::SZ_K, LDK, 16 * ti, 32);
        }
        __builtin_amdgcn_sched_barrier(kComputeMayCross);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (m == 1) {
#pragma unroll
                for (int ti = 0; ti < NT; ++ti) {
                    tf[ti][0] = O::ldc_at(tb, LDP, 16 * ti, 0);
                    tf[ti][1] = O::ldc_at(tb, LDP, 16 * ti, C);
                }
                __builtin_amdgcn_sched_barrier(kComputeMayCross);
            }
            F sh, sl;
            O::split(accS[2 * m], accS[2 * m + 1], sh, sl);
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
                ks[ti] = O::mma(kf[m][ti], sl, ks[ti]);
                qs[ti] = O::mma(sl, qf[m][ti], qs[ti]);
                ks[ti] = O::mma(kf[m][ti], sh, ks[ti]);
                qs[ti] = O::mma(sh, qf[m][ti], qs[ti]);
            }
        }
        // exchange: this wave's block, the partner's (wave ^ 1) block
        const uint32_t xo = smem_a + (uint32_t)(Cf::OFF_X + wave * Cf::SZ_XW + l * 16);
        const uint32_t xp = smem_a + (uint32_t)(Cf::OFF_X + (wave ^ 1) * Cf::SZ_XW + l * 16);
        int* flags = (int*)(smem + Cf::OFF_XF);
        *lds_ptr<f32x4>(xo) = ks[0];
        *lds_ptr<f32x4>(xo + 1024) = ks[1];
        *lds_ptr<f32x4>(xo + 2048) = h ? qs[0] : qs[1];
        __hip_atomic_store(&flags[wave], i + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        // the transposed K tiles of this wave's rows and e^{gamma_C - gamma}
        // are read while the other wave finishes its half
        const uint32_t ktb = opaque_base(sa + Cf::OFF_SK + c_kt + (uint32_t)(64 * h * Cf::ES));
        F kt_f[Cf::NKTW];
#pragma unroll
        for (int kt = 0; kt < Cf::NKTW; ++kt) kt_f[kt] = O::ldt_at(ktb, LDK, kt);
        float dl[NT][4];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            const f32x4 d4 = *lds_ptr<const f32x4>(srb + (uint32_t)((Cf::SC_DL + 16 * ti) * 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) dl[ti][e] = d4[e];
        }
        // Bounded wait for the other wave's counter: it always arrives (both
        // waves run the same steps), and the bound keeps every wave finite.
        for (int spin = 0; spin < (1 << 22); ++spin) {
            if (__hip_atomic_load(&flags[wave ^ 1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) > i) break;
        }
        const f32x4 pk0 = *lds_ptr<const f32x4>(xp);
        const f32x4 pk1 = *lds_ptr<const f32x4>(xp + 1024);
        const f32x4 pq = *lds_ptr<const f32x4>(xp + 2048);
        ks[0] += pk0;
        ks[1] += pk1;
        const f32x4 qh = (h ? qs[1] : qs[0]) + pq;
        __builtin_amdgcn_sched_barrier(kComputeMayCross);
        // R = beta V - beta e^gamma (K S0), U = T R (both token tiles)
        f32x4 r[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti)
#pragma unroll
            for (int e = 0; e < 4; ++e) r[ti][e] = pre.bt[ti][e] * pre.vv[ti][e] - pre.bk[ti][e] * ks[ti][e];
        F rh, rl;
        O::template split<true>(r[0], r[1], rh, rl, dm0, dm1);
        f32x4 u[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            u[ti] = zero4();
            u[ti] = O::mma(tf[ti][1], rh, u[ti]);
            u[ti] = O::mma(tf[ti][0], rl, u[ti]);
            u[ti] = O::mma(tf[ti][0], rh, u[ti]);
        }
        f32x4 ud[NT];
#pragma unroll
        for (int ti = 0; ti < NT; ++ti)
#pragma unroll
            for (int e = 0; e < 4; ++e) ud[ti][e] = u[ti][e] * dl[ti][e];
        F dh, dlo;
        O::template split<true>(ud[0], ud[1], dh, dlo, dm0, dm1);
        // P rows of output tile h, read while the state update runs
        const F p0 = O::ldc_at(pb, LDP, 0, 0);
        const F p1 = O::ldc_at(pb, LDP, 0, C);
        __builtin_amdgcn_sched_barrier(kComputeMayCross);
#pragma unroll
        for (int kt = 0; kt < Cf::NKTW; ++kt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) accS[kt][e] *= egC;
            accS[kt] = O::mma(kt_f[kt], dlo, accS[kt]);
            accS[kt] = O::mma(kt_f[kt], dh, accS[kt]);
        }
        cons_prefetch(i + 1, pre);
        F uh, ul;
        O::template split<true>(u[0], u[1], uh, ul, dm0, dm1);
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = qh[e] * egh;
        o = O::mma(uh, p1, o);
        o = O::mma(ul, p0, o);
        o = O::mma(uh, p0, o);
        if (wok && c0 + 16 * h + lc < S) {
            E* dst = ob + (size_t)(c0 + 16 * h + lc) * Dv + 16 * strip + lr;
            if constexpr (SP) *(bf16x4*)dst = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
            else *(f32x4*)dst = o;
        }
    };

    // ------------------------------------------------------------ schedule
    // Each role runs its own program: three prologue barriers, then one
    // barrier per step i = 0 .. NC-1. Values a role carries from step to step
    // occupy registers only in that role's code.
    //   consumers         chunk i
    //   P wave            P of chunk i+1
    //   stagers           store chunk i+LEAD (loaded during step i-1), load chunk i+LEAD+1
    //  SPREAD:
    //   A wave            A of chunk i+3
    //   inverse wave i%2  substitution for chunk i+2 (result kept in registers)
    //   other inverse     merge and T stores for chunk i+1
    //  otherwise:
    //   inverse wave      A, substitution, merge and T stores for chunk i+1
    // The upper-right 16x16 blocks of T and P are zero for every chunk; they
    // are written once, for both buffers of each.
    for (int id = threadIdx.x; id < (Cf::NTBUF + 2) * 256; id += Cf::THREADS) {
        const int which = id >> 8, r = (id >> 4) & 15, col = tpos(16 + (id & 15));
        E* base = (E*)(smem + (which < Cf::NTBUF ? Cf::OFF_T + which * Cf::SZ_TP
                                                 : Cf::OFF_P + (which - Cf::NTBUF) * Cf::SZ_TP));
        store_pair<SP>(base + r * LDP + col, C, 0.f);
    }

    if constexpr (Cf::PAIR) {
        if ((int)threadIdx.x < Cf::NCWW) ((int*)(smem + Cf::OFF_XF))[threadIdx.x] = 0;   // exchange step counters
    }

    if (wave < Cf::NCWW) {
        // state tiles kt0 .. kt0 + NKTW - 1 of the strip (all of them unless PAIR)
        const int kt0 = Cf::PAIR ? Cf::NKTW * (wave & 1) : 0;
        f32x4 accS[Cf::NKTW];
#pragma unroll
        for (int kt = 0; kt < Cf::NKTW; ++kt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dk = spos(kt0 + kt, lr >> 2, e);
                accS[kt][e] = (vok && dk < Dk) ? sb[(size_t)dk * Dv + vl] : 0.f;
            }
        }
        __syncthreads();
        __syncthreads();
        __syncthreads();
        ConsPre pre;
        cons_prefetch(0, pre);
        for (int i = 0; i < NC; ++i) {
            if constexpr (Cf::PAIR) consume_pair(i, accS, pre, wave & 1);
            else consume(i, accS, pre);
            // The only LDS reads a consumer may still have in flight here are
            // the prefetches of chunk i + 1, whose slot no wave writes before
            // step i + 2 (a PAIR wave's exchange reads were consumed within
            // the step, and its exchange writes precede its counter release):
            // they pass the barrier without waiting for those reads (a
            // compiler-only fence keeps every LDS access on its side of it).
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
        if (vok) {
#pragma unroll
            for (int kt = 0; kt < Cf::NKTW; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int dk = spos(kt0 + kt, lr >> 2, e);
                    if (dk < Dk) sb[(size_t)dk * Dv + vl] = accS[kt][e];
                }
        }
    } else if (wave == Cf::W_T0 || wave == Cf::W_T1) {
        const int pw = wave == Cf::W_T0 ? 0 : 1;
        // the solve result waits in registers for the merge
        f32x4 x[2];
        auto solve = [&](int c) __attribute__((always_inline)) {
            if constexpr (INV == 0) t_solve(c, x); else n_solve(c, x);
        };
        auto merge = [&](int c) __attribute__((always_inline)) {
            if constexpr (INV == 0) t_merge(c, x); else n_merge(c, x);
        };
        __syncthreads();
        if constexpr (!Cf::SPREAD) {
            if (NC > 0) { build_A(0); wave_lds_fence(); solve(0); merge(0); }
        } else {
            if (NC > 1 + pw) build_A(1 + pw);          // beside the A wave's chunk 0
        }
        __syncthreads();
        if constexpr (Cf::SPREAD) {
            if (pw == 0 && NC > 0) { solve(0); merge(0); }
            if (pw == 1 && NC > 1) solve(1);
        }
        __syncthreads();
        for (int i = 0; i < NC; ++i) {
            if constexpr (Cf::SPREAD) {
                if ((i & 1) == pw) {
                    if (i + 2 < NC) solve(i + 2);
                } else {
                    if (i + 1 < NC) merge(i + 1);
                }
            } else {
                if (i + 1 < NC) { build_A(i + 1); wave_lds_fence(); solve(i + 1); merge(i + 1); }
            }
            __syncthreads();
        }
    } else if (wave == Cf::W_P) {
        // P of chunk 0 after the second barrier: on the GATED bf16 path it
        // reads the norms the A wave forms between the first two.
        __syncthreads();
        __syncthreads();
        if (NC > 0) build_P(0);
        __syncthreads();
        for (int i = 0; i < NC; ++i) {
            if (i + 1 < NC) build_P(i + 1);
            __syncthreads();
        }
    } else if (wave == Cf::W_A) {
        // A of chunks 0, 1, 2 between the first two barriers: chunk 0 here,
        // chunks 1 and 2 by the inverse waves, which are idle until the second
        __syncthreads();
        build_A(0);
        __syncthreads();
        __syncthreads();
        for (int i = 0; i < NC; ++i) {
            if (i + 3 < NC) build_A(i + 3);
            __syncthreads();
        }
    } else if (wave == Cf::W_SK) {
        if constexpr (GATED) { expA = expf(A_log[h]); dtb = dt_bias[h]; }
        // Chunks 0 .. LEAD-1 are stored before the first barrier, their loads
        // running two chunks ahead of the stores (two register sets), so the
        // HBM latency is paid about once instead of once per chunk. (NC >= 1;
        // loads past the last chunk reload it, harmlessly.)
        // Then loads are issued a full step before their data is stored: at
        // step i the loads of chunk i + LEAD + 1 go out first, then chunk
        // i + LEAD (loaded during step i - 1) is stored. Two register sets
        // alternate (the loop is unrolled by two), so the HBM latency passes
        // during the rest of the step and the barrier instead of inside the
        // store.
        {
            KRegs P0, P1;
            stage_k_load(0, P0);
            stage_k_load(min(1, NC - 1), P1);
#pragma unroll
            for (int c = 0; c < Cf::LEAD; c += 2) {
                if (c < NC) stage_k_store(c, P0);
                if (c + 2 < Cf::LEAD) stage_k_load(min(c + 2, NC - 1), P0);
                if (c + 1 < NC) stage_k_store(c + 1, P1);
                if (c + 3 < Cf::LEAD) stage_k_load(min(c + 3, NC - 1), P1);
            }
        }
        KRegs Ra, Rb;
        stage_k_load(min(Cf::LEAD, NC - 1), Ra);
        __syncthreads();
        __syncthreads();
        __syncthreads();
        for (int i = 0; i < NC; i += 2) {
            stage_k_load(min(i + Cf::LEAD + 1, NC - 1), Rb);   // past the end: a harmless reload
            if (i + Cf::LEAD < NC) stage_k_store(i + Cf::LEAD, Ra);
            __syncthreads();
            if (i + 1 < NC) {
                stage_k_load(min(i + Cf::LEAD + 2, NC - 1), Ra);
                if (i + Cf::LEAD + 1 < NC) stage_k_store(i + Cf::LEAD + 1, Rb);
                __syncthreads();
            }
        }
    } else {
        {
            QVRegs P0, P1;                             // as the K stager's prologue
            stage_qv_load(0, P0);
            stage_qv_load(min(1, NC - 1), P1);
#pragma unroll
            for (int c = 0; c < Cf::LEAD; c += 2) {
                if (c < NC) stage_qv_store(c, P0);
                if (c + 2 < Cf::LEAD) stage_qv_load(min(c + 2, NC - 1), P0);
                if (c + 1 < NC) stage_qv_store(c + 1, P1);
                if (c + 3 < Cf::LEAD) stage_qv_load(min(c + 3, NC - 1), P1);
            }
        }
        QVRegs Ra, Rb;
        stage_qv_load(min(Cf::LEAD, NC - 1), Ra);
        __syncthreads();
        __syncthreads();
        __syncthreads();
        for (int i = 0; i < NC; i += 2) {
            stage_qv_load(min(i + Cf::LEAD + 1, NC - 1), Rb);   // past the end: a harmless reload
            if (i + Cf::LEAD < NC) stage_qv_store(i + Cf::LEAD, Ra);
            __syncthreads();
            if (i + 1 < NC) {
                stage_qv_load(min(i + Cf::LEAD + 2, NC - 1), Ra);
                if (i + Cf::LEAD + 1 < NC) stage_qv_store(i + Cf::LEAD + 1, Rb);
                __syncthreads();
            }
        }
    }
}

// ---------------------------------------------------------------- launch

template <typename E, int DK, int BV, bool GATED, int INV>
static hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream)
{
    using Cf = PipeCfg<E, 32, DK, BV>;
    const int nvt = (a.Dv + BV - 1) / BV;
    const long long blocks = (long long)nvt * a.Hv * a.B;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_prefill_kernel<E, 32, DK, BV, GATED, INV>), dim3((unsigned)blocks),
                       dim3(Cf::THREADS), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, a.g_log, a.beta,
                       a.A_log, a.dt_bias, a.l2_eps, a.scale,
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

template <typename E, int DK, bool GATED, int INV>
static hipError_t launch_dk(const PrefillArgs& a, int max_bv, hipStream_t stream)
{
    switch (pick_bv(a, max_bv)) {
        case 64: if constexpr (sizeof(E) == 2) return launch_cfg<E, DK, 64, GATED, INV>(a, stream);
                 [[fallthrough]];
        case 32: return launch_cfg<E, DK, 32, GATED, INV>(a, stream);
        default: return launch_cfg<E, DK, 16, GATED, INV>(a, stream);
    }
}

template <bool GATED, int INV>
static hipError_t launch_gated(const PrefillArgs& a, int dtype, hipStream_t stream)
{
    if (dtype == 1)
        return a.Dk <= 64 ? launch_dk<bf16, 64, GATED, INV>(a, 64, stream)
                          : launch_dk<bf16, 128, GATED, INV>(a, 64, stream);
    return a.Dk <= 64 ? launch_dk<float, 64, GATED, INV>(a, 32, stream)
                      : launch_dk<float, 128, GATED, INV>(a, 32, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, hipStream_t stream)
{
    if (a.inverse == 1) return launch_gated<false, 1>(a, dtype, stream);   // ungated only
    return a.gated ? launch_gated<true, 0>(a, dtype, stream) : launch_gated<false, 0>(a, dtype, stream);
}

}  // namespace gdn
