// Router: fp32 logits h = W_r x, softmax, top-k with lowest-index ties,
// gates, and per-block partial sums of the probabilities and choice counts.
//
// [SW-GLaM] "Dense Scaling 与 MoE 的核心差异": h(x) = W_r x, p = softmax(h).
// [SW-GLaM] "Switch Transformer：把 MoE 做简单": i* = argmax p, gate p_{i*}.
// [CMU-L16] section 2.3: top-k keeps k logits, gate = softmax over them;
// an all-zero router picks the lowest indices (ties -> lower index).
// [CS25-L5] "稳定训练" / [SW-RES] section 2.1: the router runs in fp32.
//
// Two kernels:
//  * router_mfma  (bf16 x, E <= 256).  The fp32 router weight is split
//    exactly into three bf16 parts, w = hi + mid + lo (each part takes the
//    round-to-nearest bf16 of what the previous parts left, so the sum
//    reproduces all 24 significand bits).  bf16 x bf16 products are exact
//    in fp32, so three bf16 MFMAs with fp32 accumulation give an fp32 dot
//    product without any fp32 vector FMA.  A block of 64 tokens (128 with
//    more than 128 experts) streams W_r (fp32, split into its three parts
//    in registers as each fragment is read) and its token rows through a
//    ring of LDS stages filled by 16-byte DMA, and each of its four waves
//    computes the logits of all the block's tokens for a quarter of the
//    experts.  The logits go through LDS to one wave per 16 tokens,
//    where row softmax and top-k use 16-lane DPP row reductions.
//  * router_generic (fp32 x, or E > 256): fp32 FMA dot products into LDS,
//    then one wave per token row.
//
// Noisy top-k ([CMU-L16] section 2.3, after Shazeer et al.): the logit
// becomes H = W_r x + eps * softplus(W_noise x) with the standard normal
// draws eps [T, E] given by the caller, and H replaces the logits in
// everything that follows.  With bf16 x and E <= 128 the MFMA router runs
// on the stacked weight [W_r; W_noise]: each half padded to a whole number
// of 16-expert groups (32, 64 or 128 rows), so the lane that holds expert
// n's logit also holds its noise logit and H is formed lane by lane.  With
// E <= 256 it runs its K loop twice, over W_r and then W_noise, keeping the
// first pass's logits in registers.  Otherwise router_generic.
#include "common.h"
#include "launch.h"

#include <math.h>

namespace moe {

namespace {

constexpr int MAXK = 8;

// ---------------------------------------------------------------------------
// MFMA router
// ---------------------------------------------------------------------------
constexpr int RM_WAVES = 4;
constexpr int RM_TOK_WAVE = 16;
constexpr int RM_TOK_BLOCK = RM_WAVES * RM_TOK_WAVE;
constexpr int RM_LDS = 128 * 1024;         // LDS bytes of the stage ring

__device__ __forceinline__ void split3(float w, uint16_t &h, uint16_t &m, uint16_t &l) {
    h = f2bf(w);
    const float r1 = w - bf2f(h);      // exact
    m = f2bf(r1);
    const float r2 = r1 - bf2f(m);     // exact
    l = f2bf(r2);
}

// The stacked noisy weight: rows [0, EH) are W_r, rows [EH, 2 EH) W_noise,
// rows past E in either half zero; the same three-part split into W3.
__global__ __launch_bounds__(256) void router_split_noisy_kernel(const float *__restrict__ Wr,
                                                                 const float *__restrict__ Wn, int E,
                                                                 int d, int EH, uint16_t *__restrict__ W3) {
    const int64_t n = (int64_t)2 * EH * d;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int r = (int)(i / d);
        const int c = (int)(i - (int64_t)r * d);
        const int h = r < EH ? r : r - EH;
        const float *src = r < EH ? Wr : Wn;
        const float w = h < E ? src[(int64_t)h * d + c] : 0.f;
        uint16_t hi, mid, lo;
        split3(w, hi, mid, lo);
        W3[i] = hi;
        W3[n + i] = mid;
        W3[2 * n + i] = lo;
    }
}

// Stage geometry of the MFMA router: a stage holds KC columns of the three
// weights (WR x EP rows: the three bf16 parts, or fp32 W_r with each row's
// KC values in two LDS rows) and of the block's 64 token rows, in LDS rows of
// KC bf16.  Piece c (16 bytes) of row r is stored at c ^ swz(r), as in the
// expert GEMM: conflict-free 16-byte fragment reads and DMA writes.
template <int NB, int KC, int WR = 3, int TB = RM_TOK_BLOCK>
struct RGeo {
    static constexpr int EP = NB * 16;
    static constexpr int ROWB = KC * 2;
    static constexpr int PIECES = KC / 8;
    static constexpr int ROWS = WR * EP + TB;
    static constexpr int STAGE = ROWS * ROWB;
    static constexpr int S = RM_LDS / STAGE > 4 ? 4 : RM_LDS / STAGE;
    static constexpr int PERW = STAGE / 4096;            // 1 KB DMA instructions per wave per stage
    static constexpr int RPI = 1024 / ROWB;              // rows per DMA instruction
    static_assert(S >= 2 && STAGE % 4096 == 0, "router stage ring");
    static __device__ __forceinline__ int swz(int r) {
        return KC == 128 ? (r & 15) : KC == 64 ? (r & 7) : ((r >> 1) & 3);
    }
};

template <int NB, int KC, int WR = 3, int TB = RM_TOK_BLOCK>
constexpr bool rgeo_ok() { return RM_LDS / ((WR * NB * 16 + TB) * KC * 2) >= 2; }

// One block = 64 tokens (4 waves x 16) and every expert.  The weights and the
// token rows flow through an S-deep ring of LDS stages filled by 16-byte DMA;
// bf16 x bf16 products are exact in fp32, so three v_mfma_f32_16x16x32_bf16
// per 16 experts and 32 columns, one per exact bf16 part of the weight, give
// the fp32 dot products.  The plain router stages W_r itself in fp32 and
// splits each fragment into its three parts in registers as it reads it
// (split3: no launch of its own, and two thirds of the weight bytes of the
// three parts: 7-12 % faster on 8 to 128 experts); with more than 128
// experts it takes 128 tokens a block, so that each staged weight fragment
// (and its split) serves twice the tokens.  The noisy forms read the parts
// that router_split_noisy_kernel made.
//
// NB = 1 (E <= 16; KC = 128): one group of 16 experts would leave three waves
// without work, so instead wave w takes the w-th 32 columns of every stage
// for all 64 tokens, and the four partial logits are added in wave order
// before the epilogue.  With 16 rather than 64 weight rows a stage holds
// twice the token bytes of the wider kernels, and the ring keeps that much
// more of x in flight.
// NZ (noisy top-k, W3 from router_split_noisy_kernel):
//  0  the plain router;
//  1  W3 is the stacked weight with NB / 2 groups of 16 rows per half; lane
//     col's column nb is expert nb 16 + col and column NB / 2 + nb its noise
//     logit, combined in the epilogue;
//  2  W3 holds NB 16 rows of W_r, then NB 16 of W_noise; the K loop runs
//     twice (the token rows are re-read, mostly from L2) and the first
//     pass's logits stay in registers, so each lane forms H for its own
//     (token, expert) entries before they go to LDS.
// TB: tokens per block, 64 or (the plain router with 256 experts) 128, which
// halves the weight bytes streamed per token (the epilogue then runs twice).
template <int NB, int KC, bool KTAIL, int KSEL, int NZ, int TB = RM_TOK_BLOCK>
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W3, const float *__restrict__ Wf,
    const float *__restrict__ br,
    int64_t T, int d, int E, int k, int32_t *__restrict__ out_idx, float *__restrict__ out_gate,
    float *__restrict__ part_prob, int32_t *__restrict__ part_cnt, float *__restrict__ part_z,
    const float *__restrict__ eps, float *__restrict__ logits) {
    constexpr bool WF32 = NZ == 0 && (NB <= 8 || TB == 128);   // fp32 W_r, split in registers
    constexpr int WR = WF32 ? 2 : 3;                     // LDS rows of weights per expert row
    constexpr int AB = TB / 16;                          // 16-token row blocks
    static_assert(TB == RM_TOK_BLOCK || (TB == 128 && NZ == 0 && NB >= RM_WAVES), "tokens per block");
    using G = RGeo<NB, KC, WR, TB>;
    constexpr int EP = G::EP, ROWB = G::ROWB, PIECES = G::PIECES, S = G::S, PERW = G::PERW;
    constexpr int STAGE = G::STAGE, RPI = G::RPI;
    constexpr int NEWER = (S - 2) * PERW;
    __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[S > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[S > 3 ? STAGE : 16];
    __shared__ float sProb[RM_WAVES][EP];
    __shared__ int sCnt[EP];
    __shared__ float sLz[TB];                           // each token's log-sum-exp, squared

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;      // expert column within a 16-block / token row of A
    const int kg = lane >> 4;       // k group (A/B operands) or row group (D)
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    for (int i = tid; i < EP; i += 256) sCnt[i] = 0;

    // DMA sources: block instruction q = wave * PERW + i fills rows
    // [q RPI, +RPI): rows 0 .. 3 EP - 1 are the weight parts (rows past the
    // part's EW rows repeat its last one), the rest the block's tokens (past
    // T: row T - 1)
    const int lr = lane / PIECES;
    const int EW = NZ == 1 ? EP : NZ == 2 ? 2 * EP : E;
    const int64_t nW = (int64_t)EW * d;
    const uint16_t *src[PERW];
    // instruction i of this lane: the K column of its piece within a chunk
    // (its row's swizzle decides which piece) and the source's 16-bit units
    // per K column (2 for fp32 weight rows)
    int coff[PERW], kmul[PERW];
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
        const int row = (wave * PERW + i) * RPI + lr;
        const int lc = (lane % PIECES) ^ G::swz(row);
        if (row < WR * EP) {
            if constexpr (WF32) {
                // fp32 row n: columns [0, KC / 2) of the chunk in LDS row 2n,
                // the rest in 2n + 1; a 16-byte piece holds 4 of them
                const int h = row & 1;
                int n = row >> 1;
                n = n < E ? n : E - 1;
                coff[i] = h * (KC / 2) + lc * 4;
                kmul[i] = 2;
                src[i] = reinterpret_cast<const uint16_t *>(Wf + (int64_t)n * d + coff[i]);
            } else {
                const int p = row / EP;
                int n = row - p * EP;
                n = n < EW ? n : EW - 1;
                coff[i] = lc * 8;
                kmul[i] = 1;
                src[i] = W3 + p * nW + (int64_t)n * d + coff[i];
            }
        } else {
            int64_t t = t0 + (row - WR * EP);
            t = t < T ? t : T - 1;
            coff[i] = lc * 8;
            kmul[i] = 1;
            src[i] = x + t * d + coff[i];
        }
    }
    const int nk = (d + KC - 1) / KC;
    auto tail_piece = [&](int i) { return KTAIL && ((nk - 1) * KC + coff[i] >= d); };
    auto issue = [&](uint8_t *base, int kt) {
#pragma unroll
        for (int i = 0; i < PERW; ++i) {
            const int k0 = ((KTAIL && kt == nk - 1 && tail_piece(i)) ? -coff[i] : kt * KC) * kmul[i];
            __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)(src[i] + k0),
                                             (MOE_LDS_AS void *)(base + (wave * PERW + i) * 1024),
                                             16, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // the pieces past d were loaded from column 0: clear them (products with a
    // zero operand on either side are zero)
    auto clear_tail = [&](uint8_t *base) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < PERW; ++i)
            if (tail_piece(i)) *reinterpret_cast<u32x4 *>(base + (wave * PERW + i) * 1024 + lane * 16) = z;
    };

    // wave w computes the logits of all 64 tokens (4 row blocks of 16) for its
    // NBW groups of 16 experts, g = w NBW .. w NBW + NBW - 1: every weight
    // fragment read from LDS feeds 4 MFMAs
    constexpr bool KSPLIT = NB < RM_WAVES;
    constexpr int NBW = KSPLIT ? 1 : NB / RM_WAVES;
    static_assert(KSPLIT ? (NB == 1 && KC == 128 && NZ == 0) : NB % RM_WAVES == 0, "expert groups per wave");
    f32x4 acc[AB][NBW];
#pragma unroll
    for (int ab = 0; ab < AB; ++ab)
#pragma unroll
        for (int g = 0; g < NBW; ++g) acc[ab][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fragment rows: A = token row ab 16 + col, B = weight row p EP + g 16 + col;
    // row bases are multiples of 16, so swz(row) = swz(col)
    const int fs = G::swz(col);
    const int arow = (WR * EP + col) * ROWB;
    const int brow = ((KSPLIT ? 0 : wave * NBW * 16) + col) * ROWB;
    // fp32 weights: expert row n = g 16 + col (+ the wave's groups) sits in LDS
    // rows 2n and 2n + 1; a lane's 8 columns k0 .. k0 + 7 (k0 = 32 sub + 8 kg)
    // are two pieces of row 2n + k0 / (KC / 2)
    auto wf_frag = [&](const uint8_t *sb, int g, int ksub, bf16x8 (&b)[3]) {
        const int k0 = ksub * 32 + kg * 8;
        const int R = 2 * ((KSPLIT ? 0 : wave * NBW * 16) + g * 16 + col) + k0 / (KC / 2);
        const int pc = (k0 % (KC / 2)) / 4;
        const int sw = G::swz(R);
        const u32x4 w0 = *reinterpret_cast<const u32x4 *>(sb + R * ROWB + ((pc ^ sw) << 4));
        const u32x4 w1 = *reinterpret_cast<const u32x4 *>(sb + R * ROWB + (((pc + 1) ^ sw) << 4));
        u32x4 ph, pm, pl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 &w = q < 2 ? w0 : w1;
            uint16_t h0, m0, l0, h1, m1, l1;
            split3(__uint_as_float(w[(2 * q) & 3]), h0, m0, l0);
            split3(__uint_as_float(w[(2 * q + 1) & 3]), h1, m1, l1);
            ph[q] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            pm[q] = (uint32_t)m0 | ((uint32_t)m1 << 16);
            pl[q] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        b[0] = as_bf16x8(ph);
        b[1] = as_bf16x8(pm);
        b[2] = as_bf16x8(pl);
    };
    auto compute = [&](const uint8_t *sb) {
#pragma unroll
        for (int sub = 0; sub < (KSPLIT ? 1 : KC / 32); ++sub) {
            const int po = (((KSPLIT ? wave : sub) * 4 + kg) ^ fs) << 4;
            bf16x8 a[AB];
#pragma unroll
            for (int ab = 0; ab < AB; ++ab)
                a[ab] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + arow + ab * 16 * ROWB + po));
            // the weight parts of group g + 1 are read (and split) while the
            // MFMAs of group g run
            auto wfrag = [&](int g, bf16x8 (&bp)[3]) {
                if constexpr (WF32) {
                    wf_frag(sb, g, KSPLIT ? wave : sub, bp);
                } else {
                    const int o = brow + g * 16 * ROWB + po;
#pragma unroll
                    for (int p = 0; p < 3; ++p)
                        bp[p] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + p * EP * ROWB + o));
                }
            };
            bf16x8 bp[2][3];
            wfrag(0, bp[0]);
#pragma unroll
            for (int g = 0; g < NBW; ++g) {
                if (g + 1 < NBW) wfrag(g + 1, bp[(g + 1) & 1]);
#pragma unroll
                for (int p = 0; p < 3; ++p) {
#pragma unroll
                    for (int ab = 0; ab < AB; ++ab)
                        acc[ab][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ab], bp[g & 1][p], acc[ab][g], 0, 0, 0);
                }
                if (g + 1 < NBW) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);          // the next group's reads
#pragma unroll
                    for (int r = 0; r < 3 * AB; ++r) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);      // the next split, a few VALU at a time
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // ---- the ring (same scheme as the expert GEMM): chunk kt lives in stage
    // kt % S; a step waits for its own DMA, passes an LDS-only barrier,
    // refills the stage of kt - 1 with kt + S - 1 and runs its MFMAs
    // prologue: K tiles 0 .. S - 2, clamped to the last one when there are
    // fewer (the duplicate loads are never read).  Unconditional on purpose:
    // a conditional DMA here makes the compiler give up tracking which stage
    // a pending DMA writes, and then it drains the whole ring before every
    // fragment read.
    constexpr int NPASS = NZ == 2 ? 2 : 1;
    int kt = 0;
    f32x4 acc0[4][NBW];                                  // NZ 2 (TB 64): the first pass's logits
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        if (pass == 1) {
            // the ring is drained; keep the W_r logits, restart on the W_noise rows
#pragma unroll
            for (int ab = 0; ab < 4; ++ab)
#pragma unroll
                for (int g = 0; g < NBW; ++g) {
                    acc0[ab][g] = acc[ab][g];
                    acc[ab][g] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int i = 0; i < PERW; ++i)
                if ((wave * PERW + i) * RPI + lr < WR * EP) src[i] += (int64_t)EP * d;
            lds_barrier();                               // every wave is done with the last stage
        }
        issue(st0, 0);
        if (S > 2) issue(st1, nk > 1 ? 1 : nk - 1);
        if (S > 3) issue(st2, nk > 2 ? 2 : nk - 1);
        kt = 0;
        // steady state: every step refills a stage (no conditional DMA, which
        // would make the compiler drain the ring before every fragment read)
#define MOE_RSTEP_S(CUR, NXT)                                                   \
        {                                                                           \
            wait_vm_lgkm0<NEWER>();                                                 \
            ring_barrier();                                                         \
            issue(NXT, kt + S - 1);                                                 \
            compute(CUR);                                                           \
            ++kt;                                                                   \
        }
        for (; kt + 2 * S - 1 <= nk;) {
            if constexpr (S == 2) {
                MOE_RSTEP_S(st0, st1)
                MOE_RSTEP_S(st1, st0)
            } else if constexpr (S == 3) {
                MOE_RSTEP_S(st0, st2)
                MOE_RSTEP_S(st1, st0)
                MOE_RSTEP_S(st2, st1)
            } else {
                MOE_RSTEP_S(st0, st3)
                MOE_RSTEP_S(st1, st0)
                MOE_RSTEP_S(st2, st1)
                MOE_RSTEP_S(st3, st2)
            }
        }
#undef MOE_RSTEP_S
        // drain: at most 2 S - 2 steps, refilling while chunks remain; kt % S == 0 here
#define MOE_RSTEP(CUR, NXT)                                                     \
        if (kt < nk) {                                                              \
            if (kt + S - 2 < nk) wait_vm_lgkm0<NEWER>();                            \
            else wait_vm_lgkm0<0>();                                                \
            if (KTAIL && kt == nk - 1) {                                            \
                clear_tail(CUR);                                                    \
                wait_vm_lgkm0<63>();          /* the zeros are in LDS */            \
            }                                                                       \
            ring_barrier();                                                         \
            if (kt + S - 1 < nk) issue(NXT, kt + S - 1);                            \
            compute(CUR);                                                           \
            ++kt;                                                                   \
        }
        if constexpr (S == 2) {
            MOE_RSTEP(st0, st1)
            MOE_RSTEP(st1, st0)
        } else if constexpr (S == 3) {
            MOE_RSTEP(st0, st2)
            MOE_RSTEP(st1, st0)
            MOE_RSTEP(st2, st1)
            MOE_RSTEP(st0, st2)
        } else {
            MOE_RSTEP(st0, st3)
            MOE_RSTEP(st1, st0)
            MOE_RSTEP(st2, st1)
            MOE_RSTEP(st3, st2)
            MOE_RSTEP(st0, st3)
            MOE_RSTEP(st1, st0)
        }
#undef MOE_RSTEP
    }

    // ---- epilogue: lane holds logits of tokens t0 + 64 h + 16 wave + 4 kg + i,
    // experts nb 16 + col
    constexpr int NE = NZ == 1 ? NB / 2 : NB;            // expert groups
    static_assert(NZ != 1 || NB % 2 == 0, "noisy halves");
    float bias[NE];                                      // (NZ 2: already in the logits)
#pragma unroll
    for (int nb = 0; nb < NE; ++nb) {
        const int n = nb * 16 + col;
        bias[nb] = (NZ != 2 && br != nullptr && n < E) ? br[n] : 0.f;
    }
    float psum[NE];
#pragma unroll
    for (int nb = 0; nb < NE; ++nb) psum[nb] = 0.f;

    // passes of 64 tokens (TB = 128: two)
#pragma unroll
    for (int h = 0; h < TB / 64; ++h) {
        // ---- logits to LDS, 64 tokens at a time (token rows 0..31 of the pass in
        // st0, 32..63 in st1; the ring is drained), then each wave takes 16 of
        // them across all experts
        constexpr int ZS = EP + 4;                           // fp32 row stride
        static_assert(32 * ZS * 4 <= STAGE, "logit rows fit a stage buffer");
        static_assert(!KSPLIT || (S == 4 && 64 * ZS * 4 <= STAGE), "one stage buffer per wave's partial logits");
        lds_barrier();
        if constexpr (KSPLIT) {
            // wave w's partial sums (its columns of every stage) for all 64 tokens
            float *zw = reinterpret_cast<float *>(wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3);
#pragma unroll
            for (int ab = 0; ab < 4; ++ab)
#pragma unroll
                for (int i = 0; i < 4; ++i) zw[(ab * 16 + 4 * kg + i) * ZS + col] = acc[ab][0][i];
        } else {
#pragma unroll
        for (int abl = 0; abl < 4; ++abl)
#pragma unroll
            for (int g = 0; g < NBW; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ab = 4 * h + abl;
                    const int tok = abl * 16 + 4 * kg + i;
                    const int n = (wave * NBW + g) * 16 + col;
                    float *zr = reinterpret_cast<float *>(tok < 32 ? st0 : st1) + (tok & 31) * ZS;
                    if constexpr (NZ == 2) {
                        // H = (W_r x + b) + eps softplus(W_noise x), softplus as
                        // max(a, 0) + log(1 + exp(-|a|)) (no overflow)
                        const int64_t t = t0 + 64 * h + tok;
                        const bool ok = t < T && n < E;
                        const float zn = acc[ab][g][i];
                        const float sp = fmaxf(zn, 0.f) + log1pf(expf(-fabsf(zn)));
                        const float b = (br != nullptr && n < E) ? br[n] : 0.f;
                        const float e = ok ? eps[t * E + n] : 0.f;
                        zr[n] = fmaf(e, sp, acc0[ab][g][i] + b);
                    } else {
                        zr[n] = acc[ab][g][i];
                    }
                }
        }
        lds_barrier();

#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + 64 * h + wave * RM_TOK_WAVE + 4 * kg + i;
            const bool tok_ok = t < T;
            float v[NE];
            float mx = -INFINITY;
            const int tok = wave * RM_TOK_WAVE + 4 * kg + i;
            const float *zr = reinterpret_cast<const float *>(tok < 32 ? st0 : st1) + (tok & 31) * ZS;
#pragma unroll
            for (int nb = 0; nb < NE; ++nb) {
                const int n = nb * 16 + col;
                // K split: the four waves' partial sums, in wave order
                float z = KSPLIT ? ((reinterpret_cast<const float *>(st0)[tok * ZS + n] +
                                     reinterpret_cast<const float *>(st1)[tok * ZS + n]) +
                                    reinterpret_cast<const float *>(st2)[tok * ZS + n]) +
                                       reinterpret_cast<const float *>(st3)[tok * ZS + n] + bias[nb]
                                 : zr[n] + bias[nb];
                if (NZ == 1) {
                    // H = z + eps softplus(zn); softplus without overflow:
                    // max(a, 0) + log(1 + exp(-|a|))
                    const float zn = zr[NE * 16 + n];
                    const float sp = fmaxf(zn, 0.f) + log1pf(expf(-fabsf(zn)));
                    const float e = (tok_ok && n < E) ? eps[t * E + n] : 0.f;
                    z = fmaf(e, sp, z);
                }
                if (logits != nullptr && tok_ok && n < E) logits[t * E + n] = z;
                if (z != z) z = -INFINITY;          // NaN ranks as -inf: indices stay in range
                v[nb] = z;
                if (n < E) mx = fmaxf(mx, z);
            }
            mx = row16_max(mx);
            // exp through the hardware exp2 (about 1 ulp): these terms only feed
            // the sum s and the per-expert probability sums, whose bounds are far
            // looser; the gate of the chosen expert is 1 / s with s from them
            const float mxl = mx * 1.44269504088896341f;
            float ex[NE];
            float s = 0.f;
#pragma unroll
            for (int nb = 0; nb < NE; ++nb) {
                const int n = nb * 16 + col;
                ex[nb] = (n < E) ? __builtin_amdgcn_exp2f(fmaf(v[nb], 1.44269504088896341f, -mxl)) : 0.f;
                s += ex[nb];
            }
            s = row16_sum(s);
            if (tok_ok) {
                const float inv = 1.0f / s;
#pragma unroll
                for (int nb = 0; nb < NE; ++nb) psum[nb] = fmaf(ex[nb], inv, psum[nb]);
            }
            if (col == 0) {
                // z-loss term: log sum_i exp z_i = max + log sum_i exp(z_i - max)
                const float l = mx + logf(s);
                sLz[64 * h + tok] = tok_ok ? l * l : 0.f;
            }

            // top-k by k rounds over the not-yet-chosen experts: the round's
            // largest logit (a 16-lane max), then the lowest expert index holding
            // it (a 16-lane min), so ties go to the lower index.  Round 0 reuses
            // the softmax max.  (KSEL = k when it is 1 or 2, so that the common
            // cases stay small code; 0 = any k up to MAXK.)
            constexpr int KMAX = KSEL ? KSEL : MAXK;
            const int kk = KSEL ? KSEL : k;
            uint32_t excl = 0u;                      // bit nb: this lane's expert nb*16+col is taken
            static_assert(NE <= 32, "exclusion mask");
            float vsel[KMAX];
            int isel[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                vsel[j] = -INFINITY;
                isel[j] = 0;
                if (j < kk) {
                    float m = mx;
                    if (j > 0) {
                        m = -INFINITY;
#pragma unroll
                        for (int nb = 0; nb < NE; ++nb)
                            if (nb * 16 + col < E && !((excl >> nb) & 1u)) m = fmaxf(m, v[nb]);
                        m = row16_max(m);
                    }
                    int best = 0x7fffffff;
#pragma unroll
                    for (int nb = 0; nb < NE; ++nb) {
                        const int n = nb * 16 + col;
                        const bool cand = n < E && !((excl >> nb) & 1u) && v[nb] == m;
                        best = cand ? min(best, n) : best;
                    }
                    best = row16_min(best);
                    if ((best & 15) == col) excl |= 1u << (best >> 4);
                    vsel[j] = m;
                    isel[j] = best;
                }
            }
            if (tok_ok && col == 0) {
                if (kk == 1) {
                    out_idx[t] = isel[0];
                    out_gate[t] = 1.0f / s;        // p_{i*} = exp(0) / sum
                    atomicAdd(&sCnt[isel[0]], 1);
                } else {
                    float ek[KMAX];
                    float sk = 0.f;
#pragma unroll
                    for (int j = 0; j < KMAX; ++j) {
                        ek[j] = (j < kk) ? expf(vsel[j] - vsel[0]) : 0.f;
                        sk += ek[j];
                    }
#pragma unroll
                    for (int j = 0; j < KMAX; ++j) {
                        if (j < kk) {
                            out_idx[t * k + j] = isel[j];
                            out_gate[t * k + j] = ek[j] / sk;
                            atomicAdd(&sCnt[isel[j]], 1);
                        }
                    }
                }
            }
        }

        lds_barrier();                                   // the pass's logits are read
    }

    // ---- block partials: probability sums and choice counts per expert
#pragma unroll
    for (int nb = 0; nb < NE; ++nb) {
        psum[nb] += __shfl_xor(psum[nb], 16);
        psum[nb] += __shfl_xor(psum[nb], 32);
    }
    if (lane < 16) {
#pragma unroll
        for (int nb = 0; nb < NE; ++nb) sProb[wave][nb * 16 + lane] = psum[nb];
    }
    __syncthreads();
    for (int n = tid; n < E; n += 256) {
        const float s = ((sProb[0][n] + sProb[1][n]) + sProb[2][n]) + sProb[3][n];
        part_prob[(int64_t)blockIdx.x * E + n] = s;
        part_cnt[(int64_t)blockIdx.x * E + n] = sCnt[n];
    }
    // the block's z-loss partial, summed in a fixed order
    if (tid < 64) {
        static_assert(TB % 64 == 0, "one wave sums the block's tokens");
        float v = sLz[tid];
#pragma unroll
        for (int h = 1; h < TB / 64; ++h) v += sLz[64 * h + tid];
        for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
        if (tid == 0) part_z[blockIdx.x] = v;
    }
}

// ---------------------------------------------------------------------------
// generic router (fp32 FMA): any dtype, any E <= 1024
// ---------------------------------------------------------------------------
constexpr int RG_TOK = 8;   // tokens per block, two rows per wave

// NOISY: noisy top-k ([CMU-L16] section 2.3, Shazeer et al.): the logit
// becomes H = z + eps * softplus(W_noise x), with eps [T, E] standard normal
// draws given by the caller, and H replaces z in everything that follows.
template <bool BF16, bool NOISY>
__global__ __launch_bounds__(256) void router_generic_kernel(
    const void *__restrict__ xv, const float *__restrict__ Wr, const float *__restrict__ br,
    int64_t T, int d, int E, int k, int32_t *__restrict__ out_idx, float *__restrict__ out_gate,
    float *__restrict__ part_prob, int32_t *__restrict__ part_cnt, float *__restrict__ part_z,
    const float *__restrict__ Wn, const float *__restrict__ eps, float *__restrict__ logits) {
    extern __shared__ float smem[];
    __shared__ float sLz[RG_TOK];                       // each token's log-sum-exp, squared
    float *sZ = smem;                                   // [RG_TOK][E]
    int *sCnt = reinterpret_cast<int *>(smem + RG_TOK * E);   // [E]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * RG_TOK;

    for (int n = tid; n < E; n += 256) sCnt[n] = 0;
    for (int p = tid; p < RG_TOK * E; p += 256) {
        const int r = p / E;
        const int n = p - r * E;
        const int64_t t = t0 + r;
        float z = 0.f;
        if (t < T) {
            const float *w = Wr + (int64_t)n * d;
            const float *wn = NOISY ? Wn + (int64_t)n * d : nullptr;
            float zn = 0.f;
            if (BF16) {
                const uint16_t *xr = reinterpret_cast<const uint16_t *>(xv) + t * d;
                for (int q = 0; q < d; ++q) {
                    const float xq = bf2f(xr[q]);
                    z = fmaf(xq, w[q], z);
                    if (NOISY) zn = fmaf(xq, wn[q], zn);
                }
            } else {
                const float *xr = reinterpret_cast<const float *>(xv) + t * d;
                for (int q = 0; q < d; ++q) {
                    z = fmaf(xr[q], w[q], z);
                    if (NOISY) zn = fmaf(xr[q], wn[q], zn);
                }
            }
            if (br != nullptr) z += br[n];
            if (NOISY) {
                // softplus without overflow: max(a, 0) + log(1 + exp(-|a|))
                const float sp = fmaxf(zn, 0.f) + log1pf(expf(-fabsf(zn)));
                z = fmaf(eps[t * E + n], sp, z);
            }
            if (logits != nullptr) logits[t * E + n] = z;
            if (z != z) z = -INFINITY;
        }
        sZ[p] = z;
    }
    __syncthreads();

    for (int rr = 0; rr < 2; ++rr) {
        const int r = wave * 2 + rr;
        const int64_t t = t0 + r;
        float *row = sZ + r * E;
        if (t < T) {
            float mx = -INFINITY;
            for (int n = lane; n < E; n += 64) mx = fmaxf(mx, row[n]);
            for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
            float s = 0.f;
            for (int n = lane; n < E; n += 64) s += expf(row[n] - mx);
            for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
            if (lane == 0) {
                const float l = mx + logf(s);           // log sum_i exp z_i
                sLz[r] = l * l;
            }
            float vsel[MAXK];
            int isel[MAXK];
            for (int j = 0; j < MAXK; ++j) {
                vsel[j] = -INFINITY;
                isel[j] = 0;
                if (j < k) {
                    Cand c{-INFINITY, 0x7fffffff, 0};
                    for (int n = lane; n < E; n += 64) {
                        bool taken = false;
                        for (int q = 0; q < j; ++q) taken |= (isel[q] == n);
                        if (!taken) {
                            const Cand o{row[n], n, 1};
                            if (cand_better(o, c)) c = o;
                        }
                    }
                    for (int m = 32; m >= 1; m >>= 1) {
                        const Cand o = cand_shfl_xor(c, m);
                        if (cand_better(o, c)) c = o;
                    }
                    vsel[j] = c.v;
                    isel[j] = c.i;
                }
            }
            // probabilities replace the logits (after every lane has read them)
            __builtin_amdgcn_wave_barrier();
            for (int n = lane; n < E; n += 64) row[n] = expf(row[n] - mx) / s;
            if (lane == 0) {
                if (k == 1) {
                    out_idx[t] = isel[0];
                    out_gate[t] = 1.0f / s;
                    atomicAdd(&sCnt[isel[0]], 1);
                } else {
                    float ek[MAXK];
                    float sk = 0.f;
                    for (int j = 0; j < MAXK; ++j) {
                        ek[j] = (j < k) ? expf(vsel[j] - vsel[0]) : 0.f;
                        sk += ek[j];
                    }
                    for (int j = 0; j < k; ++j) {
                        out_idx[t * k + j] = isel[j];
                        out_gate[t * k + j] = ek[j] / sk;
                        atomicAdd(&sCnt[isel[j]], 1);
                    }
                }
            }
        } else {
            for (int n = lane; n < E; n += 64) row[n] = 0.f;
            if (lane == 0) sLz[r] = 0.f;
        }
    }
    __syncthreads();
    if (tid == 0) {
        float v = 0.f;
        for (int r = 0; r < RG_TOK; ++r) v += sLz[r];
        part_z[blockIdx.x] = v;
    }
    for (int n = tid; n < E; n += 256) {
        float s = 0.f;
        for (int r = 0; r < RG_TOK; ++r) s += sZ[r * E + n];
        part_prob[(int64_t)blockIdx.x * E + n] = s;
        part_cnt[(int64_t)blockIdx.x * E + n] = sCnt[n];
    }
}

// ---------------------------------------------------------------------------
// reduction of the block partials: one wave per expert, fixed order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_reduce_kernel(
    const float *__restrict__ part_prob, const int32_t *__restrict__ part_cnt, int nblk, int E,
    float *__restrict__ prob_sum, int32_t *__restrict__ route_count, const float *__restrict__ part_z,
    int64_t T, float *__restrict__ z_loss) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    double s = 0.0;
    long long c = 0;
    for (int b = lane; b < nblk; b += 64) {
        s += (double)part_prob[(int64_t)b * E + e];
        c += part_cnt[(int64_t)b * E + e];
    }
    for (int m = 32; m >= 1; m >>= 1) {
        s += __shfl_xor(s, m);
        c += __shfl_xor(c, m);
    }
    if (lane == 0) {
        prob_sum[e] = (float)s;
        route_count[e] = (int32_t)c;
    }
    if (z_loss != nullptr && e == 0) {
        const float zl = z_loss_wave(part_z, nblk, T, lane);
        if (lane == 0) z_loss[0] = zl;
    }
}

bool use_mfma(int dtype_bf16, int E) { return dtype_bf16 && E <= 256; }
bool use_mfma_noisy(int dtype_bf16, int E) { return dtype_bf16 && E <= 256; }
// rows of each half of the noisy weight in W3.  E <= 128 (stacked, one K
// pass): half of one of the MFMA router's widths (64, 128, 256 rows), so
// that the noise half starts at the kernel's column NB / 2 * 16 and the four
// waves split the rows evenly.  E <= 256 (two K passes): the full width 256.
int noisy_half_rows(int E) { return E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256; }

}  // namespace

// tokens per block of the plain MFMA router: 128 with more than 128 experts
static int router_tok_block(int E) { return E > 128 ? 128 : RM_TOK_BLOCK; }

int router_blocks(int64_t T, int dtype_bf16, int E) {
    const int per = use_mfma(dtype_bf16, E) ? router_tok_block(E) : RG_TOK;
    return (int)((T + per - 1) / per);
}

hipError_t launch_router(const void *x, int dtype_bf16, const float *W_r, const float *b_r,
                         int64_t T, int d, int E, int k, int32_t *expert_idx, float *gate,
                         float *part_prob, int32_t *part_cnt, uint16_t *w3, hipStream_t s,
                         float *part_z, float *logits) {
    const int nblk = router_blocks(T, dtype_bf16, E);
    if (nblk == 0) return hipSuccess;
    if (use_mfma(dtype_bf16, E)) {
        // W_r is staged in fp32 and split into its bf16 parts in registers
        // (w3 is left unused); more than 128 experts take 128 tokens a block
        (void)w3;
        const uint16_t *xb = reinterpret_cast<const uint16_t *>(x);
        const int nb = (E + 15) / 16;
#define MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, KSV, TBV)                                           \
    hipLaunchKernelGGL((router_mfma_kernel<NBV, KCV, TAILV, KSV, 0, TBV>), dim3(nblk), dim3(256), \
                       0, s, xb, nullptr, W_r, b_r, T, d, E, k, expert_idx, gate, part_prob,     \
                       part_cnt, part_z, nullptr, logits)
#define MOE_ROUTER_K(NBV, KCV, TAILV, TBV)                                                     \
    do {                                                                                       \
        if (k == 1) MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, 1, TBV);                                \
        else if (k == 2) MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, 2, TBV);                           \
        else MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, 0, TBV);                                       \
    } while (0)
#define MOE_ROUTER_CASE(NBV, KCV, TBV)                                                         \
    if (nb <= NBV) {                                                                           \
        static_assert(rgeo_ok<NBV, KCV, 2, TBV>(), "router ring");                             \
        if (d % KCV == 0) MOE_ROUTER_K(NBV, KCV, false, TBV);                                  \
        else MOE_ROUTER_K(NBV, KCV, true, TBV);                                                \
        return hipGetLastError();                                                              \
    }
        MOE_ROUTER_CASE(1, 128, 64)
        MOE_ROUTER_CASE(4, 64, 64)
        MOE_ROUTER_CASE(8, 64, 64)
        MOE_ROUTER_CASE(16, 32, 128)
#undef MOE_ROUTER_CASE
#undef MOE_ROUTER_K
#undef MOE_ROUTER_LAUNCH
        return hipErrorInvalidValue;
    }
    const size_t shm = (size_t)(RG_TOK + 1) * E * sizeof(float);
    if (dtype_bf16)
        hipLaunchKernelGGL((router_generic_kernel<true, false>), dim3(nblk), dim3(256), shm, s, x, W_r,
                           b_r, T, d, E, k, expert_idx, gate, part_prob, part_cnt, part_z, nullptr,
                           nullptr, logits);
    else
        hipLaunchKernelGGL((router_generic_kernel<false, false>), dim3(nblk), dim3(256), shm, s, x, W_r,
                           b_r, T, d, E, k, expert_idx, gate, part_prob, part_cnt, part_z, nullptr,
                           nullptr, logits);
    return hipGetLastError();
}

int router_w3_rows(int E) { return use_mfma_noisy(1, E) ? 2 * noisy_half_rows(E) : E; }

int router_noisy_blocks(int64_t T, int dtype_bf16, int E) {
    const int per = use_mfma_noisy(dtype_bf16, E) ? RM_TOK_BLOCK : RG_TOK;
    return (int)((T + per - 1) / per);
}

hipError_t launch_router_noisy(const void *x, int dtype_bf16, const float *W_r, const float *b_r,
                               const float *W_noise, const float *eps, int64_t T, int d, int E,
                               int k, int32_t *expert_idx, float *gate, float *part_prob,
                               int32_t *part_cnt, float *part_z, uint16_t *w3, hipStream_t s) {
    const int nblk = router_noisy_blocks(T, dtype_bf16, E);
    if (nblk == 0) return hipSuccess;
    if (use_mfma_noisy(dtype_bf16, E)) {
        const int EH = noisy_half_rows(E);
        const int64_t n = (int64_t)2 * EH * d;
        const int sg = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
        hipLaunchKernelGGL(router_split_noisy_kernel, dim3(sg), dim3(256), 0, s, W_r, W_noise, E, d, EH,
                           w3);
        const uint16_t *xb = reinterpret_cast<const uint16_t *>(x);
#define MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, KSV, NZV)                                           \
    hipLaunchKernelGGL((router_mfma_kernel<NBV, KCV, TAILV, KSV, NZV>), dim3(nblk), dim3(256),   \
                       0, s, xb, w3, nullptr, b_r, T, d, E, k, expert_idx, gate, part_prob,      \
                       part_cnt, part_z, eps, nullptr)
#define MOE_ROUTER_K(NBV, KCV, TAILV, NZV)                                                     \
    do {                                                                                       \
        if (k == 1) MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, 1, NZV);                                \
        else if (k == 2) MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, 2, NZV);                           \
        else MOE_ROUTER_LAUNCH(NBV, KCV, TAILV, 0, NZV);                                       \
    } while (0)
#define MOE_ROUTER_CASE(NBV, KCV, NZV)                                                         \
    if (EH == (NZV == 1 ? NBV * 8 : NBV * 16)) {                                               \
        static_assert(rgeo_ok<NBV, KCV>(), "router ring");                                     \
        if (d % KCV == 0) MOE_ROUTER_K(NBV, KCV, false, NZV);                                  \
        else MOE_ROUTER_K(NBV, KCV, true, NZV);                                                \
        return hipGetLastError();                                                              \
    }
        MOE_ROUTER_CASE(4, 64, 1)
        MOE_ROUTER_CASE(8, 64, 1)
        MOE_ROUTER_CASE(16, 32, 1)
        MOE_ROUTER_CASE(16, 32, 2)
#undef MOE_ROUTER_CASE
#undef MOE_ROUTER_K
#undef MOE_ROUTER_LAUNCH
        return hipErrorInvalidValue;
    }
    const size_t shm = (size_t)(RG_TOK + 1) * E * sizeof(float);
    if (dtype_bf16)
        hipLaunchKernelGGL((router_generic_kernel<true, true>), dim3(nblk), dim3(256), shm, s, x, W_r,
                           b_r, T, d, E, k, expert_idx, gate, part_prob, part_cnt, part_z, W_noise, eps,
                           nullptr);
    else
        hipLaunchKernelGGL((router_generic_kernel<false, true>), dim3(nblk), dim3(256), shm, s, x, W_r,
                           b_r, T, d, E, k, expert_idx, gate, part_prob, part_cnt, part_z, W_noise, eps,
                           nullptr);
    return hipGetLastError();
}

hipError_t launch_router_reduce(const float *part_prob, const int32_t *part_cnt, int nblk,
                                int E, float *prob_sum, int32_t *route_count, hipStream_t s,
                                const float *part_z, int64_t T, float *z_loss) {
    hipLaunchKernelGGL(router_reduce_kernel, dim3((E + 3) / 4), dim3(256), 0, s, part_prob,
                       part_cnt, nblk, E, prob_sum, route_count, part_z, T, z_loss);
    return hipGetLastError();
}

}  // namespace moe
