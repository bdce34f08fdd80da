// The bf16 grouped-GEMM kernel (gemm_bf16_kernel), its tile shapes and
// the launcher of one tile shape.  Each gemm_bf16_*.hip file instantiates a
// few shapes, so that the shapes compile in parallel; gemm.hip picks the
// shape and holds the fp32 path.  What the kernel computes and how it maps
// onto gfx950 is described at the top of gemm.hip and on Tile and tile_body.
#pragma once
#include "common.h"
#include "launch.h"

#include <math.h>
#include <type_traits>

namespace moe {

// The fused forward's extras (mode 0: none): mode 1 gathers the A rows of
// expert e straight from x (row m of the expert is token row_tok[e C + m]);
// mode 2 scales output row m by row_gate[e C + m] (its token's gate) and
// writes it to row row_tok[e C + m] of y (one expert choice per token).
// kcount (null = off; K a multiple of 64): expert e's K loop covers only its
// first kcount[e] columns of K, rounded up to the 64-wide K tile (at least
// one tile), the rest being zeros it need not read (the weight-gradient
// products contract over an expert's rows, padded to the capacity).
// part (null = off): the split last wave's partial sums (tile-map launches
// only; ncu = the device's compute units, at most TAIL_SPLIT_SLOTS).
struct FuseArgs {
    const int32_t *row_tok;
    int64_t T;
    const float *gate;                                   // row_gate [E, C]
    uint16_t *y;
    int mode;
    const int32_t *kcount;
    float *part;
    int32_t *flags;                                      // the counters after the tile map
    int ncu;
    // tile order within an expert: row tile major (consecutive blocks share
    // the A panel and sweep the column tiles) instead of column tile major
    int row_major;
};

// One grouped-GEMM launch (the arguments of launch_grouped_gemm, resolved):
// expert = a tile covers all rows of an expert; wnt = non-temporal weights.
struct GemmArgs {
    const uint16_t *a, *b, *b3, *bias;
    const int32_t *count, *tile_map;
    int E;
    int64_t C;
    int N, K;
    int64_t rows_bound;
    uint16_t *out;
    hipStream_t s;
    FuseArgs fz;
    int act;
    bool expert, wnt;
};

namespace {


constexpr int MAX_E_LDS = 1024;

// A block's share of a split tile: part p of ns along K, in partial-sum slot
// `slot` (ns = 1: the whole tile, no split).
struct SplitPart {
    int ns, p, slot;
};

// The split of the last wave.  With W full waves of ncu tiles and R tiles
// left over, 0 < 2 R <= ncu, the R tiles of the last wave are each split
// into ns = min(ncu / R, nk / 8, cap) parts along K (at least 8 K tiles per
// part), so that the last wave keeps the whole chip busy for 1 / ns of a
// tile's time instead of R / ncu of it for a whole tile's.  cap = 8 for
// W < 8; 2 for 8 <= W < 32, where tiles of unequal height already stagger
// the end of the launch and each part's own prologue, partial sums and
// fence weigh more; none beyond.  Measured on the Mixtral-shaped layer: its
// second GEMM (4 waves + 80 tiles of 224 K tiles) 1960 -> 1715 us; its first
// (30 waves + 48 tiles of 64) 2 % slower with cap 8, 0.6 % faster with 2.
__device__ __forceinline__ int split_count(int total, int ncu, int nk) {
    if (ncu < 8 || total <= 0 || total >= 32 * ncu) return 1;
    const int R = total % ncu;
    if (R == 0 || 2 * R > ncu) return 1;
    const int cap = total >= 8 * ncu ? 2 : 8;
    int ns = ncu / R;
    ns = ns < nk / 8 ? ns : nk / 8;
    ns = ns < cap ? ns : cap;
    return ns < 2 ? 1 : ns;
}

// Which tile this block computes (tile_map staged in LDS).  Returns false if none.
// Order: expert-major, then column tile, then row tile (row_major: row tile,
// then column tile); block b of XCD b % 8 takes the (b / 8)-th tile of that
// XCD's contiguous share.  With a split
// last wave (split_count > 1) the first W ncu blocks take the first W ncu
// tiles that way and the blocks after them take the parts of the rest,
// tile by tile; the hardware hands out blocks in index order, so those run
// last.
__device__ __forceinline__ bool map_tile(const int32_t *__restrict__ tile_map, int E, int tiles_n,
                                         int *s_map, int &e, int &mt, int &nt, SplitPart &sp, int ncu = 0,
                                         int nk = 0, bool row_major = false) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_map[i] = tile_map[i];
    __syncthreads();
    const int total = s_map[E] * tiles_n;
    const int ns = split_count(total, ncu, nk);
    const int ndp = ns > 1 ? total - total % ncu : total;       // tiles of the whole waves
    const int b = blockIdx.x;
    int L;
    sp.ns = 1;
    sp.p = 0;
    sp.slot = 0;
    if (b < ((ndp + 7) & ~7)) {
        const int per_xcd = (ndp + 7) >> 3;
        const int slot = b >> 3;
        L = (b & 7) * per_xcd + slot;
        if (L >= ndp) return false;
    } else {
        const int q = b - ((ndp + 7) & ~7);
        if (ns == 1 || q >= (total - ndp) * ns) return false;
        const int st = q / ns;
        sp.ns = ns;
        sp.p = q - st * ns;
        sp.slot = q;
        L = ndp + st;
    }
    int lo = 0, hi = E - 1;           // largest e with s_map[e] * tiles_n <= L
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_map[mid] * tiles_n <= L) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int r = L - s_map[e] * tiles_n;
    if (row_major) {
        mt = r / tiles_n;
        nt = r - mt * tiles_n;
    } else {
        const int mtiles = s_map[e + 1] - s_map[e];
        nt = r / mtiles;
        mt = r - nt * mtiles;
    }
    return true;
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

// SiLU for the bf16 epilogue: exp through the hardware exp2 and a hardware
// reciprocal (each about 1 ulp of fp32); the result is rounded to bf16
// (8 significand bits) right after, so the difference from silu() does not
// survive.  Very negative a gives exp2 -> inf, rcp -> 0, result -0.
__device__ __forceinline__ float silu_fast(float a) {
    const float ex = __builtin_amdgcn_exp2f(-a * 1.44269504088896341f);   // e^-a = 2^(-a log2 e)
    return a * __builtin_amdgcn_rcpf(1.0f + ex);
}

// Two bf16 values times a gate, rounded back to bf16: the combine step's
// arithmetic for one kept choice (fp32 fma onto zero, one rounding).
__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t p, float g) {
    return pack_bf16x2(fmaf(g, bf2f((uint16_t)(p & 0xFFFFu)), 0.f), fmaf(g, bf2f((uint16_t)(p >> 16)), 0.f));
}

// Tile shape: block BM x BN (BN = output columns; the gated form also stages
// the matching BN rows of the second weight), K step 64, an S-deep ring of
// LDS stages filled by 16-byte DMA (global_load_lds).  4 waves in a 2 x 2
// grid; each wave owns (BM/2) x (BN/2) outputs = FM x FN fragments of
// v_mfma_f32_32x32x16_bf16 (on gfx950 one wave per SIMD keeps this form
// issuing at nearly the full rate).  Large wave tiles keep the LDS bytes read
// per MFMA low: a 128 x 128 wave tile reads 16 KB of fragments per 64 MFMAs.
// A stage holds BK columns of K: LDS rows of BK bf16 = 8 (BK = 64) or 4
// (BK = 32) pieces of 16 bytes.  Piece c of row r is stored at position
// c ^ swz(r).  A fragment read serves 16 lanes (16 consecutive rows, one
// logical piece) per LDS cycle of 256 bytes, so the 16 addresses must fall in
// 16 different 16-byte bank groups: swz(r) = (r / 2) % 8 for 128-byte rows
// (rows r and r + 8 share r % 2 and so need different positions; r % 8, which
// repeats every 8 rows, measured 2-way conflicts) and (r / 4) % 4 for 64-byte
// rows.  A DMA instruction writes 1 KB contiguously, which is conflict-free
// under any placement.  MINB = 2 sizes the ring and
// the registers for two blocks per CU, so that one block's prologue and
// epilogue overlap the other's MFMAs.
template <int BM_, int BN_, int S_, int BK_ = 64, int MINB_ = 1, int ILV_ = 0, int SB_ = 0, int WK0_ = 0>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, S = S_, BK = BK_, MINB = MINB_;
    // > 0: split ring.  A and the weights get rings of their own: S = 2
    // stages of A (one K tile ahead) and SB = 3 of weights (two ahead), so
    // the weight stream from HBM has twice the lead of the activations, which
    // come from the caches
    static constexpr int SB = SB_;
    // > 0: the DMA of the next stage is spread over the MFMAs of the first ILV
    // k steps instead of issued in one burst (a wave stalls while the address
    // unit is busy, so a burst delays the MFMAs behind it)
    static constexpr int ILV = ILV_;
    // > 0 (split ring): A's DMA is spread over k steps [0, ILV) and the
    // weights' over [WK0, BK / 16), so the address unit takes a steady share
    // of every k step instead of a double one in the first ILV; the weights,
    // needed two K tiles later, go last
    static constexpr int WK0 = WK0_;
    static constexpr int ROWB = BK * 2;                 // bytes per LDS row
    static constexpr int PIECES = BK / 8;               // 16-byte pieces per row
    static constexpr int KS = BK / 16;                  // MFMA k steps per stage
    static constexpr int FM = BM / 64, FN = BN / 64;    // 32x32 fragments per wave
    static constexpr int AI = BM * ROWB / 4096;         // 1 KB DMA instructions per wave per stage (A)
    static constexpr int BI = BN * ROWB / 4096;         // (B)
    static_assert(BM % 64 == 0 && BN % 64 == 0 && S >= 2 && S <= 4, "tile");
    static_assert((BK == 64 || BK == 32) && (MINB == 1 || MINB == 2), "tile");
    static_assert(BK == 32 || BI % 2 == 0, "B groups alternate the swizzle parity");
    static_assert(SB == 0 || (SB == 3 && S == 2), "split ring: 2 stages of A, 3 of weights");
    static_assert(WK0 == 0 || (SB > 0 && ILV > 0 && WK0 >= ILV && WK0 < BK / 16), "weight DMA after A's");
    static __device__ __forceinline__ int swz(int r) { return BK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
};

// 16-byte DMA of one lane into LDS (M0 base + 16 lane) with cache policy AUX
// (0 default, 2 non-temporal); the builtin wants literal arguments.
template <int AUX>
__device__ __forceinline__ void dma16(const uint16_t *src, uint8_t *dst) {
    if constexpr (AUX == 2)
        __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)src, (MOE_LDS_AS void *)dst, 16, 0, 2);
    else
        __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)src, (MOE_LDS_AS void *)dst, 16, 0, 0);
}


// The state of one block's tile shared by the prologue and the K loop: the LDS
// ring and the per-lane DMA sources.  A rows go to LDS in groups of RPI rows
// (one 1 KB DMA instruction); group 4 i + w belongs to instruction i of wave
// w, so the first instructions of every wave cover the first tile rows.
template <class TL, int ACT, bool WNT>
struct TileCtx {
    static constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, ROWB = TL::ROWB, PIECES = TL::PIECES;
    // cache policy of the weight DMA: non-temporal when the weights stream
    // past activations that should stay in the last-level cache
    static constexpr int WAUX = WNT ? 2 : 0;
    static constexpr int AI = TL::AI, BI = TL::BI;
    static constexpr bool DUAL = (ACT == 2);
    static constexpr int NBT = DUAL ? 2 : 1;                       // weight tiles per stage
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    static constexpr int STAGE = A_BYTES + NBT * B_BYTES;
    static constexpr int RPI = 1024 / ROWB;                        // LDS rows per DMA instruction
    uint8_t *st0, *st1, *st2, *st3, *st4;
    const uint16_t *Ae;                                            // the expert's rows of A (or all of x)
    // fused forward: row m of the expert is token rtok[m] (its A row is row
    // rtok[m] of x when gathering; its output goes to row rtok[m] of y,
    // times gate[m] (that token's gate), when scattering)
    const int32_t *rtok;
    const float *gate;
    uint16_t *y;
    int64_t T, arows;                                              // tokens; rows A may index
    bool gather, scatter;
    const uint16_t *asrc[AI];
    const uint16_t *bsrc[BI];
    int64_t b3off;
    // the logical piece this lane fetches: lcA for the A groups of this wave,
    // lcB[j & 1] for B group j (with 128-byte rows swz depends on the parity
    // of the 8-row group: 4 i + wave for A, wave BI + j for B, BI even)
    int K, m0, lane, wave, lr, lcA, lcB[2], nk;
    bool tailA, tailB[2];                                          // piece past K in the last K tile
    // split last wave: this block's K range starts kofs elements in (the DMA
    // sources are offset once, so the K loop is the same for every block);
    // sp says which part of the tile it holds
    int kofs;
    SplitPart sp;
    float *part;
    int32_t *flags;
    int *sflag;                                                    // LDS: this part is the last

    __device__ __forceinline__ void set_lanes(int lane_, int wave_, int K_) {
        lane = lane_;
        wave = wave_;
        K = K_;
        nk = (K + BK - 1) / BK;
        lr = lane / PIECES;
        const int pos = lane % PIECES;
        if (BK == 64) {
            // row 8 g + lr: swz = 4 (g % 2) + lr / 2
            lcA = pos ^ ((4 * (wave & 1)) | (lr >> 1));
            lcB[0] = pos ^ (lr >> 1);
            lcB[1] = pos ^ (4 | (lr >> 1));
        } else {
            // row 16 g + lr: swz = lr / 4
            lcA = lcB[0] = lcB[1] = pos ^ ((lr >> 2) & 3);
        }
        tailA = (nk - 1) * BK + lcA * 8 >= K;
        tailB[0] = (nk - 1) * BK + lcB[0] * 8 >= K;
        tailB[1] = (nk - 1) * BK + lcB[1] * 8 >= K;
    }

    // A sources of the first NA instructions: tile rows m0 + row, the row
    // clamped to last (rows past the count are computed but never stored).
    // Gathering, the row's token comes from rtok; an entry past the count
    // may hold anything, so the token is clamped into [0, T).
    template <int NA>
    __device__ __forceinline__ void set_a(int last) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            int am = m0 + (4 * i + wave) * RPI + lr;
            am = am < last ? am : last;
            asrc[i] = Ae + (int64_t)am * K + lcA * 8 + kofs;
        }
    }
    // gathering: the tokens of the rows the A instructions cover (rows past
    // last repeat row last), loaded first so that their latency overlaps the
    // weight DMA issued next; set_a_tok then points the A sources at them
    __device__ __forceinline__ void load_tok(int last, int32_t (&tok)[AI]) const {
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            int am = m0 + (4 * i + wave) * RPI + lr;
            tok[i] = rtok[am < last ? am : last];
        }
    }
    __device__ __forceinline__ void set_a_tok(const int32_t (&tok)[AI]) {
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            const int64_t t = (uint32_t)tok[i];
            asrc[i] = Ae + (t < arows ? t : arows - 1) * K + lcA * 8 + kofs;
        }
    }
    // K offset (elements, from the block's first K tile) of K tile kt for A
    // and for B group j: the pieces past K of the last K tile read the
    // block's first column instead (in bounds; a part other than the last of
    // a split tile has no tail: its tail flags are cleared)
    template <bool KTAIL>
    __device__ __forceinline__ int ka(int kt) const {
        return (KTAIL && kt == nk - 1 && tailA) ? -lcA * 8 : kt * BK;
    }
    template <bool KTAIL>
    __device__ __forceinline__ int kb(int kt, int j) const {
        return (KTAIL && kt == nk - 1 && tailB[j & 1]) ? -lcB[j & 1] * 8 : kt * BK;
    }
};

// DMA of K tile kt into one stage: NA instructions of A, then those of B (and
// B3).  Lane l lands at byte 16 l of its 1 KB group = row l / PIECES,
// position l % PIECES, which holds logical piece (l % PIECES) ^ swz(row).  The
// pieces past K (K % BK != 0) of the last K tile are read from the block's
// first column and cleared in LDS once they have landed.
// PARTS: 1 = the A instructions (K tile kta into abase), 2 = the weight
// instructions (K tile ktb into bbase), 3 = both (the waits count the
// instructions issued after a stage's own, so the order matters).
template <int NA, bool KTAIL, class CTX, int PARTS = 3>
__device__ __forceinline__ void tile_issue2(const CTX &c, uint8_t *abase, uint8_t *bbase, int kta, int ktb) {
    if (PARTS & 1) {
        const int ka = c.template ka<KTAIL>(kta);
#pragma unroll
        for (int i = 0; i < NA; ++i)
            __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)(c.asrc[i] + ka),
                                             (MOE_LDS_AS void *)(abase + (4 * i + c.wave) * 1024), 16, 0, 0);
    }
    if (PARTS & 2) {
#pragma unroll
        for (int j = 0; j < CTX::BI; ++j)
            dma16<CTX::WAUX>(c.bsrc[j] + c.template kb<KTAIL>(ktb, j), bbase + (c.wave * CTX::BI + j) * 1024);
        if (CTX::DUAL) {
#pragma unroll
            for (int j = 0; j < CTX::BI; ++j)
                dma16<CTX::WAUX>(c.bsrc[j] + c.b3off + c.template kb<KTAIL>(ktb, j),
                                 bbase + CTX::B_BYTES + (c.wave * CTX::BI + j) * 1024);
        }
    }
    // keep every DMA of the stage ahead of the MFMAs that follow (left to
    // itself the scheduler sinks them to the end of the step, which leaves
    // almost no time for them to land)
    __builtin_amdgcn_sched_barrier(0);
}
// A stage holding both operands: A at base, the weights after it.
template <int NA, bool KTAIL, class CTX, int PARTS = 3>
__device__ __forceinline__ void tile_issue(const CTX &c, uint8_t *base, int kt) {
    tile_issue2<NA, KTAIL, CTX, PARTS>(c, base, base + CTX::A_BYTES, kt, kt);
}

// The K loop and epilogue of a tile whose rows that hold data lie in
// [0, 64 FV): FV 32-row fragments per wave (wave row wm owns tile rows
// 64 i + 32 wm + 0..31) and the A-DMA instructions of those rows only.  The
// caller has issued K tiles 0 .. S - 2 with every A instruction.
template <class TL, int FV, int ACT, bool BIAS, bool KTAIL, class X>
__device__ __forceinline__ void tile_body(X &c, const uint16_t *__restrict__ bias_e, int cnt, int n0, int N,
                                          uint16_t *__restrict__ oe, int *s_tok, float *s_g) {
    constexpr int BN = TL::BN, S = TL::S, ROWB = TL::ROWB, KS = TL::KS, FN = TL::FN, BI = TL::BI;
    constexpr bool DUAL = X::DUAL;
    constexpr int NBT = X::NBT, A_BYTES = X::A_BYTES, B_BYTES = X::B_BYTES;
    constexpr int NA = FV * 64 / (4 * X::RPI);           // A-DMA instructions per wave
    static_assert(NA >= 1 && NA <= TL::AI && NA * 4 * X::RPI == FV * 64, "A rows per wave");
    constexpr int PER = NA + NBT * BI;
    constexpr bool SPLIT = TL::SB > 0;
    // DMA instructions a wave issues after a stage's own before that stage is
    // waited for: those of the S - 2 newer stages (the prologue's stages hold
    // more, which only makes the first waits stricter).  Split ring: step kt
    // needs A(kt) and the weights of kt, and only the weights of kt + 1 were
    // issued after A(kt).
    constexpr int NEWER = SPLIT ? NBT * BI : (S - 2) * PER;
    constexpr int ROWS = FV * 64;                        // tile rows computed and stored
    // the output rows are staged in LDS when they fit, else stored from
    // registers: two stage buffers (one per wave row), or with the split ring
    // one buffer per 64-row chunk: all five stages, or the three weight
    // stages when a chunk is larger than an A stage (tiles of 192 rows)
    constexpr int CHUNK = 64 * BN * 2;
    constexpr bool CH_IN_A = CHUNK <= A_BYTES;
    constexpr bool STAGED_OUT = SPLIT ? (CHUNK <= NBT * B_BYTES && TL::FM <= (CH_IN_A ? 5 : 3))
                                      : TL::BM * BN <= X::STAGE;
    const int lane = c.lane, wave = c.wave, nk = c.nk;
    const int wm = wave >> 1, wn = wave & 1;
    uint8_t *const st0 = c.st0, *const st1 = c.st1, *const st2 = c.st2, *const st3 = c.st3,
                   *const st4 = c.st4;
    // A sources of the data rows, clamped to the expert's last row (rows past
    // the count are computed but never stored); gathering keeps the prologue's
    // sources, whose rows past the count hold valid tokens too
    if (!c.gather) c.template set_a<NA>(cnt - 1);
    // scattering: each thread fetches the token and gate of up to two stored
    // rows now; they land during the K loop and go to LDS in the epilogue
    int ptok[2] = {0, 0};
    float pgate[2] = {0.f, 0.f};
    if (c.scatter) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = threadIdx.x + 256 * h;
            if (r < ROWS && c.m0 + r < cnt) {
                ptok[h] = c.rtok[c.m0 + r];
                pgate[h] = c.gate[c.m0 + r];
            }
        }
    }

    // na / nb: where A of K tile kta and the weights of K tile ktb go
    auto issue = [&](uint8_t *na, uint8_t *nb, int kta, int ktb) { tile_issue2<NA, KTAIL>(c, na, nb, kta, ktb); };
    auto clear_tail = [&](uint8_t *sa, uint8_t *sb) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (c.tailA) {
#pragma unroll
            for (int i = 0; i < NA; ++i) *reinterpret_cast<u32x4 *>(sa + (4 * i + wave) * 1024 + lane * 16) = z;
        }
#pragma unroll
        for (int j = 0; j < NBT * BI; ++j)
            if (c.tailB[(j % BI) & 1])
                *reinterpret_cast<u32x4 *>(sb + (j / BI) * B_BYTES + (wave * BI + (j % BI)) * 1024 + lane * 16) = z;
    };

    // accumulators hold C^T fragments: acc[i][j] = weight rows (n) x x rows (m);
    // lane l holds output row m = l % 32 of the fragment and, for g = 0..3, the
    // four consecutive columns n = 8 g + 4 (l / 32) + 0..3 in elements 4g..4g+3
    f32x16 acc[FV][FN];
    f32x16 acc3[DUAL ? FV : 1][DUAL ? FN : 1];
#pragma unroll
    for (int i = 0; i < FV; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
#pragma unroll
    for (int i = 0; i < (DUAL ? FV : 1); ++i)
#pragma unroll
        for (int j = 0; j < (DUAL ? FN : 1); ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc3[i][j][q] = 0.f;

    // fragment reads (32 x 16 operands): row (base + lane % 32), logical piece
    // 2 ks + lane / 32; fragment bases are multiples of 32, so the stored
    // position is piece ^ swz(lane % 32)
    const int arow = (32 * wm + (lane & 31)) * ROWB;
    const int brow = (wn * (BN / 2) + (lane & 31)) * ROWB;
    const int fswz = TL::swz(lane & 31);
    // fragments of two k steps: the reads of k step ks + 1 are issued between
    // the MFMAs of k step ks
    bf16x8 af[2][FV], bfr[2][FN], bf3[DUAL ? 2 : 1][DUAL ? FN : 1];
    auto rd = [&](const uint8_t *sa, const uint8_t *sb, int ks, int sl) {
        const int pofs = ((ks * 2 + (lane >> 5)) ^ fswz) << 4;
#pragma unroll
        for (int i = 0; i < FV; ++i)
            af[sl][i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sa + arow + i * 64 * ROWB + pofs));
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bfr[sl][j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + brow + j * 32 * ROWB + pofs));
        if (DUAL) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf3[DUAL ? sl : 0][DUAL ? j : 0] =
                    as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + B_BYTES + brow + j * 32 * ROWB + pofs));
        }
    };
    // per k step: R fragment reads (of the next k step) and M MFMAs, paired
    // one read after each MFMA while both last
    constexpr int R = FV + NBT * FN;
    constexpr int M = FV * FN * NBT;
    constexpr int RM = R > M ? R : M;
    // DMA instruction q of a stage (A rows, then B, then B3), for spreading a
    // stage's DMA over the MFMAs of the first ILV k steps
    auto dma_one = [&](uint8_t *na, uint8_t *nb, int kta, int ktb, int q) {
        if (q < NA)
            __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)(c.asrc[q] + c.template ka<KTAIL>(kta)),
                                             (MOE_LDS_AS void *)(na + (4 * q + wave) * 1024), 16, 0, 0);
        else if (q < NA + BI)
            dma16<X::WAUX>(c.bsrc[q - NA] + c.template kb<KTAIL>(ktb, q - NA), nb + (wave * BI + q - NA) * 1024);
        else
            dma16<X::WAUX>(c.bsrc[q - NA - BI] + c.b3off + c.template kb<KTAIL>(ktb, q - NA - BI),
                           nb + B_BYTES + (wave * BI + q - NA - BI) * 1024);
    };
    constexpr int ILV = TL::ILV < KS ? TL::ILV : KS;
    constexpr int SLOTS = (ILV > 0 ? ILV : 1) * M;
    // MFMA slot (k step * M + MFMA) after which DMA instruction q of a stage
    // goes out: all over the first ILV k steps, or A over those and the
    // weights over k steps [WK0, KS).  Issue order stays A, then weights,
    // which the split ring's wait count relies on (the k steps end in
    // scheduling barriers).
    constexpr int WK0 = TL::WK0;
    auto slot_of = [](int q) constexpr -> int {
        if (WK0 == 0) return q * SLOTS / PER;
        if (q < NA) return q * SLOTS / NA;
        return WK0 * M + (q - NA) * ((KS - WK0) * M) / (PER - NA);
    };
    // the MFMAs of one K tile; the fragments of its k step 0 are already read.
    // With ILV, the DMA of A (K tile kta into na) and of the weights (ktb
    // into nb) is spread over its first k steps.
    auto compute = [&](const uint8_t *sa, const uint8_t *sb, uint8_t *na, uint8_t *nb, int kta, int ktb,
                       auto with_dma) {
        constexpr bool IL = decltype(with_dma)::value && ILV > 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int sl = ks & 1;
            if (IL) {
#pragma unroll
                for (int q = 0; q < PER; ++q)
                    if (slot_of(q) / M == ks) dma_one(na, nb, kta, ktb, q);
            }
            if (ks < KS - 1) rd(sa, sb, ks + 1, sl ^ 1);
#pragma unroll
            for (int i = 0; i < FV; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[sl][j], af[sl][i], acc[i][j], 0, 0, 0);
            if (DUAL) {
#pragma unroll
                for (int i = 0; i < (DUAL ? FV : 1); ++i)
#pragma unroll
                    for (int j = 0; j < (DUAL ? FN : 1); ++j)
                        acc3[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf3[DUAL ? sl : 0][j], af[sl][i],
                                                                             acc3[i][j], 0, 0, 0);
            }
            if (IL) {
#pragma unroll
                for (int r = 0; r < RM; ++r) {
                    if (r < M) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    if (ks < KS - 1 && r < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
#pragma unroll
                    for (int q = 0; q < PER; ++q)
                        if (slot_of(q) == ks * M + r) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            } else if (ks < KS - 1) {
#pragma unroll
                for (int r = 0; r < RM; ++r) {
                    if (r < M) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    if (r < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- the ring: K tile kt lives in stage kt % S.  Step kt waits for its
    // own DMA (the S - 2 newer stages stay in flight), passes one barrier (all
    // waves have landed their part of kt and finished reading kt - 1), refills
    // the stage of kt - 1 with kt + S - 1, then runs the MFMAs of kt.  Split
    // ring: A of kt is in a[kt % 2] (st0, st1), its weights in b[kt % 3]
    // (st2, st3, st4); step kt refills a[(kt + 1) % 2] with A of kt + 1 and
    // b[(kt + 2) % 3] with the weights of kt + 2, both consumed at kt - 1.
    int kt = 0;
    constexpr auto DMA_ON = std::integral_constant<bool, true>();
    constexpr auto DMA_OFF = std::integral_constant<bool, false>();
    // steady state: every step refills, so the wait count is fixed and the
    // loop body has no branch
#define MOE_STEP2(CA, CB, NA_, NB_, KA, KB)                                     \
    {                                                                           \
        wait_vm_lgkm0<NEWER>();                                                 \
        ring_barrier();                                                         \
        rd(CA, CB, 0, 0);                                                       \
        if (ILV == 0) issue(NA_, NB_, KA, KB);                                  \
        compute(CA, CB, NA_, NB_, KA, KB, DMA_ON);                              \
        ++kt;                                                                   \
    }
#define MOE_STEP(CUR, NXT) MOE_STEP2(CUR, CUR + A_BYTES, NXT, NXT + A_BYTES, kt + S - 1, kt + S - 1)
#define MOE_STEPS(CA, CB, NA_, NB_) MOE_STEP2(CA, CB, NA_, NB_, kt + 1, kt + 2)
    if constexpr (SPLIT) {
        for (; kt + 8 <= nk;) {
            MOE_STEPS(st0, st2, st1, st4)
            MOE_STEPS(st1, st3, st0, st2)
            MOE_STEPS(st0, st4, st1, st3)
            MOE_STEPS(st1, st2, st0, st4)
            MOE_STEPS(st0, st3, st1, st2)
            MOE_STEPS(st1, st4, st0, st3)
        }
    } else {
        for (; kt + 2 * S - 1 <= nk;) {
            if constexpr (S == 2) {
                MOE_STEP(st0, st1)
                MOE_STEP(st1, st0)
            } else if constexpr (S == 3) {
                MOE_STEP(st0, st2)
                MOE_STEP(st1, st0)
                MOE_STEP(st2, st1)
            } else {
                MOE_STEP(st0, st3)
                MOE_STEP(st1, st0)
                MOE_STEP(st2, st1)
                MOE_STEP(st3, st2)
            }
        }
    }
#undef MOE_STEPS
#undef MOE_STEP
#undef MOE_STEP2
    // drain, refilling while K tiles remain: at most 2 S - 2 steps with
    // kt % S == 0 at the start, or 7 split steps with kt % 6 == 0
#define MOE_TAIL(CUR, NXT)                                                      \
    if (kt < nk) {                                                              \
        if (kt + S - 2 < nk) wait_vm_lgkm0<NEWER>();                            \
        else wait_vm_lgkm0<0>();                                                \
        if (KTAIL && kt == nk - 1) {                                            \
            clear_tail(CUR, CUR + A_BYTES);                                     \
            wait_vm_lgkm0<63>();          /* the zeros are in LDS */            \
        }                                                                       \
        ring_barrier();                                                         \
        rd(CUR, CUR + A_BYTES, 0, 0);                                           \
        if (kt + S - 1 < nk) issue(NXT, NXT + A_BYTES, kt + S - 1, kt + S - 1); \
        __builtin_amdgcn_sched_barrier(0);                                      \
        compute(CUR, CUR + A_BYTES, NXT, NXT + A_BYTES, 0, 0, DMA_OFF);         \
        ++kt;                                                                   \
    }
#define MOE_TAILS(CA, CB, NA_, NB_)                                             \
    if (kt < nk) {                                                              \
        if (kt + 1 < nk) wait_vm_lgkm0<NEWER>();                                \
        else wait_vm_lgkm0<0>();                                                \
        if (KTAIL && kt == nk - 1) {                                            \
            clear_tail(CA, CB);                                                 \
            wait_vm_lgkm0<63>();          /* the zeros are in LDS */            \
        }                                                                       \
        ring_barrier();                                                         \
        rd(CA, CB, 0, 0);                                                       \
        if (kt + 1 < nk) tile_issue2<NA, KTAIL, X, 1>(c, NA_, NB_, kt + 1, 0);  \
        if (kt + 2 < nk) tile_issue2<NA, KTAIL, X, 2>(c, NA_, NB_, 0, kt + 2);  \
        __builtin_amdgcn_sched_barrier(0);                                      \
        compute(CA, CB, NA_, NB_, 0, 0, DMA_OFF);                               \
        ++kt;                                                                   \
    }
    if constexpr (SPLIT) {
        MOE_TAILS(st0, st2, st1, st4)
        MOE_TAILS(st1, st3, st0, st2)
        MOE_TAILS(st0, st4, st1, st3)
        MOE_TAILS(st1, st2, st0, st4)
        MOE_TAILS(st0, st3, st1, st2)
        MOE_TAILS(st1, st4, st0, st3)
        MOE_TAILS(st0, st2, st1, st4)
    } else if constexpr (S == 2) {
        MOE_TAIL(st0, st1)
        MOE_TAIL(st1, st0)
    } else if constexpr (S == 3) {
        MOE_TAIL(st0, st2)
        MOE_TAIL(st1, st0)
        MOE_TAIL(st2, st1)
        MOE_TAIL(st0, st2)
    } else {
        MOE_TAIL(st0, st3)
        MOE_TAIL(st1, st0)
        MOE_TAIL(st2, st1)
        MOE_TAIL(st3, st2)
        MOE_TAIL(st0, st3)
        MOE_TAIL(st1, st0)
    }
#undef MOE_TAILS
#undef MOE_TAIL

    // ---- split last wave: every part stores its fp32 sums (lane-major, so
    // the stores and loads are 16-byte and coalesced); the last part to finish
    // adds all of them in part order, so the result does not depend on which
    // part finishes last, and goes on to the epilogue
    if (c.sp.ns > 1) {
        constexpr int PF4 = TAIL_SPLIT_PART_FLOATS / 4;
        static_assert(FV * FN * NBT * 16 * 256 <= TAIL_SPLIT_PART_FLOATS, "partial-sum slot");
        const int tid = threadIdx.x;
        f32x4 *own = reinterpret_cast<f32x4 *>(c.part) + (size_t)c.sp.slot * PF4;
#pragma unroll
        for (int i = 0; i < FV; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    own[(((i * FN + j) * 4 + v) << 8) + tid] =
                        f32x4{acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]};
                    if (DUAL)
                        own[((((FV + i) * FN + j) * 4 + v) << 8) + tid] =
                            f32x4{acc3[DUAL ? i : 0][DUAL ? j : 0][4 * v], acc3[DUAL ? i : 0][DUAL ? j : 0][4 * v + 1],
                                  acc3[DUAL ? i : 0][DUAL ? j : 0][4 * v + 2], acc3[DUAL ? i : 0][DUAL ? j : 0][4 * v + 3]};
                    __builtin_amdgcn_sched_barrier(0);
                }
        const int tile_slot = c.sp.slot / c.sp.ns;
        // every wave's stores have reached L2; one device-scope release fence
        // (it writes back the whole L2, so once per block) makes them visible
        // before the count, and the last part's acquire fence (it invalidates
        // this CU's L1 and the L2) comes before any wave reads the others'
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            __threadfence();
            *c.sflag = atomicAdd(c.flags + tile_slot, 1) == c.sp.ns - 1;
            if (*c.sflag) __threadfence();
        }
        __syncthreads();
        if (!*c.sflag) return;
        const f32x4 *first = reinterpret_cast<const f32x4 *>(c.part) + (size_t)(c.sp.slot - c.sp.p) * PF4 + tid;
        const int ns = c.sp.ns;
        // one 16-byte piece at a time through the parts (few live registers:
        // the accumulators fill the register file)
        auto total = [&](int f, int v) -> f32x4 {
            const f32x4 *src = first + (((f * 4 + v)) << 8);
            f32x4 t = src[0];
            for (int q = 1; q < ns; ++q) t += src[(size_t)q * PF4];
            return t;
        };
#pragma unroll
        for (int i = 0; i < FV; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const f32x4 t = total(i * FN + j, v);
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[i][j][4 * v + u] = t[u];
                    if (DUAL) {
                        const f32x4 t3 = total((FV + i) * FN + j, v);
#pragma unroll
                        for (int u = 0; u < 4; ++u) acc3[DUAL ? i : 0][DUAL ? j : 0][4 * v + u] = t3[u];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
        if (tid == 0) c.flags[tile_slot] = 0;            // cleared for the next launch
    }

    // ---- epilogue: bias, activation, bf16.  With STAGED_OUT the rows of wave
    // row wm go to stage buffer wm (16-byte pieces swizzled by row), so that
    // rows leave as coalesced 16-byte stores; otherwise each lane stores its
    // four consecutive columns (8 bytes) directly.
    constexpr int P = BN / 8;                            // 16-byte pieces per output row
    // piece swizzle of the staged rows (keeps a piece in its row): 16 rows of
    // a store phase fall in distinct 16-byte bank groups (rows of 384 bytes
    // alternate between the two 128-byte halves of a 256-byte bank line)
    auto esw = [](int r) { return (P & (P - 1)) == 0 ? (r & (P - 1)) : ((r >> 1) & 7); };
    const int m0 = c.m0;
    // scattering: the token and gate of every stored row, staged once
    const bool scatter = c.scatter;
    if (scatter) {
        static_assert(ROWS <= 512, "two rows per thread");
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = threadIdx.x + 256 * h;
            if (r < ROWS) {
                const int64_t tt = (uint32_t)ptok[h];
                s_tok[r] = (int)(tt < c.T ? tt : c.T - 1);
                s_g[r] = pgate[h];
            }
        }
    }
    if (STAGED_OUT || scatter) lds_barrier();            // every wave is past its last fragment read
    // the staging buffer of 64-row chunk i (split ring)
    auto chunk_buf = [&](int i) -> uint8_t * {
        if (!CH_IN_A) return i == 0 ? st2 : i == 1 ? st3 : st4;
        return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : i == 3 ? st3 : st4;
    };
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nl = wn * (BN / 2) + j * 32 + 8 * g + 4 * (lane >> 5);   // 4 consecutive columns
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (BIAS) {
                const int n = n0 + nl;
                if (n < N) {
                    const uint2 bb = *reinterpret_cast<const uint2 *>(bias_e + n);
                    bv[0] = bf2f((uint16_t)(bb.x & 0xFFFFu));
                    bv[1] = bf2f((uint16_t)(bb.x >> 16));
                    bv[2] = bf2f((uint16_t)(bb.y & 0xFFFFu));
                    bv[3] = bf2f((uint16_t)(bb.y >> 16));
                }
            }
#pragma unroll
            for (int i = 0; i < FV; ++i) {
                // staged row: within the wave row's buffer, or within chunk i's
                const int r = SPLIT ? 32 * wm + (lane & 31) : i * 32 + (lane & 31);
                uint8_t *so = SPLIT ? chunk_buf(i) : (wm ? st1 : st0);
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float t = acc[i][j][4 * g + q] + bv[q];
                    if (ACT == 1) t = fmaxf(t, 0.f);
                    if (ACT == 2) t = silu_fast(t) * acc3[DUAL ? i : 0][DUAL ? j : 0][4 * g + q];
                    v[q] = t;
                }
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                if (STAGED_OUT) {
                    const int pc = (nl >> 3) ^ esw(r);
                    *reinterpret_cast<uint2 *>(so + r * (BN * 2) + (pc << 4) + ((nl & 4) << 1)) = pk;
                } else {
                    const int rr = 64 * i + 32 * wm + (lane & 31);
                    const int m = m0 + rr;
                    const int n = n0 + nl;
                    if (m < cnt && n < N) {
                        if (scatter) {
                            const float gg = s_g[rr];
                            pk.x = scale_bf16x2(pk.x, gg);
                            pk.y = scale_bf16x2(pk.y, gg);
                            *reinterpret_cast<uint2 *>(c.y + (int64_t)s_tok[rr] * N + n) = pk;
                        } else {
                            *reinterpret_cast<uint2 *>(oe + (int64_t)m * N + n) = pk;
                        }
                    }
                }
            }
        }
    }
    if (STAGED_OUT) {
        lds_barrier();
        static_assert(!STAGED_OUT || (ROWS * P) % 256 == 0, "whole store rounds");
#pragma unroll
        for (int it = 0; it < ROWS * P / 256; ++it) {
            const int q = threadIdx.x + it * 256;
            const int Rw = q / P;                        // tile row
            const int p = q % P;
            // its row in the wave row's buffer, or in its 64-row chunk's
            const int r = SPLIT ? (Rw & 63) : (((Rw >> 6) << 5) | (Rw & 31));
            const uint8_t *sbuf = SPLIT ? chunk_buf(Rw >> 6) : (((Rw >> 5) & 1) ? st1 : st0);
            const uint8_t *src = sbuf + r * (BN * 2) + ((p ^ esw(r)) << 4);
            const int m = m0 + Rw;
            const int n = n0 + p * 8;
            if (m < cnt && n < N) {
                u32x4 v = *reinterpret_cast<const u32x4 *>(src);
                if (scatter) {
                    const float gg = s_g[Rw];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = scale_bf16x2(v[q], gg);
                    st16(c.y + (int64_t)s_tok[Rw] * N + n, v);
                } else {
                    st16(oe + (int64_t)m * N + n, v);
                }
            }
        }
    }
}

// One tile per block.  EXPERT: the tile covers all rows of an expert (BM >= C),
// block -> (expert, column tile) directly, and the first stages are issued
// before the expert's count is known; else the block finds its (expert, row
// tile, column tile) in tile_map.  The K loop then runs in the specialization
// for the 64-row chunks of the tile that hold data.
template <class TL, int ACT, bool BIAS, bool KTAIL, bool EXPERT, bool WNT>
__global__ __launch_bounds__(256, TL::MINB) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, const uint16_t *__restrict__ B3,
    const uint16_t *__restrict__ bias, const int32_t *__restrict__ count,
    const int32_t *__restrict__ tile_map, int E, int64_t C, int N, int K, int tiles_n,
    uint16_t *__restrict__ out, FuseArgs fz) {
    using X = TileCtx<TL, ACT, WNT>;
    constexpr int BM = TL::BM, BN = TL::BN, S = TL::S, FM = TL::FM;
    constexpr int STAGE = X::STAGE;
    constexpr bool SPLIT = TL::SB > 0;
    constexpr int SA = X::A_BYTES, SBW = X::NBT * X::B_BYTES;   // split ring: A and weight stages
    // one LDS array per stage: the compiler then sees that the fragment reads of
    // one stage cannot alias the DMA in flight into another and adds no wait
    __shared__ __attribute__((aligned(1024))) uint8_t st0[SPLIT ? SA : STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[SPLIT ? SA : STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[SPLIT ? SBW : (S > 2 ? STAGE : 16)];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[SPLIT ? SBW : (S > 3 ? STAGE : 16)];
    __shared__ __attribute__((aligned(1024))) uint8_t st4[SPLIT ? SBW : 16];
    // the tile map (read before the ring starts), the scattered rows' tokens
    // and gates and the split flag (both used after the ring has drained):
    // when the ring takes the whole LDS they live in the last weight stage,
    // which the ring first fills in its first step (after a barrier every
    // wave reaches past its tile-map reads) and which the epilogue's row
    // staging (chunks of 64 rows in the first four stages) leaves alone
    constexpr int NMAP = EXPERT ? 1 : MAX_E_LDS + 1;
    constexpr int SMALL = (NMAP + 2 * BM + 1) * 4;
    constexpr bool ALIAS = SPLIT && 2 * SA + 3 * SBW + SMALL > 160 * 1024;
    static_assert(!ALIAS || (SMALL <= SBW && FM <= 4 && 64 * BN * 2 <= SA), "small arrays in the last weight stage");
    int *s_map, *s_tok, *s_last;                         // s_tok, s_g: scattering, token and gate of each row
    float *s_g;
    if constexpr (ALIAS) {
        s_map = reinterpret_cast<int *>(st4);
        s_tok = s_map + NMAP;
        s_g = reinterpret_cast<float *>(s_tok + BM);
        s_last = reinterpret_cast<int *>(s_g + BM);
    } else {
        __shared__ int s_map_[NMAP];
        __shared__ int s_tok_[BM];
        __shared__ float s_g_[BM];
        __shared__ int s_last_;
        s_map = s_map_;
        s_tok = s_tok_;
        s_g = s_g_;
        s_last = &s_last_;
    }

    int e, mt, nt;
    SplitPart sp{1, 0, 0};
    if (EXPERT) {
        // expert-major, then column tile; block b of XCD b % 8 takes the
        // (b / 8)-th tile of that XCD's contiguous share
        const int total = E * tiles_n;
        const int per_xcd = (total + 7) >> 3;
        const int slot = blockIdx.x >> 3;
        const int L = (blockIdx.x & 7) * per_xcd + slot;
        if (slot >= per_xcd || L >= total) return;
        e = L / tiles_n;
        nt = L - e * tiles_n;
        mt = 0;
    } else {
        // the split last wave needs whole K loops (no per-expert K) and the
        // partial-sum buffer
        const int ncu = (fz.part != nullptr && fz.kcount == nullptr) ? fz.ncu : 0;
        if (!map_tile(tile_map, E, tiles_n, s_map, e, mt, nt, sp, ncu, (K + TL::BK - 1) / TL::BK,
                      fz.row_major != 0))
            return;
    }

    X c;
    c.st0 = st0; c.st1 = st1; c.st2 = st2; c.st3 = st3; c.st4 = st4;
    // wave-uniform wave index (DMA base)
    c.set_lanes(threadIdx.x & 63, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), K);
    if (fz.kcount != nullptr) {
        // this expert's rows of K only, in whole K tiles (K % 64 == 0: no tail)
        const int kc = fz.kcount[e];
        const int nke = (kc + TL::BK - 1) / TL::BK;
        c.nk = nke < 1 ? 1 : (nke < c.nk ? nke : c.nk);
    }
    c.kofs = 0;
    c.sp = SplitPart{1, 0, 0};
    c.part = fz.part;
    c.flags = fz.flags;
    c.sflag = s_last;
    if constexpr (!EXPERT) {
        // wave-uniform (scalar registers: the vector ones are all taken)
        c.sp.ns = __builtin_amdgcn_readfirstlane(sp.ns);
        c.sp.p = __builtin_amdgcn_readfirstlane(sp.p);
        c.sp.slot = __builtin_amdgcn_readfirstlane(sp.slot);
    }
    if (c.sp.ns > 1) {
        // K tiles [p nk / ns, (p + 1) nk / ns): at least 8 each; only the
        // last part holds the K tail
        const int k0 = c.sp.p * c.nk / c.sp.ns, k1 = (c.sp.p + 1) * c.nk / c.sp.ns;
        c.kofs = __builtin_amdgcn_readfirstlane(k0) * TL::BK;
        c.nk = __builtin_amdgcn_readfirstlane(k1 - k0);
        if (c.sp.p != c.sp.ns - 1) c.tailA = c.tailB[0] = c.tailB[1] = false;
    }
    c.m0 = mt * BM;
    c.b3off = X::DUAL ? (int64_t)(B3 - B) : 0;
    c.gather = fz.mode == 1;
    c.scatter = fz.mode == 2;
    c.rtok = fz.row_tok != nullptr ? fz.row_tok + (int64_t)e * C : nullptr;
    c.T = fz.T;
    c.arows = c.gather ? fz.T : C;                       // bound of the A row index
    c.gate = fz.gate != nullptr ? fz.gate + (int64_t)e * C : nullptr;
    c.y = fz.y;
    c.Ae = c.gather ? A : A + (int64_t)e * C * K;
    const int n0 = nt * BN;
    {
        const uint16_t *Be = B + (int64_t)e * N * K;
#pragma unroll
        for (int j = 0; j < TL::BI; ++j) {
            int bn = n0 + (c.wave * TL::BI + j) * X::RPI + c.lr;
            bn = bn < N ? bn : N - 1;
            c.bsrc[j] = Be + (int64_t)bn * K + c.lcB[j & 1] * 8 + c.kofs;
        }
    }
    // prologue: K tiles 0 .. S - 2 with every A row (clamped to the last row
    // of the capacity), each clamped to the last K tile when there are fewer
    // (the duplicate loads are never read).  Unconditional on purpose: a
    // conditional DMA here makes the compiler give up tracking which stage a
    // pending DMA writes, and then it drains the whole ring before every
    // fragment read.
    // The A rows: gathering, the row tokens are loaded first and stage 0's
    // weight DMA goes out while they land; otherwise the row indices
    // themselves (the DMA is issued the same way on both paths, with no
    // branch around it: a conditional DMA costs the ring its lookahead).
    {
        int32_t tok[TL::AI];
        if (c.gather) {
            c.load_tok((int)C - 1, tok);
        } else {
#pragma unroll
            for (int i = 0; i < TL::AI; ++i) {
                const int am = c.m0 + (4 * i + c.wave) * X::RPI + c.lr;
                tok[i] = am < (int)C - 1 ? am : (int)C - 1;
            }
        }
        // stage 0: weights, then A (split ring: A into st0, weights into st2)
        uint8_t *b0 = SPLIT ? st2 : st0 + X::A_BYTES;
        tile_issue2<TL::AI, KTAIL, X, 2>(c, st0, b0, 0, 0);
        c.set_a_tok(tok);
        tile_issue2<TL::AI, KTAIL, X, 1>(c, st0, b0, 0, 0);
    }
    if (SPLIT) {
        // the weights of K tile 1 (clamped), one stage further ahead
        tile_issue2<TL::AI, KTAIL, X, 2>(c, st1, st3, 0, c.nk > 1 ? 1 : c.nk - 1);
    } else {
        if (S > 2) tile_issue<TL::AI, KTAIL>(c, st1, c.nk > 1 ? 1 : c.nk - 1);
        if (S > 3) tile_issue<TL::AI, KTAIL>(c, st2, c.nk > 2 ? 2 : c.nk - 1);
    }

    const int cnt = count[e];
    const int rows = cnt - c.m0;                         // > 0 for every mapped tile
    if (rows <= 0) {
        wait_vm_lgkm0<0>();                              // no DMA may land after the block ends
        return;
    }
    const int fv = rows >= BM ? FM : (rows + 63) >> 6;
    const uint16_t *bias_e = BIAS ? bias + (int64_t)e * N : nullptr;
    uint16_t *oe = out + (int64_t)e * C * N;
    if constexpr (FM >= 5) if (fv == 5) { tile_body<TL, 5, ACT, BIAS, KTAIL>(c, bias_e, cnt, n0, N, oe, s_tok, s_g); return; }
    if constexpr (FM >= 4) if (fv == 4) { tile_body<TL, 4, ACT, BIAS, KTAIL>(c, bias_e, cnt, n0, N, oe, s_tok, s_g); return; }
    if constexpr (FM >= 3) if (fv == 3) { tile_body<TL, 3, ACT, BIAS, KTAIL>(c, bias_e, cnt, n0, N, oe, s_tok, s_g); return; }
    if (fv == 2) { tile_body<TL, 2, ACT, BIAS, KTAIL>(c, bias_e, cnt, n0, N, oe, s_tok, s_g); return; }
    tile_body<TL, 1, ACT, BIAS, KTAIL>(c, bias_e, cnt, n0, N, oe, s_tok, s_g);
}

// Blocks for at most E * ceil(C / bm) row tiles, and at most
// ceil(rows_bound / bm) + E of them (each expert wastes at most one partial tile).
inline int64_t grid_for(int64_t C, int E, int bm, int tiles_n, int64_t rows_bound) {
    int64_t m = (int64_t)E * ((C + bm - 1) / bm);
    const int64_t m2 = (rows_bound + bm - 1) / bm + E;
    if (m2 < m) m = m2;
    const int64_t g = m * tiles_n;
    return ((g + 7) / 8) * 8;
}


}  // namespace

// bf16 tile shapes: W = wide (192 or 256 output columns), N = 128 columns,
// G = gated (128 columns of each weight); the suffix is BM.  64-wide K
// stages, one block per CU and 112-160 KB rings (one or two stages ahead of
// the MFMAs), except the narrow 128-row shape, which runs two blocks per CU
// on 32-wide K stages.  The 256- and 320-row tiles spread each stage's DMA
// over the MFMAs of the first two k steps (measured faster there; neutral to
// slower on the 128-row ones).  The wide 320- and 192-row tiles (one tile per
// expert, weights streamed once) and the 256-row wide and gated tiles use the
// split ring, which keeps the weights two K tiles ahead: 3 % off both
// many-expert GEMMs for the 192-row one, where the two-stage ring left the
// weight stream waiting on HBM latency; on the Mixtral-shaped layer 1 % off
// the first GEMM and 2 % off the second (alternating runs on one device; the
// ring then fills all 160 KB of LDS, and the kernel's small arrays move into
// its last weight stage); the wide 128-row tile measured 6 % slower with it
// and keeps three uniform stages.
using TileW320 = Tile<320, 192, 2, 64, 1, 2, 3>;
using TileN320 = Tile<320, 128, 2, 64, 1, 2>;
using TileW256 = Tile<256, 256, 2, 64, 1, 2, 3, 2>;
using TileN256 = Tile<256, 128, 3, 64, 1, 2>;
using TileG256 = Tile<256, 128, 2, 64, 1, 2, 3, 2>;
using TileW192 = Tile<192, 256, 2, 64, 1, 2, 3, 2>;
using TileN192 = Tile<192, 128, 3, 64, 1, 0>;
using TileW128 = Tile<128, 256, 3, 64, 1, 0>;
using TileN128 = Tile<128, 128, 4, 32, 2, 0>;
using TileG128 = Tile<128, 128, 3, 64, 1, 0>;

// Launch tile shape TL with activation ACT (0 none, 1 ReLU, 2 SwiGLU).
template <class TL, int ACT, bool BIAS>
hipError_t launch_bf16_tile(const GemmArgs &g) {
    const int tiles_n = (g.N + TL::BN - 1) / TL::BN;
    // tile-map launches: up to ncu more blocks for the parts of a split last wave
    const int64_t extra = (!g.expert && g.fz.part != nullptr && g.fz.kcount == nullptr) ? g.fz.ncu : 0;
    const dim3 grid((unsigned)(g.expert ? (((int64_t)g.E * tiles_n + 7) / 8) * 8
                                        : grid_for(g.C, g.E, TL::BM, tiles_n, g.rows_bound) + extra));
#define MOE_GEMM_L(KT, EXP, NT)                                                                   \
    hipLaunchKernelGGL((gemm_bf16_kernel<TL, ACT, BIAS, KT, EXP, NT>), grid, dim3(256), 0, g.s, g.a, \
                       g.b, g.b3, g.bias, g.count, g.tile_map, g.E, g.C, g.N, g.K, tiles_n, g.out, g.fz)
    const bool kt = g.K % 64 != 0;
    if (!g.expert) {
        if (!kt) MOE_GEMM_L(false, false, false);
        else MOE_GEMM_L(true, false, false);
    } else if (g.wnt) {
        if (!kt) MOE_GEMM_L(false, true, true);
        else MOE_GEMM_L(true, true, true);
    } else {
        if (!kt) MOE_GEMM_L(false, true, false);
        else MOE_GEMM_L(true, true, false);
    }
#undef MOE_GEMM_L
    return hipGetLastError();
}
// no activation or ReLU, with or without bias
template <class TL>
hipError_t launch_bf16_act(const GemmArgs &g) {
    if (g.act == 1) return g.bias ? launch_bf16_tile<TL, 1, true>(g) : launch_bf16_tile<TL, 1, false>(g);
    return g.bias ? launch_bf16_tile<TL, 0, true>(g) : launch_bf16_tile<TL, 0, false>(g);
}

// the shapes, one group per translation unit (wide: the 192- or 256-column form)
hipError_t gemm_bf16_320(const GemmArgs &g, bool wide);
hipError_t gemm_bf16_256w(const GemmArgs &g);
hipError_t gemm_bf16_256n(const GemmArgs &g);
hipError_t gemm_bf16_192(const GemmArgs &g, bool wide);
hipError_t gemm_bf16_128w(const GemmArgs &g);
hipError_t gemm_bf16_128n(const GemmArgs &g);
hipError_t gemm_bf16_gated(const GemmArgs &g, int bm);

}  // namespace moe
