// The tile kernel of the fused MatMul -> slice-reduce -> epilogue block (gfx950).
//
// The block (CoCoNet record LIT-735, "Key takeaways": the model-parallel MatMul whose
// partial products an AllReduce sums, overlapped in chunks, with pointwise work fused
// into the collective) folded onto one GPU: P K-slices stand in for P ranks, and a
// fixed-order fp32 sum of the slice partials stands in for the AllReduce.
//
// A workgroup owns a 256 x 128 output tile, computed with v_mfma_f32_32x32x16_bf16 in
// 32 x 32 blocks.  With 64-deep K steps it has 8 waves, two per SIMD: wave w owns rows
// [64 (w % 4), +64) and columns [64 (w / 4), +64), as 2 x 2 blocks; the two waves of a
// SIMD take turns issuing, so one wave's operand reads, copies and waits run while the
// other's MFMAs execute.  The partials mode, and 32-deep K steps (slices that are not a
// multiple of 64), use 4 waves, one per SIMD, each owning 64 rows and all 128 columns as
// 2 x 4 blocks.  The MFMA computes the transposed block (W^T in the A slot,
// X in the B slot), so that a lane's accumulator holds one output row and, per group of
// four registers, four consecutive columns: exactly one Philox group, one 8-byte bias /
// residual load and one 16-byte fp32 store, with no cross-lane exchange.
//   * Staging: global_load_lds_dwordx4 copies (HBM/L2 -> LDS, no register round trip),
//     issued in pairs that share one M0 setting, into a ring of X stages [256][BK] and a
//     ring of W stages [BK][128] (W^T [128][BK] when W is given transposed), LEAD K steps
//     ahead; 16-byte chunks are XOR-swizzled
//     so the copies and the operand reads are bank-conflict free.  W [K, N] operands are
//     read with the LDS transpose read ds_read_b64_tr_b16, everything else with 16-byte
//     reads.
//   * Pipelining: the copies of step t+LEAD are spread between the MFMAs of step t; one
//     handshake per K step (this wave's copies done, then a workgroup barrier) placed
//     before the last k step, so the first operand fragments of step t+1 are read under
//     the last MFMAs of step t.  All waits are explicit vector-memory waits: no compiler
//     fence drains the copies in flight.
//   * Slice semantics: S starts every slice from zero (the first MFMA of a slice takes a
//     zero accumulator input); after the slice T = T + S (fp32, round to nearest even; T
//     starts at +0, and 0 + S_0 = S_0), so the partials are reduced in the fixed order
//     p = 0..P-1 without leaving registers.
//   * Modes: kModeFused applies bias + Philox dropout + residual to T and stores fp32
//     out; kModeReduced stores T; kModePartials computes one slice per work item and
//     stores S_p to a workspace; kModeLinear (the column-parallel producer MatMul before
//     the block) applies bias and GeLU or no activation and stores bf16.  All share the
//     same MFMA sequence,
//     so partials reduced by the reduce+epilogue kernel give the same bits as the fused
//     mode.
//   * Work items are visited chunk by chunk, tiles inside a chunk in groups of 4 tile
//     rows; a persistent grid walks the items with a stride of the grid size, and
//     workgroup ids are remapped so the 32 workgroups resident on one XCD (ids are
//     dealt round-robin over the 8 XCDs) take 32 consecutive items and share their
//     X rows and W columns in that XCD's L2.
//   * Epilogue: on a full fp32-output tile the residual comes in through the X ring
//     during the tile's last two K steps (their X copies would only repeat the last
//     step's operands); the epilogue adds the bias, reads the residual from LDS into
//     registers and, once every wave has, issues the next tile's first two K steps of
//     copies, which land under its Philox arithmetic and stores.  Otherwise every bias
//     and residual load of the tile is issued before the first Philox block is computed,
//     so the load latency is paid once per tile.
//
// No fused multiply-add anywhere in the epilogue (built with -ffp-contract=off and
// written with explicit round-to-nearest add / multiply).
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "mmar_internal.h"

namespace mmar {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ tile kernel
#define MMAR_LDS __attribute__((address_space(3)))
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Waves per workgroup: 8 (two per SIMD) for the modes that keep a tile's result in
// registers over all its K steps (the fused block 5-6 % faster, the producer MatMul 2-4 %
// faster than with 4 waves); 4 (one per SIMD) for the partials mode, whose work items are
// one slice long (12 % slower with 8 waves), and at BK = 32, where a W stage has too few
// 16-byte chunks for 8 waves to copy them in pairs.  The 256 x 192 tile has 4 waves, one
// per SIMD, each holding a 128 x 96 block: its slice sum and running total take 384 of
// the 512 registers a lone wave has.  The 128 x 128 tail tile follows the 256 x 128 rule
// (8 waves of 64 x 32 at BK = 64, 4 of 64 x 64 at BK = 32).
constexpr int tile_waves(int mode, int bk, int tile) {
    return tile == kTile192 ? 4
           : mode == kModeLinearWide ? 8
           : bk != 64 || mode == kModePartials ? 4 : 8;
}
// K step of a mode's kernel: the wide producer tile and the 256 x 192 tile always step by
// 32 (two 64-deep stages of either would not fit the LDS with copies two steps ahead).
constexpr int tile_bk(int mode, int bk, int tile) {
    return (mode == kModeLinearWide || tile == kTile192) ? 32 : bk;
}
constexpr bool is_linear(int mode) { return mode == kModeLinear || mode == kModeLinearWide; }

template <int BK, int NW_, int BN_, int WM_, int LEAD_, int XSTAGES_, int WSTAGES_,
          int TLDS_ = 0, int BM_ = kBM>
struct TileCfgT {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int NW = NW_;
    static constexpr int THREADS = 64 * NW;
    static constexpr int WM = WM_;                      // waves along m
    static constexpr int WN = NW / WM;                  // waves along n
    static constexpr int RW = BM / WM, CW = BN / WN;    // rows / columns of a wave
    static constexpr int MB = RW / 32, NB = CW / 32;    // 32 x 32 MFMA blocks of a wave
    static constexpr int KS = BK / 16;                  // MFMA k steps per K step
    static constexpr int LEAD = LEAD_;                  // copies run LEAD K steps ahead
    static constexpr int XSTAGES = XSTAGES_;            // X ring depth
    static constexpr int WSTAGES = WSTAGES_;            // W ring depth
    static constexpr int XS = BM * BK;                  // elements of an X stage [BM][BK]
    static constexpr int WS = BK * BN;                  // elements of a W stage [BK][BN]
    static constexpr int CPR = BK / 8;                  // 16-byte chunks per X row
    static constexpr int XQ = XS / 8 / 64 / NW;         // X copy instructions per wave
    static constexpr int WQ = WS / 8 / 64 / NW;         // W copy instructions per wave
    static constexpr int DMA = XQ + WQ;                 // copy instructions per wave per step
    // copy operations per wave per step: X copies in pairs, W copies in pairs and, when
    // their count is odd, one single copy
    static constexpr int XOPS = XQ / 2, WOPS = (WQ + 1) / 2, OPS = XOPS + WOPS;
    // running-total blocks of a wave kept in LDS (after the rings), 32 x 32 fp32 each
    static constexpr int TLDS = TLDS_;
    static constexpr int RING_BYTES = (XSTAGES * XS + WSTAGES * WS) * 2;
    static constexpr int LDS_BYTES = RING_BYTES + NW * TLDS * 4096;
    static_assert(LDS_BYTES <= 163840, "LDS budget");
    static_assert(MB * NB * NW * 1024 == BM * BN, "the waves' 32 x 32 blocks cover the tile");
    static_assert(XQ % 2 == 0, "X copies go in pairs");
    static_assert(XQ * NW * 64 * 8 == XS && WQ * NW * 64 * 8 == WS, "copies cover a stage");
    static_assert(XSTAGES >= LEAD + 1 && WSTAGES >= LEAD + 1, "ring depth");
};

// The configuration of a (mode, K step, tile shape).  The 256 x 128 and wide shapes keep
// one W stage more than X (their copies never reuse the stage of the step just read).
// The 256 x 192 tile uses LEAD + 1 = 4 stages of each (the step handshake waits for this
// wave's LDS reads, so the stage read last is free once every wave has passed it), the
// copies 3 steps (about 2000 cycles) ahead, and keeps 3 of each wave's 12 running-total
// blocks in the remaining 48 KB of LDS: with all 12 in registers the slice sum (192
// accumulation registers), the running total (192) and the operand fragments do not fit
// the 512 registers of a wave.
template <int MODE, int BK, int TILE>
struct TileCfgOf {
    static constexpr int NW = tile_waves(MODE, BK, TILE);
    static constexpr int BN = tile_bn(MODE, TILE);
    static constexpr int LEAD = TILE == kTile192 ? 3 : BK == 64 ? 2 : BN == 256 ? 3 : 5;
    using type = TileCfgT<BK, NW, BN, TILE == kTile128 ? 4 : 2, LEAD, LEAD + 1,
                          TILE == kTile192 ? LEAD + 1 : LEAD + 2, TILE == kTile192 ? 3 : 0,
                          tile_bm(TILE)>;
};

// 16-byte chunk swizzles (bank-conflict-free MFMA operand reads).  X stage rows are BK
// elements; W stage rows are BN elements.  The LDS transpose read of W takes, per
// half-wave, 64 bytes from each of 4 consecutive k rows: with 256- or 512-byte rows the
// four start on the same bank, so 64-byte groups are rotated by k mod 4; with 384-byte
// rows (BN = 192) rows k and k + 1 already sit half a bank cycle apart, so only k / 2
// mod 2 flips the 64-byte group (an XOR inside aligned 8-chunk groups: 24 chunks per
// row stay in range).
template <int BK>
__device__ __forceinline__ int swz_x(int m) {
    return BK == 64 ? ((m & 7) ^ ((m >> 3) & 1)) : ((m >> 2) & 3);
}
template <int BN>
__device__ __forceinline__ int swz_w(int k) {
    return BN == 192 ? 4 * ((k >> 1) & 1) : 4 * (k & 3);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding).
#define MMAR_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | 0x70 | 0xF00 | ((((n) >> 4) & 3) << 14))
// The same, and every LDS read of this wave complete (lgkmcnt 0).
#define MMAR_WAIT_VM_LDS(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | 0x70 | ((((n) >> 4) & 3) << 14))

// Two 16-byte global -> LDS copies per lane with one M0 setting (sbase wave-uniform in
// SGPRs, voff0 / voff1 per-lane byte offsets, lds_addr1 wave-uniform): copy 0 reads
// sbase + voff0 - 1024 and lands at lds_addr1 - 1024 + 16 lane, copy 1 reads
// sbase + voff1 and lands at lds_addr1 + 16 lane.  The instruction offset applies to both
// addresses, so voff0 holds its byte offset plus 1024 (no wrap: an offset within a tile
// of X, W or W^T, each under 2^31 elements, stays far below 2^32 - 1024).  M0 is
// declared clobbered (the compiler keeps nothing of its own in it across the asm).  Inline
// asm, so that the compiler does not turn the LDS writes into a wait on every later LDS
// read; the kernel waits on the vector-memory counter itself.  One M0 setting per pair
// instead of per copy saved about an eighth of the instructions a wave issues per K step.
__device__ __forceinline__ void dma16x2(const void* sbase, uint32_t voff0, uint32_t voff1,
                                        uint32_t lds_addr1) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %2 offset:-1024\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "v"(voff0), "v"(voff1), "s"(sbase), "s"(lds_addr1)
        : "memory", "m0");
}

// One 16-byte global -> LDS copy per lane: reads sbase + voff, lands at lds_addr + 16 lane
// (lds_addr wave-uniform).  M0 is declared clobbered.
__device__ __forceinline__ void dma16x1(const void* sbase, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds_addr)
        : "memory", "m0");
}

// Byte bias a copy's per-lane source offset carries against its instruction offset: +1 KB
// for the first copy of a pair.
template <int TILE, int NQ>
__device__ __forceinline__ uint32_t copy_bias(int q) {
    return (q % 2 == 0 && q + 1 < NQ) ? 1024u : 0u;
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const MMAR_LDS void*)p));
}

// Workgroup barrier without the memory fence of __syncthreads (which would also wait
// for the copies in flight); "memory" keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Calls f(integral_constant<int, I>) for I = B .. E-1 in order (compile-time indices for
// register arrays).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// WT = false: W is [K, N] (n contiguous) and its MFMA operand is read with the LDS
// transpose read; WT = true: W is given transposed, [N, K] (k contiguous, the layout of
// a Linear layer's weight), and both operands use plain 16-byte LDS reads.
template <int MODE, int BK, bool WT, int TILE>
__global__ __launch_bounds__(64 * tile_waves(MODE, BK, TILE))
__attribute__((amdgpu_waves_per_eu(tile_waves(MODE, BK, TILE) / 4,
                                   tile_waves(MODE, BK, TILE) / 4)))
void tile_kernel(TileArgs a) {
    using C = typename TileCfgOf<MODE, BK, TILE>::type;
    // one slice and no running total: the wide producer tile stores S itself
    constexpr bool NO_T = MODE == kModeLinearWide || MODE == kModePartials;
    constexpr int BM = C::BM, BN = C::BN, NB = C::NB, MB = C::MB, KS = C::KS;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* const xs_base = smem;                       // [XSTAGES][BM][BK], swizzled
    uint16_t* const ws_base = smem + C::XSTAGES * C::XS;  // [WSTAGES][BK][BN] or [BN][BK]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int wm = wave % C::WM, wn = wave / C::WM;      // this wave's block of the tile
    const int uwave = __builtin_amdgcn_readfirstlane(wave);

    // XCD-aware slot: ids are dealt round-robin over the 8 XCDs; give each XCD a
    // contiguous run of items per sweep.
    const int G = gridDim.x, bid = blockIdx.x;
    const int slot = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;

    const int tpcm = (a.cm + BM - 1) / BM, tpcn = (a.cn + BN - 1) / BN, tpc = tpcm * tpcn;
    const int chunks_n = a.RN / a.cn;
    const int n_tiles = (a.RM / a.cm) * chunks_n * tpc;
    const int sps = a.Ks / BK;   // K steps per slice

    // Operand reads.  X (B slot): rows C::RW wm + 32 mb + l32, 16-byte chunk 2 s + h.
    // W (A slot) through the LDS transpose read: in each 16-lane group i = lane % 16,
    // lane i points at row k = kb + i / 4 and columns 4 (i % 4) .. +3 of a 16-column
    // half; the read returns to lane j column j and rows kb .. kb + 3.
    int xrd[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) xrd[mb] = (C::RW * wm + 32 * mb + l32) * BK;
    const int gi = lane & 15, grp = lane >> 4;
    const int wk = 8 * (grp >> 1) + (gi >> 2);            // row within a 16-row k step
    const int wcn = C::CW * wn + 16 * (grp & 1) + 4 * (gi & 3);   // column (block 0)

    // Work item -> tile origin and extent (and slice range in the partials mode)
    struct ItemTile { int m0, n0, rows, cols, p_lo, p_hi; };
    auto tile_of = [&](int item) {
        int tile_item = item, p_lo = 0, p_hi = a.P;
        if (MODE == kModePartials) {
            tile_item = item % n_tiles;
            p_lo = item / n_tiles;
            p_hi = p_lo + 1;
        }
        const int chunk = tile_item / tpc, t = tile_item - chunk * tpc;
        const int cr = chunk / chunks_n, cc = chunk - cr * chunks_n;
        constexpr int GM = 4;
        const int first_tm = (t / (GM * tpcn)) * GM;
        const int gm = min(GM, tpcm - first_tm);
        const int tin = t - (t / (GM * tpcn)) * (GM * tpcn);
        const int tm = first_tm + tin % gm, tn = tin / gm;
        return ItemTile{a.rm0 + cr * a.cm + tm * BM, a.rn0 + cc * a.cn + tn * BN,
                        min(BM, a.cm - tm * BM), min(BN, a.cn - tn * BN), p_lo, p_hi};
    };
    // Copy sources: a wave-uniform base (SGPRs) per K step plus per-lane byte offsets.
    // Copy q of wave w fills 16-byte chunks 64 (Q w + q) + lane of the stage; X rows are
    // clamped to the tile, W columns to the tile.
    auto copy_offsets = [&](int rows, int cols, uint32_t (&xoff)[C::XQ], uint32_t (&woff)[C::WQ]) {
#pragma unroll
        for (int q = 0; q < C::XQ; ++q) {
            const int idx = 64 * (C::XQ * wave + q) + lane;
            const int r = idx / C::CPR, pos = idx % C::CPR;
            const int c = pos ^ swz_x<BK>(r);
            xoff[q] = static_cast<uint32_t>((static_cast<int64_t>(min(r, rows - 1)) * a.ldx + 8 * c) * 2 +
                                            copy_bias<TILE, C::XQ>(q));
        }
#pragma unroll
        for (int q = 0; q < C::WQ; ++q) {
            const int idx = 64 * (C::WQ * wave + q) + lane;
            if constexpr (WT) {   // W^T rows n, swizzled like X
                const int r = idx / C::CPR, pos = idx % C::CPR;
                const int c = pos ^ swz_x<BK>(r);
                woff[q] = static_cast<uint32_t>(
                    (static_cast<int64_t>(min(r, cols - 1)) * a.ldw + 8 * c) * 2 +
                    copy_bias<TILE, C::WQ>(q));
            } else {
                const int k = idx / (BN / 8), pos = idx % (BN / 8);
                const int c = pos ^ swz_w<BN>(k);
                woff[q] = static_cast<uint32_t>(
                    (static_cast<int64_t>(k) * a.ldw + min(8 * c, cols - 8)) * 2 +
                    copy_bias<TILE, C::WQ>(q));
            }
        }
    };
    auto x_base = [&](const ItemTile& it) {
        return static_cast<const uint16_t*>(
            uniform_ptr(a.X + static_cast<int64_t>(it.m0) * a.ldx + static_cast<int64_t>(it.p_lo) * a.Ks));
    };
    auto w_base = [&](const ItemTile& it) {
        const int64_t kf = static_cast<int64_t>(it.p_lo) * a.Ks;
        return static_cast<const uint16_t*>(uniform_ptr(
            WT ? a.W + static_cast<int64_t>(it.n0) * a.ldw + kf : a.W + kf * a.ldw + it.n0));
    };
    // bytes per K step; a step's byte offset st * step fits 32 bits (the extents of X
    // and W, rows times leading dimension, are below 2^31 elements)
    const uint32_t xstep_b = BK * 2;
    const uint32_t wstep_b = WT ? BK * 2 : static_cast<uint32_t>(BK * a.ldw * 2);
    auto step_ptr = [](const uint16_t* base, int st, uint32_t step_b) {
        return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(base) +
                                                 static_cast<uint32_t>(st) * step_b);
    };
    // copy operation j of step st from the bases and offsets of one item, into X stage xsi
    // and W stage wsi: X copies 2j, 2j+1 (j < XOPS), else W copies q, q+1
    // (q = 2 (j - XOPS)), or W copy q alone when it is the last of an odd count
    auto copy_op_of = [&](const uint16_t* xb, const uint16_t* wb, const uint32_t (&xo)[C::XQ],
                          const uint32_t (&wo)[C::WQ], int st, unsigned xsi, unsigned wsi, int j) {
        if (j < C::XOPS) {
            const int i = 2 * j;
            const uint32_t xd = lds_addr(xs_base + xsi * C::XS + (C::XQ * uwave + i + 1) * 512);
            dma16x2(step_ptr(xb, st, xstep_b), xo[i], xo[i + 1], xd);
        } else {
            const int q = 2 * (j - C::XOPS);
            if (q + 1 < C::WQ) {
                const uint32_t wd = lds_addr(ws_base + wsi * C::WS + (C::WQ * uwave + q + 1) * 512);
                dma16x2(step_ptr(wb, st, wstep_b), wo[q], wo[q + 1], wd);
            } else {
                const uint32_t wd = lds_addr(ws_base + wsi * C::WS + (C::WQ * uwave + q) * 512);
                dma16x1(step_ptr(wb, st, wstep_b), wo[q], wd);
            }
        }
    };
    // The next item's first LEAD K steps of copies may have been issued at the end of
    // this one (a fused tile whose residual came through LDS: after its last LDS reads,
    // before its Philox arithmetic and its 16 output stores per lane), so that they land
    // under that epilogue; its first handshake then lets those stores stay in flight.
    constexpr int kTileStores = 4 * NB * MB;   // 16-byte stores per lane of a full tile
    bool prefetched = false;

    for (int item = slot; item < a.total_items; item += G) {
        const ItemTile itile = tile_of(item);
        const int m0 = itile.m0, n0 = itile.n0, rows = itile.rows, cols = itile.cols;
        const int p_lo = itile.p_lo, p_hi = itile.p_hi;
        uint32_t xoff[C::XQ], woff[C::WQ];
        copy_offsets(rows, cols, xoff, woff);
        const int nsteps = (p_hi - p_lo) * sps;

        // The fused epilogue's residual tile through the X ring.  On a full tile whose
        // residual rows are 16-byte aligned, the last two K steps (whose copies would only
        // repeat the last step's operands) copy residual rows 0-127 and 128-255 into the
        // X stages they free, 16 chunks of 16 bytes per row, chunk c of row r at slot
        // c ^ (r mod 16) (so the epilogue's reads of 32 rows spread over the banks); the
        // epilogue then reads the residual from LDS instead of waiting for HBM at the end
        // of every round.
        constexpr bool RES_OK = MODE == kModeFused && TILE == kTile128 && C::LEAD == 2 &&
                                C::XQ == 4 && C::NW == 8 && BN == 128;
        bool use_res = false;
        uint32_t roff[RES_OK ? C::XQ : 1];
        if constexpr (RES_OK) {
            use_res = rows == BM && cols == BN && sps >= 3 && a.hout == nullptr &&
                      (reinterpret_cast<uintptr_t>(a.residual) % 16) == 0 && (a.ldr % 8) == 0;
#pragma unroll
            for (int q = 0; q < C::XQ; ++q) {   // slot 64 (XQ w + q) + lane of a 128-row half
                const int idx = 64 * (C::XQ * wave + q) + lane;
                const int r = idx >> 4, c = (idx & 15) ^ (r & 15);
                roff[q] = static_cast<uint32_t>(r * static_cast<uint32_t>(a.ldr) * 2u + 16u * c) +
                          copy_bias<TILE, C::XQ>(q);
            }
        }
        const uint16_t* xbase = x_base(itile);
        const uint16_t* wbase = w_base(itile);
        // stage of K step st (st >= 0: unsigned arithmetic keeps the modulo short)
        auto xstage = [](int st) { return static_cast<unsigned>(st) % C::XSTAGES; };
        auto wstage = [](int st) { return static_cast<unsigned>(st) % C::WSTAGES; };

        // residual copy pair j (j < XOPS) issued during K step cur, one of the last two
        // (cur = nsteps - 2 + half): residual rows 128 half .. +127 into the X stage of step
        // cur + LEAD, which the repeat of the last step's X operands would have filled
        // (xsi: that stage, (cur + LEAD) mod XSTAGES)
        auto res_copy_op = [&](int j, int cur, unsigned xsi) {
            const int i = 2 * j, half = cur + C::LEAD - nsteps;
            const uint32_t xd = lds_addr(xs_base + xsi * C::XS + (C::XQ * uwave + i + 1) * 512);
            dma16x2(uniform_ptr(a.residual + (static_cast<int64_t>(m0) + 128 * half) * a.ldr + n0),
                    roff[i], roff[i + 1], xd);
        };
        // copy operation j of step st of this item into X stage xsi and W stage wsi
        auto copy_op = [&](int st, unsigned xsi, unsigned wsi, int j) {
            copy_op_of(xbase, wbase, xoff, woff, st, xsi, wsi, j);
        };

        // S: this slice's sums; T: the running total (the 256 x 192 tile defines T at the
        // end of the first slice, T = 0 + S_0, so it is not cleared here)
        f32x16 S[NB][MB], T[NB][MB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                S[nb][mb] = f32x16{};
                if constexpr (TILE != kTile192) T[nb][mb] = f32x16{};
            }

        const int last = nsteps - 1;
        // operand fragment of row block mb (X) / column block nb (W) for MFMA k step s,
        // from X stage xsi / W stage wsi
        auto read_x = [&](unsigned xsi, int s, int mb) -> bf16x8 {
            const uint16_t* xs = xs_base + xsi * C::XS;
            const int m = C::RW * wm + 32 * mb + l32;
            return *reinterpret_cast<const bf16x8*>(xs + xrd[mb] + 8 * ((2 * s + h) ^ swz_x<BK>(m)));
        };
        auto read_w = [&](unsigned wsi, int s, int nb) -> bf16x8 {
            const uint16_t* wsb = ws_base + wsi * C::WS;
            if constexpr (WT) {
                const int n = C::CW * wn + 32 * nb + l32;
                return *reinterpret_cast<const bf16x8*>(wsb + n * BK +
                                                        8 * ((2 * s + h) ^ swz_x<BK>(n)));
            } else {
                const int k1 = 16 * s + wk, k2 = k1 + 4;
                const int n = wcn + 32 * nb;
                const uint16_t* p1 = wsb + k1 * BN + 8 * ((n >> 3) ^ swz_w<BN>(k1)) + (n & 7);
                const uint16_t* p2 = wsb + k2 * BN + 8 * ((n >> 3) ^ swz_w<BN>(k2)) + (n & 7);
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MMAR_LDS v4i16*)p1);
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MMAR_LDS v4i16*)p2);
                const v4i16 both[2] = {lo, hi};
                return __builtin_bit_cast(bf16x8, both);
            }
        };
        auto frags = [&](unsigned xsi, unsigned wsi, int s, bf16x8 (&xf)[MB], bf16x8 (&wf)[NB]) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) xf[mb] = read_x(xsi, s, mb);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) wf[nb] = read_w(wsi, s, nb);
        };
        // Step-boundary handshake for K step t: this wave's copies of t are done (only the
        // copies of the LEAD - 1 following steps may remain) and the barrier makes every
        // wave's copies of t visible.  Each wave also waits for its own LDS reads (the
        // operands of step t-1's last k step, read just before), so the barrier shows that
        // every wave has finished reading step t-1, whose X stage the copies issued next
        // (for step t + LEAD) overwrite, and step t-2, whose W stage they overwrite.
        auto handshake = [&]() {
            MMAR_WAIT_VM_LDS((C::LEAD - 1) * C::DMA);
            wg_barrier();
        };

        if (!prefetched) {
#pragma unroll
            for (int d = 0; d < C::LEAD; ++d)
#pragma unroll
                for (int j = 0; j < C::OPS; ++j) copy_op(min(d, last), d, d, j);
            handshake();
            // the 256 x 192 tile issues each step's X copies in the k step before its W
            // copies (right after the handshake that frees their stage), so step LEAD's X
            // copies go out here and its W copies in the first K step
            if constexpr (TILE == kTile192) {
#pragma unroll
                for (int j = 0; j < C::XOPS; ++j)
                    copy_op(min(C::LEAD, last), xstage(min(C::LEAD, last)), 0, j);
            }
        } else {
            // the copies of step 0 are done once all but the LEAD - 1 later steps' copies
            // and the previous tile's stores are
            MMAR_WAIT_VM_LDS((C::LEAD - 1) * C::DMA + kTileStores);
            wg_barrier();
        }
        prefetched = false;
        // the next item's first LEAD K steps of copies, issued while this item's epilogue
        // still has its output stores to issue (stages 0 .. LEAD - 1 of both rings)
        auto prefetch_next = [&]() {
            const int nxt = item + G;
            if (nxt >= a.total_items) return;
            const ItemTile nt = tile_of(nxt);
            uint32_t nxo[C::XQ], nwo[C::WQ];
            copy_offsets(nt.rows, nt.cols, nxo, nwo);
            const uint16_t* nxb = x_base(nt);
            const uint16_t* nwb = w_base(nt);
            const int nlast = (nt.p_hi - nt.p_lo) * sps - 1;
#pragma unroll
            for (int d = 0; d < C::LEAD; ++d)
#pragma unroll
                for (int j = 0; j < C::OPS; ++j) copy_op_of(nxb, nwb, nxo, nwo, min(d, nlast), d, d, j);
            prefetched = true;
        };

        // running-total blocks (nb = NB - 1, mb < TLDS) kept in this wave's LDS area (the
        // 256 x 192 tile): value 4q + j of lane l at float offset 256 (4 blk + q) + 4 l + j
        float* const tl = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) +
                                                   C::RING_BYTES) +
                          uwave * C::TLDS * 1024;
        auto in_lds = [](int nb, int mb) { return nb == NB - 1 && mb < C::TLDS; };

        int st = 0;
        if constexpr (TILE == kTile192) {
            // 256 x 192 tile, 4 waves of 128 x 96, K steps of 32 (two MFMA k steps).
            // MFMAs go row block by row block (mb outer); an X fragment is re-read for the
            // next k step as soon as the three MFMAs of its row block are issued, the W
            // fragments of the next k step are read into the other half of a double buffer
            // at the start of a k step.  The W copies of step st + LEAD go between the MFMAs
            // of the first k step, the handshake before the second, and the X copies of
            // step st + LEAD + 1 between the MFMAs of the second.
            static_assert(KS == 2, "the 256 x 192 tile steps K by 32");
            static_assert(C::XQ == 4 && C::WQ == 3, "copy groups of the 256 x 192 tile");
            // Fragments double-buffered: buffer 0 holds k step 0 of a K step, buffer 1 k
            // step 1; each k step starts by reading the other buffer's fragments, so the
            // reads of a stage are all issued a whole k step before the handshake waits
            // for them.
            bf16x8 xf0[MB], wf0[NB], xf1[MB], wf1[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) xf0[mb] = read_x(0, 0, mb);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) wf0[nb] = read_w(0, 0, nb);
            // One K step as two k steps of 12 MFMA slots each (mb outer, nb inner).  A single
            // wave per SIMD issues in order, so each slot holds one MFMA and at most a few
            // other instructions, which then issue while the MFMA runs: in k step 0 the
            // fragment reads for k step 1 (W first, then X in MFMA order), the W copies of
            // step st + LEAD and the handshake in the last slot (by then the reads it waits
            // for have long returned); in k step 1 the reads of the next K step's first
            // fragments and the X copies of step st + LEAD + 1.  So the copies that fill a
            // stage go out between the handshake that frees it and the next one, in four
            // groups five slots apart: bunched into four consecutive slots, the four waves'
            // copies of a step made the GPT-2 MLP block 3-4 % slower.  The handshake of step
            // st still finds exactly the copies of the two newest such windows in flight.
            auto kstep192 = [&](auto zero_tag) {
                constexpr bool ZERO = decltype(zero_tag)::value;
                const int st2 = min(st + C::LEAD, last);
                const int st3 = min(st + C::LEAD + 1, last);
                const int nx = min(st + 1, last);
                constexpr int K0A = 2, K0B = 7, K1A = 2, K1B = 7;
                // copy sources and LDS destinations: W of step st2 (computed in slot K0A - 1,
                // a pair in slot K0A and a single copy in K0B of k step 0), X of step st3
                // (slot K1A - 1, pairs in slots K1A and K1B of k step 1); past an item's last
                // step they repeat its operands
                const uint16_t* xsrc = nullptr;
                const uint16_t* wsrc = nullptr;
                uint32_t xdst = 0, wdst = 0;
                static_for<0, MB * NB>([&](auto ic) {
                    constexpr int i = decltype(ic)::value, mb = i / NB, nb = i % NB;
                    S[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        wf0[nb], xf0[mb], ZERO ? f32x16{} : S[nb][mb], 0, 0, 0);
                    if constexpr (i < NB) wf1[i] = read_w(wstage(st), 1, i);
                    else if constexpr (i < NB + MB) xf1[i - NB] = read_x(xstage(st), 1, i - NB);
                    if constexpr (i == K0A - 1) {
                        wsrc = step_ptr(wbase, st2, wstep_b);
                        wdst = lds_addr(ws_base + wstage(st2) * C::WS + C::WQ * uwave * 512);
                    } else if constexpr (i == K0A) {
                        dma16x2(wsrc, woff[0], woff[1], wdst + 1024);
                    } else if constexpr (i == K0B) {
                        dma16x1(wsrc, woff[2], wdst + 2048);
                    } else if constexpr (i == MB * NB - 1) {
                        handshake();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
                static_for<0, MB * NB>([&](auto ic) {
                    constexpr int i = decltype(ic)::value, mb = i / NB, nb = i % NB;
                    S[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf1[nb], xf1[mb],
                                                                        S[nb][mb], 0, 0, 0);
                    if constexpr (i < NB) wf0[i] = read_w(wstage(nx), 0, i);
                    else if constexpr (i < NB + MB) xf0[i - NB] = read_x(xstage(nx), 0, i - NB);
                    if constexpr (i == K1A - 1) {
                        xsrc = step_ptr(xbase, st3, xstep_b);
                        xdst = lds_addr(xs_base + xstage(st3) * C::XS + C::XQ * uwave * 512);
                    } else if constexpr (i == K1A) {
                        dma16x2(xsrc, xoff[0], xoff[1], xdst + 1024);
                    } else if constexpr (i == K1B) {
                        dma16x2(xsrc, xoff[2], xoff[3], xdst + 3072);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            };

            // T = 0 + S_0 after the first slice, then T + S_1, T + S_2, ... (fp32, nearest
            // even), in registers or in this wave's LDS area; one block at a time (the
            // barriers keep the compiler from reading every slice sum out of the
            // accumulation registers at once)
            auto update = [&](auto first_tag) {
                constexpr bool FIRST = decltype(first_tag)::value;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (in_lds(nb, mb)) {
                            float4* q = reinterpret_cast<float4*>(tl + 1024 * mb) + lane;
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                const float4 t = FIRST ? make_float4(0.f, 0.f, 0.f, 0.f) : q[64 * g];
                                q[64 * g] = make_float4(t.x + S[nb][mb][4 * g],
                                                        t.y + S[nb][mb][4 * g + 1],
                                                        t.z + S[nb][mb][4 * g + 2],
                                                        t.w + S[nb][mb][4 * g + 3]);
                            }
                        } else if (FIRST) {
                            T[nb][mb] = f32x16{} + S[nb][mb];
                        } else {
                            T[nb][mb] += S[nb][mb];
                        }
                    }
                __builtin_amdgcn_sched_barrier(0);
            };
            for (int p = p_lo; p < p_hi; ++p) {
                kstep192(std::true_type{});
                ++st;
                for (int j = 1; j < sps; ++j, ++st) kstep192(std::false_type{});
                if constexpr (!NO_T) {
                    if (p == p_lo)
                        update(std::true_type{});
                    else
                        update(std::false_type{});
                }
            }
        } else {
        // fragments are double-buffered: k step s of any K step uses buffer s % 2 (KS is
        // even), and the first fragments of step t+1 are read during the last MFMAs of t
        bf16x8 xa[MB], wa[NB], xb2[MB], wb2[NB];
        frags(0, 0, 0, xa, wa);
        // ring stages of step st, kept as running indices instead of st mod XSTAGES / mod
        // WSTAGES recomputed per use
        unsigned x3 = 0, w4 = 0;
        auto ring_next = [](unsigned i, unsigned n, unsigned by) {
            return i + by >= n ? i + by - n : i + by;
        };

        // One K step (step st): KS k steps of NB x MB MFMAs, the copies of step st+LEAD between
        // them, the step-boundary handshake before the last k step.  ZERO marks the first
        // K step of a slice: its first k step gives the MFMAs a zero accumulator input,
        // which starts the slice sums from zero without clearing any register.
        auto kstep = [&](auto zero_tag, auto res_tag) {
            constexpr bool ZERO = decltype(zero_tag)::value;
            // RES: one of the last two K steps of a tile whose residual goes through LDS;
            // its X copy slots carry residual copies (the same number of copies per step)
            constexpr bool RES = decltype(res_tag)::value;
            // copies of step st+LEAD, spread over the MFMAs of k steps 0 .. KS-2.  The last
            // LEAD steps of an item copy the last step's operands again (the same count of
            // copies every step) into the stages of steps st + LEAD, which follow the
            // item's last step: nothing reads them before the item's final drain.
            const int st2 = min(st + C::LEAD, last);
            const unsigned xc = ring_next(x3, C::XSTAGES, C::LEAD);
            const unsigned wc = ring_next(w4, C::WSTAGES, C::LEAD);
            // the NB x MB MFMAs of one k step, with copy operations c0 .. c1-1 issued between
            // them (all of them: the caller passes c1 - c0 <= OPS)
            auto mfmas = [&](const bf16x8 (&xf)[MB], const bf16x8 (&wf)[NB], int c0, int c1,
                             bool zero) {
                int c = c0;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        S[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            wf[nb], xf[mb], zero ? f32x16{} : S[nb][mb], 0, 0, 0);
                        // spread the copies evenly over the NB x MB MFMAs
                        const int upto =
                            c0 + ((nb * MB + mb + 1) * (c1 - c0) + NB * MB - 1) / (NB * MB);
                        while (c < upto) {
                            __builtin_amdgcn_sched_barrier(0);
                            if constexpr (RES) {
                                if (c < C::XOPS)
                                    res_copy_op(c, st, xc);
                                else
                                    copy_op(st2, xc, wc, c);
                            } else {
                                copy_op(st2, xc, wc, c);
                            }
                            c += 1;
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
            };
            constexpr int CPS = (C::OPS + KS - 2) / (KS - 1);   // copy operations per k step
#pragma unroll
            for (int s = 0; s < KS; s += 2) {
                // k step s (buffer a), prefetching s+1 into buffer b
                frags(x3, w4, s + 1, xb2, wb2);
                mfmas(xa, wa, min(s * CPS, C::OPS), min((s + 1) * CPS, C::OPS), ZERO && s == 0);
                // k step s+1 (buffer b), prefetching s+2, or the next K step's first (after
                // an item's last step: fragments of a stage being refilled, never used)
                if (s + 2 < KS) {
                    frags(x3, w4, s + 2, xa, wa);
                    mfmas(xb2, wb2, min((s + 1) * CPS, C::OPS), min((s + 2) * CPS, C::OPS),
                          false);
                } else {
                    handshake();
                    frags(ring_next(x3, C::XSTAGES, 1), ring_next(w4, C::WSTAGES, 1), 0, xa, wa);
                    mfmas(xb2, wb2, C::OPS, C::OPS, false);
                }
            }
        };

        // the slices' K steps; with the residual through LDS the last two steps of the
        // last slice are the residual variant (peeled after one loop with a shorter bound)
        auto advance = [&]() {
            ++st;
            x3 = ring_next(x3, C::XSTAGES, 1);
            w4 = ring_next(w4, C::WSTAGES, 1);
        };
        for (int p = p_lo; p < p_hi; ++p) {
          const bool peel = RES_OK && use_res && p == p_hi - 1;
          kstep(std::true_type{}, std::false_type{});
          advance();
          const int jend = peel ? sps - 2 : sps;
          for (int j = 1; j < jend; ++j) {
              kstep(std::false_type{}, std::false_type{});
              advance();
          }
          if constexpr (RES_OK) {
              if (peel) {
                  kstep(std::false_type{}, std::true_type{});
                  advance();
                  kstep(std::false_type{}, std::true_type{});
                  advance();
              }
          }
          if constexpr (!NO_T) {
              // T = 0 + S_0 (= S_0 exactly: an MFMA sum started from +0 is never -0),
              // then T + S_1, T + S_2, ... in fp32, round to nearest even
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                  for (int mb = 0; mb < MB; ++mb) T[nb][mb] += S[nb][mb];
          }
        }
        }
        MMAR_WAIT_VM_LDS(0);
        wg_barrier();   // every wave is done with the LDS ring (its copies landed, its reads
                        // returned) before the next item's copies

        // Store / epilogue.  Lane holds rows RW wm + 32 mb + l32 and, in registers
        // 4g..4g+3 of block nb, columns CW wn + 32 nb + 8 g + 4 h + 0..3.  A ragged tile
        // holds whole 32 x 32 blocks (rows and cols are multiples of 32); blocks outside
        // it are neither loaded nor stored.  The fused mode loads every bias and residual
        // value it needs first, so the loads are in flight together (and under the Philox
        // arithmetic) instead of one load latency per output group.
        auto col_ok = [&](int nb) { return C::CW * wn + 32 * nb < cols; };
        auto row_ok = [&](int mb) { return C::RW * wm + 32 * mb < rows; };
        if constexpr (TILE == kTile192) {
            // One 32 x 32 block at a time (nb outer), the residual loads of the block PF
            // blocks ahead in flight and the bias of a column block loaded once; the
            // barriers keep the compiler from issuing every load (and holding every address)
            // of the 128 x 96 wave block at once, which would not fit beside T.  fp32
            // output only (a second, bf16 store path alone made the registers spill; the
            // bf16-output block uses the 256 x 128 tile).  Per lane: row m_lane + 32 mb,
            // columns n_lane + 32 nb + 8 g + 0..3.
            constexpr int NBLK = NB * MB, PF = 3;
            const int64_t m_lane = static_cast<int64_t>(m0) + C::RW * wm + l32;
            const int n_lane = n0 + C::CW * wn + 4 * h;
            uint2 bq[4], rq[PF][4];
            // columns 8 g .. 8 g + 3 of block (nb, mb) of T, from registers or LDS
            auto tval = [&](int nb, int mb, int g) -> float4 {
                if (in_lds(nb, mb))
                    return reinterpret_cast<const float4*>(tl + 1024 * mb)[64 * g + lane];
                const f32x16& acc = T[nb][mb];
                return make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
            };
            // column offset of block nb (clamped into the tile), relative to n_lane
            auto ncol = [&](int nb) { return min(C::CW * wn + 32 * nb, cols - 32) - C::CW * wn; };
            auto issue = [&](auto ic) {   // residual loads of block i (clamped into the tile)
                constexpr int i = decltype(ic)::value, nb = i / MB, mb = i % MB;
                const int ml = min(C::RW * wm + 32 * mb, rows - 32) - C::RW * wm;
                const uint16_t* rp = a.residual + (m_lane + ml) * a.ldr + n_lane + ncol(nb);
#pragma unroll
                for (int g = 0; g < 4; ++g) rq[i % PF][g] = *reinterpret_cast<const uint2*>(rp + 8 * g);
            };
            if constexpr (MODE == kModeFused) static_for<0, PF>(issue);
            static_for<0, NBLK>([&](auto ic) {
                constexpr int i = decltype(ic)::value, nb = i / MB, mb = i % MB;
                __builtin_amdgcn_sched_barrier(0);
                const bool ok = col_ok(nb) && row_ok(mb);
                const int64_t m = m_lane + 32 * mb;
                if constexpr (MODE == kModeFused) {
                    if constexpr (mb == 0) {
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            bq[g] = *reinterpret_cast<const uint2*>(a.bias + n_lane + ncol(nb) + 8 * g);
                    }
                    uint2 r0[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) r0[g] = rq[i % PF][g];
                    if constexpr (i + PF < NBLK) issue(std::integral_constant<int, i + PF>{});
                    if (ok) {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int64_t n = n_lane + 32 * nb + 8 * g;
                            *reinterpret_cast<float4*>(a.out + m * a.ldo + n) =
                                epilogue4(tval(nb, mb, g), bq[g], r0[g], m * a.N + n, a.drop);
                        }
                    }
                } else {   // kModeReduced: T itself
                    if (ok) {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int64_t n = n_lane + 32 * nb + 8 * g;
                            *reinterpret_cast<float4*>(a.out + m * a.ldo + n) = tval(nb, mb, g);
                        }
                    }
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (is_linear(MODE)) {
            uint2 bb[NB][4];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = min(C::CW * wn + 32 * nb, cols - 32) + 8 * g + 4 * h;
                    bb[nb][g] = *reinterpret_cast<const uint2*>(a.bias + n0 + nl);
                }
            // bf16(act(T + bias)), the sum and the activation in fp32
            auto store_all = [&](auto act) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            if (!col_ok(nb) || !row_ok(mb)) continue;
                            const int64_t m = m0 + C::RW * wm + 32 * mb + l32;
                            const int64_t n = n0 + C::CW * wn + 32 * nb + 8 * g + 4 * h;
                            // the wide tile has one slice: S, as it comes from the MFMAs
                            // (a sum started from +0, never -0), equals T = 0 + S
                            const f32x16& acc = NO_T ? S[nb][mb] : T[nb][mb];
                            const uint2 b = bb[nb][g];
                            const float g0 = act(__fadd_rn(acc[4 * g], bf16_lo(b.x)));
                            const float g1 = act(__fadd_rn(acc[4 * g + 1], bf16_hi(b.x)));
                            const float g2 = act(__fadd_rn(acc[4 * g + 2], bf16_lo(b.y)));
                            const float g3 = act(__fadd_rn(acc[4 * g + 3], bf16_hi(b.y)));
                            *reinterpret_cast<uint2*>(a.hout + m * a.ldo + n) =
                                make_uint2(bf16x2_rne(g0, g1), bf16x2_rne(g2, g3));
                        }
            };
            if (a.act == kActGeluTanh)
                store_all([](float v) { return gelu_tanh_f32(v); });
            else
                store_all([](float v) { return v; });
        } else if constexpr (MODE == kModeFused) {
            uint2 bb[NB][4];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // clamped into the tile: an outside block reads a valid address
                    const int nl = min(C::CW * wn + 32 * nb, cols - 32) + 8 * g + 4 * h;
                    bb[nb][g] = *reinterpret_cast<const uint2*>(a.bias + n0 + nl);
                }
            // the output as fp32, or rounded once more to bf16 (nearest even) when hout is
            // set; res(nb, g, mb) gives the residual of the lane's group
            auto store_all = [&](auto store, auto res) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            if (!col_ok(nb) || !row_ok(mb)) continue;
                            const int64_t m = m0 + C::RW * wm + 32 * mb + l32;
                            const int64_t n = n0 + C::CW * wn + 32 * nb + 8 * g + 4 * h;
                            const f32x16& acc = T[nb][mb];
                            const float4 v = make_float4(acc[4 * g], acc[4 * g + 1],
                                                         acc[4 * g + 2], acc[4 * g + 3]);
                            // the counter takes the element's index in the M x N output,
                            // the address the output's leading dimension
                            store(m * a.ldo + n, epilogue4(v, bb[nb][g], res(nb, g, mb),
                                                           m * a.N + n, a.drop));
                        }
            };
            auto store_f32 = [&](int64_t o_at, float4 o) {
                *reinterpret_cast<float4*>(a.out + o_at) = o;
            };
            if (RES_OK && use_res) {
                // the residual from the ring, read next to its use (an LDS read, no load
                // latency to hide); full tile: row r, columns nl .. nl + 3 = chunk nl / 8,
                // half h
                auto res_lds = [&](int nb, int g, int mb) -> uint2 {
                    const int r = C::RW * wm + 32 * mb + l32, rr = r & 127;
                    const int nl = C::CW * wn + 32 * nb + 8 * g + 4 * h;
                    const int slot = rr * 16 + ((nl >> 3) ^ (rr & 15));
                    return *reinterpret_cast<const uint2*>(xs_base + xstage(last + 1 + (r >> 7)) * C::XS +
                                                           slot * 8 + (nl & 7));
                };
                // v = T + bias, the epilogue's first add, before anything else: the bias
                // loads are consumed (and waited for) before the next item's copies go out
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            f32x16& acc = T[nb][mb];
                            acc[4 * g] = __fadd_rn(acc[4 * g], bf16_lo(bb[nb][g].x));
                            acc[4 * g + 1] = __fadd_rn(acc[4 * g + 1], bf16_hi(bb[nb][g].x));
                            acc[4 * g + 2] = __fadd_rn(acc[4 * g + 2], bf16_lo(bb[nb][g].y));
                            acc[4 * g + 3] = __fadd_rn(acc[4 * g + 3], bf16_hi(bb[nb][g].y));
                        }
                // the whole residual into registers; once every wave has it, the ring may
                // take the next item's first copies, which then run under this epilogue's
                // Philox arithmetic and stores
                uint2 rq[NB][4][MB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) rq[nb][g][mb] = res_lds(nb, g, mb);
                wg_barrier();
                if constexpr (C::NW == 8 && BK == 64) prefetch_next();
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            const int64_t m = m0 + C::RW * wm + 32 * mb + l32;
                            const int64_t n = n0 + C::CW * wn + 32 * nb + 8 * g + 4 * h;
                            const f32x16& acc = T[nb][mb];
                            const float4 v = make_float4(acc[4 * g], acc[4 * g + 1],
                                                         acc[4 * g + 2], acc[4 * g + 3]);
                            store_f32(m * a.ldo + n, epilogue4_v(v, rq[nb][g][mb], m * a.N + n, a.drop));
                        }
            } else {
                // every residual load issued first, so they are in flight together (and
                // under the Philox arithmetic) instead of one load latency per group
                uint2 rb[NB][4][MB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int nl = min(C::CW * wn + 32 * nb, cols - 32) + 8 * g + 4 * h;
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) {
                            const int ml = min(C::RW * wm + 32 * mb, rows - 32) + l32;
                            rb[nb][g][mb] = *reinterpret_cast<const uint2*>(
                                a.residual + (static_cast<int64_t>(m0) + ml) * a.ldr + n0 + nl);
                        }
                    }
                auto res_reg = [&](int nb, int g, int mb) { return rb[nb][g][mb]; };
                if (a.hout)
                    store_all([&](int64_t o_at, float4 o) {
                        *reinterpret_cast<uint2*>(a.hout + o_at) =
                            make_uint2(bf16x2_rne(o.x, o.y), bf16x2_rne(o.z, o.w));
                    }, res_reg);
                else
                    store_all(store_f32, res_reg);
            }
        } else if constexpr (MODE == kModePartials) {
            // The slice partial S_p through the idle copy ring to whole-row stores: each
            // wave writes its 64 x 128 block into its own 32 KB (16-byte chunk c of row r at
            // chunk c ^ (r % 32) of that row, so the 32 rows a store instruction of the MFMA
            // layout touches hit different banks), reads it back two rows (2 x 512 bytes)
            // per instruction and stores them contiguously into the partials [P][RM][RN];
            // then a barrier, so no wave's next copies overwrite a block still being read.
            static_assert(C::RW == 64 && C::BN == 128 && C::NW * 32768 <= C::RING_BYTES,
                          "staging layout of the partials tile");
            float* const stg = reinterpret_cast<float*>(smem) + uwave * (64 * 128);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int r = 32 * mb + l32, c = 8 * nb + 2 * g + h;   // 16-byte chunk
                        const f32x16& acc = S[nb][mb];
                        reinterpret_cast<float4*>(stg + r * 128)[c ^ (r & 31)] =
                            make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
                    }
            float* const dst0 = a.ws + static_cast<int64_t>(p_lo) * a.RM * a.RN +
                                static_cast<int64_t>(m0 + C::RW * wm - a.rm0) * a.RN + (n0 - a.rn0);
            const int c = lane & 31;
#pragma unroll 8
            for (int i = 0; i < 32; ++i) {
                const int r = 2 * i + h;   // row of this lane within the wave's 64
                const float4 v = reinterpret_cast<const float4*>(stg + r * 128)[c ^ (r & 31)];
                if (C::RW * wm + r < rows && 4 * c < cols)
                    *reinterpret_cast<float4*>(dst0 + static_cast<int64_t>(r) * a.RN + 4 * c) = v;
            }
            MMAR_WAIT_VM_LDS(63);   // lgkmcnt(0): this wave's ring reads have returned
            wg_barrier();
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        if (!col_ok(nb) || !row_ok(mb)) continue;
                        const int64_t m = m0 + C::RW * wm + 32 * mb + l32;
                        const int64_t n = n0 + C::CW * wn + 32 * nb + 8 * g + 4 * h;
                        const f32x16& acc = T[nb][mb];
                        *reinterpret_cast<float4*>(a.out + m * a.ldo + n) = make_float4(
                            acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
                    }
        }
    }
}

// ------------------------------------------------------------------ launchers
template <int MODE, int BK, bool WT, int TILE>
static hipError_t launch_tile_t(const TileArgs& a, int grid, hipStream_t s) {
    using C = typename TileCfgOf<MODE, BK, TILE>::type;
    constexpr int lds = C::LDS_BYTES;
    // the dynamic-LDS limit is raised once per device (bit d of the mask: device d)
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
    const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
    if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
        void (*fn)(TileArgs) = tile_kernel<MODE, BK, WT, TILE>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit, std::memory_order_release);
    }
    hipLaunchKernelGGL((tile_kernel<MODE, BK, WT, TILE>), dim3(grid), dim3(C::THREADS), lds, s,
                       a);
    return hipGetLastError();
}

template <bool WT>
static hipError_t launch_tile_w(int mode, int bk, int tile, const TileArgs& a, int grid,
                                hipStream_t s) {
    if (tile == kTile192) {
        if (mode == kModeFused) return launch_tile_t<kModeFused, 32, WT, kTile192>(a, grid, s);
        if (mode == kModeReduced) return launch_tile_t<kModeReduced, 32, WT, kTile192>(a, grid, s);
        return hipErrorInvalidValue;
    }
    if (tile == kTileHalf) {
        if (mode != kModeFused) return hipErrorInvalidValue;
        return bk == 64 ? launch_tile_t<kModeFused, 64, WT, kTileHalf>(a, grid, s)
                        : launch_tile_t<kModeFused, 32, WT, kTileHalf>(a, grid, s);
    }
    if (mode == kModeLinearWide) return launch_tile_t<kModeLinearWide, 32, WT, kTile128>(a, grid, s);
    if (bk == 64) {
        if (mode == kModeFused) return launch_tile_t<kModeFused, 64, WT, kTile128>(a, grid, s);
        if (mode == kModeReduced) return launch_tile_t<kModeReduced, 64, WT, kTile128>(a, grid, s);
        if (mode == kModeLinear) return launch_tile_t<kModeLinear, 64, WT, kTile128>(a, grid, s);
        return launch_tile_t<kModePartials, 64, WT, kTile128>(a, grid, s);
    }
    if (mode == kModeFused) return launch_tile_t<kModeFused, 32, WT, kTile128>(a, grid, s);
    if (mode == kModeReduced) return launch_tile_t<kModeReduced, 32, WT, kTile128>(a, grid, s);
    if (mode == kModeLinear) return launch_tile_t<kModeLinear, 32, WT, kTile128>(a, grid, s);
    return launch_tile_t<kModePartials, 32, WT, kTile128>(a, grid, s);
}

hipError_t launch_tile(int mode, int bk, bool wt, int tile, const TileArgs& a, int grid,
                       hipStream_t s) {
    if (!tile_supported(mode, tile)) return hipErrorInvalidValue;
    return wt ? launch_tile_w<true>(mode, bk, tile, a, grid, s)
              : launch_tile_w<false>(mode, bk, tile, a, grid, s);
}

template <int MODE, int BK, int TILE>
static int occ_t() {
    using C = typename TileCfgOf<MODE, BK, TILE>::type;
    int n = 0;
    const void* fn = reinterpret_cast<const void*>(&tile_kernel<MODE, BK, false, TILE>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, C::THREADS,
                                                     static_cast<size_t>(C::LDS_BYTES)) != hipSuccess)
        return 0;
    return n;
}

int tile_occupancy(int mode, int bk, int tile) {
    if (!tile_supported(mode, tile)) return 0;
    if (tile == kTile192)
        return mode == kModeFused ? occ_t<kModeFused, 32, kTile192>()
                                  : occ_t<kModeReduced, 32, kTile192>();
    if (tile == kTileHalf)
        return bk == 64 ? occ_t<kModeFused, 64, kTileHalf>() : occ_t<kModeFused, 32, kTileHalf>();
    if (mode == kModeLinearWide) return occ_t<kModeLinearWide, 32, kTile128>();
    if (bk == 64) {
        if (mode == kModeFused) return occ_t<kModeFused, 64, kTile128>();
        if (mode == kModeReduced) return occ_t<kModeReduced, 64, kTile128>();
        if (mode == kModeLinear) return occ_t<kModeLinear, 64, kTile128>();
        return occ_t<kModePartials, 64, kTile128>();
    }
    if (mode == kModeFused) return occ_t<kModeFused, 32, kTile128>();
    if (mode == kModeReduced) return occ_t<kModeReduced, 32, kTile128>();
    if (mode == kModeLinear) return occ_t<kModeLinear, 32, kTile128>();
    return occ_t<kModePartials, 32, kTile128>();
}

}  // namespace mmar
