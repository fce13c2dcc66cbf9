// Internal interface between the host scheduler (mmar.cpp) and the gfx950 kernels
// (tile_kernel.hip, reduce_kernels.hip, unfused.hip).  Not installed; the public interface
// is include/mmar.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmar {

// What the tile kernel does with each finished output tile.
enum TileMode : int {
    kModeFused = 0,     // all P slices, reduced in registers, then bias/dropout/residual
    kModeReduced = 1,   // all P slices, reduced in registers, stored as fp32 T
    kModePartials = 2,  // one slice per work item, stored as fp32 S_p to a workspace
    kModeLinear = 3,    // all slices (the producer MatMul has P = 1), + bias, activation,
                        // bf16 out
    kModeLinearWide = 4,  // kModeLinear for one slice on 256 x 256 tiles (no running total,
                          // so the registers hold a tile twice as wide)
};
constexpr int kNumModes = 5;

// Activation of kModeLinear (the values of the public MMAR_ACT_* constants).
enum Activation : int {
    kActNone = 0,       // H = X . W + bias (the attention block's QKV projection)
    kActGeluTanh = 1,   // H = GeLU(X . W + bias), tanh form (the MLP's first MatMul)
};

// Dropout parameters as the kernels use them.
struct DropParams {
    uint32_t thr;       // drop iff Philox word < thr
    uint32_t drop_all;  // p == 1: every element is dropped
    float scale;        // fp32(1 / (1 - p)); 1 when p == 0
    uint32_t key0, key1;
    uint32_t ctr2, ctr3;  // counter words 2 and 3: the low and high word of the offset
};

// Arguments of the tile kernel.  The kernel covers the output region
// [rm0, rm0 + RM) x [rn0, rn0 + RN), split into chunks of cm x cn (which divide RM and
// RN) and each chunk into BM x BN tiles visited in chunk order.
struct TileArgs {
    const uint16_t* X;   // [M, K] bf16 bits
    const uint16_t* W;   // [K, N] bf16 bits, or W^T [N, K] for the transposed-W kernel
    const uint16_t* bias;
    const uint16_t* residual;
    float* out;          // kModeFused / kModeReduced: [M, N]
    uint16_t* hout;      // kModeLinear: bf16 [M, N]; kModeFused: bf16 output instead of out
                         // when set
    float* ws;           // kModePartials: [P][RM][RN] for the region
    int64_t M, N, K;
    // leading dimensions (elements between consecutive rows): X (>= K), W (>= N; >= K for
    // W^T), residual and out / hout (>= N)
    int64_t ldx, ldw, ldr, ldo;
    int32_t P, Ks;       // Ks = K / P
    int32_t rm0, rn0, RM, RN;
    int32_t cm, cn;
    int32_t total_items; // tiles (x P for kModePartials)
    int32_t act;         // kModeLinear: Activation
    DropParams drop;
};

struct ReduceArgs {
    const float* ws;     // [P][RM][RN]
    const uint16_t* bias;
    const uint16_t* residual;
    float* out;          // [M, N]
    int64_t N;           // leading dimension of out / residual
    int32_t P;
    int32_t rm0, rn0, RM, RN;
    DropParams drop;
};

// Arguments of the fused reduce + Adam kernel (adam.hip).
struct AdamArgs {
    const float* grads;   // [P][n]
    float* param;         // [n], updated in place
    float* m;             // [n], first moment, updated in place
    float* v;             // [n], second moment, updated in place
    uint16_t* param_bf16; // [n] bf16 copy of the new parameters, or NULL
    int64_t n;            // multiple of 4
    int32_t P;
    float inv_p, lr, b1, b2, one_minus_b1, one_minus_b2, eps, wd, c1, c2;
};

constexpr int kBM = 256;   // output rows per tile
constexpr int kBN = 128;   // output columns per tile
constexpr int kBNWide = 256;   // output columns per tile of kModeLinearWide

// Tile shapes of the block's modes (kModeFused, kModeReduced): the plan's choice, and the
// half-height tile of the split schedule's tail.
enum TileShape : int {
    kTile128 = 0,   // 256 x 128: 8 waves of 64 x 64 at BK = 64 (4 waves of 64 x 128 at BK = 32)
    kTile192 = 1,   // 256 x 192: 4 waves of 128 x 96, BK = 32
    kTileHalf = 2,  // 128 x 128 (kModeFused only): 8 waves of 64 x 32 at BK = 64 (4 waves of
                    // 64 x 64 at BK = 32); twice as many tiles for a tail region, so a last
                    // round of whole tiles that would leave CUs idle fills them instead
};
constexpr int kNumTiles = 3;
constexpr int kBMHalf = 128;
// Output rows per tile of a tile shape.
constexpr int tile_bm(int tile) { return tile == kTileHalf ? kBMHalf : kBM; }
constexpr int kBN192 = 192;
// Output columns per tile of a mode on a tile shape (the partials and producer modes
// have one shape each).
constexpr int tile_bn(int mode, int tile = kTile128) {
    return mode == kModeLinearWide ? kBNWide
           : (tile == kTile192 && (mode == kModeFused || mode == kModeReduced)) ? kBN192
                                                                               : kBN;
}
constexpr bool tile_supported(int mode, int tile) {
    return tile == kTile128 ||
           (tile == kTile192 && (mode == kModeFused || mode == kModeReduced)) ||
           (tile == kTileHalf && mode == kModeFused);
}

// Launchers (tile_kernel.hip, reduce_kernels.hip).  bk is 64 or 32 (the K step; it must
// divide Ks; kModeLinearWide and kTile192 always step by 32).  wt: a.W holds W^T [N, K]
// instead of W [K, N].  tile: a TileShape that tile_supported(mode, tile) accepts.
hipError_t launch_tile(int mode, int bk, bool wt, int tile, const TileArgs& a, int grid,
                       hipStream_t s);
hipError_t launch_transpose(const uint16_t* W, uint16_t* Wt, int64_t K, int64_t N, hipStream_t s);
hipError_t launch_reduce_epilogue(const ReduceArgs& a, int grid, hipStream_t s);
hipError_t launch_fill_bf16(uint16_t* p, int64_t n, uint32_t salt, float amp, hipStream_t s);
hipError_t launch_adam(const AdamArgs& a, int grid, hipStream_t s);
// The unfused tail (unfused.hip): sum of the P partials ws [P][M][N] into T (may alias ws),
// then bias add, dropout (keep bytes to mask [M][N]) and residual add into out, each its
// own kernel on stream s.
hipError_t launch_unfused_tail(const float* ws, float* T, const uint16_t* bias,
                               const uint16_t* residual, float* out, uint8_t* mask, int64_t M,
                               int64_t N, int32_t P, const DropParams& d, int grid, hipStream_t s);
// Host-side entry for callers that bring a fixed workspace and must not allocate
// (mmar.cpp): the fused block with the plan resolved as for mmar_fused_ex; MMAR_* codes.
int fused_fixed_ws(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
                   const uint16_t* residual, float* out, int64_t M, int64_t N, int64_t K,
                   int32_t P, float p_drop, uint64_t seed, int32_t sched, int32_t chunk_m,
                   int32_t chunk_n, int32_t ring, int32_t wmode, int32_t tile, void* ws,
                   size_t ws_cap, void* stream);
// Sets the calling thread's last-error text (mmar_last_error).
void set_error(const char* msg);

// Workgroups of the tile kernel that fit on one CU at once (0 on error or for a shape
// the mode does not have).
int tile_occupancy(int mode, int bk, int tile);
int reduce_occupancy();

}  // namespace mmar
