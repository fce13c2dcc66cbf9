/*
 * mmar.h -- C ABI of the fused MatMul -> slice-reduce -> epilogue library (gfx950).
 *
 * The block.  A row-parallel (tensor-parallel) linear layer splits its contraction over
 * P ranks; rank p computes the partial product S_p = X[:, K_p] . W[K_p, :] and an
 * AllReduce sums the partials (CoCoNet record LIT-735, "Key takeaways", second bullet:
 * the model-parallel MatMul followed by the AllReduce that consumes it, overlapped in
 * chunks).  The pointwise work after it is fused into the reduction (same page, first
 * bullet: fusing pointwise work into a collective).  This library folds the P ranks
 * onto one GPU as P K-slices and computes
 *
 *     out = residual + dropout_p( bias + sum_{p=0}^{P-1} X[:, K_p] . W[K_p, :] )
 *
 * with K_p = [p*K/P, (p+1)*K/P).  Each partial S_p is accumulated in fp32 from zero;
 * the partials are added in fp32 in the fixed order p = 0, 1, ..., P-1 starting from
 * S_0, output chunk by output chunk; then v = T + bias[n], kept elements become
 * residual + v * scale and dropped ones residual, with scale = fp32(1 / (1 - p)).  The
 * keep decision is counter-based (Philox4x32-10, Salmon et al., SC'11): for the
 * element at row m, column n, e = m*N + n, the block with counter
 * (lo32(e>>2), hi32(e>>2), 0, 0) and key (lo32(seed), hi32(seed)) gives word
 * r = block[e & 3]; the element is dropped iff r < floor(p * 2^32).  The mask therefore
 * does not depend on chunking or on the schedule, and neither do the output bits:
 * every schedule below produces identical bytes.
 *
 * Schedules (the chunk scheduler: the MatMul and the reduction overlapped chunk by chunk,
 * as the CoCoNet record's second key takeaway describes):
 *   MMAR_SCHED_SEQUENTIAL  GEMM of a chunk's P partials into a workspace, then the
 *                          reduce+epilogue of that chunk, on one stream, no overlap.
 *   MMAR_SCHED_STREAMS     the same two kernels, the reduce+epilogue of chunk c on a
 *                          second HIP stream while the GEMM of chunk c+1 runs; a ring
 *                          of R workspace slots.
 *   MMAR_SCHED_PERSISTENT  one persistent kernel: each workgroup walks output tiles in
 *                          chunk order, reduces the P slices of a tile in registers and
 *                          applies the epilogue before moving on; no partials reach HBM.
 *   MMAR_SCHED_BALANCED    PERSISTENT over a head block of whole tile columns (or rows)
 *                          whose tile count is a multiple of the device's CU count, so
 *                          every round of the persistent grid is full; the tail, whose
 *                          tiles would leave part of the last round idle, is split by
 *                          slice instead: its P one-slice partials per tile are spread
 *                          over all CUs, then the reduce+epilogue kernel sums them in
 *                          slice order.  Whole-output chunk only; the tail's partials
 *                          take P x M x (tail columns) x 4 bytes (or P x (tail rows) x
 *                          N x 4) of workspace.  Without such a split it is PERSISTENT.
 *   MMAR_SCHED_SPLIT       PERSISTENT over the same head block, then PERSISTENT again over
 *                          the tail on 128 x 128 tiles (twice as many as whole tiles, so
 *                          their round fills more CUs for half as long); no partials and no
 *                          workspace.  Whole-output chunk only.  Without a split it is
 *                          PERSISTENT.
 *
 * Layouts.  X [M,K], W [K,N], residual [M,N] row-major, contiguous, bf16 bit patterns
 * (uint16); bias [N] bf16 bits; out [M,N] row-major fp32.  All tensor pointers are
 * DEVICE pointers on the current HIP device.  mmar_fused_nt takes the weight
 * transposed, W^T [N,K] row-major (the layout of a Linear layer's weight).
 *
 * Weight modes.  The tile kernel needs each lane's MFMA operand as 8 consecutive k of one
 * column of W.  MMAR_W_DIRECT reads W [K,N] as given and transposes fragments with the LDS
 * transpose read; MMAR_W_PRETRANSPOSE first writes W^T [N,K] into the workspace
 * (4 K N bytes of memory traffic) and then reads both operands with plain 16-byte LDS
 * reads.  Both produce identical bits.
 *
 * Preconditions (checked; violations return MMAR_EINVAL before any device work and
 * leave `out` untouched): M, N, K > 0; 1 <= P <= 4096; K % P == 0; (K/P) % 32 == 0;
 * M % 32 == 0; N % 32 == 0; every tensor has fewer than 2^31 elements; p_drop finite
 * and in [0, 1]; chunk_m / chunk_n each 0 (library choice) or a multiple of 32 dividing
 * M (resp. N).  Pointers must be 16-byte aligned (else MMAR_EALIGN).  `out` must not
 * overlap any input.
 *
 * Ownership.  The caller owns every tensor and keeps it alive until the stream has
 * passed the call; the library never frees or retains caller memory.  The library owns
 * a per-device workspace (partial-product ring, pre-transposed weight), a second stream
 * and events, created on first use and freed by mmar_release().  Calls that use the
 * library workspace are serialized per device by a mutex; with a caller workspace
 * (mmar_fused_ex) calls are re-entrant.
 *
 * Errors.  Every int-returning call returns MMAR_OK (0) or a negative code; details of
 * the last failure on the calling thread are in mmar_last_error().  Asynchronous device
 * faults surface at the caller's next synchronization, as for any HIP kernel.  No C++
 * exception crosses this interface.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 * work is ordered after earlier work on `stream` and before later work on it: the
 * second stream of MMAR_SCHED_STREAMS waits for `stream` on entry and `stream` waits
 * for it before the call returns.
 *
 * Around the block: mmar_linear / mmar_gelu_linear (the column-parallel MatMul + bias and
 * GeLU, or no activation for an attention block's QKV projection, that produces the
 * block's X), mmar_unfused (the block one kernel per operation, for comparison) and
 * mmar_adam_step (the data-parallel gradient average + Adam step, one HBM pass).
 */
#ifndef MMAR_H
#define MMAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MMAR_OK = 0,
    MMAR_EINVAL = -1, /* bad argument; nothing was launched */
    MMAR_EALIGN = -2, /* a pointer is not 16-byte aligned */
    MMAR_ENODEV = -3, /* no gfx950 device is current */
    MMAR_ENOMEM = -4, /* device allocation failed or workspace too small */
    MMAR_EHIP = -5    /* a HIP runtime call failed; see mmar_last_error() */
};

enum {
    MMAR_SCHED_AUTO = 0,
    MMAR_SCHED_SEQUENTIAL = 1,
    MMAR_SCHED_STREAMS = 2,
    MMAR_SCHED_PERSISTENT = 3,
    MMAR_SCHED_BALANCED = 4,
    MMAR_SCHED_SPLIT = 5
};

enum { MMAR_W_AUTO = -1, MMAR_W_DIRECT = 0, MMAR_W_PRETRANSPOSE = 1 };

/* Output tile of the persistent fused kernel (MMAR_SCHED_PERSISTENT, and the head block of
 * MMAR_SCHED_BALANCED and MMAR_SCHED_SPLIT, whose tail always runs on 128 x 128 tiles; the
 * chunked schedules always use 256 x 128).
 *   MMAR_TILE_256x128  8 waves per workgroup, each a 64 x 64 block of the tile.
 *   MMAR_TILE_256x192  4 waves, each a 128 x 96 block: 42 % fewer operand bytes read from
 *                      LDS and 22 % fewer bytes copied into it per flop; 3 of a wave's 12
 *                      running-total blocks are kept in LDS.  K steps of 32.
 * Both give identical output bits (every 32 x 32 output block sees the same MFMA sequence
 * and the same reduction and epilogue).  AUTO: the plan's (default 256 x 128). */
enum { MMAR_TILE_AUTO = -1, MMAR_TILE_256x128 = 0, MMAR_TILE_256x192 = 1 };

/* Activation of the producer MatMul (mmar_linear). */
enum { MMAR_ACT_NONE = 0, MMAR_ACT_GELU_TANH = 1 };

/* The fused block with the library's schedule for this shape: the plan set by
 * mmar_set_plan or found by mmar_autotune, else the persistent schedule.  chunk_m /
 * chunk_n override the plan's chunk when non-zero.  Uses the library workspace. */
int mmar_fused(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
               const uint16_t* residual, float* out, int64_t M, int64_t N, int64_t K,
               int32_t P, float p_drop, uint64_t seed, int32_t chunk_m, int32_t chunk_n,
               void* stream);

/* The same block with the weight given transposed, Wt = W^T [N,K] row-major (the layout of
 * a Linear layer's weight); no transpose is needed.  Same plan, same bits as mmar_fused
 * on W = Wt^T. */
int mmar_fused_nt(const uint16_t* X, const uint16_t* Wt, const uint16_t* bias,
                  const uint16_t* residual, float* out, int64_t M, int64_t N, int64_t K,
                  int32_t P, float p_drop, uint64_t seed, int32_t chunk_m, int32_t chunk_n,
                  void* stream);

/* The block with a bf16 output, for a model that keeps its residual stream in bf16: out
 * [M,N] bf16 row-major (written; must not overlap an input) receives the fp32 result of
 * mmar_fused rounded once to bf16 (nearest even), so each element equals that rounding of
 * mmar_fused's output on the same arguments.  The fp32 tolerance of the block does not
 * carry over (the bf16 rounding alone exceeds it); the result is judged against the
 * oracle's fp64 value rounded to bf16, either neighbour accepted where that value lies
 * within the fp32 error bound of a rounding midpoint.  Persistent schedule, W as
 * [K,N], whole output in one chunk; preconditions, dropout and errors as mmar_fused.  No
 * workspace. */
int mmar_fused_bf16(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
                    const uint16_t* residual, uint16_t* out, int64_t M, int64_t N, int64_t K,
                    int32_t P, float p_drop, uint64_t seed, void* stream);

/* Workspace bytes a plan needs: K N 2 (256-aligned) for MMAR_W_PRETRANSPOSE, plus the
 * partial-product ring for MMAR_SCHED_SEQUENTIAL (P chunk_m chunk_n 4) and
 * MMAR_SCHED_STREAMS (ring times that), plus the tail partials of MMAR_SCHED_BALANCED
 * (which depend on the tile); MMAR_SCHED_SPLIT needs none.  schedule AUTO: the plan mmar_fused would use (with non-zero
 * chunk / ring and non-AUTO w_mode / tile arguments overriding).  ring = number of chunk
 * slots for MMAR_SCHED_STREAMS (0 = the default, 2).  Returns 0 and sets the last error on
 * invalid arguments. */
size_t mmar_workspace_bytes(int32_t schedule, int64_t M, int64_t N, int64_t K, int32_t P,
                            int32_t chunk_m, int32_t chunk_n, int32_t ring, int32_t w_mode,
                            int32_t tile);

/* The fused block with every choice explicit (tile: an MMAR_TILE_* value).  workspace ==
 * NULL: the library's workspace is used (serialized per device); otherwise `workspace`
 * (device memory, 16-byte aligned, at least mmar_workspace_bytes(...) bytes, owned by the
 * caller and not used by any other call until the stream passes this one) and the call is
 * re-entrant.  A too-small caller workspace returns MMAR_ENOMEM. */
int mmar_fused_ex(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
                  const uint16_t* residual, float* out, int64_t M, int64_t N, int64_t K,
                  int32_t P, float p_drop, uint64_t seed, int32_t schedule, int32_t chunk_m,
                  int32_t chunk_n, int32_t ring, int32_t w_mode, int32_t tile, void* workspace,
                  size_t ws_bytes, void* stream);

/* The fused block (the CoCoNet record LIT-735, "Key takeaways", second bullet) over
 * buffers with leading dimensions and a dropout stream offset.  ldx, ldw, ldr, ldo: elements
 * between consecutive rows of X [M,K], W [K,N], residual [M,N] and out [M,N] (each at
 * least its row length; ldx and ldw multiples of 8, ldr and ldo multiples of 4; every
 * extent (rows - 1) * ld + row below 2^31 elements), so that a rank's operand can be a view
 * into a larger buffer, as the K-slice X[:, K_p] of the shard view is a column block of X
 * with leading dimension K.  philox_offset fills counter words 2 and 3 (low, high 32 bits)
 * of the mask's Philox blocks, which every other entry point leaves 0: element (m, n) takes
 * word e & 3 of the block with counter (lo32(e>>2), hi32(e>>2), lo32(offset), hi32(offset)),
 * e = m*N + n whatever the leading dimensions, so one seed gives an independent mask per
 * offset (a layer or step index) and offset 0 reproduces mmar_fused's bits.  Runs the
 * persistent schedule (the cached plan if it is a persistent one reading W directly, else
 * the default persistent plan); needs no workspace and allocates nothing.  The residual
 * pointer needs 8-byte alignment only (the others 16).  Preconditions, dropout and errors
 * otherwise as mmar_fused; out must not overlap any input's extent. */
int mmar_fused_strided(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                       const uint16_t* bias, const uint16_t* residual, int64_t ldr, float* out,
                       int64_t ldo, int64_t M, int64_t N, int64_t K, int32_t P, float p_drop,
                       uint64_t seed, uint64_t philox_offset, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mmar_fused_ex with its workspace taken
 * from a static per-device array of mmar_noalloc_workspace_capacity() bytes (64 MiB) that
 * the library holds from load to process exit; no hipMalloc, hipFree or other allocation
 * on this path.  Arguments as mmar_fused_ex (without workspace); the plan is resolved the
 * same way.  Plans whose workspace exceeds the capacity return MMAR_ENOMEM, and
 * MMAR_SCHED_STREAMS (whose side stream and events are created on first use) returns
 * MMAR_EINVAL, both before any device work.  Every call on a device shares that device's
 * array: calls that overlap on one device (two streams, two threads) race. */
int mmar_fused_noalloc(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
                       const uint16_t* residual, float* out, int64_t M, int64_t N, int64_t K,
                       int32_t P, float p_drop, uint64_t seed, int32_t schedule,
                       int32_t chunk_m, int32_t chunk_n, int32_t ring, int32_t w_mode,
                       int32_t tile, void* stream);
size_t mmar_noalloc_workspace_capacity(void);

/* MMAR_SCHED_SEQUENTIAL with the library workspace: the comparison point of the CoCoNet
 * record that fuses the same work but does not overlap it ("Key takeaways", second
 * bullet). */
int mmar_sequential(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
                    const uint16_t* residual, float* out, int64_t M, int64_t N, int64_t K,
                    int32_t P, float p_drop, uint64_t seed, int32_t chunk_m, int32_t chunk_n,
                    void* stream);

/* W [K,N] -> W^T [N,K] (bf16 bits), for callers that keep the transposed weight and call
 * mmar_fused_nt.  K, N positive multiples of 32; Wt must not overlap W. */
int mmar_transpose_weight(const uint16_t* W, uint16_t* Wt, int64_t K, int64_t N, void* stream);

/* Measurement entry point: the persistent kernel with the epilogue removed, with the plan's
 * weight mode (its transpose included).  Writes the reduced sum T = S_0 + ... + S_{P-1}
 * (fp32, fixed order) to T_out [M,N]; the same MFMA sequence as mmar_fused, so T_out +
 * epilogue reproduces its bits.  Uses the library workspace for a pre-transposed W. */
int mmar_gemm_only(const uint16_t* X, const uint16_t* W, float* T_out, int64_t M, int64_t N,
                   int64_t K, int32_t P, int32_t chunk_m, int32_t chunk_n, void* stream);

/* Measurement entry point: the P per-slice partials S_p, fp32, written to
 * partials [P][M][N] (each slice accumulated from zero), with the plan's weight mode. */
int mmar_gemm_partials(const uint16_t* X, const uint16_t* W, float* partials, int64_t M,
                       int64_t N, int64_t K, int32_t P, void* stream);

/* The producer side of the block: the column-parallel MatMul that precedes it in a
 * transformer MLP (the block sits between two MatMuls: practices record SOTA-059, "Where
 * it stops being free"), H = GeLU(X . W + bias) with GeLU in its tanh form,
 *   X     bf16 [M, K] row-major,  W bf16 [K, N] row-major,  bias bf16 [N],
 *   H     bf16 [M, N] row-major (written; must not overlap an input),
 * computed as v = fp32 sum over k (MFMA, k ascending) + bias, gelu(v) in fp32, rounded
 * to bf16 (nearest even).  Column block p of H is what rank p of the column-parallel
 * layer would own, and it is exactly K-slice p of the block that follows, so H feeds
 * mmar_fused directly as its X.  Preconditions as mmar_fused with P = 1.  No
 * workspace.  The leading output columns (a multiple of 256) are computed on 256 x 256
 * tiles and the rest on 256 x 128 tiles, split so that the tiles fill whole rounds of the
 * CUs (one or two launches; the environment variable MMAR_LINEAR_TILE = 128 or 256 puts
 * every column on one width, for measurements); the bits do not depend on the split. */
int mmar_gelu_linear(const uint16_t* X, const uint16_t* W, const uint16_t* bias, uint16_t* H,
                     int64_t M, int64_t N, int64_t K, void* stream);

/* The producer MatMul with its activation chosen: MMAR_ACT_GELU_TANH is mmar_gelu_linear;
 * MMAR_ACT_NONE gives H = X . W + bias, the QKV projection in front of an attention
 * block's out-projection (its column block p holds the Q, K and V columns of the heads
 * of rank p, which are what that rank's attention reads), rounded once from fp32 to bf16
 * (nearest even).  Same arguments, preconditions and layout as mmar_gelu_linear; any
 * other activation value returns MMAR_EINVAL before any device work. */
int mmar_linear(const uint16_t* X, const uint16_t* W, const uint16_t* bias, uint16_t* H,
                int64_t M, int64_t N, int64_t K, int32_t activation, void* stream);

/* The MLP around the block, producer and block in one call (the block sits between two
 * MatMuls: practices record SOTA-059, "Where it stops being free"; CoCoNet overlaps a
 * producer with the collective that consumes it: LIT-735, "Key takeaways", first bullet):
 *   H   = GeLU(X0 . W1 + b1)          X0 [M, D], W1 [D, K], b1 [K], H [M, K] bf16 (written)
 *   out = residual + dropout_p(b2 + sum_p H[:, K_p] . W2[K_p, :])
 *                                     W2 [K, N], b2 [N], residual [M, N] bf16, out [M, N] fp32
 * with the arithmetic of mmar_gelu_linear and mmar_fused (same bits as calling the two in
 * turn).  chunk_m = 0: the producer over all rows, then the block, on `stream`.  chunk_m a
 * multiple of 32 dividing M: row chunks, the producer of chunk c on `stream` and the block
 * of chunk c on the library's side stream once that chunk of H is written, so the producer
 * of the next chunk runs beside it (H handed over chunk by chunk, the way an all-gathered
 * input arrives); `stream` waits for the side stream before the call returns.
 * Preconditions as mmar_gelu_linear (M, K, D) and mmar_fused (M, N, K, P); H must not
 * overlap any other argument, out no input.  Uses no workspace; the chunked form uses the
 * side stream (serialized per device). */
int mmar_mlp(const uint16_t* X0, const uint16_t* W1, const uint16_t* b1, const uint16_t* W2,
             const uint16_t* b2, const uint16_t* residual, uint16_t* H, float* out, int64_t M,
             int64_t D, int64_t K, int64_t N, int32_t P, float p_drop, uint64_t seed,
             int32_t chunk_m, void* stream);

/* The data-parallel side of the CoCoNet record ("Key takeaways", fifth bullet: the
 * gradient ReduceScatter, the optimizer and the parameter AllGather fused) folded onto
 * one GPU, one HBM pass:
 *   grads       fp32 [P][n]  the P data-parallel replicas' gradients (read)
 *   param, m, v fp32 [n]     parameters, first and second Adam moments (updated in place)
 *   param_bf16  bf16 [n]     the new parameters rounded to bf16 (written), or NULL
 * g = (G_0 + ... + G_{P-1}) * fp32(1/P) (fixed order); m = b1 m + (1-b1) g;
 * v = b2 v + (1-b2) g^2; p = p - lr ((m c1) / (sqrt(v c2) + eps) + weight_decay p), with
 * c1 = 1/(1-b1^step), c2 = 1/(1-b2^step) from fp64 on the host (Adam; weight_decay > 0
 * gives AdamW's decoupled decay).  fp32, round to nearest even, no fused multiply-add.
 * Preconditions: n > 0 and a multiple of 4; 1 <= P <= 4096; step >= 1; 0 <= b1, b2 < 1;
 * eps > 0; fp32 pointers 16-byte aligned, param_bf16 8-byte aligned; no buffer overlaps
 * another.  No workspace. */
int mmar_adam_step(const float* grads, float* param, float* m, float* v, uint16_t* param_bf16,
                   int64_t n, int32_t P, int64_t step, float lr, float beta1, float beta2,
                   float eps, float weight_decay, void* stream);

/* Comparison entry point: the same block computed unfused, one kernel per operation, the
 * way frameworks that call computation and communication as separate library kernels run
 * it (the baseline the CoCoNet record compares against, "Key takeaways", first and second
 * bullets): the P slice GEMMs write all partials to a workspace, a reduction kernel sums
 * them left to right, then separate bias-add, dropout and residual-add kernels.  The
 * dropout kernel writes the keep mask as bytes (1 = kept) to `mask` [M][N] (uint8,
 * device; NULL: to the library workspace).  Same arguments, preconditions and output bits
 * as mmar_fused; uses the library workspace, 4*P*M*N (+ M*N without `mask`) bytes. */
int mmar_unfused(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
                 const uint16_t* residual, float* out, uint8_t* mask, int64_t M, int64_t N,
                 int64_t K, int32_t P, float p_drop, uint64_t seed, void* stream);

/* The slice reduction plus epilogue alone, over P materialized fp32 partials
 * [P][M][N]: T = S_0 + S_1 + ... (fixed order), then the bias, dropout and residual
 * epilogue.  With P = 1 it is the epilogue alone over a materialized T. */
int mmar_reduce_epilogue_only(const float* partials, const uint16_t* bias,
                              const uint16_t* residual, float* out, int64_t M, int64_t N,
                              int32_t P, float p_drop, uint64_t seed, void* stream);

/* The autotuner (CoCoNet picks its schedules by automatic search; "Key takeaways", first
 * bullet): times candidate {schedule, tile, chunk, weight mode} plans for this shape on
 * library-owned buffers, 25 rounds interleaved (each round times every candidate once, in
 * an order rotated from round to round, as 4 calls back to back between two events), and
 * keeps the default plan unless a candidate's
 * median time beats it by more than the larger of the two interquartile ranges and by at
 * least 1 % of the default's median; among such candidates the fastest wins, and a
 * candidate tied with it within their interquartile ranges wins instead if it comes
 * first in candidate order (larger chunks, W read directly, the 256 x 128 tile).  The
 * choice goes to the plan cache (also written, with its margin, to the JSON file named by
 * the MMAR_PLAN_CACHE environment variable, if set).  flags: bit 0 = also try MMAR_SCHED_STREAMS and
 * MMAR_SCHED_SEQUENTIAL plans.  Synchronizes the device. */
int mmar_autotune(int64_t M, int64_t N, int64_t K, int32_t P, uint32_t flags);

/* Set / read the plan used by mmar_fused for this shape on the current device.
 * schedule is one of MMAR_SCHED_*, AUTO clears the entry; w_mode one of MMAR_W_*; tile
 * one of MMAR_TILE_*.  mmar_get_plan writes the plan that mmar_fused would use (the
 * default when none is set: persistent, whole-output chunk, MMAR_W_DIRECT,
 * MMAR_TILE_256x128). */
int mmar_set_plan(int64_t M, int64_t N, int64_t K, int32_t P, int32_t schedule,
                  int32_t chunk_m, int32_t chunk_n, int32_t ring, int32_t w_mode, int32_t tile);
int mmar_get_plan(int64_t M, int64_t N, int64_t K, int32_t P, int32_t* schedule,
                  int32_t* chunk_m, int32_t* chunk_n, int32_t* ring, int32_t* w_mode,
                  int32_t* tile);

/* Text of the last error on the calling thread ("" if none).  Valid until the next
 * call on this thread. */
const char* mmar_last_error(void);

/* Library version string, e.g. "mmar 0.1.0 gfx950". */
const char* mmar_version(void);

/* Frees the library's workspaces, streams and events on every device.  Synchronizes
 * the devices first.  Safe to call more than once. */
int mmar_release(void);

#ifdef __cplusplus
}
#endif

#endif /* MMAR_H */
