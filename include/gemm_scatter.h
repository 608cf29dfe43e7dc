/*
 * gemm_scatter.h -- C ABI of the GEMM whose epilogue stores straight into
 * reduce-scatter buffers, in librmsnorm.so, on MI355X (gfx950).
 *
 * The operation follows page "LLM System: 通信计算融合算子实现 01 - sm80GEMM +
 * ReduceScatter":
 *   - section "flux实现：sm80 gemm+rs": the second GEMM of a tensor-parallel
 *     FFN writes its output tiles into the reduce-scatter buffers in its
 *     epilogue, so no separate copy is needed;
 *   - section "cutlass自定义epilogue–sm80": the epilogue computes
 *     alpha * accumulator + beta * C and scatters each tile to the buffer
 *     that holds it, raising a per-tile flag once the tile is written;
 *   - section "gemmrs版本的swizzle如何编排": the output is cut into one chunk
 *     per rank and the tiles of the other ranks' chunks are computed first,
 *     the local chunk last.
 * On one GPU every buffer is local memory; with several GPUs dst[q] would be
 * rank q's receive buffer (mapped peer memory), and the reduction of the
 * received chunks with the residual is add_rmsnorm_fwd with k = world.
 *
 * What is computed (products accumulate in fp32 on the matrix cores):
 *     D[i][j] = alpha * sum_p A[i][p] * B[j][p] + beta * C[i][j]
 * A [m][k], B [n][k] (the weight layout of a linear layer: k contiguous),
 * C [m][n] (optional); D rounded once to the storage type (round to nearest
 * even).  The m rows form `world` chunks of m / world rows; row i goes to
 * chunk q = i / (m / world), stored at dst[q] + (i - q * m / world) * ldd.
 * The fp32 result differs from the exact value by at most about
 * k * 2^-24 * (|alpha| * sum_p |A[i][p] * B[j][p]|) + 2^-23 * |beta * C[i][j]|
 * before the final rounding.
 *
 * Conventions (shared with rmsnorm.h, whose RMSN_* codes and
 * rmsnorm_strerror / rmsnorm_last_error apply):
 *   - a, b, c, every dst[q] and flags are DEVICE pointers; `dst` itself is a
 *     HOST array of `world` pointers, read during the call only.  Strides
 *     (lda, ldb, ldc, ldd) are in elements.
 *   - dtype: RMSN_F16 or RMSN_BF16 for every tensor.
 *   - For k > 0, a and b must be 16-byte aligned with lda, ldb and k
 *     multiples of 8 (whole 16-byte chunks along k); with k == 0 they are
 *     not read.  c and dst need 2-byte alignment.
 *   - 1 <= world <= GEMM_SCATTER_WORLD_MAX, 0 <= rank < world, m divisible
 *     by world; m, n, k below 2^31; 255 * lda + k and 255 * ldb + k below
 *     2^29 (a tile's operand rows are addressed with 32-bit offsets).
 *   - tile_n: the output tile's width, GEMM_SCATTER_TILE_N (256) or
 *     GEMM_SCATTER_TILE_N_NARROW (128); 0 takes gemm_scatter_tile_n(m, n).
 *     The 128-wide tiles are GEMM_SCATTER_TILE_M (256) rows high; the
 *     256-wide ones 256, 192 or 160 rows, gemm_scatter_tile_m(m, n, tile_n)
 *     (shorter tiles fill rounds of workgroups that 256-row tiles would
 *     leave partly idle).  Every output is accumulated in the same k order
 *     at every tile shape, so the results do not depend on it.
 *   - flags (nullable): gemm_scatter_tiles(m, n, tile_n) uint32 slots.  When
 *     given, the workgroup that computes tile t stores `epoch` to flags[t]
 *     after the tile's elements are written and made visible at system
 *     scope, so a consumer that reads flags[t] == epoch sees the whole tile.
 *     Tile t covers rows [(t / T) * H, ...) and columns [(t % T) * W, ...),
 *     H and W the tile height and width used, T = ceil(n / W).
 *   - dst chunks must not overlap each other, a, b, c or flags, and flags
 *     must not overlap a, b or c (RMSN_ERR_ALIAS otherwise).
 *   - The call enqueues one kernel on `stream` (NULL: the default stream),
 *     allocates nothing and does not synchronise.  Arguments are validated
 *     before the launch; on error nothing is launched.  m == 0 or n == 0
 *     launches nothing; k == 0 gives beta * C (or zeros).
 */
#ifndef GEMM_SCATTER_H
#define GEMM_SCATTER_H

#include <stdint.h>

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_SCATTER_WORLD_MAX 16
#define GEMM_SCATTER_TILE_M 256
#define GEMM_SCATTER_TILE_N 256
#define GEMM_SCATTER_TILE_N_NARROW 128
/* The automatic width counts rounds of workgroups (one tile each) over the
 * compute units of an MI355X.  A full round of 256 x 128 tiles takes about
 * 0.63 of the time of a full round of 256 x 256 tiles (63 against 101 us on
 * the 8192 x 3584 bf16 weights), but a round the 256-wide tiles fill only in
 * part costs less than a full one (2560 tokens: 156 us in two 256-wide
 * rounds of 256 and 64 tiles, 163 us in three 128-wide rounds), so the
 * narrow width is taken only when it needs no more rounds than the wide
 * one: ceil(T128 / CUS) <= ceil(T256 / CUS), T the tile count at each width
 * (T > 0). */
#define GEMM_SCATTER_CUS 256

/*
 * gemm_scatter_fwd -- the epilogue-scattered product above.  Returns RMSN_OK,
 * RMSN_ERR_NULL, RMSN_ERR_SHAPE (sizes, strides, alignment, world, rank,
 * tile_n), RMSN_ERR_DTYPE, RMSN_ERR_ALIAS or RMSN_ERR_HIP.
 */
int gemm_scatter_fwd(void* const* dst, int64_t ldd, int world, int rank, const void* a,
                     int64_t lda, const void* b, int64_t ldb, const void* c, int64_t ldc,
                     float alpha, float beta, int64_t m, int64_t n, int64_t k, int dtype,
                     uint32_t* flags, uint32_t epoch, int tile_n, void* stream);

/* gemm_scatter_tile_n -- the tile width tile_n = 0 takes for m x n, by the
 * rule beside GEMM_SCATTER_CUS; -1 if m or n is negative or too large. */
int gemm_scatter_tile_n(int64_t m, int64_t n);

/* gemm_scatter_tile_m -- the tile height a call with this m, n and tile_n
 * (0: automatic width) uses: 256 for the 128-wide tiles; for the 256-wide
 * ones the height set by gemm_scatter_tune, else the cheapest of 256, 192
 * and 160 rows by an estimate of the rounds of workgroups each needs (a
 * partial round counting 0.7 + 0.3 f of a full one, f the fraction of the
 * CUS it keeps busy) times a round's cost (a fixed part plus a part in
 * proportion to the rows; fitted on MI355X to 8192 x 3584 bf16 weights:
 * 85.6, 68.3 and 62.5 us per full round), ties to the taller tile.  -1 if m
 * or n is negative or too large, or tile_n is not 0, 128 or 256. */
int gemm_scatter_tile_m(int64_t m, int64_t n, int tile_n);

/* gemm_scatter_tiles -- number of output tiles (and flag slots) for m x n at
 * tile width tile_n (0: automatic), at the height gemm_scatter_tile_m
 * gives; -1 if m or n is negative or too large, or tile_n is not 0, 128 or
 * 256. */
int64_t gemm_scatter_tiles(int64_t m, int64_t n, int tile_n);

/* gemm_scatter_tune -- for tuning and testing only.  From now on every call
 * of this process (gemm_scatter_fwd, gemm_scatter_tile_m, gemm_scatter_tiles,
 * gemm_scatter_schedule) makes the 256-wide tiles tile_m rows high (256,
 * 192 or 160); 0 restores the automatic height.  Set it before the calls it
 * should affect: it is not synchronised with calls running on other
 * threads.  Returns RMSN_OK, or RMSN_ERR_SHAPE for another value (nothing is
 * changed then). */
int gemm_scatter_tune(int tile_m);

/*
 * gemm_scatter_schedule -- the tile schedule of one launch (host only, no
 * GPU needed).  For workgroup w (launch order), wg_tile[w] is the tile it
 * computes; pos_tile[s] is the tile at position s of the schedule, before
 * workgroups are spread over the GPU's eight XCDs.  A tile-row belongs to
 * the chunk of its first row.  The schedule runs the other ranks' chunks
 * first, in ring order from rank + 1, in groups of up to eight tile-rows
 * (a group may hold several chunks), then the local chunk's tile-rows;
 * within a group the tiles go column-major.  tile_n as for gemm_scatter_fwd.
 * Either array may be NULL; each holds `len` >= gemm_scatter_tiles(m, n,
 * tile_n) entries.  Returns RMSN_OK or RMSN_ERR_SHAPE.
 */
int gemm_scatter_schedule(int64_t m, int64_t n, int world, int rank, int tile_n,
                          int32_t* wg_tile, int32_t* pos_tile, int64_t len);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_SCATTER_H */
