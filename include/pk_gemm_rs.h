/*
 * pk_gemm_rs.h -- C ABI of libpk_gemm_rs.so: one GPU's share of a tile-fused
 * bf16 GEMM + reduce-scatter on MI355X (gfx950).
 *
 * The operation ("ParallelKittens: Systematic and Practical Simplification of
 * Multi-GPU AI Kernels", section 3 "Scheduling Analysis", the fused GEMM +
 * reduce-scatter example; "ParallelKittens: Three Principles and Eight
 * Primitives for Multi-GPU Kernels", section 3 "Principle 2"): P tensor-
 * parallel ranks each hold A_p (M x K) and B_p (K x N); the result is
 * C = sum_p A_p * B_p and rank r keeps row shard r, rows [r*S, (r+1)*S) with
 * S = M / P.  This library runs rank `rank`'s part on one GPU:
 *
 *   C_loc = A * B                      bf16 inputs, fp32 accumulation (MFMA)
 *   for every other rank d: send slot j(d) <- bf16(C_loc rows of shard d)
 *       and, per chunk of `chunk_rows` rows, a ready word raised by one once
 *       every tile of the chunk is stored (the pages' signal primitive,
 *       "The Eight PK Primitives": signal adds to a counter, wait waits for
 *       it to reach a value; chunks as in "Syncopate: Efficient Multi-GPU AI
 *       Kernels via Automatic Chunk-Centric Compute-Communication Overlap",
 *       section 5.1);
 *   out <- sum_j peer_partials[j] + C_loc rows of shard `rank`   (fp32: the
 *       peers added in ascending slot order starting from +0, then the
 *       local partial), stored once.
 *
 * The peers' partials are already staged in device memory (what the other
 * ranks sent to this one); nothing here talks to another GPU.
 *
 * Conventions for every entry point below:
 *  - All matrices are dense row-major with no padding.  A: bf16 [M][K];
 *    B: bf16 [K][N]; peer_partials and send_bufs: bf16 [P-1][S][N]; out:
 *    fp32 or bf16 [S][N].  Slot j of peer_partials / send_bufs belongs to rank
 *    j if j < rank, else rank j+1 (ascending ranks, skipping `rank`).
 *  - flags: uint32 [pk_flags_words(P, M, chunk_rows)] = 33*(P-1)*C words:
 *    first (P-1)*C ready words (slot-major, C = S / chunk_rows chunks per
 *    slot), then the arrival counters, one per 128-byte line (counter i at
 *    word (P-1)*C + 32*i, the 31 words after it unused).  Counters (and the
 *    unused words) must be zero at launch, and are zero again when the stream
 *    reaches the end of the call.  Each call adds exactly 1
 *    to every ready word (wrapping at 2^32), whatever the tile
 *    configuration or tile order: zero the buffer once, and the n-th call on
 *    it leaves every ready word at n, so a consumer of that call waits for
 *    n.  Nothing needs to be cleared between calls.
 *  - A chunk's send rows are written through the L2 to memory and have
 *    completed before its ready word rises (an atomic add with device-scope
 *    release), so a reader on this GPU that sees the word with a
 *    device-scope acquire then reads the chunk's data.
 *  - Pointers are device pointers owned by the caller, 16-byte aligned; the
 *    output buffers (send_bufs, out, flags) must not overlap each other or
 *    the inputs.  Unused pointers may be NULL: peer_partials, send_bufs and
 *    flags when P == 1, everything when M == 0 or N == 0.
 *  - Shapes: M % P == 0, N % 8 == 0, K % 8 == 0 (16-byte rows), chunk_rows
 *    divides S, 1 <= P <= 64, 0 <= rank < P.  Ragged tiles are handled.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Calls are
 *    asynchronous: they return after the launch; no host synchronisation,
 *    no device allocation.  Arguments are validated before any HIP call.
 *  - Return value: PK_OK or a negative PK_ERR_* code; no exception crosses
 *    the ABI.  pk_strerror() names the code.
 *  - Two calls that overlap in time must not share output buffers or flags.
 */
#ifndef PK_GEMM_RS_H
#define PK_GEMM_RS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PK_OK 0
#define PK_ERR_POINTER (-1)     /* required pointer NULL or not 16-byte aligned */
#define PK_ERR_SHAPE (-2)       /* M % P, N % 8, K % 8, chunk_rows, negative sizes */
#define PK_ERR_RANK (-3)        /* P < 1, P > 64, rank outside [0, P) */
#define PK_ERR_TILE_ORDER (-4)  /* tile_order not 0, 1 or 2 */
#define PK_ERR_CONFIG (-5)      /* requested tile configuration does not exist */
#define PK_ERR_LAUNCH (-6)      /* the HIP runtime refused the launch */
#define PK_ERR_TOO_LARGE (-7)   /* a buffer exceeds the 32-bit element offsets used */
#define PK_ERR_SCRATCH (-8)     /* the shape needs more than the static workspace holds */

#define PK_TILE_ROW_MAJOR 0       /* shards 0..P-1 in order, chunk-major inside */
#define PK_TILE_OWNED_FIRST 1     /* owned shard, then rank+1, rank+2, ... (mod P) */
#define PK_TILE_DEST_ROUND_ROBIN 2 /* one tile per destination in turn, owned last */

/* The fused share with an fp32 `out` (fp32 [S][N]).  See the conventions
 * above.  tile_order: PK_TILE_*; it changes the order work is done in, never
 * a bit of any output. */
int pk_gemm_rs_local(const void* A, const void* B, const void* peer_partials,
                     void* send_bufs, void* out, uint32_t* flags,
                     int64_t M, int64_t N, int64_t K, int P, int rank,
                     int chunk_rows, int tile_order, void* stream);

/* Same as pk_gemm_rs_local with a bf16 `out` (bf16 [S][N], the fp32 sum
 * rounded to nearest even once). */
int pk_gemm_rs_local_bf16out(const void* A, const void* B, const void* peer_partials,
                             void* send_bufs, void* out, uint32_t* flags,
                             int64_t M, int64_t N, int64_t K, int P, int rank,
                             int chunk_rows, int tile_order, void* stream);

/* Tuning knobs for pk_gemm_rs_local_ex.  Zero in any field means "library
 * default".  Schedule knobs follow Syncopate section 5.3 (chunk size, tile
 * configuration and tile order are searched by measurement). */
typedef struct pk_options {
  int config;           /* tile configuration id (pk_config_info), 0 = auto */
  int max_workgroups;   /* cap on the persistent grid, 0 = fill the device */
  int group_n;          /* column tiles per locality group inside a shard; 0 = auto: 32 for
                           dest-round-robin, 8 for the other orders (at most the tile columns) */
  int gemm_only;        /* 1: store bf16(A*B) for all M rows into `out` (bf16 [M][N]);
                           no send, peers or flags.  The standalone-GEMM reference
                           the fused kernel is measured against. */
  int owned_split;      /* owned shard tiled finer than the send shards, so its
                           epilogue (P-1 peer reads per element) spreads over many
                           workgroups: 1 on, -1 off, 0 = auto (on when the walk has
                           fewer than two whole tiles per CU).  Tile configuration 1
                           with P in {2, 4, 8} (at P = 8, when the work fits one
                           round and S is a multiple of 32, as gathered rows:
                           pk_gather_rows), and configuration 6 (two workgroups
                           per CU) at P = 8 when every owned sub-tile and send tile
                           fits one grid of two workgroups per CU; elsewhere it
                           stays off, except that configuration 6 with 1 where its
                           schedule does not fit is PK_ERR_CONFIG. */
  int signal_batch;     /* finished send tiles of a workgroup whose chunk arrivals
                           share one device-scope release, 0 = auto (8).  Larger
                           batches cost fewer cache writebacks and raise ready words
                           later; the last batch of a workgroup is always flushed. */
  uint64_t* ready_clock; /* NULL, or uint64 [P-1][S/chunk_rows] (8-byte aligned): for
                           each chunk, the 100 MHz device clock when its ready word
                           rose in this call (timing of the chunk consumer only). */
  int store_policy;     /* cache policy of the output stores (send chunks, out, the
                           reduction workspace), all written through to memory:
                           1 streaming (non-temporal hint), 2 without the hint,
                           0 = auto (streaming when the call stores more than
                           64 MiB).  Results never depend on it. */
  uint64_t* timeline;   /* NULL, or uint64 [2048][32] (8-byte aligned): read only by the
                           instrumented timing build of this library
                           (libpk_gemm_rs_timeline.so, compiled with PK_TIMELINE),
                           which records per workgroup its CU placement and the
                           device clock at each phase boundary; the launch must
                           then have at most 2048 workgroups (else PK_ERR_CONFIG).
                           Results never depend on it. */
} pk_options;

/* The fused share with explicit options; out_bf16 selects bf16 (1) or fp32 (0)
 * `out`.  With opts->gemm_only the call is a plain GEMM (see pk_options). */
int pk_gemm_rs_local_ex(const void* A, const void* B, const void* peer_partials,
                        void* send_bufs, void* out, uint32_t* flags,
                        int64_t M, int64_t N, int64_t K, int P, int rank,
                        int chunk_rows, int tile_order, int out_bf16,
                        const pk_options* opts, void* stream);

/* Atomic push variant: the pages' own epilogue ("The Eight PK Primitives" of
 * the ParallelKittens summary page: store_add_async adds a tile atomically
 * into a peer's buffer; section 3 "Scheduling Analysis" sends every output
 * tile to its owner that way).  Every tile of this rank's partial
 * C_loc = A * B is added, element by element with fp32 atomic adds, into the
 * accumulator of the rank that owns its rows:
 *   accum[d] += C_loc rows of shard d      for every d in 0..P-1 (own shard too)
 * accum: fp32 [P][S][N], 16-byte aligned: accum[d] stands for rank d's
 * accumulator (on one GPU, a local buffer); what it holds before the call
 * (other ranks' contributions, or zeros) is what the adds land on.  Each
 * element receives one add per call, so the result is fl32(before + C_loc)
 * whatever the tile order.  Ready words as for pk_gemm_rs_local: for the P-1
 * other owners, a chunk's word rises by one once this rank's adds into it
 * are complete and visible at device scope.  No peer partials, no send
 * buffers.  opts: config, max_workgroups, group_n, signal_batch and
 * ready_clock apply; gemm_only and owned_split = 1 are PK_ERR_CONFIG. */
int pk_gemm_rs_push(const void* A, const void* B, float* accum, uint32_t* flags,
                    int64_t M, int64_t N, int64_t K, int P, int rank,
                    int chunk_rows, int tile_order, const pk_options* opts, void* stream);

/* Inter-CU schedule (the pages' alternative to the fused epilogue: in the
 * ParallelKittens summary page, compute workers produce tiles while
 * dedicated communication workers move them, with "num_comm_sms" tuned per
 * size; Syncopate section 5.2 backends (4)-(5), load/store on a specialized
 * SM).  One launch does what pk_gemm_rs_local_ex does (same send_bufs, out
 * and flags, bit for bit) and, on num_comm_cus dedicated workgroups (rounded
 * up to a multiple of 8, one XCD round), moves every send chunk into `dest`
 * as soon as its ready word reaches `expected` (the value this call raises
 * it to: n for the n-th call on a zeroed flags buffer), as pk_rs_consume
 * does: dest bf16 [P-1][S][N], status int32 [P-1][S/chunk_rows] (0 moved,
 * 1 gave up after spin_limit polls).  The compute grid shrinks by those
 * workgroups so that all of them are resident at once.  P >= 2; opts as
 * for pk_gemm_rs_local_ex except gemm_only.
 * Co-residency: the communicators wait for chunks that compute workgroups of
 * the same launch produce, so the move completes only when the whole grid is
 * resident together (the grid is sized for an otherwise idle device).  On a
 * device shared with other work a communicator may give up: send_bufs, out
 * and flags are still right, but `dest` rows are valid only for chunks whose
 * status is 0; read the status words after the stream has reached the end
 * of the call. */
int pk_gemm_rs_intercu(const void* A, const void* B, const void* peer_partials,
                       void* send_bufs, void* out, uint32_t* flags, void* dest,
                       int32_t* status, int64_t M, int64_t N, int64_t K, int P, int rank,
                       int chunk_rows, int tile_order, int out_bf16, uint32_t expected,
                       int num_comm_cus, int spin_limit, const pk_options* opts,
                       void* stream);

/* Inter-CU schedule, reduction role: dedicated workgroups do the owned
 * shard's reduction while the rest compute (ParallelKittens summary page,
 * "Scheduling Analysis": inter-SM overlapping gives whole SMs to
 * communication, with "num_comm_sms" tuned per size as in Figure 5; the
 * owner-side sum of the staged partials is the reading of the owned-shard
 * step documented for pk_gemm_rs_local).  One launch leaves send_bufs, out
 * and flags exactly as pk_gemm_rs_local_ex does, bit for bit, split as:
 *  - num_comm_cus workgroups (rounded up to a multiple of 8, one XCD round)
 *    sum the staged peer partials of the owned shard, in ascending slot order
 *    from +0 in fp32, into `presum` (fp32 [S][N], 16-byte aligned): the
 *    value the fused epilogue adds the local partial to;
 *  - the other workgroups run the share; an owned item waits for the
 *    pieces of presum it covers, then stores out = presum + C_own.
 * presum may be `out` itself when out is fp32 and num_comm_cus > 0 (each
 * element is read, then written, by one thread); with a bf16 out or in the
 * background mode (num_comm_cus = 0) it must be a separate buffer
 * (PK_ERR_POINTER).
 * piece_ready: uint32 [ceil(S/64)][ceil(N/64)] (pk_reduce_piece_words),
 * 4-byte aligned, zeroed once: the word of the 64 x 64 piece at rows
 * [64r, 64r+64), columns [64c, 64c+64) of the owned shard rises by one per
 * call once its sums are visible at device scope; compute workgroups wait
 * for it to reach `expected` (n for the n-th call on a zeroed buffer; signed
 * 32-bit distance).  peer_ready: NULL (the peer partials are already staged)
 * or uint32 [P-1][S/chunk_rows], the ready words of the incoming chunks by
 * slot: a reduction workgroup first waits for the words of every chunk its
 * rows touch to reach `expected`, as the owner does in a multi-GPU run.
 * Every wait polls at most spin_limit >= 1 times, so a missing producer
 * ends the kernel instead of hanging it.  A wait that gives up ORs a bit into
 * *error (int32, device memory, zeroed by the caller): 2 for an incoming chunk
 * word (the rows are summed as they are), 1 for a piece word (the owned item
 * then sums its staged peer partials itself, in the same order, so `out` is
 * unchanged).  The compute grid shrinks by the reduction workgroups so that
 * every workgroup is resident at once.
 * Co-residency: piece words are raised by other workgroups of the same
 * launch, so the split of work pays off only when the whole grid is resident
 * together (the grid is sized for an otherwise idle device).  Results are
 * valid when *error reads 0 after the stream has reached the end of the call;
 * with error bit 1 alone and presum a separate buffer they are valid too.
 * With presum == out a reduction workgroup that ran late may have stored its
 * bare peer sum over the owned shard, so then any nonzero error word means
 * `out` must not be used.
 * num_comm_cus = 0: no dedicated workgroups; the reduction runs in the
 * background of the main loops instead (the pages' intra-SM overlap applied
 * to the owner-side sum).  Every whole tile gets its own workgroup.  While a
 * send tile or an owned tile is multiplied, its workgroup sums the peer
 * partials of one 64 x 128 eighth of an owned tile (each owned tile's last
 * eighth by its own workgroup, the other seven by send tiles' workgroups),
 * stores the sums into presum and raises their pieces.  It then sends its
 * tile, or, for an owned tile, waits for the tile's pieces and stores
 * out = presum + C_own.  Same outputs, piece words and error rules as
 * above.  It needs P = 8, tile configuration 1 with the owned split (not
 * turned off by opts), and a grid that holds every tile at once
 * (8 * ceil(S/256) * ceil(N/256) workgroups); otherwise PK_ERR_CONFIG.
 * P >= 2; opts as for pk_gemm_rs_local_ex except gemm_only.  Returns PK_OK
 * or PK_ERR_* (arguments checked before any HIP call). */
int pk_gemm_rs_intercu_reduce(const void* A, const void* B, const void* peer_partials,
                              const uint32_t* peer_ready, void* send_bufs, void* out,
                              uint32_t* flags, float* presum, uint32_t* piece_ready,
                              int32_t* error, int64_t M, int64_t N, int64_t K, int P, int rank,
                              int chunk_rows, int tile_order, int out_bf16, uint32_t expected,
                              int num_comm_cus, int spin_limit, const pk_options* opts,
                              void* stream);

/* Number of piece words pk_gemm_rs_intercu_reduce reads and raises:
 * ceil((M/P)/64) * ceil(N/64), or a negative PK_ERR_* code. */
int64_t pk_reduce_piece_words(int64_t M, int64_t N, int P);

/* pk_gemm_rs_intercu_reduce without a caller-provided workspace, for callers
 * that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid it): the fp32 peer sum and the piece
 * words live in a static array of this library, one copy per GPU held until
 * the process ends (pk_static_workspace_limits gives its size).  Arguments,
 * outputs, error bits and the background mode (num_comm_cus = 0) are those
 * of pk_gemm_rs_intercu_reduce, with presum a separate buffer; `expected`
 * applies to the incoming chunk words (peer_ready) only, the piece words are
 * cleared by each call and raised once.  The call allocates nothing: it runs
 * a small fill kernel and the fused kernel on `stream`.  Shapes with
 * (M/P) * N above max_sum_elements or more piece words than max_piece_words
 * return PK_ERR_SCRATCH.  Every call on one GPU uses the same workspace: two
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and their results are undefined; calls in one stream are ordered and safe. */
int pk_gemm_rs_intercu_reduce_static(const void* A, const void* B, const void* peer_partials,
                                     const uint32_t* peer_ready, void* send_bufs, void* out,
                                     uint32_t* flags, int32_t* error, int64_t M, int64_t N,
                                     int64_t K, int P, int rank, int chunk_rows, int tile_order,
                                     int out_bf16, uint32_t expected, int num_comm_cus,
                                     int spin_limit, const pk_options* opts, void* stream);

/* Capacity of the static workspace of pk_gemm_rs_intercu_reduce_static:
 * writes the largest (M/P) * N and piece-word count it accepts (either
 * pointer may be NULL) and returns the workspace's size in bytes per GPU. */
int64_t pk_static_workspace_limits(int64_t* max_sum_elements, int64_t* max_piece_words);

/* All-gather + GEMM, the step before the reduce-scatter in a tensor-
 * parallel MLP (ParallelKittens summary page, "Data and Tensor Parallelism:
 * AG+GEMM, GEMM+RS, and GEMM+AR": local shape N x N/8 x N; Syncopate's
 * AG-GEMM).  Rank p holds rows [p*S, (p+1)*S) of A (S = M/P); the others'
 * rows arrive chunk by chunk into the gathered buffer:
 *   C = A * B,  A: bf16 [M][K] (gathered; this rank's rows already in place),
 *   B: bf16 [K][N] (this rank's columns), C: bf16 [M][N] (fp32 accumulation,
 *   rounded to nearest even once).
 * a_ready: uint32 [P][S/chunk_rows]; word (p, c) counts the arrivals of rows
 * [c*chunk_rows, (c+1)*chunk_rows) of rank p's shard (this rank's words are
 * not read).  Before a tile of rank p's rows reads A it waits (the pages'
 * wait primitive) until every chunk word its rows touch has reached
 * `expected` (signed 32-bit distance, so counts may wrap), polling each at
 * most spin_limit >= 1 times, then acquires at device scope.  A wait that
 * gives up sets *error to 1 (int32, device memory; the caller zeroes it) and
 * the tile is computed from whatever the rows hold.  tile_order as for the
 * fused share: PK_TILE_OWNED_FIRST multiplies this rank's own rows first,
 * then ranks rank+1, rank+2, ... in ring order.  opts: config,
 * max_workgroups and group_n apply (leave CUs to whatever produces the
 * chunks if it runs on the same GPU). */
int pk_ag_gemm(const void* A, const uint32_t* a_ready, const void* B, void* C, int32_t* error,
               int64_t M, int64_t N, int64_t K, int P, int rank, int chunk_rows,
               uint32_t expected, int spin_limit, int tile_order, const pk_options* opts,
               void* stream);

/* Chunk consumer: the transfer half of the reduce-scatter, the step after
 * the fused share ("The Eight PK Primitives" of the ParallelKittens summary
 * page: wait spins on a counter until it reaches an expected value; chunks
 * as in Syncopate section 5.1, moved as one unit once their tiles are
 * stored).  For every send slot j and chunk c (slot-major order, the order
 * the row-major walk completes them) it waits until the chunk's ready word
 * reaches `expected` (compared as a signed 32-bit distance, so counts may
 * wrap), acquires at device scope, and copies rows [c*chunk_rows,
 * (c+1)*chunk_rows) of send_bufs[j] into dest[j]: the staging buffer of the
 * rank that owns those rows in a multi-GPU run.
 *  - flags: the producer's flags buffer (ready words read, nothing written).
 *  - send_bufs, dest: bf16 [P-1][S][N], 16-byte aligned, not overlapping.
 *  - expected: the ready value of the producer call to consume (n for the
 *    n-th call on a zeroed flags buffer).
 *  - spin_limit >= 1: polls of one ready word (about 1-2 us apart) before
 *    the chunk is given up: then its status is 1 and its dest rows are not
 *    touched, so a producer that never signals cannot hang the consumer.
 *  - status: int32 [P-1][S/chunk_rows], per chunk 0 (copied) or 1 (timed out).
 *  - observed: NULL or uint64 [P-1][S/chunk_rows]: the 100 MHz device clock
 *    when the chunk's ready word was seen (0 on time-out).
 *  - max_workgroups: consumer workgroups, 0 = min(32, chunks).
 * It may run on another stream while the producer runs; the producer's
 * workgroups take a whole CU each, so leave the consumer CUs
 * (pk_options.max_workgroups) or it starts only as producer workgroups end.
 * Asynchronous; returns PK_OK or PK_ERR_* (arguments checked before any HIP
 * call). */
int pk_rs_consume(const uint32_t* flags, const void* send_bufs, void* dest,
                  int64_t M, int64_t N, int P, int chunk_rows, uint32_t expected,
                  int spin_limit, int32_t* status, uint64_t* observed,
                  int max_workgroups, void* stream);

/* Number of uint32 flag words for (P, M, chunk_rows): 2*(P-1)*(M/P)/chunk_rows,
 * or a negative PK_ERR_* code for invalid arguments. */
int64_t pk_flags_words(int P, int64_t M, int chunk_rows);

/* Argument check of pk_gemm_rs_local_ex without any HIP call (host only). */
int pk_validate(const void* A, const void* B, const void* peer_partials,
                const void* send_bufs, const void* out, const uint32_t* flags,
                int64_t M, int64_t N, int64_t K, int P, int rank,
                int chunk_rows, int tile_order, int out_bf16, const pk_options* opts);

/* Static description of tile configuration `id` (1..pk_config_count()):
 * block tile BM x BN x BK, wave tile WM x WN, threads per workgroup.
 * Returns PK_OK or PK_ERR_CONFIG. */
int pk_config_count(void);
int pk_config_info(int id, int* BM, int* BN, int* BK, int* WM, int* WN, int* threads);

/* Configuration id the library picks for a shape when opts->config == 0. */
int pk_select_config(int64_t M, int64_t N, int64_t K, int P);

/* Host copy of the work walk (host only): writes, for each of the first
 * min(cap, total) work items in the order they are handed out, (shard, row
 * tile, column tile, sub-tile) into out4[4*i .. 4*i+3]; sub-tile is -1 for a
 * whole tile and 0..R-1 for the R sub-tiles of an owned tile under the owned
 * split (owned_split = 1; configurations 1 and 6), where the walk is a list of
 * pairs, each send tile followed by the owned sub-tile that rides with it.
 * When the split's pairs fit in one round of the grid at P = 8 and S is a
 * multiple of 32, the kernel runs the gathered-row schedule instead
 * (pk_gather_rows); otherwise, in one round, it hands the sub-tiles of every
 * fourth pair (pairs 0, 4, 8, ...) to the workgroups that hold no send tile,
 * and those pairs' workgroups only send; the list is the same.  Configuration 6 hands send tile j to workgroup j of
 * the first half of its grid and owned sub-tile j, then send tile half + j,
 * to workgroup j of the second half.  Returns the total number of work items or a
 * negative code.  group_n as in
 * pk_options (0 = auto for this config). */
int64_t pk_tile_walk(int64_t M, int64_t N, int P, int rank, int config, int tile_order,
                     int group_n, int owned_split, int32_t* out4, int64_t cap);

/* Arrival count chunk c of every slot waits for, under configuration `config`
 * with whole tiles or the owned split's sub-tiles (not the gathered rows). */
int64_t pk_chunk_arrivals(int64_t M, int64_t N, int P, int chunk_rows, int config, int c);

/* Gathered-row schedule (host-only description).  The fused share runs it in
 * place of the owned split's sub-tiles when configuration 1 takes the owned
 * split at P = 8, S = M/P is a multiple of 32, the grid holds a workgroup for
 * every work item, there are no communicator workgroups and M*K*2 <= 2^31.
 * The M rows are cut into S/32 row groups of 256: group g holds send rows
 * 224g .. 224g+223 (the P-1 send shards' rows one after another in slot
 * order) and owned rows 32g .. 32g+31, and work item (g, u) multiplies them
 * by column tile u ((S/32) x ceil(N/256) items), so every work item stores
 * send rows and a slice of the owned shard (whose peer partials it sums while
 * it multiplies) and no workgroup holds a whole owned tile.  The sums, their
 * order and so every output bit are those of the other schedules; the ready
 * words rise once per call as there, after a different number of arrivals.
 * pk_gather_rows writes the rows of A that tile rows 0..255 of group g read
 * into rows[256]; pk_gather_arrivals writes, for chunk c of send slot d (index
 * d*(S/chunk_rows) + c), the arrivals the chunk waits for into expected[] and
 * the arrivals the work items make into made[] (both (P-1)*(S/chunk_rows)).
 * PK_ERR_CONFIG when (P, S) does not fit the schedule. */
int pk_gather_rows(int P, int rank, int64_t M, int g, int64_t* rows);
int pk_gather_arrivals(int64_t M, int64_t N, int P, int chunk_rows, uint32_t* expected,
                       uint32_t* made);

/* Human-readable name of a return code. */
const char* pk_strerror(int code);

/* Library version, 100*major + minor. */
int pk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PK_GEMM_RS_H */
