/*
 * qgemm.h — C ABI of the weight-streaming Q4_K-style GEMM for MI355X (gfx950).
 *
 * The operation (OpenJet multi-agent serving page, section on moving the
 * weights only once): one decode step stacks the rows of every active agent
 * (each agent's next token plus two draft tokens: four agents give twelve rows)
 * into one batch and streams the quantised weights from memory once; every
 * weight read is applied to all stacked rows.  For one weight matrix:
 *
 *     y[r, n] = sum_{k=0}^{K-1} w[n, k] * x[r, k]      0 <= r < R, 0 <= n < N
 *     w[n, k] = d * sc_s * q_k - dmin * m_s             (Q4_K-style block)
 *
 * with fp32 accumulation.  A block holds 256 consecutive weights of one output
 * n: binary16 d and dmin, eight 32-wide sub-blocks s with a 6-bit scale sc_s
 * and a 6-bit min m_s, and 4-bit quants q_k.
 *
 * Canonical block bytes (144 B, the input format of qgemm_pack):
 *   [0,2) d, [2,4) dmin (binary16, little endian);
 *   [4,16) a 96-bit little-endian bit stream of sixteen 6-bit fields: sc_s at
 *          bits [6s, 6s+6), m_s at bits [48+6s, 54+6s);
 *   [16,144) quants: byte i = q_{2i} | q_{2i+1} << 4.
 * Block (n, j) covers w[n, 256j .. 256j+255] at byte 144 * (n * K/256 + j).
 *
 * The pages describe the method, not an interface: every call below is this
 * library's own.  Each call's comment opens with the passage of the method it
 * serves in brackets, or says that it is an interface of this library.
 *
 * Conventions for every call:
 *   - Device pointers are hipMalloc'd (or torch) memory of the current device;
 *     the library never frees memory it did not allocate.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls that take a
 *     stream only enqueue work and return; errors of the kernels themselves
 *     appear at the caller's next synchronisation.
 *   - Every call validates its arguments on the host before touching the GPU
 *     and returns a qgemm_status; nothing aborts.  Launch failures return
 *     QGEMM_EHIP.
 *   - Shapes: K a positive multiple of 256; N >= 1; 0 <= R <= QGEMM_MAX_R; the
 *     packed quant region of one matrix (N rounded up to 16, times K/2 bytes)
 *     must stay below 2 GiB (QGEMM_ESHAPE otherwise).
 *   - x is bf16 (bit patterns, R x K row-major), y is fp32 (R x N row-major,
 *     overwritten).  x enters the matrix cores as binary16: values with
 *     2^-17 <= |x| <= 65504 (and zero) are exact there; smaller magnitudes are
 *     rounded to a multiple of 2^-24 and larger ones are outside the supported
 *     range (they become infinities).  Sums of x over 32-wide sub-blocks (used
 *     for the min term) are kept in fp32, so every x in that range is served,
 *     whatever its neighbours.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QGEMM_MAX_R 64

typedef enum {
    QGEMM_OK = 0,
    QGEMM_EINVAL = -1,    /* null pointer, bad handle or bad flag */
    QGEMM_ESHAPE = -2,    /* K not a positive multiple of 256, N < 1, or sizes overflow */
    QGEMM_EALIGN = -3,    /* a device pointer is not 16-byte aligned */
    QGEMM_ERANGE_R = -4,  /* R < 0, R > max_R of the handle, or max_R out of 1..QGEMM_MAX_R */
    QGEMM_ENOMEM = -5,    /* the library could not allocate its workspace */
    QGEMM_EHIP = -6,      /* a HIP call or kernel launch failed */
    QGEMM_EPATH = -7,     /* requested kernel path cannot serve this R */
    QGEMM_ESCRATCH = -8   /* qgemm_run_static: the run needs more than its fixed scratch */
} qgemm_status;

/* Kernel paths (the R-dependent selection chooses between them). */
typedef enum {
    QGEMM_PATH_AUTO = 0,  /* the library's choice for (R, N, K) */
    QGEMM_PATH_VALU = 1,  /* vector-ALU bandwidth path (small R only) */
    QGEMM_PATH_MFMA = 2,  /* matrix-core streaming path (any R) */
    QGEMM_PATH_TILED = 3  /* row-tiled matrix-core path (the kernel of
                             qgemm_run_prefill, with the handle's workspace):
                             handles created with max_R >= QGEMM_TILED_MIN_R */
} qgemm_path;

/* The automatic choice takes the row-tiled path from this many rows on for
 * matrices of at least 32768 outputs, from 48 rows on for matrices of at least
 * 2^26 weights, and at QGEMM_MAX_R rows for all (the measured crossovers
 * against the streaming kernel on one MI355X). */
#define QGEMM_TILED_MIN_R 24

typedef struct qgemm_handle *qgemm_t;
typedef struct qgemm_seq *qgemm_seq_t;

/* What a run of (R, path) would launch.  The streaming kernel cuts the
 * matrix into `tiles` (groups of outputs), each needing K/256 block steps, cuts
 * the `steps` = tiles * K/256 (tile, block) steps into `ranges` equal
 * contiguous ranges and deals them round-robin to `workgroups` workgroups. */
typedef struct {
    int path;               /* QGEMM_PATH_VALU, QGEMM_PATH_MFMA or QGEMM_PATH_TILED
                               (for the row-tiled path only path, tiles (output tiles),
                               workgroups, kernels, k_chunks and workspace_bytes are set) */
    int row_tiles;          /* 16-row tiles on the matrix-core path (0 on the VALU path) */
    int subtiles_per_wave;  /* 16-output sub-tiles per wave */
    int64_t tiles;          /* output tiles */
    int64_t workgroups;     /* workgroups of the streaming kernel */
    int64_t steps;          /* (tile, block) steps in total */
    int kernels;            /* kernels enqueued by qgemm_run */
    size_t workspace_bytes; /* bytes of the handle's workspace this run may touch */
    int64_t ranges;         /* step ranges */
    int waves_per_workgroup;
    int wave_columns;       /* waves of a workgroup side by side along N; the others
                               split each step range along K */
    int whole_tile_ranges;  /* 1: each step range is whole output tiles (no partial
                               sums cross workgroups); 0: equal ranges (stream-K) */
    int k_chunks;           /* K split in this many chunks (when a tile row of
                               activations does not fit in LDS); 1: whole K */
    int min_term_sums;      /* 1: the min term dmin * sum_s m_s X_s is formed from fp32
                               sums X_s of x over each 32-wide sub-block (staged once
                               per block); 0: from the activations at every step */
} qgemm_info;

/* [Interface of this library: the pages fix no weight layout.]
 * Bytes of the packed (GPU) layout of an N x K matrix: 144 B per 256 weights
 * of N rounded up to a multiple of 16 (the canonical size plus N-tail padding).
 * Errors: QGEMM_EINVAL (bytes NULL), QGEMM_ESHAPE. */
int qgemm_packed_size(int64_t N, int64_t K, size_t *bytes);

/* [Interface of this library: the pages fix no weight layout.]
 * Rearrange canonical blocks (device, N*K/256*144 bytes, 16-byte aligned) into
 * the packed layout (device, qgemm_packed_size bytes, 16-byte aligned).  Both
 * buffers belong to the caller; canon may be freed once the stream has run the
 * work.  The packed bytes are a pure re-arrangement: no value is changed.
 * Errors: QGEMM_EINVAL, QGEMM_ESHAPE, QGEMM_EALIGN, QGEMM_EHIP. */
int qgemm_pack(const void *canon_dev, void *packed_dev, int64_t N, int64_t K, void *stream);

/* [Serves the multiply of the formula above (page: moving the weights only once).]
 * Create a handle over packed weights.  The handle BORROWS packed_dev (it must
 * stay valid and unchanged until qgemm_destroy) and OWNS a device workspace
 * sized for up to max_R rows (partial output tiles and per-tile arrival
 * counters; with max_R >= QGEMM_TILED_MIN_R also the row-tiled path's
 * activation image and K-chunk partials).  flags
 * must be 0.  Synchronous.
 * Errors: QGEMM_EINVAL, QGEMM_ESHAPE, QGEMM_EALIGN, QGEMM_ERANGE_R,
 * QGEMM_ENOMEM, QGEMM_EHIP. */
int qgemm_create(qgemm_t *out, const void *packed_dev, int64_t N, int64_t K, int max_R,
                 uint32_t flags);

/* [The multiply of the formula above: every packed weight read once and applied
 * to all R rows (page: moving the weights only once).]
 * y = x . W^T for R rows on `stream`, with the R-dependent kernel choice.
 * x: device bf16 [R x K], y: device fp32 [R x N], both 16-byte aligned.
 * On the streaming paths enqueues exactly one kernel, which reads every packed
 * weight byte once, converts x itself and writes y; on the row-tiled path
 * (large R, see QGEMM_TILED_MIN_R) two or three kernels (activation image,
 * product, and the sum of K chunks).  R = 0 is a no-op.  Runs of one handle
 * share its workspace: do not run one handle on two streams at once.
 * Errors: QGEMM_EINVAL, QGEMM_EALIGN, QGEMM_ERANGE_R, QGEMM_EHIP. */
int qgemm_run(qgemm_t h, const void *x_bf16, float *y, int R, void *stream);

/* [For callers that cannot allocate: an interface of this library around the
 * same multiply.]
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): qgemm_run
 * without a handle, allocating nothing.  packed_dev holds the packed layout of
 * an N x K matrix (qgemm_pack; borrowed for the call), x_bf16 [R x K] and y
 * [R x N] as for qgemm_run; all three 16-byte aligned; 0 <= R <= QGEMM_MAX_R.
 * Always the streaming matrix-core kernel (the row-tiled path's activation
 * image would need an allocation), with the plan qgemm_run takes on that path:
 * the same result bits.  Its partial output tiles and arrival counters live in
 * a fixed device area of QGEMM_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; a run that would need more
 * returns QGEMM_ESCRATCH (large R with stream-K partials on wide matrices).
 * Enqueues two kernels on `stream`: one that zeroes the counters the run uses,
 * then the GEMM.  Every call on one GPU shares that GPU's area: calls that
 * overlap on one GPU (two streams, or two host threads) race and give wrong
 * results.  The first call on a device reads the device's properties
 * (synchronous, no allocation).
 * Errors: QGEMM_EINVAL (NULL pointers), QGEMM_ESHAPE, QGEMM_EALIGN,
 * QGEMM_ERANGE_R, QGEMM_ESCRATCH, QGEMM_EHIP. */
#define QGEMM_STATIC_SCRATCH_BYTES (16u << 20)
int qgemm_run_static(const void *packed_dev, int64_t N, int64_t K, const void *x_bf16, float *y,
                     int R, void *stream);

/* [The same multiply; the path choice is an interface of this library.]
 * As qgemm_run with an explicit path (QGEMM_PATH_AUTO = qgemm_run).
 * Extra error: QGEMM_EPATH when the VALU path is asked for an R it does not
 * serve (R > 4), or the row-tiled path of a handle created with
 * max_R < QGEMM_TILED_MIN_R. */
int qgemm_run_path(qgemm_t h, const void *x_bf16, float *y, int R, int path, void *stream);

/* Prompt-chunk rows sharing the weight pass (OpenJet multi-agent serving page,
 * section on what the design buys: another agent's long prefill runs while the
 * others decode, so a chunk of prompt rows and the agents' decode rows go
 * through the same weights): y = x . W^T for R rows, 0 <= R <= QGEMM_MAX_PREFILL_R,
 * with a kernel that tiles rows as well as outputs (128 rows x 128 or 192 per workgroup,
 * every weight read serving a 128-row tile; bound by the matrix cores at
 * hundreds of rows).  Same operands and result as qgemm_run: x device bf16
 * [R x K], y device fp32 [R x N] (overwritten), both row-major and 16-byte
 * aligned; the same arithmetic per 256-weight block (exact binary16 products
 * of sc*q with x, fp32 sums, then d and the min term).  `workspace` (device,
 * caller-owned, 16-byte aligned, at least qgemm_prefill_workspace_size bytes)
 * receives x converted once into the kernel's LDS image (binary16 operands and
 * sub-block sums per 128-row tile and block, 1.125x the padded x in bytes)
 * and, when the row and output tiles are fewer than the GPU's compute units,
 * the partial outputs of K chunks, which a last kernel adds in chunk order: the
 * result is the same bits on every run.  Does not use the handle's workspace
 * or max_R: calls with their own workspaces may run on several streams at once.
 * Enqueues two kernels (three with K chunks) on `stream`; R = 0 is a no-op.
 * Errors: QGEMM_EINVAL (bad handle, null x or y, workspace missing or too
 * small), QGEMM_EALIGN, QGEMM_ERANGE_R (R < 0, R > QGEMM_MAX_PREFILL_R,
 * R*K*2 >= 2^31, or an activation image of 2 GiB or more), QGEMM_EHIP. */
#define QGEMM_MAX_PREFILL_R 8192
int qgemm_prefill_workspace_size(qgemm_t h, int R, size_t *bytes);
int qgemm_run_prefill(qgemm_t h, const void *x_bf16, float *y, int R, void *workspace,
                      size_t workspace_bytes, void *stream);

/* [Interface of this library: the block formula above, as a check of the packed
 * weights.]
 * The dequantised weights, fp32 [N x K] row-major (device, caller-owned,
 * 16-byte aligned): w_out[n, k] is the binary32 value nearest to
 * d*sc_s*q_k - dmin*m_s (one rounding; bit-exact), decoded from the packed
 * layout by the same unpacking the GEMM kernels use.
 * Errors: QGEMM_EINVAL, QGEMM_EALIGN, QGEMM_EHIP. */
int qgemm_dequantize(qgemm_t h, float *w_out, void *stream);

/* [The output head's next-token choice that the drafts are checked against
 * (page: from one session to four agents).]
 * idx[r] = the smallest n with y[r, n] = max over n of y[r, n], for r < R
 * (y: device fp32 [R x N]; idx: device int32 [R]).  NaN entries never win;
 * a row of NaNs gives 0.  The greedy pick over the output-head logits.
 * Errors: QGEMM_EINVAL, QGEMM_ESHAPE (N < 1), QGEMM_ERANGE_R (R < 0), QGEMM_EHIP. */
int qgemm_argmax_rows(const float *y, int R, int64_t N, int32_t *idx, void *stream);

/* [Interface of this library.]
 * Bytes of the workspace qgemm_argmax_rows_ws needs for R rows of N columns.
 * Errors: QGEMM_EINVAL (bytes NULL), QGEMM_ERANGE_R, QGEMM_ESHAPE (N < 1 or
 * N > 2^31 - 1). */
int qgemm_argmax_workspace_size(int R, int64_t N, size_t *bytes);

/* [As qgemm_argmax_rows (page: from one session to four agents).]
 * As qgemm_argmax_rows (the same result), spread over many workgroups: each
 * takes a chunk of up to 8192 columns of one row; the last chunk of a row to
 * finish combines the chunks' maxima in chunk order.  workspace: device,
 * caller-owned, at least qgemm_argmax_workspace_size bytes, 16-byte aligned,
 * zero-filled before its first use; every run leaves it ready for the next (its
 * counters back at zero).  Runs sharing a workspace must not overlap.
 * Errors: QGEMM_EINVAL, QGEMM_EALIGN, QGEMM_ERANGE_R, QGEMM_ESHAPE, QGEMM_EHIP. */
int qgemm_argmax_rows_ws(const float *y, int R, int64_t N, int32_t *idx, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Greedy verification of draft tokens (OpenJet multi-agent serving page,
 * section on moving the weights only once: each agent contributes its next token
 * and draft tokens as rows of one pass, and the drafts are checked in the same
 * round).  The R rows are R / (D + 1) agents of D + 1 consecutive rows (D =
 * drafts_per_agent): the agent's current token, then its D drafts.  argmax_idx
 * (device int32 [R]) is the row argmax of the output head; drafts (device int32
 * [agents x D], may be NULL when D = 0) the draft tokens.  Draft i stands iff it
 * equals the argmax of row i, in order, up to the first rejection.  Writes
 * n_new[a] = 1 + accepted drafts (device int32 [agents]) and tokens[a (D + 1) + j]
 * = the j-th emitted token: the argmax of row 0, then of row i + 1 for each
 * accepted draft i; -1 past n_new[a] (device int32 [agents x (D + 1)]).  One small
 * kernel on `stream`.
 * Errors: QGEMM_EINVAL (R not a multiple of D + 1, D < 0, NULL pointers),
 * QGEMM_ERANGE_R, QGEMM_EHIP. */
int qgemm_verify_greedy(const int32_t *argmax_idx, int R, const int32_t *drafts, int drafts_per_agent,
                        int32_t *tokens, int32_t *n_new, void *stream);

/* [Interface of this library.]
 * Describe the launch plan for (R, path) without running it.
 * Errors: QGEMM_EINVAL, QGEMM_ERANGE_R, QGEMM_EPATH. */
int qgemm_query(qgemm_t h, int R, int path, qgemm_info *info);

/* [Interface of this library.]
 * Free the handle and its workspace (not the packed weights).  Waits for the
 * device to finish work that may use the workspace.  NULL is a no-op. */
int qgemm_destroy(qgemm_t h);

/* ---- full weight pass -------------------------------------------------------
 * [One decode step's weight pass (page: moving the weights only once); the
 * persistent launch is the page's megakernel (section: from one session to four
 * agents).]
 * A sequence of handles run back to back in the given (dependency) order, as
 * one decode step's weight pass: layer after layer of projections and then the
 * output head, each weight byte read once.  The sequence BORROWS the handles.
 * count >= 1.  flags selects how a run is launched:
 *   0                     one streaming-kernel launch per GEMM (exactly as
 *                         qgemm_run), captured into a HIP graph on the first
 *                         run for a given (R, pointer set) and replayed after;
 *   QGEMM_SEQ_PERSISTENT  one cooperative launch for all GEMMs (below).
 * and, with QGEMM_SEQ_PERSISTENT, the form of the min term (dmin m_s X_s) up to
 * 16 rows (from 17 rows on, two or three 16-row tiles, the sums are always
 * taken: measured faster there, as the products grow with the row tiles):
 *   0                          eight more matrix-core products per weight block,
 *                              of the activation operands with the mins;
 *   QGEMM_SEQ_SUB_BLOCK_SUMS   the sub-block sums X_s of x (fp32, staged as two
 *                              binary16 parts of X_s / 256 when the activations
 *                              are staged), times the mins in one fp16 product
 *                              per block and row tile.
 * (Both give results within the stated tolerance; they round differently.)
 * and, with QGEMM_SEQ_PERSISTENT, the dependency between GEMMs:
 *   0                          GEMM i + 1 starts after GEMM i has finished on
 *                              every workgroup (its input depends on all of
 *                              the previous output, as through a norm);
 *   QGEMM_SEQ_GATED_INPUTS     where GEMM i has 2 K outputs and GEMM i + 1 has
 *                              K inputs (K a multiple of 16; a fused gate|up
 *                              feeding a down projection through an element-wise
 *                              gate), input column j of GEMM i + 1 depends only
 *                              on outputs j and K + j of GEMM i: each K chunk of
 *                              GEMM i + 1 starts once the workgroups holding
 *                              those outputs have finished GEMM i (not for two
 *                              such GEMMs in a row; on up to 256 compute units).
 *                              Results are the same as without the flag.
 * Errors: QGEMM_EINVAL (also for unknown flags), QGEMM_ENOMEM, QGEMM_ESHAPE,
 * QGEMM_EHIP. */
#define QGEMM_SEQ_PERSISTENT 1u
#define QGEMM_SEQ_SUB_BLOCK_SUMS 2u
#define QGEMM_SEQ_GATED_INPUTS 4u
int qgemm_seq_create(qgemm_seq_t *out, const qgemm_t *handles, int count, uint32_t flags);

/* [One decode step's weight pass, weights read once (page: moving the weights
 * only once); the one-launch form is the page's persistent megakernel (section:
 * from one session to four agents).]
 * Run the whole sequence for R rows: GEMM i reads xs[i] and writes ys[i]
 * (arrays of `count` device pointers, shapes as for qgemm_run); GEMM i + 1
 * starts after GEMM i has finished, as when each projection's input depends on
 * the previous output.  If argmax_idx is not NULL, the row argmax of the LAST
 * GEMM's output is written to it (device int32 [R]) by one more kernel (the
 * chunked argmax of qgemm_argmax_rows_ws, on the sequence's own workspace).
 * With QGEMM_SEQ_PERSISTENT, one cooperative launch runs all GEMMs for 1 to 48
 * rows (one to three 16-row tiles per weight step): every workgroup is
 * resident, waits at a device-wide barrier between GEMMs and already streams
 * the next GEMM's weights while it waits; the first run for a given (R,
 * pointer set) uploads a descriptor table (synchronous).  Do not
 * capture a persistent run into a graph (cooperative launch).  Runs of one
 * sequence share workspace: one stream at a time.  Without the flag, the first
 * run for a given (R, pointer set, argmax_idx) captures the launches into a
 * graph that later runs replay.  The sequence keeps at most 64 such graphs (and
 * 64 descriptor tables); a run that needs one more first waits for the device
 * and drops all of them.
 * Errors: as qgemm_run, plus QGEMM_EINVAL for NULL arrays, QGEMM_ENOMEM, and
 * QGEMM_EPATH for a persistent sequence at more than 48 rows (or a GEMM whose
 * K admits no chunking that fits the kernel's LDS). */
int qgemm_seq_run(qgemm_seq_t s, const void *const *xs, float *const *ys, int R,
                  int32_t *argmax_idx, void *stream);

/* [The step's pass with the draft check in the same round (page: from one
 * session to four agents).]
 * As qgemm_seq_run with argmax_idx, and the greedy verification of
 * qgemm_verify_greedy on that argmax in the same epilogue kernel (the last row
 * to finish its argmax runs it): the whole decode step's weight pass, head argmax
 * and draft check in one call.
 * Errors: as qgemm_seq_run and qgemm_verify_greedy. */
int qgemm_seq_run_verify(qgemm_seq_t s, const void *const *xs, float *const *ys, int R,
                         int32_t *argmax_idx, const int32_t *drafts, int drafts_per_agent,
                         int32_t *tokens, int32_t *n_new, void *stream);

/* [Interface of this library.]
 * Waits for the device, then stores in *timeouts how many barrier waits of the
 * sequence's launches since the previous call gave up (a bounded wait: a
 * workgroup that waits about a second for the others proceeds and flags it;
 * results of such a launch are not reliable).  Resets the count.
 * Errors: QGEMM_EINVAL, QGEMM_EHIP. */
int qgemm_seq_errors(qgemm_seq_t s, uint32_t *timeouts);

/* [Interface of this library.]  Free the sequence and its workspace (not the
 * handles).  NULL is a no-op. */
int qgemm_seq_destroy(qgemm_seq_t s);

/* Decode attention of the agents' step rows over their own KV caches
 * (OpenJet multi-agent serving page, section on moving the weights only once:
 * every agent reads its own KV cache, and attention grows with the agents).
 * Agent a's step has `rows` (1..4) query rows (its token and drafts) at
 * positions L_a .. L_a + rows - 1 of its sequence, L_a = lengths[a] (device
 * int32 [agents], clamped to [0, max_len]); their keys and values must already
 * be in the caches at those positions.  Row i sees positions 0 .. L_a + i.
 *   q_bf16   device bf16 [agents][rows][q_heads][head_dim]
 *   k_cache, v_cache  device bf16 [agents][kv_heads][cap][head_dim] (head-major:
 *            each head's positions contiguous)
 *   out      device fp32 [agents][rows][q_heads][head_dim], overwritten:
 *            softmax(q.k / sqrt(head_dim)) . v, query head hq reading
 *            key/value head hq / (q_heads / kv_heads)
 * head_dim must be 128 and q_heads = 8 kv_heads; cap >= max_len + rows; q and
 * the caches below 2 GiB each.  Keys and queries enter the matrix cores as
 * bf16 (exact); the weights and the values as binary16 (values above 65504 in
 * magnitude are out of range).  workspace: device, caller-owned, at least
 * qgemm_attention_workspace_size bytes, 16-byte aligned (partial results of
 * the sequence splits: each (agent, key/value head) cut into splits of a
 * multiple of 32 positions, as many in all as workgroups stay resident in one
 * round, 256).  Two kernels on `stream`.
 * Errors: QGEMM_EINVAL, QGEMM_ESHAPE, QGEMM_EALIGN, QGEMM_EHIP. */
int qgemm_attention_workspace_size(int agents, int rows, int kv_heads, int max_len, size_t *bytes);
int qgemm_decode_attention(const void *q_bf16, const void *k_cache, const void *v_cache,
                           const int32_t *lengths, int agents, int rows, int q_heads, int kv_heads,
                           int head_dim, int cap, int max_len, float *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Measurement aid (an interface of this library, not a step the pages
 * describe): read `bytes` of device memory at `buf` once, as fast as the device
 * allows, so that a caller can time the practical HBM read ceiling next to the
 * weight pass.  One workgroup per compute unit, 16-byte nontemporal loads,
 * four in flight per thread.  buf: device, 16-byte aligned; bytes: a multiple
 * of 16, below 2^40.  sink: 16 KiB of device memory the kernel may write
 * (contents unspecified).  One kernel on `stream`.
 * Errors: QGEMM_EINVAL (NULL pointer, bytes not a multiple of 16 or too
 * large), QGEMM_EALIGN, QGEMM_EHIP. */
int qgemm_read_probe(const void *buf, uint64_t bytes, void *sink, void *stream);

/* [Interface of this library.]  Static text for a status code. */
const char *qgemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
