/*
 * lora_sgmv.h -- C ABI of the MI355X (gfx950) multi-adapter LoRA library.
 *
 * One call applies many LoRA adapters to one token batch. Token t, grouped
 * into a segment whose adapter is i (rank r_i, scale s_i), gets
 *
 *     u_t = A_i x_t            "shrink" to rank r_i        A_i: [r_i, h_in]
 *     y_t = y_t + s_i B_i u_t  "expand" back to h_out      B_i: [h_out, r_i]
 *
 * for all adapters of the batch in one kernel launch ("Trajectory presenta C-LoRA" (vivodigitale.it),
 * "Come funziona l'architettura": a decode batch mixes tokens of different
 * resident adapters and the per-adapter matrix-vector work is fused into a
 * single launch). The packed-training backward ("Technische Samenvatting: PLoRA" (gist.science), "LoRA
 * Execution Engine", packed kernels over concatenated adapter tensors, tiled
 * along the sequence or hidden dimension rather than the small rank) gives
 *
 *     du_t = s_i B_i^T dy_t,   dx_t += A_i^T du_t,
 *     dB_i = s_i sum_t dy_t u_t^T,   dA_i = sum_t du_t x_t^T   (fp32).
 *
 * Types: x, y, dy, dx, A_i, B_i are bfloat16 (raw 16-bit patterns); u, du,
 * dA_i, dB_i are float32. Accumulation is in float32; bf16 outputs are
 * rounded to nearest even.
 *
 * Conventions shared by every entry point
 *  - Memory: every buffer is owned by the caller. The library allocates no
 *    device memory. "DEVICE" pointers are GPU addresses, "HOST" pointers are
 *    read during the call only and may be freed when it returns. Device
 *    buffers must stay alive until the work queued on `stream` has finished.
 *  - Layout: row-major. x rows have stride ldx elements, y rows ldy, u rows
 *    ldu. Row strides and the base addresses of x, y, dx, dy and of every
 *    A_i, B_i must be multiples of 16 bytes (8 bf16 elements); h_in and
 *    h_out must be multiples of 8; u needs 4-byte alignment.
 *  - Token order: the kernels walk tokens in "sorted position" order,
 *    p = 0..T-1, in which every segment is a contiguous run. With
 *    no row table, sorted position p is row p of x/y/dx/dy. With a
 *    token_rows table (or its host copy token_rows_host, see
 *    lora_segments_t), position p reads and writes row token_rows[p] of
 *    x/y/dx/dy (an in-kernel gather/scatter, so a request-order batch need
 *    not be permuted by the caller). u and du always use sorted positions.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream). Calls only
 *    enqueue work and never synchronise the device. Calls must not be
 *    captured into a HIP graph (each launch carries a fresh hand-off id in
 *    its kernel argument, which a replayed graph would repeat), except
 *    lora_sgmv_fused_graph(), which takes its id from the device.
 *  - Workspace: size it with lora_workspace_size(). It must be filled with
 *    zero bytes once before its first use; every call returns its counters
 *    to zero when its work completes. The hand-off stamps a call leaves in
 *    it carry that call's unique 56-bit id, so no later call can take them
 *    for its own. Calls that share a workspace must be ordered (same stream,
 *    or synchronised): concurrent calls on one workspace race.
 *  - Errors: every entry point returns a lora_status_t and never aborts.
 *    All metadata checks run on the HOST mirrors before any HIP call, so a
 *    rejected call has touched no device state. A failed HIP call returns
 *    LORA_DEVICE_ERROR. lora_last_error() gives a readable reason for the
 *    last failure on the calling thread. Device faults surface at the
 *    caller's next synchronisation.
 *  - Segments with adapter id -1, with a rank-0 adapter, or with no tokens
 *    produce no work: their rows of y/dx/u/du are never written.
 */
#ifndef LORA_SGMV_H
#define LORA_SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LORA_OK = 0,
  LORA_INVALID_ARGUMENT = 1,    /* malformed metadata, pointer or size */
  LORA_UNSUPPORTED = 2,         /* valid request outside what this build does (e.g. rank > 128) */
  LORA_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below lora_workspace_size() */
  LORA_DEVICE_ERROR = 4         /* a HIP runtime call failed; see lora_last_error() */
} lora_status_t;

/* Operation codes for lora_workspace_size(). */
enum { LORA_OP_SHRINK = 0, LORA_OP_EXPAND = 1, LORA_OP_FUSED = 2, LORA_OP_BACKWARD = 3 };

/* Flags for lora_packed_backward(). */
#define LORA_GRAD_ACCUMULATE 1u /* add into dA_i / dB_i instead of overwriting them */

/* Largest supported adapter rank. */
#define LORA_MAX_RANK 128

/*
 * The adapters resident on the GPU (all of them reachable from one launch:
 * "Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona l'architettura", every adapter loaded
 * in GPU memory). Pointer tables are read on the device at every call, so
 * weights can be updated in place, or re-pointed, between calls without any
 * other call (same rank).
 *
 * A_ptrs_host / B_ptrs_host are optional HOST copies of the two tables. When
 * both are given, forward launches of up to 16 segments carry the weight
 * addresses in their launch arguments instead of reading the device tables
 * (one dependent memory round trip less at the start of every workgroup,
 * which matters for decode-sized batches). They must then hold the same
 * addresses as the device tables at the time of the call; the library only
 * reads them during the call. NULL (either one): the device tables are used.
 */
typedef struct lora_adapters_t {
  int32_t num_adapters;   /* N >= 1 */
  int32_t h_in;           /* input width (multiple of 8) */
  int32_t h_out;          /* output width (multiple of 8) */
  const uint64_t* A_ptrs; /* DEVICE [N]: address of bf16 A_i [r_i, h_in]; may be 0 if r_i == 0 */
  const uint64_t* B_ptrs; /* DEVICE [N]: address of bf16 B_i [h_out, r_i]; may be 0 if r_i == 0 */
  const int32_t* ranks;   /* HOST [N]: r_i in [0, 128] */
  const float* scales;    /* HOST [N]: s_i, finite */
  const uint64_t* A_ptrs_host; /* HOST [N] or NULL: same entries as A_ptrs */
  const uint64_t* B_ptrs_host; /* HOST [N] or NULL: same entries as B_ptrs */
} lora_adapters_t;

/*
 * A token batch in sorted-position order, cut into segments that each use
 * one adapter (a segment is a run of positions [seg_starts[g],
 * seg_starts[g+1])). Several segments may use the same adapter (packed
 * sequences, "Technische Samenvatting: PLoRA" (gist.science) "Kernelontwerp"); their tokens are summed
 * together in dA_i / dB_i.
 */
typedef struct lora_segments_t {
  int32_t num_tokens;         /* T >= 0 */
  int32_t num_segments;       /* S >= 0 */
  const int32_t* seg_starts;  /* HOST [S+1]: [0] = 0, non-decreasing, [S] = T */
  const int32_t* seg_adapter; /* HOST [S]: -1 (no adapter) or 0..N-1 */
  const int32_t* token_rows;  /* DEVICE [T] or NULL: row of x/y/dx/dy used by position p.
                                 Rows must be distinct for the writing calls. With a
                                 table, every matrix the call touches is addressed
                                 through one 2 GiB - 16 byte window from its base:
                                 the call is refused (LORA_INVALID_ARGUMENT) when
                                 T rows of its stride cannot fit in the window, and
                                 a row that is negative or does not lie wholly
                                 inside it is treated as absent (it reads as zero
                                 and is never written; the offset is computed in
                                 64 bits, so it cannot wrap onto another row). */
  const int32_t* token_rows_host; /* HOST [T] or NULL: the same rows as token_rows (the
                                 same rules apply). A forward launch of at most 16
                                 segments over at most 256 tokens then carries the
                                 rows in its launch arguments and reads no device
                                 table, so a request-order decode batch needs no
                                 upload of its rows: token_rows may be NULL for
                                 lora_sgmv_shrink, _expand, _fused, _fused_multi and
                                 _fused_noalloc calls of that size (larger ones are
                                 refused with LORA_INVALID_ARGUMENT).
                                 lora_packed_backward always needs token_rows. The
                                 library only reads the copy during the call. */
} lora_segments_t;

/*
 * Token bookkeeping for a mixed-adapter batch. A decode batch arrives with
 * the tokens of many tenants' adapters interleaved in request order
 * ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona
 * l'architettura": one batch mixes tokens of different adapters); the
 * segmented kernels want each adapter's tokens as one contiguous run.
 * Groups request-order adapter ids into segments (HOST only, no GPU):
 * segment a (0 <= a < N) holds the tokens with id a in request order, and a
 * final segment N holds the tokens with id -1. perm[p] is the request index
 * of sorted position p (usable as token_rows). Output sizes: perm [T],
 * seg_starts [N+2], seg_adapter [N+1] (seg_adapter[a] = a, last = -1).
 * Empty segments are kept. Returns LORA_INVALID_ARGUMENT for an id outside
 * [-1, N) or T/N out of range.
 */
int lora_segments_from_ids(const int32_t* ids, int32_t num_tokens, int32_t num_adapters,
                           int32_t* perm, int32_t* seg_starts, int32_t* seg_adapter);

/*
 * Device scratch of the one-launch calls: the cross-workgroup hand-off of a
 * shrink that is split along h_in before the expand of the same launch
 * ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona
 * l'architettura": the per-adapter work of a decode step runs as one launch),
 * and for the backward the du / transposed-weight buffers of the packed
 * kernels ("Technische Samenvatting: PLoRA" (gist.science), "Packed LoRA
 * Kernels"). Bytes of device workspace needed by `op` (LORA_OP_*) for these
 * adapters and this batch. The value depends only on T, S, N, h_in, h_out and the
 * largest rank in `adapters`, so one workspace serves every later batch with
 * no more tokens and segments.
 */
int lora_workspace_size(int op, const lora_adapters_t* adapters, const lora_segments_t* segments,
                        size_t* bytes);

/*
 * Shrink, the first of the two products of a LoRA-wrapped projection (the
 * low-rank factor A_i of the adapter, "Trajectory presenta C-LoRA"
 * (vivodigitale.it), "Cos'e C-LoRA e perche serve"), for all adapters of the
 * batch in one launch, tiled along tokens and h_in rather than the rank
 * ("Technische Samenvatting: PLoRA" (gist.science), "Kernelontwerp"):
 * u[p][k] = sum_d A_i[k][d] x[row(p)][d] for k < r_i (fp32), for every
 * position p of an active segment. Columns k >= r_i of u are not written.
 * x: DEVICE bf16 [*, ldx]; u: DEVICE fp32 [T, ldu], ldu >= max rank used.
 * Errors as for every call; ws may be NULL when lora_workspace_size() gives 0.
 */
int lora_sgmv_shrink(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                     const lora_segments_t* segments, float* u, int64_t ldu, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Expand, the second product (the factor B_i back to h_out, scaled by the
 * adapter's scaling factor: "Technische Samenvatting: PLoRA" (gist.science),
 * "Resultaten", rank and scaling factor per adapter), for all adapters of
 * the batch in one launch, tiled along tokens and h_out ("Kernelontwerp"):
 * y[row(p)][j] += s_i sum_k B_i[j][k] u[p][k] for j < h_out, rounded to bf16.
 * u: DEVICE fp32 [T, ldu]; y: DEVICE bf16 [*, ldy]. Needs no workspace.
 */
int lora_sgmv_expand(const float* u, int64_t ldu, const lora_adapters_t* adapters,
                     const lora_segments_t* segments, void* y, int64_t ldy, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Fused shrink + expand in ONE kernel launch for all adapters of the batch
 * ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona l'architettura"):
 * y[row(p)] += s_i B_i (A_i x[row(p)]). If u_save is not NULL the fp32
 * intermediate u is also written there (for a later backward), ldu >= max
 * rank used. x and y must not overlap.
 */
int lora_sgmv_fused(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                    const lora_segments_t* segments, void* y, int64_t ldy, float* u_save,
                    int64_t ldu, void* ws, size_t ws_bytes, void* stream);

/*
 * Several LoRA-wrapped projections that read the same x (for example the q,
 * k and v projections of one attention layer, each with its own set of
 * adapters) in ONE kernel launch: the one-launch-per-decode-step design
 * ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona
 * l'architettura") carried over to the projections of a step that share
 * their input, so that the launch latency is paid once.
 *   y[p][row(pos)] += s_p,i B_p,i (A_p,i x[row(pos)])   for p < num_proj
 * adapters[p]: HOST array of num_proj pointers; every projection has the
 * same num_adapters and h_in (the segments' adapter ids index all of them),
 * its own h_out, ranks, scales and weight tables. y[p] / ldy[p]: HOST arrays
 * of num_proj DEVICE output addresses and row strides (bf16 [*, h_out_p]);
 * the outputs must not overlap each other or x (an output that starts at x,
 * or two that start at the same address, are refused with
 * LORA_INVALID_ARGUMENT). 1 <= num_proj <= 4. No u is
 * saved. The workspace is sized by lora_workspace_size_multi() and follows
 * the rules of the other calls. Errors as for lora_sgmv_fused().
 */
int lora_workspace_size_multi(int32_t num_proj, const lora_adapters_t* const* adapters,
                              const lora_segments_t* segments, size_t* bytes);
int lora_sgmv_fused_multi(const void* x, int64_t ldx, int32_t num_proj,
                          const lora_adapters_t* const* adapters, const lora_segments_t* segments,
                          void* const* y, const int64_t* ldy, void* ws, size_t ws_bytes, void* stream);

/*
 * A decode step that can be captured into a HIP graph and replayed with new
 * token ids and new weights. The pages' serving engine keeps every tenant's
 * adapter resident, loads the trained weights in place after each optimizer
 * step, and keeps decoding the other tenants' requests without a stall
 * ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come funziona
 * l'architettura"; the Japanese page, architecture paragraph). Here the
 * batch is described only by DEVICE data, so nothing the host computes is
 * baked into a captured launch:
 *
 *   lora_sgmv_fused_graph() groups token_ids[num_tokens] (request order)
 *   per adapter on the device with a stable counting sort (adapters in id
 *   order, request order within) against the adapters' device tables, cuts
 *   the groups into 32-token tiles and runs the fused shrink + expand on
 *   them. Up to 1024 tokens this is ONE launch: every workgroup reads the
 *   ids and the tables and plans its own tile. Above, a one-workgroup plan
 *   kernel writes the tile table and the sorted-position -> row table into
 *   the workspace first, and the fused launch reads them. Either way:
 *     y[t] += s_i B_i (A_i x[t])   for every token t whose id i is active,
 *   with x and y in request order (rows 0 .. num_tokens-1). A token whose id
 *   is outside [0, N), or whose adapter has a rank outside [1, max_rank] or
 *   a null weight address, is left out (its row of y is not written).
 *
 * Everything a replay may change lives in device memory: the ids, the
 * weights (updated in place) and the four per-adapter tables (re-pointed
 * weights, new ranks up to max_rank, new scales). num_tokens, x, y, the
 * tables' addresses and the workspace are fixed by the capture. The grid is
 * laid out for the most tiles num_tokens ids can need, so a replay costs the
 * same for any id mix. Results equal lora_sgmv_fused() on the same batch.
 *
 * The workspace (lora_workspace_size_graph) must be zero-filled once before
 * its first use and must not be shared with other entry points; calls on
 * one workspace must be ordered (a graph's replays on one stream are). A
 * workspace sized for num_tokens serves calls of fewer tokens too. An epoch
 * kept in the workspace makes every call's hand-off stamps distinct, across
 * replays and batch sizes.
 * Errors are reported for the host arguments only; device data are not
 * checked beyond the rules above.
 */
typedef struct lora_graph_adapters_t {
  int32_t num_adapters;   /* N, 1..256 */
  int32_t h_in;           /* multiple of 8 */
  int32_t h_out;          /* multiple of 8 */
  int32_t max_rank;       /* HOST bound on every rank a replay may use, 1..128 */
  const uint64_t* A_ptrs; /* DEVICE [N]: bf16 A_i [r_i, h_in] */
  const uint64_t* B_ptrs; /* DEVICE [N]: bf16 B_i [h_out, r_i] */
  const int32_t* ranks;   /* DEVICE [N] */
  const float* scales;    /* DEVICE [N] */
} lora_graph_adapters_t;

int lora_workspace_size_graph(const lora_graph_adapters_t* adapters, int32_t num_tokens, size_t* bytes);
int lora_sgmv_fused_graph(const void* x, int64_t ldx, const lora_graph_adapters_t* adapters,
                          const int32_t* token_ids, int32_t num_tokens, void* y, int64_t ldy, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * lora_sgmv_fused without a workspace, for callers that cannot allocate
 * device memory or hand one over (code that must not call hipMalloc in its
 * loop, serving loops and harnesses that forbid allocation). Arguments,
 * results and errors are those of lora_sgmv_fused() minus ws / ws_bytes.
 * The hand-off scratch is a static device array of
 * LORA_NOALLOC_SCRATCH_BYTES per GPU, created with the library and held
 * until the process ends; the call allocates nothing. A batch whose
 * workspace (lora_workspace_size(LORA_OP_FUSED, ...)) exceeds it is refused
 * with LORA_UNSUPPORTED before any HIP call. Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams or
 * threads) race, so they must be ordered. Not capturable into a HIP graph
 * (each launch carries a fresh hand-off id, as for lora_sgmv_fused).
 */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int lora_sgmv_fused_noalloc(const void* x, int64_t ldx, const lora_adapters_t* adapters,
                            const lora_segments_t* segments, void* y, int64_t ldy, float* u_save,
                            int64_t ldu, void* stream);

/*
 * Packed backward over all adapters of the batch ("Technische Samenvatting: PLoRA" (gist.science), "LoRA
 * Execution Engine": forward and backward cases tiled along the sequence or
 * hidden dimension):
 *   du[p]  = s_i B_i^T dy[row(p)]                          (kept in the workspace)
 *   dx[row(p)] += A_i^T du[p]                              (skipped if dx == NULL; bf16)
 *   dB_i   = s_i sum_{p in adapter i} dy[row(p)] u[p]^T    fp32 [h_out, r_i]
 *   dA_i   =     sum_{p in adapter i} du[p] x[row(p)]^T    fp32 [r_i, h_in]
 * u: the forward's fp32 u (e.g. from lora_sgmv_fused's u_save), or NULL to
 * recompute it from x. dA_ptrs / dB_ptrs: DEVICE [N] tables of fp32 output
 * addresses (16-byte aligned); an entry of 0 skips that gradient. Without
 * LORA_GRAD_ACCUMULATE the gradients of every adapter with r_i > 0 are
 * overwritten, with zeros for adapters that have no tokens; with it they are
 * added to, and adapters without tokens are left untouched.
 */
int lora_packed_backward(const void* x, int64_t ldx, const void* dy, int64_t lddy, const float* u,
                         int64_t ldu, const lora_adapters_t* adapters,
                         const lora_segments_t* segments, void* dx, int64_t lddx,
                         const uint64_t* dA_ptrs, const uint64_t* dB_ptrs, uint32_t flags,
                         void* ws, size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* lora_status_string(int status);

/* Reason for the last failing call on this thread ("" if none). */
const char* lora_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int lora_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_SGMV_H */
