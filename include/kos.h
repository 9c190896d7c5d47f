/*
 * kos.h -- C ABI of the KOSMOS-style self-scheduling persistent kernels for
 * MI355X (gfx950): collectives fused into their GEMMs, run on one GPU's share.
 *
 * Sources of the operations (the two KOSMOS pages that describe the method):
 *   [explainer]  "KOSMOS -- Self-scheduling persistent kernels -- What does it
 *                mean?" (learnaivisually.com), paragraphs "Start with the
 *                problem", "KOSMOS removes the manager", "Role switching only
 *                works if ...", "A worked example".
 *   [abstract]   "KOSMOS: Self-scheduling Persistent Kernels for
 *                Communication-Compute Overlap", arXiv 2611.07477, abstract.
 *
 * Every entry point launches ONE persistent kernel (up to four for the
 * unfused baseline) with one workgroup per compute unit.  Workgroups take entries
 * from atomic queues laid out in the order consumers need them and switch
 * roles as ready flags show which data has landed [explainer, "KOSMOS
 * removes the manager"; "Role switching only works if ..."].
 *
 * One rank's share is computed.  The other ranks of a world of `world`
 * ranks are emulated: what they would send arrives as ordinary buffers
 * (device memory, or host memory mapped for the device to model a slower
 * link); what this rank would send them is written to output buffers.
 *
 * Conventions
 *   - Matrices are row-major and dense (leading dimension = column count).
 *   - bf16 is IEEE bfloat16; products accumulate in fp32; bf16 results are
 *     rounded to nearest even.
 *   - Every pointer argument not called "host array" is a device-accessible
 *     address (device memory, or pinned host memory mapped for the device
 *     where stated).  "host array" arguments are small host-side arrays of
 *     such pointers, read during the call only.
 *   - The caller allocates every buffer.  The library allocates nothing on
 *     the call path and keeps no pointer after the call returns.
 *   - All calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Inputs must stay valid and outputs untouched until
 *     the stream reaches the call.
 *   - `ws` is a workspace of `kos_workspace_bytes()` bytes, zeroed once with
 *     kos_workspace_init().  Every call leaves it zeroed again (the last
 *     workgroup to finish resets it), except for the sticky error word that
 *     kos_workspace_status() reads and clears.  Calls that share one
 *     workspace must be ordered on one stream; concurrent calls need
 *     separate workspaces.
 *
 * Errors
 *   - Argument errors are detected before any launch and returned
 *     synchronously; nothing is launched then.  kos_last_error() gives a
 *     thread-local message for the last non-OK status.
 *   - Device-side errors (a ready flag that never arrives within the spin
 *     limit, a capacity overflow) cannot be returned synchronously: the
 *     kernel records the first one in the workspace, every workgroup drains
 *     and exits (no hang), and kos_workspace_status() reports it.  Outputs of
 *     such a call are undefined.
 */
#ifndef KOS_H_
#define KOS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kos_status {
  KOS_OK = 0,
  KOS_ERR_ARG = 1,          /* null pointer, bad enum, world/rank out of range   */
  KOS_ERR_SHAPE = 2,        /* sizes not supported (see each entry point)        */
  KOS_ERR_ALIGN = 3,        /* a pointer is not 16-byte aligned                   */
  KOS_ERR_WORKSPACE = 4,    /* ws null or smaller than kos_workspace_bytes()     */
  KOS_ERR_HIP = 5,          /* a HIP runtime call failed (launch, sync, copy)    */
  KOS_ERR_UNSUPPORTED = 6,  /* no gfx950 device, or a mode this op lacks         */
  KOS_ERR_TIMEOUT = 7,      /* device: a ready flag did not arrive in time       */
  KOS_ERR_CAPACITY = 8      /* device: routed rows exceed a caller capacity      */
} kos_status;

typedef enum kos_dtype { KOS_BF16 = 0, KOS_F32 = 1 } kos_dtype;

/* How the collective and the GEMM share the GPU.
 *   FUSED   one persistent launch; roles switch as readiness dictates.
 *   FIXED   one persistent launch; a fixed crew of `n_movers` workgroups
 *           only communicates (or only reduces), the rest only compute:
 *           a split chosen once, before the call, and never revised
 *           [explainer, "Picture a restaurant kitchen" paragraph].
 *   UNFUSED two launches: the whole collective step, then the whole GEMM
 *           (or GEMM then reduction), same tile code. */
typedef enum kos_mode { KOS_MODE_FUSED = 0, KOS_MODE_FIXED = 1, KOS_MODE_UNFUSED = 2 } kos_mode;

/* GEMM+reduce-scatter output order: BAND finishes the first BM rows of
 * every rank's chunk before any chunk's next BM rows (the consumer order:
 * no reducer waits beyond the first band), ROW one chunk after the
 * other (the ablation the explainer reports 1.41-1.45x slower) ["Role
 * switching only works if"]. */
typedef enum kos_rs_order { KOS_RS_BAND = 0, KOS_RS_ROW = 1 } kos_rs_order;

typedef struct kos_opts {
  int32_t mode;         /* kos_mode                                            */
  int32_t n_movers;     /* workgroups that START in the communication role (and,
                           under FIXED, stay there); < 0 = the library's default
                           for the op, mode and peer link (never per shape):
                           kos_ag_gemm FUSED half the grid over device memory,
                           16 over PCIe; kos_gemm_rs FUSED 0 (builders switch
                           to reducing when the tiles run out); FIXED 16, or 8
                           over PCIe.  Unused by FUSED kos_moe_*.             */
  int32_t rs_order;     /* kos_rs_order (kos_gemm_rs only)                     */
  int32_t grid;         /* workgroups; 0 = one per compute unit.  Must not
                           exceed the compute-unit count (all co-resident).    */
  uint32_t spin_limit;  /* polls of a ready flag before KOS_ERR_TIMEOUT; 0 =
                           default (about a few seconds).                      */
  int32_t peer_link;    /* 0: peers' buffers in device memory; 1: in pinned,
                           device-mapped host memory (PCIe).  Only picks the
                           default crew size.                                  */
  int32_t trace;        /* non-zero: every workgroup records a timeline of its
                           work in the workspace's trace region (read it with
                           kos_workspace_trace).  Adds a few stores per entry;
                           leave it off for timed runs.                        */
  int32_t policy;       /* kos_policy: how roles switch under FUSED             */
} kos_opts;

/* Role-switching policy under KOS_MODE_FUSED [explainer, "KOSMOS removes
 * the manager": roles change in one direction only for the two TP+SP
 * collectives, in both directions for the expert combine; "How do the
 * policies compare?"].
 *   DEFAULT  the pages' choice per op: kos_ag_gemm one-way (movers become
 *            builders), kos_gemm_rs one-way (builders become reducers),
 *            kos_moe_combine and kos_moe_layer two-way (push a ready result,
 *            else build a tile).
 *   SWAPPED  the other choice, for the policy comparison: kos_ag_gemm and
 *            kos_gemm_rs two-way (between tiles a builder takes a move entry
 *            while any is left / the reduce queue's head when it is ready),
 *            kos_moe_combine one-way (builders push only once the tiles run
 *            out).  kos_moe_dispatch has no compute role: ignored there;
 *            kos_moe_layer: KOS_ERR_UNSUPPORTED. */
typedef enum kos_policy { KOS_POLICY_DEFAULT = 0, KOS_POLICY_SWAPPED = 1 } kos_policy;

/* Timeline of one traced call (kos_opts.trace).  The trace region holds
 * KOS_TRACE_LAUNCHES slots, one per kernel launch of the call (a fused call
 * launches once and writes slot 0; the unfused baselines launch up to four
 * kernels and write slots 0, 1, ... in launch order).  In slot l, workgroup
 * g (launch order, 0..grid-1) owns records
 * [(l*KOS_TRACE_MAX_WG + g)*KOS_TRACE_RECORDS, ... + KOS_TRACE_RECORDS).
 * Its record 0 is a header: t0 = when it started, dt = its lifetime, tag =
 * (arrival ticket << 16) | (XCD it ran on << 12) | records written (header
 * and clock record included, at most KOS_TRACE_RECORDS; later pieces of work
 * are dropped).  Record 1 is the clock record: t0 = shader-clock cycles
 * (s_memtime) over the workgroup's lifetime, dt = the lifetime again, tag =
 * KOS_TR_CLOCK << 24, so t0 / dt is the clock the workgroup ran at, in units
 * of 100 MHz.  Every other record is one piece of work: t0 = start, dt =
 * duration, tag = (kos_trace_kind << 24) | entry index (low 24 bits).  Times
 * are ticks of the GPU's constant-rate 100 MHz counter (s_memrealtime), one
 * clock for every launch, so the gaps between the launches of an unfused
 * call show in the timeline.  Used for the idle-CU fraction (the share of
 * workgroup-time outside work records, waits and gaps between launches
 * included, over the call's span) and the clock under load. */
#define KOS_TRACE_RECORDS 512
#define KOS_TRACE_MAX_WG 256
#define KOS_TRACE_LAUNCHES 4
typedef struct kos_trace_rec {
  uint64_t t0;
  uint32_t dt;
  uint32_t tag;
} kos_trace_rec;
typedef enum kos_trace_kind {
  KOS_TR_MOVE = 1,    /* a mover's copy: an all-gather slice; dispatch rows     */
  KOS_TR_TILE = 2,    /* a builder tile (combine: gate/up)                      */
  KOS_TR_WAIT = 3,    /* polling a ready counter before a dependent entry       */
  KOS_TR_REDUCE = 4,  /* a reduce-scatter slab                                  */
  KOS_TR_ROUTE = 5,   /* a router entry (16 tokens)                             */
  KOS_TR_SCAN = 6,    /* a dispatch scan entry (one expert)                     */
  KOS_TR_PUSH = 7,    /* a combine push slab                                    */
  KOS_TR_FOLD = 8,    /* a combine fold block                                   */
  KOS_TR_TILE2 = 9,   /* a combine down tile                                    */
  KOS_TR_CLOCK = 10   /* record 1: shader-clock cycles over the lifetime        */
} kos_trace_kind;

/* Fills `o` with the defaults (FUSED, default crew, band order, full grid). */
void kos_opts_default(kos_opts* o);

/* Bytes of workspace every entry point needs (a fixed size). */
size_t kos_workspace_bytes(void);

/* Zeroes a workspace on `stream` (asynchronous).  Call once after allocating. */
kos_status kos_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* A device-side error as the kernels record it: the status and the entry
 * that raised it (a queue entry index, or a code naming the check; 0 if
 * none).  Only the first error since the last read is kept. */
typedef struct kos_device_error {
  int32_t status;   /* kos_status: KOS_OK, KOS_ERR_TIMEOUT, KOS_ERR_CAPACITY, KOS_ERR_ARG */
  uint32_t entry;   /* what raised it                                          */
} kos_device_error;

/* Synchronizes `stream`, then returns the first device-side error recorded
 * in `ws` since the last call of this function (KOS_OK if none) and clears
 * it; `out` (may be NULL) receives the status and the entry that raised it.
 * KOS_ERR_HIP if the synchronization itself fails. */
kos_status kos_workspace_status(void* ws, void* stream, kos_device_error* out);

/* Synchronizes `stream`, then copies the first `n_records` records of the
 * trace region of `ws` (see kos_trace_rec) to host memory `out`.  n_records
 * is at most KOS_TRACE_LAUNCHES * KOS_TRACE_MAX_WG * KOS_TRACE_RECORDS (else
 * KOS_ERR_ARG).  The region holds the timeline of the last call made with
 * kos_opts.trace set; slots beyond that call's launches and rows of
 * workgroups beyond its grid are stale. */
kos_status kos_workspace_trace(void* ws, kos_trace_rec* out, size_t n_records, void* stream);

/* Thread-local description of the last non-OK status returned on this
 * thread ("" if none).  Valid until the next library call on the thread. */
const char* kos_last_error(void);

/* Number of compute units of the current device (0 if none). */
int32_t kos_device_cu_count(void);

/*
 * All-gather + GEMM, one rank's share [explainer, "Start with the problem":
 * under TP+SP a layer's GEMM input is first collected from every rank;
 * "Role switching only works if": tiles of the shard already held locally
 * are built first, while the movers bring the other shards over in the
 * order the tiles will consume them; "KOSMOS removes the manager": a mover
 * turns builder for good when no transfer is left].
 *
 *   G = [S_0; S_1; ...; S_{world-1}]   (rank-order concatenation of shards)
 *   C = G . W
 *
 * world      ranks, 1..8;   rank: this rank, 0..world-1
 * m_local    rows per shard (> 0);  k: columns of a shard = rows of W;
 *            n: columns of W and C
 * a_local    bf16 [m_local, k]: S_rank
 * a_peers    host array[world]: a_peers[p] = S_p, bf16 [m_local, k], for
 *            p != rank (a_peers[rank] is ignored and may be NULL); device
 *            memory or pinned device-mapped host memory
 * w          bf16 [k, n] (the weight shard, stored K x N)
 * a_gathered out bf16 [world*m_local, k]: G, a bit copy of the shards; with
 *            world == 1 it may alias a_local (then nothing is moved)
 * c          out [world*m_local, n] of c_dtype (KOS_BF16 or KOS_F32)
 * Shapes: k % 64 == 0, n % 64 == 0 and m_local % 64 == 0 (KOS_ERR_SHAPE
 * otherwise); all pointers 16-byte aligned (KOS_ERR_ALIGN).
 */
kos_status kos_ag_gemm(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                       const void* a_local, const void* const* a_peers, const void* w,
                       void* a_gathered, void* c, int32_t c_dtype,
                       const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * All-gather + GEMM that allocates nothing and takes no workspace: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same operation,
 * arguments, shapes, modes, kernels and results as kos_ag_gemm; the queue
 * heads and ready counters live in a static device array of the library
 * (68 KiB, one per GPU, held until the process ends), zeroed before its
 * first use and returned to zero by every call.
 *
 * status_out  optional device int32 (4-byte aligned): when the call's
 *             kernels finish it holds KOS_OK or the device-side error
 *             (KOS_ERR_TIMEOUT); NULL if not wanted.
 * Limits: world * (m_local / tile rows) <= 16384 ready counters, i.e. at
 * most 16384 64-row blocks of gathered rows (KOS_ERR_SHAPE beyond);
 * opts->trace must be 0 (KOS_ERR_ARG).  Every call on one GPU shares its
 * array: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.
 */
kos_status kos_ag_gemm_noalloc(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                               const void* a_local, const void* const* a_peers, const void* w,
                               void* a_gathered, void* c, int32_t c_dtype,
                               const kos_opts* opts, int32_t* status_out, void* stream);

/*
 * GEMM + reduce-scatter, one rank's share [explainer, "Start with the
 * problem": the GEMM's partial sums are split by rows over the ranks and
 * summed; "Role switching only works if": tiles come out one band of rows
 * at a time, covering that band in every rank's chunk, so each rank can
 * start summing after the first band; "KOSMOS removes the manager": a
 * builder that finds no tile left turns reducer for good].
 *
 *   P = A . W                     (this rank's fp32 partial of the output)
 *   chunk c = rows [c*m/world, (c+1)*m/world)
 *   y = sum_{p=0..world-1, ascending} X_p,  X_rank = P[chunk rank],
 *       X_p = peer_slices[p] (p's partial of chunk `rank`), fp32 adds.
 *
 * world, rank  as above;  m, k, n: A is [m, k], W is [k, n]
 * a            bf16 [m, k];  w: bf16 [k, n]
 * peer_slices  host array[world] of fp32 [m/world, n] (entry `rank` ignored)
 * partial      out fp32 [m, n]: P.  Rows of chunk c != rank stand for the
 *              pushes into peer c's inbox; rows of chunk `rank` are staging.
 * y            out fp32 [m/world, n]
 * Band height = the builder tile height; a band of chunk `rank` is reduced
 * once this rank's tiles of that band are stored (peers run the same order
 * at the same pace, so their slices of the band are taken as ready then).
 * Shapes: m % world == 0, (m/world) % 64 == 0, k % 64 == 0, n % 64 == 0.
 */
kos_status kos_gemm_rs(int32_t world, int32_t rank, int64_t m, int64_t k, int64_t n,
                       const void* a, const void* w, const float* const* peer_slices,
                       float* partial, float* y,
                       const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * The same two collectives with the weight stored transposed, W^T [n, k]
 * (row j holds output column j's k values): the data-gradient GEMMs of the
 * backward pass [abstract: each TP+SP collective of a layer is fused with
 * its GEMM; explainer, "Start with the problem"].  The backward of
 * an all-gather+GEMM (Y = AG(X) . W) is a GEMM+reduce-scatter of dY . W^T;
 * the backward of a GEMM+reduce-scatter (Y = RS(X . W)) is an
 * all-gather+GEMM of dY with W^T -- both with the forward weight as it is
 * stored, k x n, read as the n x k operand of the transposed product.
 *
 * kos_ag_gemm_wt:  as kos_ag_gemm with C = G . W^T, w_t bf16 [n, k].
 * kos_gemm_rs_wt:  as kos_gemm_rs with P = A . W^T, w_t bf16 [n, k].
 * Shapes, modes, other arguments and errors as the plain entry points.
 */
kos_status kos_ag_gemm_wt(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                          const void* a_local, const void* const* a_peers, const void* w_t,
                          void* a_gathered, void* c, int32_t c_dtype,
                          const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

kos_status kos_gemm_rs_wt(int32_t world, int32_t rank, int64_t m, int64_t k, int64_t n,
                          const void* a, const void* w_t, const float* const* peer_slices,
                          float* partial, float* y,
                          const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * MXFP8 operands for the two TP+SP collectives [abstract: the same fused
 * kernels speed up training in MXFP8 as well as in BF16].  The pages do not
 * restate the format; it is the OCP Microscaling (MX) specification v1.0:
 * elements are FP8 E4M3 codes (uint8), and every 32 consecutive elements
 * along K share one E8M0 scale (uint8 s, value 2^(s-127)); element value =
 * E4M3 value x its block's scale.  Products accumulate in fp32.
 *
 * Scale layout (both operands): K/64 slabs; slab s holds, for every row r of
 * the operand (R rows), the scales of blocks 2s and 2s+1 at bytes
 * s*2R + 2r and s*2R + 2r + 1 -- i.e. scale[r][b] sits at
 * (b/2)*2R + 2r + (b%2).  A tile's scales for one 64-k step are then one
 * contiguous run.  The weight is stored N x K (each output column's K codes
 * contiguous), with its scales in the same slab layout over its N rows.
 */

/*
 * All-gather + GEMM with MX operands: as kos_ag_gemm, with
 *
 *   G = [S_0; ...; S_{world-1}] (codes and scales gathered, rank order)
 *   C = G . W^T    (W stored [n, k])
 *
 * a_local, a_peers[p]        E4M3 [m_local, k]
 * a_local_scales,            E8M0 scales of those rows, slab layout over
 * a_peer_scales[p]           R = m_local rows (k/64 slabs of 2*m_local bytes)
 * w, w_scales                E4M3 [n, k]; scales in slab layout over R = n
 * a_gathered                 out E4M3 [world*m_local, k]: G's codes
 * a_gathered_scales          out: G's scales, slab layout over
 *                            R = world*m_local rows (each slab holds the
 *                            shards' rows in rank order)
 * c                          out [world*m_local, n] of c_dtype
 * Shapes: m_local, k, n positive multiples of 256 (KOS_ERR_SHAPE); all
 * pointers 16-byte aligned (KOS_ERR_ALIGN).  The other arguments, the
 * modes and the errors are those of kos_ag_gemm.
 */
kos_status kos_ag_gemm_mx(int32_t world, int32_t rank, int64_t m_local, int64_t k, int64_t n,
                          const void* a_local, const void* a_local_scales,
                          const void* const* a_peers, const void* const* a_peer_scales,
                          const void* w, const void* w_scales,
                          void* a_gathered, void* a_gathered_scales, void* c, int32_t c_dtype,
                          const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * GEMM + reduce-scatter with MX operands: as kos_gemm_rs with
 * P = A . W^T, A E4M3 [m, k] with scales in slab layout over R = m rows,
 * W E4M3 [n, k] with scales over R = n rows.  Partials, peer slices and y
 * are fp32 as in kos_gemm_rs.  Shapes: m % world == 0, m/world, k and n
 * positive multiples of 256 (KOS_ERR_SHAPE); pointers 16-byte aligned.
 */
kos_status kos_gemm_rs_mx(int32_t world, int32_t rank, int64_t m, int64_t k, int64_t n,
                          const void* a, const void* a_scales, const void* w, const void* w_scales,
                          const float* const* peer_slices, float* partial, float* y,
                          const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/* Shape of an expert layer seen from one rank.  Experts are spread over the
 * ranks contiguously: rank d holds experts [d*E_loc, (d+1)*E_loc),
 * E_loc = experts / world. */
typedef struct kos_moe_shape {
  int32_t world, rank;
  int32_t tokens;   /* T: this rank's tokens                                 */
  int32_t hidden;   /* H                                                      */
  int32_t experts;  /* E (global), a multiple of world, <= 1024              */
  int32_t topk;     /* k, 1..min(E, 16)                                       */
  int32_t ffn;      /* F: expert hidden width                                 */
  int32_t reserved; /* must be 0                                              */
} kos_moe_shape;

/*
 * Expert layer, dispatch direction: router -> permutation -> token movement
 * [abstract: the whole expert layer, routing through the final weighted
 * sum, in one launch per direction; explainer, "Start with the problem": a
 * token's row is sent to the rank owning its expert, and the result comes
 * back].
 *
 * Router: per token, the k experts of largest logit in descending order,
 * ties to the lowest expert index; weights = softmax over the k selected
 * logits (fp32).  Packed order: pairs (t, j) sorted by (expert, t); pair
 * (t, j) of expert e sits at offset[e] + #{t' < t routed to e}.  One row per
 * pair (a token sent twice to one rank is sent twice).
 *
 * x            bf16 [T, H];  logits: fp32 [T, E]
 * peer_send    host array[world]: rows peer p sends us (p != rank), bf16,
 *              expert-major over our local experts, in p's packed order
 * peer_counts  int32 [world, E_loc] (device): rows p sends us per local
 *              expert; row `rank` must be 0
 * topk_idx     out int32 [T, k];  topk_w: out fp32 [T, k]
 * counts       out int32 [E]: pairs routed to each expert (global)
 * perm         out int32 [T*k]: packed position of pair (t, j)
 * out_send     host array[world] of out bf16 [send_caps[d], H]: rows for
 *              peer d != rank, i.e. our packed rows of d's experts, in order
 * send_caps    host array[world]: rows out_send[d] holds (entry `rank`
 *              ignored); may be NULL when world == 1
 * x_grouped    out bf16 [grouped_cap, H]: rows of our local experts,
 *              expert-major, then by source rank, then in source order
 * grouped_offsets out int32 [E_loc + 1]: expert e's rows start here
 * row_src      out int32 [grouped_cap, 2]: (source rank, row index in what
 *              that source sends us) of every grouped row
 * With T == 0, x, logits, topk_idx, topk_w and perm may be NULL.
 * peer_send[p] may be NULL if peer p sends nothing (its peer_counts row is
 * zero) and out_send[d] if no pair routes to d's experts; a NULL buffer
 * that something would travel through is reported as KOS_ERR_ARG by
 * kos_workspace_status (the rows are skipped, never dereferenced).
 * T <= 65536 and T * E * 12 bytes within the workspace's 15 MiB scratch
 * (KOS_ERR_SHAPE otherwise).
 * Capacities overflow -> KOS_ERR_CAPACITY (device, see kos_workspace_status;
 * nothing is written past a buffer's capacity); send_caps[d] >=
 * T*min(k, E_loc) and grouped_cap >= sum(peer_counts) + T*min(k, E_loc)
 * never overflow.  Shapes: H % 64 == 0.
 */
kos_status kos_moe_dispatch(const kos_moe_shape* s, const void* x, const float* logits,
                            const void* const* peer_send, const int32_t* peer_counts,
                            int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* perm,
                            void* const* out_send, const int64_t* send_caps,
                            void* x_grouped, int64_t grouped_cap, int32_t* grouped_offsets,
                            int32_t* row_src,
                            const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * Expert layer, combine direction: grouped SwiGLU expert GEMMs, results
 * pushed back to their source ranks, and the weighted fold of this rank's
 * tokens [abstract; explainer, "KOSMOS removes the manager": here roles
 * switch both ways -- between tiles a workgroup sends back a finished
 * result if one is waiting, else it computes the next tile].
 *
 *   h  = bf16( silu(X_e . Wg_e) * (X_e . Wu_e) )      fp32 silu and product
 *   Yg = bf16( h . Wd_e )                              per local expert e
 *   out_return[p][i] = Yg[r] for the grouped row r with row_src (p, i), p != rank
 *   y[t] = bf16( sum_{j ascending} topk_w[t,j] * res(t,j) ), fp32 accumulate,
 *   res(t,j) = Yg row of pair (t,j) if its expert is local, else row
 *              perm[t*k+j] - send_off[d] of peer_return[d], d = expert's rank.
 *
 * x_grouped, grouped_offsets, row_src, topk_idx, topk_w, counts, perm,
 * peer_counts: as produced / consumed by kos_moe_dispatch (device)
 * w_gate, w_up bf16 [E_loc, H, F];  w_down bf16 [E_loc, F, H]
 * peer_return  host array[world] of bf16 [>= rows we sent d, H] (entry
 *              `rank` ignored): results d returns, in our packed order
 * h            out bf16 [grouped_cap, F] (the SwiGLU hidden, kept for
 *              inspection);  y_grouped: out bf16 [grouped_cap, H]
 * gate_save, up_save  optional out bf16 [grouped_cap, F]: bf16(X_e . Wg_e)
 *              and bf16(X_e . Wu_e) as the tiles computed them, for a
 *              backward pass that reads them instead of recomputing them
 *              (kos_moe_layer_bwd); both NULL (nothing written) or both
 *              given (else KOS_ERR_ARG)
 * out_return   host array[world] of out bf16 [return_caps[p], H]: the
 *              results of the rows p sent us, in p's packed order
 * return_caps  host array[world]: rows out_return[p] holds (entry `rank`
 *              ignored; at least the rows p sent us, else KOS_ERR_CAPACITY
 *              from kos_workspace_status and the kernel does nothing); may
 *              be NULL when world == 1
 * y            out bf16 [T, H]
 * With T == 0, topk_idx, topk_w, perm and y may be NULL.  peer_return[d]
 * may be NULL if we sent d nothing and out_return[p] if p sent us nothing;
 * otherwise a NULL peer buffer is reported as KOS_ERR_ARG by
 * kos_workspace_status and the kernel does nothing.  So are grouped
 * offsets that decrease or describe more than grouped_cap rows
 * (KOS_ERR_CAPACITY).  A grouped row whose row_src names a rank outside
 * [0, world) or a row past what that rank sent (peer_counts) is not pushed
 * and is reported as KOS_ERR_ARG.
 * Shapes: H % 128 == 0, F % 64 == 0, grouped_cap * H * 2 < 2^31 bytes
 * (else KOS_ERR_SHAPE).
 */
kos_status kos_moe_combine(const kos_moe_shape* s, const void* x_grouped,
                           const int32_t* grouped_offsets, const int32_t* row_src,
                           int64_t grouped_cap,
                           const void* w_gate, const void* w_up, const void* w_down,
                           const int32_t* topk_idx, const float* topk_w,
                           const int32_t* counts, const int32_t* perm,
                           const int32_t* peer_counts,
                           const void* const* peer_return,
                           void* h, void* gate_save, void* up_save,
                           void* y_grouped, void* const* out_return,
                           const int64_t* return_caps, void* y,
                           const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole expert layer, forward direction, in ONE persistent launch:
 * router -> permutation -> token movement -> grouped SwiGLU expert GEMMs ->
 * results pushed back -> weighted fold [abstract: KOSMOS runs the whole
 * expert layer, routing through the final weighted sum, in one launch per
 * direction; explainer, "KOSMOS removes the manager"].
 *
 * Computes exactly what kos_moe_dispatch followed by kos_moe_combine
 * computes, with the same arguments and outputs (see both): the launch
 * boundary between them is replaced by ready counters -- the grouped
 * SwiGLU tiles of a unit (256 grouped rows of one expert) start as soon as
 * the unit's rows have landed, while other workgroups still move tokens.
 *
 * Inputs: x, logits, peer_send, peer_counts (as kos_moe_dispatch); w_gate,
 * w_up, w_down, peer_return (as kos_moe_combine).  Outputs: topk_idx,
 * topk_w, counts, perm, out_send (with send_caps), x_grouped (grouped_cap
 * rows), grouped_offsets, row_src (as kos_moe_dispatch); h, the optional
 * gate_save and up_save, y_grouped (at least grouped_cap rows), out_return
 * (with return_caps), y (as kos_moe_combine).  Shapes and errors: those of both calls (H % 128 == 0,
 * F % 64 == 0; capacities -> KOS_ERR_CAPACITY from kos_workspace_status,
 * nothing written past a buffer).  opts->mode must be KOS_MODE_FUSED
 * (KOS_ERR_UNSUPPORTED otherwise): the two calls are the baseline.
 */
kos_status kos_moe_layer(const kos_moe_shape* s, const void* x, const float* logits,
                         const void* const* peer_send, const int32_t* peer_counts,
                         const void* w_gate, const void* w_up, const void* w_down,
                         const void* const* peer_return,
                         int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* perm,
                         void* const* out_send, const int64_t* send_caps,
                         void* x_grouped, int64_t grouped_cap, int32_t* grouped_offsets, int32_t* row_src,
                         void* h, void* gate_save, void* up_save, void* y_grouped,
                         void* const* out_return, const int64_t* return_caps,
                         void* y, const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

/*
 * The expert layer, backward direction (data and router gradients), in ONE
 * persistent launch [abstract: one launch per direction of the whole expert
 * layer].  The pages give no backward formulas; this is the chain rule of
 * the forward above, with y[t] = sum_j w[t,j] * res[t,j]:
 *   movers    each pair's output gradient dres = bf16(w[t,j] * dy[t]) goes
 *             where the forward sent the token row: into dres_grouped for
 *             our own experts, into out_send_grad[d] (our packed order)
 *             for rank d's; the rows peers send us (peer_send_grad) are
 *             pulled into dres_grouped (grouped order of the forward)
 *   tiles 1   per unit (256 grouped rows of one expert) and 256 columns of
 *             F (128 when F % 256 != 0): dH = dres . Wd^T (fp32, kept in
 *             dh), then per 128 of those columns g = X.Wg and u = X.Wu
 *             recomputed from the forward's grouped input and
 *             dU = bf16(dH * silu(g)), dG = bf16(dH * u * silu'(g))
 *             (the forward's bf16 rounding of h passes gradients unchanged);
 *             with gate_saved / up_saved given, g and u are those bf16
 *             values instead (no recomputation: dH and the epilogue only)
 *   tiles 2   per unit and 256 columns of H, once the unit's tiles 1 are
 *             done: dX = bf16(dG . Wg^T + dU . Wu^T)
 *   pushes    dX rows of rows a peer sent us, back to it (out_return_grad,
 *             the peer's packed order); two-way with the tiles
 *   fold      dx[t] = bf16(sum_j dX(t,j)) (fp32, j ascending; remote rows
 *             from peer_return_grad) and the router gradient
 *             dlogits[t, idx[t,j]] = w_j * (dw_j - sum_i w_i * dw_i),
 *             dw_j = <dy[t], res[t,j]> (fp32; res the forward's results:
 *             y_grouped rows or peer_return rows), 0 for other experts.
 * Weight gradients are plain grouped GEMMs with no collective: not here.
 *
 * dy           bf16 [T, H]
 * topk_idx, topk_w, perm, counts, peer_counts, x_grouped, grouped_offsets,
 * row_src, y_grouped, peer_return: the forward's (kos_moe_layer, or
 *              kos_moe_dispatch + kos_moe_combine), read only
 * w_gate, w_up bf16 [E_loc, H, F];  w_down bf16 [E_loc, F, H]
 * gate_saved, up_saved  bf16 [grouped_cap, F]: the forward's gate_save and
 *              up_save outputs, or both NULL to recompute g and u (one
 *              without the other: KOS_ERR_ARG)
 * peer_send_grad  host array[world] of bf16 [rows p sent us, H] (entry
 *              `rank` ignored): the gradients of the rows p sent us, in
 *              the order p sent them
 * out_send_grad   host array[world] of out bf16 [send_caps[d], H]: our
 *              pairs' gradients for rank d, in our packed order
 * dres_grouped out bf16 [grouped_cap, H];  dg, du: out bf16 [grouped_cap, F]
 * dh           out fp32 [grouped_cap, F]; with gate_saved it may be NULL
 *              (then not written)
 * dx_grouped   out bf16 [grouped_cap, H]
 * peer_return_grad host array[world] of bf16 [>= rows we sent d, H]: the
 *              dX rows d returns for the rows we sent it
 * out_return_grad  host array[world] of out bf16 [return_caps[p], H]
 * dx           out bf16 [T, H];  dlogits: out fp32 [T, E] (every entry
 *              written)
 * A rank's buffers may be NULL where nothing travels (world == 1: the
 * arrays themselves).  Errors, reported by kos_workspace_status with the
 * kernel then doing nothing more: a NULL peer buffer that would be read or
 * written, grouped offsets that disagree with counts + peer_counts or pass
 * grouped_cap, routing that names rows outside the forward's (KOS_ERR_ARG
 * or KOS_ERR_CAPACITY); send/return capacities below the rows that travel
 * (KOS_ERR_CAPACITY).  Shapes: H % 256 == 0, F % 128 == 0, grouped_cap * H
 * * 2 < 2^31 bytes (else KOS_ERR_SHAPE).  All buffers 16-byte aligned
 * (KOS_ERR_ALIGN).  opts->mode must be
 * KOS_MODE_FUSED with the default policy (KOS_ERR_UNSUPPORTED otherwise).
 */
kos_status kos_moe_layer_bwd(const kos_moe_shape* s, const void* dy,
                             const int32_t* topk_idx, const float* topk_w, const int32_t* perm,
                             const int32_t* counts, const int32_t* peer_counts,
                             const void* x_grouped, int64_t grouped_cap,
                             const int32_t* grouped_offsets, const int32_t* row_src,
                             const void* y_grouped, const void* const* peer_return,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* gate_saved, const void* up_saved,
                             const void* const* peer_send_grad,
                             void* const* out_send_grad, const int64_t* send_caps,
                             void* dres_grouped, void* dg, void* du, float* dh, void* dx_grouped,
                             const void* const* peer_return_grad,
                             void* const* out_return_grad, const int64_t* return_caps,
                             void* dx, float* dlogits,
                             const kos_opts* opts, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KOS_H_ */
