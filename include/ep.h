/* ep.h -- C ABI of libep: MoE token dispatch and combine on one AMD MI355X
 * (gfx950), every expert resident on this GPU.
 *
 * Three operations, each one or more launches of hand-written HIP kernels,
 * asynchronously on the caller's stream:
 *
 *   ep_layout   routing table -> per-expert counts, expert-major offsets and a
 *               stable slot for every (token, k) routing entry
 *   ep_dispatch token rows -> per-expert receive rows (bf16 copy, or E4M3FN
 *               bytes plus one fp32 scale per 128 channels)
 *   ep_combine  the k expert outputs of each token -> their routing-weighted
 *               sum in fp32, rounded to bf16
 *
 * Source of the operations.  The pages this library follows are DeepEP issue
 * and pull-request threads about the multi-GPU version of this path.
 *   - "[GH-ISSUE #282] Redundant atomics in internode_ll", code quoted in the
 *     question: the low-latency dispatch counts the tokens it sends to each
 *     expert and hands the receiver one count per (local expert, source rank).
 *     On one GPU holding every expert that is the histogram count[E]; the
 *     expert id maps to (rank = e / experts_per_rank, local = e % ...), which
 *     degenerates to (0, e).
 *   - "[GH-ISSUE #18] Reasons for not calling NVSHMEM public APIs?", maintainer
 *     answer on low-latency mode: data of one expert must keep its order.
 *     Here: inside one expert's rows, entries appear in ascending row-major
 *     (t, j) order of the routing table (a stable counting sort).
 *   - "[PR #693] Pipeline direct NVLink dispatch with triple-buffered
 *     prefetch", Summary: a dispatched token carries hidden data, scale
 *     factors, metadata and routing information.  Here: the receive row, its
 *     scale row, src_of_slot and slot_of.
 *   - "[GH-ISSUE #166] Why does DeepEP LL kernel use double send/recv/signal
 *     buffers?": the low-latency receive buffers are fixed-size per expert.
 *     Here: the fixed-capacity layout [E, capacity, H].
 * The pages do not give the arithmetic.  This library defines it as:
 *   FP8 = OCP E4M3FN (bias 7, max 448, no infinities); per block of 128
 *   channels from channel 0, scale = amax / 448 (one IEEE fp32 division),
 *   q = E4M3FN round-to-nearest-even, saturating, of the fp32 quotient
 *   x / scale (another IEEE fp32 division); amax = 0 gives scale 0 and
 *   codes 0x00.  Combine: acc = +0; for j = 0..k-1 with a slot,
 *   acc = fmaf(w[t,j], expert_out[slot][c], acc); y = bf16 RNE(acc).
 *
 * Conventions.
 *   T tokens, H hidden size, k experts per token, E experts,
 *   cap = capacity (0 selects the contiguous layout).
 *   R = number of receive rows = T*k (contiguous) or E*cap (fixed capacity).
 *   All tensors are dense, row-major, in device memory (HBM) unless noted.
 *   bf16 data is passed as 16-bit patterns, E4M3FN data as bytes.
 *   Data pointers (x, recv_x, recv_scales, expert_out, y) and topk_idx must
 *   be 16-byte aligned; the other int32 / fp32 arrays 4-byte aligned.
 *
 * Ownership.  The caller allocates and owns every buffer, including the
 * layout workspace.  The library never allocates, frees, or keeps a pointer
 * after a call returns, and keeps no mutable global state: calls are
 * re-entrant and may be issued from several host threads.  The one exception
 * is ep_layout_dispatch_noalloc, whose workspace is a fixed device array of
 * the library (one per GPU; see its declaration).
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Every call only enqueues work; nothing synchronises.  Outputs are
 * valid once the stream reaches them.  Two calls that write the same buffers
 * must be ordered by the caller.
 *
 * Errors.  Every entry point returns EP_OK (0) or a negative code.  Argument
 * checks happen on the host before anything is enqueued, so an error code
 * means nothing was launched -- except EP_ERR_HIP, returned when a launch
 * itself fails.  Data-dependent conditions (ids outside [0, E), rows beyond
 * the capacity) are not errors: they are reported in device memory through
 * slot_of = -1 and the status counters.
 */
#ifndef EP_H_
#define EP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    EP_OK = 0,
    EP_ERR_ARG = -1,          /* negative size, NULL required pointer, small workspace */
    EP_ERR_UNSUPPORTED = -2,  /* size outside the supported envelope (see ep_problem) */
    EP_ERR_ALIGN = -3,        /* data pointer not 16-byte aligned, int32/fp32 array not 4-byte */
    EP_ERR_HIP = -4           /* a kernel launch failed */
};

/* Shape of one dispatch / combine problem.  Host struct, read during the call
 * only.  Supported envelope: 0 <= T, 1 <= k <= 32, 1 <= E <= 1024, H >= 8 and
 * H % 8 == 0, H <= 65536, cap >= 0, T*k < 2^31, E*cap < 2^31, and H % 128 == 0
 * when use_fp8 != 0. */
typedef struct ep_problem {
    int32_t num_tokens;   /* T */
    int32_t hidden;       /* H, channels per token */
    int32_t num_topk;     /* k, routing entries per token */
    int32_t num_experts;  /* E */
    int32_t capacity;     /* 0: contiguous layout, rows grouped by expert, R = T*k.
                             > 0: fixed-capacity layout, expert e owns rows
                             [e*cap, (e+1)*cap), R = E*cap */
    int32_t use_fp8;      /* 0: bf16 payload.
                             1: OCP E4M3FN payload, one fp32 scale per 128
                                channels: scale = amax / 448, code = RNE(x / scale).
                             2: E4M3FN payload, one UE8M0 scale byte per 128
                                channels: the scale is 2^s for the smallest
                                s >= -127 with 448 * 2^s >= amax, stored as the
                                byte s + 127 (amax = 0: byte 0, codes 0).  The
                                format is named in "[PR #206] [MERGED] Support
                                UE8M0 data format"; the scale rule is a reading. */
} ep_problem;

/* Layout arrays, all int32 in device memory, written by ep_layout and read by
 * ep_dispatch / ep_combine.  The struct itself is a host struct. */
typedef struct ep_layout_t {
    int32_t* count;        /* [E]    valid entries routed to each expert (never clamped) */
    int32_t* offset;       /* [E+1]  exclusive prefix sum of count; offset[E] = valid entries */
    int32_t* slot_of;      /* [T*k]  receive row of entry (t, j), or -1 if the id is outside
                                     [0, E) or the entry is beyond its expert's capacity */
    int32_t* src_of_slot;  /* [R]    entry index t*k + j that fills each receive row, or -1
                                     (fixed-capacity rows left empty) */
    int32_t* status;       /* [2]    {entries with an id outside [0, E),
                                      entries dropped because their expert was full} */
} ep_layout_t;

/* R for this problem (T*k or E*cap), or -1 if the problem is invalid. */
int64_t ep_num_recv_rows(const ep_problem* prob);

/* Bytes of device workspace ep_layout and ep_layout_dispatch need for this
 * problem (a multiple of 256: two tables of 64 * (E + 1) int32, per-block
 * expert counts and their prefix sums), or -1 if the problem is invalid.
 * Its contents need no initialisation and are scratch after the call. */
int64_t ep_layout_workspace_bytes(const ep_problem* prob);

/* Routing layout.
 *   topk_idx   int32 [T, k], device, 16-byte aligned.  Expert id of each
 *              routing entry.
 *   out        host struct of device pointers, all written:
 *              count, offset, slot_of, src_of_slot (every one of the R rows
 *              is written, -1 for rows no entry fills), status.
 *   workspace  device scratch of at least ep_layout_workspace_bytes bytes.
 * Slots: entry i = t*k + j with valid id e and rank r = number of earlier
 * entries (in row-major order) with the same id gets
 *   contiguous:      slot = offset[e] + r
 *   fixed capacity:  slot = e*cap + r if r < cap, else -1 (counted in status[1]).
 * T = 0 is valid (count and offset are all zero). */
int ep_layout(const ep_problem* prob, const int32_t* topk_idx, const ep_layout_t* out,
              void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch: for every entry with slot_of >= 0, write token t's payload to
 * receive row slot.
 *   x            bf16 [T, H], device.
 *   layout       as written by ep_layout for the same problem (slot_of is read).
 *   recv_x       use_fp8 = 0: bf16 [R, H].  use_fp8 = 1, 2: E4M3FN bytes [R, H].
 *   recv_scales  the block scales of each row: use_fp8 = 1: fp32 [R, H/128];
 *                use_fp8 = 2: UE8M0 bytes [R, H/128].  Ignored (may be NULL)
 *                when use_fp8 = 0.
 * Receive rows that no entry fills are not written.  Every copy of a token is
 * bit-identical.  x must be finite. */
int ep_dispatch(const ep_problem* prob, const void* x, const ep_layout_t* layout,
                void* recv_x, void* recv_scales, void* stream);

/* Layout and dispatch in one call, with the same results as ep_layout
 * followed by ep_dispatch (every output of both is written).  Arguments as
 * for ep_layout and ep_dispatch.  For routing tables of up to 8192 entries
 * (T*k, decode-sized batches) it is one kernel launch in which no workgroup
 * waits for another: each one derives the slots of its own tokens from the
 * whole table while its rows load, then stores them; the workspace is not
 * touched.  Prefill-sized tables (8192 < T*k <= 32768, T*k a multiple of
 * 4, token rows that give every wave of one 1024-lane workgroup per CU
 * between 1 and 14 (bf16) or 16 (FP8) chunks of 64 16-byte pieces) are one
 * launch too: each workgroup histograms the whole table itself while its
 * share of the rows loads, ranks its own tokens' entries, then stores (FP8:
 * quantises and stores each chunk as it arrives); the workspace is not
 * touched.  Other tables take two launches for bf16 payloads and for FP8
 * with k >= 8: the layout's histogram kernel (which also writes per-block
 * prefix sums over experts to the workspace), then a dispatch kernel in
 * which each workgroup computes its own token's slots from those tables and
 * the routing entries ahead of the token in its block before it moves the
 * row; FP8 with k < 8 runs the ep_layout and ep_dispatch kernels in turn.
 * Either way no workgroup waits for another. */
int ep_layout_dispatch(const ep_problem* prob, const int32_t* topk_idx, const ep_layout_t* out,
                       void* workspace, size_t workspace_bytes, const void* x, void* recv_x,
                       void* recv_scales, void* stream);

/* Layout and dispatch as ep_layout_dispatch, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of ep_layout_dispatch without the workspace: the workspace is a fixed
 * device array of EP_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * copy per GPU, held until the process ends.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks the array's address up once (hipGetSymbolAddress)
 * with that device current.
 * Limit: the workspace of the problem must fit the array; every problem
 * inside the supported envelope does (E <= 1024), and a larger one would be
 * rejected with EP_ERR_UNSUPPORTED.  EP_ERR_HIP if the address lookup fails.
 * Sharing: every call on one GPU uses that GPU's array, which keeps the last
 * call's contents.  Nothing in it needs to start at zero (each call writes
 * every word it reads before reading it), but two calls that overlap in time
 * on one GPU (different streams, or different host threads without stream
 * order between them) race on the array and give undefined results; order
 * them on one stream. */
#define EP_NOALLOC_SCRATCH_BYTES 524800
int ep_layout_dispatch_noalloc(const ep_problem* prob, const int32_t* topk_idx,
                               const ep_layout_t* out, const void* x, void* recv_x,
                               void* recv_scales, void* stream);

/* Combine: y[t][c] = bf16_RNE( fixed-order fused multiply-add chain over
 * j = 0..k-1 with slot_of[t*k+j] >= 0 of topk_weights[t*k+j] *
 * expert_out[slot][c], starting from +0.0f ).
 *   expert_out    bf16 [R, H], device, in the receive-row layout.
 *   layout        as written by ep_layout (slot_of is read).
 *   topk_weights  fp32 [T, k], device; used as given (not renormalised).
 *   y             bf16 [T, H], device; every element is written.
 * Receive rows that no entry fills are never read.  Prefill-sized batches
 * take one launch of one 1024-lane workgroup per CU per range of tokens that
 * gives each wave at most 16 chunks of 64 16-byte pieces (up to 16 such
 * launches, over consecutive token ranges); other batches one launch of a
 * workgroup per (token, column tile). */
int ep_combine(const ep_problem* prob, const void* expert_out, const ep_layout_t* layout,
               const float* topk_weights, void* y, void* stream);

/* Elementwise E4M3FN encoding with the exact device encoder ep_dispatch uses
 * (round to nearest even, saturating to +-448, sign kept on zero), for
 * callers that quantise other tensors the same way.
 *   in   fp32 [n], device, finite values.
 *   out  uint8 [n], device.
 * n = 0 is valid and launches nothing. */
int ep_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream);

/* Static text for a status code. */
const char* ep_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* EP_H_ */
