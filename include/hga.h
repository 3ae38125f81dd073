/*
 * hga.h - C ABI of the MI355X (gfx950) Hierarchical Global Attention hot path.
 *
 * HGA is two-level, content-routed attention for one query block (all five
 * pages titled "Long-Context Fine-Tuning with Limited VRAM"; the method detail
 * is on gist.science, Technical Summary §2.1 "Hierarchical Global Attention"):
 *   1. a summary vector per closed 64-token chunk is scored against the query
 *      block and the best chunks are kept ("Chunk Selection");
 *   2. inside those chunks, summaries of 8-token groups are scored and the best
 *      groups are kept ("Group Selection");
 *   3. attention runs over the exact K/V of the selected groups plus the local
 *      window, here the whole active segment, causal ("Exact-Token Attention").
 * Routing has no gradient and no learned weights (same section); history K/V
 * is detached at the segment boundary (§2.2 "Segment-wise Backward and Tiered
 * Storage"), so the backward produces dQ for every query and dK/dV only for the
 * active segment.
 *
 * Readings where the pages are silent:
 *   - summary = mean of the chunk's / group's keys (fp32);
 *   - block query = mean of the block's 64 queries over the r = n_q/n_kv query
 *     heads that share one KV head; query head h uses KV head h / r;
 *   - score = unscaled fp32 dot product; top-k keeps the highest scores and the
 *     lowest index on ties (NaN ranks lowest, -0 == +0);
 *   - one routing decision per (query block, KV head), shared by its r heads
 *     and 64 queries;
 *   - selections are written in ascending index order, padded with -1;
 *   - the "fixed sink and local windows" beside the routed chunks (gist.science
 *     §2.1 "Chunk Selection"): the first n_sink_chunks history chunks are
 *     attended in full and not ranked; the local window is the W most recent
 *     segment tokens (default: the whole segment). Routing covers the closed
 *     history only, so with W < seg_len older segment tokens are not attended.
 *
 * Layouts (contiguous, head-major, batch 1; "dtype" = hga_shape.dtype, i.e.
 * fp32 or bf16 stored as raw 16-bit words):
 *   q, o, d_o, dq                [n_q_heads][seg_len][head_dim]   dtype
 *   k_hist, v_hist               [n_kv_heads][P][head_dim] dtype, first hist_len
 *                                rows of each head used, P = hist_stride or hist_len
 *   k_seg, v_seg, dk_seg, dv_seg [n_kv_heads][seg_len][head_dim]  dtype
 *   chunk_sum                    [n_kv_heads][P/64][head_dim] fp32
 *   group_sum                    [n_kv_heads][P/8][head_dim]  fp32
 *   lse                          [n_q_heads][seg_len] fp32 (natural log)
 *   sel_chunks                   [seg_len/64][n_kv_heads][top_k_chunks] int32
 *   sel_groups                   [seg_len/64][n_kv_heads][top_k_groups] int32
 *
 * Ownership: the caller allocates every buffer and the workspace; the library
 * allocates no device memory and keeps no state between calls except, for the
 * pinned-host history tier, one side stream and three events per device,
 * created on first use; host-tier calls on one device from several threads
 * take turns while they enqueue (they share that side stream). Every pointer
 * is a device pointer except k_hist / v_hist under HGA_HIST_HOST_PINNED, which
 * must come from hipHostMalloc (page-locked, mapped) memory.
 *
 * Streams: `stream` is a hipStream_t (NULL = the null stream). All work is
 * enqueued asynchronously on it; calls return before the GPU finishes.
 *
 * Errors: every argument is checked on the host before anything is launched;
 * on failure nothing is enqueued and a status code is returned (never an abort
 * or exception). A failed launch returns HGA_ERR_HIP. Faults that occur while
 * kernels run surface at the caller's next synchronisation. hga_last_error()
 * gives a human-readable detail of the last failure on the calling thread.
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HGA_ABI_VERSION 4

typedef enum {
  HGA_OK = 0,
  HGA_ERR_INVALID_ARG = 1,   /* bad shape, null pointer, bad range */
  HGA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. head_dim 96) */
  HGA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  HGA_ERR_HIP = 4            /* a HIP runtime call or launch failed */
} hga_status;

typedef enum { HGA_F32 = 0, HGA_BF16 = 1 } hga_dtype;
typedef enum { HGA_HIST_DEVICE = 0, HGA_HIST_HOST_PINNED = 1 } hga_hist_loc;
typedef enum {
  HGA_OP_ROUTE = 0,
  HGA_OP_ATTN_FWD = 1,
  HGA_OP_ATTN_BWD = 2,
  HGA_OP_ROUTE_CACHED = 3
} hga_op;

/* Problem description shared by every call. */
typedef struct {
  int32_t n_q_heads;      /* query heads; a multiple of n_kv_heads (GQA) */
  int32_t n_kv_heads;     /* key/value heads */
  int32_t head_dim;       /* 64 or 128 */
  int32_t chunk;          /* tokens per chunk; must be 64 */
  int32_t group;          /* tokens per group; must be 8 */
  int32_t block_q;        /* queries per routed block; must be 64 */
  int32_t top_k_chunks;   /* chunks kept per (block, KV head); 1..64 */
  int32_t top_k_groups;   /* groups kept per (block, KV head); 1..512 */
  int64_t hist_len;       /* H: history tokens, a multiple of 64, may be 0 */
  int32_t seg_len;        /* S: active-segment tokens, a positive multiple of 64 */
  float softmax_scale;    /* multiplies Q.K before the softmax, > 0 */
  int32_t dtype;          /* hga_dtype of Q/K/V/O/dO/dQ/dK/dV */
  int32_t hist_loc;       /* hga_hist_loc of k_hist / v_hist */
  int64_t hist_stride;    /* rows per KV head in k_hist / v_hist, 0 = hist_len; a
                             multiple of 64, >= hist_len. Summaries then hold
                             hist_stride/64 chunk and hist_stride/8 group rows
                             per KV head, so a history can grow in place */
  int32_t n_sink_chunks;  /* >= 0: the first n_sink_chunks history chunks (the
                             fixed sink) are attended in full by every query
                             and are not ranked by the router */
  int32_t local_window;   /* >= 0: query i attends segment keys t with
                             i - W < t <= i, W = local_window (0 or >= seg_len:
                             the whole segment, causal) */
} hga_shape;

/* Chunk and group summaries (gist.science Technical Summary §2.1, "Chunk
 * Selection" and "Group Selection"; pith.science review, "What carries the
 * argument": summaries are built from the model's projected keys).
 * For every chunk m with 64m in [tok_begin, tok_end):
 *   chunk_sum[j][m] = mean of k_hist[j][64m .. 64m+63]
 *   group_sum[j][n] = mean of k_hist[j][8n .. 8n+7] for its 8 groups n.
 * tok_begin, tok_end: multiples of 64 with 0 <= tok_begin <= tok_end <= hist_len
 * (incremental use: summarise only the tokens of a newly closed segment).
 * k_hist lives where shape->hist_loc says (device or pinned host); chunk_sum
 * is device memory; group_sum is device memory or page-locked host memory
 * (hipHostMalloc; recognised by its pointer attributes, written over the host
 * link) for use with hga_route_cached. Both are 16-byte aligned (rows are
 * written 16 bytes at a time), else HGA_ERR_INVALID_ARG. Summaries outside the
 * range are untouched. */
hga_status hga_build_summaries(const hga_shape* shape, const void* k_hist,
                               int64_t tok_begin, int64_t tok_end,
                               float* chunk_sum, float* group_sum, void* stream);

/* Two-level routing (gist.science Technical Summary §2.1, "Chunk Selection",
 * "Group Selection"; routing runs without gradient). For each query block b
 * and KV head j: qbar = block query; chunk scores qbar . chunk_sum[j][m] over
 * the history chunks after the sink, m in [n_sink_chunks, hist_len/64); keep
 * top_k_chunks; group scores over the 8
 * groups of each kept chunk; keep top_k_groups. Both lists are ascending and
 * padded with -1 when fewer candidates exist (e.g. hist_len == 0).
 * ws: device workspace of at least hga_workspace_size(shape, HGA_OP_ROUTE)
 * bytes, 256-byte aligned; its contents are scratch. */
hga_status hga_route(const hga_shape* shape, const void* q, const float* chunk_sum,
                     const float* group_sum, int32_t* sel_chunks, int32_t* sel_groups,
                     void* ws, size_t ws_bytes, void* stream);

/* hga_route without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same kernels and results, bit for bit, as hga_route;
 * the workspace is a static device array of HGA_NOALLOC_SCRATCH_BYTES in the
 * library, one per device, held until the process ends (its address is looked
 * up on the first call on a device). Returns HGA_ERR_WORKSPACE, with nothing
 * enqueued, when hga_workspace_size(shape, HGA_OP_ROUTE) exceeds that size.
 * Calls no allocating routine. Every call on one device shares that device's
 * array and leaves its contents behind (nothing in it needs to start at zero:
 * each call writes what it reads), so calls that overlap on one device (other
 * streams, other threads) race: the caller must order them. */
#define HGA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
hga_status hga_route_noalloc(const hga_shape* shape, const void* q, const float* chunk_sum,
                             const float* group_sum, int32_t* sel_chunks, int32_t* sel_groups,
                             void* stream);

/* Group-summary cache (gist.science Technical Summary §2.2, "Tiered Memory
 * Hierarchy", and pith.science review, Figure 2 caption: device memory keeps
 * every chunk summary but only a cache of group summaries; the rest of the
 * history lives in host memory). The cache is one device buffer of
 * hga_gcache_bytes(shape, n_slots) bytes holding n_slots chunk slots per KV
 * head, each with the 8 group summaries of one chunk, plus the chunk-to-slot
 * tables. It is tied to (n_kv_heads, head_dim, hist_stride or hist_len,
 * n_slots): reset it before first use and whenever the history it mirrors is
 * rewritten; appending history (growing hist_len under a fixed hist_stride)
 * keeps it valid. 1 <= n_slots <= 16384; 0 is returned for invalid input.
 * Layout (each part starts on a 256-byte boundary, in this order), readable
 * for inspection: slot_of_chunk int32 [n_kv][P/64] (-1: not cached),
 * chunk_of_slot int32 [n_kv][n_slots] (-1: empty), hand int32 [n_kv] (next
 * slot of the clock), data fp32 [n_kv][n_slots][8][head_dim]. */
size_t hga_gcache_bytes(const hga_shape* shape, int32_t n_slots);

/* Empties the cache (every slot free, clock hands at slot 0), on `stream`. */
hga_status hga_gcache_reset(const hga_shape* shape, void* cache, int32_t n_slots, void* stream);

/* hga_route with the group summaries in page-locked host memory (group_sum_host,
 * [n_kv][P/8][head_dim] fp32, P = hist_stride or hist_len) behind the cache.
 * Same selections, bit for bit, as hga_route on the same summaries. Runs as
 * three kernels on `stream`: chunk selection for every block; one cache update
 * per KV head (the union of the chunks the blocks kept: cached ones are hits
 * and stay; each miss, in ascending chunk order, takes the next slot in clock
 * order that no hit of this call holds, and its 8 rows are copied from host
 * memory); group selection from the cache. Requires
 * n_slots >= (seg_len/64) * top_k_chunks (every kept chunk fits),
 * (seg_len/64) * top_k_chunks <= 8192 and P/64 <= 131072 chunks. stats (device, optional): per KV head
 * {hits, misses} of this call, int32 [n_kv][2]. ws:
 * hga_workspace_size(shape, HGA_OP_ROUTE_CACHED) bytes, 256-byte aligned.
 * Calls that share one cache must be ordered (one stream). */
hga_status hga_route_cached(const hga_shape* shape, const void* q, const float* chunk_sum,
                            const float* group_sum_host, void* cache, int32_t n_slots,
                            int32_t* sel_chunks, int32_t* sel_groups, int32_t* stats,
                            void* ws, size_t ws_bytes, void* stream);

/* Decode step for a batch of sequences (gist.science §3 "Key Contributions":
 * the trained adapter runs with HGA for retrieval and generation; the routing
 * and key set of §2.1 with the history / open-segment split of §2.2).
 * Sequence b has a closed, summarised history of hist_lens[b] tokens and an
 * open segment of tail_lens[b] tokens that ends with its n_new newest tokens,
 * whose queries are q[b]. The step routes with the mean of those queries over
 * the r heads of each KV head (as hga_route does for a 64-query block) and,
 * for new token i at open-segment position p = tail_lens[b] - n_new + i,
 * attends the sink tokens, the tokens of the selected groups and the
 * open-segment tokens t with p - W < t <= p (W = local_window, default the
 * whole open segment):
 *   o[b][h][i] = sum_t softmax_t(scale * q[b][h][i] . k_t) v_t, lse likewise.
 * Layouts (device memory, except k_hist / v_hist, which live where
 * shape->hist_loc says; P = hist_stride or hist_len is the history
 * capacity, T = seg_len the open-segment capacity):
 *   q, o           [batch][n_q][n_new][head_dim]        (dtype)
 *   k_hist, v_hist [batch][n_kv][P][head_dim]           (dtype)
 *   chunk_sum      [batch][n_kv][P/64][head_dim]        fp32 (hga_build_summaries per sequence)
 *   group_sum      [batch][n_kv][P/8][head_dim]         fp32
 *   k_tail, v_tail [batch][n_kv][T][head_dim]           (dtype)
 *   hist_lens, tail_lens  int32 [batch], device memory: read by the kernels,
 *                  clamped to [0, P] (rounded down to whole chunks) and to
 *                  [n_new, T]
 *   sel_chunks [batch][n_kv][top_k_chunks], sel_groups [batch][n_kv][top_k_groups]
 *   lse            fp32 [batch][n_q][n_new]
 * With hist_loc = HGA_HIST_HOST_PINNED (gist.science §2.2 "Tiered Memory
 * Hierarchy": history in host RAM, summaries in VRAM) each call copies every
 * (sequence, KV head)'s sink rows and routed groups over the host link into
 * ws after routing, then attends to those copies; results are bit-identical
 * to device-resident history. Requires 1 <= n_new <= seg_len and
 * r * n_new <= 16 (r = n_q_heads / n_kv_heads). ws:
 * hga_decode_workspace_size(shape, batch, n_new) bytes, 256-byte aligned. */
size_t hga_decode_workspace_size(const hga_shape* shape, int32_t batch, int32_t n_new);

hga_status hga_decode(const hga_shape* shape, int32_t batch, int32_t n_new, const void* q,
                      const void* k_hist, const void* v_hist, const float* chunk_sum,
                      const float* group_sum, const void* k_tail, const void* v_tail,
                      const int32_t* hist_lens, const int32_t* tail_lens,
                      int32_t* sel_chunks, int32_t* sel_groups, void* o, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/* hga_decode with a two-pass chunk route (gist.science §2.1 "Chunk Selection":
 * the same top-k_c chunks, lowest index on ties). chunk_sum_bf16 holds bf16
 * copies of chunk_sum, same layout [batch][n_kv][P/64][head_dim], rounded to
 * nearest even (hga_summaries_to_bf16), device memory, 16-byte aligned, kept
 * by the caller beside chunk_sum. Each (sequence, KV head) scores its chunks
 * from the copies, which read half the bytes; a chunk whose copy score is
 * more than twice the rounding bound below the k_c-th largest cannot be in
 * the fp32 top k_c, and the rest are re-scored from chunk_sum. Outputs are
 * bit-identical to hga_decode on the same inputs provided the copies are
 * those of chunk_sum: a stale copy can change the selection (never a memory
 * access). Batches whose chunk scan is split over several workgroups per
 * (sequence, KV head) (at most 64 pairs) read no copies: their short scans
 * are latency bound. Non-finite or huge summaries, and routes where too many
 * chunks stay candidates, fall back to the fp32 scan inside the kernel. Same
 * arguments, requirements, workspace (hga_decode_workspace_size) and errors
 * as hga_decode, plus HGA_ERR_INVALID_ARG for a NULL or misaligned
 * chunk_sum_bf16 when the history capacity is > 0. */
hga_status hga_decode_twopass(const hga_shape* shape, int32_t batch, int32_t n_new, const void* q,
                              const void* k_hist, const void* v_hist, const float* chunk_sum,
                              const uint16_t* chunk_sum_bf16, const float* group_sum, const void* k_tail,
                              const void* v_tail, const int32_t* hist_lens, const int32_t* tail_lens,
                              int32_t* sel_chunks, int32_t* sel_groups, void* o, float* lse, void* ws,
                              size_t ws_bytes, void* stream);

/* dst[i] = src[i] rounded to bf16 (nearest even; NaN stays NaN, values
 * beyond the bf16 range become infinite) for i < n, on `stream`: the copies
 * hga_decode_twopass reads. n must be a multiple of 8 (0: nothing to do);
 * src and dst are device memory, 16-byte aligned, not overlapping.
 * HGA_ERR_INVALID_ARG otherwise. */
hga_status hga_summaries_to_bf16(const float* src, uint16_t* dst, int64_t n, void* stream);

/* Exact-token attention forward (gist.science Technical Summary §2.1,
 * "Exact-Token Attention"; pith.science review, Figure 1: summaries select
 * regions, attention uses exact K/V only). For query i of head h (block
 * b = i/64, KV head j = h/r) the keys are the sink tokens
 * 0 .. 64*n_sink_chunks-1, the 8 tokens of every group n >= 0 in
 * sel_groups[b][j] (history) and segment tokens i-W+1 .. i (the local window,
 * W = whole segment by default, causal):
 *   o[h][i] = sum_t softmax_t(scale * q[h][i] . k_t) v_t
 *   lse[h][i] = log sum_t exp(scale * q[h][i] . k_t)
 * sel_groups entries are group ids in [0, hist_len/8) or -1 (empty slot); the
 * kernels treat any other value as -1, so no entry can make them read outside
 * the history. ws: hga_workspace_size(shape, HGA_OP_ATTN_FWD)
 * bytes (zero for device-resident history; staging for the pinned-host tier,
 * whose gathers run on an internal side stream fenced back to `stream`). With
 * pinned-host history and hist_len > 0, ws holds after the call (in stream
 * order) the routed K/V rows of every query block and the sink rows, which
 * hga_attn_bwd_staged reads. */
hga_status hga_attn_fwd(const hga_shape* shape, const void* q, const void* k_hist,
                        const void* v_hist, const void* k_seg, const void* v_seg,
                        const int32_t* sel_groups, void* o, float* lse,
                        void* ws, size_t ws_bytes, void* stream);

/* Backward of hga_attn_fwd for the loss sum(o * d_o) (gist.science Technical
 * Summary §2.1: gradients flow through exact-token attention; §2.2: history
 * is detached at the segment boundary). Writes dq for every query, dk_seg and
 * dv_seg for the active segment; history K/V, summaries and selections get no
 * gradient. o and lse are the forward's outputs. Deterministic: no atomics.
 * ws: hga_workspace_size(shape, HGA_OP_ATTN_BWD) bytes, 256-byte aligned.
 * k_hist / v_hist live where shape->hist_loc says (gist.science §2.2
 * "Tiered Memory Hierarchy": history in host RAM, routed exact K/V in VRAM).
 * With page-locked host history (and hist_len > 0) the call first copies every
 * query block's routed groups and the sink rows into ws over the host link, in
 * stream order, then reads only those copies; the result is bit-identical to
 * the same call on device-resident history. sel_groups as for hga_attn_fwd:
 * ids outside [0, hist_len/8) count as -1. */
hga_status hga_attn_bwd(const hga_shape* shape, const void* q, const void* k_hist,
                        const void* v_hist, const void* k_seg, const void* v_seg,
                        const int32_t* sel_groups, const void* o, const float* lse,
                        const void* d_o, void* dq, void* dk_seg, void* dv_seg,
                        void* ws, size_t ws_bytes, void* stream);

/* hga_attn_bwd for pinned-host history (shape->hist_loc ==
 * HGA_HIST_HOST_PINNED) that reads the history rows hga_attn_fwd left in its
 * workspace instead of bringing them over the host link again (gist.science
 * §2.2 "Segment-wise Backward and Tiered Storage": the routed exact K/V of the
 * active segment stay in VRAM for its backward). fwd_ws / fwd_ws_bytes: the
 * workspace of an hga_attn_fwd call with the same shape and sel_groups, not
 * written since (stream order: enqueue this call after that one). ws:
 * hga_workspace_size(shape, HGA_OP_ATTN_BWD) bytes suffice. Outputs, ids
 * outside [0, hist_len/8) and determinism as for hga_attn_bwd; the result is
 * bit-identical to it. */
hga_status hga_attn_bwd_staged(const hga_shape* shape, const void* q, const void* fwd_ws,
                               size_t fwd_ws_bytes, const void* k_seg, const void* v_seg,
                               const int32_t* sel_groups, const void* o, const float* lse,
                               const void* d_o, void* dq, void* dk_seg, void* dv_seg,
                               void* ws, size_t ws_bytes, void* stream);

/* Exact-token gather on its own (gist.science Technical Summary §2.1 and
 * §2.2 "Tiered Memory Hierarchy": only the selected groups' exact K/V are
 * brought into the working set). Copies the 8 tokens of every selected group
 * into k_out / v_out [seg_len/64][n_kv_heads][top_k_groups*8][head_dim]
 * (dtype), zero-filling the rows of -1 entries and of ids outside
 * [0, hist_len/8). k_hist / v_hist live where
 * shape->hist_loc says (device or pinned host); outputs are device memory. */
hga_status hga_gather_groups(const hga_shape* shape, const void* k_hist,
                             const void* v_hist, const int32_t* sel_groups,
                             void* k_out, void* v_out, void* stream);

/* Internal kernels, for hga_set_kernel_events. */
typedef enum {
  HGA_KERNEL_SUMMARIES = 0,    /* hga_build_summaries */
  HGA_KERNEL_ROUTE = 1,        /* hga_route; hga_route_cached (all three kernels) */
  HGA_KERNEL_GATHER = 2,       /* hga_gather_groups, pinned-host tier gathers */
  HGA_KERNEL_ATTN_FWD = 3,     /* hga_attn_fwd */
  HGA_KERNEL_BWD_DQ = 4,       /* hga_attn_bwd: dQ (and rowsum(dO * O)) */
  HGA_KERNEL_BWD_DKDV = 5,     /* hga_attn_bwd: dK, dV of the segment (+ partial sum) */
  HGA_KERNEL_GCACHE = 6,       /* hga_route_cached: the cache update */
  HGA_KERNEL_DECODE = 7,       /* hga_decode: attention pieces + merge (its route stamps ROUTE) */
  HGA_KERNEL_COUNT = 8
} hga_kernel;

/* Instrumentation: while set, the launches of `kernel` stamp ev_start with
 * the start of the entry point's first launch of it and ev_stop with the end
 * of its last (hipExtLaunchKernel timestamps: no extra packets on the
 * stream), so hipEventElapsedTime gives the duration of the most recent call;
 * BWD_DKDV includes the fixed-order partial sum. With pinned-host history
 * (HGA_HIST_HOST_PINNED) hga_attn_fwd runs its gathers and attention in
 * phases: GATHER then spans the first gather to the last on the library's
 * side stream and ATTN_FWD the first attention phase to the last on the
 * caller's stream, waits in between included. Both NULL turns it off. The
 * setting is process-wide and not synchronised between threads; the caller
 * owns the hipEvent_t handles, created with timing enabled. */
hga_status hga_set_kernel_events(int32_t kernel, void* ev_start, void* ev_stop);

/* Bytes of workspace `op` (an hga_op) needs for this shape; 0 if the shape is
 * invalid or the op needs none. */
size_t hga_workspace_size(const hga_shape* shape, int32_t op);

/* Static string for a status code (an hga_status value); any other value
 * gives "HGA_ERR_UNKNOWN". Taken as a plain integer so that every value the
 * caller passes is well-defined. */
const char* hga_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none). The pointer stays valid until the next call on that thread. */
const char* hga_last_error(void);

/* HGA_ABI_VERSION of the loaded library. */
int32_t hga_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H */
