/*
 * moe_w4a16.h -- C ABI of the W4A16 mixture-of-experts expert layer for
 * MI355X (gfx950).
 *
 * The layer (Chord page: "vLLM x Novita AI release Chord, an INT4 MoE
 * operator for Kimi K2.x", sections "TL;DR", "Indexed kernels", "Grouped SM90
 * kernels"):
 *   activations BF16; expert weights uint4 packed eight per int32 word, low
 *   nibble first along K, one BF16 scale per group of 32 along K, zero point
 *   8, dequantised subtract-then-scale w = bf16((q - 8) * s);
 *   per routed row: h = x . W13^T (gate = rows [0, I), up = rows [I, 2I)),
 *   a = bf16(silu(gate) * up), y = a . W2^T, and a top-k-weighted combine
 *   out[t] = sum_j w[t, j] * y(t, j) (indexed layout, and contiguous layout
 *   with row_src).
 *
 * Conventions for every call:
 *   - bf16 values travel as uint16_t bit patterns.
 *   - "device" pointers point to GPU memory (hipMalloc / torch tensors) and
 *     stay owned by the caller; the library never allocates or frees device
 *     memory. "host" pointers point to CPU memory.
 *   - stream is a hipStream_t (NULL = the default stream). Every device
 *     operation is enqueued on it without host synchronisation, except
 *     moe_prepare_weights (load time), which synchronises once.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on an error nothing is enqueued and moe_last_error() describes it.
 *   - Device-side data errors cannot be seen without a synchronisation:
 *     expert ids outside [0, E) route nowhere, masked_m is clamped to
 *     [0, max_m], a contiguous row whose m_index is outside [0, E) is
 *     treated as padding, a contiguous block takes its largest expert id
 *     and skips rows of any other, and a routing buffer made for another
 *     (block, E, T, topk) makes the layer compute nothing.
 *   - MOE_W4A16_VALIDATE=1 in the environment when weights are prepared
 *     turns those cases into errors for that handle: before enqueuing the
 *     layer, a call checks its index data with small kernels on its stream
 *     (topk_ids in [-1, experts), expert_map in [-1, E), masked_m in
 *     [0, max_m], m_indices in [-1, E) with one expert per 128-row block,
 *     row_src paired with m_indices and each flat row used once, a passed-in
 *     routing's header), reads the counts back and synchronises the stream.
 *     A failed check returns INVALID_ARG, or ROUTING_MISMATCH for the
 *     routing header. The counters live in the workspace (the routing
 *     buffer's scratch for moe_align); nothing is allocated. A debugging
 *     aid: the synchronisation makes such calls uncapturable in a graph.
 *   - Calls that share a workspace or routing buffer on one stream are
 *     ordered by the stream; concurrent use of one buffer from two streams
 *     races.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_W4A16_ABI_VERSION 1

typedef void* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,        /* a NULL pointer, a bad size or count */
  MOE_ERR_UNSUPPORTED_SCHEMA = 2, /* quantisation schema not uint4/g32/BF16/zp8 */
  MOE_ERR_MODE_MISMATCH = 3,      /* weights prepared for another layout */
  MOE_ERR_OVERRIDE_REJECTED = 4,  /* tuning override on a grouped layout */
  MOE_ERR_WORKSPACE_TOO_SMALL = 5,/* workspace / routing / prepared buffer */
  MOE_ERR_HIP = 6,                /* a HIP runtime call failed */
  MOE_ERR_ROUTING_MISMATCH = 7    /* routing buffer made for other shapes
                                     (reported in the validation mode) */
} moe_status_t;

/* Layout a set of prepared weights serves (Chord page, "Grouped SM90
 * kernels", Fig. 3: where the padding lives). The layout is recorded in the
 * prepared weights and checked by every entry point. */
typedef enum {
  MOE_MODE_INDEXED = 0,    /* unpadded activations, routing with sentinels */
  MOE_MODE_CONTIGUOUS = 1, /* each expert padded to a 128-row boundary */
  MOE_MODE_MASKED = 2      /* fixed per-expert row budget, masked_m counts */
} moe_mode_t;

enum { MOE_SCALE_BF16 = 1 };
enum { MOE_PACK_INT32_LOW_NIBBLE_FIRST_K = 1 };

/* The quantisation schema and shapes of one MoE layer. Only uint4 (bits = 4),
 * group_size = 32, zero_point = 8, BF16 scales and low-nibble-first int32
 * packing along K are supported (Chord page, "vLLM integration": the schema
 * is uint4, group-32, BF16 scales; other schemas fail at load). hidden and
 * inter must be positive multiples of 32. */
typedef struct {
  int32_t num_experts; /* E, 1..4096 */
  int32_t hidden;      /* H: K of W13, N of W2 */
  int32_t inter;       /* I: W13 has N = 2I rows (gate | up), W2 has K = I */
  int32_t bits;        /* 4 */
  int32_t group_size;  /* 32 */
  int32_t zero_point;  /* 8 */
  int32_t scale_dtype; /* MOE_SCALE_BF16 */
  int32_t pack_order;  /* MOE_PACK_INT32_LOW_NIBBLE_FIRST_K */
  int32_t mode;        /* moe_mode_t */
} moe_weight_desc_t;

/* Per-call schedule overrides, accepted by the indexed entry point only
 * (Chord page, "Grouped SM90 kernels": grouped dispatch owns its layout
 * search and rejects the indexed block_m / tuning overrides). A zero field
 * means "choose automatically".
 *
 * dispatch (small-M schedule only; ignored under large-M) picks how the
 * decode GEMMs' token tiles are scheduled, for the comparison the Chord page
 * measured in "H200 and Blackwell indexed decode" (semi-static against fully
 * dynamic):
 *   0  semi-static (default): a grid fixed from host-known sizes, one
 *      workgroup per (expert, 256 weight rows), row counts read on the device
 *      (with fewer routed rows than experts, the grid covers T*topk sets,
 *      each taking the next expert that holds rows);
 *   1  persistent, static: one workgroup per resident slot, each taking an
 *      equal contiguous range of (routing block, 256 weight rows) jobs;
 *   2  persistent, fully dynamic: the same workgroups taking jobs one at a
 *      time from an atomic counter in the workspace (cleared by the call with
 *      a fill kernel on its stream);
 *   3  semi-static over routing blocks: one workgroup per (routing block,
 *      256 weight rows), the grid bounded by min(blocks, T*topk), so that a
 *      call with few routed rows launches no workgroup per idle expert.
 * With 1, 2 or 3 the routing block is one weight pass, 16 x the token tiles
 * (16, 32 or 64 rows), unless block_m sets it. The semi-static forms (0, 3)
 * may split K over several workgroups when the grid cannot fill the chip
 * (FP32 partials in the workspace, summed in split order). */
typedef struct {
  int32_t block_m;  /* alignment block (rows): 16, 32, 64 or 128 */
  int32_t schedule; /* 0 auto, 1 small-M (decode), 2 large-M (prefill) */
  int32_t dispatch; /* small-M token-tile dispatch: 0 .. 3 (above) */
  int32_t global_experts; /* expert parallelism: experts the routing is drawn
                             from (0: the handle's); rows per expert, which pick
                             the schedule, are T*topk / global_experts */
} moe_tuning_t;

typedef struct moe_weights moe_weights_t; /* opaque host handle */

/* ---- library ---------------------------------------------------------- */

/* MOE_W4A16_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

/* Thread-local description of the last error of this thread ("" if none).
 * The string stays valid until the next call on the same thread. */
const char* moe_last_error(void);

/* Static name of a status code. */
const char* moe_status_string(int status);

/* ---- load time ---------------------------------------------------------- */

/* Bytes of device memory moe_prepare_weights needs for desc, or 0 if desc is
 * invalid or unsupported (moe_last_error says why). */
size_t moe_prepared_bytes(const moe_weight_desc_t* desc);

/* Repack canonical weights into the prepared layout and fix the layout mode
 * (Chord page, "Indexed kernels": configurations and weight layouts are
 * fixed at model load, before packing; "Grouped SM90 kernels": the forward
 * path sees pre-permuted INT4 bytes and re-tiled scales).
 *   w13_q  device int32 [E, 2I, H/8]  rows [0,I) gate, [I,2I) up
 *   w13_s  device bf16  [E, 2I, H/32]
 *   w2_q   device int32 [E, H, I/8]
 *   w2_s   device bf16  [E, H, I/32]
 *   prepared  device buffer of prepared_bytes >= moe_prepared_bytes(desc),
 *             256-byte aligned, owned by the caller, kept alive and unchanged
 *             while the handle is used. The canonical inputs may be freed
 *             after the call returns.
 *   out    host: receives a new handle (release with moe_release_weights).
 * Synchronises `stream` once. Errors: INVALID_ARG, UNSUPPORTED_SCHEMA (also
 * when a scale is NaN, infinite or of magnitude >= 2^117, checked on the
 * device), WORKSPACE_TOO_SMALL, HIP. */
moe_status_t moe_prepare_weights(const moe_weight_desc_t* desc, const int32_t* w13_q,
                                 const uint16_t* w13_s, const int32_t* w2_q,
                                 const uint16_t* w2_s, void* prepared, size_t prepared_bytes,
                                 moe_stream_t stream, moe_weights_t** out);

/* Free a host handle (not the caller's prepared buffer). NULL is ignored. */
void moe_release_weights(moe_weights_t* h);

/* A handle without weights, for sizing buffers before the weights are
 * loaded: size queries (moe_routing_bytes, moe_routing_layout,
 * moe_workspace_bytes) and moe_describe work; every call that would enqueue
 * device work validates its arguments as usual and then returns
 * MOE_ERR_INVALID_ARG. Returns NULL (moe_last_error says why) for an invalid
 * or unsupported desc. Release with moe_release_weights. Makes no HIP call. */
moe_weights_t* moe_plan_create(const moe_weight_desc_t* desc);

/* ---- routing (indexed layout) -------------------------------------------- */

/* Alignment block (rows) the indexed entry point uses for T tokens x topk
 * with these overrides (NULL = none): the per-call schedule refined by
 * tokens per expert (Chord page, "H200 prefill and TP8"). 0 on error. */
int32_t moe_routing_block(const moe_weights_t* h, int32_t T, int32_t topk,
                          const moe_tuning_t* ovr);

/* Bytes of the routing buffer for (T, topk, ovr), 0 on error. */
size_t moe_routing_bytes(const moe_weights_t* h, int32_t T, int32_t topk,
                         const moe_tuning_t* ovr);

/* Layout of a routing buffer, in int32 elements from its start. */
typedef struct {
  int32_t block;        /* alignment block B */
  int32_t cap;          /* T*topk + E*(B-1): slots in sorted_ids */
  int32_t nblocks;      /* ceil(cap / B): entries of block_expert */
  int32_t sentinel;     /* T*topk */
  int64_t off_header;   /* int32[16]; [7] = total padded rows (device-written) */
  int64_t off_counts;   /* int32[E]   rows per expert */
  int64_t off_offsets;  /* int32[E+1] exclusive scan of padded counts */
  int64_t off_sorted;   /* int32[cap] flat row t*topk+j, or sentinel */
  int64_t off_block_expert; /* int32[nblocks] expert of block b, -1 past total */
  int64_t off_slot_of;  /* int32[T*topk] slot p with sorted_ids[p] = f, -1 for a dropped row */
  int64_t off_scratch;  /* internal scratch */
  int64_t total_ints;
} moe_routing_layout_t;

moe_status_t moe_routing_layout(const moe_weights_t* h, int32_t T, int32_t topk,
                                const moe_tuning_t* ovr, moe_routing_layout_t* out);

/* Token -> expert alignment for the indexed layout (Chord page, "Grouped SM90
 * kernels", Fig. 3: activations stay unpadded, the routing indices carry pad
 * sentinels). Bit-exact and deterministic:
 *   counts[e] = rows routed to e; offsets = exclusive scan of
 *   ceil(counts/B)*B; sorted_ids[offsets[e] + r] = r-th flat row of e in
 *   ascending t*topk+j order; all other slots hold the sentinel T*topk;
 *   block_expert[b] = expert owning block b, -1 past the total;
 *   slot_of[f] = the slot p with sorted_ids[p] = f, -1 for a row whose id
 *   lies outside [0, E).
 *   topk_ids  device int32 [T, topk]
 *   routing   device buffer of moe_routing_bytes(h, T, topk, ovr) bytes,
 *             4-byte aligned.
 * Errors: INVALID_ARG, MODE_MISMATCH (handle not INDEXED),
 * WORKSPACE_TOO_SMALL, HIP. T = 0 is valid and writes an empty routing. */
moe_status_t moe_align(const moe_weights_t* h, const int32_t* topk_ids, int32_t T, int32_t topk,
                       const moe_tuning_t* ovr, void* routing, size_t routing_bytes,
                       moe_stream_t stream);

/* Alignment for one GPU's share of the experts (expert parallelism: the
 * handle holds E of num_global_experts experts). topk_ids hold global ids;
 * expert_map (device int32 [num_global_experts]) gives the handle's local
 * expert for each global id, or -1 for an expert held elsewhere. Rows routed
 * elsewhere are dropped as ids outside [0, E) are: they take no slot, so the
 * indexed call given this routing adds only local experts' rows, and a token
 * with none gets 0 (the partial output an EP combine sums over GPUs).
 * Bit-exact; the same buffer layout, capacity and ovr rules as moe_align (set
 * ovr.global_experts = num_global_experts for the schedule of the share).
 * Errors: as moe_align, and INVALID_ARG for a NULL or misaligned map or
 * num_global_experts outside 1..2^20. */
moe_status_t moe_align_ep(const moe_weights_t* h, const int32_t* topk_ids, int32_t T, int32_t topk,
                          const int32_t* expert_map, int32_t num_global_experts,
                          const moe_tuning_t* ovr, void* routing, size_t routing_bytes,
                          moe_stream_t stream);

/* Gather x rows into the aligned order (the contiguous layout's producer;
 * Chord page, "Grouped SM90 kernels", Fig. 3):
 *   a_out      device bf16 [cap, H]: row p = x[sorted_ids[p] / topk], zero
 *              for sentinel slots below the routing's padded total (header
 *              word 7, the layout's M_pad); rows at or past the total are
 *              not written
 *   m_indices  device int32 [cap]: expert of row p, -1 for sentinel slots
 *   row_src    device int32 [cap]: sorted_ids[p], -1 for sentinel slots
 * Any of the three outputs may be NULL. routing must come from moe_align
 * with the same (T, topk, ovr); slots it names outside [0, cap) are not
 * written. Errors: INVALID_ARG (NULL routing, NULL x with a_out and T > 0,
 * x or a_out not 16-byte aligned, bad T / topk), MODE_MISMATCH, HIP. */
moe_status_t moe_permute(const moe_weights_t* h, const uint16_t* x, int32_t T, int32_t topk,
                         const moe_tuning_t* ovr, const void* routing, uint16_t* a_out,
                         int32_t* m_indices, int32_t* row_src, moe_stream_t stream);

/* ---- the layer ------------------------------------------------------------ */

/* Workspace bytes for one call, 0 on error.
 *   indexed:    rows = T (tokens), topk = top-k
 *   contiguous: rows = M_pad, topk = top-k if row_src will be passed (T via
 *               tokens), else 0
 *   masked:     rows = max_m, topk ignored
 * `tokens` is T when the call combines (indexed; contiguous with row_src),
 * ignored otherwise: the workspace then holds T*topk rows of H, the
 * routing-weighted outputs of the second GEMM that the combine sums, kept as
 * 16-bit integers with a power-of-two scale per 8 features, the scale's
 * exponent carried in their top bits (2 bytes a feature, each value within
 * 2^-14 of its group's largest magnitude).
 * ovr: the indexed call's overrides (they set the alignment block and so
 * the routing capacity), NULL otherwise. */
size_t moe_workspace_bytes(const moe_weights_t* h, int32_t mode, int32_t rows, int32_t topk,
                           int32_t tokens, const moe_tuning_t* ovr);

/* Indexed layout (Chord page, "Grouped SM90 kernels", Fig. 3: activations
 * stay unpadded and the padding lives in the routing indices as sentinels;
 * "Indexed kernels" and "H200 and Blackwell indexed decode": the decode
 * schedule follows rows per expert, and block_m / tuning overrides are
 * accepted on this layout only). One call runs the whole layer: W13
 * (gate | up) grouped GEMM with the uint4 dequantisation fused into the
 * weight load, SwiGLU, the W2 grouped GEMM and the top-k-weighted combine
 * out[t] = sum_j topk_w[t, j] * y(t, j).
 *   x        device bf16 [T, H]
 *   topk_ids device int32 [T, topk], topk_w device float [T, topk]
 *   routing  device buffer from moe_align(h, topk_ids, T, topk, ovr, ...) on
 *            this stream, or NULL to align internally (in the workspace)
 *   out      device bf16 [T, H] (fully written; tokens routed nowhere get 0)
 *   ws       device workspace of ws_bytes >= moe_workspace_bytes(h,
 *            MOE_MODE_INDEXED, T, topk, T, ovr), 256-byte aligned
 *   ovr      NULL or overrides (block_m, schedule)
 * Errors: INVALID_ARG, MODE_MISMATCH, WORKSPACE_TOO_SMALL, HIP. */
moe_status_t moe_w4a16_indexed(const moe_weights_t* h, const uint16_t* x, int32_t T, int32_t topk,
                               const int32_t* topk_ids, const float* topk_w, const void* routing,
                               uint16_t* out, void* ws, size_t ws_bytes, const moe_tuning_t* ovr,
                               moe_stream_t stream);

/* Contiguous layout (Chord page, "Grouped SM90 kernels", Fig. 3).
 *   a          device bf16 [M_pad, H], M_pad % 128 == 0; each expert's rows
 *              contiguous and starting on a 128-row boundary
 *   m_indices  device int32 [M_pad]: expert of each row, -1 for padding
 *   row_src    device int32 [M_pad] (t*topk+j, -1 for padding) or NULL
 *   topk_w     device float [T, topk], needed with row_src
 *   out        row_src ? bf16 [T, H] combined : bf16 [M_pad, H] per row
 *              (pad rows unspecified)
 *   ovr        must be NULL (OVERRIDE_REJECTED otherwise)
 * Errors: INVALID_ARG, MODE_MISMATCH, OVERRIDE_REJECTED,
 * WORKSPACE_TOO_SMALL, HIP. */
moe_status_t moe_w4a16_contiguous(const moe_weights_t* h, const uint16_t* a, int32_t M_pad,
                                  const int32_t* m_indices, const int32_t* row_src,
                                  const float* topk_w, int32_t T, int32_t topk, uint16_t* out,
                                  void* ws, size_t ws_bytes, const moe_tuning_t* ovr,
                                  moe_stream_t stream);

/* Indexed layout without allocation, for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same layer, kernels and results as
 * moe_w4a16_indexed with routing = NULL (aligned internally), but the
 * workspace is a fixed device array inside the library,
 * MOE_NOALLOC_SCRATCH_BYTES bytes on each GPU the library runs on, held until
 * the process ends; the caller passes only inputs and outputs.
 *   x, topk_ids, topk_w, out, ovr: as for moe_w4a16_indexed
 * The call allocates nothing (no hipMalloc / hipFree, no library routine that
 * allocates). Every call on one GPU shares that GPU's array and leaves the
 * last call's contents in it: calls that overlap on one GPU (two streams, two
 * threads) race and must be serialised by the caller.
 * Errors: as moe_w4a16_indexed, and WORKSPACE_TOO_SMALL (before anything is
 * enqueued) when the call's workspace (moe_workspace_bytes(h,
 * MOE_MODE_INDEXED, T, topk, T, ovr)) exceeds the array: 128 MiB holds the
 * Kimi decode shape (448 tokens, top-8, 384 experts, hidden 7168,
 * intermediate 2048) and smaller ones. */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
moe_status_t moe_w4a16_indexed_noalloc(const moe_weights_t* h, const uint16_t* x, int32_t T,
                                       int32_t topk, const int32_t* topk_ids, const float* topk_w,
                                       uint16_t* out, const moe_tuning_t* ovr, moe_stream_t stream);

/* Masked layout (Chord page, "Grouped SM90 kernels": expected_m is a
 * positive integer that picks the launch, masked_m holds the valid count
 * per expert, the output is flat even for a 3-D a3, rows past the valid
 * count are to be ignored).
 *   a3         device bf16 [E, max_m, H]
 *   masked_m   device int32 [E] (clamped to [0, max_m])
 *   expected_m > 0: expected rows per expert, picks the schedule only
 *   out        device bf16 [E * max_m, H]; rows >= masked_m[e] unspecified
 *   ovr        must be NULL
 * Errors: INVALID_ARG (also expected_m <= 0), MODE_MISMATCH,
 * OVERRIDE_REJECTED, WORKSPACE_TOO_SMALL, HIP. */
moe_status_t moe_w4a16_masked(const moe_weights_t* h, const uint16_t* a3, int32_t max_m,
                              const int32_t* masked_m, int32_t expected_m, uint16_t* out,
                              void* ws, size_t ws_bytes, const moe_tuning_t* ovr,
                              moe_stream_t stream);

/* ---- unfused steps (indexed layout) ---------------------------------------
 *
 * The layer split at the contract the Chord page times its grouped kernels
 * on ("Grouped SM90 kernels" and "H200 prefill and TP8": routing, activation
 * and communication outside the timed GEMMs): the two grouped GEMMs with BF16
 * outputs, and the activation, as separate calls on the rows of a routing
 * made by moe_align for the same (T, topk, ovr). The GEMMs use the schedule
 * moe_w4a16_indexed would (ovr.dispatch aside: always the semi-static grid).
 * These are BF16 hand-offs: h and y are rounded to BF16 between the steps,
 * where the fused call keeps them in FP32.
 *
 * moe_w4a16_gate_up: for every routing slot s holding flat index
 * f = t*topk + j of expert e, h_out[s][c] = bf16(x[t] . W13[e][c]) over
 * c < 2I in the canonical W13 row order (gate rows [0, I), up rows [I, 2I)).
 *   x        device bf16 [T, H]
 *   routing  device routing buffer (required)
 *   h_out    device bf16 [cap, 2I], cap from moe_routing_layout; rows of pad
 *            slots are left unspecified
 * moe_w4a16_down: y_out[s][n] = bf16(a[s] . W2[e][n]) for the same slots.
 *   a        device bf16 [cap, I] in routing-slot order (moe_swiglu of h_out)
 *   y_out    device bf16 [cap, H]
 * Errors: INVALID_ARG (NULL or misaligned pointers: x/a/outputs 16 B,
 * routing 4 B), MODE_MISMATCH, OVERRIDE_REJECTED, HIP. A routing made for
 * other (E, block, T*topk) computes nothing. Nothing is enqueued on error. */
moe_status_t moe_w4a16_gate_up(const moe_weights_t* h, const uint16_t* x, int32_t T, int32_t topk,
                               const void* routing, uint16_t* h_out, const moe_tuning_t* ovr,
                               moe_stream_t stream);
moe_status_t moe_w4a16_down(const moe_weights_t* h, const uint16_t* a, int32_t T, int32_t topk,
                            const void* routing, uint16_t* y_out, const moe_tuning_t* ovr,
                            moe_stream_t stream);

/* SwiGLU on BF16 rows (reading of the layer's activation, as in the fused
 * W13 epilogue): a[r][c] = bf16(silu(g) * u) with g = h[r][c], u = h[r][I + c]
 * widened to FP32 and silu(z) = z / (1 + exp(-z)), for r < rows, c < inter.
 *   h  device bf16 [rows, 2*inter], a device bf16 [rows, inter], 16-byte
 *   aligned; inter a positive multiple of 8.
 * Errors: INVALID_ARG, HIP. Needs no weights handle. */
moe_status_t moe_swiglu(const uint16_t* h, int64_t rows, int32_t inter, uint16_t* a,
                        moe_stream_t stream);

/* ---- inspection ------------------------------------------------------------ */

/* Dequantise one expert's prepared matrix back to canonical order with the
 * same device routine the GEMMs use: which = 13 -> out bf16 [2I, H],
 * which = 2 -> out bf16 [H, I]. */
moe_status_t moe_dequant_weights(const moe_weights_t* h, int32_t which, int32_t expert,
                                 uint16_t* out, moe_stream_t stream);

/* Write a one-line text description of the schedule a call with these
 * shapes would use (layout, rows per expert, kernel variant, tiles, grid).
 * mode/rows/topk as for moe_workspace_bytes; expected_m for masked.
 * Returns the length written (excluding NUL), or -1. */
int moe_describe(const moe_weights_t* h, int32_t mode, int32_t rows, int32_t topk,
                 int32_t expected_m, const moe_tuning_t* ovr, char* buf, size_t n);

/* Kernel timing. While enabled, every kernel the library enqueues is
 * bracketed by HIP events on its stream. moe_profile_read synchronises those
 * events and writes lines "name launches total_ms\n" (totals since the last
 * reset) into buf; it returns the length written or -1. */
moe_status_t moe_profile_enable(int enable);
void moe_profile_reset(void);
int moe_profile_read(char* buf, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
