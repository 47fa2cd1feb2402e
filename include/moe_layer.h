/*
 * moe_layer.h -- C ABI of the sparse mixture-of-experts FFN layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (sources: "Optimizing on-device inference for Apple Silicon",
 * Perplexity 2026):
 *   - the router scores every routed expert and each token keeps its top k,
 *     plus one shared expert that every token passes through
 *     (section "Qwen creates three distinct workload shapes");
 *   - routing stays on the GPU: a histogram of assignments per expert, a
 *     prefix scan to group offsets, a scatter into expert groups and a block
 *     map of fixed-size row tiles for the grouped GEMM, with no host
 *     synchronisation inside the layer (section "Keep expert routing on the
 *     GPU");
 *   - each expert applies two input projections with a gated activation,
 *     then an output projection combined with its routing score and the
 *     shared expert's result (section "Reduce intermediate and state
 *     traffic"); products accumulate in fp32 and write bf16 (section
 *     "Dequantize weights during matrix multiplication");
 *   - prefill (many rows) runs as grouped matrix-matrix products, batch-1
 *     decode as bandwidth-bound matrix-vector products over the selected
 *     experts only (sections "Apple silicon offers different paths for
 *     different workloads" and "Optimize the single-row weight path").
 *
 * Definitions fixed by this library where the pages are silent:
 *   scores     L[t,e] = x[t] . Wr[e] (+ bias[e]), fp32;
 *   selection  the top_k largest L[t,.], descending, equal scores -> lower
 *              expert index first; slot j of a token holds its rank-j expert;
 *   weights    w[t,j] = softmax over the selected scores (equal to the full
 *              softmax probabilities renormalised over the selection);
 *   expert     F(x) = Wd . (silu(Wg . x) * (Wu . x)), silu(z) = z*sigmoid(z);
 *   output     out[t] = S(x[t]) + sum_j w[t,j] * F_{ids[t,j]}(x[t]), with S the
 *              shared expert (weight 1), no capacity limit, no dropped token;
 *   groups     assignments of one expert are stored in ascending token order.
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library allocates nothing, keeps no state between calls and never
 *     frees caller memory.  Pointers must be 16-byte aligned.
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and the call returns without waiting.
 *     Buffers must stay valid until that work completes.  The library never
 *     synchronises the stream and never launches host callbacks.
 *   - Arguments are checked before anything is enqueued; a failed check
 *     returns a status and enqueues nothing.  A failed launch returns
 *     MOE_ERR_HIP (the hipError_t is available from moe_last_hip_error()).
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Calls on distinct workspaces are independent (re-entrant); two calls
 *     sharing one workspace must be ordered (same stream, or synchronised).
 *
 * Layouts (row-major, bf16 = IEEE bfloat16 bits):
 *   x          bf16 [M][H]
 *   router_w   bf16 [E][H]
 *   expert_w   bf16 [E][3*I*H]; expert e = gate [I][H], up [I][H], down [H][I]
 *   shared_w   bf16 [3*I_shared*H], same packing, or NULL when I_shared == 0
 *   out        bf16 [M][H]
 *   router_bias fp32 [E] or NULL
 * Outputs (out, the workspace, the routing buffers) must not overlap any
 * input (x, router_w, the expert and shared weights, router_bias) nor each
 * other; a call that breaks this returns MOE_ERR_INVALID_ARG.
 *
 * Supported shapes: M >= 0 (M == 0 is a no-op returning MOE_OK),
 * H % 64 == 0 and 64 <= H <= 16384, I % 64 == 0 and 64 <= I <= 16384,
 * I_shared == 0 or (I_shared % 64 == 0 and I_shared <= 16384),
 * 1 <= E <= 1024, 1 <= top_k <= min(E, 32), M * top_k < 2^31.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream handle, declared exactly as <hip/hip_runtime_api.h>
 * declares it, so that this header needs no HIP include (an identical
 * repeated typedef is valid C11 and C++).  NULL is the default stream. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,         /* null pointer, negative size, aliasing */
  MOE_ERR_UNSUPPORTED_SHAPE = 2,   /* outside the supported shapes above */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < moe_workspace_size() */
  MOE_ERR_MISALIGNED = 4,          /* a pointer is not 16-byte aligned */
  MOE_ERR_HIP = 5                  /* a HIP launch failed */
} moe_status_t;

/* Path selection.  1 <= M <= 5 (8 with 4-bit experts): the decode path, each
 * token row through its own selected experts (for M > 1 the decode kernels
 * run one grid row per token row; an expert two rows select is read for
 * each).  Larger M up to 64: the small-batch path, matrix-vector products
 * over the union of the experts the rows select, each expert's weights read
 * once for all rows routed to it (section "Limits of further optimization":
 * few-row batches pick different experts).  Both give every row the bits of
 * a one-row call.  By default the matrix-vector paths run when M <= 64 and
 * M * top_k <= 4 * E (at most four assignments per expert on average), the
 * grouped path otherwise; the flags override that choice.  Only the grouped
 * path reports counts / offsets / perm. */
#define MOE_FLAG_FORCE_GEMV 0x1u /* matrix-vector paths; requires M <= 64 */
#define MOE_FLAG_FORCE_GEMM 0x2u /* grouped (matrix-matrix) path, also at M == 1 */
/* expert_w and shared_w are in the tiled layout written by moe_tile_weights
 * (bf16), or the 4-bit experts and shared expert in the one written by
 * moe_tile_weights_q4 (moe_layer_forward_q4).  Every path reads it; results
 * are bit-identical to the row-major layout's. */
#define MOE_FLAG_TILED_WEIGHTS 0x4u
/* Decode path (M == 1) in two launches instead of three, when I and
 * I_shared <= 512, H <= 4096 and (top_k * I + I_shared) * 4 <= 64 KiB (else
 * the three launches run).  Launch 1: router scores and the shared expert's
 * gated activations side by side; launch 2: the selection, the routed
 * experts' gated activations and the down projections + combine, the down
 * workgroups loading their weights at the start and waiting inside the
 * launch for the gated activations (section "Keep each decode step on the
 * GPU": steps wait only where a dependency requires it).  Same results,
 * bit for bit, as the three launches, which are faster on MI355X: both
 * phases are bound by HBM, and the in-launch wait costs about as much as a
 * kernel boundary. */
#define MOE_FLAG_DECODE_TWO_LAUNCH 0x10u
/* Test hook, never set in normal use: the in-launch wait of the two-launch
 * decode path (see moe_routing_t.wait_status) waits for a condition that
 * never occurs, with a short bound, so that it takes its give-up path. */
#define MOE_FLAG_WAIT_PROBE 0x8u

typedef struct {
  int64_t M;                /* token rows in this call */
  int32_t H;                /* hidden size */
  int32_t E;                /* routed experts */
  int32_t I;                /* routed expert intermediate size */
  int32_t I_shared;         /* shared expert intermediate size; 0 = no shared expert */
  uint32_t flags;           /* MOE_FLAG_* */
  const float* router_bias; /* device fp32 [E] added to the scores, or NULL */
} moe_desc_t;

/* Optional routing outputs (device pointers; any may be NULL = not wanted). */
typedef struct {
  int32_t* topk_ids; /* [M][top_k] selected experts, slot order = rank order */
  float* topk_w;     /* [M][top_k] routing weights */
  float* logits;     /* [M][E] fp32 router scores (bias included) */
  int32_t* counts;   /* [E] assignments per expert (grouped path only) */
  int32_t* offsets;  /* [E+1] exclusive prefix sum of counts (grouped path only) */
  int32_t* perm;     /* [M*top_k] perm[p] = t*top_k + j of the assignment at group
                        position p (grouped path only) */
  int32_t* tiles;    /* [moe_block_map_capacity()][4] the block map of the grouped
                        GEMMs (grouped path only; section "Keep expert routing on
                        the GPU": the list of fixed-size row blocks the grouped
                        GEMM works on): per tile (group g, first row r0 in the
                        group, rows, group position of row r0); routed groups
                        g < E in expert order, then the shared expert (g == E,
                        its rows are the tokens in order); a routed group of
                        c > 0 rows is cut into one tile when c <= 288, else
                        into ceil((c - 32) / 256) tiles, all of 256 rows but
                        the last, which holds the rest (1 .. 288 rows: up to
                        32 rows past a multiple of 256 ride with the tile
                        before); the shared group is cut into ceil(M / 256)
                        tiles of 256 rows but the last */
  int32_t* num_tiles; /* [1] tiles in the block map (grouped path only) */
  int32_t* wait_status; /* [1] 0 when every wait inside the call's kernels ended
                           normally; 1 when one gave up, in which case out holds
                           NaN rows.  Only the two-launch decode path
                           (MOE_FLAG_DECODE_TWO_LAUNCH) waits inside a launch:
                           its second launch waits for the routed experts'
                           gated activations before their down projections
                           (bounded: about a second); the other paths have no
                           such wait and write 0. */
} moe_routing_t;

/* Capacity, in tiles, that moe_routing_t.tiles must have for this
 * descriptor and top_k: ceil(M*top_k/256) + E, plus ceil(M/256) with a
 * shared expert; 0 when the arguments are invalid.  Pure host computation. */
int64_t moe_block_map_capacity(const moe_desc_t* d, int top_k);

/* Bytes of device workspace moe_layer_forward / moe_route need for this
 * descriptor and top_k on the path the descriptor selects; 0 when the
 * arguments are invalid.  Pure host computation. */
size_t moe_workspace_size(const moe_desc_t* d, int top_k);

/* The whole layer: out = shared expert + weighted top-k routed experts.
 * x, router_w, expert_w, shared_w, top_k, out as documented above;
 * workspace: device buffer of workspace_bytes >= moe_workspace_size(d, top_k),
 * 256-byte aligned, contents undefined on entry and exit;
 * routing: NULL, or buffers that receive the routing decisions. */
moe_status_t moe_layer_forward(const moe_desc_t* d, const void* x, const void* router_w,
                               const void* expert_w, const void* shared_w, int top_k, void* out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream,
                               const moe_routing_t* routing);

/* Routing only (scores, top-k, weights and, on the grouped path, the
 * histogram / scan / scatter tables), written to `routing` (non-NULL). */
moe_status_t moe_route(const moe_desc_t* d, const void* x, const void* router_w, int top_k,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       const moe_routing_t* routing);

/* Kernels of the layer, as reported by moe_layer_forward_traced. */
typedef enum {
  MOE_K_ROUTER_SCORES = 1,     /* grouped path: router scores (MFMA) */
  MOE_K_TOPK = 2,              /* grouped path: top-k, weights, per-chunk histograms */
  MOE_K_ROUTE_SCAN = 3,        /* grouped path: prefix scan and block map */
  MOE_K_ROUTE_SCATTER = 4,     /* grouped path: scatter into expert groups */
  MOE_K_GEMM_GATEUP = 5,       /* grouped path: gate/up GEMM + gated activation */
  MOE_K_GEMM_DOWN = 6,         /* grouped path: down GEMM of the routed experts */
  MOE_K_COMBINE = 7,           /* grouped path without a shared expert: weighted combine */
  MOE_K_DEC_ROUTER = 8,        /* decode: router scores */
  MOE_K_DEC_GATEUP = 9,        /* decode: shared expert gate/up, top-k, routed gate/up */
  MOE_K_DEC_DOWN = 10,         /* decode: down projections + combine */
  MOE_K_SM_ROUTER = 11,        /* small batch: router scores */
  MOE_K_SM_TOPK = 12,          /* small batch: top-k, weights, union of the selected experts */
  MOE_K_SM_GATEUP = 13,        /* small batch: shared and union experts' gate/up + activation */
  MOE_K_SM_DOWN = 14,          /* small batch: down projections + combine */
  MOE_K_DEC_ROUTE = 15,        /* decode, two launches: router scores, shared expert gate/up */
  MOE_K_DEC_EXPERTS = 16,      /* decode, two launches: top-k, routed gate/up, all down projections, combine */
  MOE_K_SHARED_DOWN_COMBINE = 17, /* grouped path with a shared expert: its down GEMM + the weighted combine */
  MOE_K_ROUTE_SCAN_SCATTER = 18   /* grouped path, calls of up to 8192 tokens: scan, block map and scatter */
} moe_kernel_t;

/* Instrumentation for moe_layer_forward_traced: caller-created hipEvent_t
 * handles (timing enabled).  Each kernel of the call is launched with
 * begin[count] / end[count] as its start / stop events (hipExtLaunchKernel
 * semantics: the events take the kernel's own start and end time, the
 * interval a kernel-trace profiler reports), kernel[count] receives its
 * moe_kernel_t and count advances.  Launches beyond capacity run untimed. */
typedef struct {
  void* const* begin;
  void* const* end;
  int32_t* kernel;
  int32_t capacity;
  int32_t count;
} moe_trace_t;

/* moe_layer_forward with per-kernel event records (same arguments and
 * results; trace may be NULL, which is exactly moe_layer_forward). */
moe_status_t moe_layer_forward_traced(const moe_desc_t* d, const void* x, const void* router_w,
                                      const void* expert_w, const void* shared_w, int top_k,
                                      void* out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream, const moe_routing_t* routing,
                                      moe_trace_t* trace);

/* 4-bit group-affine expert weights ("Optimizing on-device inference for
 * Apple Silicon", section "Dequantize weights during matrix multiplication":
 * 4-bit weights whose groups of 64 share a bf16 scale and bias).
 * Every weight of the bf16 packing (expert e = gate [I][H], up [I][H],
 * down [H][I], rows along the reduction dimension) is w = s*q + b, with q
 * an unsigned 4-bit code and (s, b) the bf16 scale and bias of its group of
 * 64 consecutive elements of the block (row lengths are multiples of 64, so
 * a group never spans two rows).
 *   codes       uint8 [E][3*I*H/2]: element 2i in the low nibble of byte i,
 *               element 2i+1 in the high nibble
 *   scale_bias  uint32 [E][3*I*H/64]: group g's scale in bits 0..15, its
 *               bias in bits 16..31 (bf16 bit patterns)
 * The shared expert uses the same layout with E = 1 and I_shared.  Both
 * pointers are device pointers, 16-byte aligned. */
typedef struct {
  const void* codes;
  const void* scale_bias;
} moe_q4_t;

/* moe_layer_forward (with the optional trace of moe_layer_forward_traced)
 * on 4-bit expert weights: experts (non-NULL) and shared (NULL when
 * I_shared == 0) in the layout above.  x, the router and the output stay
 * bf16; the workspace is sized by moe_workspace_size.  Products accumulate
 * in fp32: the matrix-matrix path rounds each dequantised weight to bf16
 * for the MFMA operands, the decode path multiplies in fp32. */
moe_status_t moe_layer_forward_q4(const moe_desc_t* d, const void* x, const void* router_w,
                                  const moe_q4_t* experts, const moe_q4_t* shared, int top_k, void* out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream,
                                  const moe_routing_t* routing, moe_trace_t* trace);

/* Rewrites nblocks bf16 expert blocks (each 3*H*I elements in the row-major
 * packing above: gate [I][H], up [I][H], down [H][I]) from src into the tiled
 * layout at dst, the order in which the grouped GEMM streams its weight tiles
 * ("Optimizing on-device inference for Apple Silicon", section "Dequantize
 * weights during matrix multiplication": one small weight tile at a time is
 * staged on chip), so that each tile's K-step is one contiguous block.
 * Layout of a block (3*H*I elements, as before):
 *   gate/up part, elements [0, 2*I*H): panel p = 0 .. ceil(I/128)-1 starts at
 *     256*p*H and holds n = min(128, I - 128p) gate rows and the n up rows of
 *     the same indices as 2n tile rows, gate (m = 0) or up (m = 1) row
 *     128p + 32c + l (0 <= l < 32) being tile row 64c + 32m + l;
 *   down part, elements [2*I*H, 3*I*H): panel p = 0 .. ceil(H/256)-1 starts
 *     at 2*I*H + 256*p*I and holds the n = min(256, H - 256p) down rows
 *     256p .. 256p+n-1 as tile rows 0 .. n-1;
 *   a panel is its K/64 steps (K = H for gate/up, I for down) one after
 *     another; a step is its tile rows in order, 64 elements each (the row's
 *     elements 64s .. 64s+63), the 8-element chunk q of tile row R stored at
 *     chunk position q ^ ((R / 2) % 8).
 * For the shared expert call with nblocks = 1 and I = I_shared.  src and dst
 * are device pointers, 16-byte aligned, not overlapping; H and I follow the
 * layer's shape rules.  Asynchronous on `stream` like the layer calls. */
moe_status_t moe_tile_weights(int64_t nblocks, int32_t H, int32_t I, const void* src, void* dst, hipStream_t stream);

/* The same tiled order for 4-bit experts (moe_q4_t): rewrites nblocks blocks'
 * codes (3*H*I/2 bytes each) and group words (3*H*I/64 words each) from
 * codes / groups into codes_dst / groups_dst.  Element e of a tiled block
 * (the order above, without the chunk swizzle) is element f of the row-major
 * block; its code goes to code word e/8 (nibble e%8) and each group word to
 * position e/64, so a 4-bit K-step of a weight tile is one contiguous block
 * of codes (32 bytes per tile row) and one of group words (one per tile row).
 * With MOE_FLAG_TILED_WEIGHTS moe_layer_forward_q4 reads experts and shared
 * expert in this layout on every path, bit-identical to the row-major one.
 * It speeds up the grouped path (whole cache lines per K-step instead of a
 * quarter line of each row) and slows down the matrix-vector paths (a row's
 * codes come in 32-byte pieces, one per K-step), so it suits prefill-heavy
 * use; decode is faster on the row-major packing.  All four pointers are
 * device pointers, 16-byte aligned; the outputs overlap neither input nor
 * each other.  Asynchronous on `stream`. */
moe_status_t moe_tile_weights_q4(int64_t nblocks, int32_t H, int32_t I, const void* codes, const void* groups,
                                 void* codes_dst, void* groups_dst, hipStream_t stream);

/* moe_layer_forward for callers that cannot allocate or pass device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same layer, arguments and results, with the workspace
 * taken from a static per-device scratch array of the library instead of
 * a caller buffer.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library call.
 *   - The scratch holds MOE_NOALLOC_SCRATCH_BYTES (64 MiB) on every
 *     device the library runs on, for the life of the process; a call whose
 *     moe_workspace_size() is larger returns MOE_ERR_WORKSPACE_TOO_SMALL and
 *     enqueues nothing (at H=2048, E=256, top-8, I=512: up to 1,553
 *     rows on the grouped path; the decode and small-batch paths always fit).
 *   - The scratch of the current device is used (hipGetDevice): make the
 *     stream's device current.  The first call on a device looks up that
 *     device's scratch address once (hipGetSymbolAddress); make that first
 *     call outside graph capture.
 *   - All calls on one device share its scratch and leave their contents in
 *     it: calls that overlap in time on one device race (order them on one
 *     stream, or synchronise them).  No result depends on what a previous
 *     call left there. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_layer_forward_noalloc(const moe_desc_t* d, const void* x, const void* router_w,
                                       const void* expert_w, const void* shared_w, int top_k, void* out,
                                       hipStream_t stream, const moe_routing_t* routing);

/* Static description of a status code. */
const char* moe_status_string(moe_status_t s);

/* hipError_t (as int) behind the last MOE_ERR_HIP returned on this thread, 0 if none. */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_H */
