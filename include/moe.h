/*
 * moe.h - C ABI of a quantised mixture-of-experts feed-forward layer for one
 * AMD Instinct MI355X (gfx950): DeepSeek-V4.1-style routing with Q2_K / Q3_K
 * routed experts read against q8_1-quantised activations.
 *
 * What the layer computes, per token t of x [m, dim] (bf16):
 *   z = x W_R^T (f32 accumulation);  s = sqrt(softplus(z / gate_temp)), where
 *   softplus returns its argument above 20;  keys = s + bias;  T = the topk
 *   experts by key, descending, equal keys ordered by ascending expert id;
 *   G_i = s_{T_i} / (sum_j s_{T_j} + 1e-20) when norm_topk_prob and topk > 1,
 *   times route_scale;  y = sum_i G_i E_{T_i}(x) + y_shared(x);  out = bf16(y).
 *   A routed expert E(x) = W2 q8_1(h) with h = min(g,L) sigma(min(g,L))
 *   clip(u,-L,L) (no clamps when L <= 0), g = W1 q8_1(x), u = W3 q8_1(x); W1 and
 *   W3 are Q2_K blocks, W2 Q3_K blocks.
 * Sources: the metrale moe_v41 module documentation and moe_v41.rs source view
 * (docs.metrale.ai; fns route_from_logits, softplus, bf16_bytes; struct
 * MoeV41Cfg; methods forward / route / route_launch of struct MoeV41), and the
 * Open Model Atlas page "DeepSeek V4.1 · Mixture of experts" (router and
 * expert equations; the Gate / Expert / MoE code excerpts; config.json). The
 * Q2_K (84 B), Q3_K (110 B) and q8_1 (32 x int8 + fp16 d + fp16 d*sum) block
 * layouts are the public GGUF ones; the pages only name them.
 *
 * Conventions for every function:
 *   - returns MOE_OK (0) or a negative MOE_E* code; moe_strerror() names it;
 *   - no exception, abort or exit crosses this boundary;
 *   - pointers marked "device" are HIP device memory on the current device,
 *     borrowed for the duration of the work queued on `stream` (the caller
 *     keeps them alive until that work is done); "host" pointers are read
 *     before the call returns unless stated otherwise;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     every device-side call is asynchronous on it unless stated otherwise;
 *   - a context is not thread-safe: one host thread (or stream) per context;
 *     two calls on one context must not overlap on different streams.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)        /* an argument is out of range or NULL */
#define MOE_ENOMEM (-2)        /* a device or pinned-host allocation failed */
#define MOE_EHIP (-3)          /* a HIP runtime call failed */
#define MOE_ENONFINITE (-4)    /* a routing key (score + bias) was NaN */
#define MOE_ENOTRESIDENT (-5)  /* a picked expert had no slot and no host arena */
#define MOE_ESTATE (-6)        /* a call needs state that is not set (e.g. no slots) */
#define MOE_ESCRATCH (-7)      /* moe_forward_static: the call needs more than MOE_STATIC_SCRATCH_BYTES */

/* shared expert formats */
#define MOE_SHARED_NONE 0
#define MOE_SHARED_BF16 1      /* w1/w3 bf16 [inter, dim], w2 bf16 [dim, inter], row-major */
#define MOE_SHARED_KQUANT 2    /* w1/w3 Q2_K blocks [inter][dim/256], w2 Q3_K blocks [dim][inter/256],
                                  each in the panel order of moe_expert_layout (moe_pack_expert) */

/* Layer configuration (the fields of metrale's MoeV41Cfg). */
typedef struct moe_cfg {
    int32_t dim;            /* model dim D: a multiple of 256, 256..8192 */
    int32_t inter;          /* expert intermediate dim I: a multiple of 256, 256..8192 */
    int32_t n_routed;       /* routed experts E: 1..1024 */
    int32_t topk;           /* experts per token k: 1..min(E, 64) */
    float gate_temp;        /* router temperature, > 0 */
    int32_t norm_topk_prob; /* nonzero: renormalise the picked scores (only when topk > 1) */
    float route_scale;      /* routing weight multiplier */
    float swiglu_limit;     /* clamp L; <= 0 disables both clamps */
    int32_t max_tokens;     /* largest m any call may pass: 1..65536; sizes the scratch */
    int32_t expert_fmt;     /* MOE_EXPERT_KQUANT (0) or MOE_EXPERT_MXFP4 (1): the routed experts' format */
} moe_cfg;

/* Routed expert formats (moe_cfg.expert_fmt).
 * MOE_EXPERT_KQUANT: GGUF Q2_K gate/up and Q3_K down blocks, read against q8_1
 *   activations (metrale moe_v41 module documentation).
 * MOE_EXPERT_MXFP4: the upstream checkpoint's FP4 experts (Open Model Atlas,
 *   "DeepSeek V4.1 · Mixture of experts": float4_e2m1fn_x2 weights): per 32
 *   consecutive weights of a row one E8M0 scale byte 2^(E-127), and 32 e2m1
 *   codes, two per byte with the even weight in the low nibble (the OCP
 *   microscaling layout; the pages give only the element type). In plain
 *   order a matrix [rows, cols] is its codes [rows, cols/2] followed by its
 *   scales [rows, cols/32]; slots hold the tiled order of moe_expert_layout
 *   (moe_pack_expert). The experts run on the unquantised bf16 x with f32
 *   accumulation, h rounded to bf16 before W2. The shared expert must then be
 *   bf16 or none. */
#define MOE_EXPERT_KQUANT 0
#define MOE_EXPERT_MXFP4 1

/* One layer's resident weights (metrale's MoeV41LayerWeights). Routed experts
 * are not here: they are found through the slot table (moe_set_slots). */
typedef struct moe_weights {
    const void* router_w;      /* device, bf16 [n_routed, dim] row-major */
    const float* router_bias;  /* device, f32 [n_routed] */
    int32_t shared_fmt;        /* MOE_SHARED_* */
    const void* shared_w1;     /* device; see MOE_SHARED_* for the layout */
    const void* shared_w3;     /* device */
    const void* shared_w2;     /* device */
} moe_weights;

/* Counters of the calls since creation or moe_reset_stats: the fields of
 * metrale's MoeV41Timing (moe_v41.rs source view, struct MoeV41Timing: route,
 * fetch and compute milliseconds, hits, misses, bytes read), plus the near-tie
 * count that the stated pass criterion for the expert indices asks to be
 * reported. Only calls made with a host arena read the routing back and
 * stream. moe_get_stats and moe_reset_stats synchronise the device first
 * (all queued work of the context, and the copies). */
typedef struct moe_stats {
    uint64_t calls;         /* moe_forward / moe_forward_ex calls */
    uint64_t hits;          /* distinct picked experts already resident at a streamed call's start */
    uint64_t misses;        /* picked experts copied from the host arena */
    uint64_t bytes_copied;  /* host-to-device bytes of those copies */
    uint64_t waves;         /* slot waves run by streamed calls */
    double route_ms;        /* host time waiting for the routing read-back (includes the queued work before it) */
    double fetch_ms;        /* device time of the miss copies (events on the copy stream) */
    double compute_ms;      /* device time from the first expert kernel to the layer's last kernel (the
                               combine), summed over the calls made with a host arena or with profiling
                               on (moe_set_profiling); other calls carry no events and add nothing */
    uint64_t near_ties;     /* tokens (of moe_forward, moe_forward_ex and moe_route calls) whose k-th
                               largest key exceeded the largest key not picked by less than 1e-5, in the
                               device's own f32 keys: where rounding alone may change the selection */
} moe_stats;

typedef struct moe_ctx moe_ctx;

/* Create a context on the current HIP device: validates cfg, allocates the
 * scratch for cfg->max_tokens tokens. *out is set only on success.
 * The context is the counterpart of metrale's struct MoeV41 (moe_v41.rs source
 * view): built from a MoeV41Cfg, it owns the per-call device buffers that
 * struct lists (logits, the q8_1 activations, gate/up/h/down outputs, the
 * token rows and weights grouped by expert, the slot table) sized for
 * max_tokens, whose limit route_launch enforces (MoeV41 struct documentation:
 * m outside 1..=max_tokens is an error), plus the side stream and events of
 * shared_side. MOE_EINVAL (bad cfg / NULL), MOE_ENOMEM, MOE_EHIP. */
int moe_create(const moe_cfg* cfg, moe_ctx** out);

/* Free what the context owns (scratch, table, streams, events): the buffers
 * of struct MoeV41 above. Caller-owned memory (slot arena, host arena,
 * weights) is not touched. Synchronises the device first. NULL is accepted. */
int moe_destroy(moe_ctx* ctx);

/* Byte layout of one routed expert's slice (the analogue of metrale's
 * arena_of): [W1 Q2_K | W3 Q2_K | W2 Q3_K]; W1/W3 hold inter rows of dim/256
 * blocks of 84 B, W2 dim rows of inter/256 blocks of 110 B, the GGUF block
 * bytes unchanged. Inside each matrix the blocks are in panel order: panels
 * of 8 consecutive rows, each panel holding its rows' block 0, then their
 * block 1, ... (block s of row r at ((r/8)*nsb + s)*8*B + (r%8)*B, nsb blocks
 * per row of B bytes), so that every 8-row tile and every block column of a
 * panel is one contiguous run. moe_pack_expert turns a slice in plain GGUF
 * row order into this layout. With expert_fmt MOE_EXPERT_MXFP4 the slice is
 * [W1 | W3 | W2] of MXFP4 matrices, each [rows, cols] in tiles of 64 rows x 128
 * columns: tile (rows 64i.., columns 128s..) has index t = i * (cols/128) + s,
 * its codes (64 rows x 64 bytes, row after row) at byte 4096 t of the matrix,
 * and its scales (64 rows x 4 bytes) at byte rows*cols/2 + 256 t, after all
 * the codes. All four outputs are required. MOE_EINVAL on a bad cfg. */
int moe_expert_layout(const moe_cfg* cfg, size_t* slot_bytes, size_t* off_w1, size_t* off_w3,
                      size_t* off_w2);

/* Reorder one expert slice from plain GGUF row order (each matrix's rows one
 * after another, a row's blocks consecutive) into the slot layout of
 * moe_expert_layout. src and dst: device, slot_bytes each, 2-byte aligned, not
 * overlapping; asynchronous on `stream`. Used for routed expert slots, host
 * arena slices (pack on the device, then copy) and a K-quant shared expert.
 * MOE_EINVAL for a bad cfg, NULL or overlapping buffers; MOE_EHIP on a launch
 * error. (A layout step of this library: the blocks themselves are the
 * pages' GGUF Q2_K / Q3_K blocks, untouched.) For MXFP4 experts the source is
 * the plain layout (each matrix's codes [rows, cols/2] then its scales
 * [rows, cols/32]) and the destination the tiles above; codes and scales are
 * moved, not changed. */
int moe_pack_expert(const moe_cfg* cfg, const void* src, void* dst, void* stream);

/* Give the context a caller-owned device arena of n_slots slices of slot_bytes
 * (256-byte aligned base) and reset the slot table to "nothing resident".
 * The arena is the ExpertArena whose slots the ExpertLru fills with the picked
 * experts' raw slices (metrale moe_v41 module documentation; the analogue of
 * arena_of on the MoeV41 struct documentation), and the table the
 * [n_routed] i32 slot_table of struct MoeV41 (moe_v41.rs source view: -1 = not
 * resident). MOE_EINVAL for NULL / n_slots < 1 / a misaligned base. */
int moe_set_slots(moe_ctx* ctx, void* arena_dev, int32_t n_slots);

/* Slot table (metrale's slot_table_set): expert -> slot, -1 = not resident.
 * bind: the caller has put the expert's slice in that slot; MOE_EINVAL for an
 * id out of range or a slot already bound to another expert; MOE_ESTATE
 * without an arena. evict: forget the expert's slot. slot_of: read it. The
 * device copy of the table is refreshed on the next forward/route call. */
int moe_slot_bind(moe_ctx* ctx, int32_t expert, int32_t slot);
int moe_slot_evict(moe_ctx* ctx, int32_t expert);
int moe_slot_of(const moe_ctx* ctx, int32_t expert, int32_t* slot);

/* Optional page-locked host arena holding every routed expert's slice,
 * expert e at host + e * expert_stride (expert_stride >= slot_bytes): the
 * ExpertSource that misses are read from (metrale moe_v41 module
 * documentation; the MoeV41 struct documentation's forward takes the
 * ExpertLru and the source). With it,
 * every moe_forward reads its picks back (one host wait), copies the picked
 * experts that are not resident into device slots (least recently used slots
 * reused, hipMemcpyAsync on the context's copy stream, fenced by events) and
 * rebinds the slot table. When the distinct picks outnumber the slots the
 * experts run in waves of half the slots each (one wave's copies overlap the
 * previous wave's kernels). The memory must be page-locked (hipHostMalloc or
 * an equivalent pinned allocation); NULL disables streaming. Slots the caller
 * bound stay usable and become part of the LRU. MOE_EINVAL for a stride below
 * slot_bytes; MOE_ENOMEM / MOE_EHIP when the copy stream or its pinned
 * buffers cannot be made. */
int moe_set_host_arena(moe_ctx* ctx, const void* pinned_host, size_t expert_stride);

/* Routing only (metrale's route / route_launch, with the selection on the
 * device): writes weights_out f32 [m, topk] and idx_out i32 [m, topk] (device),
 * each token's picks in descending key order. Asynchronous. MOE_EINVAL when m
 * is outside 1..max_tokens or a pointer is NULL. A NaN key is reported by
 * moe_check as MOE_ENONFINITE (NaN keys are ordered last). */
int moe_route(moe_ctx* ctx, const moe_weights* w, const void* x_bf16, int32_t m, float* weights_out,
              int32_t* idx_out, void* stream);

/* The whole layer (metrale's forward): out_bf16 [m, dim] bf16 (device,
 * caller-owned). Asynchronous when every picked expert is resident or no host
 * arena is set; with a host arena it blocks once on the routing read-back and
 * then streams the misses. A picked expert that is not resident without a host
 * arena contributes zero and is reported by moe_check as MOE_ENOTRESIDENT. */
int moe_forward(moe_ctx* ctx, const moe_weights* w, const void* x_bf16, int32_t m, void* out_bf16,
                void* stream);

/* moe_forward that also writes the routing (either pointer may be NULL). */
int moe_forward_ex(moe_ctx* ctx, const moe_weights* w, const void* x_bf16, int32_t m, void* out_bf16,
                   float* weights_out, int32_t* idx_out, void* stream);

/* How a call of m tokens with this shared-expert format (MOE_SHARED_*) runs, for
 * callers that account the bytes each kernel class reads (the per-kernel times
 * of moe_kernel_times): which routing and expert kernels run, and where the
 * rows of a bf16 shared expert are computed. The expert path holds for calls
 * whose picks are all resident or fit one slot wave (several waves run the
 * GEMV kernels). The selection rule follows the metrale moe_v41 module
 * documentation (GEMVs for small groups, MMQ above eight rows) as this library
 * applies it per call. MOE_EINVAL for NULL, m outside 1..max_tokens or a bad
 * shared_fmt. */
#define MOE_PATH_DECODE 0   /* m <= 8, K-quant experts: gate/up writing q8_1(h), then down + combine */
#define MOE_PATH_GEMV 1     /* chunked GEMV kernels (MXFP4 experts up to 8 tokens, slot waves, MIXED groups) */
#define MOE_PATH_MMQ 2      /* the expert-grouped matrix-core kernels (above 8 tokens) */
typedef struct moe_plan {
    int32_t small_routing;      /* 1: one workgroup runs the top-k and bucketing (m <= 8, m * topk <= 512;
                                   one token on the K-quant decode kernels: the last router
                                   workgroup, in the router launch, so no top-k launch follows) */
    int32_t expert_path;        /* MOE_PATH_* */
    int32_t shared_rows_router; /* bf16 shared gate/up rows computed by extra workgroups of the router launch */
    int32_t shared_rows_topk;   /* bf16 shared down rows (0..n-1) in the top-k launch (0 when there is none) */
    int32_t shared_rows_gateup; /* the rest of them in the routed gate/up launch */
} moe_plan;
int moe_plan_call(const moe_ctx* ctx, int32_t m, int32_t shared_fmt, moe_plan* out);

/* How a call of more than 8 tokens runs the routed experts, by group size (the
 * rows that picked one expert). MOE_DISPATCH_MMQ (the default): every group on
 * the int8 matrix-core (MMQ) kernels, the smallest in 16-row tiles.
 * MOE_DISPATCH_MIXED: the rule of the metrale moe_v41 module documentation,
 * GEMVs for groups of up to eight rows and MMQ above; on gfx950 the dot4 GEMV
 * kernels stream such groups several times slower than the MMQ tiles, so it
 * is not the default. Calls of up to 8 tokens always use the GEMV kernels.
 * Takes effect for the calls queued after it. MOE_EINVAL for NULL or another
 * value. */
#define MOE_DISPATCH_MMQ 0
#define MOE_DISPATCH_MIXED 1
int moe_set_dispatch(moe_ctx* ctx, int32_t mode);

/* The layer's activation quantiser alone (q8_1 of bf16 rows), exposed so its
 * output can be checked bit for bit: x_bf16 [rows, cols] (device, 16-byte
 * aligned, cols a multiple of 32); q_out int8 [rows, cols] and d_out f32
 * [rows, cols/32] holding fp16(d) (device). Per 32 values: d = amax/127,
 * q = round-half-away-from-zero(x/d) with the unrounded d (0 when d = 0).
 * Asynchronous. MOE_EINVAL for NULL, rows < 1 or a bad cols. */
int moe_quantize_q8_1(const void* x_bf16, int32_t rows, int32_t cols, int8_t* q_out, float* d_out, void* stream);

/* Synchronise `stream` and return (then clear) the device error word of the
 * calls queued so far: MOE_OK, MOE_ENONFINITE or MOE_ENOTRESIDENT. The first
 * is metrale's route_from_logits panic on a NaN key (moe_v41.rs source view),
 * raised here as a flag by the device top-k; the second a pick whose slot
 * table entry is -1 (struct MoeV41's slot_table) with no source to read it
 * from. Other counters (near ties) are left alone. */
int moe_check(moe_ctx* ctx, void* stream);

/* Per-kernel timing for benchmarks. With profiling on, every kernel launch of
 * moe_forward / moe_forward_ex is bracketed by HIP events recorded on the
 * call's stream (a small gap is added between kernels). moe_kernel_times
 * synchronises the device and fills, for kernel class i < n (MOE_K_* order),
 * the summed milliseconds and the number of launches since profiling was
 * switched on or last read; then it restarts the sums. n < MOE_K_COUNT reads
 * the first n classes. MOE_EINVAL for NULL. */
#define MOE_K_ROUTER 0        /* router logits (+ q8_1 of x in the same launch) */
#define MOE_K_QUANT 1         /* q8_1 of the SwiGLU output h */
#define MOE_K_TOPK 2          /* selection and weights (+ bucketing when m <= 8) */
#define MOE_K_BUCKET 3        /* token -> expert bucketing (m > 8) */
#define MOE_K_GATEUP 4        /* routed (and K-quant shared) gate/up + SwiGLU */
#define MOE_K_SHARED_GATEUP 5 /* bf16 shared gate/up + SwiGLU */
#define MOE_K_DOWN 6          /* routed (and K-quant shared) down */
#define MOE_K_SHARED_DOWN 7   /* bf16 shared down */
#define MOE_K_COMBINE 8       /* weighted combine + bf16 store */
#define MOE_K_COUNT 9
int moe_set_profiling(moe_ctx* ctx, int32_t on);
int moe_kernel_times(moe_ctx* ctx, double* ms_sum, int64_t* launches, int32_t n);

/* Copy out / clear the counters. */
int moe_get_stats(const moe_ctx* ctx, moe_stats* out);
int moe_reset_stats(moe_ctx* ctx);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * path of moe_forward_ex (m <= 8 tokens, m * topk <= 512, K-quant experts),
 * with no context. Its scratch (logits, q8_1 of x, the routing, chunk list and
 * q8_1 records of h, the bf16 shared expert's h and output) is a file-scope
 * device array of MOE_STATIC_SCRATCH_BYTES, one per GPU, held until the process
 * ends; nothing is allocated, by this call or by any call it makes. The same
 * kernels run in the same order as moe_forward_ex, so the outputs are
 * identical to a context's.
 *   cfg         the layer (cfg->max_tokens is ignored; expert_fmt must be
 *               MOE_EXPERT_KQUANT)
 *   w           as for moe_forward (a bf16 shared expert's rows ride in the
 *               routed launches, as moe_plan_call describes)
 *   arena       device, the routed experts' slots (moe_expert_layout), 256-byte aligned
 *   slot_table  device, i32 [n_routed]: expert -> slot, -1 = not resident
 *   x_bf16, out_bf16, weights_out, idx_out   as for moe_forward_ex
 *   status      device, i32 [2] or NULL: the kernels OR MOE error flags into
 *               word 0 (1: a NaN key, 2: a picked expert not resident) and add
 *               the near-tie count to word 1; the caller clears it. With NULL
 *               these are dropped.
 * Every call on a GPU uses that GPU's one array, so two calls that overlap on a
 * GPU (different streams, threads) race; calls queued on one stream do not.
 * The array keeps the last call's contents; every buffer a call reads is
 * written earlier in the same call, except the one-token router launch's
 * arrival counters at its start, which every call leaves at zero (the array
 * starts zeroed). MOE_EINVAL for a bad cfg, MXFP4 experts,
 * NULL or misaligned pointers, m < 1, m > 8 or m * topk > 512; MOE_ESCRATCH if
 * the call needs more than MOE_STATIC_SCRATCH_BYTES (no valid cfg does at
 * m <= 8); MOE_EHIP on a runtime error. */
#define MOE_STATIC_SCRATCH_BYTES (8u << 20)
int moe_forward_static(const moe_cfg* cfg, const moe_weights* w, const void* arena, const int32_t* slot_table,
                       const void* x_bf16, int32_t m, void* out_bf16, float* weights_out, int32_t* idx_out,
                       int32_t* status, void* stream);

/* Static text for a status code. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
