/*
 * fd.h - C ABI of the frame-synchronous batched decode step (gfx950).
 *
 * The problem this library serves (PersonaPlex 7B page, sections "What
 * Real-time Means for a Full-duplex Agent", "Compressing the Temporal KV
 * cache" and "A server built around the conversation clock"; Nemotron
 * VoiceChat case study, "The solution" and "Under the hood"; its
 * profile.json, serving_profile):
 *
 *   - every session advances one frame per step through a decoder stack;
 *   - all sessions advance together on one clock, in fixed-shape session
 *     slots; a new session takes a free slot without changing what the GPU
 *     executes;
 *   - one read of the weights is shared by every session in the step;
 *   - conversation state (the temporal cache) stays resident between steps;
 *     it is stored in FP8 (or fp32 for the talker-style stack) and holds at
 *     most a fixed window of frames (1500 = 120 s in the profile);
 *   - a serving profile is fixed per (model, session capacity, context
 *     length) ahead of time;
 *   - the GPU does not return to the CPU per operation, and no client I/O
 *     runs inside the step.
 *
 * Conventions for every call:
 *   - The return value is an fd_status: FD_OK (0) or a negative code.
 *   - All argument checks run on the host before anything is changed, so a
 *     call that fails has no effect.  No C++ exception crosses this ABI.
 *   - "device pointer" means memory allocated on the ctx's GPU (the Python
 *     binding uses torch uint8 tensors); "host pointer" means CPU memory.
 *   - A ctx is not thread-safe: one host thread and one stream per ctx.
 *   - Streams are hipStream_t values passed as void* (NULL = the default
 *     stream).
 *   - Errors raised by the HIP runtime are reported as FD_E_DEVICE by the
 *     call that sees them; fd_last_error() gives the message.
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fd_status;

#define FD_OK             0
#define FD_E_INVAL       (-1) /* null/misaligned pointer or out-of-range argument */
#define FD_E_UNSUPPORTED (-2) /* a shape or type the kernels do not implement */
#define FD_E_NOSLOT      (-3) /* fewer free slots than requested */
#define FD_E_BADSLOT     (-4) /* slot id out of range, or not allocated */
#define FD_E_CTXFULL     (-5) /* an active slot has used its whole window */
#define FD_E_DEVICE      (-6) /* HIP runtime error or device-side fault flag */
#define FD_E_STATE       (-7) /* call not valid in the ctx's current state */

/* Storage types. */
#define FD_F32       0
#define FD_BF16      1
#define FD_FP8_E4M3  2 /* OCP E4M3 ("e4m3fn"): bias 7, max 448, one NaN pattern */

/*
 * Form of the projections' session-row inputs in FD_BF16 profiles (bf16 or
 * FP8 weights), fd_config.proj_in.  The pages keep weights and activations
 * in BF16 (PersonaPlex 7B page, "Compressing the Temporal KV cache"); these forms carry the
 * rows between phases at least that precisely:
 *   FD_PROJ_F16: each row rounded to fp16 (11 significant bits, nearest
 *     even).  bf16 weights are held as fp16 codes of w / 2^e with one
 *     power of two per output row (the row's largest magnitude lands in
 *     [2^14, 2^15)), exact for every entry of at least 2^-28 of that
 *     largest; FP8 weight codes convert to fp16 exactly.  The matrix cores
 *     multiply fp16 operands with fp32 sums, and the row scales multiply
 *     the sums.  A row value beyond fp16's range (|v| > 65504) makes that
 *     session's outputs non-finite; other sessions are unaffected.
 *   FD_PROJ_BF16X2: each row as two bf16 parts, hi = bf16(v) and
 *     lo = bf16(v - hi) (~16 significant bits), multiplied with the bf16
 *     (or FP8-decoded) weights: twice the matrix-core work and row loads of
 *     FD_PROJ_F16.
 *   FD_PROJ_AUTO: FD_PROJ_F16.
 * Both forms run in either exec_mode.  FD_F32 profiles take FD_PROJ_AUTO
 * (fp32 rows); other values give FD_E_UNSUPPORTED.  FD_F32 stacks multiply
 * in fp32 (exact fp32 products, fp32 sums; no TF32-like reduction).  As a
 * measurement option only (environment FD_TUNE containing "x3=1" at
 * fd_plan / fd_init, FD_EXEC_KERNELS), their projections and the depth
 * input projection instead multiply as three bf16 products per k-step:
 * each weight is stored as hi = bf16(w) and lo = bf16(w - hi), each
 * session row value is split the same way as it is loaded, and the matrix
 * cores add w_lo*x_hi + w_hi*x_lo + w_hi*x_hi with fp32 sums (~16
 * significant bits per operand; the dropped w_lo*x_lo term is below 2^-16
 * of the product), in the weight bytes of fp32.
 */
#define FD_PROJ_AUTO   0
#define FD_PROJ_F16    1
#define FD_PROJ_BF16X2 2

/*
 * Serving profile: the decoder shape, slot capacity and window, fixed for
 * the life of a ctx (Nemotron case study, "Under the hood": profiles are
 * compiled per model, session capacity and context length).
 *
 * Supported (w_dtype / act_dtype):
 *   FD_F32 / FD_F32, FD_BF16 / FD_BF16: weights in that type;
 *   FD_FP8_E4M3 / FD_BF16: the caller passes bf16 weight tensors (as for
 *     FD_BF16) and fd_init quantises each output row to OCP E4M3 codes of
 *     w / scale with scale = max|row| / 448 (1 for a zero row), one fp32
 *     scale per row; the step uses scale * decode(code).  Not combined with
 *     a depth stack or FD_EXEC_WALK.
 * kv_dtype in {FD_F32, FD_FP8_E4M3}; head_dim in {64, 128, 256}; n_heads a
 * multiple of n_kv_heads with n_heads / n_kv_heads in {1, 2, 4}; d_model,
 * d_ffn and n_heads*head_dim multiples of 256 (bf16), 512 (FP8 weights) or
 * 128 (fp32); max_slots in 1..4096; max_context in 1..65536.  An optional
 * depth stack (depth_steps > 0) runs after the main stack on every frame,
 * for depth_steps sequential sub-steps with its own fp32 cache cleared
 * every frame; it requires w_dtype == FD_F32 and kv_dtype == FD_F32.
 */
typedef struct {
    int32_t n_layers;
    int32_t d_model;
    int32_t n_heads;      /* query heads */
    int32_t n_kv_heads;   /* key/value heads (GQA: query head h reads kv head h*n_kv_heads/n_heads) */
    int32_t head_dim;
    int32_t d_ffn;        /* SwiGLU hidden width */
    float rms_eps;        /* RMSNorm: x * (mean(x^2) + eps)^(-1/2) * g */
    float rope_base;      /* rotary angle of pair i at position p: p * base^(-2i/head_dim) */
    int32_t max_slots;    /* S_cap: session slots, fixed launch shape */
    int32_t max_context;  /* T_max: frames a slot's cache holds */
    int32_t w_dtype;      /* FD_F32, FD_BF16 or FD_FP8_E4M3 (see above) */
    int32_t act_dtype;    /* w_dtype, or FD_BF16 with FD_FP8_E4M3 weights */
    int32_t kv_dtype;     /* FD_F32 or FD_FP8_E4M3 */
    int32_t depth_steps;  /* 0 = no depth stack */
    int32_t depth_layers;
    int32_t depth_d;
    int32_t depth_heads;
    int32_t depth_kv_heads;
    int32_t depth_head_dim;
    int32_t depth_ffn;
    int32_t exec_mode;    /* FD_EXEC_KERNELS (0) or FD_EXEC_WALK (1), see below */
    int32_t kv_ring;      /* 0: fixed window; 1: rolling window, see below */
    int32_t vocab;        /* 0: no output head; else V, a multiple of 16 (<= 2^20): see fd_step_tokens */
    int32_t proj_in;      /* FD_PROJ_AUTO, FD_PROJ_F16 or FD_PROJ_BF16X2 (see above) */
} fd_config;

/*
 * Window of a session's cache.  kv_ring = 0: a session holds at most
 * max_context frames; stepping a slot whose position reached max_context
 * fails with FD_E_CTXFULL (the 1500-frame, 120 s window of the case study's
 * profile.json serving profile).  kv_ring = 1: sessions continue past the
 * window (the vLLM-Omni recipe's realtime configuration leaves session
 * length unbounded, "Performance"): frame t's key/value live in cache
 * position t mod max_context, the frame at index p attends to frames
 * max(0, p - max_context + 1) .. p, and its rotary angle uses the absolute
 * index p.  Positions then run up to 2^30 (fd_set_position accepts them);
 * the cache layout and fd_kv_write still address cache positions
 * 0 .. max_context - 1.
 */

/*
 * Execution of a step.  FD_EXEC_KERNELS: fd_step enqueues a fixed sequence
 * of kernels (no host work or synchronisation between them).
 * FD_EXEC_WALK: fd_step enqueues ONE persistent cooperative launch (after a
 * one-block reset of its barrier counter) whose workgroups, as many as fit
 * co-resident (one per CU for the larger shapes), walk
 * the whole step -- embed, every layer's phases, final norm, and the depth
 * stack's loop when there is one -- with device-side grid barriers between
 * dependent phases, requesting each next phase's weights (or first cached
 * keys) before waiting at the barrier (the case study's persistent program,
 * "Under the hood").  Compiled for three families of shapes; others give
 * FD_E_UNSUPPORTED at fd_plan: fp32 stacks with head_dim 64, one query head
 * per kv head and no depth stack (at most 32 slots); fp32 stacks with
 * head_dim 256, 4 query heads per kv head and a depth stack of head_dim 128
 * with one query head per kv head (at most 64 slots); bf16 weights with an
 * FP8 cache, head_dim 128, one query head per kv head, no depth stack, at
 * most 5 row tiles of 16 slots per m-group of the projections (up to 80
 * slots, or more than 128, where the rows split into m-groups).
 * A barrier wait that times out makes the launch stop early and the next
 * fd_sync return FD_E_DEVICE; the slots that were active are then stale
 * (their device positions and newest cache entries are unknown): fd_step
 * and fd_step_static return FD_E_STATE until each is given a position with
 * fd_set_position or freed with fd_free.
 */
#define FD_EXEC_KERNELS 0
#define FD_EXEC_WALK 1

/* Byte sizes of the four caller-allocated device buffers. */
typedef struct {
    uint64_t packed_weights; /* weights in the kernels' tile layout + constant tables */
    uint64_t kv_arena;       /* the slot-pooled cache, layout in fd_kv_view */
    uint64_t workspace;      /* activations, partial results, counters */
    uint64_t slot_table;     /* device copy of per-slot active flag and position, and the
                                order attention takes the slots in */
} fd_sizes;

/*
 * One decoder layer's parameters: device pointers to row-major matrices in
 * nn.Linear [out, in] layout, in w_dtype (bf16 as raw 16-bit values), and
 * fp32 RMSNorm gains.
 *   wq [n_heads*head_dim][d]   wk, wv [n_kv_heads*head_dim][d]
 *   wo [d][n_heads*head_dim]   w_gate, w_up [d_ffn][d]   w_down [d][d_ffn]
 *   g_attn, g_ffn [d] (fp32)
 */
typedef struct {
    const void* wq;
    const void* wk;
    const void* wv;
    const void* wo;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const float* g_attn;
    const float* g_ffn;
} fd_layer_weights;

/*
 * All parameters.  `layers` and `depth_layers` are HOST arrays of
 * fd_layer_weights whose members are device pointers.
 *   g_final [d] fp32 (device)
 *   kv_scale [n_layers][2 (K|V)][n_kv_heads] fp32 (device); required for
 *     FD_FP8_E4M3 caches (a cached entry is stored as code(x / scale) and
 *     read back as scale * decode(code)); ignored for FD_F32 caches
 *   w_in [depth_d][d_model], depth_layers[depth_layers], depth_g_final
 *     [depth_d]: the depth stack (only when depth_steps > 0)
 *   w_head [vocab][d_model] in w_dtype: the output head (only when vocab > 0)
 */
typedef struct {
    const fd_layer_weights* layers;
    const float* g_final;
    const float* kv_scale;
    const void* w_in;
    const fd_layer_weights* depth_layers;
    const float* depth_g_final;
    const void* w_head;
} fd_weights;

/* The four device buffers, each at least the size fd_plan reports and
 * 256-byte aligned.  The ctx borrows them until fd_destroy. */
typedef struct {
    void* packed_weights;
    void* kv_arena;
    void* workspace;
    void* slot_table;
} fd_buffers;

/*
 * Cache layout (returned by fd_kv_layout).  Slot-major, one contiguous
 * region per session:
 *   element (slot s, layer l, kv (0 = K, 1 = V), kv-head g, position t, dim d)
 *   lives at byte  base + ((((s*L + l)*2 + kv)*H_kv + g)*T_max + t)*D*elem_bytes
 *                  + d*elem_bytes
 * Key vectors are stored after the rotary embedding.  For FP8 caches each
 * byte is an OCP E4M3 code of value / kv_scale[l][kv][g].
 */
typedef struct {
    void* base;              /* device pointer to the arena */
    uint64_t slot_stride;    /* bytes between consecutive slots */
    uint64_t layer_stride;   /* bytes between consecutive layers of a slot */
    uint64_t kv_stride;      /* bytes between the K and V blocks of a layer */
    uint64_t head_stride;    /* bytes between kv heads */
    uint64_t pos_stride;     /* bytes between positions (head_dim * elem_bytes) */
    int32_t elem_bytes;      /* 1 (FP8) or 4 (fp32) */
    int32_t n_layers, n_kv_heads, max_context, head_dim, max_slots;
    const float* kv_scale;   /* device copy of the scales [L][2][H_kv] (NULL for fp32) */
    int32_t* slot_active;    /* device int32 [max_slots] */
    int32_t* slot_pos;       /* device int32 [max_slots]: next frame index */
} fd_kv_view;

typedef struct fd_ctx fd_ctx;

/* Pure host function: validates cfg and reports the buffer sizes.
 * FD_E_INVAL for null pointers, FD_E_UNSUPPORTED for shapes outside the
 * supported set. */
fd_status fd_plan(const fd_config* cfg, fd_sizes* out);

/*
 * Creates a ctx.  Validates cfg and every pointer, then on `stream`:
 * repacks the weights into buf->packed_weights (the caller's weight
 * tensors may be freed once the stream has passed this point), writes the
 * constant tables (rotary cos/sin computed on the host in double and
 * rounded to fp32; FP8 scales), clears the counters in the workspace and
 * marks every slot inactive.  The ctx borrows `buf` until fd_destroy.
 * Errors: FD_E_INVAL, FD_E_UNSUPPORTED, FD_E_DEVICE.
 */
fd_status fd_init(const fd_config* cfg, const fd_weights* w, const fd_buffers* buf,
                  void* stream, fd_ctx** out);

/*
 * Admits n new sessions at frame position 0.  Takes the n lowest-numbered
 * free slots and writes their ids, ascending, to the host array slots_out.
 * All or nothing: FD_E_NOSLOT (and no change) if fewer than n slots are
 * free.  The change reaches the device with the next fd_step on the ctx's
 * stream; the launch shape of fd_step does not change.  The slot's old
 * cache bytes are not cleared: positions >= the slot's position are never
 * read.
 */
fd_status fd_alloc_slots(fd_ctx* ctx, int32_t n, int32_t* slots_out);

/*
 * Advances every active slot by one frame.
 *   x_in   device [max_slots][d_model] in act_dtype: slot s's new frame
 *          embedding in row s; rows of inactive slots are ignored.
 *   y_out  device [max_slots][d_model] in act_dtype: the final-normed
 *          output; rows of inactive slots are set to 0.
 *   depth_out device [max_slots][depth_steps][depth_d] in act_dtype, or
 *          NULL when the profile has no depth stack; inactive rows set to 0.
 * x_in, y_out and depth_out must be 16-byte aligned (FD_E_INVAL, no launch).
 * Each active slot's new key/value are appended at its position, which then
 * advances by one.  Enqueued on `stream` without waiting (the caller syncs);
 * no host I/O and no allocation.  With FD_EXEC_KERNELS it enqueues the fixed
 * kernel sequence of the profile (per layer: the QKV projection, attention,
 * the O projection, gate/up and down, plus a k-split reduction after a
 * projection split over K; embed before and the final norm after); with
 * FD_EXEC_WALK one persistent launch.  FD_E_CTXFULL (and no launch) if an
 * active slot's position equals max_context; FD_E_STATE (no launch) while a
 * slot is stale (see FD_EXEC_WALK).
 */
fd_status fd_step(fd_ctx* ctx, const void* x_in, void* y_out, void* depth_out, void* stream);

/*
 * fd_step followed by the output head on the same stream: for every active
 * slot, logits = y . W_head^T over the vocabulary (fp32 accumulation of the
 * final-normed output, before its rounding to act_dtype) and the greedy
 * token argmax(logits), ties to the lowest index -- one text token per frame,
 * chosen greedily (vLLM-Omni recipe, "Summary" and "Key flags").
 *   tokens_out device int32 [max_slots]: the token of each active slot, -1
 *          for inactive slots.
 *   logits_out device fp32 [max_slots][vocab] or NULL: the logits (rows of
 *          inactive slots 0).  Rows max_slots and beyond are never written.
 * FD_E_INVAL if the profile has no head (vocab 0), tokens_out is NULL or not
 * 4-byte aligned, or logits_out is not 16-byte aligned; otherwise as
 * fd_step.
 */
fd_status fd_step_tokens(fd_ctx* ctx, const void* x_in, void* y_out, void* depth_out,
                         int32_t* tokens_out, float* logits_out, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): fd_step
 * with the library's own static device scratch as the step's workspace.
 * The scratch is a file-scope device array of FD_STATIC_SCRATCH_BYTES bytes
 * (64 MiB) that every GPU the library runs on holds until the process ends;
 * the step's activations, projection planes, k-split partial sums, norm
 * partial sums, attention chunk partials and the depth stack's per-frame
 * cache live there instead of in the fd_init workspace.  Arguments, outputs
 * and effects on the cache and positions are those of fd_step; x_in, y_out
 * and depth_out are still the caller's.  Allocates nothing: no hipMalloc,
 * hipFree, event creation or other allocating call (the ctx's fd_profile
 * timing is skipped for this call).  The current device must be the ctx's
 * (FD_E_INVAL otherwise); its first call on a GPU resolves that GPU's copy
 * of the array.
 * FD_E_UNSUPPORTED (no launch) for FD_EXEC_WALK profiles, whose phase
 * layout is built into the fd_init workspace, and for profiles whose step
 * workspace (fd_sizes.workspace) exceeds FD_STATIC_SCRATCH_BYTES.
 * All calls on one GPU share that GPU's array and keep the last call's
 * contents: calls that overlap on one GPU (several ctxs or streams, or
 * several host threads) race and give undefined results -- serialize them.
 * Counters that must start at zero are cleared by each call.
 */
#define FD_STATIC_SCRATCH_BYTES (64ull << 20)
fd_status fd_step_static(fd_ctx* ctx, const void* x_in, void* y_out, void* depth_out, void* stream);

/*
 * Ends sessions: marks the n slots (host array) free.  FD_E_BADSLOT and no
 * change if any id is out of range, not allocated, or repeated.
 */
fd_status fd_free(fd_ctx* ctx, const int32_t* slots, int32_t n);

/* Releases the ctx's host state.  Device buffers belong to the caller. */
fd_status fd_destroy(fd_ctx* ctx);

/* ---- inspection and bench/test hooks ---- */

/* Fills *out with the cache layout and the device slot-table pointers. */
fd_status fd_kv_layout(fd_ctx* ctx, fd_kv_view* out);

/*
 * Sets an allocated slot's next frame index (0..max_context), e.g. after a
 * caller-side prefill, or to rewind a slot between timed steps.  Reaches
 * the device with the next fd_step.  FD_E_BADSLOT for an unallocated slot,
 * FD_E_INVAL for a position outside 0..max_context.
 */
fd_status fd_set_position(fd_ctx* ctx, int32_t slot, int32_t pos);

/* Host copy of a slot's state: *active (0/1) and *pos. */
fd_status fd_slot_state(fd_ctx* ctx, int32_t slot, int32_t* active, int32_t* pos);

/*
 * Writes cache entries from raw values, stored exactly as the step stores
 * new frames (FP8: code(value / kv_scale[layer][kv][g]), round to nearest
 * even, saturating at +-448; fp32: the value).
 *   src: device fp32 [2 (K|V)][n_kv_heads][n][head_dim], positions t0..t0+n-1
 * of `slot` at `layer`.  Enqueued on `stream`.  The slot need not be
 * allocated.  FD_E_INVAL for a range outside the window.
 */
fd_status fd_kv_write(fd_ctx* ctx, int32_t slot, int32_t layer, int32_t t0, int32_t n,
                      const float* src, void* stream);

/*
 * Per-kernel timing (bench hook).  With enable != 0, fd_step brackets every
 * kernel it launches with a pair of HIP events on its stream; fd_profile_read
 * waits for them and returns, per kernel kind, the summed duration in
 * milliseconds and the number of launches since the last read (then resets).
 * Kinds: 0 embed, 1 qkv, 2 attention, 3 o-projection, 4 gate/up, 5 down,
 * 6 final norm, 7 depth input projection, 8 the persistent walk of the
 * whole step (FD_EXEC_WALK; then the only step kind launched), 9 the output
 * head of fd_step_tokens (projection and argmax); 10..14 the depth stack's
 * qkv, attention, o-projection, gate/up and down (kinds 1..5 then count the
 * main stack only) (FD_N_KINDS = 15).  Timing adds a small gap between
 * launches; headline step times are taken with it off.
 */
#define FD_N_KINDS 15
fd_status fd_profile(fd_ctx* ctx, int32_t enable);
fd_status fd_profile_read(fd_ctx* ctx, double* ms_out, int64_t* launches_out, int32_t n);

/*
 * Device-clock trace of the attention kernel (bench hook, off by default).
 * With stamps != NULL, every later fd_step's attention launch of main-stack
 * layer `layer` has each workgroup write four 64-bit readings of the
 * device's constant-rate clock (s_memrealtime, 100 MHz) with ordinary
 * vector stores to stamps[4*w + i]: i = 0 on entry, 1 when its prologue
 * (the norm, rotary, cache append and query set-up) is done, 2 when its
 * stream over the cached positions is done, 3 on exit (a workgroup with no
 * work writes entry then three equal exit stamps).  w is the workgroup
 * index, (r * n_kv_heads + kv-head) * chunks + chunk, where the r-th slot
 * in the attention order is the r-th active slot by descending position
 * (ties by slot number), the inactive slots following in ascending order
 * (attention runs the longest windows first).  stamps: device,
 * 8-byte aligned, at least 4 * max_workgroups entries; max_workgroups must
 * cover the launch (FD_E_INVAL).  NULL turns it off.  FD_EXEC_KERNELS
 * profiles only (FD_E_UNSUPPORTED otherwise).
 */
fd_status fd_trace_attention(fd_ctx* ctx, uint64_t* stamps, int32_t layer, int32_t max_workgroups);

/*
 * Forces the persistent walk's abort path (test hook, FD_EXEC_WALK profiles;
 * FD_E_UNSUPPORTED otherwise): the ctx's next fd_step launches the walk with
 * its abort flag already set, so every workgroup leaves at its first grid
 * barrier wait, as after a timed-out wait, without any wait running out.
 * That step's outputs, cache entries and device positions are then
 * incomplete; fd_sync reports FD_E_DEVICE and marks the active slots stale
 * (fd_step gives FD_E_STATE until each is given a position with
 * fd_set_position or freed).  Applies to one step.
 */
fd_status fd_walk_abort_next(fd_ctx* ctx);

/*
 * HBM read probe (bench hook): enqueues one kernel that reads `bytes` of
 * device memory at `buf` (16-byte aligned) once with wide loads, `grid`
 * workgroups of 256 threads, and may write to device words sink[0..grid).
 * Timing it gives the achievable streaming-read bandwidth, the denominator
 * the bandwidth blog measures directly (section 2, "Direct Verification").
 * Needs no ctx.  FD_E_INVAL for bad arguments.
 */
fd_status fd_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int32_t grid, void* stream);

/* Waits for the ctx's last enqueued work on `stream` and reports device
 * errors (FD_E_DEVICE) including the persistent walk's timed-out barrier
 * flag (after which the active slots are stale, see FD_EXEC_WALK). */
fd_status fd_sync(fd_ctx* ctx, void* stream);

/* Message of the ctx's most recent error ("" if none); valid until the
 * next call on the ctx.  With ctx == NULL, the last fd_plan/fd_init error. */
const char* fd_last_error(fd_ctx* ctx);

/* Static name of a status code. */
const char* fd_status_str(fd_status s);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
