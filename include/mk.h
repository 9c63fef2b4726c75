/*
 * mk.h -- C ABI of a persistent decode megakernel for AMD MI355X (gfx950).
 *
 * One call of mk_decode_step runs one batch-1 autoregressive decode step of
 * a Llama-style decoder as ONE kernel launch:
 *   embedding gather -> per layer [RMSNorm -> fused QKV GEMV -> RoPE ->
 *   KV-cache append -> GQA attention over the cache -> O projection +
 *   residual -> RMSNorm -> gate/up GEMV + SwiGLU -> down GEMV + residual]
 *   -> final RMSNorm -> LM-head GEMV (-> optional greedy argmax).
 *
 * The operator chain is the one the pages name (cloud.baidu.com/article/
 * 9434380 "low-latency single-request LLM inference: from operator fusion
 * to runtime orchestration", section 三 and section 五 step 2, segments A,
 * B and C); the single launch with an in-kernel weight-prefetch pipeline is
 * that page's section 4.2 and section 五 step 3, and the MegaKernel tutorial
 * at developer.baidu.com/article/detail.html?id=8006242, sections 4.1-4.2.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major [out][in] (the layout of a Linear layer weight).
 *   - "device" pointers are HIP device allocations on the current device;
 *     "host" pointers are ordinary host memory.
 *   - Streams are passed as `void *` holding a hipStream_t (NULL = the null
 *     stream; the pages advise always passing an explicit stream, page
 *     www.stapisi.com/news/3904786 section 3.3).
 *   - Every call returns an mk_status; nothing throws across the ABI.
 *     Argument checks are done on the host before any device work is
 *     enqueued (the page cloud.baidu.com/article/9434380, section 九, asks
 *     for guards on input ranges in a fused kernel).
 *   - Device-side failures (a grid-wait timeout) are asynchronous: they set
 *     a device flag that mk_get_device_error reports, after which the handle
 *     refuses further steps (MK_ERR_STATE).
 *   - Ordering: each call that enqueues work records an event of the handle
 *     after its launches; a call on a different stream than the handle's
 *     previous call first makes its stream wait on that event (record on one
 *     stream, wait on another: www.stapisi.com/news/3904786 section 3.1).
 *     So the calls of one handle run in the order they were made, whatever
 *     streams the caller passes.  Calls on one handle from several host
 *     threads at once are not supported.
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MK_OK = 0,
    MK_ERR_NULL = 1,    /* a required pointer argument is NULL */
    MK_ERR_SHAPE = 2,   /* unsupported or inconsistent model shape */
    MK_ERR_DTYPE = 3,   /* unsupported dtype */
    MK_ERR_RANGE = 4,   /* token id, position or count out of range */
    MK_ERR_NOMEM = 5,   /* device allocation failed */
    MK_ERR_HIP = 6,     /* a HIP runtime call failed */
    MK_ERR_DEVICE = 7,  /* the device reported a failure (grid-wait timeout) */
    MK_ERR_STATE = 8,   /* the handle was disabled by an earlier device failure, or its
                           weights are not all loaded yet (mk_create_deferred) */
    MK_ERR_TUNING = 9,  /* a tuning value is out of its documented range */
    MK_ERR_SCRATCH = 10 /* the model's cross-workgroup records do not fit the static scratch
                           (mk_decode_step_device_token_noalloc) */
} mk_status;

/* Size of the library's static device scratch, the record buffer of
   mk_decode_step_device_token_noalloc (one per device, held until the
   process ends). */
#define MK_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)

/* MK_F32, MK_BF16: every weight and the KV cache in that type.
   MK_W8: weight-only INT8 -- the seven layer matrices and the LM head are
   int8 codes q with one float32 scale s per output row, standing for the
   weights W[r][c] = s[r] * q[r][c]; the embedding, the norm gains and the KV
   cache are bf16.  Quantised models stream fewer bytes per token, and the
   dequantisation runs inside the fused step (www.stapisi.com/news/3904786
   section 6.1).  The kernel multiplies the int8 codes by the activations in
   fp32 and applies each row's scale to the row's sum. */
typedef enum { MK_F32 = 0, MK_BF16 = 1, MK_W8 = 2 } mk_dtype;

/* Model shape.  Supported: n_heads % n_kv_heads == 0; head_dim * element
   size of the cache equal to 128 or 256 bytes (bf16 and MK_W8: head_dim 64
   or 128; f32: 32 or 64); hidden and ffn multiples of 8; max_seq >= 1;
   MK_W8 models are not tied (their LM head is its own int8 matrix).
   rms_eps is added to the mean square inside the square root; RoPE rotates
   pairs (i, i + head_dim/2) by pos * rope_theta^(-2i/head_dim). */
typedef struct {
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, max_seq;
    double rms_eps, rope_theta;
    mk_dtype dtype;          /* weights and KV cache */
    int32_t tied_embeddings; /* 1: the LM head is the embedding matrix */
} mk_model_desc;

/* Device pointers to one layer's weights in the model dtype:
   attn_norm [H], wq [n_heads*head_dim][H], wk [n_kv*head_dim][H],
   wv [n_kv*head_dim][H], wo [H][n_heads*head_dim], ffn_norm [H],
   w_gate [F][H], w_up [F][H], w_down [H][F].  For MK_W8 the matrices are
   int8 codes, the norms bf16, and s_* are the matrices' float32 per-row
   scales (one per output row: s_wq [n_heads*head_dim], ..., s_w_down [H]);
   the s_* pointers are ignored for the other dtypes and may be NULL. */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
    const float *s_wq, *s_wk, *s_wv, *s_wo, *s_w_gate, *s_w_up, *s_w_down;
} mk_layer_ptrs;

/* embed [V][H], final_norm [H], lm_head [V][H] (ignored when tied);
   layers is a HOST array of n_layers entries holding device pointers;
   lm_head_scale [V] is the LM head's per-row scales (MK_W8 only). */
typedef struct {
    const void *embed, *final_norm, *lm_head;
    const mk_layer_ptrs *layers;
    const float *lm_head_scale;
} mk_weight_ptrs;

/* Caller-owned contiguous KV cache, device memory in the model dtype, each of
   K and V laid out [n_layers][n_kv_heads][max_seq][head_dim]. */
typedef struct {
    void *k, *v;
    int32_t max_seq; /* must equal the model's max_seq */
} mk_kv_cache;

/* Tuning knobs.  Zero selects the default for every field.
     grid:        workgroups of the persistent grid, 1..1024 and no more than
                  can be resident at once (default: CU count);
     ring_slots:  16 KiB LDS ring slots per workgroup, 3..9 (default: 8, or as many
                  as fit beside the activation buffer);
     attn_splits: sequence splits per KV head, at most 64 (default:
                  min(grid / n_kv_heads, 64));
     timeout_ms:  grid-wait timeout before the device error flag is raised
                  (default 2000);
     cooperative: 2 = ordinary launch (default), 1 = cooperative launch.
                  Either way the host first checks that the whole grid fits
                  on the device at once (one workgroup per CU); the ordinary
                  launch skips the runtime's own co-residency handling,
                  which costs about 20 us per launch.  If workgroups are
                  nevertheless not co-resident (another kernel holds CUs),
                  the grid waits end by timeout with the device error flag,
                  never by a hang;
     trace:       1 = record a per-workgroup stage timeline on every step
                  (read it with mk_read_trace; default 0 = off);
     prefetch_depth: 16 KiB slots the weight and cache loads run ahead of
                  the slot being multiplied, slots_per_step .. ring_slots -
                  slots_per_step (default ring_slots - slots_per_step);
     stage_drain: 1 = no cross-stage prefetch: a stage's first loads wait
                  for the grid dependency before it (the consumers' opening
                  barrier of the stage); 0 = loads run ahead across stage
                  boundaries (default).  An ablation knob;
     attn_pm_slots: per-length attention mapping.  With four query heads
                  per KV head, when a split holds at least this many whole
                  KV slots (64 positions each at head_dim 64, 32 at 128) the
                  launch uses the position-major mapping (each consumer wave
                  folds a quarter of every slot's positions for all four
                  heads, so K and V are read from LDS once per workgroup);
                  shorter splits use the head-major mapping (each consumer
                  one head over all positions).  0 or -1 (default) = always
                  head-major: on MI355X the position-major mapping measured
                  slower at both the 2048- and the 32768-token contexts (the
                  slot is bound by the consumers' arithmetic, not by LDS
                  reads).  The page cloud.baidu.com/article/9434380 section
                  八 (question five) advises tiling by length;
     prefill_chunk: tokens per chunk of the batched prefill, 1..4096
                  (default 4096, or max_seq if smaller); -1 = prefill by one
                  decode launch per position.  The batched prefill needs bf16
                  or INT8 weights, a hidden size of at most 16384 and a
                  geometry whose down-stage workgroups own inputs starting at
                  multiples of 8 (true of the Llama shapes at 256
                  workgroups); otherwise mk_prefill_kv uses
                  decode launches (mk_info.prefill_chunk reports which);
     slots_per_step: the tile of the weight and cache stream: 16 KiB ring
                  slots the consumer waves take per data step, between two
                  workgroup barriers, 1 or 2 (default 1).  With 2 the loads
                  of both slots are complete before the step's barrier and
                  prefetch_depth lies in 2 .. ring_slots - 2.  The tile
                  granularity is the first tunable of
                  cloud.baidu.com/article/9434380 section 六. */
typedef struct {
    int32_t grid, ring_slots, attn_splits, timeout_ms, cooperative, trace, prefetch_depth, stage_drain;
    int32_t prefill_chunk, attn_pm_slots, slots_per_step;
} mk_tuning;

typedef struct mk_handle mk_handle;

/* Read-only facts about a created handle (for benchmarks and tests). */
typedef struct {
    int32_t grid, ring_slots, attn_splits, block_threads, lds_bytes, cu_count;
    int32_t prefetch_slots;  /* 16 KiB slots the loads run ahead of the arithmetic */
    int64_t packed_bytes;    /* library-owned pre-laid-out weight bytes */
    int64_t weight_bytes;    /* algorithmic weight bytes read per step */
    int64_t record_bytes;    /* cross-workgroup record buffer of one launch (at most
                                MK_STATIC_SCRATCH_BYTES for the no-allocation step) */
    int32_t prefill_chunk;   /* tokens per batched-prefill chunk; 0: prefill by decode launches */
    int32_t slots_per_step;  /* 16 KiB ring slots per data step (the stream's tile) */
} mk_info;

/* Create a handle: validates the shape, copies every weight into a
   library-owned buffer laid out in the kernel's access order (the weight
   pre-layout of cloud.baidu.com/article/9434380 section 九), builds the RoPE
   table, and allocates scratch.  The caller may free its weights after this
   returns.  Synchronous.  tuning may be NULL.  On success *out receives the
   handle; on failure *out is set to NULL. */
mk_status mk_create(const mk_model_desc *desc, const mk_weight_ptrs *weights, const mk_tuning *tuning,
                    mk_handle **out);

/* Create a handle whose weights are supplied afterwards with
   mk_load_weights, a part at a time.  For models whose caller-side weights
   and the library's pre-laid-out copy do not both fit in device memory at
   once (an 80-layer, hidden-8192 bf16 decoder holds about 139 GB of
   weights; the device has 288 GB): the caller can upload, load and free one
   layer at a time.  Validation, geometry and allocations are those of
   mk_create.  Steps and prefill return MK_ERR_STATE until every layer and
   the head weights (embedding, final norm, LM head) have been loaded.
   Synchronous.  On failure *out is set to NULL. */
mk_status mk_create_deferred(const mk_model_desc *desc, const mk_tuning *tuning, mk_handle **out);

/* Pre-lay out part of a model's weights into h (the same re-layout mk_create
   does, cloud.baidu.com/article/9434380 section 九): layers
   [first_layer, first_layer + n_layers) are read from weights->layers[0 ..
   n_layers) (a host array of device pointers; may be NULL when n_layers is
   0), and, when weights->embed is not NULL, the embedding, final norm and
   LM head (weights->lm_head, ignored when tied) are loaded too.  A part may
   be loaded again; the last load wins.  Synchronous: it first waits for all
   work on the device (so no step of the handle still reads the weights it
   replaces), and the caller may free the source tensors when it returns.  Errors: MK_ERR_NULL (h, weights, or a
   pointer of a part being loaded is NULL), MK_ERR_RANGE (the layer range
   is outside [0, n_layers)). */
mk_status mk_load_weights(mk_handle *h, const mk_weight_ptrs *weights, int32_t first_layer, int32_t n_layers);

/* One decode step for token_id at 0-based position pos: writes K/V of
   position pos into the cache, reads cache positions [0, pos] (never
   positions > pos) and writes vocab fp32 logits to logits_out (device).
   Enqueued on `stream`; returns immediately.  Requires 0 <= token_id < vocab
   and 0 <= pos < max_seq.
   The operation is the whole decode step of the pages' path as one launch
   (cloud.baidu.com/article/9434380 section 4.2 and section 五 steps 2-3;
   developer.baidu.com/article/detail.html?id=8006242 section 4.1); its
   arguments follow the asynchronous forward entry of
   www.stapisi.com/news/3904786 section 5.2 (a stream, the input, the output
   and the KV cache, enqueued without waiting).  Errors: MK_ERR_NULL (h,
   kv, its pointers or logits_out NULL), MK_ERR_SHAPE (kv->max_seq differs
   from the model's), MK_ERR_RANGE, MK_ERR_STATE (disabled handle or weights
   not all loaded), MK_ERR_HIP (the launch failed). */
mk_status mk_decode_step(mk_handle *h, int32_t token_id, int32_t pos, const mk_kv_cache *kv,
                         float *logits_out, void *stream);

/* Same step with the token read from device memory (token_in, one int32) and
   the greedy next token (argmax of the logits, lowest index on ties) written
   to device memory (token_out, one int32).  Lets a caller enqueue many steps
   back to back with no host round trip.  logits_out may be NULL.  A token id
   outside [0, vocab) in token_in raises the device error flag.
   The greedy choice runs on the fused path itself, where the page
   cloud.baidu.com/article/9434380 section 五 step 5 asks that sampling and
   the state carried from step to step be checked again. */
mk_status mk_decode_step_device_token(mk_handle *h, const int32_t *token_in, int32_t pos, const mk_kv_cache *kv,
                                      float *logits_out, int32_t *token_out, void *stream);

/* The step of mk_decode_step_device_token for callers that cannot allocate
   device memory at the time of the call: code under HIP graph capture, tight
   serving loops, harnesses that forbid hipMalloc.  It allocates nothing and
   calls no allocating routine: the cross-workgroup records of the launch
   (the only buffer its kernel needs beyond the handle's weights and the
   caller's inputs and outputs) live in a static device array of the library,
   MK_STATIC_SCRATCH_BYTES per device, instead of the handle's own buffer;
   the kernel and the results are those of mk_decode_step_device_token, bit
   for bit.  The caller still passes the token, cache, logits and token
   buffers.  Every call on one device shares that device's array and one tag
   counter (a record left by an earlier call never carries an awaited tag, so
   nothing needs clearing between calls); calls that overlap in time on one
   device, from any handle or stream, race on it and are not allowed.  The
   device is the one current at mk_create.  Errors: as
   mk_decode_step_device_token, plus MK_ERR_SCRATCH when the handle's record
   buffer (mk_info.record_bytes) exceeds MK_STATIC_SCRATCH_BYTES and MK_ERR_HIP
   when the array's device address could not be taken at mk_create. */
mk_status mk_decode_step_device_token_noalloc(mk_handle *h, const int32_t *token_in, int32_t pos,
                                              const mk_kv_cache *kv, float *logits_out, int32_t *token_out,
                                              void *stream);

/* Fill cache positions [start_pos, start_pos + n) from n host token ids: by
   definition under causal attention this is n decode steps at those
   positions with the LM head skipped.  Requires n >= 0 and
   start_pos + n <= max_seq.  The caller's token array may be reused as soon
   as the call returns.
   Batched (mk_info.prefill_chunk > 0): chunks of up to prefill_chunk
   positions; per layer the chunk's tokens go through matrix-core GEMMs
   (bf16 weights, or int8 codes widened to bf16 with the row scale applied
   to each sum; activations split into bf16 high and low parts; fp32
   accumulation) that read the packed weights in place, and a causal
   attention over positions [0, own].  The cache rows equal the decode
   step's to within the bf16 rounding of the stored values.  Otherwise one
   decode launch per position.
   The pages keep the prefill apart from the decode step and measure the two
   phases separately (cloud.baidu.com/article/9434380 section 八, question
   two); the cache it fills is the state handed between steps (same page,
   section 五 step 4).  Errors: MK_ERR_NULL, MK_ERR_SHAPE, MK_ERR_RANGE (a
   token id outside [0, vocab) or the range past max_seq), MK_ERR_STATE,
   MK_ERR_HIP. */
mk_status mk_prefill_kv(mk_handle *h, const int32_t *tokens, int32_t n, int32_t start_pos, const mk_kv_cache *kv,
                        void *stream);

/* Waits for the handle's last call to complete (its recorded event, on
   whatever stream that call used: no stream argument is needed) and reports
   the device failure flag: MK_OK, MK_ERR_DEVICE (after which the handle is
   disabled), or MK_ERR_STATE for a handle disabled earlier.  The stability
   advice of the pages (cloud.baidu.com/article/9434380 section 九;
   developer.baidu.com/article/detail.html?id=8006242 section 6.2) asks for
   bounds checks on a fused kernel; the kernel's device-side checks (a token
   id read from device memory, a dependency wait that times out) report
   here. */
mk_status mk_get_device_error(mk_handle *h);

/* Launch geometry and sizes of a created handle, for benchmarks and tests
   (the tunables the page cloud.baidu.com/article/9434380 section 六 asks to
   expose).  Errors: MK_ERR_NULL. */
mk_status mk_get_info(const mk_handle *h, mk_info *info);

/* Stage timeline of the most recent step (handles created with trace = 1;
   the per-stage timing points of www.stapisi.com/news/3904786 section 5.3):
   waits for the handle's last call, then copies uint64 wall-clock ticks (100 MHz
   on MI355X) into host_out, three arrays one after the other:
   1. grid * (5*n_layers + 2) * 4, laid out [workgroup][boundary][event].
      Boundary 5l+k is the start of stage k of layer l (k: 0 QKV,
      1 attention, 2 O, 3 gate/up, 4 down), 5L the LM head, 5L+1 the end of
      the step.  Events: 0 boundary reached (all of the previous stage
      consumed), 1 previous stage finished and published, 2 inputs of the
      next stage available (dependency wait over), 3 inputs loaded.
   2. grid * 64 * 2: consumer 0's first 64 data steps of layer 1
      [workgroup][step][0 barrier passed, 1 arithmetic done].
   3. grid * 96 * 2: loader 0's first 96 barriers of layer 1
      [workgroup][barrier][0 arrival, 1 exit].
   Unrecorded entries are 0.  capacity is the number of uint64 host_out can
   hold (at least the sum of the three sizes). */
mk_status mk_read_trace(mk_handle *h, uint64_t *host_out, int64_t capacity);

/* A static, human-readable name of a status ("unknown status" for values
   outside the enum).  Never NULL; the caller does not free it. */
const char *mk_status_str(mk_status s);

/* Frees everything the handle owns (packed weights, records, tables,
   event).  The caller must make sure no call of the handle is still running
   (mk_get_device_error waits for the last one).  NULL is allowed. */
void mk_destroy(mk_handle *h);

#ifdef __cplusplus
}
#endif
#endif
