// Internal definitions shared by the host runtime and the device code.
//
// Work decomposition (one persistent workgroup per CU):
//   - Every matrix-vector stage splits its output rows into "units" of four
//     consecutive packed rows; unit u of a stage goes to workgroup
//     w = the w with floor(w*U/G) <= u < floor((w+1)*U/G).  Inside a
//     workgroup, local row i belongs to consumer wave i % 4.
//   - A workgroup's weights for a stage are a sequence of 16 KiB "slots",
//     striped with the other workgroups' (slot n of workgroup w at
//     (n * grid + w) * 16 KiB of the stage's layer block).  Slot n holds,
//     for each consumer c, the next 4 KiB of c's rows (each row zero-padded
//     to whole 1 KiB chunks; see mk_stream_pos for the order).  Loader waves
//     copy slots into an LDS ring with direct-to-LDS loads; consumer waves
//     read their 4 KiB piece of the slot.
//   - Attention splits each KV head's positions [0, pos) into `splits`
//     contiguous ranges, one per workgroup; position pos (written in the same
//     step) is folded in by the last split after the producers publish it.
#pragma once
#include <stdint.h>

#define MK_SLOT_BYTES 16384
#define MK_CHUNK_BYTES 1024
#define MK_CHUNKS_PER_SLOT 16
#define MK_NUM_LOADERS 4
#define MK_NUM_CONSUMERS 4
#define MK_BLOCK_THREADS (64 * (MK_NUM_LOADERS + MK_NUM_CONSUMERS))
#define MK_MAX_RING 9  // LDS bound; the loaders wait for (ring-2)*4 outstanding loads (at most 63)
#define MK_DEFAULT_RING 8
#define MK_LDS_LIMIT 163840
#define MK_MAX_GRID 1024
#define MK_MAX_SPLITS 64  // attention splits per KV head (one lane each in the combine)

// The down projection is split along its input instead of its output rows:
// workgroup w owns the SwiGLU outputs f in [f0, f0 + nf) -- the gate/up rows
// it computes -- and multiplies them by the matching Wd columns, producing a
// partial sum for every one of the H output rows.  Its weights are streamed
// as "piece columns" of 1 KiB: 64 lanes x 16 bytes, lane i holding 16 bytes
// (EPL elements) of one output row.  Rows come in groups of 64 (one row per
// lane); consumer c takes row groups c, c + 4, ...; a row group is kp piece
// columns long (kp = ceil(nf / EPL)), and slot n carries piece columns
// [4n, 4n + 4) of each consumer's stream.
struct MkDownGeo {
    int f0, nf, kp, nsl;
};
static inline __host__ __device__ MkDownGeo mk_down_geo(int w, int G, int units_gu, int F, int H, int epl) {
    const int u0 = (int)(((long long)w * units_gu) / G), u1 = (int)(((long long)(w + 1) * units_gu) / G);
    MkDownGeo g;
    g.f0 = 2 * u0;
    const int f1 = 2 * u1 < F ? 2 * u1 : F;
    g.nf = f1 > g.f0 ? f1 - g.f0 : 0;
    g.kp = (g.nf + epl - 1) / epl;
    const int groups_per_consumer = ((H + 63) / 64 + 3) / 4;
    g.nsl = (groups_per_consumer * g.kp + 3) / 4;
    return g;
}

// Order of a consumer's chunk stream for the matrix-vector stages.  Rows
// may be interleaved in groups of four rows: the stream holds chunk 0 of
// rows 4g..4g+3, then chunk 1 of the same rows, and so on, so the four
// pieces a consumer takes from one slot multiply the same input elements
// (read once from LDS instead of once per piece).  Rows past the last whole
// group follow row after row.  Grouped: int8 rows (eb == 1) of any length --
// a 16-byte int8 piece needs 16 input floats, so re-reading them per piece
// would cost four times the weight bytes in LDS reads; float32 and bfloat16
// rows of 8, 12, 16 ... chunks.  Float32 and bfloat16 rows of exactly 4
// chunks go row after row (the kernel keeps their input slice in registers),
// and so do rows of other lengths.
static inline __host__ __device__ bool mk_row_groups(int rbp, int eb) {
    return eb == 1 ? rbp >= 1 : (rbp >= 8 && (rbp & 3) == 0);
}
// Stream position qq (in chunks) of a consumer holding `rows` rows of rbp
// chunks of eb-byte elements -> its local row and the chunk within that row.
static inline __host__ __device__ void mk_stream_pos(int qq, int rows, int rbp, int eb, int &row, int &kc) {
    const int full = mk_row_groups(rbp, eb) ? rows / 4 : 0;
    const int span = 4 * rbp;  // chunks of one group of four rows
    if (qq < full * span) {
        row = (qq / span) * 4 + (qq % 4);
        kc = (qq % span) / 4;
    } else {
        const int r = qq - full * span;
        row = full * 4 + r / rbp;
        kc = r % rbp;
    }
}

// Stage kinds with weights; the attention stage streams the KV cache.
enum { ST_QKV = 0, ST_O = 1, ST_GU = 2, ST_DOWN = 3, ST_LM = 4, ST_NUM = 5 };

struct MkStage {
    int32_t units;        // total units (4 packed rows each); for the down stage: the gate/up units
    int32_t rbp;          // packed row length in 1 KiB chunks
    int32_t k;            // input length in elements
    int32_t rows;         // logical packed rows (units*4 >= rows; the rest are zero)
    int64_t base;         // byte offset of layer 0's block in the packed buffer
    int64_t layer_stride; // bytes between consecutive layers' blocks
    const int64_t *wg_off;   // [grid] byte offset of each workgroup's first slot in a layer block
    int64_t slot_stride;     // bytes between a workgroup's consecutive slots (grid * 16 KiB: striped)
};

struct MkParams {
    // model
    int32_t L, H, nh, nkv, d, F, V, max_seq;
    float eps;
    // launch shape
    int32_t grid, ring_slots, splits, lds_vec_floats, lds_out_rows;
    int32_t prefetch_depth;  // slots the loads run ahead of the arithmetic, slots_per_step .. ring_slots-slots_per_step
    int32_t slots_per_step;  // ring slots the consumers take between two workgroup barriers (1 or 2)
    int32_t stage_drain;     // 1: no loads for a stage before its opening barrier
    int32_t attn_pm_slots;   // position-major attention when a split holds at least this many whole KV slots
    // weights
    const unsigned char *packed;
    MkStage st[ST_NUM];
    // Weight-only INT8 (dtype 2): per-row scales of the matrices, one block
    // per (layer, workgroup) of sc_blk floats -- the workgroup's QKV rows,
    // O rows, gate/up rows (packed local order) and the down-projection rows
    // of its x rows (the O rows' indices), one after the other, zero padded
    // -- at scl + (l * grid + w) * sc_blk, and the LM head's block of sc_lm
    // floats at scl + L * grid * sc_blk + w * sc_lm.  lds_sc_floats: the LDS
    // copy of one block (max(sc_blk, sc_lm)); two copies, by layer parity.
    const float *scl;
    int32_t sc_blk, sc_lm, lds_sc_floats;
    const float *g_attn;   // [L][H]
    const float *g_ffn;    // [L][H]
    const float *g_final;  // [H]
    const void *embed;     // [V][H] in the model dtype
    const float *rope;     // [max_seq][d/2][2] (cos, sin)
    // KV cache (caller-owned)
    void *kc, *vc;
    // Cross-workgroup values within a launch.  Every record is 64 bits: the
    // float's bits in the low word, the tag in the high word.  Each
    // dependency point has its own array with two buffers, [2] below, used by
    // layers of even and odd index (l & 1); a record of layer index l carries
    // the tag `tag + l`, so a reader polls until the tags equal the one of
    // its layer in this launch.
    uint64_t *ll_xq;       // [2][H]     x entering layer l >= 1, and the LM head (l = L)
    uint64_t *ll_xg;       // [2][H]     x after the O projection
    uint64_t *ll_qkv;      // [2][nkv][GQ+2][d] per KV group: rotated queries, then K and V of
                           // this step's position (bf16-rounded), next to each other
    uint64_t *ll_part;     // [2][nkv*splits][GQ][d+2] attention partials: o (unnormalised), m, l
    uint64_t *ll_o;        // [2][nh*d]  attention output
    uint64_t *ll_dpart;    // [2][grid][H] each workgroup's partial down projection
    uint64_t *ll_amax;     // [grid][2]  per-workgroup (max logit, its index), tag + L
    uint32_t *err;         // device error word
    // this call
    int32_t token;
    const int32_t *token_dev;
    int32_t pos;
    int32_t want_logits;
    float *logits;
    int32_t *token_out;
    uint32_t tag;          // this launch's tag base: a record of layer index l carries tag + l (never 0)
    int64_t timeout_ticks; // wall-clock ticks (100 MHz) before a grid wait gives up
    int64_t err_check_ticks;  // wall-clock ticks a wait lasts before it also watches the device error word
    uint64_t *trace;       // optional [grid][5L+2][4] stage timeline, or null
};

// Buffers of the batched prefill (mk_prefill.hip), sized for chunks of up
// to t_max tokens.
struct MkPrefillBufs {
    float *X;        // [t_max][H] residual stream
    uint16_t *Ah;    // [t_max][lda] bf16 high parts of the current GEMM operand
    uint16_t *Al;    // [t_max][lda] bf16 low parts (a - hi)
    float *Y;        // [t_max][ldy] QKV or gate/up outputs, packed row order
    float *Q;        // [t_max][max(nh*d, H)] rotated queries; an input split's sums in the O and down GEMMs
    int32_t *tok;    // token ids of the chunk (device)
    // [F/8][4] where the down projection keeps each block of 8 consecutive
    // inputs (one 16-byte piece or half of one): the owning workgroup's
    // byte offset in a layer block, its pieces per row group (kp), the
    // piece index q and the byte offset inside the piece
    const int32_t *dmap;
    int32_t lda, ldy, t_max;
};

// Error codes written to the device error word.
#define MK_DEVERR_TIMEOUT 1u
#define MK_DEVERR_TOKEN 2u

// Host-side launchers implemented in the .hip files.
#ifdef __cplusplus
extern "C" {
#endif
int mk_launch_decode(const MkParams *p, int dtype, int cooperative, void *stream);
int mk_launch_prelayout_stage(unsigned char *dst, const MkStage *st, int grid, int kind, int eb,
                              const void *src0, const void *src1, const void *src2, int nh, int nkv, int d,
                              void *stream);
// One block of per-row scales per workgroup (see MkParams::scl) for layer
// `layer` (src[0..6]: wq, wk, wv, wo, w_gate, w_up, w_down scales) or, with
// layer == L, the LM head's (src[0]).
int mk_launch_prelayout_scales(float *scl, const MkParams *p, int layer, const float *const *src, void *stream);
int mk_kernel_lds_bytes(int ring_slots, int vec_floats, int out_rows, int sc_floats);
int mk_launch_to_f32(float *dst, const void *src, int64_t n, int dtype, void *stream);
int mk_launch_zero(void *dst, int64_t bytes, void *stream);
int mk_prefill_chunk(const MkParams *p, const MkPrefillBufs *b, int T, int pos0, void *stream);
int mk_prefill_supported(const MkParams *p, int dtype);
#ifdef __cplusplus
}
#endif
