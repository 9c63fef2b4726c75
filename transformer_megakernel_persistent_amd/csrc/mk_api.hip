// Host runtime of the C ABI declared in include/mk.h: argument validation,
// work decomposition, weight pre-layout, scratch ownership and the one
// launch per decode step.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "mk.h"
#include "mk_internal.h"

extern "C" int mk_kernel_max_blocks_per_cu(int dtype, int gq, int lpp, int lds);

// Offsets (in records) of the cross-workgroup record arrays inside one
// record buffer, in MkParams order: xq, xg, qkv, part, o, dpart, amax; [7] is
// the total.  Each per-layer array holds two layers (even and odd index).
struct RecLayout {
    size_t off[8];
};

// ---- the static scratch of mk_decode_step_device_token_noalloc -------------
// Callers that cannot allocate device memory (code under graph capture,
// tight serving loops) get the records from this file-scope array instead
// of the handle's own buffer.  Each device the library runs on holds one
// copy until the process ends.  In host code the name `scratch` is only a
// host-side stand-in: its device address is taken once per device with
// hipGetSymbolAddress (device current) and kept in g_scratch_ptr, and only
// that address is ever passed to a kernel.
#define MK_MAX_DEVICES 64
static __device__ __align__(256) uint64_t scratch[MK_STATIC_SCRATCH_BYTES / sizeof(uint64_t)];
static std::mutex g_scratch_mu;
static uint64_t *g_scratch_ptr[MK_MAX_DEVICES];  // device address of `scratch` on each device
static uint32_t g_scratch_tag_end[MK_MAX_DEVICES];  // last tag used on that device's array

struct mk_handle {
    mk_model_desc desc;
    int emb_bytes = 0;  // bytes per embedding element (bf16 for MK_W8)
    int device = 0;
    int cu_count = 0;
    int cooperative = 0;
    MkParams base;  // launch-invariant kernel arguments
    unsigned char *packed = nullptr;
    int64_t packed_bytes = 0;
    int64_t weight_bytes = 0;
    int64_t *wg_off = nullptr;  // [ST_NUM][grid]
    float *gains = nullptr;     // attn [L][H], ffn [L][H], final [H]
    void *embed = nullptr;
    float *rope = nullptr;
    float *scl = nullptr;       // per-row scales of the INT8 matrices (MK_W8; see MkParams::scl)
    uint64_t *ll = nullptr;     // tagged cross-workgroup records (see MkParams)
    RecLayout rec;              // their layout (the same inside the static scratch)
    uint32_t *err = nullptr;    // device error word
    uint64_t *trace = nullptr;
    int64_t trace_len = 0;
    uint32_t tag_end = 0;       // last tag used on the handle's own records
    bool disabled = false;
    // Completion of the handle's last call: recorded on its stream after the
    // launches; a call on another stream first waits for it, so the launches
    // of one handle stay ordered whatever streams the caller uses.
    hipEvent_t done = nullptr;
    bool done_recorded = false;
    hipStream_t last_stream = nullptr;
    int lds_bytes = 0;
    MkPrefillBufs pf = {};           // batched prefill (pf.t_max == 0: one decode launch per position)
    int32_t *pf_tokens = nullptr;    // [max_seq] device copy of prompt token ids
    std::vector<char> layer_loaded;  // [n_layers]: weights of the layer pre-laid out
    int layers_loaded = 0;
    bool head_loaded = false;        // embedding, final norm and LM head in place
};

namespace {

mk_status hip_fail(hipError_t e) { return e == hipErrorOutOfMemory ? MK_ERR_NOMEM : MK_ERR_HIP; }

#define HIP_TRY(expr)                              \
    do {                                           \
        hipError_t e_ = (expr);                    \
        if (e_ != hipSuccess) return hip_fail(e_); \
    } while (0)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The kernel's dtype code: 0 float32, 1 bfloat16, 2 weight-only INT8 (bf16
// cache, embedding and gains).
int dtype_code(mk_dtype t) { return t == MK_W8 ? 2 : t == MK_BF16 ? 1 : 0; }
// Bytes per element of the weight matrices, and of the cache, embedding and gains.
int matrix_bytes(mk_dtype t) { return t == MK_W8 ? 1 : t == MK_BF16 ? 2 : 4; }
int cache_bytes(mk_dtype t) { return t == MK_F32 ? 4 : 2; }
// Largest block of per-row scales one workgroup keeps in LDS (four consumer
// waves of 64 lanes carry four floats each between its load and its LDS store).
constexpr int MK_SC_MAX = 1024;

// Tag base of the next launch on a record buffer whose last launch used tags
// up to `end` (a launch tags its records base + l for layer index l in
// [0, L]): the range starts right after `end` and `end` moves to its last
// tag.  A range that would hold 0 (the tag of a never-written record) or wrap
// around 2^32 starts over at 1; *wrapped is then set, and the caller clears
// the buffer first so that no record left from 2^32 tags ago can match.
uint32_t next_tag_base(uint32_t &end, int L, bool *wrapped) {
    uint64_t nb = (uint64_t)end + 1;
    *wrapped = false;
    if (nb + (uint64_t)L > 0xFFFFFFFFull) {
        nb = 1;
        *wrapped = true;
    }
    end = (uint32_t)(nb + (uint64_t)L);
    return (uint32_t)nb;
}

// The record pointers of a launch, for a record buffer at `base`.
void set_records(MkParams &P, uint64_t *base, const RecLayout &r) {
    P.ll_xq = base + r.off[0];
    P.ll_xg = base + r.off[1];
    P.ll_qkv = base + r.off[2];
    P.ll_part = base + r.off[3];
    P.ll_o = base + r.off[4];
    P.ll_dpart = base + r.off[5];
    P.ll_amax = base + r.off[6];
}

// Once per device, with that device current: the device address of the
// static scratch.  Returns false if it cannot be taken.
bool scratch_setup(int dev) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (dev < 0 || dev >= MK_MAX_DEVICES) return false;
    if (g_scratch_ptr[dev]) return true;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return false;
    g_scratch_ptr[dev] = (uint64_t *)ptr;
    return true;
}

struct StageShape {
    int rows, k;
};

mk_status validate_desc(const mk_model_desc *d) {
    if (d->dtype != MK_F32 && d->dtype != MK_BF16 && d->dtype != MK_W8) return MK_ERR_DTYPE;
    const int eb = cache_bytes(d->dtype);
    if (d->dtype == MK_W8 && d->tied_embeddings) return MK_ERR_SHAPE;  // the int8 LM head is its own matrix
    if (d->n_layers < 1 || d->hidden < 8 || d->n_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 2 || d->ffn < 8 ||
        d->vocab < 1 || d->max_seq < 1)
        return MK_ERR_SHAPE;
    if (d->hidden % 8 || d->ffn % 8 || d->n_heads % d->n_kv_heads) return MK_ERR_SHAPE;
    const int gq = d->n_heads / d->n_kv_heads;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8) return MK_ERR_SHAPE;
    if (d->head_dim * eb != 128 && d->head_dim * eb != 256) return MK_ERR_SHAPE;
    if (!(d->rms_eps >= 0.0) || !(d->rope_theta > 0.0)) return MK_ERR_SHAPE;
    if ((int64_t)d->n_heads * d->head_dim > (1 << 20) || d->hidden > (1 << 20) || d->ffn > (1 << 22))
        return MK_ERR_SHAPE;
    return MK_OK;
}

// Ranges of the tuning knobs that need no device query.
mk_status validate_tuning(const mk_tuning *t) {
    if (!t) return MK_OK;
    if (t->grid < 0 || t->grid > MK_MAX_GRID || t->ring_slots < 0 || t->attn_splits < 0 || t->attn_splits > MK_MAX_SPLITS || t->timeout_ms < 0 ||
        t->cooperative < 0 || t->cooperative > 2 || t->trace < 0 || t->trace > 1 || t->prefetch_depth < 0 ||
        t->stage_drain < 0 || t->stage_drain > 1 || t->prefill_chunk < -1 || t->prefill_chunk > 4096 ||
        t->attn_pm_slots < -1 || t->slots_per_step < 0 || t->slots_per_step > 2)
        return MK_ERR_TUNING;
    if (t->ring_slots != 0 && (t->ring_slots < 3 || t->ring_slots > MK_MAX_RING)) return MK_ERR_TUNING;
    return MK_OK;
}

}  // namespace

extern "C" const char *mk_status_str(mk_status s) {
    switch (s) {
    case MK_OK: return "ok";
    case MK_ERR_NULL: return "null pointer argument";
    case MK_ERR_SHAPE: return "unsupported or inconsistent model shape";
    case MK_ERR_DTYPE: return "unsupported dtype";
    case MK_ERR_RANGE: return "token, position or count out of range";
    case MK_ERR_NOMEM: return "device allocation failed";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_DEVICE: return "device reported a failure";
    case MK_ERR_STATE: return "handle not ready: disabled by a device failure, or weights not all loaded";
    case MK_ERR_TUNING: return "tuning value out of range";
    case MK_ERR_SCRATCH: return "the model's cross-workgroup records exceed the static scratch (MK_STATIC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

extern "C" void mk_destroy(mk_handle *h) {
    if (!h) return;
    // Teardown has no way to report a failure: the frees' statuses are
    // deliberately dropped (a failed free leaves nothing to undo).
    void *const bufs[] = {h->packed, h->wg_off, h->gains, h->embed, h->rope, h->scl, h->ll, h->err, h->trace,
                          h->pf.X, h->pf.Ah, h->pf.Al, h->pf.Y, h->pf.Q, h->pf_tokens, (void *)h->pf.dmap};
    for (void *b : bufs) (void)hipFree(b);
    if (h->done) (void)hipEventDestroy(h->done);
    delete h;
}

// Geometry, allocations, RoPE table and launch-invariant arguments; the
// weights are pre-laid out afterwards by load_impl.
static mk_status create_impl(const mk_model_desc *desc, const mk_tuning *tun, mk_handle *h) {
    const mk_model_desc &D = *desc;
    const int L = D.n_layers, H = D.hidden, nh = D.n_heads, nkv = D.n_kv_heads, d = D.head_dim, F = D.ffn,
              V = D.vocab;
    const int dtype = dtype_code(D.dtype);
    const int eb = matrix_bytes(D.dtype);  // geometry of the packed matrices
    const int ebc = cache_bytes(D.dtype);  // cache rows, embedding
    const int gq = nh / nkv;
    const int lpp = d * ebc / 16;
    h->desc = D;
    h->emb_bytes = ebc;

    HIP_TRY(hipGetDevice(&h->device));
    // the static scratch of the no-allocation entry point, taken once per
    // device at the library's set-up; if it cannot be taken, that entry
    // point reports MK_ERR_HIP and everything else works as usual
    (void)scratch_setup(h->device);
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, h->device));
    h->cu_count = prop.multiProcessorCount;
    int wclk_khz = 0;
    HIP_TRY(hipDeviceGetAttribute(&wclk_khz, hipDeviceAttributeWallClockRate, h->device));
    if (wclk_khz <= 0) wclk_khz = 100000;

    // tuning (ranges were checked by validate_tuning)
    mk_tuning t;
    memset(&t, 0, sizeof t);
    if (tun) t = *tun;
    const int grid = t.grid ? t.grid : h->cu_count;
    if (grid > MK_MAX_GRID) return MK_ERR_TUNING;
    // consumers sharing one query head (GQ < 4) each produce a partial record,
    // so the combine merges splits * cph records per head, one lane each
    const int cph = MK_NUM_CONSUMERS / (gq < MK_NUM_CONSUMERS ? gq : MK_NUM_CONSUMERS);
    int splits = t.attn_splits ? t.attn_splits : (grid / nkv > 0 ? grid / nkv : 1);
    if (!t.attn_splits && splits > MK_MAX_SPLITS / cph) splits = MK_MAX_SPLITS / cph;
    if (splits * cph > MK_MAX_SPLITS) return MK_ERR_TUNING;
    if ((int64_t)splits * nkv > grid) return MK_ERR_TUNING;
    h->cooperative = t.cooperative == 1 ? 1 : 0;
    const int timeout_ms = t.timeout_ms ? t.timeout_ms : 2000;

    // stage geometry
    const StageShape shapes[ST_NUM] = {{(nh + 2 * nkv) * d, H}, {H, nh * d}, {2 * F, H}, {H, F}, {V, H}};
    MkParams &P = h->base;
    memset(&P, 0, sizeof P);
    std::vector<int64_t> off_host((size_t)ST_NUM * grid);
    // the packed buffer opens with one zeroed 16 KiB slot that no stage owns:
    // the loaders' masked reads land there (see the allocation below)
    int64_t total = MK_SLOT_BYTES;
    int vec_floats = 0, out_rows = 0;
    const int epc = MK_CHUNK_BYTES / eb;
    int max_rows_o = 0;  // x rows a workgroup owns (O-stage rows): reduced and kept in LDS
    for (int k = 0; k < ST_NUM; ++k) {
        MkStage &s = P.st[k];
        s.rows = shapes[k].rows;
        s.k = shapes[k].k;
        // the down stage is split along its input: its geometry follows the gate/up units
        s.units = k == ST_DOWN ? (int)ceil_div(2LL * F, 4) : (int)ceil_div(s.rows, 4);
        s.rbp = k == ST_DOWN ? 0 : (int)ceil_div((int64_t)s.k * eb, MK_CHUNK_BYTES);
        int64_t block = 0, max_nsl = 0;
        for (int w = 0; w < grid; ++w) {
            const int u0 = (int)((int64_t)w * s.units / grid), u1 = (int)((int64_t)(w + 1) * s.units / grid);
            off_host[(size_t)k * grid + w] = block;
            if (k == ST_DOWN) {
                const MkDownGeo dg = mk_down_geo(w, grid, s.units, F, H, 16 / eb);
                block += (int64_t)dg.nsl * MK_SLOT_BYTES;
                if (dg.nsl > max_nsl) max_nsl = dg.nsl;
                continue;
            }
            const int64_t nsl_w = ceil_div((int64_t)(u1 - u0) * s.rbp, 4);
            block += nsl_w * MK_SLOT_BYTES;
            if (nsl_w > max_nsl) max_nsl = nsl_w;
            if ((u1 - u0) * 4 > out_rows) out_rows = (u1 - u0) * 4;
            if (k == ST_O) {
                if ((u1 - u0) * 4 > 64) return MK_ERR_SHAPE;  // residual rows kept in LDS
                if ((u1 - u0) * 4 > max_rows_o) max_rows_o = (u1 - u0) * 4;
            }
        }
        if (s.rbp * epc > vec_floats) vec_floats = s.rbp * epc;
        // Striped slots: slot n of workgroup w at (n * grid + w) * 16 KiB of
        // the layer block, so that at any moment the grid streams one compact
        // window of memory (workgroups with fewer slots leave holes).
        for (int w = 0; w < grid; ++w) off_host[(size_t)k * grid + w] = (int64_t)w * MK_SLOT_BYTES;
        s.slot_stride = (int64_t)grid * MK_SLOT_BYTES;
        block = max_nsl * s.slot_stride;
        s.base = total;
        s.layer_stride = k == ST_LM ? 0 : block;
        total += k == ST_LM ? block : block * L;
    }
    // vec also holds: the SwiGLU outputs of this workgroup (down-stage input),
    // and the G partial sums of its x rows while they are reduced
    for (int w = 0; w < grid; ++w) {
        const MkDownGeo dg = mk_down_geo(w, grid, P.st[ST_DOWN].units, F, H, 16 / eb);
        if (dg.kp * (16 / eb) > vec_floats) vec_floats = dg.kp * (16 / eb);
    }
    if ((int64_t)grid * max_rows_o > vec_floats) vec_floats = grid * max_rows_o;
    // the down partials of one layer are addressed with a 32-bit buffer resource
    if ((int64_t)grid * H * 8 >= (1LL << 32)) return MK_ERR_SHAPE;
    // the attention stage gathers its group's queries and the new K/V row into vec
    if (vec_floats < (gq + 2) * d) vec_floats = (gq + 2) * d;
    // position-major attention (groups of four query heads) merges the four
    // consumers' per-head partials in vec, after the queries and the row of pos
    if (gq == MK_NUM_CONSUMERS && vec_floats < (gq + 2) * d + MK_NUM_CONSUMERS * gq * (d + 2))
        vec_floats = (gq + 2) * d + MK_NUM_CONSUMERS * gq * (d + 2);
    // per-row scale blocks of the INT8 matrices (two LDS copies, by layer parity)
    int sc_blk = 0, sc_lm = 0;
    if (dtype == 2) {
        auto nu = [&](int k, int w) {
            return (int)((int64_t)(w + 1) * P.st[k].units / grid) - (int)((int64_t)w * P.st[k].units / grid);
        };
        for (int w = 0; w < grid; ++w) {
            const int blk = 4 * (nu(ST_QKV, w) + 2 * nu(ST_O, w) + nu(ST_GU, w));
            if (blk > sc_blk) sc_blk = blk;
            if (4 * nu(ST_LM, w) > sc_lm) sc_lm = 4 * nu(ST_LM, w);
        }
        sc_blk = (sc_blk + 63) & ~63;
        sc_lm = (sc_lm + 63) & ~63;
        if (sc_blk > MK_SC_MAX || sc_lm > MK_SC_MAX) return MK_ERR_SHAPE;
    }
    const int lds_sc = sc_blk > sc_lm ? sc_blk : sc_lm;
    const int fixed = mk_kernel_lds_bytes(0, vec_floats, out_rows, 2 * lds_sc);
    int ns = t.ring_slots ? t.ring_slots : (MK_LDS_LIMIT - fixed) / MK_SLOT_BYTES;
    if (ns > MK_DEFAULT_RING && !t.ring_slots) ns = MK_DEFAULT_RING;  // a 9th slot measured no faster
    if (ns > MK_MAX_RING) ns = MK_MAX_RING;
    if (ns < 3 || fixed + ns * MK_SLOT_BYTES > MK_LDS_LIMIT) return MK_ERR_SHAPE;
    // A load needs a ring slot already consumed, and a data step's slots
    // must all have been issued before its barrier.
    const int sps = t.slots_per_step ? t.slots_per_step : 1;
    if (t.prefetch_depth > ns - sps || (t.prefetch_depth != 0 && t.prefetch_depth < sps)) return MK_ERR_TUNING;
    h->lds_bytes = mk_kernel_lds_bytes(ns, vec_floats, out_rows, 2 * lds_sc);
    const int per_cu = mk_kernel_max_blocks_per_cu(dtype, gq, lpp, h->lds_bytes);
    if (per_cu < 1) return MK_ERR_SHAPE;
    if (grid > per_cu * h->cu_count) return MK_ERR_TUNING;  // every workgroup must be resident

    // allocations
    h->packed_bytes = total;
    // The loaders' idle reads (cache positions past a split's end, slots past
    // the end of the stream) read the first 1 KiB of the buffer, which lies in
    // the zeroed slot that opens it and that no stage owns.  The attention
    // fold multiplies masked V values by probability 0, so they must be
    // finite numbers, whatever the weights are: int8 codes read as bf16 pairs
    // can spell a NaN.  The striped layout also leaves holes that no
    // pre-layout writes (for example workgroup 0's first slot when a stage has
    // fewer units than workgroups); the whole buffer is zeroed once.
    const int64_t packed_alloc = total;
    HIP_TRY(hipMalloc(&h->packed, packed_alloc));
    HIP_TRY(hipMemset(h->packed, 0, packed_alloc));
    HIP_TRY(hipMalloc(&h->wg_off, off_host.size() * sizeof(int64_t)));
    HIP_TRY(hipMemcpy(h->wg_off, off_host.data(), off_host.size() * sizeof(int64_t), hipMemcpyHostToDevice));
    const size_t ngain = (size_t)2 * L * H + H;
    HIP_TRY(hipMalloc(&h->gains, ngain * sizeof(float)));
    HIP_TRY(hipMalloc(&h->embed, (size_t)V * H * ebc));
    HIP_TRY(hipMalloc(&h->rope, (size_t)D.max_seq * d * sizeof(float)));
    if (dtype == 2) {
        const size_t n_sc = (size_t)L * grid * sc_blk + (size_t)grid * sc_lm;
        HIP_TRY(hipMalloc(&h->scl, n_sc * sizeof(float)));
        HIP_TRY(hipMemset(h->scl, 0, n_sc * sizeof(float)));
    }
    // tagged records, one array per dependency point, each with two buffers
    // (layers of even and odd index)
    const size_t n_rec[7] = {(size_t)2 * H, (size_t)2 * H, (size_t)2 * nkv * (gq + 2) * d,
                             (size_t)2 * nkv * splits * cph * gq * (d + 2), (size_t)2 * nh * d, (size_t)2 * grid * H,
                             (size_t)grid * 2};
    size_t n_ll = 0;
    for (int i = 0; i < 7; ++i) {
        h->rec.off[i] = n_ll;
        n_ll += (n_rec[i] + 31) & ~(size_t)31;  // each array on a 256-byte boundary
    }
    h->rec.off[7] = n_ll;
    HIP_TRY(hipMalloc(&h->ll, n_ll * sizeof(uint64_t)));
    HIP_TRY(hipMemset(h->ll, 0, n_ll * sizeof(uint64_t)));  // tag 0: never a launch's tag
    HIP_TRY(hipEventCreateWithFlags(&h->done, hipEventDisableTiming));
    HIP_TRY(hipMalloc(&h->err, 64 * sizeof(uint32_t)));
    HIP_TRY(hipMemset(h->err, 0, 64 * sizeof(uint32_t)));
    if (t.trace) {
        // stage timeline, consumer data steps of layer 1, loader barriers of layer 1
        h->trace_len = (int64_t)grid * (5 * L + 2) * 4 + (int64_t)grid * 64 * 2 + (int64_t)grid * 96 * 2;
        HIP_TRY(hipMalloc(&h->trace, h->trace_len * sizeof(uint64_t)));
        HIP_TRY(hipMemset(h->trace, 0, h->trace_len * sizeof(uint64_t)));
    }

    for (int k = 0; k < ST_NUM; ++k) P.st[k].wg_off = h->wg_off + (size_t)k * grid;
    h->layer_loaded.assign((size_t)L, 0);

    // rotary table: angle pos * theta^(-2i/d), evaluated in double
    {
        std::vector<float> tab((size_t)D.max_seq * d);
        for (int pos = 0; pos < D.max_seq; ++pos)
            for (int i = 0; i < d / 2; ++i) {
                const double ang = (double)pos * pow(D.rope_theta, -2.0 * (double)i / (double)d);
                tab[((size_t)pos * (d / 2) + i) * 2] = (float)cos(ang);
                tab[((size_t)pos * (d / 2) + i) * 2 + 1] = (float)sin(ang);
            }
        HIP_TRY(hipMemcpy(h->rope, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice));
    }
    HIP_TRY(hipDeviceSynchronize());

    // launch-invariant kernel arguments
    P.L = L; P.H = H; P.nh = nh; P.nkv = nkv; P.d = d; P.F = F; P.V = V; P.max_seq = D.max_seq;
    P.eps = (float)D.rms_eps;
    P.grid = grid; P.ring_slots = ns; P.splits = splits; P.lds_vec_floats = vec_floats; P.lds_out_rows = out_rows;
    P.slots_per_step = sps;
    P.prefetch_depth = t.prefetch_depth ? t.prefetch_depth : ns - sps;
    P.stage_drain = t.stage_drain;
    // default: head-major at every length (position-major measured slower,
    // 947 against 937 us per 32K-context step; the slot is bound by the
    // consumers' arithmetic, not by their LDS reads)
    P.attn_pm_slots = t.attn_pm_slots > 0 ? t.attn_pm_slots : (1 << 30);
    P.packed = h->packed;
    P.scl = h->scl;
    P.sc_blk = sc_blk;
    P.sc_lm = sc_lm;
    P.lds_sc_floats = lds_sc;
    P.g_attn = h->gains; P.g_ffn = h->gains + (size_t)L * H; P.g_final = h->gains + (size_t)2 * L * H;
    P.embed = h->embed;
    P.rope = h->rope;
    set_records(P, h->ll, h->rec);
    P.err = h->err;
    P.timeout_ticks = (int64_t)timeout_ms * wclk_khz;
    P.err_check_ticks = (int64_t)wclk_khz / 50;  // 20 us
    P.trace = h->trace;

    // batched prefill buffers, when the geometry allows it (bf16, aligned
    // down-stage inputs) and the tuning does not ask for decode launches
    if (t.prefill_chunk != -1 && mk_prefill_supported(&P, dtype)) {
        // default: chunks of 4096 tokens, or max_seq if smaller (a prompt of
        // up to 4096 tokens in one chunk; longer prompts get twice the
        // workgroups per launch of 2048-token chunks: 32K prefill 320 -> 309 ms)
        const int T = t.prefill_chunk > 0 ? t.prefill_chunk : (D.max_seq < 4096 ? D.max_seq : 4096);
        auto r32 = [](int k) { return (k + 31) & ~31; };
        int kmax = H > nh * d ? H : nh * d;
        if (F > kmax) kmax = F;
        const int nqkv = (nh + 2 * nkv) * d;
        MkPrefillBufs &B = h->pf;
        B.lda = r32(kmax);
        B.ldy = nqkv > 2 * F ? nqkv : 2 * F;
        HIP_TRY(hipMalloc(&B.X, (size_t)T * H * sizeof(float)));
        HIP_TRY(hipMalloc(&B.Ah, (size_t)T * B.lda * sizeof(uint16_t)));
        HIP_TRY(hipMalloc(&B.Al, (size_t)T * B.lda * sizeof(uint16_t)));
        HIP_TRY(hipMalloc(&B.Y, (size_t)T * B.ldy * sizeof(float)));
        // the rotated queries, and during the O and down projections the
        // second input split's sums ([T][H])
        HIP_TRY(hipMalloc(&B.Q, (size_t)T * (nh * d > H ? nh * d : H) * sizeof(float)));
        HIP_TRY(hipMalloc(&h->pf_tokens, (size_t)D.max_seq * sizeof(int32_t)));
        // where each block of 8 down-projection inputs lives (mk_down_geo)
        {
            const int epl = 16 / eb, U = P.st[ST_DOWN].units;
            std::vector<int32_t> dm((size_t)(F / 8) * 4);
            for (int f8 = 0; f8 < F / 8; ++f8) {
                const int f = 8 * f8, u = f >> 1;
                const int w = (int)(((int64_t)(u + 1) * grid - 1) / U);  // owner of gate/up unit u
                const MkDownGeo dg = mk_down_geo(w, grid, U, F, H, epl);
                dm[(size_t)f8 * 4 + 0] = (int32_t)off_host[(size_t)ST_DOWN * grid + w];
                dm[(size_t)f8 * 4 + 1] = dg.kp;
                dm[(size_t)f8 * 4 + 2] = (f - dg.f0) / epl;
                dm[(size_t)f8 * 4 + 3] = ((f - dg.f0) % epl) * eb;
            }
            int32_t *dmap = nullptr;
            HIP_TRY(hipMalloc(&dmap, dm.size() * sizeof(int32_t)));
            HIP_TRY(hipMemcpy(dmap, dm.data(), dm.size() * sizeof(int32_t), hipMemcpyHostToDevice));
            B.dmap = dmap;
        }
        B.t_max = T;
    }

    // algorithmic bytes: every matrix (with its per-row scales when INT8),
    // the gains, the LM head and one embedding row
    const int64_t mat = (int64_t)((nh + 2 * nkv) * d) * H + (int64_t)H * nh * d + 3LL * H * F;
    const int64_t mrows = (int64_t)(nh + 2 * nkv) * d + H + 2LL * F + H;
    const int64_t sc = dtype == 2 ? 4 : 0;
    h->weight_bytes = (int64_t)L * (mat * eb + mrows * sc + 2LL * H * ebc) + (int64_t)V * H * eb + (int64_t)V * sc +
                      2LL * H * ebc;
    return MK_OK;
}


// Pre-layout of layers [first, first + n) from wp->layers[0 .. n) and, when
// wp->embed is set, of the embedding, final norm and LM head.  Synchronous.
static mk_status load_impl(mk_handle *h, const mk_weight_ptrs *wp, int first, int n) {
    const mk_model_desc &D = h->desc;
    const MkParams &P = h->base;
    const int L = D.n_layers, H = D.hidden, V = D.vocab, grid = P.grid;
    const int eb = matrix_bytes(D.dtype);
    const int gdt = D.dtype == MK_F32 ? 0 : 1;  // storage of the gains
    const bool q8 = D.dtype == MK_W8;
    // no step of this handle may still be reading the weights being replaced
    HIP_TRY(hipDeviceSynchronize());
    for (int i = 0; i < n; ++i) {
        const int l = first + i;
        const mk_layer_ptrs &lw = wp->layers[i];
        for (int k = 0; k < ST_LM; ++k) {
            const void *s0 = nullptr, *s1 = nullptr, *s2 = nullptr;
            switch (k) {
            case ST_QKV: s0 = lw.wq; s1 = lw.wk; s2 = lw.wv; break;
            case ST_O: s0 = lw.wo; break;
            case ST_GU: s0 = lw.w_gate; s1 = lw.w_up; break;
            default: s0 = lw.w_down; break;
            }
            if (mk_launch_prelayout_stage(h->packed + P.st[k].base + (int64_t)l * P.st[k].layer_stride, &P.st[k], grid,
                                          k, eb, s0, s1, s2, D.n_heads, D.n_kv_heads, D.head_dim, nullptr))
                return MK_ERR_HIP;
        }
        if (q8) {
            const float *sc[7] = {lw.s_wq, lw.s_wk, lw.s_wv, lw.s_wo, lw.s_w_gate, lw.s_w_up, lw.s_w_down};
            if (mk_launch_prelayout_scales(h->scl, &P, l, sc, nullptr)) return MK_ERR_HIP;
        }
        if (mk_launch_to_f32(h->gains + (size_t)l * H, lw.attn_norm, H, gdt, nullptr)) return MK_ERR_HIP;
        if (mk_launch_to_f32(h->gains + (size_t)(L + l) * H, lw.ffn_norm, H, gdt, nullptr)) return MK_ERR_HIP;
    }
    if (wp->embed) {
        const void *lm = D.tied_embeddings ? wp->embed : wp->lm_head;
        if (mk_launch_prelayout_stage(h->packed + P.st[ST_LM].base, &P.st[ST_LM], grid, ST_LM, eb, lm, nullptr,
                                      nullptr, D.n_heads, D.n_kv_heads, D.head_dim, nullptr))
            return MK_ERR_HIP;
        if (q8) {
            const float *sc[7] = {wp->lm_head_scale, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
            if (mk_launch_prelayout_scales(h->scl, &P, L, sc, nullptr)) return MK_ERR_HIP;
        }
        if (mk_launch_to_f32(h->gains + (size_t)2 * L * H, wp->final_norm, H, gdt, nullptr)) return MK_ERR_HIP;
        HIP_TRY(hipMemcpy(h->embed, wp->embed, (size_t)V * H * h->emb_bytes, hipMemcpyDeviceToDevice));
    }
    // the sources may be freed when this returns
    HIP_TRY(hipDeviceSynchronize());
    for (int i = 0; i < n; ++i) {
        char &done = h->layer_loaded[(size_t)(first + i)];
        if (!done) ++h->layers_loaded;
        done = 1;
    }
    if (wp->embed) h->head_loaded = true;
    return MK_OK;
}

// Null checks of the weight pointers a load will read: layers[0 .. n) and,
// when embed is set, the head tensors.
static mk_status check_weight_ptrs(const mk_model_desc *desc, const mk_weight_ptrs *w, int n) {
    const bool q8 = desc->dtype == MK_W8;
    if (w->embed && (!w->final_norm || (!desc->tied_embeddings && !w->lm_head) || (q8 && !w->lm_head_scale)))
        return MK_ERR_NULL;
    if (n > 0 && !w->layers) return MK_ERR_NULL;
    for (int l = 0; l < n; ++l) {
        const mk_layer_ptrs &lw = w->layers[l];
        if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.ffn_norm || !lw.w_gate || !lw.w_up ||
            !lw.w_down)
            return MK_ERR_NULL;
        if (q8 && (!lw.s_wq || !lw.s_wk || !lw.s_wv || !lw.s_wo || !lw.s_w_gate || !lw.s_w_up || !lw.s_w_down))
            return MK_ERR_NULL;
    }
    return MK_OK;
}

extern "C" mk_status mk_create(const mk_model_desc *desc, const mk_weight_ptrs *weights, const mk_tuning *tuning,
                               mk_handle **out) {
    if (!out) return MK_ERR_NULL;
    *out = nullptr;
    if (!desc || !weights) return MK_ERR_NULL;
    mk_status s = validate_desc(desc);
    if (s != MK_OK) return s;
    s = validate_tuning(tuning);
    if (s != MK_OK) return s;
    if (!weights->embed) return MK_ERR_NULL;
    s = check_weight_ptrs(desc, weights, desc->n_layers);
    if (s != MK_OK) return s;
    mk_handle *h = new mk_handle();
    s = create_impl(desc, tuning, h);
    if (s == MK_OK) s = load_impl(h, weights, 0, desc->n_layers);
    if (s != MK_OK) {
        mk_destroy(h);
        return s;
    }
    *out = h;
    return MK_OK;
}

extern "C" mk_status mk_create_deferred(const mk_model_desc *desc, const mk_tuning *tuning, mk_handle **out) {
    if (!out) return MK_ERR_NULL;
    *out = nullptr;
    if (!desc) return MK_ERR_NULL;
    mk_status s = validate_desc(desc);
    if (s != MK_OK) return s;
    s = validate_tuning(tuning);
    if (s != MK_OK) return s;
    mk_handle *h = new mk_handle();
    s = create_impl(desc, tuning, h);
    if (s != MK_OK) {
        mk_destroy(h);
        return s;
    }
    *out = h;
    return MK_OK;
}

extern "C" mk_status mk_load_weights(mk_handle *h, const mk_weight_ptrs *weights, int32_t first_layer,
                                     int32_t n_layers) {
    if (!h || !weights) return MK_ERR_NULL;
    if (first_layer < 0 || n_layers < 0 || (int64_t)first_layer + n_layers > h->desc.n_layers) return MK_ERR_RANGE;
    mk_status s = check_weight_ptrs(&h->desc, weights, n_layers);
    if (s != MK_OK) return s;
    return load_impl(h, weights, first_layer, n_layers);
}

static mk_status check_kv(const mk_handle *h, const mk_kv_cache *kv) {
    if (!kv || !kv->k || !kv->v) return MK_ERR_NULL;
    if (kv->max_seq != h->desc.max_seq) return MK_ERR_SHAPE;
    return MK_OK;
}

// Before a call's launches: a call on a stream other than the previous call's
// waits for the previous call to complete (the tagged records and the cache
// row at pos are shared by every launch of the handle).
static mk_status order_before(mk_handle *h, void *stream) {
    if (h->done_recorded && (hipStream_t)stream != h->last_stream)
        HIP_TRY(hipStreamWaitEvent((hipStream_t)stream, h->done, 0));
    return MK_OK;
}
// After a call's launches: mark its completion on its stream.
static mk_status order_after(mk_handle *h, void *stream) {
    HIP_TRY(hipEventRecord(h->done, (hipStream_t)stream));
    h->done_recorded = true;
    h->last_stream = (hipStream_t)stream;
    return MK_OK;
}

// One launch.  records: the record buffer (NULL: the handle's own, tagged
// from the handle's counter); tag_base: the launch's tag base when records
// is given.
static mk_status launch(mk_handle *h, const mk_kv_cache *kv, int32_t token, const int32_t *token_dev, int32_t pos,
                        int want_logits, float *logits, int32_t *token_out, void *stream,
                        uint64_t *records = nullptr, uint32_t tag_base = 0) {
    if (h->layers_loaded < h->desc.n_layers || !h->head_loaded) return MK_ERR_STATE;  // weights still missing
    MkParams p = h->base;
    p.kc = kv->k;
    p.vc = kv->v;
    p.token = token;
    p.token_dev = token_dev;
    p.pos = pos;
    p.want_logits = want_logits;
    p.logits = logits;
    p.token_out = token_out;
    if (records) {
        set_records(p, records, h->rec);
        p.tag = tag_base;
    } else {
        bool wrapped = false;
        p.tag = next_tag_base(h->tag_end, h->desc.n_layers, &wrapped);
        if (wrapped && mk_launch_zero(h->ll, (int64_t)h->rec.off[7] * 8, stream)) return MK_ERR_HIP;
    }
    int rc = mk_launch_decode(&p, dtype_code(h->desc.dtype), h->cooperative, stream);
    return rc ? MK_ERR_HIP : MK_OK;
}

// One call's launches, ordered after the handle's previous call.
static mk_status launch_one(mk_handle *h, const mk_kv_cache *kv, int32_t token, const int32_t *token_dev,
                            int32_t pos, int want_logits, float *logits, int32_t *token_out, void *stream) {
    if (h->layers_loaded < h->desc.n_layers || !h->head_loaded) return MK_ERR_STATE;
    mk_status s = order_before(h, stream);
    if (s == MK_OK) s = launch(h, kv, token, token_dev, pos, want_logits, logits, token_out, stream);
    if (s == MK_OK) s = order_after(h, stream);
    return s;
}

extern "C" mk_status mk_decode_step(mk_handle *h, int32_t token_id, int32_t pos, const mk_kv_cache *kv,
                                    float *logits_out, void *stream) {
    if (!h || !logits_out) return MK_ERR_NULL;
    if (h->disabled) return MK_ERR_STATE;
    mk_status s = check_kv(h, kv);
    if (s != MK_OK) return s;
    if (token_id < 0 || token_id >= h->desc.vocab || pos < 0 || pos >= h->desc.max_seq) return MK_ERR_RANGE;
    return launch_one(h, kv, token_id, nullptr, pos, 1, logits_out, nullptr, stream);
}

extern "C" mk_status mk_decode_step_device_token(mk_handle *h, const int32_t *token_in, int32_t pos,
                                                 const mk_kv_cache *kv, float *logits_out, int32_t *token_out,
                                                 void *stream) {
    if (!h || !token_in || !token_out) return MK_ERR_NULL;
    if (h->disabled) return MK_ERR_STATE;
    mk_status s = check_kv(h, kv);
    if (s != MK_OK) return s;
    if (pos < 0 || pos >= h->desc.max_seq) return MK_ERR_RANGE;
    return launch_one(h, kv, 0, token_in, pos, 1, logits_out, token_out, stream);
}

extern "C" mk_status mk_decode_step_device_token_noalloc(mk_handle *h, const int32_t *token_in, int32_t pos,
                                                         const mk_kv_cache *kv, float *logits_out, int32_t *token_out,
                                                         void *stream) {
    if (!h || !token_in || !token_out) return MK_ERR_NULL;
    if (h->disabled) return MK_ERR_STATE;
    mk_status s = check_kv(h, kv);
    if (s != MK_OK) return s;
    if (pos < 0 || pos >= h->desc.max_seq) return MK_ERR_RANGE;
    if (h->rec.off[7] * sizeof(uint64_t) > (size_t)MK_STATIC_SCRATCH_BYTES) return MK_ERR_SCRATCH;
    if (h->layers_loaded < h->desc.n_layers || !h->head_loaded) return MK_ERR_STATE;
    uint64_t *base = nullptr;
    uint32_t tb = 0;
    bool wrapped = false;
    {
        // every call on a device shares its array and one tag counter, so a
        // record another handle left there never carries an awaited tag
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        const int dev = h->device;
        if (dev < 0 || dev >= MK_MAX_DEVICES || !g_scratch_ptr[dev]) return MK_ERR_HIP;
        base = g_scratch_ptr[dev];
        tb = next_tag_base(g_scratch_tag_end[dev], h->desc.n_layers, &wrapped);
    }
    s = order_before(h, stream);
    if (s == MK_OK && wrapped && mk_launch_zero(base, (int64_t)MK_STATIC_SCRATCH_BYTES, stream)) s = MK_ERR_HIP;
    if (s == MK_OK) s = launch(h, kv, 0, token_in, pos, 1, logits_out, token_out, stream, base, tb);
    if (s == MK_OK) s = order_after(h, stream);
    return s;
}

extern "C" mk_status mk_prefill_kv(mk_handle *h, const int32_t *tokens, int32_t n, int32_t start_pos,
                                   const mk_kv_cache *kv, void *stream) {
    if (!h) return MK_ERR_NULL;
    if (h->disabled) return MK_ERR_STATE;
    mk_status s = check_kv(h, kv);
    if (s != MK_OK) return s;
    if (n < 0 || start_pos < 0 || (int64_t)start_pos + n > h->desc.max_seq) return MK_ERR_RANGE;
    if (n > 0 && !tokens) return MK_ERR_NULL;
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= h->desc.vocab) return MK_ERR_RANGE;
    if (n == 0) return MK_OK;
    if (h->layers_loaded < h->desc.n_layers || !h->head_loaded) return MK_ERR_STATE;
    s = order_before(h, stream);
    if (s == MK_OK && h->pf.t_max > 0) {
        // batched: the token ids go to the device once, then chunks of up to
        // t_max positions run the token-parallel kernels
        if (hipMemcpyAsync(h->pf_tokens + start_pos, tokens, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice,
                           (hipStream_t)stream) != hipSuccess)
            s = MK_ERR_HIP;
        MkParams p = h->base;
        p.kc = kv->k;
        p.vc = kv->v;
        for (int i = 0; i < n && s == MK_OK; i += h->pf.t_max) {
            const int T = n - i < h->pf.t_max ? n - i : h->pf.t_max;
            MkPrefillBufs b = h->pf;
            b.tok = h->pf_tokens + start_pos + i;
            if (mk_prefill_chunk(&p, &b, T, start_pos + i, stream)) s = MK_ERR_HIP;
        }
    } else {
        for (int i = 0; i < n && s == MK_OK; ++i)
            s = launch(h, kv, tokens[i], nullptr, start_pos + i, 0, nullptr, nullptr, stream);
    }
    if (s == MK_OK) s = order_after(h, stream);
    return s;
}

extern "C" mk_status mk_get_device_error(mk_handle *h) {
    if (!h) return MK_ERR_NULL;
    // the handle's last call, on whatever stream it was enqueued
    if (h->done_recorded) HIP_TRY(hipEventSynchronize(h->done));
    uint32_t err = 0;
    HIP_TRY(hipMemcpy(&err, h->base.err, sizeof err, hipMemcpyDeviceToHost));
    if (err) {
        h->disabled = true;
        return MK_ERR_DEVICE;
    }
    return h->disabled ? MK_ERR_STATE : MK_OK;
}

extern "C" mk_status mk_read_trace(mk_handle *h, uint64_t *host_out, int64_t capacity) {
    if (!h || !host_out) return MK_ERR_NULL;
    if (!h->trace || capacity < h->trace_len) return MK_ERR_RANGE;
    if (h->done_recorded) HIP_TRY(hipEventSynchronize(h->done));
    HIP_TRY(hipMemcpy(host_out, h->trace, h->trace_len * sizeof(uint64_t), hipMemcpyDeviceToHost));
    return MK_OK;
}

extern "C" mk_status mk_get_info(const mk_handle *h, mk_info *info) {
    if (!h || !info) return MK_ERR_NULL;
    info->grid = h->base.grid;
    info->ring_slots = h->base.ring_slots;
    info->prefetch_slots = h->base.prefetch_depth;
    info->attn_splits = h->base.splits;
    info->block_threads = MK_BLOCK_THREADS;
    info->lds_bytes = h->lds_bytes;
    info->cu_count = h->cu_count;
    info->packed_bytes = h->packed_bytes;
    info->weight_bytes = h->weight_bytes;
    info->record_bytes = (int64_t)h->rec.off[7] * (int64_t)sizeof(uint64_t);
    info->prefill_chunk = h->pf.t_max;
    info->slots_per_step = h->base.slots_per_step;
    return MK_OK;
}
