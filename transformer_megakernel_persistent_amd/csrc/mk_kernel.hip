// Persistent batch-1 decode megakernel for gfx950 (MI355X).
//
// One launch runs a whole decode step (cloud.baidu.com/article/9434380,
// section 4.2: one launch with an internal pipeline instead of one launch
// per operator; developer.baidu.com/article/detail.html?id=8006242, section
// 4.1).  Each workgroup is resident on one CU for the whole step and has two
// roles:
//
//   loader waves (4)    copy the workgroup's weight slots -- and, for the
//                       attention stage, its KV-cache blocks -- from HBM into
//                       an LDS ring with gfx950 direct-to-LDS 16-byte loads,
//                       each wave a quarter (four 1 KiB chunks) of every
//                       16 KiB slot.  A workgroup's weight slots are striped
//                       with the other workgroups': slot n of workgroup w
//                       lies at w * 16 KiB + n * slot_stride of its stage's
//                       layer block, slot_stride = grid * 16 KiB.
//                       Weights and old cache positions do not depend on
//                       activations, so the loaders run up to ring_slots-1
//                       slots ahead ACROSS stage boundaries: weight streaming
//                       continues while consumers wait on a dependency (the
//                       in-kernel prefetch pipeline of cloud.baidu.com/
//                       article/9434380 section 五 step 3, and the double-
//                       buffered prefetch of the MegaKernel tutorial 4.2.1).
//   consumer waves (4)  compute from the ring: GEMV dot products reduced with
//                       wave64 DPP (no MFMA: at batch 1 this is a
//                       matrix-vector product), split-K flash-decode attention,
//                       and the fused epilogues (RoPE + KV append, residual
//                       add, SwiGLU, logits + argmax).
//
// All waves step through the same program; each step starts with one
// s_barrier.  A step is either a data step (consumers use one ring slot) or
// a stage boundary (the consumers finish the stage's epilogue and gather the
// next stage's input).
//
// Cross-workgroup values travel as tagged records: each value is stored with
// one 64-bit device-scope store together with a tag naming the launch and
// the layer (mixed with the value's bits, see tag_word), and readers poll
// the records they need until every tag matches.  Every dependency point has
// its own record array with two buffers (layers of even and odd index), so
// the data carry their own validity: no flags, counters, store-completion
// waits or separate flag round trips.  The attention splits write tagged
// partials; each workgroup then merges a slice of the attention output
// straight from them (log-sum-exp), with no atomic counter.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mk_internal.h"

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));

#define LDS __attribute__((address_space(3)))
#define GLB __attribute__((address_space(1)))
#define MK_COMPILER_BARRIER() asm volatile("" ::: "memory")
#define MK_WAIT_VM0() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")

// ---- device-scope (sc1) accesses ----------------------------------------
__device__ __forceinline__ uint32_t ldcu(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stcu(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resources: out-of-range offsets read as zero.  aux bit 4 = sc1
// (device scope) on gfx950, so these loads observe other workgroups' sc1
// stores without an L2 invalidate.
#define MK_SC1 16
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u4v ld16c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, MK_SC1);
}
__device__ __forceinline__ f4v as_f4(u4v v) {
    return f4v{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
}

// s_waitcnt encoding (gfx9): vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
// n a multiple of 4 up to 60; anything else waits for every load
__device__ __forceinline__ void wait_vm_rt(int n) {
    switch (n) {
    case 4: wait_vm<4>(); break;
    case 8: wait_vm<8>(); break;
    case 12: wait_vm<12>(); break;
    case 16: wait_vm<16>(); break;
    case 20: wait_vm<20>(); break;
    case 24: wait_vm<24>(); break;
    case 28: wait_vm<28>(); break;
    case 32: wait_vm<32>(); break;
    case 36: wait_vm<36>(); break;
    case 40: wait_vm<40>(); break;
    case 44: wait_vm<44>(); break;
    case 48: wait_vm<48>(); break;
    case 52: wait_vm<52>(); break;
    case 56: wait_vm<56>(); break;
    case 60: wait_vm<60>(); break;
    default: wait_vm<0>(); break;
    }
}

// ---- cross-lane reductions (wave64 DPP) -----------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
// Sum over all 64 lanes; result valid in every lane (read from lane 63).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);        // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);        // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);       // row_half_mirror: 8-lane sums
    v += dpp<0x140>(v);       // row_mirror: 16-lane sums
    v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Sum within aligned groups of LPP (8 or 16) lanes, result in every lane.
template <int LPP>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    if (LPP == 16) v += dpp<0x140>(v);
    return v;
}
// Sum / max across the groups of size GS (8, 16 or 32): lanes with equal
// (lane % GS).  VALU only: DPP row_ror:8 pairs lanes i and i^8 inside a row,
// and the gfx950 permlane16/32 swaps hand each lane its i^16 / i^32 partner;
// the sum of the two swapped registers is the pair sum in both lanes.
__device__ __forceinline__ float pair16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int GS>
__device__ __forceinline__ float xgroup_sum(float v) {
    if (GS <= 8) v += dpp<0x128>(v);  // row_ror:8
    if (GS <= 16) v = pair16_sum(v);
    return pair32_sum(v);
}
template <int GS>
__device__ __forceinline__ float xgroup_max(float v) {
    if (GS <= 8) v = fmaxf(v, dpp<0x128>(v));
    if (GS <= 16) v = pair16_max(v);
    return pair32_max(v);
}
// Max over all 64 lanes, result in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, dpp<0x128>(v));  // every lane of a row now holds the row max
    v = pair16_max(v);
    return pair32_max(v);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Weight elements per 16-byte piece: float32, bfloat16, int8 (dtype 2).
constexpr int wepl(int dt) { return dt == 2 ? 16 : dt ? 8 : 4; }

// Signed byte k of w as a float (an int8 weight code; exact).
__device__ __forceinline__ float i8f(uint32_t w, int k) { return (float)((int32_t)(w << (24 - 8 * k)) >> 24); }

// Dot product of one 16-byte weight piece (in LDS) with the matching input
// elements (in LDS).  INT8 pieces give the sum of code * input; the row's
// scale is applied to the finished row sum.
template <int DT>
__device__ __forceinline__ float piece_dot(const LDS unsigned char *wp, const LDS float *hp) {
    if constexpr (DT == 2) {
        const u4v w = *(const LDS u4v *)wp;
        const f4v h0 = *(const LDS f4v *)hp;
        const f4v h1 = *(const LDS f4v *)(hp + 4);
        const f4v h2 = *(const LDS f4v *)(hp + 8);
        const f4v h3 = *(const LDS f4v *)(hp + 12);
        float a = i8f(w.x, 0) * h0.x;
        float b = i8f(w.x, 1) * h0.y;
        a = fmaf(i8f(w.x, 2), h0.z, a);
        b = fmaf(i8f(w.x, 3), h0.w, b);
        a = fmaf(i8f(w.y, 0), h1.x, a);
        b = fmaf(i8f(w.y, 1), h1.y, b);
        a = fmaf(i8f(w.y, 2), h1.z, a);
        b = fmaf(i8f(w.y, 3), h1.w, b);
        a = fmaf(i8f(w.z, 0), h2.x, a);
        b = fmaf(i8f(w.z, 1), h2.y, b);
        a = fmaf(i8f(w.z, 2), h2.z, a);
        b = fmaf(i8f(w.z, 3), h2.w, b);
        a = fmaf(i8f(w.w, 0), h3.x, a);
        b = fmaf(i8f(w.w, 1), h3.y, b);
        a = fmaf(i8f(w.w, 2), h3.z, a);
        b = fmaf(i8f(w.w, 3), h3.w, b);
        return a + b;
    } else if constexpr (DT == 1) {
        const u4v w = *(const LDS u4v *)wp;
        const f4v h0 = *(const LDS f4v *)hp;
        const f4v h1 = *(const LDS f4v *)(hp + 4);
        float a = bf_lo(w.x) * h0.x;
        a = fmaf(bf_hi(w.x), h0.y, a);
        a = fmaf(bf_lo(w.y), h0.z, a);
        a = fmaf(bf_hi(w.y), h0.w, a);
        a = fmaf(bf_lo(w.z), h1.x, a);
        a = fmaf(bf_hi(w.z), h1.y, a);
        a = fmaf(bf_lo(w.w), h1.z, a);
        a = fmaf(bf_hi(w.w), h1.w, a);
        return a;
    } else {
        const f4v w = *(const LDS f4v *)wp;
        const f4v h = *(const LDS f4v *)hp;
        float a = w.x * h.x;
        a = fmaf(w.y, h.y, a);
        a = fmaf(w.z, h.z, a);
        a = fmaf(w.w, h.w, a);
        return a;
    }
}

// Same with the input elements already in registers.
template <int DT>
__device__ __forceinline__ float piece_dot_reg(const LDS unsigned char *wp, const float (&h)[wepl(DT)]) {
    if constexpr (DT == 2) {
        const u4v w = *(const LDS u4v *)wp;
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float a = i8f(ww[0], 0) * h[0];
        float b = i8f(ww[0], 1) * h[1];
#pragma unroll
        for (int e = 2; e < 16; e += 2) {
            a = fmaf(i8f(ww[e >> 2], e & 3), h[e], a);
            b = fmaf(i8f(ww[e >> 2], (e & 3) + 1), h[e + 1], b);
        }
        return a + b;
    } else if constexpr (DT == 1) {
        const u4v w = *(const LDS u4v *)wp;
        float a = bf_lo(w.x) * h[0];
        float b = bf_hi(w.x) * h[1];
        a = fmaf(bf_lo(w.y), h[2], a);
        b = fmaf(bf_hi(w.y), h[3], b);
        a = fmaf(bf_lo(w.z), h[4], a);
        b = fmaf(bf_hi(w.z), h[5], b);
        a = fmaf(bf_lo(w.w), h[6], a);
        b = fmaf(bf_hi(w.w), h[7], b);
        return a + b;
    } else {
        const f4v w = *(const LDS f4v *)wp;
        return fmaf(w.x, h[0], w.y * h[1]) + fmaf(w.z, h[2], w.w * h[3]);
    }
}

// Elements of a 16-byte piece as floats.
template <int DT>
__device__ __forceinline__ void piece_load(const LDS unsigned char *p, float (&v)[16 / (DT ? 2 : 4)]) {
    if constexpr (DT == 1) {
        const u4v w = *(const LDS u4v *)p;
        v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
        v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
    } else {
        const f4v w = *(const LDS f4v *)p;
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    }
}

// Element e of a 16-byte piece held as raw words (bf16 pairs or floats).
template <int DT>
__device__ __forceinline__ float piece_elem(const u4v &w, int e) {
    if constexpr (DT == 1) {
        const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
        return (e & 1) ? bf_hi(x) : bf_lo(x);
    } else {
        return __uint_as_float(e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w);
    }
}

// The input elements matching a 16-byte weight piece, from LDS.
template <int DT>
__device__ __forceinline__ void piece_in(const LDS float *hp, float (&h)[wepl(DT)]) {
#pragma unroll
    for (int k = 0; k < wepl(DT); k += 4) {
        const f4v t = *(const LDS f4v *)(hp + k);
        h[k] = t.x; h[k + 1] = t.y; h[k + 2] = t.z; h[k + 3] = t.w;
    }
}

// The high word of a tagged record: the tag XOR the value's bits.  A reader
// accepts a record when its high word equals the tag it awaits XOR the low
// word it read.  So it has read the awaited value even if its 16-byte load
// combined the halves of two different stores: a stale low word passes only
// if it equals the fresh value, a stale high word only next to the fresh low
// word, and a stale record never (its tag differs).  No assumption on the
// atomicity of a 16-byte load is needed, and the check is one XOR.
__device__ __forceinline__ uint32_t tag_word(uint32_t tag, uint32_t bits) { return tag ^ bits; }

// Poll N 16-byte pieces (two tagged records each) at byte offsets off(u)
// of rs, for the lanes' bits set in mask, until both records of every piece
// carry tag; pieces already valid are not read again.  on_fail() is called
// after each incomplete round and ends the wait by returning false.
template <int N, class O, class F>
__device__ __forceinline__ bool poll16(__amdgpu_buffer_rsrc_t rs, O &&off, uint32_t mask, u4v (&v)[N], uint32_t tag,
                                       F &&on_fail) {
    uint32_t pend = mask;
    while (true) {
#pragma unroll
        for (int u = 0; u < N; ++u)
            if (pend & (1u << u)) v[u] = ld16c(rs, off(u));
#pragma unroll
        for (int u = 0; u < N; ++u)
            if ((pend & (1u << u)) && v[u].y == tag_word(tag, v[u].x) && v[u].w == tag_word(tag, v[u].z))
                pend &= ~(1u << u);
        if (!__any(pend != 0u)) return true;
        if (!on_fail()) return false;
    }
}

// Elements of the 16-byte piece at byte offset off of a buffer (plain load;
// the wave-uniform base sits in the buffer resource, so the lane's part of
// the address is one 32-bit register).
template <int DT>
__device__ __forceinline__ void piece_load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[16 / (DT ? 2 : 4)]) {
    const u4v w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    if constexpr (DT == 1) {
        v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
        v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
    } else {
        v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y); v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    }
}

__device__ __forceinline__ int wg_unit0(int w, int U, int G) { return (int)(((int64_t)w * U) / G); }

// Running attention state of NH query heads (flash decode): the lane's
// query dims, running max (wave-uniform), running sums and unnormalised
// outputs of the lane's position group.
template <int NH, int EPLT>
struct AttnSt {
    static constexpr int nh = NH;
    float qr[NH][EPLT];
    float am[NH], al[NH];
    float ao[NH][EPLT];
};
// The same without the queries (read from LDS at each fold instead).
template <int NH, int EPLT>
struct AttnStQ {
    static constexpr int nh = NH;
    float am[NH], al[NH];
    float ao[NH][EPLT];
};

struct Geo {
    int unit0[ST_NUM], units[ST_NUM], nsl[ST_NUM];
    MkDownGeo dn;
};

__device__ __forceinline__ void make_geo(const MkParams &p, int w, int epl, Geo &g) {
#pragma unroll
    for (int k = 0; k < ST_NUM; ++k) {
        const int U = p.st[k].units;
        g.unit0[k] = wg_unit0(w, U, p.grid);
        g.units[k] = wg_unit0(w + 1, U, p.grid) - g.unit0[k];
        g.nsl[k] = (g.units[k] * p.st[k].rbp + 3) / 4;
    }
    g.dn = mk_down_geo(w, p.grid, p.st[ST_DOWN].units, p.F, p.H, epl);
    g.nsl[ST_DOWN] = g.dn.nsl;
}


}  // namespace

// LOGITS = false is the cache-append variant used by prefill: the same step
// without the final norm, LM head and argmax.
// PMAP selects the position-major attention mapping (groups of four query
// heads, long splits; chosen per launch by the host from the split length).
template <int DT, int GQ, int LPP, bool LOGITS, bool PMAP>
__global__ __launch_bounds__(MK_BLOCK_THREADS, 1) void mk_decode_kernel(const MkParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_[];
    LDS unsigned char *smem = (LDS unsigned char *)smem_;
    // DT 0 float32, 1 bfloat16, 2 weight-only INT8: int8 matrices with
    // per-row scales, the cache and the embedding in bfloat16 (CDT 1).
    constexpr int CDT = DT == 2 ? 1 : DT;   // storage of the cache and the embedding
    constexpr int EB = CDT ? 2 : 4;         // bytes per cache / embedding element
    constexpr int EPL = 16 / EB;            // cache elements per 16-byte lane piece
    constexpr int EPLW = wepl(DT);          // weight elements per 16-byte lane piece
    constexpr int EBW = 16 / EPLW;          // bytes per weight element
    constexpr int EPCW = MK_CHUNK_BYTES * EPLW / 16;  // weight elements per 1 KiB chunk
    // the register input paths (rows of exactly four chunks, down row groups of
    // four pieces) are built for float32 and bfloat16 pieces
    constexpr bool REGP = DT != 2;
    constexpr int PPC = 64 / LPP;           // cache positions per 1 KiB chunk
    constexpr int BP = 8 * PPC;             // positions per KV slot (8 K chunks + 8 V chunks)
    constexpr int DH = LPP * 16 / EB;       // head dim

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int w = blockIdx.x, G = p.grid, NS = p.ring_slots, L = p.L;
    constexpr int d = DH;

    // LDS layout: ring | vec | out | xown | rope | ss | control | INT8 scales
    LDS unsigned char *ring = smem;
    LDS float *vec = (LDS float *)(smem + NS * MK_SLOT_BYTES);
    LDS float *outv = vec + p.lds_vec_floats;
    LDS float *xown = outv + p.lds_out_rows;
    LDS float *ropel = xown + 64;  // [64][4] rotary (cos, sin) pairs of the first 64 QKV units
    LDS float *ssp = ropel + 256;
    volatile LDS int *ctl = (volatile LDS int *)(ssp + MK_NUM_CONSUMERS);  // [1] abort step, [8] consumer meetings
    LDS float *sbuf = ssp + MK_NUM_CONSUMERS + 16;  // [2][lds_sc_floats] per-row scales (DT 2), by layer parity

    Geo g;
    make_geo(p, w, EPLW, g);

    // Attention split of this workgroup: KV head kvj, positions [t0, t1).
    const int S = p.splits;
    const bool has_split = w < p.nkv * S;
    const int kvj = has_split ? w / S : 0, kvs = has_split ? w % S : 0;
    const int P = p.pos;
    const int per = (P + S - 1) / S;
    const int t0 = min(P, kvs * per), t1 = min(P, t0 + per);
    const int nt = has_split ? t1 - t0 : 0;
    // Whole KV slots go through the ring; a remainder of at most one chunk
    // (PPC positions, one per lane group) is read straight into registers.
    const int nfull = nt / BP, nrem = nt - nfull * BP;
    const int ntail = nrem <= PPC ? nrem : 0;
    const int nsl_kv = nfull + (nrem > PPC ? 1 : 0);
    const bool is_last = has_split && kvs == S - 1;
    const size_t head_bytes = (size_t)p.max_seq * d * EB;
    // Per-kind slot counts as scalars (kind 0 QKV, 1 KV, 2 O, 3 GU, 4 DOWN, 5 LM);
    // a switch keeps the runtime-selected value in registers.
    const int nsl_q = g.nsl[ST_QKV], nsl_o = g.nsl[ST_O], nsl_gu = g.nsl[ST_GU], nsl_dn = g.nsl[ST_DOWN],
              nsl_lm = g.nsl[ST_LM];
    auto nslots = [&](int kind) -> int {
        switch (kind) {
        case 0: return nsl_q;
        case 1: return nsl_kv;
        case 2: return nsl_o;
        case 3: return nsl_gu;
        case 4: return nsl_dn;
        default: return nsl_lm;
        }
    };

    if (tid == 0) { ctl[0] = -1; ctl[1] = 0; ctl[8] = 0; }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    if (wave < MK_NUM_LOADERS) {
        // ============================ loader ============================
        const int wl = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: keeps buffer resources scalar
        // Each loader carries CPW of a slot's 16 chunks: chunks [wl*CPW, wl*CPW + CPW).
        // In a cache slot chunks 0-7 are K and 8-15 are V, so the first half
        // of the loaders reads K and the second half V.
        constexpr int CPW = MK_CHUNKS_PER_SLOT / MK_NUM_LOADERS;
        constexpr int HALF = MK_NUM_LOADERS / 2;
        constexpr uint32_t WAVE_BYTES = CPW * MK_CHUNK_BYTES;  // this wave's share of a slot
        const unsigned char *kv_src = (const unsigned char *)(wl < HALF ? p.kc : p.vc);
        const int64_t kv_skip = (int64_t)(wl % HALF) * CPW * MK_CHUNK_BYTES;  // bytes before this loader's first K (V) chunk

        // this workgroup's weight blocks for layer 0 (this wave's share), and
        // the per-layer strides
        const unsigned char *wb_q = p.packed + p.st[ST_QKV].base + p.st[ST_QKV].wg_off[w] + wl * WAVE_BYTES;
        const unsigned char *wb_o = p.packed + p.st[ST_O].base + p.st[ST_O].wg_off[w] + wl * WAVE_BYTES;
        const unsigned char *wb_gu = p.packed + p.st[ST_GU].base + p.st[ST_GU].wg_off[w] + wl * WAVE_BYTES;
        const unsigned char *wb_dn = p.packed + p.st[ST_DOWN].base + p.st[ST_DOWN].wg_off[w] + wl * WAVE_BYTES;
        const unsigned char *wb_lm = p.packed + p.st[ST_LM].base + p.st[ST_LM].wg_off[w] + wl * WAVE_BYTES;
        const int64_t ws_q = p.st[ST_QKV].layer_stride, ws_o = p.st[ST_O].layer_stride,
                      ws_gu = p.st[ST_GU].layer_stride, ws_dn = p.st[ST_DOWN].layer_stride;
        const unsigned char *kv_l0 = kv_src + (int64_t)kvj * (int64_t)head_bytes + (int64_t)t0 * d * EB + kv_skip;
        const int64_t kv_lstride = (int64_t)p.nkv * (int64_t)head_bytes;

        // ---- the stream: every slot of every stage, in consumption order ----
        // (it_l, it_k) is the current stage (kind 0 QKV, 1 KV, 2 O, 3 gate/up,
        // 4 down; kind 5 the LM head after the last layer), it_left the slots
        // left in it, it_ptr this wave's source of the current slot.  A slot
        // costs a pointer step; the stage bookkeeping runs once per stage.
        int it_l = 0, it_k = 0, it_left = 0;
        bool done = false, it_kv = false;
        const unsigned char *it_ptr = p.packed;
        int64_t it_step = 0, kv_rem = 0;  // kv_rem: bytes of this wave's chunks left in the split
        auto last_kind = [&]() { return it_k == 5 || (!LOGITS && it_l == L - 1 && it_k == 4); };
        // past the end of the stream: harmless re-reads of the packed buffer's
        // opening slot (zeros, owned by no stage)
        auto finish = [&]() {
            done = true;
            it_kv = false;
            it_ptr = p.packed;
            it_step = 0;
        };
        // Position on stage (it_l, it_k) or the first non-empty stage after it
        // (bounded: every stage is visited at most once).
        auto stage_setup = [&]() {
            for (int guard = 0; guard <= 5 * L + 1; ++guard) {
                const int n = nslots(it_k);
                if (n > 0) {
                    it_left = n;
                    it_kv = it_k == 1;
                    if (it_kv) {
                        it_ptr = kv_l0 + (int64_t)it_l * kv_lstride;
                        it_step = (int64_t)BP * d * EB;
                        kv_rem = (int64_t)(t1 - t0) * d * EB - kv_skip;
                    } else {
                        switch (it_k) {
                        case 0: it_ptr = wb_q + (int64_t)it_l * ws_q; break;
                        case 2: it_ptr = wb_o + (int64_t)it_l * ws_o; break;
                        case 3: it_ptr = wb_gu + (int64_t)it_l * ws_gu; break;
                        case 4: it_ptr = wb_dn + (int64_t)it_l * ws_dn; break;
                        default: it_ptr = wb_lm; break;
                        }
                        it_step = p.st[it_k == 5 ? ST_LM : it_k == 0 ? ST_QKV : it_k == 2 ? ST_O : it_k == 3 ? ST_GU : ST_DOWN]
                                      .slot_stride;
                    }
                    return;
                }
                if (last_kind()) break;
                if (++it_k == 5 && ++it_l < L) it_k = 0;  // after the last layer: the LM head
            }
            finish();
        };
        auto advance = [&]() {
            if (done) return;
            if (--it_left > 0) {
                it_ptr += it_step;
                kv_rem -= it_step;
                return;
            }
            if (last_kind()) {
                finish();
                return;
            }
            if (++it_k == 5 && ++it_l < L) it_k = 0;
            stage_setup();
        };
        stage_setup();
        // This lane's 16 bytes of chunk c of the current slot.  Cache rows
        // past the split read the packed buffer's zeroed opening slot instead
        // (the consumers mask those positions; the values they multiply by 0
        // are zeros).  Global loads: direct-to-LDS buffer loads measured
        // slower for this stream.
        auto piece_src = [&](int c) -> const GLB u4v * {
            const int64_t o = (int64_t)c * MK_CHUNK_BYTES + lane * 16;
            return (const GLB u4v *)(!it_kv || o < kv_rem ? it_ptr + o : p.packed + lane * 16);
        };
        // direct-to-LDS loads of the current slot into ring slot buf
        auto issue = [&](int buf) {
            LDS unsigned char *dst = ring + buf * MK_SLOT_BYTES + wl * WAVE_BYTES;
            if (it_kv) {
#pragma unroll
                for (int c = 0; c < CPW; ++c)
                    __builtin_amdgcn_global_load_lds((const void *)piece_src(c), (LDS void *)(dst + c * MK_CHUNK_BYTES), 16, 0, 0);
            } else {
#pragma unroll
                for (int c = 0; c < CPW; ++c)
                    __builtin_amdgcn_global_load_lds((const void *)piece_src(c), (LDS void *)(dst + c * MK_CHUNK_BYTES), 16, 0,
                                                     2 /* nt: streamed once */);
            }
            advance();
        };

        int lstep = 0;  // barriers passed; mirrors the consumers' step counter
        // optional timeline: loader 0's arrival at and exit from the barriers
        // of layer 1 (and the start of layer 2), barrier indices [b0, b0 + 96)
        const int sps = p.slots_per_step;
        auto nsteps = [&](int n) { return (n + sps - 1) / sps; };  // data steps of a stage of n slots
        const int lb0 = 5 + nsteps(nsl_q) + nsteps(nsl_kv) + nsteps(nsl_o) + nsteps(nsl_gu) + nsteps(nsl_dn);
        auto lstamp = [&](int e) {
            if (p.trace && wl == 0 && lane == 0 && lstep >= lb0 && lstep < lb0 + 96)
                p.trace[(size_t)G * (5 * L + 2) * 4 + (size_t)G * 64 * 2 + ((size_t)w * 96 + lstep - lb0) * 2 + e] =
                    wall_clock64();
        };
        const int total = L * (nsl_q + nsl_kv + nsl_o + nsl_gu + nsl_dn) + (LOGITS ? nsl_lm : 0);
        // Slot m goes straight into ring slot m % NS.  The loads run up to
        // `depth` slots ahead of the slot being consumed (at most NS -
        // slots_per_step: the ring slot must have been consumed) and, unless
        // stage_drain is set, across stage boundaries; with stage_drain a
        // stage's first loads wait for its opening barrier.  `issued` counts
        // the slots issued so far, so the wait before a data step is exact:
        // slot k's loads are done when at most (issued - 1 - k) * CPW newer
        // loads are outstanding.
        const int depth = p.prefetch_depth;
        int issued = 0, cons = 0;                  // slots issued; slots handed to the consumers
        int cap = p.stage_drain ? -1 : total - 1;  // last slot that may be issued now
        int jl = 0;                                // ring slot of the next issue
        auto issue_more = [&]() {
            int lim = cons - 1 + depth;
            if (lim > cap) lim = cap;
            while (issued <= lim) {
                issue(jl);
                jl = jl + 1 == NS ? 0 : jl + 1;
                ++issued;
            }
        };

        // ctl[1] holds the step in which a consumer aborted (0: none).  The
        // consumers pass exactly one more barrier after aborting and leave; a
        // barrier then waits for the remaining waves only.  So the loaders
        // read the word only at stage openings: the data-step path stays
        // short, and after an abort the rest of the current stage is merely
        // loaded in vain before they leave too.
        auto bar = [&]() {
            lstamp(0);
            MK_COMPILER_BARRIER();
            __builtin_amdgcn_s_barrier();
            MK_COMPILER_BARRIER();
            lstamp(1);
            ++lstep;
        };
        auto bar_check = [&]() -> bool {  // false: the consumers aborted in an earlier step
            bar();
            const int a = ctl[1];
            return a == 0 || a >= lstep;
        };
        // The consumers' barrier sequence: each stage (layer sl, kind sk)
        // opens with one barrier, then has one per data slot; one more closes
        // the step.  wleft counts the data barriers left in the current stage.
        int sl = 0, sk = -1, wleft = 0;
        bool dead = false;
        auto walk_next = [&]() -> bool {  // to the next stage; false after the last one
            if (sk < 0) {
                sk = 0;
                return true;
            }
            if (sk == 5 || (!LOGITS && sl == L - 1 && sk == 4)) return false;
            if (++sk == 5 && ++sl < L) sk = 0;
            return true;
        };
        // Opening barriers up to the next stage that has data steps.
        auto open_next = [&]() {
            for (int guard = 0; guard <= 5 * L + 1; ++guard) {
                if (!walk_next()) return;
                if (!bar_check()) {
                    dead = true;
                    return;
                }
                wleft = nslots(sk);
                if (wleft > 0) {
                    if (p.stage_drain) {  // this stage's loads may start now
                        cap = cons + wleft - 1;
                        issue_more();
                    }
                    return;
                }
            }
        };
        // The stages after the last data step (none has data steps) and the
        // closing barrier.
        auto close_walk = [&]() {
            if (dead) return;
            for (int guard = 0; guard <= 5 * L + 1; ++guard) {
                if (!walk_next()) break;
                if (!bar_check()) return;
            }
            bar();
        };

        // A data step takes TS slots of the current stage (fewer at its end):
        // the loads of all of them are complete before the step's barrier
        // (the host keeps depth >= TS, so they have been issued), and with
        // cons counting the slots handed to the consumers, the issue limit
        // cons - 1 + depth stays below the ring slots still in use (depth
        // <= ring - TS).
        const int TS = p.slots_per_step;
        issue_more();
        for (int k = 0; k < total;) {
            if (wleft == 0) open_next();
            if (dead) break;
            const int take = wleft < TS ? wleft : TS;
            wait_vm_rt((issued - k - take) * CPW);  // slots k .. k + take - 1 have landed
            bar();
            cons += take;
            wleft -= take;
            k += take;
            issue_more();
        }
        close_walk();
        wait_vm<0>();
        return;
    }

    // ============================== consumers ==============================
    // Each stage is a block: its per-lane register state (the input slice of
    // a GEMV, the attention accumulators) is declared inside the block, so
    // its registers are free again for the next stage.
    // consumer waves issue ahead of the loader wave sharing their SIMD
    __builtin_amdgcn_s_setprio(2);
    const int c = wave - MK_NUM_LOADERS;        // consumer index 0..3
    const int ct = tid - MK_NUM_LOADERS * 64;   // consumer thread 0..255
    int js = 0;     // ring slot of the next data step
    int step = 0;   // barriers passed (also the consumer-local go-flag value)
    bool ok = true;

    auto barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        ++step;
    };
    // The barrier of a data step: before slot n (stage-local) of every stage
    // when n is a multiple of slots_per_step -- the loaders' schedule.
    const bool ts2 = p.slots_per_step == 2;
    auto data_barrier = [&](int n) {
        if (!ts2 || (n & 1) == 0) barrier();
    };

    // ---- tagged records ----------------------------------------------------
    // A producer stores {value, tag} as one 64-bit device-scope store; a
    // reader polls the records it needs until every tag is the expected one.
    // No flag, no store-completion wait, no second load: the data carry
    // their own validity.  The tag names the launch and the layer: a record
    // of layer index l (the index of its array: x entering layer l, layer
    // l's queries, partials, ...; L for the argmax records) carries
    // p.tag + l, and the host advances p.tag by L + 1 per launch.  Each
    // per-layer array has two buffers, for even and odd l: a producer of
    // layer l + 2 can only run once every workgroup has finished reading
    // layer l's records (each dependency chain between them passes through
    // an all-to-all gather of layer l + 1), and the slot it overwrites holds
    // an older tag, never the awaited one.
    auto tag_of = [&](int l) -> uint32_t { return p.tag + (uint32_t)l; };
    auto stll = [&](uint64_t *dst, float v, uint32_t tg) {
        const uint32_t bits = __float_as_uint(v);
        __hip_atomic_store(dst, ((uint64_t)tag_word(tg, bits) << 32) | bits, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    };
    int64_t poll_start = 0;
    // After a failed poll round: false once this workgroup aborted, the wait
    // timed out or the device error word is set (then the abort is marked).
    // The error word is read only once a wait has lasted err_check_ticks:
    // reading it after every failed round would add a second memory round
    // trip to each poll period, and a healthy wait ends well before that.
    auto poll_ok = [&]() -> bool {
        if (ctl[1] != 0) return false;
        const int64_t waited = wall_clock64() - poll_start;
        const bool timed_out = waited > p.timeout_ticks;
        if (timed_out || (waited > p.err_check_ticks && ldcu(p.err) != 0u)) {
            if (lane == 0) {
                if (timed_out) __hip_atomic_fetch_or(p.err, MK_DEVERR_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ctl[1] = step;
            }
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
        return true;
    };
    // The consumers meet here after each gather.  An LDS counter, not
    // s_barrier: the loaders take no part, so a loader stalled on issuing
    // loads delays nobody.
    int nsync = 0;
    auto csync = [&]() -> bool {
        ++nsync;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        if (lane == 0) __hip_atomic_fetch_add((LDS int *)&ctl[8], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        while (ctl[8] < MK_NUM_CONSUMERS * nsync) {
            if (ctl[1] != 0) return false;
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        return ctl[1] == 0;
    };
    // ---- per-row scales of the INT8 matrices (DT 2) ----
    // Block bl (a layer's QKV, O, gate/up and down rows of this workgroup;
    // bl == L: its LM-head rows) is read into registers -- consumer c lane i
    // holds entries j*256 + c*64 + i -- while the gate/up weights of layer
    // bl-1 stream, and stored to LDS copy bl & 1 when the down stage of that
    // layer opens.  So the loads never stand in a dependency wait, and a
    // copy is rewritten only after the last reader of the block two layers
    // back (the down reduction) has passed a consumer meeting.  Block 0 is
    // read and stored when the step starts.
    float sreg[4];
    auto sc_fetch = [&](int bl) {
        if constexpr (DT == 2) {
            const bool head = bl == L;
            const float *src = head ? p.scl + (size_t)L * G * p.sc_blk + (size_t)w * p.sc_lm
                                    : p.scl + ((size_t)bl * G + w) * p.sc_blk;
            // entries past the block read as 0 (buffer range check)
            const __amdgpu_buffer_rsrc_t rs = rsrc(src, (uint32_t)(head ? p.sc_lm : p.sc_blk) * 4u);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sreg[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(j * 256 + ct) * 4u, 0, 0));
        }
    };
    auto sc_park = [&](int bl) {
        if constexpr (DT == 2) {
            LDS float *dst = sbuf + (bl & 1) * p.lds_sc_floats;
            const int n = bl == L ? p.sc_lm : p.sc_blk;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j * 256 + ct < n) dst[j * 256 + ct] = sreg[j];
        }
    };
    // the LDS copy of block bl
    auto scl_of = [&](int bl) -> const LDS float * { return sbuf + (bl & 1) * p.lds_sc_floats; };
    // row i's scale in the copy sc (1 when the weights are not INT8)
    auto rsc = [&](const LDS float *sc, int i) -> float {
        if constexpr (DT == 2) return sc[i];
        else return 1.0f;
    };

    // Gather n (even) tagged elements into vec (times gain, if given),
    // zero-padded to pad.  The four consumers take interleaved 16-byte pieces
    // (two records), so the workgroup reads each element once; ssp[c] gets
    // this consumer's share of the sum of squares, summed in a fixed order.
    auto gather_fn = [&](LDS float *dst, int npc, __amdgpu_buffer_rsrc_t rs, auto &&off, const float *gain,
                         int n, int pad, uint32_t tg) -> bool {
        float ss = 0.f;
        poll_start = wall_clock64();
        bool good = true;
        for (int base = ct; base < npc; base += 256 * 8) {
            uint32_t mask = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (base + u * 256 < npc) mask |= 1u << u;
            // the gain slice does not depend on the records: load it first so
            // its latency hides behind the first poll round
            f2v gg[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                gg[u] = (gain && (mask & (1u << u))) ? *(const f2v *)(gain + 2 * (base + u * 256)) : f2v{1.f, 1.f};
            u4v v[8];
            if (!poll16<8>(rs, [&](int u) { return off(base + u * 256); }, mask, v, tg, poll_ok)) {
                good = false;
                break;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (mask & (1u << u)) {
                    const int e = 2 * (base + u * 256);
                    const float x0 = __uint_as_float(v[u].x), x1 = __uint_as_float(v[u].z);
                    ss = fmaf(x0, x0, ss);
                    ss = fmaf(x1, x1, ss);
                    *(LDS f2v *)(dst + e) = gg[u] * f2v{x0, x1};
                }
            }
        }
        for (int i = n + ct; i < pad; i += 256) dst[i] = 0.f;
        ss = wave_sum(ss);
        if (lane == 0) ssp[c] = ss;
        if (!good) return false;
        return csync();
    };
    auto gather_to = [&](LDS float *dst, const uint64_t *src, int n, const float *gain, int pad, uint32_t tg) -> bool {
        return gather_fn(dst, n >> 1, rsrc(src, (uint32_t)n * 8u), [](int pc) { return (uint32_t)pc * 16u; }, gain, n,
                         pad, tg);
    };
    auto gather = [&](const uint64_t *src, int n, const float *gain, int pad, uint32_t tg) -> bool {
        return gather_to(vec, src, n, gain, pad, tg);
    };

    // ---- optional stage timeline (consumer 0, lane 0) ----
    const int nbound = 5 * L + 2;
    auto stamp = [&](int b, int e) {
        if (p.trace && c == 0 && lane == 0) p.trace[((size_t)w * nbound + b) * 4 + e] = wall_clock64();
    };
    // Data steps of layer 1 (steady state): barrier passed / compute done.
    int dstep_l1 = 0;
    auto stamp_step = [&](int l, int e) {
        if (p.trace && l == 1 && c == 0 && lane == 0 && dstep_l1 < 64)
            p.trace[(size_t)G * nbound * 4 + ((size_t)w * 64 + dstep_l1) * 2 + e] = wall_clock64();
        if (e == 1 && l == 1) ++dstep_l1;
    };

    // ---- input vectors ----
    // LDS path: vec[0..n) = gain (.) x, zero padded to `pad`, with per-consumer
    // sums of squares of x in ssp[c].  x is read with 16-byte device-scope
    // loads (or, for layer 0, from the embedding row), eight per lane before
    // any is used, so a call costs ceil(n/8192) memory round trips.
    auto load_normed = [&](const float *xsrc, const void *erow, const float *gain, int n, int pad) {
        const int nqd = n / 4;
        const __amdgpu_buffer_rsrc_t rx = rsrc(xsrc ? (const void *)xsrc : erow, (uint32_t)n * (xsrc ? 4u : (uint32_t)EB));
        float ss = 0.f;
        for (int base = ct; base < nqd; base += 256 * 8) {
            f4v xv[8], gv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int qi = base + u * 256;
                if (xsrc) {
                    xv[u] = as_f4(ld16c(rx, (uint32_t)qi * 16u));
                } else if constexpr (CDT == 1) {
                    const uint64_t e = qi < nqd ? ((const uint64_t *)erow)[qi] : 0ull;
                    xv[u] = f4v{bf_lo((uint32_t)e), bf_hi((uint32_t)e), bf_lo((uint32_t)(e >> 32)), bf_hi((uint32_t)(e >> 32))};
                } else {
                    xv[u] = qi < nqd ? ((const f4v *)erow)[qi] : f4v{0.f, 0.f, 0.f, 0.f};
                }
                gv[u] = qi < nqd ? ((const f4v *)gain)[qi] : f4v{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int qi = base + u * 256;
                if (qi < nqd) {
                    const f4v x = xv[u];
                    ss = fmaf(x.x, x.x, ss);
                    ss = fmaf(x.y, x.y, ss);
                    ss = fmaf(x.z, x.z, ss);
                    ss = fmaf(x.w, x.w, ss);
                    *(LDS f4v *)(vec + 4 * qi) = gv[u] * x;
                }
            }
        }
        for (int i = n + ct; i < pad; i += 256) vec[i] = 0.f;
        ss = wave_sum(ss);
        if (lane == 0) ssp[c] = ss;
    };
    auto inv_lds = [&](int n) {
        const float ss = ssp[0] + ssp[1] + ssp[2] + ssp[3];
        return 1.0f / sqrtf(ss / (float)n + p.eps);
    };
    // Register path (rows of exactly four chunks): every consumer loads the
    // lane's slice of the input vector -- element q*EPCW + lane*EPLW + e feeds
    // chunk q -- straight into registers with the gain applied, and returns
    // the full sum of squares of x (it sees all 4*EPCW elements).  Float32 and
    // bfloat16 weights (REGP) only.
    auto load_direct = [&](const float *xsrc, const void *erow, const float *gain, float (&hr)[4][EPLW]) -> float {
        f4v xv[4][EPLW / 4], gv[4][EPLW / 4];
        const __amdgpu_buffer_rsrc_t rx = rsrc(xsrc ? (const void *)xsrc : erow, 4u * EPCW * (xsrc ? 4u : (uint32_t)EB));
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int k4 = 0; k4 < EPLW / 4; ++k4) {
                const int el = q * EPCW + lane * EPLW + 4 * k4;  // first of 4 elements
                if (xsrc) {
                    xv[q][k4] = as_f4(ld16c(rx, (uint32_t)el * 4u));
                } else if constexpr (DT == 1) {
                    // one 16-byte load per chunk holds all 8 bf16 elements of the lane
                    if (k4 == 0) {
                        const u4v e = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)el * 2u, 0, 0);
                        xv[q][0] = f4v{bf_lo(e.x), bf_hi(e.x), bf_lo(e.y), bf_hi(e.y)};
                        xv[q][1] = f4v{bf_lo(e.z), bf_hi(e.z), bf_lo(e.w), bf_hi(e.w)};
                    }
                } else {
                    xv[q][k4] = as_f4(__builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)el * 4u, 0, 0));
                }
                gv[q][k4] = gain ? *(const f4v *)(gain + el) : f4v{1.f, 1.f, 1.f, 1.f};
            }
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int k4 = 0; k4 < EPLW / 4; ++k4) {
                const f4v x = xv[q][k4];
                ss = fmaf(x.x, x.x, ss);
                ss = fmaf(x.y, x.y, ss);
                ss = fmaf(x.z, x.z, ss);
                ss = fmaf(x.w, x.w, ss);
                const f4v hv = gv[q][k4] * x;
                hr[q][4 * k4 + 0] = hv.x;
                hr[q][4 * k4 + 1] = hv.y;
                hr[q][4 * k4 + 2] = hv.z;
                hr[q][4 * k4 + 3] = hv.w;
            }
        return wave_sum(ss);
    };
    auto inv_of = [&](float ss, int n) { return 1.0f / sqrtf(ss / (float)n + p.eps); };

    // ---- GEMV data steps ----
    // Register path: slot n holds row n of this consumer (4 chunks); the four
    // 16-byte ring reads are issued before any arithmetic.
    auto gemv_reg_steps = [&](int st, int l, const float (&hr)[4][EPLW]) {
        const int units = g.units[st];
        for (int n = 0; n < g.nsl[st]; ++n) {
            data_barrier(n);
            stamp_step(l, 0);
            if (n < units) {
                const LDS unsigned char *bp = ring + js * MK_SLOT_BYTES + c * 4 * MK_CHUNK_BYTES + lane * 16;
                float d[4];
                if constexpr (DT == 1) {
                    u4v wv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) wv[q] = *(const LDS u4v *)(bp + q * MK_CHUNK_BYTES);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float a = bf_lo(wv[q].x) * hr[q][0];
                        float b = bf_hi(wv[q].x) * hr[q][1];
                        a = fmaf(bf_lo(wv[q].y), hr[q][2], a);
                        b = fmaf(bf_hi(wv[q].y), hr[q][3], b);
                        a = fmaf(bf_lo(wv[q].z), hr[q][4], a);
                        b = fmaf(bf_hi(wv[q].z), hr[q][5], b);
                        a = fmaf(bf_lo(wv[q].w), hr[q][6], a);
                        b = fmaf(bf_hi(wv[q].w), hr[q][7], b);
                        d[q] = a + b;
                    }
                } else {
                    f4v wv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) wv[q] = *(const LDS f4v *)(bp + q * MK_CHUNK_BYTES);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        d[q] = fmaf(wv[q].x, hr[q][0], wv[q].y * hr[q][1]) + fmaf(wv[q].z, hr[q][2], wv[q].w * hr[q][3]);
                }
                const float t = wave_sum((d[0] + d[1]) + (d[2] + d[3]));
                if (lane == 0) outv[n * 4 + c] = t;
            }
            js = js + 1 == NS ? 0 : js + 1;
            stamp_step(l, 1);
        }
    };
    // LDS path: any row length; the input vector is in vec.  Whole groups of
    // four rows come first (mk_stream_pos): slot s of a group carries chunk s
    // of four rows, so the lane's eight input elements are read from LDS once
    // and multiply four weight pieces, with one accumulator per row.  The
    // remaining rows follow row after row.
    auto gemv_lds_steps = [&](int st, int l) __attribute__((always_inline)) {
        const int units = g.units[st], rbp = p.st[st].rbp;
        const int full = mk_row_groups(rbp, EBW) ? units / 4 : 0;
        int n = 0;
        for (int grp = 0; grp < full; ++grp) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < rbp; ++s, ++n) {
                data_barrier(n);
                stamp_step(l, 0);
                const LDS unsigned char *bp = ring + js * MK_SLOT_BYTES + c * 4 * MK_CHUNK_BYTES + lane * 16;
                float hv[EPLW];
                piece_in<DT>(vec + s * EPCW + lane * EPLW, hv);
                float d[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] = piece_dot_reg<DT>(bp + j * MK_CHUNK_BYTES, hv);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] += d[j];
                js = js + 1 == NS ? 0 : js + 1;
                stamp_step(l, 1);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float t = wave_sum(acc[j]);
                if (lane == 0) outv[(grp * 4 + j) * 4 + c] = t;
            }
        }
        int row_c = full * 4, kc = 0;
        float acc = 0.f;
        for (; n < g.nsl[st]; ++n) {
            data_barrier(n);
            stamp_step(l, 0);
            const LDS unsigned char *bp = ring + js * MK_SLOT_BYTES + c * 4 * MK_CHUNK_BYTES + lane * 16;
            if ((rbp & 3) == 0) {  // the piece lies inside one row
                if (row_c < units) {
                    const LDS float *hp = vec + kc * EPCW + lane * EPLW;
                    const float d0 = piece_dot<DT>(bp, hp);
                    const float d1 = piece_dot<DT>(bp + MK_CHUNK_BYTES, hp + EPCW);
                    const float d2 = piece_dot<DT>(bp + 2 * MK_CHUNK_BYTES, hp + 2 * EPCW);
                    const float d3 = piece_dot<DT>(bp + 3 * MK_CHUNK_BYTES, hp + 3 * EPCW);
                    acc += (d0 + d1) + (d2 + d3);
                    kc += 4;
                    if (kc == rbp) {
                        const float t = wave_sum(acc);
                        if (lane == 0) outv[row_c * 4 + c] = t;
                        acc = 0.f;
                        kc = 0;
                        ++row_c;
                    }
                }
            } else {
#pragma unroll
                for (int qi = 0; qi < 4; ++qi) {
                    if (row_c < units) {
                        acc += piece_dot<DT>(bp + qi * MK_CHUNK_BYTES, vec + kc * EPCW + lane * EPLW);
                        if (++kc == rbp) {
                            const float t = wave_sum(acc);
                            if (lane == 0) outv[row_c * 4 + c] = t;
                            acc = 0.f;
                            kc = 0;
                            ++row_c;
                        }
                    }
                }
            }
            js = js + 1 == NS ? 0 : js + 1;
            stamp_step(l, 1);
        }
    };

    // ---- down projection, split along its input ----
    // Lane i of consumer c accumulates output row (c + 4*gl)*64 + i over the
    // kp piece columns of its row group gl; the finished partial sum is
    // stored as a tagged record of this workgroup's partial vector.
    auto down_steps = [&](int l) {
        uint64_t *dst = p.ll_dpart + ((size_t)(l & 1) * G + w) * p.H;
        const uint32_t tg = tag_of(l);
        const int kp = g.dn.kp, ng = (p.H + 63) >> 6;
        if (kp == 0) {  // no SwiGLU outputs here: the partial is zero
            // buffer stores (scalar base, 32-bit lane offset): the same
            // device-scope 64-bit stores as stll, one register cheaper
            const __amdgpu_buffer_rsrc_t rd = rsrc(dst, (uint32_t)p.H * 8u);
            const uint64_t zero_rec = (uint64_t)tag_word(tg, 0u) << 32;
            const u4v z = u4v{0u, (uint32_t)(zero_rec >> 32), 0u, (uint32_t)(zero_rec >> 32)};
            for (int r = 2 * ct; r < p.H; r += 512)  // H is even: two records per 16-byte store
                __builtin_amdgcn_raw_buffer_store_b128(z, rd, (uint32_t)r * 8u, 0, MK_SC1);
            return;
        }
        if ((kp & 3) == 0) {
            // Every step covers four pieces of one row group: straight-line
            // code with four independent dot products; with kp == 4 the
            // workgroup's SwiGLU outputs stay in registers.
            float ar[4][EPLW];
            if (REGP && kp == 4) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                    for (int e = 0; e < EPLW; ++e) ar[qq][e] = vec[qq * EPLW + e];
            }
            int gl = 0, q = 0;
            float acc = 0.f;
            for (int n = 0; n < g.nsl[ST_DOWN]; ++n) {
                data_barrier(n);
                stamp_step(l, 0);
                const int grp = c + 4 * gl;
                if (grp < ng) {  // wave-uniform
                    const LDS unsigned char *bp = ring + js * MK_SLOT_BYTES + c * 4 * MK_CHUNK_BYTES + lane * 16;
                    float dq[4];
                    if (REGP && kp == 4) {
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) dq[qq] = piece_dot_reg<DT>(bp + qq * MK_CHUNK_BYTES, ar[qq]);
                    } else {
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) dq[qq] = piece_dot<DT>(bp + qq * MK_CHUNK_BYTES, vec + (q + qq) * EPLW);
                    }
                    acc += (dq[0] + dq[1]) + (dq[2] + dq[3]);
                    q += 4;
                    if (q == kp) {
                        const int row = grp * 64 + lane;
                        if (row < p.H) stll(dst + row, acc, tg);
                        acc = 0.f;
                        q = 0;
                        ++gl;
                    }
                }
                js = js + 1 == NS ? 0 : js + 1;
                stamp_step(l, 1);
            }
            return;
        }
        int gl = 0, q = 0;
        float acc = 0.f;
        for (int n = 0; n < g.nsl[ST_DOWN]; ++n) {
            data_barrier(n);
            stamp_step(l, 0);
            const LDS unsigned char *bp = ring + js * MK_SLOT_BYTES + c * 4 * MK_CHUNK_BYTES + lane * 16;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int grp = c + 4 * gl;
                if (grp < ng) {  // wave-uniform
                    acc += piece_dot<DT>(bp + qq * MK_CHUNK_BYTES, vec + q * EPLW);
                    if (++q == kp) {
                        const int row = grp * 64 + lane;
                        if (row < p.H) stll(dst + row, acc, tg);
                        acc = 0.f;
                        q = 0;
                        ++gl;
                    }
                }
            }
            js = js + 1 == NS ? 0 : js + 1;
            stamp_step(l, 1);
        }
    };
    // x rows of this workgroup (its O-stage rows r0 .. r0+nr-1) = residual +
    // the sum of the G partial down projections, summed in a fixed order;
    // stored as tagged records for the next stage's gather.  Ends with the
    // consumers' meeting so that vec may be overwritten afterwards.
    auto down_reduce = [&](int l, uint64_t *xdst) -> bool {
        const int r0 = g.unit0[ST_O] * 4;
        const int nr = max(0, min(g.units[ST_O] * 4, p.H - r0));
        const int hp = nr >> 1;  // 16-byte pieces per producer
        const int H = p.H;
        const __amdgpu_buffer_rsrc_t rs = rsrc(p.ll_dpart + (size_t)(l & 1) * G * H, (uint32_t)((size_t)G * H * 8u));
        // vec[wq * nr + i] = partial of producer wq for row r0 + i
        auto off = [&](int pc) {
            const int wq = pc / hp, i = pc - wq * hp;
            return (uint32_t)(((size_t)wq * H + r0 + 2 * i) * 8u);
        };
        if (!gather_fn(vec, G * hp, rs, off, nullptr, G * nr, G * nr, tag_of(l))) return false;
        // INT8: the down rows' scales follow the QKV, O and gate/up rows in the block
        const LDS float *scd = scl_of(l) + 4 * (g.units[ST_QKV] + g.units[ST_O] + g.units[ST_GU]);
        for (int i = c; i < nr; i += MK_NUM_CONSUMERS) {
            float sum = 0.f;
            for (int wq = lane; wq < G; wq += 64) sum += vec[wq * nr + i];
            sum = wave_sum(sum);
            if (lane == 0) {
                const float xn = xown[i] + sum * rsc(scd, i);
                xown[i] = xn;
                stll(xdst + r0 + i, xn, tag_of(l + 1));
            }
        }
        return csync();
    };

    // ---- attention (split-K flash decode over this workgroup's positions) ----
    // Head-major mapping: the group's GQ query heads are dealt to the four
    // consumers, HG of them distinct at a time.  Consumer c holds heads
    // c % HG + HG*k (k < HPC) and, when several consumers share a head
    // (GQ < 4), the chunk subset cs = c / HG of every KV slot.  With GQ >= 4
    // a consumer owns its heads over all positions and writes the split's
    // partial records itself; consumers sharing a head write one record each
    // (an extra "effective split" that the combine merges like any other).
    constexpr int HG = GQ < MK_NUM_CONSUMERS ? GQ : MK_NUM_CONSUMERS;
    constexpr int HPC = GQ / HG;                // heads per consumer
    constexpr int CPH = MK_NUM_CONSUMERS / HG;  // consumers per head
    constexpr int CPS = 8 / CPH;                // K (and V) chunks per slot per consumer
    // Chunks folded per softmax update: all eight of a slot when a consumer
    // holds one head of 64 dims; four otherwise (with 128-dim heads the
    // eight-chunk fold needs more than the 256 VGPRs a wave has at two waves
    // per SIMD, and the compiler spills to scratch).
    constexpr int NQB = (HPC == 1 && CPS >= 8 && LPP == 8) ? 8 : (CPS < 4 ? CPS : 4);
    const int hc = c % HG, cs = c / HG;
    const float scale = 1.0f / sqrtf((float)d);
    const int e0 = (lane % LPP) * EPL;
    using AttnState = AttnSt<HPC, EPL>;  // head-major: this consumer's HPC heads
    // Fold NQ chunks of positions (each lane holds one position of each
    // chunk, PPC positions per chunk) into the running state: all scores
    // first, then one running-max update, rescale and V accumulation per
    // head.  Invalid positions get probability 0.  Their V values are zeros
    // (the loaders read the packed buffer's zeroed opening slot, not the
    // cache, past a split's positions) or a valid row (the register tail), so
    // 0 * v adds nothing.
    // kget(q, e) / vget(q, e): element e of the lane's K / V piece of chunk q.
    // qget(h, e): element e of the lane's dims of head h's query.
    // The update from raw scores sc[q][h] (the lane's share of the dot
    // product, before the sum over the lane group).
    auto attn_update = [&](auto &A, auto nq_tag, auto &sc, auto &&vget, const bool *valid) {
        constexpr int NQ = decltype(nq_tag)::value;
        constexpr int NHS = std::remove_reference_t<decltype(A)>::nh;  // heads held by the state
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int h = 0; h < NHS; ++h) {
                const float gsum = group_sum<LPP>(sc[q][h]) * scale;  // all lanes take part
                sc[q][h] = valid[q] ? gsum : -INFINITY;
            }
#pragma unroll
        for (int h = 0; h < NHS; ++h) {
            float mx = sc[0][h];
#pragma unroll
            for (int q = 1; q < NQ; ++q) mx = fmaxf(mx, sc[q][h]);
            const float mn = fmaxf(A.am[h], xgroup_max<LPP>(mx));
            const bool any = mn != -INFINITY;
            const float alpha = any ? __expf(A.am[h] - mn) : 1.f;
            float pe[NQ];
            float lsum = A.al[h] * alpha;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                pe[q] = valid[q] ? __expf(sc[q][h] - mn) : 0.f;
                lsum += pe[q];
            }
            A.al[h] = lsum;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float o = A.ao[h][e] * alpha;
#pragma unroll
                for (int q = 0; q < NQ; ++q) o = fmaf(pe[q], vget(q, e), o);
                A.ao[h][e] = o;
            }
            A.am[h] = any ? mn : A.am[h];
        }
    };
    auto attn_fold_q = [&](auto &A, auto nq_tag, auto &&qget, auto &&kget, auto &&vget, const bool *valid) {
        constexpr int NQ = decltype(nq_tag)::value;
        constexpr int NHS = std::remove_reference_t<decltype(A)>::nh;
        float sc[NQ][NHS];
#pragma unroll
        for (int h = 0; h < NHS; ++h) {
            float qv[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) qv[e] = qget(h, e);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                float t = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) t = fmaf(qv[e], kget(q, e), t);
                sc[q][h] = t;
            }
        }
        attn_update(A, nq_tag, sc, vget, valid);
    };
    // Head-major state, bf16 cache, one head per consumer (QPAIR; with two
    // heads per consumer the 128-dim instantiation would spill): the query
    // is held as bf16 hi + lo pairs (A.qr[h][j] carries the bits of the hi
    // pair of dims 2j, 2j+1 and A.qr[h][4 + j] the lo pair; hi + lo keeps
    // about 16 bits of each element), and the scores of whole cache pieces
    // take two v_dot2c_f32_bf16 per pair of dims against the raw K words.
    constexpr bool QPAIR = CDT == 1 && HPC == 1;
    auto qpair_set = [&](float (&qr)[EPL], const float *qv) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) {
            const bf2 h2 = {(__bf16)qv[2 * j], (__bf16)qv[2 * j + 1]};
            const uint32_t hw = __builtin_bit_cast(uint32_t, h2);
            const bf2 l2 = {(__bf16)(qv[2 * j] - bf_lo(hw)), (__bf16)(qv[2 * j + 1] - bf_hi(hw))};
            qr[j] = __uint_as_float(hw);
            qr[EPL / 2 + j] = __uint_as_float(__builtin_bit_cast(uint32_t, l2));
        }
    };
    auto qpair_elem = [&](const float (&qr)[EPL], int e) -> float {
        const uint32_t hw = __float_as_uint(qr[e >> 1]), lw = __float_as_uint(qr[EPL / 2 + (e >> 1)]);
        return (e & 1) ? bf_hi(hw) + bf_hi(lw) : bf_lo(hw) + bf_lo(lw);
    };
    auto attn_fold_w = [&](auto &A, auto nq_tag, const u4v *kr, auto &&vget, const bool *valid) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        constexpr int NQ = decltype(nq_tag)::value;
        constexpr int NHS = std::remove_reference_t<decltype(A)>::nh;
        float sc[NQ][NHS];
#pragma unroll
        for (int h = 0; h < NHS; ++h)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint32_t kw[4] = {kr[q].x, kr[q].y, kr[q].z, kr[q].w};
                float t = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf2 k2 = __builtin_bit_cast(bf2, kw[j]);
                    t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, __float_as_uint(A.qr[h][j])), k2, t, false);
                    t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, __float_as_uint(A.qr[h][4 + j])), k2, t,
                                                        false);
                }
                sc[q][h] = t;
            }
        attn_update(A, nq_tag, sc, vget, valid);
    };
    // The head-major state holds its queries in registers.
    auto attn_fold = [&](auto &A, auto nq_tag, auto &&kget, auto &&vget, const bool *valid) {
        if constexpr (QPAIR)
            attn_fold_q(A, nq_tag, [&](int h, int e) { return qpair_elem(A.qr[h], e); }, kget, vget, valid);
        else
            attn_fold_q(A, nq_tag, [&](int h, int e) { return A.qr[h][e]; }, kget, vget, valid);
    };
    // This consumer's final state -> its partial records (o over its
    // positions, m, l), one per head, as tagged records.
    constexpr int PREC = DH + 2;  // partial record: o[DH], m, l
    const int S_eff = S * CPH;    // effective splits per KV head
    auto attn_finish = [&](AttnState &A, int l) {
        uint64_t *part = p.ll_part + (((size_t)(l & 1) * p.nkv + kvj) * S_eff + kvs * CPH + cs) * GQ * PREC;
        const uint32_t tg = tag_of(l);
#pragma unroll
        for (int k = 0; k < HPC; ++k) {
            const int h = hc + HG * k;
            const float lsum = xgroup_sum<LPP>(A.al[k]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ov = xgroup_sum<LPP>(A.ao[k][e]);
                if (lane < LPP) stll(part + h * PREC + e0 + e, ov, tg);
            }
            if (lane == 0) {
                stll(part + h * PREC + d, A.am[k], tg);
                stll(part + h * PREC + d + 1, lsum, tg);
            }
        }
    };

    // ---- epilogues (consumer 0) ----
    // The rotary cos/sin pairs of this workgroup's query/key units depend only
    // on the position, the same in every layer: consumer 0 parks the first 64
    // units' pairs in LDS once per step (registers are the scarcer resource;
    // consumer 0 alone writes and reads them, so no barrier is needed).
    const float *rope_row = p.rope + (size_t)P * d;  // [d/2][2]
    auto rope_of_unit = [&](int u) -> f4v {
        const int r = ((g.unit0[ST_QKV] + u) * 4) % d;  // query and key rows share the angles by head dim
        return *(const f4v *)(rope_row + r);
    };
    if (c == 0 && lane < g.units[ST_QKV]) *(LDS f4v *)(ropel + 4 * lane) = rope_of_unit(lane);
    auto epi_qkv = [&](int l, float inv) {
        const int nqd = p.nh * d, nk = p.nkv * d;
        const uint32_t tg = tag_of(l);
        uint64_t *const qkv_l = p.ll_qkv + (size_t)(l & 1) * p.nkv * (GQ + 2) * d;
        const LDS float *sc = scl_of(l);  // INT8: the QKV rows' scales open the block
        for (int u = lane; u < g.units[ST_QKV]; u += 64) {
            const int gr0 = (g.unit0[ST_QKV] + u) * 4;
            const float y0 = outv[u * 4] * inv * rsc(sc, u * 4), y1 = outv[u * 4 + 1] * inv * rsc(sc, u * 4 + 1);
            const float y2 = outv[u * 4 + 2] * inv * rsc(sc, u * 4 + 2), y3 = outv[u * 4 + 3] * inv * rsc(sc, u * 4 + 3);
            if (gr0 < nqd + nk) {
                const bool isq = gr0 < nqd;
                const int r = isq ? gr0 : gr0 - nqd;
                const int head = r / d, m0 = (r % d) / 2;
                const f4v rc = u < 64 ? *(const LDS f4v *)(ropel + 4 * u) : rope_of_unit(u);
                const float c0 = rc.x, s0 = rc.y, c1 = rc.z, s1 = rc.w;
                const float a0 = y0 * c0 - y1 * s0, b0 = y0 * s0 + y1 * c0;
                const float a1 = y2 * c1 - y3 * s1, b1 = y2 * s1 + y3 * c1;
                if (isq) {
                    uint64_t *qd = qkv_l + (size_t)(head / GQ) * (GQ + 2) * d + (size_t)(head % GQ) * d;
                    stll(qd + m0, a0, tg);
                    stll(qd + m0 + 1, a1, tg);
                    stll(qd + m0 + d / 2, b0, tg);
                    stll(qd + m0 + 1 + d / 2, b1, tg);
                } else {
                    unsigned char *row = (unsigned char *)p.kc + ((size_t)l * p.nkv + head) * head_bytes + (size_t)P * d * EB;
                    uint64_t *kn = qkv_l + (size_t)head * (GQ + 2) * d + (size_t)GQ * d;
                    if constexpr (CDT == 1) {
                        const uint32_t ba0 = f2bf(a0), ba1 = f2bf(a1), bb0 = f2bf(b0), bb1 = f2bf(b1);
                        stcu((uint32_t *)(row + m0 * 2), ba0 | (ba1 << 16));
                        stcu((uint32_t *)(row + (m0 + d / 2) * 2), bb0 | (bb1 << 16));
                        stll(kn + m0, __uint_as_float(ba0 << 16), tg);
                        stll(kn + m0 + 1, __uint_as_float(ba1 << 16), tg);
                        stll(kn + m0 + d / 2, __uint_as_float(bb0 << 16), tg);
                        stll(kn + m0 + 1 + d / 2, __uint_as_float(bb1 << 16), tg);
                    } else {
                        stc((float *)row + m0, a0);
                        stc((float *)row + m0 + 1, a1);
                        stc((float *)row + m0 + d / 2, b0);
                        stc((float *)row + m0 + 1 + d / 2, b1);
                        stll(kn + m0, a0, tg);
                        stll(kn + m0 + 1, a1, tg);
                        stll(kn + m0 + d / 2, b0, tg);
                        stll(kn + m0 + 1 + d / 2, b1, tg);
                    }
                }
            } else if (gr0 < nqd + 2 * nk) {
                const int r = gr0 - nqd - nk;
                const int head = r / d, e = r % d;
                unsigned char *row = (unsigned char *)p.vc + ((size_t)l * p.nkv + head) * head_bytes + (size_t)P * d * EB;
                uint64_t *vn = qkv_l + (size_t)head * (GQ + 2) * d + (size_t)(GQ + 1) * d;
                if constexpr (CDT == 1) {
                    const uint32_t c0 = f2bf(y0), c1 = f2bf(y1), c2 = f2bf(y2), c3 = f2bf(y3);
                    stcu((uint32_t *)(row + e * 2), c0 | (c1 << 16));
                    stcu((uint32_t *)(row + e * 2 + 4), c2 | (c3 << 16));
                    stll(vn + e, __uint_as_float(c0 << 16), tg);
                    stll(vn + e + 1, __uint_as_float(c1 << 16), tg);
                    stll(vn + e + 2, __uint_as_float(c2 << 16), tg);
                    stll(vn + e + 3, __uint_as_float(c3 << 16), tg);
                } else {
                    stc((float *)row + e, y0);
                    stc((float *)row + e + 1, y1);
                    stc((float *)row + e + 2, y2);
                    stc((float *)row + e + 3, y3);
                    stll(vn + e, y0, tg);
                    stll(vn + e + 1, y1, tg);
                    stll(vn + e + 2, y2, tg);
                    stll(vn + e + 3, y3, tg);
                }
            }
        }
    };
    auto epi_o = [&](int l, uint64_t *xdst, uint32_t tg) {  // O(l): x += out for the workgroup's rows
        const LDS float *sc = scl_of(l) + 4 * g.units[ST_QKV];  // INT8: the O rows' scales
        for (int i = lane; i < g.units[ST_O] * 4; i += 64) {
            const int r = g.unit0[ST_O] * 4 + i;
            if (r < p.H) {
                const float xn = xown[i] + outv[i] * rsc(sc, i);
                xown[i] = xn;
                stll(xdst + r, xn, tg);
            }
        }
    };
    // SwiGLU of this workgroup's gate/up rows: a[f0 + m] -> vec[m] (the
    // down stage's input stays in the workgroup), zero-padded to kp pieces.
    auto epi_gu = [&](int l, float inv) {
        const LDS float *sc = scl_of(l) + 4 * (g.units[ST_QKV] + g.units[ST_O]);  // INT8: the gate/up rows' scales
        for (int m = lane; m < g.dn.kp * EPLW; m += 64) {
            float av = 0.f;
            if (m < g.dn.nf) {
                const float gv = outv[2 * m] * inv * rsc(sc, 2 * m), uv = outv[2 * m + 1] * inv * rsc(sc, 2 * m + 1);
                av = gv / (1.0f + __expf(-gv)) * uv;
            }
            vec[m] = av;
        }
    };
    // Log-sum-exp merge of the splits (blocks of 8 elements per consumer): workgroup w produces
    // attention-output elements [w*N/G, (w+1)*N/G) of N = n_heads*d.  Lane s
    // reads effective split s's (m, l) and the element's o value; the
    // weights are exp(m_s - max m) and the result sum(w_s o_s) / sum(w_s l_s).
    auto combine_slice = [&](int l) -> bool {
        const int N = p.nh * d;
        const int e_0 = (int)((int64_t)w * N / G), e_1 = (int)((int64_t)(w + 1) * N / G);
        const uint32_t tg = tag_of(l);
        const __amdgpu_buffer_rsrc_t rp = rsrc(p.ll_part + (size_t)(l & 1) * p.nkv * S_eff * GQ * PREC,
                                               (uint32_t)((size_t)p.nkv * S_eff * GQ * PREC * 8));
        const bool ln = lane < S_eff;
        poll_start = wall_clock64();
        int cur_h = -1;
        float M = 0.f, Ls = 1.f;
        // blocks of 8 elements dealt to the four consumers, so that the
        // blocks' waits run side by side
        for (int eb = e_0 + 8 * c; eb < e_1; eb += 8 * MK_NUM_CONSUMERS) {
            uint32_t mask = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (eb + u < e_1 && ln) mask |= 3u << (2 * u);
            // piece 2u: (m, l) of element eb+u's head; piece 2u+1: the pair holding its o value
            auto off = [&](int i) {
                const int e = eb + i / 2, h = e / d;
                const uint32_t rec = (uint32_t)(((h / GQ) * S_eff + lane) * GQ + h % GQ) * PREC;
                return (rec + ((i & 1) ? ((e % d) & ~1) : d)) * 8u;
            };
            u4v v[16];
            if (!poll16<16>(rp, off, mask, v, tg, poll_ok)) return false;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = eb + u;
                if (e < e_1) {  // wave-uniform
                    const int h = e / d, dim = e % d;
                    const float ms = ln ? __uint_as_float(v[2 * u].x) : -INFINITY;
                    const bool new_head = h != cur_h;  // wave-uniform
                    if (new_head) M = wave_max(ms);
                    const float wgt = ms == -INFINITY ? 0.f : __expf(ms - M);
                    if (new_head) {
                        Ls = wave_sum(ln ? wgt * __uint_as_float(v[2 * u].z) : 0.f);
                        cur_h = h;
                    }
                    const float ov = ln ? __uint_as_float((dim & 1) ? v[2 * u + 1].z : v[2 * u + 1].x) : 0.f;
                    const float os = wave_sum(wgt * ov);
                    if (lane == 0) stll(p.ll_o + (size_t)(l & 1) * N + e, os / Ls, tg);
                }
            }
        }
        return true;
    };
    auto epi_lm = [&](float inv) {
        float best = -INFINITY;
        int besti = 0x7FFFFFFF;
        for (int i = lane; i < g.units[ST_LM] * 4; i += 64) {
            const int r = g.unit0[ST_LM] * 4 + i;
            if (r < p.V) {
                const float lg = outv[i] * inv * rsc(scl_of(L), i);
                if (p.logits) p.logits[r] = lg;
                if (lg > best) { best = lg; besti = r; }
            }
        }
        if (!p.token_out) return;
        // wave argmax, lowest index on ties
        for (int m = 1; m < 64; m <<= 1) {
            const float ob = __shfl_xor(best, m);
            const int oi = __shfl_xor(besti, m);
            if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
        }
        if (lane == 0) {
            stll(p.ll_amax + 2 * (size_t)w, best, tag_of(L));
            stll(p.ll_amax + 2 * (size_t)w + 1, __int_as_float(besti), tag_of(L));
        }
        if (w != 0) return;
        // Workgroup 0 reduces the G (max, index) records.  This is the last
        // wait of the step; if it fails the error word is already set and the
        // token is not written.
        const __amdgpu_buffer_rsrc_t ra = rsrc(p.ll_amax, (uint32_t)G * 16u);
        poll_start = wall_clock64();
        best = -INFINITY;
        besti = 0x7FFFFFFF;
        for (int k0 = 0; k0 < 16; k0 += 8) {
            uint32_t mask = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (lane + 64 * (k0 + k) < G) mask |= 1u << k;
            u4v v[8];
            if (!poll16<8>(ra, [&](int k) { return (uint32_t)(lane + 64 * (k0 + k)) * 16u; }, mask, v, tag_of(L),
                           poll_ok))
                return;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (mask & (1u << k)) {
                    const float vb = __uint_as_float(v[k].x);
                    const int ix = (int)v[k].z;
                    if (vb > best || (vb == best && ix < besti)) { best = vb; besti = ix; }
                }
            }
        }
        for (int m = 1; m < 64; m <<= 1) {
            const float ob = __shfl_xor(best, m);
            const int oi = __shfl_xor(besti, m);
            if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
        }
        if (lane == 0) p.token_out[0] = besti;
    };


    // ---- the program ----
    const int nq = p.nh * d;
    // The register path's input slice (gain (.) x) from the gathered vector.
    auto regs_from_vec = [&](float (&hr)[4][EPLW]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < EPLW; e += 4) {
                const f4v t = *(const LDS f4v *)(vec + q * EPCW + lane * EPLW + e);
                hr[q][e] = t.x;
                hr[q][e + 1] = t.y;
                hr[q][e + 2] = t.z;
                hr[q][e + 3] = t.w;
            }
    };
    // The GEMV data steps of stage st, input in vec (gathered) or, for the
    // register path, loaded from it.
    auto gemv_from_vec = [&](int st, int l, int b) __attribute__((always_inline)) {
        if (REGP && p.st[st].rbp == 4) {
            float hr[4][EPLW];
            regs_from_vec(hr);
            stamp(b, 3);
            gemv_reg_steps(st, l, hr);
        } else {
            stamp(b, 3);
            gemv_lds_steps(st, l);
        }
    };
    sc_fetch(0);  // INT8: layer 0's scales
    sc_park(0);
    for (int l = 0; l < L && ok; ++l) {
        // ===== stage QKV(l); boundary: [epilogue DOWN(l-1)] + input x =====
        float inv_q = 0.f;
        {
            barrier();
            stamp(5 * l, 0);
            const float *gain = p.g_attn + (size_t)l * p.H;
            if (l == 0) {
                int tok = p.token_dev ? p.token_dev[0] : p.token;
                if (tok < 0 || tok >= p.V) {
                    if (ct == 0) __hip_atomic_fetch_or(p.err, MK_DEVERR_TOKEN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    tok = 0;
                }
                const void *erow = (const unsigned char *)p.embed + (size_t)tok * p.H * EB;
                for (int i = ct; i < g.units[ST_O] * 4; i += 256) {
                    const int r = g.unit0[ST_O] * 4 + i;
                    float xv = 0.f;
                    if (r < p.H) {
                        if constexpr (CDT == 1) xv = __uint_as_float((uint32_t)((const uint16_t *)erow)[r] << 16);
                        else xv = ((const float *)erow)[r];
                    }
                    xown[i] = xv;
                }
                if (REGP && p.st[ST_QKV].rbp == 4) {
                    float hr[4][EPLW];
                    inv_q = inv_of(load_direct(nullptr, erow, gain, hr), p.H);
                    stamp(5 * l, 3);
                    gemv_reg_steps(ST_QKV, l, hr);
                } else {
                    load_normed(nullptr, erow, gain, p.H, p.st[ST_QKV].rbp * EPCW);
                    ok = csync();
                    if (!ok) break;
                    inv_q = inv_lds(p.H);
                    stamp(5 * l, 3);
                    gemv_lds_steps(ST_QKV, l);
                }
            } else {
                ok = down_reduce(l - 1, p.ll_xq + (size_t)(l & 1) * p.H);
                stamp(5 * l, 1);
                ok = ok && gather(p.ll_xq + (size_t)(l & 1) * p.H, p.H, gain, p.st[ST_QKV].rbp * EPCW, tag_of(l));
                stamp(5 * l, 2);
                if (!ok) break;
                inv_q = inv_lds(p.H);
                gemv_from_vec(ST_QKV, l, 5 * l);
            }
        }

        // ===== attention(l); boundary: epilogue QKV(l) + q, new K/V row =====
        {
            barrier();
            stamp(5 * l + 1, 0);
            if (c == 0) epi_qkv(l, inv_q);
            stamp(5 * l + 1, 1);
            if (has_split) {
                // Consumers of chunk subset 0 also fold the tail positions and,
                // in the last split, position pos.  The tail rows were written
                // by earlier steps: plain loads, issued first to hide latency.
                const bool fold_extra = cs == 0;
                const int tg = lane / LPP;
                const bool tvalid = fold_extra && tg < ntail;
                float kt[EPL], vt[EPL];
                if (fold_extra && ntail > 0) {
                    // the tail's rows: at most PPC positions from t0 + nfull * BP
                    const size_t rbase = (((size_t)l * p.nkv + kvj) * p.max_seq + (size_t)t0 + (size_t)nfull * BP) * d * EB;
                    const uint32_t tbytes = (uint32_t)(PPC * d * EB);
                    const uint32_t roff = (uint32_t)(((tvalid ? tg : 0) * d + e0) * EB);
                    piece_load_buf<CDT>(rsrc((const unsigned char *)p.kc + rbase, tbytes), roff, kt);
                    piece_load_buf<CDT>(rsrc((const unsigned char *)p.vc + rbase, tbytes), roff, vt);
                }
                // This group's rotated queries and, in the last split, the K/V
                // row of position pos (bf16-rounded like the cache) into LDS in
                // one gather (they are stored next to each other); vec is free
                // here (the QKV input is no longer needed).
                {
                    const int nrec = (is_last ? GQ + 2 : GQ) * d;  // the last split also takes K/V of pos
                    ok = gather_to(vec, p.ll_qkv + ((size_t)(l & 1) * p.nkv + kvj) * (GQ + 2) * d, nrec, nullptr, nrec,
                                   tag_of(l));
                }
                stamp(5 * l + 1, 2);
                if (!ok) break;
                stamp(5 * l + 1, 3);
                // Position-major mapping, for a group of exactly four query
                // heads and a split of at least attn_pm_slots KV slots (long
                // contexts): consumer c folds chunks 2c and 2c+1 of every slot
                // for all four heads, so each K/V chunk is read from LDS once
                // per workgroup instead of once per head, and each consumer
                // runs four independent softmax chains.  At the end the four
                // consumers' partials of each head are merged in LDS (log-sum-
                // exp) into the same per-head records the head-major mapping
                // writes.  Otherwise head-major (below).  The two mappings run
                // separate loops so that only one running state is live.
                constexpr bool PM_OK = PMAP && GQ == MK_NUM_CONSUMERS;
                if constexpr (PM_OK) {
                    {
                        AttnStQ<GQ, EPL> P;  // the queries stay in vec (LDS)
#pragma unroll
                        for (int h = 0; h < GQ; ++h) {
#pragma unroll
                            for (int e = 0; e < EPL; ++e) P.ao[h][e] = 0.f;
                            P.am[h] = -INFINITY;
                            P.al[h] = 0.f;
                        }
                        auto qlds = [&](int h, int e) { return vec[h * d + e0 + e]; };
                        // End of the split: consumer 0 folds the tail and
                        // position pos for all heads, every consumer's
                        // per-head partials go to LDS (after the queries and
                        // the row of pos in vec), then consumer c merges head c
                        // and writes its record.
                        auto finish_pm = [&]() {
                            if (c == 0 && ntail > 0) {
                                const bool v1[1] = {tg < ntail};
                                attn_fold_q(P, std::integral_constant<int, 1>{}, qlds, [&](int, int e) { return kt[e]; },
                                            [&](int, int e) { return vt[e]; }, v1);
                            }
                            if (c == 0 && is_last) {
                                float kp[EPL], vp[EPL];
#pragma unroll
                                for (int e = 0; e < EPL; ++e) {
                                    kp[e] = vec[GQ * d + e0 + e];
                                    vp[e] = vec[GQ * d + d + e0 + e];
                                }
                                const bool v1[1] = {lane < LPP};
                                attn_fold_q(P, std::integral_constant<int, 1>{}, qlds, [&](int, int e) { return kp[e]; },
                                            [&](int, int e) { return vp[e]; }, v1);
                            }
                            LDS float *mg = vec + (GQ + 2) * d;  // [consumer][head][d + 2]: o, m, l
#pragma unroll
                            for (int h = 0; h < GQ; ++h) {
                                LDS float *dst = mg + (c * GQ + h) * PREC;
                                const float lsum = xgroup_sum<LPP>(P.al[h]);
#pragma unroll
                                for (int e = 0; e < EPL; ++e) {
                                    const float ov = xgroup_sum<LPP>(P.ao[h][e]);
                                    if (lane < LPP) dst[e0 + e] = ov;
                                }
                                if (lane == 0) {
                                    dst[d] = P.am[h];
                                    dst[d + 1] = lsum;
                                }
                            }
                            if (!csync()) {
                                ok = false;
                                return;
                            }
                            const int hh = c;  // the head this consumer merges
                            float M = -INFINITY;
#pragma unroll
                            for (int j = 0; j < MK_NUM_CONSUMERS; ++j) M = fmaxf(M, mg[(j * GQ + hh) * PREC + d]);
                            float wj[MK_NUM_CONSUMERS], Lsum = 0.f;
#pragma unroll
                            for (int j = 0; j < MK_NUM_CONSUMERS; ++j) {
                                const float mj = mg[(j * GQ + hh) * PREC + d];
                                wj[j] = mj == -INFINITY ? 0.f : __expf(mj - M);
                                Lsum = fmaf(wj[j], mg[(j * GQ + hh) * PREC + d + 1], Lsum);
                            }
                            uint64_t *part = p.ll_part + (((size_t)(l & 1) * p.nkv + kvj) * S_eff + kvs) * GQ * PREC;
                            const uint32_t tg2 = tag_of(l);
                            for (int e = lane; e < d; e += 64) {
                                float ov = 0.f;
#pragma unroll
                                for (int j = 0; j < MK_NUM_CONSUMERS; ++j)
                                    ov = fmaf(wj[j], mg[(j * GQ + hh) * PREC + e], ov);
                                stll(part + hh * PREC + e, ov, tg2);
                            }
                            if (lane == 0) {
                                stll(part + hh * PREC + d, M, tg2);
                                stll(part + hh * PREC + d + 1, Lsum, tg2);
                            }
                        };
                        for (int n = 0; n < nsl_kv; ++n) {
                            data_barrier(n);
                            stamp_step(l, 0);
                            const LDS unsigned char *kb = ring + js * MK_SLOT_BYTES;
                            const LDS unsigned char *vb = kb + 8 * MK_CHUNK_BYTES;
                            u4v kr[2], vr[2];
                            bool valid[2];
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                const int chunk = 2 * c + q;
                                valid[q] = t0 + n * BP + chunk * PPC + lane / LPP < t1;
                                kr[q] = *(const LDS u4v *)(kb + chunk * MK_CHUNK_BYTES + lane * 16);
                                vr[q] = *(const LDS u4v *)(vb + chunk * MK_CHUNK_BYTES + lane * 16);
                            }
                            attn_fold_q(P, std::integral_constant<int, 2>{}, qlds,
                                        [&](int q, int e) { return piece_elem<CDT>(kr[q], e); },
                                        [&](int q, int e) { return piece_elem<CDT>(vr[q], e); }, valid);
                            if (n == nsl_kv - 1) finish_pm();
                            js = js + 1 == NS ? 0 : js + 1;
                            stamp_step(l, 1);
                        }
                        if (nsl_kv == 0) finish_pm();
                    }
                } else {
                AttnState A;
#pragma unroll
                for (int k = 0; k < HPC; ++k) {
                    float qv[EPL];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        qv[e] = vec[(hc + HG * k) * d + e0 + e];
                        A.ao[k][e] = 0.f;
                    }
                    if constexpr (QPAIR) {
                        qpair_set(A.qr[k], qv);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPL; ++e) A.qr[k][e] = qv[e];
                    }
                    A.am[k] = -INFINITY;
                    A.al[k] = 0.f;
                }
                auto finish = [&]() {
                    if (fold_extra && ntail > 0) {
                        const bool v1[1] = {tvalid};
                        attn_fold(A, std::integral_constant<int, 1>{}, [&](int, int e) { return kt[e]; },
                                  [&](int, int e) { return vt[e]; }, v1);
                    }
                    if (fold_extra && is_last) {
                        float kp[EPL], vp[EPL];
#pragma unroll
                        for (int e = 0; e < EPL; ++e) {
                            kp[e] = vec[GQ * d + e0 + e];
                            vp[e] = vec[GQ * d + d + e0 + e];
                        }
                        const bool v1[1] = {lane < LPP};
                        attn_fold(A, std::integral_constant<int, 1>{}, [&](int, int e) { return kp[e]; },
                                  [&](int, int e) { return vp[e]; }, v1);
                    }
                    attn_finish(A, l);
                };
                if (nsl_kv == 0) finish();
                for (int n = 0; n < nsl_kv; ++n) {
                    data_barrier(n);
                    stamp_step(l, 0);
                    const LDS unsigned char *kb = ring + js * MK_SLOT_BYTES;
                    const LDS unsigned char *vb = kb + 8 * MK_CHUNK_BYTES;
#pragma unroll
                    for (int b = 0; b < CPS; b += NQB) {
                        // raw 16-byte pieces; each element is widened where it is used
                        u4v kr[NQB], vr[NQB];
                        bool valid[NQB];
#pragma unroll
                        for (int q = 0; q < NQB; ++q) {
                            const int chunk = cs * CPS + b + q;
                            valid[q] = t0 + n * BP + chunk * PPC + lane / LPP < t1;
                            kr[q] = *(const LDS u4v *)(kb + chunk * MK_CHUNK_BYTES + lane * 16);
                            vr[q] = *(const LDS u4v *)(vb + chunk * MK_CHUNK_BYTES + lane * 16);
                        }
                        if constexpr (QPAIR)
                            attn_fold_w(A, std::integral_constant<int, NQB>{}, kr,
                                        [&](int q, int e) { return piece_elem<CDT>(vr[q], e); }, valid);
                        else
                            attn_fold(A, std::integral_constant<int, NQB>{},
                                      [&](int q, int e) { return piece_elem<CDT>(kr[q], e); },
                                      [&](int q, int e) { return piece_elem<CDT>(vr[q], e); }, valid);
                    }
                    if (n == nsl_kv - 1) finish();
                    js = js + 1 == NS ? 0 : js + 1;
                    stamp_step(l, 1);
                }
                }  // head-major
            } else {
                stamp(5 * l + 1, 3);
            }
        }

        // ===== stage O(l); boundary: attention partials, combine, input o =====
        {
            barrier();
            stamp(5 * l + 2, 0);
            const bool mine = combine_slice(l);
            stamp(5 * l + 2, 1);
            ok = mine && gather(p.ll_o + (size_t)(l & 1) * nq, nq, nullptr, p.st[ST_O].rbp * EPCW, tag_of(l));
            stamp(5 * l + 2, 2);
            if (!ok) break;
            gemv_from_vec(ST_O, l, 5 * l + 2);
        }

        // ===== stage gate/up(l); boundary: epilogue O(l) + input x =====
        float inv_g = 0.f;
        {
            barrier();
            stamp(5 * l + 3, 0);
            if (c == 0) epi_o(l, p.ll_xg + (size_t)(l & 1) * p.H, tag_of(l));
            stamp(5 * l + 3, 1);
            ok = gather(p.ll_xg + (size_t)(l & 1) * p.H, p.H, p.g_ffn + (size_t)l * p.H, p.st[ST_GU].rbp * EPCW,
                        tag_of(l));
            stamp(5 * l + 3, 2);
            if (!ok) break;
            inv_g = inv_lds(p.H);
            if (LOGITS || l + 1 < L) sc_fetch(l + 1);  // INT8: the next block (layer l + 1, or the LM head)
            gemv_from_vec(ST_GU, l, 5 * l + 3);
        }

        // ===== stage down(l); boundary: epilogue gate/up(l) + input a =====
        {
            barrier();
            stamp(5 * l + 4, 0);
            if (c == 0) epi_gu(l, inv_g);
            if (LOGITS || l + 1 < L) sc_park(l + 1);  // INT8: the next block (read during gate/up) to LDS
            stamp(5 * l + 4, 1);
            ok = csync();
            stamp(5 * l + 4, 2);
            if (!ok) break;
            stamp(5 * l + 4, 3);
            down_steps(l);
        }
    }
    if (ok && LOGITS) {
        // ===== LM head; boundary: epilogue DOWN(L-1) + input x =====
        barrier();
        stamp(5 * L, 0);
        ok = down_reduce(L - 1, p.ll_xq + (size_t)(L & 1) * p.H);
        stamp(5 * L, 1);
        ok = ok && gather(p.ll_xq + (size_t)(L & 1) * p.H, p.H, p.g_final, p.st[ST_LM].rbp * EPCW, tag_of(L));
        stamp(5 * L, 2);
        if (ok) {
            const float inv_lm = inv_lds(p.H);
            gemv_from_vec(ST_LM, L, 5 * L);
            barrier();
            stamp(5 * L + 1, 0);
            if (c == 0) epi_lm(inv_lm);
            stamp(5 * L + 1, 1);
        }
    } else if (ok) {
        // Without the LM head the last layer's output is not needed: only
        // the cache rows written by the attention stages are the result.
        barrier();
        stamp(5 * L + 1, 0);
        stamp(5 * L + 1, 1);
    }
    if (!ok) {
        // Aborted inside step `step` (ctl[1] == step): pass one more barrier,
        // after which the loaders see an abort from an earlier step and leave.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
    }
    MK_WAIT_VM0();
}

// ---- instantiations and host-side launch ----------------------------------
// The kernel is instantiated for every (dtype, group, lanes per cache row,
// LOGITS, position-major) combination the host can pick.  The build compiles
// this file once per (dtype, group) part with MK_KERNEL_PART, MK_PART_DT and
// MK_PART_GQ defined, each part instantiating its kernels, and once without,
// for the host code below, which only declares them (extern template); the
// parts compile in parallel.
#define MK_FOR_LPP_LOGITS(X, DT_, GQ_, PM_) \
    X(DT_, GQ_, 8, true, PM_) X(DT_, GQ_, 8, false, PM_) X(DT_, GQ_, 16, true, PM_) X(DT_, GQ_, 16, false, PM_)
// position-major instantiations exist for groups of four query heads only
#define MK_FOR_PM(X, DT_, GQ_) MK_FOR_LPP_LOGITS(X, DT_, GQ_, false) if_gq4_##GQ_(MK_FOR_LPP_LOGITS(X, DT_, GQ_, true))
#define if_gq4_1(...)
#define if_gq4_2(...)
#define if_gq4_4(...) __VA_ARGS__
#define if_gq4_8(...)

#ifdef MK_KERNEL_PART
#define MK_INST(DT_, GQ_, LPP_, LG_, PM_) \
    template __global__ void mk_decode_kernel<DT_, GQ_, LPP_, LG_, PM_>(const MkParams);
#define MK_PART_EXPAND(DT_, GQ_) MK_FOR_PM(MK_INST, DT_, GQ_)
#define MK_PART_EXPAND2(DT_, GQ_) MK_PART_EXPAND(DT_, GQ_)
MK_PART_EXPAND2(MK_PART_DT, MK_PART_GQ)
#else
#define MK_EXTERN(DT_, GQ_, LPP_, LG_, PM_) \
    extern template __global__ void mk_decode_kernel<DT_, GQ_, LPP_, LG_, PM_>(const MkParams);
#define MK_ALL_PARTS(X) \
    MK_FOR_PM(X, 0, 1) MK_FOR_PM(X, 0, 2) MK_FOR_PM(X, 0, 4) MK_FOR_PM(X, 0, 8) \
    MK_FOR_PM(X, 1, 1) MK_FOR_PM(X, 1, 2) MK_FOR_PM(X, 1, 4) MK_FOR_PM(X, 1, 8) \
    MK_FOR_PM(X, 2, 1) MK_FOR_PM(X, 2, 2) MK_FOR_PM(X, 2, 4) MK_FOR_PM(X, 2, 8)
MK_ALL_PARTS(MK_EXTERN)

// ---- host-side launch ---------------------------------------------------
namespace {
typedef void (*KernelFn)(const MkParams);

template <int DT, int GQ, int LPP>
KernelFn kfn(bool logits, bool pmap) {
    if constexpr (GQ == MK_NUM_CONSUMERS) {
        if (pmap) return logits ? mk_decode_kernel<DT, GQ, LPP, true, true> : mk_decode_kernel<DT, GQ, LPP, false, true>;
    }
    return logits ? mk_decode_kernel<DT, GQ, LPP, true, false> : mk_decode_kernel<DT, GQ, LPP, false, false>;
}

KernelFn pick(int dtype, int gq, int lpp, bool logits, bool pmap) {
#define MK_PICK(DT_, GQ_, LPP_) if (dtype == DT_ && gq == GQ_ && lpp == LPP_) return kfn<DT_, GQ_, LPP_>(logits, pmap);
    MK_PICK(1, 1, 8) MK_PICK(1, 2, 8) MK_PICK(1, 4, 8) MK_PICK(1, 8, 8)
    MK_PICK(1, 1, 16) MK_PICK(1, 2, 16) MK_PICK(1, 4, 16) MK_PICK(1, 8, 16)
    MK_PICK(0, 1, 8) MK_PICK(0, 2, 8) MK_PICK(0, 4, 8) MK_PICK(0, 8, 8)
    MK_PICK(0, 1, 16) MK_PICK(0, 2, 16) MK_PICK(0, 4, 16) MK_PICK(0, 8, 16)
    MK_PICK(2, 1, 8) MK_PICK(2, 2, 8) MK_PICK(2, 4, 8) MK_PICK(2, 8, 8)
    MK_PICK(2, 1, 16) MK_PICK(2, 2, 16) MK_PICK(2, 4, 16) MK_PICK(2, 8, 16)
#undef MK_PICK
    return nullptr;
}
}  // namespace

// sc_floats: both LDS copies of the INT8 scale blocks (0 for other dtypes)
extern "C" int mk_kernel_lds_bytes(int ring_slots, int vec_floats, int out_rows, int sc_floats) {
    const int floats = vec_floats + out_rows + 64 + 256 + MK_NUM_CONSUMERS + 16 + sc_floats;
    return ring_slots * MK_SLOT_BYTES + floats * 4;
}

extern "C" int mk_launch_decode(const MkParams *p, int dtype, int cooperative, void *stream) {
    const int eb = dtype ? 2 : 4;  // cache element bytes (dtype 2 keeps a bf16 cache)
    const int lpp = p->d * eb / 16;
    const int gq = p->nh / p->nkv;
    // per-length attention mapping: position-major when a split holds at
    // least attn_pm_slots whole KV slots (BP positions each)
    const int bp = 8 * (64 / lpp);
    const int per = (p->pos + p->splits - 1) / p->splits;
    const bool pmap = gq == MK_NUM_CONSUMERS && per / bp >= p->attn_pm_slots;
    KernelFn fn = pick(dtype, gq, lpp, p->want_logits != 0, pmap);
    if (!fn) return (int)hipErrorInvalidValue;
    // the dynamic-LDS limit of every instantiation was raised to MK_LDS_LIMIT
    // when the handle was created (mk_kernel_max_blocks_per_cu)
    const int lds = mk_kernel_lds_bytes(p->ring_slots, p->lds_vec_floats, p->lds_out_rows, 2 * p->lds_sc_floats);
    hipError_t e;
    MkParams copy = *p;
    void *args[] = {&copy};
    if (cooperative)
        e = hipLaunchCooperativeKernel((const void *)fn, dim3(p->grid), dim3(MK_BLOCK_THREADS), args, lds,
                                       (hipStream_t)stream);
    else
        e = hipLaunchKernel((const void *)fn, dim3(p->grid), dim3(MK_BLOCK_THREADS), args, lds, (hipStream_t)stream);
    return (int)e;
}

extern "C" int mk_kernel_max_blocks_per_cu(int dtype, int gq, int lpp, int lds) {
    int best = 1 << 30;
    for (int k = 0; k < 4; ++k) {
        KernelFn fn = pick(dtype, gq, lpp, (k & 1) != 0, (k & 2) != 0);
        if (!fn) return 0;
        if (hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, MK_LDS_LIMIT) !=
            hipSuccess)
            return 0;
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)fn, MK_BLOCK_THREADS, lds) != hipSuccess)
            return 0;
        if (n < best) best = n;
    }
    return best;
}
#endif  // MK_KERNEL_PART
