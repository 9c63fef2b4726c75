// Persistent batch-1 decode megakernel for gfx950 (MI355X).
//
// One launch runs a whole decode step (cloud.baidu.com/article/9434380,
// section 4.2: one launch with an internal pipeline instead of one launch
// per operator; developer.baidu.com/article/detail.html?id=8006242, section
// 4.1).  Each workgroup is resident on one CU for the whole step and has two
// roles:
//
//   loader waves (2)    copy the workgroup's weight slots -- and, for the
//                       attention stage, its KV-cache blocks -- from HBM into
//                       an LDS ring with gfx950 direct-to-LDS 16-byte loads.
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
// a stage boundary (consumer 0 finishes the stage, publishes progress, waits
// for the next stage's producers and the consumers load its input vector).
//
// Cross-workgroup dependencies use per-workgroup progress words instead of a
// counter barrier: a workgroup publishes epoch_base + k after point k; a
// consumer of point k polls all progress words.  Every value read by another
// workgroup within the launch (activations, q, the new K/V row, attention
// partials, progress words) is written and read with device-scope (sc1)
// accesses, so no L2 writeback/invalidate is needed.  The publisher waits for
// its stores (vmcnt 0) before the progress store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))
#define MK_COMPILER_BARRIER() asm volatile("" ::: "memory")
#define MK_WAIT_VM0() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")

// ---- device-scope (sc1) accesses ----------------------------------------
__device__ __forceinline__ float ldc(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ldc64(const void *p) {
    return __hip_atomic_load((uint64_t *)const_cast<void *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ldcu(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stcu(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stci(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt encoding (gfx9): vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
__device__ __forceinline__ void wait_vm_rt(int n) {
    switch (n) {
    case 8: wait_vm<8>(); break;
    case 16: wait_vm<16>(); break;
    case 24: wait_vm<24>(); break;
    case 32: wait_vm<32>(); break;
    case 40: wait_vm<40>(); break;
    case 48: wait_vm<48>(); break;
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
// Sum / max across the groups: lanes with equal (lane % LPP).
template <int LPP>
__device__ __forceinline__ float xgroup_sum(float v) {
#pragma unroll
    for (int m = LPP; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}
template <int LPP>
__device__ __forceinline__ float xgroup_max(float v) {
#pragma unroll
    for (int m = LPP; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
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

// Dot product of one 16-byte weight piece (in LDS) with the matching input
// elements (in LDS).
template <int DT>
__device__ __forceinline__ float piece_dot(const LDS unsigned char *wp, const LDS float *hp) {
    if constexpr (DT == 1) {
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
// Same from global memory with device-scope loads (the newly appended row).
template <int DT>
__device__ __forceinline__ void piece_load_dev(const unsigned char *p, float (&v)[16 / (DT ? 2 : 4)]) {
    uint64_t a = ldc64(p), b = ldc64(p + 8);
    if constexpr (DT == 1) {
        uint32_t w0 = (uint32_t)a, w1 = (uint32_t)(a >> 32), w2 = (uint32_t)b, w3 = (uint32_t)(b >> 32);
        v[0] = bf_lo(w0); v[1] = bf_hi(w0); v[2] = bf_lo(w1); v[3] = bf_hi(w1);
        v[4] = bf_lo(w2); v[5] = bf_hi(w2); v[6] = bf_lo(w3); v[7] = bf_hi(w3);
    } else {
        v[0] = __uint_as_float((uint32_t)a); v[1] = __uint_as_float((uint32_t)(a >> 32));
        v[2] = __uint_as_float((uint32_t)b); v[3] = __uint_as_float((uint32_t)(b >> 32));
    }
}

__device__ __forceinline__ int wg_unit0(int w, int U, int G) { return (int)(((int64_t)w * U) / G); }

struct Geo {
    int unit0[ST_NUM], units[ST_NUM], nsl[ST_NUM];
};

__device__ __forceinline__ void make_geo(const MkParams &p, int w, Geo &g) {
#pragma unroll
    for (int k = 0; k < ST_NUM; ++k) {
        const int U = p.st[k].units;
        g.unit0[k] = wg_unit0(w, U, p.grid);
        g.units[k] = wg_unit0(w + 1, U, p.grid) - g.unit0[k];
        g.nsl[k] = (g.units[k] * p.st[k].rbp + 3) / 4;
    }
}

// Order of streamed stages inside a layer; index 1 is the KV stream.
// kind 0: QKV, 1: KV, 2: O, 3: GU, 4: DOWN.  After the last layer: LM.
__device__ __forceinline__ int st_of_kind(int kind) {
    return kind == 0 ? ST_QKV : kind == 2 ? ST_O : kind == 3 ? ST_GU : kind == 4 ? ST_DOWN : ST_LM;
}

}  // namespace

template <int DT, int GQ, int LPP>
__global__ __launch_bounds__(MK_BLOCK_THREADS, 1) void mk_decode_kernel(const MkParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_[];
    LDS unsigned char *smem = (LDS unsigned char *)smem_;
    constexpr int EB = DT ? 2 : 4;          // bytes per element
    constexpr int EPL = 16 / EB;            // elements per 16-byte lane piece
    constexpr int EPC = MK_CHUNK_BYTES / EB;  // elements per 1 KiB chunk
    constexpr int PPC = 64 / LPP;           // cache positions per 1 KiB chunk
    constexpr int BP = 8 * PPC;             // positions per KV slot (8 K chunks + 8 V chunks)

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int w = blockIdx.x, G = p.grid, NS = p.ring_slots, L = p.L;
    const int d = p.d;

    // LDS layout: ring | vec | out | cstate | xown | ss | control
    LDS unsigned char *ring = smem;
    LDS float *vec = (LDS float *)(smem + NS * MK_SLOT_BYTES);
    LDS float *outv = vec + p.lds_vec_floats;
    LDS float *cst = outv + p.lds_out_rows;
    LDS float *xown = cst + MK_NUM_CONSUMERS * GQ * (d + 2);
    LDS float *ssp = xown + 64;
    volatile LDS int *ctl = (volatile LDS int *)(ssp + MK_NUM_CONSUMERS);  // [0] go step, [1] abort

    Geo g;
    make_geo(p, w, g);

    // Attention split of this workgroup: KV head kvj, positions [t0, t1).
    const int S = p.splits;
    const bool has_split = w < p.nkv * S;
    const int kvj = has_split ? w / S : 0, kvs = has_split ? w % S : 0;
    const int P = p.pos;
    const int per = (P + S - 1) / S;
    const int t0 = min(P, kvs * per), t1 = min(P, t0 + per);
    const int nt = has_split ? t1 - t0 : 0;
    const int nsl_kv = (nt + BP - 1) / BP;
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

    if (tid == 0) { ctl[0] = -1; ctl[1] = 0; }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    if (wave < MK_NUM_LOADERS) {
        // ============================ loader ============================
        const int wl = wave;
        // this workgroup's weight blocks for layer 0, and the per-layer strides
        const unsigned char *wb_q = p.packed + p.st[ST_QKV].base + p.st[ST_QKV].wg_off[w];
        const unsigned char *wb_o = p.packed + p.st[ST_O].base + p.st[ST_O].wg_off[w];
        const unsigned char *wb_gu = p.packed + p.st[ST_GU].base + p.st[ST_GU].wg_off[w];
        const unsigned char *wb_dn = p.packed + p.st[ST_DOWN].base + p.st[ST_DOWN].wg_off[w];
        const unsigned char *wb_lm = p.packed + p.st[ST_LM].base + p.st[ST_LM].wg_off[w];
        const int64_t ws_q = p.st[ST_QKV].layer_stride, ws_o = p.st[ST_O].layer_stride,
                      ws_gu = p.st[ST_GU].layer_stride, ws_dn = p.st[ST_DOWN].layer_stride;
        int it_l = 0, it_k = 0, it_n = 0;
        bool done = false;
        // position the iterator on the first non-empty stage
        auto settle = [&]() {
            while (!done && it_n >= nslots(it_k)) {
                it_n = 0;
                if (it_k == 5) { done = true; break; }
                if (++it_k == 5) {
                    if (++it_l == L) {
                        if (p.want_logits) it_k = 5; else done = true;
                    } else {
                        it_k = 0;
                    }
                }
            }
        };
        settle();
        auto issue = [&](int buf) {
            LDS unsigned char *dst = ring + buf * MK_SLOT_BYTES + wl * 8 * MK_CHUNK_BYTES;
            if (done) {
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    __builtin_amdgcn_global_load_lds((const void *)(p.packed + c * MK_CHUNK_BYTES + lane * 16),
                                                     (LDS void *)(dst + c * MK_CHUNK_BYTES),
                                                     16, 0, 0);
                return;
            }
            if (it_k == 1) {
                const unsigned char *base = (const unsigned char *)(wl == 0 ? p.kc : p.vc) +
                                            ((size_t)it_l * p.nkv + kvj) * head_bytes;
                const size_t lim = (size_t)t1 * d * EB;
                const size_t off0 = ((size_t)t0 + (size_t)it_n * BP) * d * EB + lane * 16;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    size_t off = off0 + c * MK_CHUNK_BYTES;
                    if (off >= lim) off = (lane % LPP) * 16;  // beyond the split: re-read position 0, masked by consumers
                    __builtin_amdgcn_global_load_lds((const void *)(base + off),
                                                     (LDS void *)(dst + c * MK_CHUNK_BYTES),
                                                     16, 0, 0);
                }
            } else {
                const unsigned char *blk;
                int64_t stride;
                switch (it_k) {
                case 0: blk = wb_q; stride = ws_q; break;
                case 2: blk = wb_o; stride = ws_o; break;
                case 3: blk = wb_gu; stride = ws_gu; break;
                case 4: blk = wb_dn; stride = ws_dn; break;
                default: blk = wb_lm; stride = 0; break;
                }
                const unsigned char *src = blk + (int64_t)it_l * stride + (int64_t)it_n * MK_SLOT_BYTES +
                                           wl * 8 * MK_CHUNK_BYTES + lane * 16;
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    __builtin_amdgcn_global_load_lds((const void *)(src + c * MK_CHUNK_BYTES),
                                                     (LDS void *)(dst + c * MK_CHUNK_BYTES),
                                                     16, 0, 2 /* nt: streamed once */);
            }
            ++it_n;
            settle();
        };
        for (int i = 0; i < NS - 1; ++i) issue(i);
        int j = 0;
        int lstep = 0;  // barriers passed; mirrors the consumers' step counter
        const int wait_n = (NS - 2) * 8;
        // ctl[1] holds the step in which a consumer aborted (0: none).  The
        // consumers pass exactly one more barrier after aborting, so "aborted
        // in an earlier step" is stable when read here.
        auto aborted = [&]() { const int a = ctl[1]; return a != 0 && a < lstep; };
        auto vstep = [&]() -> bool {
            MK_COMPILER_BARRIER();
            __builtin_amdgcn_s_barrier();
            MK_COMPILER_BARRIER();
            ++lstep;
            return !aborted();
        };
        auto dstep = [&]() -> bool {
            wait_vm_rt(wait_n);
            MK_COMPILER_BARRIER();
            __builtin_amdgcn_s_barrier();
            MK_COMPILER_BARRIER();
            ++lstep;
            if (aborted()) return false;
            issue((j + NS - 1) % NS);
            ++j;
            return true;
        };
        bool ok = true;
        for (int l = 0; l < L && ok; ++l)
            for (int kind = 0; kind < 5 && ok; ++kind) {
                ok = vstep();
                for (int n = 0; n < nslots(kind) && ok; ++n) ok = dstep();
            }
        if (ok && p.want_logits) {
            ok = vstep();
            for (int n = 0; n < nsl_lm && ok; ++n) ok = dstep();
        }
        if (ok) vstep();
        wait_vm<0>();
        return;
    }

    // ============================== consumers ==============================
    const int c = wave - MK_NUM_LOADERS;        // consumer index 0..3
    const int ct = tid - MK_NUM_LOADERS * 64;   // consumer thread 0..255
    int j = 0;      // next ring slot
    int step = 0;   // step counter (for the consumer-local go flag)
    bool ok = true;

    auto barrier = [&]() -> bool {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        ++step;
        return true;
    };

    // Progress publication (consumer 0, after its stores completed).
    auto publish = [&](int k) {
        MK_WAIT_VM0();
        if (lane == 0) stcu(p.flags + w, p.epoch_base + (uint32_t)k);
        MK_WAIT_VM0();
    };
    // Wait until every workgroup published point k.  Consumer 0 polls; the
    // other consumers wait for its go signal in LDS.  Returns false on abort.
    auto wait_all = [&](int k) -> bool {
        if (c == 0) {
            const uint32_t target = p.epoch_base + (uint32_t)k;
            const int64_t t_start = wall_clock64();
            bool good = true;
            while (true) {
                bool mine = true;
                for (int i = lane; i < G; i += 64) mine &= (int32_t)(ldcu(p.flags + i) - target) >= 0;
                if (__all(mine)) break;
                if (ldcu(p.err) != 0u || wall_clock64() - t_start > p.timeout_ticks) {
                    if (lane == 0) stcu(p.err, ldcu(p.err) | MK_DEVERR_TIMEOUT);
                    good = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            MK_COMPILER_BARRIER();
            if (lane == 0) {
                if (!good) ctl[1] = step;
                ctl[0] = step;
            }
            return good;
        }
        while (ctl[0] != step) __builtin_amdgcn_s_sleep(1);
        MK_COMPILER_BARRIER();
        return ctl[1] == 0;
    };

    // ---- input-vector loaders (all consumers) ----
    // vec[0..n) = gain (.) x (sc1 loads of x, or the embedding row), zero pad to
    // `pad`, and per-consumer sums of squares of x into ssp[c].
    auto load_normed = [&](const float *xsrc, const void *erow, const float *gain, int n, int pad) {
        float ss = 0.f;
        for (int i = ct; i < n / 2; i += 256) {
            float x0, x1;
            if (erow) {
                if constexpr (DT == 1) {
                    uint32_t wv = ((const uint32_t *)erow)[i];
                    x0 = bf_lo(wv); x1 = bf_hi(wv);
                } else {
                    x0 = ((const float *)erow)[2 * i]; x1 = ((const float *)erow)[2 * i + 1];
                }
            } else {
                uint64_t v = ldc64(xsrc + 2 * i);
                x0 = __uint_as_float((uint32_t)v); x1 = __uint_as_float((uint32_t)(v >> 32));
            }
            ss = fmaf(x0, x0, ss);
            ss = fmaf(x1, x1, ss);
            vec[2 * i] = gain[2 * i] * x0;
            vec[2 * i + 1] = gain[2 * i + 1] * x1;
        }
        for (int i = n + ct; i < pad; i += 256) vec[i] = 0.f;
        ss = wave_sum(ss);
        if (lane == 0) ssp[c] = ss;
    };
    auto load_plain = [&](const float *src, int n, int pad) {
        for (int i = ct; i < n / 2; i += 256) {
            uint64_t v = ldc64(src + 2 * i);
            vec[2 * i] = __uint_as_float((uint32_t)v);
            vec[2 * i + 1] = __uint_as_float((uint32_t)(v >> 32));
        }
        for (int i = n + ct; i < pad; i += 256) vec[i] = 0.f;
    };
    auto inv_rms = [&](int n) {
        const float ss = ssp[0] + ssp[1] + ssp[2] + ssp[3];
        return 1.0f / sqrtf(ss / (float)n + p.eps);
    };

    // ---- GEMV state ----
    int row_c = 0, kc = 0;
    float acc = 0.f;
    auto gemv_begin = [&]() { row_c = 0; kc = 0; acc = 0.f; };
    auto gemv_slot = [&](int st, int buf) {
        const LDS unsigned char *bp = ring + buf * MK_SLOT_BYTES + c * 4 * MK_CHUNK_BYTES + lane * 16;
        const int units = g.units[st], rbp = p.st[st].rbp;
#pragma unroll
        for (int qi = 0; qi < 4; ++qi) {
            if (row_c < units) {
                acc += piece_dot<DT>(bp + qi * MK_CHUNK_BYTES, vec + kc * EPC + lane * EPL);
                if (++kc == rbp) {
                    const float t = wave_sum(acc);
                    if (lane == 0) outv[row_c * 4 + c] = t;
                    acc = 0.f;
                    kc = 0;
                    ++row_c;
                }
            }
        }
    };

    // ---- attention state (per lane) ----
    float qr[GQ][EPL];
    float am[GQ], al[GQ], ao[GQ][EPL];
    float kp[EPL], vp[EPL];
    const float scale = 1.0f / sqrtf((float)d);
    const int e0 = (lane % LPP) * EPL;
    auto attn_begin = [&]() {
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            am[h] = -INFINITY;
            al[h] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) ao[h][e] = 0.f;
        }
    };
    // Fold one group of positions (one per lane group) into the running state.
    auto attn_fold = [&](const float (&kv)[EPL], const float (&vv)[EPL], bool valid) {
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) s = fmaf(qr[h][e], kv[e], s);
            s = group_sum<LPP>(s) * scale;
            s = valid ? s : -INFINITY;
            const float mx = xgroup_max<LPP>(s);
            const float mn = fmaxf(am[h], mx);
            if (mn == -INFINITY) continue;  // nothing valid yet (wave-uniform)
            const float alpha = __expf(am[h] - mn);
            // Masked positions contribute nothing; their V values are never
            // touched (they may be unwritten cache contents, e.g. NaN).
            const float pe = valid ? __expf(s - mn) : 0.f;
            al[h] = al[h] * alpha + pe;
#pragma unroll
            for (int e = 0; e < EPL; ++e) ao[h][e] = valid ? fmaf(pe, vv[e], ao[h][e] * alpha) : ao[h][e] * alpha;
            am[h] = mn;
        }
    };
    auto attn_finish = [&]() {
        if (c == 0 && is_last) attn_fold(kp, vp, lane < LPP);  // the position written this step
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float lsum = xgroup_sum<LPP>(al[h]);
            LDS float *dst = cst + (c * GQ + h) * (d + 2);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ov = xgroup_sum<LPP>(ao[h][e]);
                if (lane < LPP) dst[e0 + e] = ov;
            }
            if (lane == 0) { dst[d] = am[h]; dst[d + 1] = lsum; }
        }
    };
    auto kv_slot = [&](int n, int buf) {
        const LDS unsigned char *kb = ring + buf * MK_SLOT_BYTES;
        const LDS unsigned char *vb = kb + 8 * MK_CHUNK_BYTES;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int chunk = c * 2 + q;
            const int tpos = t0 + n * BP + chunk * PPC + lane / LPP;
            float kv[EPL], vv[EPL];
            piece_load<DT>(kb + chunk * MK_CHUNK_BYTES + lane * 16, kv);
            piece_load<DT>(vb + chunk * MK_CHUNK_BYTES + lane * 16, vv);
            attn_fold(kv, vv, tpos < t1);
        }
    };

    // ---- epilogues (consumer 0) ----
    auto epi_qkv = [&](int l) {
        const float inv = inv_rms(p.H);
        const int nq = p.nh * d, nk = p.nkv * d;
        const float *rope = p.rope + (size_t)P * d;  // [d/2][2]
        for (int u = lane; u < g.units[ST_QKV]; u += 64) {
            const int gr0 = (g.unit0[ST_QKV] + u) * 4;
            const float y0 = outv[u * 4] * inv, y1 = outv[u * 4 + 1] * inv;
            const float y2 = outv[u * 4 + 2] * inv, y3 = outv[u * 4 + 3] * inv;
            if (gr0 < nq + nk) {
                const bool isq = gr0 < nq;
                const int r = isq ? gr0 : gr0 - nq;
                const int head = r / d, m0 = (r % d) / 2;
                const float c0 = rope[2 * m0], s0 = rope[2 * m0 + 1];
                const float c1 = rope[2 * m0 + 2], s1 = rope[2 * m0 + 3];
                const float a0 = y0 * c0 - y1 * s0, b0 = y0 * s0 + y1 * c0;
                const float a1 = y2 * c1 - y3 * s1, b1 = y2 * s1 + y3 * c1;
                if (isq) {
                    float *qd = p.q + (size_t)head * d;
                    stc(qd + m0, a0);
                    stc(qd + m0 + 1, a1);
                    stc(qd + m0 + d / 2, b0);
                    stc(qd + m0 + 1 + d / 2, b1);
                } else {
                    unsigned char *row = (unsigned char *)p.kc + ((size_t)l * p.nkv + head) * head_bytes + (size_t)P * d * EB;
                    if constexpr (DT == 1) {
                        stcu((uint32_t *)(row + m0 * 2), f2bf(a0) | (f2bf(a1) << 16));
                        stcu((uint32_t *)(row + (m0 + d / 2) * 2), f2bf(b0) | (f2bf(b1) << 16));
                    } else {
                        stc((float *)row + m0, a0);
                        stc((float *)row + m0 + 1, a1);
                        stc((float *)row + m0 + d / 2, b0);
                        stc((float *)row + m0 + 1 + d / 2, b1);
                    }
                }
            } else if (gr0 < nq + 2 * nk) {
                const int r = gr0 - nq - nk;
                const int head = r / d, e = r % d;
                unsigned char *row = (unsigned char *)p.vc + ((size_t)l * p.nkv + head) * head_bytes + (size_t)P * d * EB;
                if constexpr (DT == 1) {
                    stcu((uint32_t *)(row + e * 2), f2bf(y0) | (f2bf(y1) << 16));
                    stcu((uint32_t *)(row + e * 2 + 4), f2bf(y2) | (f2bf(y3) << 16));
                } else {
                    stc((float *)row + e, y0);
                    stc((float *)row + e + 1, y1);
                    stc((float *)row + e + 2, y2);
                    stc((float *)row + e + 3, y3);
                }
            }
        }
    };
    auto epi_residual = [&](int st) {  // O or DOWN: x += out for the workgroup's rows
        for (int i = lane; i < g.units[st] * 4; i += 64) {
            const int r = g.unit0[st] * 4 + i;
            if (r < p.H) {
                const float xn = xown[i] + outv[i];
                xown[i] = xn;
                stc(p.x + r, xn);
            }
        }
    };
    auto epi_gu = [&]() {
        const float inv = inv_rms(p.H);
        for (int m = lane; m < g.units[ST_GU] * 2; m += 64) {
            const int f = g.unit0[ST_GU] * 2 + m;
            if (f < p.F) {
                const float gv = outv[2 * m] * inv, uv = outv[2 * m + 1] * inv;
                stc(p.a + f, gv / (1.0f + __expf(-gv)) * uv);
            }
        }
    };
    auto epi_attn = [&]() {
        if (!has_split) return;
        const int stride = d + 2;
        float *part = p.part + ((size_t)kvj * S + kvs) * GQ * stride;
        // merge the four consumers' states
        for (int h = 0; h < GQ; ++h) {
            float M = -INFINITY;
            for (int cc = 0; cc < MK_NUM_CONSUMERS; ++cc) M = fmaxf(M, cst[(cc * GQ + h) * stride + d]);
            float Lsum = 0.f;
            float wgt[MK_NUM_CONSUMERS];
            for (int cc = 0; cc < MK_NUM_CONSUMERS; ++cc) {
                const float mc = cst[(cc * GQ + h) * stride + d];
                wgt[cc] = (mc == -INFINITY) ? 0.f : __expf(mc - M);
                Lsum += wgt[cc] * cst[(cc * GQ + h) * stride + d + 1];
            }
            for (int e = lane; e < d; e += 64) {
                float o = 0.f;
                for (int cc = 0; cc < MK_NUM_CONSUMERS; ++cc) o = fmaf(wgt[cc], cst[(cc * GQ + h) * stride + e], o);
                stc(part + h * stride + e, o);
            }
            if (lane == 0) { stc(part + h * stride + d, M); stc(part + h * stride + d + 1, Lsum); }
        }
        MK_WAIT_VM0();
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(p.head_cnt + kvj, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old != (uint32_t)(S - 1)) return;
        // last arriver for this KV head: log-sum-exp merge of all splits
        MK_COMPILER_BARRIER();
        const float *pb = p.part + (size_t)kvj * S * GQ * stride;
        for (int h = 0; h < GQ; ++h) {
            float M = -INFINITY;
            for (int s = lane; s < S; s += 64) M = fmaxf(M, ldc(pb + ((size_t)s * GQ + h) * stride + d));
            M = wave_max(M);
            float Lsum = 0.f;
            float o0 = 0.f, o1 = 0.f;
            for (int s = 0; s < S; ++s) {
                const float *ps = pb + ((size_t)s * GQ + h) * stride;
                const float ms = ldc(ps + d);
                const float wgt = (ms == -INFINITY) ? 0.f : __expf(ms - M);
                Lsum = fmaf(wgt, ldc(ps + d + 1), Lsum);
                if (lane < d) o0 = fmaf(wgt, ldc(ps + lane), o0);
                if (lane + 64 < d) o1 = fmaf(wgt, ldc(ps + lane + 64), o1);
            }
            float *od = p.o + ((size_t)kvj * GQ + h) * d;
            const float invl = 1.0f / Lsum;
            if (lane < d) stc(od + lane, o0 * invl);
            if (lane + 64 < d) stc(od + lane + 64, o1 * invl);
        }
        if (lane == 0) stcu(p.head_cnt + kvj, 0u);
    };
    auto epi_lm = [&]() {
        const float inv = inv_rms(p.H);
        float best = -INFINITY;
        int besti = 0x7FFFFFFF;
        for (int i = lane; i < g.units[ST_LM] * 4; i += 64) {
            const int r = g.unit0[ST_LM] * 4 + i;
            if (r < p.V) {
                const float lg = outv[i] * inv;
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
        if (lane == 0) { stc(p.amax_val + w, best); stci(p.amax_idx + w, besti); }
        MK_WAIT_VM0();
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(p.amax_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old != (uint32_t)(G - 1)) return;
        MK_COMPILER_BARRIER();
        best = -INFINITY;
        besti = 0x7FFFFFFF;
        for (int i = lane; i < G; i += 64) {
            const float v = ldc(p.amax_val + i);
            const int ix = (int)ldcu((const uint32_t *)p.amax_idx + i);
            if (v > best || (v == best && ix < besti)) { best = v; besti = ix; }
        }
        for (int m = 1; m < 64; m <<= 1) {
            const float ob = __shfl_xor(best, m);
            const int oi = __shfl_xor(besti, m);
            if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
        }
        if (lane == 0) {
            p.token_out[0] = besti;
            stcu(p.amax_cnt, 0u);
        }
    };

    // ---- the program ----
    const int nq = p.nh * d;
    for (int l = 0; l < L && ok; ++l) {
        // stage boundary: [epilogue DOWN(l-1)] + prologue QKV(l)
        ok = barrier();
        if (!ok) break;
        if (l == 0) {
            int tok = p.token_dev ? p.token_dev[0] : p.token;
            if (tok < 0 || tok >= p.V) {
                if (ct == 0) stcu(p.err, ldcu(p.err) | MK_DEVERR_TOKEN);
                tok = 0;
            }
            const unsigned char *erow = (const unsigned char *)p.embed + (size_t)tok * p.H * EB;
            load_normed(nullptr, erow, p.g_attn, p.H, p.st[ST_QKV].rbp * EPC);
            for (int i = ct; i < g.units[ST_O] * 4; i += 256) {
                const int r = g.unit0[ST_O] * 4 + i;
                float xv = 0.f;
                if (r < p.H) {
                    if constexpr (DT == 1) xv = __uint_as_float((uint32_t)((const uint16_t *)erow)[r] << 16);
                    else xv = ((const float *)erow)[r];
                }
                xown[i] = xv;
            }
        } else {
            if (c == 0) {
                epi_residual(ST_DOWN);
                publish(5 * (l - 1) + 5);
            }
            if (!wait_all(5 * (l - 1) + 5)) ok = false;
            if (ok) load_normed(p.x, nullptr, p.g_attn + (size_t)l * p.H, p.H, p.st[ST_QKV].rbp * EPC);
        }
        gemv_begin();
        for (int n = 0; n < g.nsl[ST_QKV] && ok; ++n) {
            ok = barrier();
            if (ok) gemv_slot(ST_QKV, j % NS);
            ++j;
        }
        if (!ok) break;

        // stage boundary: epilogue QKV(l) + prologue attention(l)
        ok = barrier();
        if (!ok) break;
        if (c == 0) {
            epi_qkv(l);
            publish(5 * l + 1);
        }
        if (has_split) {
            if (!wait_all(5 * l + 1)) ok = false;
            if (ok) {
                const float *qb = p.q + (size_t)kvj * GQ * d;
#pragma unroll
                for (int h = 0; h < GQ; ++h)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) qr[h][e] = ldc(qb + h * d + e0 + e);
                if (c == 0 && is_last) {
                    const unsigned char *krow = (const unsigned char *)p.kc + ((size_t)l * p.nkv + kvj) * head_bytes + (size_t)P * d * EB;
                    const unsigned char *vrow = (const unsigned char *)p.vc + ((size_t)l * p.nkv + kvj) * head_bytes + (size_t)P * d * EB;
                    const int off = (lane < LPP ? lane : 0) * 16;
                    piece_load_dev<DT>(krow + off, kp);
                    piece_load_dev<DT>(vrow + off, vp);
                }
                attn_begin();
                if (nsl_kv == 0) attn_finish();
            }
        }
        for (int n = 0; n < nsl_kv && ok; ++n) {
            ok = barrier();
            if (ok) {
                kv_slot(n, j % NS);
                if (n == nsl_kv - 1) attn_finish();
            }
            ++j;
        }
        if (!ok) break;

        // stage boundary: epilogue attention(l) + prologue O(l)
        ok = barrier();
        if (!ok) break;
        if (c == 0) {
            epi_attn();
            publish(5 * l + 2);
        }
        if (!wait_all(5 * l + 2)) { ok = false; break; }
        load_plain(p.o, nq, p.st[ST_O].rbp * EPC);
        gemv_begin();
        for (int n = 0; n < g.nsl[ST_O] && ok; ++n) {
            ok = barrier();
            if (ok) gemv_slot(ST_O, j % NS);
            ++j;
        }
        if (!ok) break;

        // stage boundary: epilogue O(l) + prologue gate/up(l)
        ok = barrier();
        if (!ok) break;
        if (c == 0) {
            epi_residual(ST_O);
            publish(5 * l + 3);
        }
        if (!wait_all(5 * l + 3)) { ok = false; break; }
        load_normed(p.x, nullptr, p.g_ffn + (size_t)l * p.H, p.H, p.st[ST_GU].rbp * EPC);
        gemv_begin();
        for (int n = 0; n < g.nsl[ST_GU] && ok; ++n) {
            ok = barrier();
            if (ok) gemv_slot(ST_GU, j % NS);
            ++j;
        }
        if (!ok) break;

        // stage boundary: epilogue gate/up(l) + prologue down(l)
        ok = barrier();
        if (!ok) break;
        if (c == 0) {
            epi_gu();
            publish(5 * l + 4);
        }
        if (!wait_all(5 * l + 4)) { ok = false; break; }
        load_plain(p.a, p.F, p.st[ST_DOWN].rbp * EPC);
        gemv_begin();
        for (int n = 0; n < g.nsl[ST_DOWN] && ok; ++n) {
            ok = barrier();
            if (ok) gemv_slot(ST_DOWN, j % NS);
            ++j;
        }
        if (!ok) break;
    }
    if (ok && p.want_logits) {
        ok = barrier();
        if (ok) {
            if (c == 0) {
                epi_residual(ST_DOWN);
                publish(5 * (L - 1) + 5);
            }
            if (!wait_all(5 * (L - 1) + 5)) ok = false;
        }
        if (ok) load_normed(p.x, nullptr, p.g_final, p.H, p.st[ST_LM].rbp * EPC);
        gemv_begin();
        for (int n = 0; n < g.nsl[ST_LM] && ok; ++n) {
            ok = barrier();
            if (ok) gemv_slot(ST_LM, j % NS);
            ++j;
        }
        if (ok) {
            ok = barrier();
            if (ok && c == 0) epi_lm();
        }
    } else if (ok) {
        ok = barrier();
        if (ok && c == 0) {
            epi_residual(ST_DOWN);
            publish(5 * (L - 1) + 5);
        }
    }
    if (!ok) {
        // Aborted inside step `step` (ctl[1] == step): pass one more barrier,
        // after which the loaders see an abort from an earlier step and leave.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
    }
    MK_WAIT_VM0();
}

// ---- host-side launch ---------------------------------------------------
namespace {
typedef void (*KernelFn)(const MkParams);

template <int DT, int GQ, int LPP>
KernelFn kfn() { return mk_decode_kernel<DT, GQ, LPP>; }

KernelFn pick(int dtype, int gq, int lpp) {
#define MK_PICK(DT_, GQ_, LPP_) if (dtype == DT_ && gq == GQ_ && lpp == LPP_) return kfn<DT_, GQ_, LPP_>();
    MK_PICK(1, 1, 8) MK_PICK(1, 2, 8) MK_PICK(1, 4, 8) MK_PICK(1, 8, 8)
    MK_PICK(1, 1, 16) MK_PICK(1, 2, 16) MK_PICK(1, 4, 16) MK_PICK(1, 8, 16)
    MK_PICK(0, 1, 8) MK_PICK(0, 2, 8) MK_PICK(0, 4, 8) MK_PICK(0, 8, 8)
    MK_PICK(0, 1, 16) MK_PICK(0, 2, 16) MK_PICK(0, 4, 16) MK_PICK(0, 8, 16)
#undef MK_PICK
    return nullptr;
}
}  // namespace

extern "C" int mk_kernel_lds_bytes(int ring_slots, int vec_floats, int out_rows, int dtype, int d, int gq) {
    (void)dtype;
    const int floats = vec_floats + out_rows + MK_NUM_CONSUMERS * gq * (d + 2) + 64 + MK_NUM_CONSUMERS + 4;
    return ring_slots * MK_SLOT_BYTES + floats * 4;
}

extern "C" int mk_launch_decode(const MkParams *p, int dtype, int cooperative, void *stream) {
    const int eb = dtype ? 2 : 4;
    const int lpp = p->d * eb / 16;
    const int gq = p->nh / p->nkv;
    KernelFn fn = pick(dtype, gq, lpp);
    if (!fn) return (int)hipErrorInvalidValue;
    const int lds = mk_kernel_lds_bytes(p->ring_slots, p->lds_vec_floats, p->lds_out_rows, dtype, p->d, gq);
    hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return (int)e;
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
    KernelFn fn = pick(dtype, gq, lpp);
    if (!fn) return 0;
    if (hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)fn, MK_BLOCK_THREADS, lds) != hipSuccess)
        return 0;
    return n;
}
