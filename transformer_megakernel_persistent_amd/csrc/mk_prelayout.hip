// Weight pre-layout: copies row-major [out][in] weights into the order the
// decode kernel streams them, once, when a handle is created
// (cloud.baidu.com/article/9434380 section 九: arrange weights in an
// access-friendly order ahead of time instead of reordering at run time).
//
// Packed row order per stage (four consecutive packed rows form a "unit"):
//   QKV : query heads, then key heads, then value heads.  Within a query or
//         key head the rows are paired for rotary encoding: packed rows 2m and
//         2m+1 are head dims m and m + head_dim/2, so a unit holds head dims
//         {2e, 2e+1, 2e + d/2, 2e+1 + d/2}: two complete rotation pairs and
//         two adjacent storage words of the cache row.  Value rows keep their
//         natural order.
//   GU  : gate row f and up row f interleaved (packed rows 2f, 2f+1), so a
//         workgroup owns both halves of every SwiGLU product it emits.
//   O, LM: natural row order.
// The workgroups' slots are striped: slot n of workgroup w lies at
// wg_off[w] + n * slot_stride (wg_off[w] = w * 16 KiB, slot_stride = grid *
// 16 KiB).  Slot n holds for consumer c the 4 KiB of its row
// stream at [4n, 4n+4) chunks; consumer c's rows are local rows c, c+4, ...,
// and rows of 8, 12, ... chunks are interleaved in groups of four (see
// mk_stream_pos) so that one slot carries the same chunk of four rows.
//   DOWN: split along the input instead (see mk_down_geo): workgroup w's block
//         holds the Wd columns of its SwiGLU outputs as piece columns, lane i
//         of a piece column carrying 16 bytes of one output row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace {

// A 16-byte piece assembled byte by byte in registers (no private array):
// byte_at(i) returns byte i of the piece, or a negative value for a zero.
template <class F>
__device__ __forceinline__ uint4 gather_piece(F &&byte_at) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int b = byte_at(i);
        if (b >= 0) w[i >> 2] |= (uint32_t)b << (8 * (i & 3));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One 64-lane wave copies one 1 KiB chunk (16 bytes per lane).
__global__ __launch_bounds__(256) void prelayout_kernel(unsigned char *dst_block, MkStage st, int grid, int kind,
                                                        int eb, const unsigned char *src0, const unsigned char *src1,
                                                        const unsigned char *src2, int nh, int nkv, int d) {
    const int w = blockIdx.y;
    const int U = st.units;
    const int unit0 = (int)(((int64_t)w * U) / grid);
    const int units = (int)(((int64_t)(w + 1) * U) / grid) - unit0;
    const int chunk = blockIdx.x * 4 + (threadIdx.x >> 6);  // chunk index within this workgroup's block
    const int lane = threadIdx.x & 63;
    const int slot = chunk / MK_CHUNKS_PER_SLOT, cc = chunk % MK_CHUNKS_PER_SLOT;
    const int c = cc / 4, qi = cc % 4;
    const int qq = slot * 4 + qi;          // position in consumer c's chunk stream
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kind == ST_DOWN) {
        const MkDownGeo dg = mk_down_geo(w, grid, U, st.k, st.rows, 16 / eb);
        if (chunk >= dg.nsl * MK_CHUNKS_PER_SLOT) return;
        const int grp = c + 4 * (qq / (dg.kp > 0 ? dg.kp : 1)), q = qq % (dg.kp > 0 ? dg.kp : 1);
        const int row = grp * 64 + lane;
        const int epl = 16 / eb;
        if (dg.kp > 0 && row < st.rows) {
            const int fa = dg.f0 + q * epl;  // first column of this piece
            const unsigned char *srow = src0 + (int64_t)row * st.k * eb;
            // byte i of the piece: element i / eb of the piece, byte i % eb of it
            val = gather_piece([&](int i) -> int {
                const int e = i / eb;
                return q * epl + e < dg.nf ? (int)srow[(int64_t)(fa + e) * eb + i % eb] : -1;
            });
        }
        *(uint4 *)(dst_block + st.wg_off[w] + (int64_t)(chunk / MK_CHUNKS_PER_SLOT) * st.slot_stride +
                   (chunk % MK_CHUNKS_PER_SLOT) * MK_CHUNK_BYTES + lane * 16) = val;
        return;
    }
    const int nsl = (units * st.rbp + 3) / 4;
    if (chunk >= nsl * MK_CHUNKS_PER_SLOT) return;
    int row_c, kc;
    mk_stream_pos(qq, units, st.rbp, eb, row_c, kc);
    if (row_c < units) {
        const int gr = (unit0 + row_c) * 4 + c;  // packed row
        if (gr < st.rows) {
            const unsigned char *src = nullptr;
            int64_t srow = 0;
            if (kind == ST_QKV) {
                const int nq = nh * d, nk = nkv * d;
                if (gr < nq + nk) {
                    const int r = gr < nq ? gr : gr - nq;
                    const int head = r / d, wi = r % d;
                    srow = (int64_t)head * d + wi / 2 + (wi % 2) * (d / 2);
                    src = gr < nq ? src0 : src1;
                } else {
                    srow = gr - nq - nk;
                    src = src2;
                }
            } else if (kind == ST_GU) {
                srow = gr / 2;
                src = (gr % 2 == 0) ? src0 : src1;
            } else {
                srow = gr;
                src = src0;
            }
            const int64_t row_bytes = (int64_t)st.k * eb;
            const int64_t off = (int64_t)kc * MK_CHUNK_BYTES + lane * 16;
            if (off + 16 <= row_bytes) {
                val = *(const uint4 *)(src + srow * row_bytes + off);
            } else if (off < row_bytes) {  // partial 16-byte piece at the row end
                const unsigned char *sp = src + srow * row_bytes + off;
                const int nb = (int)(row_bytes - off);
                val = gather_piece([&](int i) -> int { return i < nb ? (int)sp[i] : -1; });
            }
        }
    }
    *(uint4 *)(dst_block + st.wg_off[w] + (int64_t)(chunk / MK_CHUNKS_PER_SLOT) * st.slot_stride +
               (chunk % MK_CHUNKS_PER_SLOT) * MK_CHUNK_BYTES + lane * 16) = val;
}

// Per-row scales of the INT8 matrices, one block per workgroup (layout in
// MkParams::scl): the rows of each stage in the order the workgroup's
// epilogues index them.  One workgroup of threads per block.
__global__ __launch_bounds__(256) void prelayout_scales_kernel(float *scl, const MkParams p, int layer,
                                                               const float *s_q, const float *s_k, const float *s_v,
                                                               const float *s_o, const float *s_g, const float *s_u,
                                                               const float *s_d) {
    const int w = blockIdx.x, G = p.grid;
    auto unit0 = [&](int k) { return (int)(((int64_t)w * p.st[k].units) / G); };
    auto nunits = [&](int k) { return (int)(((int64_t)(w + 1) * p.st[k].units) / G) - unit0(k); };
    if (layer == p.L) {
        float *dst = scl + (size_t)p.L * G * p.sc_blk + (size_t)w * p.sc_lm;
        const int n = nunits(ST_LM) * 4, r0 = unit0(ST_LM) * 4;
        for (int i = threadIdx.x; i < p.sc_lm; i += blockDim.x) dst[i] = (i < n && r0 + i < p.V) ? s_q[r0 + i] : 0.f;
        return;
    }
    float *dst = scl + ((size_t)layer * G + w) * p.sc_blk;
    const int nq = nunits(ST_QKV) * 4, no = nunits(ST_O) * 4, ng = nunits(ST_GU) * 4;
    const int nqd = p.nh * p.d, nk = p.nkv * p.d, d = p.d;
    for (int i = threadIdx.x; i < p.sc_blk; i += blockDim.x) {
        float v = 0.f;
        if (i < nq) {
            const int gr = unit0(ST_QKV) * 4 + i;  // packed QKV row
            if (gr < nqd + nk) {
                const int r = gr < nqd ? gr : gr - nqd;
                const int head = r / d, wi = r % d;
                const int srow = head * d + wi / 2 + (wi % 2) * (d / 2);  // rotary pairing of the packed rows
                v = gr < nqd ? s_q[srow] : s_k[srow];
            } else if (gr < nqd + 2 * nk) {
                v = s_v[gr - nqd - nk];
            }
        } else if (i < nq + no) {
            const int r = unit0(ST_O) * 4 + i - nq;
            if (r < p.H) v = s_o[r];
        } else if (i < nq + no + ng) {
            const int gr = unit0(ST_GU) * 4 + i - nq - no;  // gate and up rows interleaved
            if (gr < 2 * p.F) v = (gr % 2 == 0) ? s_g[gr / 2] : s_u[gr / 2];
        } else if (i < nq + 2 * no + ng) {
            const int r = unit0(ST_O) * 4 + i - nq - no - ng;  // the x rows this workgroup reduces
            if (r < p.H) v = s_d[r];
        }
        dst[i] = v;
    }
}

__global__ void to_f32_kernel(float *dst, const void *src, int64_t n, int dtype) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        if (dtype == 1) dst[i] = __uint_as_float((uint32_t)((const uint16_t *)src)[i] << 16);
        else dst[i] = ((const float *)src)[i];
    }
}

__global__ void zero_kernel(uint4 *dst, int64_t n16) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

// Clears `bytes` (a multiple of 16) at dst with a fill kernel on `stream`
// (a kernel rather than a memset so that the call can sit in a captured
// graph).
extern "C" int mk_launch_zero(void *dst, int64_t bytes, void *stream) {
    const int64_t n16 = bytes / 16;
    if (n16 <= 0) return 0;
    int blocks = (int)((n16 + 255) / 256);
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4 *)dst, n16);
    return (int)hipGetLastError();
}

extern "C" int mk_launch_prelayout_scales(float *scl, const MkParams *p, int layer, const float *const *src,
                                          void *stream) {
    const bool head = layer == p->L;
    hipLaunchKernelGGL(prelayout_scales_kernel, dim3(p->grid), dim3(256), 0, (hipStream_t)stream, scl, *p, layer,
                       src[0], head ? nullptr : src[1], head ? nullptr : src[2], head ? nullptr : src[3],
                       head ? nullptr : src[4], head ? nullptr : src[5], head ? nullptr : src[6]);
    return (int)hipGetLastError();
}

// eb: bytes per weight element (4 float32, 2 bfloat16, 1 int8)
extern "C" int mk_launch_prelayout_stage(unsigned char *dst, const MkStage *st, int grid, int kind, int eb,
                                         const void *src0, const void *src1, const void *src2, int nh, int nkv,
                                         int d, void *stream) {
    // the largest per-workgroup slot count bounds the x-extent of the launch
    int max_nsl = 0;
    for (int w = 0; w < grid; ++w) {
        const int U = st->units;
        const int u0 = (int)(((int64_t)w * U) / grid), u1 = (int)(((int64_t)(w + 1) * U) / grid);
        const int nsl = kind == ST_DOWN ? mk_down_geo(w, grid, U, st->k, st->rows, 16 / eb).nsl
                                        : ((u1 - u0) * st->rbp + 3) / 4;
        if (nsl > max_nsl) max_nsl = nsl;
    }
    if (max_nsl == 0) return 0;
    dim3 g((max_nsl * MK_CHUNKS_PER_SLOT + 3) / 4, grid);
    hipLaunchKernelGGL(prelayout_kernel, g, dim3(256), 0, (hipStream_t)stream, dst, *st, grid, kind, eb,
                       (const unsigned char *)src0, (const unsigned char *)src1, (const unsigned char *)src2, nh, nkv, d);
    return (int)hipGetLastError();
}

extern "C" int mk_launch_to_f32(float *dst, const void *src, int64_t n, int dtype, void *stream) {
    if (n <= 0) return 0;
    int blocks = (int)((n + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(to_f32_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, dst, src, n, dtype);
    return (int)hipGetLastError();
}
