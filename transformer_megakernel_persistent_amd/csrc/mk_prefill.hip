// Batched prefill: the prompt's positions processed T tokens at a time, so
// that every weight is read once per chunk instead of once per position, and
// the matrix products become dense contractions for the matrix cores.
//
// The pages keep prefill apart from the decode step and measure the two
// separately (cloud.baidu.com/article/9434380 section 八, question two); by
// definition under causal attention the cache after a prompt equals what n
// decode steps leave, which is what these kernels compute, in another order:
//
//   X = E[tokens]                                      [T][H] fp32
//   per layer:
//     A = split(rmsnorm(X, g_attn))                    bf16 hi + lo parts
//     Y = A . Wqkv^T                                   MFMA, packed QKV rows
//     rotate q, k; K, V rows of positions pos0..pos0+T-1 -> cache (bf16 RNE)
//     A = split(causal GQA attention of each token over positions 0..its own)
//     X += A . Wo^T
//     A = split(rmsnorm(X, g_ffn));  A' = split(silu(gate) * up) of
//       [gate; up] = A . [Wg;Wu]^T (in the GEMM's epilogue);  X += A' . Wd^T
//
// Numerics.  Weights are bf16, or int8 codes widened to bf16 (exact: an int8
// value has at most 8 significant bits) whose per-row scale multiplies the
// finished dot product; either way they enter the products exactly.  Activations
// are fp32; each is split into bf16 hi = rne(a) and lo = rne(a - hi), and a
// product is accumulated as W.hi + W.lo in fp32 by v_mfma_f32_16x16x32_bf16,
// so an activation keeps about 16 bits of mantissa (relative error below
// 2^-16) -- the decode step's activations are fp32 throughout; the cache
// rows agree with it to within the bf16 rounding of the stored values.  In
// the attention the queries and the probabilities are split the same way
// (with the probabilities rounded once to bf16, an 80-layer prefill's cache
// rows drift to several bf16 steps from the oracle's in the last layers).
//
// Weights are read in place from the decode kernel's packed layout (no
// second copy of the model): a GEMM loader lane finds the 16-byte piece
// holding consecutive inputs of a row (8 bf16 values, 16 int8 codes; 4-code
// words in the int8 down stage) from the row's owning workgroup, consumer
// and stream position (mk_stream_pos, mk_down_geo).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace {

constexpr int MK_PF_MAX_H = 16384;  // widest hidden size of the batched prefill

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bfloat16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f_to_bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---- embedding: X[t] = E[tok[t]] -----------------------------------------
__global__ __launch_bounds__(256) void pf_embed(float *X, const int32_t *tok, const uint16_t *E, int H) {
    const int t = blockIdx.x;
    const uint16_t *row = E + (size_t)tok[t] * H;
    for (int i = threadIdx.x; i < H; i += 256) X[(size_t)t * H + i] = bf_to_f(row[i]);
}

// ---- RMSNorm into the split operand ---------------------------------------
// One workgroup per token: h = g * x / sqrt(mean(x^2) + eps), written as
// bf16 hi and lo parts, zero-padded from H to kpad columns.
// Thread tid takes groups of 4 consecutive elements, 4 tid + 1024 k (H a
// multiple of 8, so a group is all inside or all past H; at most NI groups,
// H <= 1024 NI), kept in registers between the sum of squares and the
// stores of the hi and lo parts; the loads of x and g and the 8-byte stores
// are contiguous across the lanes.
template <int NI>
__global__ __launch_bounds__(256) void pf_norm_split(const float *X, const float *g, int H, float eps,
                                                     uint16_t *Ah, uint16_t *Al, int lda, int kpad) {
    __shared__ float red[8];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float *x = X + (size_t)t * H;
    f4v v[NI];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        const int i0 = 4 * tid + 1024 * k;
        v[k] = i0 < H ? *(const f4v *)(x + i0) : f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(v[k][e], v[k][e], ss);
    }
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        const int i0 = 4 * tid + 1024 * k;
        if (i0 >= kpad) break;
        const f4v gg = i0 < H ? *(const f4v *)(g + i0) : f4v{0.f, 0.f, 0.f, 0.f};
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            const float a = gg[e] * (v[k][e] * inv), b = gg[e + 1] * (v[k][e + 1] * inv);
            const uint16_t ha = f_to_bf(a), hb = f_to_bf(b);
            hw[e / 2] = ha | ((uint32_t)hb << 16);
            lw[e / 2] = f_to_bf(a - bf_to_f(ha)) | ((uint32_t)f_to_bf(b - bf_to_f(hb)) << 16);
        }
        *(u2v *)(Ah + (size_t)t * lda + i0) = u2v{hw[0], hw[1]};
        *(u2v *)(Al + (size_t)t * lda + i0) = u2v{lw[0], lw[1]};
    }
}

// ---- the packed weight layout, read by row ---------------------------------
// Owner workgroup of unit u among G workgroups holding U units (the w with
// floor(w U / G) <= u < floor((w + 1) U / G)).
__device__ __forceinline__ int unit_owner(int u, int U, int G) { return (int)(((int64_t)(u + 1) * G - 1) / U); }
__device__ __forceinline__ int unit_first(int w, int U, int G) { return (int)(((int64_t)w * U) / G); }

// Where packed row n of a row-split stage keeps its chunks: chunk kc of the
// row is at base + ((qq0 + kc*qs) / 4) * slot_stride + ((qq0 + kc*qs) % 4) * 1 KiB
// (the inverse of mk_stream_pos for the row's consumer stream).
struct RowLoc {
    const unsigned char *base;  // layer block + workgroup offset + consumer's 4 KiB of a slot
    int qq0, qs;
};
__device__ __forceinline__ RowLoc row_loc(const MkStage &st, const unsigned char *layer_block, int grid, int n,
                                          int eb) {
    const int U = st.units, u = n >> 2;
    const int w = unit_owner(u, U, grid);
    const int u0 = unit_first(w, U, grid), units = unit_first(w + 1, U, grid) - u0;
    const int i = n - 4 * u0, c = i & 3, rc = i >> 2;
    const int full = mk_row_groups(st.rbp, eb) ? units / 4 : 0;
    RowLoc r;
    r.base = layer_block + st.wg_off[w] + c * 4 * MK_CHUNK_BYTES;
    if (rc < full * 4) {
        r.qq0 = (rc >> 2) * 4 * st.rbp + (rc & 3);
        r.qs = 4;
    } else {
        r.qq0 = full * 4 * st.rbp + (rc - full * 4) * st.rbp;
        r.qs = 1;
    }
    return r;
}
// Element k of the row (eb bytes per element: 2 bf16, 1 int8).
__device__ __forceinline__ const unsigned char *row_piece(const RowLoc &r, int64_t slot_stride, int k, int eb) {
    const int epc = MK_CHUNK_BYTES / eb;  // elements per chunk
    const int kc = k / epc;
    const int qq = r.qq0 + kc * r.qs;
    return r.base + (int64_t)(qq >> 2) * slot_stride + (qq & 3) * MK_CHUNK_BYTES + (k % epc) * eb;
}
// The down stage (split along its input, piece columns): where output row n
// keeps inputs f .. f+7 (f a multiple of 8, the owning workgroup's first
// input a multiple of 8; a 16-byte piece holds 8 bf16 or 16 int8 inputs).
// e = dmap[f / 8] gives the owning workgroup's block offset, its pieces per
// row group, the piece and the byte offset inside it (mk_down_geo,
// tabulated by the host).  Output row n = 64 grp + r: with grp the same for
// a whole wave, everything but the row's 16-byte column r is wave-uniform.
__device__ __forceinline__ const unsigned char *down_piece(const MkStage &st, const unsigned char *layer_block,
                                                           const int4 e, int grp, int r) {
    const int c = grp & 3, gl = grp >> 2;
    const int qq = gl * e.y + e.z;
    return layer_block + e.x + (int64_t)(qq >> 2) * st.slot_stride + (c * 4 + (qq & 3)) * MK_CHUNK_BYTES + e.w +
           r * 16;
}

// Entry i of the down stage's map (int4 per block of 8 inputs), read at a
// wave-uniform index.
__device__ __forceinline__ int4 dmap4(const int32_t *__restrict__ dmap, int i) {
    return *(const int4 *)(dmap + 4 * i);
}

// INT8: the scale of output n of stage `kind` in one layer, read from the
// decode kernel's per-workgroup scale blocks (MkParams::scl): a block holds
// the workgroup's QKV, O and gate/up rows and then the down rows of its x
// rows (the O rows' indices), in local order.
struct ScaleIdx {
    const float *blk;  // the layer's blocks: [grid][sc_blk]
    int sc_blk, grid, uq, uo, ugu;
};
__device__ __forceinline__ float row_scale(const ScaleIdx &si, int kind, int n) {
    const int G = si.grid;
    auto first = [&](int w, int U) { return unit_first(w, U, G); };
    auto count = [&](int w, int U) { return unit_first(w + 1, U, G) - unit_first(w, U, G); };
    const int U = kind == ST_QKV ? si.uq : kind == ST_GU ? si.ugu : si.uo;  // O and down: the O rows' owner
    const int w = unit_owner(n >> 2, U, G);
    int off = n - 4 * first(w, U);
    if (kind != ST_QKV) off += 4 * count(w, si.uq);
    if (kind == ST_GU || kind == ST_DOWN) off += 4 * count(w, si.uo);
    if (kind == ST_DOWN) off += 4 * count(w, si.ugu);
    return si.blk[(size_t)w * si.sc_blk + off];
}

// The GEMM epilogue, per 64 x 64 block of a wave's products (the 128 x 256
// tiles' waves call it for each 64-column half) in the
// v_mfma_f32_16x16x32_bf16 result layout (acc[mb][nb]
// element i is C[m0 + wm*64 + mb*16 + 4*kg + i][n0 + wn*64 + nb*16 + r16]),
// stored, added to out, or (SWIGLU) turned into the down projection's
// operand.
template <bool ADD, bool Q8, bool SWIGLU>
__device__ __forceinline__ void gemm_store(const f4v (&acc)[4][4], int m0, int n0, int wm, int wn, int r16, int kg,
                                           int T, int N, float *out, int ldo, uint16_t *oh, uint16_t *ol,
                                           const ScaleIdx &si, int kind) {
    if constexpr (SWIGLU) {
        // gate/up rows interleave in the packed order (row 2f the gate, row
        // 2f + 1 the up projection of SwiGLU input f), so lane r16 ^ 1 holds
        // the partner of this lane's column: a = silu(gate) * up, split into
        // the down projection's bf16 hi + lo operand at [token][f]
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int n = n0 + wn * 64 + nb * 16 + r16;
            const float sc = Q8 && n < N ? row_scale(si, kind, n) : 1.0f;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = Q8 ? acc[mb][nb][i] * sc : acc[mb][nb][i];
                    const float up = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
                    const int m = m0 + wm * 64 + mb * 16 + 4 * kg + i;
                    if ((r16 & 1) == 0 && n < N && m < T) {
                        const float a = v / (1.0f + __expf(-v)) * up;
                        const uint16_t hi = f_to_bf(a);
                        const size_t idx = (size_t)m * ldo + (n >> 1);
                        oh[idx] = hi;
                        ol[idx] = f_to_bf(a - bf_to_f(hi));
                    }
                }
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int n = n0 + wn * 64 + nb * 16 + r16;
            if (n >= N) continue;
            const float sc = Q8 ? row_scale(si, kind, n) : 1.0f;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + wm * 64 + mb * 16 + 4 * kg + i;
                    if (m >= T) continue;
                    float *o = out + (size_t)m * ldo + n;
                    const float v = Q8 ? acc[mb][nb][i] * sc : acc[mb][nb][i];
                    if (ADD) *o += v;
                    else *o = v;
                }
        }
    }
}

// ---- GEMM: out[t][n] (=|+=) sum_k (Ah + Al)[t][k] * W[n][k] -----------------
// v_mfma_f32_16x16x32_bf16 operand layout (wave64): A[m][k] in lane
// m + 16 * (k / 8), element k % 8; B[k][n] in lane n + 16 * (k / 8); the
// result C[m][n] in lane n + 16 * (m / 4), element m % 4.
// B is taken in units of 8 consecutive inputs of one row: 16 bytes of bf16,
// or 8 int8 codes widened to bf16 (exact); Q8 multiplies each output
// column's sum by its row's scale.  Rows at or past N, tokens at or past T
// and inputs at or past K (a multiple of 32) enter as zeros.

// ---- GEMM with a load ring ---------------------------------------------------
// Organised like the decode kernel: 8 waves, 4 of them loaders that stream
// 32-input steps of A hi, A lo and B into a ring of LDS stages with
// direct-to-LDS loads, 4 of them multiplying (2 x 2).  The loads run NST - 1 steps ahead of the products,
// with one workgroup barrier per step, and no register holds an operand
// between its load and its LDS copy.
// Tile 128 tokens x BN outputs.  BN = 128: 6 stages of 24 KiB, waves of
// 64 x 64, fragments double-buffered (a wave reads step s + 1's fragments
// before it multiplies step s's).  BN = 256: 5 stages of 32 KiB, waves of
// 64 x 128; a third fewer operand bytes per product (A, the bf16 hi + lo
// pair, costs 4 bytes per element against B's 2), for GEMMs with enough
// output tiles to fill the chip.
// Stage layout: [row][32 inputs] for A hi, A lo and row-split B (64-byte
// rows, the four 16-byte pieces of row r at position piece ^ rg_swz(r), so
// that the 16 rows of one fragment read fall in distinct banks); the down
// stage's B as [8-input block][row] (its piece columns, 64 rows of one block
// contiguous in memory).  INT8 weights (Q8) stay codes in LDS, half the B
// bytes, widened when a fragment is read: row-split rows of 32 codes, their
// two 16-code halves at position half ^ ((r >> 3) & 1) (8-byte reads of 16
// rows in distinct banks); the down stage in 4-code words, [word][row], as
// its slices are aligned to 8 inputs only.  Rows past T or N and down
// inputs past F read a zeroed 1 KiB (zsrc).
constexpr int RG_BK = 32;
constexpr int RG_WIDE_MIN_TILES = 256;  // 128 x 256 tiles when they fill the 256 CUs once
constexpr int RG_SEC = 128 * RG_BK * 2;  // A hi (or A lo) of one step: 128 rows of 64 bytes
// Q8: B holds int8 codes (one byte per input), widened to bf16 when a
// fragment is read.
template <int BN, bool Q8, bool DOWN>
struct RgCfg {
    static constexpr int NST = BN == 256 && !Q8 ? 5 : 6;   // ring stages
    static constexpr int SECB = BN * RG_BK * (Q8 ? 1 : 2); // B of one step
    static constexpr int STAGE = 2 * RG_SEC + SECB;
    static constexpr int LDS = NST * STAGE;
    // B loads per loader wave and step: bf16, 16 rows (row split) or 64
    // rows of one 8-input block (down) per load; int8 row split, 32 rows of
    // 32 codes per load; int8 down, 64 rows of one 4-code block per load
    static constexpr int QB = !Q8 ? BN / 64 : DOWN ? BN / 32 : BN / 128;
    static constexpr int LOADS = 4 + QB;                   // direct-to-LDS loads per loader wave and step
    static constexpr int NB = BN / 32;                     // 16-output blocks per multiplying wave
};
template <int BN, bool Q8, bool DOWN>
constexpr bool rg_fits() {
    typedef RgCfg<BN, Q8, DOWN> C;
    return C::LDS <= MK_LDS_LIMIT && (C::NST - 2) <= 4 && (C::NST - 1) * C::LOADS < 64;
}
static_assert(rg_fits<128, false, false>() && rg_fits<128, false, true>() && rg_fits<256, false, false>() &&
                  rg_fits<256, false, true>() && rg_fits<128, true, false>() && rg_fits<128, true, true>() &&
                  rg_fits<256, true, false>() && rg_fits<256, true, true>(),
              "each ring fits the LDS, its steady-state waits are covered and its loads stay within the counter");
// eight int8 codes (two words, code e in byte e % 4 of word e / 4) -> eight
// bf16 values in the operand layout (value e in half e % 2 of word e / 2);
// exact: |code| <= 128
__device__ __forceinline__ u4v rg_widen8(uint32_t lo, uint32_t hi) {
    // the upper halves of the two floats, packed by one byte permute
    // (bytes 2, 3 of f0 then bytes 2, 3 of f1)
    auto pair = [](uint32_t w, int b) -> uint32_t {
        const float f0 = (float)(int8_t)(w >> (8 * b)), f1 = (float)(int8_t)(w >> (8 * b + 8));
        return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    };
    return u4v{pair(lo, 0), pair(lo, 2), pair(hi, 0), pair(hi, 2)};
}
__device__ __forceinline__ int rg_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void rg_wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
// n a multiple of L up to 4 L; anything else waits for every load
template <int L>
__device__ __forceinline__ void rg_wait_vm_rt(int n) {
    if (n == L) rg_wait_vm<L>();
    else if (n == 2 * L) rg_wait_vm<2 * L>();
    else if (n == 3 * L) rg_wait_vm<3 * L>();
    else if (n == 4 * L) rg_wait_vm<4 * L>();
    else rg_wait_vm<0>();
}

template <bool DOWN, bool ADD, bool SWIGLU, int BN, bool Q8>
__global__ __launch_bounds__(512, 1) void pf_gemm_ring(const MkStage st, const unsigned char *layer_block, int grid,
                                                       int F, const uint16_t *Ah, const uint16_t *Al, int lda, int T,
                                                       int K, int N, float *out, int ldo, uint16_t *oh, uint16_t *ol,
                                                       const int32_t *__restrict__ dmap,
                                                       const unsigned char *__restrict__ zsrc, float *part,
                                                       int ldp, const ScaleIdx si, int kind) {
    typedef RgCfg<BN, Q8, DOWN> C;
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    extern __shared__ __attribute__((aligned(16))) unsigned char rg_smem[];
    lds_u8 *ring = (lds_u8 *)rg_smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = blockIdx.y * 128, n0 = blockIdx.x * BN;
    // Split along the inputs (gridDim.z = 2): split 0 takes the first half
    // of the steps and stores (or adds) its sums to out as usual, split 1
    // the rest and stores its sums to part [T][ldp]; the sums of part are
    // then added in by pf_add_part or by the kernel that reads out next.
    // out (+ sums0) + sums1, in that order: deterministic.
    const int nall = K / RG_BK, kz = blockIdx.z;
    const int sbeg = kz ? nall / 2 : 0;
    const int nst = gridDim.z == 1 ? nall : kz ? nall - nall / 2 : nall / 2;

    if (wave < 4) {
        // ============================ loader ============================
        // Wave lw carries rows [32 lw, 32 lw + 32) of A hi and A lo and rows
        // [BN/4 lw, BN/4 (lw + 1)) of row-split B, 16 rows per load: lane l
        // takes row base + l / 4 and LDS position l % 4, i.e. the row's piece
        // (l % 4) ^ rg_swz(row).  Down stage: B block lw of every step, rows
        // 64 h + l.
        const int lw = wave;
        const unsigned char *zl = zsrc + lane * 16;
        const unsigned char *pah[2], *pal[2];
        int ja[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = 32 * lw + 16 * q + (lane >> 2);
            ja[q] = (lane & 3) ^ rg_swz(row);
            const int m = m0 + row;
            pah[q] = m < T ? (const unsigned char *)(Ah + (size_t)m * lda + 8 * ja[q]) : nullptr;
            pal[q] = m < T ? (const unsigned char *)(Al + (size_t)m * lda + 8 * ja[q]) : nullptr;
        }
        // B rows of this lane, per load q: bf16 row split, row (BN/4) lw +
        // 16 q + l / 4 and piece jb = (l % 4) ^ rg_swz(row); int8 row split,
        // row (BN/4) lw + 32 q + l / 2 and 16-code half jb = (l % 2) ^
        // ((row >> 3) & 1); down, row 64 (q % (BN/64)) + l
        constexpr int NQ = DOWN ? BN / 64 : C::QB;
        RowLoc rl[NQ];
        bool bok[NQ];
        int jb[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int row = Q8 ? (BN / 4) * lw + 32 * q + (lane >> 1) : (BN / 4) * lw + 16 * q + (lane >> 2);
            jb[q] = Q8 ? (lane & 1) ^ ((row >> 3) & 1) : (lane & 3) ^ rg_swz(row);
            const int n = DOWN ? n0 + 64 * q + lane : n0 + row;
            bok[q] = n < N;
            if constexpr (!DOWN) rl[q] = row_loc(st, layer_block, grid, bok[q] ? n : 0, Q8 ? 1 : 2);
        }
        // Row split: the address of each B row's current 1 KiB chunk, found
        // again only when a step enters the next chunk (every 16 steps for
        // bf16, 32 for int8; a step's 32 inputs never straddle two chunks, so
        // the chunk is wave-uniform); a load adds the step's offset inside
        // the chunk and the lane's piece.  Issued in increasing step order.
        constexpr int EB = Q8 ? 1 : 2, EPC = MK_CHUNK_BYTES / EB;  // bytes per element, elements per chunk
        const unsigned char *bch[NQ];
        int kc_cur = -1;
        auto issue = [&](int s) {
            lds_u8 *base = ring + (s % C::NST) * C::STAGE;
            const int k0 = (sbeg + s) * RG_BK;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                lds_u8 *dst = base + (32 * lw + 16 * q) * (RG_BK * 2);
                __builtin_amdgcn_global_load_lds((const void *)(pah[q] ? pah[q] + 2 * k0 : zl),
                                                 (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
                __builtin_amdgcn_global_load_lds((const void *)(pal[q] ? pal[q] + 2 * k0 : zl),
                                                 (__attribute__((address_space(3))) void *)(dst + RG_SEC), 16, 0, 0);
            }
            if constexpr (DOWN && Q8) {
                // 4-code blocks 2 lw and 2 lw + 1 of the step (8-input block
                // lw): LDS [4-code block][row], 4 bytes per row
                const int f = k0 + 8 * lw;  // wave-uniform
                const int4 e = f < F ? dmap4(dmap, f >> 3) : int4{0, 0, 0, 0};
#pragma unroll
                for (int h = 0; h < BN / 64; ++h) {
                    const unsigned char *src = f < F && bok[h] ? down_piece(st, layer_block, e, (n0 >> 6) + h, lane) : zl;
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        __builtin_amdgcn_global_load_lds(
                            (const void *)(src == zl ? zl : src + 4 * b),
                            (__attribute__((address_space(3))) void *)(base + 2 * RG_SEC + (2 * lw + b) * (BN * 4) +
                                                                       h * 256),
                            4, 0, 0);
                }
            } else if constexpr (DOWN) {
                const int f = k0 + 8 * lw;  // this wave's block of the step (wave-uniform)
                const int4 e = f < F ? dmap4(dmap, f >> 3) : int4{0, 0, 0, 0};
#pragma unroll
                for (int h = 0; h < C::QB; ++h) {
                    const unsigned char *src = f < F && bok[h] ? down_piece(st, layer_block, e, (n0 >> 6) + h, lane) : zl;
                    __builtin_amdgcn_global_load_lds(
                        (const void *)src,
                        (__attribute__((address_space(3))) void *)(base + 2 * RG_SEC + lw * (BN * 16) + h * 1024), 16, 0,
                        0);
                }
            } else {
                const int kc = k0 / EPC;  // wave-uniform
                if (kc != kc_cur) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) bch[q] = row_piece(rl[q], st.slot_stride, kc * EPC, EB);
                    kc_cur = kc;
                }
                const int ko = (k0 % EPC) * EB;  // the step's first input, bytes into the chunk
                // the lane's piece: inputs 8 jb (bf16) or 16 jb (int8) of the step
#pragma unroll
                for (int q = 0; q < C::QB; ++q) {
                    const unsigned char *src = bok[q] ? bch[q] + ko + 16 * jb[q] : zl;
                    const int row0 = Q8 ? (BN / 4) * lw + 32 * q : (BN / 4) * lw + 16 * q;  // first LDS row of the load
                    __builtin_amdgcn_global_load_lds(
                        (const void *)src,
                        (__attribute__((address_space(3))) void *)(base + 2 * RG_SEC + row0 * (RG_BK * EB)), 16, 0, 0);
                }
            }
        };
        // Step s is in stage s % NST.  Before barrier s a loader waits until
        // its loads of step s have landed (loads of later steps may still be
        // in flight); after it, every multiplying wave has read step s - 1
        // into registers, so that stage takes step s + NST - 1.
        const int pro = nst < C::NST - 1 ? nst : C::NST - 1;
        for (int s = 0; s < pro; ++s) issue(s);
        int issued = pro;
        for (int s = 0; s < nst; ++s) {
            rg_wait_vm_rt<C::LOADS>((issued - 1 - s) * C::LOADS);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (issued < nst) {
                issue(issued);
                ++issued;
            }
        }
        rg_wait_vm<0>();
        return;
    }

    // ============================ products ============================
    const int c = wave - 4, wm = c >> 1, wn = c & 1;
    const int r16 = lane & 15, kg = lane >> 4;
    int aoff[4], boff[C::NB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = wm * 64 + i * 16 + r16;
        aoff[i] = ra * (RG_BK * 2) + ((kg ^ rg_swz(ra)) << 4);
    }
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
        // B fragment of row rb, inputs 8 kg .. 8 kg + 7 of the step (int8
        // down: the first of its two 4-code words; the second is BN * 4 on)
        const int rb = wn * (BN / 2) + i * 16 + r16;
        if constexpr (Q8 && DOWN) boff[i] = 2 * RG_SEC + 2 * kg * (BN * 4) + rb * 4;
        else if constexpr (Q8) boff[i] = 2 * RG_SEC + rb * RG_BK + ((((kg >> 1) ^ ((rb >> 3) & 1)) << 4) | ((kg & 1) << 3));
        else boff[i] = 2 * RG_SEC + (DOWN ? kg * (BN * 16) + rb * 16 : rb * (RG_BK * 2) + ((kg ^ rg_swz(rb)) << 4));
    }
    f4v acc[4][C::NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f4v{0.f, 0.f, 0.f, 0.f};
    auto step_barrier = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    constexpr int NX = BN == 128 ? 2 : 1;  // fragment buffers
    u4v fh[NX][4], fl[NX][4], fb[NX][C::NB];
    auto read_step = [&](int sb, int x) {
        const lds_u8 *base = ring + sb * C::STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fh[x][i] = *(const __attribute__((address_space(3))) u4v *)(base + aoff[i]);
            fl[x][i] = *(const __attribute__((address_space(3))) u4v *)(base + RG_SEC + aoff[i]);
        }
#pragma unroll
        for (int i = 0; i < C::NB; ++i) {
            if constexpr (Q8 && DOWN)
                fb[x][i] = rg_widen8(*(const __attribute__((address_space(3))) uint32_t *)(base + boff[i]),
                                     *(const __attribute__((address_space(3))) uint32_t *)(base + boff[i] + BN * 4));
            else if constexpr (Q8) {
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                const u2v c = *(const __attribute__((address_space(3))) u2v *)(base + boff[i]);
                fb[x][i] = rg_widen8(c.x, c.y);
            } else
                fb[x][i] = *(const __attribute__((address_space(3))) u4v *)(base + boff[i]);
        }
    };
    auto products = [&](int x) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, fh[x][mb]),
                                                                      __builtin_bit_cast(bf8v, fb[x][nb]), acc[mb][nb], 0, 0, 0);
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, fl[x][mb]),
                                                                      __builtin_bit_cast(bf8v, fb[x][nb]), acc[mb][nb], 0, 0, 0);
            }
    };
    if constexpr (NX == 2) {
        // double-buffered: after barrier s + 1 read step s + 1, then multiply
        // step s (barrier s + 1 also frees step s's stage for the loaders)
        step_barrier();
        read_step(0, 0);
        int sb = 1;  // stage of step s + 1
        for (int s = 0; s + 1 < nst; s += 2) {
            step_barrier();
            read_step(sb, 1);
            sb = sb + 1 == C::NST ? 0 : sb + 1;
            products(0);
            if (s + 2 < nst) {
                step_barrier();
                read_step(sb, 0);
                sb = sb + 1 == C::NST ? 0 : sb + 1;
            }
            products(1);
        }
        if (nst & 1) products(0);  // the last step of an odd count
    } else {
        // 64 x 128 per wave: one set of fragments (a second one, or reading
        // the next step's A fragments as each block row finishes, measured
        // slower: 238 VGPRs and hazards on the matrix-core sources)
        int sb = 0;
        for (int s = 0; s < nst; ++s) {
            step_barrier();
            read_step(sb, 0);
            sb = sb + 1 == C::NST ? 0 : sb + 1;
            products(0);
        }
    }
#pragma unroll
    for (int h = 0; h < C::NB / 4; ++h) {
        f4v sub[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) sub[mb][nb] = acc[mb][4 * h + nb];
        // columns n0 + wn * BN/2 + 64 h + nb * 16 + r16
        if (kz == 0)
            gemm_store<ADD, Q8, SWIGLU>(sub, m0, n0 + wn * (BN / 2) + 64 * h, wm, 0, r16, kg, T, N, out, ldo, oh, ol, si,
                                        kind);
        else
            gemm_store<false, Q8, false>(sub, m0, n0 + wn * (BN / 2) + 64 * h, wm, 0, r16, kg, T, N, part, ldp, nullptr,
                                         nullptr, si, kind);
    }
}

// out[t][n] += part[t][n] (the second input split of a ring GEMM)
__global__ __launch_bounds__(256) void pf_add_part(float *out, int ldo, const float *part, int ldp, int N) {
    const int t = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
    if (n < N) out[(size_t)t * ldo + n] += part[(size_t)t * ldp + n];
}

// ---- rotary encoding and the cache rows of the chunk ------------------------
// Y holds each token's packed QKV rows (query and key heads with the rotary
// partners m and m + d/2 at packed rows 2m', 2m'+1, then value rows in
// order).  Thread j of token t handles query/key pair j, or value element
// j - (nh + nkv) * d / 2.
// poff > 0: the QKV GEMM ran as two input splits and left the second
// one's sums at columns [poff, poff + nqkv) of Y, added here as Y is read.
__global__ __launch_bounds__(256) void pf_rope_kv(const float *Y, int ldy, int poff, int pos0, const float *rope,
                                                  int nh, int nkv, int d, int layer, int max_seq, uint16_t *kc,
                                                  uint16_t *vc, float *Q) {
    const int t = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
    const int npair = (nh + nkv) * d / 2, nv = nkv * d;
    if (j >= npair + nv) return;
    const float *y = Y + (size_t)t * ldy;
    const int pos = pos0 + t, nq = nh * d;
    if (j < npair) {
        const int gr = 2 * j;
        const bool isq = gr < nq;
        const int r = isq ? gr : gr - nq;
        const int head = r / d, m = (r % d) / 2;
        const float c = rope[((size_t)pos * (d / 2) + m) * 2], s = rope[((size_t)pos * (d / 2) + m) * 2 + 1];
        const float y0 = poff ? y[gr] + y[poff + gr] : y[gr], y1 = poff ? y[gr + 1] + y[poff + gr + 1] : y[gr + 1];
        const float a = y0 * c - y1 * s, b = y0 * s + y1 * c;
        if (isq) {
            Q[((size_t)t * nh + head) * d + m] = a;
            Q[((size_t)t * nh + head) * d + m + d / 2] = b;
        } else {
            uint16_t *row = kc + (((size_t)layer * nkv + head) * max_seq + pos) * d;
            row[m] = f_to_bf(a);
            row[m + d / 2] = f_to_bf(b);
        }
    } else {
        const int r = j - npair;
        const int head = r / d, e = r % d;
        const int cv = nq + nkv * d + r;
        vc[(((size_t)layer * nkv + head) * max_seq + pos) * d + e] = f_to_bf(poff ? y[cv] + y[poff + cv] : y[cv]);
    }
}

// ---- causal GQA attention of the chunk on the matrix cores -----------------
// bf16 hi + lo parts of two floats, packed in pairs (v_cvt_pk_bf16_f32
// rounds to nearest even): hi = rne(a), lo = rne(a - hi)
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 h = {(__bf16)a, (__bf16)b};
    hi = __builtin_bit_cast(uint32_t, h);
    const bf2 l = {(__bf16)(a - __uint_as_float(hi << 16)), (__bf16)(b - __uint_as_float(hi & 0xFFFF0000u))};
    lo = __builtin_bit_cast(uint32_t, l);
}
// Max over the four lanes l, l^16, l^32, l^48 (the gfx950 permlane swaps
// exchange 16-lane rows 0<->1, 2<->3 and 0<->2, 1<->3).
__device__ __forceinline__ float cross4_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Column of position p (0..63) of a block in the transposed V tile.  With
// p = 32 a + 16 h + 4 g + i (i < 4) the column is 32 a + 8 g + 4 h + i: the
// eight columns 32 a + 8 g ... + 7 that one lane of the P V product reads
// as its operand (k-step a, lane group g) then hold positions 4 g + i of the
// score tiles 2 a and 2 a + 1, the positions that same lane holds in S.
__device__ __forceinline__ int vt_col(int p) {
    return (p & 32) | (((p >> 2) & 3) << 3) | (((p >> 4) & 1) << 2) | (p & 3);
}

// Workgroup (query block, KV head j): 64 RB query rows -- QB = 64 RB / GQ
// tokens x the GQ heads of group j, row m = token (m / GQ), head (m % GQ)
// -- against blocks of 64 cached positions staged in LDS (K as [pos][dim],
// V transposed to [dim][vt_col(pos)]); the next block's K and V are loaded
// into registers while the current one is multiplied.  Wave w owns the RB
// 16-row blocks 16 (w RB + r) ...  Per position block and row block, with
// v_mfma_f32_16x16x32_bf16 and the query rows as the N dimension:
//   S^T = K Q^T (Q split into bf16 hi + lo, K exact; Q carries the factor
//   log2(e) / sqrt(d), so that exp2 of a score is exp of the scaled score);
//   in the result layout lane l holds positions 4 (l / 16) + i (i < 4) of
//   each 16-position tile for the single query row l % 16, so a row's
//   running max is one lane's, completed over the four lanes l % 16 + 16 k
//   by two lane swaps (only when the reference moves).  Positions past
//   each row's own are masked (only blocks that reach past the workgroup's
//   first token need it); P =
//   exp2(S - m) for a reference m that moves only when a block's max
//   passes it by more than 8;
//   O^T += V^T P^T (V exact, P split into hi + lo), with 16 rows of ones
//   after V^T so that one more output tile holds the row sums of P.  The
//   positions of V^T's columns are permuted within each block (vt_col), so
//   that the operand of the P V product is in each lane already: its own
//   eight scores of score tiles 2 k2 and 2 k2 + 1.
// Masked scores are -inf, so exp2 makes them 0; rows past the chunk's last
// token attend everything and are never written.  The result o / l goes to
// the split operand.
template <int D, int GQ, int RB>
__global__ __launch_bounds__(256) void pf_attn_mfma(const float *Q, const uint16_t *kc, const uint16_t *vc, int layer,
                                                    int nh, int nkv, int max_seq, int pos0, int T, uint16_t *Ah,
                                                    uint16_t *Al, int lda) {
    constexpr int QB = 64 * RB / GQ;  // tokens per workgroup
    constexpr int KS = D / 32;        // k-steps of S^T = K Q^T
    constexpr int NT = D / 16;        // output tiles (16 dims each) per row block
    constexpr int BP = 64;            // positions per block
    constexpr int PPT = BP * D / 8 / 256;  // 16-byte K (and V) pieces per thread and block
    // rows padded by 16 bytes, so that the 16 rows one fragment read touches
    // (lanes l % 16) fall in different banks
    constexpr int LK = D + 8, LV = BP + 8;
    __shared__ __attribute__((aligned(16))) uint16_t ks[BP * LK];  // [pos][dim]
    // [dim][pos], then 16 rows of ones: the products with them are the row
    // sums of P (output tile NT), from the same hi + lo parts as o
    __shared__ __attribute__((aligned(16))) uint16_t vt[(D + 16) * LV];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // One-dimensional grid, KV head fastest: workgroup w runs on XCD w mod 8,
    // so with 8 KV heads each head's K/V stream stays in one XCD's L2; the
    // query blocks go last-first, so the longest causal ranges start first.
    const int nqb = (T + QB - 1) / QB;
    const int j = (int)blockIdx.x % nkv, t_base = (nqb - 1 - (int)blockIdx.x / nkv) * QB;
    const int r16 = lane & 15, kg = lane >> 4;
    const float scale = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)
    // query row of this lane in row block r: m = 16 (wv RB + r) + r16
    u4v qh[RB][KS], ql[RB][KS];
    int plast[RB];
    float mrun[RB];
    f4v o[RB][NT + 1];  // tile NT: the row sum of P
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int m = (wv * RB + r) * 16 + r16, t = t_base + m / GQ, g = m % GQ;
        const bool tv = t < T;
        const float *qp = Q + ((size_t)(tv ? t : 0) * nh + j * GQ + g) * D + 8 * kg;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2)
                split2(tv ? qp[32 * k + e] * scale : 0.f, tv ? qp[32 * k + e + 1] * scale : 0.f, hw[e / 2], lw[e / 2]);
            qh[r][k] = u4v{hw[0], hw[1], hw[2], hw[3]};
            ql[r][k] = u4v{lw[0], lw[1], lw[2], lw[3]};
        }
        plast[r] = tv ? pos0 + t : 0x7FFFFFFF;
        mrun[r] = 0.f;  // set by the first block
#pragma unroll
        for (int n = 0; n <= NT; ++n) o[r][n] = f4v{0.f, 0.f, 0.f, 0.f};
    }
    for (int i = tid; i < 16 * LV; i += 256) vt[D * LV + i] = 0x3F80;  // bf16 1.0 (the staging never writes these rows)
    const int t_last = min(T, t_base + QB) - 1;
    const int n_pos = pos0 + t_last + 1;  // positions the workgroup needs
    const uint16_t *kbase = kc + ((size_t)layer * nkv + j) * max_seq * D;
    const uint16_t *vbase = vc + ((size_t)layer * nkv + j) * max_seq * D;
    // K piece i of a block: row i / (D / 8), 16-byte column i % (D / 8).  V
    // pieces 2 u and 2 u + 1 of a thread: positions 2 pp and 2 pp + 1 of
    // the same 16-byte column vcp (pair i = tid + 256 u: pp = i % 32, vcp =
    // i / 32), so that each transposed LDS word holds two neighbouring
    // positions of one dimension (32 lanes write 32 neighbouring words)
    u4v kr[PPT], vr[PPT];
    auto fetch = [&](int p0) {
        const int nb = min(BP, n_pos - p0);
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int i = tid + 256 * u;
            const int krow = i / (D / 8), kcp = i % (D / 8);
            kr[u] = krow < nb ? *(const u4v *)(kbase + (size_t)(p0 + krow) * D + 8 * kcp) : u4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < PPT / 2; ++u) {
            const int i = tid + 256 * u, pp = i % (BP / 2), vcp = i / (BP / 2);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int vrow = 2 * pp + h;
                vr[2 * u + h] = vrow < nb ? *(const u4v *)(vbase + (size_t)(p0 + vrow) * D + 8 * vcp) : u4v{0u, 0u, 0u, 0u};
            }
        }
    };
    fetch(0);
    for (int p0 = 0; p0 < n_pos; p0 += BP) {
        __syncthreads();  // the previous block's K and V are consumed
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            const int i = tid + 256 * u;
            *(u4v *)(ks + (i / (D / 8)) * LK + 8 * (i % (D / 8))) = kr[u];
        }
#pragma unroll
        for (int u = 0; u < PPT / 2; ++u) {
            const int i = tid + 256 * u, pp = i % (BP / 2), vcp = i / (BP / 2), col = vt_col(2 * pp);
            const uint32_t a4[4] = {vr[2 * u].x, vr[2 * u].y, vr[2 * u].z, vr[2 * u].w};
            const uint32_t b4[4] = {vr[2 * u + 1].x, vr[2 * u + 1].y, vr[2 * u + 1].z, vr[2 * u + 1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // dimension 8 vcp + e at positions 2 pp (low half) and 2 pp + 1,
                // which vt_col keeps in neighbouring columns
                const uint32_t lo = (a4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, hi = (b4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                *(uint32_t *)(vt + (8 * vcp + e) * LV + col) = lo | (hi << 16);
            }
        }
        __syncthreads();
        if (p0 + BP < n_pos) fetch(p0 + BP);
        const bool diag = p0 + BP - 1 > pos0 + t_base;  // uniform
        const bool first = p0 == 0;                     // uniform
        // the block's K fragments: read once for two row blocks, in place for one
        u4v kf[4][KS];
        if constexpr (RB > 1) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int k = 0; k < KS; ++k) kf[nt][k] = *(const u4v *)(ks + (nt * 16 + r16) * LK + 32 * k + 8 * kg);
        }
        auto kfrag = [&](int nt, int k) -> u4v {
            if constexpr (RB > 1) return kf[nt][k];
            else return *(const u4v *)(ks + (nt * 16 + r16) * LK + 32 * k + 8 * kg);
        };
        // S^T - m of row block r, tile nt: lane holds positions 16 nt + 4 kg
        // + i of row r16 (the accumulators start at minus the row's running
        // max, so the products land already shifted for exp2)
        f4v sc[RB][4];
        auto qk_tile = [&](int r, int nt) {
            const float nm = -mrun[r];
            sc[r][nt] = f4v{nm, nm, nm, nm};
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const u4v ak = kfrag(nt, k);
                sc[r][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, ak),
                                                                    __builtin_bit_cast(bf8v, qh[r][k]), sc[r][nt], 0, 0, 0);
                sc[r][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, ak),
                                                                    __builtin_bit_cast(bf8v, ql[r][k]), sc[r][nt], 0, 0, 0);
            }
        };
        // Masking and lazy rescaling of row block r: the reference m moves
        // only when a row's block max passes it by more than 8 (log2 units),
        // so P stays at most 2^8; o / l is unchanged, and most blocks skip
        // the rescaling (a wave-uniform branch).  Some lane's share of a row
        // passes the reference by more than 8 exactly when the row's block
        // max does, so the row max over the four lanes is needed only inside
        // the branch.  The first block sets m to its max (every row has an
        // unmasked position there: position 0), with o and l still 0; later
        // a fully masked row (-inf) keeps its m.
        auto prep = [&](int r) {
            if (diag) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (p0 + nt * 16 + 4 * kg + i > plast[r]) sc[r][nt][i] = -INFINITY;
            }
            float mx = sc[r][0][0];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[r][nt][i]);
            if (first || __builtin_amdgcn_ballot_w64(mx > 8.0f) != 0) {
                const float bm = cross4_max(mx);  // block max minus m
                const float dm = first ? bm : fmaxf(bm, 0.f);  // m's move (0 for rows that keep theirs)
                const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-dm);
                mrun[r] += dm;
#pragma unroll
                for (int n = 0; n <= NT; ++n) o[r][n] *= alpha;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[r][nt][i] -= dm;
            }
        };
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) qk_tile(0, nt);
        prep(0);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            // P of each tile as bf16 hi / lo pairs (positions 4 kg + 0,1 and 2,3).
            // With a next row block, its score products of tile nt go first
            // and this block's exponentials of tile nt after them, fenced in
            // that order, so that the vector work issues while the matrix
            // cores run (1B, 32768 tokens: attention 116.6 -> 110.7 ms).
            uint32_t ph[4][2], pl[4][2];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                if (r + 1 < RB) {
                    qk_tile(r + 1, nt);
                    __builtin_amdgcn_sched_barrier(0);
                }
                float pe[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) pe[i] = __builtin_amdgcn_exp2f(sc[r][nt][i]);
                split2(pe[0], pe[1], ph[nt][0], pl[nt][0]);
                split2(pe[2], pe[3], ph[nt][1], pl[nt][1]);
                if (r + 1 < RB) __builtin_amdgcn_sched_barrier(0);
            }
            // O^T += V^T P^T: two 32-position k-steps, k-step k2 over the
            // columns that hold score tiles 2 k2 and 2 k2 + 1
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const u4v bp = u4v{ph[2 * k2][0], ph[2 * k2][1], ph[2 * k2 + 1][0], ph[2 * k2 + 1][1]};
                const u4v bq = u4v{pl[2 * k2][0], pl[2 * k2][1], pl[2 * k2 + 1][0], pl[2 * k2 + 1][1]};
#pragma unroll
                for (int n = 0; n <= NT; ++n) {
                    const u4v av = *(const u4v *)(vt + (n * 16 + r16) * LV + 32 * k2 + 8 * kg);
                    o[r][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, av),
                                                                      __builtin_bit_cast(bf8v, bp), o[r][n], 0, 0, 0);
                    o[r][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, av),
                                                                      __builtin_bit_cast(bf8v, bq), o[r][n], 0, 0, 0);
                }
            }
            if (r + 1 < RB) prep(r + 1);
        }
    }
    // o / l into the split operand: lane holds dims 16 n + 4 kg + i of its
    // row, and the whole row sum in tile NT
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const float l = o[r][NT][0];
        const int m = (wv * RB + r) * 16 + r16, t = t_base + m / GQ, g = m % GQ;
        if (t >= T) continue;
        const float inv = 1.0f / l;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            uint32_t hw[2], lw[2];
            split2(o[r][n][0] * inv, o[r][n][1] * inv, hw[0], lw[0]);
            split2(o[r][n][2] * inv, o[r][n][3] * inv, hw[1], lw[1]);
            const size_t idx = (size_t)t * lda + (size_t)(j * GQ + g) * D + n * 16 + 4 * kg;
            *(uint2 *)(Ah + idx) = uint2{hw[0], hw[1]};
            *(uint2 *)(Al + idx) = uint2{lw[0], lw[1]};
        }
    }
}

// ---- zero padding of the down projection's operand ------------------------
// Columns [F, kpad) of the SwiGLU operand (the gate/up GEMM writes [0, F)),
// when F is not a multiple of 32.
__global__ __launch_bounds__(64) void pf_zero_cols(uint16_t *Ah, uint16_t *Al, int lda, int F, int kpad) {
    const int t = blockIdx.x, f = F + (int)threadIdx.x;
    if (f < kpad) {
        Ah[(size_t)t * lda + f] = 0;
        Al[(size_t)t * lda + f] = 0;
    }
}

template <int D, int GQ>
void launch_attn(hipStream_t s, const float *Q, const uint16_t *kc, const uint16_t *vc, int layer, int nh, int nkv,
                 int max_seq, int pos0, int T, uint16_t *Ah, uint16_t *Al, int lda) {
    // Two 16-row blocks per wave halve the K/V fragment reads from LDS per
    // query row; for 64-dim heads that pays once the causal ranges are long
    // (a 32768-token prompt: 259 -> 246 ms of attention), while for short
    // prompts the longest query block's chain of position blocks sets the
    // time and one row block per wave is faster (1B, 2048 tokens: 17.4
    // against 18.4 ms).  For 128-dim heads two row blocks need more than 256
    // VGPRs (occupancy 1) and one is faster (an 8B-shaped 16384-token
    // prompt: 22.8 against 17.1 ms of attention).
    if constexpr (D == 64) {
        if (pos0 + T > 8192) {
            constexpr int QB = 64 * 2 / GQ;
            hipLaunchKernelGGL((pf_attn_mfma<D, GQ, 2>), dim3((T + QB - 1) / QB * nkv), dim3(256), 0, s, Q, kc, vc, layer,
                               nh, nkv, max_seq, pos0, T, Ah, Al, lda);
            return;
        }
    }
    constexpr int QB = 64 / GQ;
    hipLaunchKernelGGL((pf_attn_mfma<D, GQ, 1>), dim3((T + QB - 1) / QB * nkv), dim3(256), 0, s, Q, kc, vc, layer, nh,
                       nkv, max_seq, pos0, T, Ah, Al, lda);
}

int round32(int k) { return (k + 31) & ~31; }

// One GEMM of the chunk: bf16 or int8 weights of stage `kind`, N outputs
// per token; workgroups cover 128 tokens x 128 outputs.  SWIGLU: the
// outputs are gate/up rows and the epilogue writes the down projection's
// split operand (oh, ol with leading dimension ldo) instead of out.
// RMSNorm of T rows into the split operand, columns [0, round32(H)); H <=
// MK_PF_MAX_H (mk_prefill_supported)
void launch_norm_split(hipStream_t s, int T, const float *X, const float *g, int H, float eps, uint16_t *Ah,
                       uint16_t *Al, int lda) {
    const int kpad = round32(H), groups = (kpad + 1023) / 1024;
    if (groups <= 2)
        hipLaunchKernelGGL(pf_norm_split<2>, dim3(T), dim3(256), 0, s, X, g, H, eps, Ah, Al, lda, kpad);
    else if (groups <= 4)
        hipLaunchKernelGGL(pf_norm_split<4>, dim3(T), dim3(256), 0, s, X, g, H, eps, Ah, Al, lda, kpad);
    else if (groups <= 8)
        hipLaunchKernelGGL(pf_norm_split<8>, dim3(T), dim3(256), 0, s, X, g, H, eps, Ah, Al, lda, kpad);
    else
        hipLaunchKernelGGL(pf_norm_split<16>, dim3(T), dim3(256), 0, s, X, g, H, eps, Ah, Al, lda, kpad);
}

template <bool DOWN, bool ADD, bool SWIGLU, int BN, bool Q8>
void launch_ring(hipStream_t s, dim3 g, const MkStage &st, const unsigned char *blk, int grid, int F,
                 const uint16_t *Ah, const uint16_t *Al, int lda, int T, int K, int N, float *out, int ldo,
                 uint16_t *oh, uint16_t *ol, const int32_t *dmap, const unsigned char *zsrc, float *part, int ldp,
                 const ScaleIdx &si, int kind) {
    constexpr int lds = RgCfg<BN, Q8, DOWN>::LDS;  // above the default dynamic limit
    (void)hipFuncSetAttribute((const void *)pf_gemm_ring<DOWN, ADD, SWIGLU, BN, Q8>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    hipLaunchKernelGGL((pf_gemm_ring<DOWN, ADD, SWIGLU, BN, Q8>), g, dim3(512), lds, s, st, blk, grid, F, Ah, Al, lda, T,
                       K, N, out, ldo, oh, ol, dmap, zsrc, part, ldp, si, kind);
}

// Returns whether the GEMM ran as two input splits.  part (nullable) [T][ldp]
// takes the second split's sums; with add_part they are added to out here,
// else the caller adds them (the QKV sums, in the RoPE kernel).
template <bool DOWN, bool ADD, bool SWIGLU = false>
bool launch_gemm(bool q8, hipStream_t s, const MkStage &st, const unsigned char *blk, int grid, int F,
                 const uint16_t *Ah, const uint16_t *Al, int lda, int T, int K, int N, float *out, int ldo,
                 uint16_t *oh, uint16_t *ol, const ScaleIdx &si, int kind, const int32_t *dmap,
                 const unsigned char *zsrc, float *part, int ldp, bool add_part) {
    const int mt = (T + 127) / 128;
    const int64_t wide = (int64_t)((N + 255) / 256) * mt, narrow = (int64_t)((N + 127) / 128) * mt;
    const bool use_wide = wide >= RG_WIDE_MIN_TILES;
    const int64_t tiles = use_wide ? wide : narrow;
    auto rounds = [](int64_t n) { return (n + RG_WIDE_MIN_TILES - 1) / RG_WIDE_MIN_TILES; };
    // Two input splits (never for SwiGLU, whose epilogue needs whole sums):
    // an adding GEMM whose wide tiles fill half the chip and whose inputs
    // run long (the 1B down projection: twice the workgroups at a third
    // fewer operand bytes per product; at 2048 inputs, the 1B O projection,
    // the halves are too short to pay for the extra pass over the sums), or
    // any GEMM whose last round of tiles would leave CUs idle where twice
    // the tiles at half the length finish in fewer full-length rounds (384
    // tiles: 2 rounds against 3 half rounds; the 1B and 8B QKV products).
    const bool split_wide = ADD && wide * 2 >= RG_WIDE_MIN_TILES && wide < RG_WIDE_MIN_TILES && K >= 4096;
    const bool split_tail = tiles > RG_WIDE_MIN_TILES && rounds(2 * tiles) < 2 * rounds(tiles) && K >= 2048;
    const bool split = !SWIGLU && part && (split_wide || split_tail);
    const bool wide_tiles = use_wide || split_wide;
    const dim3 g(wide_tiles ? (N + 255) / 256 : (N + 127) / 128, mt, split ? 2 : 1);
    if (wide_tiles) {
        // 128 x 256 tiles: fewer operand bytes per product, when there are
        // enough of them for every CU
        if (q8)
            launch_ring<DOWN, ADD, SWIGLU, 256, true>(s, g, st, blk, grid, F, Ah, Al, lda, T, K, N, out, ldo, oh, ol, dmap,
                                                      zsrc, part, ldp, si, kind);
        else
            launch_ring<DOWN, ADD, SWIGLU, 256, false>(s, g, st, blk, grid, F, Ah, Al, lda, T, K, N, out, ldo, oh, ol,
                                                       dmap, zsrc, part, ldp, si, kind);
    } else {
        if (q8)
            launch_ring<DOWN, ADD, SWIGLU, 128, true>(s, g, st, blk, grid, F, Ah, Al, lda, T, K, N, out, ldo, oh, ol, dmap,
                                                      zsrc, part, ldp, si, kind);
        else
            launch_ring<DOWN, ADD, SWIGLU, 128, false>(s, g, st, blk, grid, F, Ah, Al, lda, T, K, N, out, ldo, oh, ol,
                                                       dmap, zsrc, part, ldp, si, kind);
    }
    if (split && add_part)
        hipLaunchKernelGGL(pf_add_part, dim3((N + 255) / 256, T), dim3(256), 0, s, out, ldo, (const float *)part, ldp, N);
    return split;
}

}  // namespace

// Token-parallel work for positions [pos0, pos0 + T) of prompt tokens
// tok (device, T ids): fills their cache rows in every layer.  Buffers are
// the handle's (see MkPrefillBufs).  Requires a bf16 or weight-only INT8
// model (p->scl set) whose down-stage workgroups own inputs starting at
// multiples of 8 (mk_prefill_supported).
extern "C" int mk_prefill_chunk(const MkParams *p, const MkPrefillBufs *b, int T, int pos0, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    const int L = p->L, H = p->H, nh = p->nh, nkv = p->nkv, d = p->d, F = p->F, G = p->grid;
    const int gq = nh / nkv;
    const int nqkv = (nh + 2 * nkv) * d, nq = nh * d;
    uint16_t *kc = (uint16_t *)p->kc, *vc = (uint16_t *)p->vc;
    const int lda = b->lda, ldy = b->ldy;
    const bool q8 = p->scl != nullptr;
    ScaleIdx si = {nullptr, p->sc_blk, G, p->st[ST_QKV].units, p->st[ST_O].units, p->st[ST_GU].units};
    hipLaunchKernelGGL(pf_embed, dim3(T), dim3(256), 0, s, b->X, b->tok, (const uint16_t *)p->embed, H);
    for (int l = 0; l < L; ++l) {
        const unsigned char *blk[ST_NUM];
        for (int k = 0; k < ST_LM; ++k) blk[k] = p->packed + p->st[k].base + (int64_t)l * p->st[k].layer_stride;
        if (q8) si.blk = p->scl + (size_t)l * G * p->sc_blk;
        // attention half
        launch_norm_split(s, T, b->X, p->g_attn + (size_t)l * H, H, p->eps, b->Ah, b->Al, lda);
        // an input split of the QKV product leaves its second half's sums in
        // Y's spare columns [nqkv, 2 nqkv), added by the RoPE kernel
        float *qkv_part = 2 * nqkv <= ldy ? b->Y + nqkv : nullptr;
        const bool qkv_split = launch_gemm<false, false>(q8, s, p->st[ST_QKV], blk[ST_QKV], G, F, b->Ah, b->Al, lda, T,
                                                         round32(H), nqkv, b->Y, ldy, nullptr, nullptr, si, ST_QKV,
                                                         b->dmap, p->packed, qkv_part, ldy, false);
        const int nthr = (nh + nkv) * d / 2 + nkv * d;
        hipLaunchKernelGGL(pf_rope_kv, dim3((nthr + 255) / 256, T), dim3(256), 0, s, b->Y, ldy, qkv_split ? nqkv : 0,
                           pos0, p->rope, nh, nkv, d, l, p->max_seq, kc, vc, b->Q);
        {
#define MK_PF_ATTN(D_, GQ_) \
    if (d == D_ && gq == GQ_) launch_attn<D_, GQ_>(s, b->Q, kc, vc, l, nh, nkv, p->max_seq, pos0, T, b->Ah, b->Al, lda);
            MK_PF_ATTN(64, 1) MK_PF_ATTN(64, 2) MK_PF_ATTN(64, 4) MK_PF_ATTN(64, 8)
            MK_PF_ATTN(128, 1) MK_PF_ATTN(128, 2) MK_PF_ATTN(128, 4) MK_PF_ATTN(128, 8)
#undef MK_PF_ATTN
        }
        launch_gemm<false, true>(q8, s, p->st[ST_O], blk[ST_O], G, F, b->Ah, b->Al, lda, T, round32(nq), H, b->X, H,
                                 nullptr, nullptr, si, ST_O, b->dmap, p->packed, b->Q, H, true);
        // feed-forward half
        launch_norm_split(s, T, b->X, p->g_ffn + (size_t)l * H, H, p->eps, b->Ah, b->Al, lda);
        // gate/up with SwiGLU in the epilogue: the down projection's split
        // operand goes to the Y buffer (free until the next layer's QKV; it
        // holds T x 2F floats, the operand 2 x T x round32(F) bf16 values)
        const int ldf = round32(F);
        uint16_t *Fh = (uint16_t *)b->Y, *Fl = Fh + (size_t)T * ldf;
        launch_gemm<false, false, true>(q8, s, p->st[ST_GU], blk[ST_GU], G, F, b->Ah, b->Al, lda, T, round32(H),
                                        2 * F, nullptr, ldf, Fh, Fl, si, ST_GU, b->dmap, p->packed, nullptr, 0, false);
        if (ldf != F) hipLaunchKernelGGL(pf_zero_cols, dim3(T), dim3(64), 0, s, Fh, Fl, ldf, F, ldf);
        launch_gemm<true, true>(q8, s, p->st[ST_DOWN], blk[ST_DOWN], G, F, Fh, Fl, ldf, T, ldf, H, b->X, H, nullptr,
                                nullptr, si, ST_DOWN, b->dmap, p->packed, b->Q, H, true);
    }
    return (int)hipGetLastError();
}

// Whether the batched prefill applies to a handle's geometry: bf16 or INT8
// weights (a bf16 cache), head_dim 64 or 128, hidden at most MK_PF_MAX_H,
// FFN width 16 or more, and every down-stage workgroup's first input a
// multiple of 8 (8 consecutive inputs of a row, the unit a GEMM loader lane
// fetches, then lie in one 16-byte piece of its piece columns).
extern "C" int mk_prefill_supported(const MkParams *p, int dtype) {
    if ((dtype != 1 && dtype != 2) || (p->d != 64 && p->d != 128)) return 0;
    if (p->H > MK_PF_MAX_H) return 0;  // the RMSNorm split keeps a row in registers
    // the SwiGLU operand (2 x round32(F) bf16 values per token) lives in the
    // gate/up output buffer (2F floats per token)
    if (round32(p->F) > 2 * p->F) return 0;
    const int U = p->st[ST_DOWN].units;
    for (int w = 0; w < p->grid; ++w) {
        const MkDownGeo dg = mk_down_geo(w, p->grid, U, p->F, p->H, dtype == 2 ? 16 : 8);
        if (dg.f0 % 8 != 0) return 0;
    }
    return 1;
}
