// Causal softmax attention on the gathered sub-sequence (stage (iii) of
// Sec. 3; Eq. (1) of Sec. 3.1 with scale 1/sqrt(d) and the lower-triangular
// mask) and its gradient, on gfx950.  The same kernels run at full length for
// the dense comparison.
//
// MFMA layout: v_mfma_f32_16x16x32_{f16,bf16}.  A lane l works on column l%16
// of a 16x16 output tile and supplies 8 elements of the contraction to each
// operand; which 8 is irrelevant as long as both operands use the same
// assignment, so lane group g = l/16 holds contraction indices kappa(g, e).
// Scores are computed transposed (S^T = K Q^T, one query per lane column) so
// the online-softmax statistics of a query live in the lanes that own its
// output column (O^T = V^T P^T).  Operands whose contraction index is the
// sequence position come from [H][d][Sp] transposed copies whose blocks of 32
// positions are stored in fragment order, so every operand load is one
// contiguous 16-byte vector.
//
// Precision: the pooled sub-sequence is not representable in 16 bits, and
// the backward's dS = P o (dP - D) cancels heavily on heavy-tailed inputs, so
// every product uses split operands x = hi + lo:
//   * fp16 hi/lo (22 significant bits) for Q K^T, P V, dO V^T and P^T dO;
//     stored operands carry a per-head power-of-two scale so fp16 never
//     overflows; P lies in [0, 1];
//   * bf16 hi/lo for dS^T Q (dS may be large; bf16 has the fp32 range);
//   * fp16 hi/lo of dS scaled per query row by a power of two for dS K.
// Each split product is hi*hi + hi*lo + lo*hi (lo*lo is below fp32
// rounding).  When the stored operands are exact in 16 bits (the dense path
// on bf16 inputs) the lo parts of stored operands are zero and skipped.
//
// fp32 path: one wavefront per row, double-precision arithmetic.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// forward: the softmax reference maximum lags the row maximum by up to this
// much (log2 units); P then lies in [0, 2^8], still split exactly into fp16 hi/lo
constexpr float kLazyMax = 8.0f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 ld_f16x8(const uint16_t* p) {
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 ld_b16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f32x4 mma_h(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_b(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split 8 fp32 values (two f32x4 holding elements 0..3 and 4..7) into fp16 hi/lo.
__device__ __forceinline__ void split_h(const f32x4& a, const f32x4& b, f16x8& hi, f16x8& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const _Float16 h0 = (_Float16)a[e], h1 = (_Float16)b[e];
        hi[e] = h0;
        hi[4 + e] = h1;
        lo[e] = (_Float16)(a[e] - (float)h0);
        lo[4 + e] = (_Float16)(b[e] - (float)h1);
    }
}
__device__ __forceinline__ uint16_t bf16_rne(float f) { return (uint16_t)f32_to_bf16_bits(f); }
__device__ __forceinline__ void split_b(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
    u32x4 wh, wl;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const uint16_t a0 = bf16_rne(a[2 * e]), a1 = bf16_rne(a[2 * e + 1]);
        const uint16_t b0 = bf16_rne(b[2 * e]), b1 = bf16_rne(b[2 * e + 1]);
        wh[e] = (uint32_t)a0 | ((uint32_t)a1 << 16);
        wh[2 + e] = (uint32_t)b0 | ((uint32_t)b1 << 16);
        wl[e] = (uint32_t)bf16_rne(a[2 * e] - bf16_lo(a0)) | ((uint32_t)bf16_rne(a[2 * e + 1] - bf16_lo(a1)) << 16);
        wl[2 + e] = (uint32_t)bf16_rne(b[2 * e] - bf16_lo(b0)) | ((uint32_t)bf16_rne(b[2 * e + 1] - bf16_lo(b1)) << 16);
    }
    hi = __builtin_bit_cast(bf16x8, wh);
    lo = __builtin_bit_cast(bf16x8, wl);
}

// Operand tensors of one attention problem (all [H][rows][d] row-major or
// [H][d][Sp] transposed, 2-byte elements; lo pointers unused when !SPLIT).
struct AttnK {
    const uint16_t *qh, *ql, *kh, *kl, *vh, *vl, *doh, *dol;   // fp16 rows
    const uint16_t *vTh, *vTl, *kTh, *kTl, *doTh, *doTl;       // fp16 transposed
    const uint16_t *qTbh, *qTbl;                               // bf16 transposed (unscaled)
    const float* hscale;    // [H][4]: true value = stored * hscale (q, k, v, dO)
    float* o;               // fp32 [H][Sp][d] sub-sequence output, or null
    uint16_t* o_bf16;       // bf16 output with strides ld_o/hs_o (dense), or null
    float *lse, *lse2;      // [H][Sp]: natural and base-2 log-sum-exp
    const float* D;         // [H][Sp]
    const float* rowdown;   // [H][Sp]: power-of-two down-scale of dS rows (dq kernel)
    float *dq, *dk, *dv;    // fp32 [H][Sp][d] gradients, or
    uint16_t *dq_b, *dk_b, *dv_b;   // bf16 gradients with strides ld_o/hs_o
    const uint8_t* level;           // [H][rows]
    int p;
    uint16_t *o_tok, *dq_tok, *dk_tok, *dv_tok;   // or null: bf16 token rows [N][H][d], tok_ld apart
    const int32_t* start;                         // [H][rows]: first token of each entry
    int64_t tok_ld;
    int64_t rows, Sp, ld_o, hs_o;
    float scale;            // 1/sqrt(d)
    // fp32 path (double arithmetic)
    const float *qf, *kf, *vf, *dof;
};

// ------------------------------------------------------------ LDS tiles
// Streamed operands move through double-buffered LDS in blocks of kBN
// sequence positions, shared by the 4 wavefronts of a workgroup.  Row tiles
// hold kBN rows of d elements; transposed tiles hold d rows of kBN elements.
// 16-byte slots are XOR-swizzled by row so a fragment read is free of LDS
// bank conflicts.
constexpr int kBN = 32;

template <int D>
struct Tiles {
    static constexpr int NSLOT = D / 8;              // 16-byte slots per row-tile row
    static constexpr int ROW = kBN * D;              // elements of a row tile
    static constexpr int TR = D * kBN;               // elements of a transposed tile
    static constexpr int CH_ROW = kBN * NSLOT / 256; // 16-byte chunks per thread
    static constexpr int CH_T = D * 4 / 256;
};

__device__ __forceinline__ int swz_row(int r, int slot, int nslot) { return slot ^ (r & (nslot - 1)); }
// Transposed tiles have 64-byte rows (4 slots).  A ds_read_b128 of rows
// r0..r0+15 (r0 a multiple of 16) at one slot per 16-lane group runs at the
// full 256 B/clk on gfx950 with this XOR (measured; (r >> 2) & 3 and no
// swizzle both run at half rate).
__device__ __forceinline__ int swz_t(int r, int slot) { return slot ^ ((r >> 1) & 3); }

// global [rows][D] (head base `g`, first row r0) -> registers
template <int D>
__device__ __forceinline__ void fetch_row(const uint16_t* g, int64_t r0, u32x4 (&reg)[Tiles<D>::CH_ROW]) {
    constexpr int NSLOT = Tiles<D>::NSLOT;
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_ROW; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int r = c / NSLOT, slot = c % NSLOT;
        reg[i] = *reinterpret_cast<const u32x4*>(g + (r0 + r) * D + swz_row(r, slot, NSLOT) * 8);
    }
}
template <int D>
__device__ __forceinline__ void store_row(uint16_t* lds, const u32x4 (&reg)[Tiles<D>::CH_ROW]) {
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_ROW; ++i) {
        const int c = threadIdx.x + 256 * i;
        *reinterpret_cast<u32x4*>(lds + c * 8) = reg[i];
    }
}
// global transposed [D][Sp] (head base `g`), columns c0..c0+kBN-1 -> registers
template <int D>
__device__ __forceinline__ void fetch_t(const uint16_t* g, int64_t Sp, int64_t c0, u32x4 (&reg)[Tiles<D>::CH_T]) {
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_T; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int r = c / 4, slot = c % 4;
        reg[i] = *reinterpret_cast<const u32x4*>(g + (int64_t)r * Sp + c0 + swz_t(r, slot) * 8);
    }
}
template <int D>
__device__ __forceinline__ void store_t(uint16_t* lds, const u32x4 (&reg)[Tiles<D>::CH_T]) {
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_T; ++i) {
        const int c = threadIdx.x + 256 * i;
        *reinterpret_cast<u32x4*>(lds + c * 8) = reg[i];
    }
}
// Direct global -> LDS copies of the same tiles (no staging registers): thread
// c fetches the 16-byte chunk that fetch_row / fetch_t would give it, and the
// load writes it at wave base + 16 * lane, i.e. at chunk c of the LDS tile.
// The data is in LDS once the issuing wave's vmcnt has drained.
#define LH_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
template <int D>
__device__ __forceinline__ void dma_row(const uint16_t* g, int64_t r0, uint16_t* lds) {
    constexpr int NSLOT = Tiles<D>::NSLOT;
    const int wbase = threadIdx.x & ~63;
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_ROW; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int r = c / NSLOT, slot = c % NSLOT;
        __builtin_amdgcn_global_load_lds(g + (r0 + r) * D + swz_row(r, slot, NSLOT) * 8,
                                         LH_LDS_PTR(lds + (256 * i + wbase) * 8), 16, 0, 0);
    }
}
template <int D>
__device__ __forceinline__ void dma_t(const uint16_t* g, int64_t Sp, int64_t c0, uint16_t* lds) {
    const int wbase = threadIdx.x & ~63;
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_T; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int r = c / 4, slot = c % 4;
        __builtin_amdgcn_global_load_lds(g + (int64_t)r * Sp + c0 + swz_t(r, slot) * 8,
                                         LH_LDS_PTR(lds + (256 * i + wbase) * 8), 16, 0, 0);
    }
}
// The same copies through a buffer resource over one head's operand: the
// per-lane byte offsets are computed once (row_voff / t_voff), the block's
// offset is a scalar, and `wofs` (the wave's byte offset inside a tile,
// wave * 1024) is uniform.
template <int D>
__device__ __forceinline__ void row_voff(uint32_t (&voff)[Tiles<D>::CH_ROW]) {
    constexpr int NSLOT = Tiles<D>::NSLOT;
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_ROW; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int r = c / NSLOT, slot = c % NSLOT;
        voff[i] = (uint32_t)(r * D + swz_row(r, slot, NSLOT) * 8) * 2u;
    }
}
template <int D>
__device__ __forceinline__ void t_voff(uint32_t (&voff)[Tiles<D>::CH_T], int64_t Sp) {
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_T; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int r = c / 4, slot = c % 4;
        voff[i] = (uint32_t)((int64_t)r * Sp + swz_t(r, slot) * 8) * 2u;
    }
}
// rows r0 .. r0 + kBN - 1 of a head's [rows][D] operand -> LDS row tile
template <int D>
__device__ __forceinline__ void bdma_row(const uint16_t* head, uint32_t bytes, const uint32_t* voff,
                                         int64_t r0, uint16_t* tile, uint32_t wofs) {
    const auto rs = make_rsrc(head, bytes);
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_ROW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LH_LDS_PTR(reinterpret_cast<char*>(tile) + 4096 * i + wofs), 16,
                                                 voff[i], (uint32_t)(r0 * D * 2), 0, 0);
}
// columns c0 .. c0 + kBN - 1 of a head's [D][Sp] operand -> LDS transposed tile
template <int D>
__device__ __forceinline__ void bdma_t(const uint16_t* head, uint32_t bytes, const uint32_t* voff,
                                       int64_t c0, uint16_t* tile, uint32_t wofs) {
    const auto rs = make_rsrc(head, bytes);
#pragma unroll
    for (int i = 0; i < Tiles<D>::CH_T; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LH_LDS_PTR(reinterpret_cast<char*>(tile) + 4096 * i + wofs), 16,
                                                 voff[i], (uint32_t)(c0 * 2), 0, 0);
}

// wait until this wave's outstanding vector-memory operations (its tile
// copies and loads) have completed (gfx9 s_waitcnt: vmcnt 0, others unchanged)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// fragment of row tile: row r, global 16-byte chunk c
template <int D>
__device__ __forceinline__ u32x4 frag_row(const uint16_t* lds, int r, int c) {
    return *reinterpret_cast<const u32x4*>(lds + r * D + swz_row(r, c, Tiles<D>::NSLOT) * 8);
}
// fragment of transposed tile: row r, sequence positions {4g..4g+3} and
// {16+4g..16+4g+3} of the block, which the split stores as the 16-byte run g
// (fragment order); one read, conflict-free over the 16 rows of a fragment
__device__ __forceinline__ u32x4 frag_t(const uint16_t* lds, int r, int g) {
    return *reinterpret_cast<const u32x4*>(lds + r * kBN + swz_t(r, g) * 8);
}

// p^level of row `row` of head h as a float (exact for every level that fits
// the sub-sequence's rows), for the pool adjoint's division
__device__ __forceinline__ float level_den(const AttnK& a, int h, int64_t row) {
    const int lv = a.level[(int64_t)h * a.rows + row];
    float den = 1.0f;
    for (int z = 0; z < lv; ++z) den *= (float)a.p;
    return den;
}
// 4 fp32 values / den, rounded to bf16 (round to nearest even)
__device__ __forceinline__ u32x2 bf16x4_div(const f32x4& x, float den) {
    return u32x2{pack_bf16x2(x[0] / den, x[1] / den), pack_bf16x2(x[2] / den, x[3] / den)};
}

// Scatter inside the attention kernels (Sec. 3 stage (iv), and the pool
// adjoint of the gradient path): a wavefront's 16 result rows are staged in
// LDS as bf16, then written to every token of their entries, one 16-byte
// chunk of one token row per lane, so the kernel's HBM writes overlap the
// other workgroups' MFMA work instead of running as a pass of their own.
// stage_rows: lane (lq, lg) holds columns 16v + 4lg .. +3 of row lq; the row
// is stored as bf16 of x * mul / den (den = p^level for the pool adjoint).
template <int D>
__device__ __forceinline__ void stage_rows(uint16_t* rows, const f32x4* acc, float mul, float den, int lq, int lg) {
#pragma unroll
    for (int v = 0; v < D / 16; ++v)
        *reinterpret_cast<u32x2*>(rows + lq * D + 16 * v + 4 * lg) = bf16x4_div(acc[v] * mul, den);
}
template <int D>
__device__ __forceinline__ void rows_to_tokens(const uint16_t* rows, uint16_t* tok, const AttnK& a, int h,
                                               int64_t r0, int lane) {
    constexpr int CPR = D / 8, TPI = 64 / CPR;   // 16-byte chunks per row, tokens per store
    const int c = lane % CPR, r4 = lane / CPR;
    for (int j = 0; j < 16; ++j) {
        const int64_t row = r0 + j;
        if (row >= a.rows) break;
        const int64_t st = a.start[(int64_t)h * a.rows + row];
        int64_t n = 1;
        for (int z = a.level[(int64_t)h * a.rows + row]; z > 0; --z) n *= a.p;
        const u32x4 x = *reinterpret_cast<const u32x4*>(rows + j * D + 8 * c);
        uint16_t* dst = tok + st * a.tok_ld + (int64_t)h * D + 8 * c;
        for (int64_t t = r4; t < n; t += TPI)
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst + t * a.tok_ld));
    }
}

// Work item -> (head, 64-row tile).  When H is a multiple of 8, the workgroups
// of a head are all dispatched to the same XCD (workgroup i runs on XCD i % 8),
// so the head's streamed operands stay in that XCD's L2.  `last_tile_first`
// dispatches the head's tiles from the last one down (for query tiles, the
// longest causal rows first; for key tiles, the shortest).
__device__ __forceinline__ void work_item(int nT, int H, bool last_tile_first, int& h, int& tile) {
    const int i = blockIdx.x;
    int j;
    if (H % 8 == 0) {
        const int x = i % 8, q = i / 8;
        h = x + 8 * (q / nT);
        j = q % nT;
    } else {
        h = i / nT;
        j = i % nT;
    }
    tile = last_tile_first ? nT - 1 - j : j;
}

// ------------------------------------------------------------------ forward
template <int D, bool SPLIT>
__global__ void __launch_bounds__(256) k_attn_fwd(AttnK a) {
    using T = Tiles<D>;
    constexpr int NS = D / 32, NV = D / 16;
    constexpr int NA = SPLIT ? 2 : 1;
    // K rows (read by the score phase) and V^T (read by the P V phase): one LDS
    // buffer each, refilled by direct copies while the other one is in use
    constexpr int KR = NA * T::ROW;
    __shared__ __attribute__((aligned(16))) uint16_t sm[KR + NA * T::TR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int64_t Sp = a.Sp;
    const int nT = (int)(Sp / 64);
    int h, qt;
    work_item(nT, gridDim.x / nT, true, h, qt);
    const int64_t q0 = (int64_t)qt * 64 + wave * 16;
    const int64_t myq = q0 + lq;
    const int64_t hb = (int64_t)h * Sp * D;
    const float mq = a.hscale[h * 4 + 0], mk = a.hscale[h * 4 + 1], mv = a.hscale[h * 4 + 2];
    const float c2 = a.scale * kLog2e * mq * mk;

    f16x8 qfh[NS], qfl[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = hb + myq * D + 32 * s + 8 * lg;
        qfh[s] = ld_f16x8(a.qh + off);
        if constexpr (SPLIT) qfl[s] = ld_f16x8(a.ql + off);
    }
    f32x4 o[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;

    const int nblk = (int)(((int64_t)qt * 64 + 64) / kBN);
    const uint16_t* Kh = sm;
    const uint16_t* Kl = sm + T::ROW;
    const uint16_t* Vh = sm + KR;
    const uint16_t* Vl = Vh + T::TR;
    const uint32_t wofs = __builtin_amdgcn_readfirstlane((uint32_t)wave * 1024u);
    const uint32_t hbytes = (uint32_t)(Sp * D * 2);
    uint32_t rvo[T::CH_ROW], tvo[T::CH_T];
    row_voff<D>(rvo);
    t_voff<D>(tvo, Sp);
    auto loadK = [&](int b) {
        bdma_row<D>(a.kh + hb, hbytes, rvo, (int64_t)b * kBN, sm, wofs);
        if constexpr (SPLIT) bdma_row<D>(a.kl + hb, hbytes, rvo, (int64_t)b * kBN, sm + T::ROW, wofs);
    };
    auto loadV = [&](int b) {
        bdma_t<D>(a.vTh + hb, hbytes, tvo, (int64_t)b * kBN, sm + KR, wofs);
        if constexpr (SPLIT) bdma_t<D>(a.vTl + hb, hbytes, tvo, (int64_t)b * kBN, sm + KR + T::TR, wofs);
    };
    loadK(0);
    loadV(0);
    wait_vmem();
    __syncthreads();
    // Per block: scores and softmax from K while this block's V^T may still be
    // arriving; the barrier publishes V^T and frees K, which is refilled during
    // the P V phase; the second barrier publishes K and frees V^T.
    for (int b = 0; b < nblk; ++b) {
        const bool more = b + 1 < nblk;
        const int64_t kb = (int64_t)b * kBN;
        const bool active = kb < q0 + 16;
        f32x4 sc[2];
        if (active) {
            // one accumulator per (key tile u, d step st), so consecutive MFMAs are
            // independent (a 16x16x32 MFMA chain needs many in flight); the partial
            // sums are added at the end
            f32x4 part[2][NS];
            f16x8 kfr[2][NS], klr[2][NS];
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    kfr[u][st] = __builtin_bit_cast(f16x8, frag_row<D>(Kh, 16 * u + lq, 4 * st + lg));
                    if constexpr (SPLIT) klr[u][st] = __builtin_bit_cast(f16x8, frag_row<D>(Kl, 16 * u + lq, 4 * st + lg));
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
                for (int u = 0; u < 2; ++u) part[u][st] = mma_h(kfr[u][st], qfh[st], f32x4{0.f, 0.f, 0.f, 0.f});
            if constexpr (SPLIT) {
#pragma unroll
                for (int st = 0; st < NS; ++st)
#pragma unroll
                    for (int u = 0; u < 2; ++u) part[u][st] = mma_h(kfr[u][st], qfl[st], part[u][st]);
#pragma unroll
                for (int st = 0; st < NS; ++st)
#pragma unroll
                    for (int u = 0; u < 2; ++u) part[u][st] = mma_h(klr[u][st], qfh[st], part[u][st]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                sc[u] = part[u][0];
#pragma unroll
                for (int st = 1; st < NS; ++st) sc[u] += part[u][st];
            }
            // row maximum of the unscaled scores (c2 > 0); only the block that meets
            // the diagonal needs the causal mask: key kb + 16u + 4g + r is visible to
            // query myq iff 16u + r <= myq - kb - 4g
            float mx = -INFINITY;
            if (kb + kBN - 1 > q0) {
                const int vis = (int)(myq - kb) - 4 * lg;
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = 16 * u + r > vis ? -INFINITY : sc[u][r];
                        sc[u][r] = x;
                        mx = fmaxf(mx, x);
                    }
            } else {
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[u][r]);
            }
            mx = rows4_max(mx) * c2;
            // The reference maximum m moves only when a row maximum exceeds it by
            // more than kLazyMax (log2 units), so P stays in [0, 2^kLazyMax] and
            // the rescale of O is rare; alpha is exactly 1 for rows that keep m.
            const bool grow = mx > m + kLazyMax;
            if (__ballot(grow) != 0) {
                const float mnew = grow ? mx : m;
                const float alpha = grow ? fast_exp2(m - mnew) : 1.0f;
                lsum *= alpha;
#pragma unroll
                for (int v = 0; v < NV; ++v) o[v] *= alpha;
                m = mnew;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pr = fast_exp2(fmaf(sc[u][r], c2, -m));
                    lsum += pr;
                    sc[u][r] = pr;
                }
        }
        wait_vmem();
        __syncthreads();
        if (more) loadK(b + 1);
        if (active) {
            f16x8 ph, pl;
            split_h(sc[0], sc[1], ph, pl);
            // all V^T fragments first, then the products in passes over v, so the
            // three MFMAs into one accumulator are NV issues apart
            f16x8 vfh[NV], vfl[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                vfh[v] = __builtin_bit_cast(f16x8, frag_t(Vh, 16 * v + lq, lg));
                if constexpr (SPLIT) vfl[v] = __builtin_bit_cast(f16x8, frag_t(Vl, 16 * v + lq, lg));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = 0; v < NV; ++v) o[v] = mma_h(vfh[v], ph, o[v]);
#pragma unroll
            for (int v = 0; v < NV; ++v) o[v] = mma_h(vfh[v], pl, o[v]);
            if constexpr (SPLIT) {
#pragma unroll
                for (int v = 0; v < NV; ++v) o[v] = mma_h(vfl[v], ph, o[v]);
            }
        }
        wait_vmem();
        __syncthreads();
        if (more) loadV(b + 1);
    }
    lsum = rows4_sum(lsum);
    const float mul = mv / lsum;
    // o[v][r] holds O^T[16v + 4g + r][myq]
    if (a.o) {
        float* O = a.o + hb + myq * D;
#pragma unroll
        for (int v = 0; v < NV; ++v) __builtin_nontemporal_store(o[v] * mul, reinterpret_cast<f32x4*>(O + 16 * v + 4 * lg));
    }
    if (a.o_bf16 && myq < a.rows) {
        uint16_t* O = a.o_bf16 + h * a.hs_o + myq * a.ld_o;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const f32x4 x = o[v] * mul;
            *reinterpret_cast<u32x2*>(O + 16 * v + 4 * lg) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        }
    }
    if (lg == 0) {
        const float l2 = m + log2f(lsum);
        a.lse2[(int64_t)h * Sp + myq] = l2;
        a.lse[(int64_t)h * Sp + myq] = l2 * kLn2;
    }
    if (a.o_tok) {   // the LDS tiles are idle: every wave is past the loop's last barrier
        uint16_t* rows = sm + wave * 16 * D;
        stage_rows<D>(rows, o, mul, 1.0f, lq, lg);
        __syncthreads();
        rows_to_tokens<D>(rows, a.o_tok, a, h, q0, lane);
    }
}

// ------------------------------------------------------- backward: dK, dV
// Key-stationary: wave w owns keys k0..k0+15 (lane column = key); the query
// blocks at or after the workgroup's keys stream through LDS.
template <int D, bool SPLIT, bool OUT_BF16>
__global__ void __launch_bounds__(256) k_attn_dkdv(AttnK a) {
    using T = Tiles<D>;
    constexpr int NS = D / 32, NV = D / 16;
    constexpr int NA = SPLIT ? 2 : 1;
    // LDS, one buffer each: q and dO rows (read by the score phase), q^T (bf16)
    // and dO^T (read by the gradient phase); each group is refilled as soon as
    // every wave is past its phase: 64 KiB at d = 128 with split operands
    constexpr int ROWS = NA * 2 * T::ROW;
    __shared__ __attribute__((aligned(16))) uint16_t sm[ROWS + NA * 2 * T::TR];
    // per-query lse2 and D of the block, copied with the rows: the score phase
    // then waits on no global load issued after the transposed-tile copies
    __shared__ __attribute__((aligned(16))) float qstat[2 * kBN];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int64_t Sp = a.Sp;
    const int nT = (int)(Sp / 64);
    int h, kt;
    // The last key tiles see the fewest queries.  When the kernel writes token rows,
    // they go first: their writes start soon, while the dQ kernel beside this one
    // works through its longest tiles, so HBM is not left idle at the start.
    // Without token writes the kernel is compute-bound and the longest go first.
    work_item(nT, gridDim.x / nT, a.dk_tok != nullptr, h, kt);
    const int64_t k0 = (int64_t)kt * 64 + wave * 16;
    const int64_t mykey = k0 + lq;
    const int64_t hb = (int64_t)h * Sp * D;
    const float mq = a.hscale[h * 4 + 0], mk = a.hscale[h * 4 + 1], mv = a.hscale[h * 4 + 2],
                mdo = a.hscale[h * 4 + 3];
    const float cS = a.scale * kLog2e * mq * mk;
    const float cP = mdo * mv;
    const float* lse2 = a.lse2 + (int64_t)h * Sp;
    const float* Dv = a.D + (int64_t)h * Sp;

    f16x8 kfh[NS], kfl[NS], vfh[NS], vfl[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = hb + mykey * D + 32 * s + 8 * lg;
        kfh[s] = ld_f16x8(a.kh + off);
        vfh[s] = ld_f16x8(a.vh + off);
        if constexpr (SPLIT) {
            kfl[s] = ld_f16x8(a.kl + off);
            vfl[s] = ld_f16x8(a.vl + off);
        }
    }
    f32x4 dk[NV], dv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) dk[v] = dv[v] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t qfirst = (int64_t)kt * 64;              // first query that can see the workgroup's keys
    const int nblk = (int)((a.rows - qfirst + kBN - 1) / kBN);
    // query blocks run from the last one down, so the workgroups of a head read
    // the same block at about the same time (one L2 working set per head)
    auto qblock = [&](int b) { return qfirst + (int64_t)(nblk - 1 - b) * kBN; };
    // layout: [qh][ql?][doh][dol?] rows, then [qTh][qTl?][doTh][doTl?]
    auto loadA = [&](int b) {
        const int64_t qb = qblock(b);
        if (wave == 0) {   // lanes 0..31: lse2, lanes 32..63: D (qb + 32 <= Sp)
            const float* src = (lane < kBN ? lse2 : Dv) + qb + (lane & (kBN - 1));
            __builtin_amdgcn_global_load_lds(src, LH_LDS_PTR(qstat), 4, 0, 0);
        }
        dma_row<D>(a.qh + hb, qb, sm);
        dma_row<D>(a.doh + hb, qb, sm + NA * T::ROW);
        if constexpr (SPLIT) {
            dma_row<D>(a.ql + hb, qb, sm + T::ROW);
            dma_row<D>(a.dol + hb, qb, sm + 3 * T::ROW);
        }
    };
    auto loadB = [&](int b) {
        const int64_t qb = qblock(b);
        uint16_t* base = sm + ROWS;
        dma_t<D>(a.qTbh + hb, Sp, qb, base);
        dma_t<D>(a.doTh + hb, Sp, qb, base + NA * T::TR);
        if constexpr (SPLIT) {
            dma_t<D>(a.qTbl + hb, Sp, qb, base + T::TR);
            dma_t<D>(a.doTl + hb, Sp, qb, base + 3 * T::TR);
        }
    };
    if (nblk > 0) {
        loadA(0);
        loadB(0);
    }
    wait_vmem();
    __syncthreads();
    const uint16_t* Qh = sm;
    const uint16_t* Ql = sm + T::ROW;
    const uint16_t* Oh = sm + NA * T::ROW;
    const uint16_t* Ol = Oh + T::ROW;
    const uint16_t* QTh = sm + ROWS;
    const uint16_t* QTl = QTh + T::TR;
    const uint16_t* OTh = QTh + NA * T::TR;
    const uint16_t* OTl = OTh + T::TR;
    // Per block: the score phase reads the rows while this block's transposed
    // tiles may still be arriving; the barrier after it publishes them and frees
    // the rows, which are refilled during the gradient phase; the second barrier
    // publishes the rows and frees the transposed tiles for the next block.
    for (int b = 0; b < nblk; ++b) {
        const bool more = b + 1 < nblk;
        const int64_t qb = qblock(b);
        const bool active = qb + kBN > k0;   // some query of the block sees some key of the wave
        f32x4 P[2], dS[2];
        if (active) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
                const int r = 16 * u + lq;
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    const f16x8 qh = __builtin_bit_cast(f16x8, frag_row<D>(Qh, r, 4 * st + lg));
                    const f16x8 oh = __builtin_bit_cast(f16x8, frag_row<D>(Oh, r, 4 * st + lg));
                    s = mma_h(qh, kfh[st], s);
                    dp = mma_h(oh, vfh[st], dp);
                    if constexpr (SPLIT) {
                        s = mma_h(qh, kfl[st], s);
                        s = mma_h(__builtin_bit_cast(f16x8, frag_row<D>(Ql, r, 4 * st + lg)), kfh[st], s);
                        dp = mma_h(oh, vfl[st], dp);
                        dp = mma_h(__builtin_bit_cast(f16x8, frag_row<D>(Ol, r, 4 * st + lg)), vfh[st], dp);
                    }
                }
                const int64_t qq = qb + 16 * u + 4 * lg;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(qstat + 16 * u + 4 * lg);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(qstat + kBN + 16 * u + 4 * lg);
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) {
                    const int q = (int)qq + r2;
                    float pr = fast_exp2(s[r2] * cS - l4[r2]);
                    pr = (q >= (int)mykey && q < (int)a.rows) ? pr : 0.f;
                    P[u][r2] = pr;
                    dS[u][r2] = pr * (dp[r2] * cP - d4[r2]);
                }
            }
        }
        wait_vmem();
        __syncthreads();
        if (more) loadA(b + 1);
        if (active) {
            f16x8 ph, pl;
            split_h(P[0], P[1], ph, pl);
            bf16x8 sh, sl;
            split_b(dS[0], dS[1], sh, sl);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int r = 16 * v + lq;
                const f16x8 oth = __builtin_bit_cast(f16x8, frag_t(OTh, r, lg));
                dv[v] = mma_h(oth, ph, dv[v]);
                dv[v] = mma_h(oth, pl, dv[v]);
                const bf16x8 qth = __builtin_bit_cast(bf16x8, frag_t(QTh, r, lg));
                dk[v] = mma_b(qth, sh, dk[v]);
                dk[v] = mma_b(qth, sl, dk[v]);
                if constexpr (SPLIT) {
                    dv[v] = mma_h(__builtin_bit_cast(f16x8, frag_t(OTl, r, lg)), ph, dv[v]);
                    dk[v] = mma_b(__builtin_bit_cast(bf16x8, frag_t(QTl, r, lg)), sh, dk[v]);
                }
            }
        }
        wait_vmem();
        __syncthreads();
        if (more) loadB(b + 1);
    }
    // dk[v][r], dv[v][r] hold the gradients of key mykey at d-index 16v + 4g + r
    if (mykey < a.rows) {
        if constexpr (OUT_BF16) {
            const int64_t base = h * a.hs_o + mykey * a.ld_o + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4 x = dk[v] * a.scale, y = dv[v] * mdo;
                *reinterpret_cast<u32x2*>(a.dk_b + base + 16 * v) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                *reinterpret_cast<u32x2*>(a.dv_b + base + 16 * v) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            }
        } else {
            const int64_t base = hb + mykey * D + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                __builtin_nontemporal_store(dk[v] * a.scale, reinterpret_cast<f32x4*>(a.dk + base + 16 * v));
                __builtin_nontemporal_store(dv[v] * mdo, reinterpret_cast<f32x4*>(a.dv + base + 16 * v));
            }
        }
    }
    if (a.dk_tok) {   // pool adjoint of k and v: dK~ / p^level, dV~ / p^level to the entry's tokens
        uint16_t* rk = sm + wave * 16 * D;
        uint16_t* rv = sm + (4 + wave) * 16 * D;
        const float den = mykey < a.rows ? level_den(a, h, mykey) : 1.0f;
        stage_rows<D>(rk, dk, a.scale, den, lq, lg);
        stage_rows<D>(rv, dv, mdo, den, lq, lg);
        __syncthreads();
        rows_to_tokens<D>(rk, a.dk_tok, a, h, k0, lane);
        rows_to_tokens<D>(rv, a.dv_tok, a, h, k0, lane);
    }
}

// ---------------------------------------------------------- backward: dQ
// Query-stationary: wave w owns queries q0..q0+15 and the key blocks up to the
// diagonal stream through LDS.  dS rows are scaled down by a power of two
// (rowdown) before the fp16 split, so they cannot overflow; the scale is undone
// at the end.
template <int D, bool SPLIT, bool OUT_BF16>
__global__ void __launch_bounds__(256) k_attn_dq(AttnK a) {
    using T = Tiles<D>;
    constexpr int NS = D / 32, NV = D / 16;
    constexpr int NA = SPLIT ? 2 : 1;
    // LDS: k and v rows (read by the score phase) and k^T (read by the dQ
    // phase), one buffer each, refilled by direct copies while the other one is
    // in use: 48 KiB at d = 128 with split operands
    constexpr int ROWS = NA * 2 * T::ROW;
    __shared__ __attribute__((aligned(16))) uint16_t sm[ROWS + NA * T::TR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int64_t Sp = a.Sp;
    const int nT = (int)(Sp / 64);
    int h, qt;
    work_item(nT, gridDim.x / nT, true, h, qt);
    const int64_t q0 = (int64_t)qt * 64 + wave * 16;
    const int64_t myq = q0 + lq;
    const int64_t hb = (int64_t)h * Sp * D;
    const float mq = a.hscale[h * 4 + 0], mk = a.hscale[h * 4 + 1], mv = a.hscale[h * 4 + 2],
                mdo = a.hscale[h * 4 + 3];
    const float cS = a.scale * kLog2e * mq * mk;
    const float cP = mdo * mv;

    f16x8 qfh[NS], qfl[NS], dfh[NS], dfl[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = hb + myq * D + 32 * s + 8 * lg;
        qfh[s] = ld_f16x8(a.qh + off);
        dfh[s] = ld_f16x8(a.doh + off);
        if constexpr (SPLIT) {
            qfl[s] = ld_f16x8(a.ql + off);
            dfl[s] = ld_f16x8(a.dol + off);
        }
    }
    const float l2 = a.lse2[(int64_t)h * Sp + myq];
    const float Dq = a.D[(int64_t)h * Sp + myq];
    const float down = a.rowdown[(int64_t)h * Sp + myq];
    f32x4 dq[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) dq[v] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nblk = (int)(((int64_t)qt * 64 + 64) / kBN);
    auto loadA = [&](int b) {
        const int64_t kb = (int64_t)b * kBN;
        dma_row<D>(a.kh + hb, kb, sm);
        dma_row<D>(a.vh + hb, kb, sm + NA * T::ROW);
        if constexpr (SPLIT) {
            dma_row<D>(a.kl + hb, kb, sm + T::ROW);
            dma_row<D>(a.vl + hb, kb, sm + 3 * T::ROW);
        }
    };
    auto loadB = [&](int b) {
        const int64_t kb = (int64_t)b * kBN;
        dma_t<D>(a.kTh + hb, Sp, kb, sm + ROWS);
        if constexpr (SPLIT) dma_t<D>(a.kTl + hb, Sp, kb, sm + ROWS + T::TR);
    };
    loadA(0);
    loadB(0);
    wait_vmem();
    __syncthreads();
    const uint16_t* Kh = sm;
    const uint16_t* Kl = sm + T::ROW;
    const uint16_t* Vh = sm + NA * T::ROW;
    const uint16_t* Vl = Vh + T::ROW;
    const uint16_t* KTh = sm + ROWS;
    const uint16_t* KTl = KTh + T::TR;
    // Per block: scores from the rows while this block's k^T may still be
    // arriving; the barrier publishes k^T and frees the rows, refilled during the
    // dQ phase; the second barrier publishes the rows and frees k^T.
    for (int b = 0; b < nblk; ++b) {
        const bool more = b + 1 < nblk;
        const int64_t kb = (int64_t)b * kBN;
        const bool active = kb < q0 + 16;
        f32x4 dS[2];
        if (active) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                // the key tile's fragments first, then its products in four
                // independent chains (s and dp, by parity of the d step)
                const int r = 16 * u + lq;
                f16x8 kh[NS], kl[NS], vh[NS], vl[NS];
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    kh[st] = __builtin_bit_cast(f16x8, frag_row<D>(Kh, r, 4 * st + lg));
                    vh[st] = __builtin_bit_cast(f16x8, frag_row<D>(Vh, r, 4 * st + lg));
                    if constexpr (SPLIT) {
                        kl[st] = __builtin_bit_cast(f16x8, frag_row<D>(Kl, r, 4 * st + lg));
                        vl[st] = __builtin_bit_cast(f16x8, frag_row<D>(Vl, r, 4 * st + lg));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x4 s2[2], dp2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) s2[e] = dp2[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    s2[st & 1] = mma_h(kh[st], qfh[st], s2[st & 1]);
                    dp2[st & 1] = mma_h(vh[st], dfh[st], dp2[st & 1]);
                }
                if constexpr (SPLIT) {
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        s2[st & 1] = mma_h(kh[st], qfl[st], s2[st & 1]);
                        dp2[st & 1] = mma_h(vh[st], dfl[st], dp2[st & 1]);
                    }
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        s2[st & 1] = mma_h(kl[st], qfh[st], s2[st & 1]);
                        dp2[st & 1] = mma_h(vl[st], dfh[st], dp2[st & 1]);
                    }
                }
                const f32x4 s = s2[0] + s2[1], dp = dp2[0] + dp2[1];
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) {
                    const int key = (int)kb + 16 * u + 4 * lg + r2;
                    float pr = fast_exp2(s[r2] * cS - l2);
                    pr = key <= (int)myq ? pr : 0.f;
                    dS[u][r2] = pr * (dp[r2] * cP - Dq) * down;
                }
            }
        }
        wait_vmem();
        __syncthreads();
        if (more) loadA(b + 1);
        if (active) {
            f16x8 sh, sl;
            split_h(dS[0], dS[1], sh, sl);
            // all k^T fragments first, then the products in passes over v, so the
            // three MFMAs into one accumulator are NV issues apart
            f16x8 kth[NV], ktl[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                kth[v] = __builtin_bit_cast(f16x8, frag_t(KTh, 16 * v + lq, lg));
                if constexpr (SPLIT) ktl[v] = __builtin_bit_cast(f16x8, frag_t(KTl, 16 * v + lq, lg));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = 0; v < NV; ++v) dq[v] = mma_h(kth[v], sh, dq[v]);
#pragma unroll
            for (int v = 0; v < NV; ++v) dq[v] = mma_h(kth[v], sl, dq[v]);
            if constexpr (SPLIT) {
#pragma unroll
                for (int v = 0; v < NV; ++v) dq[v] = mma_h(ktl[v], sh, dq[v]);
            }
        }
        wait_vmem();
        __syncthreads();
        if (more) loadB(b + 1);
    }
    if (myq < a.rows) {
        const float mul = a.scale * mk / down;
        if constexpr (OUT_BF16) {
            const int64_t base = h * a.hs_o + myq * a.ld_o + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4 x = dq[v] * mul;
                *reinterpret_cast<u32x2*>(a.dq_b + base + 16 * v) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
            }
        } else {
            const int64_t base = hb + myq * D + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) __builtin_nontemporal_store(dq[v] * mul, reinterpret_cast<f32x4*>(a.dq + base + 16 * v));
        }
    }
    if (a.dq_tok) {   // pool adjoint of q: dQ~ / p^level to every token of the entry
        uint16_t* rows = sm + wave * 16 * D;
        const float den = myq < a.rows ? level_den(a, h, myq) : 1.0f;
        stage_rows<D>(rows, dq, a.scale * mk / down, den, lq, lg);
        __syncthreads();
        rows_to_tokens<D>(rows, a.dq_tok, a, h, q0, lane);
    }
}

// ------------------------------------------------------------- fp32 path
// One wavefront per row; lane holds E = D/64 consecutive elements; double
// arithmetic throughout.
template <int E>
__device__ __forceinline__ double wave_dot(const double (&x)[E], const float* y) {
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) s = fma(x[e], (double)y[e], s);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    return s;
}

template <int D>
__global__ void __launch_bounds__(256) k_attn_fwd_f32(AttnK a) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= a.Sp) return;
    const int64_t hb = (int64_t)h * a.Sp * D;
    double q[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        q[e] = a.qf[hb + i * D + lane * E + e];
        acc[e] = 0.0;
    }
    const double sc = 1.0 / sqrt((double)D);
    double m = -INFINITY, l = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        const double s = wave_dot<E>(q, a.kf + hb + j * D + lane * E) * sc;
        const double mn = fmax(m, s);
        const double al = exp(m - mn);
        const double pr = exp(s - mn);
        l = l * al + pr;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = acc[e] * al + pr * (double)a.vf[hb + j * D + lane * E + e];
        m = mn;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) a.o[hb + i * D + lane * E + e] = (float)(acc[e] / l);
    if (lane == 0) {
        const double lse = m + log(l);
        a.lse[(int64_t)h * a.Sp + i] = (float)lse;
        a.lse2[(int64_t)h * a.Sp + i] = (float)(lse * 1.4426950408889634);
    }
}

// dQ (query rows) and dK/dV (key rows) in one kernel: blockIdx.z = 0 / 1.
template <int D>
__global__ void __launch_bounds__(256) k_attn_bwd_f32(AttnK a) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.y;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.rows) return;
    const int64_t hb = (int64_t)h * a.Sp * D;
    const float* lse = a.lse + (int64_t)h * a.Sp;
    const float* Dv = a.D + (int64_t)h * a.Sp;
    const double sc = 1.0 / sqrt((double)D);
    if (blockIdx.z == 0) {
        double q[E], g[E], acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            q[e] = a.qf[hb + r * D + lane * E + e];
            g[e] = a.dof[hb + r * D + lane * E + e];
            acc[e] = 0.0;
        }
        for (int64_t j = 0; j <= r; ++j) {
            const double s = wave_dot<E>(q, a.kf + hb + j * D + lane * E) * sc;
            const double pr = exp(s - (double)lse[r]);
            const double ds = pr * (wave_dot<E>(g, a.vf + hb + j * D + lane * E) - (double)Dv[r]);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fma(ds, (double)a.kf[hb + j * D + lane * E + e], acc[e]);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) a.dq[hb + r * D + lane * E + e] = (float)(acc[e] * sc);
    } else {
        double kk[E], vv[E], gk[E], gv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            kk[e] = a.kf[hb + r * D + lane * E + e];
            vv[e] = a.vf[hb + r * D + lane * E + e];
            gk[e] = gv[e] = 0.0;
        }
        for (int64_t i = r; i < a.rows; ++i) {
            const double s = wave_dot<E>(kk, a.qf + hb + i * D + lane * E) * sc;
            const double pr = exp(s - (double)lse[i]);
            const double ds = pr * (wave_dot<E>(vv, a.dof + hb + i * D + lane * E) - (double)Dv[i]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                gv[e] = fma(pr, (double)a.dof[hb + i * D + lane * E + e], gv[e]);
                gk[e] = fma(ds, (double)a.qf[hb + i * D + lane * E + e], gk[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            a.dk[hb + r * D + lane * E + e] = (float)(gk[e] * sc);
            a.dv[hb + r * D + lane * E + e] = (float)gv[e];
        }
    }
}

// ------------------------------------------------------------------ launchers
static AttnK to_k(const AttnArgs& x) {
    AttnK a{};
    a.qh = x.qh; a.ql = x.ql; a.kh = x.kh; a.kl = x.kl; a.vh = x.vh; a.vl = x.vl;
    a.doh = x.doh; a.dol = x.dol;
    a.vTh = x.vTh; a.vTl = x.vTl; a.kTh = x.kTh; a.kTl = x.kTl; a.doTh = x.doTh; a.doTl = x.doTl;
    a.qTbh = x.qTbh; a.qTbl = x.qTbl;
    a.hscale = x.hscale;
    a.o = x.o; a.o_bf16 = x.o_bf16;
    a.lse = x.lse; a.lse2 = x.lse2; a.D = x.D; a.rowdown = x.rowdown;
    a.dq = x.dq; a.dk = x.dk; a.dv = x.dv;
    a.dq_b = x.dq_b; a.dk_b = x.dk_b; a.dv_b = x.dv_b;
    a.level = x.level; a.p = x.p;
    a.o_tok = x.o_tok; a.dq_tok = x.dq_tok; a.dk_tok = x.dk_tok; a.dv_tok = x.dv_tok;
    a.start = x.start; a.tok_ld = x.tok_ld;
    a.rows = x.rows; a.Sp = x.Sp; a.ld_o = x.ld_o; a.hs_o = x.hs_o;
    a.scale = x.scale;
    a.qf = x.qf; a.kf = x.kf; a.vf = x.vf; a.dof = x.dof;
    return a;
}

#define LH_ATTN_DISPATCH(KERNEL, GRID, ...)                                                       \
    do {                                                                                          \
        if (x.d == 128) {                                                                         \
            if (x.split) hipLaunchKernelGGL((KERNEL<128, true __VA_ARGS__>), GRID, dim3(256), 0, s, a);   \
            else hipLaunchKernelGGL((KERNEL<128, false __VA_ARGS__>), GRID, dim3(256), 0, s, a);          \
        } else {                                                                                  \
            if (x.split) hipLaunchKernelGGL((KERNEL<64, true __VA_ARGS__>), GRID, dim3(256), 0, s, a);    \
            else hipLaunchKernelGGL((KERNEL<64, false __VA_ARGS__>), GRID, dim3(256), 0, s, a);           \
        }                                                                                         \
    } while (0)

hipError_t launch_attn_fwd(const AttnArgs& x, hipStream_t s) {
    AttnK a = to_k(x);
    if (x.fp32_path) {
        dim3 grid((unsigned)((x.Sp + 3) / 4), (unsigned)x.H);
        if (x.d == 128) hipLaunchKernelGGL(k_attn_fwd_f32<128>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_attn_fwd_f32<64>, grid, dim3(256), 0, s, a);
    } else {
        dim3 grid((unsigned)(x.Sp / 64 * x.H));
        LH_ATTN_DISPATCH(k_attn_fwd, grid);
    }
    return hipGetLastError();
}

hipError_t launch_attn_bwd(const AttnArgs& x, hipStream_t s, int part) {
    AttnK a = to_k(x);
    if (x.fp32_path) {
        if (part != 0) return hipSuccess;   // one kernel does both
        dim3 grid((unsigned)((x.rows + 3) / 4), (unsigned)x.H, 2);
        if (x.d == 128) hipLaunchKernelGGL(k_attn_bwd_f32<128>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_attn_bwd_f32<64>, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    dim3 grid((unsigned)(x.Sp / 64 * x.H));
    const bool ob = x.dq_b != nullptr;
    if (part == 0) {
        if (ob) LH_ATTN_DISPATCH(k_attn_dkdv, grid, , true);
        else LH_ATTN_DISPATCH(k_attn_dkdv, grid, , false);
    } else {
        if (ob) LH_ATTN_DISPATCH(k_attn_dq, grid, , true);
        else LH_ATTN_DISPATCH(k_attn_dq, grid, , false);
    }
    return hipGetLastError();
}

}  // namespace lh
