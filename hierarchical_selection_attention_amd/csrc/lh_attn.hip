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
// sequence position (V^T in P V, dO^T and Q^T in dV and dK, K^T in dQ) are
// read across the same row tiles with gfx950's transposed LDS read, which
// hands each lane its 8 positions in the order the score fragments hold them.
//
// Precision: the pooled sub-sequence is not representable in 16 bits, and
// the backward's dS = P o (dP - D) cancels heavily on heavy-tailed inputs, so
// every product uses split operands x = hi + lo in fp16 (22 significant bits;
// hi*hi + hi*lo + lo*hi, lo*lo being below fp32 rounding).  Every split
// value is first brought just below 2^14 by a power of two, so that its lo
// part stays in fp16's normal range:
//   * stored operands (q, k, v, dO rows): one power of two per head and tensor;
//   * P: the forward's softmax reference lags the row maximum by 2^6, so P
//     lies in [0, 2^14] there; the backward reads lse2 = log2-sum-exp - 14, so
//     P lies in [0, 2^14] there too (the 2^-14 is applied to dV at the end);
//   * dS (for dS K and dS^T Q): a running power of two per output column (per
//     query in dQ, per key in dK) that only decreases; when a block's largest
//     |dS| of a column would pass 2^14, the column's accumulators are
//     multiplied by the ratio of the old and new powers (exact).
// When the stored operands are exact in 16 bits (the dense path on bf16
// inputs) the lo parts of stored operands are zero and skipped.
//
// fp32 path: one wavefront per row, double-precision arithmetic.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// forward: the softmax reference m is set kPLag below the row maximum and
// moves only when the row maximum passes m + kPTop (log2 units), so the
// weights 2^(s - m) lie in [0, 2^kPTop], at least 2^kPLag for the row's
// maximum, and the rescale of O is rare (growth by more than 2^8)
constexpr float kPLag = 6.0f;
constexpr float kPTop = 14.0f;
// the backward kernels read lse2 = base-2 log-sum-exp - kPBwd, so their
// weights are P * 2^kPBwd in [0, 2^14]
constexpr float kPBwd = 14.0f;
constexpr float kInvPBwd = 1.0f / 16384.0f;

// Running power-of-two multiplier `mul` of one output column's dS values:
// keeps |dS| * mul below 2^14 for the block maximum `bm` of the column (same
// value in the column's four lanes).  Returns the factor (a power of two, or
// 1) by which the column's accumulators must be multiplied.
__device__ __forceinline__ float column_scale(float bm, float& mul) {
    if (!(bm * mul >= 16384.0f)) return 1.0f;
    int ex;
    frexpf(bm, &ex);                          // bm < 2^ex
    const float nm = ldexpf(1.0f, 14 - ex);   // bm * nm < 2^14
    const float f = nm / mul;
    mul = nm;
    return f;
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 ld_f16x8(const uint16_t* p) {
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f32x4 mma_h(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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

// Operand tensors of one attention problem (16-bit operands [H][Sp][d]
// row-major; lo pointers unused when !SPLIT).
struct AttnK {
    const uint16_t *qh, *ql, *kh, *kl, *vh, *vl, *doh, *dol;   // fp16 rows
    const float* hscale;    // [H][4]: true value = stored * hscale (q, k, v, dO)
    float* o;               // fp32 [H][Sp][d] sub-sequence output, or null
    uint16_t* o_bf16;       // bf16 output with strides ld_o/hs_o (dense), or null
    float *lse, *lse2;      // [H][Sp]: natural log-sum-exp, base-2 log-sum-exp - kPBwd
    const float* D;         // [H][Sp]
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
// Streamed operands move through LDS in blocks of kBN sequence positions,
// shared by the 4 wavefronts of a workgroup: row tiles of kBN rows of d
// elements, two stages (the copy of the next block lands in one while the
// current block is read from the other).  A tile is read along its rows
// (frag_row) or across them (frag_tr).
constexpr int kBN = 32;

template <int D>
struct Tiles {
    static constexpr int NSLOT = D / 8;              // 16-byte slots per row-tile row
    static constexpr int ROW = kBN * D;              // elements of a row tile
    static constexpr int CH_ROW = kBN * NSLOT / 256; // 16-byte chunks per thread
};

// Row tiles: slot s of row r holds the row's 16-byte chunk s ^ f(r).  At d = 128
// (16 slots) f is the linear map of r's low four bits b0..b3 to
// (b0 << 1) | (b1 << 2) | b2 | ((b2 ^ b3) << 3), chosen by measurement: with it
// both reads of a row tile, along (frag_row) and across (frag_tr), run free of
// LDS bank conflicts on gfx950 (r & 15 leaves the read across 2-way
// conflicted, a rotation of r the read along; 240 bit-linear maps were timed).
__device__ __forceinline__ int swz_row(int r, int slot, int nslot) {
    const int f = nslot == 16 ? (((r & 3) << 1) | ((r >> 2) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 3))
                              : (r & (nslot - 1));
    return slot ^ f;
}

// Direct global -> LDS copies of a row tile (no staging registers): thread c
// fetches row c / NSLOT's chunk swz_row(r, c % NSLOT), and the load writes it
// at wave base + 16 * lane, i.e. at slot c of the LDS tile.  The data is in
// LDS once the issuing wave's vmcnt has drained.
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
// The same copies through a buffer resource over one head's operand: the
// per-lane byte offsets are computed once (row_voff), the block's offset is a
// scalar, and `wofs` (the wave's byte offset inside a tile, wave * 1024) is
// uniform.
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

// wait until this wave's outstanding vector-memory operations (its tile
// copies and loads) have completed (gfx9 s_waitcnt: vmcnt 0, others unchanged)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// fragment of row tile: row r, global 16-byte chunk c
template <int D>
__device__ __forceinline__ u32x4 frag_row(const uint16_t* lds, int r, int c) {
    return *reinterpret_cast<const u32x4*>(lds + r * D + swz_row(r, c, Tiles<D>::NSLOT) * 8);
}
// Fragment of a row tile read across its rows (gfx950 ds_read_b64_tr_b16): lane
// (lq, g) receives column c0 + lq of rows 4g..4g+3 and 16+4g..16+4g+3, the
// contraction order in which the score fragments hold a block's positions.
// Within each 16-lane group the instruction hands lane t element t % 4 of the
// 8 bytes addressed by lane 4k + t / 4 as its k-th value; so lane s addresses
// row 4g + s / 4 (then 16 + 4g + s / 4), columns c0 + 4 (s % 4) .. + 3.
typedef __fp16 f16x4t __attribute__((__vector_size__(4 * sizeof(__fp16))));
template <int D>
__device__ __forceinline__ u32x4 frag_tr(const uint16_t* lds, int c0, int lq, int g) {
    const int r = 4 * g + (lq >> 2);
    const int col = c0 + 4 * (lq & 3);
    const int ch = col >> 3, e = col & 7;
    const uint16_t* p0 = lds + r * D + swz_row(r, ch, Tiles<D>::NSLOT) * 8 + e;
    const uint16_t* p1 = lds + (r + 16) * D + swz_row(r + 16, ch, Tiles<D>::NSLOT) * 8 + e;
    const f16x4t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) f16x4t*)(p0));
    const f16x4t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) f16x4t*)(p1));
    const u32x2 a = __builtin_bit_cast(u32x2, x0), b = __builtin_bit_cast(u32x2, x1);
    return u32x4{a[0], a[1], b[0], b[1]};
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
// adjoint of the gradient path): the workgroup's 64 result rows are staged in
// LDS as bf16, then written to every token of their entries, so the kernel's
// HBM writes overlap the other workgroups' MFMA work instead of running as a
// pass of their own.
// stage_rows: lane (lq, lg) holds columns 16v + 4lg .. +3 of row lq; the row
// is stored as bf16 of x * mul / den (den = p^level for the pool adjoint).
template <int D>
__device__ __forceinline__ void stage_rows(uint16_t* rows, const f32x4* acc, float mul, float den, int lq, int lg) {
#pragma unroll
    for (int v = 0; v < D / 16; ++v)
        *reinterpret_cast<u32x2*>(rows + lq * D + 16 * v + 4 * lg) = bf16x4_div(acc[v] * mul, den);
}
// Token table of the workgroup's 64 entries (rows r0 .. r0+63 of head h), by
// the first wavefront: tab[e] is the number of tokens of entries 0 .. e-1
// (tab[64] the total) and tab[65 + e] the first token of entry e.  Rows past
// the sub-sequence have no tokens.  Published by the caller's next barrier.
constexpr int kTokTab = 129;
__device__ __forceinline__ void token_table(const AttnK& a, int h, int64_t r0, int64_t* tab) {
    if (threadIdx.x >= 64) return;
    const int e = threadIdx.x;
    const int64_t row = r0 + e;
    int64_t n = 0, first = 0;
    if (row < a.rows) {
        first = a.start[(int64_t)h * a.rows + row];
        n = 1;
        for (int z = a.level[(int64_t)h * a.rows + row]; z > 0; --z) n *= a.p;
    }
    int64_t incl = n;   // inclusive prefix sum over the wavefront
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const int64_t u = __shfl_up(incl, k);
        if (e >= k) incl += u;
    }
    tab[e + 1] = incl;
    if (e == 0) tab[0] = 0;
    tab[65 + e] = first;
}
// Writes the staged rows (NT tensors; entry e's row at rows_j + e * D) to
// their tokens.  The work is flattened over (token, 16-byte chunk), so all
// four wavefronts share it evenly whatever the entries' sizes: thread t keeps
// chunk t % (D/8) and walks the workgroup's tokens 256/(D/8) apart, entry by
// entry, loading its chunk once per entry and stepping a pointer per token.
template <int D, int NT>
__device__ __forceinline__ void tile_to_tokens(const uint16_t* rows0, const uint16_t* rows1, uint16_t* tok0,
                                               uint16_t* tok1, const AttnK& a, int h, const int64_t* tab) {
    constexpr int CPR = D / 8, TPI = 256 / CPR;   // 16-byte chunks per row, tokens per pass
    const int c = threadIdx.x % CPR;
    const int64_t total = tab[64];
    const int64_t col = (int64_t)h * D + 8 * c;
    const int64_t step = (int64_t)TPI * a.tok_ld;
    int64_t t = threadIdx.x / CPR;   // this thread's next token (flat index over the 64 entries)
    for (int e = 0; e < 64 && t < total; ++e) {
        const int64_t end = tab[e + 1];
        if (t >= end) continue;
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(rows0 + e * D + 8 * c);
        u32x4 x1 = {0u, 0u, 0u, 0u};
        if constexpr (NT == 2) x1 = *reinterpret_cast<const u32x4*>(rows1 + e * D + 8 * c);
        const int64_t o = (tab[65 + e] - tab[e] + t) * a.tok_ld + col;
        uint16_t* p0 = tok0 + o;
        uint16_t* p1 = NT == 2 ? tok1 + o : nullptr;
        for (; t < end; t += TPI) {
            __builtin_nontemporal_store(x0, reinterpret_cast<u32x4*>(p0));
            p0 += step;
            if constexpr (NT == 2) {
                __builtin_nontemporal_store(x1, reinterpret_cast<u32x4*>(p1));
                p1 += step;
            }
        }
    }
}

// Work item -> (head, 64-row tile) of the forward.  When H is a multiple of
// 8, head h runs on XCD h % 8 (workgroup i runs on XCD i % 8), where its
// operands stay in that XCD's L2.  With token writes (`alternate`) the heads
// of an XCD are interleaved tile by tile and the query tiles go out in the
// order nT-1, 0, nT-2, 1, ... (the longest causal rows, then the shortest),
// so the workgroups resident at any time mix long and short rows and their
// token writes spread over the launch (at 512K: 0.507 -> 0.498 ms against the
// order below).  Without them (dense comparison, parent kept) the launch is
// bound by its MFMA work: heads one after the other, longest rows first.
__device__ __forceinline__ void work_item(int nT, int H, bool alternate, int& h, int& tile) {
    const int i = blockIdx.x;
    int j;
    if (H % 8 == 0) {
        const int G = H / 8, x = i % 8, q = i / 8;
        if (alternate) {
            h = x + 8 * (q % G);
            j = q / G;
        } else {
            h = x + 8 * (q / nT);
            j = q % nT;
        }
    } else {
        h = i / nT;
        j = i % nT;
    }
    if (alternate) j = (j & 1) ? nT - 1 - (j >> 1) : (j >> 1);
    tile = nT - 1 - j;
}

// ------------------------------------------------------------------ forward
template <int D, bool SPLIT>
__global__ void __launch_bounds__(256) k_attn_fwd(AttnK a) {
    using T = Tiles<D>;
    constexpr int NS = D / 32, NV = D / 16;
    constexpr int NA = SPLIT ? 2 : 1;
    // Per key block, one stage of row tiles: k (hi, lo) for the score phase and
    // v (hi, lo), read across (frag_tr) by the P V phase.  Two stages: the copy
    // of block b + 1 is in flight during all of block b's work, and one barrier
    // per block orders it.
    constexpr int STAGE = NA * 2 * T::ROW;
    __shared__ __attribute__((aligned(16))) uint16_t sm[2 * STAGE];
    __shared__ int64_t ttab[kTokTab];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int64_t Sp = a.Sp;
    const int nT = (int)(Sp / 64);
    int h, qt;
    work_item(nT, gridDim.x / nT, a.o_tok != nullptr, h, qt);
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
    const uint32_t wofs = __builtin_amdgcn_readfirstlane((uint32_t)wave * 1024u);
    const uint32_t hbytes = (uint32_t)(Sp * D * 2);
    uint32_t rvo[T::CH_ROW];
    row_voff<D>(rvo);
    // stage layout: [kh][kl?][vh][vl?] row tiles
    auto load = [&](int b) {
        uint16_t* base = sm + (b & 1) * STAGE;
        bdma_row<D>(a.kh + hb, hbytes, rvo, (int64_t)b * kBN, base, wofs);
        bdma_row<D>(a.vh + hb, hbytes, rvo, (int64_t)b * kBN, base + NA * T::ROW, wofs);
        if constexpr (SPLIT) {
            bdma_row<D>(a.kl + hb, hbytes, rvo, (int64_t)b * kBN, base + T::ROW, wofs);
            bdma_row<D>(a.vl + hb, hbytes, rvo, (int64_t)b * kBN, base + 3 * T::ROW, wofs);
        }
    };
    load(0);
    for (int b = 0; b < nblk; ++b) {
        // block b has landed (this wave's copies; the barrier covers the others')
        // and every wave is past block b - 1, whose stage the next copy refills
        wait_vmem();
        __syncthreads();
        if (b + 1 < nblk) load(b + 1);
        const int64_t kb = (int64_t)b * kBN;
        if (!(kb < q0 + 16)) continue;   // no key of the block is visible to the wave
        const uint16_t* Kh = sm + (b & 1) * STAGE;
        const uint16_t* Kl = Kh + T::ROW;
        const uint16_t* Vh = Kh + NA * T::ROW;
        const uint16_t* Vl = Vh + T::ROW;
        f32x4 sc[2];
        {
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
            // the small hi*lo and lo*hi products first, hi*hi last: an MFMA's
            // rounding error scales with its largest addend, accumulator included
            if constexpr (SPLIT) {
#pragma unroll
                for (int st = 0; st < NS; ++st)
#pragma unroll
                    for (int u = 0; u < 2; ++u) part[u][st] = mma_h(kfr[u][st], qfl[st], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int st = 0; st < NS; ++st)
#pragma unroll
                    for (int u = 0; u < 2; ++u) part[u][st] = mma_h(klr[u][st], qfh[st], part[u][st]);
#pragma unroll
                for (int st = 0; st < NS; ++st)
#pragma unroll
                    for (int u = 0; u < 2; ++u) part[u][st] = mma_h(kfr[u][st], qfh[st], part[u][st]);
            } else {
#pragma unroll
                for (int st = 0; st < NS; ++st)
#pragma unroll
                    for (int u = 0; u < 2; ++u) part[u][st] = mma_h(kfr[u][st], qfh[st], f32x4{0.f, 0.f, 0.f, 0.f});
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
            // The reference m moves only when a row maximum passes m + kPTop; it is
            // then set kPLag below that maximum.  alpha is exactly 1 for rows that
            // keep m.
            const bool grow = mx > m + kPTop;
            if (__ballot(grow) != 0) {
                const float mnew = grow ? mx - kPLag : m;
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
        {
            f16x8 ph, pl;
            split_h(sc[0], sc[1], ph, pl);
            // all V^T fragments first (the v rows read across), then the products
            // in passes over v, so the three MFMAs into one accumulator are NV
            // issues apart
            f16x8 vfh[NV], vfl[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                vfh[v] = __builtin_bit_cast(f16x8, frag_tr<D>(Vh, 16 * v, lq, lg));
                if constexpr (SPLIT) vfl[v] = __builtin_bit_cast(f16x8, frag_tr<D>(Vl, 16 * v, lq, lg));
            }
            __builtin_amdgcn_sched_barrier(0);
            // this block's products in fresh accumulators (small terms first), added
            // to O with fp32 adds: an MFMA that took O itself as its accumulator
            // would round at O's magnitude once per block and per split term
            f32x4 blk[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) blk[v] = mma_h(vfh[v], pl, f32x4{0.f, 0.f, 0.f, 0.f});
            if constexpr (SPLIT) {
#pragma unroll
                for (int v = 0; v < NV; ++v) blk[v] = mma_h(vfl[v], ph, blk[v]);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) blk[v] = mma_h(vfh[v], ph, blk[v]);
#pragma unroll
            for (int v = 0; v < NV; ++v) o[v] += blk[v];
        }
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
        a.lse2[(int64_t)h * Sp + myq] = l2 - kPBwd;
        a.lse[(int64_t)h * Sp + myq] = l2 * kLn2;
    }
    if (a.o_tok) {
        __syncthreads();   // every wave is done with the last stage before the LDS is reused
        token_table(a, h, (int64_t)qt * 64, ttab);
        stage_rows<D>(sm + wave * 16 * D, o, mul, 1.0f, lq, lg);
        __syncthreads();
        tile_to_tokens<D, 1>(sm, nullptr, a.o_tok, nullptr, a, h, ttab);
    }
}

// ------------------------------------------------------- backward: dK, dV
// Key-stationary: wave w owns keys k0..k0+15 (lane column = key) of key tile
// kt of head h; the query blocks at or after the workgroup's keys stream
// through LDS as row tiles (q and dO, hi and lo), two blocks' worth: the copy
// of block b + 1 is in flight during all of block b's work, and one barrier
// per block orders it.  The score phase reads the rows directly, the gradient
// phase reads them across (frag_tr): no transposed copies.  64 KiB at d = 128
// with split operands.
template <int D, bool SPLIT>
struct DkdvLds {
    static constexpr int STAGE = (SPLIT ? 2 : 1) * 2 * Tiles<D>::ROW;
    static constexpr int ELEMS = 2 * STAGE;
};
template <int D, bool SPLIT, bool OUT_BF16>
__device__ __forceinline__ void dkdv_body(const AttnK& a, uint16_t* __restrict__ sm, float* __restrict__ qstat,
                                          int64_t* __restrict__ ttab, int h, int kt) {
    using T = Tiles<D>;
    constexpr int NS = D / 32, NV = D / 16;
    constexpr int NA = SPLIT ? 2 : 1;
    constexpr int STAGE = DkdvLds<D, SPLIT>::STAGE;
    // qstat: per stage, the block's per-query lse2 and D, copied with the rows
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int64_t Sp = a.Sp;
    const int64_t k0 = (int64_t)kt * 64 + wave * 16;
    const int64_t mykey = k0 + lq;
    const int64_t hb = (int64_t)h * Sp * D;
    const float mq = a.hscale[h * 4 + 0], mk = a.hscale[h * 4 + 1], mv = a.hscale[h * 4 + 2],
                mdo = a.hscale[h * 4 + 3];
    const float cS = a.scale * kLog2e * mq * mk;
    const float cP = mdo * mv;
    const float* lse2 = a.lse2 + (int64_t)h * Sp;
    const float* Dv = a.D + (int64_t)h * Sp;
    float smul = 0x1p100f;   // running power-of-two multiplier of this key's dS column

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
    // stage layout: [qh][ql?][doh][dol?] row tiles
    auto load = [&](int b) {
        const int64_t qb = qblock(b);
        uint16_t* base = sm + (b & 1) * STAGE;
        if (wave == 0) {   // lanes 0..31: lse2, lanes 32..63: D (qb + 32 <= Sp)
            const float* src = (lane < kBN ? lse2 : Dv) + qb + (lane & (kBN - 1));
            __builtin_amdgcn_global_load_lds(src, LH_LDS_PTR(qstat + (b & 1) * 2 * kBN), 4, 0, 0);
        }
        dma_row<D>(a.qh + hb, qb, base);
        dma_row<D>(a.doh + hb, qb, base + NA * T::ROW);
        if constexpr (SPLIT) {
            dma_row<D>(a.ql + hb, qb, base + T::ROW);
            dma_row<D>(a.dol + hb, qb, base + 3 * T::ROW);
        }
    };
    if (nblk > 0) load(0);
    for (int b = 0; b < nblk; ++b) {
        // block b has landed (this wave's copies; the barrier covers the others')
        // and every wave is past block b - 1, whose stage the next copy refills
        wait_vmem();
        __syncthreads();
        if (b + 1 < nblk) load(b + 1);
        const int64_t qb = qblock(b);
        const bool active = qb + kBN > k0;   // some query of the block sees some key of the wave
        if (!active) continue;
        const uint16_t* Qh = sm + (b & 1) * STAGE;
        const uint16_t* Ql = Qh + T::ROW;
        const uint16_t* Oh = Qh + NA * T::ROW;
        const uint16_t* Ol = Oh + T::ROW;
        const float* qs = qstat + (b & 1) * 2 * kBN;
        f32x4 P[2], dS[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
            const int r = 16 * u + lq;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const f16x8 qh = __builtin_bit_cast(f16x8, frag_row<D>(Qh, r, 4 * st + lg));
                const f16x8 oh = __builtin_bit_cast(f16x8, frag_row<D>(Oh, r, 4 * st + lg));
                if constexpr (SPLIT) {
                    s = mma_h(qh, kfl[st], s);
                    s = mma_h(__builtin_bit_cast(f16x8, frag_row<D>(Ql, r, 4 * st + lg)), kfh[st], s);
                    dp = mma_h(oh, vfl[st], dp);
                    dp = mma_h(__builtin_bit_cast(f16x8, frag_row<D>(Ol, r, 4 * st + lg)), vfh[st], dp);
                }
                s = mma_h(qh, kfh[st], s);
                dp = mma_h(oh, vfh[st], dp);
            }
            const int64_t qq = qb + 16 * u + 4 * lg;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(qs + 16 * u + 4 * lg);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(qs + kBN + 16 * u + 4 * lg);
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) {
                const int q = (int)qq + r2;
                float pr = fast_exp2(s[r2] * cS - l4[r2]);   // P * 2^kPBwd
                pr = (q >= (int)mykey && q < (int)a.rows) ? pr : 0.f;
                P[u][r2] = pr;
                dS[u][r2] = pr * (dp[r2] * cP - d4[r2]);
            }
        }
        f16x8 ph, pl;
        split_h(P[0], P[1], ph, pl);
        // this key's dS column, brought below 2^14 by its running power of two
        float bm = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) bm = fmaxf(bm, fabsf(dS[u][r2]));
        bm = rows4_max(bm);
        if (__ballot(bm * smul >= 16384.0f) != 0) {
            const float f = column_scale(bm, smul);
#pragma unroll
            for (int v = 0; v < NV; ++v) dk[v] *= f;
        }
        f16x8 sh, sl;
        split_h(dS[0] * smul, dS[1] * smul, sh, sl);
        // dV^T += dO^T P and dK^T += Q^T dS: the transposed operands are the
        // rows read across; small split terms first, hi * hi last
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const f16x8 oth = __builtin_bit_cast(f16x8, frag_tr<D>(Oh, 16 * v, lq, lg));
            const f16x8 qth = __builtin_bit_cast(f16x8, frag_tr<D>(Qh, 16 * v, lq, lg));
            if constexpr (SPLIT) {
                dv[v] = mma_h(__builtin_bit_cast(f16x8, frag_tr<D>(Ol, 16 * v, lq, lg)), ph, dv[v]);
                dk[v] = mma_h(__builtin_bit_cast(f16x8, frag_tr<D>(Ql, 16 * v, lq, lg)), sh, dk[v]);
            }
            dv[v] = mma_h(oth, pl, dv[v]);
            dk[v] = mma_h(qth, sl, dk[v]);
            dv[v] = mma_h(oth, ph, dv[v]);
            dk[v] = mma_h(qth, sh, dk[v]);
        }
    }
    __syncthreads();   // every wave is done with the last stage before the LDS is reused
    // dk[v][r], dv[v][r] hold the gradients of key mykey at d-index 16v + 4g + r,
    // times smul 2^kPBwd / (scale mq) and 2^kPBwd / mdo
    const float kmul = a.scale * mq * kInvPBwd / smul, vmul = mdo * kInvPBwd;
    if (mykey < a.rows) {
        if constexpr (OUT_BF16) {
            const int64_t base = h * a.hs_o + mykey * a.ld_o + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4 x = dk[v] * kmul, y = dv[v] * vmul;
                *reinterpret_cast<u32x2*>(a.dk_b + base + 16 * v) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                *reinterpret_cast<u32x2*>(a.dv_b + base + 16 * v) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            }
        } else if (a.dk) {   // fp32 dK~, dV~ rows (null when only the token rows are wanted)
            const int64_t base = hb + mykey * D + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                __builtin_nontemporal_store(dk[v] * kmul, reinterpret_cast<f32x4*>(a.dk + base + 16 * v));
                __builtin_nontemporal_store(dv[v] * vmul, reinterpret_cast<f32x4*>(a.dv + base + 16 * v));
            }
        }
    }
    if (a.dk_tok) {   // pool adjoint of k and v: dK~ / p^level, dV~ / p^level to the entry's tokens
        token_table(a, h, (int64_t)kt * 64, ttab);
        const float den = mykey < a.rows ? level_den(a, h, mykey) : 1.0f;
        stage_rows<D>(sm + wave * 16 * D, dk, kmul, den, lq, lg);
        stage_rows<D>(sm + (4 + wave) * 16 * D, dv, vmul, den, lq, lg);
        __syncthreads();
        tile_to_tokens<D, 2>(sm, sm + 64 * D, a.dk_tok, a.dv_tok, a, h, ttab);
    }
}

// ---------------------------------------------------------- backward: dQ
// Query-stationary: wave w owns queries q0..q0+15 of query tile qt of head h,
// and the key blocks up to the diagonal stream through LDS as row tiles (k and
// v, hi and lo), two blocks' worth, like dK/dV.  dQ = dS K reads the k rows
// across (frag_tr).  Each query's dS row carries a running power of two
// (column_scale) before the fp16 split; it is undone at the end.
template <int D, bool SPLIT>
struct DqLds {
    static constexpr int STAGE = (SPLIT ? 2 : 1) * 2 * Tiles<D>::ROW;
    static constexpr int ELEMS = 2 * STAGE;
};
template <int D, bool SPLIT, bool OUT_BF16>
__device__ __forceinline__ void dq_body(const AttnK& a, uint16_t* __restrict__ sm, int64_t* __restrict__ ttab, int h,
                                        int qt) {
    using T = Tiles<D>;
    constexpr int NS = D / 32, NV = D / 16;
    constexpr int NA = SPLIT ? 2 : 1;
    constexpr int STAGE = DqLds<D, SPLIT>::STAGE;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int64_t Sp = a.Sp;
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
    float smul = 0x1p100f;   // running power-of-two multiplier of this query's dS row
    f32x4 dq[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) dq[v] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nblk = (int)(((int64_t)qt * 64 + 64) / kBN);
    // stage layout: [kh][kl?][vh][vl?] row tiles
    auto load = [&](int b) {
        const int64_t kb = (int64_t)b * kBN;
        uint16_t* base = sm + (b & 1) * STAGE;
        dma_row<D>(a.kh + hb, kb, base);
        dma_row<D>(a.vh + hb, kb, base + NA * T::ROW);
        if constexpr (SPLIT) {
            dma_row<D>(a.kl + hb, kb, base + T::ROW);
            dma_row<D>(a.vl + hb, kb, base + 3 * T::ROW);
        }
    };
    load(0);
    for (int b = 0; b < nblk; ++b) {
        wait_vmem();
        __syncthreads();
        if (b + 1 < nblk) load(b + 1);
        const int64_t kb = (int64_t)b * kBN;
        const bool active = kb < q0 + 16;
        if (!active) continue;
        const uint16_t* Kh = sm + (b & 1) * STAGE;
        const uint16_t* Kl = Kh + T::ROW;
        const uint16_t* Vh = Kh + NA * T::ROW;
        const uint16_t* Vl = Vh + T::ROW;
        f32x4 dS[2];
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
            // small split terms first, hi*hi last (an MFMA rounds at the scale of
            // its largest addend)
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
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                s2[st & 1] = mma_h(kh[st], qfh[st], s2[st & 1]);
                dp2[st & 1] = mma_h(vh[st], dfh[st], dp2[st & 1]);
            }
            const f32x4 s = s2[0] + s2[1], dp = dp2[0] + dp2[1];
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) {
                const int key = (int)kb + 16 * u + 4 * lg + r2;
                float pr = fast_exp2(s[r2] * cS - l2);   // P * 2^kPBwd
                pr = key <= (int)myq ? pr : 0.f;
                dS[u][r2] = pr * (dp[r2] * cP - Dq);
            }
        }
        float bm = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) bm = fmaxf(bm, fabsf(dS[u][r2]));
        bm = rows4_max(bm);
        if (__ballot(bm * smul >= 16384.0f) != 0) {
            const float f = column_scale(bm, smul);
#pragma unroll
            for (int v = 0; v < NV; ++v) dq[v] *= f;
        }
        f16x8 sh, sl;
        split_h(dS[0] * smul, dS[1] * smul, sh, sl);
        // all k^T fragments first (the k rows read across), then the products in
        // passes over v, so the three MFMAs into one accumulator are NV issues apart
        f16x8 kth[NV], ktl[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            kth[v] = __builtin_bit_cast(f16x8, frag_tr<D>(Kh, 16 * v, lq, lg));
            if constexpr (SPLIT) ktl[v] = __builtin_bit_cast(f16x8, frag_tr<D>(Kl, 16 * v, lq, lg));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < NV; ++v) dq[v] = mma_h(kth[v], sl, dq[v]);
        if constexpr (SPLIT) {
#pragma unroll
            for (int v = 0; v < NV; ++v) dq[v] = mma_h(ktl[v], sh, dq[v]);
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) dq[v] = mma_h(kth[v], sh, dq[v]);
    }
    __syncthreads();   // every wave is done with the last stage before the LDS is reused
    const float mul = a.scale * mk * kInvPBwd / smul;
    if (myq < a.rows) {
        if constexpr (OUT_BF16) {
            const int64_t base = h * a.hs_o + myq * a.ld_o + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4 x = dq[v] * mul;
                *reinterpret_cast<u32x2*>(a.dq_b + base + 16 * v) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
            }
        } else if (a.dq) {   // fp32 dQ~ rows (null when only the token rows are wanted)
            const int64_t base = hb + myq * D + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) __builtin_nontemporal_store(dq[v] * mul, reinterpret_cast<f32x4*>(a.dq + base + 16 * v));
        }
    }
    if (a.dq_tok) {   // pool adjoint of q: dQ~ / p^level to every token of the entry
        token_table(a, h, (int64_t)qt * 64, ttab);
        const float den = myq < a.rows ? level_den(a, h, myq) : 1.0f;
        stage_rows<D>(sm + wave * 16 * D, dq, mul, den, lq, lg);
        __syncthreads();
        tile_to_tokens<D, 1>(sm, nullptr, a.dq_tok, nullptr, a, h, ttab);
    }
}

// ------------------------------------------------------- backward: launch
// One launch runs both gradient roles: 0, dK/dV of a key tile, and 1, dQ of a
// query tile.  Key tile t of the dK/dV role and query tile nT-1-t of the dQ
// role both sweep nT - t tiles: rank t.  Workgroups are dispatched by rank in
// the order 0, nT-1, 1, nT-2, ... (a long rank, then a short one), the two
// roles of a rank side by side, so the workgroups resident at any time mix
// long and short items: their token writes, which start when an item's MFMA
// work ends, are spread over the whole launch instead of bunching where many
// similar items end together.  (Measured at 512K: 1.53 ms longest first, 1.37
// ms alternating.)  A launch that writes no token rows (dense comparison,
// parent-kept selection) is bound by its MFMA work alone and takes the ranks
// longest first (dense at 128K: 401 TFLOP/s against 328 alternating).  When H
// is a multiple of 8, head h runs on XCD h % 8 (workgroup i runs on XCD i % 8),
// where its operands sit in that XCD's L2.
__device__ __forceinline__ void bwd_item(int nT, int H, bool alternate, int& role, int& h, int& tile) {
    const int i = blockIdx.x;
    int j;
    if (H % 8 == 0) {
        const int G = H / 8, x = i % 8, q = i / 8;
        role = q & 1;
        j = q / (2 * G);
        h = x + 8 * ((q >> 1) % G);
    } else {
        role = i & 1;
        const int jj = i >> 1;
        j = jj / H;
        h = jj % H;
    }
    const int r = !alternate ? j : (j & 1) ? nT - 1 - (j >> 1) : (j >> 1);   // rank of the j-th position
    tile = role == 0 ? r : nT - 1 - r;
}

template <int D, bool SPLIT, bool OUT_BF16>
__global__ void __launch_bounds__(256) k_attn_bwd(AttnK a) {
    constexpr int E1 = DkdvLds<D, SPLIT>::ELEMS, E2 = DqLds<D, SPLIT>::ELEMS;
    __shared__ __attribute__((aligned(16))) uint16_t sm[E1 > E2 ? E1 : E2];
    __shared__ __attribute__((aligned(16))) float qstat[4 * kBN];
    __shared__ int64_t ttab[kTokTab];
    const int nT = (int)(a.Sp / 64);
    int role, h, tile;
    bwd_item(nT, (int)(gridDim.x / (2 * nT)), a.dk_tok != nullptr, role, h, tile);
    if (role == 0) dkdv_body<D, SPLIT, OUT_BF16>(a, sm, qstat, ttab, h, tile);
    else dq_body<D, SPLIT, OUT_BF16>(a, sm, ttab, h, tile);
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
        a.lse2[(int64_t)h * a.Sp + i] = (float)(lse * 1.4426950408889634 - (double)kPBwd);
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
    a.hscale = x.hscale;
    a.o = x.o; a.o_bf16 = x.o_bf16;
    a.lse = x.lse; a.lse2 = x.lse2; a.D = x.D;
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

hipError_t launch_attn_bwd(const AttnArgs& x, hipStream_t s) {
    AttnK a = to_k(x);
    if (x.fp32_path) {
        dim3 grid((unsigned)((x.rows + 3) / 4), (unsigned)x.H, 2);
        if (x.d == 128) hipLaunchKernelGGL(k_attn_bwd_f32<128>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_attn_bwd_f32<64>, grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    dim3 grid((unsigned)(2 * (x.Sp / 64) * x.H));
    if (x.dq_b != nullptr) LH_ATTN_DISPATCH(k_attn_bwd, grid, , true);
    else LH_ATTN_DISPATCH(k_attn_bwd, grid, , false);
    return hipGetLastError();
}

}  // namespace lh
