// Bandwidth-bound stages of the Lighthouse layer on gfx950.
//
// Paper: "Long Context Pre-Training with Lighthouse Attention" (arXiv
// 2605.06554), Sec. 3 stages (i) pooling and (iv) scatter, Fig. 1 (gather,
// back-scatter, gradient path) and Fig. 2 (mean-pool by p^l, l2 norm +
// max-pool).  Every kernel streams [N][H][d] rows with 16-byte vector
// accesses: a row is split over G = d/8 consecutive lanes (8 elements each),
// so one wavefront instruction touches 64*16 contiguous bytes of bf16.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

// ---------------------------------------------------------------------------
// Pooling + scoring pass (stage (i) and the scorer of stage (ii)).
// Chunks of `tok` = p^m tokens, all heads of a head group; a workgroup takes
// up to four chunks side by side (one group of threads each).  Thread (ts, h, c)
// of a group: token lane ts, head h, 8-element chunk c.  Outputs: the max-pool
// of the leaf scores for levels 1..m (and the leaf scores themselves on
// request), and the level-m means of q, k, v (fp32).
// The leaf score is ||q||^2 + ||k||^2 in fp32 in a fixed order: fma over the 8
// elements of a lane from +0, then a xor butterfly over the G lanes of the row,
// then one add of the q and k parts.  The other readings of what the norm is
// taken of are score modes: ||k||^2, ||q||^2, or ||q||^2 * ||k||^2 (one fp32
// multiply, ranking as ||q|| ||k||).
struct PoolScoreArgs {
    const void *q, *k, *v;
    float* lev[kMaxLevels];   // level l scores, [H][n_l]
    float* pool_m;            // fp32 [3][n_m][H][d]
    int64_t n[kMaxLevels];
    int N, H, HG, p, m, tok, mt;
    int score_mode;
    int store_l0;             // store level 0 too (else levels 1..m only)
    int tpc;                  // threads per chunk; a workgroup of ng * tpc threads takes ng chunks
    int lds_chunk;            // floats of LDS per chunk
    int64_t ld;               // q, k, v: token t, head h at element t * ld + h * d
    int64_t pw[kMaxLevels];
};

__device__ __forceinline__ float leaf_score(float sq, float sk, int mode) {
    return mode == 1 ? sk : mode == 2 ? sq : mode == 3 ? sq * sk : sq + sk;
}

// Tokens per load batch of the bf16 pooling pass (two batches in flight per wave).
// Two at d = 128: 110 VGPRs, four waves per SIMD, which is exactly one workgroup
// of four chunks per CU (0.961 -> 0.950 ms at 512K against one token per batch).
#ifndef LH_POOL_U
#define LH_POOL_U 2
#endif
// Tokens per load batch of the bf16 scatter adjoint (one tensor streamed).
#ifndef LH_SCATTER_U
#define LH_SCATTER_U 3
#endif

#ifndef LH_POOL_NG
#define LH_POOL_NG 4
#endif
// Token rows per load step and lane group in the gather (the q, k and v loads of
// the step's rows are issued together, then summed).  One row per step measured
// fastest at 512K: 0.1143 ms, against 0.1165 with two and 0.150 with four.
#ifndef LH_GATHER_U
#define LH_GATHER_U 1
#endif
template <int DT, int G>
__global__ void __launch_bounds__(1024) k_pool_score(PoolScoreArgs a) {
    extern __shared__ float smem_all[];
    const int d = G * 8;
    // Chunk group: a workgroup may take several chunks side by side (one per group of
    // tpc threads) and store all their results after one barrier.  The group index is
    // uniform over a wavefront: several chunks per workgroup only when tpc is a
    // multiple of 64.
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / a.tpc);
    const int tid = threadIdx.x - grp * a.tpc;
    const int64_t chunk = (int64_t)blockIdx.x * (blockDim.x / a.tpc) + grp;
    float* smem = smem_all + (size_t)grp * a.lds_chunk;
    const int c = tid % G;
    const int row = tid / G;
    const int HG = a.HG;              // heads handled by this workgroup
    const int hl = row % HG;          // local head
    const int h = blockIdx.y * HG + hl;
    const int ts = row / HG;
    const int H = a.H;
    const int64_t t0 = chunk * a.tok;
    const int iters = a.tok / a.mt;
    float* sc = smem;   // [HG][tok] leaf scores of this chunk (head-major)

    float aq[8], ak[8], av[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) aq[e] = ak[e] = av[e] = 0.f;

    // one token: fixed-order fp32 score and running sums of the pooled rows
    auto consume = [&](int tl, const float (&xq)[8], const float (&xk)[8], const float (&xv)[8]) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sq = __builtin_fmaf(xq[e], xq[e], sq);
            sk = __builtin_fmaf(xk[e], xk[e], sk);
        }
#pragma unroll
        for (int off = G / 2; off >= 1; off >>= 1) {
            sq = sq + shfl_xor_f(sq, off);
            sk = sk + shfl_xor_f(sk, off);
        }
        if (c == 0) sc[hl * a.tok + tl] = leaf_score(sq, sk, a.score_mode);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            aq[e] += xq[e];
            ak[e] += xk[e];
            av[e] += xv[e];
        }
    };
    if constexpr (DT == 0) {
        // bf16: U tokens of raw 16-byte non-temporal loads in flight (read once);
        // the butterflies of the U tokens are interleaved so the cross-lane moves
        // overlap.  Loads go through buffer resources over this workgroup's chunk:
        // one lane offset, and a uniform offset per token.
        const int64_t base0 = t0 * a.ld + (int64_t)blockIdx.y * HG * d;
        const uint32_t chunk_bytes = (uint32_t)((((int64_t)a.tok - 1) * a.ld + HG * d) * 2);
        const uint32_t tstride = (uint32_t)(a.mt * a.ld * 2);
        const uint32_t lane_off = (uint32_t)((ts * a.ld + hl * d + c * 8) * 2);
        const auto Q = make_rsrc(reinterpret_cast<const uint16_t*>(a.q) + base0, chunk_bytes);
        const auto Kp = make_rsrc(reinterpret_cast<const uint16_t*>(a.k) + base0, chunk_bytes);
        const auto V = make_rsrc(reinterpret_cast<const uint16_t*>(a.v) + base0, chunk_bytes);
        // loads of tokens i0 .. i0+U-1 into r (q, k, v per token)
        auto issue = [&](u32x4* r, int i0, auto Uc) {
            constexpr int U = decltype(Uc)::value;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t off = (uint32_t)(i0 + u) * tstride;
                r[3 * u + 0] = buf_ld16_nt(Q, lane_off, off);
                r[3 * u + 1] = buf_ld16_nt(Kp, lane_off, off);
                r[3 * u + 2] = buf_ld16_nt(V, lane_off, off);
            }
        };
        // scores and pooled sums of tokens i0 .. i0+U-1 held in r
        auto consume_batch = [&](const u32x4* r, int i0, auto Uc) {
            constexpr int U = decltype(Uc)::value;
            float sq[U], sk[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float xq[8], xk[8], xv[8];
                unpack8(r[3 * u + 0], xq);
                unpack8(r[3 * u + 1], xk);
                unpack8(r[3 * u + 2], xv);
                float a1 = 0.f, a2 = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a1 = __builtin_fmaf(xq[e], xq[e], a1);
                    a2 = __builtin_fmaf(xk[e], xk[e], a2);
                }
                sq[u] = a1;
                sk[u] = a2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    aq[e] += xq[e];
                    ak[e] += xk[e];
                    av[e] += xv[e];
                }
            }
            // Materialise the sums here.  Left to itself the compiler sinks them past
            // the score store's branch, so the loaded registers stay live across the
            // next prefetch; it then loads into other registers and copies them back
            // at the loop end behind a wait for every load in flight.
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(aq[e]), "+v"(ak[e]), "+v"(av[e]));
            // a_g <- a_g + a_(g^off), off = G/2 .. 1
#define LH_BFLY(OFF)                                                        \
            if constexpr (G / 2 >= OFF) {                                   \
                _Pragma("unroll") for (int u = 0; u < U; ++u) {             \
                    sq[u] = sq[u] + xor_lane<OFF>(sq[u]);                   \
                    sk[u] = sk[u] + xor_lane<OFF>(sk[u]);                   \
                }                                                           \
            }
            LH_BFLY(8)
            LH_BFLY(4)
            LH_BFLY(2)
            LH_BFLY(1)
#undef LH_BFLY
            if (c == 0) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    sc[hl * a.tok + ts + a.mt * (i0 + u)] = leaf_score(sq[u], sk[u], a.score_mode);
            }
        };
        // full batches of UB tokens, double-buffered: the loads of batch b+1 are
        // issued before batch b is consumed; then single tokens
        constexpr int UB = LH_POOL_U;
        using UBc = std::integral_constant<int, UB>;
        const int nb = iters / UB;
        u32x4 ra[3 * UB], rb[3 * UB];
        // (no branch between a prefetch and the consume after it, so the waits stay exact)
        if (nb > 0) issue(ra, 0, UBc{});
        int b = 0;
        for (; b + 2 < nb; b += 2) {
            issue(rb, (b + 1) * UB, UBc{});
            __builtin_amdgcn_sched_barrier(0);
            consume_batch(ra, b * UB, UBc{});
            issue(ra, (b + 2) * UB, UBc{});
            __builtin_amdgcn_sched_barrier(0);
            consume_batch(rb, (b + 1) * UB, UBc{});
        }
        if (b + 1 < nb) {
            issue(rb, (b + 1) * UB, UBc{});
            __builtin_amdgcn_sched_barrier(0);
            consume_batch(ra, b * UB, UBc{});
            consume_batch(rb, (b + 1) * UB, UBc{});
        } else if (b < nb) {
            consume_batch(ra, b * UB, UBc{});
        }
        for (int i = nb * UB; i < iters; ++i) {
            issue(ra, i, std::integral_constant<int, 1>{});
            consume_batch(ra, i, std::integral_constant<int, 1>{});
        }
    } else {
        for (int i = 0; i < iters; ++i) {
            const int64_t t = t0 + ts + (int64_t)a.mt * i;
            const int64_t el = t * a.ld + (int64_t)h * d + c * 8;
            float xq[8], xk[8], xv[8];
            load8_nt<DT>(a.q, el, xq);
            load8_nt<DT>(a.k, el, xk);
            load8_nt<DT>(a.v, el, xv);
            consume(ts + a.mt * i, xq, xk, xv);
        }
    }
    __syncthreads();

    // scores of levels 0..m for this chunk.  Level l+1 is the max over p entries of
    // level l (max is exact, so this equals the max over the covered leaves); the
    // levels alternate between sc and lb, [HG][tok / p^l] each.
    {
        float* lb = smem + (size_t)a.tok * HG;
        float* src = sc;
        float* dst = lb;
        int per = a.tok;
        for (int l = 0; l <= a.m; ++l) {
            const int64_t j0 = t0 / a.pw[l];
            float* out = a.lev[l] + (int64_t)blockIdx.y * HG * a.n[l] + j0;
            // non-temporal stores: nothing reads the scores until the selection,
            // and cached lines written inside this read stream cost more (16-byte
            // stores when every head's run is 16-byte aligned).  Leaves are stored
            // only on request: writes inside this read stream cost several times
            // their bytes, and the selection does not rank leaves.
            if (l == 0 && !a.store_l0) {
            } else if ((per & 3) == 0 && (a.n[l] & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
                for (int idx = tid; idx < HG * per / 4; idx += a.tpc) {
                    const int i4 = idx * 4, hh = i4 / per, j = i4 - hh * per;
                    const f32x4 x = *reinterpret_cast<const f32x4*>(src + i4);
                    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(out + (int64_t)hh * a.n[l] + j));
                }
            } else {
                for (int idx = tid; idx < HG * per; idx += a.tpc) {
                    const int hh = idx / per, j = idx - hh * per;
                    __builtin_nontemporal_store(src[idx], out + (int64_t)hh * a.n[l] + j);
                }
            }
            if (l == a.m) break;
            const int nper = per / a.p;
            for (int idx = tid; idx < HG * nper; idx += a.tpc) {
                const float* g = src + (int64_t)idx * a.p;   // entries idx*p .. idx*p+p-1 of [HG][per]
                float mx = g[0];
                for (int k = 1; k < a.p; ++k) mx = fmaxf(mx, g[k]);
                dst[idx] = mx;
            }
            __syncthreads();
            float* t = src; src = dst; dst = t;
            per = nper;
        }
    }

    // level-m means of q, k, v (only needed when the pyramid has levels)
    if (a.m >= 1) {
        float* red = smem + (size_t)a.tok * HG + (size_t)(a.tok / a.p) * HG;   // [mt][HG][d]
        const float inv = 1.0f / (float)a.tok;
        const int64_t blk = chunk;
        float* accs[3] = {aq, ak, av};
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            float* acc = accs[t];
            float* dst = a.pool_m + ((int64_t)t * a.n[a.m] + blk) * H * d;
            if (a.mt == 1) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = acc[e] * inv;
                store8f_nt(dst, (int64_t)h * d + c * 8, o);
            } else {
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 8; ++e) red[(ts * HG + hl) * d + c * 8 + e] = acc[e];
                __syncthreads();
                if (ts == 0) {
                    float o[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float s = 0.f;
                        for (int z = 0; z < a.mt; ++z) s += red[(z * HG + hl) * d + c * 8 + e];
                        o[e] = s * inv;
                    }
                    store8f_nt(dst, (int64_t)h * d + c * 8, o);
                }
            }
        }
    }
}

// Levels m+1..L-1 from level m: top-level means of q, k, v and max-pooled
// scores.  One workgroup per top-level block.
struct PoolUpArgs {
    float* lev[kMaxLevels];
    const float* pool_m;   // [3][n_m][H][d]
    float* pool_top;       // [3][ntop][H][d]
    int64_t n[kMaxLevels];
    int64_t pw[kMaxLevels];
    int H, d, p, m, L;
};

__global__ void __launch_bounds__(256) k_pool_up(PoolUpArgs a) {
    const int64_t b = blockIdx.x;
    const int R = (int)(a.pw[a.L - 1] / a.pw[a.m]);   // level-m rows per top block
    const int HD = a.H * a.d;
    const float inv = 1.0f / (float)R;
    for (int t = 0; t < 3; ++t) {
        const float* src = a.pool_m + ((int64_t)t * a.n[a.m] + b * R) * HD;
        float* dst = a.pool_top + ((int64_t)t * a.n[a.L - 1] + b) * HD;
        for (int idx = threadIdx.x; idx < HD; idx += blockDim.x) {
            float s = 0.f;
            for (int r = 0; r < R; ++r) s += src[(int64_t)r * HD + idx];
            dst[idx] = s * inv;
        }
    }
    for (int l = a.m + 1; l < a.L; ++l) {
        const int per = (int)(a.pw[a.L - 1] / a.pw[l]);   // level-l entries per top block
        for (int idx = threadIdx.x; idx < a.H * per; idx += blockDim.x) {
            int h = idx / per, j = idx % per;
            int64_t jj = b * per + j;
            const float* prev = a.lev[l - 1] + h * a.n[l - 1] + jj * a.p;
            float mx = prev[0];
            for (int c = 1; c < a.p; ++c) mx = fmaxf(mx, prev[c]);
            a.lev[l][h * a.n[l] + jj] = mx;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Gather (Fig. 1 "Dense Gather"): sub-sequence row i of head h is the mean of
// the pyramid entry (start_i, level_i).  One wavefront per row; the entry is
// read from the stored top level, from the stored level m (p^(l-m) rows), or
// from the input tokens (p^l rows).  Rows i in [S, Sp) are written as zeros.
// Rows differ in cost by up to p^(m-1) input rows, so each row is a workgroup
// of its own: a workgroup of several rows would hold its slot until its
// slowest row finished.
struct GatherArgs {
    const void *q, *k, *v;
    const float* pool_m;
    const float* pool_top;
    const int32_t* start;
    const uint8_t* level;
    float *qs, *ks, *vs;   // fp32 [H][Sp][d]
    float* rowmax;         // fp32 [3][H][Sp]: max |x| of each written row (q, k, v)
    int64_t S, Sp, n_m, ntop;
    int64_t ld;            // q, k, v: token t, head h at element t * ld + h * d
    int64_t pw[kMaxLevels];
    int H, m, L;
};

template <int DT, int G>
__global__ void __launch_bounds__(64) k_gather(GatherArgs a) {
    constexpr int d = G * 8;
    constexpr int NR = 64 / G;   // rows read per wavefront instruction
    const int lane = threadIdx.x & 63;
    const int c = lane % G, rs = lane / G;
    const int h = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x;
    if (i >= a.Sp) return;
    const int64_t orow = ((int64_t)h * a.Sp + i) * d + c * 8;
    if (i >= a.S) {
        if (rs == 0) {
            float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            store8f(a.qs, orow, z);
            store8f(a.ks, orow, z);
            store8f(a.vs, orow, z);
        }
        if (lane == 0)
            for (int t = 0; t < 3; ++t) a.rowmax[((int64_t)t * a.H + h) * a.Sp + i] = 0.f;
        return;
    }
    const int64_t st = a.start[h * a.S + i];
    const int l = a.level[h * a.S + i];
    const int H = a.H;
    float acc[3][8];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
    int64_t R;
    if (l >= 1 && l == a.L - 1) {
        R = 1;
        if (rs == 0) {
            const int64_t el = ((st / a.pw[l]) * H + h) * d + c * 8;
#pragma unroll
            for (int t = 0; t < 3; ++t) load8_nt<1>(a.pool_top + t * a.ntop * H * d, el, acc[t]);
        }
    } else if (l >= 1 && l >= a.m) {
        R = a.pw[l] / a.pw[a.m];
        const int64_t r0 = st / a.pw[a.m];
        for (int64_t r = rs; r < R; r += NR) {
            const int64_t el = ((r0 + r) * H + h) * d + c * 8;
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                float x[8];
                load8_nt<1>(a.pool_m + t * a.n_m * H * d, el, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[t][e] += x[e];
            }
        }
    } else {
        R = a.pw[l];
        const void* src[3] = {a.q, a.k, a.v};
        constexpr int U = LH_GATHER_U;
        for (int64_t r0 = rs; r0 < R; r0 += NR * U) {
            float x[U][3][8];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t r = r0 + (int64_t)u * NR;
                if (r < R) {
                    const int64_t el = (st + r) * a.ld + (int64_t)h * d + c * 8;
#pragma unroll
                    for (int t = 0; t < 3; ++t) load8_nt<DT>(src[t], el, x[u][t]);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (r0 + (int64_t)u * NR < R) {
#pragma unroll
                    for (int t = 0; t < 3; ++t)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[t][e] += x[u][t][e];
                }
            }
        }
    }
    if (R > 1) {
#pragma unroll
        for (int off = G; off < 64; off <<= 1)
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[t][e] += shfl_xor_f(acc[t][e], off);
    }
    float* dst[3] = {a.qs, a.ks, a.vs};
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        float o[8], mx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[e] = (R > 1) ? acc[t][e] / (float)R : acc[t][e];
            mx = fmaxf(mx, fabsf(o[e]));
        }
        if (rs == 0) store8f_nt(dst[t], orow, o);
        // the row's max |x| for the per-head scale of the 16-bit operand copies (lanes
        // rs != 0 hold the same row after the butterfly, or zeros when R == 1)
#pragma unroll
        for (int off = G / 2; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
        if (lane == 0) a.rowmax[((int64_t)t * a.H + h) * a.Sp + i] = mx;
    }
}

// ---------------------------------------------------------------------------
// Token-range mapping shared by the scatter-type kernels: a workgroup covers
// kTileTok consecutive tokens of every head; thread (ts, h, c) walks the
// contiguous sub-range ts of length kTileTok/mt with a cursor over the
// position-sorted sub-sequence of head h.
constexpr int kTileTok = 64;

struct TokMap {
    int c, h, ts;
    int64_t tb, te;
};

template <int G>
__device__ __forceinline__ TokMap tok_map(int HG, int mt, int64_t N) {
    TokMap m;
    const int tid = threadIdx.x;
    m.c = tid % G;
    const int row = tid / G;
    m.h = blockIdx.y * HG + row % HG;
    m.ts = row / HG;
    const int span = kTileTok / mt;
    m.tb = (int64_t)blockIdx.x * kTileTok + (int64_t)m.ts * span;
    m.te = m.tb + span;
    if (m.te > N) m.te = N;
    return m;
}

// Last slot whose start is <= t (starts are strictly increasing, start[0] = 0).
__device__ __forceinline__ int64_t find_slot(const int32_t* st, int64_t S, int64_t t) {
    int64_t lo = 0, hi = S - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) >> 1;
        if (st[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Scatter forward (stage (iv)): o[t][h] = O~[h][slot_h(t)], rounded once from
// the fp32 sub-sequence output to the I/O dtype.
struct ScatterArgs {
    const int32_t* start;
    const float* src;     // fp32 [H][Sp][d]
    void* dst;            // dtype [N][H][d]
    int64_t N, S, Sp;
    int H, HG, mt;
};

template <int DT, int G>
__global__ void __launch_bounds__(256) k_scatter_fwd(ScatterArgs a) {
    constexpr int d = G * 8;
    const TokMap tm = tok_map<G>(a.HG, a.mt, a.N);
    if (tm.tb >= tm.te) return;
    const int32_t* st = a.start + (int64_t)tm.h * a.S;
    int64_t slot = find_slot(st, a.S, tm.tb);
    int64_t nxt = slot + 1 < a.S ? st[slot + 1] : a.N;
    const int64_t sbase = (int64_t)tm.h * a.Sp * d + tm.c * 8;
    const int64_t H = a.H;
    float x[8];
    load8f(a.src, sbase + slot * d, x);
    for (int64_t t = tm.tb; t < tm.te; ++t) {
        if (t >= nxt) {
            ++slot;
            nxt = slot + 1 < a.S ? st[slot + 1] : a.N;
            load8f(a.src, sbase + slot * d, x);
        }
        store8<DT, true>(a.dst, (t * H + tm.h) * d + tm.c * 8, x);
    }
}

// Adjoint of the scatter: dO~[h][i] = sum over the tokens of entry i of dO.
// A thread owns one block of p^m tokens (the pooling chunk) for one
// (head, 8-element chunk) and sums dO over each entry in token order in fp32.
// Entries at levels <= m lie inside one block and are stored directly (fp32,
// both modes).  Only coarser entries span blocks; such an entry covers each
// of its blocks whole, so a block holds at most one partial sum of one:
//   mode 0: the partial is added to the entry's row with fp32 atomics;
//   mode 1 (deterministic): the partial is stored, without atomics, to the
//     block's row of `part`, and the row preparation adds an entry's partials
//     in block order (the same bits on every run, over the whole fp32 range).
struct ScatterBwdArgs {
    const int32_t* start;
    const void* dout;     // dtype [N][H][d]
    float* acc;           // fp32 [H][Sp][d]
    float* part;          // mode 1: fp32 [H][N / tok][d] partial sums of entries above level m
    int64_t N, S, Sp, tok;
    int H, HG;
};

template <int DT, int G, int MODE>
__device__ __forceinline__ void flush_entry(const ScatterBwdArgs& a, int h, int c, int64_t slot, bool whole,
                                            const float (&s)[8]) {
    constexpr int d = G * 8;
    const int64_t el = ((int64_t)h * a.Sp + slot) * d + c * 8;
    if (whole) {
        store8f_nt(a.acc, el, s);
    } else if constexpr (MODE == 0) {
        float* p = a.acc + el;
#pragma unroll
        for (int e = 0; e < 8; ++e) unsafeAtomicAdd(p + e, s[e]);
    } else {
        store8f_nt(a.part, ((int64_t)h * (a.N / a.tok) + blockIdx.x) * d + c * 8, s);
    }
}

template <int DT, int G, int MODE>
__global__ void __launch_bounds__(256) k_scatter_bwd(ScatterBwdArgs a) {
    constexpr int d = G * 8;
    const int tid = threadIdx.x;
    const int c = tid % G;
    const int hl = tid / G;
    const int h = blockIdx.y * a.HG + hl;
    const int64_t tb = (int64_t)blockIdx.x * a.tok;
    const int64_t te = tb + a.tok;
    const int32_t* st = a.start + (int64_t)h * a.S;
    const int64_t slot0 = find_slot(st, a.S, tb);
    // First tokens of the entries from slot0 on, for this head's walk: at most tok
    // entries start inside the chunk, so tok + 2 values cover every entry met and
    // the start of the one after the last (N past the end).  Kept in LDS: a load
    // from memory at each entry boundary would wait for every dO load in flight.
    extern __shared__ int32_t stab_mem[];
    int32_t* stab = stab_mem + hl * (int)(a.tok + 2);
    for (int i = c; i < (int)a.tok + 2; i += G) stab[i] = slot0 + i < a.S ? st[slot0 + i] : (int32_t)a.N;
    __syncthreads();
    int ls = 0;   // current entry: slot0 + ls
    int64_t beg = stab[0];
    int64_t nxt = stab[1];
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.f;
    const int64_t H = a.H;
    // token t's row of dO joins the running sum of its entry; an entry is
    // flushed when the next one starts
    auto add_token = [&](int64_t t, const float (&x)[8]) {
        if (t >= nxt) {
            flush_entry<DT, G, MODE>(a, h, c, slot0 + ls, beg >= tb && nxt <= te, s);
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = 0.f;
            ++ls;
            beg = nxt;
            nxt = stab[ls + 1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += x[e];
    };
    if constexpr (DT == 0) {
        // bf16: buffer loads over this workgroup's chunk (a lane offset and a
        // uniform offset per token), batches of UB tokens double-buffered: the
        // loads of batch b+1 are in flight while batch b is summed
        constexpr int UB = LH_SCATTER_U;
        const int64_t base0 = (tb * H + (int64_t)blockIdx.y * a.HG) * d;
        const uint32_t chunk_bytes = (uint32_t)((((int64_t)a.tok - 1) * H + a.HG) * d * 2);
        const uint32_t tstride = (uint32_t)(H * d * 2);
        const uint32_t lane_off = (uint32_t)((hl * d + c * 8) * 2);
        const auto R = make_rsrc(reinterpret_cast<const uint16_t*>(a.dout) + base0, chunk_bytes);
        auto issue = [&](u32x4* r, int i0, auto Uc) {
            constexpr int U = decltype(Uc)::value;
#pragma unroll
            for (int u = 0; u < U; ++u) r[u] = buf_ld16_nt(R, lane_off, (uint32_t)(i0 + u) * tstride);
        };
        auto consume_batch = [&](const u32x4* r, int i0, auto Uc) {
            constexpr int U = decltype(Uc)::value;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float x[8];
                unpack8(r[u], x);
                add_token(tb + i0 + u, x);
            }
        };
        using UBc = std::integral_constant<int, UB>;
        const int iters = a.tok;
        const int nb = iters / UB;
        u32x4 ra[UB], rb[UB];
        // (no branch between a prefetch and the consume after it, so the waits stay exact)
        if (nb > 0) issue(ra, 0, UBc{});
        int b = 0;
        for (; b + 2 < nb; b += 2) {
            issue(rb, (b + 1) * UB, UBc{});
            __builtin_amdgcn_sched_barrier(0);
            consume_batch(ra, b * UB, UBc{});
            issue(ra, (b + 2) * UB, UBc{});
            __builtin_amdgcn_sched_barrier(0);
            consume_batch(rb, (b + 1) * UB, UBc{});
        }
        if (b + 1 < nb) {
            issue(rb, (b + 1) * UB, UBc{});
            __builtin_amdgcn_sched_barrier(0);
            consume_batch(ra, b * UB, UBc{});
            consume_batch(rb, (b + 1) * UB, UBc{});
        } else if (b < nb) {
            consume_batch(ra, b * UB, UBc{});
        }
        for (int i = nb * UB; i < iters; ++i) {
            issue(ra, i, std::integral_constant<int, 1>{});
            consume_batch(ra, i, std::integral_constant<int, 1>{});
        }
    } else {
        constexpr int U = 8;
        for (int64_t t0 = tb; t0 < te; t0 += U) {
            float x[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (t0 + u < te) load8_nt<DT>(a.dout, ((t0 + u) * H + h) * d + c * 8, x[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (t0 + u < te) add_token(t0 + u, x[u]);
        }
    }
    flush_entry<DT, G, MODE>(a, h, c, slot0 + ls, beg >= tb && nxt <= te, s);
}

// Adjoint of gather + mean-pool: dX[t][h] = dX~[h][slot_h(t)] / p^level.
struct PoolBwdArgs {
    const int32_t* start;
    const uint8_t* level;
    const float *dqs, *dks, *dvs;   // fp32 [H][Sp][d]
    void *dq, *dk, *dv;             // dtype [N][H][d]
    int64_t N, S, Sp;
    int H, HG, mt, p;
};

template <int DT, int G>
__global__ void __launch_bounds__(256) k_pool_bwd(PoolBwdArgs a) {
    constexpr int d = G * 8;
    const TokMap tm = tok_map<G>(a.HG, a.mt, a.N);
    if (tm.tb >= tm.te) return;
    const int32_t* st = a.start + (int64_t)tm.h * a.S;
    int64_t slot = find_slot(st, a.S, tm.tb);
    int64_t nxt = slot + 1 < a.S ? st[slot + 1] : a.N;
    float g[3][8];
    const float* srcs[3] = {a.dqs, a.dks, a.dvs};
    void* dsts[3] = {a.dq, a.dk, a.dv};
    auto load_slot = [&](int64_t sl) {
        const int lv = a.level[(int64_t)tm.h * a.S + sl];
        float den = 1.0f;
        for (int z = 0; z < lv; ++z) den *= (float)a.p;
        const int64_t el = ((int64_t)tm.h * a.Sp + sl) * d + tm.c * 8;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            load8f(srcs[t], el, g[t]);
            if (lv > 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) g[t][e] = g[t][e] / den;
            }
        }
    };
    load_slot(slot);
    const int64_t H = a.H;
    for (int64_t t = tm.tb; t < tm.te; ++t) {
        if (t >= nxt) {
            ++slot;
            nxt = slot + 1 < a.S ? st[slot + 1] : a.N;
            load_slot(slot);
        }
        const int64_t el = (t * H + tm.h) * d + tm.c * 8;
#pragma unroll
        for (int z = 0; z < 3; ++z) store8<DT, true>(dsts[z], el, g[z]);
    }
}

__global__ void k_fill_zero(u32x4* p, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = u32x4{0, 0, 0, 0};
}

// ------------------------------------------------------------------ launchers

// Heads per workgroup: the largest divisor of H with HG * G <= 256 threads.
static int head_group(int H, int G) {
    int hg = 1;
    for (int c = 1; c <= H; ++c)
        if (H % c == 0 && c * G <= 256) hg = c;
    return hg;
}

static int pick_mt(int rows_threads, int limit) {
    // token lanes per workgroup: largest power of two keeping <= 256 threads
    int mt = 1;
    while (rows_threads * mt * 2 <= 256 && mt * 2 <= limit) mt *= 2;
    return mt;
}

// ------------------------------------------------ overlapping entries
// The "parent kept" reading of the selection (Fig. 2 step 3): a selected entry
// stays in the sub-sequence beside its p children, so up to L kept entries
// cover a token, one per level.  lmap[l][h][j] holds 1 + the slot of entry
// (level l, index j) when it is kept, else 0.

// out[z][t][h] = sum over the kept entries covering t of tab[z][h][slot], each
// divided by p^level when `divide` (z = 1: the scatter of O~; z = 3: the pool
// adjoint of dQ~, dK~, dV~, one tensor per workgroup).  fp32 tables, one
// rounding to bf16.  Threads walk tokens like the partition's row copy: the
// entries covering the first token come from the level maps; after that a
// cursor over the position-sorted slots enters each entry where it starts (its
// row is loaded once, into the register row of its level) and an entry leaves
// at its end, so rows are read once per entry and thread, not per token.
struct SumCopyArgs {
    const int32_t* lmap;          // [sum_l H * n_l] int32, level l at lmap_off[l]
    const int32_t* start;         // [H][S]
    const uint8_t* level;         // [H][S]
    const float* tab[3];          // fp32 [H][Sp][d]
    uint16_t* out[3];             // bf16; token t, head h at element t * ld + h * d
    int64_t lmap_off[kMaxLevels];
    int64_t n[kMaxLevels], pw[kMaxLevels];
    float scale[kMaxLevels];      // 1 / p^l, or 1
    int64_t N, S, Sp, ld;
    int H, HG, mt, L;
};

template <int G, int LMAX>
__global__ void __launch_bounds__(256) k_sum_copy(SumCopyArgs a) {
    constexpr int d = G * 8;
    const TokMap tm = tok_map<G>(a.HG, a.mt, a.N);
    if (tm.tb >= tm.te) return;
    const int z = blockIdx.z;
    const int h = tm.h;
    const int32_t* st = a.start + (int64_t)h * a.S;
    const uint8_t* lv = a.level + (int64_t)h * a.S;
    const float* tab = a.tab[z] + (int64_t)h * a.Sp * d + 8 * tm.c;
    uint16_t* ob = a.out[z] + (int64_t)h * d + 8 * tm.c;
    float row[LMAX][8];
    int64_t end[LMAX];   // first token after the active entry of each level (<= tm.tb: none)
    int64_t j = tm.tb;
#pragma unroll
    for (int l = 0; l < LMAX; ++l) {
        end[l] = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) row[l][e] = 0.f;
        if (l < a.L) {
            const int32_t s1 = a.lmap[a.lmap_off[l] + (int64_t)h * a.n[l] + j];
            if (s1 != 0) {
                load8f(tab, (int64_t)(s1 - 1) * d, row[l]);
#pragma unroll
                for (int e = 0; e < 8; ++e) row[l][e] *= a.scale[l];
                end[l] = (j + 1) * a.pw[l];
            }
            j /= a.pw[l + 1 < a.L ? l + 1 : l] / a.pw[l];
        }
    }
    int64_t cur = find_slot(st, a.S, tm.tb) + 1;   // first slot starting after tm.tb
    int64_t nstart = cur < a.S ? st[cur] : a.N;
    for (int64_t t = tm.tb; t < tm.te; ++t) {
        while (nstart <= t) {   // entries that start at t, coarser first
            const int l = lv[cur];
            float x[8];
            load8f(tab, cur * d, x);
#pragma unroll
            for (int q = 0; q < LMAX; ++q) {
                if (q == l) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) row[q][e] = x[e] * a.scale[q];
                    end[q] = t + a.pw[q];
                }
            }
            ++cur;
            nstart = cur < a.S ? st[cur] : a.N;
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int l = 0; l < LMAX; ++l)
            if (t < end[l]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += row[l][e];
            }
        u32x4 w;
        w[0] = pack_bf16x2(acc[0], acc[1]);
        w[1] = pack_bf16x2(acc[2], acc[3]);
        w[2] = pack_bf16x2(acc[4], acc[5]);
        w[3] = pack_bf16x2(acc[6], acc[7]);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(ob + t * a.ld));
    }
}

// Adjoint of the summed scatter: acc[h][slot] = sum of dO over the p^level
// tokens of the entry, fp32 (the layout the row preparation reads as fp32
// accumulators).  One wavefront per (head, slot): 64 / G token rows per step,
// lane group r takes rows r, r + 64/G, ...; the row groups are added with
// xor shuffles at the end.  Every slot is summed by one wavefront in a fixed
// order, so the result is the same on every run.
struct EntrySumArgs {
    const int32_t* start;   // [H][S]
    const uint8_t* level;   // [H][S]
    const uint16_t* dout;   // bf16 [N][H][d]
    float* acc;             // fp32 [H][Sp][d]
    int64_t S, Sp, pw[kMaxLevels];
    int H;
};

template <int G>
__global__ void __launch_bounds__(256) k_entry_sum(EntrySumArgs a) {
    constexpr int d = G * 8, R = 64 / G;
    const int lane = threadIdx.x & 63;
    const int64_t slot = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int h = blockIdx.y;
    if (slot >= a.S) return;
    const int c = lane % G, r = lane / G;
    const int64_t t0 = a.start[(int64_t)h * a.S + slot];
    const int64_t len = a.pw[a.level[(int64_t)h * a.S + slot]];
    float acc[8];
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    // four rows per lane group in flight; the order of the additions is fixed
    constexpr int U = 4;
    int64_t t = t0 + r;
    for (; t + (U - 1) * R < t0 + len; t += U * R) {
        float x[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load8<0>(a.dout, ((t + u * R) * a.H + h) * d + 8 * c, x[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += x[u][e];
    }
    for (; t < t0 + len; t += R) {
        float x[8];
        load8<0>(a.dout, (t * a.H + h) * d + 8 * c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += shfl_xor_f(acc[e], off);
    if (r == 0) store8f(a.acc, ((int64_t)h * a.Sp + slot) * d + 8 * c, acc);
}

hipError_t launch_pool_score(const Plan& P, const void* q, const void* k, const void* v, char* ws,
                             hipStream_t s) {
    PoolScoreArgs a{};
    a.q = q; a.k = k; a.v = v;
    float* sc = reinterpret_cast<float*>(ws + P.off_scores);
    for (int l = 0; l < P.L; ++l) {
        a.lev[l] = sc + P.lev_off[l];
        a.n[l] = P.n[l];
        a.pw[l] = P.pw[l];
    }
    a.pool_m = reinterpret_cast<float*>(ws + P.off_pool_m);
    a.N = P.N; a.H = P.H; a.p = P.p; a.m = P.m; a.tok = (int)P.tok;
    a.score_mode = P.score_mode;
    // level 0 is read by the selection only when it is the top level, and by
    // the upper pooling pass only when it is the level this pass ends at
    a.store_l0 = (P.keep_leaves || P.L == 1 || P.m == 0) ? 1 : 0;
    a.ld = P.in_ld;
    const int G = P.d / 8;
    a.HG = head_group(P.H, G);
    // token lanes must divide tok (a power of p): use powers of p
    int mt = 1;
    while (a.HG * G * mt * P.p <= 256 && mt * P.p <= P.tok) mt *= P.p;
    a.mt = mt;
    const int threads = a.HG * G * mt;
    // leaf scores [HG][tok], the level buffer [HG][tok/p], the mean partials [mt][HG][d]
    size_t lds = sizeof(float) * (size_t)P.tok * a.HG;
    if (P.m >= 1) lds += sizeof(float) * (size_t)(P.tok / P.p) * a.HG;
    if (P.m >= 1 && mt > 1) lds += sizeof(float) * (size_t)mt * a.HG * P.d;
    // Chunks per workgroup: up to LH_POOL_NG side by side, so that one workgroup fills a
    // CU.  Workgroups sharing a CU progress unevenly (the oldest is served first) and
    // their result stores then trickle into the read stream, where writes cost several
    // times their bytes; with one workgroup per CU they all finish together.
    const int64_t nchunks = P.N / P.tok;
    int ng = 1;
    while (threads % 64 == 0 && ng * 2 <= LH_POOL_NG && ng * 2 * threads <= 1024 && nchunks % (ng * 2) == 0 &&
           (size_t)(ng * 2) * lds <= 96 * 1024)
        ng *= 2;
    a.tpc = threads;
    a.lds_chunk = (int)(lds / sizeof(float));
    lds *= (size_t)ng;
    dim3 grid((unsigned)(nchunks / ng), (unsigned)(P.H / a.HG));
    if (P.dtype == BF16) {
        if (G == 16) hipLaunchKernelGGL((k_pool_score<0, 16>), grid, dim3(threads * ng), lds, s, a);
        else hipLaunchKernelGGL((k_pool_score<0, 8>), grid, dim3(threads * ng), lds, s, a);
    } else {
        if (G == 16) hipLaunchKernelGGL((k_pool_score<1, 16>), grid, dim3(threads * ng), lds, s, a);
        else hipLaunchKernelGGL((k_pool_score<1, 8>), grid, dim3(threads * ng), lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_pool_up(const Plan& P, char* ws, hipStream_t s) {
    PoolUpArgs a{};
    float* sc = reinterpret_cast<float*>(ws + P.off_scores);
    for (int l = 0; l < P.L; ++l) {
        a.lev[l] = sc + P.lev_off[l];
        a.n[l] = P.n[l];
        a.pw[l] = P.pw[l];
    }
    a.pool_m = reinterpret_cast<const float*>(ws + P.off_pool_m);
    a.pool_top = reinterpret_cast<float*>(ws + P.off_pool_top);
    a.H = P.H; a.d = P.d; a.p = P.p; a.m = P.m; a.L = P.L;
    hipLaunchKernelGGL(k_pool_up, dim3((unsigned)P.ntop), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gather(const Plan& P, const void* q, const void* k, const void* v, char* ws,
                         hipStream_t s) {
    GatherArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.pool_m = reinterpret_cast<const float*>(ws + P.off_pool_m);
    a.pool_top = reinterpret_cast<const float*>(ws + P.off_pool_top);
    a.start = reinterpret_cast<const int32_t*>(ws + P.off_start);
    a.level = reinterpret_cast<const uint8_t*>(ws + P.off_level);
    a.qs = reinterpret_cast<float*>(ws + P.off_qs);
    a.ks = reinterpret_cast<float*>(ws + P.off_ks);
    a.vs = reinterpret_cast<float*>(ws + P.off_vs);
    a.rowmax = reinterpret_cast<float*>(ws + P.off_rowmax);
    a.S = P.S; a.Sp = P.Sp; a.n_m = P.n[P.m]; a.ntop = P.ntop;
    a.ld = P.in_ld;
    for (int l = 0; l < P.L; ++l) a.pw[l] = P.pw[l];
    a.H = P.H; a.m = P.m; a.L = P.L;
    dim3 grid((unsigned)P.Sp, (unsigned)P.H);
    const int G = P.d / 8;
    if (P.dtype == BF16) {
        if (G == 16) hipLaunchKernelGGL((k_gather<0, 16>), grid, dim3(64), 0, s, a);
        else hipLaunchKernelGGL((k_gather<0, 8>), grid, dim3(64), 0, s, a);
    } else {
        if (G == 16) hipLaunchKernelGGL((k_gather<1, 16>), grid, dim3(64), 0, s, a);
        else hipLaunchKernelGGL((k_gather<1, 8>), grid, dim3(64), 0, s, a);
    }
    return hipGetLastError();
}

static int scatter_threads(const Plan& P, int* hg_out, int* mt_out) {
    const int G = P.d / 8;
    const int hg = head_group(P.H, G);
    const int mt = pick_mt(hg * G, kTileTok);
    *hg_out = hg;
    *mt_out = mt;
    return hg * G * mt;
}

hipError_t launch_scatter_fwd(const Plan& P, char* ws, void* o, hipStream_t s) {
    ScatterArgs a{};
    a.start = reinterpret_cast<const int32_t*>(ws + P.off_start);
    a.src = reinterpret_cast<const float*>(ws + P.off_os);
    a.dst = o;
    a.N = P.N; a.S = P.S; a.Sp = P.Sp; a.H = P.H;
    const int threads = scatter_threads(P, &a.HG, &a.mt);
    dim3 grid((unsigned)((P.N + kTileTok - 1) / kTileTok), (unsigned)(P.H / a.HG));
    const int G = P.d / 8;
    if (P.dtype == BF16) {
        if (G == 16) hipLaunchKernelGGL((k_scatter_fwd<0, 16>), grid, dim3(threads), 0, s, a);
        else hipLaunchKernelGGL((k_scatter_fwd<0, 8>), grid, dim3(threads), 0, s, a);
    } else {
        if (G == 16) hipLaunchKernelGGL((k_scatter_fwd<1, 16>), grid, dim3(threads), 0, s, a);
        else hipLaunchKernelGGL((k_scatter_fwd<1, 8>), grid, dim3(threads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<u32x4*>(p), n16);
    return hipGetLastError();
}

hipError_t launch_scatter_bwd(const Plan& P, const void* dout, int mode, char* ws, hipStream_t s) {
    ScatterBwdArgs a{};
    a.start = reinterpret_cast<const int32_t*>(ws + P.off_start);
    a.dout = dout;
    a.acc = reinterpret_cast<float*>(ws + P.off_acc);
    a.part = reinterpret_cast<float*>(ws + P.off_part);
    a.N = P.N; a.S = P.S; a.Sp = P.Sp; a.H = P.H; a.tok = P.tok;
    const int G = P.d / 8;
    a.HG = head_group(P.H, G);
    const int threads = a.HG * G;
    dim3 grid((unsigned)(P.N / P.tok), (unsigned)(P.H / a.HG));
    const size_t lds = (size_t)a.HG * (size_t)(P.tok + 2) * sizeof(int32_t);   // entry starts per head
#define LH_SB(DT, GG, MD) hipLaunchKernelGGL((k_scatter_bwd<DT, GG, MD>), grid, dim3(threads), lds, s, a)
    if (P.dtype == BF16) {
        if (G == 16) { if (mode == 0) LH_SB(0, 16, 0); else LH_SB(0, 16, 1); }
        else { if (mode == 0) LH_SB(0, 8, 0); else LH_SB(0, 8, 1); }
    } else {
        if (G == 16) { if (mode == 0) LH_SB(1, 16, 0); else LH_SB(1, 16, 1); }
        else { if (mode == 0) LH_SB(1, 8, 0); else LH_SB(1, 8, 1); }
    }
#undef LH_SB
    return hipGetLastError();
}

hipError_t launch_pool_bwd(const Plan& P, char* ws, void* dq, void* dk, void* dv, hipStream_t s) {
    PoolBwdArgs a{};
    a.start = reinterpret_cast<const int32_t*>(ws + P.off_start);
    a.level = reinterpret_cast<const uint8_t*>(ws + P.off_level);
    a.dqs = reinterpret_cast<const float*>(ws + P.off_dq);
    a.dks = reinterpret_cast<const float*>(ws + P.off_dk);
    a.dvs = reinterpret_cast<const float*>(ws + P.off_dv);
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.N = P.N; a.S = P.S; a.Sp = P.Sp; a.H = P.H; a.p = P.p;
    const int threads = scatter_threads(P, &a.HG, &a.mt);
    dim3 grid((unsigned)((P.N + kTileTok - 1) / kTileTok), (unsigned)(P.H / a.HG));
    const int G = P.d / 8;
    if (P.dtype == BF16) {
        if (G == 16) hipLaunchKernelGGL((k_pool_bwd<0, 16>), grid, dim3(threads), 0, s, a);
        else hipLaunchKernelGGL((k_pool_bwd<0, 8>), grid, dim3(threads), 0, s, a);
    } else {
        if (G == 16) hipLaunchKernelGGL((k_pool_bwd<1, 16>), grid, dim3(threads), 0, s, a);
        else hipLaunchKernelGGL((k_pool_bwd<1, 8>), grid, dim3(threads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_sum_copy(const Plan& P, const char* ws, const float* const* tab, void* const* out, int Z,
                           bool divide, int64_t out_ld, hipStream_t s) {
    if (Z < 1 || Z > 3 || P.dtype != BF16 || !P.pk) return hipErrorInvalidValue;
    if (out_ld < (int64_t)P.H * P.d || out_ld % 8 != 0) return hipErrorInvalidValue;
    SumCopyArgs a{};
    a.lmap = reinterpret_cast<const int32_t*>(ws + P.off_lmap);
    a.start = reinterpret_cast<const int32_t*>(ws + P.off_start);
    a.level = reinterpret_cast<const uint8_t*>(ws + P.off_level);
    for (int z = 0; z < Z; ++z) {
        a.tab[z] = tab[z];
        a.out[z] = reinterpret_cast<uint16_t*>(out[z]);
    }
    for (int l = 0; l < P.L; ++l) {
        a.lmap_off[l] = (int64_t)P.lmap_off[l];
        a.n[l] = P.n[l];
        a.pw[l] = P.pw[l];
        a.scale[l] = divide ? 1.0f / (float)P.pw[l] : 1.0f;
    }
    a.N = P.N; a.S = P.S; a.Sp = P.Sp; a.ld = out_ld;
    a.H = P.H; a.L = P.L;
    const int G = P.d / 8;
    const int threads = scatter_threads(P, &a.HG, &a.mt);
    dim3 grid((unsigned)((P.N + kTileTok - 1) / kTileTok), (unsigned)(P.H / a.HG), (unsigned)Z);
#define LH_SUMC(GG, LM) hipLaunchKernelGGL((k_sum_copy<GG, LM>), grid, dim3(threads), 0, s, a)
    if (P.L <= 6) {
        if (G == 16) LH_SUMC(16, 6); else LH_SUMC(8, 6);
    } else if (P.L <= 12) {
        if (G == 16) LH_SUMC(16, 12); else LH_SUMC(8, 12);
    } else {
        if (G == 16) LH_SUMC(16, kMaxLevels); else LH_SUMC(8, kMaxLevels);
    }
#undef LH_SUMC
    return hipGetLastError();
}

hipError_t launch_entry_sum(const Plan& P, const void* dout, char* ws, hipStream_t s) {
    if (P.dtype != BF16 || !P.pk) return hipErrorInvalidValue;
    EntrySumArgs a{};
    a.start = reinterpret_cast<const int32_t*>(ws + P.off_start);
    a.level = reinterpret_cast<const uint8_t*>(ws + P.off_level);
    a.dout = reinterpret_cast<const uint16_t*>(dout);
    a.acc = reinterpret_cast<float*>(ws + P.off_acc);
    a.S = P.S; a.Sp = P.Sp; a.H = P.H;
    for (int l = 0; l < P.L; ++l) a.pw[l] = P.pw[l];
    if (P.S == 0) return hipSuccess;
    dim3 grid((unsigned)((P.S + 3) / 4), (unsigned)P.H);
    if (P.d == 128) hipLaunchKernelGGL((k_entry_sum<16>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_entry_sum<8>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace lh
