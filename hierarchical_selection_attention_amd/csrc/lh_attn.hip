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
// sequence position come from [H][d][Sp] transposed copies, so every operand
// load is one contiguous vector.
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16x8 ld_f16x8(const uint16_t* p) {
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 ld_b16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
// elements {4g..4g+3} and {16+4g..16+4g+3} of a 32-wide block of a transposed row
__device__ __forceinline__ u32x4 ld_split_raw(const uint16_t* p) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
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
    int64_t rows, Sp, ld_o, hs_o;
    float scale;            // 1/sqrt(d)
    // fp32 path (double arithmetic)
    const float *qf, *kf, *vf, *dof;
};

// ------------------------------------------------------------------ forward
template <int D, bool SPLIT>
__global__ void __launch_bounds__(256) k_attn_fwd(AttnK a) {
    constexpr int NS = D / 32, NV = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int h = blockIdx.y;
    const int64_t Sp = a.Sp;
    const int64_t qt = gridDim.x - 1 - blockIdx.x;   // longest rows first
    const int64_t q0 = qt * 64 + wave * 16;
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

    for (int64_t kb = 0; kb < q0 + 16; kb += 64) {
        f32x4 sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int64_t off = hb + (kb + 16 * u + lq) * D + 8 * lg;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const f16x8 kh = ld_f16x8(a.kh + off + 32 * s);
                sc[u] = mma_h(kh, qfh[s], sc[u]);
                if constexpr (SPLIT) {
                    sc[u] = mma_h(kh, qfl[s], sc[u]);
                    sc[u] = mma_h(ld_f16x8(a.kl + off + 32 * s), qfh[s], sc[u]);
                }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t key = kb + 16 * u + 4 * lg + r;
                float x = sc[u][r] * c2;
                x = key > myq ? -INFINITY : x;
                sc[u][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, shfl_xor_f(mx, 16));
        mx = fmaxf(mx, shfl_xor_f(mx, 32));
        const float mnew = fmaxf(m, mx);
        const float alpha = exp2f(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int v = 0; v < NV; ++v) o[v] *= alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pr = exp2f(sc[u][r] - m);
                lsum += pr;
                sc[u][r] = pr;
            }
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            f16x8 ph, pl;
            split_h(sc[2 * w], sc[2 * w + 1], ph, pl);
            const int64_t col = kb + 32 * w + 4 * lg;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int64_t off = hb + (int64_t)(16 * v + lq) * Sp + col;
                const f16x8 vh = __builtin_bit_cast(f16x8, ld_split_raw(a.vTh + off));
                o[v] = mma_h(vh, ph, o[v]);
                o[v] = mma_h(vh, pl, o[v]);
                if constexpr (SPLIT) o[v] = mma_h(__builtin_bit_cast(f16x8, ld_split_raw(a.vTl + off)), ph, o[v]);
            }
        }
    }
    lsum += shfl_xor_f(lsum, 16);
    lsum += shfl_xor_f(lsum, 32);
    const float mul = mv / lsum;
    // o[v][r] holds O^T[16v + 4g + r][myq]
    if (a.o) {
        float* O = a.o + hb + myq * D;
#pragma unroll
        for (int v = 0; v < NV; ++v) *reinterpret_cast<f32x4*>(O + 16 * v + 4 * lg) = o[v] * mul;
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
}

// ------------------------------------------------------- backward: dK, dV
// Key-stationary: wave w owns keys k0..k0+15 (lane column = key) and walks the
// query blocks at or after its keys.
template <int D, bool SPLIT, bool OUT_BF16>
__global__ void __launch_bounds__(256) k_attn_dkdv(AttnK a) {
    constexpr int NS = D / 32, NV = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int h = blockIdx.y;
    const int64_t Sp = a.Sp;
    const int64_t k0 = (int64_t)blockIdx.x * 64 + wave * 16;
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

    for (int64_t qb = k0 & ~(int64_t)31; qb < a.rows; qb += 32) {
        f32x4 P[2], dS[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
            const int64_t off = hb + (qb + 16 * u + lq) * D + 8 * lg;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const f16x8 qh = ld_f16x8(a.qh + off + 32 * st);
                const f16x8 oh = ld_f16x8(a.doh + off + 32 * st);
                s = mma_h(qh, kfh[st], s);
                dp = mma_h(oh, vfh[st], dp);
                if constexpr (SPLIT) {
                    s = mma_h(qh, kfl[st], s);
                    s = mma_h(ld_f16x8(a.ql + off + 32 * st), kfh[st], s);
                    dp = mma_h(oh, vfl[st], dp);
                    dp = mma_h(ld_f16x8(a.dol + off + 32 * st), vfh[st], dp);
                }
            }
            const int64_t qq = qb + 16 * u + 4 * lg;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + qq);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dv + qq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t q = qq + r;
                float pr = exp2f(s[r] * cS - l4[r]);
                pr = (q >= mykey && q < a.rows) ? pr : 0.f;
                P[u][r] = pr;
                dS[u][r] = pr * (dp[r] * cP - d4[r]);
            }
        }
        f16x8 ph, pl;
        split_h(P[0], P[1], ph, pl);
        bf16x8 sh, sl;
        split_b(dS[0], dS[1], sh, sl);
        const int64_t col = qb + 4 * lg;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int64_t off = hb + (int64_t)(16 * v + lq) * Sp + col;
            const f16x8 oth = __builtin_bit_cast(f16x8, ld_split_raw(a.doTh + off));
            dv[v] = mma_h(oth, ph, dv[v]);
            dv[v] = mma_h(oth, pl, dv[v]);
            const bf16x8 qth = __builtin_bit_cast(bf16x8, ld_split_raw(a.qTbh + off));
            dk[v] = mma_b(qth, sh, dk[v]);
            dk[v] = mma_b(qth, sl, dk[v]);
            if constexpr (SPLIT) {
                dv[v] = mma_h(__builtin_bit_cast(f16x8, ld_split_raw(a.doTl + off)), ph, dv[v]);
                dk[v] = mma_b(__builtin_bit_cast(bf16x8, ld_split_raw(a.qTbl + off)), sh, dk[v]);
            }
        }
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
                *reinterpret_cast<f32x4*>(a.dk + base + 16 * v) = dk[v] * a.scale;
                *reinterpret_cast<f32x4*>(a.dv + base + 16 * v) = dv[v] * mdo;
            }
        }
    }
}

// ---------------------------------------------------------- backward: dQ
// Query-stationary: wave w owns queries q0..q0+15 and walks the keys up to the
// diagonal.  dS rows are scaled down by a power of two (rowdown) before the
// fp16 split, so they cannot overflow; the scale is undone at the end.
template <int D, bool SPLIT, bool OUT_BF16>
__global__ void __launch_bounds__(256) k_attn_dq(AttnK a) {
    constexpr int NS = D / 32, NV = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lq = lane & 15, lg = lane >> 4;
    const int h = blockIdx.y;
    const int64_t Sp = a.Sp;
    const int64_t qt = gridDim.x - 1 - blockIdx.x;
    const int64_t q0 = qt * 64 + wave * 16;
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

    for (int64_t kb = 0; kb < q0 + 16; kb += 32) {
        f32x4 dS[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
            const int64_t off = hb + (kb + 16 * u + lq) * D + 8 * lg;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const f16x8 kh = ld_f16x8(a.kh + off + 32 * st);
                const f16x8 vh = ld_f16x8(a.vh + off + 32 * st);
                s = mma_h(kh, qfh[st], s);
                dp = mma_h(vh, dfh[st], dp);
                if constexpr (SPLIT) {
                    s = mma_h(kh, qfl[st], s);
                    s = mma_h(ld_f16x8(a.kl + off + 32 * st), qfh[st], s);
                    dp = mma_h(vh, dfl[st], dp);
                    dp = mma_h(ld_f16x8(a.vl + off + 32 * st), dfh[st], dp);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t key = kb + 16 * u + 4 * lg + r;
                float pr = exp2f(s[r] * cS - l2);
                pr = key <= myq ? pr : 0.f;
                dS[u][r] = pr * (dp[r] * cP - Dq) * down;
            }
        }
        f16x8 sh, sl;
        split_h(dS[0], dS[1], sh, sl);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int64_t off = hb + (int64_t)(16 * v + lq) * Sp + kb + 4 * lg;
            const f16x8 kth = __builtin_bit_cast(f16x8, ld_split_raw(a.kTh + off));
            dq[v] = mma_h(kth, sh, dq[v]);
            dq[v] = mma_h(kth, sl, dq[v]);
            if constexpr (SPLIT) dq[v] = mma_h(__builtin_bit_cast(f16x8, ld_split_raw(a.kTl + off)), sh, dq[v]);
        }
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
            for (int v = 0; v < NV; ++v) *reinterpret_cast<f32x4*>(a.dq + base + 16 * v) = dq[v] * mul;
        }
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
        dim3 grid((unsigned)(x.Sp / 64), (unsigned)x.H);
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
    dim3 grid((unsigned)(x.Sp / 64), (unsigned)x.H);
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
