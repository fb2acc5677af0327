// Operand preparation for the attention kernels on gfx950: per-head scale
// exponents, fp16 hi/lo row splits, and the per-row
// quantities of the backward pass (D_i, and for the dense path the base-2 lse).
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

// ---------------------------------------------------------------- max |x|
// Per-head maximum of |x| over [rows][d] (fp32 [H][Sp][d] or bf16 rows with
// strides), accumulated as float bits with atomicMax (values are >= 0), for up
// to three tensors of the same layout (tensor blockIdx.z).
struct MaxAbsArgs {
    const void* src[3];
    unsigned int* out[3];   // [H][4] word of the tensor's slot
    int64_t ld, hs, rows;
    int d;
};
template <int SRC_BF16>
__global__ void __launch_bounds__(256) k_maxabs(MaxAbsArgs a) {
    const int h = blockIdx.y, t = blockIdx.z;
    const void* src = a.src[t];
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int G = a.d / 8;
    float mx = 0.f;
    for (int idx = threadIdx.x; idx < 64 * G; idx += 256) {
        const int64_t r = r0 + idx / G;
        if (r >= a.rows) break;
        float x[8];
        const int64_t el = h * a.hs + r * a.ld + (idx % G) * 8;
        if constexpr (SRC_BF16) load8<0>(src, el, x);
        else load8f(reinterpret_cast<const float*>(src), el, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[e]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
    __shared__ float wm[4];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float m = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
        atomicMax(a.out[t] + h * 4, __float_as_uint(m));
    }
}

// Per-head maximum of per-row maxima: out[t][h * 4] = max over rows of
// rowmax[t][h][0..rows), as float bits (values are >= 0).  One workgroup per
// (head, tensor); no atomics, so the words need no clearing first.
struct HeadMaxArgs {
    const float* rowmax;    // [T][H][rows_ld]
    unsigned int* out[4];   // [H][4] word of tensor t's slot
    int64_t rows, rows_ld;
    int H;
};
// 1024 threads, four independent loads in flight per thread per pass.
constexpr int kHeadMaxThreads = 1024;
__global__ void __launch_bounds__(kHeadMaxThreads) k_head_max(HeadMaxArgs a) {
    const int h = blockIdx.x, t = blockIdx.y;
    const float* r = a.rowmax + ((int64_t)t * a.H + h) * a.rows_ld;
    float mx = 0.f;
    for (int64_t i0 = threadIdx.x; i0 < a.rows; i0 += 4 * kHeadMaxThreads) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = i0 + (int64_t)u * kHeadMaxThreads;
            v[u] = i < a.rows ? r[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) mx = fmaxf(mx, v[u]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
    constexpr int NW = kHeadMaxThreads / 64;
    __shared__ float wm[NW];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = wm[0];
        for (int w = 1; w < NW; ++w) m = fmaxf(m, wm[w]);
        a.out[t][h * 4] = __float_as_uint(m);
    }
}

// Power of two s with max|x| * s in [2^13, 2^14) (1 when max is 0).
__device__ __forceinline__ float down_scale(float mx) {
    if (!(mx > 0.f)) return 1.0f;
    int ex;
    frexpf(mx, &ex);           // mx = f * 2^ex, f in [0.5, 1)
    return ldexpf(1.0f, 14 - ex);
}

// ---------------------------------------------------------------- splits
// One 64x64 tile of head h: x = src * down (down = power-of-two scale of the
// head); writes fp16 hi/lo rows.  Rows >= `rows` are written as zeros.
// Up to three tensors of the same layout per launch: blockIdx.z = tensor * H + head.
struct SplitArgs {
    const void* src[3];
    int64_t ld, hs, rows, Sp;
    int d, H, src_bf16;
    const unsigned int* hmax;   // [H][4], slot `slot`
    float* hscale;              // [H][4]: stored * hscale = true value
    int slot[3];
    uint16_t *rh[3], *rl[3];    // fp16 [H][Sp][d] (scaled); rl may be null
};

__device__ __forceinline__ uint16_t h16(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float f16f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__global__ void __launch_bounds__(256) k_split(SplitArgs a) {
    const int t = blockIdx.z / a.H, h = blockIdx.z % a.H;
    const void* src = a.src[t];
    uint16_t *rh = a.rh[t], *rl = a.rl[t];
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int c0 = blockIdx.y * 64;
    const float mx = __uint_as_float(a.hmax[h * 4 + a.slot[t]]);
    const float down = down_scale(mx);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.hscale[h * 4 + a.slot[t]] = 1.0f / down;
    // each thread: 2 (row, 8-column chunk) items of the 64x64 tile
    for (int it = threadIdx.x; it < 64 * 8; it += 256) {
        const int r = it / 8, cc = (it % 8) * 8;
        float x[8];
        if (r0 + r < a.rows) {
            const int64_t el = h * a.hs + (r0 + r) * a.ld + c0 + cc;
            if (a.src_bf16) load8<0>(src, el, x);
            else load8f(reinterpret_cast<const float*>(src), el, x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
        u32x4 wh, wl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = x[2 * e] * down, x1 = x[2 * e + 1] * down;
            const uint16_t h0 = h16(x0), h1 = h16(x1);
            wh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            wl[e] = (uint32_t)h16(x0 - f16f(h0)) | ((uint32_t)h16(x1 - f16f(h1)) << 16);
        }
        const int64_t o = ((int64_t)h * a.Sp + r0 + r) * a.d + c0 + cc;
        *reinterpret_cast<u32x4*>(rh + o) = wh;
        if (rl) *reinterpret_cast<u32x4*>(rl + o) = wl;
    }
}

// ---------------------------------------------------------- backward rows
// Per sub-sequence row: finish dO~ and D_i = <dO~_i, O~_i> in double; for the
// dense path also the base-2 lse minus the backward kernels' offset 14 (their
// weights are then P * 2^14).  dO~ of an entry is its row of `acc`, except in
// the deterministic mode for entries above level m: those are the sum, in
// block order and in double, of the entry's per-block partial sums.  In place
// (dos == acc), only the rows that change are written: those sums, and zeros
// for the padding rows S .. Sp-1.
struct RowPrepArgs {
    const void* acc;       // fp32 [H][Sp][d]; unused when dense
    const float* part;     // mode 1: fp32 [H][N / tok][d]
    const int32_t* start;  // [H][S]
    const uint8_t* level;  // [H][S]
    int64_t tok, nblk;
    int m, p;
    const void* dout;      // dense: bf16 rows with strides ld/hs
    const void* o;         // fp32 [H][Sp][d] attention output
    int64_t ld, hs;        // dense strides of dout
    float* dos;            // fp32 [H][Sp][d] finished dO~ (sub-sequence) or null
    float* D;              // [H][Sp]
    const float* lse_in;   // dense: natural-log lse [H][N], converted to base 2 in lse2
    float* lse2;
    float* rowmax;             // optional fp32 [H][Sp]: max |dO~| of each row
    int64_t S, Sp;
    int H, d, mode, dense;
    int in_place;              // dos is acc: store only the rows that change
};

template <int G>
__global__ void __launch_bounds__(256) k_row_prep(RowPrepArgs a) {
    constexpr int d = G * 8;
    const int c = threadIdx.x % G;
    const int64_t r = (int64_t)blockIdx.x * (256 / G) + threadIdx.x / G;   // over [H][Sp]
    const bool live = r < (int64_t)a.H * a.Sp;
    const int64_t h = live ? r / a.Sp : 0;
    const int64_t i = live ? r % a.Sp : 0;
    float x[8], o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = o[e] = 0.f;
    bool changed = i >= a.S;   // rows whose dO~ differs from what `acc` holds
    if (live && i < a.S) {
        if (a.dense) {
            load8<0>(a.dout, h * a.hs + i * a.ld + c * 8, x);
            load8f(reinterpret_cast<const float*>(a.o), r * d + c * 8, o);
        } else {
            const int64_t el = r * d + c * 8;
            const int lv = a.mode == 1 ? (int)a.level[h * a.S + i] : 0;
            if (lv > a.m) {
                changed = true;
                // p^(lv - m) blocks of tok tokens, from the entry's first one
                const int64_t b0 = a.start[h * a.S + i] / a.tok;
                int64_t nb = 1;
                for (int z = a.m; z < lv; ++z) nb *= a.p;
                double acc8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc8[e] = 0.0;
                for (int64_t b = 0; b < nb; ++b) {
                    float y[8];
                    load8f(a.part, (h * a.nblk + b0 + b) * d + c * 8, y);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc8[e] += (double)y[e];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (float)acc8[e];
            } else {
                load8f(reinterpret_cast<const float*>(a.acc), el, x);
            }
            load8f(reinterpret_cast<const float*>(a.o), el, o);
        }
    }
    if (live && a.dos && (changed || !a.in_place)) store8f(a.dos, r * d + c * 8, x);
    double dot = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fma((double)x[e], (double)o[e], dot);
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (a.rowmax) {   // the row's max |dO~| for the per-head scale of its 16-bit copies
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[e]));
#pragma unroll
        for (int off = G / 2; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
        if (live && c == 0) a.rowmax[r] = mx;
    }
    if (live && c == 0) {
        if (a.lse_in) a.lse2[r] = (float)((double)a.lse_in[r] * 1.4426950408889634 - 14.0);
        a.D[r] = (float)dot;
    }
}

__global__ void k_clear_slot(unsigned int* hmax, int H, int slot) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h < H) hmax[h * 4 + slot] = 0u;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_clear_slot(unsigned int* hmax, int H, int slot, hipStream_t s) {
    hipLaunchKernelGGL(k_clear_slot, dim3((unsigned)((H + 63) / 64)), dim3(64), 0, s, hmax, H, slot);
    return hipGetLastError();
}

hipError_t launch_maxabs(const void* const* src, unsigned int* const* out, int T, bool src_bf16, int64_t ld,
                         int64_t hs, int64_t rows, int d, int H, hipStream_t s) {
    if (T < 1 || T > 3) return hipErrorInvalidValue;
    MaxAbsArgs a{};
    for (int t = 0; t < T; ++t) {
        a.src[t] = src[t];
        a.out[t] = out[t];
    }
    a.ld = ld; a.hs = hs; a.rows = rows; a.d = d;
    dim3 grid((unsigned)((rows + 63) / 64), (unsigned)H, (unsigned)T);
    if (src_bf16) hipLaunchKernelGGL(k_maxabs<1>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_maxabs<0>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_split(const SplitSpec* sp, int T, hipStream_t s) {
    if (T < 1 || T > 3) return hipErrorInvalidValue;
    SplitArgs a{};
    const SplitSpec& s0 = sp[0];
    a.ld = s0.ld; a.hs = s0.hs; a.rows = s0.rows; a.Sp = s0.Sp;
    a.d = s0.d; a.H = s0.H; a.src_bf16 = s0.src_bf16; a.hmax = s0.hmax; a.hscale = s0.hscale;
    for (int t = 0; t < T; ++t) {
        const SplitSpec& x = sp[t];
        if (x.ld != s0.ld || x.hs != s0.hs || x.rows != s0.rows || x.Sp != s0.Sp || x.d != s0.d || x.H != s0.H ||
            x.src_bf16 != s0.src_bf16 || x.hmax != s0.hmax || x.hscale != s0.hscale)
            return hipErrorInvalidValue;
        a.src[t] = x.src; a.slot[t] = x.slot;
        if (!x.rh) return hipErrorInvalidValue;
        a.rh[t] = x.rh; a.rl[t] = x.rl;
    }
    dim3 grid((unsigned)(s0.Sp / 64), (unsigned)(s0.d / 64), (unsigned)(s0.H * T));
    hipLaunchKernelGGL(k_split, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_head_max(const float* rowmax, unsigned int* const* out, int T, int64_t rows, int64_t rows_ld,
                           int H, hipStream_t s) {
    if (T < 1 || T > 4 || rows < 0 || rows > rows_ld) return hipErrorInvalidValue;
    HeadMaxArgs a{};
    a.rowmax = rowmax;
    for (int t = 0; t < T; ++t) a.out[t] = out[t];
    a.rows = rows; a.rows_ld = rows_ld; a.H = H;
    hipLaunchKernelGGL(k_head_max, dim3((unsigned)H, (unsigned)T), dim3(kHeadMaxThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_row_prep(const RowPrepSpec& sp, hipStream_t s) {
    RowPrepArgs a{};
    a.acc = sp.acc; a.dout = sp.dout; a.o = sp.o; a.ld = sp.ld; a.hs = sp.hs;
    a.part = sp.part; a.start = sp.start; a.level = sp.level; a.tok = sp.tok > 0 ? sp.tok : 1;
    a.m = sp.m; a.p = sp.p; a.nblk = sp.nblk;
    a.dos = sp.dos; a.D = sp.D;
    a.lse_in = sp.lse_in; a.lse2 = sp.lse2; a.rowmax = sp.rowmax;
    a.S = sp.S; a.Sp = sp.Sp; a.H = sp.H; a.d = sp.d; a.mode = sp.mode; a.dense = sp.dense;
    a.in_place = sp.in_place;
    const int G = sp.d / 8;
    const int64_t rows = (int64_t)sp.H * sp.Sp;
    dim3 grid((unsigned)((rows + (256 / G) - 1) / (256 / G)));
    if (G == 16) hipLaunchKernelGGL(k_row_prep<16>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_row_prep<8>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace lh
