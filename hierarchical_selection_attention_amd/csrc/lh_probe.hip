// Achievable-peak probes, reported beside the vendor peaks so that a stage's
// fraction of peak can be read against what a plain kernel reaches on the same
// GPU.  They are not part of the layer.  Streams use the pattern the layer's
// streaming stages use: each workgroup owns a contiguous chunk (1 MiB to read
// or copy, 256 KiB to write) and moves it in 16-byte non-temporal accesses.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

namespace {

constexpr int64_t kChunk16 = 65536;   // 16-byte words per workgroup (1 MiB)
constexpr size_t kMfmaRoundRecord = 3072;   // bytes per trial of the rounding probe
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr int kInFlight = 8;

// XOR-fold v over the workgroup and store it to this workgroup's 16 bytes of
// out (no atomics: one shared word would serialise every workgroup's update).
__device__ __forceinline__ void fold_out(u32x4 v, unsigned* out) {
    __shared__ unsigned red[4][4];
    unsigned x[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] ^= (unsigned)__shfl_xor((int)x[j], off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][j] = x[j];
    __syncthreads();
    if (threadIdx.x < 4) {
        unsigned t = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t ^= red[w][threadIdx.x];
        out[4 * (size_t)blockIdx.x + threadIdx.x] = t;
    }
}

// kind 0: read n16 words, fold them into out; kind 2: copy them to dst.  Full
// batches of kInFlight loads per lane are unconditional; the ragged end of
// the last chunk takes a guarded loop.
template <bool COPY>
__global__ void __launch_bounds__(256) k_probe_stream(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                      int64_t n16, unsigned* out) {
    const int64_t b0 = (int64_t)blockIdx.x * kChunk16;
    const int64_t b1 = b0 + kChunk16 < n16 ? b0 + kChunk16 : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = b0 + threadIdx.x;
    for (; i + (int64_t)(kInFlight - 1) * 256 < b1; i += 256 * kInFlight) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + (int64_t)u * 256);
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            if constexpr (COPY) __builtin_nontemporal_store(v[u], dst + i + (int64_t)u * 256);
            else acc ^= v[u];
        }
    }
    for (; i < b1; i += 256) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        if constexpr (COPY) __builtin_nontemporal_store(v, dst + i);
        else acc ^= v;
    }
    if constexpr (!COPY) fold_out(acc, out);
}

// kind 1: write a fixed pattern over n16 words, 256 KiB per workgroup
constexpr int64_t kWriteChunk16 = 16384;
__global__ void __launch_bounds__(256) k_probe_write(u32x4* __restrict__ dst, int64_t n16) {
    const int64_t b0 = (int64_t)blockIdx.x * kWriteChunk16;
    const int64_t b1 = b0 + kWriteChunk16 < n16 ? b0 + kWriteChunk16 : n16;
    const u32x4 z = {0x3f800000u, (unsigned)blockIdx.x, (unsigned)threadIdx.x, 0u};
    for (int64_t i = b0 + threadIdx.x; i < b1; i += 256) __builtin_nontemporal_store(z, dst + i);
}

// kind 5: the token-row write pattern of the attention kernels' scatter: bf16
// rows [T][16 heads][128], each workgroup writing one head's 256-byte pieces
// (4 KiB apart) for 16384 consecutive tokens (4 MiB, about what one work item
// of the backward writes), 16 tokens per pass of its 256 threads, one pointer
// step per store.  Thread t's store i goes to token tb + t / 16 + 16 i, chunk
// t % 16; its value is {1.0f bits, workgroup, thread, 0}.  n16 is a multiple of
// 16 heads x 16384 tokens x 16 words.
constexpr int kTokHeads = 16, kTokPerWg = 16384;
__global__ void __launch_bounds__(256) k_probe_token_write(u32x4* __restrict__ dst) {
    const int64_t g = blockIdx.x;
    const int h = (int)(g % kTokHeads);
    const int64_t tb = (g / kTokHeads) * kTokPerWg;
    const int c = threadIdx.x % 16;
    const u32x4 z = {0x3f800000u, (unsigned)blockIdx.x, (unsigned)threadIdx.x, 0u};
    u32x4* p = dst + ((tb + threadIdx.x / 16) * kTokHeads + h) * 16 + c;
    const int64_t step = (int64_t)16 * kTokHeads * 16;   // 16 tokens, in 16-byte words
    for (int i = 0; i < kTokPerWg / 16; ++i, p += step) __builtin_nontemporal_store(z, p);
}

// kind 3: every wave issues `iters` rounds of 4 independent
// v_mfma_f32_32x32x16_bf16 on register operands (32768 flops each); four
// accumulation chains per wave keep the matrix pipe full
__global__ void __launch_bounds__(256) k_probe_mfma(int iters, unsigned* out) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
        b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e & 3] += acc[j][e];
    fold_out(u32x4{__float_as_uint(t[0]), __float_as_uint(t[1]), __float_as_uint(t[2]), __float_as_uint(t[3])}, out);
}

// kind 4: one v_mfma_f32_16x16x32_f16 per trial, one wavefront per trial, on
// operands from memory (a record of 64 lanes x 8 fp16 A values, 64 x 8 fp16
// B values and 64 x 4 fp32 accumulator values); the 64 x 4 results go to dst.
// Lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16] for
// e < 8, and holds C and D at rows 4 (l / 16) + r, column l % 16, for r < 4.
__global__ void __launch_bounds__(64) k_probe_mfma_round(const unsigned char* __restrict__ src, float* __restrict__ dst) {
    const int lane = threadIdx.x;
    const unsigned char* rec = src + (size_t)blockIdx.x * kMfmaRoundRecord;
    const f16x8 a = *reinterpret_cast<const f16x8*>(rec + 16 * lane);
    const f16x8 b = *reinterpret_cast<const f16x8*>(rec + 1024 + 16 * lane);
    const f32x4 c = *reinterpret_cast<const f32x4*>(rec + 2048 + 16 * lane);
    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    *reinterpret_cast<f32x4*>(dst + ((size_t)blockIdx.x * 64 + lane) * 4) = d;
}

}  // namespace

// Grid of the MFMA probe: 4 waves per workgroup, 4 workgroups per CU of 256.
constexpr int kMfmaGrid = 1024;
static_assert(kMfmaGrid * 4 == 4096, "the header documents 4096 wavefronts");

hipError_t launch_peak_probe(int kind, const void* src, void* dst, size_t n, hipStream_t s) {
    if (kind == 4) {
        hipLaunchKernelGGL(k_probe_mfma_round, dim3((unsigned)n), dim3(64), 0, s,
                           reinterpret_cast<const unsigned char*>(src), reinterpret_cast<float*>(dst));
        return hipGetLastError();
    }
    if (kind == 3) {
        hipLaunchKernelGGL(k_probe_mfma, dim3(kMfmaGrid), dim3(256), 0, s, (int)n, reinterpret_cast<unsigned*>(dst));
        return hipGetLastError();
    }
    if (kind == 5) {
        const int64_t words = (int64_t)(n / 16);
        hipLaunchKernelGGL(k_probe_token_write, dim3((unsigned)(words / (16 * kTokPerWg))), dim3(256), 0, s,
                           reinterpret_cast<u32x4*>(dst));
        return hipGetLastError();
    }
    const int64_t n16 = (int64_t)(n / 16);
    const int64_t chunk = kind == 1 ? kWriteChunk16 : kChunk16;
    const dim3 grid((unsigned)((n16 + chunk - 1) / chunk));
    const u32x4* in = reinterpret_cast<const u32x4*>(src);
    u32x4* o = reinterpret_cast<u32x4*>(dst);
    if (kind == 0) hipLaunchKernelGGL((k_probe_stream<false>), grid, dim3(256), 0, s, in, o, n16,
                                      reinterpret_cast<unsigned*>(dst));
    else if (kind == 1) hipLaunchKernelGGL(k_probe_write, grid, dim3(256), 0, s, o, n16);
    else hipLaunchKernelGGL((k_probe_stream<true>), grid, dim3(256), 0, s, in, o, n16, nullptr);
    return hipGetLastError();
}

}  // namespace lh
