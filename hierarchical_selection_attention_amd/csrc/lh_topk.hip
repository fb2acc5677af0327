// Hierarchical selector (stage (ii) of Sec. 3; Fig. 2 step 3 "bitonic argsort
// + tree-prune") on gfx950.  One workgroup of 1024 threads per head.
//
// From the top level down, the candidates of a level are scored by 64-bit
// keys (fp32 score bits << 32 | ~index): scores are >= +0 so the bit pattern
// orders them, and the complemented index makes equal scores rank the lower
// index first; keys are unique, so the K selected candidates are exactly those
// whose key is at least the K-th largest key.  That key is found by an
// MSB-first radix selection (eight 8-bit digits, a 256-bin LDS histogram per
// digit) -- the set an argsort would select, without sorting.  Selected
// entries are replaced by their p children, the others are kept; finally
// every kept entry gets its slot in the position-ordered sub-sequence from
// entry counts (bottom-up) and prefix offsets (top-down).  In the "parent
// kept" reading a selected entry is kept as well, in the slot just before its
// children's (the coarser entry first where two start together), and the
// slot of every kept entry is also written to a per-level map.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr int kTopkThreads = 1024;

struct TopkArgs {
    const float* lev[kMaxLevels];   // scores of level l: [H][n_l]
    int32_t* start;                 // [H][S]
    uint8_t* level;                 // [H][S]
    int32_t* bfirst;                // [H][ntop + 1]
    int32_t* scratch;               // [H][L][5][cap]
    int32_t* lmap;                  // parent kept: [sum_l H * n_l], 1 + slot of kept entries (zeroed)
    int64_t lmap_off[kMaxLevels];
    int pk;                         // 1: parent kept
    int64_t n[kMaxLevels];
    int64_t pw[kMaxLevels];
    int64_t ncand[kMaxLevels];      // candidates at level l: ntop at the top, p*min(K, .) below
    int64_t S, cap, ntop;
    int L, p, K;
    // per-level arrays in LDS when they fit (lds = 1): level l's five arrays of llen[l]
    // words each from word loff[l]; the candidates' scores of the level being ranked from ks_off
    int lds;
    int64_t loff[kMaxLevels], llen[kMaxLevels], ks_off;
};
constexpr size_t kTopkLdsMax = 144 * 1024;   // gfx950: 160 KiB of LDS per workgroup

__device__ __forceinline__ uint64_t make_key(float s, int32_t idx) {
    return ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(uint32_t)(~idx);
}

// The k-th largest (1 <= k <= nc) of the unique keys of candidates idx[0..nc)
// of level scores sc.  Each pass fixes one 8-bit digit, from the most
// significant: among the keys that match the digits fixed so far, a histogram
// of the next digit is counted, and wavefront 0 walks it from the top to the
// bin that holds the k-th largest, which becomes the next digit of the answer.
// When that bin holds a single key, one more pass reads the key itself.
__device__ uint64_t kth_largest_key(const float* sc, const int32_t* idx, const float* ks, int64_t nc, int64_t k,
                                    int32_t* hist, int64_t* bcast) {
    // candidate i's score: from the level's scores, or from the copy ks[i] made for this level
    auto score = [&](int64_t i) { return ks ? ks[i] : sc[idx[i]]; };
    const int tid = threadIdx.x, lane = tid & 63;
    uint64_t pre = 0, mask = 0;
    int64_t krem = k;   // rank of the answer among the keys that match `pre`
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (int64_t i = tid; i < nc; i += blockDim.x) {
            const uint64_t key = make_key(score(i), idx[i]);
            if ((key & mask) == pre) atomicAdd(&hist[(key >> shift) & 0xFF], 1);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 255-4l .. 252-4l (descending); x = keys in bins >= its lowest
            int c[4], sum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[255 - 4 * lane - q];
                sum += c[q];
            }
            int x = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            int64_t acc = x - sum;   // keys in bins above this lane's
            if (acc < krem && x >= krem) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (acc + c[q] >= krem) {
                        bcast[0] = 255 - 4 * lane - q;
                        bcast[1] = krem - acc;
                        bcast[2] = c[q];
                        break;
                    }
                    acc += c[q];
                }
            }
        }
        __syncthreads();
        pre |= (uint64_t)bcast[0] << shift;
        mask |= (uint64_t)0xFF << shift;
        krem = bcast[1];
        const bool unique = bcast[2] == 1;   // one key left with this prefix: it is the answer
        __syncthreads();                     // bcast is rewritten below
        if (unique) {
            for (int64_t i = tid; i < nc; i += blockDim.x) {
                const uint64_t key = make_key(score(i), idx[i]);
                if ((key & mask) == pre) bcast[3] = (int64_t)key;
            }
            __syncthreads();
            const uint64_t key = (uint64_t)bcast[3];
            __syncthreads();
            return key;
        }
    }
    return pre;
}

// Exclusive prefix sum of in[0..n) into out[0..n); returns the total.
__device__ int64_t block_scan_excl(const int32_t* in, int32_t* out, int64_t n, int32_t* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    int64_t carry = 0;
    for (int64_t base = 0; base < n; base += blockDim.x) {
        const int64_t i = base + tid;
        const int32_t v = i < n ? in[i] : 0;
        int32_t x = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int32_t y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        if (tid == 0) {
            int32_t acc = 0;
            for (int w = 0; w < nw; ++w) {
                int32_t t = wsum[w];
                wsum[w] = acc;
                acc += t;
            }
            wsum[nw] = acc;
        }
        __syncthreads();
        if (i < n) out[i] = (int32_t)(carry + wsum[wave] + x - v);
        carry += wsum[nw];
        __syncthreads();
    }
    return carry;
}

__global__ void __launch_bounds__(kTopkThreads) k_topk(TopkArgs a) {
    __shared__ int32_t hist[256];
    __shared__ int64_t bcast[4];
    __shared__ int32_t wsum[kTopkThreads / 64 + 1];
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = a.L, p = a.p, K = a.K;
    const int64_t cap = a.cap;
    int32_t* base = a.scratch + (int64_t)h * L * 5 * cap;
    // The selection is a chain of dependent passes over small arrays: kept in LDS
    // (when they fit) every pass waits for LDS instead of memory.
    extern __shared__ int32_t tk_lds[];
    auto arr = [&](int l, int which) -> int32_t* {
        return a.lds ? tk_lds + a.loff[l] + which * a.llen[l] : base + ((int64_t)l * 5 + which) * cap;
    };
    float* ks = a.lds ? reinterpret_cast<float*>(tk_lds + a.ks_off) : nullptr;
    // which: 0 idx, 1 flag, 2 rank, 3 cnt, 4 first
    const int64_t* ncand = a.ncand;

    for (int64_t i = tid; i < a.ntop; i += blockDim.x) arr(L - 1, 0)[i] = (int32_t)i;
    __syncthreads();

    for (int l = L - 1; l >= 1; --l) {
        int32_t* idx = arr(l, 0);
        int32_t* flag = arr(l, 1);
        const float* sc = a.lev[l] + (int64_t)h * a.n[l];
        const int64_t nc = ncand[l];
        const int64_t nsel = nc < K ? nc : K;   // equals ncand[l-1] / p
        if (nc <= K || K == 0) {
            const int32_t all = nc <= K ? 1 : 0;
            for (int64_t i = tid; i < nc; i += blockDim.x) flag[i] = all;
        } else {
            if (ks) {
                for (int64_t i = tid; i < nc; i += blockDim.x) ks[i] = sc[idx[i]];
                __syncthreads();
            }
            const uint64_t tau = kth_largest_key(sc, idx, ks, nc, K, hist, bcast);
            for (int64_t i = tid; i < nc; i += blockDim.x) {
                const float v = ks ? ks[i] : sc[idx[i]];
                flag[i] = make_key(v, idx[i]) >= tau ? 1 : 0;
            }
        }
        __syncthreads();
        block_scan_excl(flag, arr(l, 2), nc, wsum);
        // children of the selected candidates, in index order
        int32_t* rank = arr(l, 2);
        int32_t* nidx = arr(l - 1, 0);
        for (int64_t i = tid; i < nc; i += blockDim.x) {
            if (flag[i]) {
                const int64_t r = rank[i];
                const int32_t j = idx[i];
                for (int c = 0; c < p; ++c) nidx[r * p + c] = j * p + c;
            }
        }
        (void)nsel;
        __syncthreads();
    }

    // entry counts, bottom-up
    for (int64_t i = tid; i < ncand[0]; i += blockDim.x) arr(0, 3)[i] = 1;
    __syncthreads();
    for (int l = 1; l < L; ++l) {
        const int32_t* flag = arr(l, 1);
        const int32_t* rank = arr(l, 2);
        const int32_t* ccnt = arr(l - 1, 3);
        int32_t* cnt = arr(l, 3);
        for (int64_t i = tid; i < ncand[l]; i += blockDim.x) {
            int32_t c = 1;
            if (flag[i]) {
                c = a.pk;   // the entry itself, when it stays beside its children
                const int64_t r = rank[i];
                for (int z = 0; z < p; ++z) c += ccnt[r * p + z];
            }
            cnt[i] = c;
        }
        __syncthreads();
    }
    // slots, top-down
    block_scan_excl(arr(L - 1, 3), arr(L - 1, 4), ncand[L - 1], wsum);
    __syncthreads();
    for (int l = L - 1; l >= 1; --l) {
        const int32_t* flag = arr(l, 1);
        const int32_t* rank = arr(l, 2);
        const int32_t* first = arr(l, 4);
        const int32_t* ccnt = arr(l - 1, 3);
        int32_t* cfirst = arr(l - 1, 4);
        for (int64_t i = tid; i < ncand[l]; i += blockDim.x) {
            if (flag[i]) {
                const int64_t r = rank[i];
                int32_t f = first[i] + a.pk;
                for (int z = 0; z < p; ++z) {
                    cfirst[r * p + z] = f;
                    f += ccnt[r * p + z];
                }
            }
        }
        __syncthreads();
    }
    // emit kept entries
    int32_t* st = a.start + (int64_t)h * a.S;
    uint8_t* lv = a.level + (int64_t)h * a.S;
    for (int l = 0; l < L; ++l) {
        const int32_t* idx = arr(l, 0);
        const int32_t* flag = arr(l, 1);
        const int32_t* first = arr(l, 4);
        int32_t* lm = a.pk ? a.lmap + a.lmap_off[l] + (int64_t)h * a.n[l] : nullptr;
        for (int64_t i = tid; i < ncand[l]; i += blockDim.x) {
            if (l == 0 || !flag[i] || a.pk) {
                const int32_t s = first[i];
                st[s] = (int32_t)(idx[i] * a.pw[l]);
                lv[s] = (uint8_t)l;
                if (lm) lm[idx[i]] = s + 1;
            }
        }
    }
    int32_t* bf = a.bfirst + (int64_t)h * (a.ntop + 1);
    const int32_t* tfirst = arr(L - 1, 4);
    for (int64_t i = tid; i < a.ntop; i += blockDim.x) bf[i] = tfirst[i];
    if (tid == 0) bf[a.ntop] = (int32_t)a.S;
}

hipError_t launch_topk(const Plan& P, char* ws, hipStream_t s) {
    TopkArgs a{};
    const float* sc = reinterpret_cast<const float*>(ws + P.off_scores);
    for (int l = 0; l < P.L; ++l) {
        a.lev[l] = sc + P.lev_off[l];
        a.n[l] = P.n[l];
        a.pw[l] = P.pw[l];
    }
    a.start = reinterpret_cast<int32_t*>(ws + P.off_start);
    a.level = reinterpret_cast<uint8_t*>(ws + P.off_level);
    a.bfirst = reinterpret_cast<int32_t*>(ws + P.off_bfirst);
    a.scratch = reinterpret_cast<int32_t*>(ws + P.off_tk);
    a.S = P.S; a.cap = P.tk_cap; a.ntop = P.ntop;
    a.L = P.L; a.p = P.p; a.K = P.K;
    a.pk = P.pk;
    if (P.pk) {
        a.lmap = reinterpret_cast<int32_t*>(ws + P.off_lmap);
        for (int l = 0; l < P.L; ++l) a.lmap_off[l] = (int64_t)P.lmap_off[l];
    }
    int64_t nc = P.ntop;
    for (int l = P.L - 1; l >= 0; --l) {
        a.ncand[l] = nc;
        nc = (nc < P.K ? nc : P.K) * P.p;
    }
    // LDS layout: each level's five arrays (lengths rounded up to 4 words), then the
    // score copy of the largest ranked level
    int64_t words = 0, ksw = 0;
    for (int l = P.L - 1; l >= 0; --l) {
        a.llen[l] = (a.ncand[l] + 3) & ~(int64_t)3;
        a.loff[l] = words;
        words += 5 * a.llen[l];
        if (l >= 1 && a.llen[l] > ksw) ksw = a.llen[l];
    }
    a.ks_off = words;
    words += ksw;
    const size_t lds = (size_t)words * sizeof(int32_t);
    a.lds = lds <= kTopkLdsMax ? 1 : 0;
    hipLaunchKernelGGL(k_topk, dim3((unsigned)P.H), dim3(kTopkThreads), a.lds ? lds : 0, s, a);
    return hipGetLastError();
}

}  // namespace lh
