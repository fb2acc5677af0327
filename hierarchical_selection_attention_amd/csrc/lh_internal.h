// Internal plan of the Lighthouse layer on gfx950: shapes, workspace layout
// and the host-side launchers of every kernel.  Shared by the kernel sources
// and the C ABI (lh_api.cpp); not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lh {

constexpr int kMaxLevels = 24;
constexpr int kMaxK = 2048;        // largest K accepted when K < #candidates (a validation limit)
constexpr int kRowPad = 64;        // sub-sequence rows are padded to a multiple of this
constexpr int kChunkTokMax = 256;  // tokens per workgroup in the pooling/scoring pass
constexpr int kChunkScoreMax = 8192;  // tokens*heads of leaf scores kept in LDS per workgroup

enum Dtype { BF16 = 0, FP32 = 1 };

// Stage ids for event timing (order of launch).
enum Stage {
    ST_POOL_SCORE = 0, ST_POOL_UP, ST_TOPK, ST_GATHER, ST_SUB_PREP, ST_ATTN_FWD,
    ST_SCATTER_FWD, ST_ZERO_ACC, ST_SCATTER_BWD, ST_BWD_PREP, ST_ATTN_BWD, ST_POOL_BWD,
    // projections around the layer (lh_block_*)
    ST_PROJ_QKV, ST_PROJ_OUT, ST_PROJ_OUT_DX, ST_PROJ_OUT_DW, ST_PROJ_QKV_DX, ST_PROJ_QKV_DW, ST_COUNT
};

// Event pair around one stage when stage timing is on (lh_stage_timing).
struct StageMark {
    hipEvent_t a = nullptr, b = nullptr;
};
StageMark stage_open(hipStream_t s);
void stage_close(int id, hipStream_t s, const StageMark& m);
// Runs `fn`, which enqueues one stage, between the two events.
template <class F>
hipError_t stage(int id, hipStream_t s, F&& fn) {
    const StageMark m = stage_open(s);
    const hipError_t e = fn();
    stage_close(id, s, m);
    return e;
}

// lh_forward_sel with q, k, v rows in_ld elements apart (in_ld >= H*d, a multiple of 8)
// fwd_only: ws need only hold the forward's state (Plan::fwd_total); no matching
// backward may then use it
int forward_strided(const void* q, const void* k, const void* v, void* o, int N, int H, int d, int p, int L, int K,
                    int dtype, int score_mode, int select_mode, void* ws, size_t ws_bytes, void* stream,
                    int64_t in_ld, bool fwd_only = false);
// lh_backward with dq, dk, dv rows grad_ld elements apart (grad_ld = H*d for
// [N][H][d] tensors; larger strides need the bf16 path, grad_ld % 8 == 0)
int backward_strided(const void* dout, void* dq, void* dk, void* dv, int N, int H, int d, int p, int L, int K,
                     int dtype, int scatter_mode, void* ws, size_t ws_bytes, void* stream, int64_t grad_ld,
                     int select_mode = 0);

struct Plan {
    int N, H, d, p, L, K, dtype, esz;
    int score_mode;         // leaf score: 0 |q|^2+|k|^2, 1 |k|^2, 2 |q|^2, 3 |q|^2*|k|^2
    int keep_leaves;        // store the level-0 scores (inspection only; the selection ranks levels >= 1)
    int64_t in_ld;          // token stride of q, k, v in elements (H*d unless a caller strides them)
    int64_t S, Sp;
    int m;                  // pyramid level produced per workgroup by the pooling pass
    int rowcopy;            // bf16 partition: the attention kernels scatter their results to the tokens
    int pk;                 // "parent kept": selected entries stay beside their children (bf16 only)
    int64_t tok;            // p^m tokens per pooling workgroup
    int64_t ntop;           // N / p^(L-1)
    int64_t n[kMaxLevels];  // entries at level l
    int64_t pw[kMaxLevels]; // p^l
    int64_t tk_cap;         // capacity of one level's candidate list in the selection scratch
    // byte offsets inside the workspace
    size_t off_scores;
    size_t lev_off[kMaxLevels];   // float offset of level l inside the score block
    size_t off_pool_m;            // fp32 [3][n_m][H][d]
    size_t off_pool_top;          // fp32 [3][ntop][H][d] (aliases off_pool_m when m == L-1)
    size_t off_start, off_level, off_bfirst;
    size_t off_tk;                // selection scratch: [H][L][5][tk_cap] int32
    size_t off_qs, off_ks, off_vs;   // fp32 [H][Sp][d] gathered sub-sequence
    // 16-bit operand copies (bf16 path): fp16 hi/lo rows [H][Sp][d]
    size_t off_qh, off_ql, off_kh, off_kl, off_vh, off_vl;
    size_t off_hmax;              // uint32 [2][H][4]: forward (q, k, v) and backward (dO) max |x|
    size_t off_rowmax;            // fp32 [4][H][Sp]: max |x| per row of q~, k~, v~ (gather) and dO~
    size_t off_hscale;            // fp32 [H][4]: per-head multipliers of the fp16 copies
    size_t off_os;                // fp32 [H][Sp][d]
    size_t off_lse, off_lse2;     // fp32 [H][Sp]
    size_t off_acc;               // fp32 [H][Sp][d]: sums of dO over each entry (dO~)
    size_t off_part;              // fp32 [H][N / tok][d]: deterministic mode's per-block partial sums
    size_t off_dos;               // fp32 [H][Sp][d] finished dO~: the rows of off_acc, completed in place
    size_t off_doh, off_dol;      // fp16 hi/lo rows of dO~
    size_t off_D;                 // fp32 [H][Sp]
    size_t off_dq, off_dk, off_dv;   // fp32 [H][Sp][d]
    // parent kept: int32 [sum_l H * n_l], 1 + the slot of entry (l, j) of head h
    // at lmap_off[l] + h * n_l + j, 0 when that entry is not kept
    size_t off_lmap;
    size_t lmap_off[kMaxLevels];
    size_t fwd_total;             // bytes of the forward's state (a prefix of the workspace)
    size_t total;
    size_t off_lmap_bytes() const {
        size_t n = 0;
        for (int l = 0; l < L; ++l) n += (size_t)H * this->n[l];
        return sizeof(int32_t) * n;
    }
};

// Fills `pl`; returns 0 or a negative lh_status.  select_mode 0: the kept
// entries partition [0, N); 1: parent kept (bf16 only).
int make_plan(int N, int H, int d, int p, int L, int K, int dtype, Plan* pl, int select_mode = 0);
int64_t subseq_len(int N, int p, int L, int K, int select_mode = 0);

// ------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.  All pointers are device
// pointers; `ws` is the workspace base.

hipError_t launch_pool_score(const Plan& P, const void* q, const void* k, const void* v, char* ws,
                             hipStream_t s);
hipError_t launch_pool_up(const Plan& P, char* ws, hipStream_t s);
hipError_t launch_topk(const Plan& P, char* ws, hipStream_t s);
hipError_t launch_gather(const Plan& P, const void* q, const void* k, const void* v, char* ws,
                         hipStream_t s);
hipError_t launch_scatter_fwd(const Plan& P, char* ws, void* o, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_scatter_bwd(const Plan& P, const void* dout, int mode, char* ws, hipStream_t s);
hipError_t launch_pool_bwd(const Plan& P, char* ws, void* dq, void* dk, void* dv, hipStream_t s);
// parent kept: out[z][t][h] = sum over the kept entries covering t of tab[z][h][slot]
// (divided by p^level when `divide`), fp32 tables, bf16 output rows out_ld apart
hipError_t launch_sum_copy(const Plan& P, const char* ws, const float* const* tab, void* const* out, int Z,
                           bool divide, int64_t out_ld, hipStream_t s);
// parent kept: fp32 acc[h][slot] = sum of dO over the entry's tokens (bf16 dO)
hipError_t launch_entry_sum(const Plan& P, const void* dout, char* ws, hipStream_t s);

// Attention operands: 16-bit copies laid out [H][Sp][d]; lo parts are used
// when `split`.
struct AttnArgs {
    const uint16_t *qh, *ql, *kh, *kl, *vh, *vl, *doh, *dol;
    const float* hscale;
    float* o;                  // fp32 [H][Sp][d] or null
    uint16_t* o_bf16;          // bf16 output rows (ld_o, hs_o) or null
    float *lse, *lse2;
    const float* D;
    float *dq, *dk, *dv;       // fp32 [H][Sp][d] or null
    uint16_t *dq_b, *dk_b, *dv_b;   // bf16 rows (ld_o, hs_o) or null
    const uint8_t* level;           // [H][rows] (the in-kernel scatters)
    int p;
    // optional: the kernels scatter their results to bf16 token rows [N][H][d]
    // (tok_ld elements apart) themselves -- O~ (forward), dQ~/p^level (dQ),
    // dK~/p^level and dV~/p^level (dK/dV) -- for the entries start [H][rows]
    uint16_t *o_tok, *dq_tok, *dk_tok, *dv_tok;
    const int32_t* start;
    int64_t tok_ld;
    int64_t rows, Sp, ld_o, hs_o;
    int H, d;
    bool split, fp32_path;
    float scale;
    const float *qf, *kf, *vf, *dof;   // fp32 path operands [H][Sp][d]
};
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
// dK/dV and dQ in one launch (bf16: the two roles of k_attn_bwd; fp32: one kernel)
hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t s);

struct SplitSpec {
    const void* src;
    int64_t ld, hs, rows, Sp;
    int d, H, src_bf16;
    const unsigned int* hmax;
    float* hscale;
    int slot;
    uint16_t *rh, *rl;
};
struct RowPrepSpec {
    const void *acc, *dout, *o;
    // deterministic mode: entries above level m are summed from `part` (start, level: [H][S])
    const float* part;
    const int32_t* start;
    const uint8_t* level;
    int64_t tok, nblk;            // tokens per block, blocks per head (N / tok)
    int m, p;
    int64_t ld, hs;
    float *dos, *D;
    const float* lse_in;       // dense: natural-log lse [H][N] -> lse2 (base 2, minus the backward's offset)
    float* lse2;
    float* rowmax;             // optional: per-row max |dO~| [H][Sp]
    int64_t S, Sp;
    int H, d, mode, dense;
    int in_place;              // dos is acc: only the rows that change are stored
};
// out[t][h * 4] = max over rows of rowmax[t][h][0..rows) (rows_ld apart), T <= 4 tensors
hipError_t launch_head_max(const float* rowmax, unsigned int* const* out, int T, int64_t rows, int64_t rows_ld,
                           int H, hipStream_t s);
// max |x| per head of T <= 3 tensors of one layout (out[t]: the tensor's [H][4] slot word)
hipError_t launch_maxabs(const void* const* src, unsigned int* const* out, int T, bool src_bf16, int64_t ld,
                         int64_t hs, int64_t rows, int d, int H, hipStream_t s);
// splits of T <= 3 tensors of one layout (same strides, rows, hmax and hscale) in one launch
hipError_t launch_split(const SplitSpec* sp, int T, hipStream_t s);
hipError_t launch_clear_slot(unsigned int* hmax, int H, int slot, hipStream_t s);
hipError_t launch_row_prep(const RowPrepSpec& sp, hipStream_t s);

// Achievable-peak probes (kind 0 read, 1 write, 2 copy, 3 bf16 MFMA loop).
hipError_t launch_peak_probe(int kind, const void* src, void* dst, size_t n, hipStream_t s);

}  // namespace lh
