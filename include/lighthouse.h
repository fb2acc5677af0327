/*
 * lighthouse.h — C ABI of the MI355X (gfx950) Lighthouse attention layer.
 *
 * The layer follows "Long Context Pre-Training with Lighthouse Attention"
 * (Peng, Ghosh, Quesnelle, arXiv 2605.06554; read from the P1 mirror of the
 * arXiv HTML, Sec. 3, Sec. 3.1 Eq. (1), Fig. 1 and Fig. 2, and the P3/P4
 * summaries).  It replaces softmax attention by four stages around an
 * unmodified causal attention kernel:
 *   (i)   average-pool q, k and v symmetrically into an L-level pyramid with
 *         factor p (level l averages p^l tokens; level 0 is the input);
 *   (ii)  score every pyramid entry without parameters (squared l2 norm of
 *         q and k, max-pooled up the levels) and select, from the top level
 *         down, the K best entries per level and head; a selected entry is
 *         replaced by its p children, so the kept entries partition [0, N);
 *   (iii) order the kept entries by first token into a hole-free causal
 *         sub-sequence of length S (see lh_subseq_len), gather their pooled
 *         q, k, v and run ordinary causal softmax attention (Eq. (1), scale
 *         1/sqrt(d)) on it;
 *   (iv)  scatter every sub-sequence output back to the p^l tokens of its
 *         entry.
 * Gradients flow through (iv), (iii), the gather and the pooling; the
 * selection carries none (Fig. 1, gradient path).
 *
 * Conventions for every entry point below:
 *   - q, k, v, o, dout, dq, dk, dv are device pointers to contiguous
 *     [N][H][d] tensors (token-major, one batch element), 16-byte aligned,
 *     in the element type given by `dtype` (lh_dtype).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call only enqueues work on it and returns; nothing synchronises.
 *   - The library never allocates device memory on these paths: the caller
 *     provides a workspace of at least lh_workspace_bytes(...) bytes
 *     (256-byte aligned).  lh_backward reads what lh_forward left in the
 *     workspace, so the workspace must stay untouched between the two and
 *     both calls must use the same parameters and stream order.
 *   - Arguments are validated on the host before any launch; on error the
 *     call returns a negative lh_status and enqueues nothing.  Launch
 *     failures return LH_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Supported shapes: d in {64, 128}; 1 <= H, H*d <= 8192; p >= 2; L >= 1;
 *     p^(L-1) divides N; N < 2^31; K >= 0, and K <= 2048 unless K covers
 *     every candidate at every level.
 */
#ifndef LIGHTHOUSE_H
#define LIGHTHOUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LH_OK = 0,
    LH_ERR_ARG = -1,        /* null pointer or parameter out of range            */
    LH_ERR_SHAPE = -2,      /* shape not supported (d, H, N divisibility, sizes)  */
    LH_ERR_DTYPE = -3,      /* unknown dtype or scatter mode                      */
    LH_ERR_WORKSPACE = -4,  /* workspace missing, misaligned or too small         */
    LH_ERR_HIP = -5,        /* a HIP launch or runtime call failed                */
    LH_ERR_GEMM = -6,       /* the GEMM library (hipBLASLt) failed or has no algorithm */
    LH_ERR_SCRATCH = -7     /* lh_forward_static: the shape's forward state exceeds its array */
} lh_status;

typedef enum { LH_BF16 = 0, LH_FP32 = 1 } lh_dtype;

/* How the adjoint of the scatter sums dO over the tokens of an entry when the
 * entry spans several workgroups.  "Lighthouse Attention Technique" (closing
 * paragraph) describes an fp-atomic default and a deterministic int-atomic
 * variant kept for reproducibility.  Here an entry at pyramid level <= m (the
 * level one workgroup pools, p^m <= 256 tokens) is summed by one thread in
 * token order in both modes.  A coarser entry is summed per block of p^m
 * tokens, and the block sums are combined:
 *   LH_SCATTER_FP_ATOMIC: with fp32 atomic adds (the order, and so the last
 *     bits, can differ between runs);
 *   LH_SCATTER_INT_ATOMIC (= LH_SCATTER_DETERMINISTIC): each block stores its
 *     sum, and the sums are added in block order in double.  The bits are the
 *     same on every run.  Unlike fixed-point integer atomics, there is no range
 *     limit or quantum: every fp32 dO whose sums stay finite is handled. */
typedef enum {
    LH_SCATTER_FP_ATOMIC = 0,
    LH_SCATTER_INT_ATOMIC = 1,
    LH_SCATTER_DETERMINISTIC = 1
} lh_scatter_mode;

/* Length S of the gathered sub-sequence (Sec. 1: S = O(LpK + N/p^(L-1))):
 * N/p^(L-1) top entries, plus (p-1) for every selection made.  Host only.
 * Returns S, or a negative lh_status for invalid arguments. */
int64_t lh_subseq_len(int N, int p, int L, int K);

/* Bytes of workspace lh_forward/lh_backward need; 0 for invalid arguments. */
size_t lh_workspace_bytes(int N, int H, int d, int p, int L, int K, int dtype);

/* Forward pass, stages (i)-(iv).  Writes o [N][H][d] and keeps the selection,
 * the gathered sub-sequence, its output and log-sum-exp in the workspace. */
int lh_forward(const void* q, const void* k, const void* v, void* o,
               int N, int H, int d, int p, int L, int K, int dtype,
               void* ws, size_t ws_bytes, void* stream);

/* lh_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation and output as lh_forward (partition selection, default
 * score), with its workspace in a static device array of
 * LH_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on each device it
 * runs on until the process ends.  The first call on a device looks up that
 * device's array; the call allocates nothing.  Its state serves no
 * lh_backward.  Every call on one device shares that device's array: calls
 * that overlap in time on one device (on different streams, or from other
 * threads) race and give wrong results.  The shape must fit: its forward state
 * (scores, selection, gathered sub-sequence and operand copies, about 53 MiB at
 * N = 16384, H = 16, d = 128, K = 32) may not exceed the array, else
 * LH_ERR_SCRATCH and nothing is enqueued.  `stream` must belong to the current
 * device (LH_ERR_ARG otherwise).  Other arguments, layouts and errors as
 * lh_forward. */
#define LH_STATIC_SCRATCH_BYTES (64u << 20)
int lh_forward_static(const void* q, const void* k, const void* v, void* o,
                      int N, int H, int d, int p, int L, int K, int dtype, void* stream);

/* What the parameter-free score is taken of.  The pages call the scoring
 * bidirectional (Sec. 1) and label Fig. 2's scores "qk" / "kq" without fixing
 * the formula.  LH_SCORE_QK, the reading lh_forward uses, scores a leaf by
 * ||q||^2 + ||k||^2; the alternatives score it by ||k||^2, by ||q||^2, or by
 * ||q||^2 * ||k||^2 (ranks as ||q|| ||k||).  Each squared norm is summed in
 * fp32 in the fixed order of the default score (fma over 8 consecutive
 * elements from +0, then a xor butterfly over the d/8 groups); the product
 * is one fp32 multiply.  Coarser levels take the max of their p children in
 * every mode. */
typedef enum {
    LH_SCORE_QK = 0,
    LH_SCORE_K = 1,
    LH_SCORE_Q = 2,
    LH_SCORE_QK_PRODUCT = 3
} lh_score_mode;

/* Option bit for the score_mode argument of lh_forward_scored / lh_forward_sel:
 * also store the leaf scores (level 0 of LH_VIEW_SCORES).  The selection never
 * ranks leaves -- the p children of a selected level-1 entry are all kept -- so
 * the layer itself needs only levels 1..L-1, and without this bit level 0 of
 * the score view is left unwritten (except when L = 1, where level 0 is the
 * top).  Leaf scores are computed either way: level 1 is their max-pool. */
#define LH_SCORE_KEEP_LEAVES 0x100

/* lh_forward with the score of `score_mode` (lh_score_mode, optionally ORed
 * with LH_SCORE_KEEP_LEAVES; LH_ERR_DTYPE for an unknown mode).  Everything
 * else, lh_backward included, is unchanged. */
int lh_forward_scored(const void* q, const void* k, const void* v, void* o,
                      int N, int H, int d, int p, int L, int K, int dtype, int score_mode,
                      void* ws, size_t ws_bytes, void* stream);

/* Which entries the selection keeps (Fig. 2 step 3 "tree-prune", "parent
 * kept").  LH_SELECT_PARTITION, the reading of lh_forward: a selected entry
 * is replaced by its p children, so the kept entries partition [0, N) and
 * every token takes the output of the one entry covering it.
 * LH_SELECT_PARENT_KEPT: a selected entry stays in the sub-sequence beside its
 * children, so every candidate of every level is kept (S = N/p^(L-1) plus
 * p * min(K, #candidates) per selecting level, lh_subseq_len_sel); entries
 * are ordered by first token, the coarser first where two start together; a
 * token's output is the sum of the outputs of the (up to L) entries covering
 * it, and the adjoints sum likewise (the gradient of an entry is the sum of
 * dO over its tokens; a token's dq, dk, dv sum dX~ / p^level over its
 * entries).  Both sums are taken by one thread or wavefront per output in a
 * fixed order, so the result does not depend on scatter_mode and is the same
 * on every run.  Parent kept is bf16 only (LH_ERR_DTYPE otherwise). */
typedef enum {
    LH_SELECT_PARTITION = 0,
    LH_SELECT_PARENT_KEPT = 1
} lh_select_mode;

/* The entry points of the layer with a selection mode (lh_select_mode;
 * LH_ERR_DTYPE for an unknown one).  A workspace filled by lh_forward_sel
 * must be read with the same select_mode (lh_backward_sel,
 * lh_read_selection_sel, lh_workspace_view_sel). */
int64_t lh_subseq_len_sel(int N, int p, int L, int K, int select_mode);
size_t lh_workspace_bytes_sel(int N, int H, int d, int p, int L, int K, int dtype, int select_mode);
int lh_forward_sel(const void* q, const void* k, const void* v, void* o,
                   int N, int H, int d, int p, int L, int K, int dtype, int score_mode,
                   int select_mode, void* ws, size_t ws_bytes, void* stream);
int lh_backward_sel(const void* dout, void* dq, void* dk, void* dv,
                    int N, int H, int d, int p, int L, int K, int dtype, int scatter_mode,
                    int select_mode, void* ws, size_t ws_bytes, void* stream);

/* Option bit for the scatter_mode argument of lh_backward / lh_backward_sel:
 * also store the fp32 gradients of the gathered sub-sequence, dQ~, dK~, dV~
 * (LH_VIEW_DQSUB .. LH_VIEW_DVSUB).  On the bf16 partition path the attention
 * kernels write dq, dk, dv to the tokens themselves and nothing reads these
 * rows, so without the bit they are not stored and those views keep whatever
 * the workspace held.  The fp32 path and the parent-kept selection store them
 * either way (their pool adjoint reads them). */
#define LH_BWD_KEEP_SUB 0x100

/* Backward pass through the scatter, the attention, the gather and the pool
 * (Fig. 1 gradient path).  q, k, v are not needed: everything is read from
 * the workspace of the matching lh_forward.  Writes dq, dk, dv [N][H][d].
 * scatter_mode is an lh_scatter_mode, optionally ORed with LH_BWD_KEEP_SUB.
 * Every kernel is enqueued on `stream`; the library keeps no stream or
 * buffer of its own (events only while lh_stage_timing is on), so calls with
 * distinct workspaces on distinct streams may run concurrently. */
int lh_backward(const void* dout, void* dq, void* dk, void* dv,
                int N, int H, int d, int p, int L, int K, int dtype, int scatter_mode,
                void* ws, size_t ws_bytes, void* stream);

/* Locations of intermediate results inside a workspace, for inspection.
 * Host only; pure address arithmetic on `ws`. */
typedef enum {
    LH_VIEW_SCORES = 0,     /* fp32, levels 0..L-1 concatenated, each [H][N/p^l]
                               (level 0 only with LH_SCORE_KEEP_LEAVES or L = 1) */
    LH_VIEW_SEL_START = 1,  /* int32 [H][S]: first token of each kept entry        */
    LH_VIEW_SEL_LEVEL = 2,  /* uint8 [H][S]: pyramid level of each kept entry      */
    LH_VIEW_QSUB = 3,       /* fp32 [H][Sp][d]: gathered q (rows >= S are zero)    */
    LH_VIEW_KSUB = 4,       /* fp32 [H][Sp][d]                                     */
    LH_VIEW_VSUB = 5,       /* fp32 [H][Sp][d]                                     */
    LH_VIEW_OSUB = 6,       /* fp32 [H][Sp][d]: attention output on the sub-seq.   */
    LH_VIEW_LSE = 7,        /* fp32 [H][Sp]: natural-log log-sum-exp per row       */
    LH_VIEW_DOSUB = 8,      /* fp32 [H][Sp][d]: dO summed over each entry's tokens */
    LH_VIEW_DQSUB = 9,      /* fp32 [H][Sp][d]: gradient of the gathered q (bf16
                               partition path: only with LH_BWD_KEEP_SUB)          */
    LH_VIEW_DKSUB = 10,     /* fp32 [H][Sp][d], as LH_VIEW_DQSUB                 */
    LH_VIEW_DVSUB = 11,     /* fp32 [H][Sp][d], as LH_VIEW_DQSUB                 */
    LH_VIEW_BLOCK_FIRST = 12 /* int32 [H][N/p^(L-1)+1]: first slot of each top block */
} lh_view;

/* Sp = S rounded up to a multiple of 64 (row padding of the sub-sequence). */
int lh_workspace_view(void* ws, int N, int H, int d, int p, int L, int K, int dtype,
                      int view, void** ptr, size_t* bytes);
int lh_workspace_view_sel(void* ws, int N, int H, int d, int p, int L, int K, int dtype,
                          int select_mode, int view, void** ptr, size_t* bytes);

/* Copy the kept entries' descriptors out of a workspace that lh_forward
 * filled: start (int32 [H][S], first token of each entry of the causal
 * sub-sequence, strictly increasing per head) and level (uint8 [H][S],
 * pyramid level; the entry covers p^level tokens) -- the partition of
 * [0, N) selected in stage (ii) and ordered in stage (iii) (Sec. 3, Fig. 2).
 * start and level are device pointers owned by the caller (either may be
 * NULL, not both); the copies are enqueued on `stream`.  Parameters must be
 * those of the forward call.  Returns LH_OK, LH_ERR_ARG/SHAPE/DTYPE for bad
 * arguments (nothing enqueued), or LH_ERR_HIP. */
int lh_read_selection(const void* ws, int N, int H, int d, int p, int L, int K, int dtype,
                      int32_t* start, uint8_t* level, void* stream);
int lh_read_selection_sel(const void* ws, int N, int H, int d, int p, int L, int K, int dtype,
                          int select_mode, int32_t* start, uint8_t* level, void* stream);

/* Achievable-peak probes (not part of the layer), reported beside the vendor
 * peaks.  kind 0 reads n bytes at src in 1 MiB chunks and stores the XOR fold
 * of each chunk's 16-byte words to dst[16c .. 16c+15] (dst: ceil(n / 2^20) * 16
 * bytes); kind 1 writes n bytes at dst; kind 2 copies n bytes from src to dst
 * (these three use 16-byte non-temporal accesses; n a multiple of 16, pointers
 * 16-byte aligned); kind 3 runs n rounds (n <= 2^30) of 4 independent bf16
 * 32x32x16 MFMAs in each of 4096 wavefronts (4096 * n * 4 * 32768 flops) and
 * stores a checksum per workgroup of 4 wavefronts (dst: 1024 * 16 bytes); kind 4
 * measures the rounding of the attention kernels' matrix instruction: for each
 * of n trials (n <= 2^20) one v_mfma_f32_16x16x32_f16 on the 3072-byte record
 * src + 3072 t (lanes 0..63 of fp16 A[8], then fp16 B[8], then fp32 C[4]; lane
 * l holds A[l % 16][8 (l / 16) + e], B[8 (l / 16) + e][l % 16] and C, D at rows
 * 4 (l / 16) + r, column l % 16) writes D to dst + 1024 t (lanes 0..63 of fp32
 * D[4]); kind 5 writes n bytes at dst (n a multiple of 64 MiB, at most 2^40,
 * dst 16-byte aligned) in the token-row pattern of the attention kernels'
 * scatter: dst read as bf16 rows [n / 4096][16][128], each workgroup of 256
 * threads writing one head's 256-byte pieces of 16384 consecutive tokens, 16
 * tokens per pass, in 16-byte non-temporal stores (the 16-byte word of token t,
 * head h, chunk c holds {1.0f bits, workgroup 16 (t / 16384) + h, thread
 * 16 (t % 16) + c, 0}).  Device pointers; enqueued on `stream`.  Returns LH_OK,
 * LH_ERR_ARG, or LH_ERR_HIP. */
int lh_peak_probe(int kind, const void* src, void* dst, size_t n, void* stream);

/* Dense causal attention over all N tokens with the same attention kernels
 * (the comparison path of the benchmark).  lse is fp32 [H][N] (natural log);
 * N must be a multiple of 64; bf16 only.  Workspace: lh_dense_workspace_bytes.
 * lh_dense_attn_bwd reads the operand copies and the fp32 output that the
 * matching lh_dense_attn_fwd left in the workspace (same workspace, same
 * stream order); q, k, v and o must be the tensors of that forward call. */
size_t lh_dense_workspace_bytes(int N, int H, int d, int dtype);
int lh_dense_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int N, int H, int d, int dtype, void* ws, size_t ws_bytes, void* stream);
int lh_dense_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      int N, int H, int d, int dtype, void* ws, size_t ws_bytes, void* stream);

/* The attention block around the layer (Sec. 3.1 Eq. (1) and Fig. 1: the
 * projections W_Q, W_K, W_V from the block input feed the pyramid pool; the
 * layer output leaves through an output projection W_O, as in the Llama-style
 * models of Sec. 4).  bf16 only.  With dm the model width and Hd = H*d, all
 * row-major device tensors, 16-byte aligned:
 *   x      [N][dm]      block input
 *   w_qkv  [dm][3*Hd]   columns [0, Hd) give q = x W_Q, read as [N][H][d];
 *                       [Hd, 2Hd) give k and [2Hd, 3Hd) give v
 *   w_o    [Hd][dm]
 *   o      [N][H][d]    the layer output: written by lh_block_forward and
 *                       read by lh_block_backward (the caller keeps it)
 *   y      [N][dm]      y = o W_O
 * lh_block_backward takes dy [N][dm] and writes dx [N][dm] (bf16) and the
 * weight gradients dw_qkv [dm][3*Hd] and dw_o [Hd][dm] in fp32; all three
 * are overwritten, not accumulated.  x, w_qkv, w_o and o must be those of the
 * matching forward.  Products accumulate in fp32; q, k, v and dO = dy W_O^T
 * are rounded to bf16 (round to nearest even), the layer's I/O type.  The six
 * weight products run in hipBLASLt; the first call on a device creates its
 * handle and each new GEMM shape chooses an algorithm once (host state kept
 * until the process ends).  Workspace: lh_block_workspace_bytes (256-byte
 * aligned); it begins with the layer's workspace, so lh_read_selection and
 * lh_workspace_view (dtype LH_BF16) read it directly.  At the next 256-byte
 * boundary after it the forward leaves q, k, v ([N][3][H][d] bf16: the q, k
 * and v rows of a token side by side), which the backward overwrites with the
 * gradients in the same layout; at the next 256-byte boundary after those the backward
 * leaves dO = dy W_O^T ([N][H][d] bf16).  The workspace must stay untouched
 * between the forward and the backward.  dm must be a multiple of
 * 8; the other shape limits are the layer's.  `stream` must belong to the
 * current device, whose hipBLASLt handle runs the products (LH_ERR_ARG
 * otherwise).  Returns LH_OK, a negative lh_status for bad arguments (nothing
 * enqueued), LH_ERR_HIP or LH_ERR_GEMM. */
size_t lh_block_workspace_bytes(int N, int H, int d, int dm, int p, int L, int K);
int lh_block_forward(const void* x, const void* w_qkv, const void* w_o, void* o, void* y,
                     int N, int H, int d, int dm, int p, int L, int K,
                     void* ws, size_t ws_bytes, void* stream);
int lh_block_backward(const void* x, const void* w_qkv, const void* w_o, const void* o,
                      const void* dy, void* dx, float* dw_qkv, float* dw_o,
                      int N, int H, int d, int dm, int p, int L, int K, int scatter_mode,
                      void* ws, size_t ws_bytes, void* stream);

/* Per-stage timing with HIP events recorded on the caller's stream around
 * each kernel of lh_forward/lh_backward and each GEMM of lh_block_*.  enable != 0 starts recording (and
 * clears earlier results); lh_stage_timing_read synchronises on the recorded
 * events, adds each stage's elapsed milliseconds into ms[stage] and the
 * number of times the stage ran into count[stage] for stage < n, and returns
 * the number of stages.  lh_stage_name gives a stage's name. */
int lh_stage_timing(int enable);
int lh_stage_timing_read(double* ms, int* count, int n);
const char* lh_stage_name(int stage);

/* Human-readable text for an lh_status value. */
const char* lh_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTHOUSE_H */
