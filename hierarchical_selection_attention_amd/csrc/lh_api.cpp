// C ABI of the Lighthouse layer (declared in include/lighthouse.h): argument
// validation, workspace layout and the launch order of the stages on the
// caller's stream.  Stage order follows Fig. 1 of "Long Context Pre-Training
// with Lighthouse Attention": pyramid pool -> selector -> dense gather ->
// attention -> back-scatter, and the reverse for the gradient.
#include <math.h>
#include <stdint.h>
#include <mutex>
#include <vector>

#include "lighthouse.h"
#include "lh_internal.h"

namespace lh {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t subseq_len(int N, int p, int L, int K, int select_mode) {
    if (N <= 0 || p < 2 || L < 1 || L > kMaxLevels || K < 0) return LH_ERR_ARG;
    if (select_mode != LH_SELECT_PARTITION && select_mode != LH_SELECT_PARENT_KEPT) return LH_ERR_DTYPE;
    int64_t top = 1;
    for (int l = 0; l < L - 1; ++l) {
        top *= p;
        if (top > N) return LH_ERR_SHAPE;
    }
    if (N % top != 0) return LH_ERR_SHAPE;
    int64_t n = N / top, S = n, cand = n;
    for (int l = L - 1; l >= 1; --l) {
        const int64_t sel = cand < K ? cand : K;
        // a selected entry gives way to its p children, or stays beside them (parent kept)
        S += sel * (select_mode == LH_SELECT_PARENT_KEPT ? p : p - 1);
        cand = sel * p;
    }
    return S;
}

int make_plan(int N, int H, int d, int p, int L, int K, int dtype, Plan* P, int select_mode) {
    if (dtype != BF16 && dtype != FP32) return LH_ERR_DTYPE;
    if (select_mode != LH_SELECT_PARTITION && select_mode != LH_SELECT_PARENT_KEPT) return LH_ERR_DTYPE;
    if (select_mode == LH_SELECT_PARENT_KEPT && dtype != BF16) return LH_ERR_DTYPE;
    if (N <= 0 || H <= 0 || p < 2 || L < 1 || L > kMaxLevels || K < 0) return LH_ERR_ARG;
    if (d != 64 && d != 128) return LH_ERR_SHAPE;
    if ((int64_t)H * d > 8192) return LH_ERR_SHAPE;
    const int64_t S = subseq_len(N, p, L, K, select_mode);
    if (S < 0) return (int)S;
    if (S > INT32_MAX - 1) return LH_ERR_SHAPE;
    Plan& pl = *P;
    pl = Plan{};
    pl.pk = select_mode == LH_SELECT_PARENT_KEPT;
    pl.in_ld = (int64_t)H * d;
    pl.N = N; pl.H = H; pl.d = d; pl.p = p; pl.L = L; pl.K = K; pl.dtype = dtype;
    pl.esz = dtype == BF16 ? 2 : 4;
    pl.S = S;
    pl.Sp = (S + kRowPad - 1) / kRowPad * kRowPad;
    pl.pw[0] = 1;
    for (int l = 1; l < L; ++l) pl.pw[l] = pl.pw[l - 1] * p;
    for (int l = 0; l < L; ++l) pl.n[l] = N / pl.pw[l];
    pl.ntop = pl.n[L - 1];
    int m = 0;
    while (m + 1 <= L - 1 && pl.pw[m + 1] <= kChunkTokMax && pl.pw[m + 1] * H <= kChunkScoreMax) ++m;
    if (L > 1 && m < 1) return LH_ERR_SHAPE;
    pl.m = m;
    pl.tok = pl.pw[m];
    // candidate counts per level; the top-K network handles K <= kMaxK
    int64_t nc = pl.ntop, cap = pl.ntop;
    for (int l = L - 1; l >= 1; --l) {
        if (nc > K && K > kMaxK) return LH_ERR_SHAPE;
        nc = (nc < K ? nc : K) * p;
        if (nc > cap) cap = nc;
    }
    pl.tk_cap = cap > 0 ? cap : 1;

    const size_t HSd = (size_t)H * pl.Sp * d;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    size_t nscore = 0;
    for (int l = 0; l < L; ++l) {
        pl.lev_off[l] = nscore;
        nscore += (size_t)H * pl.n[l];
    }
    pl.off_scores = take(sizeof(float) * nscore);
    pl.off_pool_m = take(m >= 1 ? sizeof(float) * 3 * (size_t)pl.n[m] * H * d : 0);
    pl.off_pool_top = (m == L - 1) ? pl.off_pool_m : take(sizeof(float) * 3 * (size_t)pl.ntop * H * d);
    pl.off_start = take(sizeof(int32_t) * (size_t)H * S);
    pl.off_level = take((size_t)H * S);
    pl.off_bfirst = take(sizeof(int32_t) * (size_t)H * (pl.ntop + 1));
    pl.off_tk = take(sizeof(int32_t) * (size_t)H * L * 5 * pl.tk_cap);
    pl.off_qs = take(sizeof(float) * HSd);
    pl.off_ks = take(sizeof(float) * HSd);
    pl.off_vs = take(sizeof(float) * HSd);
    const size_t h16 = dtype == BF16 ? 2 * HSd : 0;
    pl.off_qh = take(h16); pl.off_ql = take(h16);
    pl.off_kh = take(h16); pl.off_kl = take(h16);
    pl.off_vh = take(h16); pl.off_vl = take(h16);
    pl.off_hmax = take(sizeof(uint32_t) * 8 * (size_t)H);
    pl.off_rowmax = take(sizeof(float) * 4 * (size_t)H * pl.Sp);
    pl.off_hscale = take(sizeof(float) * 4 * (size_t)H);
    pl.off_os = take(sizeof(float) * HSd);
    pl.off_lse = take(sizeof(float) * (size_t)H * pl.Sp);
    pl.off_lse2 = take(sizeof(float) * (size_t)H * pl.Sp);
    size_t nmap = 0;
    for (int l = 0; l < L; ++l) {
        pl.lmap_off[l] = nmap;
        nmap += (size_t)H * pl.n[l];
    }
    pl.off_lmap = take(pl.pk ? sizeof(int32_t) * nmap : 0);
    // everything above is the forward's state; what follows only the backward uses
    pl.fwd_total = off;
    pl.off_acc = take(sizeof(float) * HSd);
    pl.off_part = take(m < L - 1 ? sizeof(float) * (size_t)H * (size_t)(N / pl.tok) * d : 0);
    // the finished dO~ is the accumulator itself: the row preparation completes its
    // rows in place
    pl.off_dos = pl.off_acc;
    pl.off_doh = take(h16); pl.off_dol = take(h16);
    pl.off_D = take(sizeof(float) * (size_t)H * pl.Sp);
    pl.off_dq = take(sizeof(float) * HSd);
    pl.off_dk = take(sizeof(float) * HSd);
    pl.off_dv = take(sizeof(float) * HSd);
    pl.rowcopy = dtype == BF16 && !pl.pk;
    pl.total = off;
    return LH_OK;
}

// ------------------------------------------------------------ stage timing
namespace {
struct TimedLaunch {
    int stage;
    hipEvent_t a, b;
};
std::mutex g_mu;
bool g_timing = false;
// set while lh_forward_static runs on this thread: its stages take no events
// (creating one may allocate)
thread_local bool t_untimed = false;
std::vector<TimedLaunch> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

const char* kStageNames[ST_COUNT] = {
    "pool_score", "pool_up", "topk", "gather", "sub_prep", "attn_fwd", "scatter_fwd",
    "zero_acc", "scatter_bwd", "bwd_prep", "attn_bwd", "pool_bwd",
    "proj_qkv", "proj_out", "proj_out_dx", "proj_out_dw", "proj_qkv_dx", "proj_qkv_dw"};

}  // namespace

StageMark stage_open(hipStream_t s) {
    StageMark m;
    if (t_untimed) return m;
    {
        std::lock_guard<std::mutex> g(g_mu);
        if (!g_timing) return m;
        m.a = take_event();
        m.b = take_event();
    }
    if (m.a && m.b) (void)hipEventRecord(m.a, s);
    return m;
}

void stage_close(int id, hipStream_t s, const StageMark& m) {
    if (!m.a || !m.b) return;
    (void)hipEventRecord(m.b, s);
    std::lock_guard<std::mutex> g(g_mu);
    g_recs.push_back({id, m.a, m.b});
}

// ------------------------------------------------ forward without allocation
// The workspace of lh_forward_static: one array per device, allocated with the
// library's code on each device and held until the process ends.  Host code
// never uses the symbol itself (on the host it is only a stand-in): the device
// address is looked up once per device and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[LH_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];

// The array's address on the current device, looked up on the first call
// there; null when the lookup fails.
void* scratch_on_current_device(int* dev_out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    *dev_out = dev;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_dev[dev] = ptr;
    }
    return g_scratch_dev[dev];
}
}  // namespace

}  // namespace lh

using namespace lh;

#define LH_TRY(expr)                               \
    do {                                           \
        if ((expr) != hipSuccess) return LH_ERR_HIP; \
    } while (0)

extern "C" {

int64_t lh_subseq_len(int N, int p, int L, int K) { return subseq_len(N, p, L, K); }

size_t lh_workspace_bytes(int N, int H, int d, int p, int L, int K, int dtype) {
    Plan P;
    if (make_plan(N, H, d, p, L, K, dtype, &P) != LH_OK) return 0;
    return P.total;
}

static int check_ws(const Plan& P, const void* ws, size_t ws_bytes, bool fwd_only = false) {
    if (!ws) return LH_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return LH_ERR_WORKSPACE;
    if (ws_bytes < (fwd_only ? P.fwd_total : P.total)) return LH_ERR_WORKSPACE;
    return LH_OK;
}

static bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

static const uint16_t* u16(char* w, size_t off) { return reinterpret_cast<const uint16_t*>(w + off); }
static uint16_t* u16m(char* w, size_t off) { return reinterpret_cast<uint16_t*>(w + off); }
static float* f32(char* w, size_t off) { return reinterpret_cast<float*>(w + off); }

static AttnArgs sub_attn_args(const Plan& P, char* w) {
    AttnArgs a{};
    a.qh = u16(w, P.off_qh); a.ql = u16(w, P.off_ql);
    a.kh = u16(w, P.off_kh); a.kl = u16(w, P.off_kl);
    a.vh = u16(w, P.off_vh); a.vl = u16(w, P.off_vl);
    a.doh = u16(w, P.off_doh); a.dol = u16(w, P.off_dol);
    a.hscale = f32(w, P.off_hscale);
    a.o = f32(w, P.off_os);
    a.lse = f32(w, P.off_lse);
    a.lse2 = f32(w, P.off_lse2);
    a.D = f32(w, P.off_D);
    a.dq = f32(w, P.off_dq); a.dk = f32(w, P.off_dk); a.dv = f32(w, P.off_dv);
    a.rows = P.S; a.Sp = P.Sp;
    a.H = P.H; a.d = P.d;
    a.split = true;
    a.fp32_path = P.dtype == FP32;
    a.scale = 1.0f / sqrtf((float)P.d);
    a.qf = f32(w, P.off_qs); a.kf = f32(w, P.off_ks); a.vf = f32(w, P.off_vs); a.dof = f32(w, P.off_dos);
    return a;
}

// fp16 hi/lo rows of one [H][Sp][d] fp32 tensor
static SplitSpec split_spec(const Plan& P, char* w, size_t src, unsigned int* hmax, int slot, size_t rh, size_t rl) {
    SplitSpec sp{};
    sp.src = w + src; sp.ld = P.d; sp.hs = P.Sp * P.d; sp.rows = P.Sp; sp.Sp = P.Sp;
    sp.d = P.d; sp.H = P.H; sp.src_bf16 = 0;
    sp.hmax = hmax; sp.hscale = f32(w, P.off_hscale); sp.slot = slot;
    sp.rh = u16m(w, rh); sp.rl = u16m(w, rl);
    return sp;
}

int lh_forward(const void* q, const void* k, const void* v, void* o, int N, int H, int d, int p, int L,
               int K, int dtype, void* ws, size_t ws_bytes, void* stream) {
    return lh_forward_scored(q, k, v, o, N, H, d, p, L, K, dtype, LH_SCORE_QK, ws, ws_bytes, stream);
}

int lh_forward_scored(const void* q, const void* k, const void* v, void* o, int N, int H, int d, int p, int L,
                      int K, int dtype, int score_mode, void* ws, size_t ws_bytes, void* stream) {
    return lh_forward_sel(q, k, v, o, N, H, d, p, L, K, dtype, score_mode, LH_SELECT_PARTITION, ws, ws_bytes,
                          stream);
}

int lh_forward_sel(const void* q, const void* k, const void* v, void* o, int N, int H, int d, int p, int L, int K,
                   int dtype, int score_mode, int select_mode, void* ws, size_t ws_bytes, void* stream) {
    return forward_strided(q, k, v, o, N, H, d, p, L, K, dtype, score_mode, select_mode, ws, ws_bytes, stream,
                           (int64_t)H * d);
}

}  // extern "C"

namespace lh {
int forward_strided(const void* q, const void* k, const void* v, void* o, int N, int H, int d, int p, int L, int K,
                    int dtype, int score_mode, int select_mode, void* ws, size_t ws_bytes, void* stream,
                    int64_t in_ld, bool fwd_only) {
    Plan P;
    int rc = make_plan(N, H, d, p, L, K, dtype, &P, select_mode);
    if (rc) return rc;
    if (in_ld < (int64_t)H * d || in_ld % 8 != 0) return LH_ERR_ARG;
    P.in_ld = in_ld;
    P.keep_leaves = (score_mode & LH_SCORE_KEEP_LEAVES) ? 1 : 0;
    score_mode &= ~LH_SCORE_KEEP_LEAVES;
    if (score_mode < LH_SCORE_QK || score_mode > LH_SCORE_QK_PRODUCT) return LH_ERR_DTYPE;
    P.score_mode = score_mode;
    if (!q || !k || !v || !o) return LH_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LH_ERR_ARG;
    if ((rc = check_ws(P, ws, ws_bytes, fwd_only))) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    LH_TRY(stage(ST_POOL_SCORE, s, [&] { return launch_pool_score(P, q, k, v, w, s); }));
    if (L > 1 && P.m < L - 1) LH_TRY(stage(ST_POOL_UP, s, [&] { return launch_pool_up(P, w, s); }));
    LH_TRY(stage(ST_TOPK, s, [&] {
        // parent kept: the level maps start empty; the selector fills in the kept entries
        // (rounded up to 16 bytes, inside the segment's 256-byte alignment)
        const size_t mb = (P.off_lmap_bytes() + 15) & ~(size_t)15;
        hipError_t e = P.pk ? launch_fill_zero(w + P.off_lmap, mb, s) : hipSuccess;
        return e == hipSuccess ? launch_topk(P, w, s) : e;
    }));
    LH_TRY(stage(ST_GATHER, s, [&] { return launch_gather(P, q, k, v, w, s); }));
    unsigned int* hmax = reinterpret_cast<unsigned int*>(w + P.off_hmax);
    LH_TRY(stage(ST_SUB_PREP, s, [&] {
        if (dtype != BF16) return hipSuccess;
        // per-head max |x| of q~, k~, v~ from the row maxima the gather left
        unsigned int* out[3] = {hmax, hmax + 1, hmax + 2};
        hipError_t e = launch_head_max(f32(w, P.off_rowmax), out, 3, P.S, P.Sp, H, s);
        const SplitSpec sp[3] = {
            split_spec(P, w, P.off_qs, hmax, 0, P.off_qh, P.off_ql),
            split_spec(P, w, P.off_ks, hmax, 1, P.off_kh, P.off_kl),
            split_spec(P, w, P.off_vs, hmax, 2, P.off_vh, P.off_vl)};
        if (e == hipSuccess) e = launch_split(sp, 3, s);
        return e;
    }));
    AttnArgs a = sub_attn_args(P, w);
    if (P.rowcopy) {
        // the attention kernel scatters O~ to the tokens itself (stage (iv)), rounded once to bf16
        a.o_tok = reinterpret_cast<uint16_t*>(o);
        a.start = reinterpret_cast<const int32_t*>(w + P.off_start);
        a.level = reinterpret_cast<const uint8_t*>(w + P.off_level);
        a.p = p;
        a.tok_ld = (int64_t)H * d;
    }
    LH_TRY(stage(ST_ATTN_FWD, s, [&] { return launch_attn_fwd(a, s); }));
    if (!P.rowcopy) LH_TRY(stage(ST_SCATTER_FWD, s, [&] {
        if (P.pk) {
            // overlapping entries: every token sums the outputs of the entries that cover it
            const float* tab[1] = {f32(w, P.off_os)};
            void* out[1] = {o};
            return launch_sum_copy(P, w, tab, out, 1, false, (int64_t)H * d, s);
        }
        return launch_scatter_fwd(P, w, o, s);
    }));
    return LH_OK;
}

int backward_strided(const void* dout, void* dq, void* dk, void* dv, int N, int H, int d, int p, int L, int K,
                     int dtype, int scatter_mode, void* ws, size_t ws_bytes, void* stream, int64_t grad_ld,
                     int select_mode) {
    Plan P;
    int rc = make_plan(N, H, d, p, L, K, dtype, &P, select_mode);
    if (rc) return rc;
    const bool keep_sub = (scatter_mode & LH_BWD_KEEP_SUB) != 0;
    scatter_mode &= ~LH_BWD_KEEP_SUB;
    if (scatter_mode != LH_SCATTER_FP_ATOMIC && scatter_mode != LH_SCATTER_INT_ATOMIC) return LH_ERR_DTYPE;
    if (grad_ld != (int64_t)H * d &&
        (!(P.rowcopy || P.pk) || grad_ld < (int64_t)H * d || grad_ld % 8 != 0))
        return LH_ERR_ARG;
    if (!dout || !dq || !dk || !dv) return LH_ERR_ARG;
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return LH_ERR_ARG;
    if ((rc = check_ws(P, ws, ws_bytes))) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    const size_t HSd = (size_t)H * P.Sp * d;
    unsigned int* hmax = reinterpret_cast<unsigned int*>(w + P.off_hmax);
    unsigned int* hmax_b = hmax + 4 * (size_t)H;
    // the fp32 atomics add into cleared rows.  They only run for entries above level m,
    // which span several blocks; with m = L-1 every entry is stored whole, as in the
    // deterministic mode, and row preparation reads no row it has not written
    if ((scatter_mode == LH_SCATTER_FP_ATOMIC && P.m < P.L - 1) || P.pk)
        LH_TRY(stage(ST_ZERO_ACC, s, [&] { return launch_fill_zero(w + P.off_acc, sizeof(float) * HSd, s); }));
    // parent kept: each entry's sum of dO is taken by one wavefront (no atomics), in the
    // fp32 layout of the fp-atomic accumulators
    const int acc_mode = P.pk ? LH_SCATTER_FP_ATOMIC : scatter_mode;
    LH_TRY(stage(ST_SCATTER_BWD, s, [&] {
        return P.pk ? launch_entry_sum(P, dout, w, s) : launch_scatter_bwd(P, dout, scatter_mode, w, s);
    }));
    LH_TRY(stage(ST_BWD_PREP, s, [&] {
        RowPrepSpec rp{};
        rp.acc = w + P.off_acc; rp.o = w + P.off_os;
        rp.part = f32(w, P.off_part);
        rp.start = reinterpret_cast<const int32_t*>(w + P.off_start);
        rp.level = reinterpret_cast<const uint8_t*>(w + P.off_level);
        rp.tok = P.tok; rp.nblk = P.N / P.tok; rp.m = P.m; rp.p = P.p;
        rp.dos = f32(w, P.off_dos); rp.D = f32(w, P.off_D);
        rp.in_place = 1;
        rp.S = P.S; rp.Sp = P.Sp; rp.H = H; rp.d = d; rp.mode = acc_mode; rp.dense = 0;
        float* rowmax_b = f32(w, P.off_rowmax) + 3 * (size_t)H * P.Sp;
        rp.rowmax = dtype == BF16 ? rowmax_b : nullptr;
        hipError_t e = launch_row_prep(rp, s);
        if (e != hipSuccess || dtype != BF16) return e;
        unsigned int* out[1] = {hmax_b + 3};
        e = launch_head_max(rowmax_b, out, 1, P.S, P.Sp, H, s);
        const SplitSpec sp = split_spec(P, w, P.off_dos, hmax_b, 3, P.off_doh, P.off_dol);
        if (e == hipSuccess) e = launch_split(&sp, 1, s);
        return e;
    }));
    AttnArgs a = sub_attn_args(P, w);
    if (P.rowcopy) {
        // the gradient kernels apply the pool adjoint themselves: dX~ / p^level to every
        // token of the entry, rounded once to bf16
        a.dq_tok = reinterpret_cast<uint16_t*>(dq);
        a.dk_tok = reinterpret_cast<uint16_t*>(dk);
        a.dv_tok = reinterpret_cast<uint16_t*>(dv);
        a.start = reinterpret_cast<const int32_t*>(w + P.off_start);
        a.level = reinterpret_cast<const uint8_t*>(w + P.off_level);
        a.p = p;
        a.tok_ld = grad_ld;
        // the fp32 dQ~, dK~, dV~ rows are read by nothing after the attention here:
        // stored only on request
        if (!keep_sub) a.dq = a.dk = a.dv = nullptr;
    }
    // dK/dV and dQ in one launch: each role's token writes overlap the other's MFMA work
    LH_TRY(stage(ST_ATTN_BWD, s, [&] { return launch_attn_bwd(a, s); }));
    if (!P.rowcopy) LH_TRY(stage(ST_POOL_BWD, s, [&] {
        if (P.pk) {
            // a token sums dX~ / p^level over the entries that cover it
            const float* tab[3] = {f32(w, P.off_dq), f32(w, P.off_dk), f32(w, P.off_dv)};
            void* out[3] = {dq, dk, dv};
            return launch_sum_copy(P, w, tab, out, 3, true, grad_ld, s);
        }
        return launch_pool_bwd(P, w, dq, dk, dv, s);
    }));
    return LH_OK;
}
}  // namespace lh

extern "C" {

int lh_forward_static(const void* q, const void* k, const void* v, void* o, int N, int H, int d, int p, int L,
                      int K, int dtype, void* stream) {
    Plan P;
    int rc = make_plan(N, H, d, p, L, K, dtype, &P);
    if (rc) return rc;
    if (P.fwd_total > (size_t)LH_STATIC_SCRATCH_BYTES) return LH_ERR_SCRATCH;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev = -1;
    void* ws = scratch_on_current_device(&dev);
    if (!ws) return LH_ERR_HIP;
    if (s) {   // the stream must belong to the current device, whose array is used
        int sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return LH_ERR_HIP;
        if (sdev != dev) return LH_ERR_ARG;
    }
    t_untimed = true;
    rc = forward_strided(q, k, v, o, N, H, d, p, L, K, dtype, LH_SCORE_QK, LH_SELECT_PARTITION, ws,
                         (size_t)LH_STATIC_SCRATCH_BYTES, stream, (int64_t)H * d, true);
    t_untimed = false;
    return rc;
}

int lh_backward(const void* dout, void* dq, void* dk, void* dv, int N, int H, int d, int p, int L, int K,
                int dtype, int scatter_mode, void* ws, size_t ws_bytes, void* stream) {
    return backward_strided(dout, dq, dk, dv, N, H, d, p, L, K, dtype, scatter_mode, ws, ws_bytes, stream,
                            (int64_t)H * d);
}

int lh_backward_sel(const void* dout, void* dq, void* dk, void* dv, int N, int H, int d, int p, int L, int K,
                    int dtype, int scatter_mode, int select_mode, void* ws, size_t ws_bytes, void* stream) {
    return backward_strided(dout, dq, dk, dv, N, H, d, p, L, K, dtype, scatter_mode, ws, ws_bytes, stream,
                            (int64_t)H * d, select_mode);
}

int64_t lh_subseq_len_sel(int N, int p, int L, int K, int select_mode) {
    return subseq_len(N, p, L, K, select_mode);
}

size_t lh_workspace_bytes_sel(int N, int H, int d, int p, int L, int K, int dtype, int select_mode) {
    Plan P;
    if (make_plan(N, H, d, p, L, K, dtype, &P, select_mode) != LH_OK) return 0;
    return P.total;
}

int lh_workspace_view(void* ws, int N, int H, int d, int p, int L, int K, int dtype, int view, void** ptr,
                      size_t* bytes) {
    return lh_workspace_view_sel(ws, N, H, d, p, L, K, dtype, LH_SELECT_PARTITION, view, ptr, bytes);
}

int lh_workspace_view_sel(void* ws, int N, int H, int d, int p, int L, int K, int dtype, int select_mode, int view,
                          void** ptr, size_t* bytes) {
    Plan P;
    int rc = make_plan(N, H, d, p, L, K, dtype, &P, select_mode);
    if (rc) return rc;
    if (!ws || !ptr || !bytes) return LH_ERR_ARG;
    char* w = reinterpret_cast<char*>(ws);
    const size_t HSd = (size_t)H * P.Sp * d;
    size_t off = 0, n = 0;
    switch (view) {
        case LH_VIEW_SCORES: {
            off = P.off_scores;
            size_t tot = 0;
            for (int l = 0; l < L; ++l) tot += (size_t)H * P.n[l];
            n = sizeof(float) * tot;
            break;
        }
        case LH_VIEW_SEL_START: off = P.off_start; n = sizeof(int32_t) * (size_t)H * P.S; break;
        case LH_VIEW_SEL_LEVEL: off = P.off_level; n = (size_t)H * P.S; break;
        case LH_VIEW_QSUB: off = P.off_qs; n = sizeof(float) * HSd; break;
        case LH_VIEW_KSUB: off = P.off_ks; n = sizeof(float) * HSd; break;
        case LH_VIEW_VSUB: off = P.off_vs; n = sizeof(float) * HSd; break;
        case LH_VIEW_OSUB: off = P.off_os; n = sizeof(float) * HSd; break;
        case LH_VIEW_LSE: off = P.off_lse; n = sizeof(float) * (size_t)H * P.Sp; break;
        case LH_VIEW_DOSUB: off = P.off_dos; n = sizeof(float) * HSd; break;
        case LH_VIEW_DQSUB: off = P.off_dq; n = sizeof(float) * HSd; break;
        case LH_VIEW_DKSUB: off = P.off_dk; n = sizeof(float) * HSd; break;
        case LH_VIEW_DVSUB: off = P.off_dv; n = sizeof(float) * HSd; break;
        case LH_VIEW_BLOCK_FIRST: off = P.off_bfirst; n = sizeof(int32_t) * (size_t)H * (P.ntop + 1); break;
        default: return LH_ERR_ARG;
    }
    *ptr = w + off;
    *bytes = n;
    return LH_OK;
}

int lh_read_selection(const void* ws, int N, int H, int d, int p, int L, int K, int dtype, int32_t* start,
                      uint8_t* level, void* stream) {
    return lh_read_selection_sel(ws, N, H, d, p, L, K, dtype, LH_SELECT_PARTITION, start, level, stream);
}

int lh_read_selection_sel(const void* ws, int N, int H, int d, int p, int L, int K, int dtype, int select_mode,
                          int32_t* start, uint8_t* level, void* stream) {
    Plan P;
    int rc = make_plan(N, H, d, p, L, K, dtype, &P, select_mode);
    if (rc) return rc;
    if (!ws || (!start && !level)) return LH_ERR_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const char* w = reinterpret_cast<const char*>(ws);
    const size_t n = (size_t)H * P.S;
    if (start && hipMemcpyAsync(start, w + P.off_start, n * sizeof(int32_t), hipMemcpyDeviceToDevice, s) != hipSuccess)
        return LH_ERR_HIP;
    if (level && hipMemcpyAsync(level, w + P.off_level, n, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return LH_ERR_HIP;
    return LH_OK;
}

int lh_peak_probe(int kind, const void* src, void* dst, size_t n, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!dst || n == 0) return LH_ERR_ARG;
    if (kind >= 0 && kind <= 2) {
        if (n % 16 != 0 || (kind != 1 && !src)) return LH_ERR_ARG;
        if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16 != 0) return LH_ERR_ARG;
    } else if (kind == 5) {
        // whole 64 MiB groups (16 heads x 16384 tokens x 256 bytes), within a 32-bit grid
        if (n % ((size_t)64 << 20) != 0 || n > ((size_t)1 << 40) || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
            return LH_ERR_ARG;
    } else if (kind == 4) {
        if (!src || n > (1u << 20) || (reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16 != 0)
            return LH_ERR_ARG;
    } else if (kind != 3 || n > (1u << 30)) {
        return LH_ERR_ARG;
    }
    return launch_peak_probe(kind, src, dst, n, s) == hipSuccess ? LH_OK : LH_ERR_HIP;
}

// ------------------------------------------------------------ dense path
static int dense_check(int N, int H, int d, int dtype) {
    if (dtype != BF16) return LH_ERR_DTYPE;
    if (N <= 0 || H <= 0) return LH_ERR_ARG;
    if (d != 64 && d != 128) return LH_ERR_SHAPE;
    if (N % 64 != 0 || (int64_t)H * d > 8192) return LH_ERR_SHAPE;
    return LH_OK;
}

struct DenseLayout {
    size_t qh, kh, vh, doh, o32, hmax, hscale, lse2, D, total;
};
static DenseLayout dense_layout(int N, int H, int d) {
    DenseLayout L{};
    const size_t t = 2 * (size_t)H * d * N;
    const size_t r = sizeof(float) * (size_t)H * N;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.qh = take(t); L.kh = take(t); L.vh = take(t); L.doh = take(t);
    L.o32 = take(2 * t);
    L.hmax = take(sizeof(uint32_t) * 4 * (size_t)H);
    L.hscale = take(sizeof(float) * 4 * (size_t)H);
    L.lse2 = take(r); L.D = take(r);
    L.total = off;
    return L;
}

size_t lh_dense_workspace_bytes(int N, int H, int d, int dtype) {
    if (dense_check(N, H, d, dtype)) return 0;
    return dense_layout(N, H, d).total;
}

// Dense operands are bf16 inputs [N][H][d]: exact in the 16-bit formats, so
// no lo parts are needed.
static hipError_t dense_split(const void* src, int N, int H, int d, char* w, const DenseLayout& DL, int slot,
                              size_t rh, hipStream_t s) {
    SplitSpec sp{};
    sp.src = src; sp.ld = (int64_t)H * d; sp.hs = d; sp.rows = N; sp.Sp = N;
    sp.d = d; sp.H = H; sp.src_bf16 = 1;
    sp.hmax = reinterpret_cast<const unsigned int*>(w + DL.hmax);
    sp.hscale = f32(w, DL.hscale); sp.slot = slot;
    sp.rh = u16m(w, rh);
    return launch_split(&sp, 1, s);
}

static AttnArgs dense_args(int N, int H, int d, char* w, const DenseLayout& DL) {
    AttnArgs a{};
    a.qh = u16(w, DL.qh); a.kh = u16(w, DL.kh); a.vh = u16(w, DL.vh); a.doh = u16(w, DL.doh);
    a.hscale = f32(w, DL.hscale);
    a.lse2 = f32(w, DL.lse2); a.D = f32(w, DL.D);
    a.rows = N; a.Sp = N; a.ld_o = (int64_t)H * d; a.hs_o = d;
    a.H = H; a.d = d; a.split = false; a.fp32_path = false;
    a.scale = 1.0f / sqrtf((float)d);
    return a;
}

// Per-head max |x| of the given bf16 [N][H][d] tensors into slots first..n-1
// (the slots are cleared first; other slots are kept).
static hipError_t dense_maxabs(const void* const* src, int n, int N, int H, int d, char* w, const DenseLayout& DL,
                               hipStream_t s, int first = 0) {
    unsigned int* hmax = reinterpret_cast<unsigned int*>(w + DL.hmax);
    hipError_t e = hipSuccess;
    if (first == 0) e = launch_fill_zero(hmax, sizeof(uint32_t) * 4 * (size_t)H, s);
    else e = launch_clear_slot(hmax, H, first, s);
    for (int t = first; t < n && e == hipSuccess; ++t)
        if (src[t]) {
            unsigned int* out = hmax + t;
            e = launch_maxabs(&src[t], &out, 1, true, (int64_t)H * d, d, N, d, H, s);
        }
    return e;
}

int lh_dense_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int N, int H, int d,
                      int dtype, void* ws, size_t ws_bytes, void* stream) {
    int rc = dense_check(N, H, d, dtype);
    if (rc) return rc;
    if (!q || !k || !v || !o || !lse) return LH_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LH_ERR_ARG;
    const DenseLayout DL = dense_layout(N, H, d);
    if (!ws || reinterpret_cast<uintptr_t>(ws) % 256 || ws_bytes < DL.total) return LH_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    const void* src[3] = {q, k, v};
    LH_TRY(dense_maxabs(src, 3, N, H, d, w, DL, s));
    // every q/k/v copy the matching backward needs is made here
    LH_TRY(dense_split(q, N, H, d, w, DL, 0, DL.qh, s));
    LH_TRY(dense_split(k, N, H, d, w, DL, 1, DL.kh, s));
    LH_TRY(dense_split(v, N, H, d, w, DL, 2, DL.vh, s));
    AttnArgs a = dense_args(N, H, d, w, DL);
    a.o_bf16 = reinterpret_cast<uint16_t*>(o);
    a.o = f32(w, DL.o32);
    a.lse = lse;
    LH_TRY(launch_attn_fwd(a, s));
    return LH_OK;
}

int lh_dense_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int N, int H, int d, int dtype, void* ws,
                      size_t ws_bytes, void* stream) {
    int rc = dense_check(N, H, d, dtype);
    if (rc) return rc;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return LH_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return LH_ERR_ARG;
    const DenseLayout DL = dense_layout(N, H, d);
    if (!ws || reinterpret_cast<uintptr_t>(ws) % 256 || ws_bytes < DL.total) return LH_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    // q, k, v copies and the fp32 output come from the matching forward's workspace
    const void* src[4] = {nullptr, nullptr, nullptr, dout};
    LH_TRY(dense_maxabs(src, 4, N, H, d, w, DL, s, 3));
    LH_TRY(dense_split(dout, N, H, d, w, DL, 3, DL.doh, s));
    RowPrepSpec rp{};
    rp.dout = dout; rp.o = w + DL.o32; rp.ld = (int64_t)H * d; rp.hs = d;
    rp.D = f32(w, DL.D);
    rp.lse_in = lse; rp.lse2 = f32(w, DL.lse2);
    rp.S = N; rp.Sp = N; rp.H = H; rp.d = d; rp.dense = 1;
    LH_TRY(launch_row_prep(rp, s));
    AttnArgs a = dense_args(N, H, d, w, DL);
    a.dq_b = reinterpret_cast<uint16_t*>(dq);
    a.dk_b = reinterpret_cast<uint16_t*>(dk);
    a.dv_b = reinterpret_cast<uint16_t*>(dv);
    LH_TRY(launch_attn_bwd(a, s));
    return LH_OK;
}

// ------------------------------------------------------------ timing / misc
int lh_stage_timing(int enable) {
    std::lock_guard<std::mutex> g(g_mu);
    for (auto& r : g_recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    g_timing = enable != 0;
    return LH_OK;
}

int lh_stage_timing_read(double* ms, int* count, int n) {
    std::vector<TimedLaunch> recs;
    {
        std::lock_guard<std::mutex> g(g_mu);
        recs.swap(g_recs);
    }
    int rc = ST_COUNT;
    for (auto& r : recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
            rc = LH_ERR_HIP;
        } else if (r.stage < n) {
            if (ms) ms[r.stage] += t;
            if (count) count[r.stage] += 1;
        }
    }
    std::lock_guard<std::mutex> g(g_mu);
    for (auto& r : recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    return rc;
}

const char* lh_stage_name(int stage) {
    if (stage < 0 || stage >= ST_COUNT) return "unknown";
    return kStageNames[stage];
}

const char* lh_status_str(int status) {
    switch (status) {
        case LH_OK: return "ok";
        case LH_ERR_ARG: return "invalid argument";
        case LH_ERR_SHAPE: return "unsupported shape";
        case LH_ERR_DTYPE: return "unknown dtype or mode";
        case LH_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case LH_ERR_HIP: return "HIP launch or runtime error";
        case LH_ERR_GEMM: return "GEMM library error or no algorithm for the shape";
        case LH_ERR_SCRATCH: return "the shape needs more forward state than lh_forward_static's static array holds";
        default: return "unknown status";
    }
}

}  // extern "C"
