// C ABI of the block-sparse attention library: argument validation and
// kernel launches.  Every check runs before anything is enqueued, so a call
// that fails did no work.  No device memory is allocated or freed here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "bsa.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

bsa_status fail(bsa_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bsa_status hip_fail(hipError_t e, const char *what)
{
    return fail(BSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates one [B][H][N][D] bfloat16 tensor descriptor.
bsa_status check_tensor(const bsa_tensor *t, const char *name)
{
    if (!t) return fail(BSA_ERR_INVALID_ARG, "%s: null descriptor", name);
    if (!t->data) return fail(BSA_ERR_INVALID_ARG, "%s: null data pointer", name);
    if (t->B <= 0 || t->H <= 0 || t->N <= 0 || t->D <= 0)
        return fail(BSA_ERR_INVALID_ARG, "%s: shape must be positive (B=%lld H=%lld N=%lld D=%lld)",
                    name, (long long)t->B, (long long)t->H, (long long)t->N, (long long)t->D);
    if (t->D != 64 && t->D != 128)
        return fail(BSA_ERR_UNSUPPORTED, "%s: head dim %lld not supported (64 or 128)", name,
                    (long long)t->D);
    if (t->N > (1ll << 30) || t->B * t->H > (1ll << 30))
        return fail(BSA_ERR_UNSUPPORTED, "%s: N or B*H too large", name);
    if (!aligned16(t->data)) return fail(BSA_ERR_INVALID_ARG, "%s: data not 16-byte aligned", name);
    if (t->stride_b % 8 || t->stride_h % 8 || t->stride_n % 8 || t->stride_b < 0 ||
        t->stride_h < 0 || t->stride_n < t->D)
        return fail(BSA_ERR_INVALID_ARG,
                    "%s: strides must be non-negative multiples of 8 with stride_n >= D", name);
    // The kernels address one head's rows through a 32-bit buffer range from
    // the head's base, (N - 1) * stride_n + D elements of 2 bytes.
    if (((t->N - 1) * t->stride_n + t->D) * 2 >= (1ll << 32))
        return fail(BSA_ERR_UNSUPPORTED,
                    "%s: one head spans 4 GiB or more ((N - 1) * stride_n + D elements of 2 bytes)", name);
    return BSA_OK;
}

bool same_shape(const bsa_tensor *a, const bsa_tensor *b)
{
    return a->B == b->B && a->H == b->H && a->N == b->N && a->D == b->D;
}

bsa::Tensor4 t4(const bsa_tensor *t)
{
    return bsa::Tensor4{static_cast<const uint16_t *>(t->data), t->stride_b, t->stride_h,
                        t->stride_n};
}

bool block_ok(int32_t block) { return block == 64 || block == 128; }


size_t exact_slot_bytes(int64_t nB, int32_t block) { return (size_t)nB * block * sizeof(float); }

int64_t select_row_bound(int64_t nB, int64_t tb, const bsa_group *g, int32_t ng)
{
    int64_t k = tb;
    for (int32_t x = 0; x < ng; ++x) k += g[x].k;
    return k < nB ? k : nB;
}

// Byte layout of the long-row splitting workspace: counts, work list, split
// rows, partial-result slots (each region 256-byte aligned).
struct SplitLayout {
    size_t items, split_rows, partials, total;
};

SplitLayout split_layout(int64_t rows, int32_t block, int64_t D, int32_t max_chunks, int64_t max_split_rows)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    SplitLayout l;
    const int64_t n_items = rows + max_split_rows * (max_chunks - 1);
    l.items = 256;
    l.split_rows = l.items + up((size_t)n_items * 16);
    l.partials = l.split_rows + up((size_t)max_split_rows * 8);
    l.total = l.partials + (size_t)max_split_rows * max_chunks *
                               (size_t)bsa::partial_slot_floats(block, (int)D) * sizeof(float);
    return l;
}

// FP8 operands: shape of the descriptor and alignment of its arrays.
bsa_status check_fp8(const bsa_fp8_qkv *t, const char *name)
{
    if (!t) return fail(BSA_ERR_INVALID_ARG, "%s: null descriptor", name);
    if (!t->q8 || !t->q_scale || !t->k8 || !t->k_scale || !t->v8t || !t->v_scale)
        return fail(BSA_ERR_INVALID_ARG, "%s: null array", name);
    if (t->B <= 0 || t->H <= 0 || t->N <= 0 || t->D <= 0)
        return fail(BSA_ERR_INVALID_ARG, "%s: shape must be positive", name);
    if (t->D != 64 && t->D != 128)
        return fail(BSA_ERR_UNSUPPORTED, "%s: head dim %lld not supported (64 or 128)", name, (long long)t->D);
    if (t->N > (1ll << 24) || t->B * t->H > (1ll << 30))
        return fail(BSA_ERR_UNSUPPORTED, "%s: N above 2^24 or B*H too large", name);
    if (!aligned16(t->q8) || !aligned16(t->q_scale) || !aligned16(t->k8) || !aligned16(t->k_scale) ||
        !aligned16(t->v8t) || !aligned16(t->v_scale))
        return fail(BSA_ERR_INVALID_ARG, "%s: arrays must be 16-byte aligned", name);
    return BSA_OK;
}

// Quantisation workspace: reciprocal channel scales [B*H][D], then the
// channel maxima of 256-key chunks [B*H][ceil(N/256)][D] (256-byte aligned).
size_t fp8_ws_inv_bytes(int64_t BH, int64_t D) { return ((size_t)(BH * D) * sizeof(float) + 255) & ~(size_t)255; }

// RSE chunks: about 64 K elements per workgroup, at most 1024 per head.
int32_t rse_chunks(int64_t N, int64_t D)
{
    int64_t c = ceil_div(N * D, 65536);
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(c, 1024));
}

}  // namespace

extern "C" {

const char *bsa_status_string(bsa_status s)
{
    switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARG: return "BSA_ERR_INVALID_ARG";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_CAPACITY: return "BSA_ERR_CAPACITY";
    case BSA_ERR_WORKSPACE: return "BSA_ERR_WORKSPACE";
    case BSA_ERR_HIP: return "BSA_ERR_HIP";
    default: return "BSA_ERR_UNKNOWN";
    }
}

const char *bsa_last_error(void) { return g_err; }

int32_t bsa_reuse_full_steps(int32_t steps, double skip)
{
    if (steps < 1 || !(skip >= 0.0 && skip <= 1.0)) return -1;
    // floor of steps * skip; the guard keeps a product rounded just below an
    // integer (10 * 0.3 = 2.9999999999999996) at that integer
    const double f = std::floor((double)steps * skip + 1e-9);
    return (int32_t)std::min<double>(steps, f);
}

int32_t bsa_reuse_step_action(int32_t steps, double skip, int32_t step)
{
    const int32_t n_full = bsa_reuse_full_steps(steps, skip);
    if (n_full < 0 || step < 0 || step >= steps) return -1;
    if (step < n_full) return BSA_STEP_FULL;
    return step == n_full ? BSA_STEP_SELECT : BSA_STEP_SPARSE;
}

const char *bsa_version(void) { return "bsa 0.1.0 gfx950"; }

// ---------------------------------------------------------------------------
size_t bsa_pool_scores_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int32_t block,
                                      int32_t mode, int32_t r)
{
    (void)D;
    if (B <= 0 || H <= 0 || N <= 0 || !block_ok(block)) return 0;
    const int64_t nB = ceil_div(N, block);
    if (mode == BSA_SCORE_MEANPOOL_PROJ) {
        if (r <= 0) return 0;
        return (size_t)(2 * B * H * nB * (int64_t)r) * sizeof(float);
    }
    if (mode == BSA_SCORE_EXACT_AVGPOOL) {
        int64_t slots = B * H * nB;
        if (slots > bsa::kExactSlots) slots = bsa::kExactSlots;
        return (size_t)slots * exact_slot_bytes(nB, block);
    }
    return 0;
}

bsa_status bsa_pool_scores(const bsa_tensor *q, const bsa_tensor *k, int32_t block, int32_t mode,
                           const float *w, int32_t r, float scale, float *scores, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if ((st = check_tensor(k, "k")) != BSA_OK) return st;
    if (!same_shape(q, k)) return fail(BSA_ERR_INVALID_ARG, "q and k shapes differ");
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (!scores) return fail(BSA_ERR_INVALID_ARG, "scores is null");
    if (mode != BSA_SCORE_MEANPOOL_PROJ && mode != BSA_SCORE_EXACT_AVGPOOL)
        return fail(BSA_ERR_UNSUPPORTED, "unknown scoring mode %d", mode);
    if (std::isnan(scale)) return fail(BSA_ERR_INVALID_ARG, "scale is NaN");
    const int64_t nB = ceil_div(q->N, block);
    const size_t need = bsa_pool_scores_workspace_size(q->B, q->H, q->N, q->D, block, mode, r);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;

    if (mode == BSA_SCORE_MEANPOOL_PROJ) {
        if (!w) return fail(BSA_ERR_INVALID_ARG, "projection w is null");
        if (r < 1 || r > 64) return fail(BSA_ERR_INVALID_ARG, "projection width r=%d outside 1..64", r);
        if (!workspace || workspace_bytes < need)
            return fail(BSA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
        bsa::PoolParams pp{};
        pp.x[0] = t4(q);
        pp.x[1] = t4(k);
        pp.w = w;
        pp.proj = static_cast<float *>(workspace);
        pp.B = (int32_t)q->B; pp.H = (int32_t)q->H; pp.N = (int32_t)q->N;
        pp.nB = (int32_t)nB; pp.r = r;
        if ((e = bsa::launch_pool_proj(pp, block, (int)q->D, s)) != hipSuccess)
            return hip_fail(e, "pool launch");
        bsa::ScoreParams sp{};
        sp.proj = pp.proj;
        sp.S = scores;
        sp.BH = (int32_t)(q->B * q->H);
        sp.nB = (int32_t)nB;
        sp.r = r;
        if ((e = bsa::launch_scores(sp, s)) != hipSuccess) return hip_fail(e, "score launch");
        return BSA_OK;
    }

    // EXACT_AVGPOOL
    const size_t slot = exact_slot_bytes(nB, block);
    if (!workspace || workspace_bytes < slot)
        return fail(BSA_ERR_WORKSPACE, "workspace needs at least %zu bytes (%zu for full speed)", slot,
                    need);
    int64_t slots = (int64_t)(workspace_bytes / slot);
    const int64_t items = q->B * q->H * nB;
    if (slots > items) slots = items;
    if (slots > bsa::kExactSlots) slots = bsa::kExactSlots;
    bsa::ExactParams ep{};
    ep.q = t4(q);
    ep.k = t4(k);
    ep.S = scores;
    ep.scratch = static_cast<float *>(workspace);
    ep.B = (int32_t)q->B; ep.H = (int32_t)q->H; ep.N = (int32_t)q->N; ep.nB = (int32_t)nB;
    const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)q->D);
    ep.scale_log2 = sc * 1.4426950408889634f;
    if ((e = bsa::launch_exact_scores(ep, block, (int)q->D, (int)slots, s)) != hipSuccess)
        return hip_fail(e, "exact score launch");
    return BSA_OK;
}

// ---------------------------------------------------------------------------
// Block scores without a caller workspace, for callers that cannot allocate.
// The workspace is a file-scope device array; host code only ever uses the
// address hipGetSymbolAddress returns for it on each device (the array's
// name is a host-side stand-in, not a device address).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[BSA_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices];   // per device, resolved on its first call

// The current device's copy of the scratch array (resolved once per device,
// with that device current).
bsa_status device_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(BSA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(BSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return BSA_OK;
}
}  // namespace

bsa_status bsa_pool_scores_noalloc(const bsa_tensor *q, const bsa_tensor *k, int32_t block, int32_t mode,
                                   const float *w, int32_t r, float scale, float *scores, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    size_t bytes = 0;
    if (mode == BSA_SCORE_MEANPOOL_PROJ) {
        if (r < 1 || r > 64) return fail(BSA_ERR_INVALID_ARG, "projection width r=%d outside 1..64", r);
        bytes = bsa_pool_scores_workspace_size(q->B, q->H, q->N, q->D, block, mode, r);
        if (bytes > BSA_SCRATCH_BYTES)
            return fail(BSA_ERR_WORKSPACE,
                        "needs %zu bytes of scratch, above the %u this entry point holds per device "
                        "(use bsa_pool_scores with a workspace)", bytes, (unsigned)BSA_SCRATCH_BYTES);
    } else if (mode == BSA_SCORE_EXACT_AVGPOOL) {
        const size_t slot = exact_slot_bytes(ceil_div(q->N, block), block);
        if (slot > BSA_SCRATCH_BYTES)
            return fail(BSA_ERR_WORKSPACE,
                        "one exact-score slot needs %zu bytes, above the %u of scratch this entry point "
                        "holds per device (use bsa_pool_scores with a workspace)", slot,
                        (unsigned)BSA_SCRATCH_BYTES);
        // as many slots as the scratch holds, up to what bsa_pool_scores would use
        const size_t full = bsa_pool_scores_workspace_size(q->B, q->H, q->N, q->D, block, mode, r);
        bytes = std::min<size_t>(full, (BSA_SCRATCH_BYTES / slot) * slot);
    } else {
        return fail(BSA_ERR_UNSUPPORTED, "unknown scoring mode %d", mode);
    }
    void *ws = nullptr;
    if ((st = device_scratch(&ws)) != BSA_OK) return st;
    return bsa_pool_scores(q, k, block, mode, w, r, scale, scores, ws, bytes, stream);
}

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bsa_score_grad_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int32_t block, int32_t r)
{
    if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || !block_ok(block) || r < 1 || r > 64) return 0;
    const size_t rows = (size_t)(B * H * ceil_div(N, block));
    const size_t f = sizeof(float);
    const size_t parts = (size_t)(B * H) * (size_t)ceil_div(ceil_div(N, block), bsa::kGradChunk);
    return up256(2 * rows * r * f) + up256(2 * rows * D * f) + up256(2 * rows * r * f) + up256(parts * D * r * f);
}

bsa_status bsa_score_grad(const bsa_tensor *q, const bsa_tensor *k, int32_t block, const float *w, int32_t r,
                          const float *dscores, float *dw, float *dq_pool, float *dk_pool, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if ((st = check_tensor(k, "k")) != BSA_OK) return st;
    if (!same_shape(q, k)) return fail(BSA_ERR_INVALID_ARG, "q and k shapes differ");
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (!w || !dscores || !dw) return fail(BSA_ERR_INVALID_ARG, "w / dscores / dw null");
    if (r < 1 || r > 64) return fail(BSA_ERR_INVALID_ARG, "projection width r=%d outside 1..64", r);
    const int64_t nB = ceil_div(q->N, block);
    if (q->B * q->H * nB >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many blocks");
    const size_t need = bsa_score_grad_workspace_size(q->B, q->H, q->N, q->D, block, r);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need)
        return fail(BSA_ERR_WORKSPACE, "score gradient workspace needs %zu bytes (16-byte aligned)", need);
    const size_t rows = (size_t)(q->B * q->H * nB);
    char *ws = static_cast<char *>(workspace);
    float *proj = reinterpret_cast<float *>(ws);
    ws += up256(2 * rows * r * sizeof(float));
    float *mean = reinterpret_cast<float *>(ws);
    ws += up256(2 * rows * q->D * sizeof(float));
    float *g = reinterpret_cast<float *>(ws);
    ws += up256(2 * rows * r * sizeof(float));
    float *wpart = reinterpret_cast<float *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;

    bsa::PoolParams pp{};
    pp.x[0] = t4(q);
    pp.x[1] = t4(k);
    pp.w = w;
    pp.proj = proj;
    pp.mean = mean;
    pp.B = (int32_t)q->B; pp.H = (int32_t)q->H; pp.N = (int32_t)q->N;
    pp.nB = (int32_t)nB; pp.r = r;
    if ((e = bsa::launch_pool_proj(pp, block, (int)q->D, s)) != hipSuccess) return hip_fail(e, "pool launch");
    bsa::ScoreGradParams gp{};
    gp.proj = proj;
    gp.mean = mean;
    gp.dS = dscores;
    gp.w = w;
    gp.g = g;
    gp.dpool[0] = dq_pool;
    gp.dpool[1] = dk_pool;
    gp.wpart = wpart;
    gp.dw = dw;
    gp.BH = (int32_t)(q->B * q->H);
    gp.nB = (int32_t)nB;
    gp.D = (int32_t)q->D;
    gp.r = r;
    if ((e = bsa::launch_score_grad(gp, s)) != hipSuccess) return hip_fail(e, "score gradient launch");
    return BSA_OK;
}

// ---------------------------------------------------------------------------
// Fused content-driven selection (mean-pool, projection, scores, top-k)
// ---------------------------------------------------------------------------
size_t bsa_select_meanpool_workspace_size(int64_t B, int64_t H, int64_t N, int32_t block, int32_t r)
{
    if (B <= 0 || H <= 0 || N <= 0 || !block_ok(block) || r < 1 || r > 64) return 0;
    const size_t bh = (size_t)(B * H), nB = (size_t)ceil_div(N, block);
    return 2 * bh * nB * (size_t)r * sizeof(float);
}

// The groups in ascending column order (a stable insertion sort of at most
// 8): the selection kernels that write a row's columns as they choose them
// (disjoint groups clear of the text columns) take the groups in this order;
// the bitmask path does not depend on it.
static void groups_by_column(const bsa_group *groups, int32_t n_groups, int32_t *g_begin, int32_t *g_end,
                             int32_t *g_k)
{
    int32_t order[8];
    for (int32_t g = 0; g < n_groups; ++g) {
        int32_t at = g;
        while (at > 0 && groups[order[at - 1]].col_begin > groups[g].col_begin) {
            order[at] = order[at - 1];
            --at;
        }
        order[at] = g;
    }
    for (int32_t g = 0; g < n_groups; ++g) {
        g_begin[g] = groups[order[g]].col_begin;
        g_end[g] = groups[order[g]].col_end;
        g_k[g] = groups[order[g]].k;
    }
}

bsa_status bsa_select_meanpool(const bsa_tensor *q, const bsa_tensor *k, int32_t block, const float *w, int32_t r,
                               int32_t text_blocks, const bsa_group *groups, int32_t n_groups, float *scores,
                               int32_t *row_ptr, int32_t *col_idx, int64_t capacity, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if ((st = check_tensor(k, "k")) != BSA_OK) return st;
    if (!same_shape(q, k)) return fail(BSA_ERR_INVALID_ARG, "q and k shapes differ");
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (!w || !row_ptr || !col_idx) return fail(BSA_ERR_INVALID_ARG, "w, row_ptr or col_idx null");
    if (r < 1 || r > 64) return fail(BSA_ERR_INVALID_ARG, "projection width r=%d outside 1..64", r);
    const int64_t nB = ceil_div(q->N, block);
    if (nB > bsa::kMpsMaxBlocks || nB * ((r + 3) & ~3) > bsa::kMpsMaxProj)
        return fail(BSA_ERR_UNSUPPORTED,
                    "fused selection holds at most %d blocks and %d projection values (r rounded up to a multiple "
                    "of 4) per head (nB=%lld, r=%d); "
                    "use bsa_pool_scores and bsa_select_topk", bsa::kMpsMaxBlocks, bsa::kMpsMaxProj,
                    (long long)nB, r);
    if (q->B * q->H * nB >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many blocks");
    if (text_blocks < 0 || text_blocks > nB)
        return fail(BSA_ERR_INVALID_ARG, "text_blocks %d outside [0, %lld]", text_blocks, (long long)nB);
    if (n_groups < 0 || n_groups > 8) return fail(BSA_ERR_UNSUPPORTED, "at most 8 groups");
    if (n_groups > 0 && !groups) return fail(BSA_ERR_INVALID_ARG, "groups is null");
    for (int32_t g = 0; g < n_groups; ++g) {
        const bsa_group &x = groups[g];
        if (x.col_begin < 0 || x.col_end > nB || x.col_begin >= x.col_end || x.k < 0 || x.k > x.col_end - x.col_begin)
            return fail(BSA_ERR_INVALID_ARG, "group %d = [%d, %d) k=%d invalid for %lld blocks", g, x.col_begin,
                        x.col_end, x.k, (long long)nB);
        if (x.k == 0) continue;
        if (x.col_begin < text_blocks)
            return fail(BSA_ERR_UNSUPPORTED, "fused selection needs groups clear of the text columns; "
                                             "use bsa_pool_scores and bsa_select_topk");
        for (int32_t h = g + 1; h < n_groups; ++h) {
            const bsa_group &y = groups[h];
            if (y.k > 0 && x.col_begin < y.col_end && y.col_begin < x.col_end)
                return fail(BSA_ERR_UNSUPPORTED, "fused selection needs disjoint groups; "
                                                 "use bsa_pool_scores and bsa_select_topk");
        }
    }
    const int64_t need = bsa_select_capacity(q->B, q->H, (int32_t)nB, text_blocks, groups, n_groups);
    if (need >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "nnz bound exceeds int32");
    if (capacity < need)
        return fail(BSA_ERR_CAPACITY, "capacity %lld below bound %lld", (long long)capacity, (long long)need);
    const size_t ws = bsa_select_meanpool_workspace_size(q->B, q->H, q->N, block, r);
    if (!workspace || !aligned16(workspace) || workspace_bytes < ws)
        return fail(BSA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned)", ws);

    char *wsp = static_cast<char *>(workspace);
    bsa::MeanpoolSelectParams mp{};
    mp.q = t4(q);
    mp.k = t4(k);
    mp.w = w;
    mp.proj = reinterpret_cast<float *>(wsp);
    mp.scores = scores;
    mp.row_ptr = row_ptr;
    mp.col_idx = col_idx;
    mp.capacity = capacity;
    mp.B = (int32_t)q->B; mp.H = (int32_t)q->H; mp.N = (int32_t)q->N; mp.nB = (int32_t)nB; mp.r = r;
    mp.text_blocks = text_blocks;
    mp.n_groups = n_groups;
    mp.row_len = (int32_t)select_row_bound(nB, text_blocks, groups, n_groups);
    groups_by_column(groups, n_groups, mp.g_begin, mp.g_end, mp.g_k);
    hipError_t e = bsa::launch_meanpool_select(mp, block, (int)q->D, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "mean-pool selection launch");
    return BSA_OK;
}

// ---------------------------------------------------------------------------
int64_t bsa_select_capacity(int64_t B, int64_t H, int32_t n_blocks, int32_t text_blocks,
                            const bsa_group *groups, int32_t n_groups)
{
    if (B <= 0 || H <= 0 || n_blocks <= 0 || text_blocks < 0 || text_blocks > n_blocks ||
        n_groups < 0 || (n_groups > 0 && !groups))
        return -1;
    const int64_t per_row = select_row_bound(n_blocks, text_blocks, groups, n_groups);
    return B * H * ((int64_t)text_blocks * n_blocks + (int64_t)(n_blocks - text_blocks) * per_row);
}

size_t bsa_select_workspace_size(int64_t B, int64_t H, int32_t n_blocks)
{
    if (B <= 0 || H <= 0 || n_blocks <= 0) return 0;
    return (size_t)(B * H * n_blocks) * (size_t)ceil_div(n_blocks, 32) * sizeof(uint32_t);
}

bsa_status bsa_select_topk(const float *scores, int64_t B, int64_t H, int32_t n_blocks,
                           int32_t text_blocks, const bsa_group *groups, int32_t n_groups,
                           int32_t *row_ptr, int32_t *col_idx, int64_t capacity, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    if (!scores || !row_ptr || !col_idx) return fail(BSA_ERR_INVALID_ARG, "null pointer argument");
    if (B <= 0 || H <= 0 || n_blocks <= 0)
        return fail(BSA_ERR_INVALID_ARG, "B, H and n_blocks must be positive");
    if (n_blocks > bsa::kMaxSelectBlocks)
        return fail(BSA_ERR_UNSUPPORTED, "n_blocks %d above %d", n_blocks, bsa::kMaxSelectBlocks);
    if (text_blocks < 0 || text_blocks > n_blocks)
        return fail(BSA_ERR_INVALID_ARG, "text_blocks %d outside [0, %d]", text_blocks, n_blocks);
    if (n_groups < 0 || n_groups > 8) return fail(BSA_ERR_UNSUPPORTED, "at most 8 groups");
    if (n_groups > 0 && !groups) return fail(BSA_ERR_INVALID_ARG, "groups is null");
    for (int32_t g = 0; g < n_groups; ++g) {
        const bsa_group &x = groups[g];
        if (x.col_begin < 0 || x.col_end > n_blocks || x.col_begin >= x.col_end || x.k < 0 ||
            x.k > x.col_end - x.col_begin)
            return fail(BSA_ERR_INVALID_ARG, "group %d = [%d, %d) k=%d invalid for %d blocks", g,
                        x.col_begin, x.col_end, x.k, n_blocks);
    }
    const int64_t rows = B * H * n_blocks;
    if (rows >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many rows");
    const int64_t need = bsa_select_capacity(B, H, n_blocks, text_blocks, groups, n_groups);
    if (need >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "nnz bound exceeds int32");
    if (capacity < need)
        return fail(BSA_ERR_CAPACITY, "capacity %lld below bound %lld", (long long)capacity,
                    (long long)need);
    const size_t ws = bsa_select_workspace_size(B, H, n_blocks);
    if (!workspace || workspace_bytes < ws)
        return fail(BSA_ERR_WORKSPACE, "workspace needs %zu bytes", ws);

    hipStream_t s = static_cast<hipStream_t>(stream);
    bsa::SelectParams sp{};
    sp.S = scores;
    sp.row_ptr = row_ptr;
    sp.bits = static_cast<uint32_t *>(workspace);
    sp.rows = rows;
    sp.nB = n_blocks;
    sp.words = (int32_t)ceil_div(n_blocks, 32);
    sp.text_blocks = text_blocks;
    sp.n_groups = n_groups;
    groups_by_column(groups, n_groups, sp.g_begin, sp.g_end, sp.g_k);
    // disjoint groups that leave the text columns alone fix every row's length
    bool direct = true;
    for (int32_t g = 0; g < n_groups && direct; ++g) {
        const bsa_group &a = groups[g];
        if (a.k == 0) continue;
        if (a.col_begin < text_blocks) direct = false;
        for (int32_t h = g + 1; h < n_groups && direct; ++h) {
            const bsa_group &b = groups[h];
            if (b.k > 0 && a.col_begin < b.col_end && b.col_begin < a.col_end) direct = false;
        }
    }
    sp.direct = direct ? 1 : 0;
    sp.row_len = (int32_t)select_row_bound(n_blocks, text_blocks, groups, n_groups);
    sp.col_idx = col_idx;
    sp.capacity = capacity;
    hipError_t e;
    if ((e = bsa::launch_select(sp, s)) != hipSuccess) return hip_fail(e, "select launch");
    if (direct) return BSA_OK;
    if ((e = bsa::launch_scan(row_ptr, rows, s)) != hipSuccess) return hip_fail(e, "scan launch");
    bsa::ExpandParams xp{};
    xp.bits = sp.bits;
    xp.row_ptr = row_ptr;
    xp.col_idx = col_idx;
    xp.rows = rows;
    xp.capacity = capacity;
    xp.words = sp.words;
    if ((e = bsa::launch_expand(xp, s)) != hipSuccess) return hip_fail(e, "expand launch");
    return BSA_OK;
}

// ---------------------------------------------------------------------------
static bsa_status arrow_check(int64_t B, int64_t H, int64_t N, int32_t block, int64_t text_len,
                              const int8_t *modes, const int32_t *windows)
{
    if (B <= 0 || H <= 0 || N <= 0) return fail(BSA_ERR_INVALID_ARG, "B, H, N must be positive");
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (text_len < 0 || text_len > N) return fail(BSA_ERR_INVALID_ARG, "text_len outside [0, N]");
    if (!modes || !windows) return fail(BSA_ERR_INVALID_ARG, "head_modes / head_windows null");
    if (H > bsa::kMaxArrowHeads) return fail(BSA_ERR_UNSUPPORTED, "H above %d", bsa::kMaxArrowHeads);
    if (ceil_div(N, block) > 65536) return fail(BSA_ERR_UNSUPPORTED, "more than 65536 blocks");
    for (int64_t h = 0; h < H; ++h) {
        if (modes[h] != BSA_HEAD_FULL && modes[h] != BSA_HEAD_ARROW && modes[h] != BSA_HEAD_SKIP)
            return fail(BSA_ERR_INVALID_ARG, "head %lld: unknown mode %d", (long long)h, modes[h]);
        if (modes[h] == BSA_HEAD_ARROW && windows[h] < 0)
            return fail(BSA_ERR_INVALID_ARG, "head %lld: negative window", (long long)h);
    }
    return BSA_OK;
}

int64_t bsa_arrow_capacity(int64_t B, int64_t H, int64_t N, int32_t block, int64_t text_len,
                           const int8_t *head_modes, const int32_t *head_windows)
{
    if (arrow_check(B, H, N, block, text_len, head_modes, head_windows) != BSA_OK) return -1;
    const int64_t nB = ceil_div(N, block), tb = ceil_div(text_len, block);
    int64_t per_batch = 0;
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t i = 0; i < nB; ++i) {
            const int m = head_modes[h];
            if (m == BSA_HEAD_SKIP) continue;
            if (m == BSA_HEAD_FULL || i < tb) { per_batch += nB; continue; }
            const int64_t w = head_windows[h];
            const int64_t lo = std::max(tb, i - w), hi = std::min(nB - 1, i + w);
            per_batch += tb + (hi >= lo ? hi - lo + 1 : 0);
        }
    }
    return B * per_batch;
}

bsa_status bsa_build_arrow_layout(int64_t B, int64_t H, int64_t N, int32_t block, int64_t text_len,
                                  const int8_t *head_modes, const int32_t *head_windows,
                                  int32_t *row_ptr, int32_t *col_idx, int64_t capacity, void *stream)
{
    bsa_status st = arrow_check(B, H, N, block, text_len, head_modes, head_windows);
    if (st != BSA_OK) return st;
    if (!row_ptr || !col_idx) return fail(BSA_ERR_INVALID_ARG, "row_ptr / col_idx null");
    const int64_t need = bsa_arrow_capacity(B, H, N, block, text_len, head_modes, head_windows);
    if (need >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "nnz %lld exceeds int32", (long long)need);
    if (capacity < need)
        return fail(BSA_ERR_CAPACITY, "capacity %lld below %lld", (long long)capacity, (long long)need);
    bsa::ArrowParams ap{};
    ap.row_ptr = row_ptr;
    ap.col_idx = col_idx;
    ap.capacity = capacity;
    ap.per_batch = need / B;
    ap.B = (int32_t)B;
    ap.H = (int32_t)H;
    ap.nB = (int32_t)ceil_div(N, block);
    ap.text_blocks = (int32_t)ceil_div(text_len, block);
    for (int64_t h = 0; h < H; ++h) {
        ap.mode[h] = head_modes[h];
        ap.window[h] = head_modes[h] == BSA_HEAD_ARROW ? head_windows[h] : 0;
    }
    hipError_t e = bsa::launch_arrow(ap, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "arrow launch");
    return BSA_OK;
}

// ---------------------------------------------------------------------------
size_t bsa_forward_split_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int32_t block,
                                        int32_t max_chunks, int64_t max_split_rows)
{
    if (B <= 0 || H <= 0 || N <= 0 || (D != 64 && D != 128) || !block_ok(block) || max_chunks < 2 ||
        max_chunks > 64 || max_split_rows < 1)
        return 0;
    const int64_t rows = B * H * ceil_div(N, block);
    return split_layout(rows, block, D, max_chunks, std::min(max_split_rows, rows)).total;
}

// Head modes of a forward call: the SKIP bitmask (o_cache then required,
// with the output's shape).
static bsa_status parse_head_modes(const int8_t *head_modes, int64_t H, const bsa_tensor *o_cache,
                                   const bsa_tensor *o, uint32_t *skip_bits, bool *any_skip)
{
    *any_skip = false;
    if (H > bsa::kMaxSkipHeads) return fail(BSA_ERR_UNSUPPORTED, "H above %d", bsa::kMaxSkipHeads);
    if (head_modes) {
        for (int64_t h = 0; h < H; ++h) {
            const int8_t m = head_modes[h];
            if (m != BSA_HEAD_FULL && m != BSA_HEAD_ARROW && m != BSA_HEAD_SKIP)
                return fail(BSA_ERR_INVALID_ARG, "head %lld: unknown mode %d", (long long)h, m);
            if (m == BSA_HEAD_SKIP) {
                skip_bits[h >> 5] |= 1u << (h & 31);
                *any_skip = true;
            }
        }
    }
    if (*any_skip) {
        bsa_status st;
        if ((st = check_tensor(o_cache, "o_cache")) != BSA_OK) return st;
        if (!same_shape(o, o_cache)) return fail(BSA_ERR_INVALID_ARG, "o_cache shape differs");
    }
    return BSA_OK;
}

// Long-row splitting of a forward call: validates the request, launches the
// plan kernel and returns the work list and partial-result slots for the
// forward kernel, and the launch size.
struct SplitRun {
    const int4 *items = nullptr;
    const int32_t *counts = nullptr;
    float *partials = nullptr;
    const int2 *split_rows = nullptr;
    int32_t max_chunks = 0;
    int64_t n_split_rows = 0;
    int64_t grid = 0;
};

static bsa_status split_begin(const bsa_split *split, int64_t BH, int64_t nB, int32_t block, int64_t D,
                              SplitRun *run)
{
    const int64_t rows = BH * nB;
    run->grid = rows;
    if (!split) return BSA_OK;
    if (split->chunk_blocks < 1 || split->max_chunks < 2 || split->max_chunks > 64 || split->max_split_rows < 1)
        return fail(BSA_ERR_INVALID_ARG,
                    "split: chunk_blocks >= 1, max_chunks in 2..64 and max_split_rows >= 1 required");
    const int64_t split_rows = std::min<int64_t>(split->max_split_rows, rows);
    const SplitLayout sl = split_layout(rows, block, D, split->max_chunks, split_rows);
    if (!split->workspace || !aligned16(split->workspace) || split->workspace_bytes < sl.total)
        return fail(BSA_ERR_WORKSPACE, "split workspace needs %zu bytes (16-byte aligned)", sl.total);
    const int64_t grid = rows + split_rows * (split->max_chunks - 1);
    if (grid >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "split work list too long");
    char *ws = static_cast<char *>(split->workspace);
    run->items = reinterpret_cast<const int4 *>(ws + sl.items);
    run->counts = reinterpret_cast<const int32_t *>(ws);
    run->partials = reinterpret_cast<float *>(ws + sl.partials);
    run->split_rows = reinterpret_cast<const int2 *>(ws + sl.split_rows);
    run->max_chunks = split->max_chunks;
    run->n_split_rows = split_rows;
    run->grid = grid;
    return BSA_OK;
}

static bsa_status split_plan(const SplitRun &run, const int32_t *row_ptr, int64_t BH, int64_t H, int64_t nB,
                             const bsa_split *split, const uint32_t *skip_bits, hipStream_t s)
{
    bsa::PlanParams pp{};
    pp.row_ptr = row_ptr;
    pp.items = const_cast<int4 *>(run.items);
    pp.counts = const_cast<int32_t *>(run.counts);
    pp.split_rows = const_cast<int2 *>(run.split_rows);
    pp.BH = (int32_t)BH;
    pp.H = (int32_t)H;
    pp.nB = (int32_t)nB;
    std::memcpy(pp.skip_bits, skip_bits, sizeof pp.skip_bits);
    pp.chunk_blocks = split->chunk_blocks;
    pp.max_chunks = split->max_chunks;
    pp.max_split_rows = run.n_split_rows;
    hipError_t e = bsa::launch_plan(pp, s);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    return BSA_OK;
}

static bsa_status split_combine(const SplitRun &run, const bsa_tensor *o, float *lse, int64_t H, int64_t N, int64_t nB,
                                int64_t D, int32_t block, int natural, const bsa::NbGeom *nb, hipStream_t s)
{
    bsa::CombineParams cp{};
    cp.partials = run.partials;
    cp.counts = run.counts;
    cp.split_rows = run.split_rows;
    cp.o = static_cast<uint16_t *>(o->data);
    cp.o_sb = o->stride_b;
    cp.o_sh = o->stride_h;
    cp.o_sn = o->stride_n;
    cp.lse = lse;
    cp.H = (int32_t)H;
    cp.N = (int32_t)N;
    cp.nB = (int32_t)nB;
    cp.D = (int32_t)D;
    cp.block = block;
    cp.max_chunks = run.max_chunks;
    cp.natural = natural;
    if (nb) cp.nb = *nb;
    hipError_t e = bsa::launch_combine(cp, run.n_split_rows, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return BSA_OK;
}

// SKIP heads: O (and LSE when a cache is given) copied from the caches.
static bsa_status skip_heads_copy(const bsa_tensor *o_cache, const float *lse_cache, const bsa_tensor *o, float *lse,
                                  const uint32_t *skip_bits, hipStream_t s)
{
    bsa::SkipCopyParams cp{};
    cp.src = t4(o_cache);
    cp.dst = static_cast<uint16_t *>(o->data);
    cp.d_sb = o->stride_b;
    cp.d_sh = o->stride_h;
    cp.d_sn = o->stride_n;
    cp.lse_src = lse_cache;
    cp.lse_dst = lse;
    cp.B = (int32_t)o->B;
    cp.H = (int32_t)o->H;
    cp.N = (int32_t)o->N;
    cp.D = (int32_t)o->D;
    cp.copy_o = !(o_cache->data == o->data && o_cache->stride_b == o->stride_b &&
                  o_cache->stride_h == o->stride_h && o_cache->stride_n == o->stride_n);
    std::memcpy(cp.skip_bits, skip_bits, sizeof cp.skip_bits);
    if (cp.copy_o || (lse_cache && lse && lse_cache != lse)) {
        hipError_t e = bsa::launch_skip_copy(cp, s);
        if (e != hipSuccess) return hip_fail(e, "skip copy launch");
    }
    return BSA_OK;
}

// ---------------------------------------------------------------------------
// Long-row split policy (host computation from the layout's closed-form row
// lengths; no device data).  The model takes the rows query-block-major (the
// order of a split launch's work list; a whole-row launch also starts with
// the leading query blocks of every head); a row of L blocks costs L +
// kItemOverhead block steps of
// one workgroup, and `slots` workgroups run at once (two per CU at block
// 128, about four at block 64).  Rows longer than L0 = max(typical,
// ceil(nB / 4)) would be cut into at most ceil(nB / L0) chunks; the split is
// recommended only when the greedy list-schedule makespan with the cut rows,
// plus the plan and combine cost, beats the makespan of whole rows by 5 %.
// The costs were calibrated by forcing splits on the FLUX 1024^2 mix, the
// 2K MMDiT arrow layout and the content-driven DiT.
// ---------------------------------------------------------------------------
static bsa_status check_nb(const bsa_neighborhood *g, int64_t N, int32_t block, bsa::NbGeom *out);

namespace {
constexpr double kItemOverhead = 0.5;
constexpr double kSplitGain = 0.95;
constexpr int kTargetChunks = 4;

int policy_slots(int32_t block) { return block == 128 ? 512 : 1024; }
double policy_overhead(int32_t block) { return block == 128 ? 4.0 : 20.0; }

// Greedy list schedule of costs (in order) on `slots` workgroups: the
// finishing time of the last one.
double makespan(const std::vector<double> &costs, int slots)
{
    if (costs.empty()) return 0.0;
    if ((int64_t)costs.size() <= slots) return *std::max_element(costs.begin(), costs.end());
    std::priority_queue<double, std::vector<double>, std::greater<double>> heap;
    for (int x = 0; x < slots; ++x) heap.push(0.0);
    double end = 0.0;
    for (double c : costs) {
        const double t = heap.top() + c;
        heap.pop();
        heap.push(t);
        end = std::max(end, t);
    }
    return end;
}

// 1 and *out filled when splitting pays, else 0.
int32_t split_from_rows(int64_t nB, const std::vector<int64_t> &lens, int64_t typical, int32_t block,
                        bsa_split *out)
{
    const int64_t L = std::max<int64_t>({1, typical, ceil_div(nB, kTargetChunks)});
    const int64_t S = std::min<int64_t>(64, std::max<int64_t>(2, ceil_div(nB, L)));
    int64_t long_rows = 0;
    std::vector<double> whole, cut;
    whole.reserve(lens.size());
    for (int64_t x : lens) {
        whole.push_back((double)x + kItemOverhead);
        if (x > L) {
            ++long_rows;
            const int64_t c = std::min<int64_t>(S, ceil_div(x, L));
            for (int64_t y = 0; y < c; ++y) cut.push_back((double)x / (double)c + kItemOverhead);
        } else {
            cut.push_back((double)x + kItemOverhead);
        }
    }
    if (long_rows == 0) return 0;
    const int slots = policy_slots(block);
    if (makespan(cut, slots) + policy_overhead(block) >= kSplitGain * makespan(whole, slots)) return 0;
    std::memset(out, 0, sizeof *out);
    out->chunk_blocks = (int32_t)L;
    out->max_chunks = (int32_t)S;
    out->max_split_rows = long_rows;
    return 1;
}
}  // namespace

int32_t bsa_split_policy_arrow(int64_t B, int64_t H, int64_t N, int32_t block, int64_t text_len,
                               const int8_t *head_modes, const int32_t *head_windows, bsa_split *out)
{
    if (B <= 0 || H <= 0 || N <= 0 || !block_ok(block) || text_len < 0 || text_len > N || !head_modes ||
        !head_windows || !out)
        return -1;
    const int64_t nB = ceil_div(N, block), tb = ceil_div(text_len, block);
    if (B * H * nB > (1ll << 26)) return -1;
    std::vector<int64_t> per(H * nB);
    int64_t typical = 1;
    bool all_full = true;
    for (int64_t h = 0; h < H; ++h) {
        const int8_t m = head_modes[h];
        if (m != BSA_HEAD_FULL && m != BSA_HEAD_ARROW && m != BSA_HEAD_SKIP) return -1;
        if (m == BSA_HEAD_ARROW && head_windows[h] < 0) return -1;
        all_full = all_full && m == BSA_HEAD_FULL;
        for (int64_t i = 0; i < nB; ++i) {
            int64_t len;
            if (m == BSA_HEAD_SKIP) len = 0;
            else if (m == BSA_HEAD_FULL || i < tb) len = nB;
            else {
                const int64_t w = head_windows[h];
                const int64_t lo = std::max(tb, i - w), hi = std::min(nB - 1, i + w);
                len = tb + std::max<int64_t>(0, hi - lo + 1);
                typical = std::max(typical, len);
            }
            per[h * nB + i] = len;
        }
    }
    if (all_full) typical = ceil_div(nB, kTargetChunks);
    std::vector<int64_t> lens;
    lens.reserve(B * H * nB);
    for (int64_t i = 0; i < nB; ++i)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < H; ++h) lens.push_back(per[h * nB + i]);
    return split_from_rows(nB, lens, typical, block, out);
}

int32_t bsa_split_policy_select(int64_t B, int64_t H, int32_t n_blocks, int32_t text_blocks,
                                const bsa_group *groups, int32_t n_groups, int32_t block, bsa_split *out)
{
    if (B <= 0 || H <= 0 || n_blocks <= 0 || text_blocks < 0 || text_blocks > n_blocks || n_groups < 0 ||
        (n_groups > 0 && !groups) || !block_ok(block) || !out || B * H * n_blocks > (1ll << 26))
        return -1;
    const int64_t nB = n_blocks;
    const int64_t typical = select_row_bound(nB, text_blocks, groups, n_groups);
    std::vector<int64_t> lens;
    lens.reserve(B * H * nB);
    for (int64_t i = 0; i < nB; ++i)
        for (int64_t x = 0; x < B * H; ++x) lens.push_back(i < text_blocks ? nB : typical);
    return split_from_rows(nB, lens, typical, block, out);
}

int32_t bsa_split_policy_neighborhood(int64_t B, int64_t H, int32_t block, const bsa_neighborhood *nb,
                                      bsa_split *out)
{
    if (B <= 0 || H <= 0 || !nb || !out) return -1;
    bsa::NbGeom g;
    const int64_t N = (int64_t)nb->text_len + (int64_t)nb->rows * nb->cols;
    if (check_nb(nb, N, block, &g) != BSA_OK) return -1;
    const int64_t nB = ceil_div(N, block);
    if (B * H * nB > (1ll << 26)) return -1;
    std::vector<int64_t> per(nB);
    int64_t typical = 1;
    for (int64_t i = 0; i < nB; ++i) {
        per[i] = bsa::nb_row_len(g, (int32_t)nB, (int32_t)i);
        if (per[i] < nB) typical = std::max(typical, per[i]);
    }
    std::vector<int64_t> lens;
    lens.reserve(B * H * nB);
    for (int64_t i = 0; i < nB; ++i)
        for (int64_t x = 0; x < B * H; ++x) lens.push_back(per[i]);
    return split_from_rows(nB, lens, typical, block, out);
}

static bsa_status forward_impl(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, int32_t block,
                               const int32_t *row_ptr, const int32_t *col_idx, const int8_t *head_modes,
                               const bsa_tensor *o_cache, const float *lse_cache, float scale,
                               const bsa_tensor *o, float *lse, const bsa_split *split, void *stream,
                               const int32_t *entry_flags, const bsa::NbGeom *nb, int natural = 0)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if ((st = check_tensor(k, "k")) != BSA_OK) return st;
    if ((st = check_tensor(v, "v")) != BSA_OK) return st;
    if ((st = check_tensor(o, "o")) != BSA_OK) return st;
    if (!same_shape(q, k) || !same_shape(q, v) || !same_shape(q, o))
        return fail(BSA_ERR_INVALID_ARG, "q, k, v and o shapes differ");
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (!row_ptr || !col_idx) return fail(BSA_ERR_INVALID_ARG, "row_ptr / col_idx null");
    if (std::isnan(scale)) return fail(BSA_ERR_INVALID_ARG, "scale is NaN");
    const int64_t H = q->H;
    const int64_t nB = ceil_div(q->N, block);
    if (q->B * H * nB >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many query blocks");

    bsa::FwdParams fp{};
    bool any_skip = false;
    if ((st = parse_head_modes(head_modes, H, o_cache, o, fp.skip_bits, &any_skip)) != BSA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    SplitRun run;
    if ((st = split_begin(split, q->B * H, nB, block, q->D, &run)) != BSA_OK) return st;

    fp.q = t4(q);
    fp.k = t4(k);
    fp.v = t4(v);
    fp.flags = entry_flags;
    if (nb) fp.nb = *nb;
    fp.natural = natural;
    fp.o = static_cast<uint16_t *>(o->data);
    fp.o_sb = o->stride_b;
    fp.o_sh = o->stride_h;
    fp.o_sn = o->stride_n;
    fp.lse = lse;
    fp.row_ptr = row_ptr;
    fp.col_idx = col_idx;
    fp.B = (int32_t)q->B;
    fp.H = (int32_t)H;
    fp.N = (int32_t)q->N;
    fp.nB = (int32_t)nB;
    const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)q->D);
    fp.scale_log2 = sc * 1.4426950408889634f;
    fp.items = run.items;
    fp.counts = run.counts;
    fp.partials = run.partials;
    fp.max_chunks = run.max_chunks;

    if (any_skip) {   // the forward's SKIP-row workgroups copy the caches
        fp.oc = t4(o_cache);
        fp.lse_src = (lse_cache && lse && lse_cache != lse) ? lse_cache : nullptr;
        fp.copy_o = !(o_cache->data == o->data && o_cache->stride_b == o->stride_b &&
                      o_cache->stride_h == o->stride_h && o_cache->stride_n == o->stride_n);
    }
    if (split && (st = split_plan(run, row_ptr, q->B * H, H, nB, split, fp.skip_bits, s)) != BSA_OK) return st;
    hipError_t e;
    if ((e = bsa::launch_forward(fp, block, (int)q->D, run.grid, s)) != hipSuccess)
        return hip_fail(e, "forward launch");
    if (split && (st = split_combine(run, o, lse, H, q->N, nB, q->D, block, natural, nb, s)) != BSA_OK) return st;
    return BSA_OK;
}

bsa_status bsa_forward(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, int32_t block,
                       const int32_t *row_ptr, const int32_t *col_idx, const int8_t *head_modes,
                       const bsa_tensor *o_cache, const float *lse_cache, float scale,
                       const bsa_tensor *o, float *lse, const bsa_split *split, void *stream)
{
    return forward_impl(q, k, v, block, row_ptr, col_idx, head_modes, o_cache, lse_cache, scale, o, lse, split,
                        stream, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// 2-D neighbourhood attention
// ---------------------------------------------------------------------------
static bsa_status check_nb(const bsa_neighborhood *g, int64_t N, int32_t block, bsa::NbGeom *out)
{
    if (!g) return fail(BSA_ERR_INVALID_ARG, "neighborhood: null descriptor");
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (g->rows <= 0 || g->cols <= 0 || g->tile_rows <= 0 || g->tile_cols <= 0 || g->text_len < 0)
        return fail(BSA_ERR_INVALID_ARG, "neighborhood: grid and tile must be positive");
    if ((int64_t)g->tile_rows * g->tile_cols != block || (g->tile_cols & (g->tile_cols - 1)))
        return fail(BSA_ERR_INVALID_ARG, "neighborhood: tile_rows * tile_cols must equal the block, tile_cols a power of two");
    if (g->rows % g->tile_rows || g->cols % g->tile_cols || g->text_len % block)
        return fail(BSA_ERR_INVALID_ARG, "neighborhood: grid not a whole number of tiles, or text_len not a whole number of blocks");
    if (g->text_len + (int64_t)g->rows * g->cols != N)
        return fail(BSA_ERR_INVALID_ARG, "neighborhood: text_len + rows * cols must equal N");
    if (g->window_rows < 1 || g->window_rows > g->rows || g->window_cols < 1 || g->window_cols > g->cols ||
        g->stride_rows < 1 || g->stride_cols < 1)
        return fail(BSA_ERR_INVALID_ARG, "neighborhood: window must lie in 1..grid and strides be >= 1");
    if (N / block > 65536) return fail(BSA_ERR_UNSUPPORTED, "neighborhood: more than 65536 blocks");
    bsa::NbGeom x{};
    x.T = (int32_t)g->text_len;
    x.Tb = (int32_t)(g->text_len / block);
    x.R = g->rows;
    x.C = g->cols;
    x.th = g->tile_rows;
    x.tw = g->tile_cols;
    x.tw_log2 = 0;
    while ((1 << x.tw_log2) < x.tw) ++x.tw_log2;
    x.tpr = g->cols / g->tile_cols;
    x.kh = g->window_rows;
    x.kw = g->window_cols;
    x.sh = g->stride_rows;
    x.sw = g->stride_cols;
    x.rep = 1;
    for (int b = x.tw; x.tw < 64 && b < 64; b += x.tw) x.rep |= 1ull << b;
    *out = x;
    return BSA_OK;
}

static int64_t nb_head_nnz(const bsa::NbGeom &g, int32_t nB)
{
    int64_t n = 0;
    for (int32_t i = 0; i < nB; ++i) n += bsa::nb_row_len(g, nB, i);
    return n;
}

int64_t bsa_neighborhood_capacity(int64_t B, int64_t H, int32_t block, const bsa_neighborhood *nb)
{
    if (B <= 0 || H <= 0 || !nb) return -1;
    bsa::NbGeom g;
    const int64_t N = nb->text_len + (int64_t)nb->rows * nb->cols;
    if (check_nb(nb, N, block, &g) != BSA_OK) return -1;
    return B * H * nb_head_nnz(g, (int32_t)(N / block));
}

bsa_status bsa_build_neighborhood_layout(int64_t B, int64_t H, int32_t block, const bsa_neighborhood *nb,
                                         int32_t *row_ptr, int32_t *col_idx, int32_t *entry_flags,
                                         int64_t capacity, void *stream)
{
    if (B <= 0 || H <= 0) return fail(BSA_ERR_INVALID_ARG, "B and H must be positive");
    if (!nb) return fail(BSA_ERR_INVALID_ARG, "neighborhood: null descriptor");
    bsa::NbGeom g;
    bsa_status st;
    const int64_t N = nb->text_len + (int64_t)nb->rows * nb->cols;
    if ((st = check_nb(nb, N, block, &g)) != BSA_OK) return st;
    if (!row_ptr || !col_idx || !entry_flags) return fail(BSA_ERR_INVALID_ARG, "row_ptr / col_idx / entry_flags null");
    const int32_t nB = (int32_t)(N / block);
    const int64_t per_head = nb_head_nnz(g, nB);
    if (B * H * nB >= (1ll << 31) || B * H * per_head >= (1ll << 31))
        return fail(BSA_ERR_UNSUPPORTED, "layout too large for int32 indices");
    if (capacity < B * H * per_head)
        return fail(BSA_ERR_CAPACITY, "capacity %lld below %lld", (long long)capacity, (long long)(B * H * per_head));
    bsa::NbLayoutParams p{};
    p.nb = g;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.flags = entry_flags;
    p.capacity = capacity;
    p.per_head = per_head;
    p.B = (int32_t)B;
    p.H = (int32_t)H;
    p.nB = nB;
    hipError_t e = bsa::launch_neighborhood_layout(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "neighborhood layout launch");
    return BSA_OK;
}

bsa_status bsa_permute_tokens(const bsa_tensor *in, const bsa_tensor *out, const float *lse_in, float *lse_out,
                              int32_t block, const bsa_neighborhood *nb, int32_t inverse, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(in, "in")) != BSA_OK) return st;
    if ((st = check_tensor(out, "out")) != BSA_OK) return st;
    if (!same_shape(in, out)) return fail(BSA_ERR_INVALID_ARG, "in and out shapes differ");
    if (in->data == out->data) return fail(BSA_ERR_INVALID_ARG, "permutation cannot run in place");
    if ((lse_in == nullptr) != (lse_out == nullptr) || (lse_in && lse_in == lse_out))
        return fail(BSA_ERR_INVALID_ARG, "lse_in and lse_out: both or neither, distinct");
    bsa::NbGeom g;
    if ((st = check_nb(nb, in->N, block, &g)) != BSA_OK) return st;
    bsa::PermuteParams p{};
    p.in = t4(in);
    p.out = static_cast<uint16_t *>(out->data);
    p.o_sb = out->stride_b;
    p.o_sh = out->stride_h;
    p.o_sn = out->stride_n;
    p.lse_in = lse_in;
    p.lse_out = lse_out;
    p.nb = g;
    p.B = (int32_t)in->B;
    p.H = (int32_t)in->H;
    p.N = (int32_t)in->N;
    p.D = (int32_t)in->D;
    p.inverse = inverse ? 1 : 0;
    if (in->B * in->H > 65535) return fail(BSA_ERR_UNSUPPORTED, "B*H above 65535");
    hipError_t e = bsa::launch_permute_tokens(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "permute launch");
    return BSA_OK;
}

bsa_status bsa_forward_neighborhood(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, int32_t block,
                                    const int32_t *row_ptr, const int32_t *col_idx, const int32_t *entry_flags,
                                    const bsa_neighborhood *nb, float scale, const bsa_tensor *o, float *lse,
                                    const bsa_split *split, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if (!entry_flags) return fail(BSA_ERR_INVALID_ARG, "entry_flags null");
    bsa::NbGeom g;
    if ((st = check_nb(nb, q->N, block, &g)) != BSA_OK) return st;
    return forward_impl(q, k, v, block, row_ptr, col_idx, nullptr, nullptr, nullptr, scale, o, lse, split, stream,
                        entry_flags, &g);
}

bsa_status bsa_forward_neighborhood_natural(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                            int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                                            const int32_t *entry_flags, const bsa_neighborhood *nb, float scale,
                                            const bsa_tensor *o, float *lse, const bsa_split *split,
                                            void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if (!entry_flags) return fail(BSA_ERR_INVALID_ARG, "entry_flags null");
    bsa::NbGeom g;
    if ((st = check_nb(nb, q->N, block, &g)) != BSA_OK) return st;
    return forward_impl(q, k, v, block, row_ptr, col_idx, nullptr, nullptr, nullptr, scale, o, lse, split, stream,
                        entry_flags, &g, 1);
}

// ---------------------------------------------------------------------------
size_t bsa_backward_workspace_size(int64_t B, int64_t H, int64_t N)
{
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    return 2 * (((size_t)(B * H * N) * sizeof(float) + 255) & ~(size_t)255);
}

static bsa_status backward_impl(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, const bsa_tensor *o,
                                const bsa_tensor *dO, int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                                const float *lse, float scale, const bsa_tensor *dq, const bsa_tensor *dk,
                                const bsa_tensor *dv, void *workspace, size_t workspace_bytes, void *stream,
                                const int32_t *entry_flags, const bsa::NbGeom *nb, int natural = 0)
{
    bsa_status st;
    const bsa_tensor *ts[] = {q, k, v, o, dO, dq, dk, dv};
    const char *names[] = {"q", "k", "v", "o", "dO", "dq", "dk", "dv"};
    for (int x = 0; x < 8; ++x) {
        if ((st = check_tensor(ts[x], names[x])) != BSA_OK) return st;
        if (!same_shape(q, ts[x])) return fail(BSA_ERR_INVALID_ARG, "%s shape differs from q", names[x]);
    }
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (!row_ptr || !col_idx || !lse) return fail(BSA_ERR_INVALID_ARG, "row_ptr / col_idx / lse null");
    if (std::isnan(scale)) return fail(BSA_ERR_INVALID_ARG, "scale is NaN");
    const int64_t nB = ceil_div(q->N, block);
    if (nB > bsa::kBwdMaxBlocks) return fail(BSA_ERR_UNSUPPORTED, "more than %d blocks", bsa::kBwdMaxBlocks);
    if (q->B * q->H * nB >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many blocks");
    const size_t need = bsa_backward_workspace_size(q->B, q->H, q->N);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need)
        return fail(BSA_ERR_WORKSPACE, "backward workspace needs %zu bytes (16-byte aligned)", need);
    bsa::BwdParams p{};
    p.q = t4(q);
    p.k = t4(k);
    p.v = t4(v);
    p.o = t4(o);
    p.dO = t4(dO);
    p.lse = lse;
    p.lse2 = static_cast<float *>(workspace);
    p.delta = reinterpret_cast<float *>(static_cast<char *>(workspace) + need / 2);
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.dq = static_cast<uint16_t *>(dq->data);
    p.dk = static_cast<uint16_t *>(dk->data);
    p.dv = static_cast<uint16_t *>(dv->data);
    p.dq_sb = dq->stride_b; p.dq_sh = dq->stride_h; p.dq_sn = dq->stride_n;
    p.dk_sb = dk->stride_b; p.dk_sh = dk->stride_h; p.dk_sn = dk->stride_n;
    p.dv_sb = dv->stride_b; p.dv_sh = dv->stride_h; p.dv_sn = dv->stride_n;
    p.B = (int32_t)q->B;
    p.H = (int32_t)q->H;
    p.N = (int32_t)q->N;
    p.D = (int32_t)q->D;
    p.nB = (int32_t)nB;
    p.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)q->D);
    p.scale_log2 = p.scale * 1.4426950408889634f;
    p.flags = entry_flags;
    if (nb) p.nb = *nb;
    p.natural = (nb && natural) ? block : 0;
    hipError_t e = bsa::launch_backward(p, block, (int)q->D, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return BSA_OK;
}

bsa_status bsa_backward(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, const bsa_tensor *o,
                        const bsa_tensor *dO, int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                        const float *lse, float scale, const bsa_tensor *dq, const bsa_tensor *dk,
                        const bsa_tensor *dv, void *workspace, size_t workspace_bytes, void *stream)
{
    return backward_impl(q, k, v, o, dO, block, row_ptr, col_idx, lse, scale, dq, dk, dv, workspace,
                         workspace_bytes, stream, nullptr, nullptr);
}

bsa_status bsa_backward_neighborhood(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                     const bsa_tensor *o, const bsa_tensor *dO, int32_t block,
                                     const int32_t *row_ptr, const int32_t *col_idx, const int32_t *entry_flags,
                                     const bsa_neighborhood *nb, const float *lse, float scale,
                                     const bsa_tensor *dq, const bsa_tensor *dk, const bsa_tensor *dv,
                                     void *workspace, size_t workspace_bytes, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if (!entry_flags) return fail(BSA_ERR_INVALID_ARG, "entry_flags null");
    bsa::NbGeom g;
    if ((st = check_nb(nb, q->N, block, &g)) != BSA_OK) return st;
    return backward_impl(q, k, v, o, dO, block, row_ptr, col_idx, lse, scale, dq, dk, dv, workspace,
                         workspace_bytes, stream, entry_flags, &g);
}

bsa_status bsa_backward_neighborhood_natural(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                             const bsa_tensor *o, const bsa_tensor *dO, int32_t block,
                                             const int32_t *row_ptr, const int32_t *col_idx,
                                             const int32_t *entry_flags, const bsa_neighborhood *nb,
                                             const float *lse, float scale, const bsa_tensor *dq,
                                             const bsa_tensor *dk, const bsa_tensor *dv, void *workspace,
                                             size_t workspace_bytes, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if (!entry_flags) return fail(BSA_ERR_INVALID_ARG, "entry_flags null");
    bsa::NbGeom g;
    if ((st = check_nb(nb, q->N, block, &g)) != BSA_OK) return st;
    return backward_impl(q, k, v, o, dO, block, row_ptr, col_idx, lse, scale, dq, dk, dv, workspace,
                         workspace_bytes, stream, entry_flags, &g, 1);
}

// ---------------------------------------------------------------------------
size_t bsa_quantize_fp8_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D)
{
    if (B <= 0 || H <= 0 || N <= 0 || (D != 64 && D != 128)) return 0;
    const int64_t BH = B * H;
    return fp8_ws_inv_bytes(BH, D) + (size_t)(BH * ceil_div(N, 256) * D) * sizeof(float);
}

static bsa_status quantize_fp8_impl(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                    const bsa_fp8_qkv *out, void *workspace, size_t workspace_bytes, void *stream,
                                    const bsa::NbGeom *nb, int32_t nb_block)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    if ((st = check_tensor(k, "k")) != BSA_OK) return st;
    if ((st = check_tensor(v, "v")) != BSA_OK) return st;
    if (!same_shape(q, k) || !same_shape(q, v)) return fail(BSA_ERR_INVALID_ARG, "q, k and v shapes differ");
    if ((st = check_fp8(out, "out")) != BSA_OK) return st;
    if (out->B != q->B || out->H != q->H || out->N != q->N || out->D != q->D)
        return fail(BSA_ERR_INVALID_ARG, "out shape differs from q");
    const size_t need = bsa_quantize_fp8_workspace_size(q->B, q->H, q->N, q->D);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need)
        return fail(BSA_ERR_WORKSPACE, "quantisation workspace needs %zu bytes (16-byte aligned)", need);
    const int64_t BH = q->B * q->H;
    if (BH * ceil_div(q->N, 64) >= (1ll << 31) || ceil_div(q->N, 256) > 65535)
        return fail(BSA_ERR_UNSUPPORTED, "too many tiles");

    bsa::Fp8QuantParams p{};
    p.q = t4(q);
    p.k = t4(k);
    p.v = t4(v);
    p.q8 = static_cast<uint8_t *>(out->q8);
    p.k8 = static_cast<uint8_t *>(out->k8);
    p.v8t = static_cast<uint8_t *>(out->v8t);
    p.q_scale = out->q_scale;
    p.k_scale = out->k_scale;
    p.v_scale = out->v_scale;
    p.v_inv = static_cast<float *>(workspace);
    p.vmax_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + fp8_ws_inv_bytes(BH, q->D));
    p.BHN = BH * q->N;
    p.B = (int32_t)q->B;
    p.H = (int32_t)q->H;
    p.N = (int32_t)q->N;
    p.NT = (int32_t)ceil_div(q->N, 64);
    p.NP = 64 * p.NT;
    p.S = (int32_t)ceil_div(q->N, 256);
    if (nb) {
        p.nb = *nb;
        p.nb_block = nb_block;
    }
    hipError_t e = bsa::launch_quantize_fp8(p, (int)q->D, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "fp8 quantisation launch");
    return BSA_OK;
}

bsa_status bsa_quantize_fp8(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v, const bsa_fp8_qkv *out,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    return quantize_fp8_impl(q, k, v, out, workspace, workspace_bytes, stream, nullptr, 0);
}

bsa_status bsa_quantize_fp8_neighborhood(const bsa_tensor *q, const bsa_tensor *k, const bsa_tensor *v,
                                         int32_t block, const bsa_neighborhood *nb, const bsa_fp8_qkv *out,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(q, "q")) != BSA_OK) return st;
    bsa::NbGeom g;
    if ((st = check_nb(nb, q->N, block, &g)) != BSA_OK) return st;
    return quantize_fp8_impl(q, k, v, out, workspace, workspace_bytes, stream, &g, block);
}

static bsa_status forward_fp8_impl(const bsa_fp8_qkv *in, int32_t block, const int32_t *row_ptr,
                                   const int32_t *col_idx, const int8_t *head_modes, const bsa_tensor *o_cache,
                                   const float *lse_cache, float scale, const bsa_tensor *o, float *lse,
                                   const bsa_split *split, void *stream, const int32_t *entry_flags,
                                   const bsa::NbGeom *nb, int natural = 0)
{
    bsa_status st;
    if ((st = check_fp8(in, "in")) != BSA_OK) return st;
    if ((st = check_tensor(o, "o")) != BSA_OK) return st;
    if (o->B != in->B || o->H != in->H || o->N != in->N || o->D != in->D)
        return fail(BSA_ERR_INVALID_ARG, "o shape differs from the fp8 inputs");
    if (!block_ok(block)) return fail(BSA_ERR_UNSUPPORTED, "block size %d not supported", block);
    if (!row_ptr || !col_idx) return fail(BSA_ERR_INVALID_ARG, "row_ptr / col_idx null");
    if (std::isnan(scale)) return fail(BSA_ERR_INVALID_ARG, "scale is NaN");
    const int64_t nB = ceil_div(in->N, block);
    if (in->B * in->H * nB >= (1ll << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many query blocks");

    bsa::Fp8FwdParams p{};
    bool any_skip = false;
    if ((st = parse_head_modes(head_modes, in->H, o_cache, o, p.skip_bits, &any_skip)) != BSA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    SplitRun run;
    if ((st = split_begin(split, in->B * in->H, nB, block, in->D, &run)) != BSA_OK) return st;
    p.q8 = static_cast<const uint8_t *>(in->q8);
    p.k8 = static_cast<const uint8_t *>(in->k8);
    p.v8t = static_cast<const uint8_t *>(in->v8t);
    p.q_scale = in->q_scale;
    p.k_scale = in->k_scale;
    p.v_scale = in->v_scale;
    p.o = static_cast<uint16_t *>(o->data);
    p.o_sb = o->stride_b;
    p.o_sh = o->stride_h;
    p.o_sn = o->stride_n;
    p.lse = lse;
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.B = (int32_t)in->B;
    p.H = (int32_t)in->H;
    p.N = (int32_t)in->N;
    p.nB = (int32_t)nB;
    p.NT = (int32_t)ceil_div(in->N, 64);
    p.NP = 64 * p.NT;
    const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)in->D);
    p.scale_log2 = sc * 1.4426950408889634f;
    p.flags = entry_flags;
    if (nb) p.nb = *nb;
    p.natural = nb ? natural : 0;
    p.items = run.items;
    p.counts = run.counts;
    p.partials = run.partials;
    p.max_chunks = run.max_chunks;
    if (split && (st = split_plan(run, row_ptr, in->B * in->H, in->H, nB, split, p.skip_bits, s)) != BSA_OK)
        return st;
    hipError_t e = bsa::launch_forward_fp8(p, block, (int)in->D, run.grid, s);
    if (e != hipSuccess) return hip_fail(e, "fp8 forward launch");
    if (split && (st = split_combine(run, o, lse, in->H, in->N, nB, in->D, block, p.natural, nb, s)) != BSA_OK)
        return st;
    if (any_skip && (st = skip_heads_copy(o_cache, lse_cache, o, lse, p.skip_bits, s)) != BSA_OK) return st;
    return BSA_OK;
}

bsa_status bsa_forward_fp8(const bsa_fp8_qkv *in, int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                           const int8_t *head_modes, const bsa_tensor *o_cache, const float *lse_cache, float scale,
                           const bsa_tensor *o, float *lse, const bsa_split *split, void *stream)
{
    return forward_fp8_impl(in, block, row_ptr, col_idx, head_modes, o_cache, lse_cache, scale, o, lse, split,
                            stream, nullptr, nullptr);
}

bsa_status bsa_forward_fp8_neighborhood(const bsa_fp8_qkv *in, int32_t block, const int32_t *row_ptr,
                                        const int32_t *col_idx, const int32_t *entry_flags,
                                        const bsa_neighborhood *nb, float scale, const bsa_tensor *o, float *lse,
                                        void *stream)
{
    bsa_status st;
    if ((st = check_fp8(in, "in")) != BSA_OK) return st;
    if (!entry_flags) return fail(BSA_ERR_INVALID_ARG, "entry_flags null");
    bsa::NbGeom g;
    if ((st = check_nb(nb, in->N, block, &g)) != BSA_OK) return st;
    return forward_fp8_impl(in, block, row_ptr, col_idx, nullptr, nullptr, nullptr, scale, o, lse, nullptr, stream,
                            entry_flags, &g);
}

bsa_status bsa_forward_fp8_neighborhood_natural(const bsa_fp8_qkv *in, int32_t block, const int32_t *row_ptr,
                                                const int32_t *col_idx, const int32_t *entry_flags,
                                                const bsa_neighborhood *nb, float scale, const bsa_tensor *o,
                                                float *lse, void *stream)
{
    bsa_status st;
    if ((st = check_fp8(in, "in")) != BSA_OK) return st;
    if (!entry_flags) return fail(BSA_ERR_INVALID_ARG, "entry_flags null");
    bsa::NbGeom g;
    if ((st = check_nb(nb, in->N, block, &g)) != BSA_OK) return st;
    return forward_fp8_impl(in, block, row_ptr, col_idx, nullptr, nullptr, nullptr, scale, o, lse, nullptr, stream,
                            entry_flags, &g, 1);
}

// ---------------------------------------------------------------------------
size_t bsa_output_rse_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D)
{
    if (B <= 0 || H <= 0 || N <= 0 || (D != 64 && D != 128)) return 0;
    return (size_t)(B * H) * rse_chunks(N, D) * 3 * sizeof(double);
}

bsa_status bsa_output_rse(const bsa_tensor *test, const bsa_tensor *ref, double *rse, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    bsa_status st;
    if ((st = check_tensor(test, "test")) != BSA_OK) return st;
    if ((st = check_tensor(ref, "ref")) != BSA_OK) return st;
    if (!same_shape(test, ref)) return fail(BSA_ERR_INVALID_ARG, "test and ref shapes differ");
    if (!rse) return fail(BSA_ERR_INVALID_ARG, "rse null");
    const size_t need = bsa_output_rse_workspace_size(ref->B, ref->H, ref->N, ref->D);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need)
        return fail(BSA_ERR_WORKSPACE, "rse workspace needs %zu bytes (16-byte aligned)", need);
    bsa::RseParams p{};
    p.test = t4(test);
    p.ref = t4(ref);
    p.partials = static_cast<double *>(workspace);
    p.rse = rse;
    p.B = (int32_t)ref->B;
    p.H = (int32_t)ref->H;
    p.N = (int32_t)ref->N;
    p.D = (int32_t)ref->D;
    p.chunks = rse_chunks(ref->N, ref->D);
    p.rows_per_chunk = (int32_t)ceil_div(ref->N, p.chunks);
    hipError_t e = bsa::launch_output_rse(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "rse launch");
    return BSA_OK;
}

bsa_status bsa_mask_jaccard(int64_t B, int64_t H, int32_t n_blocks, const int32_t *row_ptr_a,
                            const int32_t *col_idx_a, const int32_t *row_ptr_b, const int32_t *col_idx_b,
                            double *jaccard, void *stream)
{
    if (B <= 0 || H <= 0 || n_blocks <= 0) return fail(BSA_ERR_INVALID_ARG, "B, H, n_blocks must be positive");
    if (!row_ptr_a || !col_idx_a || !row_ptr_b || !col_idx_b || !jaccard)
        return fail(BSA_ERR_INVALID_ARG, "null array");
    if (n_blocks > 65536 || B * H > INT32_MAX) return fail(BSA_ERR_UNSUPPORTED, "n_blocks above 65536 or B*H too large");
    bsa::JaccardParams p{};
    p.row_ptr_a = row_ptr_a;
    p.col_idx_a = col_idx_a;
    p.row_ptr_b = row_ptr_b;
    p.col_idx_b = col_idx_b;
    p.jaccard = jaccard;
    p.B = (int32_t)B;
    p.H = (int32_t)H;
    p.nB = n_blocks;
    hipError_t e = bsa::launch_mask_jaccard(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "jaccard launch");
    return BSA_OK;
}

}  // extern "C"
