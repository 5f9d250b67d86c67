// api.hip -- the C ABI of include/csa_attn.h: host-side validation, workspace
// sizing, dispatch to the kernel launchers and error reporting.
//
// Every argument check runs before the first HIP call, so a non-OK status
// means nothing was enqueued (and every error path can be exercised without a
// GPU).  No device memory is allocated here.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/csa_attn.h"
#include "launch.hpp"

#define CSA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

csa_status fail(csa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

csa_status ok() {
    g_err.clear();
    return CSA_OK;
}

csa_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_kv_fmt(int f) { return f == CSA_F32 || f == CSA_BF16 || f == CSA_FP8_E4M3; }
bool is_idx_fmt(int f) { return f == CSA_F32 || f == CSA_BF16 || f == CSA_FP4_E2M1; }
bool is_act_fmt(int f) { return f == CSA_F32 || f == CSA_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t idx_row_bytes(int fmt, int di) { return fmt == CSA_F32 ? 4 * di : fmt == CSA_BF16 ? 2 * di : di / 2; }

constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kIdxWsBudget = (int64_t)1 << 30;   // rows of the large top-k path per launch batch

int64_t idx_rows_per_batch(int64_t rows, int64_t cap, int32_t topk) {
    const int64_t rb = csa::idx_ws_row_bytes(cap, topk);
    int64_t n = kIdxWsBudget / rb;
    if (n < 1) n = 1;
    if (n > kMaxGridY) n = kMaxGridY;
    return rows < n ? rows : n;
}

// window ring / compressed cache checks shared by both attention calls
csa_status check_attn_common(const void* q, int32_t q_dtype, const int32_t* q_pos, const csa_kv_cache* comp,
                             const csa_kv_cache* win, const float* sink, const csa_attn_params* p, int32_t B,
                             int32_t Tq, int32_t H, void* out, int32_t out_dtype) {
    if (!p) return fail(CSA_ERR_INVALID_ARG, "params is null");
    if (B < 0 || Tq < 0 || H < 1) return fail(CSA_ERR_INVALID_ARG, "bad sizes B=%d Tq=%d H=%d", B, Tq, H);
    if ((int64_t)B * Tq > kMaxGridY) return fail(CSA_ERR_UNSUPPORTED, "B*Tq=%lld exceeds %lld query rows", (long long)B * Tq, (long long)kMaxGridY);
    if (H > 256) return fail(CSA_ERR_UNSUPPORTED, "H=%d > 256", H);
    const int d = p->head_dim, dr = p->rope_dim;
    if (d < 2 || d > 1024 || d % 2) return fail(CSA_ERR_INVALID_ARG, "head_dim %d must be even and in [2, 1024]", d);
    if (dr < 0 || dr > d || dr % 2) return fail(CSA_ERR_INVALID_ARG, "rope_dim %d must be even and <= head_dim", dr);
    if (dr > 128) return fail(CSA_ERR_UNSUPPORTED, "rope_dim %d > 128", dr);
    if (p->window < 0 || p->m < 1) return fail(CSA_ERR_INVALID_ARG, "window %d / m %d", p->window, p->m);
    if (p->split_policy != CSA_SPLIT_BY_CHUNK && p->split_policy != CSA_SPLIT_FIXED)
        return fail(CSA_ERR_INVALID_ARG, "split_policy %d", p->split_policy);
    if (!is_act_fmt(q_dtype)) return fail(CSA_ERR_UNSUPPORTED, "q dtype %d", q_dtype);
    if (!is_act_fmt(out_dtype)) return fail(CSA_ERR_UNSUPPORTED, "out dtype %d", out_dtype);
    if (!comp) return fail(CSA_ERR_INVALID_ARG, "comp cache is null");
    if (!is_kv_fmt(comp->fmt)) return fail(CSA_ERR_UNSUPPORTED, "comp fmt %d", comp->fmt);
    if (comp->d != d || comp->d_rope != dr) return fail(CSA_ERR_INVALID_ARG, "comp cache d/d_rope %d/%d differ from params %d/%d", comp->d, comp->d_rope, d, dr);
    if (comp->ring) return fail(CSA_ERR_INVALID_ARG, "the compressed cache must be linear (ring = 0)");
    if (comp->cap < 1) return fail(CSA_ERR_INVALID_ARG, "comp cap %lld", (long long)comp->cap);
    if (p->window > 0) {
        if (!win) return fail(CSA_ERR_INVALID_ARG, "window %d needs a window cache", p->window);
        if (!is_kv_fmt(win->fmt)) return fail(CSA_ERR_UNSUPPORTED, "win fmt %d", win->fmt);
        if (win->d != d || win->d_rope != dr) return fail(CSA_ERR_INVALID_ARG, "win cache d/d_rope %d/%d differ from params", win->d, win->d_rope);
        if (!win->ring) return fail(CSA_ERR_INVALID_ARG, "the window cache must be a ring (ring = 1)");
        if (win->cap < (int64_t)p->window + (Tq > 0 ? Tq - 1 : 0))
            return fail(CSA_ERR_CAPACITY, "window ring cap %lld < window + Tq - 1 = %lld", (long long)win->cap, (long long)p->window + Tq - 1);
    }
    if ((int64_t)B * Tq > 0) {
        if (!q || !q_pos || !sink || !out) return fail(CSA_ERR_INVALID_ARG, "q / q_pos / sink / out is null");
        if (!comp->rec) return fail(CSA_ERR_INVALID_ARG, "comp->rec is null");
        if (p->window > 0 && !win->rec) return fail(CSA_ERR_INVALID_ARG, "win->rec is null");
    }
    return CSA_OK;
}

csa_status run_attention(const void* q, int32_t q_dtype, const int32_t* q_pos, const int32_t* topk_idx, int32_t topk,
                         const csa_kv_cache* comp, const csa_kv_cache* win, const float* gamma_q, const float* sink,
                         const csa_attn_params* p, int32_t B, int32_t Tq, int32_t H, void* out, int32_t out_dtype,
                         void* workspace, size_t ws_bytes, void* stream) {
    const int64_t max_entries = topk_idx ? topk : comp->cap;
    if (max_entries + p->window > (int64_t)1024 * 256)
        return fail(CSA_ERR_UNSUPPORTED, "entry list of %lld exceeds 262144", (long long)(max_entries + p->window));
    const int64_t rows = (int64_t)B * Tq;
    const size_t need =
        csa_attn_workspace_size(B, Tq, H, p->head_dim, max_entries, p->window, q_dtype, comp->fmt, p->split_policy);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace ? ws_bytes : (size_t)0, need);
    if (rows == 0) return ok();
    csa::AttnArgs a{};
    a.q = q;
    a.q_fmt = q_dtype;
    a.q_pos = q_pos;
    a.topk = topk_idx;
    a.k = topk;
    a.comp = static_cast<const uint8_t*>(comp->rec);
    a.comp_fmt = comp->fmt;
    a.ccap = comp->cap;
    a.comp_rec = (int32_t)csa_kv_record_bytes(comp->fmt, comp->d, comp->d_rope);
    if (p->window > 0) {
        a.win = static_cast<const uint8_t*>(win->rec);
        a.win_fmt = win->fmt;
        a.wcap = win->cap;
        a.win_rec = (int32_t)csa_kv_record_bytes(win->fmt, win->d, win->d_rope);
    } else {
        a.win = nullptr;
        a.win_fmt = comp->fmt;
        a.wcap = 1;
        a.win_rec = a.comp_rec;
    }
    a.gamma_q = gamma_q;
    a.sink = sink;
    a.d = p->head_dim;
    a.dr = p->rope_dim;
    a.W = p->window;
    a.m = p->m;
    a.base = p->rope_base;
    a.scale = p->softmax_scale;
    a.eps = p->rms_eps;
    csa::fill_rope_table(a.rope, a.dr, a.base);
    a.Tq = Tq;
    a.split_tq = p->split_policy == CSA_SPLIT_FIXED ? 1 : Tq;
    a.H = H;
    a.rows = (int32_t)rows;
    a.out = out;
    a.out_fmt = out_dtype;
    a.ws = workspace;
    a.ws_bytes = (int64_t)ws_bytes;
    return hip_status(csa::launch_attention(a, max_entries + p->window, static_cast<hipStream_t>(stream)), "attention launch");
}

}  // namespace

namespace csa {
// the fp64 inverse RoPE frequencies base^(-2i/dr) of every kernel launch
void fill_rope_table(RopeTable& t, int dr, float base) {
    for (int i = 0; i < 64; i++) t.f[i] = (i < dr / 2) ? pow((double)base, -2.0 * i / dr) : 0.0;
}
}  // namespace csa

CSA_API size_t csa_kv_record_bytes(int32_t fmt, int32_t d, int32_t d_rope) {
    if (d < 1 || d_rope < 0 || d_rope > d) return 0;
    if (fmt == CSA_F32) return (size_t)4 * d;
    if (fmt == CSA_BF16) return (size_t)2 * d;
    if (fmt == CSA_FP8_E4M3) return (size_t)(((d - d_rope) + 2 * d_rope + 4 + 15) / 16 * 16);
    return 0;
}

CSA_API const char* csa_last_error(void) { return g_err.c_str(); }

// validates one compression request and fills its launch arguments
static csa_status compress_args(const void* x, int32_t x_dtype, int32_t B, int64_t T, int32_t d,
                                const int32_t* tok_start, int32_t m, const float* score_bias,
                                const float* score_proj, const float* gamma, float eps, int32_t rope_dim,
                                float rope_base, const csa_kv_cache* kv_out, const csa_idx_cache* idx_out,
                                csa::CompressArgs& a) {
    if (B < 0 || T < 0) return fail(CSA_ERR_INVALID_ARG, "bad sizes B=%d T=%lld", B, (long long)T);
    if (B > kMaxGridY) return fail(CSA_ERR_UNSUPPORTED, "B=%d > %lld", B, (long long)kMaxGridY);
    if (d < 2 || d > 1024 || d % 2) return fail(CSA_ERR_INVALID_ARG, "d %d must be even and in [2, 1024]", d);
    if (m < 1 || m > 1024) return fail(CSA_ERR_INVALID_ARG, "m %d must be in [1, 1024]", m);
    if (rope_dim < 0 || rope_dim > d || rope_dim % 2) return fail(CSA_ERR_INVALID_ARG, "rope_dim %d", rope_dim);
    if (rope_dim > 128) return fail(CSA_ERR_UNSUPPORTED, "rope_dim %d > 128", rope_dim);
    if (!is_act_fmt(x_dtype)) return fail(CSA_ERR_UNSUPPORTED, "x dtype %d", x_dtype);
    if ((kv_out != nullptr) == (idx_out != nullptr)) return fail(CSA_ERR_INVALID_ARG, "give exactly one of kv_out / idx_out");
    if (T / m > (int64_t)0x7FFFFFFF) return fail(CSA_ERR_UNSUPPORTED, "too many blocks");
    a = csa::CompressArgs{};
    if (kv_out) {
        if (!is_kv_fmt(kv_out->fmt)) return fail(CSA_ERR_UNSUPPORTED, "kv_out fmt %d", kv_out->fmt);
        if (kv_out->d != d || kv_out->d_rope != rope_dim) return fail(CSA_ERR_INVALID_ARG, "kv_out d/d_rope %d/%d differ from call %d/%d", kv_out->d, kv_out->d_rope, d, rope_dim);
        if (kv_out->cap < 1) return fail(CSA_ERR_INVALID_ARG, "kv_out cap %lld", (long long)kv_out->cap);
        if (!kv_out->rec) return fail(CSA_ERR_INVALID_ARG, "kv_out->rec is null");
        a.out_kind = 0;
        a.fmt = kv_out->fmt;
        a.out = static_cast<uint8_t*>(kv_out->rec);
        a.out_scales = nullptr;
        a.cap = kv_out->cap;
        a.ring = kv_out->ring ? 1 : 0;
        a.rec_bytes = (int32_t)csa_kv_record_bytes(kv_out->fmt, d, rope_dim);
    } else {
        if (!is_idx_fmt(idx_out->fmt)) return fail(CSA_ERR_UNSUPPORTED, "idx_out fmt %d", idx_out->fmt);
        if (idx_out->di != d) return fail(CSA_ERR_INVALID_ARG, "idx_out di %d differs from d %d", idx_out->di, d);
        if (idx_out->fmt == CSA_FP4_E2M1 && (d % 32 || !idx_out->scales))
            return fail(idx_out->scales ? CSA_ERR_UNSUPPORTED : CSA_ERR_INVALID_ARG, "FP4 rows need di %% 32 == 0 and a scales plane");
        if (idx_out->cap < 1) return fail(CSA_ERR_INVALID_ARG, "idx_out cap %lld", (long long)idx_out->cap);
        if (!idx_out->codes) return fail(CSA_ERR_INVALID_ARG, "idx_out->codes is null");
        a.out_kind = 1;
        a.fmt = idx_out->fmt;
        a.out = static_cast<uint8_t*>(idx_out->codes);
        a.out_scales = idx_out->scales;
        a.cap = idx_out->cap;
        a.ring = 0;
        a.rec_bytes = (int32_t)idx_row_bytes(idx_out->fmt, d);
    }
    if ((int64_t)B * (T / m) > 0 && (!x || !tok_start || !score_bias))
        return fail(CSA_ERR_INVALID_ARG, "x / tok_start / score_bias is null");
    a.x = x;
    a.B = B;
    a.d = d;
    a.m = m;
    a.T = T;
    a.tok_start = tok_start;
    a.sbias = score_bias;
    a.sproj = score_proj;
    a.gamma = gamma;
    a.eps = eps;
    a.dr = rope_dim;
    a.base = rope_base;
    csa::fill_rope_table(a.rope, rope_dim, rope_base);
    return CSA_OK;
}

CSA_API csa_status csa_compress_kv(const void* x, int32_t x_dtype, int32_t B, int64_t T, int32_t d,
                                   const int32_t* tok_start, int32_t m, const float* score_bias,
                                   const float* score_proj, const float* gamma, float eps, int32_t rope_dim,
                                   float rope_base, const csa_kv_cache* kv_out, const csa_idx_cache* idx_out,
                                   void* stream) {
    csa::CompressArgs a;
    const csa_status st = compress_args(x, x_dtype, B, T, d, tok_start, m, score_bias, score_proj, gamma, eps,
                                        rope_dim, rope_base, kv_out, idx_out, a);
    if (st != CSA_OK) return st;
    return hip_status(csa::launch_compress(a, x_dtype, static_cast<hipStream_t>(stream)), "compress launch");
}

CSA_API csa_status csa_compress_kv_batch(const csa_compress_job* jobs, int32_t njobs, int32_t x_dtype,
                                         void* stream) {
    if (njobs < 0 || (njobs > 0 && !jobs))
        return fail(CSA_ERR_INVALID_ARG, "njobs %d with jobs %p", njobs, (const void*)jobs);
    std::vector<csa::CompressArgs> args((size_t)njobs);
    for (int k = 0; k < njobs; k++) {
        const csa_compress_job& j = jobs[k];
        const csa_status st = compress_args(j.x, x_dtype, j.B, j.T, j.d, j.tok_start, j.m, j.score_bias, j.score_proj,
                                            j.gamma, j.eps, j.rope_dim, j.rope_base, j.kv_out, j.idx_out, args[k]);
        if (st != CSA_OK) return st;
    }
    if (njobs == 0) return CSA_OK;
    return hip_status(csa::launch_compress_batch(args.data(), njobs, x_dtype, static_cast<hipStream_t>(stream)),
                      "compress batch launch");
}

CSA_API csa_status csa_compress_kv_step(const csa_compress_step_job* jobs, int32_t njobs, int32_t x_dtype,
                                        void* stream) {
    if (njobs < 0 || (njobs > 0 && !jobs))
        return fail(CSA_ERR_INVALID_ARG, "njobs %d with jobs %p", njobs, (const void*)jobs);
    std::vector<csa::CompressArgs> args((size_t)njobs);
    for (int k = 0; k < njobs; k++) {
        const csa_compress_step_job& j = jobs[k];
        // the checks of a call over one block of m tokens
        const csa_status st = compress_args(j.x, x_dtype, j.B, j.m, j.d, j.tok_pos, j.m, j.score_bias, j.score_proj,
                                            j.gamma, j.eps, j.rope_dim, j.rope_base, j.kv_out, j.idx_out, args[k]);
        if (st != CSA_OK) return st;
        if (j.m > 1 && j.B > 0 && !j.state) return fail(CSA_ERR_INVALID_ARG, "job %d: m %d needs a state", k, j.m);
        args[k].T = 1;
        args[k].state = j.m > 1 ? j.state : nullptr;
    }
    if (njobs == 0) return CSA_OK;
    return hip_status(csa::launch_compress_step(args.data(), njobs, x_dtype, static_cast<hipStream_t>(stream)),
                      "compress step launch");
}

CSA_API size_t csa_indexer_topk_workspace_size(int32_t B, int32_t Tq, int64_t key_cap, int32_t topk) {
    const int64_t rows = (int64_t)(B > 0 ? B : 0) * (Tq > 0 ? Tq : 0);
    if (rows == 0 || key_cap <= csa::kIdxSmallMaxKeys || topk < 1) return 0;
    int64_t need = idx_rows_per_batch(rows, key_cap, topk) * csa::idx_ws_row_bytes(key_cap, topk);
    // room for the query-batched prefill path too (used for FP4 queries and keys)
    if (csa::idx_prefill_eligible(64, 4, Tq, key_cap, topk))
        need = std::max<int64_t>(need, rows * csa::idx_prefill_row_bytes());
    // and for the decode path (FP4 queries and keys, every row at once)
    if (csa::idx_decode_eligible(64, 4, Tq, key_cap, topk))
        need = std::max<int64_t>(need, rows * csa::idx_decode_row_bytes(key_cap));
    return (size_t)need;
}

CSA_API csa_status csa_indexer_topk(const void* q_idx, const uint8_t* q_idx_scales, int32_t q_dtype, const float* w_idx,
                                    const csa_idx_cache* keys, const int32_t* q_pos, int32_t B, int32_t Tq, int32_t Hi,
                                    int32_t m, int32_t topk, int32_t* out_idx, void* workspace, size_t ws_bytes,
                                    void* stream) {
    if (!keys) return fail(CSA_ERR_INVALID_ARG, "keys is null");
    if (B < 0 || Tq < 0) return fail(CSA_ERR_INVALID_ARG, "bad sizes B=%d Tq=%d", B, Tq);
    if (Hi < 1 || Hi > 16) return fail(Hi < 1 ? CSA_ERR_INVALID_ARG : CSA_ERR_UNSUPPORTED, "Hi %d must be in [1, 16]", Hi);
    if (m < 1) return fail(CSA_ERR_INVALID_ARG, "m %d", m);
    if (topk < 1) return fail(CSA_ERR_INVALID_ARG, "topk %d", topk);
    if (topk > csa::kIdxMaxTopk) return fail(CSA_ERR_UNSUPPORTED, "topk %d > %d", topk, csa::kIdxMaxTopk);
    const int di = keys->di;
    if (di < 32 || di > 256 || di % 32) return fail(CSA_ERR_UNSUPPORTED, "di %d must be a multiple of 32 in [32, 256]", di);
    if (!is_idx_fmt(q_dtype)) return fail(CSA_ERR_UNSUPPORTED, "q dtype %d", q_dtype);
    if (!is_idx_fmt(keys->fmt)) return fail(CSA_ERR_UNSUPPORTED, "key fmt %d", keys->fmt);
    if (keys->cap < 1) return fail(CSA_ERR_INVALID_ARG, "key cap %lld", (long long)keys->cap);
    const int64_t rows = (int64_t)B * Tq;
    if (rows > 0) {
        if (!q_idx || !w_idx || !q_pos || !out_idx || !keys->codes)
            return fail(CSA_ERR_INVALID_ARG, "q_idx / w_idx / q_pos / out_idx / keys->codes is null");
        if (q_dtype == CSA_FP4_E2M1 && !q_idx_scales) return fail(CSA_ERR_INVALID_ARG, "FP4 queries need q_idx_scales");
        if (keys->fmt == CSA_FP4_E2M1 && !keys->scales) return fail(CSA_ERR_INVALID_ARG, "FP4 keys need a scales plane");
        if (!aligned16(keys->codes) || !aligned16(q_idx)) return fail(CSA_ERR_INVALID_ARG, "key / query rows must be 16-byte aligned");
    }
    const size_t need = csa_indexer_topk_workspace_size(B, Tq, keys->cap, topk);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(CSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace ? ws_bytes : (size_t)0, need);
    if (need > 0 && !aligned16(workspace)) return fail(CSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (rows == 0) return ok();
    csa::IndexerArgs a{};
    a.q = q_idx;
    a.q_scales = q_idx_scales;
    a.q_fmt = q_dtype;
    a.w = w_idx;
    a.keys = static_cast<const uint8_t*>(keys->codes);
    a.key_scales = keys->scales;
    a.key_fmt = keys->fmt;
    a.cap = keys->cap;
    a.di = di;
    a.Hi = Hi;
    a.m = m;
    a.topk = topk;
    a.Tq = Tq;
    a.q_pos = q_pos;
    a.out = out_idx;
    a.ws = static_cast<uint8_t*>(workspace);
    a.ws_row_bytes = csa::idx_ws_row_bytes(keys->cap, topk);
    const int64_t batch = need > 0 ? (int64_t)(ws_bytes / (size_t)a.ws_row_bytes) : 0;
    const int64_t per = batch > kMaxGridY ? kMaxGridY : batch;
    return hip_status(csa::launch_indexer_topk(a, rows, per * a.ws_row_bytes, static_cast<hipStream_t>(stream)),
                      "indexer launch");
}

// ---- the indexer without a caller workspace: a static device array
// (kNoAllocScratchBytes on every GPU the library runs on, held until the
// process ends) takes the workspace's place.  Its address is taken once per
// device with hipGetSymbolAddress, on the first call with that device
// current; in host code the array's name is not a device address.
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

csa_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CSA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(CSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CSA_OK;
}
}  // namespace

CSA_API csa_status csa_indexer_topk_noalloc(const void* q_idx, const uint8_t* q_idx_scales, int32_t q_dtype,
                                            const float* w_idx, const csa_idx_cache* keys, const int32_t* q_pos,
                                            int32_t B, int32_t Tq, int32_t Hi, int32_t m, int32_t topk,
                                            int32_t* out_idx, void* stream) {
    if (!keys) return fail(CSA_ERR_INVALID_ARG, "keys is null");
    const size_t need = csa_indexer_topk_workspace_size(B, Tq, keys->cap, topk);
    if (need > kNoAllocScratchBytes)
        return fail(CSA_ERR_WORKSPACE, "the call needs %zu bytes of scratch; the static scratch holds %zu", need,
                    kNoAllocScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        const csa_status st = scratch_address(&ws);
        if (st != CSA_OK) return st;
    }
    return csa_indexer_topk(q_idx, q_idx_scales, q_dtype, w_idx, keys, q_pos, B, Tq, Hi, m, topk, out_idx, ws,
                            need > 0 ? kNoAllocScratchBytes : 0, stream);
}

CSA_API size_t csa_attn_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t head_dim, int64_t max_comp_entries,
                                       int32_t window, int32_t q_dtype, int32_t comp_fmt, int32_t split_policy) {
    const int64_t rows = (int64_t)(B > 0 ? B : 0) * (Tq > 0 ? Tq : 0);
    if (rows == 0 || H < 1 || head_dim < 1) return 0;
    (void)q_dtype;
    (void)comp_fmt;
    const int32_t split_tq = split_policy == CSA_SPLIT_FIXED ? 1 : Tq;
    return (size_t)csa::attn_ws_bytes(rows, split_tq, H, head_dim, max_comp_entries + (window > 0 ? window : 0));
}

CSA_API csa_status csa_sparse_mqa_attn(const void* q, int32_t q_dtype, const int32_t* q_pos, const int32_t* topk_idx,
                                       int32_t topk, const csa_kv_cache* comp, const csa_kv_cache* win,
                                       const float* gamma_q, const float* sink, const csa_attn_params* p, int32_t B,
                                       int32_t Tq, int32_t H, void* out, int32_t out_dtype, void* workspace,
                                       size_t ws_bytes, void* stream) {
    csa_status st = check_attn_common(q, q_dtype, q_pos, comp, win, sink, p, B, Tq, H, out, out_dtype);
    if (st != CSA_OK) return st;
    if (topk < 1) return fail(CSA_ERR_INVALID_ARG, "topk %d", topk);
    if ((int64_t)B * Tq > 0 && !topk_idx) return fail(CSA_ERR_INVALID_ARG, "topk_idx is null");
    return run_attention(q, q_dtype, q_pos, topk_idx, topk, comp, win, gamma_q, sink, p, B, Tq, H, out, out_dtype,
                         workspace, ws_bytes, stream);
}

CSA_API csa_status hca_dense_mqa_attn(const void* q, int32_t q_dtype, const int32_t* q_pos, const csa_kv_cache* comp,
                                      const csa_kv_cache* win, const float* gamma_q, const float* sink,
                                      const csa_attn_params* p, int32_t B, int32_t Tq, int32_t H, void* out,
                                      int32_t out_dtype, void* workspace, size_t ws_bytes, void* stream) {
    csa_status st = check_attn_common(q, q_dtype, q_pos, comp, win, sink, p, B, Tq, H, out, out_dtype);
    if (st != CSA_OK) return st;
    return run_attention(q, q_dtype, q_pos, nullptr, 0, comp, win, gamma_q, sink, p, B, Tq, H, out, out_dtype,
                         workspace, ws_bytes, stream);
}

CSA_API csa_status attn_out_proj_grouped(const void* o, int32_t o_dtype, const void* W, int32_t w_dtype, int64_t M,
                                         int32_t Hd, int32_t D, int32_t G, void* y, int32_t y_dtype, void* stream) {
    if (M < 0 || Hd < 1 || D < 1 || G < 1) return fail(CSA_ERR_INVALID_ARG, "bad sizes M=%lld Hd=%d D=%d G=%d", (long long)M, Hd, D, G);
    if (Hd % G || D % G) return fail(CSA_ERR_INVALID_ARG, "Hd %d and D %d must be multiples of G %d", Hd, D, G);
    if (!is_act_fmt(o_dtype) || o_dtype != w_dtype) return fail(CSA_ERR_UNSUPPORTED, "o / W dtypes %d / %d", o_dtype, w_dtype);
    if (!is_act_fmt(y_dtype)) return fail(CSA_ERR_UNSUPPORTED, "y dtype %d", y_dtype);
    if ((M + 31) / 32 > kMaxGridY) return fail(CSA_ERR_UNSUPPORTED, "M=%lld too large", (long long)M);
    if (M > 0 && (!o || !W || !y)) return fail(CSA_ERR_INVALID_ARG, "o / W / y is null");
    csa::ProjArgs a{};
    a.o = o;
    a.W = W;
    a.y = y;
    a.M = M;
    a.Hd = Hd;
    a.D = D;
    a.G = G;
    a.fmt = o_dtype;
    a.y_fmt = y_dtype;
    return hip_status(csa::launch_proj(a, static_cast<hipStream_t>(stream)), "projection launch");
}

namespace {

// shape checks shared by the FP8-weight projections
csa_status check_lin8(const void* x, int32_t x_dtype, int64_t M, int32_t K, const uint8_t* W, const float* w_scale,
                      int64_t N, int32_t G) {
    if (M < 0 || K < 1 || N < 1 || G < 1) return fail(CSA_ERR_INVALID_ARG, "bad sizes M=%lld K=%d N=%lld G=%d", (long long)M, K, (long long)N, G);
    if (K % G || N % G) return fail(CSA_ERR_INVALID_ARG, "K %d and N %lld must be multiples of G %d", K, (long long)N, G);
    if (N > 0x7fffffff) return fail(CSA_ERR_UNSUPPORTED, "N=%lld too large", (long long)N);
    if (x_dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "x dtype %d (bf16 activations only)", x_dtype);
    if ((K / G) % 64) return fail(CSA_ERR_UNSUPPORTED, "group width K/G=%d is not a multiple of 64", K / G);
    if (M > 0 && (!x || !W || !w_scale)) return fail(CSA_ERR_INVALID_ARG, "x / W / w_scale is null");
    if (M > 0 && (!aligned16(x) || !aligned16(W))) return fail(CSA_ERR_UNSUPPORTED, "x and W must be 16-byte aligned");
    const int64_t grid = M <= csa::kLinSkinnyMaxM ? (int64_t)G * ((N / G + 15) / 16) : csa::lin8_max_tiles(M, (int32_t)N, G);
    if (grid > 0x7fffffff) return fail(CSA_ERR_UNSUPPORTED, "M=%lld N=%lld too large for one launch", (long long)M, (long long)N);
    return CSA_OK;
}

}  // namespace

CSA_API csa_status csa_linear_fp8(const void* x, int32_t x_dtype, int64_t M, int32_t K, const uint8_t* W,
                                  const float* w_scale, int32_t N, int32_t G, void* y, int32_t y_dtype, void* stream) {
    const csa_status st = check_lin8(x, x_dtype, M, K, W, w_scale, N, G);
    if (st != CSA_OK) return st;
    if (!is_act_fmt(y_dtype)) return fail(CSA_ERR_UNSUPPORTED, "y dtype %d", y_dtype);
    if (M > 0 && !y) return fail(CSA_ERR_INVALID_ARG, "y is null");
    csa::LinArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.M = M;
    a.K = K;
    a.N = N;
    a.G = G;
    a.W = W;
    a.scale = w_scale;
    a.nseg = 1;
    a.seg[0] = csa::LinSeg{0, y_dtype, N, y};
    return hip_status(csa::launch_lin8(a, static_cast<hipStream_t>(stream)), "fp8 projection launch");
}

CSA_API size_t csa_layer_in_proj_workspace_size(int64_t M, int32_t Hi, int32_t di) {
    if (M < 0 || Hi < 1 || di < 1) return 0;
    return (size_t)M * Hi * di * sizeof(float);
}

CSA_API csa_status csa_layer_in_proj(const void* h, int32_t h_dtype, int64_t M, int32_t D, const uint8_t* W,
                                     const float* w_scale, int32_t H, int32_t d, int32_t di, int32_t Hi, void* q,
                                     void* kv, void* k_idx, uint8_t* q_idx, uint8_t* q_idx_scales, float* w_idx,
                                     void* workspace, size_t ws_bytes, void* stream) {
    if (H < 1 || d < 1 || di < 1 || Hi < 1) return fail(CSA_ERR_INVALID_ARG, "bad sizes H=%d d=%d di=%d Hi=%d", H, d, di, Hi);
    const int64_t nq = (int64_t)H * d, nqi = (int64_t)Hi * di;
    const int64_t N = nq + d + di + nqi + Hi;
    const csa_status st = check_lin8(h, h_dtype, M, D, W, w_scale, N, 1);
    if (st != CSA_OK) return st;
    if (di % 32 || di > 256) return fail(CSA_ERR_UNSUPPORTED, "di=%d: FP4 queries need a multiple of 32, at most 256", di);
    if (M > 0 && (!q || !kv || !k_idx || !q_idx || !q_idx_scales || !w_idx))
        return fail(CSA_ERR_INVALID_ARG, "an output pointer is null");
    const size_t need = csa_layer_in_proj_workspace_size(M, Hi, di);
    if (M > 0 && (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 3u)))
        return fail(CSA_ERR_WORKSPACE, "workspace %zu bytes (need %zu, 4-byte aligned)", ws_bytes, need);
    if (M == 0) return ok();
    csa::LinArgs a{};
    a.x = static_cast<const uint16_t*>(h);
    a.M = M;
    a.K = D;
    a.N = (int32_t)N;
    a.G = 1;
    a.W = W;
    a.scale = w_scale;
    a.nseg = 5;
    int32_t n0 = 0;
    a.seg[0] = csa::LinSeg{n0, CSA_BF16, nq, q};
    n0 += (int32_t)nq;
    a.seg[1] = csa::LinSeg{n0, CSA_BF16, d, kv};
    n0 += d;
    a.seg[2] = csa::LinSeg{n0, CSA_BF16, di, k_idx};
    n0 += di;
    a.seg[3] = csa::LinSeg{n0, CSA_F32, nqi, workspace};
    n0 += (int32_t)nqi;
    a.seg[4] = csa::LinSeg{n0, CSA_F32, Hi, w_idx};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = csa::launch_lin8(a, s);
    if (e == hipSuccess) e = csa::launch_fp4_rows(static_cast<const float*>(workspace), M * Hi, di, q_idx, q_idx_scales, s);
    return hip_status(e, "input projection launch");
}
