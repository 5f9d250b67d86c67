// attn.hip -- csa_sparse_mqa_attn / hca_dense_mqa_attn.
//
// Method: "DeepSeek-V4 ... open-source declaration" (peacm.com) section 3.2:
// CSA step 3 (multi-query attention over the top-k compressed blocks), the
// HCA paragraph (dense attention over every compressed entry) and the four
// tricks (query RMSNorm, partial RoPE with a RoPE at -i on the output, the
// raw 128-token window visible to every query, a learnable sink logit in the
// softmax denominator); "DeepSeek V4 (Flash & Pro)" wiki article: HCA is a
// dense MQA stream plus a 128-token window.
//
// Decomposition (flash-decoding): a query row's entry list -- its compressed
// entries (top-k slots, or every visible block) followed by its W window
// positions -- is cut into splits (attn_split_len, launch.hpp); one workgroup
// per (split, row, head group) keeps a running max / sum / output per head,
// and a combine kernel merges the splits in split order, adds the sink and
// applies the output RoPE.  A row whose list fits in one split is finished
// in place.  Split sizes depend only on the row's own entry count, so the
// result of a row does not depend on the batch it is in.
//
// This file holds the generic kernel (fp32 VALU, any cache format); the MFMA
// kernel for bf16 queries lives in attn_mfma.hip.
#include <map>
#include <mutex>
#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kAttnThreads = 256;
constexpr int kAttnTile = 8;
constexpr int kAttnMaxD = 1024;
// combine: one workgroup per (head, query row); every thread's partial loads
// in flight at once (d / 4 columns x groups of splits)
constexpr int kCombThreads = 1024;
constexpr int kCombMaxSplits = 64;
constexpr int kCombLoads = kCombMaxSplits / (kCombThreads / (kAttnMaxD / 4));
constexpr int kComb256Loads = 8;           // loads per split group in the 256-thread combine
constexpr int kAttnQFloats = 4096;

__device__ __forceinline__ int64_t comp_slots(const AttnArgs& a, int64_t t) {
    if (a.topk) return a.k;
    int64_t n = t < 0 ? 0 : (t + 1) / a.m;
    return n < a.ccap ? n : a.ccap;
}

// record of entry e of a row (nullptr if masked)
__device__ __forceinline__ const uint8_t* entry_rec(const AttnArgs& a, int64_t row, int64_t b, int64_t t,
                                                    int64_t nc, int64_t e, int& fmt) {
    if (e < nc) {
        int64_t j = e;
        if (a.topk) {
            j = a.topk[row * a.k + e];
            int64_t vis = t < 0 ? 0 : (t + 1) / a.m;
            if (vis > a.ccap) vis = a.ccap;
            if (j < 0 || j >= vis) return nullptr;
        }
        fmt = a.comp_fmt;
        return a.comp + (b * a.ccap + j) * a.comp_rec;
    }
    int64_t s = t - a.W + 1 + (e - nc);
    if (s < 0) return nullptr;
    fmt = a.win_fmt;
    return a.win + (b * a.wcap + s % a.wcap) * a.win_rec;
}

__device__ __forceinline__ float rec_value(const uint8_t* rec, int fmt, int d, int dr, int k) {
    if (fmt == CSA_F32) return reinterpret_cast<const float*>(rec)[k];
    if (fmt == CSA_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(rec)[k]);
    const int dn = d - dr;
    if (k < dn) return e4m3_to_f32(rec[k]) * *reinterpret_cast<const float*>(rec + dn + 2 * dr);
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(rec + dn)[k - dn]);
}

// q^ = RoPE_t(RMSNorm(q)) for heads [h0, h0+hg) into qs[hh*d + k]; one wave per head
template <typename QT>
__device__ void query_prologue(const AttnArgs& a, int64_t row, int h0, int hg, int64_t t, float* qs, const double* rf) {
    const int d = a.d, lane = threadIdx.x & (kWave - 1), nw = blockDim.x / kWave;
    const QT* q = reinterpret_cast<const QT*>(a.q) + (row * a.H + h0) * d;
    for (int hh = threadIdx.x / kWave; hh < hg; hh += nw) {
        float ss = 0.0f;
        for (int k = lane; k < d; k += kWave) {
            float v = ld_scalar<QT>(q, (size_t)hh * d + k);
            ss += v * v;
        }
        ss = wave_sum(ss);
        const float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
        for (int k = lane; k < d; k += kWave) {
            float v = ld_scalar<QT>(q, (size_t)hh * d + k) * inv;
            qs[hh * d + k] = a.gamma_q ? v * a.gamma_q[k] : v;
        }
        // RoPE_t on the last dr dims (each lane rotates its own pairs)
        const int off = d - a.dr;
        for (int p = lane; p < a.dr / 2; p += kWave) {
            float sn, cs;
            rope_sincos((double)t, rf[p], sn, cs);
            float x0 = qs[hh * d + off + 2 * p], x1 = qs[hh * d + off + 2 * p + 1];
            qs[hh * d + off + 2 * p] = x0 * cs - x1 * sn;
            qs[hh * d + off + 2 * p + 1] = x0 * sn + x1 * cs;
        }
    }
}

// output RoPE_{-t} on the last dr dims of one head's vector v[0..d), by
// nthreads threads starting at lane0
__device__ __forceinline__ void rotate_out(const AttnArgs& a, int64_t t, float* v, int lane0, int nthreads,
                                           const double* rf) {
    const int d = a.d, off = d - a.dr;
    for (int p = lane0; p < a.dr / 2; p += nthreads) {
        float sn, cs;
        rope_sincos(-(double)t, rf[p], sn, cs);
        float x0 = v[off + 2 * p], x1 = v[off + 2 * p + 1];
        v[off + 2 * p] = x0 * cs - x1 * sn;
        v[off + 2 * p + 1] = x0 * sn + x1 * cs;
    }
}

template <typename QT, typename OT>
__global__ __launch_bounds__(kAttnThreads) void k_attn_valu(AttnArgs a, int HG) {
    __shared__ float qs[kAttnQFloats];
    __shared__ float kv[kAttnTile * (kAttnMaxD + 1)];
    __shared__ float pz[kAttnQFloats / 64 * kAttnTile];   // [hg][tile]
    __shared__ float mrun[kAttnQFloats / 64], lrun[kAttnQFloats / 64], alph[kAttnQFloats / 64];
    __shared__ int valid[kAttnTile];
    __shared__ double rf[64];

    const int64_t row = blockIdx.y, b = row / a.Tq;
    const int64_t t = a.q_pos[row];
    const int64_t nc = comp_slots(a, t);
    const int64_t ne = nc + a.W;
    const int64_t split = attn_split_len(ne, a.split_tq);
    const int64_t nsplit = attn_nsplit(ne, a.split_tq);
    const int64_t s = blockIdx.x;
    if (s >= nsplit) return;
    const int64_t e0 = s * split, e1 = min(e0 + split, ne);
    const int h0 = blockIdx.z * HG, hg = min(HG, a.H - h0);
    const int d = a.d, ld = d + 1;
    const int tid = threadIdx.x;

    stage_rope_arg(offsetof(AttnArgs, rope), rf, a.dr / 2);
    __syncthreads();
    query_prologue<QT>(a, row, h0, hg, t, qs, rf);
    for (int hh = tid; hh < hg; hh += blockDim.x) { mrun[hh] = -INFINITY; lrun[hh] = 0.0f; }
    constexpr int kMaxOwn = kAttnQFloats / kAttnThreads;
    float o[kMaxOwn];
#pragma unroll
    for (int q = 0; q < kMaxOwn; q++) o[q] = 0.0f;
    __syncthreads();

    for (int64_t et = e0; et < e1; et += kAttnTile) {
        const int nt = (int)min((int64_t)kAttnTile, e1 - et);
        if (tid < kAttnTile) {
            int fmt;
            valid[tid] = tid < nt && entry_rec(a, row, b, t, nc, et + tid, fmt) != nullptr;
        }
        for (int idx = tid; idx < kAttnTile * d; idx += blockDim.x) {
            const int ee = idx / d, k = idx % d;
            float v = 0.0f;
            if (ee < nt) {
                int fmt = 0;
                const uint8_t* rec = entry_rec(a, row, b, t, nc, et + ee, fmt);
                if (rec) v = rec_value(rec, fmt, d, a.dr, k);
            }
            kv[ee * ld + k] = v;
        }
        __syncthreads();
        for (int idx = tid; idx < hg * kAttnTile; idx += blockDim.x) {
            const int hh = idx / kAttnTile, ee = idx % kAttnTile;
            float z = -INFINITY;
            if (ee < nt && valid[ee]) {
                float acc = 0.0f;
                for (int k = 0; k < d; k++) acc = fmaf(qs[hh * d + k], kv[ee * ld + k], acc);
                z = acc * a.scale;
            }
            pz[hh * kAttnTile + ee] = z;
        }
        __syncthreads();
        for (int hh = tid; hh < hg; hh += blockDim.x) {
            float mt = -INFINITY;
            for (int ee = 0; ee < kAttnTile; ee++) mt = fmaxf(mt, pz[hh * kAttnTile + ee]);
            const float mo = mrun[hh], mn = fmaxf(mo, mt);
            float al = 1.0f, sum = 0.0f;
            if (mn != -INFINITY) {
                al = expf(mo - mn);
                for (int ee = 0; ee < kAttnTile; ee++) {
                    float p = expf(pz[hh * kAttnTile + ee] - mn);
                    pz[hh * kAttnTile + ee] = p;
                    sum += p;
                }
            } else {
                for (int ee = 0; ee < kAttnTile; ee++) pz[hh * kAttnTile + ee] = 0.0f;
            }
            lrun[hh] = lrun[hh] * al + sum;
            mrun[hh] = mn;
            alph[hh] = al;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kMaxOwn; q++) {
            const int idx = tid + q * kAttnThreads;
            if (idx < hg * d) {
                const int hh = idx / d, k = idx % d;
                float acc = o[q] * alph[hh];
                for (int ee = 0; ee < kAttnTile; ee++) acc = fmaf(pz[hh * kAttnTile + ee], kv[ee * ld + k], acc);
                o[q] = acc;
            }
        }
        __syncthreads();
    }

    if (nsplit <= 1) {
        // whole list in this split: normalise with the sink, rotate, store
#pragma unroll
        for (int q = 0; q < kMaxOwn; q++) {
            const int idx = tid + q * kAttnThreads;
            if (idx < hg * d) {
                const int hh = idx / d;
                const float sk = a.sink[h0 + hh], mr = mrun[hh];
                const float M = fmaxf(mr, sk);
                float v = 0.0f;
                if (M != -INFINITY) {
                    const float den = lrun[hh] * expf(mr - M) + expf(sk - M);
                    v = (mr == -INFINITY) ? 0.0f : o[q] * expf(mr - M) / den;
                }
                qs[idx] = v;
            }
        }
        __syncthreads();
        const int lane = tid & (kWave - 1), nw = blockDim.x / kWave;
        for (int hh = tid / kWave; hh < hg; hh += nw) rotate_out(a, t, qs + hh * d, lane, kWave, rf);
        __syncthreads();
        OT* out = reinterpret_cast<OT*>(a.out) + (row * a.H + h0) * d;
        for (int idx = tid; idx < hg * d; idx += blockDim.x) st_scalar<OT>(out, idx, qs[idx]);
        return;
    }
    // partials: o (relative to mrun), m, l
    float* wo = reinterpret_cast<float*>(a.ws);
    float* wml = wo + (size_t)a.rows * a.nsplit_max * a.H * d;
    const size_t base = ((size_t)row * a.nsplit_max + s) * a.H + h0;
#pragma unroll
    for (int q = 0; q < kMaxOwn; q++) {
        const int idx = tid + q * kAttnThreads;
        if (idx < hg * d) wo[base * d + idx] = o[q];
    }
    for (int hh = tid; hh < hg; hh += blockDim.x) {
        wml[(base + hh) * 2] = mrun[hh];
        wml[(base + hh) * 2 + 1] = lrun[hh];
    }
}

// merge the splits of (row, head): weights exp(m_s - M) with M over the split
// maxima and the sink.  Thread t sums float4 column t % (d/4) over the splits
// of group t / (d/4) (splits g, g + G, ... in order); the groups are then
// added in group order.  Loads return in order: the position and the split
// maxima and sums go out first, then every partial, so the split weights and
// the output's RoPE factors are formed while the partials are in flight.
//
// The split groups are those of a 1,024-thread workgroup (Gc = 1,024 / (d/4)
// groups, whatever the launch) and every group is summed in the same order,
// so the result bits do not depend on NT.  NT = 256 (bf16 partials, d/4
// dividing 256, at most kComb256Loads loads per group): each thread runs R =
// 4 of those groups, so four workgroups fit on a CU where one of 1,024
// threads does (the launcher takes it when (head, row) pairs outnumber the
// CUs).
template <typename OT, int NT, bool PB>
__global__ __launch_bounds__(NT) void k_attn_combine(AttnArgs a) {
    constexpr int R = kCombThreads / NT;                        // canonical split groups per thread
    constexpr int LQ = R == 1 ? kCombLoads : kComb256Loads;     // loads per group at most
    warm_kernargs(offsetof(AttnArgs, rope));
    __shared__ float v[kAttnMaxD];
    __shared__ float wsc[kCombMaxSplits];
    __shared__ float den_s;
    __shared__ double rf[64];
    __shared__ float4 part[kCombThreads];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int NS = a.nsplit_max;
    const int d = a.d;
    const float* wo = reinterpret_cast<const float*>(a.ws);
    const float* wml = wo + (size_t)a.rows * NS * a.H * d;
    const size_t mbase = (size_t)row * NS * a.H + h;           // split s at mbase + s * H
    const int lane = tid & (kWave - 1);
    const int64_t t = a.q_pos[row];
    float ms = -INFINITY, ls = 0.0f;
    if (tid < kWave) {
        const size_t i = (mbase + (size_t)min(lane, NS - 1) * a.H) * 2;
        ms = wml[i];
        ls = wml[i + 1];
    }
    // ---- then this thread's partial columns of its splits (addresses
    // clamped to the buffer; splits past the row's count get weight 0 and
    // are skipped)
    const int nc4 = d / 4 > 0 ? d / 4 : 1;
    const int G = kCombThreads / nc4;                           // split groups (canonical)
    const int c = tid % nc4, g0 = R * (tid / nc4);              // this thread's column and first group
    const float4* wo4 = reinterpret_cast<const float4*>(wo + mbase * d) + c;
    const uint2* wb4 = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.ws) + mbase * d) + c;
    const size_t sstride = (size_t)a.H * d / 4;                 // 4-value groups between splits
    const bool vec = d % 4 == 0;
    constexpr bool pb = PB;                                     // partials in bf16 (a.part_bf16)
    const int nq = vec ? (NS + G - 1) / G : 0;
    // group g0 + r, load q: split g0 + r + q G (bf16 partials stay packed
    // until the weights are known)
    uint2 xb[PB ? R : 1][PB ? LQ : 1];
    float4 xf[PB ? 1 : LQ];
    static_assert(PB || R == 1, "fp32 partials: the 1,024-thread combine");
    if constexpr (PB) {
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int q = 0; q < LQ; q++) {
                xb[r][q] = make_uint2(0u, 0u);
                if (q < nq) xb[r][q] = wb4[(size_t)min(g0 + r + q * G, NS - 1) * sstride];
            }
    } else {
#pragma unroll
        for (int q = 0; q < LQ; q++) {
            xf[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (q < nq) xf[q] = wo4[(size_t)min(g0 + q * G, NS - 1) * sstride];
        }
    }
    stage_rope_arg(offsetof(AttnArgs, rope), rf, a.dr / 2);
    const int64_t nc = comp_slots(a, t);
    const int nsplit = (int)attn_nsplit<int64_t>(nc + a.W, a.split_tq);
    if (nsplit <= 1) return;
    // ---- split weights, one wave (at most 64 splits)
    if (tid < kWave) {
        const float sk = a.sink[h];
        const bool live = lane < nsplit;
        const float M = fmaxf(sk, wave_max_dpp(live ? ms : -INFINITY));
        const float w = (!live || ms == -INFINITY) ? 0.0f : expf(ms - M);
        // lanes past the row's split count hold whatever the buffer held
        // (possibly NaN): they add an exact zero, not 0 * ls
        float den = wave_sum_dpp(live ? ls * w : 0.0f);
        if (M != -INFINITY) den += expf(sk - M);
        wsc[lane] = w;
        if (lane == 0) den_s = den;
    }
    // the -t rotation of this thread's RoPE pairs (vector path: thread c <
    // d / 4 owns dims 4c .. 4c + 3; pairs start at even dims and d - dr is
    // even, so a pair never straddles two threads), from the argument block
    float rsn[2] = {0.0f, 0.0f}, rcs[2] = {1.0f, 1.0f};
    if (vec && tid < nc4) {
        const double* rfa = (const double*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(AttnArgs, rope));
        const int k0 = 4 * tid, off = d - a.dr;
#pragma unroll
        for (int u = 0; u < 2; u++)
            if (k0 + 2 * u >= off) rope_sincos(-(double)t, rfa[(k0 + 2 * u - off) / 2], rsn[u], rcs[u]);
    }
    __syncthreads();
    if (!vec) {
        // head dims not a multiple of 4: one dim per thread, splits in order
        const float den = den_s;
        const float* wo_h = wo + mbase * d;
        const uint16_t* wb_h = reinterpret_cast<const uint16_t*>(a.ws) + mbase * d;
        for (int k = tid; k < d; k += blockDim.x) {
            float acc = 0.0f;
            for (int s2 = 0; s2 < nsplit; s2++) {
                const size_t i = (size_t)s2 * a.H * d + k;
                acc = fmaf(wsc[s2], pb ? __uint_as_float((uint32_t)wb_h[i] << 16) : wo_h[i], acc);
            }
            v[k] = den > 0.0f ? acc / den : 0.0f;
        }
        __syncthreads();
        rotate_out(a, t, v, tid, blockDim.x, rf);
        __syncthreads();
        OT* out = reinterpret_cast<OT*>(a.out) + (row * a.H + h) * d;
        for (int k = tid; k < d; k += blockDim.x) st_scalar<OT>(out, k, v[k]);
        return;
    }
    // ---- each group's splits in order, then the groups in order
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int g = g0 + r;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (g < G) {
#pragma unroll
            for (int q = 0; q < LQ; q++) {
                const int s = g + q * G;
                if (q < nq && s < nsplit) {
                    const float w = wsc[s];
                    float4 x;
                    if constexpr (PB) {
                        const uint2 u = xb[r][q];
                        x = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                                        __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
                    } else {
                        x = xf[q];
                    }
                    acc.x = fmaf(w, x.x, acc.x);
                    acc.y = fmaf(w, x.y, acc.y);
                    acc.z = fmaf(w, x.z, acc.z);
                    acc.w = fmaf(w, x.w, acc.w);
                }
            }
            part[g * nc4 + c] = acc;
        }
    }
    __syncthreads();
    // ---- thread c < d / 4 adds the groups in order, normalises its four
    // dims, rotates the RoPE pairs among them and stores them as one vector
    if (tid < nc4) {
        const float den = den_s;
        float4 r = part[tid];
        for (int q = 1; q < G; q++) {
            const float4 y = part[q * nc4 + tid];
            r.x += y.x; r.y += y.y; r.z += y.z; r.w += y.w;
        }
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        float o[4] = {den > 0.0f ? r.x * inv : 0.0f, den > 0.0f ? r.y * inv : 0.0f,
                      den > 0.0f ? r.z * inv : 0.0f, den > 0.0f ? r.w * inv : 0.0f};
        const int k0 = 4 * tid, off = d - a.dr;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            if (k0 + 2 * u >= off) {
                const float x0 = o[2 * u], x1 = o[2 * u + 1];
                o[2 * u] = x0 * rcs[u] - x1 * rsn[u];
                o[2 * u + 1] = x0 * rsn[u] + x1 * rcs[u];
            }
        }
        OT* out = reinterpret_cast<OT*>(a.out) + (row * a.H + h) * d + k0;
        if ((reinterpret_cast<uintptr_t>(out) & (4 * sizeof(OT) - 1)) != 0) {   // an unaligned output
#pragma unroll
            for (int u = 0; u < 4; u++) st_scalar<OT>(out, u, o[u]);
        } else if constexpr (sizeof(OT) == 2) {
            *reinterpret_cast<uint2*>(out) = make_uint2(
                (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16),
                (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16));
        } else {
            *reinterpret_cast<float4*>(out) = make_float4(o[0], o[1], o[2], o[3]);
        }
    }
}

int64_t attn_ws_bytes(int64_t rows, int32_t split_tq, int32_t H, int32_t d, int64_t max_entries) {
    const int64_t nb = attn_nsplit_bound(max_entries, split_tq);
    if (nb <= 1) return 0;
    return rows * nb * H * ((int64_t)d + 2) * 4;
}

// compute units of the current device, cached per device (a large number
// when the runtime cannot say, which keeps the default combine)
static int device_cus() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1 << 30;
    std::lock_guard<std::mutex> lk(mu);
    const auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 1 << 30;
    cache[dev] = n;
    return n;
}

hipError_t launch_attention(const AttnArgs& a0, int64_t max_entries, hipStream_t st) {
    if (a0.rows == 0) return hipSuccess;
    const int64_t nb = attn_nsplit_bound(max_entries, a0.split_tq);
    AttnArgs a = a0;
    a.nsplit_max = (int32_t)nb;
    // the matrix-core kernel keeps bf16 partials for bf16 outputs (the partial
    // store and the combine read agree through this flag)
    const bool mfma = attn_mfma_supported(a);
    a.part_bf16 = mfma && a.out_fmt == CSA_BF16 ? 1 : 0;
    if (mfma) {
        hipError_t e = launch_attention_mfma(a, nb, st);
        if (e != hipSuccess) return e;
    } else {
        const int HG = min(min(a.H, kAttnQFloats / 64), kAttnQFloats / a.d);
        const int ngroups = (a.H + HG - 1) / HG;
        dim3 grid((unsigned)nb, (unsigned)a.rows, (unsigned)ngroups);
        const bool qb = a.q_fmt == CSA_BF16, ob = a.out_fmt == CSA_BF16;
        if (!qb && !ob) hipLaunchKernelGGL((k_attn_valu<float, float>), grid, dim3(kAttnThreads), 0, st, a, HG);
        if (!qb && ob) hipLaunchKernelGGL((k_attn_valu<float, uint16_t>), grid, dim3(kAttnThreads), 0, st, a, HG);
        if (qb && !ob) hipLaunchKernelGGL((k_attn_valu<uint16_t, float>), grid, dim3(kAttnThreads), 0, st, a, HG);
        if (qb && ob) hipLaunchKernelGGL((k_attn_valu<uint16_t, uint16_t>), grid, dim3(kAttnThreads), 0, st, a, HG);
    }
    if (nb > 1) {
        dim3 g2((unsigned)a.H, (unsigned)a.rows);
        // more (head, row) pairs than CUs: the 256-thread combine (same bits,
        // four workgroups per CU) where it applies
        const int nc4 = a.d / 4;
        const int Gc = nc4 > 0 ? kCombThreads / nc4 : 0;
        const bool small = a.part_bf16 && a.d % 4 == 0 && nc4 > 0 && 256 % nc4 == 0 &&
                           (nb + Gc - 1) / Gc <= kComb256Loads && (int64_t)a.H * a.rows > device_cus();
        if (small) hipLaunchKernelGGL((k_attn_combine<uint16_t, 256, true>), g2, dim3(256), 0, st, a);
        else if (a.part_bf16) hipLaunchKernelGGL((k_attn_combine<uint16_t, kCombThreads, true>), g2, dim3(kCombThreads), 0, st, a);
        else if (a.out_fmt == CSA_BF16) hipLaunchKernelGGL((k_attn_combine<uint16_t, kCombThreads, false>), g2, dim3(kCombThreads), 0, st, a);
        else hipLaunchKernelGGL((k_attn_combine<float, kCombThreads, false>), g2, dim3(kCombThreads), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace csa
