// attn_mfma.hip -- MFMA kernel of csa_sparse_mqa_attn / hca_dense_mqa_attn for
// bf16 queries over bf16 / FP8 caches (gfx950, v_mfma_f32_16x16x32_bf16).
//
// Same method and decomposition as attn.hip (peacm.com section 3.2: MQA over
// the selected compressed entries plus the raw window, Q/KV RMSNorm, partial
// RoPE with the -i output RoPE, sink logit in the denominator), arranged for
// the matrix cores:
//   - one query row per workgroup and split; each wave owns 16 heads, whose
//     normalised and rotated queries sit in registers as MFMA A-fragments;
//   - all heads of the workgroup share one LDS tile of 32 entries (MQA: one
//     KV vector per entry serves every head); FP8 records are expanded to
//     bf16 on the way in with the hardware OCP-E4M3 conversion, their per-row
//     scale kept aside and applied to the logits of the non-RoPE part and to
//     the probabilities of the non-RoPE output dims (exactly the decoded
//     value, since scale * <q, code> = <q, scale * code>);
//   - S = Q K^T and O += P V run as 16x16x32 MFMAs with fp32 accumulation; P
//     goes through a small per-wave LDS buffer to turn the accumulator layout
//     into the A-operand layout; the online softmax keeps running max / sum
//     per head in registers and skips the O rescale when no max moved.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMTE = 32;       // entries per LDS tile
constexpr int kMSplit = 128;   // entries per workgroup (fixed: results independent of the batch)
constexpr int kPStride = kMTE + 8;

template <int D>
struct MfmaSmem {
    uint8_t tile[kMTE][D * 2 + 16];          // bf16 entries, rows padded by 16 bytes
    const uint8_t* rec[kMTE];
    int fmt[kMTE];
    float scale[kMTE];
    uint16_t p[4][2][16][kPStride];          // per wave: [scaled, plain] P, 16 heads x 32 entries
};

// same entry enumeration as the generic kernel
__device__ __forceinline__ const uint8_t* mfma_entry_rec(const AttnArgs& a, int64_t row, int64_t b, int64_t t,
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

__device__ __forceinline__ uint32_t pack_bf16x2(bf16x2_t v) {
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}

template <int D, typename OT>
__global__ __launch_bounds__(256) void k_attn_mfma(AttnArgs a, int nsplit_max) {
    constexpr int NS = D / 32;   // QK K-steps
    constexpr int ND = D / 16;   // PV N-tiles
    __shared__ MfmaSmem<D> sm;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t row = blockIdx.y, b = row / a.Tq;
    const int64_t t = a.q_pos[row];
    int64_t nc;
    if (a.topk) nc = a.k;
    else {
        nc = t < 0 ? 0 : (t + 1) / a.m;
        if (nc > a.ccap) nc = a.ccap;
    }
    const int64_t ne = nc + a.W;
    const int64_t nsplit = (ne + kMSplit - 1) / kMSplit;
    const int64_t sp = blockIdx.x;
    if (sp >= nsplit && !(sp == 0 && ne == 0)) return;
    const int64_t e0 = sp * kMSplit, e1 = min(e0 + (int64_t)kMSplit, ne);
    const int hw = blockIdx.z * 64 + 16 * w;          // first head of this wave
    const bool active = hw < a.H;
    const int dn = D - a.dr;                           // non-RoPE dims (multiple of 32)
    const int nsr = dn / 32, ndr = dn / 16;

    // ---- query prologue: q^ = RoPE_t(RMSNorm(q)) as bf16 A-fragments
    bf16x8_t qf[NS];
    if (active) {
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (row * a.H + hw + l16) * D;
        float v[NS][8];
        float ss = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g4);
            uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[s][2 * j] = __uint_as_float(wd[j] << 16);
                v[s][2 * j + 1] = __uint_as_float(wd[j] & 0xFFFF0000u);
            }
#pragma unroll
            for (int j = 0; j < 8; j++) ss += v[s][j] * v[s][j];
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
        for (int s = 0; s < NS; s++) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int dim = 32 * s + 8 * g4 + j;
                v[s][j] *= inv;
                if (a.gamma_q) v[s][j] *= a.gamma_q[dim];
            }
            if (s >= nsr) {
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const int p = (32 * s + 8 * g4 + j - dn) / 2;
                    float sn, cs;
                    rope_sincos((double)t, a.rope.f[p], sn, cs);
                    const float x0 = v[s][j], x1 = v[s][j + 1];
                    v[s][j] = x0 * cs - x1 * sn;
                    v[s][j + 1] = x0 * sn + x1 * cs;
                }
            }
#pragma unroll
            for (int j = 0; j < 8; j++) qf[s][j] = (__bf16)v[s][j];
        }
    }

    f32x4_t o[ND];
#pragma unroll
    for (int nd = 0; nd < ND; nd++) o[nd] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun[4], lrun[4];
#pragma unroll
    for (int i = 0; i < 4; i++) { mrun[i] = -INFINITY; lrun[i] = 0.0f; }

    for (int64_t et = e0; et < e1; et += kMTE) {
        const int nt = (int)min((int64_t)kMTE, e1 - et);
        __syncthreads();                                   // previous tile consumed
        if (tid < kMTE) {
            int fmt = 0;
            const uint8_t* r = tid < nt ? mfma_entry_rec(a, row, b, t, nc, et + tid, fmt) : nullptr;
            sm.rec[tid] = r;
            sm.fmt[tid] = fmt;
            float sc = 1.0f;
            if (r && fmt == CSA_FP8_E4M3) sc = *reinterpret_cast<const float*>(r + dn + 2 * a.dr);
            sm.scale[tid] = sc;
        }
        __syncthreads();
        // ---- stage the tile: 16-byte chunks of 8 bf16 dims
        for (int idx = tid; idx < kMTE * (D / 8); idx += blockDim.x) {
            const int ee = idx / (D / 8), c = idx % (D / 8);
            const uint8_t* r = sm.rec[ee];
            uint4 out = make_uint4(0u, 0u, 0u, 0u);
            if (r) {
                if (sm.fmt[ee] == CSA_BF16) {
                    out = *reinterpret_cast<const uint4*>(r + 16 * c);
                } else if (8 * c < dn) {
                    const uint2 codes = *reinterpret_cast<const uint2*>(r + 8 * c);
                    out.x = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, 1.0f, false));
                    out.y = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, 1.0f, true));
                    out.z = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, 1.0f, false));
                    out.w = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, 1.0f, true));
                } else {
                    out = *reinterpret_cast<const uint4*>(r + dn + 2 * (8 * c - dn));
                }
            }
            *reinterpret_cast<uint4*>(&sm.tile[ee][16 * c]) = out;
        }
        __syncthreads();
        if (!active) continue;

        // ---- S = Q K^T: two 16-entry N-tiles, split into non-RoPE / RoPE parts
        f32x4_t snr[2], sr[2];
#pragma unroll
        for (int n = 0; n < 2; n++) {
            snr[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            sr[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            const uint8_t* kr = &sm.tile[16 * n + l16][16 * g4];
#pragma unroll
            for (int s = 0; s < NS; s++) {
                const bf16x8_t kb = *reinterpret_cast<const bf16x8_t*>(kr + 64 * s);
                if (s < nsr) snr[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[s], kb, snr[n], 0, 0, 0);
                else sr[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[s], kb, sr[n], 0, 0, 0);
            }
        }
        // ---- online softmax (rows = heads 4*g4 + i; this lane's entries 16n + l16)
        float pz[2][4];
        float alpha[4];
        bool moved = false;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float mt = -INFINITY;
#pragma unroll
            for (int n = 0; n < 2; n++) {
                const int e = 16 * n + l16;
                const float z = sm.rec[e] ? a.scale * (sm.scale[e] * snr[n][i] + sr[n][i]) : -INFINITY;
                pz[n][i] = z;
                mt = fmaxf(mt, z);
            }
#pragma unroll
            for (int o2 = 1; o2 < 16; o2 <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o2, kWave));
            const float mn = fmaxf(mrun[i], mt);
            float al = 1.0f, rs = 0.0f;
            if (mn != -INFINITY) {
                al = expf(mrun[i] - mn);
#pragma unroll
                for (int n = 0; n < 2; n++) {
                    pz[n][i] = expf(pz[n][i] - mn);
                    rs += pz[n][i];
                }
            } else {
                pz[0][i] = 0.0f;
                pz[1][i] = 0.0f;
            }
#pragma unroll
            for (int o2 = 1; o2 < 16; o2 <<= 1) rs += __shfl_xor(rs, o2, kWave);
            lrun[i] = lrun[i] * al + rs;
            mrun[i] = mn;
            alpha[i] = al;
            moved |= (al != 1.0f);
        }
        if (__any(moved)) {
#pragma unroll
            for (int nd = 0; nd < ND; nd++)
#pragma unroll
                for (int i = 0; i < 4; i++) o[nd][i] *= alpha[i];
        }
        // ---- P (scaled for the non-RoPE dims, plain for the RoPE dims) to LDS
#pragma unroll
        for (int n = 0; n < 2; n++) {
            const int e = 16 * n + l16;
            const float sc = sm.scale[e];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const __bf16 ps = (__bf16)(pz[n][i] * sc), pp = (__bf16)pz[n][i];
                sm.p[w][0][4 * g4 + i][e] = __builtin_bit_cast(uint16_t, ps);
                sm.p[w][1][4 * g4 + i][e] = __builtin_bit_cast(uint16_t, pp);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const bf16x8_t pa = *reinterpret_cast<const bf16x8_t*>(&sm.p[w][0][l16][8 * g4]);
        const bf16x8_t pb = *reinterpret_cast<const bf16x8_t*>(&sm.p[w][1][l16][8 * g4]);
        // ---- O += P V (V read down the entry axis, one dim per lane)
#pragma unroll
        for (int nd = 0; nd < ND; nd++) {
            bf16x8_t vb;
#pragma unroll
            for (int j = 0; j < 8; j++)
                vb[j] = *reinterpret_cast<const __bf16*>(&sm.tile[8 * g4 + j][2 * (16 * nd + l16)]);
            o[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nd < ndr ? pa : pb, vb, o[nd], 0, 0, 0);
        }
    }
    if (!active) return;

    const int hb = hw + 4 * g4;                         // this lane's first head row
    if (nsplit <= 1) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float sk = a.sink[hb + i], mr = mrun[i];
            const float M = fmaxf(mr, sk);
            f[i] = 0.0f;
            if (mr != -INFINITY && M != -INFINITY) {
                const float em = expf(mr - M);
                f[i] = em / (lrun[i] * em + expf(sk - M));
            }
        }
        OT* out = reinterpret_cast<OT*>(a.out) + (row * a.H) * D;
#pragma unroll
        for (int nd = 0; nd < ND; nd++) {
            const int dim = 16 * nd + l16;
            float sn = 0.0f, cs = 1.0f;
            if (nd >= ndr) rope_sincos(-(double)t, a.rope.f[(dim - dn) / 2], sn, cs);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float v = o[nd][i] * f[i];
                if (nd >= ndr) {
                    const float pv = __shfl_xor(v, 1, kWave);
                    v = (dim & 1) ? pv * sn + v * cs : v * cs - pv * sn;
                }
                st_scalar<OT>(out, (size_t)(hb + i) * D + dim, v);
            }
        }
        return;
    }
    float* wo = reinterpret_cast<float*>(a.ws);
    float* wml = wo + (size_t)a.rows * nsplit_max * a.H * D;
    const size_t base = ((size_t)row * nsplit_max + sp) * a.H;
#pragma unroll
    for (int nd = 0; nd < ND; nd++)
#pragma unroll
        for (int i = 0; i < 4; i++) wo[(base + hb + i) * D + 16 * nd + l16] = o[nd][i];
    if (l16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            wml[(base + hb + i) * 2] = mrun[i];
            wml[(base + hb + i) * 2 + 1] = lrun[i];
        }
    }
}

bool attn_mfma_supported(const AttnArgs& a) {
    if (a.q_fmt != CSA_BF16) return false;
    if (a.comp_fmt == CSA_F32 || (a.W > 0 && a.win_fmt == CSA_F32)) return false;
    if (a.d != 128 && a.d != 256 && a.d != 512) return false;
    if (a.H % 16 != 0) return false;
    if ((a.d - a.dr) % 32 != 0) return false;
    return true;
}

int attn_mfma_split() { return kMSplit; }

template <typename OT>
static void launch_d(const AttnArgs& a, int nsplit, hipStream_t st) {
    const int groups = (a.H + 63) / 64;
    const int threads = 64 * min(4, a.H / 16);
    dim3 grid((unsigned)nsplit, (unsigned)a.rows, (unsigned)groups);
    if (a.d == 128) hipLaunchKernelGGL((k_attn_mfma<128, OT>), grid, dim3(threads), 0, st, a, nsplit);
    else if (a.d == 256) hipLaunchKernelGGL((k_attn_mfma<256, OT>), grid, dim3(threads), 0, st, a, nsplit);
    else hipLaunchKernelGGL((k_attn_mfma<512, OT>), grid, dim3(threads), 0, st, a, nsplit);
}

hipError_t launch_attention_mfma(const AttnArgs& a, int64_t max_entries, hipStream_t st) {
    const int64_t nsplit = max((int64_t)1, (max_entries + kMSplit - 1) / kMSplit);
    if (a.out_fmt == CSA_BF16) launch_d<uint16_t>(a, (int)nsplit, st);
    else launch_d<float>(a, (int)nsplit, st);
    return hipGetLastError();
}

}  // namespace csa
