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
//     bf16 with the hardware OCP-E4M3 conversion, their per-row scale kept
//     aside and applied to the logits of the non-RoPE part and to the
//     probabilities of the non-RoPE output dims (exactly the decoded value,
//     since scale * <q, code> = <q, scale * code>);
//   - the tile loop is software-pipelined: each wave loads the raw records of
//     its 8 entries of tile t+1 into registers (16-byte pieces, one lane per
//     piece) while tile t is computed, so HBM latency overlaps the MFMAs;
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

constexpr int kMTE = 32;                  // entries per LDS tile
constexpr int kPStride = kMTE + 8;
constexpr int kEntPerWave = kMTE / 4;     // entries of a tile staged by one wave (4 waves per workgroup)

template <int D>
struct MfmaSmem {
    uint8_t tile[kMTE][D * 2 + 16];       // bf16 entries, rows padded by 16 bytes
    float scale[kMTE];                    // FP8 row scale (1 for bf16 records)
    int valid[kMTE];
    uint16_t p[4][2][16][kPStride];       // per wave: [scaled, plain] P, 16 heads x 32 entries
    double rf[64];                        // RoPE inverse frequencies
};

// record of entry e of a row (nullptr if masked); same enumeration as attn.hip
__device__ __forceinline__ const uint8_t* mfma_entry_rec(const AttnArgs& a, int64_t row, int64_t b, int64_t t,
                                                         int64_t nc, int64_t vis, int64_t e, int& fmt) {
    if (e < nc) {
        int64_t j = e;
        if (a.topk) {
            j = a.topk[row * a.k + e];
            if (j < 0 || j >= vis) return nullptr;
        }
        fmt = a.comp_fmt;
        return a.comp + (b * a.ccap + j) * a.comp_rec;
    }
    const int64_t s = t - a.W + 1 + (e - nc);
    if (s < 0) return nullptr;
    fmt = a.win_fmt;
    return a.win + (b * a.wcap + s % a.wcap) * a.win_rec;
}

__device__ __forceinline__ uint32_t pack_bf16x2(bf16x2_t v) {
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}

// raw 16-byte pieces of one wave's entries of a tile, one piece per lane.
// FP8 records: pieces 0 .. dn/16-1 hold 16 E4M3 codes, the next DR/8 the bf16
// RoPE dims, the next one the row scale; bf16 records: D/8 pieces of 8 dims.
struct TileRegs {
    uint4 piece[kEntPerWave];
    const uint8_t* rec[kEntPerWave];
    int fmt[kEntPerWave];
};

template <int D, int DR>
__device__ __forceinline__ void tile_load(const AttnArgs& a, int64_t row, int64_t b, int64_t t, int64_t nc,
                                          int64_t vis, int64_t et, int64_t e1, int w, int lane, TileRegs& R) {
    constexpr int fp8_pieces = (D - DR) / 16 + DR / 8 + 1;
#pragma unroll
    for (int u = 0; u < kEntPerWave; u++) {
        const int64_t e = et + w + 4 * u;
        int fmt = 0;
        const uint8_t* r = e < e1 ? mfma_entry_rec(a, row, b, t, nc, vis, e, fmt) : nullptr;
        R.rec[u] = r;
        R.fmt[u] = fmt;
        R.piece[u] = make_uint4(0u, 0u, 0u, 0u);
        if (r) {
            const int npieces = fmt == CSA_FP8_E4M3 ? fp8_pieces : D / 8;
            if (lane < npieces) R.piece[u] = *reinterpret_cast<const uint4*>(r + 16 * lane);
        }
    }
}

template <int D, int DR>
__device__ __forceinline__ void tile_store(MfmaSmem<D>& sm, int w, int lane, const TileRegs& R) {
    constexpr int dn = D - DR;
#pragma unroll
    for (int u = 0; u < kEntPerWave; u++) {
        const int ee = w + 4 * u;
        uint8_t* dst = sm.tile[ee];
        const uint4 pc = R.piece[u];
        if (!R.rec[u]) {
            // masked entry: a zero row keeps 0 * garbage out of P V
            if (lane < D / 8) *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
            if (lane == 0) {
                sm.scale[ee] = 1.0f;
                sm.valid[ee] = 0;
            }
        } else if (R.fmt[u] == CSA_FP8_E4M3) {
            if (lane < dn / 16) {
                uint4 lo, hi;
                lo.x = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.x, 1.0f, false));
                lo.y = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.x, 1.0f, true));
                lo.z = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.y, 1.0f, false));
                lo.w = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.y, 1.0f, true));
                hi.x = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.z, 1.0f, false));
                hi.y = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.z, 1.0f, true));
                hi.z = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.w, 1.0f, false));
                hi.w = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc.w, 1.0f, true));
                *reinterpret_cast<uint4*>(dst + 32 * lane) = lo;
                *reinterpret_cast<uint4*>(dst + 32 * lane + 16) = hi;
            } else if (lane < dn / 16 + DR / 8) {
                *reinterpret_cast<uint4*>(dst + 2 * dn + 16 * (lane - dn / 16)) = pc;
            } else if (lane == dn / 16 + DR / 8) {
                sm.scale[ee] = __uint_as_float(pc.x);
                sm.valid[ee] = 1;
            }
        } else {
            if (lane < D / 8) *reinterpret_cast<uint4*>(dst + 16 * lane) = pc;
            if (lane == 0) {
                sm.scale[ee] = 1.0f;
                sm.valid[ee] = 1;
            }
        }
    }
}

template <int D, int DR, typename OT>
__global__ __launch_bounds__(256) void k_attn_mfma(AttnArgs a, int nsplit_max) {
    constexpr int NS = D / 32;   // QK K-steps
    constexpr int ND = D / 16;   // PV N-tiles
    constexpr int dn = D - DR;   // non-RoPE dims (multiple of 32)
    constexpr int nsr = dn / 32, ndr = dn / 16;
    __shared__ MfmaSmem<D> sm;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t row = blockIdx.y, b = row / a.Tq;
    const int64_t t = a.q_pos[row];
    int64_t vis = t < 0 ? 0 : (t + 1) / a.m;
    if (vis > a.ccap) vis = a.ccap;
    const int64_t nc = a.topk ? a.k : vis;
    const int64_t ne = nc + a.W;
    const int64_t split = attn_split_len(ne, a.Tq);
    const int64_t nsplit = attn_nsplit(ne, a.Tq);
    const int64_t sp = blockIdx.x;
    if (sp >= nsplit) return;
    const int64_t e0 = sp * split, e1 = min(e0 + split, ne);
    const int hw = blockIdx.z * 64 + 16 * w;          // first head of this wave
    const bool active = hw < a.H;

    // the first tile's loads go out before the query prologue
    TileRegs R;
    tile_load<D, DR>(a, row, b, t, nc, vis, e0, e1, w, lane, R);

    stage_rope(a.rope, sm.rf, a.dr / 2);
    __syncthreads();
    // ---- query prologue: q^ = RoPE_t(RMSNorm(q)) as bf16 A-fragments
    bf16x8_t qf[NS];
    if (active) {
        // two passes over this lane's 16-byte chunks of its head row: the sum of
        // squares, then scale, rotate and round (no large private array)
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (row * a.H + hw + l16) * D;
        float ss = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g4);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x0 = __uint_as_float(wd[j] << 16), x1 = __uint_as_float(wd[j] & 0xFFFF0000u);
                ss += x0 * x0 + x1 * x1;
            }
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
        // non-RoPE steps, then the RoPE steps (kept apart so both loops unroll)
#pragma unroll
        for (int s = 0; s < nsr; s++) {
            const uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g4);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int dim = 32 * s + 8 * g4 + 2 * j;
                float x0 = __uint_as_float(wd[j] << 16) * inv, x1 = __uint_as_float(wd[j] & 0xFFFF0000u) * inv;
                if (a.gamma_q) {
                    x0 *= a.gamma_q[dim];
                    x1 *= a.gamma_q[dim + 1];
                }
                qf[s][2 * j] = (__bf16)x0;
                qf[s][2 * j + 1] = (__bf16)x1;
            }
        }
#pragma unroll
        for (int s = nsr; s < NS; s++) {
            const uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * g4);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int dim = 32 * s + 8 * g4 + 2 * j;
                float x0 = __uint_as_float(wd[j] << 16) * inv, x1 = __uint_as_float(wd[j] & 0xFFFF0000u) * inv;
                if (a.gamma_q) {
                    x0 *= a.gamma_q[dim];
                    x1 *= a.gamma_q[dim + 1];
                }
                float sn, cs;
                rope_sincos((double)t, sm.rf[(dim - dn) / 2], sn, cs);
                qf[s][2 * j] = (__bf16)(x0 * cs - x1 * sn);
                qf[s][2 * j + 1] = (__bf16)(x0 * sn + x1 * cs);
            }
        }
    }

    f32x4_t o[ND];
#pragma unroll
    for (int nd = 0; nd < ND; nd++) o[nd] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun[4], lrun[4];
#pragma unroll
    for (int i = 0; i < 4; i++) { mrun[i] = -INFINITY; lrun[i] = 0.0f; }

    for (int64_t et = e0; et < e1; et += kMTE) {
        __syncthreads();                                   // previous tile consumed
        tile_store<D, DR>(sm, w, lane, R);
        __syncthreads();
        // the next tile's loads are issued after the barrier (whose fence would
        // otherwise wait for them) and complete while this tile is computed
        if (et + kMTE < e1) tile_load<D, DR>(a, row, b, t, nc, vis, et + kMTE, e1, w, lane, R);
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
                if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
        // ---- online softmax (rows = heads 4*g4 + i; this lane's entries 16n + l16)
        float pz[2][4];
        float alpha[4];
        bool moved = false;
        float esc[2];
        int eok[2];
#pragma unroll
        for (int n = 0; n < 2; n++) {
            esc[n] = sm.scale[16 * n + l16];
            eok[n] = sm.valid[16 * n + l16];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float mt = -INFINITY;
#pragma unroll
            for (int n = 0; n < 2; n++) {
                const float z = eok[n] ? a.scale * (esc[n] * snr[n][i] + sr[n][i]) : -INFINITY;
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
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const __bf16 ps = (__bf16)(pz[n][i] * esc[n]), pp = (__bf16)pz[n][i];
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
            if (nd % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bound the B-fragments kept in flight
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
            if (nd >= ndr) rope_sincos(-(double)t, sm.rf[(dim - dn) / 2], sn, cs);
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
    if (a.dr != 64) return false;
    return true;
}

template <typename OT>
static void launch_d(const AttnArgs& a, int nsplit, hipStream_t st) {
    const int groups = (a.H + 63) / 64;
    dim3 grid((unsigned)nsplit, (unsigned)a.rows, (unsigned)groups);
    // four waves per workgroup always (tile staging is spread over four waves);
    // waves beyond H stage but do not compute
    if (a.d == 128) hipLaunchKernelGGL((k_attn_mfma<128, 64, OT>), grid, dim3(256), 0, st, a, nsplit);
    else if (a.d == 256) hipLaunchKernelGGL((k_attn_mfma<256, 64, OT>), grid, dim3(256), 0, st, a, nsplit);
    else hipLaunchKernelGGL((k_attn_mfma<512, 64, OT>), grid, dim3(256), 0, st, a, nsplit);
}

hipError_t launch_attention_mfma(const AttnArgs& a, int64_t nsplit_bound, hipStream_t st) {
    if (a.out_fmt == CSA_BF16) launch_d<uint16_t>(a, (int)nsplit_bound, st);
    else launch_d<float>(a, (int)nsplit_bound, st);
    return hipGetLastError();
}

}  // namespace csa
