// attn_mfma.hip -- MFMA kernel of csa_sparse_mqa_attn / hca_dense_mqa_attn for
// bf16 queries over bf16 / FP8 caches (gfx950, v_mfma_f32_16x16x32_bf16).
//
// Same method and decomposition as attn.hip (peacm.com section 3.2: MQA over
// the selected compressed entries plus the raw window, Q/KV RMSNorm, partial
// RoPE with the -i output RoPE, sink logit in the denominator), arranged for
// the matrix cores of one CU:
//   - one query row (up to 64 heads) per workgroup and split, eight waves
//     (two per SIMD): wave w takes the 32 heads of half w/4 and the quarter
//     w%4 of the head dimension D.  It holds those queries as MFMA
//     A-fragments and that block of the output as accumulators (64 fp32
//     per lane at D = 512, so everything stays in plain VGPRs);
//   - a tile of 32 entries is shared by all heads (MQA: one KV vector per
//     entry serves every head).  FP8 records are expanded exactly to bf16
//     codes with the hardware OCP-E4M3 conversion; the row scale multiplies
//     the non-RoPE part of the logits and the probabilities used for the
//     non-RoPE output dims (scale * <q, code> = <q, scale * code>);
//   - the partial logits of the four quarters meet in LDS; wave g (< 4) owns
//     16-head group g, adds them in quarter order and runs the online softmax of
//     those heads (base-2 exponentials; the running maximum is raised only
//     when a tile exceeds it by more than a factor 2^8, so the accumulators
//     are rescaled rarely); P goes to LDS entry-major;
//   - P and V reach the MFMA through the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16).  The P V k index runs over the tile's entries in
//     a permuted order chosen so that the rows read together fall in disjoint
//     LDS banks;
//   - records are fetched straight into an LDS staging area with the gfx950
//     global-to-LDS load (global_load_lds_dwordx4), one tile ahead, and
//     expanded into the double-buffered bf16 tile by the wave that fetched
//     them; record addresses are computed one lane per entry and the top-k
//     indices are read two tiles ahead; two barriers per tile.
#include <stddef.h>

#include "common.hpp"
#include "launch.hpp"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kMTE = 32;                  // entries per LDS tile
constexpr int kNW = 8;                    // waves per workgroup
constexpr int kEntPerWave = kMTE / kNW;   // entries of a tile fetched by one wave (slots w + 8u)
constexpr int kPRow = 80;                 // bf16 per P row (64 heads + pad: 160-byte rows)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;          // base-2 headroom before the running max is raised

template <int D>
struct MfmaSmem {
    uint8_t tile[2][kMTE][D * 2 + 16];    // bf16 entries (FP8 codes expanded), double-buffered
    uint8_t raw[kMTE][D * 2];             // records of the next tile as fetched (bf16 records are the largest)
    float scale[2][kMTE];                 // FP8 row scale (1 for bf16 records)
    int valid[2][kMTE];
    float zx[kNW][2][2][64][4];           // partial logits [wave][local head group][n][lane][i]
    uint16_t pt[2][kMTE][kPRow];          // P [scaled, plain] by (k index, head)
    float alpha[64];                      // per-head rescale factor of the current tile
    float fin[64];                        // per-head final factor (single-split rows)
    float ssq[4][64];                     // per-quarter sums of squares of the queries
    int moved[4];                         // per head group: accumulators need rescaling
    double rf[64];                        // RoPE inverse frequencies
};

// ---- per-row entry enumeration (wave-uniform)
struct RowCtx {
    const uint8_t* comp;      // this sequence's compressed records
    const int32_t* top;       // this row's top-k list (null: dense)
    const uint8_t* win;       // this sequence's window ring
    int32_t nc, vis;          // compressed slots, visible blocks
    int32_t slot0;            // ring slot of entry nc (< 0: before the sequence start)
};

__device__ __forceinline__ uint32_t pack_bf16x2(bf16x2_t v) {
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}

// Per-wave fetch state of one tile: lane u < 4 holds the record address of
// the wave's entry u (tile slot w + 8u); the masks say which entries exist
// and which are FP8 records.
struct Fetch {
    uint64_t ptr;         // per lane
    uint32_t vmask, fmask;
};

// index of this lane's entry in the top-k list (lanes 0..3), read ahead of use
__device__ __forceinline__ int32_t fetch_index(const AttnArgs& a, const RowCtx& c, int32_t et, int32_t e1, int w,
                                               int lane) {
    const int32_t e = et + w + kNW * lane;
    int32_t j = 0;
    if (c.top && lane < kEntPerWave && e < e1 && e < c.nc) j = c.top[e];
    return j;
}

// record addresses of the wave's entries of the tile at et (j: fetch_index)
__device__ __forceinline__ Fetch fetch_plan(const AttnArgs& a, const RowCtx& c, int32_t et, int32_t e1, int w,
                                            int lane, int32_t j) {
    const int32_t e = et + w + kNW * lane;
    bool ok = lane < kEntPerWave && e < e1, fp8 = false;
    const uint8_t* p = nullptr;
    if (ok) {
        if (e < c.nc) {
            const int32_t jj = c.top ? j : e;
            ok = jj >= 0 && jj < c.vis;
            p = c.comp + (int64_t)jj * a.comp_rec;
            fp8 = a.comp_fmt == CSA_FP8_E4M3;
        } else {
            int32_t sl = c.slot0 + (e - c.nc);
            ok = sl >= 0;
            if (sl >= a.wcap) sl -= (int32_t)a.wcap;
            p = c.win + (int64_t)sl * a.win_rec;
            fp8 = a.win_fmt == CSA_FP8_E4M3;
        }
    }
    Fetch f;
    f.ptr = (uint64_t)(uintptr_t)p;
    f.vmask = (uint32_t)__ballot(ok);
    f.fmask = (uint32_t)__ballot(ok && fp8);
    return f;
}

// issue the global-to-LDS copies of the wave's records into the staging area
template <int D, int DR>
__device__ __forceinline__ void fetch_issue(MfmaSmem<D>& sm, int w, int lane, const Fetch& f) {
    constexpr int fp8_pieces = (D - DR) / 16 + DR / 8 + 1;
#pragma unroll
    for (int u = 0; u < kEntPerWave; u++) {
        if (f.vmask & (1u << u)) {
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)f.ptr, u);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(f.ptr >> 32), u);
            const uint8_t* rec = (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
            const int npieces = (f.fmask & (1u << u)) ? fp8_pieces : D / 8;
            if (lane < npieces)
                __builtin_amdgcn_global_load_lds(rec + 16 * lane,
                                                 (__attribute__((address_space(3))) void*)&sm.raw[w + kNW * u][0], 16, 0, 0);
        }
    }
}

// expand the wave's fetched records into bf16 tile rows (FP8 codes exactly,
// RoPE dims copied, row scale and validity aside)
template <int D, int DR>
__device__ __forceinline__ void fetch_expand(MfmaSmem<D>& sm, int buf, int w, int lane, const Fetch& f) {
    constexpr int dn = D - DR;
#pragma unroll
    for (int u = 0; u < kEntPerWave; u++) {
        const int ee = w + kNW * u;
        uint8_t* dst = sm.tile[buf][ee];
        const uint8_t* src = sm.raw[ee];
        if (!(f.vmask & (1u << u))) {
            // masked entry: a zero row keeps 0 * garbage out of P V
            if (lane < D / 8) *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
            if (lane == 0) sm.scale[buf][ee] = 1.0f;
        } else if (f.fmask & (1u << u)) {
            if (lane < dn / 8) {
                const uint2 cd = *reinterpret_cast<const uint2*>(src + 8 * lane);
                uint4 o;
                o.x = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cd.x, 1.0f, false));
                o.y = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cd.x, 1.0f, true));
                o.z = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cd.y, 1.0f, false));
                o.w = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cd.y, 1.0f, true));
                *reinterpret_cast<uint4*>(dst + 16 * lane) = o;
            } else if (lane < dn / 8 + DR / 8) {
                const int q = lane - dn / 8;
                *reinterpret_cast<uint4*>(dst + 2 * dn + 16 * q) = *reinterpret_cast<const uint4*>(src + dn + 16 * q);
            }
            if (lane == 0) sm.scale[buf][ee] = *reinterpret_cast<const float*>(src + dn + 2 * DR);
        } else {
            if (lane < D / 8) *reinterpret_cast<uint4*>(dst + 16 * lane) = *reinterpret_cast<const uint4*>(src + 16 * lane);
            if (lane == 0) sm.scale[buf][ee] = 1.0f;
        }
        if (lane == 0) sm.valid[buf][ee] = (f.vmask >> u) & 1u;
    }
}

// wait for this wave's global-to-LDS copies (vmcnt 0), and for its LDS reads
// before the staging area is refilled (lgkmcnt 0)
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// gfx950 transposing LDS read of four bf16 (ds_read_b64_tr_b16).  Within each
// 16-lane group, lane s points at 4 consecutive bf16; lane i then receives,
// for j = 0..3, element i%4 of the 4 values addressed by lane i/4 + 4j.
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* p) {
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// eight bf16 from two transposing reads (one vector reinterpretation: element
// by element casts of the 16-bit lanes have been lowered incorrectly)
__device__ __forceinline__ bf16x8_t tr_pair(const void* p0, const void* p1) {
    const s16x4_t v0 = lds_read_tr16(p0), v1 = lds_read_tr16(p1);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// position of tile entry e in the P V k order: k = 8g + 4h + j holds entry
// 8g + h + 2j, so the four V rows one transposing read covers are two apart
// (row pitch = 4 banks mod 32: offsets 0, 8, 16, 24 banks)
__device__ __forceinline__ int pv_k_of_entry(int e) { return (e & ~7) + 4 * (e & 1) + ((e & 7) >> 1); }

// all-reduce over the 16 lanes of a DPP row (rotations, then quad swaps);
// commutative steps give every lane the same bits
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0x128>(v));     // row_ror:8
    v = fmaxf(v, dpp_f<0x124>(v));     // row_ror:4
    v = fmaxf(v, dpp_f<0x4E>(v));      // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0xB1>(v));      // quad_perm [1,0,3,2]
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v = v + dpp_f<0x128>(v);
    v = v + dpp_f<0x124>(v);
    v = v + dpp_f<0x4E>(v);
    v = v + dpp_f<0xB1>(v);
    return v;
}

template <int D, int DR, typename OT>
__global__ __launch_bounds__(kNW * 64) void k_attn_mfma(AttnArgs a, int nsplit_max) {
    constexpr int DQ = D / 4;              // dims per quarter
    constexpr int KS = DQ / 32;            // Q K^T K-steps per wave
    constexpr int NT = DQ / 16;            // P V N-tiles per wave
    constexpr int dn = D - DR;             // non-RoPE dims (multiple of 32)
    constexpr int RS = D * 2 + 16;         // tile row stride in bytes
    __shared__ MfmaSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qd = w & 3, hp = w >> 2;                 // dim quarter, head half
    const int l16 = lane & 15, g4 = lane >> 4;
    const int row = blockIdx.y;
    const int b = row / a.Tq;
    const int t = a.q_pos[row];
    RowCtx c;
    c.vis = t < 0 ? 0 : (t + 1) / a.m;
    if (c.vis > a.ccap) c.vis = (int32_t)a.ccap;
    c.nc = a.topk ? a.k : c.vis;
    c.comp = a.comp + (int64_t)b * a.ccap * a.comp_rec;
    c.top = a.topk ? a.topk + (int64_t)row * a.k : nullptr;
    c.win = a.win + (int64_t)b * a.wcap * a.win_rec;
    {
        const int32_t s0 = t - a.W + 1;
        c.slot0 = (a.W > 0 && s0 >= 0) ? s0 % (int32_t)a.wcap : s0;
    }
    const int32_t ne = c.nc + a.W;
    const int32_t split = attn_split_len<int32_t>(ne, a.Tq);
    const int32_t nsplit = attn_nsplit<int32_t>(ne, a.Tq);
    const int32_t sp = blockIdx.x;
    if (sp >= nsplit) return;
    const int32_t e0 = sp * split, e1 = min(e0 + split, ne);
    const int h0 = blockIdx.z * 64;
    const int MT = min(4, (a.H - h0) / 16);           // 16-head groups in this workgroup
    const bool active = 2 * hp < MT;                   // this wave's head half exists
    const bool owner = w < MT;                         // wave w runs the softmax of head group w
    const int dbase = qd * DQ;                         // first dim of this wave's quarter
    // non-RoPE K-steps / N-tiles of this quarter
    const int nks = max(0, min(KS, (dn - dbase) / 32));
    const int nnt = max(0, min(NT, (dn - dbase) / 16));
    const float zscale = a.scale * kLog2e;             // logits in base-2 units

    // the first tile's records go out before the query prologue; the top-k
    // indices are read two tiles ahead of their records
    Fetch fr = fetch_plan(a, c, e0, e1, w, lane, fetch_index(a, c, e0, e1, w, lane));
    fetch_issue<D, DR>(sm, w, lane, fr);
    int32_t jn = fetch_index(a, c, e0 + kMTE, e1, w, lane);
    {
        // RoPE inverse frequencies, read lane-parallel from the argument block
        const double* rtab = (const double*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(AttnArgs, rope));
        if (tid < a.dr / 2) sm.rf[tid] = rtab[tid];
    }

    // ---- query prologue: q^ = RoPE_t(RMSNorm(q)), this wave's 32 heads and quarter
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)row * a.H + h0 + 32 * hp) * D;
    uint4 qraw[2][KS];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            qraw[mt][ks] = make_uint4(0u, 0u, 0u, 0u);
            if (2 * hp + mt < MT)
                qraw[mt][ks] = *reinterpret_cast<const uint4*>(qb + (16 * mt + l16) * D + dbase + 32 * ks + 8 * g4);
        }
    float4 gam[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        gam[ks][0] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        gam[ks][1] = gam[ks][0];
        if (a.gamma_q) {
            const float4* gp = reinterpret_cast<const float4*>(a.gamma_q + dbase + 32 * ks + 8 * g4);
            gam[ks][0] = gp[0];
            gam[ks][1] = gp[1];
        }
    }
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const uint32_t wd[4] = {qraw[mt][ks].x, qraw[mt][ks].y, qraw[mt][ks].z, qraw[mt][ks].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x0 = __uint_as_float(wd[j] << 16), x1 = __uint_as_float(wd[j] & 0xFFFF0000u);
                ss += x0 * x0 + x1 * x1;
            }
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        if (g4 == 0) sm.ssq[qd][32 * hp + 16 * mt + l16] = ss;
    }
    __syncthreads();
    float inv[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        const int hl = 32 * hp + 16 * mt + l16;
        const float ss = ((sm.ssq[0][hl] + sm.ssq[1][hl]) + sm.ssq[2][hl]) + sm.ssq[3][hl];
        inv[mt] = 1.0f / sqrtf(ss / (float)D + a.eps);
    }
    bf16x8_t qf[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const float gv[8] = {gam[ks][0].x, gam[ks][0].y, gam[ks][0].z, gam[ks][0].w,
                             gam[ks][1].x, gam[ks][1].y, gam[ks][1].z, gam[ks][1].w};
        float sn[4], cs[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            sn[j] = 0.0f;
            cs[j] = 1.0f;
        }
        if (ks >= nks) {
#pragma unroll
            for (int j = 0; j < 4; j++)
                rope_sincos((double)t, sm.rf[(dbase + 32 * ks + 8 * g4 + 2 * j - dn) / 2], sn[j], cs[j]);
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            const uint32_t wd[4] = {qraw[mt][ks].x, qraw[mt][ks].y, qraw[mt][ks].z, qraw[mt][ks].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x0 = __uint_as_float(wd[j] << 16) * inv[mt] * gv[2 * j];
                const float x1 = __uint_as_float(wd[j] & 0xFFFF0000u) * inv[mt] * gv[2 * j + 1];
                qf[mt][ks][2 * j] = (__bf16)(x0 * cs[j] - x1 * sn[j]);
                qf[mt][ks][2 * j + 1] = (__bf16)(x0 * sn[j] + x1 * cs[j]);
            }
        }
    }

    // P rows of a head group beyond MT are never written: its accumulators
    // collect garbage and are never stored
    f32x4_t o[2][NT];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nd = 0; nd < NT; nd++) o[mt][nd] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // running max (base 2) / sum of the owned heads 16w + 4*g4 + i
    float mrun[4], lrun[4];
#pragma unroll
    for (int i = 0; i < 4; i++) { mrun[i] = -INFINITY; lrun[i] = 0.0f; }

    wait_vm();
    fetch_expand<D, DR>(sm, 0, w, lane, fr);
    wait_lgkm();
    if (e0 + kMTE < e1) {
        fr = fetch_plan(a, c, e0 + kMTE, e1, w, lane, jn);
        fetch_issue<D, DR>(sm, w, lane, fr);
        jn = fetch_index(a, c, e0 + 2 * kMTE, e1, w, lane);
    }
    __syncthreads();
    // per-lane LDS coordinates of the transposing reads
    const int v_row = 8 * g4 + 2 * (l16 >> 2);
    const int v_col = 2 * (dbase + 4 * (l16 & 3));
    const int p_row = 8 * g4 + (l16 >> 2);
    const int p_col = 32 * hp + 4 * (l16 & 3);
    int buf = 0;
    for (int32_t et = e0; et < e1; et += kMTE, buf ^= 1) {
        // ---- partial logits of this quarter for the wave's head groups, to LDS:
        // scale * <q, code>_non-RoPE + <q, k>_RoPE
        if (active) {
#pragma unroll
            for (int n = 0; n < 2; n++) {
                const float esc = sm.scale[buf][16 * n + l16];
                f32x4_t acc[2];
#pragma unroll
                for (int mt = 0; mt < 2; mt++) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                const uint8_t* kr = &sm.tile[buf][16 * n + l16][2 * dbase + 16 * g4];
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const bf16x8_t kb = *reinterpret_cast<const bf16x8_t*>(kr + 64 * ks);
                    if (ks == nks && ks > 0) {
#pragma unroll
                        for (int mt = 0; mt < 2; mt++) acc[mt] *= esc;
                    }
#pragma unroll
                    for (int mt = 0; mt < 2; mt++)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[mt][ks], kb, acc[mt], 0, 0, 0);
                }
                if (nks == KS) {
#pragma unroll
                    for (int mt = 0; mt < 2; mt++) acc[mt] *= esc;
                }
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
                    *reinterpret_cast<f32x4_t*>(&sm.zx[w][mt][n][lane][0]) = acc[mt];
            }
        }
        __syncthreads();
        // ---- expand the next tile into the other buffer (last read by P V of
        // the previous tile, which every wave finished before the barrier),
        // then refill the staging area with the tile after it
        if (et + kMTE < e1) {
            wait_vm();
            fetch_expand<D, DR>(sm, buf ^ 1, w, lane, fr);
            wait_lgkm();
            if (et + 2 * kMTE < e1) {
                fr = fetch_plan(a, c, et + 2 * kMTE, e1, w, lane, jn);
                fetch_issue<D, DR>(sm, w, lane, fr);
                jn = fetch_index(a, c, et + 3 * kMTE, e1, w, lane);
            }
        }
        // ---- owner waves: add the quarters in order, online softmax, publish P
        if (owner) {
            float esc[2];
            bool eok[2];
#pragma unroll
            for (int n = 0; n < 2; n++) {
                esc[n] = sm.scale[buf][16 * n + l16];
                eok[n] = sm.valid[buf][16 * n + l16] != 0;
            }
            const int src = 4 * (w >> 1), lg = w & 1;    // waves holding this group's quarters
            f32x4_t z[2];
#pragma unroll
            for (int n = 0; n < 2; n++) {
                z[n] = *reinterpret_cast<const f32x4_t*>(&sm.zx[src][lg][n][lane][0]);
#pragma unroll
                for (int q = 1; q < 4; q++) z[n] += *reinterpret_cast<const f32x4_t*>(&sm.zx[src + q][lg][n][lane][0]);
            }
            bool moved = false;
            float pz[2][4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float zz[2];
#pragma unroll
                for (int n = 0; n < 2; n++) zz[n] = eok[n] ? z[n][i] * zscale : -INFINITY;
                const float mx = row16_max(fmaxf(zz[0], zz[1]));
                float mn = mrun[i], al = 1.0f;
                if (mx > mrun[i] + kLazyMax) {           // also the first finite maximum
                    mn = mx;
                    al = exp2f(mrun[i] - mx);            // 0 when mrun was -inf (O and l are 0)
                    moved |= mrun[i] != -INFINITY;
                }
#pragma unroll
                for (int n = 0; n < 2; n++) pz[n][i] = mn == -INFINITY ? 0.0f : exp2f(zz[n] - mn);
                const float rs = row16_sum(pz[0][i] + pz[1][i]);
                lrun[i] = lrun[i] * al + rs;
                mrun[i] = mn;
                if (l16 == 0) sm.alpha[16 * w + 4 * g4 + i] = al;
            }
            const bool any_moved = __any(moved);
            if (lane == 0) sm.moved[w] = any_moved ? 1 : 0;
#pragma unroll
            for (int n = 0; n < 2; n++) {
                const int kk = pv_k_of_entry(16 * n + l16);
                uint2 ps, pp;
                ps.x = pack_bf16x2(bf16x2_t{(__bf16)(pz[n][0] * esc[n]), (__bf16)(pz[n][1] * esc[n])});
                ps.y = pack_bf16x2(bf16x2_t{(__bf16)(pz[n][2] * esc[n]), (__bf16)(pz[n][3] * esc[n])});
                pp.x = pack_bf16x2(bf16x2_t{(__bf16)pz[n][0], (__bf16)pz[n][1]});
                pp.y = pack_bf16x2(bf16x2_t{(__bf16)pz[n][2], (__bf16)pz[n][3]});
                *reinterpret_cast<uint2*>(&sm.pt[0][kk][16 * w + 4 * g4]) = ps;
                *reinterpret_cast<uint2*>(&sm.pt[1][kk][16 * w + 4 * g4]) = pp;
            }
        }
        __syncthreads();
        if (active) {
            // ---- rescale O of the head groups whose max moved (rare), then O += P V
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                const int g = 2 * hp + mt;
                if (g < MT && sm.moved[g]) {
                    const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[16 * g + 4 * g4]);
#pragma unroll
                    for (int nd = 0; nd < NT; nd++) {
                        o[mt][nd][0] *= al.x;
                        o[mt][nd][1] *= al.y;
                        o[mt][nd][2] *= al.z;
                        o[mt][nd][3] *= al.w;
                    }
                }
            }
            // P A-fragments: scaled P for the non-RoPE dims, plain P for the RoPE dims
            bf16x8_t pf[2];
            {
                const int pa = nnt > 0 ? 0 : 1;
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
                    pf[mt] = tr_pair(&sm.pt[pa][p_row][16 * mt + p_col], &sm.pt[pa][p_row + 4][16 * mt + p_col]);
            }
            const uint8_t* vp = &sm.tile[buf][v_row][v_col];
#pragma unroll
            for (int nd = 0; nd < NT; nd++) {
                if (nd == nnt && nd > 0) {
#pragma unroll
                    for (int mt = 0; mt < 2; mt++)
                        pf[mt] = tr_pair(&sm.pt[1][p_row][16 * mt + p_col], &sm.pt[1][p_row + 4][16 * mt + p_col]);
                }
                const bf16x8_t vb = tr_pair(vp + 32 * nd, vp + RS + 32 * nd);
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
                    o[mt][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[mt], vb, o[mt][nd], 0, 0, 0);
            }
        }
    }

    // ---- epilogue
    if (nsplit <= 1) {
        if (owner) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int hr = 16 * w + 4 * g4 + i;
                const float sk = a.sink[h0 + hr] * kLog2e, mr = mrun[i];
                const float M = fmaxf(mr, sk);
                float f = 0.0f;
                if (mr != -INFINITY && M != -INFINITY) {
                    const float em = exp2f(mr - M);
                    f = em / (lrun[i] * em + exp2f(sk - M));
                }
                if (l16 == 0) sm.fin[hr] = f;
            }
        }
        __syncthreads();
        if (!active) return;
        OT* out = reinterpret_cast<OT*>(a.out) + ((int64_t)row * a.H + h0) * D;
#pragma unroll
        for (int nd = 0; nd < NT; nd++) {
            const int dim = dbase + 16 * nd + l16;
            const bool rope = nd >= nnt;
            float sn = 0.0f, cs = 1.0f;
            if (rope) rope_sincos(-(double)t, sm.rf[(dim - dn) / 2], sn, cs);
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                const int g = 2 * hp + mt;
                if (g < MT) {
                    const float4 f = *reinterpret_cast<const float4*>(&sm.fin[16 * g + 4 * g4]);
                    const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        float v = o[mt][nd][i] * fv[i];
                        if (rope) {
                            const float pv = __shfl_xor(v, 1, kWave);
                            v = (dim & 1) ? pv * sn + v * cs : v * cs - pv * sn;
                        }
                        st_scalar<OT>(out, (size_t)(16 * g + 4 * g4 + i) * D + dim, v);
                    }
                }
            }
        }
        return;
    }
    // partial results of this split: unnormalised O, and (max, sum) in natural-log units
    float* wo = reinterpret_cast<float*>(a.ws);
    float* wml = wo + (size_t)a.rows * nsplit_max * a.H * D;
    const size_t base = ((size_t)row * nsplit_max + sp) * a.H + h0;
    if (active) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
            if (2 * hp + mt < MT)
#pragma unroll
                for (int nd = 0; nd < NT; nd++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        wo[(base + 16 * (2 * hp + mt) + 4 * g4 + i) * D + dbase + 16 * nd + l16] = o[mt][nd][i];
    }
    if (owner && l16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const size_t hr = base + 16 * w + 4 * g4 + i;
            wml[hr * 2] = mrun[i] * kLn2;
            wml[hr * 2 + 1] = lrun[i];
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
    // eight waves per workgroup always (head halves x dim quarters); a
    // workgroup covers up to 64 heads
    if (a.d == 128) hipLaunchKernelGGL((k_attn_mfma<128, 64, OT>), grid, dim3(kNW * 64), 0, st, a, nsplit);
    else if (a.d == 256) hipLaunchKernelGGL((k_attn_mfma<256, 64, OT>), grid, dim3(kNW * 64), 0, st, a, nsplit);
    else hipLaunchKernelGGL((k_attn_mfma<512, 64, OT>), grid, dim3(kNW * 64), 0, st, a, nsplit);
}

hipError_t launch_attention_mfma(const AttnArgs& a, int64_t nsplit_bound, hipStream_t st) {
    if (a.out_fmt == CSA_BF16) launch_d<uint16_t>(a, (int)nsplit_bound, st);
    else launch_d<float>(a, (int)nsplit_bound, st);
    return hipGetLastError();
}

}  // namespace csa
