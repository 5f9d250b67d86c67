"""GPU parity of the projections with FP8 weights and of a CSA layer run
from its hidden states (MI355X only).

  - csa_linear_fp8: every E4M3 code through identity activations (exact, in
    both kernels), ragged shapes of both kernels against the oracle within
    the fp32 summation bound, rows independent of the other rows within a
    size class, the grouped output projection at the 1M-decode shape;
  - csa_layer_in_proj: on exact inputs (grid activations, power-of-two
    weights: every fp32 sum exact) every output equals the oracle's bit for
    bit, FP4 queries included; on general inputs within the summation bound
    (queries within one FP4 code);
  - a CSA layer from hidden states (input projections, compression of the
    projected tokens, FP4 indexer, sparse attention, FP8 output projection)
    at a 2,048-token prefill and at a 4-sequence decode step with the 1M
    model widths: top-k sets bit for bit, attention and output within the
    bf16 bounds.

Error bound of an fp32 sum of K products: |got - exact| <= gamma_K * sum |x w|
with gamma_K = K u / (1 - K u), u = 2^-24 (any summation order); a bf16
output adds half an ulp of the value (2^-9 relative).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from helpers import BF16_NORM_REL, abs_err, dev, dev_bf16, host_bf16_bits, norm_rel, out_to_f64, report, say
from long_context_attention_23_amd import api, synth

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def gamma(K):
    return K * U32 / (1 - K * U32)


def abs_products(x, W, s, G=1):
    """sum_c |x w| * s per output (the scale of the summation error)."""
    return O.linear_fp8(np.abs(x), W & 0x7F, s, G=G)


def as_bf16_values(bits):
    return O.bf16_decode(bits)


def run_linear(x_bits, W, s, G, y_dtype):
    y = api.linear_fp8(dev_bf16(x_bits), dev(W), dev(s), G=G, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return out_to_f64(y)


# ---------------------------------------------------------------------- codes
@pytest.mark.parametrize("M", [16, 64, 256])
def test_every_e4m3_code_through_identity(M):
    """Row r of x = e_r picks weight column r: y[r][n] = scale[n] * e4m3(W[n][r]);
    M = 16 and 64 take the weight-stream kernel, 256 the tiled GEMM."""
    K = 256
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0                                         # the NaN codes
    W = np.stack([np.roll(codes, 16 * n) for n in range(48)])       # every code in the first 16 columns
    s = np.array([2.0 ** (n % 7 - 3) for n in range(48)], np.float32)
    eye = np.zeros((M, K), np.float32)
    eye[np.arange(M), np.arange(M)] = 1.0
    xb = (eye.view(np.uint32) >> 16).astype(np.uint16)
    say(f"linear_fp8 identity M={M}")
    got = run_linear(xb, W, s, 1, torch.float32)
    ref = O.linear_fp8(eye.astype(np.float64), W, s)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------- shapes
LIN_CASES = [
    # M, K, N, G
    (1, 64, 16, 1),
    (3, 128, 40, 1),          # ragged column block
    (16, 1024, 1476, 1),      # C1-width input projection
    (17, 512, 200, 1),
    (33, 256, 70, 2),
    (64, 1024, 1000, 8),
    (65, 512, 130, 1),        # first row count of the tiled kernel; ragged column tile
    (300, 1024, 260, 4),      # ragged row tile
    (513, 128, 128, 1),
]


@pytest.mark.parametrize("case", LIN_CASES, ids=[f"M{c[0]}_K{c[1]}_N{c[2]}_G{c[3]}" for c in LIN_CASES])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_fp8_parity(case, out):
    M, K, N, G = case
    g = synth.rng(3100 + M + K + N + G)
    xb = synth.bf16_bits(g, (M, K))
    W = synth.e4m3_codes(g, (N, K // G))
    s = (np.abs(synth.normal(g, N)) * np.float32(1e-3) + np.float32(1e-4)).astype(np.float32)
    say(f"linear_fp8 M={M} K={K} N={N} G={G} out={out}")
    got = run_linear(xb, W, s, G, torch.float32 if out == "f32" else torch.bfloat16)
    x = as_bf16_values(xb)
    ref = O.linear_fp8(x, W, s, G=G)
    bound = gamma(K // G) * abs_products(x, W, s, G) * (1 + 1e-6) + 1e-30
    if out == "bf16":
        bound = bound + np.abs(ref) * 2.0 ** -8
    report(f"linear_fp8 {case} {out}", abs=abs_err(got, ref), norm_rel=norm_rel(got, ref))
    assert np.all(np.abs(got - ref) <= bound)


def test_linear_fp8_rows_independent_of_batch():
    """A row's bits depend only on the row, the weights and M's size class
    (M <= 32, M <= 64, larger): rows of one call equal the same rows computed
    in other calls of the same class, for a small and a large grid."""
    g = synth.rng(3150)
    xb = synth.bf16_bits(g, (300, 1024))
    for K, N in ((1024, 96), (1024, 20000)):
        W = synth.e4m3_codes(g, (N, K))
        s = np.full(N, 1e-3, np.float32)
        ref32 = run_linear(xb[:32], W, s, 1, torch.float32)
        for M in (1, 5, 17):
            assert np.array_equal(run_linear(xb[:M], W, s, 1, torch.float32), ref32[:M]), (N, M)
        ref64 = run_linear(xb[:64], W, s, 1, torch.float32)
        for M in (33, 50):
            assert np.array_equal(run_linear(xb[:M], W, s, 1, torch.float32), ref64[:M]), (N, M)
    full_big = run_linear(xb, W, s, 1, torch.float32)
    for lo, hi in ((0, 65), (100, 300), (37, 290)):
        assert np.array_equal(run_linear(np.ascontiguousarray(xb[lo:hi]), W, s, 1, torch.float32), full_big[lo:hi])


def test_fp8_output_projection_c4_shape():
    """The grouped output projection with FP8 weights at the 1M-decode shape:
    4 rows, 64 heads x 512 -> 7168 in 8 groups (W [7168][4096] codes)."""
    g = synth.rng(3160)
    M, K, N, G = 4, 32768, 7168, 8
    xb = synth.bf16_bits(g, (M, K), std=0.05)
    W = synth.e4m3_codes(g, (N, K // G))
    s = np.full(N, 0.02 / 64 / math.sqrt(K // G), np.float32)
    say("fp8 output projection C4 shape")
    got = run_linear(xb, W, s, G, torch.float32)
    x = as_bf16_values(xb)
    ref = O.linear_fp8(x, W, s, G=G)
    report("fp8 out proj c4", abs=abs_err(got, ref), norm_rel=norm_rel(got, ref))
    assert np.all(np.abs(got - ref) <= gamma(K // G) * abs_products(x, W, s, G) * (1 + 1e-6))


# ---------------------------------------------------------------------- input projections
def in_proj_weights(g, D, H, d, di, Hi, exact):
    """The five weight matrices (codes, scales).  exact: power-of-two codes
    and scales; the indexer head weights read only hidden dimension 0, which
    the exact tests hold at 1, so every head weight is a power of two and the
    indexer's weighted sums stay exact downstream."""
    mats = {}
    for name, n in (("q", H * d), ("kv", d), ("kI", di), ("qI", Hi * di), ("w", Hi)):
        if exact:
            W = synth.e4m3_pow2_codes(g, (n, D))
            if name == "w":
                W = np.zeros((n, D), np.uint8)
                W[:, 0] = synth.E4M3_POW2[1 + np.arange(n) % 3]       # 0.25, 0.5, 1, ...
            s = np.full(n, 2.0 ** -4, np.float32)
        else:
            W = synth.e4m3_codes(g, (n, D))
            s = np.full(n, 1.0 / 64 / math.sqrt(D), np.float32)
        mats[name] = (W, s)
    return mats


def packed(mats):
    order = ("q", "kv", "kI", "qI", "w")
    return np.concatenate([mats[k][0] for k in order]), np.concatenate([mats[k][1] for k in order])


def run_in_proj(hb, mats, H, d, di, Hi):
    W, s = packed(mats)
    out = api.layer_in_proj(dev_bf16(hb), dev(W), dev(s), H, d, di, Hi)
    torch.cuda.synchronize()
    return out


def oracle_in_proj(hb, mats, Hi):
    return O.layer_in_proj(as_bf16_values(hb), *mats["q"], *mats["kv"], *mats["kI"], *mats["qI"], *mats["w"], Hi)


IN_CASES = [
    # M, D, H, d, di, Hi
    (2048, 1024, 8, 128, 64, 4),      # the 2,048-token prefill layer (tiled kernel)
    (4, 7168, 64, 512, 64, 4),        # a 4-sequence decode step at the 1M model widths
    (37, 1024, 8, 128, 64, 4),        # weight-stream kernel, ragged rows
]


@pytest.mark.parametrize("case", IN_CASES, ids=[f"M{c[0]}_D{c[1]}" for c in IN_CASES])
def test_layer_in_proj_exact_inputs_bit_exact(case):
    M, D, H, d, di, Hi = case
    g = synth.rng(3200 + M)
    h = synth.grid(g, (M, D))                                       # multiples of 1/8 in [-2, 2]: bf16 numbers
    h[:, 0] = 1.0
    hb = (h.view(np.uint32) >> 16).astype(np.uint16)
    mats = in_proj_weights(g, D, H, d, di, Hi, exact=True)
    say(f"layer_in_proj exact M={M} D={D}")
    got = run_in_proj(hb, mats, H, d, di, Hi)
    q, kv, kI, qc, qs, w = oracle_in_proj(hb, mats, Hi)
    assert np.array_equal(host_bf16_bits(got["q"]).reshape(M, H * d), q)
    assert np.array_equal(host_bf16_bits(got["kv"]), kv)
    assert np.array_equal(host_bf16_bits(got["k_idx"]), kI)
    assert np.array_equal(got["w_idx"].cpu().numpy(), w)
    assert np.array_equal(got["q_idx"].cpu().numpy(), qc)
    assert np.array_equal(got["q_idx_scales"].cpu().numpy(), qs)


def fp4_values(codes, scales, di):
    flat_c = codes.reshape(-1, di // 2)
    flat_s = scales.reshape(-1, di // 32)
    return O.idx_decode(flat_c, flat_s, O.FP4_E2M1, di).reshape(codes.shape[:-1] + (di,))


@pytest.mark.parametrize("case", IN_CASES, ids=[f"M{c[0]}_D{c[1]}" for c in IN_CASES])
def test_layer_in_proj_general_inputs(case):
    M, D, H, d, di, Hi = case
    g = synth.rng(3300 + M)
    hb = synth.bf16_bits(g, (M, D))
    mats = in_proj_weights(g, D, H, d, di, Hi, exact=False)
    say(f"layer_in_proj general M={M} D={D}")
    got = run_in_proj(hb, mats, H, d, di, Hi)
    h = as_bf16_values(hb)
    for name, key, shape in (("q", "q", (M, H * d)), ("kv", "kv", (M, d)), ("kI", "k_idx", (M, di))):
        W, s = mats[name]
        ref = O.linear_fp8(h, W, s)
        bound = gamma(D) * abs_products(h, W, s) * (1 + 1e-6) + np.abs(ref) * 2.0 ** -8
        val = out_to_f64(got[key]).reshape(shape)
        report(f"in_proj {name} M={M}", abs=abs_err(val, ref), norm_rel=norm_rel(val, ref))
        assert np.all(np.abs(val - ref) <= bound), name
    W, s = mats["w"]
    ref = O.linear_fp8(h, W, s)
    assert np.all(np.abs(got["w_idx"].cpu().numpy() - ref) <= gamma(D) * abs_products(h, W, s) * (1 + 1e-6) + 1e-30)
    # FP4 queries: the quantiser's input differs from the oracle's by the
    # summation error only, so a block keeps its scale and a code moves by at
    # most one step (an E2M1 step is at most 2 at the block scale)
    W, s = mats["qI"]
    ref32 = O.linear_fp8(h, W, s).astype(np.float32).reshape(M, Hi, di)
    oc, os_ = np.empty((M, Hi, di // 2), np.uint8), np.empty((M, Hi, di // 32), np.uint8)
    for r in range(M):
        for hh in range(Hi):
            oc[r, hh], os_[r, hh] = O.fp4_quant_row(ref32[r, hh])
    gc, gs = got["q_idx"].cpu().numpy(), got["q_idx_scales"].cpu().numpy()
    same_scale = np.mean(gs == os_)
    same_code = np.mean(gc == oc)
    report(f"in_proj qI M={M}", same_scale=float(same_scale), same_code_bytes=float(same_code))
    assert same_scale >= 0.999 and same_code >= 0.995
    gv, ov = fp4_values(gc, gs, di), fp4_values(oc, os_, di)
    step = 2.0 * np.repeat(2.0 ** (os_.astype(np.float64) - 127), 32, axis=-1)
    ok = (np.abs(gv - ov) <= step) | np.repeat(gs != os_, 32, axis=-1)
    assert np.all(ok)


# ---------------------------------------------------------------------- a layer from hidden states
def test_csa_layer_from_hidden_states_prefill():
    """A CSA layer over a 2,048-token prefill from hidden states (D = 1024,
    8 heads x 128 with 64 RoPE dims, m = 4, top-64, window 128, FP4 indexer
    4 x 64, FP8 records, FP8 output projection 1024 -> 1024 in 8 groups).
    Exact inputs make the projections, the indexer keys and the indexer
    scores exact, so the top-k sets must match the oracle's bit for bit."""
    g = synth.rng(3400)
    T, D, H, d, dr, m, k, Wn, Hi, di, G = 2048, 1024, 8, 128, 64, 4, 64, 128, 4, 64, 8
    h = synth.grid(g, (T, D))
    h[:, 0] = 1.0
    hb = (h.view(np.uint32) >> 16).astype(np.uint16)
    mats = in_proj_weights(g, D, H, d, di, Hi, exact=True)
    Wo = synth.e4m3_codes(g, (D, H * d // G))
    so = np.full(D, 1.0 / 64 / math.sqrt(H * d // G), np.float32)
    b = synth.normal(g, m)
    bI = np.zeros(m, np.float32)                                    # uniform pooling of the indexer keys
    sink = synth.normal(g, H, std=0.5)
    gam = np.ones(d, np.float32)
    pos = np.arange(T, dtype=np.int32)[None]
    say("csa layer from hidden states: prefill 2048")
    p = run_in_proj(hb, mats, H, d, di, Hi)
    z = dev(np.zeros(1, np.int32))
    comp = api.KVCache(1, T // m, d, dr, O.FP8_E4M3)
    win = api.KVCache(1, Wn + T, d, dr, O.FP8_E4M3, ring=True)
    keys = api.IdxCache(1, T // m, di, O.FP4_E2M1)
    kv = p["kv"].view(1, T, d)
    api.compress_kv(kv, z, m, dev(b), gamma=dev(gam), rope_dim=dr, kv_out=comp)
    api.compress_kv(kv, z, 1, dev(np.zeros(1, np.float32)), gamma=dev(gam), rope_dim=dr, kv_out=win)
    api.compress_kv(p["k_idx"].view(1, T, di), z, m, dev(bI), idx_out=keys)
    top = api.indexer_topk(p["q_idx"].view(1, T, Hi, di // 2), api.FP4_E2M1, p["w_idx"].view(1, T, Hi), keys,
                           dev(pos), m, k, q_scales=p["q_idx_scales"].view(1, T, Hi, di // 32))
    o = api.sparse_mqa_attn(p["q"].view(1, T, H, d), dev(pos), top, comp, win, dev(sink),
                            api.attn_params(d, dr, Wn, m))
    y = api.linear_fp8(o.view(T, H * d), dev(Wo), dev(so), G=G, y_dtype=torch.float32)
    torch.cuda.synchronize()
    # the oracle's chain from the same hidden states
    q, kvb, kIb, qc, qs, w = oracle_in_proj(hb, mats, Hi)
    oc, _, _ = O.compress(kvb.reshape(1, T, d), O.BF16, [0], m, b, gamma=gam, dr=dr, out_kind=0,
                          out_fmt=O.FP8_E4M3, cap=T // m)
    ow, _, _ = O.compress(kvb.reshape(1, T, d), O.BF16, [0], 1, [0.0], gamma=gam, dr=dr, out_kind=0,
                          out_fmt=O.FP8_E4M3, cap=Wn + T, ring=True)
    okc, oks, _ = O.compress(kIb.reshape(1, T, di), O.BF16, [0], m, bI, out_kind=1, out_fmt=O.FP4_E2M1, cap=T // m)
    otop = O.indexer_topk(qc, qs, O.FP4_E2M1, w, pos[0], okc[0], oks[0], O.FP4_E2M1, m, k)
    assert np.array_equal(top.cpu().numpy()[0], otop)
    # attention and projection: the oracle on its own records (the GPU's agree
    # within one code), compared within the bf16 bounds
    oo = O.attention(q.reshape(T, H, d), O.BF16, pos[0], gam, sink, d, dr, Wn, m, 10000.0, 1 / math.sqrt(d), 1e-6,
                     oc[0], O.FP8_E4M3, ow[0], O.FP8_E4M3, otop)
    go = out_to_f64(o)[0]
    report("layer prefill attention", abs=abs_err(go, oo), norm_rel=norm_rel(go, oo))
    assert norm_rel(go, oo) <= BF16_NORM_REL
    oy = O.linear_fp8(oo.reshape(T, H * d), Wo, so, G=G)
    gy = out_to_f64(y)
    report("layer prefill output", abs=abs_err(gy, oy), norm_rel=norm_rel(gy, oy))
    assert norm_rel(gy, oy) <= BF16_NORM_REL


def test_csa_layer_from_hidden_states_decode_1m_widths():
    """One decode step of a CSA layer for 4 sequences with the 1M model
    widths (D = 7168, 64 heads x 512, indexer 4 x 64, top-1024, FP8 output
    projection 32768 -> 7168 in 8 groups) over 16,384 compressed blocks (FP8
    records and FP4 keys of a seeded prefix).  The step projects the new
    token at t = 65,535, writes its window entry, compresses the block it
    completes (with three earlier raw tokens) into the last cache slot,
    selects, attends and projects.  Exact inputs: the new indexer key and the
    top-k sets bit for bit."""
    g = synth.rng(3500)
    B, D, H, d, dr, m, k, Wn, Hi, di, G = 4, 7168, 64, 512, 64, 4, 1024, 128, 4, 64, 8
    ncap = 16384
    t = m * ncap - 1
    j = t // m
    h = synth.grid(g, (B, D))
    h[:, 0] = 1.0
    hb = (h.view(np.uint32) >> 16).astype(np.uint16)
    mats = in_proj_weights(g, D, H, d, di, Hi, exact=True)
    Wo = synth.e4m3_codes(g, (D, H * d // G))
    so = np.full(D, 1.0 / 64 / math.sqrt(H * d // G), np.float32)
    b = synth.normal(g, m)
    bI = np.zeros(m, np.float32)
    sink = synth.normal(g, H, std=0.5)
    gam = np.ones(d, np.float32)
    # the prefix: normalised entries through the oracle's encoder, FP4 keys,
    # window entries; the block's three earlier raw tokens
    prev_kv = synth.bf16_bits(g, (B, m - 1, d))
    prev_kI = (synth.grid(g, (B, m - 1, di)).view(np.uint32) >> 16).astype(np.uint16)
    ent = synth.normal(g, (B, ncap, d))
    ent = ent / np.sqrt(np.mean(ent.astype(np.float64) ** 2, axis=-1, keepdims=True))
    comp_h = O.kv_encode(ent, O.FP8_E4M3, dr)
    comp_h[:, j] = 0
    kc_h, ks_h = synth.fp4_rows(g, (B, ncap), di)
    kc_h[:, j] = 0
    ks_h[:, j] = 0
    wins = O.kv_encode(synth.normal(g, (B, Wn, d)), O.FP8_E4M3, dr)
    say("csa layer from hidden states: decode B=4 at the 1M widths")
    p = run_in_proj(hb, mats, H, d, di, Hi)
    comp = api.KVCache(B, ncap, d, dr, O.FP8_E4M3, rec=dev(comp_h))
    win = api.KVCache(B, Wn, d, dr, O.FP8_E4M3, ring=True, rec=dev(wins))
    keys = api.IdxCache(B, ncap, di, O.FP4_E2M1, codes=dev(kc_h), scales=dev(ks_h))
    blk_kv = torch.cat([dev_bf16(prev_kv), p["kv"].view(B, 1, d)], dim=1).contiguous()
    blk_kI = torch.cat([dev_bf16(prev_kI), p["k_idx"].view(B, 1, di)], dim=1).contiguous()
    tok_blk = dev(np.full(B, t - (m - 1), np.int32))
    tok_new = dev(np.full(B, t, np.int32))
    api.compress_kv_batch([
        dict(x=p["kv"].view(B, 1, d).contiguous(), tok_start=tok_new, m=1, score_bias=dev(np.zeros(1, np.float32)),
             gamma=dev(gam), rope_dim=dr, kv_out=win),
        dict(x=blk_kv, tok_start=tok_blk, m=m, score_bias=dev(b), gamma=dev(gam), rope_dim=dr, kv_out=comp),
        dict(x=blk_kI, tok_start=tok_blk, m=m, score_bias=dev(bI), idx_out=keys)])
    pos = np.full((B, 1), t, np.int32)
    top = api.indexer_topk(p["q_idx"].view(B, 1, Hi, di // 2), api.FP4_E2M1, p["w_idx"].view(B, 1, Hi), keys,
                           dev(pos), m, k, q_scales=p["q_idx_scales"].view(B, 1, Hi, di // 32))
    o = api.sparse_mqa_attn(p["q"].view(B, 1, H, d), dev(pos), top, comp, win, dev(sink),
                            api.attn_params(d, dr, Wn, m))
    y = api.linear_fp8(o.view(B, H * d), dev(Wo), dev(so), G=G, y_dtype=torch.float32)
    torch.cuda.synchronize()
    # the oracle: the same step from the same hidden states and prefix
    q, kvb, kIb, qc, qs, w = oracle_in_proj(hb, mats, Hi)
    blk = np.concatenate([prev_kv, kvb.reshape(B, 1, d)], axis=1)
    blkI = np.concatenate([prev_kI, kIb.reshape(B, 1, di)], axis=1)
    ts = [t - (m - 1)] * B
    rc, _, _ = O.compress(blk, O.BF16, ts, m, b, gamma=gam, dr=dr, out_kind=0, out_fmt=O.FP8_E4M3, cap=ncap)
    kc, ks, _ = O.compress(blkI, O.BF16, ts, m, bI, out_kind=1, out_fmt=O.FP4_E2M1, cap=ncap)
    we, _, _ = O.compress(kvb.reshape(B, 1, d), O.BF16, [t] * B, 1, [0.0], gamma=gam, dr=dr, out_kind=0,
                          out_fmt=O.FP8_E4M3, cap=Wn, ring=True)
    comp_o, kc_o, ks_o, win_o = comp_h.copy(), kc_h.copy(), ks_h.copy(), wins.copy()
    comp_o[:, j], kc_o[:, j], ks_o[:, j], win_o[:, t % Wn] = rc[:, j], kc[:, j], ks[:, j], we[:, t % Wn]
    # cache writes: the key bit for bit (exact pooled input), records within one code
    assert np.array_equal(keys.codes.cpu().numpy()[:, j], kc[:, j])
    assert np.array_equal(keys.scales.cpu().numpy()[:, j], ks[:, j])
    for got_rec, ref_rec in ((comp.rec.cpu().numpy()[:, j], rc[:, j]), (win.rec.cpu().numpy()[:, t % Wn], we[:, t % Wn])):
        dv = O.kv_decode(got_rec, O.FP8_E4M3, d, dr) - O.kv_decode(ref_rec, O.FP8_E4M3, d, dr)
        assert np.max(np.abs(dv)) <= 0.1
    otops = top.cpu().numpy()
    for bb in range(B):
        otop = O.indexer_topk(qc[bb:bb + 1], qs[bb:bb + 1], O.FP4_E2M1, w[bb:bb + 1], pos[bb], kc_o[bb], ks_o[bb],
                              O.FP4_E2M1, m, k)
        assert np.array_equal(otops[bb], otop), bb
    oo = np.stack([O.attention(q[bb].reshape(1, H, d), O.BF16, pos[bb], gam, sink, d, dr, Wn, m, 10000.0,
                               1 / math.sqrt(d), 1e-6, comp_o[bb], O.FP8_E4M3, win_o[bb], O.FP8_E4M3, otops[bb])
                   for bb in range(B)])
    go = out_to_f64(o)
    report("layer decode attention", abs=abs_err(go, oo), norm_rel=norm_rel(go, oo))
    assert norm_rel(go, oo) <= BF16_NORM_REL
    oy = O.linear_fp8(oo.reshape(B, H * d), Wo, so, G=G)
    gy = out_to_f64(y)
    report("layer decode output", abs=abs_err(gy, oy), norm_rel=norm_rel(gy, oy))
    assert norm_rel(gy, oy) <= BF16_NORM_REL
