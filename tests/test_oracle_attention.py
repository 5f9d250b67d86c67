"""Pins for the oracle's pooling, RMSNorm, RoPE, indexer, top-k, attention and
projection (CPU only).  Each check compares against something other than the
oracle itself: an independent dense numpy formulation (tests/bruteforce.py),
torch library routines (rms_norm, scaled_dot_product_attention, sorts),
closed forms and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import bruteforce as bf
from long_context_attention_23_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bytes(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint8)


def run_oracle_layer(orc, x, xI, q, qI, w, sink, *, m, k, W, dr, base, eps, b, bI, gamma_kv,
                     gamma_q, sparse=True, start=0, q_pos=None, topk=None):
    """Oracle pipeline for one sequence whose tokens sit at start..start+T-1.
    Caches are f32 records; the window is a ring of capacity T."""
    T, d = x.shape
    N = T // m
    cap = start // m + N
    comp, _, _ = orc.compress(x[None], orc.F32, [start], m, b, gamma=gamma_kv, eps=eps, dr=dr,
                              base=base, out_kind=0, out_fmt=orc.F32, cap=cap)
    win, _, _ = orc.compress(x[None], orc.F32, [start], 1, [0.0], gamma=gamma_kv, eps=eps, dr=dr,
                             base=base, out_kind=0, out_fmt=orc.F32, cap=T, ring=True)
    if q_pos is None:
        q_pos = start + np.arange(T, dtype=np.int32)
    if sparse and topk is None:
        keys, _, _ = orc.compress(xI[None], orc.F32, [start], m, bI, out_kind=1, out_fmt=orc.F32, cap=cap)
        Hi, di = qI.shape[1:]
        topk = orc.indexer_topk(f32_bytes(qI).reshape(T, Hi, 4 * di), None, orc.F32, w, q_pos,
                                keys[0], None, orc.F32, m, k)
    out = orc.attention(q, orc.F32, q_pos, gamma_q, sink, d, dr, W, m, base, 1 / math.sqrt(d), eps,
                        comp[0], orc.F32, win[0], orc.F32, topk if sparse else None)
    return out, topk


def tiny_inputs(seed, T=48, d=16, H=3, di=8, Hi=2, m=4, dr=8):
    g = synth.rng(seed)
    return dict(
        x=synth.normal(g, (T, d)), xI=synth.normal(g, (T, di)), q=synth.normal(g, (T, H, d)),
        qI=synth.normal(g, (T, Hi, di)), w=synth.normal(g, (T, Hi)), sink=synth.normal(g, H),
        b=synth.normal(g, m), bI=synth.normal(g, m), gamma_kv=1 + 0.3 * synth.normal(g, d),
        gamma_q=1 + 0.3 * synth.normal(g, d))


# ------------------------------------------------------------------ P1
@pytest.mark.parametrize("m,k,W,sparse", [(4, 3, 5, True), (4, 100, 5, True), (2, 4, 0, True),
                                          (3, 2, 7, True), (4, 0, 6, False), (1, 5, 3, True)])
def test_bruteforce_layer(orc, m, k, W, sparse):
    inp = tiny_inputs(100 + m * 10 + k, m=m)
    kw = dict(m=m, k=k, W=W, dr=8, base=10000.0, eps=1e-6)
    ref, ref_top = bf.layer(**inp, **kw, sparse=sparse)
    out, top = run_oracle_layer(orc, **inp, **kw, sparse=sparse)
    if sparse:
        assert np.array_equal(top, ref_top)
    assert np.max(np.abs(out - ref)) <= 1e-10 * np.max(np.abs(ref))


# ------------------------------------------------------------------ P2
def test_full_topk_equals_dense(orc):
    inp = tiny_inputs(7)
    T = inp["x"].shape[0]
    m = 4
    allk = np.full((T, T // m), -1, np.int32)
    for t in range(T):
        n = (t + 1) // m
        allk[t, :n] = np.arange(n)
    kw = dict(m=m, k=T // m, W=5, dr=8, base=10000.0, eps=1e-6)
    sparse, _ = run_oracle_layer(orc, **inp, **kw, topk=allk)
    dense, _ = run_oracle_layer(orc, **inp, **kw, sparse=False)
    assert np.array_equal(sparse, dense)


# ------------------------------------------------------------------ P3
@pytest.mark.parametrize("W", [0, 4])
def test_m1_is_causal_mqa(orc, W):
    """m = 1, sink = -inf: dense attention over every token equals textbook
    causal softmax attention (torch SDPA in fp64), with a +ln 2 logit bias on
    the last W keys when the window duplicates them."""
    T, d, H, dr, base, eps = 40, 32, 4, 16, 10000.0, 1e-6
    g = synth.rng(31 + W)
    x = synth.normal(g, (T, d))
    q = synth.normal(g, (T, H, d))
    gkv = 1 + 0.2 * synth.normal(g, d)
    gq = 1 + 0.2 * synth.normal(g, d)
    sink = np.full(H, -np.inf, np.float32)
    out, _ = run_oracle_layer(orc, x, None, q, None, None, sink, m=1, k=0, W=W, dr=dr, base=base, eps=eps,
                              b=[0.0], bI=None, gamma_kv=gkv, gamma_q=gq, sparse=False)
    t = np.arange(T)
    xt = torch.from_numpy(x.astype(np.float64))
    kn = torch.nn.functional.rms_norm(xt, (d,), weight=torch.from_numpy(gkv.astype(np.float64)), eps=eps).numpy()
    keys = bf.f32(bf.rope_complex(kn, t, dr, base))
    qt = torch.from_numpy(q.astype(np.float64))
    qn = torch.nn.functional.rms_norm(qt, (d,), weight=torch.from_numpy(gq.astype(np.float64)), eps=eps).numpy()
    qh = bf.rope_complex(qn, t[:, None] * np.ones((1, H)), dr, base)
    Q = torch.from_numpy(qh).permute(1, 0, 2)[None]                    # [1, H, T, d]
    K = torch.from_numpy(keys)[None, None].expand(1, H, T, d)
    bias = torch.full((T, T), -math.inf, dtype=torch.float64)
    for i in range(T):
        bias[i, :i + 1] = 0.0
        if W > 0:
            bias[i, max(0, i - W + 1):i + 1] = math.log(2.0)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, K, attn_mask=bias)
    o = o[0].permute(1, 0, 2).numpy()
    o = bf.rope_complex(o, -t[:, None] * np.ones((1, H)), dr, base)
    assert np.max(np.abs(out - o)) <= 1e-12 * np.max(np.abs(o))


# ------------------------------------------------------------------ P4
def test_relative_position_invariance(orc):
    """Shifting every position by a multiple of m leaves the outputs unchanged
    (query RoPE at t, key RoPE at its position, output RoPE at -t)."""
    m, W, dr = 4, 6, 8
    inp = tiny_inputs(41, m=m)
    T = inp["x"].shape[0]
    g = synth.rng(42)
    qs = np.arange(W - 1, T, dtype=np.int32)             # queries whose window is full
    n_vis = (qs + 1) // m
    top = synth.topk_lists(g, n_vis, 5, len(qs))
    kw = dict(m=m, k=5, W=W, dr=dr, base=10000.0, eps=1e-6)
    sub = dict(inp, q=inp["q"][qs])
    a, _ = run_oracle_layer(orc, **sub, **kw, q_pos=qs, topk=top)
    delta = 4 * 1000
    shifted = np.where(top >= 0, top + delta // m, -1).astype(np.int32)
    b, _ = run_oracle_layer(orc, **sub, **kw, start=delta, q_pos=qs + delta, topk=shifted)
    assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(a))
    # a wrong-signed output rotation would break it: R_{+t} instead of R_{-t}
    t = qs.astype(np.float64)
    a_bad = bf.rope_complex(a, 2 * t[:, None] * np.ones((1, 3)), dr, 10000.0)
    b_bad = bf.rope_complex(b, 2 * (t + delta)[:, None] * np.ones((1, 3)), dr, 10000.0)
    assert np.max(np.abs(a_bad - b_bad)) > 1e-2 * np.max(np.abs(a))


# ------------------------------------------------------------------ P5, P6
def test_weights_sum_to_one_and_sink(orc):
    T, d, H, dr = 33, 16, 1, 8
    g = synth.rng(51)
    x = synth.normal(g, (T, d))
    q = synth.normal(g, (1, H, d)) * 3
    comp, _, _ = orc.compress(x[None], orc.F32, [0], 4, [0.1, 0.2, -0.3, 0.0], dr=dr,
                              out_kind=0, out_fmt=orc.F32, cap=8)
    win, _, _ = orc.compress(x[None], orc.F32, [0], 1, [0.0], dr=dr, out_kind=0, out_fmt=orc.F32,
                             cap=T, ring=True)
    pos = np.array([T - 1], np.int32)
    res = {}
    for s in (-np.inf, -1.0, 0.0, 2.5, 60.0):
        o, p, ps = orc.attention(q, orc.F32, pos, None, np.array([s], np.float32), d, dr, 7, 4,
                                 10000.0, 0.25, 1e-6, comp[0], orc.F32, win[0], orc.F32, want_p=True)
        assert len(p) == 8 + 7
        assert abs(p.sum() + ps - 1.0) < 1e-12
        res[s] = (o, p, ps)
    o_inf, p_inf, ps_inf = res[-np.inf]
    assert ps_inf == 0.0
    for s in (-1.0, 0.0, 2.5):
        o, p, ps = res[s]
        # weights shrink uniformly by (1 - p_sink) and the output with them
        assert np.allclose(p, p_inf * (1 - ps), rtol=1e-12, atol=0)
        assert np.allclose(o, o_inf * (1 - ps), rtol=1e-10, atol=1e-14)
    # odds of the sink scale with exp(sigma)
    odds = {s: res[s][2] / (1 - res[s][2]) for s in (-1.0, 0.0, 2.5)}
    assert abs(odds[2.5] / odds[-1.0] - math.exp(3.5)) < 1e-9 * math.exp(3.5)
    assert np.max(np.abs(res[60.0][0])) < 1e-20


# ------------------------------------------------------------------ P7, P8, P9
def test_rmsnorm_matches_torch(orc):
    g = synth.rng(61)
    for d in (16, 512):
        v = synth.normal(g, d).astype(np.float64) * 5
        gam = synth.normal(g, d).astype(np.float64)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (d,), weight=torch.from_numpy(gam), eps=1e-6).numpy()
        assert np.allclose(orc.rmsnorm(v, gam, 1e-6), ref, rtol=1e-14, atol=1e-14)
        out = orc.rmsnorm(v, None, 0.0)
        assert abs(np.sqrt(np.mean(out ** 2)) - 1.0) < 1e-14


def test_rope_complex_and_group_laws(orc):
    g = synth.rng(62)
    v = synth.normal(g, 128).astype(np.float64)
    for pos in (0, 1, 7, 1048575, -5000):
        ours = orc.rope(v, 64, pos)
        # fp64 angles: one ulp of frequency times |pos| bounds the difference
        assert np.allclose(ours, bf.rope_complex(v, pos, 64, 10000.0), rtol=0, atol=1e-12 + 1e-15 * abs(pos))
        assert np.array_equal(ours[:64], v[:64])
        assert abs(np.linalg.norm(ours) - np.linalg.norm(v)) < 1e-12
    assert np.array_equal(orc.rope(v, 64, 0), v)
    ab = orc.rope(orc.rope(v, 64, 1234), 64, 4321)
    assert np.allclose(ab, orc.rope(v, 64, 5555), atol=1e-11)
    assert np.allclose(orc.rope(orc.rope(v, 64, 987654), 64, -987654), v, atol=1e-9)
    # pair (0,1) of the rotated block turns by exactly pos radians (frequency 1)
    e = np.zeros(128); e[64] = 1.0
    r = orc.rope(e, 64, 3)
    assert np.allclose(r[64:66], [math.cos(3), math.sin(3)], atol=1e-15)


def test_pooling_special_cases(orc):
    g = synth.rng(63)
    x = synth.normal(g, (4, 10)).astype(np.float64)
    c, pi = orc.pool(x, np.zeros(4))
    assert np.allclose(c, x.mean(axis=0), atol=1e-15) and np.allclose(pi, 0.25)
    c, pi = orc.pool(x, np.array([0.0, 800.0, 0.0, 0.0]))
    assert np.allclose(c, x[1], atol=0) and pi[1] == 1.0
    c, pi = orc.pool(x[:1], np.array([3.3]))
    assert np.array_equal(c, x[0])
    b = synth.normal(g, 4).astype(np.float64)
    u = synth.normal(g, 10).astype(np.float64)
    c, pi = orc.pool(x, b, u)
    assert abs(pi.sum() - 1) < 1e-15
    z = b + x @ u
    ref = torch.softmax(torch.from_numpy(z), 0).numpy()
    assert np.allclose(pi, ref, rtol=1e-14) and np.allclose(c, ref @ x, atol=1e-14)


# ------------------------------------------------------------------ indexer / top-k (P11)
def test_topk_definition_on_ties(orc):
    S = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -1.0, np.nan, 2.0])
    assert list(orc.topk(S, 3)) == [1, 2, 4]
    assert list(orc.topk(S, 4)) == [1, 2, 3, 4]
    assert list(orc.topk(S, 5)) == [1, 2, 3, 4, 7]
    assert list(orc.topk(S, 10)) == [0, 1, 2, 3, 4, 5, 6, 7, -1, -1]
    assert list(orc.topk(S[:0], 2)) == [-1, -1]


def test_topk_ranks_the_scores_themselves(orc):
    """Selection orders the scores S as they are: scores that differ below
    fp32 resolution are still distinct, not ties broken by index."""
    S = np.array([1.0, 1.0 + 2.0 ** -40, 1.0 + 2.0 ** -41, 0.5])
    assert np.float32(S[0]) == np.float32(S[1]) == np.float32(S[2])
    assert list(orc.topk(S, 1)) == [1]
    assert list(orc.topk(S, 2)) == [1, 2]


def test_indexer_general_topk_fp64(orc):
    """General (normal) f32 inputs: the set equals the first k of a full sort
    of the fp64 scores computed by numpy, (score desc, index asc)."""
    g = synth.rng(74)
    n, Hi, di, k = 4000, 4, 64, 100
    keys = synth.normal(g, (n, di))
    qI = synth.normal(g, (1, Hi, di))
    w = synth.normal(g, (1, Hi))
    out = orc.indexer_topk(f32_bytes(qI).reshape(1, Hi, 4 * di), None, orc.F32, w,
                           np.array([4 * n - 1], np.int32), f32_bytes(keys).reshape(n, 4 * di),
                           None, orc.F32, 4, k)
    ref_S = np.maximum(keys.astype(np.float64) @ qI[0].astype(np.float64).T, 0) @ w[0].astype(np.float64)
    order = np.lexsort((np.arange(n), -ref_S))
    assert np.array_equal(out[0], np.sort(order[:k]))


def test_indexer_grid_topk_exact(orc):
    """q, w and keys on the 1/8 grid in [-2, 2]: every score is exact, and the
    top-k set equals a full torch sort by (score desc, index asc)."""
    g = synth.rng(71)
    n, Hi, di, k = 3000, 4, 64, 64
    keys = synth.grid(g, (n, di))
    qI = synth.grid(g, (1, Hi, di))
    w = synth.grid(g, (1, Hi))
    out, S = orc.indexer_topk(f32_bytes(qI).reshape(1, Hi, 4 * di), None, orc.F32, w,
                              np.array([4 * n - 1], np.int32), f32_bytes(keys).reshape(n, 4 * di),
                              None, orc.F32, 4, k, want_scores=True)
    dots = keys.astype(np.float64) @ qI[0].astype(np.float64).T
    ref_S = np.maximum(dots, 0) @ w[0].astype(np.float64)
    assert np.array_equal(S[0], ref_S)
    assert np.all(np.abs(ref_S * 512 - np.round(ref_S * 512)) == 0)   # on the 1/512 grid
    # torch sort: stable descending sort keeps smaller index first on ties
    order = torch.sort(torch.from_numpy(-ref_S), stable=True).indices.numpy()
    assert np.array_equal(out[0], np.sort(order[:k]))
    # ties are common on the grid, so the tie rule is exercised
    assert len(np.unique(ref_S)) < n


def test_indexer_fp4_codes_drawn(orc):
    g = synth.rng(72)
    n, Hi, di, k = 2048, 4, 64, 128
    kc, ks = synth.fp4_rows(g, n, di, -2, 0)
    qc, qs = synth.fp4_rows(g, (1, Hi), di, -2, 0)
    w = synth.grid(g, (1, Hi))
    out, S = orc.indexer_topk(qc, qs, orc.FP4_E2M1, w, np.array([4 * n - 1], np.int32), kc, ks,
                              orc.FP4_E2M1, 4, k, want_scores=True)
    # decode codes with the OCP table directly
    table = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])

    def dec(c, s):
        vals = np.stack([table[c & 15], table[c >> 4]], axis=-1).reshape(c.shape[:-1] + (di,))
        return vals * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=-1)
    K = dec(kc, ks)
    Q = dec(qc, qs)[0]
    ref_S = np.maximum(K @ Q.T, 0) @ w[0].astype(np.float64)
    assert np.array_equal(S[0], ref_S)
    order = torch.sort(torch.from_numpy(-ref_S), stable=True).indices.numpy()
    assert np.array_equal(out[0], np.sort(order[:k]))


def test_indexer_causal_visibility(orc):
    g = synth.rng(73)
    n, di = 40, 32
    keys = synth.normal(g, (n, di))
    qI = synth.normal(g, (5, 1, di))
    w = np.ones((5, 1), np.float32)
    pos = np.array([0, 2, 3, 9, 200], np.int32)
    out = orc.indexer_topk(f32_bytes(qI).reshape(5, 1, 4 * di), None, orc.F32, w, pos,
                           f32_bytes(keys).reshape(n, 4 * di), None, orc.F32, 4, 3)
    assert list(out[0]) == [-1, -1, -1] and list(out[1]) == [-1, -1, -1]
    assert list(out[2]) == [0, -1, -1]
    assert len(set(out[3]) - {-1}) == 2 and max(out[3]) <= 1
    assert max(out[4]) < n


# ------------------------------------------------------------------ P12
def test_grouped_projection(orc):
    g = synth.rng(81)
    M, H, d, D, G = 5, 8, 16, 48, 4
    o = synth.normal(g, (M, H * d)).astype(np.float64)
    W = synth.normal(g, (G, D // G, H * d // G)).astype(np.float64)
    y = orc.out_proj(o, W)
    ref = o @ scipy.linalg.block_diag(*[W[i].T for i in range(G)])
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    W1 = synth.normal(g, (1, D, H * d)).astype(np.float64)
    assert np.allclose(orc.out_proj(o, W1), o @ W1[0].T, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ page constants
def test_page_constants_entry_counts(orc):
    """At a 1M-token context the HCA layer attends every 128:1 entry plus the
    128-token window, and a CSA query attends its top-k blocks plus the
    window (golden/page_constants.json)."""
    cst = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    L = cst["context_tokens"]["value"]
    mh = cst["hca_ratio"]["value"]
    Wn = cst["window"]["value"]
    k = cst["csa_blocks_attended_at_1M"]["value"]
    dr = cst["rope_dims"]["value"]
    d = dr + 16
    t = np.array([L - 1], np.int32)
    nh = L // mh
    comp = np.zeros((nh, 4 * d), np.uint8)
    win = np.zeros((Wn, 4 * d), np.uint8)
    q = np.ones((1, 1, d), np.float32)
    _, p, _ = orc.attention(q, orc.F32, t, None, np.zeros(1, np.float32), d, dr, Wn, mh, 10000.0, 0.1,
                            1e-6, comp, orc.F32, win, orc.F32, want_p=True)
    assert len(p) == nh + Wn == 8192 + 128
    comp4 = np.zeros((L // 4, 4 * d), np.uint8)
    top = np.arange(k, dtype=np.int32)[None] * 256
    _, p, _ = orc.attention(q, orc.F32, t, None, np.zeros(1, np.float32), d, dr, Wn, 4, 10000.0, 0.1,
                            1e-6, comp4, orc.F32, win, orc.F32, topk_idx=top, want_p=True)
    assert len(p) == k + Wn
    # all-zero entries: uniform weights, every entry and the sink (logit 0) equal
    assert np.allclose(p, 1.0 / (k + Wn + 1))
