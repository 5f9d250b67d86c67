"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded
inputs (MI355X only).

Tolerances (from the method's accuracy targets): fp32 attention outputs
within 1e-4 relative (max |d| / max |ref|); bf16 / fp8 paths within 2e-2
absolute; top-k sets bit-exact on exact (grid / drawn-code) inputs and
recall >= 99.9% on general inputs; quantised caches bit-exact on identical
fp32 input and within one code otherwise.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from helpers import (BF16_NORM_REL, abs_err, dev, dev_bf16, host_bf16_bits, norm_rel, out_to_f64, recall, rel_err,
                     report, say)
from long_context_attention_23_amd import api, synth

pytestmark = pytest.mark.gpu


# ====================================================================== compress
def run_compress_both(x32, xfmt, tok, m, b, u, gamma, dr, kind, fmt, cap, ring, seed):
    B, T, d = x32.shape
    if xfmt == O.BF16:
        bits = (x32.view(np.uint32) >> 16).astype(np.uint16)
        xin_orc = bits
        xdev = dev_bf16(bits)
    else:
        xin_orc = x32
        xdev = dev(x32)
    codes, scales, _ = O.compress(xin_orc, xfmt, tok, m, b, u=u, gamma=gamma, dr=dr, out_kind=kind,
                                  out_fmt=fmt, cap=cap, ring=ring)
    say(f"compress kind={kind} fmt={fmt} xfmt={xfmt} m={m} d={d} dr={dr} cap={cap} ring={ring} seed={seed}")
    if kind == 0:
        c = api.KVCache(B, cap, d, dr, fmt, ring=ring)
        api.compress_kv(xdev, dev(np.array(tok, np.int32)), m, dev(np.asarray(b, np.float32)),
                        score_proj=None if u is None else dev(u), gamma=None if gamma is None else dev(gamma),
                        rope_dim=dr, kv_out=c)
        torch.cuda.synchronize()
        return codes, scales, c.rec.cpu().numpy(), None
    c = api.IdxCache(B, cap, d, fmt)
    api.compress_kv(xdev, dev(np.array(tok, np.int32)), m, dev(np.asarray(b, np.float32)),
                    score_proj=None if u is None else dev(u), gamma=None if gamma is None else dev(gamma),
                    rope_dim=dr, idx_out=c)
    torch.cuda.synchronize()
    return codes, scales, c.codes.cpu().numpy(), None if c.scales is None else c.scales.cpu().numpy()


@pytest.mark.parametrize("kind,fmt", [(0, O.F32), (0, O.BF16), (0, O.FP8_E4M3), (1, O.F32), (1, O.BF16),
                                      (1, O.FP4_E2M1)])
@pytest.mark.parametrize("xfmt", [O.F32, O.BF16])
def test_compress_bit_exact_on_identical_input(kind, fmt, xfmt):
    """m = 1, no norm, no RoPE: the quantiser sees the same fp32 value on both
    sides, so the bytes must be identical."""
    g = synth.rng(300 + 10 * kind + fmt + 100 * xfmt)
    B, T, d = 3, 37, 128
    x = synth.normal(g, (B, T, d)) * np.float32(3.0)
    x[0, 0, :64] *= np.float32(1e-5)                  # a row with a wide block spread (FP4 clamp)
    x[1, 1] = 0.0                                      # an all-zero row
    tok = [0, 5, 1000]
    codes, scales, gc, gs = run_compress_both(x, xfmt, tok, 1, [0.0], None, None, 0, kind, fmt, 1100, False, 0)
    assert np.array_equal(gc, codes)
    if scales is not None:
        assert np.array_equal(gs, scales)


def decoded(kind, fmt, codes, scales, d, dr):
    if kind == 0:
        return O.kv_decode(codes, fmt, d, dr)
    return O.idx_decode(codes, scales, fmt, d)


@pytest.mark.parametrize("kind,fmt,m,dr,xfmt,ring,content", [
    (0, O.FP8_E4M3, 4, 64, O.BF16, False, True), (0, O.BF16, 128, 64, O.BF16, False, False),
    (0, O.F32, 4, 64, O.F32, False, True), (0, O.FP8_E4M3, 1, 64, O.BF16, True, False),
    (0, O.F32, 3, 16, O.F32, True, True), (1, O.FP4_E2M1, 4, 0, O.BF16, False, True),
    (1, O.BF16, 4, 0, O.F32, False, True), (1, O.F32, 128, 0, O.F32, False, False),
    # position-only scores: the latency-oriented kernel (all loads first, lane-pair RoPE)
    (0, O.FP8_E4M3, 4, 64, O.BF16, False, False), (0, O.FP8_E4M3, 128, 64, O.BF16, False, False),
    (0, O.FP8_E4M3, 16, 64, O.F32, True, False), (1, O.FP4_E2M1, 4, 0, O.BF16, False, False),
    (1, O.FP4_E2M1, 128, 0, O.BF16, False, False), (0, O.FP8_E4M3, 200, 64, O.BF16, False, False)])
def test_compress_pooled_within_one_code(kind, fmt, m, dr, xfmt, ring, content):
    g = synth.rng(400 + m + fmt + 7 * kind + 1000 * content)
    d = 512 if kind == 0 and fmt != O.F32 else (64 if kind == 1 else 128)
    B = 3
    T = m * 5 + (m - 1 if m > 1 else 0)                # ragged tail ignored
    x = synth.normal(g, (B, T, d))
    b = synth.normal(g, m)
    u = synth.normal(g, d) * np.float32(0.05) if content else None
    gamma = (1 + 0.2 * synth.normal(g, d)).astype(np.float32) if kind == 0 else None
    tok = [0, m * 3, m * 1000]
    cap = 7 if ring else 1010
    codes, scales, gc, gs = run_compress_both(x, xfmt, tok, m, b, u, gamma, dr, kind, fmt, cap, ring, 0)
    check_pooled(kind, fmt, d, dr, codes, scales, gc, gs)


def check_pooled(kind, fmt, d, dr, codes, scales, gc, gs):
    """Device record bytes gc/gs against the oracle's codes/scales: within one
    quantisation step of the stored format."""
    ref = decoded(kind, fmt, codes, scales, d, dr)
    got = decoded(kind, fmt, gc, gs, d, dr)
    written = np.any(codes != 0, axis=-1)
    assert np.array_equal(np.any(gc != 0, axis=-1), written)
    r, q = ref[written], got[written]
    if fmt == O.F32:
        assert rel_err(q, r) < 1e-5
    elif fmt == O.BF16:
        assert np.all(np.abs(q - r) <= 2.0 ** -7 * np.abs(r) + 1e-30)
    elif fmt == O.FP8_E4M3:
        step = 2.0 ** -3 * np.abs(r[:, :d - dr]) + 2.0 ** -9 * np.max(np.abs(r[:, :d - dr]), axis=1, keepdims=True) / 448
        assert np.all(np.abs(q[:, :d - dr] - r[:, :d - dr]) <= step * 1.0001)
        assert np.all(np.abs(q[:, d - dr:] - r[:, d - dr:]) <= 2.0 ** -7 * np.abs(r[:, d - dr:]) + 1e-30)
        assert np.mean(gc[written][:, :d - dr] == codes[written][:, :d - dr]) > 0.99
    else:  # FP4
        assert np.mean(gc[written] == codes[written]) > 0.97
        e = gs[written].astype(np.int64) - 127
        step = np.repeat(2.0 ** (e + 1), 32, axis=-1)
        assert np.all(np.abs(q - r) <= step)


@pytest.mark.parametrize("kind,fmt,m,dr,xfmt,ring,content", [
    (0, O.FP8_E4M3, 4, 64, O.BF16, False, False), (0, O.FP8_E4M3, 128, 64, O.BF16, False, False),
    (1, O.FP4_E2M1, 4, 0, O.BF16, False, False), (0, O.BF16, 16, 64, O.F32, False, True),
    (1, O.F32, 4, 0, O.F32, False, True), (0, O.FP8_E4M3, 1, 64, O.BF16, True, False)])
def test_compress_step_matches_oracle(kind, fmt, m, dr, xfmt, ring, content):
    """csa_compress_kv_step fed one token per call: every entry against the
    oracle's pooling of the same tokens (within one code, as the block kernel;
    m = 1 entries bit for bit against csa_compress_kv); a block's last token
    writes one entry per sequence, leaves the state alone, and repeating it
    changes nothing."""
    g = synth.rng(4400 + m + fmt + 7 * kind + 1000 * content)
    d = 512 if kind == 0 and fmt != O.F32 else (64 if kind == 1 else 128)
    B = 3
    T = 3 * m if m > 1 else 4
    x = synth.normal(g, (B, T, d))
    b = synth.normal(g, m)
    u = synth.normal(g, d) * np.float32(0.05) if content else None
    gamma = (1 + 0.2 * synth.normal(g, d)).astype(np.float32) if kind == 0 else None
    tok = [0, m * 3, m * 1000]
    cap = 7 if ring else 1010
    codes, scales, gc_blk, _ = run_compress_both(x, xfmt, tok, m, b, u, gamma, dr, kind, fmt, cap, ring, 0)
    say(f"compress step kind={kind} fmt={fmt} xfmt={xfmt} m={m} d={d} T={T}")
    xdev = dev_bf16((x.view(np.uint32) >> 16).astype(np.uint16)) if xfmt == O.BF16 else dev(x)
    out = api.KVCache(B, cap, d, dr, fmt, ring=ring) if kind == 0 else api.IdxCache(B, cap, d, fmt)
    state = api.compress_state(B, d) if m > 1 else None
    job = dict(m=m, score_bias=dev(np.asarray(b, np.float32)), score_proj=None if u is None else dev(u),
               gamma=None if gamma is None else dev(gamma), rope_dim=dr, state=state)
    job["kv_out" if kind == 0 else "idx_out"] = out

    def step(i):
        pos = dev(np.array([t0 + i for t0 in tok], np.int32))
        api.compress_kv_step([dict(job, x=xdev[:, i].contiguous(), tok_pos=pos)])
        torch.cuda.synchronize()
        if kind == 0:
            return out.rec.cpu().numpy(), None
        return out.codes.cpu().numpy(), None if out.scales is None else out.scales.cpu().numpy()

    for i in range(T - 1):
        c1, _ = step(i)
    st1 = None if state is None else state.clone()
    gc, gs = step(T - 1)
    assert np.sum(np.any(c1 != gc, axis=-1)) == B          # one new entry per sequence
    if m == 1:
        assert np.array_equal(gc, gc_blk)
    else:
        check_pooled(kind, fmt, d, dr, codes, scales, gc, gs)
        assert torch.equal(state, st1)
    again, _ = step(T - 1)
    assert np.array_equal(again, gc)
    if state is not None:
        assert torch.equal(state, st1)


@pytest.mark.parametrize("case", ["decode_step", "multi_block", "five_jobs", "content_score"])
def test_compress_batch_matches_single_calls(case):
    """csa_compress_kv_batch: every job's output equals that of its own
    csa_compress_kv call byte for byte, and the oracle's within one step."""
    g = synth.rng(4700 + len(case))
    B = 3
    # (kind, fmt, m, d, dr, ring, cap, T, content)
    jobs = [(0, O.FP8_E4M3, 1, 512, 64, True, 9, 1, False),        # window entry
            (0, O.FP8_E4M3, 4, 512, 64, False, 2100, 4, False),    # CSA block
            (1, O.FP4_E2M1, 4, 128, 0, False, 2100, 4, False),     # indexer key
            (0, O.FP8_E4M3, 128, 512, 64, False, 70, 128, False)]  # HCA block
    if case == "multi_block":
        jobs = [(0, O.FP8_E4M3, 4, 512, 64, False, 2100, 4 * 5 + 3, False),
                (1, O.FP4_E2M1, 4, 128, 0, False, 2100, 4 * 7 + 1, False),
                (0, O.BF16, 16, 256, 64, True, 11, 16 * 3, False)]
    elif case == "five_jobs":
        jobs = jobs + [(0, O.BF16, 2, 128, 64, False, 5000, 6, False)]
    elif case == "content_score":
        jobs = jobs[:2] + [(1, O.BF16, 4, 128, 0, False, 2100, 8, True)]
    tok = [0, 128 * 3, 128 * 15]
    dev_jobs, singles, refs = [], [], []
    for (kind, fmt, m, d, dr, ring, cap, T, content) in jobs:
        x32 = synth.normal(g, (B, T, d))
        bits = (x32.view(np.uint32) >> 16).astype(np.uint16)
        b = synth.normal(g, m)
        u = synth.normal(g, d) * np.float32(0.05) if content else None
        gamma = (1 + 0.2 * synth.normal(g, d)).astype(np.float32) if kind == 0 else None
        codes, scales, _ = O.compress(bits, O.BF16, tok, m, b, u=u, gamma=gamma, dr=dr, out_kind=kind,
                                      out_fmt=fmt, cap=cap, ring=ring)
        refs.append((kind, fmt, d, dr, codes, scales))
        args = dict(x=dev_bf16(bits), tok_start=dev(np.array(tok, np.int32)), m=m,
                    score_bias=dev(np.asarray(b, np.float32)), score_proj=None if u is None else dev(u),
                    gamma=None if gamma is None else dev(gamma), rope_dim=dr)
        mk = (lambda: api.KVCache(B, cap, d, dr, fmt, ring=ring)) if kind == 0 else (lambda: api.IdxCache(B, cap, d, fmt))
        one, many = mk(), mk()
        key = "kv_out" if kind == 0 else "idx_out"
        api.compress_kv(args["x"], args["tok_start"], m, args["score_bias"], score_proj=args["score_proj"],
                        gamma=args["gamma"], rope_dim=dr, **{key: one})
        singles.append(one)
        dev_jobs.append(dict(args, **{key: many}))
    say(f"compress batch case={case} jobs={len(jobs)}")
    api.compress_kv_batch(dev_jobs)
    torch.cuda.synchronize()
    for j, one, (kind, fmt, d, dr, codes, scales) in zip(dev_jobs, singles, refs):
        many = j.get("kv_out") or j.get("idx_out")
        if kind == 0:
            gc, gs, oc, osc = many.rec.cpu().numpy(), None, one.rec.cpu().numpy(), None
        else:
            gc, oc = many.codes.cpu().numpy(), one.codes.cpu().numpy()
            gs = None if many.scales is None else many.scales.cpu().numpy()
            osc = None if one.scales is None else one.scales.cpu().numpy()
        assert np.array_equal(gc, oc)
        if gs is not None:
            assert np.array_equal(gs, osc)
        check_pooled(kind, fmt, d, dr, codes, scales, gc, gs)


# ====================================================================== indexer
def run_indexer(qI_bytes, qI_scales, qfmt, w, pos, keys_bytes, key_scales, kfmt, m, k, di):
    B, Tq, Hi = w.shape
    cap = keys_bytes.shape[1]
    say(f"indexer B={B} Tq={Tq} Hi={Hi} cap={cap} k={k} qfmt={qfmt} kfmt={kfmt}")
    keys = api.IdxCache(B, cap, di, kfmt, codes=dev(keys_bytes),
                        scales=None if key_scales is None else dev(key_scales))
    out = api.indexer_topk(dev(qI_bytes), qfmt, dev(w), keys, dev(pos), m, k,
                           q_scales=None if qI_scales is None else dev(qI_scales))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = np.stack([O.indexer_topk(qI_bytes[b], None if qI_scales is None else qI_scales[b], qfmt, w[b], pos[b],
                                   keys_bytes[b], None if key_scales is None else key_scales[b], kfmt, m, k)
                    for b in range(B)])
    return got, ref


def f32_rows(a):
    a = np.ascontiguousarray(a, np.float32)
    return a.view(np.uint8).reshape(a.shape[:-1] + (a.shape[-1] * 4,))


def bf16_rows(a):
    bits = (np.ascontiguousarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits.view(np.uint8).reshape(a.shape[:-1] + (a.shape[-1] * 2,))


@pytest.mark.parametrize("cap,k,Tq,kfmt", [(512, 64, 96, O.F32), (3000, 256, 8, O.BF16), (20000, 1024, 3, O.F32),
                                           (20000, 100, 2, O.BF16), (70000, 2048, 1, O.F32)])
def test_indexer_grid_exact(cap, k, Tq, kfmt):
    """Grid inputs make every fp32 score exact: the sets must match exactly,
    across both the one-workgroup and the multi-kernel paths, including rows
    with fewer visible blocks than k and ties."""
    g = synth.rng(500 + cap + k)
    B, Hi, di, m = 2, 4, 64, 4
    keys = synth.grid(g, (B, cap, di))
    qI = synth.grid(g, (B, Tq, Hi, di))
    w = synth.grid(g, (B, Tq, Hi))
    pos = g.integers(0, 4 * cap + 50, size=(B, Tq)).astype(np.int32)
    pos[0, 0] = 4 * cap - 1                                   # every block visible
    pos[-1, -1] = 2                                           # no visible block
    if Tq > 2:
        pos[0, 1] = 4 * min(k, cap) // 2                      # fewer blocks than k
    conv = f32_rows if kfmt == O.F32 else bf16_rows
    got, ref = run_indexer(f32_rows(qI), None, O.F32, w, pos, conv(keys), None, kfmt, m, k, di)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("qkind", ["bf16", "fp4"])
def test_indexer_bf16_keys_mfma_exact(qkind):
    """bf16 keys (grid values are exact in bf16) scored on the matrix cores,
    queries in bf16 or FP4 codes: exact sets."""
    g = synth.rng(540 if qkind == "bf16" else 541)
    B, Tq, Hi, di, m, k, cap = 2, 2, 4, 64, 4, 1024, 40000
    keys = synth.grid(g, (B, cap, di))
    w = synth.grid(g, (B, Tq, Hi))
    pos = np.array([[4 * cap - 1, 4 * 7000 + 3], [4 * 100, 4 * cap + 50]], np.int32)
    if qkind == "bf16":
        qI = synth.grid(g, (B, Tq, Hi, di))
        got, ref = run_indexer(bf16_rows(qI), None, O.BF16, w, pos, bf16_rows(keys), None, O.BF16, m, k, di)
    else:
        qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
        got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, bf16_rows(keys), None, O.BF16, m, k, di)
    assert np.array_equal(got, ref)


def test_indexer_very_large_cap_exact():
    """More blocks than the final kernel's LDS bitmaps cover (2^18): the
    sorted-gather fallback."""
    g = synth.rng(545)
    B, Tq, Hi, di, m, k, cap = 1, 1, 4, 64, 4, 1024, 600000
    kc, ks = synth.fp4_rows(g, (B, cap), di, -2, 0)
    qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
    w = synth.grid(g, (B, Tq, Hi))
    pos = np.array([[4 * cap - 1]], np.int32)
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, m, k, di)
    assert np.array_equal(got, ref)


def test_indexer_tie_heavy_rows_exact():
    """Rows whose weights are all negative (every key with no positive head
    product ties at score 0) or all zero (every key ties): more candidates
    than the final kernel keeps in LDS, and the tie rule (smaller block index)
    decides most of the set."""
    g = synth.rng(546)
    B, Tq, Hi, di, m, k, cap = 2, 2, 4, 64, 4, 1024, 70000
    kc, ks = synth.fp4_rows(g, (B, cap), di, -2, 0)
    qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
    w = synth.grid(g, (B, Tq, Hi))
    w[0, 0] = -np.abs(w[0, 0]) - np.float32(0.125)          # all negative
    w[1, 1] = 0.0                                            # all zero: every score ties
    pos = np.array([[4 * cap - 1, 4 * cap - 1], [4 * 50000 + 2, 4 * cap - 1]], np.int32)
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, m, k, di)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[1, 1], np.arange(k))           # all tied: the first k blocks


def test_indexer_tie_tiers_exact():
    """Rows where every visible key ties (all weights zero), one per size class
    of the final selection's candidate storage: 3,000 / 12,000 / 20,000 /
    40,000 tied candidates (four per thread in registers, sixteen, twenty,
    re-read from memory).  The tie rule gives the first k blocks; an
    all-negative row beside them mixes ties at 0 with the rest."""
    g = synth.rng(547)
    B, Tq, Hi, di, m, k, cap = 1, 5, 4, 64, 4, 1024, 41000
    kc, ks = synth.fp4_rows(g, (B, cap), di, -2, 0)
    qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
    w = synth.grid(g, (B, Tq, Hi))
    w[0, :4] = 0.0
    w[0, 4] = -np.abs(w[0, 4]) - np.float32(0.125)
    pos = np.array([[4 * 3000 + 1, 4 * 12000 + 3, 4 * 20000, 4 * 40000 + 2, 4 * cap - 1]], np.int32)
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, m, k, di)
    assert np.array_equal(got, ref)
    for i in range(4):
        assert np.array_equal(got[0, i], np.arange(k))


@pytest.mark.parametrize("Tq", [96, 40])
def test_indexer_prefill_chunk_exact(Tq):
    """A chunk of query rows (FP4 queries and keys, four heads): the
    query-batched path -- sampled thresholds, candidate filter, exact select.
    Every row against the oracle, with a ragged chunk (Tq not a multiple of 32)
    and rows that see fewer blocks than k."""
    g = synth.rng(560 + Tq)
    B, Hi, di, m, k, cap = 2, 4, 64, 4, 1024, 20000
    kc, ks = synth.fp4_rows(g, (B, cap), di, -2, 0)
    qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
    w = synth.grid(g, (B, Tq, Hi))
    pos = np.stack([4 * (cap - Tq) + np.arange(Tq, dtype=np.int32) * 4 + 3,
                    4 * 12000 + np.arange(Tq, dtype=np.int32) * 37]).astype(np.int32)
    pos[1, :3] = [5, 4 * 1000, 4 * 1023 + 3]                # fewer blocks than k, exactly k
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, m, k, di)
    assert np.array_equal(got, ref)


def test_indexer_prefill_fallback_rows_exact():
    """Rows the sampled threshold cannot serve, recomputed exactly: one with
    all weights zero (every score ties: candidates overflow) and one whose
    sampled key tiles score far above the rest (too few candidates)."""
    g = synth.rng(570)
    B, Tq, Hi, di, m, k, cap = 1, 64, 4, 64, 4, 1024, 20000
    kc, ks = synth.fp4_rows(g, (B, cap), di, -2, 0)
    qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
    w = synth.grid(g, (B, Tq, Hi))
    w[0, 5] = 0.0
    # row 9: positive query codes and weights; the keys of every 64th 32-key
    # tile (the sampled ones) are all +6, so they outrank the rest
    qc[0, 9] = 0x22                                          # +1.0 in both nibbles
    qs[0, 9] = 127
    w[0, 9] = 1.0
    for t0 in range(0, cap, 64 * 32):
        kc[0, t0:t0 + 32] = 0x77
        ks[0, t0:t0 + 32] = 127
    pos = (4 * (cap - Tq) + np.arange(Tq, dtype=np.int32) * 4 + 3)[None].astype(np.int32)
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, m, k, di)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[0, 5], np.arange(k))           # all tied: the first k blocks


def test_indexer_decode_fallback_rows_exact():
    """Decode rows (a few queries per sequence, FP4) that a sampled threshold
    cannot serve, recomputed exactly: all weights zero (every key ties: more
    ties than the lists hold), and, for a query with positive codes and
    weights, the first four keys of every tile the decode filter samples
    (one per window of ceil(tiles / 64) tiles, at offset
    floor(((37 i + 11) mod 64) window / 64) in window i) made to outrank the
    rest: the sample's threshold is
    then the top score, which fewer than k keys of the row reach (too few
    candidates)."""
    g = synth.rng(571)
    B, Tq, Hi, di, m, k, cap = 2, 3, 4, 64, 4, 1024, 90000
    kc, ks = synth.fp4_rows(g, (B, cap), di, -2, 0)
    qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
    w = synth.grid(g, (B, Tq, Hi))
    w[0, 1] = 0.0
    qc[1, 2] = 0x22                                          # +1.0 in both nibbles
    qs[1, 2] = 127
    w[1, 2] = 1.0
    ntile = -(-cap // 32)                                    # query (1, 2) sees every block
    stride = -(-ntile // 32)                                 # the decode filter samples 32 tiles per row
    for i in range(-(-ntile // stride)):
        t0 = 32 * (i * stride + (((i * 37 + 11) & 63) * stride >> 6))
        kc[1, t0:t0 + 4] = 0x77
        ks[1, t0:t0 + 4] = 127
    pos = np.array([[4 * cap - 1, 4 * cap - 1, 4 * 30000 + 1], [4 * 60000, 4 * cap - 1, 4 * cap - 1]], np.int32)
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, m, k, di)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[0, 1], np.arange(k))           # all tied: the first k blocks


def test_indexer_fp4_codes_exact():
    """FP4 keys and queries drawn as codes with a narrow exponent range: exact."""
    g = synth.rng(510)
    B, Tq, Hi, di, m, k, cap = 2, 2, 4, 64, 4, 512, 30000
    kc, ks = synth.fp4_rows(g, (B, cap), di, -2, 0)
    qc, qs = synth.fp4_rows(g, (B, Tq, Hi), di, -2, 0)
    w = synth.grid(g, (B, Tq, Hi))
    pos = np.array([[4 * cap - 1, 4 * 1000 + 1], [4 * 20000, 4 * cap + 9]], np.int32)
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, m, k, di)
    assert np.array_equal(got, ref)
    # small path too
    got, ref = run_indexer(qc, qs, O.FP4_E2M1, w, np.minimum(pos, 4 * 4000 - 1), kc[:, :4000], ks[:, :4000],
                           O.FP4_E2M1, m, 64, di)
    assert np.array_equal(got, ref)


def test_indexer_general_recall():
    g = synth.rng(520)
    B, Tq, Hi, di, m, k, cap = 4, 2, 4, 64, 4, 1024, 50000
    keys = synth.normal(g, (B, cap, di))
    qI = synth.normal(g, (B, Tq, Hi, di))
    w = synth.normal(g, (B, Tq, Hi))
    pos = np.full((B, Tq), 4 * cap - 1, np.int32)
    got, ref = run_indexer(f32_rows(qI), None, O.F32, w, pos, f32_rows(keys), None, O.F32, m, k, di)
    r = recall(got, ref)
    say(f"recall {r}")
    assert r >= 0.999
    assert np.all(np.diff(got, axis=-1) > 0)                 # ascending, distinct


def test_indexer_deterministic_and_batch_invariant():
    g = synth.rng(530)
    B, Tq, Hi, di, m, k, cap = 3, 1, 4, 64, 4, 300, 10000
    keys = synth.normal(g, (B, cap, di))
    qI = synth.normal(g, (B, Tq, Hi, di))
    w = synth.normal(g, (B, Tq, Hi))
    pos = np.full((B, Tq), 4 * cap - 1, np.int32)
    kc = api.IdxCache(B, cap, di, O.F32, codes=dev(f32_rows(keys)))
    a = api.indexer_topk(dev(f32_rows(qI)), O.F32, dev(w), kc, dev(pos), m, k).cpu().numpy()
    b = api.indexer_topk(dev(f32_rows(qI)), O.F32, dev(w), kc, dev(pos), m, k).cpu().numpy()
    assert np.array_equal(a, b)
    k1 = api.IdxCache(1, cap, di, O.F32, codes=dev(f32_rows(keys[1:2])))
    c = api.indexer_topk(dev(f32_rows(qI[1:2])), O.F32, dev(w[1:2]), k1, dev(pos[1:2]), m, k).cpu().numpy()
    assert np.array_equal(c[0], a[1])


# ====================================================================== attention
def build_caches(g, B, ccap, wcap, d, dr, cfmt, wfmt):
    comp_v = synth.normal(g, (B, ccap, d)).astype(np.float64)
    win_v = synth.normal(g, (B, wcap, d)).astype(np.float64)
    return O.kv_encode(comp_v, cfmt, dr), O.kv_encode(win_v, wfmt, dr)


def run_attention(sparse, q32, qfmt, pos, topk, comp, cfmt, win, wfmt, gamma, sink, d, dr, W, m, ofmt,
                  nan_ws=False):
    B, Tq, H, _ = q32.shape
    say(f"attention sparse={sparse} B={B} Tq={Tq} H={H} d={d} dr={dr} W={W} m={m} cfmt={cfmt} wfmt={wfmt} "
        f"qfmt={qfmt} ofmt={ofmt} ccap={comp.shape[1]} wcap={win.shape[1]}")
    if qfmt == O.BF16:
        qbits = (np.ascontiguousarray(q32).view(np.uint32) >> 16).astype(np.uint16)
        qdev, qorc = dev_bf16(qbits), qbits
    else:
        qdev, qorc = dev(q32), q32
    cc = api.KVCache(B, comp.shape[1], d, dr, cfmt, rec=dev(comp))
    wc = api.KVCache(B, win.shape[1], d, dr, wfmt, ring=True, rec=dev(win))
    p = api.attn_params(d, dr, W, m)
    kw = dict(gamma_q=None if gamma is None else dev(gamma),
              out_dtype=torch.bfloat16 if ofmt == O.BF16 else torch.float32)
    if nan_ws:                                    # a workspace full of NaN bit patterns
        n = api.attn_workspace_bytes(B, Tq, H, d, comp.shape[1] if topk is None else topk.shape[-1], W, qfmt, cfmt)
        kw["workspace"] = torch.full((max(n, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    if sparse:
        out = api.sparse_mqa_attn(qdev, dev(pos), dev(topk), cc, wc, dev(sink), p, **kw)
    else:
        out = api.hca_dense_mqa_attn(qdev, dev(pos), cc, wc, dev(sink), p, **kw)
    torch.cuda.synchronize()
    got = out_to_f64(out)
    ref = np.stack([O.attention(qorc[b], qfmt, pos[b], gamma, sink, d, dr, W, m, 10000.0, 1 / math.sqrt(d), 1e-6,
                                comp[b], cfmt, win[b], wfmt, None if topk is None else topk[b]) for b in range(B)])
    return got, ref


ATTN_CASES = [
    # sparse, B, Tq, H, d, dr, W, m, k, ccap, cfmt, qfmt, ofmt
    (True, 1, 40, 8, 128, 64, 128, 4, 64, 512, O.F32, O.F32, O.F32),         # C1-like, fp32
    (True, 2, 3, 32, 512, 64, 128, 4, 1024, 32768, O.BF16, O.BF16, O.BF16),  # C3-like decode
    (True, 2, 2, 64, 512, 64, 128, 4, 1024, 20000, O.FP8_E4M3, O.BF16, O.BF16),  # C4-like CSA
    (False, 3, 1, 32, 512, 64, 128, 128, 0, 512, O.BF16, O.BF16, O.BF16),   # C2-like HCA
    (False, 2, 1, 64, 512, 64, 128, 128, 0, 1500, O.FP8_E4M3, O.BF16, O.BF16),  # C4-like HCA (multi-split)
    (False, 1, 33, 8, 64, 16, 5, 3, 0, 40, O.F32, O.F32, O.F32),            # ragged prefill, dense
    (True, 2, 17, 4, 96, 32, 0, 2, 7, 50, O.F32, O.F32, O.BF16),            # no window
    (True, 1, 9, 16, 256, 64, 300, 4, 20, 100, O.BF16, O.F32, O.F32),       # window > split
    # bf16 queries over bf16 / FP8 caches take the MFMA kernel when d in {128, 256, 512}, H % 16 == 0
    (True, 2, 5, 16, 128, 64, 37, 4, 100, 300, O.BF16, O.BF16, O.F32),     # d 128, odd window
    (False, 2, 3, 48, 256, 64, 128, 16, 0, 300, O.FP8_E4M3, O.BF16, O.BF16),  # d 256, 3 waves
    (True, 1, 2, 96, 512, 64, 0, 4, 700, 5000, O.FP8_E4M3, O.BF16, O.BF16),  # 2 head groups, no window
    (True, 2, 2, 8, 512, 64, 128, 4, 64, 1000, O.BF16, O.BF16, O.BF16),     # H 8: generic kernel, bf16 q
    (False, 2, 2, 32, 512, 64, 128, 4, 0, 900, (O.BF16, O.FP8_E4M3), O.BF16, O.BF16),  # mixed cache formats
    (True, 3, 4, 64, 512, 64, 128, 4, 1024, 8000, O.FP8_E4M3, O.BF16, O.F32),  # prefill-like rows, f32 out
    # FP8 records with one 16-head group per wave, and the dim-quarter classes
    # of d = 128 (quarters 2 and 3 all RoPE) and d = 256 (quarter 3 all RoPE)
    (True, 2, 2, 32, 512, 64, 128, 4, 256, 2000, O.FP8_E4M3, O.BF16, O.BF16),   # 32 heads, sparse
    (False, 1, 3, 16, 512, 64, 64, 16, 0, 300, O.FP8_E4M3, O.BF16, O.F32),      # 16 heads: half the waves idle
    (True, 2, 3, 16, 128, 64, 40, 4, 50, 400, O.FP8_E4M3, O.BF16, O.BF16),      # d 128
    (False, 1, 2, 32, 256, 64, 128, 8, 0, 600, O.FP8_E4M3, O.BF16, O.BF16),     # d 256, 32 heads
]


@pytest.mark.parametrize("ci", range(len(ATTN_CASES)), ids=[f"c{i}" for i in range(len(ATTN_CASES))])
def test_attention_parity(ci):
    sparse, B, Tq, H, d, dr, W, m, k, ccap, cfmt, qfmt, ofmt = ATTN_CASES[ci]
    cfmt, wfmt = cfmt if isinstance(cfmt, tuple) else (cfmt, cfmt)
    g = synth.rng(600 + ci)
    wcap = W + Tq + 7 if W > 0 else 4
    comp, win = build_caches(g, B, ccap, wcap, d, dr, cfmt, wfmt)
    q = synth.normal(g, (B, Tq, H, d))
    gamma = (1 + 0.3 * synth.normal(g, d)).astype(np.float32)
    sink = synth.normal(g, H)
    tmax = m * ccap + 40
    pos = np.sort(g.integers(0, tmax, size=(B, Tq)), axis=1).astype(np.int32)
    pos[0, 0] = min(pos[0, 0], m - 2) if m > 1 else 0        # a row with no visible block
    topk = None
    if sparse:
        vis = np.minimum((pos.reshape(-1) + 1) // m, ccap)
        topk = synth.topk_lists(g, vis, k, B * Tq).reshape(B, Tq, k)
        topk[..., -1] = np.where(topk[..., -1] >= 0, ccap + 5, -1)   # an invisible index is skipped
    got, ref = run_attention(sparse, q, qfmt, pos, topk, comp, cfmt, win, wfmt, gamma, sink, d, dr, W, m, ofmt)
    report(f"attention c{ci}", max_rel=rel_err(got, ref), abs=abs_err(got, ref), norm_rel=norm_rel(got, ref))
    if ofmt == O.F32 and qfmt == O.F32 and cfmt == O.F32:
        assert rel_err(got, ref) <= 1e-4
    else:
        assert abs_err(got, ref) <= 2e-2
        assert norm_rel(got, ref) <= BF16_NORM_REL


@pytest.mark.parametrize("ci", [2, 4, 10])
def test_attention_split_workspace_holds_nan(ci):
    """The split partials' workspace starts out as NaN bit patterns: splits a
    row does not use must not reach its output (the combine's weights of
    unused splits are exact zeros, not 0 * stale value)."""
    sparse, B, Tq, H, d, dr, W, m, k, ccap, cfmt, qfmt, ofmt = ATTN_CASES[ci]
    g = synth.rng(680 + ci)
    comp, win = build_caches(g, B, ccap, W + Tq + 7, d, dr, cfmt, cfmt)
    q = synth.normal(g, (B, Tq, H, d))
    sink = synth.normal(g, H)
    pos = np.sort(g.integers(0, m * ccap + 40, size=(B, Tq)), axis=1).astype(np.int32)
    pos[0, 0] = 5                                          # a short row: few of the splits
    topk = None
    if sparse:
        vis = np.minimum((pos.reshape(-1) + 1) // m, ccap)
        topk = synth.topk_lists(g, vis, k, B * Tq).reshape(B, Tq, k)
    got, ref = run_attention(sparse, q, qfmt, pos, topk, comp, cfmt, win, cfmt, None, sink, d, dr, W, m, ofmt,
                             nan_ws=True)
    assert np.all(np.isfinite(got))
    report(f"attention NaN workspace c{ci}", abs=abs_err(got, ref), norm_rel=norm_rel(got, ref))
    assert abs_err(got, ref) <= 2e-2
    assert norm_rel(got, ref) <= BF16_NORM_REL


@pytest.mark.parametrize("sink", [-np.inf, 0.0, 30.0])
def test_attention_sink_edges(sink):
    g = synth.rng(650)
    B, Tq, H, d, dr, W, m, ccap = 1, 4, 8, 128, 64, 3, 4, 16
    comp, win = build_caches(g, B, ccap, W + Tq + 2, d, dr, O.F32, O.F32)
    q = synth.normal(g, (B, Tq, H, d))
    pos = np.array([[0, 1, 5, 60]], np.int32)
    sk = np.full(H, sink, np.float32)
    got, ref = run_attention(False, q, O.F32, pos, None, comp, O.F32, win, O.F32, None, sk, d, dr, W, m, O.F32)
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) <= 1e-4 or abs_err(got, ref) < 1e-12


def test_attention_deterministic_and_batch_invariant():
    g = synth.rng(660)
    B, Tq, H, d, dr, W, m, ccap = 3, 1, 32, 512, 64, 128, 128, 700
    comp, win = build_caches(g, B, ccap, W + 8, d, dr, O.FP8_E4M3, O.FP8_E4M3)
    q = synth.normal(g, (B, Tq, H, d))
    qb = dev_bf16((q.view(np.uint32) >> 16).astype(np.uint16))
    pos = np.full((B, Tq), 128 * ccap - 1, np.int32)
    sink = synth.normal(g, H)
    p = api.attn_params(d, dr, W, m)
    cc = api.KVCache(B, ccap, d, dr, O.FP8_E4M3, rec=dev(comp))
    wc = api.KVCache(B, W + 8, d, dr, O.FP8_E4M3, ring=True, rec=dev(win))
    a = api.hca_dense_mqa_attn(qb, dev(pos), cc, wc, dev(sink), p)
    b = api.hca_dense_mqa_attn(qb, dev(pos), cc, wc, dev(sink), p)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c1 = api.KVCache(1, ccap, d, dr, O.FP8_E4M3, rec=dev(comp[2:3]))
    w1 = api.KVCache(1, W + 8, d, dr, O.FP8_E4M3, ring=True, rec=dev(win[2:3]))
    c = api.hca_dense_mqa_attn(qb[2:3], dev(pos[2:3]), c1, w1, dev(sink), p)
    assert torch.equal(c[0].view(torch.int16), a[2].view(torch.int16))


def test_sparse_attention_deterministic_and_batch_invariant():
    """The CSA path (top-k lists, FP8 records, decode splits): two runs are
    bitwise equal, and a sequence computed alone equals the same sequence
    computed inside a batch."""
    g = synth.rng(661)
    B, Tq, H, d, dr, W, m, ccap, k = 3, 1, 64, 512, 64, 128, 4, 6000, 1024
    comp, win = build_caches(g, B, ccap, W + 8, d, dr, O.FP8_E4M3, O.FP8_E4M3)
    q = synth.normal(g, (B, Tq, H, d))
    qb = dev_bf16((q.view(np.uint32) >> 16).astype(np.uint16))
    pos = np.array([[m * ccap - 1], [m * 3000 + 1], [m * ccap + 17]], np.int32)
    vis = np.minimum((pos.reshape(-1) + 1) // m, ccap)
    topk = synth.topk_lists(g, vis, k, B * Tq).reshape(B, Tq, k)
    sink = synth.normal(g, H)
    p = api.attn_params(d, dr, W, m)
    cc = api.KVCache(B, ccap, d, dr, O.FP8_E4M3, rec=dev(comp))
    wc = api.KVCache(B, W + 8, d, dr, O.FP8_E4M3, ring=True, rec=dev(win))
    say("sparse attention determinism / batch invariance")
    a = api.sparse_mqa_attn(qb, dev(pos), dev(topk), cc, wc, dev(sink), p)
    b = api.sparse_mqa_attn(qb, dev(pos), dev(topk), cc, wc, dev(sink), p)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for i in range(B):
        c1 = api.KVCache(1, ccap, d, dr, O.FP8_E4M3, rec=dev(comp[i:i + 1]))
        w1 = api.KVCache(1, W + 8, d, dr, O.FP8_E4M3, ring=True, rec=dev(win[i:i + 1]))
        c = api.sparse_mqa_attn(qb[i:i + 1], dev(pos[i:i + 1]), dev(topk[i:i + 1]), c1, w1, dev(sink), p)
        assert torch.equal(c[0].view(torch.int16), a[i].view(torch.int16))


def test_attention_workgroups_running_several_splits_are_bit_exact():
    """At 32 sequences the decode splits outnumber the workgroups the chip
    holds (32 rows x 36 splits of the 1,152 entries), so each workgroup runs
    several splits of its row in turn; every row must equal, bit for bit, the
    same row computed alone (36 workgroups, one split each), for the sparse
    and the dense path."""
    g = synth.rng(663)
    B, H, d, dr, W, m, ccap, k = 32, 64, 512, 64, 128, 4, 2048, 1024
    comp, win = build_caches(g, B, ccap, W + 8, d, dr, O.FP8_E4M3, O.FP8_E4M3)
    q = synth.normal(g, (B, 1, H, d))
    qb = dev_bf16((q.view(np.uint32) >> 16).astype(np.uint16))
    pos = (m * ccap - 1 - 3 * np.arange(B, dtype=np.int32)).reshape(B, 1)
    vis = np.minimum((pos.reshape(-1) + 1) // m, ccap)
    topk = synth.topk_lists(g, vis, k, B).reshape(B, 1, k)
    sink = synth.normal(g, H)
    cc = api.KVCache(B, ccap, d, dr, O.FP8_E4M3, rec=dev(comp))
    wc = api.KVCache(B, W + 8, d, dr, O.FP8_E4M3, ring=True, rec=dev(win))
    # dense rows: m = 128 over the same 2,048-record caches (~2,176 entries, 34 splits)
    pos_d = (128 * ccap - 1 - 3 * np.arange(B, dtype=np.int32)).reshape(B, 1)
    for dense in (False, True):
        p = api.attn_params(d, dr, W, 128 if dense else m)
        if dense:
            pos = pos_d
        say(f"several splits per workgroup, dense={dense}")
        if dense:
            a = api.hca_dense_mqa_attn(qb, dev(pos), cc, wc, dev(sink), p)
        else:
            a = api.sparse_mqa_attn(qb, dev(pos), dev(topk), cc, wc, dev(sink), p)
        for i in (0, 1, 13, 31):
            c1 = api.KVCache(1, ccap, d, dr, O.FP8_E4M3, rec=dev(comp[i:i + 1]))
            w1 = api.KVCache(1, W + 8, d, dr, O.FP8_E4M3, ring=True, rec=dev(win[i:i + 1]))
            if dense:
                c = api.hca_dense_mqa_attn(qb[i:i + 1], dev(pos[i:i + 1]), c1, w1, dev(sink), p)
            else:
                c = api.sparse_mqa_attn(qb[i:i + 1], dev(pos[i:i + 1]), dev(topk[i:i + 1]), c1, w1, dev(sink), p)
            assert torch.equal(c[0].view(torch.int16), a[i].view(torch.int16)), (dense, i)


@pytest.mark.parametrize("fmt", [O.F32, O.BF16, O.FP8_E4M3])
def test_sparse_with_every_block_equals_dense(fmt):
    """CSA with a top-k list holding every visible block, in ascending order,
    is the HCA dense attention at the same m (the full-top-k identity, GPU
    against GPU).  Rows whose visible count equals k take identical entry
    lists and must agree bit for bit; rows with fewer visible blocks than k
    carry -1 padding and agree within rounding."""
    g = synth.rng(662 + fmt)
    B, Tq, H, d, dr, W, m, ccap = 2, 3, 64 if fmt != O.F32 else 8, 512 if fmt != O.F32 else 128, 64, 128, 4, 700
    comp, win = build_caches(g, B, ccap, W + Tq + 7, d, dr, fmt, fmt)
    q = synth.normal(g, (B, Tq, H, d))
    qfmt = O.F32 if fmt == O.F32 else O.BF16
    if qfmt == O.BF16:
        qdev = dev_bf16((q.view(np.uint32) >> 16).astype(np.uint16))
    else:
        qdev = dev(q)
    pos = np.array([[m * ccap - 1, m * ccap - 1, m * 300 + 2], [m * ccap - 1, 5, m * ccap + 40]], np.int32)
    vis = np.minimum((pos + 1) // m, ccap)
    k = ccap
    topk = np.full((B, Tq, k), -1, np.int32)
    for b in range(B):
        for i in range(Tq):
            topk[b, i, :vis[b, i]] = np.arange(vis[b, i])
    sink = synth.normal(g, H)
    p = api.attn_params(d, dr, W, m)
    cc = api.KVCache(B, ccap, d, dr, fmt, rec=dev(comp))
    wc = api.KVCache(B, W + Tq + 7, d, dr, fmt, ring=True, rec=dev(win))
    say(f"full top-k vs dense fmt={fmt}")
    od = torch.float32 if fmt == O.F32 else torch.bfloat16
    sp = api.sparse_mqa_attn(qdev, dev(pos), dev(topk), cc, wc, dev(sink), p, out_dtype=od)
    de = api.hca_dense_mqa_attn(qdev, dev(pos), cc, wc, dev(sink), p, out_dtype=od)
    torch.cuda.synchronize()
    full = torch.from_numpy(vis == k).cuda()
    assert int(full.sum()) == 4
    assert torch.equal(sp[full].float(), de[full].float())
    a, b = out_to_f64(sp), out_to_f64(de)
    report(f"full top-k vs dense fmt={fmt}", max_rel=rel_err(a, b), norm_rel=norm_rel(a, b))
    if fmt == O.F32:
        assert rel_err(a, b) <= 1e-5
    else:
        assert abs_err(a, b) <= 2e-2 and norm_rel(a, b) <= BF16_NORM_REL


def test_relative_position_invariance_f32():
    """Shifting every position by a multiple of m (the block structure kept)
    leaves the CSA output unchanged: the caches are written by the GPU's own
    compression at both offsets, the top-k lists shift by the same number of
    blocks, and the outputs must agree to 1e-4 (f32)."""
    g = synth.rng(663)
    T, H, d, dr, W, m, k = 640, 8, 128, 64, 128, 4, 48
    x = synth.normal(g, (1, T, d))
    q = synth.normal(g, (1, 6, H, d))
    gam = (1 + 0.3 * synth.normal(g, d)).astype(np.float32)
    gk = (1 + 0.3 * synth.normal(g, d)).astype(np.float32)
    b = synth.normal(g, m)
    sink = synth.normal(g, H)
    t = np.array([[W - 1, 200, 333, 401, 598, T - 1]], np.int32)
    vis = (t.reshape(-1) + 1) // m
    top0 = synth.topk_lists(g, vis, k, t.size).reshape(1, 6, k)
    outs = []
    for shift in (0, 4 * 250_000, 4 * 262_143):
        nblk = (shift + T) // m
        comp = api.KVCache(1, nblk, d, dr, O.F32)
        win = api.KVCache(1, W + 8, d, dr, O.F32, ring=True)
        say(f"position shift {shift}")
        api.compress_kv(dev(x), dev(np.array([shift], np.int32)), m, dev(b), gamma=dev(gk), rope_dim=dr, kv_out=comp)
        api.compress_kv(dev(x[:, T - W - 8:]), dev(np.array([shift + T - W - 8], np.int32)), 1,
                        dev(np.zeros(1, np.float32)), gamma=dev(gk), rope_dim=dr, kv_out=win)
        top = np.where(top0 >= 0, top0 + shift // m, -1).astype(np.int32)
        # the window ring holds positions shift + T - W - 8 .. shift + T - 1: queries at the last
        # position only see raw entries inside it; earlier queries see none of them beyond t
        o = api.sparse_mqa_attn(dev(q[:, -1:]), dev(t[:, -1:] + shift), dev(top[:, -1:]), comp, win, dev(sink),
                                api.attn_params(d, dr, W, m), gamma_q=dev(gam))
        p0 = api.attn_params(d, dr, 0, m)
        o2 = api.sparse_mqa_attn(dev(q[:, :-1]), dev(t[:, :-1] + shift), dev(top[:, :-1]), comp, win, dev(sink), p0,
                                 gamma_q=dev(gam))
        torch.cuda.synchronize()
        outs.append(np.concatenate([out_to_f64(o2), out_to_f64(o)], axis=1))
    for o in outs[1:]:
        report("position shift (f32)", max_rel=rel_err(o, outs[0]))
        assert rel_err(o, outs[0]) <= 1e-4


# ====================================================================== projection
@pytest.mark.parametrize("M,H,d,D,G,fmt", [(2048, 8, 128, 1024, 8, O.F32), (4, 64, 512, 7168, 8, O.BF16),
                                           (16, 32, 512, 4096, 8, O.BF16), (37, 6, 40, 96, 3, O.F32),
                                           (1, 16, 256, 1024, 4, O.F32), (8, 64, 512, 7168, 8, O.BF16),
                                           (2, 8, 128, 384, 2, O.BF16), (3, 8, 64, 200, 8, O.BF16),
                                           # bf16 with M > 16 runs on the matrix cores: a ragged 256-row
                                           # tile, ragged 128-column tiles (D/G = 200), a single 32-wide
                                           # slab, and the prefill chunk's grouping at a smaller M
                                           (300, 16, 128, 1024, 8, O.BF16), (40, 8, 64, 1600, 8, O.BF16),
                                           (17, 4, 32, 96, 4, O.BF16), (600, 64, 512, 7168, 8, O.BF16),
                                           # group widths that are not a whole 16-byte vector (scalar kernel)
                                           (5, 3, 20, 60, 3, O.BF16), (45, 3, 20, 60, 3, O.BF16),
                                           # the skinny matrix-core path (4 < M <= 64): row blocks of 16
                                           # with a ragged last block, ragged 16-column blocks
                                           (33, 8, 256, 520, 4, O.BF16), (64, 16, 128, 1024, 8, O.BF16),
                                           (32, 32, 512, 4096, 8, O.BF16)])
def test_projection_parity(M, H, d, D, G, fmt):
    g = synth.rng(700 + M)
    Hd = H * d
    o = synth.normal(g, (M, Hd))
    W = synth.normal(g, (G, D // G, Hd // G)) * np.float32(0.02)
    say(f"projection M={M} Hd={Hd} D={D} G={G} fmt={fmt}")
    if fmt == O.BF16:
        ob = (o.view(np.uint32) >> 16).astype(np.uint16)
        Wb = (W.view(np.uint32) >> 16).astype(np.uint16)
        y = api.out_proj_grouped(dev_bf16(ob), dev_bf16(Wb), y_dtype=torch.float32)
        ref = O.out_proj(O.bf16_decode(ob), O.bf16_decode(Wb))
    else:
        y = api.out_proj_grouped(dev(o), dev(W))
        ref = O.out_proj(o.astype(np.float64), W.astype(np.float64))
    torch.cuda.synchronize()
    assert rel_err(out_to_f64(y), ref) <= 1e-5


def test_projection_mfma_bf16_out():
    """The matrix-core projection with a bf16 output: each element is the fp32
    sum rounded once to bf16 (within half a bf16 ulp of the exact value, plus
    the fp32 accumulation error)."""
    g = synth.rng(790)
    M, Hd, D, G = 333, 2048, 1024, 8
    ob = synth.bf16_bits(g, (M, Hd))
    Wb = (synth.normal(g, (G, D // G, Hd // G)).astype(np.float32) * np.float32(0.05)).view(np.uint32)
    Wb = (Wb >> 16).astype(np.uint16)
    say(f"projection bf16 out M={M} Hd={Hd} D={D} G={G}")
    y = api.out_proj_grouped(dev_bf16(ob), dev_bf16(Wb), y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = O.out_proj(O.bf16_decode(ob), O.bf16_decode(Wb))
    got = out_to_f64(y)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-5 * np.max(np.abs(ref)))


# ====================================================================== end to end (C1 shape)
def test_csa_layer_c1_end_to_end_grid():
    """Single CSA layer, fp32, batch 1, causal prefill of 2048 tokens: 8 heads
    x 128, m = 4, top-k 64, window 128, sink 0, indexer 4 x 64, grouped
    projection 1024 -> 1024 in 8 groups.  Indexer inputs on the 1/8 grid with
    uniform indexer pooling make every score exact, so the chain must match
    the oracle's chain (attention to 1e-4)."""
    g = synth.rng(2001)
    T, H, d, dr, m, k, W, Hi, di, D, G = 2048, 8, 128, 64, 4, 64, 128, 4, 64, 1024, 8
    x = synth.normal(g, (1, T, d))
    xI = synth.grid(g, (1, T, di))
    q = synth.normal(g, (1, T, H, d))
    qI = synth.grid(g, (1, T, Hi, di))
    w = synth.grid(g, (1, T, Hi))
    b = synth.normal(g, m)
    bI = np.zeros(m, np.float32)
    sink = np.zeros(H, np.float32)
    Wo = (synth.normal(g, (G, D // G, H * d // G)) / np.float32(math.sqrt(H * d // G))).astype(np.float32)
    gam = np.ones(d, np.float32)
    pos = np.arange(T, dtype=np.int32)[None]
    say("c1 end-to-end")
    comp = api.KVCache(1, T // m, d, dr, O.F32)
    win = api.KVCache(1, W + T, d, dr, O.F32, ring=True)
    keys = api.IdxCache(1, T // m, di, O.F32)
    z = dev(np.zeros(1, np.int32))
    api.compress_kv(dev(x), z, m, dev(b), gamma=dev(gam), rope_dim=dr, kv_out=comp)
    api.compress_kv(dev(x), z, 1, dev(np.zeros(1, np.float32)), gamma=dev(gam), rope_dim=dr, kv_out=win)
    api.compress_kv(dev(xI), z, m, dev(bI), idx_out=keys)
    top = api.indexer_topk(dev(f32_rows(qI)), O.F32, dev(w), keys, dev(pos), m, k)
    o = api.sparse_mqa_attn(dev(q), dev(pos), top, comp, win, dev(sink), api.attn_params(d, dr, W, m))
    y = api.out_proj_grouped(o.reshape(T, H * d), dev(Wo))
    torch.cuda.synchronize()
    # oracle chain
    oc, _, _ = O.compress(x, O.F32, [0], m, b, gamma=gam, dr=dr, out_kind=0, out_fmt=O.F32, cap=T // m)
    ow, _, _ = O.compress(x, O.F32, [0], 1, [0.0], gamma=gam, dr=dr, out_kind=0, out_fmt=O.F32, cap=W + T, ring=True)
    ok, _, _ = O.compress(xI, O.F32, [0], m, bI, out_kind=1, out_fmt=O.F32, cap=T // m)
    otop = O.indexer_topk(f32_rows(qI[0]), None, O.F32, w[0], pos[0], ok[0], None, O.F32, m, k)
    assert np.array_equal(top.cpu().numpy()[0], otop)
    oo = O.attention(q[0], O.F32, pos[0], gam, sink, d, dr, W, m, 10000.0, 1 / math.sqrt(d), 1e-6, oc[0], O.F32,
                     ow[0], O.F32, otop)
    assert rel_err(out_to_f64(o)[0], oo) <= 1e-4
    oy = O.out_proj(oo.reshape(T, H * d), Wo.astype(np.float64))
    assert rel_err(out_to_f64(y), oy) <= 1e-4
