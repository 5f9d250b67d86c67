"""Benchmark: one decode step of an alternating CSA / HCA layer pair at a
1,048,576-token context (DeepSeek-V4-Pro shape), batch 4, on one MI355X.

A step is the whole hot path for one new token per sequence:
  CSA layer: window append (m=1) + the new token folded into its 4-token
             block's pooling state, which completes the block (FP8 entry),
             and likewise into its indexer key (FP4) + indexer top-1024 over
             262,144 blocks + sparse MQA (64 heads x 512, 1024 blocks + 128
             window, FP8 cache) + grouped output projection 32768 -> 7168
             (8 groups)
  HCA layer: window append + the new token completing its 128-token block
             from the pooling state + dense MQA over 8,192 entries + window +
             grouped output projection.
The timed step is the one whose token completes a block in both layers (the
position L - 1); the pooling states hold the blocks' earlier tokens, folded
in by the per-token compression call before timing.
Inputs are resident in HBM before timing; R copies of every cache, weight and
workspace are rotated so that consecutive reuse of a buffer is separated by
more traffic than the 256 MB last-level cache holds.

Prints one JSON line (metric, value = query tokens per second, roofline of the
dominant kernel from HIP events, CPU-oracle baseline on the host cores).

Profiling helpers (the summaries under profiles/ are made with these):
  --copy-calibration       a plain 1 GiB device copy, three times (the
                           reference for FETCH_SIZE / WRITE_SIZE scaling);
  --summarize DIR          per-kernel duration summary of a rocprofv3
                           --kernel-trace run written under DIR;
  --summarize-pmc DIR ...  per-call sums of the counters of rocprofv3 --pmc
                           runs of this benchmark (one counter per run);
  --summarize-prefill DIR  per-call kernel durations of the prefill section;
  --summarize-pmc-kernels DIR ...
                           per-kernel counter means with MFMA / VALU busy;
  --summarize-launches DIR ...
                           per kernel and grid: trace durations and counter
                           means (tells apart launches of one kernel over
                           different problem sizes).
"""
import glob
import hashlib
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA/HCA attention query-tokens/s at 1M ctx; decode HBM GB/s & prefill MFMA %"
HBM_PEAK_GBS = 8000.0

# workload: 1M-context layer pair decode, V4-Pro shaped
B, L, H, D_HEAD, DR, W = 4, 1 << 20, 64, 512, 64, 128
HIDDEN, G = 7168, 8
M_CSA, K_CSA, M_HCA = 4, 1024, 128
HI, DI = 4, 64
N_CSA, N_HCA = L // M_CSA, L // M_HCA
REC = 592                      # FP8 record bytes (448 E4M3 + 64 bf16 + f32 scale + pad)
REC_ALGO = 580


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=6, help="rotated buffer sets (defeats the last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk measurement")
    ap.add_argument("--prefill-only", action="store_true", help="only the prefill-chunk measurement (for profiling)")
    ap.add_argument("--no-decode-configs", action="store_true", help="skip the HCA b16 / CSA b32 decode workloads")
    ap.add_argument("--no-layer-proj", action="store_true", help="skip the FP8-weight projection measurement")
    ap.add_argument("--layer-proj-only", action="store_true", help="only the FP8-weight projections (for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-prefill-seconds", type=float, default=25.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--summarize-pmc", metavar="DIR", nargs="+")
    ap.add_argument("--summarize-prefill", metavar="DIR")
    ap.add_argument("--summarize-pmc-kernels", metavar="DIR", nargs="+")
    ap.add_argument("--summarize-pmc-dispatches", metavar="DIR", nargs="+",
                    help="per-dispatch counter sums of k_attn_mfma in launch order (one counter per run)")
    ap.add_argument("--summarize-launches", metavar="DIR", nargs="+",
                    help="per kernel and grid: trace durations and counter means of trace / --pmc runs")
    return ap.parse_args()


def algorithmic_bytes():
    """Bytes the method itself must move per step, per call (sizes of the
    inputs read and outputs written, each once)."""
    q = B * H * D_HEAD * 2
    o = B * H * D_HEAD * 2
    win = B * W * REC_ALGO
    return {
        "csa_compress_kv": B * (D_HEAD * 2 + (D_HEAD + 2) * 4 + DI * 2 + (DI + 2) * 4) + 2 * B * REC_ALGO
                           + B * (DI // 2 + DI // 32),
        "csa_indexer_topk": B * N_CSA * (DI // 2 + DI // 32) + B * HI * (DI // 2 + DI // 32 + 4) + B * K_CSA * 4,
        "csa_sparse_mqa_attn": q + B * K_CSA * REC_ALGO + win + o + B * K_CSA * 4,
        "csa_out_proj": G * (HIDDEN // G) * (H * D_HEAD // G) * 2 + B * H * D_HEAD * 2 + B * HIDDEN * 2,
        "hca_compress_kv": B * (D_HEAD * 2 + (D_HEAD + 2) * 4) + 2 * B * REC_ALGO,
        "hca_dense_mqa_attn": q + B * N_HCA * REC_ALGO + win + o,
        "hca_out_proj": G * (HIDDEN // G) * (H * D_HEAD // G) * 2 + B * H * D_HEAD * 2 + B * HIDDEN * 2,
    }


def build_state(torch, api, copies, seed=4004):
    """Caches, weights and per-step inputs, R copies.  The prefix caches are
    made by the library's own compression call from seeded random raw tokens."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn(*shape, std=1.0, dtype=torch.bfloat16):
        return (torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32) * std).to(dtype)

    b_csa = randn(M_CSA, dtype=torch.float32)
    b_idx = randn(M_CSA, dtype=torch.float32)
    b_hca = torch.zeros(M_HCA, device=dev)
    gam = torch.ones(D_HEAD, device=dev)
    csa_c = api.KVCache(B, N_CSA, D_HEAD, DR, api.FP8_E4M3)
    hca_c = api.KVCache(B, N_HCA, D_HEAD, DR, api.FP8_E4M3)
    keys = api.IdxCache(B, N_CSA, DI, api.FP4_E2M1)
    wins = [api.KVCache(B, W, D_HEAD, DR, api.FP8_E4M3, ring=True) for _ in range(2)]
    chunk = 1 << 16
    for c0 in range(0, L, chunk):
        start = torch.full((B,), c0, dtype=torch.int32, device=dev)
        x = randn(B, chunk, D_HEAD)
        api.compress_kv(x, start, M_CSA, b_csa, gamma=gam, rope_dim=DR, kv_out=csa_c)
        xi = randn(B, chunk, DI)
        api.compress_kv(xi, start, M_CSA, b_idx, idx_out=keys)
        x = randn(B, chunk, D_HEAD)
        api.compress_kv(x, start, M_HCA, b_hca, gamma=gam, rope_dim=DR, kv_out=hca_c)
        if c0 + chunk == L:
            ws = torch.full((B,), L - W, dtype=torch.int32, device=dev)
            for wc in wins:
                api.compress_kv(x[:, chunk - W:].contiguous(), ws, 1, torch.zeros(1, device=dev), gamma=gam,
                                rope_dim=DR, kv_out=wc)
    torch.cuda.synchronize()
    t = L - 1
    sets = []
    for r in range(copies):
        s = {}
        if r == 0:
            s["csa_c"], s["hca_c"], s["keys"], s["win_csa"], s["win_hca"] = csa_c, hca_c, keys, wins[0], wins[1]
        else:
            s["csa_c"] = api.KVCache(B, N_CSA, D_HEAD, DR, api.FP8_E4M3, rec=csa_c.rec.clone())
            s["hca_c"] = api.KVCache(B, N_HCA, D_HEAD, DR, api.FP8_E4M3, rec=hca_c.rec.clone())
            s["keys"] = api.IdxCache(B, N_CSA, DI, api.FP4_E2M1, codes=keys.codes.clone(), scales=keys.scales.clone())
            s["win_csa"] = api.KVCache(B, W, D_HEAD, DR, api.FP8_E4M3, ring=True, rec=wins[0].rec.clone())
            s["win_hca"] = api.KVCache(B, W, D_HEAD, DR, api.FP8_E4M3, ring=True, rec=wins[1].rec.clone())
        s["Wo_csa"] = randn(G, HIDDEN // G, H * D_HEAD // G, std=0.02)
        s["Wo_hca"] = randn(G, HIDDEN // G, H * D_HEAD // G, std=0.02)
        # per-step inputs: the new token's raw KV (and the rest of its block), queries
        s["x_csa"] = randn(B, M_CSA, D_HEAD)
        s["xi_csa"] = randn(B, M_CSA, DI)
        s["x_hca"] = randn(B, M_HCA, D_HEAD)
        s["x_new_csa"] = s["x_csa"][:, M_CSA - 1].contiguous()
        s["xi_new_csa"] = s["xi_csa"][:, M_CSA - 1].contiguous()
        s["x_new_hca"] = s["x_hca"][:, M_HCA - 1].contiguous()
        # online pooling states of the blocks the step completes, holding the
        # blocks' earlier tokens (folded in below, one call per token)
        s["st_csa"] = torch.empty((B, D_HEAD + 2), dtype=torch.float32, device=dev)
        s["st_idx"] = torch.empty((B, DI + 2), dtype=torch.float32, device=dev)
        s["st_hca"] = torch.empty((B, D_HEAD + 2), dtype=torch.float32, device=dev)
        for r_ in range(M_HCA - 1):
            pos_r = lambda m: torch.full((B,), t + 1 - m + r_, dtype=torch.int32, device=dev)
            jobs = [dict(x=s["x_hca"][:, r_].contiguous(), tok_pos=pos_r(M_HCA), m=M_HCA, score_bias=b_hca,
                         state=s["st_hca"], gamma=gam, rope_dim=DR, kv_out=s["hca_c"])]
            if r_ < M_CSA - 1:
                jobs += [dict(x=s["x_csa"][:, r_].contiguous(), tok_pos=pos_r(M_CSA), m=M_CSA, score_bias=b_csa,
                              state=s["st_csa"], gamma=gam, rope_dim=DR, kv_out=s["csa_c"]),
                         dict(x=s["xi_csa"][:, r_].contiguous(), tok_pos=pos_r(M_CSA), m=M_CSA, score_bias=b_idx,
                              state=s["st_idx"], idx_out=s["keys"])]
            api.compress_kv_step(jobs)
        s["q_csa"] = randn(B, 1, H, D_HEAD)
        s["q_hca"] = randn(B, 1, H, D_HEAD)
        qc = torch.randint(0, 256, (B, 1, HI, DI // 2), generator=gen, device=dev, dtype=torch.int32).to(torch.uint8)
        qs = torch.randint(124, 128, (B, 1, HI, DI // 32), generator=gen, device=dev, dtype=torch.int32).to(torch.uint8)
        s["qI"], s["qI_s"] = qc, qs
        s["w_idx"] = randn(B, 1, HI, dtype=torch.float32)
        s["sink_csa"] = randn(H, dtype=torch.float32)
        s["sink_hca"] = randn(H, dtype=torch.float32)
        s["top"] = torch.empty((B, 1, K_CSA), dtype=torch.int32, device=dev)
        s["idx_ws"] = torch.empty(api.indexer_workspace_bytes(B, 1, N_CSA, K_CSA), dtype=torch.uint8, device=dev)
        s["o_csa"] = torch.empty((B, 1, H, D_HEAD), dtype=torch.bfloat16, device=dev)
        s["o_hca"] = torch.empty((B, 1, H, D_HEAD), dtype=torch.bfloat16, device=dev)
        s["y_csa"] = torch.empty((B, HIDDEN), dtype=torch.bfloat16, device=dev)
        s["y_hca"] = torch.empty((B, HIDDEN), dtype=torch.bfloat16, device=dev)
        s["attn_ws_csa"] = torch.empty(max(1, api.attn_workspace_bytes(B, 1, H, D_HEAD, K_CSA, W, api.BF16, api.FP8_E4M3)),
                                       dtype=torch.uint8, device=dev)
        s["attn_ws_hca"] = torch.empty(max(1, api.attn_workspace_bytes(B, 1, H, D_HEAD, N_HCA, W, api.BF16, api.FP8_E4M3)),
                                       dtype=torch.uint8, device=dev)
        sets.append(s)
    shared = dict(
        b_csa=b_csa, b_idx=b_idx, b_hca=b_hca, gam=gam, zero1=torch.zeros(1, device=dev),
        pos=torch.full((B, 1), t, dtype=torch.int32, device=dev),
        tok_new=torch.full((B,), t, dtype=torch.int32, device=dev),
        p_csa=api.attn_params(D_HEAD, DR, W, M_CSA), p_hca=api.attn_params(D_HEAD, DR, W, M_HCA))
    torch.cuda.synchronize()
    return sets, shared


CALLS = ["csa_compress_kv", "csa_indexer_topk", "csa_sparse_mqa_attn", "csa_out_proj",
         "hca_compress_kv", "hca_dense_mqa_attn", "hca_out_proj"]

# the kernels each call launches, in launch order (for matching rocprof traces)
CALL_KERNELS = {
    "csa_compress_kv": ["k_compress_step"],
    "csa_indexer_topk": ["k_idxd_filter", "k_idxd_select"],
    "csa_sparse_mqa_attn": ["k_attn_mfma", "k_attn_combine"],
    "csa_out_proj": ["k_proj_gemv"],
    "hca_compress_kv": ["k_compress_step"],
    "hca_dense_mqa_attn": ["k_attn_mfma", "k_attn_combine"],
    "hca_out_proj": ["k_proj_gemv"],
}


def call_fns(api):
    """One function per call of the decode step (each launches that call's kernels)."""
    # the step's three CSA compressions (window entry, the block's last token,
    # the indexer key's last token) and two HCA ones are each one per-token call
    def c0(s, sh):
        api.compress_kv_step([
            dict(x=s["x_new_csa"], tok_pos=sh["tok_new"], m=1, score_bias=sh["zero1"], gamma=sh["gam"],
                 rope_dim=DR, kv_out=s["win_csa"]),
            dict(x=s["x_new_csa"], tok_pos=sh["tok_new"], m=M_CSA, score_bias=sh["b_csa"], state=s["st_csa"],
                 gamma=sh["gam"], rope_dim=DR, kv_out=s["csa_c"]),
            dict(x=s["xi_new_csa"], tok_pos=sh["tok_new"], m=M_CSA, score_bias=sh["b_idx"], state=s["st_idx"],
                 idx_out=s["keys"])])

    def c1(s, sh):
        api.indexer_topk(s["qI"], api.FP4_E2M1, s["w_idx"], s["keys"], sh["pos"], M_CSA, K_CSA, q_scales=s["qI_s"],
                         out=s["top"], workspace=s["idx_ws"])

    def c2(s, sh):
        api.sparse_mqa_attn(s["q_csa"], sh["pos"], s["top"], s["csa_c"], s["win_csa"], s["sink_csa"], sh["p_csa"],
                            out=s["o_csa"], workspace=s["attn_ws_csa"])

    def c3(s, sh):
        api.out_proj_grouped(s["o_csa"].view(B, H * D_HEAD), s["Wo_csa"], y=s["y_csa"])

    def c4(s, sh):
        api.compress_kv_step([
            dict(x=s["x_new_hca"], tok_pos=sh["tok_new"], m=1, score_bias=sh["zero1"], gamma=sh["gam"],
                 rope_dim=DR, kv_out=s["win_hca"]),
            dict(x=s["x_new_hca"], tok_pos=sh["tok_new"], m=M_HCA, score_bias=sh["b_hca"], state=s["st_hca"],
                 gamma=sh["gam"], rope_dim=DR, kv_out=s["hca_c"])])

    def c5(s, sh):
        api.hca_dense_mqa_attn(s["q_hca"], sh["pos"], s["hca_c"], s["win_hca"], s["sink_hca"], sh["p_hca"],
                               out=s["o_hca"], workspace=s["attn_ws_hca"])

    def c6(s, sh):
        api.out_proj_grouped(s["o_hca"].view(B, H * D_HEAD), s["Wo_hca"], y=s["y_hca"])

    return [c0, c1, c2, c3, c4, c5, c6]


# prefill chunk: 8,192 new query tokens of one sequence over a 1,048,576-token
# prefix (the chunk's own blocks included), m = 4, top-1024, FP4 indexer,
# FP8 records, 64 heads x 512 -- reported beside the decode line
PF_T, PF_TOPK = 8192, 1024
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense FP4 (the indexer runs the FP4 MFMA)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16


def _pctl(ts):
    """median, p10 and p90 (ms) of a list of event times."""
    return {"median": round(float(np.median(ts)), 4), "p10": round(float(np.percentile(ts, 10)), 4),
            "p90": round(float(np.percentile(ts, 90)), 4)}


def _timed(torch, f, reps, flush=None):
    """Event times (ms) of f over reps runs after one warm-up; flush() (an
    L2 / last-level-cache eviction) runs before each, outside the events."""
    f()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        f()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return ts


def _compressed_prefix(torch, api, gen, ntok, caches, chunk=1 << 16):
    """Fill caches with the library's own compression of seeded N(0,1) raw
    tokens at positions 0 .. ntok-1: caches = [(cache, m, bias, kind)], kind
    0 a KV cache (RMSNorm + RoPE), 1 an indexer-key cache (no norm)."""
    dev = "cuda"
    gam = torch.ones(D_HEAD, device=dev)
    for c0 in range(0, ntok, chunk):
        n = min(chunk, ntok - c0)
        start = torch.full((caches[0][0].B,), c0, dtype=torch.int32, device=dev)
        x = xi = None
        for cache, m, bias, kind in caches:
            if kind == 0:
                if x is None:
                    x = torch.randn(cache.B, n, D_HEAD, generator=gen, device=dev).to(torch.bfloat16)
                api.compress_kv(x, start, m, bias, gamma=gam, rope_dim=DR, kv_out=cache)
            else:
                if xi is None:
                    xi = torch.randn(cache.B, n, DI, generator=gen, device=dev).to(torch.bfloat16)
                api.compress_kv(xi, start, m, bias, idx_out=cache)
    torch.cuda.synchronize()


def fp4_queries(torch, api, gen, B, T, Hi):
    """FP4 indexer queries quantised by the library from an N(0,1) draw:
    every (b, t, h) row of di values is one FP4 row (E2M1 codes, E8M0 scales
    per 32)."""
    x = torch.randn(1, B * T * Hi, DI, generator=gen, device="cuda").to(torch.bfloat16)
    c = api.IdxCache(1, B * T * Hi, DI, api.FP4_E2M1)
    api.compress_kv(x, torch.zeros(1, dtype=torch.int32, device="cuda"), 1, torch.zeros(1, device="cuda"), idx_out=c)
    torch.cuda.synchronize()
    return c.codes.view(B, T, Hi, DI // 2), c.scales.view(B, T, Hi, DI // 32)


def prefill_measure(torch, api, reps=10, seed=5005):
    """Times the indexer, the sparse attention and the grouped output
    projection of one prefill chunk, and the HCA layer's dense attention over
    the same chunk (events around each call; median, p10, p90 over reps runs
    after a warm-up), and prices their contractions against the MFMA peaks.
    Caches are the library's own compression of seeded N(0,1) raw tokens (RMS-
    normalised FP8 records, FP4 keys); the chunk's indexer queries are N(0,1)
    quantised to FP4 by the same quantiser."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    ntok = L + PF_T
    n = ntok // M_CSA
    n_h = ntok // M_HCA
    keys = api.IdxCache(1, n, DI, api.FP4_E2M1)
    comp = api.KVCache(1, n, D_HEAD, DR, api.FP8_E4M3)
    comp_h = api.KVCache(1, n_h, D_HEAD, DR, api.FP8_E4M3)
    b_csa = torch.randn(M_CSA, generator=gen, device=dev)
    b_idx = torch.randn(M_CSA, generator=gen, device=dev)
    _compressed_prefix(torch, api, gen, ntok, [(comp, M_CSA, b_csa, 0), (comp_h, M_HCA, torch.zeros(M_HCA, device=dev), 0),
                                              (keys, M_CSA, b_idx, 1)])
    win = api.KVCache(1, W + PF_T, D_HEAD, DR, api.FP8_E4M3, ring=True)
    xw = torch.randn(1, W + PF_T, D_HEAD, generator=gen, device=dev).to(torch.bfloat16)
    api.compress_kv(xw, torch.full((1,), L - W, dtype=torch.int32, device=dev), 1, torch.zeros(1, device=dev),
                    gamma=torch.ones(D_HEAD, device=dev), rope_dim=DR, kv_out=win)
    qc, qsc = fp4_queries(torch, api, gen, 1, PF_T, HI)
    w = torch.randn(1, PF_T, HI, generator=gen, device=dev)
    pos = (torch.arange(PF_T, device=dev, dtype=torch.int32) + L).view(1, PF_T)
    ws = torch.empty(api.indexer_workspace_bytes(1, PF_T, n, PF_TOPK), dtype=torch.uint8, device=dev)
    top = torch.empty(1, PF_T, PF_TOPK, dtype=torch.int32, device=dev)
    q = torch.randn(1, PF_T, H, D_HEAD, generator=gen, device=dev).to(torch.bfloat16)
    sink = torch.randn(H, generator=gen, device=dev)
    p = api.attn_params(D_HEAD, DR, W, M_CSA)
    out = torch.empty(1, PF_T, H, D_HEAD, dtype=torch.bfloat16, device=dev)
    aws = torch.empty(max(1, api.attn_workspace_bytes(1, PF_T, H, D_HEAD, PF_TOPK, W, api.BF16, api.FP8_E4M3)),
                      dtype=torch.uint8, device=dev)

    def idx():
        api.indexer_topk(qc, api.FP4_E2M1, w, keys, pos, M_CSA, PF_TOPK, q_scales=qsc, out=top, workspace=ws)

    def att():
        api.sparse_mqa_attn(q, pos, top, comp, win, sink, p, out=out, workspace=aws)

    # the HCA layer's prefill over the same chunk: every compressed entry of
    # the 1M prefix (m = 128) plus the window, dense
    p_h = api.attn_params(D_HEAD, DR, W, M_HCA)
    aws_h = torch.empty(max(1, api.attn_workspace_bytes(1, PF_T, H, D_HEAD, n_h, W, api.BF16, api.FP8_E4M3)),
                        dtype=torch.uint8, device=dev)
    out_h = torch.empty_like(out)

    def att_h():
        api.hca_dense_mqa_attn(q, pos, comp_h, win, sink, p_h, out=out_h, workspace=aws_h)

    # the chunk's grouped output projection: [8192, 64 x 512] -> [8192, 7168]
    wo = (torch.randn(G, HIDDEN // G, H * D_HEAD // G, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    y = torch.empty(PF_T, HIDDEN, dtype=torch.bfloat16, device=dev)

    def proj():
        api.out_proj_grouped(out.view(PF_T, H * D_HEAD), wo, y=y)

    ti, ta, th, tp = (_timed(torch, f, reps) for f in (idx, att, att_h, proj))
    mi, ma, mh, mp = (float(np.median(t)) for t in (ti, ta, th, tp))
    fi, fa, fh, fp = prefill_flops()
    return {"workload": "CSA prefill chunk, 8,192 queries over a 1M prefix, 64 heads x 512, top-1024, FP4 indexer, "
                        "FP8 records, grouped projection to 7,168; and the HCA layer's dense attention over the same "
                        "chunk (8,256 blocks + window); caches compressed by the library from N(0,1) tokens",
            "indexer_ms": _pctl(ti), "attn_ms": _pctl(ta), "proj_ms": _pctl(tp), "hca_attn_ms": _pctl(th),
            "query_tokens_per_s": round(PF_T / ((mi + ma + mp) * 1e-3), 1),
            "query_tokens_per_s_calls": "CSA indexer + sparse attention + projection (medians)",
            "indexer_TFLOPs": round(fi / (mi * 1e-3) / 1e12, 1),
            "indexer_mfma_frac": round(fi / (mi * 1e-3) / 1e12 / FP4_PEAK_TFLOPS, 4),
            "indexer_peak": "fp4 10.1 PFLOP/s",
            "attn_TFLOPs": round(fa / (ma * 1e-3) / 1e12, 1), "attn_mfma_frac": round(fa / (ma * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "attn_peak": "bf16 2.5 PFLOP/s",
            "hca_attn_TFLOPs": round(fh / (mh * 1e-3) / 1e12, 1),
            "hca_attn_mfma_frac": round(fh / (mh * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "proj_TFLOPs": round(fp / (mp * 1e-3) / 1e12, 1),
            "proj_mfma_frac": round(fp / (mp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "timing": f"HIP events around each call, median (p10, p90) of {reps} runs after a warm-up"}


def prefill_flops():
    """Algorithmic flops of the prefill chunk's calls: indexer q.k products,
    CSA attention (Q K^T and P V over top-k + window), HCA attention (every
    block of the prefix + window), grouped projection."""
    n_mean = (L + PF_T / 2) / M_CSA                       # blocks visible to the average query
    fi = 2.0 * PF_T * HI * DI * n_mean
    fa = 2.0 * PF_T * H * (PF_TOPK + W) * 2 * D_HEAD
    fh = 2.0 * PF_T * H * ((L + PF_T / 2) / M_HCA + W) * 2 * D_HEAD
    fp = 2.0 * PF_T * H * D_HEAD * (HIDDEN // G)
    return fi, fa, fh, fp


def decode_configs_measure(torch, api, reps=20, seed=6006):
    """The two other decode workloads, each one step per rep with L2 and the
    last-level cache evicted before it (a 1 GiB write outside the events):
      HCA decode, bf16, batch 16 at 65,536 tokens: window append + the token
        completing its 128-token block (per-token compression), dense attention over 512 entries + window (32 heads x
        512), grouped projection 16384 -> 4096 (8 groups);
      CSA decode, bf16, batch 32 at 131,072 tokens: window append + the token
        completing its block and its indexer key, indexer top-1024 over 32,768 bf16 keys, sparse
        attention over 1,024 entries + window (32 heads x 512), grouped
        projection 16384 -> 4096.
    Caches are the library's compression of seeded N(0,1) raw tokens.
    Returns per-call and per-step medians and the attention-side HBM rate."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device=dev)        # 1 GiB
    flush_out = torch.empty((), dtype=torch.int64, device=dev)

    def flush():
        # a read of 1 GiB: the caches end up holding clean lines of it, so the
        # timed kernel neither hits its own data nor pays for dirty write-backs
        torch.sum(flush_buf, dim=0, out=flush_out)

    res = {}
    Hq, hid = 32, 4096
    zero1 = torch.zeros(1, device=dev)
    gam = torch.ones(D_HEAD, device=dev)
    for name, Bc, Lc, m, sparse in (("hca_decode_b16_64k_bf16", 16, 65536, 128, False),
                                    ("csa_decode_b32_128k_bf16", 32, 131072, 4, True)):
        n = Lc // m
        t = Lc - 1
        comp = api.KVCache(Bc, n, D_HEAD, DR, api.BF16)
        win = api.KVCache(Bc, W, D_HEAD, DR, api.BF16, ring=True)
        bias = torch.randn(m, generator=gen, device=dev) if sparse else torch.zeros(m, device=dev)
        caches = [(comp, m, bias, 0)]
        keys = None
        if sparse:
            keys = api.IdxCache(Bc, n, DI, api.BF16)
            caches.append((keys, m, torch.randn(m, generator=gen, device=dev), 1))
        _compressed_prefix(torch, api, gen, Lc, caches)
        xw = torch.randn(Bc, W, D_HEAD, generator=gen, device=dev).to(torch.bfloat16)
        api.compress_kv(xw, torch.full((Bc,), Lc - W, dtype=torch.int32, device=dev), 1, zero1, gamma=gam,
                        rope_dim=DR, kv_out=win)
        pos = torch.full((Bc, 1), t, dtype=torch.int32, device=dev)
        x_blk = torch.randn(Bc, m, D_HEAD, generator=gen, device=dev).to(torch.bfloat16)
        x_new = x_blk[:, m - 1].contiguous()
        xi_blk = torch.randn(Bc, m, DI, generator=gen, device=dev).to(torch.bfloat16)
        xi_new = xi_blk[:, m - 1].contiguous()
        tok_new = torch.full((Bc,), t, dtype=torch.int32, device=dev)
        # pooling states of the block the timed step completes, holding its
        # earlier tokens
        st_kv = torch.empty((Bc, D_HEAD + 2), dtype=torch.float32, device=dev)
        st_ix = torch.empty((Bc, DI + 2), dtype=torch.float32, device=dev)
        for r_ in range(m - 1):
            pr = torch.full((Bc,), t + 1 - m + r_, dtype=torch.int32, device=dev)
            jobs = [dict(x=x_blk[:, r_].contiguous(), tok_pos=pr, m=m, score_bias=bias, state=st_kv, gamma=gam,
                         rope_dim=DR, kv_out=comp)]
            if sparse:
                jobs.append(dict(x=xi_blk[:, r_].contiguous(), tok_pos=pr, m=m, score_bias=caches[1][2], state=st_ix,
                                 idx_out=keys))
            api.compress_kv_step(jobs)
        q = torch.randn(Bc, 1, Hq, D_HEAD, generator=gen, device=dev).to(torch.bfloat16)
        qI = torch.randn(Bc, 1, HI, DI, generator=gen, device=dev).to(torch.bfloat16)
        wI = torch.randn(Bc, 1, HI, generator=gen, device=dev)
        sink = torch.randn(Hq, generator=gen, device=dev) * (1.0 if sparse else 0.02)
        Wo = (torch.randn(G, hid // G, Hq * D_HEAD // G, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        o = torch.empty(Bc, 1, Hq, D_HEAD, dtype=torch.bfloat16, device=dev)
        y = torch.empty(Bc, hid, dtype=torch.bfloat16, device=dev)
        prm = api.attn_params(D_HEAD, DR, W, m)
        aws = torch.empty(max(1, api.attn_workspace_bytes(Bc, 1, Hq, D_HEAD, K_CSA if sparse else n, W, api.BF16,
                                                          api.BF16)), dtype=torch.uint8, device=dev)
        top = torch.empty(Bc, 1, K_CSA, dtype=torch.int32, device=dev)
        iws = torch.empty(max(1, api.indexer_workspace_bytes(Bc, 1, n, K_CSA)), dtype=torch.uint8, device=dev)

        def comp_call():
            jobs = [dict(x=x_new, tok_pos=tok_new, m=1, score_bias=zero1, gamma=gam, rope_dim=DR, kv_out=win),
                    dict(x=x_new, tok_pos=tok_new, m=m, score_bias=bias, state=st_kv, gamma=gam, rope_dim=DR,
                         kv_out=comp)]
            if sparse:
                jobs.append(dict(x=xi_new, tok_pos=tok_new, m=m, score_bias=caches[1][2], state=st_ix,
                                 idx_out=keys))
            api.compress_kv_step(jobs)

        def idx_call():
            api.indexer_topk(qI, api.BF16, wI, keys, pos, m, K_CSA, out=top, workspace=iws)

        def attn_call():
            if sparse:
                api.sparse_mqa_attn(q, pos, top, comp, win, sink, prm, out=o, workspace=aws)
            else:
                api.hca_dense_mqa_attn(q, pos, comp, win, sink, prm, out=o, workspace=aws)

        def proj_call():
            api.out_proj_grouped(o.view(Bc, Hq * D_HEAD), Wo, y=y)

        calls = [("compress_kv", comp_call)] + ([("indexer_topk", idx_call)] if sparse else []) + \
                [("attention", attn_call), ("out_proj", proj_call)]

        def step():
            for _, f in calls:
                f()
        per = {c: float(np.median(_timed(torch, f, reps, flush))) for c, f in calls}
        st = _timed(torch, step, reps, flush)
        ms = float(np.median(st))
        qo = Bc * Hq * D_HEAD * 2
        ne = (K_CSA if sparse else n) + W
        algo = {"compress_kv": Bc * (D_HEAD * 2 + (D_HEAD + 2) * 4) + 2 * Bc * 2 * D_HEAD
                               + (Bc * (DI * 2 + (DI + 2) * 4) + Bc * DI * 2 if sparse else 0),
                "attention": 2 * qo + Bc * ne * 2 * D_HEAD + (Bc * K_CSA * 4 if sparse else 0),
                "out_proj": G * (hid // G) * (Hq * D_HEAD // G) * 2 + qo + Bc * hid * 2}
        if sparse:
            algo["indexer_topk"] = Bc * n * DI * 2 + Bc * HI * (DI * 2 + 4) + Bc * K_CSA * 4
        attn_side = sum(v for c, v in algo.items() if c != "out_proj")
        attn_ms = sum(per[c] for c in algo if c != "out_proj")
        res[name] = {
            "batch": Bc, "context": Lc, "m": m, "heads": Hq, "entries_per_query": ne,
            "step_ms": _pctl(st), "query_tokens_per_s": round(Bc / (ms * 1e-3), 1),
            "calls_us": {c: round(v * 1e3, 2) for c, v in per.items()},
            "calls_GBs": {c: round(algo[c] / (per[c] * 1e-3) / 1e9, 1) for c in per},
            "algo_MB": {c: round(v / 1e6, 3) for c, v in algo.items()},
            "attention_side": {"algo_MB": round(attn_side / 1e6, 2), "ms": round(attn_ms, 4),
                               "GBs": round(attn_side / (attn_ms * 1e-3) / 1e9, 1),
                               "frac_hbm": round(attn_side / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "query_tokens_per_s": round(Bc / (attn_ms * 1e-3), 1)},
            "timing": f"HIP events, median (p10, p90) of {reps} runs, L2 and last-level cache evicted before each "
                      "(a 1 GiB read)"}
        del comp, win, keys, aws, iws
        torch.cuda.empty_cache()
    return res


def layer_proj_measure(torch, api, reps=20, seed=7007):
    """The projections either side of the attention with FP8 weights (E4M3
    codes, one f32 scale per output row; bf16 activations), at the 1M model
    widths (hidden 7168, 64 heads x 512, indexer 4 x 64):
      in_proj : csa_layer_in_proj, one launch for q, the raw KV token, the
                raw indexer key, the FP4 indexer queries and the head weights
                (33,604 weight rows), plus the FP4 quantisation of the queries;
      out_proj: csa_linear_fp8, the grouped output projection 32768 -> 7168
                in 8 groups.
    At a 4-sequence decode step (M = 4: weight streams, HBM-bound; caches
    evicted before each run by a 1 GiB read) and at the 8,192-token prefill
    chunk (matrix-core bound: bf16 MFMA on the widened weights)."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device=dev)
    flush_out = torch.empty((), dtype=torch.int64, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_out)

    def codes(n, k):
        x = (torch.randn(n, k, generator=gen, device=dev) * 64.0).clamp_(-448.0, 448.0)
        return x.to(torch.float8_e4m3fn).view(torch.uint8)

    N_in = H * D_HEAD + D_HEAD + DI + HI * DI + HI
    K_out = H * D_HEAD
    W_in, s_in = codes(N_in, HIDDEN), torch.full((N_in,), 1e-3, device=dev)
    W_out, s_out = codes(HIDDEN, K_out // G), torch.full((HIDDEN,), 1e-3, device=dev)
    res = {"weights_MB": {"in_proj": round(N_in * HIDDEN / 1e6, 2), "out_proj": round(HIDDEN * K_out // G / 1e6, 2)}}
    for name, M in (("decode_b4", B), ("prefill_chunk_8192", PF_T)):
        h = (torch.randn(M, HIDDEN, generator=gen, device=dev)).to(torch.bfloat16)
        o = (torch.randn(M, K_out, generator=gen, device=dev) * 0.05).to(torch.bfloat16)
        out = dict(q=torch.empty((M, H, D_HEAD), dtype=torch.bfloat16, device=dev),
                   kv=torch.empty((M, D_HEAD), dtype=torch.bfloat16, device=dev),
                   k_idx=torch.empty((M, DI), dtype=torch.bfloat16, device=dev),
                   q_idx=torch.empty((M, HI, DI // 2), dtype=torch.uint8, device=dev),
                   q_idx_scales=torch.empty((M, HI, DI // 32), dtype=torch.uint8, device=dev),
                   w_idx=torch.empty((M, HI), dtype=torch.float32, device=dev))
        ws = torch.empty(api.layer_in_proj_workspace_size(M, HI, DI), dtype=torch.uint8, device=dev)
        y = torch.empty((M, HIDDEN), dtype=torch.bfloat16, device=dev)

        def fin():
            api.layer_in_proj(h, W_in, s_in, H, D_HEAD, DI, HI, out=out, workspace=ws)

        def fout():
            api.linear_fp8(o, W_out, s_out, G=G, y=y)

        decode = M <= 64
        t_in = _timed(torch, fin, reps, flush if decode else None)
        t_out = _timed(torch, fout, reps, flush if decode else None)
        r = {"rows": M, "in_proj_ms": _pctl(t_in), "out_proj_ms": _pctl(t_out)}
        mi, mo = float(np.median(t_in)), float(np.median(t_out))
        if decode:
            bytes_in = N_in * HIDDEN + 4 * N_in + M * HIDDEN * 2 + M * (H * D_HEAD * 2 + D_HEAD * 2 + DI * 2 +
                                                                        HI * DI // 2 + HI * DI // 32 + HI * 4) \
                + 2 * M * HI * DI * 4
            bytes_out = HIDDEN * K_out // G + 4 * HIDDEN + M * K_out * 2 + M * HIDDEN * 2
            r["algo_MB"] = {"in_proj": round(bytes_in / 1e6, 2), "out_proj": round(bytes_out / 1e6, 2)}
            r["GBs"] = {"in_proj": round(bytes_in / (mi * 1e-3) / 1e9, 1),
                        "out_proj": round(bytes_out / (mo * 1e-3) / 1e9, 1)}
            r["frac_hbm"] = {k: round(v / HBM_PEAK_GBS, 4) for k, v in r["GBs"].items()}
        else:
            f_in, f_out = 2.0 * M * HIDDEN * N_in, 2.0 * M * K_out // G * HIDDEN
            r["tflop"] = {"in_proj": round(f_in / 1e12, 3), "out_proj": round(f_out / 1e12, 3)}
            r["tflops"] = {"in_proj": round(f_in / (mi * 1e-3) / 1e12, 1),
                           "out_proj": round(f_out / (mo * 1e-3) / 1e12, 1)}
            r["frac_bf16_peak"] = {k: round(v / BF16_PEAK_TFLOPS, 4) for k, v in r["tflops"].items()}
        res[name] = r
        del h, o, out, ws, y
    res["timing"] = (f"HIP events, median (p10, p90) of {reps} runs; decode runs with L2 and the last-level "
                     "cache evicted before each (a 1 GiB read)")
    return res


def capture_step_graphs(torch, fns, sets, sh):
    """One HIP graph per rotated buffer set, each holding one whole decode step
    (every call's kernels, in order).  The calls allocate nothing and issue no
    memsets, so the graphs hold only kernel nodes."""
    side = torch.cuda.Stream()                        # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up on a side stream before capture
        for s_ in sets:
            for f in fns:
                f(s_, sh)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for s_ in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f(s_, sh)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def cpu_baseline(target_s):
    """The oracle, as it stands, on one decode step of the same layer pair for
    the whole batch (synthetic records drawn at the same shapes), repeated up
    to ~target_s seconds; returns query tokens per second."""
    import oracle as O
    from long_context_attention_23_amd import synth
    g = synth.rng(2004)
    t = L - 1
    csa = synth.fp8_records(g, (B, N_CSA), D_HEAD, DR, REC)
    hca = synth.fp8_records(g, (B, N_HCA), D_HEAD, DR, REC)
    win = synth.fp8_records(g, (B, W), D_HEAD, DR, REC)
    kc, ks = synth.fp4_rows(g, (B, N_CSA), DI, -3, 0)
    qc, qs = synth.fp4_rows(g, (B, 1, HI), DI, -3, 0)
    w = synth.normal(g, (B, 1, HI))
    q = synth.bf16_bits(g, (B, 1, H, D_HEAD))
    x_csa = synth.normal(g, (B, M_CSA, D_HEAD))
    xi = synth.normal(g, (B, M_CSA, DI))
    x_hca = synth.normal(g, (B, M_HCA, D_HEAD))
    sink = synth.normal(g, H)
    b4 = synth.normal(g, M_CSA)
    Wo = [synth.bf16_bits(g, (G, HIDDEN // G, H * D_HEAD // G), std=0.02) for _ in range(2)]
    Wo64 = [O.bf16_decode(x) for x in Wo]
    gam = np.ones(D_HEAD, np.float32)
    sc = 1.0 / math.sqrt(D_HEAD)
    n_steps, t0 = 0, time.perf_counter()
    while True:
        for bi in range(B):
            O.compress(x_csa[bi:bi + 1, -1:], O.F32, [t], 1, [0.0], gamma=gam, dr=DR, out_kind=0, out_fmt=O.FP8_E4M3,
                       cap=W, ring=True)
            O.compress(x_csa[bi:bi + 1], O.F32, [t + 1 - M_CSA], M_CSA, b4, gamma=gam, dr=DR, out_kind=0,
                       out_fmt=O.FP8_E4M3, cap=N_CSA)
            O.compress(xi[bi:bi + 1], O.F32, [t + 1 - M_CSA], M_CSA, b4, out_kind=1, out_fmt=O.FP4_E2M1, cap=N_CSA)
            top = O.indexer_topk(qc[bi], qs[bi], O.FP4_E2M1, w[bi], [t], kc[bi], ks[bi], O.FP4_E2M1, M_CSA, K_CSA)
            oc = O.attention(q[bi], O.BF16, [t], gam, sink, D_HEAD, DR, W, M_CSA, 10000.0, sc, 1e-6, csa[bi],
                             O.FP8_E4M3, win[bi], O.FP8_E4M3, top)
            O.out_proj(oc.reshape(1, H * D_HEAD), Wo64[0])
            O.compress(x_hca[bi:bi + 1, -1:], O.F32, [t], 1, [0.0], gamma=gam, dr=DR, out_kind=0, out_fmt=O.FP8_E4M3,
                       cap=W, ring=True)
            O.compress(x_hca[bi:bi + 1], O.F32, [t + 1 - M_HCA], M_HCA, np.zeros(M_HCA), gamma=gam, dr=DR,
                       out_kind=0, out_fmt=O.FP8_E4M3, cap=N_HCA)
            oh = O.attention(q[bi], O.BF16, [t], gam, sink, D_HEAD, DR, W, M_HCA, 10000.0, sc, 1e-6, hca[bi],
                             O.FP8_E4M3, win[bi], O.FP8_E4M3)
            O.out_proj(oh.reshape(1, H * D_HEAD), Wo64[1])
        n_steps += 1
        el = time.perf_counter() - t0
        if el >= target_s or n_steps >= 200:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return {"value": n_steps * B / el, "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_steps} full decode step(s) of the batch-4 layer pair at 1M context (fp64 oracle, "
                      f"synthetic FP8/FP4 caches of the same shapes), {el:.1f} s"}


def cpu_baseline_prefill(target_s, nq=512):
    """The oracle on the prefill chunk's CSA calls (indexer top-1024 over
    264,192 FP4 keys, sparse attention over 1,024 FP8 records + window, and
    the grouped projection) for nq strided query rows (every 8,192/nq-th),
    in batches until the sample is done or about target_s seconds have
    passed; the rate per query row is extrapolated to the chunk."""
    import oracle as O
    from long_context_attention_23_amd import synth
    g = synth.rng(2005)
    n = (L + PF_T) // M_CSA
    kc, ks = synth.fp4_rows(g, (n,), DI, -3, 0)
    comp = synth.fp8_records(g, (n,), D_HEAD, DR, REC)
    win = synth.fp8_records(g, (W + PF_T,), D_HEAD, DR, REC)
    Wo = O.bf16_decode(synth.bf16_bits(g, (G, HIDDEN // G, H * D_HEAD // G), std=0.02))
    sink = synth.normal(g, H)
    rows = np.arange(0, PF_T, PF_T // nq)[:nq]
    done, t0 = 0, time.perf_counter()
    for b0 in range(0, len(rows), 32):
        r = rows[b0:b0 + 32]
        qc, qs = synth.fp4_rows(g, (len(r), HI), DI, -3, 0)
        w = synth.normal(g, (len(r), HI))
        q = synth.bf16_bits(g, (len(r), H, D_HEAD))
        pos = (L + r).astype(np.int32)
        top = O.indexer_topk(qc, qs, O.FP4_E2M1, w, pos, kc, ks, O.FP4_E2M1, M_CSA, PF_TOPK)
        o = O.attention(q, O.BF16, pos, None, sink, D_HEAD, DR, W, M_CSA, 10000.0, 1.0 / math.sqrt(D_HEAD), 1e-6,
                        comp, O.FP8_E4M3, win, O.FP8_E4M3, top)
        O.out_proj(o.reshape(len(r), H * D_HEAD), Wo)
        done += len(r)
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return {"value": done / el, "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
            "extrapolated": True,
            "sample": f"{done} of the chunk's 8,192 query rows (every {PF_T // nq}th) through the CSA indexer, sparse "
                      f"attention and projection (fp64 oracle, synthetic FP4 keys and FP8 records of the 1M prefix's "
                      f"shapes), {el:.1f} s; the per-row rate stands for the whole chunk"}


# HBM traffic per launch of a call, from rocprofv3 FETCH_SIZE and WRITE_SIZE
# runs of this benchmark scaled by the copy calibration (the summary under
# profiles/ gives the counts and commands); valid only while the kernels'
# sources are unchanged (src_hash below).
TRAFFIC = {
    "csa_indexer_topk": {"bytes": 37_406_758, "src": "13de0a391c729277"},
    "csa_sparse_mqa_attn": {"bytes": 25_893_189, "src": "13de0a391c729277"},
    "hca_dense_mqa_attn": {"bytes": 54_513_159, "src": "13de0a391c729277"},
    "csa_out_proj": {"bytes": 59_135_011, "src": "13de0a391c729277"},
    "hca_out_proj": {"bytes": 59_135_011, "src": "13de0a391c729277"},
}
TRAFFIC_SRC = ["long_context_attention_23_amd/csrc/indexer.hip", "long_context_attention_23_amd/csrc/attn_mfma.hip",
               "long_context_attention_23_amd/csrc/attn.hip", "long_context_attention_23_amd/csrc/proj.hip",
               "long_context_attention_23_amd/csrc/compress.hip", "long_context_attention_23_amd/csrc/common.hpp"]


def src_hash():
    h = hashlib.sha256()
    for f in TRAFFIC_SRC:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, three times."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def _kernel_rows(db):
    import sqlite3
    c = sqlite3.connect(db)
    cols = [r[1] for r in c.execute("pragma table_info(kernels)")]
    ni = cols.index("name") if "name" in cols else cols.index("kernel_name")
    st, en = cols.index("start"), cols.index("end")
    return sorted(((r[ni], r[st], r[en]) for r in c.execute("select * from kernels")), key=lambda r: r[1])


def _short(name):
    return name.split("(")[0].replace("void ", "")


def summarize(d, last=20):
    """Per-kernel and per-call durations of a kernel-trace run of this
    benchmark over its last `last` steps (the timed region).  A step is the
    fixed sequence of launches of CALL_KERNELS in CALLS order; a call's span
    runs from its first kernel's start to its last kernel's end."""
    db = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))[0]
    rows = _kernel_rows(db)
    seq = [k for c in CALLS for k in CALL_KERNELS[c]]
    anchor = CALL_KERNELS["csa_indexer_topk"][0]
    first = seq.index(anchor)
    zero = [i for i, (n, _, _) in enumerate(rows) if anchor in n]
    steps = []
    for z in zero:
        st = z - first
        if st < 0 or st + len(seq) > len(rows):
            continue
        blk = rows[st:st + len(seq)]
        if all(k in _short(n) for k, (n, _, _) in zip(seq, blk)):
            steps.append(blk)
    steps = steps[-last:]
    out = [f"steps summarised: {len(steps)} (the last {last} whole steps of the run)", "",
           "Per kernel:", "",
           "| kernel | dispatches | avg us | min us | max us | total us |", "|---|---|---|---|---|---|"]
    agg = {}
    for blk in steps:
        for n, a, b in blk:
            agg.setdefault(_short(n), []).append((b - a) / 1e3)
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {len(v)} | {np.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} | {sum(v):.1f} |")
    out += ["", "Per call (span = first kernel start to last kernel end, per step):", "",
            "| call | kernels | avg span us | median span us | avg sum of kernel us |", "|---|---|---|---|---|"]
    for c in CALLS:
        i0 = sum(len(CALL_KERNELS[x]) for x in CALLS[:CALLS.index(c)])
        n = len(CALL_KERNELS[c])
        spans = [(blk[i0 + n - 1][2] - blk[i0][1]) / 1e3 for blk in steps]
        sums = [sum(b - a for _, a, b in blk[i0:i0 + n]) / 1e3 for blk in steps]
        out.append(f"| {c} | {' '.join(CALL_KERNELS[c])} | {np.mean(spans):.2f} | {np.median(spans):.2f} | "
                   f"{np.mean(sums):.2f} |")
    wall = [(steps[i + 1][0][1] - steps[i][0][1]) / 1e3 for i in range(len(steps) - 1)]
    if wall:
        out += ["", f"step period (start to start): avg {np.mean(wall):.2f} us"]
    print("\n".join(out))


def summarize_prefill(d):
    """Per-call kernel durations of the prefill section in a kernel-trace run
    of this benchmark.  The section runs each call once to warm up, then
    `reps` times, in the order indexer, CSA attention, HCA attention,
    projection; the indexer's kernels are k_idxp_*, each attention call is one
    k_attn_mfma launch (one split per row), the projection k_proj_mfma."""
    db = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))[0]
    rows = [(_short(n), (b - a) / 1e3) for n, a, b in _kernel_rows(db) if "csa::" in n]
    # the section runs from its first threshold kernel (decode steps use the
    # decode threshold kernel) to the next compression launch (the caches of
    # the workloads measured after it)
    i0 = next(i for i, (n, _) in enumerate(rows) if "k_idxp_thresh" in n)
    i1 = next((i for i in range(i0, len(rows)) if "k_compress" in rows[i][0]), len(rows))
    pre = rows[i0:i1]
    att = [t for n, t in pre if "k_attn_mfma" in n]
    nrep = len(att) // 2
    calls = {"csa_indexer_topk (k_idxp_*)": None, "csa_sparse_mqa_attn": att[:nrep],
             "hca_dense_mqa_attn": att[nrep:2 * nrep], "attn_out_proj_grouped": [t for n, t in pre if "k_proj_mfma" in n]}
    per = {}
    for n, t in pre:
        if "k_idxp_" in n:
            per.setdefault(n.replace("csa::", ""), []).append(t)
    out = ["Prefill section, per kernel of the indexer call (every launch: warm-up and timed):", "",
           "| kernel | launches | avg us | min us |", "|---|---|---|---|"]
    for k, v in per.items():
        out.append(f"| {k} | {len(v)} | {np.mean(v):.1f} | {min(v):.1f} |")
    out += ["", "Per call (kernel-only):", "", "| call | launches | avg us | min us |", "|---|---|---|---|"]
    nidx = len(per.get("k_idxp_filter", []))
    idx_sum = [sum(v[i] for v in per.values() if len(v) == nidx) for i in range(nidx)]
    calls["csa_indexer_topk (k_idxp_*)"] = idx_sum
    for c, v in calls.items():
        if v:
            out.append(f"| {c} | {len(v)} | {np.mean(v):.1f} | {min(v):.1f} |")
    print("\n".join(out))


def summarize_pmc(dirs):
    """Per-call counter sums (mean over the timed steps) from --pmc runs of
    this benchmark; calls are told apart by their kernels and step order."""
    import sqlite3
    res = {}
    for d in dirs:
        db = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))[0]
        c = sqlite3.connect(db)
        rows = c.execute("select name, counter_name, counter_value, dispatch_id from pmc_events").fetchall()
        per = {}
        for name, cn, v, did in rows:
            key = (did, _short(name), cn)
            per[key] = per.get(key, 0.0) + v
        seq = sorted(per.items())                   # dispatch order
        counters = sorted({k[2] for k, _ in seq})
        for cn in counters:
            ks = [(k[1], v) for k, v in seq if k[2] == cn]
            sums = {"csa_indexer_topk": [], "csa_sparse_mqa_attn": [], "hca_dense_mqa_attn": [],
                    "out_proj (one launch)": []}
            i = 0
            attn_seen = 0
            while i < len(ks):
                n = ks[i][0]
                nk = len(CALL_KERNELS["csa_indexer_topk"])
                if n.endswith(CALL_KERNELS["csa_indexer_topk"][0]) and i + nk - 1 < len(ks):
                    sums["csa_indexer_topk"].append(sum(v for _, v in ks[i:i + nk]))
                    attn_seen = 0
                    i += nk
                    continue
                if "k_attn_mfma" in n and i + 1 < len(ks) and "k_attn_combine" in ks[i + 1][0]:
                    key = "csa_sparse_mqa_attn" if attn_seen == 0 else "hca_dense_mqa_attn"
                    sums[key].append(ks[i][1] + ks[i + 1][1])
                    attn_seen += 1
                    i += 2
                    continue
                if "k_proj_gemv" in n:
                    sums["out_proj (one launch)"].append(ks[i][1])
                i += 1
            res[cn] = {k: (float(np.mean(v[-10:])) if v else None, len(v)) for k, v in sums.items() if v}
            if not res[cn]:                         # a --copy-calibration run
                cp = [v for n, v in ks if "copy" in n.lower() or "elementwise" in n]
                res[cn]["copy (per launch)"] = (float(np.median(cp)) if cp else None, len(cp))
    print(json.dumps(res, indent=1))


def summarize_pmc_dispatches(dirs, match="k_attn_mfma"):
    """Per-dispatch counter sums (over the counter's instances) in dispatch
    order, for kernels whose name holds `match`, from rocprofv3 --pmc runs of
    this benchmark (one counter per run); tells apart launches of one kernel
    over the same grid (the prefill section's CSA launches come before its
    HCA launches)."""
    import sqlite3
    cols = {}
    for d in dirs:
        db = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))[0]
        c = sqlite3.connect(db)
        acc = {}
        for name, cn, v, did in c.execute("select name, counter_name, counter_value, dispatch_id from pmc_events"):
            if match not in _short(name):
                continue
            acc[(did, cn)] = acc.get((did, cn), 0.0) + v
        for (did, cn), v in acc.items():
            cols.setdefault(cn, {})[did] = v
        c.close()
    names = sorted(cols)
    print("| launch | " + " | ".join(names) + " |")
    print("|---|" + "---|" * len(names))
    per = [sorted(cols[n].items()) for n in names]
    for i in range(min(len(p) for p in per) if per else 0):
        print(f"| {i} | " + " | ".join(f"{p[i][1]:.1f}" for p in per) + " |")


def summarize_pmc_kernels(dirs, match=("k_idxp_", "k_attn_mfma", "k_proj_mfma")):
    """Per-kernel counter means (per dispatch) from rocprofv3 --pmc runs of
    this benchmark (any counters, several runs), for kernels whose name holds
    one of `match`, with the derived figures:
      MFMA busy = sum SQ_VALU_MFMA_BUSY_CYCLES / (max GRBM_GUI_ACTIVE x 1024 SIMDs)
      MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_* x 512
      VALU busy = sum SQ_ACTIVE_INST_VALU / 256 CUs / max GRBM_GUI_ACTIVE
        (= 4 x the quad-cycles the counter counts per SIMD / 1024 SIMDs)
    (per-dispatch sums over the counter's instances; GRBM_GUI_ACTIVE is taken
    as its largest instance, the busy time of the GPU)."""
    import sqlite3
    per = {}                                  # (kernel, counter) -> list of per-dispatch (sum, max)
    for d in dirs:
        db = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))[0]
        c = sqlite3.connect(db)
        acc = {}
        for name, cn, v, did in c.execute("select name, counter_name, counter_value, dispatch_id from pmc_events"):
            k = _short(name)
            if not any(mm in k for mm in match):
                continue
            a = acc.setdefault((did, k, cn), [0.0, -1e300])
            a[0] += v
            a[1] = max(a[1], v)
        for (did, k, cn), (sm, mx) in acc.items():
            per.setdefault((k, cn), []).append((sm, mx))
    kernels = sorted({k for k, _ in per})
    out = []
    for k in kernels:
        cs = {cn: v for (kk, cn), v in per.items() if kk == k}
        mean = {cn: float(np.mean([a for a, _ in v])) for cn, v in cs.items()}
        gmax = float(np.mean([b for _, b in cs["GRBM_GUI_ACTIVE"]])) if "GRBM_GUI_ACTIVE" in cs else None
        row = {"dispatches": max(len(v) for v in cs.values()), "counters": {cn: round(v, 1) for cn, v in mean.items()}}
        if gmax:
            row["GRBM_GUI_ACTIVE_max"] = round(gmax, 1)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                row["mfma_busy"] = round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (gmax * 1024), 4)
            if "SQ_ACTIVE_INST_VALU" in mean:
                row["valu_busy"] = round(mean["SQ_ACTIVE_INST_VALU"] / 256 / gmax, 4)
        for t in ("BF16", "F6F4", "F8", "F16", "F32"):
            cn = "SQ_INSTS_VALU_MFMA_MOPS_" + t
            if cn in mean:
                row["mfma_flops_" + t] = float(f"{mean[cn] * 512:.4g}")
        out.append((k, row))
    print(json.dumps(dict(out), indent=1))


def summarize_launches(dirs):
    """Per launch shape (kernel, grid) of the library's kernels in rocprofv3
    runs of this benchmark: launches and duration from a --kernel-trace run,
    per-dispatch counter means (summed over the counter's instances; the
    largest instance for GRBM_GUI_ACTIVE) from --pmc runs, joined on the
    dispatch id.  Launches of one kernel over different problem sizes (an
    input and an output projection) fall into different rows."""
    import sqlite3
    rows = {}                                        # (kernel, grid) -> {"us": [...], counter: [...]}
    for d in dirs:
        db = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))[0]
        c = sqlite3.connect(db)
        have = {r[0] for r in c.execute("select name from sqlite_master where type in ('table','view')")}
        pmc = "pmc_events" in have and c.execute("select count(*) from pmc_events").fetchone()[0] > 0
        shape = {}
        for name, gx, gy, gz, wx, did, a, b in c.execute(
                "select name, grid_x, grid_y, grid_z, workgroup_x, dispatch_id, start, end from kernels"):
            if "csa::" not in name:
                continue
            key = (_short(name).replace("csa::", ""), f"{gx // max(wx, 1)}x{gy}x{gz} wg of {wx}")
            shape[did] = key
            r = rows.setdefault(key, {"us": []})
            if not pmc:                              # durations from trace runs only (counter runs serialise)
                r["us"].append((b - a) / 1e3)
        if not pmc:
            continue
        acc = {}
        for cn, v, did in c.execute("select counter_name, counter_value, dispatch_id from pmc_events"):
            if did not in shape:
                continue
            a = acc.setdefault((did, cn), [0.0, -1e300])
            a[0] += v
            a[1] = max(a[1], v)
        for (did, cn), (sm, mx) in acc.items():
            rows[shape[did]].setdefault(cn, []).append(mx if cn == "GRBM_GUI_ACTIVE" else sm)
    cns = sorted({cn for r in rows.values() for cn in r if cn != "us"})
    out = ["| kernel | grid | launches | avg us | min us | " + " | ".join(cns) + " |",
           "|---|---|---|---|---|" + "---|" * len(cns)]
    for (k, g), r in sorted(rows.items()):
        us = r["us"]
        t = f"{len(us)} | {np.mean(us):.2f} | {min(us):.2f}" if us else " | | "
        cells = [f"{np.mean(r[cn]):.6g}" if cn in r else "" for cn in cns]
        out.append(f"| {k} | {g} | {t} | " + " | ".join(cells) + " |")
    print("\n".join(out))


def main():
    args = parse()
    if args.copy_calibration:
        return copy_calibration()
    if args.summarize:
        return summarize(args.summarize)
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc)
    if args.summarize_prefill:
        return summarize_prefill(args.summarize_prefill)
    if args.summarize_pmc_kernels:
        return summarize_pmc_kernels(args.summarize_pmc_kernels)
    if args.summarize_pmc_dispatches:
        return summarize_pmc_dispatches(args.summarize_pmc_dispatches)
    if args.summarize_launches:
        return summarize_launches(args.summarize_launches)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this path runs on a single "
              "MI355X; multi-GPU sharding is not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    from long_context_attention_23_amd import api
    api.lib()
    torch.cuda.set_device(0)
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_measure(torch, api)}), flush=True)
        return
    if args.layer_proj_only:
        print(json.dumps({"layer_proj_fp8": layer_proj_measure(torch, api)}), flush=True)
        return
    sets, sh = build_state(torch, api, args.copies)
    R = len(sets)
    fns = call_fns(api)
    for s_ in sets:                                   # eager warm-up of every call
        for f in fns:
            f(s_, sh)
    torch.cuda.synchronize()

    # calibration: events around every call of eagerly launched steps -> per-call GPU time
    ncal = max(10, min(50, args.steps))
    evc = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in CALLS]
           for _ in range(ncal)]
    for i in range(ncal):
        for j, f in enumerate(fns):
            evc[i][j][0].record()
            f(sets[i % R], sh)
            evc[i][j][1].record()
    torch.cuda.synchronize()
    per_call = {c: float(np.median([evc[i][j][0].elapsed_time(evc[i][j][1]) for i in range(ncal)]))
                for j, c in enumerate(CALLS)}
    dom = max(CALLS, key=lambda c: per_call[c])
    di = CALLS.index(dom)

    # eager pass: K whole steps launched eagerly on the current stream (the
    # host stays ahead of the GPU, so the kernels run back to back), with a
    # pair of events around the dominant call in every step.
    for i in range(args.warmup):
        for f in fns:
            f(sets[i % R], sh)
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s_ = sets[i % R]
        for j, f in enumerate(fns):
            if j == di:
                ev[i][0].record()
            f(s_, sh)
            if j == di:
                ev[i][1].record()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    dom_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))

    # timed region: the same K steps as HIP graph replays (graph i % R holds
    # one whole step on rotated set i % R), W untimed replays first
    graphs = capture_step_graphs(torch, fns, sets, sh)
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    algo = algorithmic_bytes()
    calls = {c: {"us": round(per_call[c] * 1e3, 2), "algo_MB": round(algo[c] / 1e6, 3),
                 "GBs": round(algo[c] / (per_call[c] * 1e-3) / 1e9, 1), "kernels": sorted(set(CALL_KERNELS[c]))}
             for c in CALLS}
    achieved = algo[dom] / (dom_ms * 1e-3) / 1e9
    total_algo = sum(algo.values())
    gpu_ms = sum(per_call.values())
    res = {
        "metric": METRIC, "value": round(B / (ms_step * 1e-3), 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "CSA+HCA layer-pair decode, 1M context, batch 4, V4-Pro shape (hidden 7168, 64 heads "
                               "x 512, FP8 KV + FP4 indexer, top-1024, window 128)", "global_batch": B,
                   "seq_len": L, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": dom, "kernels": sorted(set(CALL_KERNELS[dom])),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (TRAFFIC[dom]["bytes"] if dom in TRAFFIC and TRAFFIC[dom]["src"] == src_hash()
                                 else None),
                     "us_per_launch": round(dom_ms * 1e3, 2), "algo_MB_per_launch": round(algo[dom] / 1e6, 3)},
        "step_hbm": {"algo_MB": round(total_algo / 1e6, 2), "gpu_us": round(gpu_ms * 1e3, 2),
                     "GBs_gpu": round(total_algo / (gpu_ms * 1e-3) / 1e9, 1),
                     "frac_gpu": round(total_algo / (gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "calls": calls,
        "timing": "value and ms_per_step: wall clock over K timed steps, each one HIP graph replay holding the "
                  "step's calls (one graph per rotated buffer set), synchronised before and after; roofline from "
                  "events around the dominant call in every step of an eager pass over the same steps; per-call "
                  "GPU times from events around every call (median over an eager calibration pass)",
    }
    res["eager"] = {"ms_per_step": round(ms_eager, 4), "query_tokens_per_s": round(B / (ms_eager * 1e-3), 1),
                    "how": "the same steps launched call by call on one stream (dispatch gaps between kernels)"}
    del graphs, sets
    torch.cuda.empty_cache()
    if not args.no_prefill:
        res["prefill"] = prefill_measure(torch, api)
        torch.cuda.empty_cache()
    if not args.no_decode_configs:
        res["decode_configs"] = decode_configs_measure(torch, api)
        torch.cuda.empty_cache()
    if not args.no_layer_proj:
        res["layer_proj_fp8"] = layer_proj_measure(torch, api)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        if not args.no_prefill:
            res["prefill"]["cpu_baseline"] = cpu_baseline_prefill(args.cpu_prefill_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
