"""Shared helpers for the GPU parity tests: host <-> device marshalling and the
comparison metrics.  Inputs come from long_context_attention_23_amd.synth;
expected values only from the oracle."""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def out_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def abs_err(got, ref):
    return float(np.max(np.abs(got - ref)))


def recall(got, ref):
    """mean over rows of |got & ref| / |ref| (ignoring -1 padding)."""
    vals = []
    for g, r in zip(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1])):
        rs = set(int(v) for v in r if v >= 0)
        if not rs:
            continue
        vals.append(len(rs & set(int(v) for v in g if v >= 0)) / len(rs))
    return float(np.mean(vals)) if vals else 1.0
