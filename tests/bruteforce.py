"""Independent dense numpy formulation of one CSA / HCA layer (test pin only).

Written against the method's description, not against the oracle: every step
is a whole-array operation (pooling as a softmax-weighted einsum, RoPE as a
complex multiplication, the indexer as a masked score matrix, top-k as a full
lexicographic sort, attention as one masked matrix over [all compressed
entries ; all raw tokens ; the sink]).  Only for tiny inputs.
"""
import numpy as np


def rope_complex(v, pos, dr, base):
    """Rotate the last dr dims of v [..., d] as complex pairs
    (v[2i] + i v[2i+1]) * exp(i * pos * base^(-2i/dr)); pos broadcasts over
    the leading dims."""
    v = np.array(v, dtype=np.float64, copy=True)
    if dr == 0:
        return v
    d = v.shape[-1]
    tail = v[..., d - dr:]
    z = tail[..., 0::2] + 1j * tail[..., 1::2]
    freq = base ** (-np.arange(0, dr, 2) / dr)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    z = z * np.exp(1j * ang)
    out = np.empty_like(tail)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    v[..., d - dr:] = out
    return v


def rms(v, gamma, eps):
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * gamma


def f32(v):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def softmax_pool(x, m, b):
    """x [T, d] -> [T//m, d], pooled with softmax(b) per block."""
    N = x.shape[0] // m
    blocks = x[:N * m].reshape(N, m, x.shape[1]).astype(np.float64)
    w = np.exp(b - np.max(b))
    w = w / w.sum()
    return np.einsum("nmd,m->nd", blocks, w)


def layer(x, xI, q, qI, w, sink, *, m, k, W, dr, base, eps, b, bI, gamma_kv, gamma_q,
          sparse=True):
    """One sequence, tokens at positions 0..T-1, one query per token.
    Returns (out [T, H, d], topk [T, k] or None)."""
    T, d = x.shape
    H = q.shape[1]
    N = T // m
    # compressed entries at block start positions, stored as f32
    comp = f32(rope_complex(rms(softmax_pool(x, m, np.asarray(b, np.float64)), gamma_kv, eps),
                            np.arange(N) * m, dr, base))
    win = f32(rope_complex(rms(x.astype(np.float64), gamma_kv, eps), np.arange(T), dr, base))
    t = np.arange(T)
    visible = np.arange(N)[None, :] < ((t + 1) // m)[:, None]          # [T, N]
    sel = visible.copy()
    top = None
    if sparse:
        keys = f32(softmax_pool(xI, m, np.asarray(bI, np.float64)))      # [N, di]
        dots = np.einsum("thi,ni->thn", qI.astype(np.float64), keys)
        S = np.einsum("th,thn->tn", w.astype(np.float64), np.maximum(dots, 0.0))
        sel = np.zeros_like(visible)
        top = np.full((T, k), -1, np.int32)
        for ti in range(T):
            cand = np.nonzero(visible[ti])[0]
            order = np.lexsort((cand, -S[ti, cand]))                  # score desc, index asc
            chosen = np.sort(cand[order[:k]])
            sel[ti, chosen] = True
            top[ti, :len(chosen)] = chosen
    in_win = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - W)  # [T, T]
    mask = np.concatenate([sel, in_win], axis=1)                          # [T, N+T]
    E = np.concatenate([comp, win], axis=0)                               # [N+T, d]
    qh = rope_complex(rms(q.astype(np.float64), gamma_q, eps), t[:, None] * np.ones((1, H)), dr, base)
    logits = np.einsum("thd,ed->the", qh, E) / np.sqrt(d)
    logits = np.where(mask[:, None, :], logits, -np.inf)
    full = np.concatenate([logits, np.broadcast_to(np.asarray(sink, np.float64)[None, :, None], (T, H, 1))], axis=2)
    mx = np.max(full, axis=2, keepdims=True)
    p = np.exp(full - mx)
    p = p / p.sum(axis=2, keepdims=True)
    o = np.einsum("the,ed->thd", p[:, :, :-1], E)
    o = rope_complex(o, -t[:, None] * np.ones((1, H)), dr, base)
    return o, top
