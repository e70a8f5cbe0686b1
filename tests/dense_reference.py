"""Dense brute-force form of the MoE layer, for pinning the oracle.

Independent of ``oracle/``: numpy float64 matrix products over ALL experts,
with a 0/1 mask from a library sort, instead of the oracle's routing loops,
counting-sort dispatch and per-pair evaluation.

  out[t] = sum_e mask[t, e] * p[t, e] * y_e(h[t])
         + sigmoid(h[t] . w_sg) * sum_j y^sh_j(h[t])

p = softmax over all experts; mask = the K largest logits, ties to the lower
id (np.lexsort); y_e = SwiGLU expert e (blog page, section 2.2 Steps 1-5).
Tiny sizes only.
"""
import numpy as np


def f64(a):
    return np.asarray(a, dtype=np.float64)


def topk_mask(logits32: np.ndarray, K: int) -> np.ndarray:
    T, E = logits32.shape
    mask = np.zeros((T, E), bool)
    ids = np.arange(E)
    for t in range(T):
        order = np.lexsort((ids, -logits32[t].astype(np.float64)))
        mask[t, order[:K]] = True
    return mask


def swiglu(x, g, u, d):
    a = x @ f64(g).T
    b = x @ f64(u).T
    hm = (a / (1.0 + np.exp(-a))) * b
    return hm @ f64(d).T


def dense_layer(h, w_router, bias, w_sg, experts, shared, K, expert_mask=None,
                x_override=None):
    """experts: list over logical experts of (g, u, d); shared: list or None.
    expert_mask [E] bool: experts whose output this GPU contributes (rank
    share); x_override [T, H]: the values the experts see (fp8 path)."""
    x = f64(h)
    lg = x @ f64(w_router).T
    logits32 = lg.astype(np.float32)
    if bias is not None:
        logits32 = logits32 + bias.astype(np.float32)
    l64 = logits32.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    p32 = p.astype(np.float32).astype(np.float64)
    mask = topk_mask(logits32, K)
    xe = x if x_override is None else f64(x_override)
    out = np.zeros_like(x)
    for e, (g, u, d) in enumerate(experts):
        if expert_mask is not None and not expert_mask[e]:
            continue
        sel = mask[:, e]
        if not sel.any():
            continue
        y = swiglu(xe[sel], g, u, d).astype(np.float32).astype(np.float64)
        out[sel] += p32[sel, e][:, None] * y
    if shared:
        gs = 1.0 / (1.0 + np.exp(-(x @ f64(w_sg)).astype(np.float32).astype(np.float64)))
        sh = sum(swiglu(x, *s).astype(np.float32).astype(np.float64) for s in shared)
        out += gs[:, None] * sh
    return out, logits32, mask
