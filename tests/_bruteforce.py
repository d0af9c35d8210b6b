"""Scalar-loop brute force of the looped decoder for tiny shapes (pins the
vectorised oracle's indexing: which operand is transposed, which positions a
query sees, where each weight enters). Pure Python floats, no numpy algebra;
exact arithmetic (no rounding points). Written from the model description on
the TinyLoop architecture-exclusive features page (introduction and 'Store-h
KV cache'): h = RMSNorm(x); K_j = W_k h_j and V_j = W_v h_j rebuilt from the
stored h of every visible position; per-head softmax attention; W_o; RMSNorm;
GELU MLP; final RMSNorm; LM head.
"""
import math


def _matvec(W, v):
    return [sum(W[r][c] * v[c] for c in range(len(v))) for r in range(len(W))]


def _rms(x, g, eps):
    ms = sum(t * t for t in x) / len(x)
    inv = 1.0 / math.sqrt(ms + eps)
    return [g[i] * x[i] * inv for i in range(len(x))]


def _gelu(t):
    return 0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0)))


def run_sequence(weights, n_heads, n_pre, loops, tokens, eps):
    """Feed ``tokens`` one position at a time; return per-position logits and
    the stored h per (layer, position)."""
    embed = weights["embed"]
    D = len(embed[0])
    d = D // n_heads
    layers = weights["layers"]
    stored = {}            # (layer, pos) -> h
    all_logits = []
    for pos, tok in enumerate(tokens):
        x = list(embed[tok])
        for layer in range(n_pre + loops):
            lw = layers[min(layer, n_pre)]
            wq = lw["w_qkv"][0:D]
            wk = lw["w_qkv"][D:2 * D]
            wv = lw["w_qkv"][2 * D:3 * D]
            h = _rms(x, lw["norm1"], eps)
            stored[(layer, pos)] = h
            q = [t / math.sqrt(d) for t in _matvec(wq, h)]
            o = [0.0] * D
            for head in range(n_heads):
                cols = range(head * d, (head + 1) * d)
                scores = []
                vals = []
                for j in range(pos + 1):
                    kj = _matvec(wk, stored[(layer, j)])
                    vj = _matvec(wv, stored[(layer, j)])
                    scores.append(sum(q[c] * kj[c] for c in cols))
                    vals.append([vj[c] for c in cols])
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                z = sum(e)
                for jj in range(len(e)):
                    for t, c in enumerate(cols):
                        o[c] += e[jj] / z * vals[jj][t]
            ao = _matvec(lw["w_o"], o)
            x = [x[i] + ao[i] for i in range(D)]
            u = _rms(x, lw["norm2"], eps)
            a = [_gelu(t) for t in _matvec(lw["w_up"], u)]
            dn = _matvec(lw["w_down"], a)
            x = [x[i] + dn[i] for i in range(D)]
        z = _rms(x, weights["final_norm"], eps)
        all_logits.append(_matvec(weights["lm_head"], z))
    return all_logits, stored
