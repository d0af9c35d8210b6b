"""Scalar-loop brute force of the looped decoder for tiny shapes (pins the
vectorised oracle's indexing: which operand is transposed, which positions a
query sees, where each weight enters, and where the fp16 model rounds). Pure
Python floats, no numpy algebra. Written from the model description on the
TinyLoop architecture-exclusive features page (introduction and 'Store-h KV
cache'): h = RMSNorm(x) is stored per position and layer; K_j = W_k h_j and
V_j = W_v h_j are rebuilt from the stored h of every visible position;
per-head softmax attention; W_o; RMSNorm; GELU MLP; final RMSNorm; LM head.

Rounding points (names used by ``run_sequence(rounding=...)``; each one rounds
a value to fp16, IEEE round-to-nearest-even, through the standard library's
binary16 packing rather than numpy):
  R1   h, the pre-QKV norm output, before it is stored and projected;
  R3   the dequantised h' = fp16(q * s) of the INT4 / INT8 codecs;
  R4o  the attention output o before W_o;
  R4u  the norm-2 output before the MLP up-projection;
  R4a  the GELU output before the down-projection;
  R4z  the final-norm output before the LM head;
  R5   stored K and V (the stored-K/V mode) at write time.
The codec (mode "int4": groups of 32 along d_model, divisor 7, clamp [-8, 7];
"int8": one group per token, divisor 127, clamp [-127, 127]) follows the
symmetric absmax rule: s = fp16(fp32(absmax / qmax)), q = round half to even
of fp32(h / s), q = 0 when s is 0. A float32 quotient of two float32 values
is obtained exactly by dividing in double and rounding once to float32 (the
double has more than twice the float32 precision plus two bits).
"""
import math
import struct

ALL_ROUNDING = frozenset(("R1", "R3", "R4o", "R4u", "R4a", "R4z", "R5"))


def f16(t):
    """Round a Python float to the nearest binary16 value (ties to even)."""
    try:
        return struct.unpack("<e", struct.pack("<e", t))[0]
    except OverflowError:
        return math.copysign(math.inf, t)


def f32(t):
    """Round a Python float to the nearest binary32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", t))[0]


def _matvec(W, v):
    return [sum(W[r][c] * v[c] for c in range(len(v))) for r in range(len(W))]


def _rms(x, g, eps):
    ms = sum(t * t for t in x) / len(x)
    inv = 1.0 / math.sqrt(ms + eps)
    return [g[i] * x[i] * inv for i in range(len(x))]


def _gelu(t):
    return 0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0)))


def codec_roundtrip(h, group, qmax, qmin):
    """Encode fp16 values h (a list) in groups of ``group`` and decode them:
    returns (codes, scales, h') with h' = fp16(q * s)."""
    codes, scales, out = [], [], []
    for g0 in range(0, len(h), group):
        grp = h[g0:g0 + group]
        am = max(abs(t) for t in grp)
        s = f16(f32(am / float(qmax)))
        scales.append(s)
        for t in grp:
            q = 0 if s == 0 else max(qmin, min(qmax, round(f32(t / s))))
            codes.append(q)
            out.append(q * s)
    return codes, scales, out


def run_sequence(weights, n_heads, n_pre, loops, tokens, eps, rounding=frozenset(), mode="h"):
    """Feed ``tokens`` one position at a time; return per-position logits and
    the stored h per (layer, position).

    ``mode``: "h" (h stored as is), "kv" (K = W_k h and V = W_v h stored at
    write time), "int4" / "int8" (h stored through the codec). ``rounding``:
    the rounding points to apply (see the module docstring)."""
    rd = {p: (f16 if p in rounding else (lambda t: t)) for p in ALL_ROUNDING}
    embed = weights["embed"]
    D = len(embed[0])
    d = D // n_heads
    layers = weights["layers"]
    stored = {}            # (layer, pos) -> h (float modes) or h' (codec modes)
    stored_kv = {}         # (layer, pos) -> (K, V) in the stored-K/V mode
    all_logits = []
    for pos, tok in enumerate(tokens):
        x = list(embed[tok])
        for layer in range(n_pre + loops):
            lw = layers[min(layer, n_pre)]
            wq = lw["w_qkv"][0:D]
            wk = lw["w_qkv"][D:2 * D]
            wv = lw["w_qkv"][2 * D:3 * D]
            h = [rd["R1"](t) for t in _rms(x, lw["norm1"], eps)]
            if mode in ("int4", "int8"):
                group, qmax, qmin = (32, 7, -8) if mode == "int4" else (D, 127, -127)
                _, _, hp = codec_roundtrip(h, group, qmax, qmin)
                stored[(layer, pos)] = [rd["R3"](t) for t in hp]
            else:
                stored[(layer, pos)] = h
            if mode == "kv":
                stored_kv[(layer, pos)] = ([rd["R5"](t) for t in _matvec(wk, h)],
                                           [rd["R5"](t) for t in _matvec(wv, h)])
            q = [t / math.sqrt(d) for t in _matvec(wq, h)]
            o = [0.0] * D
            for head in range(n_heads):
                cols = range(head * d, (head + 1) * d)
                scores = []
                vals = []
                for j in range(pos + 1):
                    if mode == "kv":
                        kj, vj = stored_kv[(layer, j)]
                    else:
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
            ao = _matvec(lw["w_o"], [rd["R4o"](t) for t in o])
            x = [x[i] + ao[i] for i in range(D)]
            u = [rd["R4u"](t) for t in _rms(x, lw["norm2"], eps)]
            a = [rd["R4a"](_gelu(t)) for t in _matvec(lw["w_up"], u)]
            dn = _matvec(lw["w_down"], a)
            x = [x[i] + dn[i] for i in range(D)]
        z = [rd["R4z"](t) for t in _rms(x, weights["final_norm"], eps)]
        all_logits.append(_matvec(weights["lm_head"], z))
    return all_logits, stored
