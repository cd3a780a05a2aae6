"""Scalar-loop reference for tiny shapes (test helper, pure Python).

An independent restatement of the oracle's forward with explicit index loops:
no numpy matmul, rotary embedding written as complex multiplication, softmax
written term by term. Used only to pin oracle.model on shapes of a few
elements, where a transposed operand, a wrong rotary pairing or a missing
scale shows up immediately.
"""
import cmath
import math


def _matvec(W, x):
    # W stored [out][in]; y_o = sum_i W[o][i] * x[i]
    return [sum(W[o][i] * x[i] for i in range(len(x))) for o in range(len(W))]


def _rms(x, g, eps):
    s = math.sqrt(sum(v * v for v in x) / len(x) + eps)
    return [x[i] / s * g[i] for i in range(len(x))]


def _rope_head(u, pos, base):
    D = len(u)
    half = D // 2
    out = [0.0] * D
    for i in range(half):
        theta = pos * base ** (-2.0 * i / D)
        z = complex(u[i], u[i + half]) * cmath.exp(1j * theta)
        out[i], out[i + half] = z.real, z.imag
    return out


def forward(weights, tokens, rows, cache, n_heads, eps=1e-5, base=10000.0, rnd=lambda v: v):
    """weights: dict of nested lists (embed, layers[...], final_norm, lm_head).

    cache: list per layer of [K, V], each a list of L row-lists; rows of
    ``rows`` are overwritten. Returns (hidden rows, logits rows).
    """
    d = len(weights["embed"][0])
    D = d // n_heads
    L = len(cache[0][0]) if cache else len(tokens)
    h = [list(weights["embed"][tokens[p]]) for p in rows]
    for li, lw in enumerate(weights["layers"]):
        K, V = cache[li]
        qs = []
        for j, p in enumerate(rows):
            a = [rnd(v) for v in _rms(h[j], lw["attn_norm"], eps)]
            qkv = _matvec(lw["wqkv"], a)
            q, k, v = qkv[:d], qkv[d:2 * d], qkv[2 * d:]
            qr, kr = [], []
            for hh in range(n_heads):
                qr += _rope_head(q[hh * D:(hh + 1) * D], p, base)
                kr += _rope_head(k[hh * D:(hh + 1) * D], p, base)
            qs.append([rnd(x) for x in qr])
            K[p] = [rnd(x) for x in kr]
            V[p] = [rnd(x) for x in v]
        for j, p in enumerate(rows):
            o = [0.0] * d
            for hh in range(n_heads):
                sl = slice(hh * D, (hh + 1) * D)
                qv = qs[j][sl]
                scores = [sum(a * b for a, b in zip(qv, K[t][sl])) / math.sqrt(D) for t in range(L)]
                # weights against the power of two 2^M just above the largest one (M integer):
                # w_t = e^(s_t) / 2^M; the ones that multiply V pass through rnd, the
                # normaliser is their unrounded sum
                M = math.ceil(max(scores) / math.log(2.0))
                w = [math.exp(s - M * math.log(2.0)) for s in scores]
                tot = sum(w)
                wr = [rnd(x) for x in w]
                for e in range(D):
                    o[hh * D + e] = sum(wr[t] * V[t][hh * D + e] for t in range(L)) / tot
            o = [rnd(x) for x in o]
            h[j] = [h[j][i] + y for i, y in enumerate(_matvec(lw["wo"], o))]
            b = [rnd(v) for v in _rms(h[j], lw["mlp_norm"], eps)]
            g = _matvec(lw["w_gate"], b)
            u = _matvec(lw["w_up"], b)
            s = [rnd(gi / (1.0 + math.exp(-gi)) * ui) for gi, ui in zip(g, u)]
            h[j] = [h[j][i] + y for i, y in enumerate(_matvec(lw["w_down"], s))]
    logits = []
    for j in range(len(rows)):
        xn = [rnd(v) for v in _rms(h[j], weights["final_norm"], eps)]
        logits.append([rnd(v) for v in _matvec(weights["lm_head"], xn)])
    return h, logits
