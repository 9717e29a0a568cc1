"""Pure-Python brute force (nested loops, math module only) for tiny inputs.

Written independently of the oracle's numpy code: no numpy, no scipy.  Used
only to pin the oracle on tiny shapes.
"""
import math


def matmul(X, W):
    n, k, m = len(X), len(W), len(W[0])
    assert all(len(r) == k for r in X)
    return [[sum(X[i][t] * W[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def add_row(Y, b):
    return [[y + bb for y, bb in zip(r, b)] for r in Y]


def gelu(x):
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def silu(x):
    return x / (1.0 + math.exp(-x))


def apply(f, Y):
    return [[f(v) for v in r] for r in Y]


def mlp_gelu(X, A, a, B, b):
    Z = matmul(X, A)
    if a is not None:
        Z = add_row(Z, a)
    Y = matmul(apply(gelu, Z), B)
    if b is not None:
        Y = add_row(Y, b)
    return Y


def mlp_swiglu(X, Wg, Wu, Wd):
    G = matmul(X, Wg)
    U = matmul(X, Wu)
    H = [[silu(g) * u for g, u in zip(rg, ru)] for rg, ru in zip(G, U)]
    return matmul(H, Wd)


def attention(Q, K, V, batch, seq, heads):
    d = len(Q[0]) // heads
    out = [[0.0] * len(Q[0]) for _ in Q]
    for b in range(batch):
        for h in range(heads):
            for t in range(seq):
                qi = b * seq + t
                scores = []
                for s in range(t + 1):
                    ki = b * seq + s
                    dot = 0.0
                    for c in range(d):
                        dot += Q[qi][h * d + c] * K[ki][h * d + c]
                    scores.append(dot / math.sqrt(d))
                mx = max(scores)
                w = [math.exp(x - mx) for x in scores]
                z = sum(w)
                for c in range(d):
                    out[qi][h * d + c] = sum(w[s] * V[b * seq + s][h * d + c] for s in range(t + 1)) / z
    return out


def attention_block(X, Wq, Wk, Wv, Wo, batch, seq, heads):
    O = attention(matmul(X, Wq), matmul(X, Wk), matmul(X, Wv), batch, seq, heads)
    return matmul(O, Wo)


def rmsnorm(X, g, eps):
    out = []
    for row in X:
        ms = sum(v * v for v in row) / len(row)
        inv = 1.0 / math.sqrt(ms + eps)
        out.append([v * inv * gg for v, gg in zip(row, g)])
    return out


def cross_entropy(logits, labels):
    """-log softmax at the label, per row, with plain loops."""
    out = []
    for row, y in zip(logits, labels):
        m = max(row)
        s = sum(math.exp(v - m) for v in row)
        out.append(math.log(s) + m - row[y])
    return out



def layernorm(X, g, b, eps):
    """Plain loops: mean, biased variance, then (x - mean)/sqrt(var + eps)*g + b."""
    out = []
    for row in X:
        n = len(row)
        mean = sum(row) / n
        var = sum((v - mean) ** 2 for v in row) / n
        inv = 1.0 / math.sqrt(var + eps)
        out.append([(v - mean) * inv * gg + bb for v, gg, bb in zip(row, g, b)])
    return out
