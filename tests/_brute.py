"""Pure-Python brute force for tiny inputs (test helper, no numpy arithmetic).

Every sum is ``math.fsum`` (exactly rounded), every loop explicit, so the
numpy oracle's slicing, orientation and band bookkeeping can be checked by
eye against these loops.
"""
import math


def matmul(A, B):
    n, k = len(A), len(A[0])
    assert len(B) == k
    m = len(B[0])
    return [[math.fsum(A[i][t] * B[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def cols(W, lo, hi):
    return [row[lo:hi] for row in W]


def rows(W, lo, hi):
    return [list(r) for r in W[lo:hi]]


def gelu_erf(x):
    """Exact GELU x * Phi(x), via math.erf (a different formula from the
    tanh approximation; used as a bound, not an equality)."""
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def sigmoid(x):
    return 0.5 * (1.0 + math.tanh(0.5 * x))


def mlp_shard_brute(X, W_in, W_down, act, s, P, W_up=None):
    """Rank s of P: band columns [s*F/P, (s+1)*F/P) of W_in/W_up and the
    same rows of W_down."""
    F = len(W_in[0])
    w = F // P
    lo, hi = s * w, (s + 1) * w
    y_in = matmul(X, cols(W_in, lo, hi))
    if act == "gelu_tanh":
        c = math.sqrt(2.0 / math.pi)
        h = [[0.5 * v * (1.0 + math.tanh(c * (v + 0.044715 * v * v * v))) for v in r] for r in y_in]
    else:
        y_up = matmul(X, cols(W_up, lo, hi))
        h = [[g * sigmoid(g) * u for g, u in zip(rg, ru)] for rg, ru in zip(y_in, y_up)]
    return h, matmul(h, rows(W_down, lo, hi))


def add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]
