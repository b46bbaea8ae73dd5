"""Brute-force triangle multiplicative update in pure Python loops.

Written element by element from the operator's definition (scalar math only,
no NumPy), for tiny inputs: the independent check the fp64 oracle is pinned to.
Nested lists in, nested lists out.
"""

import math


def _ln(vec, gamma, beta, eps):
    n = len(vec)
    mu = sum(vec) / n
    var = sum((v - mu) * (v - mu) for v in vec) / n
    inv = 1.0 / math.sqrt(var + eps)
    return [(vec[t] - mu) * inv * gamma[t] + beta[t] for t in range(n)]


def _sig(t):
    return 1.0 / (1.0 + math.exp(-t))


def _dot(row, vec):
    s = 0.0
    for t in range(len(vec)):
        s += row[t] * vec[t]
    return s


def brute_force(z, mask, w, direction, eps=1e-5):
    """z[b][i][j][ch], mask[b][i][j], w: dict of nested lists (matrices [out][in])."""
    B, N = len(z), len(z[0])
    c_z, c = len(z[0][0][0]), len(w["b_a_gate"])
    zhat = [[[_ln(z[b][i][j], w["ln_in_gamma"], w["ln_in_beta"], eps) for j in range(N)]
             for i in range(N)] for b in range(B)]

    def operand(b, i, j, which):
        zz = zhat[b][i][j]
        res = []
        for ch in range(c):
            gate = _dot(w[f"w_{which}_gate"][ch], zz) + w[f"b_{which}_gate"][ch]
            proj = _dot(w[f"w_{which}_proj"][ch], zz) + w[f"b_{which}_proj"][ch]
            res.append(mask[b][i][j] * _sig(gate) * proj)
        return res

    A = [[[operand(b, i, j, "a") for j in range(N)] for i in range(N)] for b in range(B)]
    Bo = [[[operand(b, i, j, "b") for j in range(N)] for i in range(N)] for b in range(B)]
    out = [[[[0.0] * c_z for _ in range(N)] for _ in range(N)] for _ in range(B)]
    for b in range(B):
        for i in range(N):
            for j in range(N):
                x = [0.0] * c
                for k in range(N):
                    for ch in range(c):
                        if direction == "outgoing":
                            x[ch] += A[b][i][k][ch] * Bo[b][j][k][ch]
                        else:
                            x[ch] += A[b][k][i][ch] * Bo[b][k][j][ch]
                xh = _ln(x, w["ln_out_gamma"], w["ln_out_beta"], eps)
                for o in range(c_z):
                    p = _dot(w["w_out"][o], xh) + w["b_out"][o]
                    g = _sig(_dot(w["w_gate"][o], zhat[b][i][j]) + w["b_gate"][o])
                    out[b][i][j][o] = mask[b][i][j] * g * p
    return out
