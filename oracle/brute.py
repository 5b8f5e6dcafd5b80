"""Pure-Python loop versions for tiny inputs: a second, independently
written statement of what the hot path computes, used only to pin
``oracle.reference`` in the CPU tests.

TEST INFRASTRUCTURE ONLY.  Nested lists and the ``math`` module, nothing
else; the formulas are taken straight from their definitions and not from
the vectorised oracle:

* attention uses exp(s_j) / sum_k exp(s_k) with no max subtraction (fine for
  the small scores these tests use), unlike the oracle's max-shifted form;
* the Ulysses exchanges are stated end to end on the *global* tensor (which
  rows and heads a rank owns before and after), never through the
  pack / unpack index maps.
"""

from __future__ import annotations

import math


def attention(q, k, v, scale):
    """q [B][Sq][H][D], k/v [B][Skv][H][D] nested lists -> (O, LSE).

    edge-dit.cpp "Parallel execution", Ulysses section: softmax(Q K^T *
    scale) V per head; LSE = ln sum_j exp(s_j).
    """
    B, Sq, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Skv = len(k[0])
    O = [[[[0.0] * D for _ in range(H)] for _ in range(Sq)] for _ in range(B)]
    LSE = [[[-math.inf] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                if Skv == 0:
                    continue
                e = []
                for j in range(Skv):
                    s = scale * sum(q[b][i][h][d] * k[b][j][h][d] for d in range(D))
                    e.append(math.exp(s))
                z = sum(e)
                for d in range(D):
                    O[b][i][h][d] = sum(e[j] * v[b][j][h][d] for j in range(Skv)) / z
                LSE[b][h][i] = math.log(z)
    return O, LSE


def ulysses_seq_to_head(X, U, S_loc, H_loc):
    """What Ulysses rank r holds after the sequence-to-head exchange.

    X is the *global* tensor [B][S][H][D] (S real rows).  Rank r owns heads
    r*H_loc .. r*H_loc + H_loc - 1 for the whole sequence; a head index at or
    past H is a pad head and holds zeros (cache-dit "Any Head Num").
    Returns, per rank, [B][S][H_loc][D].
    """
    B, S, H, D = len(X), len(X[0]), len(X[0][0]), len(X[0][0][0])
    out = []
    for r in range(U):
        Y = [[[[0.0] * D for _ in range(H_loc)] for _ in range(S)] for _ in range(B)]
        for b in range(B):
            for t in range(S):
                for hh in range(H_loc):
                    g = r * H_loc + hh
                    if g < H:
                        for d in range(D):
                            Y[b][t][hh][d] = X[b][t][g][d]
        out.append(Y)
    return out


def ulysses_head_to_seq(O, U, S_loc):
    """What Ulysses rank r holds after the head-to-sequence exchange.

    O is the *global* result [B][S][H][D].  Rank r owns global rows
    r*S_loc .. r*S_loc + S_loc - 1 with all H heads; a row at or past S is a
    pad row and holds zeros.  Returns, per rank, [B][S_loc][H][D].
    """
    B, S, H, D = len(O), len(O[0]), len(O[0][0]), len(O[0][0][0])
    out = []
    for r in range(U):
        Z = [[[[0.0] * D for _ in range(H)] for _ in range(S_loc)] for _ in range(B)]
        for b in range(B):
            for s in range(S_loc):
                t = r * S_loc + s
                if t < S:
                    for h in range(H):
                        for d in range(D):
                            Z[b][s][h][d] = O[b][t][h][d]
        out.append(Z)
    return out


def local_shard(X, r, S_loc):
    """Rows r*S_loc .. r*S_loc + S_loc - 1 of the global [B][S][H][D] tensor,
    zero-filled past S: the sequence-sharded input of Ulysses rank r
    (edge-dit.cpp: padded global tensor, then the rank's local view)."""
    B, S, H, D = len(X), len(X[0]), len(X[0][0]), len(X[0][0][0])
    Y = [[[[0.0] * D for _ in range(H)] for _ in range(S_loc)] for _ in range(B)]
    for b in range(B):
        for s in range(S_loc):
            t = r * S_loc + s
            if t < S:
                for h in range(H):
                    for d in range(D):
                        Y[b][s][h][d] = X[b][t][h][d]
    return Y


def cfg(u, c, g):
    """edge-dit.cpp CFG section, elementwise on flat lists."""
    return [ui + g * (ci - ui) for ui, ci in zip(u, c)]
