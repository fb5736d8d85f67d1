"""Chunk-parallel fp64 form of the KDA forward (a cross-check, not the oracle).

TEST INFRASTRUCTURE ONLY.  This computes the same forward as the token
recurrence in ``kda_oracle.c`` through the per-chunk (WY / UT) algebra that the
GPU kernels also follow, so that the algebra itself is pinned on the CPU:

per chunk of L <= C tokens entering with state S0 (K x V), with gamma the
chunk-local inclusive cumulative sum of the log-decay g (a K-vector per row):

    Akk[r,i] = sum_c k^[r,c] k^[i,c] exp(gamma[r,c] - gamma[i,c])      i <  r
    Aqk[r,i] = sum_c q^[r,c] k^[i,c] exp(gamma[r,c] - gamma[i,c])      i <= r
    Tinv     = (I + Diag(beta) Akk)^-1
    W = Tinv Diag(beta) (K^ * exp(gamma)),  U = Tinv Diag(beta) V
    Delta = U - W S0
    O     = scale ((Q^ * exp(gamma)) S0 + Aqk Delta)
    S_L   = Diag(exp(gamma_L)) S0 + (K^ * exp(gamma_L - gamma))^T Delta

It uses numpy's matmul and solve as steps and nothing else; it takes its
q^/k^/g/beta from the oracle's prologue.  It is not used as a parity
reference for the GPU path.
"""
from __future__ import annotations

import numpy as np


def chunk_step(qn, kn, v, g, b, S0, scale):
    """One chunk.  qn, kn, g: [L,K]; v: [L,V]; b: [L]; S0: [K,V].  Returns (O, S_L)."""
    L = qn.shape[0]
    gam = np.cumsum(g, axis=0)
    diff = gam[:, None, :] - gam[None, :, :]            # [r, i, c] = gamma_r - gamma_i
    lower_strict = np.tril(np.ones((L, L), bool), -1)
    lower = np.tril(np.ones((L, L), bool), 0)
    # exp only where i <= r (there gamma_r - gamma_i <= 0 because g <= 0)
    dec = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
    Akk = np.einsum("rc,ic,ric->ri", kn, kn, dec) * lower_strict
    Aqk = np.einsum("rc,ic,ric->ri", qn, kn, dec) * lower
    M = np.eye(L) + b[:, None] * Akk
    W = np.linalg.solve(M, b[:, None] * (kn * np.exp(gam)))
    U = np.linalg.solve(M, b[:, None] * v)
    Delta = U - W @ S0
    O = scale * ((qn * np.exp(gam)) @ S0 + Aqk @ Delta)
    gl = gam[-1]
    SL = np.exp(gl)[:, None] * S0 + (kn * np.exp(gl[None, :] - gam)).T @ Delta
    return O, SL


def kda_fwd_chunked(qn, kn, v, g, b, scale, chunk_size, cu_seqlens=None, initial_state=None):
    """Chunked forward over [B,T,H,*] fp64 inputs.  Chunks restart at every sequence start."""
    B, T, H, K = qn.shape
    V = v.shape[-1]
    if cu_seqlens is None:
        seqs = [(bb, 0, T) for bb in range(B)]
    else:
        cu = np.asarray(cu_seqlens)
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, H, V))
    fin = np.zeros((len(seqs), H, K, V))
    for n, (row, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((K, V)) if initial_state is None else np.array(initial_state[n, h], np.float64)
            for c0 in range(t0, t1, chunk_size):
                c1 = min(c0 + chunk_size, t1)
                O, S = chunk_step(qn[row, c0:c1, h], kn[row, c0:c1, h], np.asarray(v[row, c0:c1, h], np.float64),
                                  g[row, c0:c1, h], b[row, c0:c1, h], S, scale)
                o[row, c0:c1, h] = O
            fin[n, h] = S
    return o, fin
