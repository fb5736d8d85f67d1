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

``kda_bwd_chunked`` is the reverse mode of the same chunk algebra (the
decomposition the GPU backward follows): a forward pass keeping each chunk's
entering state S0 and Delta, a reverse pass over chunks carrying the state
gradient (dDelta = scale Aqk^T dO + Kbar dS_L, dS0 = scale Q~^T dO +
e^gamma_L dS_L - W^T dDelta), and per chunk the gradients through Tinv, the WY
factors and the pairwise decayed products.  It returns the gradients of
q^, k^, v, g, beta and the initial state and is pinned against finite
differences of the token recurrence.
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


def kda_bwd_chunked(qn, kn, v, g, b, d_o, d_final, scale, chunk_size, cu_seqlens=None,
                    initial_state=None):
    """Gradients of sum(d_o * O) + sum(d_final * S_final) for the chunked
    forward with respect to qn, kn, v, g, b ([B,T,H,*]) and the initial state
    ([N,H,K,V]).  Returns a dict dqn, dkn, dv, dg, db, dinit."""
    B, T, H, K = qn.shape
    V = v.shape[-1]
    C = chunk_size
    seqs = [(bb, 0, T) for bb in range(B)] if cu_seqlens is None else \
        [(0, int(cu_seqlens[n]), int(cu_seqlens[n + 1])) for n in range(len(cu_seqlens) - 1)]
    N = len(seqs)
    out = dict(dqn=np.zeros(qn.shape), dkn=np.zeros(kn.shape), dv=np.zeros(v.shape),
               dg=np.zeros(g.shape), db=np.zeros(b.shape), dinit=np.zeros((N, H, K, V)))
    for n, (bb, t0, t1) in enumerate(seqs):
        for h in range(H):
            chunks = []
            for s0 in range(t0, t1, C):
                e0 = min(s0 + C, t1)
                L = e0 - s0
                q_, k_, v_ = qn[bb, s0:e0, h], kn[bb, s0:e0, h], v[bb, s0:e0, h]
                gam = np.cumsum(g[bb, s0:e0, h], axis=0)
                b_ = b[bb, s0:e0, h]
                lower = np.tril(np.ones((L, L), bool), 0)
                strict = np.tril(np.ones((L, L), bool), -1)
                diff = gam[:, None, :] - gam[None, :, :]
                E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
                Akk = np.einsum("rc,ic,ric->ri", k_, k_, E) * strict
                Aqk = np.einsum("rc,ic,ric->ri", q_, k_, E) * lower
                Tm = np.linalg.inv(np.eye(L) + b_[:, None] * Akk)
                Kt, Qt = k_ * np.exp(gam), q_ * np.exp(gam)
                gL = gam[-1]
                Kb = k_ * np.exp(gL[None] - gam)
                W, U = Tm @ (b_[:, None] * Kt), Tm @ (b_[:, None] * v_)
                chunks.append(dict(s=s0, e=e0, L=L, q=q_, k=k_, v=v_, gam=gam, b=b_, E=E, Akk=Akk,
                                   Aqk=Aqk, Tm=Tm, Kt=Kt, Qt=Qt, gL=gL, Kb=Kb, W=W, U=U,
                                   lower=lower, strict=strict))
            S = initial_state[n, h].copy() if initial_state is not None else np.zeros((K, V))
            for P in chunks:
                P["S0"] = S.copy()
                P["D"] = P["U"] - P["W"] @ S
                S = np.exp(P["gL"])[:, None] * S + P["Kb"].T @ P["D"]
            dS = d_final[n, h].copy() if d_final is not None else np.zeros((K, V))
            for P in reversed(chunks):
                dO = d_o[bb, P["s"]:P["e"], h]
                P["dSL"] = dS.copy()
                P["dD"] = scale * P["Aqk"].T @ dO + P["Kb"] @ dS
                dS = scale * P["Qt"].T @ dO + np.exp(P["gL"])[:, None] * dS - P["W"].T @ P["dD"]
            out["dinit"][n, h] = dS
            for P in chunks:
                dO = d_o[bb, P["s"]:P["e"], h]
                q_, k_, E, S0, dSL, D, dD = P["q"], P["k"], P["E"], P["S0"], P["dSL"], P["D"], P["dD"]
                dq = np.zeros_like(q_)
                dk = np.zeros_like(k_)
                dgam = np.zeros_like(q_)
                # Aqk (incl. diagonal) and the Q~ S0 term of O
                dAqk = np.where(P["lower"], scale * dO @ D.T, 0.0)
                Em = np.where(P["lower"][:, :, None], E, 0.0)
                dq += np.einsum("ri,ic,ric->rc", dAqk, k_, Em)
                dk += np.einsum("ri,rc,ric->ic", dAqk, q_, Em)
                t = np.einsum("ri,rc,ic,ric->ric", dAqk, q_, k_, Em)
                dgam += t.sum(1) - t.sum(0)
                dQt = scale * dO @ S0.T
                dq += dQt * np.exp(P["gam"])
                dgam += dQt * P["Qt"]
                # S_L = e^gamma_L S0 + Kbar^T Delta
                dKb = D @ dSL.T
                dk += dKb * np.exp(P["gL"][None] - P["gam"])
                tt = dKb * P["Kb"]
                dgam -= tt
                dgam[-1] += tt.sum(0) + np.exp(P["gL"]) * (dSL * S0).sum(1)
                # W, U through Tinv
                dW, dU = -dD @ S0.T, dD
                Xk, Xv = P["b"][:, None] * P["Kt"], P["b"][:, None] * P["v"]
                dT = dW @ Xk.T + dU @ Xv.T
                dXk, dXv = P["Tm"].T @ dW, P["Tm"].T @ dU
                out["dv"][bb, P["s"]:P["e"], h] = P["b"][:, None] * dXv
                db = (dXk * P["Kt"]).sum(1) + (dXv * P["v"]).sum(1)
                dKt = P["b"][:, None] * dXk
                dk += dKt * np.exp(P["gam"])
                dgam += dKt * P["Kt"]
                dN = -P["Tm"].T @ dT @ P["Tm"].T
                dAkk = np.where(P["strict"], P["b"][:, None] * dN, 0.0)
                db += np.where(P["strict"], dN * P["Akk"], 0.0).sum(1)
                Es = np.where(P["strict"][:, :, None], E, 0.0)
                dk += np.einsum("ri,ic,ric->rc", dAkk, k_, Es)
                dk += np.einsum("ri,rc,ric->ic", dAkk, k_, Es)
                t = np.einsum("ri,rc,ic,ric->ric", dAkk, k_, k_, Es)
                dgam += t.sum(1) - t.sum(0)
                out["dqn"][bb, P["s"]:P["e"], h] = dq
                out["dkn"][bb, P["s"]:P["e"], h] = dk
                out["dg"][bb, P["s"]:P["e"], h] = np.cumsum(dgam[::-1], 0)[::-1]
                out["db"][bb, P["s"]:P["e"], h] = db
    return out
