"""fp64 chunkwise form of the (gated) delta rule -- TEST INFRASTRUCTURE.

Used only by the tests, to pin the chunk equations that the GPU kernels
implement against the token-by-token oracle (``gdn_oracle.c``).  It shares no
code with the GPU library.  Plain NumPy, small sizes only.

The chunkwise-parallel algorithm is the one of "Decoding Hybrid Linear Attention
Architectures", sec. 5 (inter-chunk state recursion and intra-chunk output), with
the WY / UT representation of "Linear Attention Variants (RetNet, GLA, DeltaNet,
Based)", section "DeltaNet: Error-Correcting Writes".  The printed formulas are
garbled; the reading used here (derived from the recurrence, and checked against
it by the tests) is, for one chunk of C positions entering with state M0 = S^T:

  G         chunk-local inclusive cumulative sum of log alpha (sec. 5: gate
            products accumulated in log space)
  Gamma     Gamma[r,i,c] = exp(G[r,c] - G[i,c]) for i <= r  (decay from i to r)
  A         A[r,i] = beta_r * sum_c K[r,c] K[i,c] Gamma[r,i,c] for i < r, else 0
  T         (I + A)^-1, unit lower triangular, by forward substitution
  W, U      W = T diag(beta) (K * e^G),  U = T diag(beta) V
  Delta     U - W M0          (the "net correction" U - W S of sec. 5)
  P         P[r,i] = sum_c Q[r,c] K[i,c] Gamma[r,i,c] for i <= r (inclusive)
  O         (Q * e^G) M0 + P Delta
  M_C       diag(e^{G_C}) M0 + (K * e^{G_C - G})^T Delta

e^G is the decay from the chunk start to position r, e^{G_C - G} the decay from
position i to the chunk end (the Gamma^{i->C} of sec. 5), e^{G_C} the whole-chunk
decay (gamma^C of sec. 5).  The causal mask is strict for A (a token's write does
not see itself) and inclusive for P (the read at t happens after the write at t).
"""
from __future__ import annotations

import numpy as np


def chunk_cumsum(log_alpha_chunk):
    """G: inclusive cumulative sum over the chunk positions (axis 0)."""
    return np.cumsum(log_alpha_chunk, axis=0)


def forward_substitution_inverse(A):
    """T = (I + A)^-1 for strictly lower triangular A, one row at a time:
    row r of T is e_r minus the A[r, i]-weighted sum of the earlier rows."""
    C = A.shape[0]
    T = np.zeros_like(A)
    for r in range(C):
        T[r, r] = 1.0
        for i in range(r):
            T[r] -= A[r, i] * T[i]
    return T


def chunk_step(q, k, v, beta, G, M0):
    """One chunk.  q,k [C,dk], v [C,dv], beta [C], G [C,dk] (already expanded to
    every key channel: zeros without a gate), M0 [dk,dv].  Returns a dict of the
    intermediates and the results O [C,dv], M_C [dk,dv]."""
    C = q.shape[0]
    causal_strict = np.tril(np.ones((C, C), dtype=bool), -1)
    causal_incl = np.tril(np.ones((C, C), dtype=bool), 0)
    # Gamma[r, i, c] = exp(G[r, c] - G[i, c]); only used where i <= r (exponent <= 0
    # when the gates are decays), the rest is masked before exponentiation.
    diff = G[:, None, :] - G[None, :, :]
    Gamma = np.exp(np.where(causal_incl[:, :, None], diff, 0.0)) * causal_incl[:, :, None]
    A = beta[:, None] * np.einsum("rc,ic,ric->ri", k, k, Gamma) * causal_strict
    T = forward_substitution_inverse(A)
    eG = np.exp(G)
    W = T @ (beta[:, None] * (k * eG))
    U = T @ (beta[:, None] * v)
    Delta = U - W @ M0
    P = np.einsum("rc,ic,ric->ri", q, k, Gamma) * causal_incl
    O = (q * eG) @ M0 + P @ Delta
    gC = G[-1]
    MC = np.exp(gC)[:, None] * M0 + (k * np.exp(gC[None, :] - G)).T @ Delta
    return dict(A=A, T=T, W=W, U=U, Delta=Delta, P=P, O=O, M=MC)


def fwd_sequence(q, k, v, beta, log_alpha, M0, chunk: int):
    """One sequence, one head.  q,k [T,dk], v [T,dv], beta [T], log_alpha None |
    [T] | [T,dk], M0 [dk,dv] or None.  The last chunk may be partial (it is simply
    shorter).  Returns (O [T,dv], M_T [dk,dv])."""
    T, dk = q.shape
    dv = v.shape[1]
    M = np.zeros((dk, dv)) if M0 is None else np.array(M0, dtype=np.float64)
    if log_alpha is None:
        la = np.zeros((T, dk))
    elif np.ndim(log_alpha) == 1:
        la = np.repeat(np.asarray(log_alpha, dtype=np.float64)[:, None], dk, axis=1)
    else:
        la = np.asarray(log_alpha, dtype=np.float64)
    O = np.zeros((T, dv))
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        G = chunk_cumsum(la[s:e])
        res = chunk_step(q[s:e], k[s:e], v[s:e], beta[s:e], G, M)
        O[s:e] = res["O"]
        M = res["M"]
    return O, M


def fwd(q, k, v, beta, log_alpha=None, initial_state=None, chunk: int = 64):
    """Batch mode over [B,T,H,*] arrays (fp64 numpy).  Returns (o, final_state)."""
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    fs = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            la = None if log_alpha is None else np.asarray(log_alpha, dtype=np.float64)[b, :, h]
            m0 = None if initial_state is None else np.asarray(initial_state)[b, h]
            o[b, :, h], fs[b, h] = fwd_sequence(q[b, :, h], k[b, :, h], v[b, :, h], beta[b, :, h],
                                                la, m0, chunk)
    return o, fs


def chunk_step_bwd(q, k, v, beta, g, M0, dO, dM, write="delta"):
    """Gradients of one chunk of the scalar-gated (or ungated: g = 0) delta rule, or of
    the additive write (write="add", beta None: Delta = V, no A or T, dbeta None).

    q,k [C,dk], v [C,dv], beta [C], g [C] (log decay per position), M0 [dk,dv] the
    state entering the chunk, dO [C,dv] the gradient of O and dM [dk,dv] the gradient
    of M_C.  Returns (dq, dk, dv, dbeta, dg [C], dM0).  Reverse mode through the chunk
    equations of the module docstring, step by step:
      dDelta = P^T dO + Khat dM                 (O = Qt M0 + P Delta, M_C = gam M0 + Khat^T Delta)
      Y      = T^T dDelta,  X = diag(beta)(V - Kt M0),  Delta = T X
      dM0    = Qt^T dO + gam dM - Kt^T diag(beta) Y
      dV = diag(beta) Y,  dbeta_r += Y_r . (V - Kt M0)_r,  dKt = -diag(beta) Y M0^T
      dT = dDelta X^T,  dA = -(T^T dT T^T) on the strictly lower part
      dP = dO Delta^T on the inclusive lower part,  dQt = dO M0^T,  dKhat = Delta dM^T
    then A = strict(diag(beta)(K K^T * Gamma)) and P = incl(Q K^T * Gamma) give the K,
    Q, beta and Gamma terms, Kt = e^G K, Qt = e^G Q and Khat = e^{G_C - G} K the
    rest, and dlog alpha_t is the sum of dG_r over r >= t plus dG_C."""
    C = q.shape[0]
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    incl = np.tril(np.ones((C, C), dtype=bool), 0)
    G = np.cumsum(g)
    gC = G[-1]
    Gam = np.where(incl, np.exp(np.where(incl, G[:, None] - G[None, :], 0.0)), 0.0)
    S, R = k @ k.T, q @ k.T
    if write == "add":
        return _chunk_step_bwd_add(q, k, v, G, Gam, R, M0, dO, dM)
    A = np.where(strict, beta[:, None] * S * Gam, 0.0)
    T = forward_substitution_inverse(A)
    eG, eT, gam = np.exp(G), np.exp(gC - G), np.exp(gC)
    Kt, Qt, Kh = eG[:, None] * k, eG[:, None] * q, eT[:, None] * k
    P = np.where(incl, R * Gam, 0.0)
    VmK = v - Kt @ M0
    X = beta[:, None] * VmK
    Delta = T @ X
    # backward
    dDelta = P.T @ dO + Kh @ dM
    Y = T.T @ dDelta
    dM0 = Qt.T @ dO + gam * dM - Kt.T @ (beta[:, None] * Y)
    dv = beta[:, None] * Y
    dbeta = np.sum(Y * VmK, axis=1)
    dKt = -(beta[:, None] * Y) @ M0.T
    dT = dDelta @ X.T
    dA = np.where(strict, -(T.T @ dT @ T.T), 0.0)
    dP = np.where(incl, dO @ Delta.T, 0.0)
    dQt = dO @ M0.T
    dKh = Delta @ dM.T
    dgam = np.sum(M0 * dM)
    # A = strict(diag(beta) (K K^T * Gamma))
    dbeta = dbeta + np.sum(dA * S * Gam, axis=1)
    Ea = dA * beta[:, None] * Gam
    dk = Ea @ k + Ea.T @ k
    dGam = dA * beta[:, None] * S
    # P = incl(Q K^T * Gamma)
    Ep = dP * Gam
    dq = Ep @ k
    dk = dk + Ep.T @ q
    dGam = dGam + dP * R
    # Gamma[r, i] = exp(G_r - G_i)
    wG = dGam * Gam
    dG = wG.sum(axis=1) - wG.sum(axis=0)
    # Kt, Qt, Khat and gam
    dk = dk + eG[:, None] * dKt + eT[:, None] * dKh
    dq = dq + eG[:, None] * dQt
    dG = dG + np.sum(dKt * Kt, axis=1) + np.sum(dQt * Qt, axis=1) - np.sum(dKh * Kh, axis=1)
    dgC = np.sum(dKh * Kh) + gam * dgam
    dG[-1] += dgC
    dg = np.cumsum(dG[::-1])[::-1]
    return dq, dk, dv, dbeta, dg, dM0


def _chunk_step_bwd_add(q, k, v, G, Gam, R, M0, dO, dM):
    """The additive write's chunk: O = Qt M0 + P V, M_C = gam M0 + Khat^T V (Delta = V).
    Reverse mode:
      dV = P^T dO + Khat dM,  dM0 = Qt^T dO + gam dM,
      dP = dO V^T on the inclusive lower part,  dQt = dO M0^T,  dKhat = V dM^T,
    then P = incl(Q K^T * Gamma), Qt, Khat and gam as for the delta rule."""
    C = q.shape[0]
    incl = np.tril(np.ones((C, C), dtype=bool), 0)
    gC = G[-1]
    eG, eT, gam = np.exp(G), np.exp(gC - G), np.exp(gC)
    Qt, Kh = eG[:, None] * q, eT[:, None] * k
    P = np.where(incl, R * Gam, 0.0)
    dv = P.T @ dO + Kh @ dM
    dM0 = Qt.T @ dO + gam * dM
    dP = np.where(incl, dO @ v.T, 0.0)
    dQt = dO @ M0.T
    dKh = v @ dM.T
    dgam = np.sum(M0 * dM)
    Ep = dP * Gam
    dq = Ep @ k + eG[:, None] * dQt
    dk = Ep.T @ q + eT[:, None] * dKh
    wG = dP * R * Gam
    dG = wG.sum(axis=1) - wG.sum(axis=0)
    dG = dG + np.sum(dQt * Qt, axis=1) - np.sum(dKh * Kh, axis=1)
    dG[-1] += np.sum(dKh * Kh) + gam * dgam
    dg = np.cumsum(dG[::-1])[::-1]
    return dq, dk, dv, None, dg, dM0


def chunk_step_bwd_key(q, k, v, beta, la, M0, dO, dM, write="delta"):
    """Gradients of one chunk with one decay per key channel (la [C,dk], log decays),
    for the delta write or the additive write (beta None).  The chunk equations are
    those of the module docstring with per-channel Gamma[r,i,c] = e^{G[r,c] - G[i,c]}
    inside the A and P contractions, Kt = K e^G, Qt = Q e^G, Khat = K e^{G_C - G} and
    gam = e^{G_C} per channel.  Reverse mode, step by step:
      dDelta, Y, dM0 (= Qt^T dO + diag(gam) dM - Kt^T diag(beta) Y), dV, dbeta, dKt, dT,
      dA = -(T^T dT T^T) strictly lower, dP = dO Delta^T inclusive lower, dQt = dO M0^T,
      dKhat = Delta dM^T, dgam_c = sum_j M0[c,j] dM[c,j]   (as for the scalar gate);
    then with Z[r,c] = sum_i dA[r,i] K[i,c] Gamma[r,i,c] (the A rows),
      Zc[i,c] = sum_r beta_r dA[r,i] K[r,c] Gamma[r,i,c] (the A columns),
      Pr[r,c] = sum_i dP[r,i] K[i,c] Gamma[r,i,c] and Pc[i,c] = sum_r dP[r,i] Q[r,c] Gamma[r,i,c]:
      dq = Pr + e^G dQt,   dk = beta Z + Zc + Pc + e^G dKt + e^{G_C - G} dKhat,
      dbeta += sum_c K Z,
      dG = beta K Z - K Zc + Q Pr - K Pc + Kt dKt + Qt dQt - Khat dKhat  (elementwise),
      dG_C = sum_r Khat dKhat + gam dgam,
    and d log alpha[t, c] = sum_{r >= t} dG[r, c] + dG_C[c].  Returns (dq, dk, dv, dbeta or
    None, dlog_alpha [C,dk], dM0)."""
    C, dk_ = q.shape
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    incl = np.tril(np.ones((C, C), dtype=bool), 0)
    G = np.cumsum(la, axis=0)
    gC = G[-1]
    diff = G[:, None, :] - G[None, :, :]
    Gam = np.exp(np.where(incl[:, :, None], diff, 0.0)) * incl[:, :, None]
    eG, eT, gam = np.exp(G), np.exp(gC[None, :] - G), np.exp(gC)
    Kt, Qt, Kh = eG * k, eG * q, eT * k
    P = np.einsum("rc,ic,ric->ri", q, k, Gam)
    dbeta = None
    if write == "add":
        Delta = v
        dv = P.T @ dO + Kh @ dM
        dM0 = Qt.T @ dO + gam[:, None] * dM
        dKt = np.zeros_like(k)
        Z = Zc = np.zeros_like(k)
    else:
        SG = np.einsum("rc,ic,ric->ri", k, k, Gam) * strict
        T = forward_substitution_inverse(beta[:, None] * SG)
        VmK = v - Kt @ M0
        X = beta[:, None] * VmK
        Delta = T @ X
        dDelta = P.T @ dO + Kh @ dM
        Y = T.T @ dDelta
        dM0 = Qt.T @ dO + gam[:, None] * dM - Kt.T @ (beta[:, None] * Y)
        dv = beta[:, None] * Y
        dKt = -(beta[:, None] * Y) @ M0.T
        dA = np.where(strict, -(T.T @ (dDelta @ X.T) @ T.T), 0.0)
        Z = np.einsum("ri,ic,ric->rc", dA, k, Gam)
        Zc = np.einsum("ri,rc,ric->ic", beta[:, None] * dA, k, Gam)
        dbeta = np.sum(Y * VmK, axis=1) + np.sum(k * Z, axis=1)
    dP = np.where(incl, dO @ Delta.T, 0.0)
    dQt, dKh = dO @ M0.T, Delta @ dM.T
    dgam = np.sum(M0 * dM, axis=1)
    Pr = np.einsum("ri,ic,ric->rc", dP, k, Gam)
    Pc = np.einsum("ri,rc,ric->ic", dP, q, Gam)
    bz = 0.0 if beta is None or write == "add" else beta[:, None] * Z
    dq = Pr + eG * dQt
    dk = bz + Zc + Pc + eG * dKt + eT * dKh
    dG = bz * k - k * Zc + q * Pr - k * Pc + Kt * dKt + Qt * dQt - Kh * dKh
    dG[-1] += np.sum(Kh * dKh, axis=0) + gam * dgam
    dla = np.cumsum(dG[::-1], axis=0)[::-1]
    return dq, dk, dv, dbeta, dla, dM0


def chunked_bwd(q, k, v, beta, log_alpha, M0, dO, dMT, C=64, write="delta"):
    """Gradients over one sequence by chunks: q,k [T,dk], v [T,dv], beta [T] (None with
    write="add"), log_alpha None | [T] | [T,dk] (one decay per key channel), M0 [dk,dv],
    dO [T,dv], dMT None | [dk,dv].  The chunk states are recomputed forward, then the
    chunks are walked in reverse.  A partial last chunk is padded with zero rows (beta =
    0, log alpha = 0)."""
    Tn, dk_ = q.shape
    dv_ = v.shape[1]
    key = log_alpha is not None and np.ndim(log_alpha) == 2
    la = np.zeros(Tn) if log_alpha is None else log_alpha
    if beta is None:
        beta = np.zeros(Tn)
    nch = (Tn + C - 1) // C
    pad = nch * C - Tn
    padf = lambda x: np.concatenate([x, np.zeros((pad,) + x.shape[1:])]) if pad else x
    qp, kp, vp, bp, lp, dOp = (padf(x) for x in (q, k, v, beta, la, dO))
    states = [M0]
    for c in range(nch):
        sl = slice(c * C, (c + 1) * C)
        G = np.cumsum(lp[sl], axis=0)
        Gk = G if key else np.repeat(G[:, None], dk_, axis=1)
        if write == "add":  # M_C = diag(e^{G_C}) M0 + (e^{G_C - G} K)^T V
            states.append(np.exp(Gk[-1])[:, None] * states[-1] + (np.exp(Gk[-1][None, :] - Gk) * kp[sl]).T @ vp[sl])
        else:
            res = chunk_step(qp[sl], kp[sl], vp[sl], bp[sl], Gk, states[-1])
            states.append(res["M"])
    dM = np.zeros((dk_, dv_)) if dMT is None else dMT
    out = [np.zeros_like(x) for x in (qp, kp, vp, bp, lp)]
    for c in reversed(range(nch)):
        sl = slice(c * C, (c + 1) * C)
        step = chunk_step_bwd_key if key else chunk_step_bwd
        dq, dk, dv, db, dg, dM = step(qp[sl], kp[sl], vp[sl], bp[sl], lp[sl], states[c], dOp[sl], dM, write=write)
        for o_, x in zip(out, (dq, dk, dv, db, dg)):
            if x is not None:
                o_[sl] = x
    return tuple(x[:Tn] for x in out) + (dM,)


def chunk_step_dplr(q, k, v, a, b, g, M0):
    """One chunk of the diagonal-plus-low-rank transition with one decay per position
    (g [C] log decays; zeros without a gate) or one per position and key channel (g
    [C,dk]: every exponential below is then per channel, inside the contractions over
    the key channels).  With u_j = a_j^T M_{j-1} (the rows U), G the inclusive prefix of
    g and G_{-1} = 0:
      (I - A_ab) U = diag(e^{G_{j-1}}) A M0 + A_ak V,
      A_ab[j,i] = (a_j . b_i) e^{G_{j-1} - G_i},  A_ak[j,i] = (a_j . k_i) e^{G_{j-1} - G_i}  (i < j)
      O   = diag(e^G) Q M0 + P_qb U + P_qk V,
      P_qb[r,j] = (q_r . b_j) e^{G_r - G_j},  P_qk[r,j] = (q_r . k_j) e^{G_r - G_j}  (j <= r)
      M_C = e^{G_C} M0 + (diag(e^{G_C - G}) B)^T U + (diag(e^{G_C - G}) K)^T V.
    Returns (O, M_C)."""
    C = q.shape[0]
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    incl = np.tril(np.ones((C, C), dtype=bool), 0)
    if np.ndim(g) == 2:
        return _chunk_step_dplr_key(q, k, v, a, b, np.asarray(g, dtype=np.float64), M0, strict, incl)
    G = np.cumsum(g)
    Gp = np.concatenate([[0.0], G[:-1]])  # G_{j-1}
    E1 = np.where(strict, np.exp(np.where(strict, Gp[:, None] - G[None, :], 0.0)), 0.0)
    E2 = np.where(incl, np.exp(np.where(incl, G[:, None] - G[None, :], 0.0)), 0.0)
    Aab, Aak = (a @ b.T) * E1, (a @ k.T) * E1
    U = np.linalg.solve(np.eye(C) - Aab, np.exp(Gp)[:, None] * (a @ M0) + Aak @ v)
    O = np.exp(G)[:, None] * (q @ M0) + ((q @ b.T) * E2) @ U + ((q @ k.T) * E2) @ v
    w = np.exp(G[-1] - G)[:, None]
    MC = np.exp(G[-1]) * M0 + (w * b).T @ U + (w * k).T @ v
    return O, MC


def _chunk_step_dplr_key(q, k, v, a, b, g, M0, strict, incl):
    """chunk_step_dplr with one decay per key channel: G [C,dk] the per-channel prefix,
    Gp its shift (G_{j-1}, G_{-1} = 0), and with E1[j,i,c] = e^{Gp[j,c] - G[i,c]} (i < j)
    and E2[r,i,c] = e^{G[r,c] - G[i,c]} (i <= r):
      A_ab[j,i] = sum_c a_j[c] b_i[c] E1[j,i,c],  A_ak likewise with k,
      (I - A_ab) U = (A * e^{Gp}) M0 + A_ak V,
      O = (Q * e^G) M0 + P_qb U + P_qk V,  P_qb[r,i] = sum_c q_r[c] b_i[c] E2[r,i,c],
      M_C = diag(e^{G_C}) M0 + (B * e^{G_C - G})^T U + (K * e^{G_C - G})^T V."""
    G = np.cumsum(g, axis=0)
    Gp = np.concatenate([np.zeros((1, G.shape[1])), G[:-1]])
    E1 = np.exp(np.where(strict[:, :, None], Gp[:, None, :] - G[None, :, :], 0.0)) * strict[:, :, None]
    E2 = np.exp(np.where(incl[:, :, None], G[:, None, :] - G[None, :, :], 0.0)) * incl[:, :, None]
    Aab = np.einsum("jc,ic,jic->ji", a, b, E1)
    Aak = np.einsum("jc,ic,jic->ji", a, k, E1)
    U = np.linalg.solve(np.eye(q.shape[0]) - Aab, (a * np.exp(Gp)) @ M0 + Aak @ v)
    O = (q * np.exp(G)) @ M0 + np.einsum("rc,ic,ric->ri", q, b, E2) @ U + np.einsum("rc,ic,ric->ri", q, k, E2) @ v
    w = np.exp(G[-1][None, :] - G)
    MC = np.exp(G[-1])[:, None] * M0 + (w * b).T @ U + (w * k).T @ v
    return O, MC


def chunked_dplr(q, k, v, a, b, log_alpha, M0, C=64):
    """The chunked form over one sequence (q, k, a, b [T,dk], v [T,dv], log_alpha None
    | [T] | [T,dk]); a partial last chunk is padded with zero rows and log alpha = 0."""
    Tn, dk_ = q.shape
    la = np.zeros(Tn) if log_alpha is None else log_alpha
    O = np.zeros((Tn, v.shape[1]))
    M = M0
    for c0 in range(0, Tn, C):
        sl = slice(c0, min(c0 + C, Tn))
        Oc, M = chunk_step_dplr(q[sl], k[sl], v[sl], a[sl], b[sl], la[sl], M)
        O[sl] = Oc
    return O, M
