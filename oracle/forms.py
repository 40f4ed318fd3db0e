"""Independent float64 numpy formulations of the SSD scan -- TEST INFRASTRUCTURE.

These do not call the sequential oracle; they are other ways of writing the
same result, used to pin it.

* ``ssd_dual``: the quadratic ("dual", attention-like) form Y = M X with a
  causal semiseparable M, page "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모
  클러스터 학습", §3 and §3.1:
      M[t, s] = (C_t · B_s) · exp(Σ_{k=s+1..t} Δ_k A) · Δ_s     for s <= t, 0 otherwise
      y_t     = Σ_s M[t, s] x_s + exp(Σ_{k=0..t} Δ_k A) · C_tᵀ h0 + D x_t
* ``ssd_chunked``: the block decomposition of §3.2 with chunks of length Q:
  diagonal blocks as masked quadratic products inside each chunk, off-diagonal
  blocks through an N x P state handed from chunk to chunk.  Stage by stage:
      cs_i    = Σ_{k<=i} Δ_k A                 (within-chunk inclusive cumsum)
      S_c     = Σ_i B_i exp(cs_end - cs_i) Δ_i x_iᵀ          (chunk state)
      H_c     = exp(cs_end) H_{c-1} + S_c,  H_{-1} = h0      (state passing)
      Y_diag  = (C Bᵀ ∘ exp(cs_i - cs_j) ∘ Δ_j, j <= i) X_c  (intra-chunk)
      Y_off_i = exp(cs_i) C_iᵀ H_{c-1}                       (state -> output)
      y       = Y_diag + Y_off + D x
  The last chunk may be shorter than Q.
* ``selective_scan_dual``: the Mamba-1 diagonal-A scan of §2.1 written as a
  sum over source tokens, y_t = Σ_{s<=t} Σ_n C_t[n] B_s[n] exp(A[n] Σ_{k=s+1..t} Δ_k) Δ_s u_s.

* ``ssd_packed_reset``: the packing of §4.3 written literally: one sequential
  recurrence over the packed tokens whose state transition is set to zero at
  the first token of every sequence (there the previous state is replaced by
  that sequence's initial state, zero by default).

* ``ssd_chunked_bwd``: the gradient of ``ssd_chunked`` in the same block
  form, derived by hand from the chunk equations above (not from the
  sequential adjoint).  With G_out the gradient w.r.t. the state leaving a
  chunk (dL/dh_final for the last), K = X dYᵀ (K[s,u] = x_s·dy_u) and the
  anti-causal decay E[s,u] = exp(cs_u - cs_s) for u >= s:
      dxr_s = Σ_u (C_u·B_s) E[s,u] dy_u + exp(cs_end - cs_s) B_sᵀ G_out
      dx    = Δ·dxr + D dy
      dB_s  = Δ_s Σ_u K[s,u] E[s,u] C_u + Δ_s exp(cs_end - cs_s) G_out x_s
      dC_u  = Σ_s K[s,u] E[s,u] Δ_s B_s + exp(cs_u) h_in dy_u
      G_in  = exp(cs_end) G_out + Σ_u exp(cs_u) C_u dy_uᵀ   (= G_out of the chunk before)
  and for the decays, with cs taken as free variables inside the chunk,
  Z[u,s] = M[u,s] K[s,u] (M the forward's intra-chunk matrix) and
  q_s = Δ_s exp(cs_end - cs_s) x_s·(B_sᵀ G_out):
      dcs_u += Σ_s Z[u,s] + exp(cs_u) dy_u·(h_inᵀ C_u);   dcs_s -= Σ_u Z[u,s] + q_s
      dcs_end += exp(cs_end) <G_out, h_in> + Σ_s q_s
      dℓ_t   = Σ_{v >= t in the chunk} dcs_v   (cs_v = Σ_{k<=v} ℓ_k, ℓ = Δ·A)
      dΔ     = A·dℓ + x·dxr;  dA = Σ Δ·dℓ;  dD = Σ x·dy;  dh0 = G_in of chunk 0

Only for small inputs (the dual forms build L x L matrices).
"""
from __future__ import annotations

import numpy as np


def softplus(r):
    r = np.asarray(r, dtype=np.float64)
    return np.where(r > 0, r + np.log1p(np.exp(-np.abs(r))), np.log1p(np.exp(np.minimum(r, 0))))


def _causal_decay(cum):
    """exp(cum[t] - cum[s]) for s <= t, else 0 (exponent masked before exp)."""
    diff = cum[:, None] - cum[None, :]
    mask = np.tril(np.ones_like(diff, dtype=bool))
    return np.exp(np.where(mask, diff, -np.inf))


def ssd_dual(x, dt, A, B, C, D=None, h0=None, dt_softplus=True):
    """Returns (y, final_state) of the quadratic form."""
    x = np.asarray(x, np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    R = H // G
    delta = softplus(dt) if dt_softplus else np.asarray(dt, np.float64)
    y = np.zeros_like(x)
    hf = np.zeros((b, H, N, P))
    for bb in range(b):
        for h in range(H):
            g = h // R
            d = delta[bb, :, h]
            cum = np.cumsum(d * A[h])
            Bm = np.asarray(B[bb, :, g], np.float64)
            Cm = np.asarray(C[bb, :, g], np.float64)
            X = x[bb, :, h]
            M = (Cm @ Bm.T) * _causal_decay(cum) * d[None, :]
            yy = M @ X
            fin = (Bm * (np.exp(cum[-1] - cum) * d)[:, None]).T @ X
            if h0 is not None:
                s0 = np.asarray(h0[bb, h], np.float64)
                yy += np.exp(cum)[:, None] * (Cm @ s0)
                fin += np.exp(cum[-1]) * s0
            if D is not None:
                yy += D[h] * X
            y[bb, :, h] = yy
            hf[bb, h] = fin
    return y, hf


def ssd_chunked(x, dt, A, B, C, D=None, h0=None, chunk=64, dt_softplus=True,
                return_stages=False):
    """Block decomposition.  Returns (y, final_state) and, on request, a dict of
    the per-chunk stages: delta, cs [b,H,K,Q] (padded with nan past the end),
    S (chunk states) and Hprev (state entering each chunk), [b,K,H,N,P]."""
    x = np.asarray(x, np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    R = H // G
    Q = chunk
    K = (L + Q - 1) // Q
    delta = softplus(dt) if dt_softplus else np.asarray(dt, np.float64)
    y = np.zeros_like(x)
    hf = np.zeros((b, H, N, P))
    st = None
    if return_stages:
        st = dict(delta=np.full((b, H, K, Q), np.nan), cs=np.full((b, H, K, Q), np.nan),
                  S=np.zeros((b, K, H, N, P)), Hprev=np.zeros((b, K, H, N, P)))
    for bb in range(b):
        for h in range(H):
            g = h // R
            state = np.zeros((N, P)) if h0 is None else np.array(h0[bb, h], np.float64)
            for c in range(K):
                s0, s1 = c * Q, min(L, c * Q + Q)
                d = delta[bb, s0:s1, h]
                cs = np.cumsum(d * A[h])
                X = x[bb, s0:s1, h]
                Bc = np.asarray(B[bb, s0:s1, g], np.float64)
                Cc = np.asarray(C[bb, s0:s1, g], np.float64)
                # diagonal block: masked quadratic form inside the chunk
                y_diag = ((Cc @ Bc.T) * _causal_decay(cs) * d[None, :]) @ X
                # off-diagonal blocks: state entering the chunk, read out by C
                y_off = np.exp(cs)[:, None] * (Cc @ state)
                y[bb, s0:s1, h] = y_diag + y_off + (D[h] * X if D is not None else 0.0)
                # chunk state and hand-off to the next chunk
                S_c = Bc.T @ ((np.exp(cs[-1] - cs) * d)[:, None] * X)
                if st is not None:
                    st["delta"][bb, h, c, :s1 - s0] = d
                    st["cs"][bb, h, c, :s1 - s0] = cs
                    st["S"][bb, c, h] = S_c
                    st["Hprev"][bb, c, h] = state
                state = np.exp(cs[-1]) * state + S_c
            hf[bb, h] = state
    if return_stages:
        return y, hf, st
    return y, hf


def selective_scan_dual(u, delta, A, B, C, D=None, z=None, delta_softplus=True):
    """Mamba-1 output as a causal sum over source tokens; returns (out, final_state)."""
    u = np.asarray(u, np.float64)
    b, L, dim = u.shape
    N = A.shape[1]
    dl = softplus(delta) if delta_softplus else np.asarray(delta, np.float64)
    out = np.zeros_like(u)
    hf = np.zeros((b, dim, N))
    for bb in range(b):
        Bm = np.asarray(B[bb], np.float64)
        Cm = np.asarray(C[bb], np.float64)
        for d in range(dim):
            w = dl[bb, :, d] * u[bb, :, d]
            yy = np.zeros(L)
            for n in range(N):
                cum = np.cumsum(dl[bb, :, d] * A[d, n])
                Kn = Cm[:, n][:, None] * Bm[:, n][None, :] * _causal_decay(cum)
                yy += Kn @ w
                hf[bb, d, n] = np.sum(np.exp(cum[-1] - cum) * Bm[:, n] * w)
            if D is not None:
                yy += D[d] * u[bb, :, d]
            if z is not None:
                zz = np.asarray(z[bb, :, d], np.float64)
                yy *= zz / (1.0 + np.exp(-zz))
            out[bb, :, d] = yy
    return out, hf


def ssd_packed_reset(x, dt, A, B, C, cu_seqlens, D=None, h0s=None, dt_softplus=True):
    """Returns (y [T,H,P], final states [nseq,H,N,P]) of the packed recurrence."""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    A = np.asarray(A, np.float64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    cu = [int(v) for v in cu_seqlens]
    nseq = len(cu) - 1
    start = {}
    for s_ in range(nseq):
        if cu[s_ + 1] > cu[s_]:
            start[cu[s_]] = s_
    delta = softplus(dt) if dt_softplus else dt
    y = np.zeros((T, H, P))
    hf = np.zeros((nseq, H, N, P)) if h0s is None else np.array(h0s, np.float64)
    for h in range(H):
        g = h // (H // G)
        state = np.zeros((N, P))
        for t in range(T):
            a_t = np.exp(delta[t, h] * A[h])
            if t in start:  # transition zeroed: the sequence starts from its own state
                s_ = start[t]
                state = np.zeros((N, P)) if h0s is None else np.array(h0s[s_][h], np.float64)
            state = a_t * state + delta[t, h] * np.outer(B[t, g], x[t, h])
            y[t, h] = C[t, g] @ state + (0.0 if D is None else D[h] * x[t, h])
            if t + 1 in cu[1:] or t == T - 1:
                for s_ in range(nseq):
                    if cu[s_ + 1] == t + 1 and cu[s_ + 1] > cu[s_]:
                        hf[s_, h] = state
    return y, hf


def ssd_chunked_bwd(x, dt, A, B, C, dy, D=None, h0=None, dhfinal=None, chunk=64, dt_softplus=True):
    """Gradient of the chunked SSD scan (see the module notes), chunk by chunk:
    states entering each chunk forward, then the adjoint backwards.  Returns the
    dict of ``oracle.ssd_scan_bwd``."""
    x, dt, B, C, dy = (np.asarray(v, np.float64) for v in (x, dt, B, C, dy))
    A = np.asarray(A, np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    R = H // G
    out = dict(dx=np.zeros_like(x), ddt=np.zeros_like(dt), dA=np.zeros(H), dB=np.zeros_like(B),
               dC=np.zeros_like(C), dD=np.zeros(H), dh0=np.zeros((b, H, N, P)))
    starts = list(range(0, L, chunk))
    for bi in range(b):
        for h in range(H):
            g = h // R
            raw = dt[bi, :, h]
            delta = softplus(raw) if dt_softplus else raw.copy()
            ell = delta * A[h]
            # forward: the state entering every chunk
            hin = []
            Hs = np.zeros((N, P)) if h0 is None else np.asarray(h0, np.float64)[bi, h].copy()
            for t0 in starts:
                sl = slice(t0, min(t0 + chunk, L))
                cs = np.cumsum(ell[sl])
                hin.append(Hs.copy())
                w = np.exp(cs[-1] - cs) * delta[sl]
                Hs = np.exp(cs[-1]) * Hs + B[bi, sl, g].T @ (w[:, None] * x[bi, sl, h])
            # backward over chunks
            Gout = np.zeros((N, P)) if dhfinal is None else np.asarray(dhfinal, np.float64)[bi, h].copy()
            for c in range(len(starts) - 1, -1, -1):
                t0 = starts[c]
                sl = slice(t0, min(t0 + chunk, L))
                Xc, dYc, Bc, Cc, dl = x[bi, sl, h], dy[bi, sl, h], B[bi, sl, g], C[bi, sl, g], delta[sl]
                cs = np.cumsum(ell[sl])
                Hin = hin[c]
                Ecaus = np.exp(cs[:, None] - cs[None, :])           # [u, s] = exp(cs_u - cs_s)
                mask = np.tril(np.ones((len(cs), len(cs)), bool))     # s <= u
                Ecaus = np.where(mask, Ecaus, 0.0)
                Gm = Cc @ Bc.T                                        # [u, s] = C_u·B_s
                M = Gm * Ecaus * dl[None, :]                          # forward intra-chunk matrix
                K = Xc @ dYc.T                                        # [s, u] = x_s·dy_u
                einter = np.exp(cs[-1] - cs)                          # exp(cs_end - cs_s)
                dxr_inter = einter[:, None] * (Bc @ Gout)
                dxr = (Gm * Ecaus).T @ dYc + dxr_inter
                out["dx"][bi, sl, h] = dl[:, None] * dxr + (0.0 if D is None else D[h]) * dYc
                dBc = (dl[:, None] * (K * Ecaus.T)) @ Cc + (dl * einter)[:, None] * (Xc @ Gout.T)
                dC_off = np.exp(cs)[:, None] * (dYc @ Hin.T)
                dCc = (K.T * Ecaus * dl[None, :]) @ Bc + dC_off
                out["dB"][bi, sl, g] += dBc
                out["dC"][bi, sl, g] += dCc
                # decays
                Z = M * K.T                                           # [u, s]
                q = dl * einter * np.sum(Xc * (Bc @ Gout), axis=1)
                dcs = Z.sum(axis=1) - Z.sum(axis=0) + np.sum(Cc * dC_off, axis=1) - q
                dcs[-1] += np.exp(cs[-1]) * np.sum(Gout * Hin) + q.sum()
                dell = np.cumsum(dcs[::-1])[::-1]
                ddelta = A[h] * dell + np.sum(Xc * dxr, axis=1)
                out["ddt"][bi, sl, h] = ddelta / (1.0 + np.exp(-raw[sl])) if dt_softplus else ddelta
                out["dA"][h] += np.sum(dl * dell)
                out["dD"][h] += np.sum(Xc * dYc)
                Gout = np.exp(cs[-1]) * Gout + Cc.T @ (np.exp(cs)[:, None] * dYc)
            out["dh0"][bi, h] = Gout
    return out
