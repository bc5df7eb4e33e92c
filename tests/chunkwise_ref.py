"""Chunkwise re-association of the complex SSD scan, in numpy float64.

Test-only. It restates, step by step, the chunkwise algorithm that the
Mamba-3-Lite pages describe (index.html lab 03 "CHUNK" and "STATE" lines;
"Extending" guide Path B Step 2):

  a       = softplus(dt) * A                        per token
  A_cs[l] = inclusive running sum of a inside the chunk
  L[l,s]  = exp(A_cs[l] - A_cs[s]) for l >= s, else 0
  Y_diag  = ((C B^T) o L) X                          intra-chunk term
  state_c = sum_s B[s] (outer) X[s] * exp(A_cs[Q-1] - A_cs[s])
  H_{c+1} = exp(A_cs[Q-1]) H_c + state_c            inter-chunk passing
  Y_off   = exp(A_cs[l]) * C[l] H_c                  state-to-output term
  y       = Y_diag + Y_off

A last chunk shorter than Q is the same computation on fewer rows.

Its only use is to show, against the oracle, that this re-association
reproduces the plain recurrence for every chunk size (the algebra the GPU
kernels implement). It is never used as the reference for GPU parity.
"""

import numpy as np


def softplus(v):
    return np.logaddexp(0.0, v)


def chunkwise_scan(x, A, B_t, C_t, dt, chunk, initial_state=None):
    x = np.asarray(x, np.complex128)
    A = np.asarray(A, np.complex128)
    Bm = np.asarray(B_t, np.complex128)
    Cm = np.asarray(C_t, np.complex128)
    dt = np.asarray(dt, np.float64)
    Bsz, T, H, D = x.shape
    N = Bm.shape[-1]
    y = np.zeros((Bsz, T, H, D), np.complex128)
    final = np.zeros((Bsz, H, N, D), np.complex128)
    for b in range(Bsz):
        for h in range(H):
            Hst = np.zeros((N, D), np.complex128)
            if initial_state is not None:
                Hst = np.array(initial_state[b, h], np.complex128)
            for c0 in range(0, T, chunk):
                c1 = min(c0 + chunk, T)
                a = softplus(dt[b, c0:c1, h]) * A[h]
                Acs = np.cumsum(a)
                diff = Acs[:, None] - Acs[None, :]
                mask = np.tril(np.ones((c1 - c0, c1 - c0), bool))
                L = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
                Cc, Bc, Xc = Cm[b, c0:c1, h], Bm[b, c0:c1, h], x[b, c0:c1, h]
                y_diag = ((Cc @ Bc.T) * L) @ Xc
                y_off = np.exp(Acs)[:, None] * (Cc @ Hst)
                y[b, c0:c1, h] = y_diag + y_off
                decay_states = np.exp(Acs[-1] - Acs)
                state = (Bc * decay_states[:, None]).T @ Xc
                Hst = np.exp(Acs[-1]) * Hst + state
            final[b, h] = Hst
    return y, final


def chunkwise_scan_backward(x, A, B_t, C_t, dt, grad_y, chunk, grad_final=None,
                            initial_state=None):
    """Gradients of sum(grad_y * Re y) + sum(Re(conj(grad_final) * final_state)),
    re-associated by chunks (complex gradients as dl/dRe + i dl/dIm).

    Per chunk, with H the state entering it (forward pass), G the adjoint of
    the state leaving it written without conjugation (G = conj(adjoint)), the
    chunk-local running sums Lam, L = exp(Lam[l] - Lam[s]) on l >= s,
    e_end = exp(Lam[-1] - Lam) and e_in = exp(Lam):

      Gram      K[l,s]  = C[l] . B[s]                (no conjugation)
      M = K o L,   W[l,s] = gy[l] . x[s],   V = W o L
      conj(gx)  = M^T gy + diag(e_end) B G
      conj(gB)  = V^T C  + diag(e_end) x G^T
      conj(gC)  = V B    + diag(e_in) gy H^T
      dF/da_t   = sum_{j>=t} (O_j - I_j + Off_j) + sum_{s<t} In_s + T
          O_j = sum_s (K o V)[j,s],  I_j = sum_l (K o V)[l,j]
          Off_j = e_in[j] C[j] . (gy H^T)[j],  In_s = e_end[s] B[s] . (x G^T)[s]
          T = exp(Lam[-1]) sum(H o G)
      ga = conj(dF/da),  gdt = Re(conj(A) ga) sigmoid(dt),  gA = sum softplus(dt) ga
      G  <- exp(Lam[-1]) G + (diag(e_in) C)^T gy     (the next chunk to the left)

    The reading behind dF/da: y is linear in exp(Lam[l] - Lam[s]) for every
    pair (l >= s) of tokens, so the derivative of a running sum collects the
    pairs whose output side (O, Off) or input side (I, In) it sits on, and
    a token's step a_t moves every running sum from t on."""
    x = np.asarray(x, np.complex128)
    A = np.asarray(A, np.complex128)
    Bm = np.asarray(B_t, np.complex128)
    Cm = np.asarray(C_t, np.complex128)
    dt = np.asarray(dt, np.float64)
    gy = np.asarray(grad_y, np.float64)
    Bsz, T, H, D = x.shape
    N = Bm.shape[-1]
    gx = np.zeros_like(x)
    gB = np.zeros_like(Bm)
    gC = np.zeros_like(Cm)
    gdt = np.zeros_like(dt)
    gA = np.zeros(H, np.complex128)
    ginit = np.zeros((Bsz, H, N, D), np.complex128)
    starts = list(range(0, T, chunk))
    for b in range(Bsz):
        for h in range(H):
            Hst = np.zeros((N, D), np.complex128)
            if initial_state is not None:
                Hst = np.array(initial_state[b, h], np.complex128)
            entering = []
            for c0 in starts:
                c1 = min(c0 + chunk, T)
                entering.append(Hst)
                a = softplus(dt[b, c0:c1, h]) * A[h]
                Lam = np.cumsum(a)
                Bc, Xc = Bm[b, c0:c1, h], x[b, c0:c1, h]
                Hst = np.exp(Lam[-1]) * Hst + (Bc * np.exp(Lam[-1] - Lam)[:, None]).T @ Xc
            G = np.zeros((N, D), np.complex128)
            if grad_final is not None:
                G = np.conj(np.array(grad_final[b, h], np.complex128))
            for ci in reversed(range(len(starts))):
                c0 = starts[ci]
                c1 = min(c0 + chunk, T)
                Hc = entering[ci]
                sp = softplus(dt[b, c0:c1, h])
                Lam = np.cumsum(sp * A[h])
                q = c1 - c0
                mask = np.tril(np.ones((q, q), bool))
                L = np.where(mask, np.exp(np.where(mask, Lam[:, None] - Lam[None, :], 0.0)), 0.0)
                e_end = np.exp(Lam[-1] - Lam)
                e_in = np.exp(Lam)
                Bc, Cc, Xc, gyc = Bm[b, c0:c1, h], Cm[b, c0:c1, h], x[b, c0:c1, h], gy[b, c0:c1, h]
                K = Cc @ Bc.T
                M = K * L
                V = (gyc @ Xc.T) * L
                gx[b, c0:c1, h] = np.conj(M.T @ gyc + e_end[:, None] * (Bc @ G))
                R = Xc @ G.T
                gB[b, c0:c1, h] = np.conj(V.T @ Cc + e_end[:, None] * R)
                P = gyc @ Hc.T
                gC[b, c0:c1, h] = np.conj(V @ Bc + e_in[:, None] * P)
                Z = K * V
                O = Z.sum(axis=1)
                I = Z.sum(axis=0)
                Off = e_in * (Cc * P).sum(axis=1)
                In = e_end * (Bc * R).sum(axis=1)
                Tc = np.exp(Lam[-1]) * (Hc * G).sum()
                tail = np.cumsum((O - I + Off)[::-1])[::-1]
                head = np.concatenate([[0.0], np.cumsum(In)[:-1]])
                ga = np.conj(tail + head + Tc)
                gdt[b, c0:c1, h] = (np.conj(A[h]) * ga).real / (1.0 + np.exp(-dt[b, c0:c1, h]))
                gA[h] += (sp * ga).sum()
                G = np.exp(Lam[-1]) * G + (e_in[:, None] * Cc).T @ gyc
            ginit[b, h] = np.conj(G)
    return gx, gA, gB, gC, gdt, ginit
