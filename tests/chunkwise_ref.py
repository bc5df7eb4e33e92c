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
