"""Float64 steps of the chunked SSD algorithm -- TEST INFRASTRUCTURE ONLY.

The chunked algorithm (Mamba-2 review, docsaid.org "Mamba-2", section
"2つのルートを半分ずつ"; SSD summary page, section "チャンク化アルゴリズム")
cuts the sequence into blocks of Q steps: inside a block it uses the matrix
(masked attention) form, across blocks it passes only the state at the end of
each block to the next one, and the two contributions are added.  Each
function below is one step of that algorithm, written from its definition in
the order the pages give it, with numpy matmul as the only library primitive.
They let the tests check each GPU kernel's intermediate on its own.

Conventions (shared with the GPU only through this documentation):
  chunk c covers steps s = c*Q .. e = min(s+Q, L) - 1 (the last may be short);
  nc = ceil(L / Q); i, j index steps inside a chunk; g = h // (H // G).

  cs[b,h,c,i]  = sum_{k=s..s+i} dt[b,k,h] * A[h]      (log of the decay product)
  G[b,c,g,i,j] = C[b,s+i,g,:] . B[b,s+j,g,:]           (used for j <= i)
  Yintra[s+i]  = sum_{j<=i} exp(cs_i - cs_j) G[i,j] x[s+j]
  S[b,c,h]     = sum_j exp(cs_e - cs_j) x[s+j] B[s+j]^T          ([P, N])
  hprev[c]     = state entering chunk c: hprev[0] = init (or 0),
                 hprev[c+1] = exp(cs_e(c)) hprev[c] + S[c]
  y[s+i]       = Yintra[s+i] + exp(cs_i) hprev[c] C[s+i] + D x[s+i]

The mask entries exp(cs_i - cs_j) are the products a_{j+1} ... a_i of the
per-step decays (review page, section "A を一つの数に簡略化する", definition
of L), and S / hprev are the low-rank blocks below the diagonal carried as
states (section "2つのルートを半分ずつ").  The inter-block formula printed
on the summary page omits the within-block weights exp(cs_e - cs_j); with
them the decomposition reproduces the recurrence exactly (pinned by the
chunk-size invariance test), without them it does not.
Padded positions of a short last chunk are NaN in cs and unused elsewhere.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _nchunks(L: int, Q: int) -> int:
    return (L + Q - 1) // Q


def _span(c: int, Q: int, L: int):
    s = c * Q
    return s, min(s + Q, L)


def chunk_cumsum(dt, A, Q: int):
    """cs [b, H, nc, Q]: inclusive prefix of dt*A inside each chunk."""
    dt, A = _f64(dt), _f64(A)
    b, L, H = dt.shape
    nc = _nchunks(L, Q)
    cs = np.full((b, H, nc, Q), np.nan)
    for c in range(nc):
        s, e = _span(c, Q, L)
        dA = dt[:, s:e, :] * A[None, None, :]            # [b, q, H]
        run = np.zeros((b, H))
        for i in range(e - s):
            run = run + dA[:, i, :]
            cs[:, :, c, i] = run
    return cs


def chunk_cb(C, B, Q: int):
    """G [b, nc, G, Q, Q]: G[i, j] = C_i . B_j inside each chunk (zero-padded)."""
    C, B = _f64(C), _f64(B)
    b, L, Gr, N = B.shape
    nc = _nchunks(L, Q)
    out = np.zeros((b, nc, Gr, Q, Q))
    for c in range(nc):
        s, e = _span(c, Q, L)
        for g in range(Gr):
            out[:, c, g, : e - s, : e - s] = C[:, s:e, g, :] @ np.swapaxes(B[:, s:e, g, :], 1, 2)
    return out


def chunk_scan_intra(Gm, cs, x, Q: int):
    """Yintra [b, L, H, P]: the masked quadratic form inside each chunk."""
    Gm, cs, x = _f64(Gm), _f64(cs), _f64(x)
    b, L, H, P = x.shape
    Gr = Gm.shape[2]
    nc = _nchunks(L, Q)
    y = np.zeros((b, L, H, P))
    for c in range(nc):
        s, e = _span(c, Q, L)
        q = e - s
        for h in range(H):
            g = h // (H // Gr)
            lc = cs[:, h, c, :q]                                   # [b, q]
            diff = lc[:, :, None] - lc[:, None, :]                 # cs_i - cs_j
            causal = np.tril(np.ones((q, q), dtype=bool))
            mask = np.where(causal[None], np.exp(np.where(causal[None], diff, 0.0)), 0.0)
            M = mask * Gm[:, c, g, :q, :q]                          # [b, i, j]
            y[:, s:e, h, :] = M @ x[:, s:e, h, :]
    return y


def chunk_state(x, B, cs, Q: int):
    """S [b, nc, H, P, N]: each chunk's own contribution to its end state."""
    x, B, cs = _f64(x), _f64(B), _f64(cs)
    b, L, H, P = x.shape
    Gr, N = B.shape[2], B.shape[3]
    nc = _nchunks(L, Q)
    S = np.zeros((b, nc, H, P, N))
    for c in range(nc):
        s, e = _span(c, Q, L)
        q = e - s
        for h in range(H):
            g = h // (H // Gr)
            lc = cs[:, h, c, :q]
            w = np.exp(lc[:, q - 1 : q] - lc)                      # exp(cs_e - cs_j), [b, q]
            xw = x[:, s:e, h, :] * w[:, :, None]                   # [b, q, P]
            S[:, c, h] = np.swapaxes(xw, 1, 2) @ B[:, s:e, g, :]   # [b, P, N]
    return S


def state_passing(S, cs, init=None, L: int | None = None, Q: int | None = None):
    """(hprev [b, nc, H, P, N], final [b, H, P, N]).

    hprev[c] is the state entering chunk c; the chunk decay is
    exp(cs at the chunk's last valid step).  ``L``/``Q`` locate that step for
    a short last chunk (default: the last non-NaN entry of cs).
    """
    S, cs, init = _f64(S), _f64(cs), _f64(init)
    b, nc, H, P, N = S.shape
    h = np.zeros((b, H, P, N)) if init is None else init.copy()
    hprev = np.zeros_like(S)
    for c in range(nc):
        if L is not None and Q is not None:
            last = min(Q, L - c * Q) - 1
            lam = np.exp(cs[:, :, c, last])
        else:
            row = cs[:, :, c, :]
            last = np.max(np.where(~np.isnan(row[0, 0]))[0])
            lam = np.exp(row[:, :, last])
        hprev[:, c] = h
        h = lam[:, :, None, None] * h + S[:, c]
    return hprev, h


def output_combine(yintra, C, cs, hprev, x, D, Q: int):
    """y = Yintra + exp(cs_i) hprev C_i + D x, chunk by chunk."""
    yintra, C, cs, hprev, x, D = (_f64(v) for v in (yintra, C, cs, hprev, x, D))
    b, L, H, P = x.shape
    Gr = C.shape[2]
    nc = _nchunks(L, Q)
    y = yintra.copy()
    for c in range(nc):
        s, e = _span(c, Q, L)
        q = e - s
        for h in range(H):
            g = h // (H // Gr)
            decay = np.exp(cs[:, h, c, :q])                                   # [b, q]
            off = C[:, s:e, g, :] @ np.swapaxes(hprev[:, c, h], 1, 2)         # [b, q, P]
            y[:, s:e, h, :] += decay[:, :, None] * off
            if D is not None:
                y[:, s:e, h, :] += D[h] * x[:, s:e, h, :]
    return y


def forward_chunked(x, dt, A, B, C, D=None, init=None, Q: int = 64):
    """All steps composed: (y, final, intermediates dict)."""
    x = _f64(x)
    b, L, H, P = x.shape
    cs = chunk_cumsum(dt, A, Q)
    Gm = chunk_cb(C, B, Q)
    yin = chunk_scan_intra(Gm, cs, x, Q)
    S = chunk_state(x, B, cs, Q)
    hprev, final = state_passing(S, cs, init, L=L, Q=Q)
    y = output_combine(yin, C, cs, hprev, x, D, Q)
    if L == 0:
        N = _f64(B).shape[3]
        final = np.zeros((b, H, P, N)) if init is None else _f64(init).copy()
    return y, final, {"cs": cs, "G": Gm, "yintra": yin, "S": S, "hprev": hprev}
