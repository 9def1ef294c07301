"""Chunked evaluation of the Mamba-2 SSD layer in float64 -- TEST INFRASTRUCTURE.

The sequence is cut into chunks of Q tokens.  Inside a chunk the layer is a
causal quadratic (attention-like) block; across chunks only the running state
is carried.  The steps below are the chunked algorithm of the Mamba-2 SSD
("state space duality") scan that the Zyphra/AMD post ("Training Transformers
and Hybrid models on AMD Instinct MI300X Accelerators", section "Mamba-2")
ports, written out from its definition in the recurrence:

  per chunk k, local index i in [0, Q), global t = kQ + i:
    cs_i     = sum_{j <= i} dt_j A                      (inclusive cumsum, per chunk)
    S_k      = sum_i exp(cs_{Q-1} - cs_i) dt_i x_i B_i^T  (chunk state, P x N)
    Hin_0    = 0,  Hin_{k+1} = exp(cs_{Q-1}) Hin_k + S_k   (state passing)
    W_ij     = C_i . B_j                                (per group)
    Lam_ij   = exp(cs_i - cs_j) for j <= i, else 0
    y_i      = sum_{j<=i} Lam_ij W_ij dt_j x_j + exp(cs_i) Hin_k C_i + D x_i

and the backward, the reverse-mode gradient of <dy, y> through those steps:

    dHloc_k  = sum_i exp(cs_i) dy_i C_i^T
    Gk       = dH_{k+1},  dH_K = dS_fin (final-state cotangent, default 0),
    dH_k     = dHloc_k + exp(cs_{Q-1}) dH_{k+1},   dS0 = dH_0
    dxt_j    = sum_{i>=j} Lam_ij W_ij dy_i + exp(cs_{Q-1} - cs_j) Gk B_j    (xt = dt x)
    dP_ij    = <dy_i, xt_j>,  R = dP o Lam o W
    dcs_i    = sum_j R_ij - sum_i' R_i'i + <dy_i, yoff_i> - q_i
    dcs_{Q-1} += sum_j q_j + exp(cs_{Q-1}) <Gk, Hin_k>,
               q_j = exp(cs_{Q-1} - cs_j) <xt_j, Gk B_j>
    dl_j     = sum_{i >= j} dcs_i   (reverse cumsum in the chunk)
    ddt_j    = A dl_j + <dxt_j, x_j>,   dA = sum dt_j dl_j
    dx_j     = dt_j dxt_j + D dy_j,     dD = sum <dy_j, x_j>
    dW_ij    = sum_{heads of group} dP_ij Lam_ij
    dC_i     = sum_j dW_ij B_j + sum_heads exp(cs_i) Hin_k^T dy_i
    dB_j     = sum_i dW_ij C_i + sum_heads exp(cs_{Q-1} - cs_j) Gk^T xt_j

States are kept as [P][N] (headdim x dstate).  numpy einsum serves as the
matrix product; nothing is blocked or fused beyond the chunking itself.

When Q does not divide the sequence length, the last chunk is shorter: it
holds the remaining L mod Q tokens, and the same steps apply with its own
length.  It is evaluated as a chunk of that length that starts from the state
the full chunks leave, and its initial-state gradient is the cotangent of the
state leaving the full chunks.
"""
from __future__ import annotations

import numpy as np


def _split(x, dt, B, C, Q):
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert L % Q == 0
    K = L // Q
    return (b, L, H, P, N, G, K,
            x.reshape(b, K, Q, H, P), dt.reshape(b, K, Q, H),
            B.reshape(b, K, Q, G, N), C.reshape(b, K, Q, G, N))


def _masked_decay(cs):
    """Lam[b,k,h,i,j] = exp(cs_i - cs_j) for j <= i else 0 (cs: [b,K,Q,H])."""
    csT = np.moveaxis(cs, 2, 3)                     # [b,K,H,Q]
    diff = csT[..., :, None] - csT[..., None, :]    # [b,K,H,i,j]
    Q = cs.shape[2]
    mask = np.tril(np.ones((Q, Q), dtype=bool))
    return np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)


def _group_sum(a, G):
    """Sum [..., H, N] over the heads of each group -> [..., G, N]."""
    sh = a.shape
    H = sh[-2]
    return a.reshape(sh[:-2] + (G, H // G, sh[-1])).sum(-2)


def ssd_chunked(x, dt, A, B, C, D, chunk, dy=None, initial_state=None, dfinal_state=None):
    """Forward (and, with dy, backward) of the chunked algorithm, started from
    initial_state (zero if None) with final-state cotangent dfinal_state
    (zero if None).

    Returns a dict holding the outputs and the gradients (dinitial_state
    among them).  When the chunk length divides the sequence length it also
    holds every intermediate (cs, S, Hin, W, dHloc, Gk, dcs, dl, dxt, dW,
    dC_off, dB_state); with a shorter last chunk it holds the dicts of the two
    parts under "full" and "tail" instead."""
    x, dt, A, B, C, D = (np.asarray(a, dtype=np.float64) for a in (x, dt, A, B, C, D))
    Q = int(chunk)
    L = x.shape[1]
    Lf = (L // Q) * Q
    if Lf in (0, L):
        return _chunked_aligned(x, dt, A, B, C, D, Q if Lf else L, dy, initial_state, dfinal_state)
    # Shorter last chunk of L - Lf tokens.  Its entry state is what the full
    # chunks leave; the full chunks' backward needs the tail's dS0 as their
    # final-state cotangent, so the full part runs forward first.
    dyf = None if dy is None else np.asarray(dy, dtype=np.float64)
    full_fwd = _chunked_aligned(x[:, :Lf], dt[:, :Lf], A, B[:, :Lf], C[:, :Lf], D, Q, None, initial_state, None)
    tail = _chunked_aligned(x[:, Lf:], dt[:, Lf:], A, B[:, Lf:], C[:, Lf:], D, L - Lf,
                            None if dyf is None else dyf[:, Lf:], full_fwd["final_state"], dfinal_state)
    out = dict(y=np.concatenate([full_fwd["y"], tail["y"]], axis=1), final_state=tail["final_state"],
               tail=tail)
    if dyf is None:
        out["full"] = full_fwd
        return out
    full = _chunked_aligned(x[:, :Lf], dt[:, :Lf], A, B[:, :Lf], C[:, :Lf], D, Q, dyf[:, :Lf], initial_state,
                            tail["dinitial_state"])
    out["full"] = full
    for k in ("dx", "ddt", "dB", "dC"):
        out[k] = np.concatenate([full[k], tail[k]], axis=1)
    out["dA"] = full["dA"] + tail["dA"]
    out["dD"] = full["dD"] + tail["dD"]
    out["dinitial_state"] = full["dinitial_state"]
    return out


def _chunked_aligned(x, dt, A, B, C, D, Q, dy, initial_state, dfinal_state):
    b, L, H, P, N, G, K, xc, dtc, Bc, Cc = _split(x, dt, B, C, Q)
    hg = np.arange(H) // (H // G)
    Bh, Ch = Bc[:, :, :, hg, :], Cc[:, :, :, hg, :]           # [b,K,Q,H,N]

    cs = np.cumsum(dtc * A, axis=2)                           # [b,K,Q,H]
    cs_last = cs[:, :, -1, :]                                 # [b,K,H]
    w = np.exp(cs_last[:, :, None, :] - cs) * dtc
    S = np.einsum("bkqh,bkqhp,bkqhn->bkhpn", w, xc, Bh)
    Hin = np.zeros((b, K + 1, H, P, N))
    if initial_state is not None:
        Hin[:, 0] = initial_state
    for k in range(K):
        Hin[:, k + 1] = np.exp(cs_last[:, k])[..., None, None] * Hin[:, k] + S[:, k]

    W = np.einsum("bkign,bkjgn->bkgij", Cc, Bc)               # [b,K,G,Q,Q]
    Wh = W[:, :, hg]                                          # [b,K,H,Q,Q]
    Lam = _masked_decay(cs)
    Pm = Lam * Wh
    xt = dtc[..., None] * xc                                  # [b,K,Q,H,P]
    y_intra = np.einsum("bkhij,bkjhp->bkihp", Pm, xt)
    ecs = np.exp(cs)
    y_off = np.einsum("bkih,bkihn,bkhpn->bkihp", ecs, Ch, Hin[:, :K])
    y = y_intra + y_off + D[None, None, None, :, None] * xc

    out = dict(y=y.reshape(b, L, H, P), final_state=Hin[:, K].copy(), cs=cs, S=S, Hin=Hin, W=W,
               y_off=y_off.reshape(b, L, H, P))
    if dy is None:
        return out

    dyc = np.asarray(dy, dtype=np.float64).reshape(b, K, Q, H, P)
    dHloc = np.einsum("bkih,bkihp,bkihn->bkhpn", ecs, dyc, Ch)
    dH = np.zeros((b, K + 1, H, P, N))
    if dfinal_state is not None:
        dH[:, K] = dfinal_state
    for k in reversed(range(K)):
        dH[:, k] = dHloc[:, k] + np.exp(cs_last[:, k])[..., None, None] * dH[:, k + 1]
    Gk = dH[:, 1:]                                            # Gk[:, k] = dH_{k+1}

    e = np.exp(cs_last[:, :, None, :] - cs)                   # [b,K,Q,H]
    GB = np.einsum("bkjhn,bkhpn->bkjhp", Bh, Gk)
    dxt = np.einsum("bkhij,bkihp->bkjhp", Pm, dyc) + e[..., None] * GB
    dP = np.einsum("bkihp,bkjhp->bkhij", dyc, xt)
    R = dP * Pm
    dcs = np.moveaxis(R.sum(-1), 2, 3) - np.moveaxis(R.sum(-2), 2, 3)
    dcs = dcs + np.einsum("bkihp,bkihp->bkih", dyc, y_off)
    q = e * np.einsum("bkjhp,bkjhp->bkjh", xt, GB)
    dcs = dcs - q
    dcs[:, :, -1, :] += q.sum(2) + np.exp(cs_last) * np.einsum("bkhpn,bkhpn->bkh", Gk, Hin[:, :K])
    dl = np.flip(np.cumsum(np.flip(dcs, 2), 2), 2)
    ddt = A * dl + np.einsum("bkjhp,bkjhp->bkjh", dxt, xc)
    dA = np.einsum("bkjh,bkjh->h", dtc, dl)
    dx = dtc[..., None] * dxt + D[None, None, None, :, None] * dyc
    dD = np.einsum("bkjhp,bkjhp->h", dyc, xc)

    dWh = dP * Lam                                            # [b,K,H,i,j]
    dW = dWh.reshape(b, K, G, H // G, Q, Q).sum(3)            # [b,K,G,Q,Q]
    dC_off = _group_sum(np.einsum("bkih,bkihp,bkhpn->bkihn", ecs, dyc, Hin[:, :K]), G)
    dB_state = _group_sum(np.einsum("bkjh,bkjhp,bkhpn->bkjhn", e, xt, Gk), G)
    dC = np.einsum("bkgij,bkjgn->bkign", dW, Bc) + dC_off
    dB = np.einsum("bkgij,bkign->bkjgn", dW, Cc) + dB_state

    out.update(dx=dx.reshape(b, L, H, P), ddt=ddt.reshape(b, L, H), dA=dA,
               dB=dB.reshape(b, L, G, N), dC=dC.reshape(b, L, G, N), dD=dD,
               dinitial_state=dH[:, 0].copy(), dHloc=dHloc, Gk=Gk, dcs=dcs, dl=dl, dxt=dxt.reshape(b, L, H, P), dW=dW,
               dC_off=dC_off.reshape(b, L, G, N), dB_state=dB_state.reshape(b, L, G, N))
    return out
