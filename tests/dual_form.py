"""The SSD in its dual (quadratic, attention-like) form, brute force in numpy.

Unrolling the recurrence of the reference page
(burn_dragon_kernel src/sequence/mamba2/backward.rs, ssd_forward_state_history_reference)
gives, per head with A = -exp(A_log) and the global inclusive cumulative sum
S_t = sum_{r<=t} dt_r A,

    h_t = exp(S_t) h0 + sum_{s<=t} exp(S_t - S_s) dt_s x_s (outer) B_s
    y_t = sum_{s<=t} exp(S_t - S_s) dt_s (C_t . B_s) x_s + exp(S_t) (h0 C_t) + D x_t

and differentiating that closed form directly (not the recurrence) gives
every gradient of L = sum(dy * y).  The decay enters only through
exp(S_i - S_j) and exp(S_i); d/da_t of S_i - S_j is 1 exactly when j < t <= i,
so the decay gradient is a rectangle sum

    da_t = sum_{i>=t} [ sum_{0<=j<t} M_ij + exp(S_i) dy_i.(h0 C_i) ],
    M_ij = exp(S_i - S_j) dt_j (dy_i . x_j)(C_i . B_j).

O(T^2) work per head: for tiny inputs only.  This is test code, independent of
both the oracle and the HIP path.
"""
import numpy as np


def _setup(x, dt, A_log, B, C):
    b, T, H, P = x.shape
    G = B.shape[2]
    hpg = H // G
    A = -np.exp(np.asarray(A_log, dtype=np.float64))
    S = np.cumsum(np.asarray(dt, np.float64) * A[None, None, :], axis=1)  # [b,T,H]
    return b, T, H, P, G, hpg, A, S


def states(x, dt, A_log, B, h0=None):
    """h_t for every t, [b,T,H,P,N], from the unrolled sum."""
    x, dt, B = (np.asarray(a, np.float64) for a in (x, dt, B))
    b, T, H, P, G, hpg, A, S = _setup(x, dt, A_log, B, B)
    N = B.shape[-1]
    hs = np.zeros((b, T, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            for t in range(T):
                acc = np.zeros((P, N))
                if h0 is not None:
                    acc += np.exp(S[bi, t, h]) * np.asarray(h0, np.float64)[bi, h]
                for s in range(t + 1):
                    acc += np.exp(S[bi, t, h] - S[bi, s, h]) * dt[bi, s, h] * np.outer(x[bi, s, h], B[bi, s, g])
                hs[bi, t, h] = acc
    return hs


def forward(x, dt, A_log, B, C, D, h0=None):
    x, dt, B, C = (np.asarray(a, np.float64) for a in (x, dt, B, C))
    b, T, H, P, G, hpg, A, S = _setup(x, dt, A_log, B, C)
    y = np.zeros_like(x)
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            for t in range(T):
                acc = D[h] * x[bi, t, h]
                for s in range(t + 1):
                    acc = acc + np.exp(S[bi, t, h] - S[bi, s, h]) * dt[bi, s, h] * (C[bi, t, g] @ B[bi, s, g]) * x[bi, s, h]
                if h0 is not None:
                    acc = acc + np.exp(S[bi, t, h]) * (np.asarray(h0, np.float64)[bi, h] @ C[bi, t, g])
                y[bi, t, h] = acc
    return y


def backward(x, dt, A_log, B, C, D, dy, h0=None):
    x, dt, B, C, dy = (np.asarray(a, np.float64) for a in (x, dt, B, C, dy))
    b, T, H, P, G, hpg, A, S = _setup(x, dt, A_log, B, C)
    N = B.shape[-1]
    dx = D[None, None, :, None] * dy
    ddt = np.zeros_like(dt)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    dh0 = np.zeros((b, H, P, N))
    dA = np.zeros(H)
    dD = np.einsum("bthp,bthp->h", dy, x)
    h0d = None if h0 is None else np.asarray(h0, np.float64)
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            Sh = S[bi, :, h]
            for j in range(T):
                for i in range(j, T):
                    L = np.exp(Sh[i] - Sh[j])
                    cb = C[bi, i, g] @ B[bi, j, g]
                    yx = dy[bi, i, h] @ x[bi, j, h]
                    dx[bi, j, h] += L * dt[bi, j, h] * cb * dy[bi, i, h]
                    dB[bi, j, g] += L * dt[bi, j, h] * yx * C[bi, i, g]
                    dC[bi, i, g] += L * dt[bi, j, h] * yx * B[bi, j, g]
                    ddt[bi, j, h] += L * cb * yx
            for i in range(T):
                dh0[bi, h] += np.exp(Sh[i]) * np.outer(dy[bi, i, h], C[bi, i, g])
                if h0d is not None:
                    dC[bi, i, g] += np.exp(Sh[i]) * (dy[bi, i, h] @ h0d[bi, h])
            # rectangle sums for the decay gradient
            da = np.zeros(T)
            for t in range(T):
                tot = 0.0
                for i in range(t, T):
                    for j in range(t):
                        tot += np.exp(Sh[i] - Sh[j]) * dt[bi, j, h] * (dy[bi, i, h] @ x[bi, j, h]) * (C[bi, i, g] @ B[bi, j, g])
                    if h0d is not None:
                        tot += np.exp(Sh[i]) * (dy[bi, i, h] @ (h0d[bi, h] @ C[bi, i, g]))
                da[t] = tot
            ddt[bi, :, h] += A[h] * da
            dA[h] += np.sum(dt[bi, :, h] * da)
    return dict(dx=dx, ddt=ddt, dA_log=A * dA, dB=dB, dC=dC, dD=dD, dh0=dh0)
