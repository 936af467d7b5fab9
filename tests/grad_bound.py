"""Per-element error bound for the attention backward's gradients (test tolerance).

Test infrastructure: the GPU parity tests gate every gradient element with this
bound; nothing in the library imports it.

The gradients are those of L = sum_i dO_i . O_i (the derivation that the llm.c
page's attention_backward and the flash-attention page's backward kernel
implement):
    P = softmax(scale * Q K^T) over the allowed keys,   O = P V
    dV = P^T dO,   dP = dO V^T,   D_i = dO_i . O_i,   dS = P * (dP - D)
    dQ = scale * dS K,   dK = scale * dS^T Q
The kernels take 16-bit inputs (unit roundoff u: 2^-8 bf16, 2^-11 fp16),
compute in fp32 (2^-24) and round to nearest even at these steps (a rounding to the
16-bit type moves x by at most u |x| + tau, tau being half the subnormal spacing:
2^-25 fp16, 2^-134 bf16):
  * P is rebuilt in fp32 from the forward's fp32 LSE, exp2(scale*log2e*s - log2e*LSE),
    then rounded to the input dtype before dV = P^T dO;
  * D comes from the forward's output O, which is itself rounded (its P rounded
    before P V, and the result rounded to the input dtype);
  * dS = P (dP - D) is formed in fp32 and rounded to the input dtype before
    dQ = dS K and dK = dS^T Q;
  * the fp32 sums are rounded to the input dtype on output.
Rounding errors of distinct operations are taken as independent and mean-zero, as in
the probabilistic rounding-error analysis of Higham and Mary ("A new approach to
probabilistic rounding error analysis", SIAM J. Sci. Comput. 41(5), 2019): a sum
sum_t delta_t x_t of roundings |delta_t| <= u then exceeds LAM u ||x||_2 with
probability at most 2 exp(-LAM^2 / 2) (Hoeffding), and an n-term fp32 sum is off by
at most LAM sqrt(n) 2^-24 sum |x| with a like probability. With LAM = 8 that is
below 1e-13 per element. Errors shared by many terms (the rebuilt P's relative
error eta, which carries the forward's LSE error, and the error of D_i, shared by
the whole row) are bounded in the worst case instead. For row i, key j, column c:
  eta_ij  relative error of the rebuilt P_ij: the fp32 score (d 2^-24 sum_c |q_ic k_jc|),
          the fp32 argument of exp2 and exp2 itself, the forward's LSE (its Nk-term
          sum, and the score errors it weights);
  E_i     error of D_i: the forward's output rounding (LAM ||dO_i (u |O_i| + tau)||),
          the forward's rounded P, whose effect on D_i is sum_j r_j (dP_ij - D_i) for
          roundings |r_j| <= u P_ij + tau (LAM ||(u P_i + tau)(dP_i - D_i)||), eta
          (sum_j eta_ij |dS_ij|), fp32 sums;
  W_ij    the rest of dS_ij's error apart from its own rounding and D:
          eta_ij |dS_ij| + P_ij LAM sqrt(d) 2^-24 sum_c |dO_ic v_jc| (dP in fp32);
  |dV_jc err| <= u |dV_jc| + tau + LAM ||(u P_:j + tau) dO_:c|| + sum_i P_ij eta_ij |dO_ic|
                 + LAM sqrt(n) 2^-24 sum_i P_ij |dO_ic|
  |dK_jc err| <= u |dK_jc| + tau + scale (LAM ||(u |dS_:j| + tau) Q_:c|| + sum_i (W_ij + E_i P_ij) |Q_ic|
                 + LAM sqrt(n) 2^-24 sum_i |dS_ij Q_ic|)
  |dQ_ic err| <= u |dQ_ic| + tau + scale (LAM ||(u |dS_i:| + tau) K_:c|| + sum_j W_ij |K_jc|
                 + E_i |sum_j P_ij K_jc| + LAM sqrt(Nk) 2^-24 sum_j |dS_ij K_jc|)
(n = group * Nq for dK and dV, whose sums run over the kv-head's query heads; the
output rounding u |g| + tau is taken in the worst case; tau counts on every allowed
pair, masked ones being exact zeros). The whole is multiplied by
1 + 16 u for the second-order terms. Masked pairs have P = dS = 0 and contribute
nothing; a row with no allowed key has a zero gradient and a zero bound.
"""
import numpy as np
import torch

U = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
TAU = {"bf16": 2.0 ** -134, "fp16": 2.0 ** -25}
EPS32 = 2.0 ** -24
LAM = 8.0



def _f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def allowed(Nq, Nk, causal):
    """Key j is allowed for row i iff j <= i + (Nk - Nq) (bottom-right causal)."""
    if not causal:
        return np.ones((Nq, Nk), dtype=bool)
    return np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)


def head_terms(Q, K, V, dO, scale, mask):
    """Exact fp64 P, LSE, O, dS and the gradients' per-head pieces for one query head."""
    s = Q @ K.T
    x = np.where(mask, scale * s, -np.inf)
    rows_ok = mask.any(axis=1)
    m = np.where(rows_ok, x.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(mask, np.exp(x - m[:, None]), 0.0)
    l = e.sum(axis=1)
    P = np.where(rows_ok[:, None], e / np.where(rows_ok, l, 1.0)[:, None], 0.0)
    lse = np.where(rows_ok, m + np.log(np.where(rows_ok, l, 1.0)), 0.0)
    O = P @ V
    dP = dO @ V.T
    D = (dO * O).sum(axis=1)
    dS = P * (dP - D[:, None])
    return s, P, lse, O, dS


def grad_bound(q, k, v, do, dtype, scale, causal):
    """(bound_dq, bound_dk, bound_dv), fp64 arrays shaped like q, k, v: the largest
    error the kernels' rounding allows in each gradient element. q/do [B,Hq,Nq,d],
    k/v [B,Hkv,Nk,d] (any real dtype; the 16-bit values are what count)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    scale = float(np.float32(scale))  # the boundary takes the scale as fp32
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    u, tau = U[dtype], TAU[dtype]
    gd = d * EPS32                    # one fp32 dot product over d, worst case
    n_kv = group * Nq                 # dK / dV sums run over the group's rows
    r32 = LAM * EPS32                 # fp32 sums, probabilistic (times sqrt(n))
    mask = allowed(Nq, Nk, causal)
    tau_q = np.where(mask.any(axis=1), tau, 0.0)[:, None]   # rows / keys with no allowed
    tau_k = np.where(mask.any(axis=0), tau, 0.0)[:, None]   # pair are exact zeros
    bq = np.zeros(q.shape)
    bk = np.zeros(k.shape)
    bv = np.zeros(k.shape)
    sk2 = np.zeros(k.shape)           # sum_i (dS_ij Q_ic)^2 over the group's rows
    sv2 = np.zeros(k.shape)           # sum_i (P_ij dO_ic)^2
    gk = np.zeros(k.shape)
    gv = np.zeros(k.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            Q, K, V, dO = q[b, h], k[b, g], v[b, g], do[b, h]
            s, P, lse, O, dS = head_terms(Q, K, V, dO, scale, mask)
            aQ, aK, adO = np.abs(Q), np.abs(K), np.abs(dO)
            aS = np.abs(dS)
            QK = aQ @ aK.T                       # sum_c |q_ic k_jc|
            M = adO @ np.abs(V).T                # sum_c |dO_ic v_jc|
            A = (adO * np.abs(O)).sum(axis=1)    # sum_c |dO_ic O_ic|
            lam = (P * (gd * scale * QK)).sum(axis=1)   # forward LSE: score errors
            sx = np.where(mask, np.abs(scale * s), 0.0)
            eta = np.where(mask, gd * scale * QK
                           + EPS32 * (4.0 * (sx + np.abs(lse)[:, None]) + Nk + 8)
                           + lam[:, None], 0.0)
            tm = np.where(mask, tau, 0.0)       # subnormal floor of a rounded P or dS
            rS = u * aS + tm                     # rounding of dS_ij
            rP = u * P + tm                      # rounding of P_ij
            dPD = np.abs(dO @ V.T - (dO * O).sum(axis=1)[:, None])
            E = LAM * (np.sqrt(((adO * (u * np.abs(O) + tau)) ** 2).sum(axis=1))
                       + np.sqrt(((rP * dPD) ** 2).sum(axis=1))) \
                + (eta * aS).sum(axis=1) \
                + r32 * (np.sqrt(Nk) * ((P * M).sum(axis=1) + A) + np.sqrt(d) * A)
            W = eta * aS + P * (r32 * np.sqrt(d) * M)
            dq = scale * (dS @ K)
            bq[b, h] = u * np.abs(dq) + tau_q + scale * (LAM * np.sqrt((rS ** 2) @ (K ** 2))
                                                 + W @ aK + E[:, None] * np.abs(P @ K)
                                                 + r32 * np.sqrt(Nk) * (aS @ aK))
            bk[b, g] += scale * ((W + E[:, None] * P).T @ aQ
                                 + r32 * np.sqrt(n_kv) * (aS.T @ aQ))
            sk2[b, g] += (rS ** 2).T @ (Q ** 2)
            bv[b, g] += (P * eta).T @ adO + r32 * np.sqrt(n_kv) * (P.T @ adO)
            sv2[b, g] += (rP ** 2).T @ (dO ** 2)
            gk[b, g] += scale * (dS.T @ Q)
            gv[b, g] += P.T @ dO
    bk += u * np.abs(gk) + tau_k + scale * LAM * np.sqrt(sk2)
    bv += u * np.abs(gv) + tau_k + LAM * np.sqrt(sv2)
    f = 1.0 + 16.0 * u
    return f * bq, f * bk, f * bv


def grads(q, k, v, do, scale, causal):
    """The exact gradients in matrix form, fp64 (used only to pin the bound)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    scale = float(np.float32(scale))  # the boundary takes the scale as fp32
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    mask = allowed(Nq, Nk, causal)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(k.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            _, P, _, _, dS = head_terms(q[b, h], k[b, g], v[b, g], do[b, h], scale, mask)
            dq[b, h] = scale * (dS @ k[b, g])
            dk[b, g] += scale * (dS.T @ q[b, h])
            dv[b, g] += P.T @ do[b, h]
    return dq, dk, dv

