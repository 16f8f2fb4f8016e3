"""Per-element error bounds for the bf16 kernels' outputs: the tolerance the
GPU parity tests hold each element of O, dQ, dK and dV to.

The bound is first order in the rounding the kernels perform (u = 2^-8, the
unit roundoff of bf16 with 8 significant bits under round to nearest even;
g = 2^-24 for fp32), summed in absolute value over every term, so it holds
whatever the signs of the individual rounding errors:

* O_i = sum_j P_ij v_j with P rounded to bf16 before the product and O
  rounded to bf16 at the end, fp32 accumulation over the row's keys:
      |dO_it| <= u |O_it| + (u + eps + n_i g) sum_j P_ij |v_jt|
* the backward forms D_i = sum_t dO_it O_it from that rounded O:
      |dD_i| <= eta_i = sum_t |dO_it| (u |O_it| + (u + eps) sum_j P_ij |v_jt|) + d g sum_t |dO_it O_it|
* dS_ij = P_ij (dP_ij - D_i) is formed in fp32 and rounded to bf16 before
  the dQ and dK products:
      |d(dS_ij)| <= P_ij eta_i + (u + eps) |dS_ij|
* dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i,
  dV_j = sum_i P_ij dO_i (P rounded to bf16), each rounded to bf16:
      |d(dQ_it)| <= scale sum_j |d(dS_ij)| |k_jt| + n_i g scale sum_j |dS_ij| |k_jt| + u |dQ_it|
      (dK alike over i with q), |d(dV_jt)| <= (u + eps + m_j g) sum_i P_ij |dO_it| + u |dV_jt|
  (n_i keys in row i, m_j rows reaching key j).

P itself is formed in fp32 as exp2(scale log2(e) s - lse log2(e)) before any
rounding to bf16: its relative error is at most eps = 2^-14 (the rounding of
the exponent's argument for arguments up to 2^9 in magnitude, the exp2
instruction's own error, and lse's), added to u wherever P's rounding
enters.

Every bound also carries an absolute 2^-100: weights below the smallest
normal fp32 number (2^-126) flush to zero on the GPU, so results that small
(which bf16 cannot hold either) come back as zeros.

P, dP, D and dS are formed here densely in fp64 from the oracle's lse and O
(so only for small n), as the quantities the bound is written in; the
expected values themselves always come from the oracle.  Where the softmax
is nearly one-hot the true gradients are tiny and the D term dominates:
there a relative bar is meaningless and this absolute one still holds.
"""
import numpy as np

from tests import brute

U = 2.0 ** -8
G = 2.0 ** -24
EPS_P = 2.0 ** -14
FLOOR = 2.0 ** -100


def error_bounds(pattern, l, c, q, k, v, do, scale, o_ref, lse_ref, backward=True):
    """Elementwise bounds (same shapes as O, dQ, dK, dV) for one head; all
    arguments fp64 [n, d] (lse [n]), o_ref and lse_ref from the oracle."""
    n, d = q.shape
    m = brute.mask(pattern, n, l, c)
    s = scale * (q @ k.T)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(m, np.exp(s - np.where(np.isfinite(lse_ref), lse_ref, 0.0)[:, None]), 0.0)
    n_i = m.sum(1)[:, None].astype(np.float64)
    m_j = m.sum(0)[:, None].astype(np.float64)
    pav = p @ np.abs(v)
    out = {"o": U * np.abs(o_ref) + (U + EPS_P + n_i * G) * pav + FLOOR}
    if not backward:
        return out
    eta = (np.abs(do) * (U * np.abs(o_ref) + (U + EPS_P) * pav)).sum(1) + d * G * np.abs(do * o_ref).sum(1)
    dp = do @ v.T
    dd = (do * o_ref).sum(1)
    ds = p * (dp - dd[:, None])
    dds = p * eta[:, None] + (U + EPS_P) * np.abs(ds)
    dq_ref = scale * (ds @ k)
    dk_ref = scale * (ds.T @ q)
    dv_ref = p.T @ do
    out["dq"] = scale * (dds @ np.abs(k)) + n_i * G * scale * (np.abs(ds) @ np.abs(k)) + U * np.abs(dq_ref) + FLOOR
    out["dk"] = scale * (dds.T @ np.abs(q)) + m_j * G * scale * (np.abs(ds).T @ np.abs(q)) + U * np.abs(dk_ref) + FLOOR
    out["dv"] = (U + EPS_P + m_j * G) * (p.T @ np.abs(do)) + U * np.abs(dv_ref) + FLOOR
    return out
