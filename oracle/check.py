"""Parity checker: compares a quantized layer against the float64 oracle.

TEST INFRASTRUCTURE ONLY (tests/, smoke check, benchmark CPU baseline).

Rules (tolerances are the ones the quantizer is specified with):
  * H: element-wise |dH_ij| <= 1e-4 * sqrt(H_ii H_jj) and
    ||dH||_F / ||H||_F <= 1e-4.
  * perm: a permutation; identity when act_order is off; with act_order on,
    any pair that the candidate orders against the oracle's descending
    diag(H) must be a near-tie (relative gap <= 1e-4).  The oracle then
    replays the candidate's order.
  * codes and zero points: the oracle runs its own loop; wherever the
    candidate's integer differs by exactly one and the oracle's pre-round
    value lies within `window` (1e-4, in code units) of the half-integer
    between the two, the oracle adopts the candidate's value (an exact-tie
    case where either integer is correct), counts it exempt and keeps
    propagating from it.  Any other difference is a mismatch.  Exempt entries
    must be <= 0.1% of codes + zeros.
  * scales: relative 1e-3 on the followed path.
  * proxy loss ||(W - W_hat) X^T||^2 within 0.5% of the oracle's own
    (unfollowed) run.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import gptq_oracle as O


def check_hessian(H_cand: np.ndarray, H_ref: np.ndarray, rel: float = 1e-4) -> dict:
    H_cand = np.asarray(H_cand, dtype=np.float64)
    d = np.sqrt(np.abs(np.diag(H_ref)))
    scale = np.outer(d, d)
    diff = np.abs(H_cand - H_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        elem = np.where(scale > 0, diff / scale, np.where(diff > 0, np.inf, 0.0))
    norm = float(np.linalg.norm(H_cand - H_ref) / max(np.linalg.norm(H_ref), 1e-300))
    return dict(max_elem=float(elem.max()) if elem.size else 0.0, norm=norm,
                ok=bool((elem.max() if elem.size else 0.0) <= rel and norm <= rel),
                symmetric=bool(np.array_equal(H_cand, H_cand.T)))


def check_perm(perm: np.ndarray, diag_ref: np.ndarray, act_order: bool, rel: float = 1e-4) -> dict:
    perm = np.asarray(perm, dtype=np.int64)
    d = diag_ref.shape[0]
    if perm.shape != (d,) or not np.array_equal(np.sort(perm), np.arange(d)):
        return dict(ok=False, reason="not a permutation")
    if not act_order:
        ok = bool(np.array_equal(perm, np.arange(d)))
        return dict(ok=ok, reason="" if ok else "act_order off but perm is not the identity")
    v = diag_ref[perm]
    # largest value that appears later in the candidate order
    later_max = np.maximum.accumulate(v[::-1])[::-1]
    tol = rel * np.maximum(np.abs(v), np.abs(later_max))
    bad = np.nonzero(later_max - v > tol)[0]
    return dict(ok=bad.size == 0, reason="" if bad.size == 0 else f"{bad.size} out-of-order positions",
                inversions=int(np.sum(v[:-1] < v[1:])))


@dataclass
class _Follow:
    cand_codes: np.ndarray      # [d_out, d_in]
    cand_zeros: np.ndarray      # [G, d_out]
    maxq: int
    window: float
    exempt_codes: int = 0
    exempt_zeros: int = 0
    mism_codes: int = 0
    mism_zeros: int = 0
    worst: list = field(default_factory=list)

    def _follow(self, ours, theirs, pre, zshift):
        diff = theirs != ours
        if not diff.any():
            return ours, 0, 0
        lo = np.minimum(ours, theirs)
        tie = np.abs(pre - (lo - zshift + 0.5)) < self.window
        take = diff & (np.abs(theirs - ours) == 1) & tie
        out = np.where(take, theirs, ours)
        return out, int(take.sum()), int((diff & ~take).sum())

    def code(self, k, q, t, z):
        out, ex, mm = self._follow(q, self.cand_codes[:, k].astype(np.float64), t, z)
        self.exempt_codes += ex
        self.mism_codes += mm
        if mm and len(self.worst) < 8:
            r = int(np.nonzero(self.cand_codes[:, k] != out)[0][0])
            self.worst.append(("code", r, k, float(t[r]), int(q[r]), int(self.cand_codes[r, k])))
        return out

    def zero(self, gi, z, tz):
        out, ex, mm = self._follow(z, self.cand_zeros[gi].astype(np.float64), tz, 0.0)
        self.exempt_zeros += ex
        self.mism_zeros += mm
        if mm and len(self.worst) < 8:
            r = int(np.nonzero(self.cand_zeros[gi] != out)[0][0])
            self.worst.append(("zero", r, gi, float(tz[r]), int(z[r]), int(self.cand_zeros[gi, r])))
        return out


def check_layer(W0: np.ndarray, H_ref: np.ndarray, bits: int, group_size: int, block_size: int,
                damp: float, act_order: bool, qpacked: np.ndarray, scales: np.ndarray,
                zeros: np.ndarray, perm: np.ndarray, window: float = 1e-4,
                exempt_frac: float = 1e-3, scale_rel: float = 1e-3, loss_rel: float = 5e-3,
                ref_run: dict | None = None, U=None) -> dict:
    """Full parity verdict for one layer.  W0: float64 [d_out, d_in] original order.
    U: optional inverse factor from this package's oracle for H_ref in the
    candidate's order and this damping (large layers compute it once)."""
    W0 = np.asarray(W0, dtype=np.float64)
    d_out, d_in = W0.shape
    g = O._eff_group(d_in, group_size)
    G = (d_in + g - 1) // g
    maxq = (1 << bits) - 1
    res: dict = {}

    codes = O.unpack(qpacked, bits, d_in)
    scales = np.asarray(scales, dtype=np.float64).reshape(G, d_out)
    zeros = np.asarray(zeros, dtype=np.float64).reshape(G, d_out)
    pc = check_perm(perm, np.diag(H_ref), act_order)
    res["perm"] = pc
    if not pc["ok"]:
        res["ok"] = False
        return res
    res["codes_in_range"] = bool(codes.min() >= 0 and codes.max() <= maxq)
    res["zeros_integral"] = bool(np.all(zeros == np.rint(zeros)) and zeros.min() >= 0 and zeros.max() <= maxq)

    fol = _Follow(codes, zeros, maxq, window)
    run = O.gptq(W0, H_ref, bits, group_size, block_size, damp, act_order, perm=np.asarray(perm),
                 decide_code=fol.code, decide_zero=fol.zero, U=U)
    total = codes.size + zeros.size
    res.update(exempt_codes=fol.exempt_codes, exempt_zeros=fol.exempt_zeros,
               mismatch_codes=fol.mism_codes, mismatch_zeros=fol.mism_zeros,
               exempt_frac=(fol.exempt_codes + fol.exempt_zeros) / max(total, 1), worst=fol.worst)
    # how close the oracle's own pre-round values came to a rounding boundary
    # (distance to the nearest half-integer, code units) where both sides agree
    dist = np.abs(run["t"] - np.floor(run["t"]) - 0.5)
    res["min_boundary_dist"] = float(dist.min()) if dist.size else 0.0
    res["within_1e-3_of_boundary"] = int(np.count_nonzero(dist < 1e-3))
    with np.errstate(divide="ignore", invalid="ignore"):
        srel = np.abs(scales - run["scales"]) / np.abs(run["scales"])
    res["scale_max_rel"] = float(np.nanmax(srel)) if srel.size else 0.0

    # loss against the oracle's own, unfollowed run
    if ref_run is None:
        own = O.act_order_perm(H_ref) if act_order else np.arange(d_in)
        same = np.array_equal(own, np.asarray(perm))     # then the factor is the same one
        ref_run = O.gptq(W0, H_ref, bits, group_size, block_size, damp, act_order,
                         U=run["U"] if same else None)
    W_ref = O.dequantize(ref_run["codes"], ref_run["scales"], ref_run["zeros"], ref_run["perm"], g)
    W_cand = O.dequantize(codes, scales, zeros, perm, g)
    l_ref = O.proxy_loss(W0, W_ref, H_ref)
    l_cand = O.proxy_loss(W0, W_cand, H_ref)
    res.update(loss_ref=l_ref, loss_cand=l_cand,
               loss_rel=abs(l_cand - l_ref) / l_ref if l_ref > 0 else abs(l_cand))
    res["ok"] = bool(res["codes_in_range"] and res["zeros_integral"]
                     and fol.mism_codes == 0 and fol.mism_zeros == 0
                     and res["exempt_frac"] <= exempt_frac
                     and res["scale_max_rel"] <= scale_rel
                     and (res["loss_rel"] <= loss_rel or (l_ref == 0 and l_cand == 0)))
    return res
