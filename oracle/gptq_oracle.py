"""Plain float64 CPU oracle of the GPTQ layer quantizer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code with the HIP library.

Sources (web pages on GPTQ; cited by page title and section):
  [OBQ]   "GPTQ (GPT Quantization)" (brain.gartu.xyz), section
          "Fondation theorique : OBQ": quantize column i, take its error,
          move the remaining columns F by -e_i / (H^-1)_ii * (H^-1)_{i,F},
          with H = 2 X^T X over the calibration inputs.
  [ALGO]  same page, section "Algorithme complet (pseudo-code)": H = 2 X^T X,
          add lambda*I, invert through Cholesky, quantize the columns in
          batches and push each batch's error onto the later columns once
          (lazy update).
  [SCAL]  same page, section "Optimisations de GPTQ pour la scalabilite":
          naive OBQ is far too slow for LLMs, hence the batched form.
  [GROUP] "Optimization Gptq" skill page (skillsdirectory.com), section
          "Quantizacao group-wise": every group of consecutive weights
          (typically 128) has its own scale and zero point.
  [CONF]  same page, "Configuracoes de quantizacao": bits, group_size,
          desc_act (activation order), damp_percent = 0.01.
  [TECH]  "GPTQ" (wikiprompt.org), "Abordagem Tecnica": greedy column
          order with a closed-form compensation of the remaining weights.

Readings where the pages are silent or garbled (each also listed with the
design notes of this repository):
  * W is d_out x d_in and a column is one input channel (the pseudo-code's
    header says d_in x d_out but indexes W[:, i:i+bs] over d_in).
  * The update uses the inverse over the *remaining* columns F ([OBQ]).  Its
    needed row equals U_kk * U[k, k:] where U is the upper Cholesky factor of
    H_d^-1 = U^T U, so the step is E_k = (w_k - q_k) / U_kk and
    W[:, j] -= E_k * U[k, j].  The pseudo-code's single static inverse with a
    division by diag(H_inv[block]) after the product is read as this.
  * Inside a batch the columns are quantized one at a time with immediate
    updates; only the update of the columns after the batch is deferred.
  * Group parameters are taken at the group's first column from the current
    (already compensated) values of all its columns.  This needs
    block_size % group_size == 0 unless one group spans the whole row.
  * Quantizer: asymmetric min-max with the range widened to contain 0:
    xmin = min(0, min w), xmax = max(0, max w); an all-zero group uses
    [0, 1] (every entry still maps to 0, and the zero point is not a
    rounding tie in any precision); s = (xmax - xmin) / (2^b - 1);
    z = rint(-xmin / s);
    q = clamp(rint(w / s) + z, 0, 2^b - 1); w_hat = s * (q - z).
    Rounding is round-half-to-even.
  * lambda = damp * mean(diag H), added after the activation-order gather.
  * Activation order: stable sort of diag(H) (undamped) descending, ties to
    the lower index; groups are consecutive in processing order.
  * H = 2 X^T X exactly (no 1/n).
"""
from __future__ import annotations

import numpy as np
import scipy.linalg

__all__ = [
    "widen", "hessian", "act_order_perm", "damping", "inverse_cholesky_upper",
    "inverse_cholesky_upper_reverse", "group_params", "quantize_values", "gptq",
    "obq_naive", "rtn", "pack", "unpack", "packed_words", "dequantize",
    "proxy_loss", "n_groups", "dequant_matmul",
]


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bytes -> float64 values.  'bf16' arrays hold uint16 bit patterns."""
    if dtype == "bf16":
        u = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f64"):
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# stage 1: Hessian  ([OBQ] definition of H, [ALGO] step 1)
# ----------------------------------------------------------------------------
def hessian(chunks, dtype: str, d_in: int) -> np.ndarray:
    """H = 2 * sum over token chunks of X_c^T X_c, in float64."""
    H = np.zeros((d_in, d_in), dtype=np.float64)
    for xc in chunks:
        x = widen(xc, dtype)
        H += x.T @ x
    return 2.0 * H


# ----------------------------------------------------------------------------
# stage 2: order, damping, inverse factor  ([ALGO] steps 1-2, [CONF])
# ----------------------------------------------------------------------------
def act_order_perm(H: np.ndarray) -> np.ndarray:
    """Processing order by descending diag(H); equal values keep index order."""
    return np.argsort(-np.diag(H), kind="stable").astype(np.int64)


def damping(H: np.ndarray, damp: float) -> float:
    """lambda = damp * mean(diag H)."""
    return float(damp) * float(np.mean(np.diag(H)))


def inverse_cholesky_upper(Hd: np.ndarray) -> np.ndarray:
    """U upper-triangular with H_d^-1 = U^T U (plain route).

    L = chol(H_d) (lower), H_d^-1 = L^-T L^-1, U = chol(H_d^-1)^T.
    Raises numpy.linalg.LinAlgError when H_d is not positive definite.
    """
    L = np.linalg.cholesky(Hd)
    Linv, info = scipy.linalg.lapack.dtrtri(L, lower=1)     # L^-1 (LAPACK triangular inverse)
    if info != 0:
        raise np.linalg.LinAlgError("singular Cholesky factor")
    del L
    Hinv = Linv.T @ Linv
    del Linv
    Hinv += Hinv.T
    Hinv *= 0.5
    return np.linalg.cholesky(Hinv).T


def inverse_cholesky_upper_reverse(Hd: np.ndarray) -> np.ndarray:
    """Same U by a second route: factor H_d in reversed index order.

    With J the reversal, J H_d J = L' L'^T gives H_d = V V^T, V = J L' J upper;
    then U = V^-1 (upper with positive diagonal, so equal to the plain route's
    U by uniqueness of the Cholesky factor).  It costs a quarter of the plain
    route's flops, so the large parity tests take their factor from here.
    """
    Lr = np.linalg.cholesky(np.ascontiguousarray(Hd[::-1, ::-1]))
    V = np.ascontiguousarray(Lr[::-1, ::-1])
    del Lr
    U, info = scipy.linalg.lapack.dtrtri(V, lower=0)          # V^-1 (LAPACK triangular inverse)
    if info != 0:
        raise np.linalg.LinAlgError("singular Cholesky factor")
    return U


# ----------------------------------------------------------------------------
# quantizer  ([GROUP]; formula: reading above)
# ----------------------------------------------------------------------------
def group_params(x: np.ndarray, maxq: int):
    """Per-row scale and zero point of a group.

    x: [rows, cols] current values of the group's columns.
    Returns (s, z, tz) with tz = -xmin/s, the zero point's pre-round value.
    """
    xmin = np.minimum(x.min(axis=1), 0.0)
    xmax = np.maximum(x.max(axis=1), 0.0)
    flat = xmax == xmin                      # only an all-zero group
    xmax = np.where(flat, 1.0, xmax)
    s = (xmax - xmin) / maxq
    tz = -xmin / s
    z = np.rint(tz)
    return s, z, tz


def quantize_values(w: np.ndarray, s: np.ndarray, z: np.ndarray, maxq: int):
    """Returns (q, w_hat, t) with t = w/s the code's pre-round value."""
    t = w / s
    q = np.clip(np.rint(t) + z, 0, maxq)
    return q, s * (q - z), t


def n_groups(d_in: int, group_size: int) -> int:
    g = _eff_group(d_in, group_size)
    return (d_in + g - 1) // g


def _eff_group(d_in: int, group_size: int) -> int:
    if group_size == -1 or group_size >= d_in:
        return d_in
    if group_size < 1:
        raise ValueError("group_size must be -1 or >= 1")
    return group_size


# ----------------------------------------------------------------------------
# stages 3+4: the blocked quantize-and-compensate loop  ([OBQ], [ALGO])
# ----------------------------------------------------------------------------
def gptq(W0: np.ndarray, H: np.ndarray, bits: int, group_size: int, block_size: int,
         damp: float, act_order: bool, perm=None, decide_code=None, decide_zero=None,
         on_column=None, U=None) -> dict:
    """GPTQ on one layer, float64.

    W0: [d_out, d_in] values (float64); H: [d_in, d_in] undamped Hessian.
    perm: optional processing order to use instead of the one derived from H
          (the parity checker replays a valid GPU order this way).
    decide_code(k, q, t, z) / decide_zero(group, z, tz): optional hooks that
          may replace a rounding decision (used by the parity checker to
          follow the other side at exact rounding ties); they must return
          arrays of the same shape.
    on_column(k, W): optional observer called after column k is done.
    U: optional inverse factor already computed by this module for the same
          H, order and damping (the parity checker's two runs share one).

    Returns a dict; every per-column array is in processing order:
      codes [d_out, d_in] int, scales/zeros [n_groups, d_out], perm [d_in],
      w_hat [d_out, d_in] (processing order), t and tz pre-round values,
      E [d_out, d_in] normalized errors, U, lam.
    """
    W0 = np.asarray(W0, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    d_out, d_in = W0.shape
    maxq = (1 << bits) - 1
    g = _eff_group(d_in, group_size)
    if block_size < 1:
        raise ValueError("block_size must be >= 1")
    if g < d_in and block_size < d_in and block_size % g != 0:
        raise ValueError("block_size must be a multiple of group_size")
    B = min(int(block_size), d_in)

    if perm is None:
        perm = act_order_perm(H) if act_order else np.arange(d_in)
    perm = np.asarray(perm, dtype=np.int64)
    W = W0[:, perm].copy()
    lam = damping(H, damp)
    if U is None:
        Hd = H[np.ix_(perm, perm)]
        Hd[np.diag_indices(d_in)] += lam
        U = inverse_cholesky_upper(Hd)
        del Hd

    G = (d_in + g - 1) // g
    codes = np.zeros((d_out, d_in), dtype=np.int64)
    w_hat = np.zeros((d_out, d_in))
    t_all = np.zeros((d_out, d_in))
    E = np.zeros((d_out, d_in))
    scales = np.zeros((G, d_out))
    zeros = np.zeros((G, d_out))
    tz_all = np.zeros((G, d_out))
    s = z = None
    for b in range(0, d_in, B):
        e = min(b + B, d_in)
        for k in range(b, e):
            if k % g == 0:
                gi = k // g
                s, z, tz = group_params(W[:, k:min(k + g, d_in)], maxq)
                if decide_zero is not None:
                    z = decide_zero(gi, z, tz)
                scales[gi], zeros[gi], tz_all[gi] = s, z, tz
            q, wq, t = quantize_values(W[:, k], s, z, maxq)
            if decide_code is not None:
                q = decide_code(k, q, t, z)
                wq = s * (q - z)
            err = (W[:, k] - wq) / U[k, k]
            codes[:, k], w_hat[:, k], t_all[:, k], E[:, k] = q, wq, t, err
            W[:, k + 1:e] -= np.outer(err, U[k, k + 1:e])
            if on_column is not None:
                on_column(k, W)
        W[:, e:] -= E[:, b:e] @ U[b:e, e:]
    return dict(codes=codes, scales=scales, zeros=zeros, perm=perm, w_hat=w_hat,
                t=t_all, tz=tz_all, E=E, U=U, lam=lam, group=g, maxq=maxq)


# ----------------------------------------------------------------------------
# naive OBQ: the inverse over the remaining columns recomputed every column
# ([OBQ] with F = remaining columns; [SCAL]: far too slow, tiny inputs only)
# ----------------------------------------------------------------------------
def obq_naive(W0: np.ndarray, H: np.ndarray, bits: int, group_size: int, damp: float,
              act_order: bool) -> dict:
    W0 = np.asarray(W0, dtype=np.float64)
    d_out, d_in = W0.shape
    maxq = (1 << bits) - 1
    g = _eff_group(d_in, group_size)
    perm = act_order_perm(H) if act_order else np.arange(d_in)
    W = W0[:, perm].copy()
    Hd = H[np.ix_(perm, perm)] + damping(H, damp) * np.eye(d_in)
    codes = np.zeros((d_out, d_in), dtype=np.int64)
    t_all = np.zeros((d_out, d_in))
    w_hat = np.zeros((d_out, d_in))
    for k in range(d_in):
        if k % g == 0:
            s, z, _ = group_params(W[:, k:min(k + g, d_in)], maxq)
        q, wq, t = quantize_values(W[:, k], s, z, maxq)
        Ginv = np.linalg.inv(Hd[k:, k:])            # (H_F)^-1, F = columns k..d_in-1
        e = W[:, k] - wq
        W[:, k:] -= np.outer(e / Ginv[0, 0], Ginv[0, :])
        codes[:, k], t_all[:, k], w_hat[:, k] = q, t, wq
    return dict(codes=codes, t=t_all, w_hat=w_hat, perm=perm)


def rtn(W0: np.ndarray, bits: int, group_size: int) -> dict:
    """Round-to-nearest baseline: every weight rounded on its own group's grid."""
    W0 = np.asarray(W0, dtype=np.float64)
    d_out, d_in = W0.shape
    maxq = (1 << bits) - 1
    g = _eff_group(d_in, group_size)
    G = (d_in + g - 1) // g
    codes = np.zeros((d_out, d_in), dtype=np.int64)
    w_hat = np.zeros((d_out, d_in))
    scales = np.zeros((G, d_out))
    zeros = np.zeros((G, d_out))
    for gi in range(G):
        c0, c1 = gi * g, min((gi + 1) * g, d_in)
        s, z, _ = group_params(W0[:, c0:c1], maxq)
        scales[gi], zeros[gi] = s, z
        for k in range(c0, c1):
            codes[:, k], w_hat[:, k], _ = quantize_values(W0[:, k], s, z, maxq)
    return dict(codes=codes, w_hat=w_hat, scales=scales, zeros=zeros)


# ----------------------------------------------------------------------------
# stage 5: bit packing (storage form implied by the pages' 4x memory figures)
# ----------------------------------------------------------------------------
def packed_words(d_in: int, bits: int) -> int:
    return (bits * d_in + 31) // 32


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [d_out, d_in] -> words [ceil(bits*d_in/32), d_out] uint32.

    Row r is a little-endian bit stream: code k occupies stream bits
    [bits*k, bits*k + bits); word w holds stream bits [32w, 32w + 32).
    """
    codes = np.asarray(codes, dtype=np.uint64)
    d_out, d_in = codes.shape
    nw = packed_words(d_in, bits)
    acc = np.zeros((nw + 1, d_out), dtype=np.uint64)
    for k in range(d_in):
        pos = bits * k
        w, off = divmod(pos, 32)
        v = codes[:, k] << np.uint64(off)
        acc[w] |= v & np.uint64(0xFFFFFFFF)
        acc[w + 1] |= v >> np.uint64(32)
    return acc[:nw].astype(np.uint32)


def unpack(words: np.ndarray, bits: int, d_in: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint64)
    nw, d_out = words.shape
    ext = np.concatenate([words, np.zeros((1, d_out), dtype=np.uint64)], axis=0)
    mask = np.uint64((1 << bits) - 1)
    out = np.zeros((d_out, d_in), dtype=np.int64)
    for k in range(d_in):
        w, off = divmod(bits * k, 32)
        v = (ext[w] >> np.uint64(off)) | (ext[w + 1] << np.uint64(32 - off))
        out[:, k] = (v & mask).astype(np.int64)
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, perm: np.ndarray,
               group: int) -> np.ndarray:
    """W_hat in original column order: W_hat[:, perm[k]] = s * (q - z) of column k."""
    codes = np.asarray(codes, dtype=np.float64)
    d_out, d_in = codes.shape
    gi = np.arange(d_in) // group
    deq = np.asarray(scales, dtype=np.float64)[gi].T * (codes - np.asarray(zeros, dtype=np.float64)[gi].T)
    out = np.empty_like(deq)
    out[:, np.asarray(perm)] = deq
    return out


def dequant_matmul(A: np.ndarray, qpacked: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                   perm: np.ndarray, bits: int, group_size: int, d_in: int) -> np.ndarray:
    """Y = A W_hat^T for a packed layer, in float64: unpack the codes,
    dequantize them into the original column order, multiply.

    The product that inference runs on the quantized weights ("Optimization
    Gptq", section "Backends de kernel"; "GPTQ (GPT Quantization)",
    "Limitations": dequantization before each product).  A: [m, d_in]
    activations in the original column order (float64 values).
    """
    codes = unpack(qpacked, bits, d_in)
    W_hat = dequantize(codes, scales, zeros, perm, _eff_group(d_in, group_size))
    return np.asarray(A, dtype=np.float64) @ W_hat.T


def proxy_loss(W0: np.ndarray, W_hat: np.ndarray, H: np.ndarray) -> float:
    """||(W0 - W_hat) X^T||_F^2 = 1/2 tr(dW H dW^T) with the undamped H (original order)."""
    dW = np.asarray(W0, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    return 0.5 * float(np.sum((dW @ H) * dW))
