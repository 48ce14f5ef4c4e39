"""Stochastic verification at temperature T > 0 (oracle; test infrastructure
only).

The pages: the dequant step brings the logits back to high precision before
softmax and the acceptance test, so the rejection-sampling criterion of
speculative decoding keeps its lossless guarantee: the emitted tokens follow
the verifier's distribution, which the pages take to match the original
model's ([de] §2 "De-Quantisierung"; [it] §2 item 3 "Campionamento di
rifiuto lossless"; [fr] §2 "Échantillonnage de rejet"; [ja] §2.2 item 4);
the speedup holds from T = 0 to T = 1 ([de] §3 "Robustheit"; [it] §4;
[ja] §4).

What is computed (standard speculative sampling, specialised to drafts that
are single tokens, i.e. the drafter's distribution at each position is a
point mass on its token, as for N-gram or greedy self-drafting):

  for each sequence b, positions i = 0..G-1 in order:
      p_i = softmax(y32[b*(G+1)+i] / T)
      accept draft d_i with probability p_i(d_i); stop at the first rejection
  n = number accepted
  if n < G: next token ~ p_n with d_n removed, renormalised
            (the residual max(0, p_n - q_n) for q_n = point mass on d_n)
  else:     next token ~ p_G (the bonus token)

Readings (the pages give no formulas for this step), chosen so that the
result is a deterministic function of the inputs and identical on any
hardware:

* T enters as one fp32 multiply by inv_t = fp32(1/T) (correctly rounded):
  x_j = fp32(fp32(y_j - m) * inv_t), m = the row maximum; x_j is clamped
  below at -32;
* e^x is :func:`exp_f32`, an fp32 routine written out below (Cody-Waite
  reduction by ln 2, degree-7 Taylor polynomial in Horner form, exact
  scaling by 2^k): every step is one IEEE operation, so any
  implementation that performs the same steps gets the same bits;
* the weights are fixed point, W_j = floor(e^{x_j} * 2^40) (the maximum is
  exactly 2^40; weights below 2^-40 of the maximum are 0, which the clamp
  at -32 guarantees for x < -32).  Sums of W are exact integers, so they do
  not depend on the order of summation;
* the random numbers are inputs: u_accept[b][i], uint32, accepts d_i iff
  u * Z < W(d_i) * 2^32 (probability ceil(W(d_i) 2^32 / Z) / 2^32, with
  Z = sum_j W_j); u_sample[b], uint64, picks the first token j with
  S_j > floor(u * Z' / 2^64), S_j the inclusive prefix sum of the sampled
  row's weights (d_n's weight set to 0 after a rejection) and Z' its total
  (inverse-CDF sampling; every token j gets probability W_j / Z' up to
  2^-64);
* a draft id outside [0, V) has weight 0: it is never accepted, and it
  removes nothing from the residual.
"""
import numpy as np

EXP_CLAMP = np.float32(-32.0)
FIXED_BITS = 40
_LOG2E = np.float32(1.4426950408889634)       # fp32(1/ln 2)
_LN2_HI = np.float32(0.693145751953125)       # 15 significant bits: k*_LN2_HI is exact
_LN2_LO = np.float32(1.4286068203094173e-06)  # fp32(ln 2 - _LN2_HI)
# Taylor coefficients 1/n!, n = 7..2, rounded to fp32
_TAYLOR = [np.float32(1.0 / f) for f in (5040.0, 720.0, 120.0, 24.0, 6.0, 2.0)]


def exp_f32(x) -> np.ndarray:
    """e^x for fp32 x in [-32, 0], step by step in fp32:
    k = rint(x * LOG2E); r = (x - k*LN2_HI) - k*LN2_LO;
    p = Horner(1/7!, 1/6!, ..., 1/2!, 1, 1) at r; result = p * 2^k.
    Each multiply and add is a separate correctly rounded fp32 operation
    (no fused multiply-add)."""
    x = np.asarray(x, dtype=np.float32)
    if np.any(x < EXP_CLAMP) or np.any(x > 0) or not np.all(np.isfinite(x)):
        raise ValueError("exp_f32 is defined on [-32, 0]")
    k = np.rint(x * _LOG2E).astype(np.float32)
    r = ((x - k * _LN2_HI).astype(np.float32) - k * _LN2_LO).astype(np.float32)
    p = np.full_like(r, _TAYLOR[0])
    for c in _TAYLOR[1:]:
        p = (p * r).astype(np.float32) + c
    p = (p * r).astype(np.float32) + np.float32(1.0)   # + r * 1
    p = (p * r).astype(np.float32) + np.float32(1.0)   # + 1
    return np.ldexp(p, k.astype(np.int32)).astype(np.float32)


def inv_temperature(temperature) -> np.float32:
    t = np.float32(temperature)
    if not (np.isfinite(t) and t > 0):
        raise ValueError("temperature must be finite and > 0")
    with np.errstate(over="raise"):
        inv = np.float32(1.0) / t
    return np.float32(inv)


def fixed_weights(y_row, inv_t) -> np.ndarray:
    """uint64 W_j = floor(exp_f32(max(fp32((y_j - m) * inv_t), -32)) * 2^40)
    for one fp32 logits row y (finite), m = max_j y_j."""
    y = np.asarray(y_row, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("logits must be finite")
    m = np.max(y)
    x = ((y - m).astype(np.float32) * np.float32(inv_t)).astype(np.float32)
    x = np.maximum(x, EXP_CLAMP)
    w = exp_f32(x)
    return np.floor(w.astype(np.float64) * float(1 << FIXED_BITS)).astype(np.uint64)


def accept_threshold(w_draft: int, z: int) -> int:
    """Number of uint32 values u with u * z < w_draft * 2^32, i.e. the
    acceptance probability times 2^32."""
    return min(1 << 32, -(-(int(w_draft) << 32) // int(z)))


def sample_index(weights, u64: int) -> int:
    """First j with S_j > floor(u64 * Z / 2^64), S the inclusive prefix sums
    of the uint64 weights and Z their total (Z > 0)."""
    w = np.asarray(weights, dtype=np.uint64)
    s = np.cumsum(w, dtype=np.uint64)
    z = int(s[-1])
    if z == 0:
        raise ValueError("all weights are zero")
    t = (int(u64) * z) >> 64
    return int(np.searchsorted(s, np.uint64(t), side="right"))


def verify_sample(logits, draft, temperature, u_accept, u_sample) -> tuple:
    """Stochastic verification of B sequences of G drafts.

    logits fp32 [B*(G+1)][V] (row b*(G+1)+i: the verifier after position i),
    draft int [B][G], u_accept uint32 [B][G], u_sample uint64 [B].
    Returns (accept_len int32[B], next_token int32[B])."""
    y = np.asarray(logits, dtype=np.float32)
    d = np.asarray(draft, dtype=np.int64)
    if d.ndim != 2:
        raise ValueError("draft must be [B][G]")
    B, G = d.shape
    R, V = y.shape
    if R != B * (G + 1) or V == 0:
        raise ValueError("logits must be [B*(G+1)][V] with V > 0")
    ua = np.asarray(u_accept, dtype=np.uint64).reshape(B, G)
    us = np.asarray(u_sample, dtype=np.uint64).reshape(B)
    inv_t = inv_temperature(temperature)
    accept_len = np.zeros(B, dtype=np.int32)
    next_token = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n < G:
            w = fixed_weights(y[b * (G + 1) + n], inv_t)
            z = int(np.sum(w, dtype=np.uint64))
            dn = int(d[b, n])
            wd = int(w[dn]) if 0 <= dn < V else 0
            if int(ua[b, n]) * z < (wd << 32):
                n += 1
            else:
                break
        w = fixed_weights(y[b * (G + 1) + n], inv_t)
        if n < G and 0 <= int(d[b, n]) < V:
            w[int(d[b, n])] = 0       # the residual: the rejected draft removed
        accept_len[b] = n
        next_token[b] = sample_index(w, int(us[b]))
    return accept_len, next_token
