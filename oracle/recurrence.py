"""The online-softmax recurrence for one query, in fp64. Test infrastructure only.

Follows "transformer math: flash attention math" (aicassindra.com), sections
"The running state: a max, a denominator, and an output", "The rescaling
identity, derived" and "The block-wise update, and the full algorithm", in the
page's notation:

    start:  m = -inf, l = 0, o~ = 0
    per block B (in the order given):
        m_blk = max over j in B of s_j
        m_new = max(m, m_blk)
        alpha = exp(m - m_new)          (rescales the old state, <= 1)
        p_j   = exp(s_j - m_new)        (each <= 1)
        l     = alpha * l + sum_j p_j
        o~    = alpha * o~ + sum_j p_j v_j
        m     = m_new
    result: o = o~ / l   (one division, after the last block)

The same two updates appear as l_new and a_new on "FlashAttention tiles exact
softmax without materializing the score matrix" (nalar.dev), sections "Online
softmax carries a maximum and a normalizer" and "The output accumulator must be
rescaled with the same state".

Masked keys (causal or padding) are given the score -inf before the block
maximum is taken ("Pitfalls in implementing the recurrence" on the aicassindra
page), so they carry no probability mass.

``pitfall`` plants one of the four mistakes listed under that "Pitfalls"
heading; the oracle tests use it to show that the pins catch each mistake:
  "no_rescale_o"        alpha is applied to l but not to o~
  "finite_m0"           the running max starts at 0 instead of -inf
  "mask_after_max"      the block max is taken before masked scores become -inf
  "normalize_per_block" o~ is divided by l after every block and the
                        normalised value is carried as the state
"""
import math

import numpy as np

PITFALLS = ("no_rescale_o", "finite_m0", "mask_after_max", "normalize_per_block")


def blocks_of(n, size):
    """Consecutive blocks [0,size), [size,2*size), ... covering range(n)."""
    return [np.arange(s, min(s + size, n)) for s in range(0, n, size)]


def online_softmax(s, v, blocks, allowed=None, pitfall=None):
    """Run the recurrence over ``blocks`` (index arrays into s, in visiting order).

    s       : [N] scores of one query (fp64).
    v       : [N] or [N, dv] values.
    allowed : optional boolean [N]; False keys are masked.
    Returns (o, trace) where trace is a list of dicts with the state after each
    block: m, l, o_tilde, alpha, p.
    """
    if pitfall is not None and pitfall not in PITFALLS:
        raise ValueError(f"unknown pitfall {pitfall!r}")
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scalar_v = v.ndim == 1
    if scalar_v:
        v = v[:, None]
    if allowed is None:
        allowed = np.ones(s.shape[0], dtype=bool)
    allowed = np.asarray(allowed, dtype=bool)

    m = 0.0 if pitfall == "finite_m0" else -math.inf
    l = 0.0
    o_t = np.zeros(v.shape[1], dtype=np.float64)
    trace = []
    for blk in blocks:
        blk = np.asarray(blk, dtype=np.int64)
        s_b = s[blk].copy()
        masked = ~allowed[blk]
        if pitfall == "mask_after_max":
            m_blk = float(np.max(s_b))
            s_b[masked] = -math.inf
        else:
            s_b[masked] = -math.inf
            m_blk = float(np.max(s_b))
        m_new = max(m, m_blk)
        alpha = math.exp(m - m_new)
        p = np.exp(s_b - m_new)
        l = alpha * l + float(np.sum(p))
        contrib = p @ v[blk]
        if pitfall == "no_rescale_o":
            o_t = o_t + contrib
        else:
            o_t = alpha * o_t + contrib
        if pitfall == "normalize_per_block":
            o_t = o_t / l
        m = m_new
        trace.append({"m": m, "l": l, "o_tilde": o_t.copy(), "alpha": alpha, "p": p.copy()})
    o = o_t if pitfall == "normalize_per_block" else o_t / l
    return (o[0] if scalar_v else o), trace
