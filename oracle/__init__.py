"""CPU oracle for exact softmax attention: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from here. The GPU library and its Python
binding never do, and this package imports nothing from them.

Contents
  core        ctypes front end of ``fa_oracle.c``: fp64 three-pass safe-softmax
              attention (the definition written out), and its gradients with
              respect to q, k, v by the chain rule (``attention_backward``), and the
              definition under a sliding-window / key-padding mask
              (``attention_masked``) and under a mask over blocks of the score
              matrix (``attention_blocksparse``); the gradients under the
              window / key-padding mask (``attention_backward_masked``) and under
              a block mask (``attention_backward_blocksparse``).
  recurrence  the online-softmax recurrence for one query in fp64, block by
              block, in any block partition and order, with switches that plant
              the four classic implementation mistakes (used only to show that
              the pins catch them).
  brute       50-digit decimal evaluation of the definition with no
              max-subtraction, for tiny inputs, and gradients of the loss
              sum(dO * O) by 50-digit central differences of it.

Pins (tests/test_oracle_*.py): the two worked examples printed on the pages
(tests/golden/), closed forms (uniform keys, a single key, causal row 0),
softmax rows summing to 1, shift invariance, block order/size invariance and
the brute force. The gradients (tests/test_oracle_bwd_pins.py): decimal
finite differences, fp64 autograd, sum rules, translation invariance,
linearity and closed forms. The masked definition
(tests/test_oracle_mask_pins.py): brute force with the same predicate,
reductions to unmasked attention over each row's key slice and over truncated
keys, and the causal / unmasked special cases. The block-sparse definition
(tests/test_oracle_blocksparse_pins.py): brute force, all-ones and
block-diagonal and block-triangular reductions, a per-row gather, mask forms
and empty rows. The masked gradients (tests/test_oracle_bwd_mask_pins.py):
decimal finite differences with the same predicate, fp64 autograd through a
masked softmax, reductions to the unmasked and causal gradients, sum rules and
zero cases; the block-masked gradients (tests/test_oracle_bwd_blocksparse_pins.py)
likewise, with block-diagonal and all-ones reductions. Every function here is pinned; none is "parity unpinned"
except the second worked example's output vector, whose value vectors the
page does not print.
"""
