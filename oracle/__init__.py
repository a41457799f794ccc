"""CPU oracle for attention against a KV cache -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain definition that the GPU library is checked
against.  Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product: the two share no code.  Inputs come from ``synth``,
which only draws random numbers.

What it computes (all arithmetic in float64 unless a rounding step is named):

* ``numerics`` -- round-to-nearest-even into float32 and bfloat16 storage.
* ``rope``     -- rotary embedding at absolute positions (Tiny-GPT post,
  "Two Gotchas That Break It Quietly", Gotcha 1).
* ``attention``-- softmax attention with GQA head sharing and absolute-position
  causal visibility, and the no-cache recompute built on it (Tiny-GPT post,
  "What the No-Cache Loop Wastes"; nanochat post, "What the KV cache looks
  like on disk"; Cake paper, Section 3 "Background").
* ``model``    -- the single fp32 layer and the six-layer tiny GPT, each rerun
  over the whole token history at every step (Tiny-GPT post, "The Cache, in
  Code").
* ``brute``    -- the same definitions written as pure-Python loops for tiny
  inputs, used to pin the NumPy version.

Parity status: every function here is pinned by a CPU test (brute force,
a library routine for a special case, closed forms, or identities); see
``tests/test_oracle_pins.py``.  None of the pages prints attention output
values, so no pin is a page-printed attention number.
"""
from . import numerics, rope, attention, model, brute  # noqa: F401
