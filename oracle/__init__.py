"""CPU oracle for the Block-GTQ packed-cache decode path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the GPU path computes.  Only the test-suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The HIP library never calls it and shares no code, header, table or
constant generator with it.

Source: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (Liang, Zhang,
Jia; arXiv 2606.24033), abstract as printed on paperdance.org/p/2606.24033 and
mirrored on the other pages.  The abstract fixes the structure of the method:

* RoPE splits a key's contribution to a later logit into a position-dependent
  sum over 2-D frequency blocks (``rope``);
* per layer and KV head a label-free energy score is computed for every RoPE
  block (``energy``);
* integer bit widths are handed out greedily by marginal gain under a matched
  K bit budget (``allocate``);
* keys are quantized with TurboQuant-MSE at those widths and values at a
  uniform width (``codebook``, ``layout``, ``quantize``);
* a packed-cache serving path attends directly over the packed cache
  (``pack``, ``decode``);
* the method is judged by the key-only RoPE logit error against uniform
  TQ-MSE at the same budget (``diagnostic``).

Everything numeric that the abstract leaves open is a stated reading; each
function names the reading it follows.  Floating point is fp64 except where
the reading fixes the quantizer's bit-exact fp32 arithmetic.

Parity status: every function here is pinned by a ``-m "not gpu"`` test to a
closed form, a textbook value, brute force or a library routine; none is
"parity unpinned" except the comparison with the authors' own implementation,
which is not available.
"""

# submodules: codebook, rope, energy, allocate, layout, quantize, pack, decode, diagnostic
