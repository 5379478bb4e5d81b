"""Block-GTQ packed-cache decode path for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libbgtq.so`` (C ABI declared in
``include/bgtq.h``); ``decode_attention_rope_amd.bgtq`` is its thin Python
binding.  ``decode_attention_rope_amd.synth`` draws the seeded synthetic
inputs.  Importing the package does not load the library; the first call into
``bgtq`` does, and raises if it is missing.
"""

__all__ = ["bgtq", "synth"]
