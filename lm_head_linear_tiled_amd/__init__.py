"""MI355X (gfx950) fused linear + cross-entropy.

Import is lazy: ``lm_head_linear_tiled_amd.inputs`` and ``.roofline`` are pure host
modules; ``lm_head_linear_tiled_amd.binding`` loads the HIP library (``libflce.so``)
and raises if it is missing.
"""
__all__ = ["binding", "inputs", "roofline"]
