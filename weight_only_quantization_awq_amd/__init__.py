"""AWQ per-linear-layer hot path for AMD MI355X (gfx950).

The GPU library (``libawq_mi355x.so``) is loaded lazily by the binding module
``weight_only_quantization_awq_amd.awq``; importing this package does not
touch the GPU.
"""
__all__ = ["awq", "synth"]
