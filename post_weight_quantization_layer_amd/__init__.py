"""GPTQ layer quantization on MI355X (gfx950): HIP kernels behind a C ABI.

The native library (libgptq_mi355x.so) is loaded on first use by
``post_weight_quantization_layer_amd.binding``; importing the package itself
does not touch the GPU.
"""
__all__ = ["inputs", "binding"]
