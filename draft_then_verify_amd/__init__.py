"""MI355X (gfx950) verify hot path of speculative decoding.

``binding`` exposes the C ABI of ``libspecverify.so`` (HIP kernels); ``runner``
drives speculative rounds through it; ``build`` compiles the library.
Importing the package does not touch the GPU.
"""
