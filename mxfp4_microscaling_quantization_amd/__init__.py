"""MXFP4 (OCP MX) quantized-training hot path for AMD MI355X (gfx950).

The compute lives in a HIP shared library with a plain C ABI (include/mx.h);
this package is only its Python binding plus seeded synthetic inputs.
"""
