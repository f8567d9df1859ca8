"""MI355X (gfx950) implementation of APB's per-host prefill path.

The compute lives in the HIP library libapb.so (C ABI declared in include/apb.h).
`binding` wraps its entry points for torch tensors; `synth` draws the seeded
synthetic inputs.  Importing the package does not load the library; the first
call into `binding` does, and raises if it is missing.
"""
__all__ = ["binding", "synth"]
