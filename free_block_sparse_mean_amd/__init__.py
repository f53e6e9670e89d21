"""Sol-Attn on-the-fly block-sparse attention forward for AMD MI355X (gfx950).

The compute path is the HIP library libsolattn.so (C ABI in include/sol_attn.h);
`binding` is its ctypes binding, `workloads` the seeded synthetic inputs.
Nothing is imported eagerly, so importing the package never loads the library.
"""
__all__ = ["binding", "workloads", "build"]
