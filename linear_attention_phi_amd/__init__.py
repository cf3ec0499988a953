"""Causal linear attention with phi(x) = elu(x) + 1 on one MI355X (gfx950).

The compute lives in the HIP library ``liblinattn.so`` (built from ``csrc/``)
behind the C ABI declared in ``include/linattn.h``.  ``binding`` marshals torch
tensors into that ABI; there is no fallback path: a missing library raises.
"""
