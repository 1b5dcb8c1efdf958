"""MI355X (gfx950) chunk-parallel gated linear attention: forward and backward.

The compute lives in a HIP shared library with a C ABI (``include/gla.h``);
``ssm_recurrence_amd.binding`` marshals torch tensors to it.  Importing this
package does not load the library; ``binding.load()`` does, and raises if it
has not been built.
"""
__all__ = ["binding", "inputs"]
