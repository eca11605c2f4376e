"""MI355X (gfx950) library of the dual-phase policy step, with its Python binding.

The compute path is libvla.so (HIP kernels behind the C ABI of include/vla.h);
`prefix_cache_flow_amd.vla` marshals torch tensors to it.  Importing this
package loads nothing; `prefix_cache_flow_amd.vla.lib()` loads the library and
raises if it is missing.
"""
__all__ = ["vla", "build"]
