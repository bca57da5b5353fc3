"""libsvq: SVQ decode-and-multiply for MI355X (gfx950), HIP kernels behind a C ABI.

``bit_spherical_vector_amd.svq`` is the ctypes binding of ``libsvq.so``
(built in-tree by ``bit_spherical_vector_amd.build``).  Importing it raises
if the library is not built; nothing falls back to a CPU path.
"""
__all__ = ["svq", "build"]
