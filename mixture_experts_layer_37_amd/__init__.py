"""MI355X (gfx950) Mixture-of-Experts FFN layer forward: HIP kernels behind the C ABI of
include/moe.h (libmoe.so), with a thin ctypes binding.

Submodules: ``configs`` (the workloads), ``inputs`` (seeded synthetic inputs), ``_lib``
(the binding), ``layer`` (torch plumbing), ``build`` (hipcc build of libmoe.so)."""
from . import configs  # noqa: F401
