"""libmla: DeepSeek-V3 Multi-head Latent Attention on AMD MI355X (gfx950).

The compute path is the HIP library ``libmla.so`` behind the C ABI in
``include/mla.h``; ``libmla`` is its ctypes binding and ``layer`` holds thin
device-buffer helpers.
"""
from . import libmla  # noqa: F401
