"""MI355X-native decoder-only transformer block forward (prefill + batched decode).

The compute path is the C-ABI library `libdec.so` built from `csrc/` (HIP for
gfx950); `dec.py` is its thin ctypes binding.  Importing this package loads
nothing: `decoder_only_forward_amd.dec.load()` opens the library and raises if
it has not been built.
"""
from .configs import ModelConfig, CONFIGS  # noqa: F401
