"""MI355X-native bidirectional multi-head attention for ViT encoders (``vitattn``).

The compute path is the HIP library ``libvitattn.so`` (hand-written gfx950
kernels behind a C ABI); :mod:`.binding` marshals torch tensors into it.
"""
from .binding import fwd, qkv_prologue, VitattnError, library_path, load_library  # noqa: F401
