"""MI355X-native block-diffusion denoising step (libdllm.so + ctypes binding).

The compute path is entirely in the HIP library; this package only marshals
arguments.  Importing it fails loudly if the library has not been built."""
from .binding import *  # noqa: F401,F403
from .binding import LIB_PATH, load_library  # noqa: F401
