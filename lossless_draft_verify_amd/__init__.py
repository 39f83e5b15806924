"""MI355X-native DSpark draft-and-verify round (libdspark.so + thin ctypes binding).

The binding functions load the in-tree HIP library on first use and raise if it is missing;
there is no CPU fallback.
"""
from .binding import *  # noqa: F401,F403
