"""MI355X-native packed KV-cache quantization and fused dequant-attend decode.

The compute lives in libkvq.so (HIP, gfx950) behind the C ABI of
include/kvq.h; ``kvq`` is its ctypes binding.
"""
from . import kvq  # noqa: F401
from .kvq import KVQCache, KVQError, config_from_workload, make_config  # noqa: F401
