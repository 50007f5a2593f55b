"""fp64 CPU oracle for the paged-KV attention step.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline import this package.  The GPU library never does.
"""
from .pagedkv_oracle import *  # noqa: F401,F403
from .pagedkv_oracle import KVPool, store_kv, build_metadata, paged_attention, attend, softmax  # noqa: F401
