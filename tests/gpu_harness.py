"""Helpers of the GPU tests: timestamped progress lines and the package's
device-side step (uploads a synthetic workload and runs the paged-KV step
through the C ABI).  Nothing here imports the oracle."""
from __future__ import annotations

import sys
import time

from paged_kv_attention_08_amd.device_step import BF16_NAN_BITS, DeviceStep, bf16_tensor, i32  # noqa: F401


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()
