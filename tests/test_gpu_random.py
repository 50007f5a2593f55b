"""GPU parity on seeded random batches: head groupings, KV head counts, page
sizes, decode / extend mixes, padding requests and lengths drawn at random
(sizes the oracle finishes in seconds), each through the whole step and the
same checks as the fixed cases (bit-exact metadata and store, whole pool,
plan coverage, the attention bar), once with metadata and store as two calls
and once as one."""
import numpy as np
import pytest

from tests.gpu_harness import log
from tests.test_gpu_parity import run_case
from workloads import RequestSpec, build_workload

pytestmark = pytest.mark.gpu

N_CASES = 16


def random_workload(seed: int):
    """A random batch: decode requests first (some of them padding, at the
    end of the decode part), then extend requests (some a pure prefill)."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    page = int(rng.choice([1, 2, 16, 32, 64]))
    n_dec = int(rng.integers(0, 9))
    n_pad = int(rng.integers(0, 3)) if n_dec else 0
    n_ext = int(rng.integers(0 if n_dec else 1, 4))
    reqs = []
    for _ in range(n_dec):
        c = int(rng.integers(0, 700))
        reqs.append(RequestSpec(c, c + 1))
    reqs += [RequestSpec(0, 1, padding=True) for _ in range(n_pad)]
    for _ in range(n_ext):
        c = int(rng.integers(0, 300)) if rng.random() < 0.75 else 0
        reqs.append(RequestSpec(c, c + int(rng.integers(1, 200))))
    rows_needed = sum(-(-r.device_len // page) + 1 for r in reqs) * page
    pool = max(64 * page, 1 << int(np.ceil(np.log2(rows_needed * 2 + 4 * page))))
    w = build_workload(f"random{seed}", 9000 + seed, reqs, num_qo_heads=hkv * group, num_kv_heads=hkv,
                       head_dim=128, page_size=page, num_pool_rows=pool, num_decode=n_dec + n_pad)
    return w


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "one_call"])
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_batch(seed, fused):
    w = random_workload(seed)
    log(f"random batch {seed}: {w.summary()}")
    ds, _, _ = run_case(w, label=f"random{seed}", fused_store=fused)
    ds.free()
