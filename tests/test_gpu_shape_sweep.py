"""GPU parity over a seeded sweep of small stream shapes.

Few (head, query tile) units per compute unit is where the work split is
busiest: units cut into key ranges, pieces of one unit in several workgroups,
the merge kernel after them.  Each case draws T (log-uniform over 1 .. 1499),
the condition length, H, D, W, the number of sinks and the launch
configuration, runs the stream past the point where the window is full and
evicts, and checks every call from the first eviction on (output,
log-sum-exp, cache indices) against the oracle.
Every fourth case uses an fp8 cache (T and Lc multiples of 16, as such caches
require)."""
import numpy as np
import pytest

import synthetic
from streams import run_stream, say

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fp8 = i % 4 == 3
        D = int(rng.choice([64, 128]))
        T = int(np.exp(rng.uniform(0.0, np.log(1500.0))))  # 1 .. 1499, log-uniform
        Lc = int(rng.integers(0, 300))
        if fp8:
            T = max(16, T // 16 * 16)
            Lc = Lc // 16 * 16
        W = int(rng.integers(1, 6))
        n_sink = int(rng.integers(0, 3))
        configs = 3 if fp8 else (6 if D == 64 else 5)
        out.append(dict(name="sweep%d" % i, n_chunks=n_sink + W + 2, chunk_tokens=T, cond_len=Lc,
                        heads=int(rng.integers(1, 17)), head_dim=D, window=W, n_sink=n_sink,
                        seed=100 + i, outlier_frac=0.01, kv_dtype="fp8" if fp8 else "bf16",
                        config=int(rng.integers(0, configs))))
    return out


CASES = _cases()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kw", CASES, ids=[c["name"] for c in CASES])
def test_shape_sweep(kw):
    kw = dict(kw)
    config = kw.pop("config")
    spec = synthetic.small_spec(**kw)
    say("sweep", spec, "config", config)
    first_evict = spec.n_sink + spec.window
    run_stream(spec, range(first_evict, spec.n_chunks), config=config)
