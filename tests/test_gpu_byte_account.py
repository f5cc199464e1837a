"""The byte account, the sweep's latency model, the measured crossing and the
latency gate through the C ABI, against the oracle, in the GPU suite ("Where
Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding", §3.3
"Crossover Length and Speedup Bounds" with its "Dispatch and batching"
paragraph, §4.3 "Locating the Crossing").  The calls are host-only; running
them here checks the library build that the GPU runs and the benchmark reads."""

import pytest

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd", reason="libsd.so not built")

import account_cases as ac  # noqa: E402


def _dims():
    return sd.make_dims(**ac.DIMS8B, w_dtype=sd.SD_BF16, kv_dtype=sd.SD_BF16)


@pytest.mark.parametrize("proj,code", ac.PROJ)
@pytest.mark.parametrize("point", ac.POINTS)
@pytest.mark.parametrize("latency", ac.LATENCY)
def test_byte_account(proj, code, point, latency):
    ac.check_account(sd, _dims(), proj, code, point, latency)


@pytest.mark.parametrize("proj,code", ac.PROJ)
@pytest.mark.parametrize("case", ac.BATCH)
def test_byte_crossover_batch(proj, code, case):
    ac.check_batched(sd, _dims(), proj, code, case)


@pytest.mark.parametrize("seed", range(4))
def test_latency_fit_and_crossing(seed):
    ac.check_sweep(sd, seed)


@pytest.mark.parametrize("seed", range(3))
def test_latency_gate(seed):
    ac.check_gate(sd, seed)
