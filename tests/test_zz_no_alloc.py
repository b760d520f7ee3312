"""The allocation-free exchange probe (kie_barrier_probe_noalloc) against the
same probe with a caller-allocated workspace (kie_barrier_probe): both must
read every exchanged value right (0 errors, an integer result compared
exactly), on two calls in a row, the second with fewer rounds, so that the
second no-alloc call starts from the array the first one left behind (the
fenced variant would pass its barriers on stale round counters if the call
did not clear them)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kie_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from memory_bandwidth_bound_amd import kie
    return kie


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_noalloc_probe_matches_workspace_probe(kie_gpu, variant):
    kie = kie_gpu
    for rounds in (3000, 400):
        print(f"variant {variant}, {rounds} rounds", flush=True)
        us_n, err_n = kie.barrier_probe_noalloc(rounds, variant)
        us_w, err_w = kie.barrier_probe(rounds, variant)
        print(f"  no-alloc {us_n:.2f} us/round, errors {err_n}; workspace {us_w:.2f} us/round, errors {err_w}",
              flush=True)
        assert err_n == err_w == 0
        assert us_n > 0 and us_w > 0
        # the same kernel: per-round times within a few times of each other
        # (the no-alloc call is host-timed, so launch latency is included)
        assert 0.2 < us_n / us_w < 5.0


def test_noalloc_probe_rejects_bad_arguments(kie_gpu):
    kie = kie_gpu
    with pytest.raises(kie.KieError) as e:
        kie.barrier_probe_noalloc(0, 1)
    assert e.value.code == -1
    with pytest.raises(kie.KieError) as e:
        kie.barrier_probe_noalloc(10, 3)
    assert e.value.code == -1
