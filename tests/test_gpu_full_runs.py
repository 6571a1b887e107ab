"""GPU: whole-run lockstep parity, each workload for its full length (the runner and its protocol:
tests/full_length_parity.py).  About a minute in all on an MI355X."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoding_step_amd import _native
    _native.load()


@pytest.mark.parametrize("name", ["tiny_threshold_f32", "threshold_b1_l32", "credit_b1_l32",
                                  "hierarchical_b1_l64", "mixed_b16_l32"])
def test_full_run_in_lockstep(name):
    from full_length_parity import run
    run(name)
