"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


def test_golden_hand_example():
    """The hand-worked two-token example in tests/golden/kda_hand_example.json."""
    import json
    import os

    import numpy as np

    import oracle

    with open(os.path.join(os.path.dirname(__file__), "golden", "kda_hand_example.json")) as f:
        g = json.load(f)
    f32 = lambda x: np.array(x, dtype=np.float32)
    la = np.log(np.array(g["alpha"], dtype=np.float64)).astype(np.float32)
    o, S = oracle.prefill(f32(g["q"]), f32(g["k"]), f32(g["v"]), f32(g["beta"]), la,
                          np.array(g["initial_state"], dtype=np.float64))
    np.testing.assert_allclose(o, np.array(g["expected_o"]), rtol=1e-6)
    np.testing.assert_allclose(S, np.array(g["expected_final_state"]), rtol=1e-6)
