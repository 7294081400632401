"""The CPU oracle against its pins (no GPU needed)."""
import json
import os

import numpy as np
import pytest

import synth
from tests import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__[4:])
def test_oracle_pin(orc, pin):
    pin(orc)


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")


def test_page_shape_constants():
    """The gate+up shapes and chunk counts printed on the pages match the workloads."""
    with open(GOLDEN) as f:
        g = json.load(f)
    for case in g["bf16_gateup"]:
        rows, k = case["rows"], case["k"]
        assert k * 2 // 16 == case["row_chunks_16B"]  # a row of bf16 in 16-byte chunks of 8 values
        assert rows - 1 == case["last_row_index"]
    ops = synth.q8_stack_08b()
    gateup = [o for o in ops if o.name.endswith("gateup")]
    hidden_case = g["bf16_gateup"][0]
    assert all(o.n == hidden_case["rows"] and o.k == hidden_case["k"] for o in gateup)
    assert len(ops) == 24 * 4 + 1


def test_decode_intensity_about_two_ops_per_byte():
    """A decode step touches each weight once, two flops per weight (Phobos, Fast Decode):
    with 1-byte codes plus a 2-byte scale per 32, the ratio sits just under 2."""
    n, k = 7168, 1024
    ops_per_byte = 2 * n * k / synth.q8_gemv_bytes(n, k)
    assert 1.8 < ops_per_byte < 2.0
    with open(GOLDEN) as f:
        g = json.load(f)
    assert g["decode_ops_per_byte"]["value"] == 2


def test_generator_is_seeded_and_shaped():
    a = synth.q8_weights(synth.rng_for(0, 0), 8, 64)
    b = synth.q8_weights(synth.rng_for(0, 0), 8, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert a[0].dtype == np.int8 and a[0].min() >= -127 and a[1].shape == (8, 2)
    c = synth.q8_weights(synth.rng_for(0, 1), 8, 64)
    assert not np.array_equal(a[0], c[0])
