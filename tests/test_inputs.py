"""The seeded input generators: the fast E4M3FN quantizer gives the same codes
and scales as the frexp/ldexp reference, and weights are reproducible."""
import numpy as np

import dllm_inputs as di


def test_fast_e4m3fn_quantizer_matches_reference():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((700, 512)) * 0.02).astype(np.float32)
    w[0, :6] = np.array([0.0, 1e-12, -1e-12, 0.02, -0.3, 0.3], np.float32)
    w[1] = 0.0                                           # zero row (scale 1)
    w[2] = np.linspace(-1, 1, 512, dtype=np.float32)     # every binade, ties
    # values exactly half-way between grid points after scaling (amax 448)
    w[3] = 0.0
    w[3, 0] = 448.0
    w[3, 1:9] = np.array([17.0, 19.0, 0.5 + 1 / 32, 2.0 ** -7 * 3, 2.0 ** -10, 2.0 ** -6 * 1.0625,
                          3 * 2.0 ** -10, 240.0 + 8.0], np.float32)
    c1, s1 = di.quantize_rows_e4m3fn(w, chunk_rows=64)
    c2, s2 = di.quantize_rows_e4m3fn_reference(w)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1, c2)


def test_weights_reproducible_and_expert_seeds_independent():
    m = di.workload("small_fp8").model
    a = di.make_weights(m, 4)
    b = di.make_weights(m, 4)
    for k in ("w_gate", "s_gate", "w_down", "w_qkv"):
        assert np.array_equal(a[k], b[k])
    c = di.make_weights(m, 5)
    assert not np.array_equal(a["w_gate"], c["w_gate"])
    # each expert matrix has its own stream: experts differ from each other
    assert not np.array_equal(a["w_up"][0, 0], a["w_up"][0, 1])
