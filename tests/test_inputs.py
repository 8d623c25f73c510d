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


# ----------------------------------------------------------------------------
# counter-based streams (dllm_inputs.counter)
# ----------------------------------------------------------------------------

def test_philox_known_answers():
    """Philox4x32-10 against the published known-answer vectors
    (tests/golden/philox4x32_10_kat.txt)."""
    import os
    from dllm_inputs import counter as CT
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        assert r[0] == "10"
        c = [int(x, 16) for x in r[1:5]]
        k = [int(x, 16) for x in r[5:7]]
        want = [int(x, 16) for x in r[7:11]]
        got = CT.philox4x32_10(*[np.uint32(x) for x in c], k[0], k[1])
        assert [int(g) for g in got] == want


def test_counter_streams_distribution_and_independence():
    from dllm_inputs import counter as CT
    x = CT.normal(3, "w_gate", 2, 7, 1 << 20)
    assert abs(float(x.mean())) < 1e-4 and abs(float(x.std()) - 0.02) < 2e-4
    assert np.abs(x).max() <= 0.02 * 3.47                 # Irwin-Hall(4) bound
    # a window of the stream equals the same elements of the whole stream
    assert np.array_equal(CT.normal(3, "w_gate", 2, 7, 100, start=1000), x[1000:1100])
    # other experts, layers, tags, seeds: other values
    for other in (CT.normal(3, "w_gate", 2, 8, 64), CT.normal(3, "w_gate", 3, 7, 64),
                  CT.normal(3, "w_up", 2, 7, 64), CT.normal(4, "w_gate", 2, 7, 64)):
        assert not np.array_equal(other, x[:64])
    b = CT.uniform(1, "router_bias", 0, 4096, 0.1)
    assert b.min() >= -0.1 and b.max() < 0.1 and abs(float(b.mean())) < 0.01


def test_counter_weights_layout():
    from dllm_inputs import counter as CT
    m = di.workload("small_fp8").model
    w = CT.make_weights_counter(m, 2)
    ref = di.make_weights(m, 2)
    for k, v in ref.items():
        if k == "dtypes" or v is None:
            continue
        assert w[k].shape == v.shape and w[k].dtype == v.dtype, k
    sub = CT.make_weights_counter(m, 2, layers=[1])
    assert sub["w_qkv"][0] is None and np.array_equal(sub["w_qkv"][1], w["w_qkv"][1])
    assert np.array_equal(sub["s_down"][1], w["s_down"][1])
