"""Self-checks of the seeded input generators (CPU)."""
import kvsynth


def test_stress_isotropic_tokens_are_the_worst_covered():
    """Adversarial workload at full size (65536 tokens, 8 heads): the isotropic
    5 % of the keys are the tokens least covered by a dictionary of the keys
    themselves (every 128th token): at least 99 % of them rank among the |iso|
    lowest largest-cosines of their head, and their share is about 5 %."""
    w = kvsynth.WORKLOADS["stress_64k"]
    for h, d in enumerate(kvsynth.stress_isotropic_check(w, seq=0, layer=0)):
        assert abs(d["iso"] / w.n_tokens - 0.05) < 0.005, (h, d)
        assert d["frac_lowest"] >= 0.99, (h, d)
        assert d["iso_max"] < 0.5, (h, d)


def test_generators_are_deterministic():
    w = kvsynth.WORKLOADS["tiny_f32"]
    a = kvsynth.unit_inputs(w, 0, 0)
    b = kvsynth.unit_inputs(w, 0, 0)
    for x, y in zip(a, b):
        assert (x == y).all()
    assert (kvsynth.decode_queries(w, 3) == kvsynth.decode_queries(w, 3)).all()
