"""The seeded input generators (CPU only)."""
import numpy as np

from workloads import get, make_inputs, round_to_bf16, bf16_bits
from workloads.hilbert import hilbert_index, hilbert_order


def test_hilbert_index_is_a_bijection_with_unit_steps():
    for bits in (1, 2, 3, 4):
        s = 1 << bits
        t, h, w = np.meshgrid(np.arange(s), np.arange(s), np.arange(s), indexing="ij")
        idx = hilbert_index([t.ravel(), h.ravel(), w.ravel()], bits)
        assert sorted(idx.tolist()) == list(range(s ** 3))
        pts = np.stack([t.ravel(), h.ravel(), w.ravel()], 1)[np.argsort(idx)]
        steps = np.abs(np.diff(pts, axis=0)).sum(axis=1)
        assert (steps == 1).all()


def test_hilbert_order_is_a_permutation_of_the_grid():
    perm = hilbert_order((5, 6, 7))
    assert sorted(perm.tolist()) == list(range(5 * 6 * 7))


def test_round_to_bf16_ties_to_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)           # bf16 spacing at 1.0
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, -(one + ulp / 2)], np.float32)
    got = round_to_bf16(x)
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 * float(ulp), 1.0, -1.0]
    assert bf16_bits(np.array([1.0], np.float32)).tolist() == [0x3F80]


def test_generator_is_seeded_and_head_subsets_agree():
    w = get("tiny")
    a = make_inputs(w, dtype="fp32")
    b = make_inputs(w, dtype="fp32", heads=[(0, 1)])
    assert np.array_equal(a["q"][0, 1], b["q"][0, 1])
    assert not np.array_equal(a["q"][0, 0], a["q"][0, 1])
    c = make_inputs(w, dtype="bf16")
    assert np.array_equal(c["k"], round_to_bf16(a["k"]))
    assert w.N == 1024 and w.nb == 16


def test_workload_shapes():
    assert get("cogvideox").N == 17776 and get("cogvideox").nb == 139
    assert get("wan").N == 32760 and get("wan").steps == 5
    assert abs(get("wan").top_p[0] - 0.80) < 1e-12 and abs(get("wan").top_p[-1] - 0.95) < 1e-12
    assert get("hunyuan").N == 118800 and get("hunyuan").nb == 929
    assert get("dsv_train").N == 16384 and get("dsv_train").nb == 256


def test_text_prefix_and_stripes():
    w = get("cogvideox")
    x = make_inputs(w, dtype="fp32", heads=[(0, 0)])
    # text rows are plain N(0,1): no shared Fourier component between q and k
    q, k = x["q"][0, 0], x["k"][0, 0]
    assert abs(float(np.corrcoef(q[:226].ravel(), k[:226].ravel())[0, 1])) < 0.05
    assert float(np.corrcoef(q[226:].ravel(), k[226:].ravel())[0, 1]) > 0.5
