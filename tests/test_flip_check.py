"""CPU checks of the GPU tests' code-flip proof (tests/_gpu_util.flip_explained):
rows whose codes were produced from the same h with an element moved one
fp16 ulp across a rounding boundary are accepted; codes no such move reaches
are rejected."""
import numpy as np
import pytest

from oracle import looped
from tests._gpu_util import flip_explained


def _flips(h16, group, qmax, qmin, off=None):
    """Every (moved row codes, scales) that one fp16-ulp move of one element
    produces and that differs from the row's own codes."""
    off = np.zeros(h16.shape, np.float32) if off is None else off
    q0, s0 = looped._encode_f32(h16.astype(np.float32) - off, group, qmax, qmin)
    out = []
    for i in range(h16.shape[0]):
        for d in (np.float16(np.inf), np.float16(-np.inf)):
            hm = h16.copy()
            hm[i] = np.nextafter(hm[i], d)
            q, s = looped._encode_f32(hm.astype(np.float32) - off, group, qmax, qmin)
            if not (np.array_equal(q, q0) and np.array_equal(s.view(np.uint16), s0.view(np.uint16))):
                out.append((q, s))
    return q0, s0, out


@pytest.mark.parametrize("group,qmax,qmin", [(32, 7, -8), (64, 127, -127)])
def test_one_ulp_flips_are_explained(group, qmax, qmin):
    rng = np.random.default_rng(4)
    n_found = 0
    for trial in range(300):
        # codes near rounding boundaries: h at s * (k + 0.5) within an ulp
        s = np.float16(rng.uniform(0.05, 2.0))
        k = rng.integers(qmin, qmax, size=group).astype(np.float32)
        h16 = (np.float32(s) * (k + 0.5)).astype(np.float16)
        h16[0] = np.float16(np.float32(s) * qmax)          # pins the scale
        q0, s0, flips = _flips(h16, group, qmax, qmin)
        cin = h16.astype(np.float32)
        for q, sc in flips[:4]:
            n_found += 1
            assert flip_explained(h16, cin, q, sc.view(np.uint16), q0, s0.view(np.uint16), group, qmax, qmin)
            # a code two steps from a reachable one is not: moves of at most
            # one ulp per element change a code by at most one step
            bad = q.copy()
            j = int(np.argmax(q != q0)) if np.any(q != q0) else 1
            bad[j] = bad[j] + 2 if bad[j] <= qmax - 2 else bad[j] - 2
            assert not flip_explained(h16, cin, bad, sc.view(np.uint16), q0, s0.view(np.uint16),
                                      group, qmax, qmin)
    assert n_found > 50


def test_delta_offset_flip_is_explained():
    """The delta mode codes h minus the reconstruction below: the proof moves
    h, not the coded difference."""
    rng = np.random.default_rng(9)
    found = 0
    for _ in range(200):
        h16 = (rng.standard_normal(64) * 0.3).astype(np.float16)
        below = (h16.astype(np.float32) + rng.standard_normal(64).astype(np.float32) * 0.01)
        q0, s0, flips = _flips(h16, 64, 127, -127, off=below)
        cin = h16.astype(np.float32) - below
        for q, sc in flips[:2]:
            found += 1
            assert flip_explained(h16, cin, q, sc.view(np.uint16), q0, s0.view(np.uint16), 64, 127, -127)
    assert found > 10


def test_identical_codes_pass_and_unrelated_codes_fail():
    rng = np.random.default_rng(2)
    h16 = rng.standard_normal(64).astype(np.float16)
    q, s = looped._encode_f32(h16.astype(np.float32), 32, 7, -8)
    cin = h16.astype(np.float32)
    assert flip_explained(h16, cin, q, s.view(np.uint16), q, s.view(np.uint16), 32, 7, -8)
    other = rng.standard_normal(64).astype(np.float16)
    q2, s2 = looped._encode_f32(other.astype(np.float32), 32, 7, -8)
    assert not flip_explained(h16, cin, q2, s2.view(np.uint16), q, s.view(np.uint16), 32, 7, -8)


def test_several_elements_moved_one_ulp_each():
    """FP32 and FP64 residuals can move several h elements of one group by an
    ulp each, one of them the absmax element (which moves the scale): the
    proof accepts any such combination, and no move of two ulps."""
    rng = np.random.default_rng(13)
    found = 0
    for _ in range(400):
        s = np.float16(rng.uniform(0.05, 2.0))
        k = rng.integers(-8, 7, size=32).astype(np.float32)
        h16 = (np.float32(s) * (k + 0.5)).astype(np.float16)
        h16[5] = np.float16(np.float32(s) * 7 * rng.uniform(0.999, 1.001))
        moves = rng.integers(-1, 2, size=32)
        hm = h16.copy()
        for i in np.flatnonzero(moves):
            hm[i] = np.nextafter(hm[i], np.float16(np.inf) if moves[i] > 0 else np.float16(-np.inf))
        q0, s0 = looped._encode_f32(h16.astype(np.float32), 32, 7, -8)
        q1, s1 = looped._encode_f32(hm.astype(np.float32), 32, 7, -8)
        if np.array_equal(q0, q1) and s0.view(np.uint16)[0] == s1.view(np.uint16)[0]:
            continue
        found += 1
        assert flip_explained(h16, h16.astype(np.float32), q1, s1.view(np.uint16), q0, s0.view(np.uint16), 32, 7, -8)
        # a code two steps from the moved row's is not explained
        bad = q1.copy()
        bad[9] = bad[9] + 2 if bad[9] <= 5 else bad[9] - 2
        assert not flip_explained(h16, h16.astype(np.float32), bad, s1.view(np.uint16), q0, s0.view(np.uint16),
                                  32, 7, -8)
    assert found > 50
