"""The arithmetic fact behind the local reduce's integer sums, checked on the
CPU with numpy (independently of the GPU code).

For eight peers of b-bit codes, term p of an output element's sum is
q_p * s_p with |q_p| <= qmax and s_p a binary16 scale.  When the peers'
nonzero scales of a block have binary16 exponents (1 for subnormals) within D
of each other -- D = 5 at 4 bits, 3 at 8 bits -- every partial sum of the
peer-ordered binary32 reduction is exact, so the reduction equals the exact
sum of the terms.  Beyond D it does not hold in general (shown for 8 bits).
"""
import numpy as np
import pytest

QMAX = {4: 7, 8: 127}
SPREAD = {4: 5, 8: 3}


def _f16(exp_field, frac):
    return np.array([(int(e) << 10) | int(f) for e, f in zip(exp_field, frac)],
                    np.uint16).view(np.float16).astype(np.float32)


def _sequential(q, s):
    acc = np.float32(q[0]) * s[0]
    for p in range(1, len(q)):
        acc = np.float32(acc + np.float32(q[p]) * s[p])
    return acc


def _exact(q, s):
    return sum(float(qi) * float(si) for qi, si in zip(q, s))


@pytest.mark.parametrize("bits", [4, 8])
def test_sequential_sum_is_exact_within_spread(bits):
    g = np.random.default_rng(bits)
    qmax, D = QMAX[bits], SPREAD[bits]
    for trial in range(20000):
        lo = int(g.integers(0, 31 - D))            # exponent field of the smallest scale
        e = lo + g.integers(0, D + 1, 8)
        e[g.integers(0, 8)] = lo
        frac = g.integers(0, 1024, 8)
        if trial % 4 == 0:                          # worst magnitudes
            frac[:] = 1023
            e[:] = lo + D
            e[0] = lo
        s = _f16(e, frac)
        s[g.random(8) < 0.1] = 0.0                  # some all-zero peer blocks
        q = g.integers(-qmax, qmax + 1, 8)
        if trial % 3 == 0:
            q = np.where(g.random(8) < 0.5, qmax, -qmax)
        assert float(_sequential(q, s)) == _exact(q, s)


def test_beyond_the_spread_a_sum_rounds():
    """8-bit codes with exponents 4 apart (one past the limit): five peers at
    the largest scale and code take the partial sum past 2^24 units of the
    smallest scale, and a sixth term of one odd unit then rounds."""
    lo = 10
    s = _f16([lo + 4] * 5 + [lo, lo, lo], [1023] * 5 + [1, 0, 0])
    q = np.array([127] * 5 + [1, 0, 0])
    assert float(_sequential(q, s)) != _exact(q, s)
    # the same terms with exponents only 3 apart stay exact
    s3 = _f16([lo + 3] * 5 + [lo, lo, lo], [1023] * 5 + [1, 0, 0])
    assert float(_sequential(q, s3)) == _exact(q, s3)
