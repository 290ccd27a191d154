"""Exact pins of the oracle's stochastic-rounding generator (CPU).

The generator is a reading (the pages name stochastic rounding but no
generator): the MurmurHash3 32-bit finaliser keyed by the seed and applied to
the global element index, the top 24 bits giving the uniform.  The published
MurmurHash3 vectors pin the finaliser (``test_oracle_formats.py``); the
hand-worked values in ``golden/sr_generator_vectors.txt`` pin how the seed and
the index are fed to it and which bits become the uniform.  A planted mistake
in any of those three choices, made in a copy of the oracle, fails them.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sr_generator_vectors.txt")
ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                          "lowbit_oracle.c")


def _vectors():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = (s.strip() for s in line.split("="))
        kind, *args = lhs.split()
        out.append((kind, [int(a, 0) for a in args], rhs))
    return out


VECTORS = _vectors()


def _mismatches(fmix32, key, bits, uniform):
    """Golden vectors the given generator functions do not reproduce."""
    bad = []
    for kind, args, rhs in VECTORS:
        if kind == "fmix32":
            ok = fmix32(*args) == int(rhs, 0)
        elif kind == "key":
            ok = key(*args) == int(rhs, 0)
        elif kind == "hash":
            ok = bits(*args) == int(rhs, 0)
        else:
            ok = f"{uniform(*args):.8f}" == rhs
        if not ok:
            bad.append((kind, args, rhs))
    return bad


def test_vector_file_is_complete():
    kinds = [k for k, _, _ in VECTORS]
    assert kinds.count("key") == 3 and kinds.count("hash") == 10 and kinds.count("uniform") == 10
    # the printed uniforms are the top 24 bits of the printed hashes
    h = {tuple(a): int(r, 0) for k, a, r in VECTORS if k == "hash"}
    for k, a, r in VECTORS:
        if k == "uniform":
            assert f"{(h[tuple(a)] >> 8) / 16777216:.8f}" == r


def test_oracle_generator_vectors(oracle_mod):
    L = oracle_mod.lib()
    bad = _mismatches(lambda x: int(L.oracle_fmix32(x)), lambda s: int(L.oracle_sr_key(s)),
                      lambda s, i: int(L.oracle_sr_bits(s, i)),
                      lambda s, i: float(L.oracle_sr_uniform(s, i)))
    assert bad == []
    # the array entry point the codec tests use gives the same uniforms
    r = oracle_mod.sr_uniform(42, 0, 8)
    want = [rhs for k, a, rhs in VECTORS if k == "uniform" and a[1] < 8]
    assert [f"{v:.8f}" for v in r] == want


def test_sr_worked_example_from_printed_uniforms(oracle_mod):
    """The 4-bit SR worked case (scale 0.5, inv 2) recomputed from the printed
    uniforms rather than from the oracle's generator."""
    x = np.array([0.3, -0.3, 1.75, -2.6, 3.5, 0.0, -3.5, 1.0], np.float32)
    h = {a[1]: int(rhs, 0) for k, a, rhs in VECTORS if k == "hash" and a[0] == 42}
    r = np.array([np.float32(h[i] >> 8) * np.float32(2.0 ** -24) for i in range(8)], np.float32)
    v = x * np.float32(2.0)
    q = np.clip(np.floor((v + r).astype(np.float32)), -7, 7).astype(np.int64)
    assert list(q) == [0, -1, 4, -6, 7, 0, -7, 2]
    word = sum(int(u) << (4 * j) for j, u in enumerate(q + 8))
    assert word == 0xA18F2C78
    codes, scales = oracle_mod.quantize_pack(x, 4, 128, stochastic=True, seed=42)
    assert int(codes[0]) == word and int(scales[0]) == 0x3800


def _oracle_cflags():
    from oracle import oracle as impl
    return impl.CFLAGS


# (original text in the oracle, planted mistake)
PLANTED = {
    "index halves swapped": ("return oracle_fmix32(lo ^ oracle_fmix32(hi ^ key));",
                             "return oracle_fmix32(hi ^ oracle_fmix32(lo ^ key));"),
    "seed halves swapped": ("return oracle_fmix32(lo ^ oracle_fmix32(hi ^ 0x9E3779B9u));",
                            "return oracle_fmix32(hi ^ oracle_fmix32(lo ^ 0x9E3779B9u));"),
    "low 24 bits as the uniform": ("return (float)(h >> 8) * (1.0f / 16777216.0f);",
                                   "return (float)(h & 0xFFFFFFu) * (1.0f / 16777216.0f);"),
    "seed constant dropped": ("oracle_fmix32(hi ^ 0x9E3779B9u)", "oracle_fmix32(hi)"),
    "key outside the inner hash": ("oracle_fmix32(hi ^ key)", "(oracle_fmix32(hi) ^ key)"),
    "key not applied": ("oracle_fmix32(lo ^ oracle_fmix32(hi ^ key))",
                        "oracle_fmix32(lo ^ oracle_fmix32(hi))"),
    "finaliser shift 13 -> 15": ("h ^= h >> 13;", "h ^= h >> 15;"),
}


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_generator_mistake_is_caught(oracle_mod, tmp_path, name):
    old, new = PLANTED[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"the oracle no longer contains {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", *_oracle_cflags(), "-o", str(so), str(path), "-lm"])
    M = ctypes.CDLL(str(so))
    u32, u64 = ctypes.c_uint32, ctypes.c_uint64
    for fn, res, args in (("oracle_fmix32", u32, [u32]), ("oracle_sr_key", u32, [u64]),
                          ("oracle_sr_bits", u32, [u64, u64]),
                          ("oracle_sr_uniform", ctypes.c_float, [u64, u64])):
        getattr(M, fn).restype = res
        getattr(M, fn).argtypes = args
    bad = _mismatches(lambda x: int(M.oracle_fmix32(x)), lambda s: int(M.oracle_sr_key(s)),
                      lambda s, i: int(M.oracle_sr_bits(s, i)),
                      lambda s, i: float(M.oracle_sr_uniform(s, i)))
    assert bad, f"planted mistake '{name}' reproduces every vector"
