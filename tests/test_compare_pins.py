"""Pins of the comparison metrics every parity assertion rests on.

The juejin post (§三, its numeric check) defines the two acceptance metrics
on the flattened outputs: the largest absolute difference and the cosine
similarity.  The relative L2 error, ||got - ref|| / ||ref||, is normalised
by the reference (the second argument).  Each metric is pinned here by
hand-computed values on small vectors, by the post's own torch calls on
random tensors, and by planted mistakes that must fail at least one pin:
the mean in place of the max, a missing normaliser, the norm of the first
argument in place of the reference's, a missing square root.
"""
import importlib
import math

import numpy as np
import pytest
import torch

# the package re-exports a function named compare, so take the module itself
C = importlib.import_module("oracle.compare")


# ------------------------------------------------------------------ pin sets
def _pins_max_abs_err(f):
    """Hand values: |1-1|, |-2-2|, |3-0| -> 4 (the mean would be 7/3)."""
    assert f([1.0, -2.0, 3.0], [1.0, 2.0, 0.0]) == 4.0
    assert f([0.5], [-0.25]) == 0.75
    # sign-symmetric and argument-symmetric
    assert f([1.0, 2.0], [3.0, -1.0]) == f([3.0, -1.0], [1.0, 2.0]) == 3.0
    # shape does not matter: the maximum is over every element
    a = np.zeros((2, 3, 4))
    a[1, 2, 3] = -5.0
    assert f(a, np.zeros((2, 3, 4))) == 5.0
    assert f(np.zeros(0), np.zeros(0)) == 0.0


def _pins_cosine(f):
    """Hand values: parallel 1, scaled 1, antiparallel -1, orthogonal 0,
    45 degrees 1/sqrt(2); zero-norm conventions (both zero 1, one zero 0)."""
    assert f([1.0, 2.0, 3.0], [1.0, 2.0, 3.0]) == pytest.approx(1.0, abs=1e-15)
    assert f([1.0, 2.0, 3.0], [3.0, 6.0, 9.0]) == pytest.approx(1.0, abs=1e-15)
    assert f([1.0, 2.0], [-1.0, -2.0]) == pytest.approx(-1.0, abs=1e-15)
    assert f([1.0, 0.0], [0.0, 7.0]) == 0.0
    assert f([1.0, 0.0], [1.0, 1.0]) == pytest.approx(1.0 / math.sqrt(2.0), abs=1e-15)
    # flattened over every axis: a [2, 2] pair at a known angle
    assert f([[1.0, 0.0], [0.0, 0.0]], [[1.0, 1.0], [0.0, 0.0]]) == \
        pytest.approx(1.0 / math.sqrt(2.0), abs=1e-15)
    assert f([0.0, 0.0], [0.0, 0.0]) == 1.0
    assert f([0.0, 0.0], [1.0, 0.0]) == 0.0


def _pins_rel_l2(f):
    """Hand values of ||a - b|| / ||b||: the normaliser is the reference b."""
    assert f([1.0, 1.0], [1.0, 0.0]) == pytest.approx(1.0, abs=1e-15)
    # the same pair swapped is normalised by the other vector
    assert f([1.0, 0.0], [1.0, 1.0]) == pytest.approx(1.0 / math.sqrt(2.0), abs=1e-15)
    # a 1 % scaling of the reference is a 1 % error
    b = np.array([3.0, -4.0, 12.0])
    assert f(1.01 * b, b) == pytest.approx(0.01, abs=1e-14)
    # a 3-4-5 difference over a reference of norm 13
    assert f(b + np.array([3.0, 4.0, 0.0]), b) == pytest.approx(5.0 / 13.0, abs=1e-15)
    assert f(b, b) == 0.0
    # a zero reference leaves the plain norm of the difference
    assert f([3.0, 4.0], [0.0, 0.0]) == pytest.approx(5.0, abs=1e-15)


# ------------------------------------------------------------- the real ones
def test_max_abs_err_pins():
    _pins_max_abs_err(C.max_abs_err)


def test_cosine_pins():
    _pins_cosine(C.cosine)


def test_rel_l2_pins():
    _pins_rel_l2(C.rel_l2)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_metrics_match_the_posts_torch_calls(seed):
    """The post's check: (a - b).abs().max() and cosine_similarity of the
    flattened tensors, in fp64, on random [B, S, H, D] tensors; rel-L2 against
    torch.linalg.vector_norm of the difference over that of the reference."""
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(2, 17, 3, 8, generator=g, dtype=torch.float64)
    b = a + 0.05 * torch.randn(2, 17, 3, 8, generator=g, dtype=torch.float64)
    want_max = (a - b).abs().max().item()
    want_cos = torch.nn.functional.cosine_similarity(a.flatten(), b.flatten(), dim=0).item()
    want_rel = (torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b)).item()
    assert C.max_abs_err(a, b) == want_max
    assert C.cosine(a, b) == pytest.approx(want_cos, abs=1e-14)
    assert C.rel_l2(a, b) == pytest.approx(want_rel, rel=1e-13)
    got = C.compare(a, b)
    assert got == {"max_abs_err": C.max_abs_err(a, b), "cos": C.cosine(a, b),
                   "rel_l2": C.rel_l2(a, b)}


def test_metrics_read_bf16_exactly():
    """A bf16 tensor is compared through its exact fp64 value: 1 + 2^-7 is a
    bf16 number, so its distance from 1 is exactly 2^-7."""
    a = torch.tensor([1.0 + 2.0 ** -7], dtype=torch.bfloat16)
    b = torch.tensor([1.0], dtype=torch.bfloat16)
    assert C.max_abs_err(a, b) == 2.0 ** -7
    assert C.rel_l2(a, b) == 2.0 ** -7


# ----------------------------------------------------------- planted mistakes
def _fails(pins, f):
    try:
        pins(f)
    except AssertionError:
        return True
    return False


def _v(x):
    return np.asarray(x, dtype=np.float64).ravel()


def test_planted_mistakes_fail_the_pins():
    """Each plausible slip in a metric fails at least one of its pins."""
    mean_for_max = lambda a, b: float(np.mean(np.abs(_v(a) - _v(b)))) if _v(a).size else 0.0
    signed_max = lambda a, b: float(np.max(_v(a) - _v(b))) if _v(a).size else 0.0
    assert _fails(_pins_max_abs_err, mean_for_max)
    assert _fails(_pins_max_abs_err, signed_max)

    def cos_no_norm(a, b):
        a, b = _v(a), _v(b)
        return float(a @ b)

    def cos_one_norm(a, b):
        a, b = _v(a), _v(b)
        n = np.linalg.norm(a) ** 2
        return float(a @ b / n) if n else 1.0

    assert _fails(_pins_cosine, cos_no_norm)
    assert _fails(_pins_cosine, cos_one_norm)

    def rel_norm_a(a, b):
        a, b = _v(a), _v(b)
        n = np.linalg.norm(a)
        return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))

    def rel_no_norm(a, b):
        a, b = _v(a), _v(b)
        return float(np.linalg.norm(a - b))

    def rel_no_sqrt(a, b):
        a, b = _v(a), _v(b)
        n = float(b @ b)
        return float((a - b) @ (a - b) / (n if n > 0 else 1.0))

    assert _fails(_pins_rel_l2, rel_norm_a)
    assert _fails(_pins_rel_l2, rel_no_norm)
    assert _fails(_pins_rel_l2, rel_no_sqrt)
