"""Pins of the top-K cache-writer oracle against facts that do not come from it:
Python's own sort on tie-heavy rows, closed-form special cases and
invariances.  Each planted mistake (in the oracle, on the CPU) must fail at
least one pin."""
import numpy as np
import pytest

from oracle import topk_oracle as TO


def _brute(row, K):
    """Python's sorted() with the key (-logit, id): the definition, written out."""
    order = sorted(range(len(row)), key=lambda i: (-float(row[i]), i))[:K]
    return np.array(order, dtype=np.int32), np.array([float(row[i]) for i in order])


def pin_brute_force_ties():
    r = np.random.default_rng(11)
    for V, K in ((7, 3), (33, 5), (64, 64), (100, 17), (257, 100)):
        L = r.integers(-3, 4, size=(6, V)).astype(np.float32) * 0.5   # many ties
        ids, vals = TO.topk_select(L, K)
        for n in range(L.shape[0]):
            bi, bv = _brute(L[n], K)
            assert (ids[n] == bi).all() and (vals[n] == bv).all()


def pin_constant_row():
    L = np.full((3, 50), 1.25, dtype=np.float32)
    ids, vals = TO.topk_select(L, 10)
    assert (ids == np.arange(10)).all() and (vals == 1.25).all()


def pin_k_equals_v_is_a_full_sort():
    r = np.random.default_rng(12)
    L = r.standard_normal((4, 40)).astype(np.float32)
    ids, vals = TO.topk_select(L, 40)
    for n in range(4):
        assert sorted(ids[n].tolist()) == list(range(40))
        assert (np.diff(vals[n]) <= 0).all()
        assert (vals[n] == np.sort(L[n].astype(np.float64))[::-1]).all()


def pin_signed_zero_and_infinities():
    row = np.array([-1.0, -0.0, -np.inf, 0.0, np.inf, -0.0, 2.0], dtype=np.float32)
    ids, vals = TO.topk_select(row[None, :], 7)
    # +inf, 2, then the three zeros by id (-0.0 == +0.0), -1, -inf
    assert ids[0].tolist() == [4, 6, 1, 3, 5, 0, 2]
    assert vals[0][0] == np.inf and vals[0][-1] == -np.inf


def pin_permutation_equivariance():
    r = np.random.default_rng(13)
    V, K = 300, 20
    row = r.standard_normal(V).astype(np.float32)   # distinct with probability 1
    assert len(set(row.tolist())) == V
    perm = r.permutation(V)
    ids_a, vals_a = TO.topk_select(row[None, :], K)
    ids_b, vals_b = TO.topk_select(row[perm][None, :], K)
    assert (vals_a == vals_b).all()
    assert (perm[ids_b[0]] == ids_a[0]).all()


def pin_bf16_widening():
    # bf16 bit patterns: 1.0 = 0x3F80, 2.0 = 0x4000, -0.5 = 0xBF00, 1.0078125 = 0x3F81
    bits = np.array([[0x3F80, 0x4000, 0xBF00, 0x3F81, 0x3F80]], dtype=np.uint16)
    ids, vals = TO.topk_select(bits, 3)
    assert ids[0].tolist() == [1, 3, 0] and vals[0].tolist() == [2.0, 1.0078125, 1.0]


def pin_selected_dominate_unselected():
    r = np.random.default_rng(14)
    L = np.round(r.standard_normal((5, 500)) * 4).astype(np.float32) / 4
    ids, vals = TO.topk_select(L, 64)
    for n in range(5):
        mask = np.ones(500, bool)
        mask[ids[n]] = False
        rest = L[n][mask].astype(np.float64)
        assert vals[n].min() >= rest.max()
        # at the boundary value, every selected id is below every unselected one
        b = vals[n].min()
        sel_b = [int(i) for i, v in zip(ids[n], vals[n]) if v == b]
        uns_b = [i for i in np.nonzero(mask)[0] if L[n][i] == b]
        assert not uns_b or max(sel_b) < min(uns_b)


PINS = [pin_brute_force_ties, pin_constant_row, pin_k_equals_v_is_a_full_sort,
        pin_signed_zero_and_infinities, pin_permutation_equivariance, pin_bf16_widening,
        pin_selected_dominate_unselected]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        TO.topk_select(np.zeros((1, 4), np.float32), 5)
    with pytest.raises(ValueError):
        TO.topk_select(np.zeros((1, 4), np.float32), 0)


# planted mistakes, each in the oracle's one building block
def _mut_higher_id_wins(row):
    ids = np.arange(row.shape[0])
    return np.lexsort((-ids, -row))


def _mut_ascending(row):
    ids = np.arange(row.shape[0])
    return np.lexsort((ids, row))


def _mut_off_by_one(row):
    ids = np.arange(row.shape[0])
    o = np.lexsort((ids, -row))
    return np.concatenate([o[1:], o[:1]])


def _mut_abs(row):
    ids = np.arange(row.shape[0])
    return np.lexsort((ids, -np.abs(row)))


MUTANTS = {"higher_id_wins": _mut_higher_id_wins, "ascending": _mut_ascending,
           "rotated": _mut_off_by_one, "abs_value": _mut_abs}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    monkeypatch.setattr(TO, "_row_order", MUTANTS[name])
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant {name} passed every pin"
