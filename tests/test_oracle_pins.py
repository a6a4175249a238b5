"""The fp64 oracle against its pins (format definitions, library routines,
brute force, closed forms, invariants).  CPU only."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_bad_block_id_is_an_error(orc):
    import oracle

    p = pins.tiny_problem(seed=20, lens=(5, 9, 2))
    p["bt"][1, 1] = 10_000  # needed by token 4..7 of sequence 1
    with pytest.raises(oracle.OracleError):
        pins.run(orc, p)


def test_units_subset_matches_full(orc):
    p = pins.tiny_problem(seed=21, lens=(7, 30, 11))
    full = pins.run(orc, p)
    units = [(2, 1), (0, 0), (1, 1)]
    sub = pins.run(orc, p, units=units)
    for i, (s, h) in enumerate(units):
        assert (sub[i] == full[s, h * 4:(h + 1) * 4]).all()


def test_threads_do_not_change_bits(orc):
    p = pins.tiny_problem(seed=22, lens=(70, 3, 41), S=3)
    assert (pins.run(orc, p, nthreads=1) == pins.run(orc, p, nthreads=5)).all()
