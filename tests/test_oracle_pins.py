"""The CPU oracle against its pins (CPU only; see oracle_checks for what pins what)."""
import numpy as np
import pytest

import oracle
import oracle_checks as oc


def test_golden_worked_examples(orc):
    oc.check_golden(orc)


@pytest.mark.slow
@pytest.mark.parametrize("wire", [oc.BF16, oc.F16], ids=["bf16", "f16"])
def test_round_exhaustive_vs_torch(orc, wire):
    oc.check_round_exhaustive(orc, wire)


def test_round_f16_vs_numpy_sample(orc):
    oc.check_round_f16_numpy_sample(orc)


def test_widen_exhaustive(orc):
    oc.check_widen_exhaustive(orc)


def test_add_matches_fp64_route_and_numpy(orc):
    oc.check_add_theorem(orc)


@pytest.mark.parametrize("R", [2, 3])
def test_fold_bruteforce_edge_grid(orc, R):
    oc.check_fold_bruteforce(orc, R)


def test_fold_bruteforce_r4_subgrid(orc):
    g = oc._edge_grid()[::2]
    oc.check_fold_bruteforce(orc, 4, grid=g)


def test_ordered_sum(orc):
    oc.check_ordered_sum(orc)


def test_closed_form(orc):
    oc.check_closed_form(orc)


def test_order_sensitivity(orc):
    oc.check_order_sensitivity(orc)


def test_broadcast_and_wire_typed_sources(orc):
    oc.check_broadcast_and_wire_srcs(orc)


def test_inactive_ranks(orc):
    oc.check_inactive_ranks(orc)


def test_empty_and_single_element(orc):
    z = np.zeros(0, dtype=np.float32)
    assert oracle.reduce([z, z], oracle.BF16, lib=orc).shape == (1, 0)
    one = np.array([1.5], dtype=np.float32)
    assert oracle.reduce([one, one], oracle.F16, lib=orc)[0, 0] == np.float32(3.0)


def test_rejects_mismatched_source_type(orc):
    a = np.zeros(4, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.reduce([a, a], oracle.BF16, src_type=oracle.F16, lib=orc)


def test_residual(orc):
    oc.check_residual(orc)


def test_narrow_destinations(orc):
    oc.check_narrow_dst(orc)


def test_rejects_undefined_residual_and_narrow_combinations(orc):
    a = np.ones(12, dtype=np.float32)
    with pytest.raises(ValueError):      # residual length must divide n
        oracle.reduce([a, a], oracle.BF16, residual=np.ones(5, dtype=np.float32), lib=orc)
    with pytest.raises(ValueError):      # a narrow destination needs the same wire type
        oracle.reduce([a, a], oracle.BF16, dst_type=oracle.F16, lib=orc)
    h = np.zeros(12, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.reduce([h, h], oracle.BF16, src_type=oracle.BF16, dst_type=oracle.F16, lib=orc)
    with pytest.raises(TypeError):       # residual of the wrong type
        oracle.reduce([h, h], oracle.F16, src_type=oracle.F16, dst_type=oracle.F16,
                      residual=np.ones(12, dtype=np.float32), lib=orc)


def test_row_strided(orc):
    oc.check_rows(orc)
