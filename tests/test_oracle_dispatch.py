"""Pins of the oracle's Dispatch rule ([LoKA] section III-C, "Library and
Recipe Selection": filter by MERE < 0.2 and speedup > 1.05x, then take the
highest measured throughput) on hand-built candidate tables whose answer
follows from the pages' sentence alone: each pin isolates one clause, so a
dropped filter, a flipped comparison or a max taken over the wrong quantity
fails one of them."""

import math

from oracle import dispatch


def test_fastest_of_the_eligible():
    # all pass both filters: the shortest time wins
    assert dispatch.select([(8.0, 0.01), (6.0, 0.05), (7.0, 0.001)], baseline_us=10.0) == 1


def test_accuracy_filter_excludes_the_fastest():
    # the fastest has MERE 0.3 > 0.2: the next fastest eligible one is chosen
    assert dispatch.select([(5.0, 0.3), (6.0, 0.1), (9.0, 0.01)], baseline_us=10.0) == 1


def test_speedup_filter():
    # 10 / 9.6 = 1.042 < 1.05: no candidate is fast enough, stay on the baseline
    assert dispatch.select([(9.6, 0.0), (9.9, 0.0)], baseline_us=10.0) == -1
    # 10 / 9.5 = 1.0526 > 1.05
    assert dispatch.select([(9.6, 0.0), (9.5, 0.0)], baseline_us=10.0) == 1


def test_thresholds_are_strict():
    # MERE exactly at the threshold, speedup exactly at the factor: both fail
    assert dispatch.select([(5.0, 0.2)], baseline_us=10.0) == -1
    assert dispatch.select([(8.0, 0.0)], baseline_us=8.4) == -1  # 1.05 exactly
    assert dispatch.select([(8.0, 0.0)], baseline_us=8.41) == 0


def test_accuracy_before_speed_not_a_tradeoff():
    # a very fast but inaccurate recipe never wins over an accurate slower one,
    # and there is no weighting between error and time
    assert dispatch.select([(1.0, 0.21), (9.0, 0.19)], baseline_us=10.0) == 1
    assert dispatch.select([(1.0, 0.21)], baseline_us=10.0) == -1


def test_ties_and_non_finite():
    assert dispatch.select([(6.0, 0.1), (6.0, 0.0)], baseline_us=10.0) == 0
    assert dispatch.select([(math.nan, 0.0), (7.0, math.inf), (0.0, 0.0), (8.0, 0.0)], baseline_us=10.0) == 3
    assert dispatch.select([], baseline_us=10.0) == -1


def test_custom_thresholds():
    assert dispatch.select([(5.0, 0.3)], baseline_us=10.0, mere_max=0.5) == 0
    assert dispatch.select([(9.0, 0.0)], baseline_us=10.0, min_speedup=1.2) == -1
