"""Pins for oracle.route: bucket boundaries by hand."""
import pytest

from oracle import route


def test_buckets_20_steps():
    # 20 sampler steps over 10 equal intervals: two steps per bucket
    assert [route.bucket(s, 20) for s in range(20)] == [s // 2 for s in range(20)]


def test_buckets_short_and_long_schedules():
    assert [route.bucket(s, 4) for s in range(4)] == [0, 2, 5, 7]
    assert route.bucket(0, 1) == 0
    assert route.bucket(999, 1000) == 9 and route.bucket(100, 1000) == 1
    with pytest.raises(ValueError):
        route.bucket(5, 5)


def test_table_lookup():
    table = [1] * 10 + [2] * 5 + [3] * 5
    assert route.act_format(table, 10, 1, 0, 20) == 2
    assert route.act_format(table, 10, 1, 19, 20) == 3
    assert route.act_format(table, 10, 0, 7, 20) == 1
