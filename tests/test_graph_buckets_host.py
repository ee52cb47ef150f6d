"""Host logic of the decode-batch graph buckets (no GPU: bucket choice only)."""
import pytest

from weight_quantized_linear_qlinear_amd.graphs import DEFAULT_BUCKETS, GraphBuckets


def _buckets(sizes):
    gb = object.__new__(GraphBuckets)            # no capture: only the size logic
    gb.buckets = tuple(sorted(set(sizes)))
    return gb


def test_default_buckets_are_powers_of_two_up_to_512():
    assert DEFAULT_BUCKETS == tuple(2 ** i for i in range(10))


@pytest.mark.parametrize("M,b", [(1, 1), (2, 2), (3, 4), (5, 8), (13, 16), (16, 16), (17, 32), (100, 128),
                                 (300, 512), (512, 512)])
def test_smallest_bucket_that_holds_the_batch(M, b):
    assert _buckets(DEFAULT_BUCKETS).bucket_for(M) == b


def test_batches_above_the_largest_bucket_are_rejected():
    with pytest.raises(ValueError):
        _buckets(DEFAULT_BUCKETS).bucket_for(513)
    assert _buckets([3, 48]).bucket_for(4) == 48
