"""Selection rules of the bounded-graph set (host logic, no GPU): the CPU length hints of every
live request must fit the graphs' window, the smallest capture that holds the batch wins, and
sizes the loaded library cannot serve are not captured."""
import pytest

from verify_attention_e4m3_amd import attention as A
from verify_attention_e4m3_amd.graphs import VerifyGraphs, capturable_batch_sizes, select_batch_size

CAPTURED = [1, 2, 4, 8, 16, 32]


def test_smallest_capture_that_holds_the_batch():
    assert select_batch_size(CAPTURED, 262144, [100]) == 1
    assert select_batch_size(CAPTURED, 262144, [5, 6]) == 2
    assert select_batch_size(CAPTURED, 262144, [1] * 3) == 4          # padded capture
    assert select_batch_size(CAPTURED, 262144, [1] * 9) == 16
    assert select_batch_size(CAPTURED, 262144, [1] * 32) == 32
    assert select_batch_size([8, 2], 262144, [1] * 3) == 8              # order of captures is irrelevant


def test_eager_route_cases():
    assert select_batch_size(CAPTURED, 262144, []) is None               # nothing live
    assert select_batch_size(CAPTURED, 262144, [1] * 33) is None         # beyond the largest capture
    assert select_batch_size([], 262144, [1]) is None


def test_every_hint_must_fit_the_window():
    bound = 131072
    assert select_batch_size(CAPTURED, bound, [bound, 0, 7]) == 4        # the window itself fits
    assert select_batch_size(CAPTURED, bound, [10, bound + 1, 7]) is None  # one oversized peer
    assert select_batch_size(CAPTURED, bound, [10, -1]) is None          # not a length
    assert select_batch_size(CAPTURED, bound, [0, 0]) == 2               # zero-length rows are fine


def test_capture_sizes_follow_the_library_and_the_plan():
    assert capturable_batch_sizes(CAPTURED, 256, 32) == [32, 16, 8, 4, 2, 1]   # largest first
    assert capturable_batch_sizes(CAPTURED, 1, 32) == [1]                       # a B1-only library
    assert capturable_batch_sizes(CAPTURED, 256, 8) == [8, 4, 2, 1]             # plan capacity
    assert capturable_batch_sizes([4, 4, 0, -2, 3], 256, 8) == [4, 3]


def test_loaded_library_reports_its_capacity():
    assert A.capabilities()["max_batch"] >= 32


def test_graph_set_needs_a_device_plan():
    p = A.Plan(q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=1648, max_seq_len=131072,
               batch_capacity=8)
    with pytest.raises(ValueError):
        VerifyGraphs(p, [])
