"""The box closed forms (box_map.py) against the oracle on small boxes, so
that the size-limit GPU test compares the library with something checked."""
import numpy as np
import pytest
import torch

import box_map
import oracle


@pytest.mark.parametrize("K,boxes", [
    (3, [(0, (5, 6, 7)), (1, (1, 2, 9))]),
    (3, [(2, (1, 1, 1)), (0, (3, 1, 4))]),
    (5, [(0, (4, 5, 6)), (3, (2, 7, 1))]),
    (7, [(0, (4, 8, 9)), (1, (2, 2, 5))])])
def test_box_lists_and_degrees_match_the_oracle(K, boxes):
    c = box_map.box_rows(boxes, "cpu").numpy()
    ref = oracle.build_map(c, K)
    deg = np.zeros(c.shape[0], np.int64)
    for k in range(K ** 3):
        assert box_map.offset_of(k, K) == oracle.offset_of(k, K)
        p, q = box_map.box_list(boxes, K, k, "cpu")
        ra, rb = ref.lists[k]
        assert np.array_equal(q.numpy(), rb) and np.array_equal(p.numpy(), ra), f"offset {k}"
        np.add.at(deg, rb, 1)
    assert np.array_equal(box_map.box_degree(boxes, K, "cpu").numpy(), deg)
