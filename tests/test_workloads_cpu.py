"""The block-mask generators of workloads.py against their definitions."""
import numpy as np

import workloads


def test_dilated_block_mask():
    for n_q, n_k, r, w, causal in ((1024, 1024, 2, 3, True), (512, 700, 3, 1, False), (16384, 16384, 2, 64, True),
                                   (300, 5000, 4, 10, False), (128, 64, 1, 0, True)):
        m = workloads.dilated_block_mask(n_q, n_k, r, w, causal)
        n_qb, n_kb = -(-n_q // 128), -(-n_k // 64)
        assert m.shape == (n_qb, n_kb) and m.dtype == np.uint8
        for qb in range(n_qb):
            k0, k1 = 2 * qb, 2 * qb + 1  # 128 rows = two 64-key blocks
            want = set(range(k0, min(k1, n_kb - 1) + 1))
            want |= {k0 - r * t for t in range(1, w + 1) if k0 - r * t >= 0}
            if not causal:
                want |= {k1 + r * t for t in range(1, w + 1) if k1 + r * t < n_kb}
            assert set(np.flatnonzero(m[qb]).tolist()) == want, (n_q, n_k, r, w, causal, qb)


def test_random_block_mask_is_seeded():
    a = workloads.random_block_mask((2, 3, 4, 5), 0.3, 7)
    assert np.array_equal(a, workloads.random_block_mask((2, 3, 4, 5), 0.3, 7)) and a.dtype == np.uint8
    assert set(np.unique(a).tolist()) <= {0, 1}
