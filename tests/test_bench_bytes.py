"""The bench's algorithmic byte count (CPU): weights + KV a layer step must move, against the
count written out here term by term for the configurations whose shapes the pages fix."""

import numpy as np
import pytest

import bench


class _W:
    def __init__(self, b, q_rows=8, dense_inter=0):
        self.b, self.q_rows, self.dense_inter = b, q_rows, dense_inter


def _wk(H, Hq, Hkv, D, E, I, b, lens, window=0):
    import torch
    dims = dict(hidden=H, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_experts=E, inter=I)
    lay = dict(seq_lens=torch.tensor(lens, dtype=torch.int32), window=window)
    return dict(dims=dims, workload=_W(b), layers=[lay])


def test_layer_step_bytes_at_the_8k_shape():
    H, Hq, Hkv, D, E, I, b, L = 4096, 32, 8, 128, 32, 1536, 8, 8192
    counts = np.zeros(E, dtype=np.int64)
    counts[:19] = 1                                   # 19 touched experts
    total, experts = bench.algorithmic_bytes(_wk(H, Hq, Hkv, D, E, I, b, [L]), [counts])
    w_qkv = (2 * Hq + 2 * Hkv) * D * H * 2            # bf16 [q | k | v | gate, H]
    w_o = H * Hq * D * 2
    w_r = E * H * 2
    gains = 4 * H * 4
    expert = 3 * H * I // 2 + 3 * H * I // 16 + 8    # E2M1 codes, E4M3 scales, 2 fp32 gscales
    kv = L * Hkv * D * 2 * 2 + b * Hkv * D * 2 * 2   # K and V read (bf16) + the new rows written
    assert experts == 19 * expert
    assert total == w_qkv + w_o + w_r + gains + 19 * expert + kv
    assert total == 353075352


@pytest.mark.parametrize("window", [100, 4096])
def test_window_limits_the_kv_bytes(window):
    H, Hq, Hkv, D, E, I, b, L = 4096, 32, 8, 128, 32, 1536, 8, 8192
    counts = np.ones(E, dtype=np.int64)
    full, _ = bench.algorithmic_bytes(_wk(H, Hq, Hkv, D, E, I, b, [L]), [counts])
    win, _ = bench.algorithmic_bytes(_wk(H, Hq, Hkv, D, E, I, b, [L], window), [counts])
    seen = min(L, window + 8 - 1)                    # the rows see the last w + q - 1 tokens
    assert full - win == (L - seen) * Hkv * D * 2 * 2


def test_untouched_experts_cost_nothing():
    H, Hq, Hkv, D, E, I, b = 256, 4, 1, 64, 8, 128, 8
    zero = np.zeros(E, dtype=np.int64)
    one = zero.copy()
    one[3] = 2
    a, _ = bench.algorithmic_bytes(_wk(H, Hq, Hkv, D, E, I, b, [128]), [zero])
    c, e = bench.algorithmic_bytes(_wk(H, Hq, Hkv, D, E, I, b, [128]), [one])
    assert c - a == e == 3 * H * I * (0.5 + 1.0 / 16) + 8


def test_rotation_copies_divide_the_timed_steps():
    from bench import rotation_copies
    step = 353.1e6
    assert rotation_copies(20, step) == (10, 0)      # 20 steps: ten copies, whole replays only
    assert rotation_copies(200, step) == (8, 0)
    assert rotation_copies(5, step) == (5, 0)        # fewer steps than the usual copies
    assert rotation_copies(1, step) == (1, 0)
    assert rotation_copies(37, step) == (8, 5)       # no divisor in range: one remainder graph
    assert rotation_copies(24, 0.9e6) == (24, 0)     # a tiny step: 16..32 copies
    for K in range(1, 120):
        R, rest = rotation_copies(K, step)
        assert 1 <= R <= 32 and rest == K % R
        assert rest == 0 or K > 32
