"""The seeded input generator: determinism, shapes and the uniform/bf16 formats."""
import numpy as np

import workloads


def test_configs_shapes_small_overrides():
    for name in ("c1", "c2", "c3", "c4"):
        cfg = workloads.get_config(name, V=257, B=3)
        a = workloads.generate(cfg)
        b = workloads.generate(cfg)
        for key in a:
            assert np.array_equal(a[key], b[key]), key
        assert a["draft_probs"].shape == (3, cfg.R, 257)
        assert a["target"].shape == (3, cfg.N, 257)
        if cfg.mode == "stochastic":
            assert np.allclose(a["target"].sum(-1), 1, atol=1e-5)
            for u in (a["u_accept"], a["u_draw"]):
                kk = u.astype(np.float64) * 2 ** 24
                assert (kk == np.floor(kk)).all() and (kk >= 0).all() and (kk < 2 ** 24).all()
        if cfg.has_attention:
            assert a["q"].dtype == np.uint16 and a["q"].shape == (3, cfg.N, cfg.Hq, cfg.D)
            P = cfg.page
            tab = a["page_table"]
            used = []
            for r in range(3):
                n = (int(a["prefix_len"][r]) + cfg.N + P - 1) // P
                assert (tab[r, :n] >= 0).all() and (tab[r, n:] == -1).all()
                used += tab[r, :n].tolist()
            assert len(set(used)) == len(used)
            assert a["k_pool"].shape[0] >= (max(used) + 1) * P


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    b = workloads.to_bf16_bits(x)
    back = workloads.bf16_bits_to_f32(b)
    assert back.tolist()[:4] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]


def test_pool_and_row_counts():
    assert workloads.num_draft_rows(8, 5) == 33 and workloads.pool_size(8, 5) == 264
    assert workloads.num_draft_rows(4, 4) == 13 and workloads.pool_size(4, 4) == 52
    assert workloads.pool_size(1, 4) == 4
