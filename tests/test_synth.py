"""The seeded input generator: determinism and the stated recipe (CPU only)."""
import numpy as np
import pytest

from sparse_attention_decode_page_amd import synth as S


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    got = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0], dtype=np.float32)
    assert np.array_equal(got, want)


def _small_spec():
    return S.custom_spec(batch=3, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, dtype="bf16",
                         lens=("list", [100, 16, 1]), budget=("tokens", 64), outlier_channels=4)


def test_same_seed_same_arrays_other_seed_differs():
    a = S.make_workload(_small_spec(), seed=3)
    b = S.make_workload(_small_spec(), seed=3)
    c = S.make_workload(_small_spec(), seed=4)
    for f in ("q", "page_table", "k_pool", "v_pool", "lens", "budget_pages"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert not np.array_equal(a.q, c.q)
    assert not np.array_equal(a.k_pool, c.k_pool)


def test_pool_layout_matches_unit_draws_and_poison():
    wl = S.make_workload(_small_spec(), seed=0, headroom=8)
    ps = wl.spec.page_size
    for b in range(wl.spec.batch):
        for g in range(wl.spec.num_kv_heads):
            kt, vt = S.unit_tokens(wl, b, g)
            for t in range(int(wl.lens[b])):
                phys = wl.page_table[b, t // ps]
                assert np.array_equal(wl.k_pool[phys, g, t % ps], kt[t])
                assert np.array_equal(wl.v_pool[phys, g, t % ps], vt[t])
        L = int(wl.lens[b])
        if L % ps:
            phys = wl.page_table[b, L // ps]
            tail = S.bf16_bits_to_f32(wl.k_pool[phys, :, L % ps:])
            assert np.all(tail == S.POISON)
    used = wl.page_table[wl.page_table >= 0]
    assert len(np.unique(used)) == len(used) == wl.num_phys


def test_unit_prefix_property():
    wl = S.make_workload(_small_spec(), seed=0, build_pool=False)
    k1, v1 = S.unit_tokens(wl, 0, 1)
    k2, v2 = S.unit_tokens(wl, 0, 1, n=150)
    assert np.array_equal(k2[:100], k1) and np.array_equal(v2[:100], v1)


def test_outlier_channels_scaled():
    wl = S.make_workload(_small_spec(), seed=0, build_pool=False)
    k, v = S.unit_tokens(wl, 0, 0, n=4000)
    k = S.bf16_bits_to_f32(k)
    ch = wl.outliers[0]
    assert len(set(ch.tolist())) == 4
    others = np.setdiff1d(np.arange(64), ch)
    assert 6.5 < k[:, ch].std() < 9.5 and 0.9 < k[:, others].std() < 1.1
    assert 0.9 < S.bf16_bits_to_f32(v).std() < 1.1


def test_ragged_lengths_and_budget_schedule():
    spec = S.SPECS["qwen3-8b-ragged"]
    wl = S.make_workload(spec, seed=0, build_pool=False)
    assert wl.lens.min() >= 8192 and wl.lens.max() <= 32768
    tok = S.budget_tokens(spec, np.array([8192, 32768, 20480]))
    assert tok.tolist() == [1024, 4096, 1024 + 3072 * 12288 // 24576]
    assert np.array_equal(wl.budget_pages, (S.budget_tokens(spec, wl.lens) // 16).astype(np.int32))
    assert wl.budget_pages.min() >= 64 and wl.budget_pages.max() <= 256


def test_planted_block_position_and_sign():
    spec = S.custom_spec(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=32, page_size=16, dtype="bf16",
                         lens=("fixed", 1024), budget=("tokens", 256), planted_block=64)
    wl = S.make_workload(spec, seed=5, build_pool=False)
    q = S.bf16_bits_to_f32(wl.q)
    for b in range(2):
        for g in range(2):
            s0 = wl.plant_start[b, g]
            assert 64 <= s0 <= 1024 - 128
            k = S.bf16_bits_to_f32(S.unit_tokens(wl, b, g)[0])
            sign = np.sign(q[b, 4 * g:4 * g + 4].sum(axis=0))
            assert np.all(np.sign(k[s0:s0 + 64].mean(axis=0)) == sign)
            assert np.abs(k[s0:s0 + 64]).mean() > 6


def test_heavy_rows_count_and_noise():
    spec = S.SPECS["qwen3-8b-L32k-acceptance"]
    a, b, heavy = S.make_logits(spec, 0)
    assert a.shape == (64, 151936) and len(heavy) == 3
    d = b - a
    stds = d.std(axis=1)
    assert np.all(np.abs(stds[heavy] - 3.0) < 0.05)
    light = np.setdiff1d(np.arange(64), heavy)
    assert np.all(np.abs(stds[light] - 0.3) < 0.01)
    assert abs(a.std() - 3.0) < 0.01


@pytest.mark.parametrize("name", sorted(S.SPECS))
def test_specs_are_consistent(name):
    spec = S.SPECS[name]
    assert spec.num_q_heads % spec.num_kv_heads == 0
    wl = S.make_workload(spec, seed=0, build_pool=False)
    assert wl.page_table.shape == (spec.batch, wl.max_pages)
    assert np.all(wl.budget_pages >= 2)
