"""Host-side arithmetic of the streaming composition (no device)."""
from long_context_attention_paged_amd import streaming


def test_budget_split():
    # the pages' decode working set: 2100 MiB over 16 layers of a 262K cache
    n_res = streaming.resident_pages_for_budget(2100 << 20, 16, 2048, 4)
    page = 4 * 53248
    assert 16 * n_res * page + 2 * (2048 - n_res) * page <= 2100 << 20
    assert 16 * (n_res + 1) * page + 2 * (2047 - n_res) * page > 2100 << 20
    assert streaming.resident_pages_for_budget(1 << 40, 16, 2048, 4) == 2048


def test_prefill_ranges_tile_the_read_pages():
    for pos0, chunk, S, n_logical in [(262144, 512, 1107, 2052), (36 * 128 + 50, 200, 15, 40),
                                      (0, 128, 1, 1), (0, 1, 4, 4), (127, 2, 2, 2),
                                      (5 * 128, 128, 3, 6), (1000, 24, 100, 10)]:
        rng = streaming.prefill_ranges(pos0, chunk, S, n_logical)
        n_read = (pos0 + chunk + 127) // 128
        assert rng[0][0] == 0 and rng[-1][1] == n_read
        assert all(rng[i][1] == rng[i + 1][0] for i in range(len(rng) - 1))
        assert all(0 < b - a <= S for a, b in rng)
        assert rng[-1][0] <= pos0 // 128      # the last range holds the chunk's pages
    # the pages' 450 MiB prefill budget at 262K: two slots of 1107 pages, two ranges
    page = 4 * 53248
    S = (450 << 20) // (2 * page)
    assert S == 1107
    assert len(streaming.prefill_ranges(262144, 512, S, 2052)) == 2


def test_prefill_ranges_reject_what_cannot_fit():
    import pytest
    with pytest.raises(ValueError):
        streaming.prefill_ranges(127, 130, 2, 8)   # the chunk spans 3 pages, a slot holds 2
    with pytest.raises(ValueError):
        streaming.prefill_ranges(1000, 100, 16, 8)  # past the host tier
