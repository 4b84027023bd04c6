"""Host-side arithmetic of the streaming composition (no device)."""
from long_context_attention_paged_amd import streaming


def test_budget_split():
    # the pages' decode working set: 2100 MiB over 16 layers of a 262K cache
    n_res = streaming.resident_pages_for_budget(2100 << 20, 16, 2048, 4)
    page = 4 * 53248
    assert 16 * n_res * page + 2 * (2048 - n_res) * page <= 2100 << 20
    assert 16 * (n_res + 1) * page + 2 * (2047 - n_res) * page > 2100 << 20
    assert streaming.resident_pages_for_budget(1 << 40, 16, 2048, 4) == 2048
