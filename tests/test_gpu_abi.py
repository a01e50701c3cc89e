"""C ABI facts that need a device: the KV slot count and the AcrossKV aliasing of the cache views.

The library's skv_num_kv_slots must be l + ceil((L - l) / g) (the AcrossKV
memory formula of the summary page, section 3.4, whose printed reductions
tests/golden/acrosskv_kv_memory.json pins), and the views of the layers of
one AcrossKV group must alias one slot."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L_,l,g", [(32, 16, 1), (32, 16, 2), (32, 16, 4), (32, 16, 8), (32, 16, 16), (32, 24, 4),
                                    (80, 40, 1), (5, 1, 3), (4, 4, 1), (4, 0, 2)])
def test_slot_count_and_view_aliasing(L_, l, g):
    from swiftkv_prefill_skipping_amd import _lib as L
    from oracle import swiftkv_oracle as O
    cfg = L.make_config(L_, 512, 4, 1, 128, 512, 256, 10000.0, 1e-5, l, g, L.SKV_BF16, 16, 1, 16)
    m = L.skv_model_create(cfg)
    try:
        n = L.skv_num_kv_slots(m)
        assert n == l + -(-(L_ - l) // g)
        c = L.skv_kv_cache_create(m, 4)
        try:
            base = {}
            for j in range(1, L_ + 1):
                k, v = L.skv_kv_cache_view(c, j)
                s = O.slot_of_layer(j, L_, l, g)
                if s in base:
                    assert (k.data, v.data) == base[s], f"layer {j} does not alias its group's slot"
                else:
                    assert all(k.data != kd for kd, _ in base.values()), f"layer {j} shares another slot"
                    base[s] = (k.data, v.data)
            assert len(base) == n
        finally:
            L.skv_kv_cache_destroy(c)
    finally:
        L.skv_model_destroy(m)
