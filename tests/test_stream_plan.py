"""Prefix pinning against a least-recently-used cache for the cyclic layer scan (in-c post,
section on streaming the trunk: every token visits the layers in the same order; with 93
layers and 90 slots LRU hits nothing, pinning the first 90 hits 90 of 93 every pass), and
the pinning plan for the K3 expert stack on one 288 GB GPU."""
from mxfp4_expert_gemm_amd.stream import cache_hits, plan_prefix


def test_lru_never_hits_a_cyclic_scan_longer_than_the_cache():
    assert cache_hits(93, 10, 90, "lru") == 0          # the post's example
    for n, s in [(5, 4), (12, 11), (93, 1), (92, 0)]:
        assert cache_hits(n, 7, s, "lru") == 0


def test_prefix_pinning_hits_its_layers_every_pass():
    assert cache_hits(93, 10, 90, "prefix") == 900
    assert round(cache_hits(93, 1, 90, "prefix") / 93, 3) == 0.968   # 96.8%
    assert cache_hits(5, 3, 0, "prefix") == 0


def test_with_room_for_every_layer_lru_misses_only_the_first_pass():
    assert cache_hits(8, 5, 8, "lru") == 8 * 4
    assert cache_hits(8, 5, 9, "lru") == 8 * 4
    assert cache_hits(8, 5, 9, "prefix") == 8 * 5


def test_plan_prefix_for_the_k3_stack():
    layer = 896 * 17_547_264                            # 15.72 GB of experts per routed layer
    assert plan_prefix(92, layer, 288 * 10**9) == 18
    # the dense weights of 92 layers (router 12.85 MB, two latent projections of 51.38 MB)
    # and the slot buffer of a one-token batch stay in HBM too
    reserved = 92 * (12_845_056 + 2 * 51_380_224) + 16 * 17_547_264
    assert plan_prefix(92, layer, 288 * 10**9, reserved) == 17
    assert plan_prefix(3, layer, 10**15) == 3
    assert plan_prefix(3, layer, 0) == 0
    assert plan_prefix(3, layer, 10**12, 2 * 10**12) == 0
