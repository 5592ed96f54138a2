"""Host logic of the overlapped decode-loop schedule: the layer groups cover
the cache once, in order, with descriptors that name their calibration layers."""
import pytest
import torch

from long_reasoning_decode_amd.decode_loop import LayerGroups


@pytest.mark.parametrize("n_layers,n_groups", [(24, 4), (24, 1), (24, 24), (7, 3), (36, 5)])
def test_layer_groups_partition_the_cache(n_layers, n_groups):
    n_seq, hkv, cap, d = 3, 2, 8, 64
    n_seg = n_layers * n_seq * hkv
    cache = {"k": torch.zeros(n_seg, cap, d, dtype=torch.bfloat16), "v": torch.zeros(n_seg, cap, d, dtype=torch.bfloat16),
             "pos": torch.zeros(n_seg, cap, dtype=torch.int32), "lengths": torch.zeros(n_seg, dtype=torch.int32)}
    g = LayerGroups(cache, n_layers=n_layers, n_seq=n_seq, n_kv_heads=hkv, n_groups=n_groups)
    assert len(g.descs) == n_groups
    assert g.layers[0][0] == 0 and g.layers[-1][1] == n_layers
    assert all(a < b for a, b in g.layers) and all(g.layers[i][1] == g.layers[i + 1][0] for i in range(n_groups - 1))
    row = cap * d * 2
    for (a, b), (s0, s1), desc, ln in zip(g.layers, g.segs, g.descs, g.lengths):
        assert (s0, s1) == (a * n_seq * hkv, b * n_seq * hkv)
        assert desc.layer0 == a and desc.n_layers == b - a and desc.n_seq == n_seq and desc.n_kv_heads == hkv
        assert desc.k == cache["k"].data_ptr() + s0 * row and desc.v == cache["v"].data_ptr() + s0 * row
        assert desc.pos == cache["pos"].data_ptr() + s0 * cap * 4
        assert desc.lengths == ln.data_ptr() == cache["lengths"].data_ptr() + s0 * 4 and ln.numel() == s1 - s0


def test_layer_groups_refuse_bad_counts():
    cache = {"k": torch.zeros(4, 8, 64), "v": torch.zeros(4, 8, 64), "pos": torch.zeros(4, 8, dtype=torch.int32),
             "lengths": torch.zeros(4, dtype=torch.int32)}
    for n in (0, 5):
        with pytest.raises(ValueError):
            LayerGroups(cache, n_layers=4, n_seq=1, n_kv_heads=1, n_groups=n)
