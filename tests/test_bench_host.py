"""Host-side pieces of bench.py (no GPU): the tile list the gather probe reads and the
CPU description recorded beside the oracle baseline."""
import torch

import bench
import workloads as W

bench.torch = torch


def test_decode_tiles_are_the_decode_reads():
    """Every (sequence, KV head, block) the decode visits contributes its K tile and
    then its V tile, at byte offset tile * (phys * Hkv + g) in the K half of a
    [2, blocks, Hkv, bs, D] pool and one pool further for V; nothing else."""
    s = W.random_small(3, batch=5, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                       max_ctx=100, min_ctx=0, dtype=torch.bfloat16)
    off, tile = bench.decode_tiles(s)
    assert tile == 16 * 128 * 2
    NB, H = s.k_cache.shape[0], s.k_cache.shape[1]
    want = []
    for b, n in enumerate(s.context_lens.tolist()):
        for g in range(H):
            for j in range((n + 15) // 16):
                t = int(s.block_tables[b, j]) * H + g
                want += [t * tile, (NB * H + t) * tile]
    assert off.tolist() == want
    assert int(off.max()) + tile <= 2 * NB * H * tile


def test_cpu_description_names_the_host():
    d = bench.cpu_description()
    assert d["logical_cpus"] and d["cpu_model"]
