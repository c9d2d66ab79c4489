"""GPU tests of block swaps between a GPU pool and a pinned host pool (and between two
GPU pools) against the CPU oracle: bit-exact."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_374_amd as pkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _pool(seed, nblocks, dt, shape=(8, 16, 128), device=DEV, pinned=False):
    g = torch.Generator().manual_seed(seed)
    if dt == torch.uint8:
        x = torch.randint(0, 256, (nblocks,) + shape, generator=g, dtype=torch.uint8)
    else:
        x = torch.randn((nblocks,) + shape, generator=g).to(dt)
    if pinned:
        return x.pin_memory()
    return x.to(device)


def _pairs(seed, n, nsrc, ndst):
    g = torch.Generator().manual_seed(seed)
    src = torch.randperm(nsrc, generator=g)[:n]
    dst = torch.randperm(ndst, generator=g)[:n]
    return torch.stack([src, dst], 1).to(torch.int32)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16, torch.float32, torch.uint8],
                         ids=["bf16", "f16", "f32", "u8"])
def test_swap_out_and_in_match_the_oracle(dt):
    _say(f"swap out/in {dt}")
    gpu = _pool(1, 40, dt)
    host = _pool(2, 25, dt, pinned=True)
    out_pairs = _pairs(3, 17, 40, 25)
    want_host = oracle.swap_blocks(host, gpu, out_pairs)
    pkv.swap_blocks(host, gpu, out_pairs.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(host.view(torch.uint8), want_host.view(torch.uint8)), "swap out"
    in_pairs = _pairs(4, 11, 25, 40)
    want_gpu = oracle.swap_blocks(gpu, host, in_pairs)
    pkv.swap_blocks(gpu, host, in_pairs.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(gpu.cpu().view(torch.uint8), want_gpu.view(torch.uint8)), "swap in"


def test_swap_pairs_in_pinned_host_memory():
    """The pair list may itself live in pinned host memory: the kernel reads it through
    the device mapping of that memory."""
    _say("swap with pinned host pairs")
    gpu = _pool(11, 40, torch.bfloat16)
    host = _pool(12, 25, torch.bfloat16, pinned=True)
    out_pairs = _pairs(13, 17, 40, 25).pin_memory()
    want_host = oracle.swap_blocks(host, gpu, out_pairs)
    pkv.swap_blocks(host, gpu, out_pairs)
    torch.cuda.synchronize()
    assert torch.equal(host.view(torch.uint8), want_host.view(torch.uint8)), "swap out"
    in_pairs = _pairs(14, 11, 25, 40).pin_memory()
    want_gpu = oracle.swap_blocks(gpu, host, in_pairs)
    pkv.swap_blocks(gpu, host, in_pairs)
    torch.cuda.synchronize()
    assert torch.equal(gpu.cpu().view(torch.uint8), want_gpu.view(torch.uint8)), "swap in"


def test_swap_between_two_gpu_pools_and_odd_block_bytes():
    """Two device pools; a block of 12 bytes (the 4-byte path)."""
    _say("swap gpu->gpu, 12-byte blocks")
    a = _pool(5, 30, torch.float32, shape=(3,))
    b = _pool(6, 9, torch.float32, shape=(3,))
    pairs = _pairs(7, 9, 30, 9)
    want = oracle.swap_blocks(b, a, pairs)
    pkv.swap_blocks(b, a, pairs.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(b.cpu(), want)


def test_swap_8b_shape_round_trip():
    """1024 blocks of the 8B batch's layout (8 KV heads x 16 x 128, bf16: 32 KiB) out
    to the host and back into other GPU blocks: bit for bit the originals."""
    _say("swap 8B-shape round trip")
    gpu = _pool(8, 4096, torch.bfloat16)
    host = torch.empty((1024,) + gpu.shape[1:], dtype=gpu.dtype).pin_memory()
    src = torch.randperm(4096, generator=torch.Generator().manual_seed(9))[:2048]
    out_pairs = torch.stack([src[:1024], torch.arange(1024)], 1).to(torch.int32)
    in_pairs = torch.stack([torch.arange(1024), src[1024:]], 1).to(torch.int32)
    orig = gpu.clone()
    pkv.swap_blocks(host, gpu, out_pairs.to(DEV))
    pkv.swap_blocks(gpu, host, in_pairs.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(gpu[src[1024:].to(DEV)], orig[src[:1024].to(DEV)])
    keep = torch.ones(4096, dtype=torch.bool)
    keep[src[1024:]] = False
    assert torch.equal(gpu[keep.to(DEV)], orig[keep.to(DEV)])


def test_swap_refuses_pageable_host_memory():
    """A pool the device cannot reach (pageable host memory) is refused on the host,
    before anything is enqueued, by the binding and by the C ABI itself."""
    gpu = _pool(10, 4, torch.float32, shape=(4,))
    pageable = torch.zeros(4, 4)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        pkv.swap_blocks(pageable, gpu, pairs)
    buf = np.zeros(16, dtype=np.float32)
    # the pair names a destination block outside the pool, so even a launch would move
    # nothing: the refusal is checked without any chance of a device access to buf
    skip = torch.tensor([[0, 99]], dtype=torch.int32, device=DEV)
    rc = pkv.load().pkv_swap_blocks(buf.ctypes.data_as(ctypes.c_void_p), gpu.data_ptr(),
                                    skip.data_ptr(), 1, 4, 4, 16, None)
    assert rc == -4, pkv.strerror(rc)
    assert np.all(buf == 0)
    # the failed pointer query leaves no error behind for the next call
    pkv.swap_blocks(gpu, gpu.clone(), pairs)
    torch.cuda.synchronize()
