"""The streaming-read probe that bench.py uses for the read ceiling runs on the GPU over
a small tile list (every index inside the caches) and returns success (GPU only)."""
import ctypes
from pathlib import Path

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from paged_kv_cache_27_amd._binding import LIB_PATH

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tile_bytes", [1024, 2048, 4096, 8192])
def test_probe_reads_tiles(tile_bytes):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib = ctypes.CDLL(str(LIB_PATH.with_name("libpkv_probe.so")))  # built beside the package library
    f = lib.pkv_probe_read_tiles
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    n_cache_tiles = 512
    k = torch.randint(0, 255, (n_cache_tiles * tile_bytes,), dtype=torch.uint8, device="cuda")
    v = torch.randint(0, 255, (n_cache_tiles * tile_bytes,), dtype=torch.uint8, device="cuda")
    for n in (1, 7, 3000):  # fewer tiles than waves, and several per wave
        tiles = torch.from_numpy(np.random.default_rng(n).integers(0, n_cache_tiles, n).astype(np.int32)).cuda()
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        print(f"probe tile_bytes {tile_bytes} n {n}", flush=True)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert f(k.data_ptr(), v.data_ptr(), tiles.data_ptr(), n, tile_bytes, sink.data_ptr(), stream) == 0
        torch.cuda.synchronize()
