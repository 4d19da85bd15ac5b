"""moe_build_offsets_noalloc (static device scratch, no workspace) against moe_build_offsets.

Both are called through the C ABI on the same ids; offsets, sorted_rows and row_pos must be
bitwise equal.  Two calls in a row, the second with a smaller input, show that the scratch
the first call left behind does not leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

from helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _ids(R, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E + 1, R).astype(np.int32)
    ids[rng.random(R) < 0.05] = E                     # sentinel rows
    return torch.from_numpy(ids).to(DEV)


def _noalloc(lib, ids, E):
    R = ids.numel()
    off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    sr = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    rp = torch.full((R,), -7, dtype=torch.int32, device=DEV)
    st = lib.build_offsets_noalloc(ctypes.c_void_p(ids.data_ptr()), R, E, ctypes.c_void_p(off.data_ptr()),
                                   ctypes.c_void_p(sr.data_ptr()), ctypes.c_void_p(rp.data_ptr()),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.last_error()
    return off, sr, rp


def _with_workspace(lib, ids, E):
    R = ids.numel()
    ws = torch.empty(max(1, lib.build_offsets_workspace(R, E)), dtype=torch.uint8, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sr = torch.empty(R, dtype=torch.int32, device=DEV)
    rp = torch.empty(R, dtype=torch.int32, device=DEV)
    st = lib.build_offsets(ctypes.c_void_p(ids.data_ptr()), R, E, ctypes.c_void_p(off.data_ptr()),
                           ctypes.c_void_p(sr.data_ptr()), ctypes.c_void_p(rp.data_ptr()),
                           ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.last_error()
    return off, sr, rp


# (R, E) pairs of consecutive calls: large then smaller, over the chunked (three-kernel) path
# with 1024- and 256-row chunks and the one-workgroup path
SEQUENCES = [((70000, 1024), (5000, 64)), ((65536, 256), (16384, 32)), ((16384, 128), (900, 8))]


@pytest.mark.parametrize("seq", SEQUENCES)
def test_build_offsets_noalloc_matches(seq):
    import grouped_gemm_histogram_amd as g
    lib = g.load()
    for i, (R, E) in enumerate(seq):
        say(f"build_offsets_noalloc call {i}: R={R} E={E}")
        ids = _ids(R, E, R + E)
        got = _noalloc(lib, ids, E)
        ref = _with_workspace(lib, ids, E)
        torch.cuda.synchronize()
        for name, a, b in zip(("offsets", "sorted_rows", "row_pos"), got, ref):
            assert torch.equal(a, b), name


def test_build_offsets_noalloc_rejects_oversized():
    import grouped_gemm_histogram_amd as g
    lib = g.load()
    # 2^21 rows at E = 1024 need 2048 chunk histograms of 1025 bins: 8.4 MB > 4 MiB
    R, E = 1 << 21, 1024
    assert lib.build_offsets_workspace(R, E) > 4 << 20
    fake = ctypes.c_void_p(0x1000)
    assert lib.build_offsets_noalloc(fake, R, E, fake, fake, fake, None) == 3   # MOE_ERR_WORKSPACE
    assert b"static scratch" in lib.last_error()
