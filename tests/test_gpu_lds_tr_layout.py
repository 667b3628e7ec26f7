"""The lane layout of gfx950's transposing LDS read (ds_read_b64_tr_b16), on which the selected-branch
kernels build their V^T fragments: within each group of 16 lanes, result lane i receives as its
element e element i % 4 of the four 16-bit values that source lane 4e + i / 4 names.  Checked with
the probe library's in-bounds kernel (LDS filled with lds[i] = i) for two address patterns."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_lds_transpose_read_layout():
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_feed_amd", "libnsa_probe.so"))
    lib.nsa_probe_lds_tr_layout.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.nsa_probe_lds_tr_layout.restype = ctypes.c_int
    out = torch.full((512,), -1, dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    print("[case] lds transpose read layout", flush=True)
    assert lib.nsa_probe_lds_tr_layout(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(2, 64, 4)
    lanes = np.arange(64)
    named = [4 * lanes, 64 * (lanes % 16) + 4 * (lanes // 16)]      # first element each lane names
    for pattern in range(2):
        want = np.zeros((64, 4), dtype=np.int64)
        for lane in range(64):
            grp, i = divmod(lane, 16)
            for e in range(4):
                src = 16 * grp + 4 * e + i // 4
                want[lane, e] = named[pattern][src] + i % 4
        np.testing.assert_array_equal(got[pattern], want)
