"""bpe_train_static (training in the library's static workspace, for
callers that cannot allocate) against bpe_train, through the C ABI."""
import ctypes

import numpy as np
import pytest

import corpus
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bpe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bpe_merge_amd
    return bpe_merge_amd


def _dev(data):
    import torch
    return torch.from_numpy(np.array(data, dtype=np.uint8)).to("cuda:0")


def _np(t, dtype):
    return t.cpu().numpy().astype(dtype)


def test_static_workspace_training_matches_bpe_train_twice(bpe):
    # two calls in a row on one device, the second on a smaller input: the
    # shared workspace keeps the first call's contents, which must not leak
    # into the second
    cases = [(3, bpe.STATIC_MAX_BYTES, 300, 0), (5, 300_001, 200, 16)]
    for cfg, n, k, tlog2 in cases:
        d = corpus.generate(corpus.CONFIGS[cfg].scaled(n, seed=300 + cfg))
        print("static workspace: recipe %d, %d bytes, %d merges" % (cfg, n, k), flush=True)
        sm, stok = bpe.train_static(_dev(d), k, tlog2 or None)
        rm, rtok = bpe.train(_dev(d), k, tlog2 or min(20, 22))
        assert np.array_equal(_np(sm, np.int64), _np(rm, np.int64)), cfg
        assert np.array_equal(_np(stok, np.uint32), _np(rtok, np.uint32)), cfg
        om, ot, _ = oracle.train_chunks(d, k)
        assert np.array_equal(_np(sm, np.int64), om) and np.array_equal(_np(stok, np.uint32), ot), cfg


def test_static_workspace_rejects_what_it_cannot_hold(bpe):
    lib = bpe._lib
    buf = (ctypes.c_uint8 * 16)()
    merges = (ctypes.c_uint32 * 12)()
    n_done = ctypes.c_uint32(7)
    # beyond the byte limit: rejected on the host before anything runs
    assert lib.bpe_train_static(ctypes.addressof(buf), bpe.STATIC_MAX_BYTES + 1, 4, 0, None,
                                ctypes.addressof(merges), ctypes.byref(n_done), None, 0, None) == bpe.EINVAL
    assert b"static workspace" in lib.bpe_last_error()
    # a table larger than the workspace takes
    assert lib.bpe_train_static(ctypes.addressof(buf), 16, 4, bpe.STATIC_MAX_TABLE_LOG2 + 1, None,
                                ctypes.addressof(merges), ctypes.byref(n_done), None, 0, None) == bpe.EINVAL
    # the empty corpus is valid
    assert lib.bpe_train_static(None, 0, 4, 0, None, ctypes.addressof(merges), ctypes.byref(n_done), None, 0,
                                None) == bpe.OK and n_done.value == 0
