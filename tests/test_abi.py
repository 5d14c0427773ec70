"""The C-ABI library loads and exports what include/bpe.h declares; host-side
argument validation (no GPU needed: every check here runs before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bpe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(bpe_[a-z_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def bpe():
    import bpe_merge_amd
    return bpe_merge_amd


def test_every_declared_function_is_exported(bpe):
    declared = _declared()
    assert "bpe_train" in declared and "bpe_step" in declared
    lib = ctypes.CDLL(bpe.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(bpe.EXPORTED)


def test_library_is_gfx950_only():
    import subprocess
    lib = os.path.join(ROOT, "bpe_merge_amd", "libbpe.so")
    out = subprocess.run(["strings", lib], capture_output=True, text=True).stdout
    assert "gfx950" in out
    for other in ("gfx942", "gfx90a", "gfx1100", "sm_"):
        assert "amdgcn-amd-amdhsa--" + other not in out


def test_strerror(bpe):
    lib = bpe._lib
    for st, word in [(0, "ok"), (1, "pair"), (-1, "invalid"), (-2, "table"), (-3, "id space"),
                     (-4, "memory"), (-5, "HIP"), (-6, "device error"), (-99, "unknown")]:
        assert word in lib.bpe_strerror(st).decode()


def test_workspace_bytes(bpe):
    n = 1 << 28
    ws = bpe.workspace_bytes(n, 22)
    # two buffers of 16-bit symbols + the global pair table of 2^22 8-byte
    # slots, plus small parts (control block, look-back status, merges,
    # the class of every id)
    assert 2 * 2 * n + 8 * (1 << 22) <= ws <= 2 * 2 * n + 8 * (1 << 22) + (8 << 20)
    assert bpe.workspace_bytes(n, 24) - ws == 8 * ((1 << 24) - (1 << 22))
    assert bpe.workspace_bytes(10, 0) > 0
    assert bpe.workspace_bytes(1 << 31, 22) == 0       # above the size limit
    assert bpe.workspace_bytes(100, 9) == 0            # table_log2 out of range
    assert bpe.workspace_bytes(100, 31) == 0


def test_train_argument_validation_before_any_device_call(bpe):
    lib = bpe._lib
    n_done = ctypes.c_uint32(7)
    n_tok = ctypes.c_size_t(7)
    buf = (ctypes.c_uint8 * 16)()
    merges = (ctypes.c_uint32 * 3 * 8)()
    toks = (ctypes.c_uint32 * 16)()
    # too many merges for 16-bit ids
    st = lib.bpe_train(ctypes.addressof(buf), 16, 65281, None, ctypes.addressof(merges),
                       ctypes.byref(n_done), None, 0, None)
    assert st == bpe.EIDSPACE
    assert "65281" in lib.bpe_last_error().decode()
    # null pointers
    assert lib.bpe_train(None, 16, 4, None, ctypes.addressof(merges), ctypes.byref(n_done), None, 0,
                         None) == bpe.EINVAL
    assert lib.bpe_train(ctypes.addressof(buf), 16, 4, None, None, ctypes.byref(n_done), None, 0,
                         None) == bpe.EINVAL
    assert lib.bpe_train(ctypes.addressof(buf), 16, 4, None, ctypes.addressof(merges), None, None, 0,
                         None) == bpe.EINVAL
    # token capacity below n
    assert lib.bpe_train(ctypes.addressof(buf), 16, 4, None, ctypes.addressof(merges), ctypes.byref(n_done),
                         ctypes.addressof(toks), 15, ctypes.byref(n_tok)) == bpe.EINVAL
    # bad config
    cfg = bpe.Config(); cfg.table_log2 = 5
    assert lib.bpe_train(ctypes.addressof(buf), 16, 4, ctypes.byref(cfg), ctypes.addressof(merges),
                         ctypes.byref(n_done), None, 0, None) == bpe.EINVAL
    cfg = bpe.Config(); cfg.flags = 4  # an unknown flag bit (1 and 2 are testing aids)
    assert lib.bpe_train(ctypes.addressof(buf), 16, 4, ctypes.byref(cfg), ctypes.addressof(merges),
                         ctypes.byref(n_done), None, 0, None) == bpe.EINVAL
    # an empty corpus is valid and needs no device
    n_done.value = 9
    assert lib.bpe_train(None, 0, 4, None, ctypes.addressof(merges), ctypes.byref(n_done), None, 0,
                         ctypes.byref(n_tok)) == bpe.OK
    assert n_done.value == 0 and n_tok.value == 0


def test_chunked_training_argument_validation_before_any_device_call(bpe):
    lib = bpe._lib
    buf = (ctypes.c_uint8 * 16)()
    merges = (ctypes.c_uint32 * 12)()
    toks = (ctypes.c_uint32 * 16)()
    n_done = ctypes.c_uint32(7)
    n_tok = ctypes.c_size_t(7)
    call = lib.bpe_train_chunked
    assert call(ctypes.addressof(buf), 16, bpe.MAX_MERGES + 1, None, ctypes.addressof(merges),
                ctypes.byref(n_done), None, 0, None) == bpe.EIDSPACE
    assert call(None, 16, 4, None, ctypes.addressof(merges), ctypes.byref(n_done), None, 0, None) == bpe.EINVAL
    assert call(ctypes.addressof(buf), 16, 4, None, None, ctypes.byref(n_done), None, 0, None) == bpe.EINVAL
    assert call(ctypes.addressof(buf), 16, 4, None, ctypes.addressof(merges), None, None, 0, None) == bpe.EINVAL
    assert call(ctypes.addressof(buf), 16, 4, None, ctypes.addressof(merges), ctypes.byref(n_done),
                ctypes.addressof(toks), 15, ctypes.byref(n_tok)) == bpe.EINVAL
    cfg = bpe.Config(); cfg.flags = 4
    assert call(ctypes.addressof(buf), 16, 4, ctypes.byref(cfg), ctypes.addressof(merges), ctypes.byref(n_done),
                None, 0, None) == bpe.EINVAL
    cfg = bpe.Config(); cfg.workspace = ctypes.addressof(buf); cfg.workspace_bytes = 16
    assert call(ctypes.addressof(buf), 16, 4, ctypes.byref(cfg), ctypes.addressof(merges), ctypes.byref(n_done),
                None, 0, None) == bpe.EINVAL
    assert b"workspace" in lib.bpe_last_error()
    assert call(None, 0, 4, None, ctypes.addressof(merges), ctypes.byref(n_done), None, 0,
                ctypes.byref(n_tok)) == bpe.OK
    assert n_done.value == 0 and n_tok.value == 0


def test_state_calls_reject_null(bpe):
    lib = bpe._lib
    h = ctypes.c_void_p()
    buf = (ctypes.c_uint8 * 4)()
    assert lib.bpe_init(None, 4, None, ctypes.byref(h)) == bpe.EINVAL
    assert lib.bpe_init(ctypes.addressof(buf), 0, None, ctypes.byref(h)) == bpe.EINVAL
    assert lib.bpe_init(ctypes.addressof(buf), 4, None, None) == bpe.EINVAL
    assert lib.bpe_run(None, 1) == bpe.EINVAL
    assert lib.bpe_sync(None, None) == bpe.EINVAL
    assert lib.bpe_step(None, None) == bpe.EINVAL
    assert lib.bpe_tokens(None, None, 0, None) == bpe.EINVAL
    assert lib.bpe_merges(None, None, 0, None) == bpe.EINVAL
    assert lib.bpe_lengths(None, None, 0, None) == bpe.EINVAL
    assert lib.bpe_pair_counts(None, None, None, 0, None) == bpe.EINVAL
    assert lib.bpe_profile(None, 1, None, None) == bpe.EINVAL
    lib.bpe_free(None)  # no-op


def test_binding_has_no_fallback(bpe):
    # the product path must not import the oracle or any CPU implementation
    src = open(os.path.join(ROOT, "bpe_merge_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("oracle/", "")
    assert "import corpus" not in src


def test_encode_and_replay_argument_validation_before_any_device_call(bpe):
    lib = bpe._lib
    buf = (ctypes.c_uint8 * 16)()
    merges = (ctypes.c_uint32 * 3 * 4)()
    n_tok = ctypes.c_size_t(5)
    assert lib.bpe_replay(None, ctypes.addressof(merges), 1) == bpe.EINVAL
    # null bytes with n > 0, null merges with n_merges > 0, null n_tokens
    assert lib.bpe_encode(None, 16, ctypes.addressof(merges), 1, None, None, 0, ctypes.byref(n_tok)) == bpe.EINVAL
    assert lib.bpe_encode(ctypes.addressof(buf), 16, None, 1, None, None, 0, ctypes.byref(n_tok)) == bpe.EINVAL
    assert lib.bpe_encode(ctypes.addressof(buf), 16, ctypes.addressof(merges), 1, None, None, 0, None) == bpe.EINVAL
    assert lib.bpe_encode(ctypes.addressof(buf), 16, ctypes.addressof(merges), 65281, None, None, 0,
                          ctypes.byref(n_tok)) == bpe.EIDSPACE
    toks = (ctypes.c_uint32 * 8)()
    assert lib.bpe_encode(ctypes.addressof(buf), 16, ctypes.addressof(merges), 1, None, ctypes.addressof(toks), 8,
                          ctypes.byref(n_tok)) == bpe.EINVAL          # capacity below n
    # an empty text is valid and needs no device
    assert lib.bpe_encode(None, 0, ctypes.addressof(merges), 1, None, None, 0, ctypes.byref(n_tok)) == bpe.OK
    assert n_tok.value == 0


def _merges(bpe, pairs):
    arr = (bpe.Merge * max(len(pairs), 1))()
    for i, (left, right) in enumerate(pairs):
        arr[i].left, arr[i].right, arr[i].count = left, right, 0
    return arr


def test_trie_and_encoder_reject_bad_lists_before_any_device_call(bpe):
    lib = bpe._lib
    h = ctypes.c_void_p()
    for build in (lib.bpe_trie_build, lib.bpe_encoder_build):
        assert build(None, 1, ctypes.byref(h)) == bpe.EINVAL                       # NULL merges
        assert build(ctypes.addressof(_merges(bpe, [(97, 98)])), 1, None) == bpe.EINVAL  # NULL out
        assert build(ctypes.addressof(_merges(bpe, [(97, 256)])), 1, ctypes.byref(h)) == bpe.EINVAL
        assert build(ctypes.addressof(_merges(bpe, [(97, 98), (300, 97)])), 2, ctypes.byref(h)) == bpe.EINVAL
        assert build(ctypes.addressof(_merges(bpe, [(97, 98)])), 65281, ctypes.byref(h)) == bpe.EIDSPACE
        assert not h.value
    # a merge joining two byte classes cannot be part of a longest-match vocabulary
    assert lib.bpe_trie_build(ctypes.addressof(_merges(bpe, [(97, 32)])), 1, ctypes.byref(h)) == bpe.EINVAL
    assert "byte classes" in lib.bpe_last_error().decode()


def test_trie_and_encoder_encode_argument_validation(bpe):
    lib = bpe._lib
    buf = (ctypes.c_uint8 * 16)()
    n_tok = ctypes.c_size_t(7)
    for enc in (lib.bpe_trie_encode, lib.bpe_encoder_encode):
        assert enc(None, ctypes.addressof(buf), 16, None, None, 0, ctypes.byref(n_tok)) == bpe.EINVAL
    for prof in (lib.bpe_trie_profile, lib.bpe_encoder_profile):
        assert prof(None, ctypes.addressof(buf), 16, 1, None, ctypes.byref(n_tok)) == bpe.EINVAL
    assert lib.bpe_encoder_cache(None, 0xFFFFFFFF, 32) == bpe.EINVAL
    lib.bpe_trie_free(None)
    lib.bpe_encoder_free(None)


def test_bench_refuses_more_than_one_gpu_before_touching_one():
    # the measurement is one GPU's: --gpus N > 1 (or a multi-rank launch)
    # exits with a message, before importing torch or the library
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                           timeout=60, env={**os.environ, **env})
        assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == "", (args, env, r.stderr)
