"""GPU parity of training over the distinct words (bpe_train_chunked,
through the C ABI) against the chunk-multiset C oracle.

The merge list (pairs and counts) and the final tokens must be identical to
the oracle's: on every workload recipe at ragged sizes, on the degenerate
inputs (empty, no pair at all, one word), on words at and past the longest
a 64-byte record holds, on a corpus with more distinct words than the word
table holds (so that most words are kept once per occurrence and the list
of such words outgrows its first allocation), and with host buffers. These
run over the chunks whatever memory their records take
(BPE_FLAG_ALWAYS_CHUNKS); one test also checks the default. The full-size
workloads are compared in test_gpu_full.py."""
import ctypes
import sys

import numpy as np
import pytest

import corpus
import oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def bpe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bpe_merge_amd
    return bpe_merge_amd


def _dev(data):
    import torch
    return torch.from_numpy(np.array(data, dtype=np.uint8)).to("cuda:0")  # a writable copy


def _check(bpe, data, n_merges, what, table_log2=None, always=True):
    _say("chunked: %s (%d bytes, %d merges)" % (what, data.size, n_merges))
    gm, gt = bpe.train_chunked(_dev(data), n_merges, table_log2, always_chunks=always)
    om, ot, _ = oracle.train_chunks(data, n_merges)
    gm = gm.cpu().numpy().astype(np.int64)
    gt = gt.cpu().numpy().astype(np.uint32)
    assert gm.shape == om.shape and np.array_equal(gm, om), "merges of %s" % what
    assert gt.shape == ot.shape and np.array_equal(gt, ot), "tokens of %s" % what
    return om


SIZES = [1, 2, 3, 17, 4097, 65537, 300_001, 2_000_003]


def test_every_recipe_at_ragged_sizes(bpe):
    for i, n in enumerate(SIZES):
        for cfg in sorted(corpus.CONFIGS):
            spec = corpus.CONFIGS[cfg].scaled(n, seed=500 + 10 * i + cfg)
            k = 300 if n < 65537 else 1500
            _check(bpe, corpus.generate(spec), k, "%s at %d" % (spec.kind, n))


def test_merge_counts_zero_and_one(bpe):
    d = corpus.generate(corpus.CONFIGS[3].scaled(100_000, seed=531))
    _check(bpe, d, 0, "no merges")
    _check(bpe, d, 1, "one merge")
    m, t = bpe.train_chunked(_dev(d), 200, tokens=False, always_chunks=True)
    om, _, _ = oracle.train_chunks(d, 200, want_tokens=False)
    assert t is None and np.array_equal(m.cpu().numpy().astype(np.int64), om)


def test_degenerate_inputs(bpe):
    m, t = bpe.train_chunked(_dev(np.zeros(0, np.uint8)), 10, always_chunks=True)
    assert m.shape[0] == 0 and t.shape[0] == 0
    # every word one byte long (letters and punctuation alternate): no pair
    one = np.frombuffer(b"a.b,c;d:" * 5000, dtype=np.uint8)
    assert _check(bpe, one, 50, "one-byte words").shape[0] == 0
    # one word: a run of a single byte, merged into doublings
    _check(bpe, np.full(300_000, ord("a"), np.uint8), 40, "one long run")
    # a long word among ordinary text, before and after it
    text = corpus.generate(corpus.CONFIGS[3].scaled(200_000, seed=532))
    long_word = np.frombuffer(b"xyzzy" * 40_000, dtype=np.uint8)
    _check(bpe, np.concatenate([long_word, text, long_word[:77_777]]), 800, "long words at both ends")


def test_words_at_the_table_length_limit(bpe):
    rng = np.random.default_rng(533)
    parts = []
    for _ in range(20_000):
        ln = int(rng.choice([30, 31, 32, 33, 34, 40]))
        # few distinct words of each length: many repeats, so their counts matter
        w = bytes(97 + (int(rng.integers(0, 3)) + j * 7) % 26 for j in range(ln))
        parts.append(w + b" ")
    d = np.frombuffer(b"".join(parts), dtype=np.uint8)
    _check(bpe, d, 600, "words of 30..40 bytes")


def test_more_distinct_words_than_the_word_table_holds(bpe):
    # ~450k random words of 4..12 letters: the word table of 2^16 slots holds
    # a fraction; the rest are kept once per occurrence, and their list grows
    # past its first allocation
    rng = np.random.default_rng(534)
    n_words = 450_000
    lens = rng.integers(4, 13, size=n_words)
    letters = rng.integers(97, 123, size=int(lens.sum()), dtype=np.uint8)
    out = np.empty(int(lens.sum()) + n_words, dtype=np.uint8)
    ends = np.cumsum(lens + 1)
    starts = ends - lens - 1
    pos = np.repeat(starts - np.cumsum(np.r_[0, lens[:-1]]), lens) + np.arange(int(lens.sum()))
    out[pos] = letters
    out[ends - 1] = ord(" ")
    # every tenth word repeated many times, so that weights differ
    common = out[: ends[9]].copy()
    d = np.concatenate([out, np.tile(common, 300)])
    _check(bpe, d, 1000, "random words")


def test_host_buffers_through_the_c_abi(bpe):
    d = corpus.generate(corpus.CONFIGS[2].scaled(500_000, seed=535))
    k = 700
    om, ot, _ = oracle.train_chunks(d, k)
    merges = np.zeros((k, 3), dtype=np.uint32)
    tokens = np.zeros(d.size, dtype=np.uint32)
    n_done = ctypes.c_uint32(0)
    n_tok = ctypes.c_size_t(0)
    cfg = bpe.Config()
    cfg.flags = bpe.FLAG_ALWAYS_CHUNKS
    st = bpe._lib.bpe_train_chunked(d.ctypes.data, d.size, k, ctypes.byref(cfg), merges.ctypes.data,
                                    ctypes.byref(n_done), tokens.ctypes.data, tokens.size, ctypes.byref(n_tok))
    assert st == 0, bpe._lib.bpe_last_error()
    assert np.array_equal(merges[: n_done.value].astype(np.int64), om)
    assert np.array_equal(tokens[: n_tok.value], ot)


def test_default_path_choice_gives_the_same_results(bpe):
    # as called: over the chunks or, past the records' bound, over the full array
    for cfg, n in ((3, 1_000_003), (5, 1_000_003), (2, 300_001)):
        spec = corpus.CONFIGS[cfg].scaled(n, seed=540 + cfg)
        _check(bpe, corpus.generate(spec), 1200, "default path, %s" % spec.kind, always=False)


def test_a_full_pair_table_is_reported(bpe):
    # a 2^10-slot pair table cannot hold this corpus's pairs: BPE_ETABLE,
    # never a result with a count missing; a large table trains bit-exactly
    d = corpus.generate(corpus.CONFIGS[5].scaled(200_000, seed=545))
    with pytest.raises(bpe.BpeError) as e:
        bpe.train_chunked(_dev(d), 30, 10, always_chunks=True)
    assert e.value.status == bpe.ETABLE
    _check(bpe, d, 30, "the same corpus with a large table", table_log2=22)


def test_default_stream_work_is_ordered_before_and_after(bpe):
    # the corpus is produced by torch kernels on the default stream, queued
    # behind other work, with no synchronisation before the call
    import torch
    data = corpus.generate(corpus.CONFIGS[3].scaled(1 << 20, seed=546))
    om, ot, _ = oracle.train_chunks(data, 500)
    src = torch.from_numpy(data.copy()).pin_memory()
    torch.cuda.synchronize()
    a = torch.randn(2048, 2048, device="cuda:0")
    for _ in range(20):
        a = a @ a
        a = a / a.abs().amax()
    d = torch.empty(data.size, dtype=torch.uint8, device="cuda:0")
    d.copy_(src, non_blocking=True)
    d = d ^ (a[0, 0] * 0).to(torch.uint8)  # a kernel that waits for the busy work
    m, t = bpe.train_chunked(d, 500, always_chunks=True)
    assert np.array_equal(m.cpu().numpy().astype(np.int64), om)
    assert np.array_equal(t.cpu().numpy().astype(np.uint32), ot)


def test_a_merge_with_more_count_changes_than_the_one_workgroup_route_holds(bpe):
    # 3,000 words "uv" (3,001 times each) and "uvab" (once each): the first
    # 3,000 merges make each "uv" one symbol, then merging (a, b) changes the
    # counts of about 6,000 pairs (each "uv" symbol next to a, and next to
    # the new one), past the one-workgroup route's change table: it gives up
    # and the multi-workgroup passes train from the start, with the same result
    import oracle as orc
    letters = [c for c in range(256) if orc.char_class(c) == 0 and c not in (ord("a"), ord("b"))]
    pairs = [(u, v) for u in letters for v in letters][:3000]
    parts = []
    for u, v in pairs:
        parts.append(bytes([u, v, 32]) * 3001)
        parts.append(bytes([u, v, ord("a"), ord("b"), 32]))
    d = np.frombuffer(b"".join(parts), dtype=np.uint8)
    om = _check(bpe, d, 3002, "a wide merge")
    assert om[3000].tolist() == [ord("a"), ord("b"), 3000]
