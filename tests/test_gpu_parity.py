"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact everywhere: all work is integer. Inputs are the seeded synthetic
corpora at sizes that span several 8192-symbol scan tiles and end in a
ragged tail, plus adversarial runs and the degenerate cases."""
import os
import sys

import numpy as np
import pytest

import corpus
import oracle

from checks import WS, ID, check_invariants

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
    return torch.from_numpy(np.ascontiguousarray(data, dtype=np.uint8)).to("cuda:0")


def gpu_train(bpe, data, n_merges, table_log2=None):
    m, t = bpe.train(_dev(data), n_merges, table_log2)
    return m.cpu().numpy().astype(np.int64), t.cpu().numpy().astype(np.uint32)


def exact_counts(tokens):
    """Exact pair-count map of a symbol sequence, as sorted (keys, counts)."""
    s = np.asarray(tokens, dtype=np.int64)
    if s.size < 2:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    ok = (s[1:] & WS) == 0
    keys = ((s[:-1] & ID) << 16 | (s[1:] & ID))[ok]
    u, c = np.unique(keys, return_counts=True)
    return u, c.astype(np.int64)


RAGGED = [1, 2, 3, 15, 16, 17, 255, 4095, 4096, 4097, 12289, 65537, 300_001]


def test_tagging_matches_oracle(bpe):
    data = np.arange(256, dtype=np.uint8)
    cases = [data, data[::-1].copy(), np.repeat(data, 3)]
    for i, n in enumerate(RAGGED):
        cases.append(corpus.generate(corpus.CONFIGS[1 + i % 5].scaled(n, seed=40 + i)))
    for d in cases:
        _say("tag n=%d" % d.size)
        with bpe.State(_dev(d), table_log2=16) as st:
            t = st.tokens().cpu().numpy().astype(np.uint32)
            assert np.array_equal(t, oracle.tag(d))
            assert st.lengths().cpu().numpy().tolist() == [d.size]


def test_count_map_iteration0_and_after_merges(bpe):
    for i, n in enumerate([4097, 65537, 300_001]):
        d = corpus.generate(corpus.CONFIGS[1 + i].scaled(n, seed=60 + i))
        _say("counts n=%d" % n)
        with bpe.State(_dev(d), table_log2=18) as st:
            k, c = st.pair_counts()
            ek, ec = exact_counts(oracle.tag(d))
            assert np.array_equal(k, ek) and np.array_equal(c, ec)
            for steps in (1, 5, 20):
                while len(st.merges()) < steps:
                    assert st.step() is not None
                _, ot, _ = oracle.train_chunks(d, steps)
                k, c = st.pair_counts()
                ek, ec = exact_counts(ot)
                assert np.array_equal(k, ek) and np.array_equal(c, ec), steps


def test_step_by_step_matches_oracle(bpe):
    d = corpus.generate(corpus.CONFIGS[2].scaled(50_000, seed=71))
    om, ot, ol = oracle.train_chunks(d, 40)
    with bpe.State(_dev(d), table_log2=17) as st:
        for k in range(40):
            m = st.step()
            assert m == tuple(int(x) for x in om[k]), k
        assert np.array_equal(st.tokens().cpu().numpy().astype(np.uint32), ot)
        assert np.array_equal(st.lengths().cpu().numpy().astype(np.int64), ol)
        assert np.array_equal(st.merges().cpu().numpy().astype(np.int64), om)


def test_train_bit_exact_ragged_sizes_all_generators(bpe):
    for i, n in enumerate(RAGGED):
        for c in (1, 2, 4, 5):
            d = corpus.generate(corpus.CONFIGS[c].scaled(n, seed=1000 + 10 * i + c))
            gm, gt = gpu_train(bpe, d, 64, table_log2=19)
            om, ot, _ = oracle.train_chunks(d, 64)
            assert np.array_equal(gm, om), (n, c)
            assert np.array_equal(gt, ot), (n, c)


def test_runs_of_identical_pairs(bpe):
    # run-length parity: (a,a) chains, runs crossing tile boundaries, and
    # alternating pairs that chain into (X,X) runs after the first merge
    cases = [np.full(r, 0x61, np.uint8) for r in [2, 3, 4, 5, 63, 64, 65, 4095, 4096, 4097, 8193, 100_003]]
    cases.append(np.frombuffer(b"ab" * 50_001, dtype=np.uint8))
    rng = np.random.default_rng(5)
    parts = []
    for _ in range(400):
        parts.append(np.full(int(rng.integers(1, 9000)), rng.choice([0x61, 0x62, 0x7A]), np.uint8))
        if rng.random() < 0.3:
            parts.append(np.array([0x20], np.uint8))
    cases.append(np.concatenate(parts))
    for d in cases:
        _say("runs n=%d" % d.size)
        gm, gt = gpu_train(bpe, d, 40, table_log2=16)
        om, ot, _ = oracle.train_chunks(d, 40)
        assert np.array_equal(gm, om) and np.array_equal(gt, ot), d.size


def test_degenerate_inputs(bpe):
    for raw in [b"a", b"a1", b" ", b"\n\n", b"ab ab", b"aaaaa", bytes(range(256))]:
        d = np.frombuffer(raw, dtype=np.uint8)
        gm, gt = gpu_train(bpe, d, 8, table_log2=12)
        om, ot, _ = oracle.train_chunks(d, 8)
        assert np.array_equal(gm, om) and np.array_equal(gt, ot), raw
    import torch
    m, t = bpe.train(torch.zeros(0, dtype=torch.uint8, device="cuda:0"), 5)
    assert m.shape[0] == 0 and t.shape[0] == 0
    # more merges requested than pairs exist: stops early, no error
    d = np.frombuffer(b"abcabc abc", dtype=np.uint8)
    gm, gt = gpu_train(bpe, d, 100, table_log2=12)
    om, ot, _ = oracle.train_chunks(d, 100)
    assert len(om) < 100 and np.array_equal(gm, om) and np.array_equal(gt, ot)
    with bpe.State(_dev(d), table_log2=12) as st:
        st.run(100)
        assert st.sync() == len(om)
        assert st.step() is None


def test_host_pointer_input(bpe):
    import ctypes
    d = corpus.generate(corpus.CONFIGS[1].scaled(20_000, seed=3))
    merges = (bpe.Merge * 32)()
    toks = np.zeros(d.size, dtype=np.uint32)
    n_done = ctypes.c_uint32(0)
    n_tok = ctypes.c_size_t(0)
    st = bpe._lib.bpe_train(d.ctypes.data, d.size, 32, None, ctypes.addressof(merges), ctypes.byref(n_done),
                            toks.ctypes.data, toks.size, ctypes.byref(n_tok))
    assert st == bpe.OK
    om, ot, _ = oracle.train_chunks(d, 32)
    gm = np.array([[m.left, m.right, m.count] for m in merges[: n_done.value]], dtype=np.int64)
    assert np.array_equal(gm, om)
    assert np.array_equal(toks[: n_tok.value], ot)


def test_tokens_read_into_host_memory_between_merges(bpe):
    # bpe_tokens into host memory passes through the symbol buffer the next
    # merge pass writes (in two halves); training goes on unchanged after it
    import ctypes
    for n in (1, 2, 3, 4097, 100_001):
        d = corpus.generate(corpus.CONFIGS[3].scaled(n, seed=70 + n % 7))
        _say("host tokens n=%d" % n)
        with bpe.State(_dev(d), table_log2=16) as st:
            for k in (0, 5, 40):
                while len(st.merges()) < k and st.step() is not None:
                    pass
                done = len(st.merges())
                toks = np.zeros(max(d.size, 1), dtype=np.uint32)
                n_tok = ctypes.c_size_t(0)
                assert bpe._lib.bpe_tokens(st._h, toks.ctypes.data, toks.size, ctypes.byref(n_tok)) == bpe.OK
                _, ot, _ = oracle.train_chunks(d, done)
                assert np.array_equal(toks[: n_tok.value], ot), (n, k)
                assert np.array_equal(st.tokens().cpu().numpy().astype(np.uint32), ot), (n, k)


def test_determinism_and_table_size_independence(bpe):
    d = corpus.generate(corpus.CONFIGS[5].scaled(400_000, seed=11))
    ref = gpu_train(bpe, d, 120, table_log2=17)
    for tl in (17, 18, 19):
        out = gpu_train(bpe, d, 120, table_log2=tl)
        assert np.array_equal(out[0], ref[0]) and np.array_equal(out[1], ref[1]), tl
    om, ot, _ = oracle.train_chunks(d, 120)
    assert np.array_equal(ref[0], om) and np.array_equal(ref[1], ot)


def test_full_pair_table_is_reported_not_dropped(bpe):
    # random bytes have far more distinct countable pairs than 7/8 of a
    # 2^10-slot table: training must stop with BPE_ETABLE, never go on with
    # a count missing; the same input trains bit-exactly with a large table
    d = corpus.generate(corpus.CONFIGS[5].scaled(200_000, seed=12))
    with pytest.raises(RuntimeError, match="table"):
        gpu_train(bpe, d, 30, table_log2=10)
    big = gpu_train(bpe, d, 30, table_log2=22)
    om, ot, _ = oracle.train_chunks(d, 30)
    assert np.array_equal(big[0], om) and np.array_equal(big[1], ot)


def test_config1_full_with_invariants(bpe):
    spec = corpus.CONFIGS[1]
    d = corpus.generate(spec)
    gm, gt = gpu_train(bpe, d, spec.n_merges, spec.table_log2)
    om, ot, ol = oracle.train_literal(d, spec.n_merges)
    assert np.array_equal(gm, om) and np.array_equal(gt, ot)
    check_invariants(d, gm, gt, ol)


def test_bench_launch_path_matches_train(bpe):
    # the state API the benchmark times (init, run, sync, profile) gives the
    # same result as bpe_train
    d = corpus.generate(corpus.CONFIGS[3].scaled(2_000_000, seed=13))
    gm, gt = gpu_train(bpe, d, 300, table_log2=20)
    with bpe.State(_dev(d), table_log2=20) as st:
        st.run(150)
        r = st.profile(150)
        assert r.launches == 150 and r.merges_done == len(gm)
        assert np.array_equal(st.merges().cpu().numpy().astype(np.int64), gm)
        assert np.array_equal(st.tokens().cpu().numpy().astype(np.uint32), gt)
    om, ot, _ = oracle.train_chunks(d, 300)
    assert np.array_equal(gm, om) and np.array_equal(gt, ot)


def test_large_corpus_uses_the_large_tiles_and_matches(bpe):
    # above 2 x 256 tiles of 16384 symbols the merge pass runs 1024-thread
    # workgroups on 16384-symbol tiles; below, 512 threads on 8192
    # words (unequal pairs mostly), then runs (every merge an equal pair,
    # many tiles entered inside a chain of occurrences)
    for cfg, seed in [(3, 91), (5, 92)]:
        d = corpus.generate(corpus.CONFIGS[cfg].scaled(10_000_000, seed=seed))
        _say("train 10 MB of %s, 400 merges" % corpus.CONFIGS[cfg].kind)
        gm, gt = bpe.train(_dev(d), 400, 21)
        om, ot, _ = oracle.train_chunks(d, 400)
        assert np.array_equal(gm.cpu().numpy().astype(np.int64), om), cfg
        assert np.array_equal(gt.cpu().numpy().astype(np.uint32), ot), cfg


def test_interleaved_state_calls_match_training(bpe):
    # run, step, profile and run again on one state: the merge of every
    # iteration is selected on the device from state the previous launch
    # left (candidate list or table sweep), whatever call enqueued it
    d = corpus.generate(corpus.CONFIGS[3].scaled(3_000_000, seed=17))
    om, ot, _ = oracle.train_chunks(d, 200)
    with bpe.State(_dev(d), table_log2=20) as st:
        r = st.profile(20)
        assert r.launches == 20 and r.merges_done == 20
        assert 1 <= r.sweeps <= 20  # a fresh state has no candidate list yet
        st.run(30)
        assert st.sync() == 50
        for k in range(50, 60):
            assert st.step() == tuple(int(x) for x in om[k]), k
        st.run(40)
        r = st.profile(30)
        assert r.launches == 30 and r.merges_done == 130 and 0 <= r.sweeps <= 30
        st.run(70)
        assert st.sync() == 200
        assert np.array_equal(st.merges().cpu().numpy().astype(np.int64), om)
        assert np.array_equal(st.tokens().cpu().numpy().astype(np.uint32), ot)


def test_words_of_uniform_letters_many_near_ties(bpe):
    # flat pair counts: hundreds of pairs within a few percent of the
    # maximum keep the candidate list long and its threshold busy
    rng = np.random.default_rng(23)
    letters = np.frombuffer(b"abcdefghijklmnopqrstuvwxyz", dtype=np.uint8)
    words = [letters[rng.integers(0, 26, int(rng.integers(2, 9)))].tobytes() for _ in range(3000)]
    text = b" ".join(words[int(i)] for i in rng.integers(0, 3000, 120_000))
    d = np.frombuffer(text, dtype=np.uint8)
    _say("uniform letters n=%d" % d.size)
    gm, gt = gpu_train(bpe, d, 600, table_log2=18)
    om, ot, _ = oracle.train_chunks(d, 600)
    assert np.array_equal(gm, om) and np.array_equal(gt, ot)


def test_oversubscribed_grid_needs_no_coresidency(bpe):
    # merge passes launched with four times the workgroups the device holds
    # at once: most start only after earlier ones have finished. No
    # workgroup waits for one that has not started (tiles are handed out in
    # order; table sweeps are claimed in chunks; the next merge is prepared
    # by the last workgroup to finish), so results are unchanged.
    cases = [(1, 65_536, 60), (3, 3_000_000, 150), (5, 2_000_000, 120), (2, 1_000_000, 200)]
    for cfg, n, k in cases:
        d = corpus.generate(corpus.CONFIGS[cfg].scaled(n, seed=200 + cfg))
        _say("oversubscribed grid: recipe %d, %d bytes, %d merges" % (cfg, n, k))
        m, t = bpe.train(_dev(d), k, 18, flags=bpe.FLAG_OVERSUBSCRIBE)
        om, ot, _ = oracle.train_chunks(d, k)
        assert np.array_equal(m.cpu().numpy().astype(np.int64), om), cfg
        assert np.array_equal(t.cpu().numpy().astype(np.uint32), ot), cfg
