"""GPU parity of the encoder and of resume by merge-list replay (the HIP
path through the C ABI against the oracle). Bit-exact: all work is integer."""
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


def _np(t):
    return t.cpu().numpy()


def _say(msg):
    print(msg, flush=True)


def test_encoding_the_training_corpus_gives_training_tokens(bpe):
    d = corpus.generate(corpus.CONFIGS[3].scaled(600_000, seed=41))
    _say("encode training corpus")
    gm, gt = bpe.train(_dev(d), 150, 19)
    tokens = bpe.encode(_dev(d), gm, 19)
    assert np.array_equal(_np(tokens).astype(np.uint32), _np(gt).astype(np.uint32))
    _, ot = oracle.encode(d, _np(gm))
    assert np.array_equal(_np(tokens).astype(np.uint32), ot)


@pytest.mark.parametrize("c", [3, 5])
def test_encoding_a_large_training_corpus_gives_training_tokens(bpe, c):
    # many tiles per workgroup: LDS reuse from one tile to the next (the
    # staged word-start bits of a tile were once cleared by the next tile
    # while its output was still being written)
    spec = corpus.CONFIGS[c].scaled(48 << 20, n_merges=600, seed=77)
    d = _dev(corpus.generate(spec))
    _say("encode large training corpus c=%d" % c)
    gm, gt = bpe.train(d, spec.n_merges, 22)
    with bpe.Encoder(gm) as e:
        for slots in (0, 0xFFFFFFFF):
            e.cache(slots)
            got = e.encode(d)
            assert got.shape == gt.shape and bool((got == gt).all()), (c, slots)


@pytest.mark.parametrize("c", [1, 2, 4, 5])
@pytest.mark.parametrize("n", [1, 3, 8191, 8193, 70_001])
def test_encode_new_text_matches_oracle(bpe, c, n):
    learn = corpus.generate(corpus.CONFIGS[c].scaled(50_000, seed=300 + c))
    om, _, _ = oracle.train_chunks(learn, 90)
    text = corpus.generate(corpus.CONFIGS[c].scaled(n, seed=400 + c + n))
    _, ot = oracle.encode(text, om)
    _say("encode new text c=%d n=%d" % (c, n))
    gt = _np(bpe.encode(_dev(text), om, 18)).astype(np.uint32)
    assert np.array_equal(gt, ot), (c, n)


@pytest.mark.parametrize("k", [0, 1, 60, 120])
def test_replay_then_train_equals_training_straight_through(bpe, k):
    d = corpus.generate(corpus.CONFIGS[5].scaled(400_000, seed=52))
    _say("replay k=%d" % k)
    gm, gt = bpe.train(_dev(d), 120, 20)
    with bpe.State(_dev(d), table_log2=20) as st:
        st.replay(gm[:k])
        mk = _np(st.merges())
        assert np.array_equal(mk, _np(gm)[:k])      # counts recorded as in training
        st.run(120 - k)
        st.sync()
        assert np.array_equal(_np(st.merges()), _np(gm))
        assert np.array_equal(_np(st.tokens()), _np(gt))
        k2, c2 = st.pair_counts()
    # the count table after replay and training equals a recount of the result
    s = _np(gt).astype(np.int64)
    ok = (s[1:] & 0x10000) == 0
    keys = ((s[:-1] & 0xFFFF) << 16 | (s[1:] & 0xFFFF))[ok]
    u, c = np.unique(keys, return_counts=True)
    assert np.array_equal(np.asarray(k2, dtype=np.int64), u) and np.array_equal(np.asarray(c2, dtype=np.int64), c)


def test_replay_of_absent_pairs_and_runs(bpe):
    # runs of identical bytes (L == R merges) and pairs that never occur:
    # an absent pair records count 0, changes nothing, and uses up its id
    d = np.array(list(b"aaaaaaa bbbb aaab ab ") * 3000, dtype=np.uint8)
    merges = np.array([[97, 97, 0], [120, 121, 0], [256, 256, 0], [256, 97, 0], [98, 98, 0], [259, 98, 0]])
    oc, ot = oracle.encode(d, merges)
    _say("replay absent pairs and runs")
    with bpe.State(_dev(d), table_log2=16) as st:
        st.replay(merges)
        gm = _np(st.merges())
        assert np.array_equal(gm[:, :2], merges[:, :2]) and np.array_equal(gm[:, 2], oc)
        assert np.array_equal(_np(st.tokens()).astype(np.uint32), ot)


def test_replay_rejects_an_unknown_id_and_the_state_stays_usable(bpe):
    d = corpus.generate(corpus.CONFIGS[1].scaled(20_000, seed=61))
    _say("replay rejection")
    with bpe.State(_dev(d), table_log2=17) as st:
        with pytest.raises(RuntimeError):
            st.replay(np.array([[97, 98], [300, 97]]))   # id 300 cannot exist before merge 1
        st.run(10)
        st.sync()
        om, ot, _ = oracle.train_chunks(d, 10)
        assert np.array_equal(_np(st.merges()).astype(np.int64), om)
        assert np.array_equal(_np(st.tokens()).astype(np.uint32), ot)


def test_encoder_object_repeated_calls_and_count(bpe):
    learn = corpus.generate(corpus.CONFIGS[4].scaled(300_000, seed=71))
    om, _, _ = oracle.train_chunks(learn, 700)
    with bpe.Encoder(om) as e:
        for i, n in enumerate((5, 1_500_000, 4095, 4096, 4097, 5121, 70_000)):
            text = corpus.generate(corpus.CONFIGS[4].scaled(n, seed=720 + i))
            _say("encoder call %d n=%d" % (i, n))
            _, ot = oracle.encode(text, om)
            got = _np(e.encode(_dev(text))).astype(np.uint32)
            assert np.array_equal(got, ot), (i, n)


def test_encoder_words_longer_than_a_tile(bpe):
    # runs past a tile's LDS range are encoded from global scratch
    merges = [(97, 97), (256, 256), (257, 257), (258, 97), (98, 98), (260, 260), (256, 97)]
    parts = [b"x" * 3, b"a" * 20_001, b" ", b"b" * 7_000, b"ab" * 3_000, b" ", b"a" * 5_000, b"1" * 9_999]
    text = np.frombuffer(b"".join(parts), np.uint8)
    with bpe.Encoder(merges) as e:
        for shift in (0, 7, 4090):
            tt = np.concatenate([np.full(shift, 32, np.uint8), text])
            _say("encoder long words shift=%d" % shift)
            _, ot = oracle.encode(tt, merges)
            assert np.array_equal(_np(e.encode(_dev(tt))).astype(np.uint32), ot), shift


def test_encoder_host_input_and_output_through_the_abi(bpe):
    import ctypes
    learn = corpus.generate(corpus.CONFIGS[2].scaled(100_000, seed=81))
    om, _, _ = oracle.train_chunks(learn, 300)
    text = corpus.generate(corpus.CONFIGS[2].scaled(40_000, seed=82))
    _, ot = oracle.encode(text, om)
    with bpe.Encoder(om) as e:
        out = np.zeros(text.size, np.uint32)
        n_tok = ctypes.c_size_t(0)
        st = bpe._lib.bpe_encoder_encode(e._h, text.ctypes.data, text.size, None, out.ctypes.data, out.size,
                                         ctypes.byref(n_tok))
        assert st == 0 and np.array_equal(out[: n_tok.value], ot)
        st = bpe._lib.bpe_encoder_encode(e._h, text.ctypes.data, text.size, None, None, 0, ctypes.byref(n_tok))
        assert st == 0 and n_tok.value == ot.size


# word cache: (log2 slots, key bits). 2^8 slots fill up, so most words
# take the uncached path; 0 key bits give every word of one length the same
# key, 4 bits nearly so (records whose bytes differ, probing past them); 0
# slots turn the cache off.
CACHE_SETTINGS = [(0xFFFFFFFF, 32), (0, 32), (8, 32), (10, 0), (12, 4), (16, 32)]


@pytest.mark.parametrize("c", [2, 3, 5])
def test_word_cache_settings_do_not_change_tokens(bpe, c):
    learn = corpus.generate(corpus.CONFIGS[c].scaled(200_000, seed=900 + c))
    om, _, _ = oracle.train_chunks(learn, 400)
    text = corpus.generate(corpus.CONFIGS[c].scaled(300_001, seed=910 + c))
    _, ot = oracle.encode(text, om)
    d = _dev(text)
    with bpe.Encoder(om) as e:
        for slots, bits in CACHE_SETTINGS:
            _say("word cache c=%d slots=%d bits=%d" % (c, slots, bits))
            e.cache(slots, bits)
            got = _np(e.encode(d)).astype(np.uint32)
            assert np.array_equal(got, ot), (c, slots, bits)


def test_word_cache_lengths_and_alignments(bpe):
    # words of 2..40 letters (the cache takes 2..32) at every offset modulo
    # 32 of a tile, some across tile edges, with merges that make tokens of
    # several lengths inside them
    rng = np.random.default_rng(5)
    words = [bytes(rng.choice(list(b"abcd"), size=L).tolist()) for L in range(2, 41) for _ in range(3)]
    parts = []
    for i in range(4000):
        w = words[rng.integers(len(words))]
        parts.append(w)
        parts.append(b" " * int(rng.integers(1, 4)))
        if i % 97 == 0:
            parts.append(b"7" * int(rng.integers(1, 40)))
    text = np.frombuffer(b"".join(parts), np.uint8)
    om, _, _ = oracle.train_chunks(text, 120)
    with bpe.Encoder(om) as e:
        for shift in (0, 1, 13, 31):
            tt = np.concatenate([np.full(shift, 32, np.uint8), text])
            _, ot = oracle.encode(tt, om)
            d = _dev(tt)
            for slots, bits in CACHE_SETTINGS:
                _say("word cache lengths shift=%d slots=%d bits=%d" % (shift, slots, bits))
                e.cache(slots, bits)
                assert np.array_equal(_np(e.encode(d)).astype(np.uint32), ot), (shift, slots, bits)


def test_word_cache_rejects_bad_settings(bpe):
    with bpe.Encoder([(97, 98)]) as e:
        for slots, bits in ((7, 32), (25, 32), (16, 33)):
            with pytest.raises(bpe.BpeError):
                e.cache(slots, bits)
        e.cache(8, 0)
        text = np.frombuffer(b"ab abab ba " * 100, np.uint8)
        assert np.array_equal(_np(e.encode(_dev(text))).astype(np.uint32), oracle.encode(text, [(97, 98)])[1])


def test_outputs_at_every_word_offset(bpe):
    # the copy passes store four tokens at a time from a 16-byte boundary of
    # the output: views of one buffer starting 0..3 words in, with texts
    # whose tiles end at every residue of the token count
    import torch
    learn = corpus.generate(corpus.CONFIGS[2].scaled(100_000, seed=91))
    om, _, _ = oracle.train_chunks(learn, 250)
    big = torch.zeros(300_000, dtype=torch.int32, device="cuda:0")
    with bpe.Encoder(om) as e, bpe.Trie(om) as tr:
        for k, n in enumerate((5, 4099, 70_003, 250_001)):
            text = corpus.generate(corpus.CONFIGS[2].scaled(n, seed=930 + k))
            d = _dev(text)
            _, oe = oracle.encode(text, om)
            ot = oracle.trie_encode(text, om)
            for off in range(4):
                _say("outputs at offset %d n=%d" % (off, n))
                big.fill_(-1)
                got = _np(e.encode(d, out=big[off:])).astype(np.uint32)
                assert np.array_equal(got, oe), (off, n)
                assert int(big[off + oe.size:].max()) == -1 if off + oe.size < big.numel() else True
                got = _np(tr.encode(d, out=big[off:])).astype(np.uint32)
                assert np.array_equal(got, ot.astype(np.uint32)), (off, n)


def test_encoder_reports_long_words_past_its_scratch(bpe):
    # one word longer than the 2^24 positions of scratch a call may use for
    # words past a tile's LDS copy: BPE_ENOMEM (the walk skips the word, so
    # nothing is written past the scratch), and the encoder stays usable
    merges = [(97, 97), (256, 256)]
    text = np.full((1 << 24) + 5000, 97, np.uint8)
    small = np.frombuffer(b"aaaa ab " * 500, np.uint8)
    with bpe.Encoder(merges) as e:
        _say("encoder scratch overflow")
        with pytest.raises(bpe.BpeError) as ei:
            e.encode(_dev(text))
        assert ei.value.status == bpe.ENOMEM
        assert np.array_equal(_np(e.encode(_dev(small))).astype(np.uint32), oracle.encode(small, merges)[1])
