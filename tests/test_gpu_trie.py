"""GPU parity of greedy longest-match inference (the HIP path through the C
ABI against the oracle, token for token)."""
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
    return torch.from_numpy(np.array(data, dtype=np.uint8)).to("cuda:0")


def _vocab(c, merges, seed):
    learn = corpus.generate(corpus.CONFIGS[c].scaled(200_000, seed=seed))
    m, _, _ = oracle.train_chunks(learn, merges)
    return m


@pytest.fixture(scope="module")
def vocabs():
    return {c: _vocab(c, 600, 900 + c) for c in (1, 2, 4, 5)}


@pytest.mark.parametrize("c", [1, 2, 4, 5])
def test_ragged_sizes_match_oracle(bpe, vocabs, c):
    m = vocabs[c]
    with bpe.Trie(m) as t:
        for n in (1, 2, 15, 16, 17, 8191, 8192, 8193, 10239, 10240, 10241, 24_577, 300_001):
            text = corpus.generate(corpus.CONFIGS[c].scaled(n, seed=1000 + n + c))
            _say("trie c=%d n=%d" % (c, n))
            got = t.encode(_dev(text)).cpu().numpy().astype(np.uint32)
            assert np.array_equal(got, oracle.trie_encode(text, m)), (c, n)


def test_large_text_matches_oracle(bpe, vocabs):
    m = vocabs[2]
    text = corpus.generate(corpus.CONFIGS[2])           # the 16 MiB generator at full size
    _say("trie 16 MiB")
    with bpe.Trie(m) as t:
        got = t.encode(_dev(text)).cpu().numpy().astype(np.uint32)
    assert np.array_equal(got, oracle.trie_encode(text, m))


def test_words_longer_than_a_tile(bpe):
    # runs of one letter far longer than a tile and its halo: the tile that
    # owns the word's start walks it to the end and writes the tokens past
    # its recorded range after the look-back
    merges = [(97, 97), (256, 256), (257, 257), (258, 258), (259, 97), (98, 98), (261, 261)]
    parts = [b"x" * 3, b"a" * 70_001, b" ", b"b" * 20_000, b"ab" * 9_000, b" ", b"a" * 9_000, b"1" * 33_333]
    text = np.frombuffer(b"".join(parts), np.uint8)
    want = oracle.trie_encode(text, merges)
    with bpe.Trie(merges) as t:
        for shift in (0, 5, 8190):
            _say("trie long words shift=%d" % shift)
            tt = np.concatenate([np.full(shift, 32, np.uint8), text])
            got = t.encode(_dev(tt)).cpu().numpy().astype(np.uint32)
            assert np.array_equal(got, oracle.trie_encode(tt, merges)), shift
    assert want.size > 0


def test_unaligned_device_input_host_input_and_count(bpe, vocabs):
    import torch
    m = vocabs[1]
    text = corpus.generate(corpus.CONFIGS[1].scaled(50_000, seed=77))
    want = oracle.trie_encode(text, m)
    d = _dev(np.concatenate([np.zeros(64, np.uint8), text]))
    with bpe.Trie(m) as t:
        for off in (64, 63, 61, 57, 49):
            _say("trie unaligned off=%d" % off)
            sub = d[off:]
            w = oracle.trie_encode(d[off:].cpu().numpy(), m)
            assert np.array_equal(t.encode(sub).cpu().numpy().astype(np.uint32), w), off
        # host bytes in, host tokens out, through the C ABI
        import ctypes
        out = np.zeros(text.size, np.uint32)
        n_tok = ctypes.c_size_t(0)
        st = bpe._lib.bpe_trie_encode(t._h, text.ctypes.data, text.size, None, out.ctypes.data, out.size,
                                      ctypes.byref(n_tok))
        assert st == 0 and np.array_equal(out[: n_tok.value], want)
        assert t.count(_dev(text)) == want.size
        torch.cuda.synchronize()


def test_repeated_calls_on_one_trie_and_pool_growth(bpe, vocabs):
    m = vocabs[4]
    with bpe.Trie(m) as t:
        for i, n in enumerate((100, 2_000_000, 7, 65_536, 1_000_003, 0, 12_345)):
            text = corpus.generate(corpus.CONFIGS[4].scaled(max(n, 1), seed=1200 + i))[:n]
            _say("trie call %d n=%d" % (i, n))
            got = t.encode(_dev(text)).cpu().numpy().astype(np.uint32)
            assert np.array_equal(got, oracle.trie_encode(text, m)), (i, n)


def test_trained_on_gpu_then_inferred_on_gpu(bpe):
    d = corpus.generate(corpus.CONFIGS[3].scaled(1_000_000, seed=88))
    gm, _ = bpe.train(_dev(d), 500, 20)
    text = corpus.generate(corpus.CONFIGS[3].scaled(400_000, seed=89))
    _say("trie after GPU training")
    with bpe.Trie(gm) as t:
        slots, longest = t.info()
        assert slots >= 512 and longest >= 2
        got = t.encode(_dev(text)).cpu().numpy().astype(np.uint32)
    assert np.array_equal(got, oracle.trie_encode(text, gm.cpu().numpy()))


def test_bytes_only_vocabulary_and_rejections(bpe):
    text = corpus.generate(corpus.CONFIGS[5].scaled(30_000, seed=5))
    with bpe.Trie(np.zeros((0, 2), np.int64)) as t:
        assert np.array_equal(t.encode(_dev(text)).cpu().numpy().astype(np.uint32), text.astype(np.uint32))
    with pytest.raises(bpe.BpeError):
        bpe.Trie([(97, 300)])                      # id 300 does not exist before merge 0
    with pytest.raises(bpe.BpeError):
        bpe.Trie([(97, 32)])                       # letter + space: crosses a class change


def test_profile_calls_agree_with_encode(bpe, vocabs):
    m = vocabs[1]
    text = corpus.generate(corpus.CONFIGS[1].scaled(200_000, seed=31))
    d = _dev(text)
    with bpe.Trie(m) as t:
        n_tok, ms = t.profile(d, 3)
        assert n_tok == t.count(d) == oracle.trie_encode(text, m).size
        assert ms.shape == (3, 3) and (ms > 0).all()
    with bpe.Encoder(m) as e:
        n_tok, ms = e.profile(d, 3)
        assert n_tok == oracle.encode(text, m)[1].size
        assert ms.shape == (3, 4) and (ms > 0).all()
