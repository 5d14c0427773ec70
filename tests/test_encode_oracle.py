"""Pins of the encoder oracle (a learned merge list applied to text in the
order it was learned) against results fixed independently of it: the
training oracles' own output, a lowest-rank-first encoder, brute force
between the Python and C forms, and the closed form of runs."""
import itertools

import numpy as np
import pytest

import corpus
import oracle
from oracle import reference as ref

from checks import BASE, WS, rank_encode

GENERATORS = (1, 2, 4, 5)


@pytest.mark.parametrize("c", GENERATORS)
def test_encoding_the_training_corpus_reproduces_training(c):
    # merge k of training is the argmax of the counts of the sequence after
    # k merges, so replaying the list must meet the same counts and end in
    # the same tokens (computed by the chunk-multiset trainer, an unrelated
    # algorithm)
    d = corpus.generate(corpus.CONFIGS[c].scaled(30_000, seed=70 + c))
    m, t, _ = oracle.train_chunks(d, 80)
    counts, tokens = oracle.encode(d, m)
    assert np.array_equal(counts, m[:, 2])
    assert np.array_equal(tokens, t)


@pytest.mark.parametrize("k", [0, 1, 7, 40])
def test_encoding_with_a_prefix_equals_training_that_far(k):
    d = corpus.generate(corpus.CONFIGS[5].scaled(20_000, seed=81))
    m, _, _ = oracle.train_chunks(d, 40)
    mk, tk, _ = oracle.train_chunks(d, k)
    _, tokens = oracle.encode(d, m[:k])
    assert np.array_equal(mk, m[:k])
    assert np.array_equal(tokens, tk)


@pytest.mark.parametrize("c", GENERATORS)
def test_new_text_matches_lowest_rank_first_encoding(c):
    # learn on one corpus, encode another of the same kind: applying merges
    # in learned order equals repeatedly merging the lowest-rank pair inside
    # each chunk (checks.rank_encode, written without the merge loop)
    learn = corpus.generate(corpus.CONFIGS[c].scaled(40_000, seed=90 + c))
    text = corpus.generate(corpus.CONFIGS[c].scaled(15_000, seed=190 + c))
    m, _, _ = oracle.train_chunks(learn, 120)
    _, tokens = oracle.encode(text, m)
    assert np.array_equal(tokens, rank_encode(text, m))


def test_python_and_c_encoders_agree_on_every_tiny_string():
    alphabet = [ord("a"), ord("b"), ord("1"), ord(" ")]
    lists = [
        [(97, 97), (256, 97), (256, 256)],
        [(97, 98), (98, 97), (256, 257), (97, 97)],
        [(32, 32), (49, 49), (97, 256), (256, 97)],
    ]
    for pairs in lists:
        for n in range(0, 7):
            for combo in itertools.product(alphabet, repeat=n):
                d = bytes(combo)
                pc, pt = ref.encode(d, pairs)
                cc, ct = oracle.encode(np.frombuffer(d, dtype=np.uint8), np.array(pairs))
                assert list(cc) == pc, (d, pairs)
                assert list(ct) == pt, (d, pairs)


def test_runs_closed_form():
    # a run of r letters under (a,a): r - 1 occurrences, floor(r / 2) merged
    for r in range(1, 300):
        counts, tokens = oracle.encode(np.full(r, 97, dtype=np.uint8), [(97, 97)])
        assert counts[0] == r - 1
        assert tokens.size == r - r // 2
        assert tokens[0] == (BASE if r >= 2 else 97) | WS


def test_unknown_ids_are_rejected():
    d = np.frombuffer(b"abab", dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.encode(d, [(97, 256)])          # id 256 does not exist before merge 0
    with pytest.raises(ValueError):
        oracle.encode(d, [(97, 98), (257, 97)])
    with pytest.raises(ValueError):
        ref.encode(b"abab", [(97, 256)])
    counts, tokens = oracle.encode(d, [(97, 98), (256, 256)])
    assert list(counts) == [2, 1] and list(tokens) == [257 | WS]
