"""Pins of the inference oracle (greedy longest match over the vocabulary of
a merge list) against results fixed independently of it: hand-worked
examples of the page's walk, a dictionary form against the C trie form on
every tiny string, the definition checked token by token, and the special
case of a bytes-only vocabulary."""
import itertools
import json
import os

import numpy as np
import pytest

import corpus
import oracle
from oracle import reference as ref

from checks import CLASS, chunk_starts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "trie_examples.json")


def _u8(b):
    return np.frombuffer(bytes(b), dtype=np.uint8)


def test_hand_worked_examples():
    ex = json.load(open(GOLDEN))["examples"]
    for e in ex:
        t = e["text"].encode()
        assert ref.trie_encode(t, e["merges"]) == e["tokens"], e["id"]
        assert oracle.trie_encode(_u8(t), e["merges"]).tolist() == e["tokens"], e["id"]


def test_bytes_only_vocabulary_is_the_identity():
    d = corpus.generate(corpus.CONFIGS[5].scaled(5000, seed=3))
    assert np.array_equal(oracle.trie_encode(d, np.zeros((0, 2))), d.astype(np.uint32))


def test_dictionary_and_trie_forms_agree_on_every_tiny_string():
    alphabet = [ord("a"), ord("b"), ord("c"), ord(" ")]
    lists = [
        [(97, 98), (98, 99), (256, 99), (97, 257)],     # duplicate spelling abc
        [(97, 97), (256, 256), (257, 97), (98, 97)],
        [(99, 97), (256, 98), (97, 98), (32, 32), (258, 99)],
    ]
    for pairs in lists:
        for n in range(0, 7):
            for combo in itertools.product(alphabet, repeat=n):
                d = bytes(combo)
                assert oracle.trie_encode(_u8(d), pairs).tolist() == ref.trie_encode(d, pairs), (d, pairs)


def _check_definition(d, merges, tokens):
    """Decode equals the text, and each token is the longest vocabulary
    string at its position (all lengths tried through a dictionary) with the
    smallest id among equal strings."""
    v = ref.vocab_strings([tuple(m[:2]) for m in np.asarray(merges).tolist()])
    first = {}
    for i, s in enumerate(v):
        first.setdefault(s, i)
    longest = max(len(s) for s in v)
    b = bytes(d)
    p = 0
    for t in np.asarray(tokens).tolist():
        s = v[t]
        assert b[p:p + len(s)] == s and first[s] == t
        for ln in range(len(s) + 1, min(longest, len(b) - p) + 1):
            assert b[p:p + ln] not in first, (p, ln)
        p += len(s)
    assert p == len(b)


@pytest.mark.parametrize("c", [1, 2, 4, 5])
def test_definition_holds_on_trained_vocabularies(c):
    learn = corpus.generate(corpus.CONFIGS[c].scaled(30_000, seed=500 + c))
    m, _, _ = oracle.train_chunks(learn, 150)
    text = corpus.generate(corpus.CONFIGS[c].scaled(6_000, seed=600 + c))
    toks = oracle.trie_encode(text, m)
    _check_definition(text, m, toks)
    assert toks.tolist() == ref.trie_encode(bytes(text), m[:, :2].tolist())


@pytest.mark.parametrize("c", [1, 2, 4, 5])
def test_trained_tokens_stay_inside_one_class_so_words_encode_alone(c):
    # every string a trained list spells has bytes of one class, so no match
    # crosses a class change: encoding the text whole equals encoding each
    # maximal same-class run on its own and concatenating
    learn = corpus.generate(corpus.CONFIGS[c].scaled(40_000, seed=700 + c))
    m, _, _ = oracle.train_chunks(learn, 200)
    for s in ref.vocab_strings(m[:, :2].tolist()):
        assert len(set(CLASS[np.frombuffer(s, np.uint8)].tolist())) == 1
    text = corpus.generate(corpus.CONFIGS[c].scaled(20_000, seed=800 + c))
    whole = oracle.trie_encode(text, m)
    starts = np.flatnonzero(chunk_starts(text)).tolist() + [text.size]
    parts = [oracle.trie_encode(text[a:b], m) for a, b in zip(starts[:-1], starts[1:])]
    assert np.array_equal(whole, np.concatenate(parts))


def test_unknown_ids_are_rejected():
    with pytest.raises(ValueError):
        oracle.trie_encode(_u8(b"ab"), [(97, 256)])
    with pytest.raises(ValueError):
        ref.trie_encode(b"ab", [(97, 98), (300, 97)])
