"""Pins of the CPU oracles against what the page and the mathematics fix.

The oracle is only trusted once these pass: the character classes the page
prints, hand-worked examples, brute-force agreement between the literal
definition and the chunk-multiset oracle on every tiny string over a small
alphabet, closed forms for runs, an independent rank encoder, and
invariants that any correct result satisfies.
"""
import itertools
import json
import os

import numpy as np
import pytest

import corpus
import oracle
from oracle import reference as ref

from checks import (BASE, CLASS, ID, WS, byte_class, check_invariants, rank_encode,
                    selected_occurrences, vocab_bytes)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


# ---------------------------------------------------------------- classes

def test_char_class_matches_the_stated_classes():
    # the class the page states for every byte, written with Python's
    # character predicates (tests/checks.py), against both oracles' tables
    for b in range(256):
        assert ref.char_class(b) == byte_class(b), b
        assert oracle.char_class(b) == byte_class(b), b


def test_char_class_sizes_and_named_bytes():
    counts = np.bincount(CLASS, minlength=5).tolist()
    # Letter: 52 ASCII letters + 128 bytes >= 0x80; Digit 10; Space 1; Punct 64; Newline 1
    assert counts == [180, 10, 1, 64, 1]
    # every UTF-8 lead and continuation byte of the Turkish letters is a Letter
    for ch in "ışğçöüİŞĞÇÖÜ":
        for b in ch.encode("utf-8"):
            assert ref.char_class(b) == 0
    assert ref.char_class(ord("\n")) == 4 and ref.char_class(ord(" ")) == 2
    assert [ref.char_class(ord(c)) for c in "09"] == [1, 1]
    assert [ref.char_class(ord(c)) for c in "\t\r.,!~\x7f\x00"] == [3] * 8


def test_tag_marks_class_changes_and_position_zero():
    data = b"ab 12\n\nx.."
    s = ref.tag(data)
    starts = [i for i, v in enumerate(s) if v & WS]
    assert starts == [0, 2, 3, 5, 7, 8]
    assert [v & ID for v in s] == list(data)
    assert np.array_equal(oracle.tag(np.frombuffer(data, np.uint8)), np.array(s, dtype=np.uint32))


# ---------------------------------------------------------------- worked examples

def _golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    return g["n_merges"], g["examples"]


@pytest.mark.parametrize("impl", ["python", "literal", "chunks"])
def test_worked_examples(impl):
    n_merges, examples = _golden()
    fn = {"python": oracle.train_python, "literal": oracle.train_literal,
          "chunks": oracle.train_chunks}[impl]
    for ex in examples:
        data = bytes.fromhex(ex["hex"])
        m, t, _ = fn(data, n_merges)
        assert m.tolist() == ex["merges"], ex["id"]
        assert t.tolist() == ex["tokens"], ex["id"]


# ---------------------------------------------------------------- brute force

ALPHA = [0x61, 0x62, 0x31, 0x20, 0xC3]  # a, b, 1, space, a UTF-8 lead byte


def _same(a, b):
    return all(np.array_equal(x, y) for x, y in zip(a, b))


def test_literal_vs_chunks_every_string_up_to_length_7():
    n = 0
    for length in range(0, 8):
        for tup in itertools.product(ALPHA, repeat=length):
            d = np.array(tup, dtype=np.uint8)
            a = oracle.train_literal(d, 8)
            b = oracle.train_chunks(d, 8)
            assert _same(a, b), bytes(d)
            n += 1
    assert n == sum(5 ** L for L in range(8))


def test_literal_vs_chunks_sampled_length_8_and_10():
    rng = np.random.default_rng(8)
    for length in (8, 10):
        for _ in range(6000):
            d = np.array(ALPHA, dtype=np.uint8)[rng.integers(0, 5, length)]
            assert _same(oracle.train_literal(d, 8), oracle.train_chunks(d, 8)), bytes(d)


def test_python_vs_c_every_string_up_to_length_5():
    for length in range(0, 6):
        for tup in itertools.product(ALPHA, repeat=length):
            d = np.array(tup, dtype=np.uint8)
            assert _same(oracle.train_python(d, 8), oracle.train_literal(d, 8)), bytes(d)


def _small_corpora(count, max_bytes, seed0=100):
    rng = np.random.default_rng(seed0)
    for i in range(count):
        spec = corpus.CONFIGS[1 + i % 5]
        n = int(rng.integers(1, max_bytes + 1))
        yield corpus.generate(spec.scaled(n, seed=seed0 + i))


def test_python_vs_c_small_corpora():
    for d in _small_corpora(15, 3000):
        assert _same(oracle.train_python(d, 40), oracle.train_literal(d, 40))


def test_literal_vs_chunks_small_corpora_all_generators():
    for d in _small_corpora(400, 16384, seed0=1000):
        a = oracle.train_literal(d, 64)
        b = oracle.train_chunks(d, 64)
        assert _same(a, b)


def test_literal_vs_chunks_config1_full():
    spec = corpus.CONFIGS[1]
    d = corpus.generate(spec)
    a = oracle.train_literal(d, spec.n_merges)
    b = oracle.train_chunks(d, spec.n_merges)
    assert _same(a, b)
    assert len(a[0]) == spec.n_merges


# ---------------------------------------------------------------- closed forms

def test_single_run_closed_form():
    # a run of r equal letters: the first merge counts r-1 overlapping pairs
    # and shrinks the run by floor(r/2); repeated halving ends in one token
    for r in list(range(1, 70)) + [255, 256, 257, 1000, 4095, 4096]:
        d = np.full(r, 0x61, dtype=np.uint8)
        m, t, lengths = oracle.train_literal(d, 16)
        if r == 1:
            assert len(m) == 0 and t.tolist() == [0x61 | WS]
            continue
        assert m[0].tolist() == [0x61, 0x61, r - 1]
        assert lengths[1] == r - r // 2
        assert len(t) == 1 or len(m) == 16
        assert _same((m, t, lengths), oracle.train_chunks(d, 16))


def test_shrink_equals_closed_form_each_step():
    # stepwise through the literal Python oracle: count_k is the brute-force
    # maximum, and each merge shrinks the sequence by ceil(m/2) per chain
    for d in list(_small_corpora(10, 1500, seed0=77)) + [np.frombuffer(b"aaaaaaa bbbb aaaa", np.uint8)]:
        s = ref.tag(bytes(d))
        for k in range(30):
            c = {}
            for i in range(1, len(s)):
                if not s[i] & WS:
                    c[(s[i - 1] & ID, s[i] & ID)] = c.get((s[i - 1] & ID, s[i] & ID), 0) + 1
            m, s2 = ref.step(s, k)
            if m is None:
                assert not c
                break
            top = max(c.values())
            assert m[2] == top and (m[0], m[1]) == min(p for p in c if c[p] == top)
            assert len(s) - len(s2) == selected_occurrences(s, m[0], m[1])
            s = s2


# ---------------------------------------------------------------- independent encoder + invariants

def test_rank_encoding_identity_and_invariants():
    for d in list(_small_corpora(40, 8192, seed0=500)) + [corpus.generate(1)]:
        m, t, lengths = oracle.train_chunks(d, 200)
        check_invariants(d, m, t, lengths)
        assert np.array_equal(rank_encode(d, m), t)


def test_word_start_is_a_class_change_between_tokens():
    """After any number of merges, a token carries the word-start bit
    exactly when its class (that of its first byte) differs from the class
    of the token before it, or it is the first: a word is a maximal run of
    one class ("Ne Yapar? 1") and no merge crosses a word start, so
    neighbouring words differ in class and every token lies in one word.
    The merge pass stores 16-bit ids and derives the bit this way."""
    cases = list(_small_corpora(30, 8192, seed0=700))
    cases.append(corpus.generate(corpus.CONFIGS[5].scaled(200_000, seed=701)))
    cases.append(np.frombuffer(b"aa  bb\n\n11,,aa", dtype=np.uint8))
    for d in cases:
        for k in (0, 1, 50, 400):
            m, t, _ = oracle.train_chunks(d, k)
            v = vocab_bytes(m)
            cls_of = np.array([CLASS[v[i][0]] for i in range(len(v))], dtype=np.int8)
            c = cls_of[t & ID]
            ws = np.ones(t.size, dtype=bool)
            ws[1:] = c[1:] != c[:-1]
            assert np.array_equal((t & WS) != 0, ws)


def test_invariant_checker_catches_planted_mistakes():
    d = corpus.generate(corpus.CONFIGS[1].scaled(4096, seed=9))
    m, t, lengths = oracle.train_chunks(d, 50)
    check_invariants(d, m, t, lengths)
    bad_t = t.copy(); bad_t[3] ^= WS
    with pytest.raises(AssertionError):
        check_invariants(d, m, bad_t, lengths)
    bad_m = m.copy(); bad_m[[4, 5]] = bad_m[[5, 4]]
    if bad_m[4, 2] != bad_m[5, 2]:
        with pytest.raises(AssertionError):
            check_invariants(d, bad_m, t, lengths)
    i = int(np.flatnonzero((t & ID) != 0x20)[5])
    bad_t2 = t.copy(); bad_t2[i] = (bad_t2[i] & WS) | 0x20
    with pytest.raises(AssertionError):
        check_invariants(d, m, bad_t2, lengths)


def test_early_stop_and_empty_inputs():
    for fn in (oracle.train_python, oracle.train_literal, oracle.train_chunks):
        m, t, lengths = fn(b"", 10)
        assert len(m) == 0 and len(t) == 0 and lengths.tolist() == [0]
        m, t, lengths = fn(b"x", 10)
        assert len(m) == 0 and t.tolist() == [0x78 | WS]
        # "abab": (a,b)=2, then (X,X)=1, then nothing is left
        m, t, lengths = fn(b"abab", 10)
        assert m.tolist() == [[97, 98, 2], [256, 256, 1]] and t.tolist() == [257 | WS]
        assert lengths.tolist() == [4, 2, 1]


def test_merge_count_limit():
    with pytest.raises(ValueError):
        oracle.train_literal(b"ab", 0x10000 - BASE + 1)
    with pytest.raises(ValueError):
        ref.train(b"ab", 0x10000 - BASE + 1)
