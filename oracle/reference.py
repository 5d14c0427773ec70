"""Oracle A: BPE training written out literally, in plain Python.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module;
only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark do.

Sources (page "bpe - GPU BPE Tokenizer Pipeline (Egitim + Cikarim)",
llm.istanbul/learn/tr/13_bpe):

* "Nedir bu ya?": training repeatedly finds the most frequent adjacent pair
  of symbols, gives it one new symbol, and repeats.
* "Ne Yapar? section 1 (bpe_word_boundary)": every symbol gets a character
  class (Letter, Digit, Space, Punct, Newline); at a class change that
  symbol is tagged with WORD_START_BIT = 0x10000, and pair counting does not
  count across that bit.
* "Satir Satir Analiz 1) char_class": the class function, byte by byte.
* Head of the page (training pipeline list): the table is cleared and all
  pairs are counted again on every iteration, then a deterministic maximum
  is taken.
* "Ne Yapar? section 3": the merged symbol carries WORD_START_BIT.
* "Nedir bu ya?" again, for encoding: text is encoded with a learned merge
  list by applying its merges in the order they were learned.
* "Nedir bu ya?", inference paragraph, and "Ne Yapar? 4": inference walks a
  prefix tree of the vocabulary and takes, at each position, the longest
  vocabulary string the text continues with (greedy longest match).

Readings where the page is silent (each one also listed in the design notes):
  - position 0 carries WORD_START_BIT (the first symbol starts a word);
  - the bit goes on the right-hand symbol of a class change;
  - every adjacent position is counted, overlapping ones included (aaa -> 2);
  - ties go to the smallest (left, right) pair; the new id is 256 + k;
  - merging is left to right and non-overlapping, and never crosses the bit;
  - the merged symbol keeps the left symbol's bit; tagging happens once;
  - training stops early when no countable pair is left (any count >= 1 merges).

Symbols are 32-bit: bits 0-15 hold the id, bit 16 the word-start flag.
"""
from __future__ import annotations

WS = 0x10000          # WORD_START_BIT
ID = 0xFFFF           # id field of a symbol
BASE = 256            # byte-level base vocabulary: new ids start here
MAX_MERGES = 0x10000 - BASE   # ids must fit in 16 bits


# Byte classes of the page's char_class ("Satir Satir Analiz 1)"), as sets:
# letters are the ASCII letters and every byte of a multi-byte UTF-8
# sequence (so UTF-8 letters stay letters); 3 is everything not listed.
_CLASS_MEMBERS = {
    0: set(range(ord("A"), ord("Z") + 1)) | set(range(ord("a"), ord("z") + 1)) | set(range(0x80, 0x100)),
    1: set(range(ord("0"), ord("9") + 1)),
    2: {ord(" ")},
    4: {ord("\n")},
}


def char_class(x: int) -> int:
    """Character class of one byte: newline 4, space 2, ASCII digit 1, any
    byte >= 0x80 and ASCII letters 0, everything else 3."""
    for cls, members in _CLASS_MEMBERS.items():
        if x in members:
            return cls
    return 3


def tag(data: bytes) -> list[int]:
    """Byte -> symbol, with WORD_START_BIT where the class changes (and at 0)."""
    s = []
    for i, b in enumerate(data):
        start = i == 0 or char_class(b) != char_class(data[i - 1])
        s.append(b | (WS if start else 0))
    return s


def count_pairs(s: list[int]) -> dict[tuple[int, int], int]:
    """Exact count of every adjacent (left id, right id) whose right symbol
    does not carry the word-start bit; overlapping positions all count."""
    c: dict[tuple[int, int], int] = {}
    for i in range(1, len(s)):
        if not (s[i] & WS):
            p = (s[i - 1] & ID, s[i] & ID)
            c[p] = c.get(p, 0) + 1
    return c


def best_pair(c: dict[tuple[int, int], int]) -> tuple[int, int]:
    """Highest count; among equal counts the smallest (left, right)."""
    return min(c, key=lambda p: (-c[p], p))


def merge_pair(s: list[int], left: int, right: int, new_id: int) -> list[int]:
    """Replace occurrences of (left, right) scanning left to right, never
    reusing a symbol that was just merged and never crossing a word start.
    The merged symbol keeps the left symbol's word-start bit."""
    t = []
    i = 0
    while i < len(s):
        if (i + 1 < len(s) and not (s[i + 1] & WS)
                and (s[i] & ID) == left and (s[i + 1] & ID) == right):
            t.append(new_id | (s[i] & WS))
            i += 2
        else:
            t.append(s[i])
            i += 1
    return t


def step(s: list[int], k: int):
    """One training iteration k on sequence s.

    Returns ((left, right, count), new_s), or (None, s) if no pair is left."""
    c = count_pairs(s)
    if not c:
        return None, s
    left, right = best_pair(c)
    return (left, right, c[(left, right)]), merge_pair(s, left, right, BASE + k)


def train(data: bytes, n_merges: int, lengths: list[int] | None = None):
    """Train up to n_merges merges on data.

    Returns (merges, tokens): merges is a list of (left, right, count) with
    merge k creating id 256 + k; tokens are the final symbols (id | bit).
    If ``lengths`` is given, the sequence length before each merge and the
    final length are appended to it."""
    if not 0 <= n_merges <= MAX_MERGES:
        raise ValueError("n_merges must be in [0, %d]" % MAX_MERGES)
    s = tag(bytes(data))
    merges = []
    for k in range(n_merges):
        if lengths is not None:
            lengths.append(len(s))
        m, s2 = step(s, k)
        if m is None:
            if lengths is not None:
                lengths.pop()
            break
        merges.append(m)
        s = s2
    if lengths is not None:
        lengths.append(len(s))
    return merges, s


def encode(data: bytes, pairs):
    """Encode data with a merge list: tag it, then apply merge k (the pair
    pairs[k] = (left, right), new id 256 + k) over the whole sequence for
    k = 0, 1, ... in order, each exactly as a training iteration applies
    its chosen pair. Returns (counts, tokens): counts[k] is the number of
    adjacent positions holding pairs[k] just before merge k (0 if none),
    tokens the final symbols. A pair naming an id that does not exist yet
    (>= 256 + k) is an error."""
    s = tag(bytes(data))
    counts = []
    for k, (left, right) in enumerate(pairs):
        if not (0 <= left < BASE + k and 0 <= right < BASE + k):
            raise ValueError("merge %d names an id that does not exist yet" % k)
        counts.append(count_pairs(s).get((left, right), 0))
        s = merge_pair(s, left, right, BASE + k)
    return counts, s


def vocab_strings(pairs) -> list[bytes]:
    """The byte string of every id of a merge list: id b < 256 is the byte
    b, id 256 + k the string of pairs[k][0] followed by that of pairs[k][1]."""
    out = [bytes([b]) for b in range(BASE)]
    for k, (left, right) in enumerate(pairs):
        if not (0 <= left < BASE + k and 0 <= right < BASE + k):
            raise ValueError("merge %d names an id that does not exist yet" % k)
        out.append(out[left] + out[right])
    return out


def trie_encode(data: bytes, pairs) -> list[int]:
    """Greedy longest-match inference with the vocabulary of a merge list:
    from the current position, emit the id of the longest vocabulary string
    that the text continues with there and move past it. Every single byte
    is in the vocabulary, so some string always matches. A string that
    several ids spell maps to the smallest of them. Tokens are plain ids."""
    data = bytes(data)
    vocab: dict[bytes, int] = {}
    for i, v in enumerate(vocab_strings(pairs)):
        vocab.setdefault(v, i)
    longest = max(len(v) for v in vocab)
    out = []
    i = 0
    while i < len(data):
        for ln in range(min(longest, len(data) - i), 0, -1):
            t = vocab.get(data[i:i + ln])
            if t is not None:
                out.append(t)
                i += ln
                break
    return out
