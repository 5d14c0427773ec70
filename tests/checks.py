"""Independent checks of a BPE training result (merges + final tokens).

These do not reuse the oracle's training loop: they decode, re-encode by
merge rank, and test invariants that any correct result must satisfy.
"""
from __future__ import annotations

import numpy as np

WS = 0x10000
ID = 0xFFFF
BASE = 256


def byte_class(x: int) -> int:
    """Class of a byte as the page states it for char_class ("Satir Satir
    Analiz 1)"): a line break is 4, a space 2, an ASCII digit 1, an ASCII
    letter or any byte of a multi-byte UTF-8 sequence (0x80 and above) 0,
    anything else 3. Written with Python's character predicates, not with
    the oracle's range tests."""
    c = chr(x)
    if x >= 0x80 or (c.isascii() and c.isalpha()):
        return 0
    if c.isascii() and c.isdigit():
        return 1
    return {" ": 2, "\n": 4}.get(c, 3)


CLASS = np.array([byte_class(b) for b in range(256)], dtype=np.int8)


def chunk_starts(data: np.ndarray) -> np.ndarray:
    """Boolean mask of positions that start a chunk (class change or 0)."""
    c = CLASS[data]
    m = np.ones(data.size, dtype=bool)
    if data.size > 1:
        m[1:] = c[1:] != c[:-1]
    return m


def vocab_bytes(merges) -> list[bytes]:
    v = [bytes([i]) for i in range(BASE)]
    for left, right, _ in np.asarray(merges).reshape(-1, 3).tolist():
        v.append(v[left] + v[right])
    return v


def decode(tokens, merges) -> bytes:
    v = vocab_bytes(merges)
    return b"".join(v[int(t) & ID] for t in np.asarray(tokens).tolist())


def check_invariants(data, merges, tokens, lengths=None) -> None:
    """Raise AssertionError if any property of a correct result fails.

    (i) decoding reproduces the input; (ii) no token spans a class change,
    and a token carries the word-start bit iff it starts a chunk; (iv) merge
    counts never increase; (v) no pair is merged twice; (vi) both ids of
    merge k exist before it; lengths (if given) strictly decrease and end at
    the token count."""
    data = np.asarray(data, dtype=np.uint8).reshape(-1)
    merges = np.asarray(merges, dtype=np.int64).reshape(-1, 3)
    tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
    v = vocab_bytes(merges)
    ids = tokens & ID
    assert np.all((tokens >> 17) == 0), "bits above the word-start flag are set"
    assert np.all(ids < BASE + len(merges)), "token id out of range"
    tl = np.array([len(v[i]) for i in ids.tolist()], dtype=np.int64)
    assert int(tl.sum()) == data.size, "decoded length differs from the input"
    assert decode(tokens, merges) == data.tobytes(), "decoding does not reproduce the input"
    starts = np.concatenate([[0], np.cumsum(tl)[:-1]]) if tokens.size else np.zeros(0, np.int64)
    cs = chunk_starts(data)
    # a token spans no class change: no chunk start strictly inside it
    cum = np.concatenate([[0], np.cumsum(cs.astype(np.int64))])
    inside = cum[starts + tl] - cum[starts + 1] if tokens.size else np.zeros(0)
    assert np.all(inside == 0), "a token spans a class change"
    assert np.array_equal((tokens & WS) != 0, cs[starts]), "word-start bit does not match chunk starts"
    if len(merges):
        c = merges[:, 2]
        assert np.all(c >= 1), "merge with zero count"
        assert np.all(c[1:] <= c[:-1]), "merge counts increase"
        keys = merges[:, 0] * 65536 + merges[:, 1]
        assert np.unique(keys).size == keys.size, "a pair is merged twice"
        k = np.arange(len(merges))
        assert np.all(merges[:, 0] < BASE + k) and np.all(merges[:, 1] < BASE + k), "merge uses a future id"
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        assert lengths[0] == data.size and lengths[-1] == tokens.size
        assert len(lengths) == len(merges) + 1
        assert np.all(np.diff(lengths) < 0), "a merge did not shrink the sequence"


def rank_encode(data, merges) -> np.ndarray:
    """Encode data with a learned merge list by merge rank: inside each chunk,
    repeatedly replace the lowest-rank adjacent pair (all its occurrences,
    left to right) until no ranked pair is left. Training on the same bytes
    must produce exactly this sequence."""
    data = np.asarray(data, dtype=np.uint8).reshape(-1)
    merges = np.asarray(merges, dtype=np.int64).reshape(-1, 3)
    rank = {(int(a), int(b)): i for i, (a, b, _) in enumerate(merges.tolist())}
    cs = chunk_starts(data)
    bounds = np.flatnonzero(cs).tolist() + [data.size]
    raw = data.tobytes()
    cache: dict[bytes, list[int]] = {}
    out: list[int] = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        ch = raw[a:b]
        enc = cache.get(ch)
        if enc is None:
            s = list(ch)
            while len(s) > 1:
                best = None
                for i in range(len(s) - 1):
                    r = rank.get((s[i], s[i + 1]))
                    if r is not None and (best is None or r < best):
                        best = r
                if best is None:
                    break
                left, right = merges[best, 0], merges[best, 1]
                t, i = [], 0
                while i < len(s):
                    if i + 1 < len(s) and s[i] == left and s[i + 1] == right:
                        t.append(BASE + best)
                        i += 2
                    else:
                        t.append(s[i])
                        i += 1
                s = t
            enc = s
            cache[ch] = enc
        out.append(enc[0] | WS)
        out.extend(enc[1:])
    return np.array(out, dtype=np.uint32)


def selected_occurrences(s: list[int], left: int, right: int) -> int:
    """Closed form of the shrink of one merge: split the occurrences of
    (left, right) into maximal chains of consecutive positions; a chain of
    m occurrences removes ceil(m / 2) symbols (only m = 1 chains exist
    when left != right)."""
    occ = [i for i in range(1, len(s))
           if not (s[i] & WS) and (s[i - 1] & ID) == left and (s[i] & ID) == right]
    total, run, prev = 0, 0, -2
    for i in occ:
        run = run + 1 if i == prev + 1 else 1
        prev = i
        total += 1 if run % 2 == 1 else 0
    return total
