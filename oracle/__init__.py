"""CPU oracles for BPE training.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

* ``reference``      - oracle A, the literal definition in pure Python (tiny inputs).
* ``train_literal``  - oracle A in plain C: full recount every iteration.
* ``train_chunks``   - oracle B in plain C: the same result computed on the
                        multiset of distinct chunks with incremental counts.
* ``encode``         - the encoder in plain C: a merge list applied in order
                        (``reference.encode`` is the same in Python).
* ``trie_encode``    - greedy longest-match inference with the vocabulary of a
                        merge list, in plain C over a pointer trie
                        (``reference.trie_encode`` is a dictionary form).

All three return ``(merges, tokens, lengths)``: merges is an int64 array of
shape [k, 3] (left, right, count; merge i creates id 256 + i), tokens a
uint32 array of final symbols (id | 0x10000 on chunk starts), lengths the
sequence length before each merge plus the final length.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import reference  # noqa: F401  (oracle A in Python)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bpe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

WS = 0x10000
ID = 0xFFFF
BASE = 256
MAX_MERGES = 0x10000 - BASE


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
_CHECK_SRC = os.path.join(_HERE, "sanitize_check.c")
_GEN_SRC = os.path.join(os.path.dirname(_HERE), "corpus", "gen.c")


def build(force: bool = True, sanitize: bool = False, out_dir: str | None = None) -> str:
    """Compile bpe_oracle.c into liboracle.so with gcc.

    With ``sanitize``, build instead the executable sanitize_check (the C
    oracle, the corpus generator and sanitize_check.c, which runs the
    brute-force pins through them) with AddressSanitizer and
    UndefinedBehaviorSanitizer, into ``out_dir`` (default: this directory),
    and return its path."""
    if sanitize:
        exe = os.path.join(out_dir or _HERE, "sanitize_check")
        if force or not os.path.exists(exe):
            tmp = exe + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", "-O1", "-std=c11", "-Wall", *SANITIZE_FLAGS, "-o", tmp, _CHECK_SRC, _SRC,
                                   _GEN_SRC, "-lm"])
            os.replace(tmp, exe)
        return exe
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        vp = ctypes.c_void_p
        for fn in (lib.oracle_train_literal, lib.oracle_train_chunks):
            fn.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint32, vp, vp, vp, vp, vp]
            fn.restype = ctypes.c_int
        lib.oracle_char_class.argtypes = [ctypes.c_uint32]
        lib.oracle_char_class.restype = ctypes.c_uint32
        lib.oracle_tag.argtypes = [vp, ctypes.c_uint64, vp]
        lib.oracle_tag.restype = None
        lib.oracle_encode.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_uint32, vp, vp, vp]
        lib.oracle_encode.restype = ctypes.c_int
        lib.oracle_trie_encode.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_uint32, vp, vp]
        lib.oracle_trie_encode.restype = ctypes.c_int
        _lib = lib
    return _lib


def _as_u8(data) -> np.ndarray:
    if isinstance(data, (bytes, bytearray, memoryview)):
        return np.frombuffer(bytes(data), dtype=np.uint8)
    a = np.ascontiguousarray(data)
    if a.dtype != np.uint8:
        raise TypeError("corpus must be uint8 bytes")
    return a.reshape(-1)


def char_class(x: int) -> int:
    return int(_load().oracle_char_class(x))


def tag(data) -> np.ndarray:
    b = _as_u8(data)
    out = np.empty(max(b.size, 1), dtype=np.uint32)
    _load().oracle_tag(b.ctypes.data, b.size, out.ctypes.data)
    return out[: b.size]


def _train(fn, data, n_merges: int, want_tokens: bool = True):
    if not 0 <= n_merges <= MAX_MERGES:
        raise ValueError("n_merges must be in [0, %d]" % MAX_MERGES)
    b = _as_u8(data)
    merges = np.zeros((max(n_merges, 1), 3), dtype=np.uint32)
    tokens = np.empty(max(b.size, 1), dtype=np.uint32) if want_tokens else None
    lengths = np.zeros(n_merges + 1, dtype=np.uint64)
    n_done = ctypes.c_uint32(0)
    n_tok = ctypes.c_uint64(0)
    rc = fn(b.ctypes.data if b.size else None, b.size, n_merges, merges.ctypes.data,
            ctypes.addressof(n_done), tokens.ctypes.data if want_tokens else None,
            ctypes.addressof(n_tok), lengths.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle failed with code %d" % rc)
    k = n_done.value
    return (merges[:k].astype(np.int64), tokens[: n_tok.value] if want_tokens else None,
            lengths[: k + 1].astype(np.int64))


def train_literal(data, n_merges: int, want_tokens: bool = True):
    """Oracle A in C: the definition with a full recount each iteration."""
    return _train(_load().oracle_train_literal, data, n_merges, want_tokens)


def train_chunks(data, n_merges: int, want_tokens: bool = True):
    """Oracle B in C: distinct-chunk multiset with incremental pair counts."""
    return _train(_load().oracle_train_chunks, data, n_merges, want_tokens)


def train_python(data, n_merges: int):
    """Oracle A in pure Python, converted to the same array form."""
    lengths: list[int] = []
    merges, toks = reference.train(bytes(_as_u8(data)), n_merges, lengths)
    return (np.array(merges, dtype=np.int64).reshape(-1, 3), np.array(toks, dtype=np.uint32),
            np.array(lengths, dtype=np.int64))


def encode(data, pairs):
    """The encoder in C: ``pairs`` is [k, 2] (left, right) or [k, 3] (a
    merge list with counts; the counts are ignored). Returns (counts,
    tokens): counts[k] = occurrences of pair k just before merge k."""
    b = _as_u8(data)
    p = np.asarray(pairs, dtype=np.int64)
    p = p.reshape(0, 2) if p.size == 0 else p.reshape(p.shape[0], -1)
    p = np.ascontiguousarray(p[:, :2], dtype=np.uint32)
    k = p.shape[0]
    if k > MAX_MERGES:
        raise ValueError("at most %d merges" % MAX_MERGES)
    counts = np.zeros(max(k, 1), dtype=np.uint32)
    tokens = np.empty(max(b.size, 1), dtype=np.uint32)
    n_tok = ctypes.c_uint64(0)
    rc = _load().oracle_encode(b.ctypes.data if b.size else None, b.size, p.ctypes.data if k else None, k,
                               counts.ctypes.data, tokens.ctypes.data, ctypes.addressof(n_tok))
    if rc == -1:
        raise ValueError("bad merge list (an id that does not exist yet)")
    if rc != 0:
        raise RuntimeError("oracle failed with code %d" % rc)
    return counts[:k].astype(np.int64), tokens[: n_tok.value]


def trie_encode(data, pairs):
    """Greedy longest-match inference in C: ``pairs`` is [k, 2] or [k, 3]
    (counts ignored). Returns the uint32 array of token ids (no flags)."""
    b = _as_u8(data)
    p = np.asarray(pairs, dtype=np.int64)
    p = p.reshape(0, 2) if p.size == 0 else p.reshape(p.shape[0], -1)
    p = np.ascontiguousarray(p[:, :2], dtype=np.uint32)
    k = p.shape[0]
    if k > MAX_MERGES:
        raise ValueError("at most %d merges" % MAX_MERGES)
    tokens = np.empty(max(b.size, 1), dtype=np.uint32)
    n_tok = ctypes.c_uint64(0)
    rc = _load().oracle_trie_encode(b.ctypes.data if b.size else None, b.size, p.ctypes.data if k else None, k,
                                    tokens.ctypes.data, ctypes.addressof(n_tok))
    if rc == -1:
        raise ValueError("bad merge list (an id that does not exist yet)")
    if rc != 0:
        raise RuntimeError("oracle failed with code %d" % rc)
    return tokens[: n_tok.value]
