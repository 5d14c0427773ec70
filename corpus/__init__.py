"""Seeded synthetic corpora (bytes only).

This package makes the input bytes that both the oracle and the GPU path
train on. It contains none of the training method's arithmetic. The five
workloads below follow the corpus descriptions of the BPE training
benchmark (sizes, vocabulary sizes, Zipf exponents, digit/punctuation
rates, letter mixes); the concrete choices the descriptions leave open are
fixed in ``gen.c``.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libcorpus.so")
_lib = None


def build(force: bool = True, sanitize: bool = False, out_dir: str | None = None) -> str:
    """Compile gen.c into libcorpus.so with gcc (host code only).

    With ``sanitize``, build the sanitizer checker that links gen.c with the
    C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (see
    ``oracle.build``) and return the executable's path."""
    if sanitize:
        import oracle
        return oracle.build(force=force, sanitize=True, out_dir=out_dir)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.corpus_words.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                     ctypes.c_double, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_uint32]
        lib.corpus_words.restype = ctypes.c_int
        lib.corpus_runs.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, ctypes.c_double]
        lib.corpus_runs.restype = ctypes.c_int
        u64p = ctypes.POINTER(ctypes.c_uint64)
        lib.corpus_rng_raw.argtypes = [ctypes.c_uint64, u64p, ctypes.c_uint64]
        lib.corpus_rng_raw.restype = None
        lib.corpus_splitmix_raw.argtypes = [ctypes.c_uint64, u64p, ctypes.c_uint64]
        lib.corpus_splitmix_raw.restype = ctypes.c_uint64
        lib.corpus_rng_raw_state.argtypes = [u64p, u64p, ctypes.c_uint64]
        lib.corpus_rng_raw_state.restype = None
        _lib = lib
    return _lib


@dataclass(frozen=True)
class CorpusSpec:
    """One benchmark workload: corpus recipe plus training parameters."""
    name: str
    kind: str               # "words" or "runs"
    n_bytes: int
    seed: int
    n_merges: int
    table_log2: int
    n_words: int = 0
    zipf_s: float = 0.0
    min_len: int = 0
    max_len: int = 0
    alphabet: int = 0       # 0 ascii a..z, 1 Turkish 29 letters, 2 mixed 1/2/3-byte
    digit_p: float = 0.0
    punct_p: float = 0.0
    max_digits: int = 4
    run_mean: float = 0.0
    rand_mean: float = 0.0

    def scaled(self, n_bytes: int, n_merges: int | None = None, seed: int | None = None) -> "CorpusSpec":
        """Same recipe at another size (and optionally another merge count / seed)."""
        return replace(self, n_bytes=int(n_bytes),
                       n_merges=self.n_merges if n_merges is None else int(n_merges),
                       seed=self.seed if seed is None else int(seed))


MiB = 1 << 20
CONFIGS = {
    1: CorpusSpec("ascii64k", "words", 64 * 1024, 1, 200, 17, n_words=500, zipf_s=1.1, min_len=2,
                  max_len=8, alphabet=0, digit_p=0.03, punct_p=0.02, max_digits=4),
    2: CorpusSpec("turkish16m", "words", 16 * MiB, 2, 8000, 21, n_words=50_000, zipf_s=1.1, min_len=2,
                  max_len=14, alphabet=1, digit_p=0.05, punct_p=0.03, max_digits=6),
    3: CorpusSpec("ascii256m", "words", 256 * MiB, 3, 32000, 22, n_words=200_000, zipf_s=1.05,
                  min_len=2, max_len=8, alphabet=0, digit_p=0.03, punct_p=0.02, max_digits=4),
    4: CorpusSpec("mixed1g", "words", 1024 * MiB, 4, 64000, 24, n_words=1_000_000, zipf_s=1.0,
                  min_len=2, max_len=8, alphabet=2, digit_p=0.03, punct_p=0.02, max_digits=4),
    5: CorpusSpec("runs128m", "runs", 128 * MiB, 5, 4000, 23, run_mean=64.0, rand_mean=256.0),
}


def generate(spec: CorpusSpec | int, out: np.ndarray | None = None) -> np.ndarray:
    """Fill (or allocate) a uint8 array with the corpus of ``spec``."""
    if isinstance(spec, int):
        spec = CONFIGS[spec]
    lib = _load()
    n = spec.n_bytes
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    if out.dtype != np.uint8 or out.size < n or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous uint8 array of at least n_bytes")
    ptr = out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    if spec.kind == "words":
        rc = lib.corpus_words(ptr, n, spec.seed, spec.n_words, spec.zipf_s, spec.min_len, spec.max_len,
                              spec.alphabet, spec.digit_p, spec.punct_p, spec.max_digits)
    elif spec.kind == "runs":
        rc = lib.corpus_runs(ptr, n, spec.seed, spec.run_mean, spec.rand_mean)
    else:
        raise ValueError("unknown corpus kind %r" % spec.kind)
    if rc != 0:
        raise RuntimeError("corpus generation failed for %s" % spec.name)
    return out[:n]


def sha256(data: np.ndarray) -> str:
    return hashlib.sha256(memoryview(np.ascontiguousarray(data))).hexdigest()


def rng_raw(seed: int, count: int) -> np.ndarray:
    """First ``count`` outputs of the seeded xoshiro256** stream."""
    out = np.empty(count, dtype=np.uint64)
    _load().corpus_rng_raw(seed, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), count)
    return out


def splitmix_raw(seed: int, count: int) -> np.ndarray:
    """First ``count`` outputs of SplitMix64 started at ``seed``."""
    out = np.empty(count, dtype=np.uint64)
    _load().corpus_splitmix_raw(seed, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), count)
    return out


def rng_raw_state(state, count: int) -> np.ndarray:
    """xoshiro256** outputs from an explicit 4-word state."""
    st = np.ascontiguousarray(np.asarray(state, dtype=np.uint64))
    out = np.empty(count, dtype=np.uint64)
    p = ctypes.POINTER(ctypes.c_uint64)
    _load().corpus_rng_raw_state(st.ctypes.data_as(p), out.ctypes.data_as(p), count)
    return out
