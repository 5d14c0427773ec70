"""Python binding of the MI355X BPE training library (``libbpe.so``).

Argument marshalling only: every step of training runs in the library's HIP
kernels; torch supplies device memory (inputs, outputs, workspace) and the
stream. The C functions keep their names (``bpe_train`` -> ``train`` etc.);
``include/bpe.h`` documents arguments, layouts, ownership and errors.

Importing fails loudly if the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbpe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("bpe_merge_amd: %s is not built (run __graft_entry__.build())" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

OK, DONE = 0, 1
EINVAL, ETABLE, EIDSPACE, ENOMEM, EHIP, ESTATE = -1, -2, -3, -4, -5, -6
WORD_START = 0x10000
ID_MASK = 0xFFFF
BASE_VOCAB = 256
MAX_MERGES = 65280
MAX_BYTES = 0x7FFFFFFF
FLAG_OVERSUBSCRIBE = 1  # testing aid: merge passes with 4x the resident workgroups
FLAG_ALWAYS_CHUNKS = 2  # train_chunked: over the distinct words whatever memory their records take


class BpeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.bpe_strerror(status).decode()
        detail = _lib.bpe_last_error().decode()
        super().__init__("%s: %s%s" % (where, msg, (" (%s)" % detail) if detail else ""))


class Config(ctypes.Structure):
    _fields_ = [("table_log2", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class Merge(ctypes.Structure):
    _fields_ = [("left", ctypes.c_uint32), ("right", ctypes.c_uint32), ("count", ctypes.c_uint32)]


class ProfileResult(ctypes.Structure):
    _fields_ = [("merge_ms", ctypes.c_double), ("launches", ctypes.c_uint32), ("merges_done", ctypes.c_uint32),
                ("sweeps", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_vp, _sz, _u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32
_cfgp = ctypes.POINTER(Config)
_SIGS = {
    "bpe_workspace_bytes": (_sz, [_sz, _cfgp]),
    "bpe_train": (ctypes.c_int, [_vp, _sz, _u32, _cfgp, _vp, ctypes.POINTER(_u32), _vp, _sz,
                                 ctypes.POINTER(_sz)]),
    "bpe_train_chunked": (ctypes.c_int, [_vp, _sz, _u32, _cfgp, _vp, ctypes.POINTER(_u32), _vp, _sz,
                                         ctypes.POINTER(_sz)]),
    "bpe_train_static": (ctypes.c_int, [_vp, _sz, _u32, _u32, _vp, _vp, ctypes.POINTER(_u32), _vp, _sz,
                                        ctypes.POINTER(_sz)]),
    "bpe_init": (ctypes.c_int, [_vp, _sz, _cfgp, ctypes.POINTER(_vp)]),
    "bpe_run": (ctypes.c_int, [_vp, _u32]),
    "bpe_sync": (ctypes.c_int, [_vp, ctypes.POINTER(_u32)]),
    "bpe_step": (ctypes.c_int, [_vp, ctypes.POINTER(Merge)]),
    "bpe_merges": (ctypes.c_int, [_vp, _vp, _u32, ctypes.POINTER(_u32)]),
    "bpe_tokens": (ctypes.c_int, [_vp, _vp, _sz, ctypes.POINTER(_sz)]),
    "bpe_lengths": (ctypes.c_int, [_vp, _vp, _u32, ctypes.POINTER(_u32)]),
    "bpe_pair_counts": (ctypes.c_int, [_vp, _vp, _vp, _sz, ctypes.POINTER(_sz)]),
    "bpe_table_usage": (ctypes.c_int, [_vp, ctypes.POINTER(_u32), ctypes.POINTER(_u32), ctypes.POINTER(_u32)]),
    "bpe_profile": (ctypes.c_int, [_vp, _u32, ctypes.POINTER(ProfileResult), _vp]),
    "bpe_replay": (ctypes.c_int, [_vp, _vp, _u32]),
    "bpe_encode": (ctypes.c_int, [_vp, _sz, _vp, _u32, _cfgp, _vp, _sz, ctypes.POINTER(_sz)]),
    "bpe_trie_build": (ctypes.c_int, [_vp, _u32, ctypes.POINTER(_vp)]),
    "bpe_trie_info": (ctypes.c_int, [_vp, ctypes.POINTER(_u32), ctypes.POINTER(_u32)]),
    "bpe_trie_encode": (ctypes.c_int, [_vp, _vp, _sz, _vp, _vp, _sz, ctypes.POINTER(_sz)]),
    "bpe_trie_profile": (ctypes.c_int, [_vp, _vp, _sz, _u32, _vp, ctypes.POINTER(_sz)]),
    "bpe_trie_free": (None, [_vp]),
    "bpe_encoder_build": (ctypes.c_int, [_vp, _u32, ctypes.POINTER(_vp)]),
    "bpe_encoder_encode": (ctypes.c_int, [_vp, _vp, _sz, _vp, _vp, _sz, ctypes.POINTER(_sz)]),
    "bpe_encoder_profile": (ctypes.c_int, [_vp, _vp, _sz, _u32, _vp, ctypes.POINTER(_sz)]),
    "bpe_encoder_free": (None, [_vp]),
    "bpe_encoder_cache": (ctypes.c_int, [_vp, _u32, _u32]),
    "bpe_free": (None, [_vp]),
    "bpe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "bpe_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def _check(st: int, where: str) -> int:
    if st < 0:
        raise BpeError(st, where)
    return st


def _config(table_log2=None, stream=None, workspace=None, flags=0) -> Config:
    c = Config()
    c.table_log2 = int(table_log2 or 0)
    c.flags = int(flags)
    c.stream = stream
    if workspace is not None:
        c.workspace = workspace.data_ptr()
        c.workspace_bytes = workspace.numel() * workspace.element_size()
    return c


def _torch():
    import torch
    return torch


def _stream_handle(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(n: int, table_log2: int | None = None) -> int:
    """bpe_workspace_bytes: device workspace for n corpus bytes (0 if invalid)."""
    cfg = _config(table_log2)
    return int(_lib.bpe_workspace_bytes(n, ctypes.byref(cfg)))


def _workspace(n, table_log2, device):
    torch = _torch()
    nbytes = workspace_bytes(n, table_log2)
    if nbytes == 0:
        raise BpeError(EINVAL, "bpe_workspace_bytes")
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    shift = (-ws.data_ptr()) % 256
    return ws[shift: shift + nbytes]


def train(data, n_merges: int, table_log2: int | None = None, flags: int = 0):
    """bpe_train on a uint8 CUDA tensor.

    Returns (merges, tokens): int32 CUDA tensors of shape [k, 3] (left,
    right, count; merge i creates id 256 + i) and [n_final] (id | 0x10000
    on word starts)."""
    torch = _torch()
    if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
        raise TypeError("data must be a uint8 CUDA tensor")
    data = data.contiguous().reshape(-1)
    n = data.numel()
    dev = data.device
    merges = torch.empty((max(n_merges, 1), 3), dtype=torch.int32, device=dev)
    tokens = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    if n == 0:
        return merges[:0], tokens[:0]
    ws = _workspace(n, table_log2, dev)
    cfg = _config(table_log2, _stream_handle(dev), ws, flags)
    n_done = _u32(0)
    n_tok = _sz(0)
    st = _lib.bpe_train(data.data_ptr(), n, n_merges, ctypes.byref(cfg), merges.data_ptr(), ctypes.byref(n_done),
                        tokens.data_ptr(), tokens.numel(), ctypes.byref(n_tok))
    _check(st, "bpe_train")
    return merges[: n_done.value], tokens[: n_tok.value]


def train_chunked(data, n_merges: int, table_log2: int | None = None, tokens: bool = True,
                  always_chunks: bool = False):
    """bpe_train_chunked on a uint8 CUDA tensor: training over the corpus's
    distinct words, each weighted by its frequency (or over the full symbol
    array where their records would take more than 8 bytes per input
    byte, unless always_chunks). Returns (merges, tokens) as train() does (tokens is
    None when tokens=False)."""
    torch = _torch()
    if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
        raise TypeError("data must be a uint8 CUDA tensor")
    data = data.contiguous().reshape(-1)
    n = data.numel()
    dev = data.device
    merges = torch.empty((max(n_merges, 1), 3), dtype=torch.int32, device=dev)
    tok = torch.empty(max(n, 1), dtype=torch.int32, device=dev) if tokens else None
    cfg = _config(table_log2, _stream_handle(dev), flags=FLAG_ALWAYS_CHUNKS if always_chunks else 0)
    n_done = _u32(0)
    n_tok = _sz(0)
    st = _lib.bpe_train_chunked(data.data_ptr() if n else None, n, n_merges, ctypes.byref(cfg), merges.data_ptr(),
                                ctypes.byref(n_done), tok.data_ptr() if tokens else None,
                                tok.numel() if tokens else 0, ctypes.byref(n_tok) if tokens else None)
    _check(st, "bpe_train_chunked")
    return merges[: n_done.value], (tok[: n_tok.value] if tokens else None)


STATIC_SCRATCH_BYTES = 32 << 20
STATIC_MAX_BYTES = 2 << 20
STATIC_MAX_TABLE_LOG2 = 20


def train_static(data, n_merges: int, table_log2: int | None = None):
    """bpe_train_static on a uint8 CUDA tensor: training in the library's own
    static workspace (no device allocation by the library; at most
    STATIC_MAX_BYTES bytes). Returns (merges, tokens) as train() does; the
    output tensors are allocated here, by torch, before the call."""
    torch = _torch()
    if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
        raise TypeError("data must be a uint8 CUDA tensor")
    data = data.contiguous().reshape(-1)
    n = data.numel()
    dev = data.device
    merges = torch.empty((max(n_merges, 1), 3), dtype=torch.int32, device=dev)
    tokens = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    n_done = _u32(0)
    n_tok = _sz(0)
    st = _lib.bpe_train_static(data.data_ptr() if n else None, n, n_merges, int(table_log2 or 0),
                               _stream_handle(dev), merges.data_ptr(), ctypes.byref(n_done), tokens.data_ptr(),
                               tokens.numel(), ctypes.byref(n_tok))
    _check(st, "bpe_train_static")
    return merges[: n_done.value], tokens[: n_tok.value]


def _merge_list(merges, device):
    """A [k, 2] or [k, 3] merge list as a contiguous int32 [k, 3] CUDA tensor
    (bpe_merge layout: left, right, count; the count is not read)."""
    torch = _torch()
    m = torch.as_tensor(merges)
    if m.numel() == 0:
        m = m.reshape(0, 3)
    if m.dim() != 2 or m.shape[1] not in (2, 3):
        raise ValueError("merges must have shape [k, 2] or [k, 3]")
    if m.shape[1] == 2:
        m = torch.cat([m, torch.zeros((m.shape[0], 1), dtype=m.dtype, device=m.device)], dim=1)
    return m.to(device=device, dtype=torch.int32).contiguous()


def encode(data, merges, table_log2: int | None = None):
    """bpe_encode on a uint8 CUDA tensor with a merge list ([k, 2] or [k, 3];
    merge i creates id 256 + i). Returns the int32 CUDA tensor of final
    symbols (id | 0x10000 on word starts). table_log2 is accepted for the
    bpe_config but not used by encoding."""
    torch = _torch()
    if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
        raise TypeError("data must be a uint8 CUDA tensor")
    data = data.contiguous().reshape(-1)
    n = data.numel()
    dev = data.device
    m = _merge_list(merges, dev)
    tokens = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    if n == 0:
        return tokens[:0]
    ws = _workspace(n, table_log2, dev)
    cfg = _config(table_log2, _stream_handle(dev), ws)
    n_tok = _sz(0)
    _check(_lib.bpe_encode(data.data_ptr(), n, m.data_ptr(), m.shape[0], ctypes.byref(cfg), tokens.data_ptr(),
                           tokens.numel(), ctypes.byref(n_tok)), "bpe_encode")
    return tokens[: n_tok.value]


class Encoder:
    """bpe_encoder_build ... bpe_encoder_free: a merge list ([k, 2] or [k, 3];
    merge i is id 256 + i) applied to new text word by word, lowest rank
    first, on the current CUDA device. Tokens carry 0x10000 on word starts."""

    def __init__(self, merges):
        torch = _torch()
        dev = torch.device("cuda", torch.cuda.current_device())
        m = _merge_list(merges, dev)
        self.device = dev
        self._h = _vp(None)
        _check(_lib.bpe_encoder_build(m.data_ptr() if m.numel() else None, m.shape[0], ctypes.byref(self._h)),
               "bpe_encoder_build")

    def encode(self, data, out=None):
        """Encode a uint8 CUDA tensor on the current stream; returns the int32
        CUDA tensor of tokens (a prefix of ``out`` if given)."""
        torch = _torch()
        if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
            raise TypeError("data must be a uint8 CUDA tensor")
        data = data.contiguous().reshape(-1)
        n = data.numel()
        if out is None:
            out = torch.empty(max(n, 1), dtype=torch.int32, device=data.device)
        if not (out.is_cuda and out.dtype == torch.int32 and out.is_contiguous() and out.numel() >= n):
            raise ValueError("out must be a contiguous int32 CUDA tensor with room for n tokens")
        n_tok = _sz(0)
        _check(_lib.bpe_encoder_encode(self._h, data.data_ptr() if n else None, n, _stream_handle(data.device),
                                       out.data_ptr(), out.numel(), ctypes.byref(n_tok)), "bpe_encoder_encode")
        return out[: n_tok.value]

    def profile(self, data, reps: int):
        """bpe_encoder_profile: (n_tokens, device ms of shape [reps, 4]: word
        cache, walk, scan and copy of each run)."""
        import numpy as np
        data = data.contiguous().reshape(-1)
        ms = np.zeros(4 * max(reps, 1), dtype=np.float32)
        n_tok = _sz(0)
        _check(_lib.bpe_encoder_profile(self._h, data.data_ptr(), data.numel(), reps, ms.ctypes.data,
                                        ctypes.byref(n_tok)), "bpe_encoder_profile")
        return n_tok.value, ms[: 4 * reps].reshape(reps, 4)

    CACHE_AUTO = 0xFFFFFFFF
    CACHE_KEY_BITS = 32

    def cache(self, log2_slots=CACHE_AUTO, key_bits=CACHE_KEY_BITS):
        """bpe_encoder_cache: word-cache size for later calls (CACHE_AUTO, 0 =
        off, or 8..24) and key bits (fewer share keys more; a testing aid)."""
        _check(_lib.bpe_encoder_cache(self._h, log2_slots, key_bits), "bpe_encoder_cache")
        return self

    def free(self) -> None:
        if self._h:
            _lib.bpe_encoder_free(self._h)
            self._h = _vp(None)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Trie:
    """bpe_trie_build ... bpe_trie_free: greedy longest-match inference with
    the vocabulary of a merge list ([k, 2] or [k, 3]; merge i is id 256 + i),
    built on the current CUDA device."""

    def __init__(self, merges):
        torch = _torch()
        dev = torch.device("cuda", torch.cuda.current_device())
        m = _merge_list(merges, dev)
        self.device = dev
        self._h = _vp(None)
        _check(_lib.bpe_trie_build(m.data_ptr() if m.numel() else None, m.shape[0], ctypes.byref(self._h)),
               "bpe_trie_build")

    def info(self):
        """(slots of the double array, longest vocabulary string in bytes)."""
        a, b = _u32(0), _u32(0)
        _check(_lib.bpe_trie_info(self._h, ctypes.byref(a), ctypes.byref(b)), "bpe_trie_info")
        return a.value, b.value

    def encode(self, data, out=None):
        """Tokenize a uint8 CUDA tensor on the current stream. Returns the
        int32 CUDA tensor of token ids (a prefix of ``out`` if given; it
        needs room for data.numel() ids)."""
        torch = _torch()
        if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
            raise TypeError("data must be a uint8 CUDA tensor")
        data = data.contiguous().reshape(-1)
        n = data.numel()
        if out is None:
            out = torch.empty(max(n, 1), dtype=torch.int32, device=data.device)
        if not (out.is_cuda and out.dtype == torch.int32 and out.is_contiguous() and out.numel() >= n):
            raise ValueError("out must be a contiguous int32 CUDA tensor with room for n ids")
        n_tok = _sz(0)
        _check(_lib.bpe_trie_encode(self._h, data.data_ptr() if n else None, n, _stream_handle(data.device),
                                    out.data_ptr(), out.numel(), ctypes.byref(n_tok)), "bpe_trie_encode")
        return out[: n_tok.value]

    def profile(self, data, reps: int):
        """bpe_trie_profile: (n_tokens, device ms as a numpy array of shape
        [reps, 3]: walk, scan and copy kernels of each run)."""
        import numpy as np
        data = data.contiguous().reshape(-1)
        ms = np.zeros(3 * max(reps, 1), dtype=np.float32)
        n_tok = _sz(0)
        _check(_lib.bpe_trie_profile(self._h, data.data_ptr(), data.numel(), reps, ms.ctypes.data,
                                     ctypes.byref(n_tok)), "bpe_trie_profile")
        return n_tok.value, ms[: 3 * reps].reshape(reps, 3)

    def count(self, data) -> int:
        """Number of tokens only (no token output)."""
        torch = _torch()
        if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
            raise TypeError("data must be a uint8 CUDA tensor")
        data = data.contiguous().reshape(-1)
        n_tok = _sz(0)
        _check(_lib.bpe_trie_encode(self._h, data.data_ptr() if data.numel() else None, data.numel(),
                                    _stream_handle(data.device), None, 0, ctypes.byref(n_tok)), "bpe_trie_encode")
        return n_tok.value

    def free(self) -> None:
        if self._h:
            _lib.bpe_trie_free(self._h)
            self._h = _vp(None)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class State:
    """bpe_init ... bpe_free on a uint8 CUDA tensor, with a torch workspace."""

    def __init__(self, data, table_log2: int | None = None, flags: int = 0):
        torch = _torch()
        if not (isinstance(data, torch.Tensor) and data.is_cuda and data.dtype == torch.uint8):
            raise TypeError("data must be a uint8 CUDA tensor")
        self.data = data.contiguous().reshape(-1)
        self.n = self.data.numel()
        self.device = self.data.device
        self.ws = _workspace(self.n, table_log2, self.device)
        self.cfg = _config(table_log2, _stream_handle(self.device), self.ws, flags)
        self._h = _vp(None)
        _check(_lib.bpe_init(self.data.data_ptr(), self.n, ctypes.byref(self.cfg), ctypes.byref(self._h)),
               "bpe_init")

    def run(self, n_merges: int) -> None:
        _check(_lib.bpe_run(self._h, n_merges), "bpe_run")

    def sync(self) -> int:
        d = _u32(0)
        _check(_lib.bpe_sync(self._h, ctypes.byref(d)), "bpe_sync")
        return d.value

    def step(self):
        m = Merge()
        st = _check(_lib.bpe_step(self._h, ctypes.byref(m)), "bpe_step")
        return None if st == DONE else (m.left, m.right, m.count)

    def replay(self, merges) -> None:
        """bpe_replay: apply a merge list ([k, 2] or [k, 3]) as the next k
        iterations; training can continue afterwards."""
        m = _merge_list(merges, self.device)
        _check(_lib.bpe_replay(self._h, m.data_ptr(), m.shape[0]), "bpe_replay")

    def merges(self):
        torch = _torch()
        k = _u32(0)
        _check(_lib.bpe_merges(self._h, None, 0, ctypes.byref(k)), "bpe_merges")
        out = torch.empty((max(k.value, 1), 3), dtype=torch.int32, device=self.device)
        _check(_lib.bpe_merges(self._h, out.data_ptr(), k.value, ctypes.byref(k)), "bpe_merges")
        return out[: k.value]

    def tokens(self):
        torch = _torch()
        n = _sz(0)
        _check(_lib.bpe_tokens(self._h, None, 0, ctypes.byref(n)), "bpe_tokens")
        out = torch.empty(max(n.value, 1), dtype=torch.int32, device=self.device)
        _check(_lib.bpe_tokens(self._h, out.data_ptr(), out.numel(), ctypes.byref(n)), "bpe_tokens")
        return out[: n.value]

    def lengths(self):
        torch = _torch()
        c = _u32(0)
        _check(_lib.bpe_lengths(self._h, None, 0, ctypes.byref(c)), "bpe_lengths")
        out = torch.empty(max(c.value, 1), dtype=torch.int32, device=self.device)
        _check(_lib.bpe_lengths(self._h, out.data_ptr(), c.value, ctypes.byref(c)), "bpe_lengths")
        return out[: c.value]

    def table_usage(self):
        """bpe_table_usage: (slots, claimed slots, claim limit) of the pair table."""
        a, b, c = _u32(0), _u32(0), _u32(0)
        _check(_lib.bpe_table_usage(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "bpe_table_usage")
        return a.value, b.value, c.value

    def pair_counts(self):
        """(keys, counts) int64 host arrays of the current pair table, sorted by key."""
        import numpy as np
        n = _sz(0)
        _check(_lib.bpe_pair_counts(self._h, None, None, 0, ctypes.byref(n)), "bpe_pair_counts")
        keys = np.zeros(max(n.value, 1), dtype=np.uint32)
        cnts = np.zeros(max(n.value, 1), dtype=np.uint32)
        _check(_lib.bpe_pair_counts(self._h, keys.ctypes.data, cnts.ctypes.data, keys.size, ctypes.byref(n)),
               "bpe_pair_counts")
        keys, cnts = keys[: n.value].astype(np.int64), cnts[: n.value].astype(np.int64)
        o = np.argsort(keys)
        return keys[o], cnts[o]

    def profile(self, n_merges: int, per_iteration: bool = False):
        """bpe_profile; with per_iteration also the per-iteration times (ms, float32)."""
        import numpy as np
        r = ProfileResult()
        m = np.zeros(max(n_merges, 1), dtype=np.float32) if per_iteration else None
        _check(_lib.bpe_profile(self._h, n_merges, ctypes.byref(r), m.ctypes.data if per_iteration else None),
               "bpe_profile")
        return (r, m[:n_merges]) if per_iteration else r

    def free(self) -> None:
        if self._h:
            _lib.bpe_free(self._h)
            self._h = _vp(None)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
