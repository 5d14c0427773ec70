"""GPU parity at the benchmark workloads' full sizes, and at the end of the
16-bit id space (the HIP path through the C ABI against the oracle).

Every workload is trained at its full size with its own merge count and
pair-table size, and the merge list and the final token sequence are
compared with the chunk-multiset C oracle element by element (bit-exact:
all work is integer). The same corpus is then encoded with the learned list
by the GPU encoder, which must give the oracle's training tokens (a learned
list applied to its own training text reproduces training's result).

Training over the distinct words (bpe_train_chunked) must give the same
merges and tokens at every full size.

The id-space test trains to the last id (65,535 = 256 + 65,279) on corpora
small enough for the oracle to follow, checks that nothing more can be
merged (BPE_EIDSPACE), and builds the encoder and the trie from the full
list."""
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
    return torch.from_numpy(np.ascontiguousarray(data, dtype=np.uint8)).to("cuda:0")


def first_difference(a, b):
    """Index of the first differing element of two 1-D arrays (the shorter
    length if one is a prefix of the other), or None if they are equal."""
    a = np.asarray(a).reshape(-1)
    b = np.asarray(b).reshape(-1)
    m = min(a.size, b.size)
    d = np.flatnonzero(a[:m] != b[:m])
    if d.size:
        return int(d[0])
    return None if a.size == b.size else m


def assert_same(what, got, want):
    i = first_difference(got, want)
    if i is not None:
        g = got.reshape(-1)[i] if i < got.size else "end"
        w = want.reshape(-1)[i] if i < want.size else "end"
        pytest.fail("%s: first difference at index %d (GPU %s, oracle %s; lengths %d and %d)"
                    % (what, i, g, w, got.size, want.size))


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 5, 3, 4])
def test_full_size_workload_matches_oracle(bpe, cfg):
    spec = corpus.CONFIGS[cfg]
    _say("full size: %s (%d bytes, %d merges, table 2^%d)" % (spec.name, spec.n_bytes, spec.n_merges,
                                                                spec.table_log2))
    data = corpus.generate(spec)
    d = _dev(data)
    gm, gt = bpe.train(d, spec.n_merges, spec.table_log2)
    gm = gm.cpu().numpy().astype(np.int64)
    _say("  GPU: %d merges, %d tokens" % (gm.shape[0], gt.shape[0]))
    om, ot, _ = oracle.train_chunks(data, spec.n_merges)
    _say("  oracle: %d merges, %d tokens" % (om.shape[0], ot.shape[0]))
    assert_same("merges of %s" % spec.name, gm, om)
    assert_same("tokens of %s" % spec.name, gt.cpu().numpy().astype(np.uint32), ot)
    # the learned list applied to its own training text gives training's tokens
    with bpe.Encoder(gm) as enc:
        et = enc.encode(d).cpu().numpy().astype(np.uint32)
    assert_same("encoding of %s with its own merges" % spec.name, et, ot)
    del gt, et
    # training over the distinct words, each weighted by its frequency, gives
    # the same (as called, and forced past the memory bound it checks)
    for always in (False, True):
        cm, ct = bpe.train_chunked(d, spec.n_merges, spec.table_log2, always_chunks=always)
        _say("  chunked (always %s): %d merges, %d tokens" % (always, cm.shape[0], ct.shape[0]))
        assert_same("chunked merges of %s" % spec.name, cm.cpu().numpy().astype(np.int64), om)
        assert_same("chunked tokens of %s" % spec.name, ct.cpu().numpy().astype(np.uint32), ot)
        del cm, ct


@pytest.mark.timeout(600)
# 8 MiB and 4 MiB: 16384-symbol tiles; 3 MiB: 8192-symbol tiles (one half)
@pytest.mark.parametrize("cfg,n_bytes", [(2, 8 << 20), (5, 4 << 20), (5, 3 << 20)])
def test_training_to_the_last_id(bpe, cfg, n_bytes):
    # 65,280 merges: ids 256 .. 65,535; the last merge creates id 0xFFFF,
    # after which no pair is counted and no further merge is allowed
    spec = corpus.CONFIGS[cfg].scaled(n_bytes, n_merges=bpe.MAX_MERGES, seed=77)
    data = corpus.generate(spec)
    _say("id space: %s at %d bytes, %d merges" % (spec.kind, n_bytes, spec.n_merges))
    om, ot, _ = oracle.train_chunks(data, spec.n_merges)
    assert om.shape[0] == bpe.MAX_MERGES, "the corpus must not run out of pairs first"
    d = _dev(data)
    with bpe.State(d, table_log2=22) as st:
        st.run(bpe.MAX_MERGES)
        assert st.sync() == bpe.MAX_MERGES
        gm = st.merges().cpu().numpy().astype(np.int64)
        gt = st.tokens().cpu().numpy().astype(np.uint32)
        assert_same("merges", gm, om)
        assert_same("tokens", gt, ot)
        for call in (lambda: st.step(), lambda: st.run(1)):
            with pytest.raises(bpe.BpeError) as e:
                call()
            assert e.value.status == bpe.EIDSPACE
        # the state is still usable after the rejected calls
        assert st.sync() == bpe.MAX_MERGES
        assert np.array_equal(st.tokens().cpu().numpy().astype(np.uint32), ot)
    # one-call training asked for the whole id space gives the same
    m2, t2 = bpe.train(d, bpe.MAX_MERGES, 22)
    assert_same("bpe_train merges", m2.cpu().numpy().astype(np.int64), om)
    assert_same("bpe_train tokens", t2.cpu().numpy().astype(np.uint32), ot)
    # and so does training over the distinct words (its last merge, X = 0xFFFF, updates no counts)
    for always in (True, False):
        m3, t3 = bpe.train_chunked(d, bpe.MAX_MERGES, 22, always_chunks=always)
        assert_same("bpe_train_chunked merges (always %s)" % always, m3.cpu().numpy().astype(np.int64), om)
        assert_same("bpe_train_chunked tokens (always %s)" % always, t3.cpu().numpy().astype(np.uint32), ot)
    # the full list drives the encoder and the trie
    text = corpus.generate(corpus.CONFIGS[cfg].scaled(300_000, seed=78))
    dt = _dev(text)
    with bpe.Encoder(gm) as enc:
        assert_same("encoding with the full list", enc.encode(dt).cpu().numpy().astype(np.uint32),
                    oracle.encode(text, om)[1])
        assert_same("encoding the training text", enc.encode(d).cpu().numpy().astype(np.uint32), ot)
    with bpe.Trie(gm) as tr:
        assert_same("inference with the full list", tr.encode(dt).cpu().numpy().astype(np.uint32),
                    oracle.trie_encode(text, om))


@pytest.mark.timeout(600)
def test_automatic_table_holds_a_corpus_past_the_old_default(bpe):
    # 32 MiB of byte runs and random bytes trained to 20,000 merges claims
    # about 4.6M pair-table slots, past the 3.67M a 2^22 table holds (the
    # largest automatic size before it depended on the merge count)
    spec = corpus.CONFIGS[5].scaled(32 << 20, n_merges=20000, seed=400 + 20000 % 97)
    data = corpus.generate(spec)
    _say("automatic table: %d bytes of runs, %d merges" % (spec.n_bytes, spec.n_merges))
    d = _dev(data)
    gm, gt = bpe.train(d, spec.n_merges)  # table_log2 0: automatic, from n and n_merges
    om, ot, _ = oracle.train_chunks(data, spec.n_merges)
    assert_same("merges", gm.cpu().numpy().astype(np.int64), om)
    assert_same("tokens", gt.cpu().numpy().astype(np.uint32), ot)
    with bpe.State(d) as st:  # bpe_init: automatic size for up to 65,280 merges
        st.run(spec.n_merges)
        assert st.sync() == spec.n_merges
        slots, claimed, limit = st.table_usage()
        _say("  slots %d, claimed %d, limit %d" % (slots, claimed, limit))
        assert 3_670_016 < claimed <= limit < slots
        assert_same("merges through bpe_init", st.merges().cpu().numpy().astype(np.int64), om)


def _busy(torch):
    """Queue a few milliseconds of work on the current stream."""
    a = torch.randn(2048, 2048, device="cuda:0")
    for _ in range(20):
        a = a @ a
        a = a / a.abs().amax()
    return a


@pytest.mark.parametrize("kind", ["encoder", "trie"])
def test_default_stream_work_is_ordered_before_and_after_calls(bpe, kind):
    # the input is produced and the output filled by torch kernels on the
    # default stream, queued behind other work, with no synchronisation
    # before the call: the library's own stream (used when the caller's is
    # the default one) must wait for them
    import torch
    text = corpus.generate(corpus.CONFIGS[2].scaled(1 << 20, seed=90))
    spec = corpus.CONFIGS[2].scaled(200_000, n_merges=300, seed=91)
    train = corpus.generate(spec)
    om, _, _ = oracle.train_chunks(train, spec.n_merges)
    want = oracle.encode(text, om)[1] if kind == "encoder" else oracle.trie_encode(text, om)
    obj = bpe.Encoder(om) if kind == "encoder" else bpe.Trie(om)
    with obj:
        src = torch.from_numpy(text.copy()).pin_memory()
        for off in (0, 3):
            torch.cuda.synchronize()
            busy = _busy(torch)
            d = torch.empty(text.size, dtype=torch.uint8, device="cuda:0")
            d.copy_(src, non_blocking=True)
            d = d ^ (busy[0, 0] * 0).to(torch.uint8)  # a kernel that waits for the busy work
            big = torch.empty(text.size + 8, dtype=torch.int32, device="cuda:0")
            big.fill_(-1)
            got = obj.encode(d, out=big[off:])
            assert_same("%s output at offset %d" % (kind, off), got.cpu().numpy().astype(np.uint32), want)
            assert bool((big[:off] == -1).all())
