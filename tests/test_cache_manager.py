"""The host-side KV pool manager (include/lazyattn_cache.h), no GPU.

* Hand-worked scenarios pin the policy model (oracle/cache_policy.py) and the
  native manager alike: block ids, frame starts, hits, misses and evictions
  written out from the rules (16-token blocks and a free list, [KVF]
  "PagedAttention" / "Exercícios" 3; reuse by content at any position versus
  position-aware and prefix reuse, [LA] "Declaração do Problema").
* Random operation traces: the native manager agrees with the model exactly
  (integer work: every table word, miss flag, request id, error and counter).
* Invariants: every block is free, held by one cached document or by one
  live prompt; a referenced document is never evicted.
* A Zipf-skewed document trace under a fixed budget: reuse by content hits at
  least as often as position-aware reuse, which beats prefix reuse ([LA]
  "Principais Contribuições" 2 and "Resultados Experimentais" report this
  ordering for skewed access).
"""

import numpy as np
import pytest

from oracle.cache_policy import AGNOSTIC, AWARE, PREFIX, BadArgument, BadPosition, CachePolicyModel, NoSpace

C = pytest.importorskip("position_agnostic_kv_amd.cache")


def w(block, off):
    return block | (off << 16)


@pytest.fixture(params=["native", "model"])
def mk(request):
    """Factory for the native manager or the model behind one interface."""
    def make(num_blocks, mode):
        if request.param == "native":
            return Native(num_blocks, mode)
        return Model(num_blocks, mode)
    return make


class Native:
    def __init__(self, n, mode):
        self.m = C.CacheManager(n, mode)

    def acquire(self, ids, lens, prompt=0, max_blocks=None):
        try:
            row, miss, rid = self.m.acquire(ids, lens, prompt, max_blocks)
        except C.CacheError as e:
            return {C.ERR_NOSPACE: "nospace", C.ERR_POSITION: "position"}.get(e.status, "arg")
        return [int(x) for x in row], [int(x) for x in miss], rid

    def release(self, rid):
        self.m.release(rid)

    def stats(self):
        return self.m.stats()


class Model:
    def __init__(self, n, mode):
        self.m = CachePolicyModel(n, C.MODES[mode])

    def acquire(self, ids, lens, prompt=0, max_blocks=None):
        if max_blocks is None:
            max_blocks = sum(L // 16 for L in lens) + -(-prompt // 16)
        try:
            return self.m.acquire(ids, lens, prompt, max_blocks)
        except NoSpace:
            return "nospace"
        except BadPosition:
            return "position"
        except BadArgument:
            return "arg"

    def release(self, rid):
        self.m.release(rid)

    def stats(self):
        return self.m.stats()


# ----------------------------------------------------------- hand-worked pins
def test_first_request_takes_blocks_in_order(mk):
    c = mk(8, "agnostic")
    row, miss, rid = c.acquire([7, 9], [32, 48], 20)
    # doc 7: blocks 0,1 at frame 0; doc 9: blocks 2,3,4 at frame 32; prompt
    # (20 tokens -> 2 blocks) 5,6 at frame 80
    assert row == [w(0, 0), w(1, 0), w(2, 32), w(3, 32), w(4, 32), w(5, 80), w(6, 80)]
    assert miss == [1, 1] and rid == 0
    s = c.stats()
    assert (s["free_blocks"], s["doc_blocks"], s["prompt_blocks"], s["cached_docs"]) == (1, 5, 2, 2)


def test_agnostic_reuses_at_any_position(mk):
    c = mk(8, "agnostic")
    _, _, r0 = c.acquire([7, 9], [32, 48], 20)
    c.release(r0)
    row, miss, _ = c.acquire([9, 7], [48, 32], 16)
    # same physical blocks, new frame starts; the prompt reuses the freed 5
    assert row == [w(2, 0), w(3, 0), w(4, 0), w(0, 48), w(1, 48), w(5, 80)]
    assert miss == [0, 0]
    s = c.stats()
    assert (s["doc_hits"], s["doc_misses"], s["tokens_hit"], s["tokens_missed"]) == (2, 2, 80, 80)


def test_aware_copies_per_position_and_evicts_lru(mk):
    c = mk(8, "aware")
    _, _, r0 = c.acquire([7, 9], [32, 48], 0)      # 7@0 -> [0,1], 9@32 -> [2,3,4]
    c.release(r0)                                   # unreferenced, oldest first: 7@0, 9@32
    row, miss, _ = c.acquire([9, 7], [48, 32], 0)   # 9@0 and 7@48 are new keys
    # 9@0 needs 3 blocks: free are 5,6,7 (top first) -> [5,6,7]; 7@48 needs 2:
    # none free, evict 7@0 (oldest) -> blocks 0,1 come back -> [0,1]
    assert row == [w(5, 0), w(6, 0), w(7, 0), w(0, 48), w(1, 48)]
    assert miss == [1, 1]
    s = c.stats()
    assert (s["evicted"], s["cached_docs"], s["free_blocks"]) == (1, 3, 0)


def test_prefix_hits_only_with_identical_prefix(mk):
    c = mk(16, "prefix")
    _, _, r0 = c.acquire([1, 2, 3], [16, 16, 16], 0)
    c.release(r0)
    _, miss, _ = c.acquire([1, 2, 4], [16, 16, 16], 0)
    assert miss == [0, 0, 1]
    _, miss, _ = c.acquire([2, 1], [16, 16], 0)
    assert miss == [1, 1]                   # same documents, other prefix


def test_referenced_documents_are_never_evicted(mk):
    c = mk(6, "agnostic")
    _, _, r0 = c.acquire([1], [64], 0)      # 4 blocks, held
    assert c.acquire([2], [48], 0) == "nospace"   # 2 free, doc 1 is referenced
    c.release(r0)
    row, miss, _ = c.acquire([2], [48], 0)  # now doc 1 is evicted
    assert miss == [1] and len(row) == 3
    assert c.stats()["evicted"] == 1


def test_failed_request_changes_nothing(mk):
    c = mk(6, "agnostic")
    _, _, r0 = c.acquire([1, 2], [32, 32], 0)
    c.release(r0)
    before = c.stats()
    assert c.acquire([3, 1], [96, 32], 0) == "nospace"   # 6 + 2 blocks > 6
    assert c.stats() == before
    row, miss, _ = c.acquire([1], [32], 0)               # doc 1 is still cached
    assert miss == [0] and row == [w(0, 0), w(1, 0)]


def test_repeat_within_one_request_shares_blocks(mk):
    c = mk(8, "agnostic")
    row, miss, _ = c.acquire([5, 6, 5], [32, 16, 32], 0)
    assert miss == [1, 1, 0]
    assert row == [w(0, 0), w(1, 0), w(2, 32), w(0, 48), w(1, 48)]


def test_document_length_is_part_of_its_identity(mk):
    """Naming a cached document with another length, or one document twice in
    a request with two lengths, is an argument error that changes nothing.
    (The native manager once placed the cached blocks regardless and wrote
    them past a row sized for the request's own lengths.)"""
    for mode in ("agnostic", "aware"):
        c = mk(16, mode)
        _, _, r0 = c.acquire([4], [48], 0)                       # 3 blocks
        before = c.stats()
        assert c.acquire([4], [16], 0, max_blocks=1) == "arg"     # claims 1 block
        assert c.acquire([4], [64], 0) == "arg"
        if mode == "agnostic":   # position-aware: two positions are two documents
            assert c.acquire([9, 9], [32, 48], 0) == "arg"        # not cached, two lengths
        assert c.stats() == before
        row, miss, _ = c.acquire([4, 9, 9], [48, 32, 32], 0)     # consistent: placed
        assert miss == ([0, 1, 0] if mode == "agnostic" else [0, 1, 1]) and len(row) == 3 + 2 + 2
        c.release(r0)


def test_positions_beyond_the_offset_field(mk):
    c = mk(4096, "agnostic")
    assert c.acquire([1, 2], [32768, 32768], 1) == "position"   # prompt at 65536
    row, _, _ = c.acquire([1, 2], [32768, 32752], 16)            # last position 65535
    assert row[-1] >> 16 == 65520


def test_arguments_are_checked():
    with pytest.raises(C.CacheError):
        C.CacheManager(0)
    with pytest.raises(C.CacheError):
        C.CacheManager(65537)
    with pytest.raises(KeyError):
        C.CacheManager(8, "lru")
    m = C.CacheManager(8)
    with pytest.raises(C.CacheError):
        m.acquire([1], [20])                 # not a whole number of blocks
    with pytest.raises(C.CacheError):
        m.release(42)                        # unknown request
    with pytest.raises(C.CacheError):
        m.acquire([1, 2], [16, 16], 0, max_blocks=1)   # table row too short


# ------------------------------------------------------------ native == model
def _check_partition(model):
    held = []
    for d in model.m.docs.values():
        held += d["blocks"]
    for _, prompt in model.m.requests.values():
        held += prompt
    allb = held + model.m.free
    assert sorted(allb) == list(range(model.m.num_blocks)), "a block is lost or owned twice"


@pytest.mark.parametrize("mode", ["agnostic", "aware", "prefix"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_native_matches_model_on_random_traces(mode, seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(12, 64))
    nat, mod = Native(nb, mode), Model(nb, mode)
    live = []
    for step in range(400):
        if live and rng.random() < 0.45:
            rid = live.pop(int(rng.integers(len(live))))
            nat.release(rid)
            mod.release(rid)
        else:
            k = int(rng.integers(0, 5))
            ids = [int(x) for x in rng.integers(0, 12, size=k)]
            lens = [16 * (1 + (i * 7919) % 4) for i in ids]   # a document's length is fixed
            prompt = int(rng.integers(0, 40))
            a, b = nat.acquire(ids, lens, prompt), mod.acquire(ids, lens, prompt)
            assert a == b, f"step {step}: native {a} model {b}"
            if not isinstance(a, str):
                live.append(a[2])
        assert nat.stats() == mod.stats(), f"step {step}"
        _check_partition(mod)
        for d in mod.m.docs.values():
            assert d["refs"] >= 0


@pytest.mark.parametrize("mode", ["agnostic", "aware", "prefix"])
def test_native_matches_model_with_inconsistent_lengths(mode):
    """Random traces in which a tenth of the documents are named with a wrong
    length: both reject the same requests and otherwise agree exactly."""
    rng = np.random.default_rng(200)
    nb = 48
    nat, mod = Native(nb, mode), Model(nb, mode)
    live, rejected = [], 0
    for step in range(400):
        if live and rng.random() < 0.45:
            rid = live.pop(int(rng.integers(len(live))))
            nat.release(rid)
            mod.release(rid)
            continue
        ids = [int(x) for x in rng.integers(0, 10, size=int(rng.integers(1, 4)))]
        lens = [16 * (1 + (i * 7919) % 4) + (16 if rng.random() < 0.1 else 0) for i in ids]
        prompt = int(rng.integers(0, 40))
        maxb = sum(L // 16 for L in lens) + -(-prompt // 16)
        a, b = nat.acquire(ids, lens, prompt, maxb), mod.acquire(ids, lens, prompt, maxb)
        assert a == b, f"step {step}: native {a} model {b}"
        rejected += a == "arg"
        if not isinstance(a, str):
            live.append(a[2])
        assert nat.stats() == mod.stats(), f"step {step}"
    assert rejected > 0


# --------------------------------------------------- hit rates under a budget
def _zipf_trace(rng, n_req, catalogue, s, docs_per_req, lens):
    p = 1.0 / np.arange(1, catalogue + 1) ** s
    p /= p.sum()
    out = []
    for _ in range(n_req):
        k = int(rng.integers(docs_per_req[0], docs_per_req[1] + 1))
        ids = [int(x) for x in rng.choice(catalogue, size=k, replace=False, p=p)]
        out.append((ids, [int(lens[i]) for i in ids]))
    return out


def simulate(mode, trace, budget_blocks, prompt=64):
    m = C.CacheManager(budget_blocks, mode)
    for ids, lens in trace:
        row, miss, rid = m.acquire(ids, lens, prompt)
        m.release(rid)
    s = m.stats()
    return s["tokens_hit"] / (s["tokens_hit"] + s["tokens_missed"])


def test_skewed_reuse_hit_rate_ordering():
    rng = np.random.default_rng(7)
    lens = 16 * rng.integers(16, 129, size=300)
    trace = _zipf_trace(rng, 1500, 300, 1.2, (3, 6), lens)
    budget = 2048   # blocks: ~20 average documents
    hr = {mode: simulate(mode, trace, budget) for mode in ("agnostic", "aware", "prefix")}
    assert hr["agnostic"] > hr["aware"] > hr["prefix"] >= 0.0, hr
    assert hr["agnostic"] > 1.5 * hr["aware"], hr
