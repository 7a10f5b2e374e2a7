"""A short serving trace driven by the library's block manager: requests with
shared prompt prefixes are admitted (prefix-cache hits on live and on freed
pages), prefilled in one ragged launch, decoded for a few steps, finished and
replaced, in a pool small enough that pages are taken back and overwritten.

Every token's K/V row is a fixed function of its token prefix (a seeded draw
keyed by the prefix), as a model's would be, so a page found through the
prefix cache must hold exactly the rows this request would have written.
After every launch the GPU output is compared with the fp64 oracle run on a
pool rebuilt from those ground-truth rows through the manager's block
tables: a wrong or stale page would show up as a mismatch."""

import hashlib

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_parity, say

pytestmark = pytest.mark.gpu

HQ, HKV, D, B, NPAGES = 16, 8, 128, 16, 96
DT = torch.bfloat16
SCALE = D ** -0.5


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


def kv_row(prefix: tuple):
    """K and V rows [HKV, D] of the last token of `prefix` (deterministic)."""
    seed = int.from_bytes(hashlib.blake2b(np.asarray(prefix, dtype=np.int32).tobytes(), digest_size=8).digest(),
                          "little")
    g = np.random.default_rng(seed)
    kv = torch.from_numpy(g.standard_normal((2, HKV, D), dtype=np.float32)).to(DT)
    return kv[0], kv[1]


class Trace:
    def __init__(self, pka):
        self.pka = pka
        self.bm = pka.BlockManager(NPAGES, B)
        self.tokens = {}
        self.kc = torch.full((NPAGES, B, HKV, D), float("nan"), dtype=DT, device="cuda")
        self.vc = torch.full_like(self.kc, float("nan"))
        self.rng = np.random.default_rng(5)

    def truth_pool(self, rids):
        """A NaN pool holding the ground-truth rows of these requests' computed
        tokens, placed through the manager's block tables."""
        kc = torch.full((NPAGES, B, HKV, D), float("nan"), dtype=DT)
        vc = torch.full_like(kc, float("nan"))
        for r in rids:
            toks, n = self.tokens[r], self.bm.computed(r)
            for p, s in enumerate(self.bm.slot_mapping(r, 0, n).tolist()):
                kc[s // B, s % B], vc[s // B, s % B] = kv_row(tuple(toks[:p + 1]))
        return kc, vc

    def tables(self, rids):
        rows = [self.bm.block_table(r) for r in rids]
        width = max(len(t) for t in rows)
        return torch.tensor([t + [0] * (width - len(t)) for t in rows], dtype=torch.int32)

    def write_rows(self, r, start, n):
        slots = self.bm.slot_mapping(r, start, n)
        ks, vs = zip(*[kv_row(tuple(self.tokens[r][:p + 1])) for p in range(start, start + n)])
        return torch.stack(ks), torch.stack(vs), torch.from_numpy(slots)

    def prefill(self, rids, starts):
        """Write and attend the uncomputed prompt rows of `rids` in one launch."""
        ks, vs, ss, qlens, ctx = [], [], [], [], []
        for r, c in zip(rids, starts):
            n = len(self.tokens[r]) - c
            k, v, s = self.write_rows(r, c, n)
            ks.append(k), vs.append(v), ss.append(s), qlens.append(n), ctx.append(len(self.tokens[r]))
        k, v, s = torch.cat(ks), torch.cat(vs), torch.cat(ss)
        self.pka.kv_cache_write(k.cuda(), v.cuda(), s.cuda(), self.kc, self.vc)
        for r, n in zip(rids, qlens):
            self.bm.commit(r, n)
        q = torch.from_numpy(self.rng.standard_normal((sum(qlens), HQ, D), dtype=np.float32)).to(DT)
        qsl = torch.tensor([0] + list(np.cumsum(qlens)), dtype=torch.int32)
        bt, cl = self.tables(rids), torch.tensor(ctx, dtype=torch.int32)
        out = self.pka.paged_attn_prefill(q.cuda(), self.kc, self.vc, bt.cuda(), cl.cuda(), qsl.cuda(), SCALE,
                                          max(qlens), max(ctx))
        torch.cuda.synchronize()
        tk, tv = self.truth_pool(rids)
        ref = oracle.prefill(q, tk, tv, bt, cl, qsl, SCALE)
        return out, ref

    def decode(self, rids):
        for r in rids:
            t = int(self.rng.integers(0, 1000))
            self.bm.append_token(r, t)
            self.tokens[r].append(t)
            assert self.bm.allocate(r, 1), "pool too small for the trace"
        ks, vs, ss = zip(*[self.write_rows(r, len(self.tokens[r]) - 1, 1) for r in rids])
        self.pka.kv_cache_write(torch.cat(ks).cuda(), torch.cat(vs).cuda(), torch.cat(ss).cuda(), self.kc, self.vc)
        for r in rids:
            self.bm.commit(r, 1)
        q = torch.from_numpy(self.rng.standard_normal((len(rids), HQ, D), dtype=np.float32)).to(DT)
        bt = self.tables(rids)
        cl = torch.tensor([len(self.tokens[r]) for r in rids], dtype=torch.int32)
        out = self.pka.paged_attn_decode(q.cuda(), self.kc, self.vc, bt.cuda(), cl.cuda(), SCALE, int(cl.max()))
        torch.cuda.synchronize()
        tk, tv = self.truth_pool(rids)
        return out, oracle.decode(q, tk, tv, bt, cl, SCALE)


def _check(out, ref, what, weights_rounded=False):
    assert_parity(out, ref, DT, what, weights_rounded=weights_rounded)


def test_serving_trace_with_prefix_reuse(pka):
    tr = Trace(pka)
    rng = np.random.default_rng(11)
    shared = [rng.integers(0, 1000, size=n).tolist() for n in (3 * B, 2 * B + 5)]
    rid = 0

    def new_request(prefix, extra):
        nonlocal rid
        rid += 1
        tr.tokens[rid] = list(prefix) + rng.integers(0, 1000, size=extra).tolist()
        tr.bm.add_request(rid, tr.tokens[rid])
        return rid

    live = []
    for wave in range(4):
        batch = [new_request(shared[i % 2] if i % 3 else [], int(rng.integers(3, 60))) for i in range(5)]
        starts = []
        for r in batch:
            c = tr.bm.admit(r, len(tr.tokens[r]))
            assert c is not None, "pool too small for the trace"
            starts.append(c)
        hits = sum(1 for c in starts if c > 0)
        say(f"wave {wave}: admitted {len(batch)}, {hits} with cached prefixes {starts}, {tr.bm.num_free()} pages free")
        if wave > 0:
            assert hits > 0, "shared prefixes should hit the cache after the first wave"
        out, ref = tr.prefill(batch, starts)
        _check(out, ref, f"wave {wave} prefill", weights_rounded=True)
        live += batch
        for step in range(3):
            out, ref = tr.decode(live)
            _check(out, ref, f"wave {wave} decode step {step}")
        # finish the oldest half: their pages go back with registrations kept
        for r in live[: len(live) // 2]:
            tr.bm.free_request(r)
        live = live[len(live) // 2:]
    held = [0] * NPAGES
    for r in live:
        for b in tr.bm.block_table(r):
            held[b] += 1
    assert held == [tr.bm.refcount(b) for b in range(NPAGES)]
    assert tr.bm.num_free() == sum(1 for h in held if h == 0)
