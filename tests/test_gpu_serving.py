"""End to end: the block manager drives the kernels over several steps of a
small serving loop (prefix-cache hits, chunked prefill of the uncached part,
decode, fork + copy-on-write, free + reuse). Every attention output is checked
against the oracle computed on each sequence's logical tokens in private blocks,
so block sharing must be invisible in the results."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import dev_bf16, dev_i32, host_bits
from tests.util import assert_close, bf16_f64

pytestmark = pytest.mark.gpu

BS, NB, HQ, HKV, D = 16, 96, 8, 2, 128
SCALE = np.float32(1 / math.sqrt(D))
TOL = (1e-2, 1e-2)


def oracle_private(seq_tokens):
    """Oracle pools holding each sequence's K/V in private contiguous blocks."""
    nblk = [math.ceil(len(t) / BS) for t in seq_tokens]
    total = sum(nblk) + 1
    ks, vs = oracle.cache.pool_shapes(total, HKV, BS, D)
    kc, vc = np.zeros(ks, np.uint16), np.zeros(vs, np.uint16)
    tables = np.zeros((len(seq_tokens), max(nblk)), np.int32)
    b0 = 0
    for i, toks in enumerate(seq_tokens):
        tables[i, :nblk[i]] = np.arange(b0, b0 + nblk[i])
        K, V = W.prefix_kv(toks, HKV, D)
        slots = (b0 * BS + np.arange(len(toks))).astype(np.int32)
        oracle.cache.store(K, V, slots, kc, vc, BS)
        b0 += nblk[i]
    return kc, vc, tables


class Server:
    def __init__(self):
        import paged_kv_cache_store_amd as pa
        self.pa = pa
        self.bm = pa.BlockManager(NB, BS)
        self.kc, self.vc = pa.empty_pools(NB, HKV, BS, D)
        self.kc.view(torch.int16).fill_(int(W.BF16_NAN))
        self.vc.view(torch.int16).fill_(int(W.BF16_NAN))
        self.tokens = {}

    def store(self, sid, first, count):
        toks = self.tokens[sid]
        K, V = W.prefix_kv(toks[:first + count], HKV, D)
        slots = self.bm.slots(sid, first, count)
        self.pa.store_kv(dev_bf16(K[first:]), dev_bf16(V[first:]), dev_i32(slots), self.kc, self.vc)

    def add(self, toks):
        sid, cached = self.bm.add_sequence(toks)
        self.tokens[sid] = list(toks)
        self.store(sid, cached, len(toks) - cached)
        return sid, cached

    def table(self, sids):
        mb = max(self.bm.info(s)[1] for s in sids)
        return np.array([self.bm.block_table(s, mb, 0) for s in sids], np.int32)

    def prefill(self, sids, cached):
        q_rows, cu_q, cu_k = [], [0], [0]
        for s, c in zip(sids, cached):
            toks = self.tokens[s]
            q_rows.append(W.prefix_q(toks, HQ, D)[c:])
            cu_q.append(cu_q[-1] + len(toks) - c)
            cu_k.append(cu_k[-1] + len(toks))
        q = np.concatenate(q_rows)
        out = self.pa.prefill_varlen(dev_bf16(q), self.kc, self.vc, dev_i32(cu_q), dev_i32(cu_k),
                                     dev_i32(self.table(sids)), float(SCALE), int(np.diff(cu_q).max()),
                                     int(np.diff(cu_k).max()))
        got = bf16_f64(host_bits(out))
        kc, vc, tab = oracle_private([self.tokens[s] for s in sids])
        ref = oracle.attention.prefill(q, kc, vc, np.array(cu_q), np.array(cu_k), tab, SCALE, BS)
        assert_close(got, ref, *TOL, what="prefill")

    def append(self, sid, token):
        slot, cow = self.bm.append_token(sid, token)
        if cow is not None:
            self.pa.copy_blocks(self.kc, self.vc, dev_i32(np.array([cow], np.int32)))
        self.tokens[sid].append(token)
        n = len(self.tokens[sid])
        K, V = W.prefix_kv(self.tokens[sid], HKV, D)
        self.pa.store_kv(dev_bf16(K[n - 1:]), dev_bf16(V[n - 1:]), dev_i32([slot]), self.kc, self.vc)
        return cow

    def decode(self, sids):
        lens = np.array([len(self.tokens[s]) for s in sids], np.int32)
        q = np.stack([W.prefix_q(self.tokens[s], HQ, D)[-1] for s in sids])
        out = self.pa.decode(dev_bf16(q), self.kc, self.vc, dev_i32(self.table(sids)), dev_i32(lens),
                             float(SCALE), int(lens.max()))
        got = bf16_f64(host_bits(out))
        kc, vc, tab = oracle_private([self.tokens[s] for s in sids])
        ref = oracle.attention.decode(q, kc, vc, tab, lens, SCALE, BS)
        assert_close(got, ref, *TOL, what="decode")


def test_serving_loop_with_prefix_cache_fork_and_reuse():
    rng = np.random.default_rng(9)
    srv = Server()
    system = rng.integers(0, 1000, 40).tolist()          # 2 full blocks + 8 tokens
    prompts = [system + rng.integers(0, 1000, n).tolist() for n in (5, 17, 30, 1)]
    sids, cached = [], []
    for p in prompts:
        s, c = srv.add(p)
        sids.append(s)
        cached.append(c)
    assert cached == [0, 32, 32, 32]                       # later prompts hit the system blocks
    srv.prefill(sids, cached)
    for _ in range(3):                                     # decode steps
        for s in sids:
            srv.append(s, int(rng.integers(0, 1000)))
        srv.decode(sids)
    # fork a sequence whose last block is partial, then let both diverge
    while len(srv.tokens[sids[0]]) % BS == 0:
        srv.append(sids[0], int(rng.integers(0, 1000)))
    f = srv.bm.fork(sids[0])
    srv.tokens[f] = list(srv.tokens[sids[0]])
    cow = srv.append(f, 5)
    assert cow is not None                                 # shared partial block was copied
    srv.append(sids[0], 6)
    srv.decode([sids[0], f] + sids[1:])
    # end two requests; a new prompt with the system prefix reuses cached blocks
    srv.bm.free(sids[1])
    srv.bm.free(sids[2])
    del srv.tokens[sids[1]], srv.tokens[sids[2]]
    s_new, c_new = srv.add(system + rng.integers(0, 1000, 9).tolist())
    assert c_new == 32
    srv.prefill([s_new], [c_new])
    srv.decode([s_new, sids[0], f, sids[3]])
