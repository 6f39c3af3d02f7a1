"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the format definition, a closed form, a library routine (torch's float8 cast,
torch's scaled_dot_product_attention in float64) or an invariant the pages
imply. ``test_oracle.py`` runs them on the real oracle; ``test_oracle_mutations.py``
plants plausible mistakes in the oracle and checks that some pin fails.
The oracle modules are looked up at call time so planted mistakes take effect.
"""
import numpy as np
import torch

import oracle
import workloads as W
from tests.util import bf16_f64, logical_kv, oracle_pools, poisoned_pools, relabel_blocks, slot_index


# ---------------------------------------------------------------- fp8 codec
def pin_fp8_code_table():
    """Closed forms of OCP E4M3 without infinities (bias 7, 3 mantissa bits)."""
    v = oracle.fp8.decode(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x3F] == 1.875 and v[0x40] == 2.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isfinite(v).sum() == 254
    # codes of one sign increase with value
    assert np.all(np.diff(v[:0x7F]) > 0)


def _torch_e4m3(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_fp8_encode_vs_torch():
    """Every finite bf16 pattern (as float32) divided by several float32 scales,
    pre-clamped to +-448 (torch does not saturate), against torch's e4m3fn cast."""
    x = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    x = x[np.isfinite(x)]
    for s in [1.0, 0.01276507, 2.0 ** -9, 3.0, 1.0 / 448.0, 0.7]:
        with np.errstate(over="ignore"):
            q = (x / np.float32(s)).astype(np.float32)
        q = q[np.isfinite(q)]
        got = oracle.fp8.encode(q)
        ref = _torch_e4m3(np.clip(q, -448.0, 448.0))
        assert np.array_equal(got, ref), f"scale {s}: {np.count_nonzero(got != ref)} codes differ"
    # exact midpoints between neighbouring codes (the table taken from torch)
    tv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    pos = tv[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    for m in (mids, -mids):
        assert np.array_equal(oracle.fp8.encode(m), _torch_e4m3(m)), "tie-breaking differs"


def pin_fp8_hand_cases():
    e = oracle.fp8.encode
    cases = {448.0: 0x7E, 470.0: 0x7E, 1e30: 0x7E, -1e30: 0xFE, 2.0 ** -9: 0x01,
             2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, -(2.0 ** -11): 0x80, 1.0625: 0x38,
             1.1875: 0x3A, 2.0 ** -6: 0x08, 15 * 2.0 ** -10: 0x08, 240.0: 0x77}
    for val, code in cases.items():
        got = int(e(np.float32(val)))
        assert got == code, f"encode({val}) = {got:#x}, expected {code:#x}"
    assert int(e(np.float32(np.nan))) & 0x7F == 0x7F


def pin_fp8_roundtrip():
    c = np.arange(256, dtype=np.uint8)
    v = oracle.fp8.decode(c)
    fin = np.isfinite(v)
    assert np.array_equal(oracle.fp8.encode(v[fin].astype(np.float32)), c[fin])


def pin_fp8_tables_equal_direct_calls():
    """The looked-up forms used for large pools give the direct calls' results:
    every bf16 pattern under several scales, and every code's value."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    for sc in (1.0, 0.0087, 3.5e-3, 1.7, 2.0 ** -10):
        s = np.float32(sc)
        assert np.array_equal(oracle.fp8.quantize_bf16(bits, s), oracle.fp8.quantize(f32, s))
    a = oracle.fp8.decode_table()
    b = oracle.fp8.decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(a[np.isfinite(b)], b[np.isfinite(b)]) and np.isnan(a[~np.isfinite(b)]).all()


# ---------------------------------------------------------------- cache store / depage
def _small_workloads():
    yield W.custom(seed=11, Hq=4, Hkv=2, D=64, bs=16, context_lens=(1, 16, 17, 40, 0, 33))
    yield W.custom(seed=12, Hq=8, Hkv=2, D=128, bs=32, context_lens=(5, 64, 65),
                   prefill=[(0, 7), (32, 9)])
    yield W.custom(seed=13, Hq=6, Hkv=3, D=64, bs=16, context_lens=(40, 50, 60),
                   sharers=(0, 2), shared_prefix_blocks=2)
    yield W.custom(seed=14, Hq=4, Hkv=1, D=128, bs=32, context_lens=(3, 31, 70), kv_dtype="fp8")


def pin_store_roundtrip():
    """De-paging what was stored returns the stored rows bit for bit (bf16), or
    their e4m3fn codes (fp8); blocks no table uses keep their NaN sentinel."""
    for w in _small_workloads():
        kc, vc = oracle_pools(w)
        idx = slot_index(w)
        rows = [(w.block_tables[s], int(w.context_lens[s])) for s in range(w.num_seqs)]
        if w.has_prefill:
            rows += [(w.p_block_tables[i], int(w.cu_seqlens_k[i + 1] - w.cu_seqlens_k[i]))
                     for i in range(len(w.cu_seqlens_q) - 1)]
        for row, n in rows:
            K, V = oracle.cache.depage_raw(kc, vc, row, n, w.block_size)
            Kl, Vl = logical_kv(w, row, n, idx)
            if w.kv_dtype == "fp8":
                Kl = _quant_ref(Kl, w.k_scale)
                Vl = _quant_ref(Vl, w.v_scale)
            assert np.array_equal(K, Kl) and np.array_equal(V, Vl)
        sentinel = W.FP8_NAN if w.kv_dtype == "fp8" else W.BF16_NAN
        assert np.all(kc[w.unused_blocks] == sentinel) and np.all(vc[w.unused_blocks] == sentinel)


def _quant_ref(bits, scale):
    """e4m3fn codes of float32(bf16)/scale via torch's cast (pre-clamped)."""
    x = W.bf16_bits_to_f32(bits) / np.asarray(scale, np.float32)[None, :, None]
    return _torch_e4m3(np.clip(x.astype(np.float32), -448.0, 448.0))


def pin_store_skip_and_sentinel():
    """Rows whose slot is -1 write nothing; a store touches exactly its slots."""
    w = W.custom(seed=21, Hq=2, Hkv=2, D=64, bs=16, context_lens=(20, 9))
    kc, vc = poisoned_pools(w)
    slots = w.fill_slots.copy()
    slots[::3] = -1
    oracle.cache.store(w.fill_k, w.fill_v, slots, kc, vc, w.block_size)
    x = 8
    for t, s in enumerate(w.fill_slots.tolist()):
        b, o = divmod(s, w.block_size)
        kr = kc[b, :, :, o, :].reshape(w.num_kv_heads, w.head_dim)
        vr = vc[b, :, o // x, :, o % x]
        if t % 3 == 0:
            assert np.all(kr == W.BF16_NAN) and np.all(vr == W.BF16_NAN)
        else:
            assert np.array_equal(kr, w.fill_k[t]) and np.array_equal(vr, w.fill_v[t])
    written = np.count_nonzero(kc != W.BF16_NAN)
    assert written == np.count_nonzero(slots >= 0) * w.num_kv_heads * w.head_dim


def pin_layout_offsets():
    """Flat offsets worked out by hand from the documented layout, for a pool of
    2 blocks, 2 KV heads, block 16, D 16 (bf16, x = 8):
    K (b,h,o,d) -> ((((b*2+h)*2 + d//8)*16 + o)*8 + d%8
    V (b,h,o,d) -> ((((b*2+h)*2 + o//8)*16 + d)*8 + o%8
    slot 19 = block 1, offset 3. Head 1, d = 10:
      K: ((((1*2+1)*2 + 1)*16 + 3)*8 + 2 = ((7*16)+3)*8 + 2 = 922
      V: ((((1*2+1)*2 + 0)*16 + 10)*8 + 3 = ((6*16)+10)*8 + 3 = 851
    slot 12 = block 0, offset 12. Head 0, d = 5:
      K: ((((0)*2 + 0)*16 + 12)*8 + 5 = 101
      V: ((((0)*2 + 1)*16 + 5)*8 + 4 = 172"""
    ks, vs = oracle.cache.pool_shapes(2, 2, 16, 16, "bf16")
    for slot, h, d, k_off, v_off in [(19, 1, 10, 922, 851), (12, 0, 5, 101, 172)]:
        kc = np.zeros(ks, np.uint16)
        vc = np.zeros(vs, np.uint16)
        k = np.zeros((1, 2, 16), np.uint16)
        v = np.zeros((1, 2, 16), np.uint16)
        k[0, h, d] = 0x3F80
        v[0, h, d] = 0x4000
        oracle.cache.store(k, v, np.array([slot], np.int32), kc, vc, 16)
        assert np.flatnonzero(kc.ravel()).tolist() == [k_off]
        assert np.flatnonzero(vc.ravel()).tolist() == [v_off]


# ---------------------------------------------------------------- attention
def _sdpa(Q, K, V, scale, causal=False):
    """torch SDPA in float64: Q [Lq,Hq,D], K/V [Lk,Hkv,D] -> [Lq,Hq,D]."""
    q = torch.from_numpy(Q).permute(1, 0, 2)[None]
    k = torch.from_numpy(K).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=causal, scale=float(scale), enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def pin_decode_vs_sdpa():
    for w in _small_workloads():
        kc, vc = oracle_pools(w)
        out = oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                      w.block_size, w.k_scale, w.v_scale)
        idx = slot_index(w)
        for s in range(w.num_seqs):
            n = int(w.context_lens[s])
            if n == 0:
                assert np.all(out[s] == 0)
                continue
            Kb, Vb = logical_kv(w, w.block_tables[s], n, idx)
            if w.kv_dtype == "fp8":
                K = _deq(Kb, w.k_scale)
                V = _deq(Vb, w.v_scale)
            else:
                K, V = bf16_f64(Kb), bf16_f64(Vb)
            ref = _sdpa(bf16_f64(w.q[s])[None], K, V, w.scale)[0]
            np.testing.assert_allclose(out[s], ref, rtol=1e-11, atol=1e-12)


def _deq(bits, scale):
    codes = _quant_ref(bits, scale)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals * np.asarray(scale, np.float32).astype(np.float64)[None, :, None]


def pin_prefill_vs_sdpa():
    """Chunks with no cached prefix (Lq = Lk) against torch's causal SDPA."""
    w = W.custom(seed=31, Hq=8, Hkv=2, D=64, bs=16, context_lens=(),
                 prefill=[(0, 1), (0, 17), (0, 40)])
    kc, vc = oracle_pools(w)
    out = oracle.attention.prefill(w.pq, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k,
                                   w.p_block_tables, w.scale, w.block_size)
    idx = slot_index(w)
    for i in range(3):
        q0, q1 = w.cu_seqlens_q[i], w.cu_seqlens_q[i + 1]
        n = int(w.cu_seqlens_k[i + 1] - w.cu_seqlens_k[i])
        Kb, Vb = logical_kv(w, w.p_block_tables[i], n, idx)
        ref = _sdpa(bf16_f64(w.pq[q0:q1]), bf16_f64(Kb), bf16_f64(Vb), w.scale, causal=True)
        np.testing.assert_allclose(out[q0:q1], ref, rtol=1e-11, atol=1e-12)


def pin_chunk_is_tail_of_full_prefill():
    """A chunk of Lq queries on a cached prefix of p tokens gives the last Lq rows
    of the full causal prefill of all p + Lq tokens (chunked prefill computes the
    same attention as one prefill)."""
    p, Lq = 37, 23
    w = W.custom(seed=41, Hq=4, Hkv=2, D=64, bs=16, context_lens=(), prefill=[(p, Lq)])
    kc, vc = oracle_pools(w)
    out = oracle.attention.prefill(w.pq, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k,
                                   w.p_block_tables, w.scale, w.block_size)
    # full prefill: queries for every position; the chunk's queries are the last Lq rows
    rng = np.random.default_rng(5)
    qfull = np.concatenate([W.f32_to_bf16_bits(rng.standard_normal((p, 4, 64)).astype(np.float32)), w.pq])
    full = oracle.attention.prefill(qfull, kc, vc, np.array([0, p + Lq]), np.array([0, p + Lq]),
                                    w.p_block_tables, w.scale, w.block_size)
    np.testing.assert_allclose(out, full[p:], rtol=1e-12, atol=1e-13)


def pin_decode_is_prefill_of_one_row():
    w = W.custom(seed=51, Hq=4, Hkv=2, D=64, bs=16, context_lens=(1, 18, 49))
    kc, vc = oracle_pools(w)
    dec = oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size)
    S = w.num_seqs
    cu_q = np.arange(S + 1)
    cu_k = np.concatenate([[0], np.cumsum(w.context_lens)])
    pre = oracle.attention.prefill(w.q, kc, vc, cu_q, cu_k, w.block_tables, w.scale, w.block_size)
    np.testing.assert_allclose(dec, pre, rtol=1e-12, atol=1e-13)


def pin_decode_closed_forms():
    bs, D, H = 16, 64, 2
    ks, vs = oracle.cache.pool_shapes(4, H, bs, D)
    rng = np.random.default_rng(3)

    def pools_with(krows, vrows):
        kc = np.full(ks, W.BF16_NAN, np.uint16)
        vc = np.full(vs, W.BF16_NAN, np.uint16)
        n = krows.shape[0]
        oracle.cache.store(krows, vrows, np.arange(n, dtype=np.int32) + bs, kc, vc, bs)
        return kc, vc

    q = W.f32_to_bf16_bits(rng.standard_normal((1, 4, D)).astype(np.float32))
    table = np.array([[1, 2, 3]], np.int32)
    v = W.f32_to_bf16_bits(rng.standard_normal((40, H, D)).astype(np.float32))
    k = W.f32_to_bf16_bits(rng.standard_normal((40, H, D)).astype(np.float32))
    # context 1: the output is v0 exactly
    kc, vc = pools_with(k, v)
    o = oracle.attention.decode(q, kc, vc, table, np.array([1]), np.float32(0.125), bs)
    assert np.array_equal(o[0].reshape(H, 2, D), np.repeat(bf16_f64(v[0])[:, None], 2, axis=1))
    # identical keys: mean of V
    kc, vc = pools_with(np.repeat(k[:1], 40, axis=0), v)
    o = oracle.attention.decode(q, kc, vc, table, np.array([40]), np.float32(0.125), bs)
    mean = bf16_f64(v).mean(axis=0)
    np.testing.assert_allclose(o[0].reshape(H, 2, D), np.repeat(mean[:, None], 2, axis=1), atol=1e-13)
    # scale 0: mean of V
    kc, vc = pools_with(k, v)
    o = oracle.attention.decode(q, kc, vc, table, np.array([33]), np.float32(0.0), bs)
    mean = bf16_f64(v[:33]).mean(axis=0)
    np.testing.assert_allclose(o[0].reshape(H, 2, D), np.repeat(mean[:, None], 2, axis=1), atol=1e-13)
    # a key far more aligned with q than the others returns its value
    kd = np.zeros((40, H, D), np.uint16)
    j = 29
    for g in range(H):
        kd[j, g] = q[0, 2 * g]   # both query heads of group g see a huge score at j
    kc, vc = pools_with(kd, v)
    o = oracle.attention.decode(q, kc, vc, table, np.array([40]), np.float32(8.0), bs)
    np.testing.assert_allclose(o[0].reshape(H, 2, D)[:, 0], bf16_f64(v[j]), atol=1e-9)


def pin_permutation_invariance():
    """Renaming physical blocks (storage is non-contiguous) leaves outputs unchanged."""
    for w in _small_workloads():
        w2 = relabel_blocks(w, seed=9)
        outs = []
        for ww in (w, w2):
            kc, vc = oracle_pools(ww)
            outs.append(oracle.attention.decode(ww.q, kc, vc, ww.block_tables, ww.context_lens,
                                                ww.scale, ww.block_size, ww.k_scale, ww.v_scale))
        assert np.array_equal(outs[0], outs[1])


def pin_shared_prefix_equals_private_copy():
    """Tables pointing at one shared copy of a prefix give the outputs of tables
    pointing at private copies holding the same values."""
    w = W.custom(seed=61, Hq=4, Hkv=2, D=64, bs=16, context_lens=(40, 50, 60),
                 sharers=(0, 1, 2), shared_prefix_blocks=2, num_blocks=16)
    kc, vc = oracle_pools(w)
    shared_out = oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size)
    # copy the shared blocks into unused blocks and point sequences 1 and 2 at the copies
    bt = w.block_tables.copy()
    free = list(w.unused_blocks[1:])
    for s in (1, 2):
        for j in range(2):
            nb = free.pop()
            kc[nb] = kc[bt[s, j]]
            vc[nb] = vc[bt[s, j]]
            bt[s, j] = nb
    assert len(set(bt[:, 0].tolist())) == 3
    private_out = oracle.attention.decode(w.q, kc, vc, bt, w.context_lens, w.scale, w.block_size)
    assert np.array_equal(shared_out, private_out)


def pin_gqa_equals_replicated_mha():
    """Grouped heads equal multi-head attention with each KV head repeated for its group."""
    w = W.custom(seed=71, Hq=8, Hkv=2, D=64, bs=16, context_lens=(5, 37))
    kc, vc = oracle_pools(w)
    gqa = oracle.attention.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size)
    G = 4
    kr = np.repeat(kc, G, axis=1)
    vr = np.repeat(vc, G, axis=1)
    mha = oracle.attention.decode(w.q, kr, vr, w.block_tables, w.context_lens, w.scale, w.block_size)
    assert np.array_equal(gqa, mha)


# ---------------------------------------------------------------- add + RMSNorm
def _bits(a):
    return np.asarray(a, dtype=np.uint16)


def pin_bf16_round_hand_cases():
    """float64 -> bf16 rounding: ties to even, one rounding step, range ends."""
    cases = [(1.0, 0x3F80), (3.140625, 0x4049), (1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82),
             (1 + 2 ** -8 + 2 ** -30, 0x3F81),      # via float32 this would tie and go to 0x3F80
             (-(1 + 2 ** -8 + 2 ** -30), 0xBF81), (0.0, 0x0000), (-0.0, 0x8000),
             ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F), ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),
             ((2 - 2 ** -8 - 2 ** -20) * 2.0 ** 127, 0x7F7F), (2.0 ** -126, 0x0080),
             (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002),
             (np.inf, 0x7F80), (-np.inf, 0xFF80), (1e300, 0x7F80)]
    v = np.array([c[0] for c in cases])
    got = oracle.norm.f64_to_bf16_bits(v)
    want = _bits([c[1] for c in cases])
    assert np.array_equal(got, want), [(c[0], hex(g)) for c, g, e in zip(cases, got, want) if g != e]
    assert (oracle.norm.f64_to_bf16_bits(np.array([np.nan])) & 0x7FC0) == 0x7FC0


def pin_bf16_round_vs_torch():
    """On float32 inputs (where one rounding from float64 equals one from float32)
    the rounding equals torch's float32 -> bfloat16 cast, exact ties included."""
    rng = np.random.default_rng(81)
    u = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, ties ^ 1])
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.norm.f64_to_bf16_bits(f.astype(np.float64)), want)


def pin_rmsnorm_vs_torch():
    """y against torch's rms_norm (float64) of x + r, with and without a residual."""
    for seed, T, H, eps, res in ((84, 7, 64, 1e-6, True), (85, 3, 1000, 1e-5, True),
                                 (86, 5, 128, 0.5, False), (87, 2, 4096, 1e-6, True),
                                 (88, 4, 96, 3.0, True)):
        x, r, w = W.norm_inputs(seed, T, H)
        y, hb = oracle.norm.add_rmsnorm(x, w, eps, r if res else None)
        h = torch.from_numpy(bf16_f64(x))
        if res:
            h = h + torch.from_numpy(bf16_f64(r))
        ref = torch.nn.functional.rms_norm(h, (H,), torch.from_numpy(bf16_f64(w)), eps).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
        assert (hb is None) == (not res)


def pin_residual_sum_vs_torch_bf16_add():
    """The new residual equals torch's bfloat16 addition (float32 sum rounded to
    nearest even, which is exact rounding for two bf16 operands) — over rows
    whose residual is scaled by 2^-24 .. 2^24, r = -x rows and r = 0 rows."""
    T, H = 52, 256
    x, r, w = W.norm_inputs(89, T, H)
    k = np.arange(T) - 24
    r = W.f32_to_bf16_bits(W.bf16_bits_to_f32(r) * np.exp2(k).astype(np.float32)[:, None])
    r[-2] = x[-2] ^ np.uint16(0x8000)          # h = 0
    r[-1] = 0
    _, hb = oracle.norm.add_rmsnorm(x, w, 1e-6, r)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    want = (tx + tr).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(hb, want)
    assert np.array_equal(hb[-1], x[-1]) and not hb[-2].any()


def pin_rmsnorm_closed_forms():
    """Constant rows give sign(c) (eps 0, w 1); a one-hot row gives ±sqrt(H) at its
    entry; scaling x by a power of two changes nothing (eps 0); mean((y/w)^2) is
    ms / (ms + eps)."""
    H = 96
    ones = W.f32_to_bf16_bits(np.ones(H, np.float32))
    c = np.array([-3.0, 0.5, 2.0 ** -10, 1024.0])
    x = W.f32_to_bf16_bits(np.repeat(c[:, None], H, 1).astype(np.float32))
    y, _ = oracle.norm.add_rmsnorm(x, ones, 0.0)
    assert np.array_equal(y, np.repeat(np.sign(c)[:, None], H, 1))
    oh = np.zeros((2, H), np.float32)
    oh[0, 5], oh[1, 77] = 3.0, -0.25
    y, _ = oracle.norm.add_rmsnorm(W.f32_to_bf16_bits(oh), ones, 0.0)
    want = np.zeros((2, H))
    want[0, 5], want[1, 77] = np.sqrt(H), -np.sqrt(H)
    np.testing.assert_allclose(y, want, rtol=1e-15, atol=0)
    xb, rb, wb = W.norm_inputs(90, 3, H)
    y1, _ = oracle.norm.add_rmsnorm(xb, wb, 0.0, rb)
    s = np.float32(2.0 ** 9)
    y2, _ = oracle.norm.add_rmsnorm(W.f32_to_bf16_bits(W.bf16_bits_to_f32(xb) * s), wb, 0.0,
                                    W.f32_to_bf16_bits(W.bf16_bits_to_f32(rb) * s))
    assert np.array_equal(y1, y2)
    eps = 7.0
    y3, _ = oracle.norm.add_rmsnorm(xb, wb, eps, rb)
    h = bf16_f64(xb) + bf16_f64(rb)
    ms = (h ** 2).sum(1) / H
    np.testing.assert_allclose(((y3 / bf16_f64(wb)) ** 2).sum(1) / H, ms / (ms + eps), rtol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
