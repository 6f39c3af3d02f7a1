"""Decode and chunked-prefill attention by definition — TEST INFRASTRUCTURE.

The pages say the attention layer follows the FlashAttention idea, an exact
memory-efficient attention ("Nano-vLLM：轻量高效的大模型推理框架…", 三.3 模型层适配),
and that PagedAttention only changes where keys/values live
("DeepSeek复刻vLLM反超原版：AI推理新标杆", section vLLM：大模型推理的加速引擎与挑战).
Both reach the plain result, so this module is the plain result: softmax of
scale * q.k over the de-paged keys, applied to the de-paged values, in float64.

Readings where the pages are silent:
* query head h reads KV head h // (Hq / Hkv) (grouped-query attention, named
  as a variant on "nano-vllm-lite…", 潜在贡献方向);
* a decode sequence of context length n attends to positions 0..n-1, its own
  newest token included; n = 0 gives a zero output;
* a prefill chunk of Lq queries on Lk keys (its cached prefix plus itself) is
  causal with the mask aligned bottom-right: query i sits at absolute
  position Lk - Lq + i and attends to keys 0..Lk - Lq + i (chunked prefill,
  "nano-vllm-lite…", 核心技术改进 §2); a query that sees no key outputs zeros.
"""
import numpy as np

from .cache import bf16_to_f64, depage


def _kv_head(h, group, num_kv_heads):
    """Query head h reads KV head h // group (contiguous groups of query heads)."""
    return h // group


def _causal_mask(Lq, Lk):
    """mask[i, j] is True when query row i may attend to key j."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return j <= (Lk - Lq) + i


def _softmax_rows(z, mask=None):
    """exp(z - max) / sum over the last axis, restricted to mask; rows with no
    admissible entry give all-zero weights."""
    if mask is not None:
        z = np.where(mask, z, -np.inf)
    m = np.max(z, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(z - m)
    if mask is not None:
        p = np.where(mask, p, 0.0)
    s = p.sum(axis=-1, keepdims=True)
    return p / np.where(s > 0, s, 1.0)


def _attend(Q, K, V, scale, mask=None):
    """Q [Lq, Hq, D], K/V [Lk, Hkv, D] float64 -> [Lq, Hq, D]."""
    Lq, Hq, D = Q.shape
    Hkv = K.shape[1]
    group = Hq // Hkv
    out = np.zeros((Lq, Hq, D))
    for h in range(Hq):
        kv = _kv_head(h, group, Hkv)
        z = float(scale) * (Q[:, h, :] @ K[:, kv, :].T)       # [Lq, Lk]
        w = _softmax_rows(z, mask)
        out[:, h, :] = w @ V[:, kv, :]
    return out


def decode(q_bits, k_cache, v_cache, block_tables, context_lens, scale, block_size,
           k_scale=None, v_scale=None, seqs=None):
    """One query per sequence. q_bits [S, Hq, D] bf16 patterns; returns float64
    [S, Hq, D] (rows of sequences not in `seqs`, when given, stay zero)."""
    q = np.asarray(q_bits)
    S, Hq, D = q.shape
    out = np.zeros((S, Hq, D))
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n <= 0:
            continue
        K, V = depage(k_cache, v_cache, block_tables[s], n, block_size, k_scale, v_scale)
        out[s] = _attend(bf16_to_f64(q[s])[None], K, V, scale)[0]
    return out


def prefill(q_bits, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables, scale,
            block_size, k_scale=None, v_scale=None, seqs=None):
    """Causal varlen attention of packed query chunks ([Tq, Hq, D] bf16 patterns,
    sequence s owns rows cu_seqlens_q[s]:cu_seqlens_q[s+1]) over each sequence's
    Lk = cu_seqlens_k[s+1] - cu_seqlens_k[s] keys read through its block table.
    Returns float64 [Tq, Hq, D]."""
    q = np.asarray(q_bits)
    out = np.zeros(q.shape)
    P = len(cu_seqlens_q) - 1
    for s in (range(P) if seqs is None else seqs):
        q0, q1 = int(cu_seqlens_q[s]), int(cu_seqlens_q[s + 1])
        Lq = q1 - q0
        Lk = int(cu_seqlens_k[s + 1]) - int(cu_seqlens_k[s])
        if Lq <= 0:
            continue
        if Lk <= 0:
            continue
        K, V = depage(k_cache, v_cache, block_tables[s], Lk, block_size, k_scale, v_scale)
        out[q0:q1] = _attend(bf16_to_f64(q[q0:q1]), K, V, scale, _causal_mask(Lq, Lk))
    return out
