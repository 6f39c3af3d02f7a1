"""Block-pool store and de-paging — TEST INFRASTRUCTURE (see the package docstring).

What the pages fix: the KV cache is cut into fixed-size blocks stored
non-contiguously ("nano-vllm：轻量级大模型推理引擎的技术探索与实践", PagedAttention
原理回顾); each block holds the KV of a fixed number of tokens, allocated per
request ("Nano-vLLM：轻量高效的大模型推理框架…", 三.1 推理引擎架构, 块管理器);
a block table maps a sequence's logical blocks to physical blocks
("DeepSeek复刻vLLM反超原版：AI推理新标杆", section vLLM：大模型推理的加速引擎与挑战).

What the library fixes (the pages give no layout), with x = 16 bytes / element
size (8 for bf16, 16 for fp8):
* token slot s lives in block s // block_size at offset s % block_size;
* K pool  [num_blocks][Hkv][D/x][block_size][x]: element (b, h, o, d) is at
  ((((b*Hkv + h)*(D/x) + d//x)*block_size + o)*x + d%x);
* V pool  [num_blocks][Hkv][block_size/x][D][x]: element (b, h, o, d) is at
  ((((b*Hkv + h)*(block_size/x) + o//x)*D + d)*x + o%x).
The oracle writes these as numpy arrays of those five dimensions.
"""
import math

import numpy as np

from . import fp8 as _fp8


def _x(cache: np.ndarray) -> int:
    return 16 // cache.itemsize


def pool_shapes(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype="bf16"):
    x = 16 if kv_dtype == "fp8" else 8
    k = (num_blocks, num_kv_heads, head_dim // x, block_size, x)
    v = (num_blocks, num_kv_heads, block_size // x, head_dim, x)
    return k, v


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def store(k_bits, v_bits, slot_mapping, k_cache, v_cache, block_size,
          k_scale=None, v_scale=None):
    """Write token t's K/V rows ([T, Hkv, D] bf16 bit patterns) into the slot
    slot_mapping[t]; a negative slot means "skip". For an fp8 pool (uint8) the
    stored byte is the e4m3fn code of float32(value) / scale[h]."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    if slots.size == 0:
        return
    k = np.asarray(k_bits)[keep]
    v = np.asarray(v_bits)[keep]
    T, H, D = k.shape
    if k_cache.dtype == np.uint8:
        # per KV head h: the code of float32(value) / scale[h] (fp8.quantize,
        # through its table over the bf16 patterns)
        kq = np.empty(k.shape, np.uint8)
        vq = np.empty(v.shape, np.uint8)
        for h in range(H):
            kq[:, h] = _fp8.quantize_bf16(k[:, h], np.float32(np.asarray(k_scale, np.float32)[h]))
            vq[:, h] = _fp8.quantize_bf16(v[:, h], np.float32(np.asarray(v_scale, np.float32)[h]))
        k, v = kq, vq
    x = _x(k_cache)
    block = slots // block_size
    off = slots % block_size
    # K: the D values of a row split into D/x chunks of x, chunk c at [b, h, c, off, :]
    k_cache[block, :, :, off, :] = k.reshape(T, H, D // x, x)
    # V: value d of a row at [b, h, off // x, d, off % x]
    v_cache[block, :, off // x, :, off % x] = v


def depage(k_cache, v_cache, table_row, length, block_size, k_scale=None, v_scale=None):
    """float64 K and V ([length, Hkv, D]) of one sequence: logical position j is
    read from block table_row[j // block_size] at offset j % block_size. Table
    entries past ceil(length / block_size) are not read."""
    nb = math.ceil(length / block_size)
    blocks = np.asarray(table_row[:nb], dtype=np.int64)
    H = k_cache.shape[1]
    x = _x(k_cache)
    D = k_cache.shape[2] * x
    K = k_cache[blocks].transpose(0, 3, 1, 2, 4).reshape(nb * block_size, H, D)[:length]
    V = v_cache[blocks].transpose(0, 2, 4, 1, 3).reshape(nb * block_size, H, D)[:length]
    if k_cache.dtype == np.uint8:
        values = _fp8.decode_table()
        K = values[K] * np.asarray(k_scale, np.float32).astype(np.float64)[None, :, None]
        V = values[V] * np.asarray(v_scale, np.float32).astype(np.float64)[None, :, None]
    else:
        K = bf16_to_f64(K)
        V = bf16_to_f64(V)
    return K, V


def depage_raw(k_cache, v_cache, table_row, length, block_size):
    """Stored bit patterns (uint16 / uint8) of one sequence, [length, Hkv, D]."""
    nb = math.ceil(length / block_size)
    blocks = np.asarray(table_row[:nb], dtype=np.int64)
    H = k_cache.shape[1]
    x = _x(k_cache)
    D = k_cache.shape[2] * x
    K = k_cache[blocks].transpose(0, 3, 1, 2, 4).reshape(nb * block_size, H, D)[:length]
    V = v_cache[blocks].transpose(0, 2, 4, 1, 3).reshape(nb * block_size, H, D)[:length]
    return K, V
