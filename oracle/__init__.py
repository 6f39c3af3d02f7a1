"""CPU oracle for the paged KV-cache path — TEST INFRASTRUCTURE, not product code.

Plain, slow, obviously correct numpy implementations of what the GPU path
computes, in float64 (float32 only where the fp8 encoding step fixes it).
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library
and imports nothing from ``paged_kv_cache_store_amd``.

Modules
* ``fp8``       — OCP FP8 E4M3 ("e4m3fn") encode/decode from the format's definition.
* ``cache``     — slot-mapping store into the block pool and de-paging through
                  a block table, in the library's physical layout.
* ``attention`` — decode and causal varlen prefill attention, written as the
                  dense definition on the de-paged keys/values.
* ``norm``      — residual add + RMSNorm, and float64 -> bf16 rounding.

What pins each function (none is pinned only against itself):
* fp8.encode/decode — exhaustive comparison with torch's float8_e4m3fn cast
  (an OCP e4m3fn conversion) on every bf16 pattern divided by several scales,
  hand cases (largest value, tie-to-even in the subnormal range, saturation),
  and the code table's closed forms.
* cache.store/depage — bit-exact round trip, untouched slots keep their
  sentinel, hand-derived flat offsets of the documented layout.
* attention.decode/prefill — closed forms (context 1 returns v0; identical
  keys or scale 0 return mean(V); a dominant key returns its value), torch's
  scaled_dot_product_attention in float64 with an explicit boolean mask,
  and invariants (physical-block permutation, shared prefix vs private
  copies, GQA vs replicated MHA, chunked prefill vs full causal prefill,
  decode vs prefill with one query row).
* norm.f64_to_bf16_bits — hand cases (ties to even, a case where rounding via
  float32 would differ, overflow, subnormals, signed zero, NaN) and torch's
  float32 -> bfloat16 cast on float32 inputs.
* norm.add_rmsnorm — torch's rms_norm in float64, torch's bfloat16 addition
  for the residual sum, and closed forms (constant rows, one-hot rows, scale
  invariance).
"""
from . import fp8, cache, attention, norm  # noqa: F401
