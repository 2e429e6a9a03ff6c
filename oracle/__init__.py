"""CPU oracle for paged GQA/MQA decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The
library under ``paged_gqa_decode_lgm_amd/`` never does: it fails loudly when
its HIP extension is missing instead of falling back here.

What it is: a plain, slow, obviously correct fp64 NumPy statement of what the
decode hot path computes, written from the pages (Loom Kernels' README on
fused NeoX RoPE + paged-KV write, static FP8 E4M3 KV write, paged MQA/GQA
decode and local split-K/LSE merge; mainarch's README, decode-attention
section, on FlashDecoding split-KV, paged block tables, GQA sharing and OCP
e4m3fn KV; microLLM-rocm's ledger on split-half RoPE and per-row positions).
It shares no code with the HIP path: no kernels, headers, helpers, tables or
constant generators, and imports nothing from it.

Modules
  codecs     bf16 round-to-nearest-even, OCP E4M3 (e4m3fn) decode / encode
  rope       NeoX (split-half) rotary embedding, fp64 and the fp32 recipe
  append     fused RoPE + paged-KV append of the new token
  attention  block-table gather, softmax attention, split-K partials, LSE merge

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, library routines or hand-derived fixtures in
``tests/golden/``.  None is "parity unpinned".
"""
from . import codecs, rope, append, attention  # noqa: F401
