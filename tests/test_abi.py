"""C-ABI contract on the CPU: the library loads, exports every function the
header declares, and rejects every invalid argument with its own status and
a message naming the function and the argument, before any HIP call (so
these run without a GPU; fake but aligned addresses are never dereferenced)."""
import ctypes
import math

import pytest

import paged_gqa_decode_lgm_amd as L
from paged_gqa_decode_lgm_amd import _binding as Bn

INV, UNS, WS = L.LGM_ERR_INVALID_ARGUMENT, L.LGM_ERR_UNSUPPORTED, L.LGM_ERR_WORKSPACE_TOO_SMALL
A = 1 << 32  # fake device addresses, far apart, 256-byte aligned


def addr(i):
    return A * (i + 1)


SLOT = 4096  # LGM_COUNTER_SLOT_BYTES: the counters at the start of every nonzero attention workspace


def test_counter_slot_constant():
    import re
    from pathlib import Path
    text = (Path(L.__file__).resolve().parents[1] / "include" / "lgm.h").read_text()
    assert int(re.search(r"#define\s+LGM_COUNTER_SLOT_BYTES\s+(\d+)u", text).group(1)) == SLOT


def dims(**kw):
    d = dict(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=1000,
             max_blocks_per_seq=512)
    d.update(kw)
    return L.make_dims(**d)


def test_library_loads_and_exports_every_header_function():
    lib = L.lib()
    names = L.header_functions()
    assert set(names) == {"lgm_rope_kv_append", "lgm_paged_decode_partition_size", "lgm_paged_decode_workspace_size",
                          "lgm_paged_decode_attn", "lgm_paged_decode_attn_static", "lgm_check_block_tables",
                          "lgm_lse_merge", "lgm_last_error",
                          "lgm_abi_version", "lgm_stream_read_probe", "lgm_paged_mla_partition_size",
                          "lgm_paged_mla_workspace_size", "lgm_paged_mla_decode"}
    for n in names:
        assert hasattr(lib, n), n
    assert L.lgm_abi_version() == 7


def test_build_entry_abi_check_matches_header():
    import __graft_entry__

    __graft_entry__.check_abi()


# ------------------------------------------------------------------ append
def _append(**over):
    a = dict(qkv=addr(0), qkv_row_stride=(32 + 16) * 128, q_out=addr(1), k_cache=addr(2), v_cache=addr(3),
             block_tables=addr(4), context_lens=addr(5), k_scale=None, v_scale=None, rope_theta=5e5, dims=dims(),
             act_dtype=L.LGM_BF16, cache_dtype=L.LGM_BF16, stream=0)
    a.update(over)
    return L.lgm_rope_kv_append(**a)


APPEND_BAD = [
    (dict(dims=dims(num_seqs=-1)), INV, "num_seqs"),
    (dict(dims=dims(num_q_heads=30)), INV, "num_q_heads"),
    (dict(dims=dims(num_kv_heads=0)), INV, "num_kv_heads"),
    (dict(dims=dims(head_dim=127)), INV, "head_dim"),
    (dict(dims=dims(head_dim=512), qkv_row_stride=48 * 512), UNS, "head_dim"),
    (dict(dims=dims(block_size=0)), INV, "block_size"),
    (dict(dims=dims(num_blocks=0)), INV, "num_blocks"),
    (dict(dims=dims(max_blocks_per_seq=0)), INV, "max_blocks_per_seq"),
    (dict(act_dtype=L.LGM_F32), UNS, "act_dtype"),
    (dict(act_dtype=7), INV, "act_dtype"),
    (dict(cache_dtype=9), INV, "cache_dtype"),
    (dict(rope_theta=0.0), INV, "rope_theta"),
    (dict(rope_theta=float("nan")), INV, "rope_theta"),
    (dict(qkv_row_stride=100), INV, "qkv_row_stride"),
    (dict(cache_dtype=L.LGM_FP8_E4M3), INV, "k_scale"),
    (dict(cache_dtype=L.LGM_FP8_E4M3, k_scale=addr(6)), INV, "v_scale"),
    (dict(k_scale=addr(6), v_scale=addr(7)), INV, "k_scale"),
    (dict(cache_dtype=L.LGM_FP4_E2M1, k_scale=addr(6), v_scale=addr(7)), INV, "k_scale"),
    (dict(flags=0x8), INV, "flags"),
    (dict(flags=L.LGM_SCALE_PER_TENSOR), INV, "LGM_SCALE_PER_TENSOR"),
    # a per-tensor scale is 4 bytes: v_scale 4 bytes after k_scale is fine, inside the per-head span is not
    (dict(cache_dtype=L.LGM_FP8_E4M3, k_scale=addr(6), v_scale=addr(6) + 16, q_out=addr(6) + 8), INV, "q_out"),
    (dict(cache_dtype=L.LGM_FP4_E2M1, dims=dims(head_dim=48), qkv_row_stride=48 * 48), UNS, "multiple of 32"),
    (dict(cache_dtype=L.LGM_FP4_E2M1, act_dtype=L.LGM_F32), UNS, "FP4_E2M1"),
    # an FP4 pool is num_blocks * block_size * Hkv * (D/2 + D/32) bytes = 1000 * 16 * 8 * 68
    (dict(cache_dtype=L.LGM_FP4_E2M1, v_cache=addr(2) + 1000 * 16 * 8 * 68 - 16), INV, "k_cache"),
    (dict(qkv=None), INV, "qkv"),
    (dict(q_out=None), INV, "q_out"),
    (dict(k_cache=None), INV, "k_cache"),
    (dict(v_cache=None), INV, "v_cache"),
    (dict(block_tables=None), INV, "block_tables"),
    (dict(context_lens=None), INV, "context_lens"),
    (dict(q_out=addr(0) + 256), INV, "q_out"),          # overlaps qkv
    (dict(v_cache=addr(2) + 1024), INV, "k_cache"),     # pools overlap
]


@pytest.mark.parametrize("over,status,word", APPEND_BAD)
def test_append_rejects(over, status, word):
    with pytest.raises(L.LgmError) as e:
        _append(**over)
    assert e.value.status == status
    assert e.value.message.startswith("lgm_rope_kv_append:")
    assert word in e.value.message


def test_append_empty_batch_is_a_noop():
    _append(dims=dims(num_seqs=0), qkv=None, q_out=None)
    assert L.lgm_last_error() == ""


# ------------------------------------------------------------------ attention
def _attn(**over):
    a = dict(out=addr(0), out_lse=addr(1), q=addr(2), q_seq_stride=32 * 128, k_cache=addr(3), v_cache=addr(4),
             block_tables=addr(5), context_lens=addr(6), k_scale=None, v_scale=None, softmax_scale=0.0883883,
             partition_size=512, max_context_len=8192, workspace=addr(7), workspace_bytes=1 << 30, dims=dims(),
             act_dtype=L.LGM_BF16, cache_dtype=L.LGM_BF16, stream=0)
    a.update(over)
    return L.lgm_paged_decode_attn(**a)


ATTN_BAD = [
    (dict(dims=dims(head_dim=96)), UNS, "head_dim"),
    (dict(dims=dims(block_size=32, max_blocks_per_seq=256)), UNS, "block_size"),
    (dict(dims=dims(num_q_heads=64, num_kv_heads=2), q_seq_stride=64 * 128), UNS, "group"),
    (dict(dims=dims(num_q_heads=32, num_kv_heads=2), act_dtype=L.LGM_F32, cache_dtype=L.LGM_F32), UNS, "group"),
    (dict(act_dtype=L.LGM_F32), UNS, "act"),
    (dict(act_dtype=5), INV, "act_dtype"),
    (dict(softmax_scale=float("inf")), INV, "softmax_scale"),
    (dict(q_seq_stride=100), INV, "q_seq_stride"),
    (dict(max_context_len=8193), INV, "max_context_len"),
    (dict(max_context_len=-1), INV, "max_context_len"),
    (dict(partition_size=24), INV, "partition_size"),
    (dict(partition_size=-16), INV, "partition_size"),
    (dict(workspace=None), WS, "workspace"),
    (dict(workspace_bytes=1000), WS, "workspace_bytes"),
    (dict(workspace=addr(7) + 8), INV, "workspace"),
    (dict(cache_dtype=L.LGM_FP8_E4M3), INV, "k_scale"),
    (dict(k_scale=addr(8), v_scale=addr(9)), INV, "k_scale"),
    (dict(cache_dtype=L.LGM_FP4_E2M1, k_scale=addr(8), v_scale=addr(9)), INV, "k_scale"),
    (dict(flags=L.LGM_ROPE_INTERLEAVED), INV, "flags"),
    (dict(flags=0x10), INV, "flags"),
    (dict(flags=L.LGM_SCALE_PER_TENSOR), INV, "LGM_SCALE_PER_TENSOR"),
    (dict(cache_dtype=L.LGM_FP4_E2M1, dims=dims(head_dim=64), q_seq_stride=32 * 64), UNS, "FP4_E2M1"),
    (dict(cache_dtype=L.LGM_FP4_E2M1, act_dtype=L.LGM_FP4_E2M1), UNS, "act"),
    (dict(cache_dtype=L.LGM_FP4_E2M1, workspace=addr(3) + 1000 * 16 * 8 * 68 - 256), INV, "workspace"),
    (dict(out=None), INV, "out"),
    (dict(q=None), INV, "q"),
    (dict(k_cache=None), INV, "k_cache"),
    (dict(v_cache=None), INV, "v_cache"),
    (dict(block_tables=None), INV, "block_tables"),
    (dict(context_lens=None), INV, "context_lens"),
    (dict(k_cache=addr(3) + 8), INV, "aligned"),
    (dict(out=addr(2) + 512), INV, "'out' overlaps input 'q'"),
    (dict(out_lse=addr(0) + 64), INV, "'out' overlaps output 'out_lse'"),
    (dict(workspace=addr(3)), INV, "workspace"),
]


@pytest.mark.parametrize("over,status,word", ATTN_BAD)
def test_attention_rejects(over, status, word):
    with pytest.raises(L.LgmError) as e:
        _attn(**over)
    assert e.value.status == status
    assert e.value.message.startswith("lgm_paged_decode_attn:")
    assert word in e.value.message


def test_attention_empty_batch_is_a_noop():
    _attn(dims=dims(num_seqs=0), out=None, q=None)


# ------------------------------------------------------------------ block-table check
def _tcheck(**over):
    a = dict(block_tables=addr(5), context_lens=addr(6), dims=dims(), max_context_len=8192, status=addr(7), stream=0)
    a.update(over)
    return L.lgm_check_block_tables(**a)


TCHECK_BAD = [
    (dict(dims=dims(num_q_heads=30)), INV, "num_q_heads"),
    (dict(dims=dims(num_blocks=0)), INV, "num_blocks"),
    (dict(max_context_len=8193), INV, "max_context_len"),
    (dict(max_context_len=-1), INV, "max_context_len"),
    (dict(dims=dims(num_seqs=70000)), UNS, "num_seqs"),
    (dict(block_tables=None), INV, "block_tables"),
    (dict(context_lens=None), INV, "context_lens"),
    (dict(status=None), INV, "status"),
    (dict(status=addr(7) + 2), INV, "aligned"),
    (dict(status=addr(5) + 64), INV, "'status' overlaps input 'block_tables'"),
]


@pytest.mark.parametrize("over,status,word", TCHECK_BAD)
def test_table_check_rejects(over, status, word):
    with pytest.raises(L.LgmError) as e:
        _tcheck(**over)
    assert e.value.status == status
    assert e.value.message.startswith("lgm_check_block_tables:")
    assert word in e.value.message


def test_table_check_empty_batch_is_a_noop():
    _tcheck(dims=dims(num_seqs=0), block_tables=None, context_lens=None, status=None)


# ------------------------------------------------------------------ attention without a workspace
def _attn_static(**over):
    a = dict(out=addr(0), out_lse=addr(1), q=addr(2), q_seq_stride=32 * 128, k_cache=addr(3), v_cache=addr(4),
             block_tables=addr(5), context_lens=addr(6), k_scale=None, v_scale=None, softmax_scale=0.0883883,
             partition_size=512, max_context_len=8192, dims=dims(), act_dtype=L.LGM_BF16, cache_dtype=L.LGM_BF16,
             stream=0)
    a.update(over)
    return L.lgm_paged_decode_attn_static(**a)


STATIC_BAD = [(over, status, word) for over, status, word in ATTN_BAD if not any(k.startswith("workspace") for k in over)] + [
    # C4-shaped long contexts in partitions of 64 need 66 MB of partial records: more than the array holds
    (dict(dims=dims(num_seqs=4, max_blocks_per_seq=8192), max_context_len=131072, partition_size=64), WS,
     "LGM_STATIC_SCRATCH_BYTES"),
]


@pytest.mark.parametrize("over,status,word", STATIC_BAD)
def test_attention_static_rejects(over, status, word):
    """The allocation-free entry point validates exactly as the workspace one
    does, and refuses plans whose workspace exceeds its device array, before
    any HIP call."""
    with pytest.raises(L.LgmError) as e:
        _attn_static(**over)
    assert e.value.status == status
    assert e.value.message.startswith("lgm_paged_decode_attn_static:")
    assert word in e.value.message


def test_attention_static_capacity_covers_the_workloads():
    """The array holds the workspace of every benchmarked shape: 64 contexts
    of up to 8192 tokens in equal ranges, 128 FP8 or FP4 contexts of up to
    4096, and four 131072-token contexts in partitions of 512."""
    cap = 32 << 20
    assert L.lgm_paged_decode_workspace_size(dims(), 8192, 0, L.LGM_BF16) <= cap
    for cache in (L.LGM_FP8_E4M3, L.LGM_FP4_E2M1):
        assert L.lgm_paged_decode_workspace_size(dims(num_seqs=128, max_blocks_per_seq=256), 4096, 0, cache) <= cap
    assert L.lgm_paged_decode_workspace_size(dims(num_seqs=4, max_blocks_per_seq=8192), 131072, 512,
                                             L.LGM_BF16) <= cap
    too_big = L.lgm_paged_decode_workspace_size(dims(num_seqs=4, max_blocks_per_seq=8192), 131072, 64, L.LGM_BF16)
    assert too_big > cap


def test_attention_static_empty_batch_is_a_noop():
    _attn_static(dims=dims(num_seqs=0), out=None, q=None)


# ------------------------------------------------------------------ plan queries
@pytest.mark.parametrize("d,max_ctx,ps,want", [
    (dims(), 8192, 0, 0),                                                 # whole-row ranges
    (dims(num_seqs=128, max_blocks_per_seq=256), 4096, 0, 0),
    (dims(num_seqs=4, max_blocks_per_seq=8192), 131072, 0, 0),
    (dims(num_q_heads=16, num_kv_heads=2), 8192, 0, 0),                   # head groups of 2: token slices
    (dims(num_q_heads=24, num_kv_heads=6), 8192, 0, 0),
    (dims(num_seqs=256, num_q_heads=16, num_kv_heads=2), 8192, 0, 0),
    (dims(num_seqs=128, num_q_heads=8, num_kv_heads=1), 8192, 0, 0),      # head groups of 1
    # single launch (<= 1022 streams, <= 16384 tiles): partitions that balance the workgroups, 128-token steps
    (dims(num_seqs=2, num_q_heads=12, num_kv_heads=2, max_blocks_per_seq=128), 2048, 0, 128),
    (dims(num_seqs=1, max_blocks_per_seq=512), 8192, 0, 256),             # 8 streams x 256 tiles
    (dims(num_seqs=1, num_q_heads=4, num_kv_heads=1, max_blocks_per_seq=4096), 65536, 0, 1024),  # <= 64 per context
    (dims(num_seqs=1022, num_q_heads=16, num_kv_heads=1, max_blocks_per_seq=8), 100, 0, 128),
    (dims(num_seqs=1023, num_q_heads=16, num_kv_heads=1, max_blocks_per_seq=8), 100, 0, 0),  # 1023 streams: ranges
    (dims(num_seqs=1, max_blocks_per_seq=4096), 65536, 0, 2048),          # 8 x 2048 = 16384 tiles
    (dims(num_seqs=1, max_blocks_per_seq=4098), 65537, 0, 0),             # 8 x 2049 tiles: whole-row ranges
    (dims(head_dim=64), 8192, 0, 512),                                    # vector-ALU shape
    (dims(num_seqs=2, num_q_heads=12, num_kv_heads=2, head_dim=64, max_blocks_per_seq=128), 2048, 0, 64),
    (dims(num_seqs=4, max_blocks_per_seq=8192), 131072, 512, 512),         # explicit
    (dims(num_seqs=1, num_q_heads=4, num_kv_heads=1, head_dim=64, max_blocks_per_seq=16), 256, 256, 256),
    (dims(), 8192, 16384, 8192),                                          # larger than the context: no split
    (dims(), 100, 512, 112),                                              # clamped to the rounded-up context
])
def test_partition_plan(d, max_ctx, ps, want):
    assert L.lgm_paged_decode_partition_size(d, max_ctx, ps, L.LGM_BF16) == want


@pytest.mark.parametrize("cache,want", [(L.LGM_BF16, 0), (L.LGM_FP4_E2M1, 0), (L.LGM_FP8_E4M3, 4096)])
def test_single_launch_tile_cap_by_cache(cache, want):
    """8 streams x 4096 tiles = 32768: within the FP8 cap (half the bytes per tile) only."""
    assert L.lgm_paged_decode_partition_size(dims(num_seqs=1, max_blocks_per_seq=8192), 131072, 0, cache) == want


def partitions_brute_force(max_ctx, ps, tps):
    """Most partitions any context 0..max_ctx is cut into: its full partitions
    of ps tokens plus the rest in partitions of tps tokens (one if empty)."""
    return max(1 if c == 0 else c // ps + -(-(c % ps) // tps) for c in range(max_ctx + 1))


def test_workspace_size_formula():
    al = lambda x: (x + 255) // 256 * 256
    # whole-row partition plan: whole-tile partitions of >= 256 tokens, >= 64 of them at the longest
    # context and >= 256 units in the batch; plain ceil(L / ps) partitions after the counter slot
    long = dims(num_seqs=4, max_blocks_per_seq=8192)
    long2 = dims(num_seqs=4, num_q_heads=12, num_kv_heads=2, max_blocks_per_seq=8192)   # head groups of 2
    assert L.lgm_paged_decode_workspace_size(long2, 131072, 512, L.LGM_BF16) == (
        SLOT + al(4 * 12 * 256 * 128 * 4) + al(4 * 12 * 256 * 4))
    long1 = dims(num_seqs=4, num_q_heads=8, num_kv_heads=1, max_blocks_per_seq=8192)  # one kv head: work queue
    P1 = partitions_brute_force(131072, 512, 256)
    assert P1 == 257
    assert L.lgm_paged_decode_workspace_size(long1, 131072, 512, L.LGM_BF16) == (
        SLOT + al(4 * 8 * P1 * 128 * 4) + al(4 * 8 * P1 * 4))
    assert L.lgm_paged_decode_workspace_size(long, 131072, 512, L.LGM_BF16) == (
        SLOT + al(4 * 32 * 256 * 128 * 4) + al(4 * 32 * 256 * 4))
    assert L.lgm_paged_decode_workspace_size(long, 131072, 2048, L.LGM_FP8_E4M3) == (
        SLOT + al(4 * 32 * 64 * 128 * 4) + al(4 * 32 * 64 * 4))
    d = dims()                                     # 16 partitions at the longest context: work-queue kernel
    assert L.lgm_paged_decode_workspace_size(d, 8192, 8192, L.LGM_BF16) == SLOT    # one partition
    assert L.lgm_paged_decode_workspace_size(d, 8192, 8192, L.LGM_FP8_E4M3) == SLOT
    d2 = dims(num_q_heads=16, num_kv_heads=2)      # work-queue shape: 256 bytes of work counters first
    assert L.lgm_paged_decode_workspace_size(d2, 8192, 8192, L.LGM_BF16) == SLOT    # one partition
    P = partitions_brute_force(8192, 512, 256)     # tails in half partitions
    assert P == 17
    out_b = 64 * 16 * P * 128 * 4
    lse_b = 64 * 16 * P * 4
    assert L.lgm_paged_decode_workspace_size(d2, 8192, 512, L.LGM_BF16) == SLOT + al(out_b) + al(lse_b)
    # below the whole-row partition minimum: the work-queue kernel, tails included
    P64 = partitions_brute_force(8192, 64, 32)
    assert L.lgm_paged_decode_workspace_size(d, 8192, 64, L.LGM_BF16) == (
        SLOT + al(64 * 32 * P64 * 128 * 4) + al(64 * 32 * P64 * 4))
    lse_b = 64 * 32 * P * 4
    v = dims(head_dim=64)                          # vector-ALU shape: the counter slot, then the partials
    assert L.lgm_paged_decode_workspace_size(v, 8192, 8192, L.LGM_BF16) == 0
    assert L.lgm_paged_decode_workspace_size(v, 8192, 512, L.LGM_BF16) == (
        SLOT + al(64 * 32 * P * 64 * 4) + al(lse_b))


@pytest.mark.parametrize("max_ctx,ps", [(100, 16), (100, 64), (1000, 96), (3000, 512), (4096, 1024), (17, 16),
                                        (5000, 4096), (2048, 2048)])
def test_partition_count_bound(max_ctx, ps):
    """The library's partition count bound equals the brute-force maximum."""
    tps = ps if max_ctx <= ps else max(16, ps // 2 // 16 * 16)
    P = partitions_brute_force(max_ctx, ps, tps)
    d = dims(head_dim=64, max_blocks_per_seq=(max_ctx + 15) // 16)
    al = lambda x: (x + 255) // 256 * 256
    want = 0 if P == 1 else SLOT + al(64 * 32 * P * 64 * 4) + al(64 * 32 * P * 4)
    assert L.lgm_paged_decode_workspace_size(d, max_ctx, ps, L.LGM_BF16) == want
    assert L.lgm_last_error() == ""
    with pytest.raises(L.LgmError):
        L.lgm_paged_decode_workspace_size(d, 8192, 10, L.LGM_BF16)


def test_row_plan_workspace_formula():
    al = lambda x: (x + 255) // 256 * 256
    d = dims()                                     # 8 kv heads per workgroup, 64 streams of 256 tiles
    W, rows = 256, 8 * 4
    want = SLOT + al(W * 2 * rows * 128 * 4) + al(W * 2 * rows * 4) + 2 * al(64 * 4)
    assert L.lgm_paged_decode_workspace_size(d, 8192, 0, L.LGM_BF16) == want
    assert L.lgm_paged_decode_workspace_size(d, 8192, 0, L.LGM_FP8_E4M3) == want
    assert L.lgm_paged_decode_workspace_size(d, 8192, 0, L.LGM_FP4_E2M1) == want
    # 2 and 1 kv heads: head groups of 2 and 1 (HG * G rows per record)
    h2 = dims(num_q_heads=16, num_kv_heads=2)
    assert L.lgm_paged_decode_workspace_size(h2, 8192, 0, L.LGM_BF16) == (
        SLOT + al(256 * 2 * 16 * 128 * 4) + al(256 * 2 * 16 * 4) + 2 * al(64 * 4))
    h1 = dims(num_seqs=128, num_q_heads=8, num_kv_heads=1)
    assert L.lgm_paged_decode_workspace_size(h1, 8192, 0, L.LGM_FP4_E2M1) == (
        SLOT + al(256 * 2 * 8 * 128 * 4) + al(256 * 2 * 8 * 4) + 2 * al(128 * 4))
    # 8 kv heads in groups of 8 up to 8 query heads per kv head, in groups of 4 past that
    g8 = dims(num_q_heads=64)
    assert L.lgm_paged_decode_workspace_size(g8, 8192, 0, L.LGM_BF16) == (
        SLOT + al(256 * 2 * 64 * 128 * 4) + al(256 * 2 * 64 * 4) + 2 * al(64 * 4))
    g16 = dims(num_q_heads=128)
    assert L.lgm_paged_decode_workspace_size(g16, 8192, 0, L.LGM_FP8_E4M3) == (
        SLOT + al(256 * 2 * 64 * 128 * 4) + al(256 * 2 * 64 * 4) + 2 * al(128 * 4))
    # 8 streams x 4096 tiles, past the single-launch cap: 2 head groups of 4 x 4096 tiles, two a range
    long = dims(num_seqs=2, num_q_heads=16, num_kv_heads=4, max_blocks_per_seq=8192)
    W, rows = 256, 4 * 4
    assert L.lgm_paged_decode_workspace_size(long, 131072, 0, L.LGM_BF16) == (
        SLOT + al(W * 2 * rows * 128 * 4) + al(W * 2 * rows * 4) + 2 * al(2 * 4))
    few = dims(num_seqs=1100, num_q_heads=16, num_kv_heads=4, max_blocks_per_seq=1)  # 4400 streams of one tile
    W = 1100 // 2
    W = 256 if W > 256 else W
    assert L.lgm_paged_decode_workspace_size(few, 16, 0, L.LGM_BF16) == (
        SLOT + al(W * 2 * rows * 128 * 4) + al(W * 2 * rows * 4) + 2 * al(1100 * 4))


def test_single_launch_workspace_formula():
    """The counter slot (its words 2.. are the arrival counters), then one
    record per (stream, partition): G fp32 rows of D, then G LSEs."""
    al = lambda x: (x + 255) // 256 * 256
    c2 = dims(num_seqs=2, num_q_heads=12, num_kv_heads=2, max_blocks_per_seq=128)  # 4 streams x 16 partitions
    for cache in (L.LGM_BF16, L.LGM_FP8_E4M3, L.LGM_FP4_E2M1):
        assert L.lgm_paged_decode_workspace_size(c2, 2048, 0, cache) == SLOT + al(4 * 16 * 6 * 128 * 4) + al(4 * 16 * 6 * 4)
    assert L.lgm_paged_decode_workspace_size(c2, 100, 0, L.LGM_BF16) == SLOT    # one partition: no records
    assert L.lgm_paged_decode_workspace_size(c2, 0, 0, L.LGM_BF16) == SLOT


def test_too_many_partitions_is_unsupported():
    d = dims(num_seqs=1, max_blocks_per_seq=1 << 17)
    with pytest.raises(L.LgmError) as e:
        L.lgm_paged_decode_workspace_size(d, 1 << 21, 16, L.LGM_BF16)
    assert "partitions: at most 65535" in e.value.message


# ------------------------------------------------------------------ merge
def _merge(**over):
    a = dict(out=addr(0), out_lse=addr(1), partial_out=addr(2), partial_lse=addr(3), num_partitions=None,
             num_seqs=4, num_q_heads=32, head_dim=128, max_partitions=256, out_dtype=L.LGM_BF16, stream=0)
    a.update(over)
    return L.lgm_lse_merge(**a)


MERGE_BAD = [
    (dict(num_seqs=-2), INV, "num_seqs"),
    (dict(num_q_heads=0), INV, "num_q_heads"),
    (dict(max_partitions=0), INV, "max_partitions"),
    (dict(out_dtype=L.LGM_FP8_E4M3), UNS, "out_dtype"),
    (dict(head_dim=96), UNS, "head_dim"),
    (dict(out=None), INV, "out"),
    (dict(partial_out=None), INV, "partial_out"),
    (dict(partial_lse=None), INV, "partial_lse"),
    (dict(partial_out=addr(2) + 4), INV, "aligned"),
    (dict(out=addr(2) + 64), INV, "overlaps"),
]


@pytest.mark.parametrize("over,status,word", MERGE_BAD)
def test_merge_rejects(over, status, word):
    with pytest.raises(L.LgmError) as e:
        _merge(**over)
    assert e.value.status == status
    assert e.value.message.startswith("lgm_lse_merge:")
    assert word in e.value.message


def test_binding_refuses_to_run_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(Bn, "_lib", None)
    monkeypatch.setattr(Bn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        Bn.lib()


# ------------------------------------------------------------------ streaming probe
@pytest.mark.parametrize("kw, msg", [
    (dict(src=None), "src is NULL"),
    (dict(sink=None), "sink is NULL"),
    (dict(src=addr(0) + 8), "16-byte aligned"),
    (dict(num_workgroups=0), "num_workgroups"),
    (dict(num_workgroups=65537), "num_workgroups"),
    (dict(nbytes=0), "positive multiple"),
    (dict(nbytes=4 * 16384 + 16), "positive multiple"),
    (dict(nbytes=(1 << 31) * 4, num_workgroups=2), "INT32_MAX"),
    (dict(sink=addr(0) + 64), "overlap"),
])
def test_stream_probe_rejects_before_launch(kw, msg):
    a = dict(src=addr(0), nbytes=4 * 16384, num_workgroups=4, nontemporal=1, sink=addr(1), stream=0)
    a.update(kw)
    with pytest.raises(L.LgmError) as e:
        Bn.lgm_stream_read_probe(**a)
    assert e.value.status == L.LGM_ERR_INVALID_ARGUMENT
    assert msg in e.value.message



# ------------------------------------------------------------------ paged MLA
def mla_dims(**kw):
    d = dict(num_seqs=1, num_heads=8, latent_dim=512, rope_dim=64, block_size=64, num_blocks=1000,
             max_blocks_per_seq=800)
    d.update(kw)
    return L.make_mla_dims(**d)


def _mla(**over):
    a = dict(out=addr(0), out_lse=addr(1), q_latent=addr(2), q_pe=addr(3), ckv_cache=addr(4), kpe_cache=addr(5),
             block_tables=addr(6), context_lens=addr(7), ckv_scale=addr(8), softmax_scale=0.0722,
             partition_size=832, max_context_len=51200, workspace=addr(9), workspace_bytes=1 << 30,
             dims=mla_dims(), ckv_dtype=L.LGM_FP8_E4M3, stream=0)
    a.update(over)
    return L.lgm_paged_mla_decode(**a)


MLA_BAD = [
    (dict(dims=mla_dims(latent_dim=256)), UNS, "latent_dim"),
    (dict(dims=mla_dims(rope_dim=32)), UNS, "rope_dim"),
    (dict(dims=mla_dims(num_heads=17)), UNS, "num_heads"),
    (dict(dims=mla_dims(num_heads=0)), INV, "num_heads"),
    (dict(dims=mla_dims(block_size=48, max_blocks_per_seq=1100)), UNS, "block_size"),
    (dict(dims=mla_dims(block_size=24, max_blocks_per_seq=3000)), UNS, "block_size"),
    (dict(dims=mla_dims(num_seqs=-1)), INV, "num_seqs"),
    (dict(dims=mla_dims(num_seqs=70000)), UNS, "num_seqs"),
    (dict(dims=mla_dims(num_blocks=0)), INV, "num_blocks"),
    (dict(ckv_dtype=L.LGM_BF16), UNS, "ckv_dtype"),
    (dict(ckv_dtype=9), INV, "ckv_dtype"),
    (dict(softmax_scale=float("nan")), INV, "softmax_scale"),
    (dict(max_context_len=51201), INV, "max_context_len"),
    (dict(partition_size=48), INV, "partition_size"),
    (dict(partition_size=-32), INV, "partition_size"),
    (dict(workspace=None), WS, "workspace"),
    (dict(workspace_bytes=4096), WS, "workspace_bytes"),
    (dict(workspace=addr(9) + 16), INV, "workspace"),
    (dict(ckv_scale=None), INV, "ckv_scale"),
    (dict(out=None), INV, "out"),
    (dict(q_latent=None), INV, "q_latent"),
    (dict(q_pe=None), INV, "q_pe"),
    (dict(ckv_cache=None), INV, "ckv_cache"),
    (dict(kpe_cache=None), INV, "kpe_cache"),
    (dict(block_tables=None), INV, "block_tables"),
    (dict(context_lens=None), INV, "context_lens"),
    (dict(q_pe=addr(3) + 8), INV, "aligned"),
    (dict(out=addr(0) + 2), INV, "aligned"),
    (dict(out=addr(2) + 1024), INV, "'out' overlaps input 'q_latent'"),
    (dict(workspace=addr(4) + 256), INV, "overlaps input 'ckv_cache'"),
]


@pytest.mark.parametrize("over,status,word", MLA_BAD)
def test_mla_rejects(over, status, word):
    with pytest.raises(L.LgmError) as e:
        _mla(**over)
    assert e.value.status == status
    assert e.value.message.startswith("lgm_paged_mla_decode:")
    assert word in e.value.message


def test_mla_empty_batch_is_a_noop():
    _mla(dims=mla_dims(num_seqs=0), out=None, q_latent=None, workspace=None, workspace_bytes=0)


@pytest.mark.parametrize("B,max_ctx,ps,want", [
    (1, 51200, 832, 832),      # explicit: kept
    (1, 51200, 0, 256),        # ceil(51200 / 256) = 200 -> 256 (whole 64-token tiles)
    (2, 51200, 0, 448),        # ceil(102400 / 256) = 400 -> 448
    (16, 51200, 0, 3200),      # already whole tiles
    (64, 4096, 0, 1024),       # 64 * 4096 / 256
    (1, 1000, 0, 128),         # at least one tile per wave
    (1, 100, 0, 128),          # capped to the context rounded up to 32
    (1, 100, 4096, 128),
    (1, 0, 0, 32),
    (3, 70, 64, 64),
])
def test_mla_partition_plan(B, max_ctx, ps, want):
    assert L.lgm_paged_mla_partition_size(mla_dims(num_seqs=B), max_ctx, ps) == want


@pytest.mark.parametrize("B", [1, 2, 3, 7, 16, 64, 300])
@pytest.mark.parametrize("max_ctx", [1, 31, 129, 1000, 4097, 51200, 131072])
def test_mla_auto_partition_properties(B, max_ctx):
    """Library-chosen partitions are whole 64-token tiles of at least 128
    tokens, unless one partition covers the context (then the context rounded
    up to 32); a batch spreads over about one workgroup per compute unit."""
    d = mla_dims(num_seqs=B, max_blocks_per_seq=-(-max_ctx // 64) + 1)
    ps = L.lgm_paged_mla_partition_size(d, max_ctx, 0)
    cap = -(-max_ctx // 32) * 32
    assert 0 < ps <= cap
    if ps < cap:
        assert ps % 64 == 0 and ps >= 128
        # one 64-token tile fewer per partition would need more than 256 workgroups
        assert ps == 128 or B * max_ctx > 256 * (ps - 64)


@pytest.mark.parametrize("B,H,max_ctx,ps", [(1, 8, 51200, 832), (1, 8, 51200, 0), (4, 16, 3000, 96),
                                            (2, 1, 100, 0), (5, 8, 64, 64)])
def test_mla_workspace_formula(B, H, max_ctx, ps):
    d = mla_dims(num_seqs=B, num_heads=H)
    p = L.lgm_paged_mla_partition_size(d, max_ctx, ps)
    P = max(1, -(-max_ctx // p))
    al = lambda x: -(-x // 256) * 256
    want = 0 if P == 1 else al(B * H * P * 512 * 4) + al(B * H * P * 4)
    assert L.lgm_paged_mla_workspace_size(d, max_ctx, ps) == want


def test_merge_accepts_the_latent_width():
    # rejected only for its NULL output, after the head_dim check passed
    with pytest.raises(L.LgmError) as e:
        _merge(head_dim=512, out=None)
    assert "out is NULL" in e.value.message
