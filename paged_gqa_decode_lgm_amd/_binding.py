"""ctypes binding of liblgm.so (include/*.h): argument marshalling only.

Each function has the name and argument order of its C entry point.  Tensor
arguments may be torch tensors (their data_ptr() is passed), raw integer
addresses, or None for NULL.  ``stream`` defaults to torch's current stream
on the current device.  A nonzero lgm_status raises LgmError carrying the
status and the library's message.  If liblgm.so has not been built, every
call raises: there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import re

# LGM_LIBRARY selects another build of the library (e.g. the sanitizer build).
LIB_PATH = os.environ.get("LGM_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblgm.so")
INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "lgm.h")

LGM_OK, LGM_ERR_INVALID_ARGUMENT, LGM_ERR_UNSUPPORTED, LGM_ERR_WORKSPACE_TOO_SMALL, LGM_ERR_HIP = range(5)
LGM_F32, LGM_BF16, LGM_FP8_E4M3, LGM_FP4_E2M1 = 0, 1, 2, 3
LGM_ROPE_INTERLEAVED, LGM_CACHE_HND, LGM_SCALE_PER_TENSOR = 0x1, 0x2, 0x4
STATUS_NAMES = {0: "LGM_OK", 1: "LGM_ERR_INVALID_ARGUMENT", 2: "LGM_ERR_UNSUPPORTED",
                3: "LGM_ERR_WORKSPACE_TOO_SMALL", 4: "LGM_ERR_HIP"}


class LgmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class lgm_paged_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "max_blocks_per_seq")]

    def __repr__(self):
        return "lgm_paged_dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class lgm_mla_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_heads", "latent_dim", "rope_dim", "block_size", "num_blocks", "max_blocks_per_seq")]

    def __repr__(self):
        return "lgm_mla_dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_gqa_decode_lgm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        u32 = ctypes.c_uint32
        L.lgm_rope_kv_append.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, f32, lgm_paged_dims, i32, i32, u32, vp]
        L.lgm_rope_kv_append.restype = i32
        L.lgm_paged_decode_partition_size.argtypes = [lgm_paged_dims, i32, i32, i32]
        L.lgm_paged_decode_partition_size.restype = i32
        L.lgm_paged_decode_workspace_size.argtypes = [lgm_paged_dims, i32, i32, i32]
        L.lgm_paged_decode_workspace_size.restype = sz
        L.lgm_paged_decode_attn.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, f32, i32, i32, vp, sz,
                                            lgm_paged_dims, i32, i32, u32, vp]
        L.lgm_paged_decode_attn.restype = i32
        L.lgm_paged_decode_attn_static.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, f32, i32, i32,
                                                   lgm_paged_dims, i32, i32, u32, vp]
        L.lgm_paged_decode_attn_static.restype = i32
        L.lgm_check_block_tables.argtypes = [vp, vp, lgm_paged_dims, i32, vp, vp]
        L.lgm_check_block_tables.restype = i32
        L.lgm_lse_merge.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.lgm_lse_merge.restype = i32
        L.lgm_last_error.argtypes = []
        L.lgm_last_error.restype = ctypes.c_char_p
        L.lgm_abi_version.argtypes = []
        L.lgm_abi_version.restype = i32
        L.lgm_paged_mla_partition_size.argtypes = [lgm_mla_dims, i32, i32]
        L.lgm_paged_mla_partition_size.restype = i32
        L.lgm_paged_mla_workspace_size.argtypes = [lgm_mla_dims, i32, i32]
        L.lgm_paged_mla_workspace_size.restype = sz
        L.lgm_paged_mla_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, vp, sz, lgm_mla_dims,
                                           i32, vp]
        L.lgm_paged_mla_decode.restype = i32
        L.lgm_stream_read_probe.argtypes = [vp, sz, i32, i32, vp, vp]
        L.lgm_stream_read_probe.restype = i32
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions the headers under include/ declare."""
    names = []
    for h in sorted(os.listdir(INCLUDE)):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+(lgm_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return names


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is not None:
        return s if isinstance(s, int) else s.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def _check(status: int):
    if status != LGM_OK:
        raise LgmError(status, lib().lgm_last_error().decode())


def make_dims(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq):
    return lgm_paged_dims(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq)


def lgm_rope_kv_append(qkv, qkv_row_stride, q_out, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale,
                       rope_theta, dims, act_dtype, cache_dtype, flags=0, stream=None):
    _check(lib().lgm_rope_kv_append(_ptr(qkv), qkv_row_stride, _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_tables), _ptr(context_lens), _ptr(k_scale), _ptr(v_scale),
                                    rope_theta, dims, act_dtype, cache_dtype, flags, _stream(stream)))


def lgm_paged_decode_partition_size(dims, max_context_len, partition_size, cache_dtype) -> int:
    r = lib().lgm_paged_decode_partition_size(dims, max_context_len, partition_size, cache_dtype)
    if r < 0:
        raise LgmError(LGM_ERR_INVALID_ARGUMENT, lib().lgm_last_error().decode())
    return r


def lgm_paged_decode_workspace_size(dims, max_context_len, partition_size, cache_dtype) -> int:
    r = lib().lgm_paged_decode_workspace_size(dims, max_context_len, partition_size, cache_dtype)
    err = lib().lgm_last_error().decode()
    if r == 0 and err:
        raise LgmError(LGM_ERR_INVALID_ARGUMENT, err)
    return r


def lgm_paged_decode_attn(out, out_lse, q, q_seq_stride, k_cache, v_cache, block_tables, context_lens, k_scale,
                          v_scale, softmax_scale, partition_size, max_context_len, workspace, workspace_bytes, dims,
                          act_dtype, cache_dtype, flags=0, stream=None):
    _check(lib().lgm_paged_decode_attn(_ptr(out), _ptr(out_lse), _ptr(q), q_seq_stride, _ptr(k_cache),
                                       _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(k_scale),
                                       _ptr(v_scale), softmax_scale, partition_size, max_context_len,
                                       _ptr(workspace), workspace_bytes, dims, act_dtype, cache_dtype, flags,
                                       _stream(stream)))


def lgm_paged_decode_attn_static(out, out_lse, q, q_seq_stride, k_cache, v_cache, block_tables, context_lens,
                                 k_scale, v_scale, softmax_scale, partition_size, max_context_len, dims, act_dtype,
                                 cache_dtype, flags=0, stream=None):
    _check(lib().lgm_paged_decode_attn_static(_ptr(out), _ptr(out_lse), _ptr(q), q_seq_stride, _ptr(k_cache),
                                              _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(k_scale),
                                              _ptr(v_scale), softmax_scale, partition_size, max_context_len, dims,
                                              act_dtype, cache_dtype, flags, _stream(stream)))


def lgm_check_block_tables(block_tables, context_lens, dims, max_context_len, status, stream=None):
    _check(lib().lgm_check_block_tables(_ptr(block_tables), _ptr(context_lens), dims, max_context_len, _ptr(status),
                                        _stream(stream)))


def lgm_lse_merge(out, out_lse, partial_out, partial_lse, num_partitions, num_seqs, num_q_heads, head_dim,
                  max_partitions, out_dtype, stream=None):
    _check(lib().lgm_lse_merge(_ptr(out), _ptr(out_lse), _ptr(partial_out), _ptr(partial_lse),
                               _ptr(num_partitions), num_seqs, num_q_heads, head_dim, max_partitions, out_dtype,
                               _stream(stream)))


def make_mla_dims(num_seqs, num_heads, latent_dim, rope_dim, block_size, num_blocks, max_blocks_per_seq):
    return lgm_mla_dims(num_seqs, num_heads, latent_dim, rope_dim, block_size, num_blocks, max_blocks_per_seq)


def lgm_paged_mla_partition_size(dims, max_context_len, partition_size) -> int:
    r = lib().lgm_paged_mla_partition_size(dims, max_context_len, partition_size)
    if r < 0:
        raise LgmError(LGM_ERR_INVALID_ARGUMENT, lib().lgm_last_error().decode())
    return r


def lgm_paged_mla_workspace_size(dims, max_context_len, partition_size) -> int:
    r = lib().lgm_paged_mla_workspace_size(dims, max_context_len, partition_size)
    err = lib().lgm_last_error().decode()
    if r == 0 and err:
        raise LgmError(LGM_ERR_INVALID_ARGUMENT, err)
    return r


def lgm_paged_mla_decode(out, out_lse, q_latent, q_pe, ckv_cache, kpe_cache, block_tables, context_lens, ckv_scale,
                         softmax_scale, partition_size, max_context_len, workspace, workspace_bytes, dims, ckv_dtype,
                         stream=None):
    _check(lib().lgm_paged_mla_decode(_ptr(out), _ptr(out_lse), _ptr(q_latent), _ptr(q_pe), _ptr(ckv_cache),
                                      _ptr(kpe_cache), _ptr(block_tables), _ptr(context_lens), _ptr(ckv_scale),
                                      softmax_scale, partition_size, max_context_len, _ptr(workspace),
                                      workspace_bytes, dims, ckv_dtype, _stream(stream)))


def lgm_last_error() -> str:
    return lib().lgm_last_error().decode()


def lgm_abi_version() -> int:
    return lib().lgm_abi_version()


def lgm_stream_read_probe(src, nbytes, num_workgroups, nontemporal, sink, stream=None):
    _check(lib().lgm_stream_read_probe(_ptr(src), nbytes, num_workgroups, nontemporal, _ptr(sink), _stream(stream)))
