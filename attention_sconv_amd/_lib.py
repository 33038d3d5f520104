"""ctypes binding of libinkattn (declarations in include/inkattn.h).

Argument marshalling only: torch tensors are turned into device pointers,
the current HIP stream is passed along, and a non-OK status raises
:class:`InkattnError`.  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  Importing this module without the built
library raises ImportError.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libinkattn.so")

OK, EINVAL, ENOTSUP, EHIP, ESCRATCH = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 8 << 20       # INKATTN_NOALLOC_SCRATCH_BYTES
FP32, BF16 = 0, 1

EXPORTED = (
    "inkattn_sconv",
    "inkattn_sconv_paged",
    "inkattn_sconv_out",
    "inkattn_sconv_fp8",
    "inkattn_relattn_decode_fp8",
    "inkattn_relattn_prefill",
    "inkattn_relattn_prefill_fp8",
    "inkattn_relattn_prefill_fp8_workspace_size",
    "inkattn_relattn_prefill_fp8_mma",
    "inkattn_relattn_decode_num_splits",
    "inkattn_relattn_decode_workspace_size",
    "inkattn_relattn_decode",
    "inkattn_relattn_decode_noalloc",
    "inkattn_relattn_decode_mq_num_splits",
    "inkattn_relattn_decode_mq_workspace_size",
    "inkattn_relattn_decode_mq",
    "inkattn_status_string",
    "inkattn_probe_mfma_bf16",
    "inkattn_probe_stream_read",
)

PROBE_MFMA_WAVES, PROBE_MFMA_CHAINS, PROBE_READ_GROUPS = 8, 8, 256


class InkattnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class AttnDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("window", ctypes.c_int32),
                ("bias_len", ctypes.c_int32)]


def make_desc(dtype, num_q_heads, num_kv_heads, window, bias_len, head_dim=128,
              block_size=128):
    return AttnDesc(dtype, num_q_heads, num_kv_heads, head_dim, block_size, window, bias_len)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python attention_sconv_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(AttnDesc)
    lib.inkattn_sconv.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                  vp, vp, vp]
    lib.inkattn_sconv.restype = i32
    lib.inkattn_sconv_paged.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                        i32, vp, vp, vp, vp, vp, vp]
    lib.inkattn_sconv_paged.restype = i32
    lib.inkattn_sconv_out.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.inkattn_sconv_out.restype = i32
    f32 = ctypes.c_float
    lib.inkattn_sconv_fp8.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                      f32, f32, vp, vp, vp]
    lib.inkattn_sconv_fp8.restype = i32
    lib.inkattn_relattn_decode_fp8.argtypes = [dp, i32, i32, i32, i32, vp, vp, vp, f32, f32, vp,
                                               i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.inkattn_relattn_decode_fp8.restype = i32
    lib.inkattn_relattn_prefill.argtypes = [dp, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp,
                                            vp, vp, vp, vp]
    lib.inkattn_relattn_prefill.restype = i32
    lib.inkattn_relattn_prefill_fp8.argtypes = [dp, i32, i32, i32, vp, vp, vp, f32, f32, vp,
                                                i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.inkattn_relattn_prefill_fp8.restype = i32
    lib.inkattn_relattn_prefill_fp8_mma.argtypes = [dp, i32, i32, i32, vp, vp, vp, f32, f32,
                                                    vp, i32, vp, vp, vp, vp, vp, vp]
    lib.inkattn_relattn_prefill_fp8_mma.restype = i32
    lib.inkattn_relattn_prefill_fp8_workspace_size.argtypes = [dp, i32, i32]
    lib.inkattn_relattn_prefill_fp8_workspace_size.restype = sz
    lib.inkattn_relattn_decode_num_splits.argtypes = [dp, i32, i32]
    lib.inkattn_relattn_decode_num_splits.restype = i32
    lib.inkattn_relattn_decode_workspace_size.argtypes = [dp, i32, i32, i32]
    lib.inkattn_relattn_decode_workspace_size.restype = sz
    lib.inkattn_relattn_decode.argtypes = [dp, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                           i32, vp, sz, vp]
    lib.inkattn_relattn_decode.restype = i32
    lib.inkattn_relattn_decode_noalloc.argtypes = [dp, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp,
                                                   vp, i32, vp]
    lib.inkattn_relattn_decode_noalloc.restype = i32
    lib.inkattn_relattn_decode_mq_num_splits.argtypes = [dp, i32, i32, i32]
    lib.inkattn_relattn_decode_mq_num_splits.restype = i32
    lib.inkattn_relattn_decode_mq_workspace_size.argtypes = [dp, i32, i32, i32, i32, i32]
    lib.inkattn_relattn_decode_mq_workspace_size.restype = sz
    lib.inkattn_relattn_decode_mq.argtypes = [dp, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp,
                                              vp, vp, vp, vp, i32, vp, sz, vp]
    lib.inkattn_relattn_decode_mq.restype = i32
    lib.inkattn_status_string.argtypes = [i32]
    lib.inkattn_status_string.restype = ctypes.c_char_p
    lib.inkattn_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
    lib.inkattn_probe_mfma_bf16.restype = i32
    lib.inkattn_probe_stream_read.argtypes = [vp, sz, vp, vp]
    lib.inkattn_probe_stream_read.restype = i32
    return lib


_lib = _load()


def status_string(status):
    return _lib.inkattn_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libinkattn takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libinkattn takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != OK:
        raise InkattnError(status, where)


def inkattn_sconv(dtype, num_kv_heads, head_dim, num_seqs, num_tokens, max_chunk_len, k_in,
                  v_in, conv_w, conv_state, state_slot, cu_seqlens, slot_mapping, k_cache,
                  v_cache, stream=None):
    st = _lib.inkattn_sconv(dtype, num_kv_heads, head_dim, num_seqs, num_tokens,
                            max_chunk_len, _ptr(k_in), _ptr(v_in), _ptr(conv_w),
                            _ptr(conv_state), _ptr(state_slot), _ptr(cu_seqlens),
                            _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), _stream(stream))
    _check(st, "inkattn_sconv")


def inkattn_relattn_prefill(desc, num_seqs, num_tokens, max_q_len, q, k_cache, v_cache,
                            block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens, bias,
                            out, lse=None, stream=None):
    st = _lib.inkattn_relattn_prefill(ctypes.byref(desc), num_seqs, num_tokens, max_q_len,
                                      _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                      max_blocks_per_seq, _ptr(cu_seqlens_q), _ptr(seq_lens),
                                      _ptr(bias), _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "inkattn_relattn_prefill")


def inkattn_relattn_prefill_fp8_workspace_size(desc, num_seqs, max_blocks_per_seq):
    return int(_lib.inkattn_relattn_prefill_fp8_workspace_size(ctypes.byref(desc), num_seqs,
                                                               max_blocks_per_seq))


def inkattn_relattn_prefill_fp8(desc, num_seqs, num_tokens, max_q_len, q, k_cache, v_cache,
                                k_scale, v_scale, block_table, max_blocks_per_seq,
                                cu_seqlens_q, seq_lens, bias, out, lse=None, workspace=None,
                                workspace_bytes=0, stream=None):
    st = _lib.inkattn_relattn_prefill_fp8(ctypes.byref(desc), num_seqs, num_tokens, max_q_len,
                                          _ptr(q), _ptr(k_cache), _ptr(v_cache), k_scale,
                                          v_scale, _ptr(block_table), max_blocks_per_seq,
                                          _ptr(cu_seqlens_q), _ptr(seq_lens), _ptr(bias),
                                          _ptr(out), _ptr(lse), _ptr(workspace),
                                          workspace_bytes, _stream(stream))
    _check(st, "inkattn_relattn_prefill_fp8")


def inkattn_relattn_prefill_fp8_mma(desc, num_seqs, num_tokens, max_q_len, q, k_cache, v_cache,
                                    k_scale, v_scale, block_table, max_blocks_per_seq,
                                    cu_seqlens_q, seq_lens, bias, out, lse=None, stream=None):
    st = _lib.inkattn_relattn_prefill_fp8_mma(ctypes.byref(desc), num_seqs, num_tokens,
                                              max_q_len, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                              k_scale, v_scale, _ptr(block_table),
                                              max_blocks_per_seq, _ptr(cu_seqlens_q),
                                              _ptr(seq_lens), _ptr(bias), _ptr(out), _ptr(lse),
                                              _stream(stream))
    _check(st, "inkattn_relattn_prefill_fp8_mma")


def inkattn_relattn_decode_num_splits(desc, num_seqs, max_seq_len):
    return int(_lib.inkattn_relattn_decode_num_splits(ctypes.byref(desc), num_seqs,
                                                      max_seq_len))


def inkattn_relattn_decode_workspace_size(desc, num_seqs, max_seq_len, num_splits=0):
    return int(_lib.inkattn_relattn_decode_workspace_size(ctypes.byref(desc), num_seqs,
                                                          max_seq_len, num_splits))


def inkattn_relattn_decode(desc, num_seqs, max_seq_len, q, k_cache, v_cache, block_table,
                           max_blocks_per_seq, seq_lens, bias, out, lse, num_splits,
                           workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.inkattn_relattn_decode(ctypes.byref(desc), num_seqs, max_seq_len, _ptr(q),
                                     _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                     max_blocks_per_seq, _ptr(seq_lens), _ptr(bias), _ptr(out),
                                     _ptr(lse), num_splits, _ptr(workspace), workspace_bytes,
                                     _stream(stream))
    _check(st, "inkattn_relattn_decode")


def inkattn_relattn_decode_noalloc(desc, num_seqs, max_seq_len, q, k_cache, v_cache,
                                   block_table, max_blocks_per_seq, seq_lens, bias, out, lse,
                                   num_splits, stream=None):
    st = _lib.inkattn_relattn_decode_noalloc(ctypes.byref(desc), num_seqs, max_seq_len, _ptr(q),
                                             _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                             max_blocks_per_seq, _ptr(seq_lens), _ptr(bias),
                                             _ptr(out), _ptr(lse), num_splits, _stream(stream))
    _check(st, "inkattn_relattn_decode_noalloc")


def inkattn_probe_mfma_bf16(num_groups, iters, out, stream=None):
    """Dense bf16 MFMA loop; ``out`` is a float32 device tensor of 3*num_groups."""
    st = _lib.inkattn_probe_mfma_bf16(num_groups, iters, _ptr(out), _stream(stream))
    _check(st, "inkattn_probe_mfma_bf16")


def inkattn_probe_stream_read(buf, out, stream=None):
    """Streaming read of the whole device tensor ``buf``; ``out`` is a float32
    device tensor of PROBE_READ_GROUPS elements."""
    st = _lib.inkattn_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                        _stream(stream))
    _check(st, "inkattn_probe_stream_read")


def inkattn_relattn_decode_mq_num_splits(desc, num_seqs, max_q_len, max_seq_len):
    return int(_lib.inkattn_relattn_decode_mq_num_splits(ctypes.byref(desc), num_seqs,
                                                         max_q_len, max_seq_len))


def inkattn_relattn_decode_mq_workspace_size(desc, num_seqs, num_tokens, max_q_len,
                                             max_seq_len, num_splits=0):
    return int(_lib.inkattn_relattn_decode_mq_workspace_size(
        ctypes.byref(desc), num_seqs, num_tokens, max_q_len, max_seq_len, num_splits))


def inkattn_relattn_decode_mq(desc, num_seqs, num_tokens, max_q_len, max_seq_len, q, k_cache,
                              v_cache, block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens,
                              bias, out, lse, num_splits, workspace, workspace_bytes=None,
                              stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib.inkattn_relattn_decode_mq(ctypes.byref(desc), num_seqs, num_tokens, max_q_len,
                                        max_seq_len, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(block_table), max_blocks_per_seq,
                                        _ptr(cu_seqlens_q), _ptr(seq_lens), _ptr(bias),
                                        _ptr(out), _ptr(lse), num_splits, _ptr(workspace),
                                        workspace_bytes, _stream(stream))
    _check(st, "inkattn_relattn_decode_mq")


def inkattn_sconv_paged(dtype, num_kv_heads, head_dim, num_seqs, num_tokens, max_chunk_len,
                        k_in, v_in, conv_w, cu_seqlens, seq_lens, state_block_table, k_state,
                        v_state, slot_mapping, k_cache, v_cache, stream=None):
    st = _lib.inkattn_sconv_paged(dtype, num_kv_heads, head_dim, num_seqs, num_tokens,
                                  max_chunk_len, _ptr(k_in), _ptr(v_in), _ptr(conv_w),
                                  _ptr(cu_seqlens), _ptr(seq_lens), _ptr(state_block_table),
                                  state_block_table.shape[1], _ptr(k_state), _ptr(v_state),
                                  _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                                  _stream(stream))
    _check(st, "inkattn_sconv_paged")


def inkattn_sconv_out(dtype, channels, num_seqs, num_tokens, max_chunk_len, x, conv_w,
                      conv_state, state_slot, cu_seqlens, y, stream=None):
    st = _lib.inkattn_sconv_out(dtype, channels, num_seqs, num_tokens, max_chunk_len, _ptr(x),
                                _ptr(conv_w), _ptr(conv_state), _ptr(state_slot),
                                _ptr(cu_seqlens), _ptr(y), _stream(stream))
    _check(st, "inkattn_sconv_out")


def inkattn_sconv_fp8(dtype, num_kv_heads, head_dim, num_seqs, num_tokens, max_chunk_len, k_in,
                      v_in, conv_w, conv_state, state_slot, cu_seqlens, slot_mapping, k_scale,
                      v_scale, k_cache, v_cache, stream=None):
    st = _lib.inkattn_sconv_fp8(dtype, num_kv_heads, head_dim, num_seqs, num_tokens,
                                max_chunk_len, _ptr(k_in), _ptr(v_in), _ptr(conv_w),
                                _ptr(conv_state), _ptr(state_slot), _ptr(cu_seqlens),
                                _ptr(slot_mapping), k_scale, v_scale, _ptr(k_cache),
                                _ptr(v_cache), _stream(stream))
    _check(st, "inkattn_sconv_fp8")


def inkattn_relattn_decode_fp8(desc, num_seqs, num_tokens, max_q_len, max_seq_len, q, k_cache,
                               v_cache, k_scale, v_scale, block_table, max_blocks_per_seq,
                               cu_seqlens_q, seq_lens, bias, out, lse=None, num_splits=0,
                               workspace=None, workspace_bytes=0, stream=None):
    st = _lib.inkattn_relattn_decode_fp8(ctypes.byref(desc), num_seqs, num_tokens, max_q_len,
                                         max_seq_len, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         k_scale, v_scale, _ptr(block_table),
                                         max_blocks_per_seq, _ptr(cu_seqlens_q),
                                         _ptr(seq_lens), _ptr(bias), _ptr(out), _ptr(lse),
                                         num_splits, _ptr(workspace), workspace_bytes,
                                         _stream(stream))
    _check(st, "inkattn_relattn_decode_fp8")
