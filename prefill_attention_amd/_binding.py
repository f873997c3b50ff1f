"""ctypes binding of libpfa.so: argument marshalling only.

Every step of the attention runs in the HIP library; this module checks tensor metadata, reads
device pointers and the current stream from torch, and forwards them to the C ABI. There is no
fallback path: if the library is missing or the call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpfa.so")

# Mirrors of include/pfa.h
NO_CAUSAL = -1
FLAG_NO_SKIP = 1
MAX_LEN = 1 << 30
STATUS = {
    0: "PFA_OK", 1: "PFA_ERR_NULL", 2: "PFA_ERR_SIZE", 3: "PFA_ERR_GQA", 4: "PFA_ERR_HEAD_DIM",
    5: "PFA_ERR_MASK_ARGS", 6: "PFA_ERR_ALIGN", 7: "PFA_ERR_ALIAS", 8: "PFA_ERR_LAUNCH",
    9: "PFA_ERR_FLAGS", 10: "PFA_ERR_SCALE", 11: "PFA_ERR_WORKSPACE", 12: "PFA_ERR_RING",
}
DECODE_MAX_L = 64
DECODE_SCRATCH_BYTES = 64 << 20
EXPORTS = ("prefill_attn_gqa", "prefill_attn_gqa_ex", "prefill_attn_gqa_opt", "prefill_attn_gqa_varlen",
           "prefill_attn_gqa_varlen_opt", "prefill_attn_gqa_ring_opt",
           "prefill_attn_gqa_ring", "prefill_attn_gqa_decode", "prefill_attn_gqa_decode_opt",
           "prefill_attn_gqa_decode_noalloc", "prefill_attn_gqa_ws", "pfa_prefill_workspace_bytes",
           "pfa_decode_workspace_bytes", "pfa_status_str", "pfa_version")


class Options(ctypes.Structure):
    """Mirror of struct pfa_options."""
    _fields_ = [("flags", ctypes.c_uint), ("softcap", ctypes.c_float), ("bias", ctypes.c_void_p),
                ("bias_stride_b", ctypes.c_int64), ("bias_stride_h", ctypes.c_int64), ("bias_stride_l", ctypes.c_int64),
                ("sinks", ctypes.c_void_p), ("block_sel", ctypes.c_void_p), ("block_q", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("sel_stride_b", ctypes.c_int64), ("sel_stride_h", ctypes.c_int64),
                ("sel_stride_q", ctypes.c_int64)]

_lib = None


class PfaError(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load libpfa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m prefill_attention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, ci, cf, cu = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint
        sig = [vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp, vp, vp]
        lib.prefill_attn_gqa.argtypes = sig
        lib.prefill_attn_gqa.restype = ci
        lib.prefill_attn_gqa_ex.argtypes = sig + [cu]
        lib.prefill_attn_gqa_ex.restype = ci
        lib.prefill_attn_gqa_opt.argtypes = sig + [ctypes.POINTER(Options)]
        lib.prefill_attn_gqa_opt.restype = ci
        lib.prefill_attn_gqa_varlen.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, ci, ci,
                                                vp, vp]
        lib.prefill_attn_gqa_varlen.restype = ci
        lib.prefill_attn_gqa_varlen_opt.argtypes = lib.prefill_attn_gqa_varlen.argtypes + [ctypes.POINTER(Options)]
        lib.prefill_attn_gqa_varlen_opt.restype = ci
        lib.prefill_attn_gqa_decode.argtypes = sig[:-1] + [vp, ctypes.c_int64, vp]
        lib.prefill_attn_gqa_decode.restype = ci
        lib.prefill_attn_gqa_decode_opt.argtypes = sig[:-1] + [vp, ctypes.c_int64, vp, ctypes.POINTER(Options)]
        lib.prefill_attn_gqa_decode_opt.restype = ci
        lib.prefill_attn_gqa_decode_noalloc.argtypes = sig + [ctypes.POINTER(Options)]
        lib.prefill_attn_gqa_decode_noalloc.restype = ci
        lib.prefill_attn_gqa_ws.argtypes = sig[:-1] + [vp, ctypes.c_int64, vp, ctypes.POINTER(Options)]
        lib.prefill_attn_gqa_ws.restype = ci
        lib.pfa_prefill_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
        lib.pfa_prefill_workspace_bytes.restype = ctypes.c_int64
        lib.pfa_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
        lib.pfa_decode_workspace_bytes.restype = ctypes.c_int64
        lib.prefill_attn_gqa_ring.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, ci, vp, vp]
        lib.prefill_attn_gqa_ring.restype = ci
        lib.prefill_attn_gqa_ring_opt.argtypes = lib.prefill_attn_gqa_ring.argtypes + [ctypes.POINTER(Options)]
        lib.prefill_attn_gqa_ring_opt.restype = ci
        lib.pfa_status_str.argtypes = [ci]
        lib.pfa_status_str.restype = ctypes.c_char_p
        lib.pfa_version.argtypes = []
        lib.pfa_version.restype = ci
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return library().pfa_status_str(int(status)).decode()


def version() -> int:
    return int(library().pfa_version())


def prefill_attn_gqa_raw(q_ptr: int, k_ptr: int, v_ptr: int, B: int, Hq: int, Hkv: int, L: int,
                         S: int, D: int, scale: float, causal_offset: int, window: int,
                         key_mask_ptr: int | None, o_ptr: int, stream: int | None,
                         flags: int = 0, softcap: float = 0.0, bias_ptr: int | None = None,
                         bias_strides=(0, 0, 0), sinks_ptr: int | None = None, sel_ptr: int | None = None,
                         sel_blocks=(0, 0), sel_strides=(0, 0, 0)) -> int:
    """Direct C-ABI call with integer pointers; returns the status code."""
    if softcap == 0.0 and not bias_ptr and not sinks_ptr and not sel_ptr:
        return int(library().prefill_attn_gqa_ex(
            q_ptr, k_ptr, v_ptr, B, Hq, Hkv, L, S, D, ctypes.c_float(scale), causal_offset, window,
            key_mask_ptr or None, o_ptr, stream or None, flags))
    opts = Options(flags, softcap, bias_ptr or None, *bias_strides, sinks_ptr or None, sel_ptr or None,
                   *sel_blocks, *sel_strides)
    return int(library().prefill_attn_gqa_opt(
        q_ptr, k_ptr, v_ptr, B, Hq, Hkv, L, S, D, ctypes.c_float(scale), causal_offset, window,
        key_mask_ptr or None, o_ptr, stream or None, ctypes.byref(opts)))


def prefill_workspace_bytes(B: int, Hq: int, Hkv: int, L: int, S: int, D: int) -> int:
    """Bytes of workspace prefill_attn_gqa_ws needs for this shape (-1 if invalid)."""
    return int(library().pfa_prefill_workspace_bytes(B, Hq, Hkv, L, S, D))


def prefill_attn_gqa_ws_raw(q_ptr: int, k_ptr: int, v_ptr: int, B: int, Hq: int, Hkv: int, L: int,
                            S: int, D: int, scale: float, causal_offset: int, window: int,
                            key_mask_ptr: int | None, o_ptr: int, ws_ptr: int | None, ws_bytes: int,
                            stream: int | None, flags: int = 0, softcap: float = 0.0,
                            sinks_ptr: int | None = None, bias_ptr: int | None = None, bias_strides=(0, 0, 0),
                            sel_ptr: int | None = None, sel_blocks=(0, 0), sel_strides=(0, 0, 0)) -> int:
    """Direct C-ABI call of the key-split prefill entry point; returns the status code."""
    opts = Options(flags, softcap, bias_ptr or None, *bias_strides, sinks_ptr or None, sel_ptr or None,
                   *sel_blocks, *sel_strides)
    return int(library().prefill_attn_gqa_ws(
        q_ptr, k_ptr, v_ptr, B, Hq, Hkv, L, S, D, ctypes.c_float(scale), causal_offset, window,
        key_mask_ptr or None, o_ptr, ws_ptr or None, ws_bytes, stream or None, ctypes.byref(opts)))


def _sinks_ptr(sinks, Hq, device):
    """Device pointer of a float32 [Hq] sink-logit tensor (None passes through)."""
    if sinks is None:
        return None
    import torch

    if (not isinstance(sinks, torch.Tensor) or sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,)
            or sinks.device != device or not sinks.is_contiguous()):
        raise ValueError(f"sinks must be a contiguous float32 [Hq]=({Hq},) tensor on {device}")
    return sinks.data_ptr()


def prefill_attn_gqa(q, k, v, *, scale: float | None = None, causal: bool = True,
                     causal_offset: int | None = None, window: int = 0, key_mask=None, out=None,
                     no_skip: bool = False, softcap: float = 0.0, bias=None, sinks=None,
                     block_sel=None, block_q: int = 0, block_k: int = 0, stream=None, workspace=None):
    """Grouped-query prefill attention on torch tensors.

    q: bf16 [B,Hq,L,D]; k, v: bf16 [B,Hkv,S,D]; key_mask: optional uint8/bool [B,S] (nonzero =
    valid). scale defaults to 1/sqrt(D). With causal=True the causal offset defaults to S - L
    (the chunk is the tail of the S keys); causal=False is bidirectional. window > 0 adds a
    sliding window of that many keys. softcap > 0 applies logit soft-capping. bias: optional
    float32 additive bias broadcastable to [B,Hq,L,S] (last dimension contiguous), added to the
    scaled scores before the masks. sinks: optional float32 [Hq] attention-sink logits (one extra
    softmax term per head, with no value). block_sel: optional uint8/bool block bitmap broadcastable
    to [B, Hq, ceil(L/block_q), ceil(S/block_k)] (last dimension contiguous); key j is visible to
    row i only where block_sel[b, h, i // block_q, j // block_k] is nonzero. workspace: optional
    zero-filled contiguous uint8 tensor on q's device of at least prefill_workspace_bytes(...)
    bytes; with it a call with at most 192 query blocks of 256 rows splits its keys over the whole
    chip (prefill_attn_gqa_ws), others run as without it. Every call leaves it ready for the next
    (of any shape it is large enough for); calls sharing it must be ordered on one stream. Returns
    `out` (allocated if None), bf16 [B,Hq,L,D].
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    B, Hq, L, D = q.shape
    Bk, Hkv, S, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k and v shapes differ: {tuple(k.shape)} vs {tuple(v.shape)}")
    if Bk != B or Dk != D:
        raise ValueError(f"batch / head dim mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if causal:
        if causal_offset is None:
            causal_offset = S - L
        if causal_offset < 0:
            raise ValueError(f"causal attention needs causal_offset >= 0 (got {causal_offset})")
    else:
        if causal_offset is not None and causal_offset >= 0:
            raise ValueError("causal=False takes no causal_offset")
        if window > 0:
            raise ValueError("a sliding window needs causal=True")
        causal_offset = NO_CAUSAL
    mask_ptr = None
    if key_mask is not None:
        if key_mask.dtype == torch.bool:
            key_mask = key_mask.view(torch.uint8)
        if key_mask.dtype != torch.uint8:
            raise ValueError("key_mask must be uint8 or bool")
        if tuple(key_mask.shape) != (B, S) or key_mask.device != q.device or not key_mask.is_contiguous():
            raise ValueError(f"key_mask must be a contiguous [B,S]=({B},{S}) tensor on {q.device}")
        mask_ptr = key_mask.data_ptr()
    bias_ptr, bias_strides = None, (0, 0, 0)
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32 or bias.device != q.device:
            raise ValueError(f"bias must be a float32 tensor on {q.device}")
        while bias.dim() < 4:
            bias = bias.unsqueeze(0)
        try:
            bias = bias.expand(B, Hq, L, S)
        except RuntimeError as e:
            raise ValueError(f"bias {tuple(bias.shape)} does not broadcast to [B,Hq,L,S]=({B},{Hq},{L},{S})") from e
        if bias.stride(3) != 1:
            raise ValueError("bias must be contiguous along the key dimension")
        bias_ptr, bias_strides = bias.data_ptr(), (bias.stride(0), bias.stride(1), bias.stride(2))
    sinks_ptr = _sinks_ptr(sinks, Hq, q.device)
    sel_ptr, sel_strides = None, (0, 0, 0)
    if block_sel is not None:
        if not isinstance(block_sel, torch.Tensor) or block_sel.device != q.device:
            raise ValueError(f"block_sel must be a tensor on {q.device}")
        if block_sel.dtype == torch.bool:
            block_sel = block_sel.view(torch.uint8)
        if block_sel.dtype != torch.uint8:
            raise ValueError("block_sel must be uint8 or bool")
        if block_q <= 0 or block_k <= 0:
            raise ValueError("block_sel needs block_q > 0 and block_k > 0")
        nqb, nkb = -(-L // block_q), -(-S // block_k)
        while block_sel.dim() < 4:
            block_sel = block_sel.unsqueeze(0)
        try:
            block_sel = block_sel.expand(B, Hq, nqb, nkb)
        except RuntimeError as e:
            raise ValueError(f"block_sel {tuple(block_sel.shape)} does not broadcast to "
                             f"[B,Hq,nqb,nkb]=({B},{Hq},{nqb},{nkb})") from e
        if nkb > 1 and block_sel.stride(3) != 1:
            raise ValueError("block_sel must be contiguous along the key-block dimension")
        sel_ptr, sel_strides = block_sel.data_ptr(), (block_sel.stride(0), block_sel.stride(1), block_sel.stride(2))
    if out is None:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 tensor shaped like q on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    stream_ptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if workspace is not None:
        # the key-split entry point (prefill_attn_gqa_ws): a zero-filled uint8 GPU tensor of at least
        # prefill_workspace_bytes(...) bytes, reused by calls ordered on one stream
        if (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or workspace.device != q.device
                or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous uint8 tensor on {q.device}")
        with torch.cuda.device(q.device):
            rc = prefill_attn_gqa_ws_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq, Hkv, L, S, D,
                                         float(scale), int(causal_offset), int(window), mask_ptr, out.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(), stream_ptr,
                                         FLAG_NO_SKIP if no_skip else 0, float(softcap), sinks_ptr,
                                         bias_ptr, bias_strides, sel_ptr, (int(block_q), int(block_k)), sel_strides)
        if rc != 0:
            raise PfaError(rc, status_str(rc))
        return out
    with torch.cuda.device(q.device):
        rc = prefill_attn_gqa_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq, Hkv, L, S, D,
                                  float(scale), int(causal_offset), int(window), mask_ptr,
                                  out.data_ptr(), stream_ptr, FLAG_NO_SKIP if no_skip else 0, float(softcap),
                                  bias_ptr, bias_strides, sinks_ptr, sel_ptr, (int(block_q), int(block_k)),
                                  sel_strides)
    if rc != 0:
        raise PfaError(rc, status_str(rc))
    return out


def prefill_attn_gqa_varlen_raw(q_ptr: int, k_ptr: int, v_ptr: int, cu_q_ptr: int, cu_k_ptr: int,
                                n_seq: int, max_seqlen_q: int, total_q: int, total_k: int, Hq: int,
                                Hkv: int, D: int, scale: float, causal: bool, window: int,
                                o_ptr: int, stream: int | None, flags: int = 0, softcap: float = 0.0,
                                sinks_ptr: int | None = None) -> int:
    """Direct C-ABI call of the packed variable-length entry point; returns the status code."""
    if flags == 0 and softcap == 0.0 and not sinks_ptr:
        return int(library().prefill_attn_gqa_varlen(
            q_ptr, k_ptr, v_ptr, cu_q_ptr, cu_k_ptr, n_seq, max_seqlen_q, total_q, total_k, Hq, Hkv, D,
            ctypes.c_float(scale), 1 if causal else 0, window, o_ptr, stream or None))
    opts = Options(flags, softcap, None, 0, 0, 0, sinks_ptr or None)
    return int(library().prefill_attn_gqa_varlen_opt(
        q_ptr, k_ptr, v_ptr, cu_q_ptr, cu_k_ptr, n_seq, max_seqlen_q, total_q, total_k, Hq, Hkv, D,
        ctypes.c_float(scale), 1 if causal else 0, window, o_ptr, stream or None, ctypes.byref(opts)))


def prefill_attn_gqa_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, *,
                            scale: float | None = None, causal: bool = True, window: int = 0,
                            out=None, no_skip: bool = False, softcap: float = 0.0, sinks=None, stream=None):
    """Packed variable-length grouped-query attention on torch tensors.

    q: bf16 [total_q, Hq, D]; k, v: bf16 [total_k, Hkv, D]; cu_seqlens_q / cu_seqlens_k: int32
    [n_seq + 1] prefix sums on the same device. max_seqlen_q bounds every sequence's query
    length. With causal=True local row i of a sequence sees local keys j <= i + (Lk - Lq).
    no_skip, softcap and sinks as in prefill_attn_gqa. Returns `out` (allocated if None), bf16
    [total_q, Hq, D].
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 GPU tensor")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1
                or not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor on {q.device}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Dk != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    n_seq = cu_seqlens_q.numel() - 1
    if n_seq < 1 or cu_seqlens_k.numel() != n_seq + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have n_seq + 1 >= 2 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if window > 0 and not causal:
        raise ValueError("a sliding window needs causal=True")
    if out is None:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 tensor shaped like q on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    stream_ptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        rc = prefill_attn_gqa_varlen_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                         cu_seqlens_k.data_ptr(), n_seq, int(max_seqlen_q), total_q, total_k,
                                         Hq, Hkv, D, float(scale), bool(causal), int(window), out.data_ptr(),
                                         stream_ptr, FLAG_NO_SKIP if no_skip else 0, float(softcap),
                                         _sinks_ptr(sinks, Hq, q.device))
    if rc != 0:
        raise PfaError(rc, status_str(rc))
    return out


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, L: int, S: int, D: int) -> int:
    """Bytes of workspace the decode entry point needs for this shape (-1 if invalid)."""
    return int(library().pfa_decode_workspace_bytes(B, Hq, Hkv, L, S, D))


def prefill_attn_gqa_decode_raw(q_ptr: int, k_ptr: int, v_ptr: int, B: int, Hq: int, Hkv: int, L: int,
                                S: int, D: int, scale: float, causal_offset: int, window: int,
                                key_mask_ptr: int | None, o_ptr: int, ws_ptr: int | None, ws_bytes: int,
                                stream: int | None, softcap: float = 0.0, flags: int = 0,
                                sinks_ptr: int | None = None) -> int:
    """Direct C-ABI call of the short-query (decode) entry point; returns the status code."""
    if softcap == 0.0 and flags == 0 and not sinks_ptr:
        return int(library().prefill_attn_gqa_decode(
            q_ptr, k_ptr, v_ptr, B, Hq, Hkv, L, S, D, ctypes.c_float(scale), causal_offset, window,
            key_mask_ptr or None, o_ptr, ws_ptr or None, ws_bytes, stream or None))
    opts = Options(flags, softcap, None, 0, 0, 0, sinks_ptr or None)
    return int(library().prefill_attn_gqa_decode_opt(
        q_ptr, k_ptr, v_ptr, B, Hq, Hkv, L, S, D, ctypes.c_float(scale), causal_offset, window,
        key_mask_ptr or None, o_ptr, ws_ptr or None, ws_bytes, stream or None, ctypes.byref(opts)))


def prefill_attn_gqa_decode_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, B: int, Hq: int, Hkv: int, L: int,
                                        S: int, D: int, scale: float, causal_offset: int, window: int,
                                        key_mask_ptr: int | None, o_ptr: int, stream: int | None,
                                        softcap: float = 0.0, flags: int = 0, sinks_ptr: int | None = None) -> int:
    """Direct C-ABI call of the allocation-free decode entry point; returns the status code."""
    opts = Options(flags, softcap, None, 0, 0, 0, sinks_ptr or None)
    return int(library().prefill_attn_gqa_decode_noalloc(
        q_ptr, k_ptr, v_ptr, B, Hq, Hkv, L, S, D, ctypes.c_float(scale), causal_offset, window,
        key_mask_ptr or None, o_ptr, stream or None, ctypes.byref(opts)))


def prefill_attn_gqa_decode_noalloc(q, k, v, *, scale: float | None = None, causal: bool = True,
                                    causal_offset: int | None = None, window: int = 0, key_mask=None, out=None,
                                    softcap: float = 0.0, sinks=None, stream=None):
    """prefill_attn_gqa_decode with the partials in the library's own device scratch array instead
    of a workspace (nothing is allocated by the call; `out` must then be given by callers that cannot
    allocate). Calls that overlap in time on one GPU race on that array."""
    return prefill_attn_gqa_decode(q, k, v, scale=scale, causal=causal, causal_offset=causal_offset,
                                   window=window, key_mask=key_mask, out=out, softcap=softcap, sinks=sinks,
                                   stream=stream, _noalloc=True)


def prefill_attn_gqa_decode(q, k, v, *, scale: float | None = None, causal: bool = True,
                            causal_offset: int | None = None, window: int = 0, key_mask=None, out=None,
                            workspace=None, softcap: float = 0.0, sinks=None, stream=None, _noalloc=False):
    """Short-query (decode, L <= 64) grouped-query attention on torch tensors: the same arguments
    and result as prefill_attn_gqa, computed with the key range split over the chip and a
    deterministic merge. `workspace` is an optional uint8 GPU tensor of at least
    decode_workspace_bytes(...) bytes (allocated here if None; the library itself never allocates).
    sinks: optional float32 [Hq] attention-sink logits, as in prefill_attn_gqa."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 GPU tensor")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    B, Hq, L, D = q.shape
    Bk, Hkv, S, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if causal:
        if causal_offset is None:
            causal_offset = S - L
        if causal_offset < 0:
            raise ValueError(f"causal attention needs causal_offset >= 0 (got {causal_offset})")
    else:
        if window > 0:
            raise ValueError("a sliding window needs causal=True")
        causal_offset = NO_CAUSAL
    mask_ptr = None
    if key_mask is not None:
        if key_mask.dtype == torch.bool:
            key_mask = key_mask.view(torch.uint8)
        if key_mask.dtype != torch.uint8 or tuple(key_mask.shape) != (B, S) or key_mask.device != q.device \
                or not key_mask.is_contiguous():
            raise ValueError(f"key_mask must be a contiguous uint8 [B,S]=({B},{S}) tensor on {q.device}")
        mask_ptr = key_mask.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 tensor shaped like q on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    stream_ptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if _noalloc:
        with torch.cuda.device(q.device):
            rc = prefill_attn_gqa_decode_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq, Hkv, L, S, D,
                                                     float(scale), int(causal_offset), int(window), mask_ptr,
                                                     out.data_ptr(), stream_ptr, float(softcap), 0,
                                                     _sinks_ptr(sinks, Hq, q.device))
        if rc != 0:
            raise PfaError(rc, status_str(rc))
        return out
    need = decode_workspace_bytes(B, Hq, Hkv, L, S, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        rc = prefill_attn_gqa_decode_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq, Hkv, L, S, D,
                                         float(scale), int(causal_offset), int(window), mask_ptr,
                                         out.data_ptr(), workspace.data_ptr(), workspace.numel(), stream_ptr,
                                         float(softcap), 0, _sinks_ptr(sinks, Hq, q.device))
    if rc != 0:
        raise PfaError(rc, status_str(rc))
    return out


def prefill_attn_gqa_ring_raw(q_ptr: int, kn_ptr: int, vn_ptr: int, kr_ptr: int, vr_ptr: int, B: int, Hq: int,
                              Hkv: int, L: int, pos0: int, ring: int, D: int, scale: float, window: int,
                              o_ptr: int, stream: int | None, flags: int = 0, softcap: float = 0.0,
                              sinks_ptr: int | None = None) -> int:
    """Direct C-ABI call of the rotating-cache entry point; returns the status code."""
    if flags == 0 and softcap == 0.0 and not sinks_ptr:
        return int(library().prefill_attn_gqa_ring(q_ptr, kn_ptr, vn_ptr, kr_ptr, vr_ptr, B, Hq, Hkv, L, pos0, ring,
                                                   D, ctypes.c_float(scale), window, o_ptr, stream or None))
    opts = Options(flags, softcap, None, 0, 0, 0, sinks_ptr or None)
    return int(library().prefill_attn_gqa_ring_opt(q_ptr, kn_ptr, vn_ptr, kr_ptr, vr_ptr, B, Hq, Hkv, L, pos0, ring,
                                                   D, ctypes.c_float(scale), window, o_ptr, stream or None,
                                                   ctypes.byref(opts)))


def prefill_attn_gqa_ring(q, k_new, v_new, k_ring, v_ring, pos0: int, *, scale: float | None = None,
                          window: int = 0, out=None, no_skip: bool = False, softcap: float = 0.0, sinks=None,
                          stream=None):
    """Causal (optionally windowed) prefill of a chunk at positions pos0.. against a rotating cache,
    appending the chunk's keys first. q: bf16 [B,Hq,L,D]; k_new, v_new: bf16 [B,Hkv,L,D]; k_ring,
    v_ring: bf16 [B,Hkv,ring,D] (position j in slot j % ring; updated in place). no_skip, softcap and
    sinks as in prefill_attn_gqa. Returns `out`."""
    import torch

    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_ring", k_ring), ("v_ring", v_ring)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 4 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous 4-D bfloat16 tensor on {q.device}")
    B, Hq, L, D = q.shape
    Bn, Hkv, Ln, Dn = k_new.shape
    if tuple(v_new.shape) != tuple(k_new.shape) or (Bn, Ln, Dn) != (B, L, D):
        raise ValueError(f"k_new / v_new must be [B,Hkv,L,D]: q {tuple(q.shape)}, k_new {tuple(k_new.shape)}")
    ring = k_ring.shape[2]
    if tuple(k_ring.shape) != (B, Hkv, ring, D) or tuple(v_ring.shape) != tuple(k_ring.shape):
        raise ValueError(f"k_ring / v_ring must be [B,Hkv,ring,D]: {tuple(k_ring.shape)}, {tuple(v_ring.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bf16 tensor shaped like q on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    stream_ptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        rc = prefill_attn_gqa_ring_raw(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_ring.data_ptr(),
                                       v_ring.data_ptr(), B, Hq, Hkv, L, int(pos0), ring, D, float(scale),
                                       int(window), out.data_ptr(), stream_ptr, FLAG_NO_SKIP if no_skip else 0,
                                       float(softcap), _sinks_ptr(sinks, Hq, q.device))
    if rc != 0:
        raise PfaError(rc, status_str(rc))
    return out
