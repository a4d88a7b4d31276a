"""ctypes binding over libfa.so (include/fa.h).

Argument marshalling only: every function here turns torch tensors into device pointers and
sizes, calls the C entry point of the same name on torch's current HIP stream and raises
``FaError`` on a non-zero status.  No attention arithmetic happens in Python, and there is no
fallback: if the library is missing or the call fails, the call raises.
"""

import ctypes
import math
import os

import torch

__all__ = [
    "FA_BF16",
    "FA_F32",
    "FaError",
    "fa_bwd",
    "fa_bwd_workspace_bytes",
    "fa_fwd_fp8",
    "fa_fwd",
    "fa_fwd_unfused",
    "fa_fwd_unfused_workspace_bytes",
    "fa_paged_decode",
    "fa_paged_decode_noalloc",
    "fa_paged_decode_workspace_bytes",
    "fa_paged_prefill",
    "fa_paged_prefill_workspace_bytes",
    "fa_status_str",
    "library_path",
    "load_library",
]

FA_BF16 = 0
FA_F32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {fa_status_str(status)} (status {status})")


def library_path():
    return os.path.join(_HERE, "libfa.so")


def load_library():
    """Load libfa.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with io_aware_attention_02_amd.build.build_library() "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.restype = i32
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, i32, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, f32, f32, f32, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                               vp, vp]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.fa_bwd.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp,
                           i32, vp, sz, vp]
    lib.fa_paged_decode_workspace_bytes.restype = sz
    lib.fa_paged_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_paged_decode.restype = i32
    lib.fa_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, vp, sz, vp]
    lib.fa_paged_decode_noalloc.restype = i32
    lib.fa_paged_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, i32, f32, vp]
    lib.fa_paged_prefill.restype = i32
    lib.fa_paged_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i32, f32, vp, sz, vp]
    lib.fa_paged_prefill_workspace_bytes.restype = sz
    lib.fa_paged_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_fwd_unfused_workspace_bytes.restype = sz
    lib.fa_fwd_unfused_workspace_bytes.argtypes = [i32, i32, i32]
    lib.fa_fwd_unfused.restype = i32
    lib.fa_fwd_unfused.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [i32]
    _LIB = lib
    return lib


def fa_status_str(status):
    return load_library().fa_status_str(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_device_tensor(name, t, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def fa_fwd(q, k, v, o=None, lse=None, scale=None, causal=False, seq_lens=None, stream=None):
    """Attention forward.  q [B,H,N,d], k/v [B,Hkv,N,d] (bf16 or fp32, same dtype).

    Returns (o, lse): o like q, lse [B,H,N] fp32.  ``scale`` defaults to 1/sqrt(d).
    ``seq_lens`` is None or a device int32 [B] tensor of valid lengths.
    """
    lib = load_library()
    if q.dtype == torch.bfloat16:
        dtype = FA_BF16
    elif q.dtype == torch.float32:
        dtype = FA_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t, q.dtype)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B,H,N,d] and k, v [B,Hkv,N,d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_device_tensor("o", o, q.dtype)
    _check_device_tensor("lse", lse, torch.float32)
    if seq_lens is not None:
        _check_device_tensor("seq_lens", seq_lens, torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale),
                    int(bool(causal)), _ptr(seq_lens), dtype, _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd")
    return o, lse


def fa_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o=None, lse=None, scale=None, causal=False,
               seq_lens=None, stream=None):
    """FP8 attention forward.  q [B,H,N,d], k/v [B,Hkv,N,d]: e4m3 codes (uint8 or
    torch.float8_e4m3fn tensors); the real tensors are ``q_scale * q`` etc.

    Returns (o, lse): o [B,H,N,d] bf16, lse [B,H,N] fp32.  ``scale`` defaults to 1/sqrt(d).
    """
    lib = load_library()
    codes = []
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        _check_device_tensor(name, t, torch.uint8)
        codes.append(t)
    q, k, v = codes
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B,H,N,d] and k, v [B,Hkv,N,d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_device_tensor("o", o, torch.bfloat16)
    _check_device_tensor("lse", lse, torch.float32)
    if seq_lens is not None:
        _check_device_tensor("seq_lens", seq_lens, torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), float(q_scale), float(k_scale), float(v_scale),
                        _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale), int(bool(causal)),
                        _ptr(seq_lens), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_fp8")
    return o, lse


def fa_bwd_workspace_bytes(B, H, N):
    return int(load_library().fa_bwd_workspace_bytes(int(B), int(H), int(N)))


def fa_bwd(q, k, v, o, lse, dout, dq=None, dk=None, dv=None, scale=None, causal=False,
           seq_lens=None, workspace=None, stream=None):
    """Attention backward.  q, o, dout [B,H,N,d] bf16; k, v [B,Hkv,N,d] bf16; lse [B,H,N] fp32
    as written by fa_fwd for the same inputs.  Returns (dq, dk, dv) shaped like q, k, v.

    ``workspace`` is an optional preallocated uint8 device tensor; if None one is allocated
    with torch (the library itself never allocates).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_device_tensor(name, t, torch.bfloat16)
    _check_device_tensor("lse", lse, torch.float32)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or o.shape != q.shape or \
            dout.shape != q.shape:
        raise ValueError("q, o, dout must be [B,H,N,d] and k, v [B,Hkv,N,d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_device_tensor(name, t, torch.bfloat16)
        if t.shape != like.shape:
            raise ValueError(f"{name} must have shape {tuple(like.shape)}")
    if seq_lens is not None:
        _check_device_tensor("seq_lens", seq_lens, torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_device_tensor("workspace", workspace)
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                    _ptr(dv), B, H, Hkv, N, d, float(scale), int(bool(causal)), _ptr(seq_lens),
                    FA_BF16, _ptr(workspace), workspace.numel() * workspace.element_size(),
                    _stream(stream))
    if st != 0:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fa_paged_decode_workspace_bytes(num_seqs, Hq, d, max_blocks_per_seq, block_size=16):
    return int(load_library().fa_paged_decode_workspace_bytes(
        int(num_seqs), int(Hq), int(d), int(max_blocks_per_seq), int(block_size)))


def fa_paged_decode(q, k_cache, v_cache, block_table, seq_lens, o=None, lse=None, scale=None,
                    workspace=None, stream=None):
    """Paged decode.  q [S,Hq,d] bf16; caches [P,block_size,Hkv,d] bf16; block_table [S,M]
    int32; seq_lens [S] int32.  Returns (o [S,Hq,d] bf16, lse [S,Hq] fp32).

    ``workspace`` is an optional preallocated uint8 device tensor; if None one is allocated
    with torch (the library itself never allocates).
    """
    lib = load_library()
    _check_device_tensor("q", q, torch.bfloat16)
    _check_device_tensor("k_cache", k_cache, torch.bfloat16)
    _check_device_tensor("v_cache", v_cache, torch.bfloat16)
    _check_device_tensor("block_table", block_table, torch.int32)
    _check_device_tensor("seq_lens", seq_lens, torch.int32)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape or block_table.dim() != 2:
        raise ValueError("q [S,Hq,d], caches [P,bs,Hkv,d], block_table [S,M]")
    S, Hq, d = q.shape
    P, bs, Hkv, _ = k_cache.shape
    M = block_table.shape[1]
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    _check_device_tensor("o", o, torch.bfloat16)
    _check_device_tensor("lse", lse, torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_paged_decode_workspace_bytes(S, Hq, d, M, bs)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_device_tensor("workspace", workspace)
    st = lib.fa_paged_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                             _ptr(seq_lens), _ptr(o), _ptr(lse), S, Hq, Hkv, d, bs, M, P,
                             float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream))
    if st != 0:
        raise FaError(st, "fa_paged_decode")
    return o, lse


def fa_paged_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse, scale=None,
                            stream=None):
    """fa_paged_decode without a workspace: the library keeps the partial results in its static
    device scratch (FA_DECODE_SCRATCH_BYTES per GPU).  ``o`` [S,Hq,d] bf16 and ``lse`` [S,Hq]
    fp32 (or None) are the caller's preallocated outputs; nothing is allocated here or in the
    library.  Calls that overlap on one GPU race."""
    lib = load_library()
    _check_device_tensor("q", q, torch.bfloat16)
    _check_device_tensor("k_cache", k_cache, torch.bfloat16)
    _check_device_tensor("v_cache", v_cache, torch.bfloat16)
    _check_device_tensor("block_table", block_table, torch.int32)
    _check_device_tensor("seq_lens", seq_lens, torch.int32)
    _check_device_tensor("o", o, torch.bfloat16)
    if lse is not None:
        _check_device_tensor("lse", lse, torch.float32)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape or block_table.dim() != 2:
        raise ValueError("q [S,Hq,d], caches [P,bs,Hkv,d], block_table [S,M]")
    S, Hq, d = q.shape
    P, bs, Hkv, _ = k_cache.shape
    M = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.fa_paged_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                     _ptr(seq_lens), _ptr(o), _ptr(lse), S, Hq, Hkv, d, bs, M, P,
                                     float(scale), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_paged_decode_noalloc")
    return o, lse


def fa_paged_prefill_workspace_bytes(S, Qmax, Hq, Hkv, d, M):
    return int(load_library().fa_paged_prefill_workspace_bytes(int(S), int(Qmax), int(Hq), int(Hkv),
                                                               int(d), int(M)))


def fa_paged_prefill(q, k_cache, v_cache, block_table, seq_lens, q_lens, o=None, lse=None,
                     scale=None, workspace=None, stream=None):
    """Chunked prefill against a paged cache.  q [S,Hq,Qmax,d] bf16 (each sequence's newest
    q_lens[b] tokens, head-major); caches [P,bs,Hkv,d] bf16; block_table [S,M], seq_lens [S],
    q_lens [S] int32.  Returns (o [S,Hq,Qmax,d] bf16, lse [S,Hq,Qmax] fp32).  ``workspace``:
    optional uint8 device tensor of fa_paged_prefill_workspace_bytes(S, Qmax, Hq, Hkv, d, M)
    bytes (allocated with torch if None)."""
    lib = load_library()
    _check_device_tensor("q", q, torch.bfloat16)
    _check_device_tensor("k_cache", k_cache, torch.bfloat16)
    _check_device_tensor("v_cache", v_cache, torch.bfloat16)
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens), ("q_lens", q_lens)):
        _check_device_tensor(name, t, torch.int32)
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape or block_table.dim() != 2:
        raise ValueError("q [S,Hq,Qmax,d], caches [P,bs,Hkv,d], block_table [S,M]")
    S, Hq, Qmax, d = q.shape
    P, bs, Hkv, _ = k_cache.shape
    M = block_table.shape[1]
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((S, Hq, Qmax), dtype=torch.float32, device=q.device)
    _check_device_tensor("o", o, torch.bfloat16)
    _check_device_tensor("lse", lse, torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        need = fa_paged_prefill_workspace_bytes(S, Qmax, Hq, Hkv, d, M) if Hkv > 0 else 0
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_device_tensor("workspace", workspace)
    st = lib.fa_paged_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                              _ptr(seq_lens), _ptr(q_lens), _ptr(o), _ptr(lse), S, Qmax, Hq, Hkv,
                              d, bs, M, P, float(scale), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_paged_prefill")
    return o, lse


def fa_fwd_unfused_workspace_bytes(B, H, N):
    return int(load_library().fa_fwd_unfused_workspace_bytes(int(B), int(H), int(N)))


def fa_fwd_unfused(q, k, v, o=None, lse=None, scale=None, causal=False, workspace=None,
                   stream=None):
    """The standard three-kernel forward (baseline).  q [B,H,N,d], k/v [B,Hkv,N,d] bf16 with N a
    multiple of 8.  Returns (o, lse) like fa_fwd.  ``workspace``: optional uint8 device tensor of
    fa_fwd_unfused_workspace_bytes(B, H, N) bytes (allocated with torch if None)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t, torch.bfloat16)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B,H,N,d] and k, v [B,Hkv,N,d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = torch.empty_like(q) if o is None else o
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_device_tensor("o", o, torch.bfloat16)
    _check_device_tensor("lse", lse, torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_fwd_unfused_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_device_tensor("workspace", workspace)
    st = lib.fa_fwd_unfused(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                            float(scale), int(bool(causal)), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise FaError(st, "fa_fwd_unfused")
    return o, lse
