"""MI355X (gfx950) tiled FlashAttention forward: thin Python binding of ``libfa.so``.

The binding only marshals arguments: every step of the computation runs in the HIP kernels
of ``csrc/fa_fwd.hip``.  PyTorch supplies device buffers and the current stream.  There is
no fallback: if the library is missing, importing the functions below raises.

Names follow include/fa.h:
  ``fa_fwd`` / ``fa_fwd_tiled`` / ``fa_fwd_splitkv`` / ``fa_fwd_ext`` /
  ``fa_splitkv_default_keys`` / ``fa_splitkv_workspace_bytes`` / ``fa_status_str``: the C entry
  points over raw pointers.
  ``forward(q, k, v, ...)``, ``forward_splitkv(q, k, v, ...)``, ``forward_paged(q, k_pool,
  v_pool, block_table, ...)``, ``forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, ...)``: the
  same calls over torch tensors (strides taken from them).
"""
import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_OK, FA_EINVAL, FA_ESHAPE, FA_EUNSUPPORTED, FA_EDEVICE, FA_ESCRATCH = range(6)
FA_NOALLOC_SCRATCH_BYTES = 32 << 20
FA_F32, FA_BF16 = 0, 1


class FaError(RuntimeError):
    """A non-OK fa_status; ``.status`` holds the code."""

    def __init__(self, status, msg):
        super().__init__(f"{msg} (fa_status {status})")
        self.status = status


class fa_strides(ctypes.Structure):
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3), ("v", ctypes.c_int64 * 3),
                ("o", ctypes.c_int64 * 3), ("lse", ctypes.c_int64 * 2), ("mask", ctypes.c_int64 * 4)]


class fa_tiling(ctypes.Structure):
    _fields_ = [("rows_per_block", ctypes.c_int32), ("heads_per_block", ctypes.c_int32)]


class fa_ext(ctypes.Structure):
    _fields_ = [("size", ctypes.c_uint32), ("rows_per_block", ctypes.c_int32), ("heads_per_block", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("split_keys", ctypes.c_int64), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("block_table", ctypes.c_void_p),
                ("block_table_stride", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("num_blocks", ctypes.c_int64), ("seqlens_k", ctypes.c_void_p), ("cu_seqlens_q", ctypes.c_void_p),
                ("cu_seqlens_k", ctypes.c_void_p), ("softcap", ctypes.c_float), ("reserved2", ctypes.c_int32),
                ("alibi_slopes", ctypes.c_void_p)]

    def __init__(self, **kw):
        super().__init__(size=ctypes.sizeof(fa_ext), **kw)


_lib = None
_FWD_ARGS = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int64] * 6 + [
    ctypes.c_float, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(fa_strides), ctypes.c_int, ctypes.c_void_p]
EXPORTED = ("fa_fwd", "fa_fwd_ext", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_fwd_tiled",
            "fa_splitkv_default_keys", "fa_splitkv_workspace_bytes", "fa_status_str")


def load_library(path=None):
    """Loads libfa.so (built by ``build.build()``); raises ImportError if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m flashattention_forward_flash_amd.build` "
                          "(there is no fallback path)")
    # torch carries its own HIP runtime.  Imported first, it is the one the library binds to
    # (the dynamic linker reuses the loaded libamdhip64), so torch's streams and allocations are
    # valid in the library's calls.  Loaded the other way round, the process would hold two HIP
    # runtimes and every launch on a torch stream would fail.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = _FWD_ARGS
    lib.fa_fwd_tiled.restype = ctypes.c_int
    lib.fa_fwd_tiled.argtypes = _FWD_ARGS + [ctypes.POINTER(fa_tiling)]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = _FWD_ARGS + [ctypes.POINTER(fa_tiling), ctypes.c_int64, ctypes.c_void_p,
                                               ctypes.c_size_t]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = _FWD_ARGS + [ctypes.POINTER(fa_tiling), ctypes.c_int64]
    lib.fa_fwd_ext.restype = ctypes.c_int
    lib.fa_fwd_ext.argtypes = _FWD_ARGS + [ctypes.POINTER(fa_ext)]
    lib.fa_splitkv_default_keys.restype = ctypes.c_int64
    lib.fa_splitkv_default_keys.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    lib.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_splitkv_workspace_bytes.argtypes = [ctypes.c_int64] * 6
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def fa_status_str(status):
    return load_library().fa_status_str(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks, mask,
           strides, dtype, stream):
    """The C entry point over raw device pointers (ints or None); returns the fa_status."""
    return load_library().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, int(causal),
                                  window, sinks, mask, strides, dtype, stream)


def fa_fwd_tiled(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks, mask,
                 strides, dtype, stream, tiling):
    return load_library().fa_fwd_tiled(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset,
                                        int(causal), window, sinks, mask, strides, dtype, stream, tiling)


def fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks, mask,
                   strides, dtype, stream, tiling, split_keys, workspace, workspace_bytes):
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset,
                                          int(causal), window, sinks, mask, strides, dtype, stream, tiling,
                                          split_keys, workspace, workspace_bytes)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks,
                           mask, strides, dtype, stream, tiling, split_keys):
    """fa_fwd_splitkv with the library's static scratch as the workspace (no allocation)."""
    return load_library().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset,
                                                  int(causal), window, sinks, mask, strides, dtype, stream, tiling,
                                                  split_keys)


def fa_fwd_ext(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, causal, window, sinks, mask, strides,
               dtype, stream, ext):
    return load_library().fa_fwd_ext(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, scale, q_offset, int(causal),
                                      window, sinks, mask, strides, dtype, stream, ext)


def fa_splitkv_default_keys(B, Hq, Hkv, Tq, Tk, q_offset=0, causal=True, window=0, dtype=FA_BF16):
    return load_library().fa_splitkv_default_keys(B, Hq, Hkv, Tq, Tk, q_offset, int(causal), window, dtype)


def fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split_keys):
    return load_library().fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split_keys)


def _check(status):
    if status != FA_OK:
        raise FaError(status, fa_status_str(status))


def _on_device(name, t, q):
    """Raises FaError unless `t` (a tensor or None) lives on q's GPU: the library receives raw
    device pointers, and a host pointer handed to a kernel would fault the GPU."""
    if t is not None and (not t.is_cuda or t.device != q.device):
        raise FaError(FA_EINVAL, f"{name} must be a GPU tensor on {q.device} (got {t.device})")


def _check_out(out, q, shape):
    """`out` must have q's dtype and the output shape, or the kernels would write out of bounds."""
    if out.dtype != q.dtype or tuple(out.shape) != tuple(shape):
        raise FaError(FA_EINVAL, f"out must be {q.dtype} {tuple(shape)} (got {out.dtype} {tuple(out.shape)})")


def forward(q, k, v, *, scale=None, q_offset=0, causal=True, window=0, sinks=None, mask=None,
            out=None, lse=None, return_lse=True, tiling=None, stream=None, softcap=0.0, alibi_slopes=None):
    """O = softmax(scale * Q K^T + mask) V over torch tensors on the GPU.

    q: [B, Hq, Tq, d]; k, v: [B, Hkv, Tk, d]; float32 or bfloat16, any strides with the d axis
    contiguous (e.g. a [B, T, H, d] tensor viewed with ``.transpose(1, 2)``).  ``mask``: float32
    tensor broadcastable to [B, Hq, Tq, Tk] (broadcast axes get stride 0).  ``sinks``: float32
    [Hq].  ``scale`` defaults to 1/sqrt(d) rounded to fp32.  Returns (o, lse) with lse float32
    [B, Hq, Tq] (None when ``return_lse`` is False and no ``lse`` buffer is given).
    ``tiling``: (rows_per_block, heads_per_block) or None for automatic; results do not depend
    on it.  ``softcap``: c > 0 caps the logit as c tanh(logit / c); ``alibi_slopes``: float32
    [Hq] slopes adding -slope |p_i - j| to the score.
    """
    return _forward(q, k, v, scale, q_offset, causal, window, sinks, mask, out, lse, return_lse, tiling,
                    stream, None, None, ext=_variants(None, softcap, alibi_slopes, tiling, q))


def forward_splitkv(q, k, v, *, split_keys=0, workspace=None, scale=None, q_offset=0, causal=True, window=0,
                    sinks=None, mask=None, out=None, lse=None, return_lse=True, tiling=None, stream=None,
                    softcap=0.0, alibi_slopes=None):
    """``forward`` with the keys cut into splits of ``split_keys`` keys (a multiple of 64; 0 picks
    ``fa_splitkv_default_keys``), the splits run in parallel and merged per row (split-KV /
    Flash-Decoding).  ``workspace``: a GPU tensor of at least ``fa_splitkv_workspace_bytes``
    bytes, 16-byte aligned; allocated here when None.  Results depend on ``split_keys`` (not on
    chunking or tiling); with one split they equal ``forward``'s.
    """
    import torch
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if split_keys == 0:
        dtype = FA_BF16 if q.dtype == torch.bfloat16 else FA_F32
        split_keys = fa_splitkv_default_keys(B, Hq, Hkv, Tq, Tk, int(q_offset), bool(causal), int(window), dtype)
    if workspace is None:
        nbytes = fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, int(split_keys)) if split_keys > 0 else 0
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if workspace.numel():
        _on_device("workspace", workspace, q)
    ext = _variants(None, softcap, alibi_slopes, tiling, q)
    if ext is not None:
        ext.split_keys = int(split_keys)
        ext.workspace = workspace.data_ptr()
        ext.workspace_bytes = workspace.numel() * workspace.element_size()
    return _forward(q, k, v, scale, q_offset, causal, window, sinks, mask, out, lse, return_lse, tiling,
                    stream, int(split_keys), workspace, ext=ext)


def forward_paged(q, k_pool, v_pool, block_table, *, Tk=None, seqlens_k=None, split_keys=0, workspace=None,
                  scale=None, q_offset=0, causal=True, window=0, sinks=None, mask=None, out=None, lse=None,
                  return_lse=True, tiling=None, stream=None, softcap=0.0, alibi_slopes=None):
    """``forward`` over paged K/V: ``k_pool``, ``v_pool`` are [num_blocks, Hkv, block_size, d] (any
    strides, d contiguous; e.g. a [num_blocks, block_size, Hkv, d] pool viewed with
    ``.transpose(1, 2)``), ``block_table`` int32 [B, max_blocks] on the GPU.  ``Tk``: keys per
    sequence (default max_blocks * block_size).  ``seqlens_k``: int32 [B] per-sequence key counts
    on the GPU; the query rows are then each sequence's last Tq positions (q_offset must be 0).
    ``split_keys``: 0 no split, > 0 keys per split, -1 the default split (``workspace`` allocated
    here when None).  Results equal ``forward`` on the same keys laid out contiguously.
    """
    import torch
    B, Hq, Tq, d = q.shape
    nb, Hkv, bs, dk = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape) or dk != d:
        raise FaError(FA_EINVAL, f"pool shapes k {tuple(k_pool.shape)} v {tuple(v_pool.shape)} d {d}")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B or (
            block_table.numel() and block_table.stride(1) != 1):
        raise FaError(FA_EINVAL, "block_table must be int32 [B, max_blocks] with a contiguous last axis")
    if Tk is None:
        Tk = block_table.shape[1] * bs
    if seqlens_k is not None and (seqlens_k.dtype != torch.int32 or tuple(seqlens_k.shape) != (B,)
                                  or not seqlens_k.is_contiguous()):
        raise FaError(FA_EINVAL, "seqlens_k must be a contiguous int32 [B] tensor")
    if q.numel() and not q.is_cuda:
        raise FaError(FA_EINVAL, "q must be a GPU tensor")
    for name, t in (("block_table", block_table), ("seqlens_k", seqlens_k)):
        if t is not None and t.numel():
            _on_device(name, t, q)
    ext = fa_ext(block_table=block_table.data_ptr() if block_table.numel() else None,
                 block_table_stride=block_table.stride(0) if block_table.shape[0] > 1 else block_table.shape[1],
                 block_size=bs, num_blocks=nb,
                 seqlens_k=seqlens_k.data_ptr() if seqlens_k is not None else None)
    keepalive = None
    if split_keys != 0:
        if split_keys < 0:
            dtype = FA_BF16 if q.dtype == torch.bfloat16 else FA_F32
            qo = max(0, Tk - Tq) if seqlens_k is not None else int(q_offset)
            split_keys = fa_splitkv_default_keys(B, Hq, Hkv, Tq, Tk, qo, bool(causal), int(window), dtype)
        if workspace is None:
            nbytes = fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, int(split_keys)) if split_keys > 0 else 0
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        if not workspace.is_cuda:
            raise FaError(FA_EINVAL, "workspace must be a GPU tensor")
        keepalive = workspace
        ext.split_keys = int(split_keys)
        ext.workspace = workspace.data_ptr()
        ext.workspace_bytes = workspace.numel() * workspace.element_size()
    _variants(ext, softcap, alibi_slopes, tiling, q)
    res = _forward(q, k_pool, v_pool, scale, q_offset, causal, window, sinks, mask, out, lse, return_lse, None,
                   stream, None, None, ext=ext, Tk=Tk)
    del keepalive
    return res


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, scale=None, causal=True,
                   window=0, sinks=None, out=None, lse=None, return_lse=True, split_keys=0, workspace=None,
                   tiling=None, stream=None, block_table=None, seqlens_k=None, softcap=0.0, alibi_slopes=None):
    """Packed sequences: q [total_q, Hq, d], k, v [total_k, Hkv, d] (token and head strides free, d
    contiguous), ``cu_seqlens_q``, ``cu_seqlens_k`` int32 [B + 1] prefix sums on the GPU,
    ``max_seqlen_q`` / ``max_seqlen_k`` at least the longest sequence.  Row i of sequence b sits
    at position n_b - m_b + i (its keys n_b, its rows m_b).  Returns (o [total_q, Hq, d],
    lse [Hq, total_q]); every row equals the single-sequence ``forward`` on its own tokens.
    ``split_keys``: 0 no split, > 0 keys per split, -1 the default (workspace allocated here
    when None).  Paged keys: ``block_table`` int32 [B, max_blocks] with k, v pools
    [num_blocks, Hkv, block_size, d] (as ``forward_paged``), ``cu_seqlens_k`` None and the key
    counts from ``seqlens_k`` (int32 [B]; None: max_seqlen_k each).
    """
    import torch
    if q.dtype == torch.float32:
        dtype = FA_F32
    elif q.dtype == torch.bfloat16:
        dtype = FA_BF16
    else:
        raise FaError(FA_EUNSUPPORTED, f"dtype {q.dtype} (float32 or bfloat16 only)")
    paged = block_table is not None
    kdim = 4 if paged else 3
    if q.dim() != 3 or k.dim() != kdim or k.shape != v.shape or k.shape[-1] != q.shape[2]:
        raise FaError(FA_EINVAL, f"packed shapes q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise FaError(FA_EINVAL, "q, k and v must share a dtype")
    if paged == (cu_seqlens_k is not None):
        raise FaError(FA_EINVAL, "give cu_seqlens_k (packed keys) or block_table (paged keys), not both")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k), ("seqlens_k", seqlens_k),
                    ("block_table", block_table)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda):
            raise FaError(FA_EINVAL, f"{name} must be a contiguous int32 GPU tensor")
    B = cu_seqlens_q.shape[0] - 1
    if B < 0 or (cu_seqlens_k is not None and tuple(cu_seqlens_k.shape) != (B + 1,)) or (
            seqlens_k is not None and tuple(seqlens_k.shape) != (B,)) or (
            paged and (block_table.dim() != 2 or block_table.shape[0] != B)):
        raise FaError(FA_EINVAL, "cu_seqlens_q [B + 1] with cu_seqlens_k [B + 1] or block_table [B, n] (seqlens_k [B])")
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.numel() and t.stride(-1) != 1:
            raise FaError(FA_EINVAL, f"{name}: the d axis must be contiguous")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.numel() and not t.is_cuda:
            raise FaError(FA_EINVAL, f"{name} must be a GPU tensor")
    for name, t in (("k", k), ("v", v), ("sinks", sinks), ("out", out), ("lse", lse), ("workspace", workspace)):
        if t is not None and (t.numel() or name in ("sinks", "workspace")):
            _on_device(name, t, q)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty((total_q, Hq, d), dtype=q.dtype, device=q.device)
    _check_out(out, q, (total_q, Hq, d))
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q)
                            or (lse.numel() and lse.stride(1) != 1)):
        raise FaError(FA_EINVAL, "lse must be float32 [Hq, total_q] with a contiguous last axis")
    st = fa_strides()
    st.q[:] = [0, q.stride(1), q.stride(0)]
    if paged:  # pools [block, head, key in block, d]
        st.k[:] = [k.stride(0), k.stride(1), k.stride(2)]
        st.v[:] = [v.stride(0), v.stride(1), v.stride(2)]
    else:
        st.k[:] = [0, k.stride(1), k.stride(0)]
        st.v[:] = [0, v.stride(1), v.stride(0)]
    st.o[:] = [0, out.stride(1), out.stride(0)]
    st.lse[:] = [0, lse.stride(0) if lse is not None else 0]
    st.mask[:] = [0, 0, 0, 0]
    if sinks is not None and (sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,) or not sinks.is_contiguous()):
        raise FaError(FA_EINVAL, "sinks must be a contiguous float32 [Hq] tensor")
    if paged:
        ext = fa_ext(cu_seqlens_q=cu_seqlens_q.data_ptr(), block_table=block_table.data_ptr(),
                     block_table_stride=block_table.shape[1], block_size=k.shape[2], num_blocks=k.shape[0],
                     seqlens_k=seqlens_k.data_ptr() if seqlens_k is not None else None)
    else:
        ext = fa_ext(cu_seqlens_q=cu_seqlens_q.data_ptr(), cu_seqlens_k=cu_seqlens_k.data_ptr())
    _variants(ext, softcap, alibi_slopes, tiling, q)
    Tq, Tk = int(max_seqlen_q), int(max_seqlen_k)
    if split_keys != 0:
        if split_keys < 0:
            split_keys = fa_splitkv_default_keys(B, Hq, Hkv, Tq, Tk, max(0, Tk - Tq), bool(causal), int(window), dtype)
        if workspace is None:
            nbytes = fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, int(split_keys)) if split_keys > 0 else 0
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        _on_device("workspace", workspace, q)
        ext.split_keys = int(split_keys)
        ext.workspace = workspace.data_ptr()
        ext.workspace_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream

    def ptr(t):
        return t.data_ptr() if (t is not None and t.numel()) else None

    status = fa_fwd_ext(ptr(q), ptr(k), ptr(v), ptr(out), ptr(lse), B, Hq, Hkv, Tq, Tk, d, float(scale), 0,
                        bool(causal), int(window), ptr(sinks), None, ctypes.byref(st), dtype, stream,
                        ctypes.byref(ext))
    _check(status)
    return out, lse


def _variants(ext, softcap, alibi_slopes, tiling, q):
    """Puts the score variants and the tiling into `ext` (made when needed); returns it, or None
    when there is neither an ext nor a variant."""
    import torch
    if ext is None and not softcap and alibi_slopes is None:
        return None
    if ext is None:
        ext = fa_ext()
    if tiling is not None:
        ext.rows_per_block, ext.heads_per_block = int(tiling[0]), int(tiling[1])
    ext.softcap = float(softcap)
    if alibi_slopes is not None:
        if (alibi_slopes.dtype != torch.float32 or alibi_slopes.dim() != 1 or not alibi_slopes.is_contiguous()
                or not alibi_slopes.is_cuda or alibi_slopes.shape[0] != q.shape[-3 if q.dim() == 4 else 1]):
            raise FaError(FA_EINVAL, "alibi_slopes must be a contiguous float32 [Hq] GPU tensor")
        ext.alibi_slopes = alibi_slopes.data_ptr()
    return ext


def _forward(q, k, v, scale, q_offset, causal, window, sinks, mask, out, lse, return_lse, tiling, stream,
             split_keys, workspace, ext=None, Tk=None):
    """Marshals the arguments of one call (strides from the tensors) and calls the library."""
    import torch
    if q.dtype == torch.float32:
        dtype = FA_F32
    elif q.dtype == torch.bfloat16:
        dtype = FA_BF16
    else:
        raise FaError(FA_EUNSUPPORTED, f"dtype {q.dtype} (float32 or bfloat16 only)")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise FaError(FA_EINVAL, "q, k and v must share a dtype")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise FaError(FA_EINVAL, "q, k, v must be 4-d [B, H, T, d]")
    B, Hq, Tq, d = q.shape
    if ext is None or not ext.block_table:
        Bk, Hkv, Tk_, dk = k.shape
        Tk = Tk_ if Tk is None else Tk
        if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
            raise FaError(FA_EINVAL, f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    else:
        Hkv = k.shape[1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.numel() and t.stride(3) != 1:
            raise FaError(FA_EINVAL, f"{name}: the d axis must be contiguous")
        if t.numel() and not t.is_cuda:
            raise FaError(FA_EINVAL, f"{name} must be a GPU tensor")
    for name, t in (("k", k), ("v", v), ("sinks", sinks), ("mask", mask), ("out", out), ("lse", lse),
                    ("workspace", workspace)):
        if t is not None and (t.numel() or name in ("sinks", "mask", "workspace")):
            _on_device(name, t, q)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty((B, Hq, Tq, d), dtype=q.dtype, device=q.device)
    _check_out(out, q, (B, Hq, Tq, d))
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    st = fa_strides()
    st.q[:] = [q.stride(0), q.stride(1), q.stride(2)]
    st.k[:] = [k.stride(0), k.stride(1), k.stride(2)]
    st.v[:] = [v.stride(0), v.stride(1), v.stride(2)]
    st.o[:] = [out.stride(0), out.stride(1), out.stride(2)]
    if out.numel() and out.stride(3) != 1:
        raise FaError(FA_EINVAL, "out: the d axis must be contiguous")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Tq) or (lse.numel() and lse.stride(2) != 1):
            raise FaError(FA_EINVAL, "lse must be float32 [B, Hq, Tq] with a contiguous last axis")
        st.lse[:] = [lse.stride(0), lse.stride(1)]
    mask_ptr = None
    if mask is not None:
        if mask.dtype != torch.float32:
            raise FaError(FA_EINVAL, "mask must be float32")
        mview = mask.expand(B, Hq, Tq, Tk)
        st.mask[:] = [mview.stride(i) if mview.shape[i] > 1 else 0 for i in range(4)]
        mask_ptr = mview.data_ptr() if mview.numel() else None
    else:
        st.mask[:] = [0, 0, 0, 0]
    if sinks is not None:
        if sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,) or not sinks.is_contiguous():
            raise FaError(FA_EINVAL, "sinks must be a contiguous float32 [Hq] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else None

    def ptr(t):
        return t.data_ptr() if (t is not None and t.numel()) else None

    til = None
    if tiling is not None:
        til = fa_tiling(int(tiling[0]), int(tiling[1]))
    args = (ptr(q), ptr(k), ptr(v), ptr(out), ptr(lse), B, Hq, Hkv, Tq, Tk, d, float(scale), int(q_offset),
            bool(causal), int(window), ptr(sinks), mask_ptr, ctypes.byref(st), dtype, stream,
            ctypes.byref(til) if til is not None else None)
    if ext is not None:
        status = fa_fwd_ext(*args[:-1], ctypes.byref(ext))
    elif split_keys is None:
        status = fa_fwd_tiled(*args)
    else:
        if not workspace.is_cuda:
            raise FaError(FA_EINVAL, "workspace must be a GPU tensor")
        nbytes = workspace.numel() * workspace.element_size()
        status = fa_fwd_splitkv(*args, split_keys, workspace.data_ptr(), nbytes)
    _check(status)
    return out, lse
