"""Python binding of the gfx950 BA-Att library.

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI (include/ba_att.h).  torch supplies device memory
and the current stream; tensors must already live on the GPU.
"""

from __future__ import annotations

import math

import torch

from . import _lib

BA_BF16, BA_F32 = 0, 1

__all__ = [
    "load", "num_blocks", "keep_count", "select_workspace_bytes", "select", "select_noalloc", "mask_to_index",
    "forward", "forward_split", "forward_split_workspace_bytes", "forward_split_parts", "forward_auto",
    "merge", "forward_ext", "dense",
    "ba_attention", "block_map", "score_full_workspace_bytes", "score_full", "rank_agreement",
]


def load():
    return _lib.load()


def _check(status: int) -> None:
    if status != 0:
        msg = _lib.load().ba_att_status_string(status).decode()
        raise RuntimeError(f"BA-Att call failed: {msg} (status {status})")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype | None, ndim: int | None = None,
          device: torch.device | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _on(t: torch.Tensor):
    """The library launches on the current device: make it the arguments' device."""
    return torch.cuda.device(t.device)


def _workspace(ws: torch.Tensor | None, need: int, device: torch.device) -> tuple[torch.Tensor, int]:
    """A caller's workspace (any dtype, contiguous, on the arguments' device) or a new one;
    returns it with its size in bytes."""
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    else:
        _need(ws, "workspace", None, device=device)
    return ws, ws.numel() * ws.element_size()


def num_blocks(N: int, block: int) -> int:
    return int(_lib.load().ba_att_num_blocks(N, block))


def keep_count(n_blocks: int, sparsity: float) -> int:
    return int(_lib.load().ba_att_keep_count(n_blocks, float(sparsity)))


def select_workspace_bytes(B: int, H: int, N: int, D: int, block: int) -> int:
    return int(_lib.load().ba_att_select_workspace_bytes(B, H, N, D, block))


def _qkv_shape(q: torch.Tensor):
    _need(q, "q", torch.bfloat16, 4)
    return tuple(int(x) for x in q.shape)


def select(q: torch.Tensor, k: torch.Tensor, block: int, sparsity: float, scale: float | None = None,
           return_score: bool = False, workspace: torch.Tensor | None = None):
    """Selection pass: returns (mask uint8 [B,H,n,n], idx int32 [B,H,n,keep],
    cnt int32 [B,H,n]) and, with return_score, the fp32 score map."""
    B, H, N, D = _qkv_shape(q)
    _need(k, "k", torch.bfloat16, 4, q.device)
    if tuple(k.shape) != (B, H, N, D):
        raise ValueError("q and k must have the same shape")
    lib = _lib.load()
    n = num_blocks(N, block)
    keep = keep_count(n, sparsity)
    if keep < 1:
        raise ValueError("sparsity must lie in [0, 1)")
    dev = q.device
    mask = torch.empty((B, H, n, n), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, H, n, keep), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    score = torch.empty((B, H, n, n), dtype=torch.float32, device=dev) if return_score else None
    workspace, ws_bytes = _workspace(workspace, select_workspace_bytes(B, H, N, D, block), dev)
    with _on(q):
        _check(lib.ba_att_select(B, H, N, D, block, float(scale or 0.0), float(sparsity),
                                 q.data_ptr(), k.data_ptr(), mask.data_ptr(), idx.data_ptr(),
                                 cnt.data_ptr(), score.data_ptr() if score is not None else None,
                                 workspace.data_ptr(), ws_bytes, _stream(q)))
    if return_score:
        return mask, idx, cnt, score
    return mask, idx, cnt


def select_noalloc(q: torch.Tensor, k: torch.Tensor, block: int, sparsity: float, scale: float | None = None,
                   return_score: bool = False, out=None):
    """ba_att_select_noalloc: the selection pass with the library's fixed
    device scratch instead of a workspace.  `out` = (mask, idx, cnt) lets a
    caller that cannot allocate pass its own outputs (shapes as returned by
    select); otherwise they are allocated here."""
    B, H, N, D = _qkv_shape(q)
    _need(k, "k", torch.bfloat16, 4, q.device)
    if tuple(k.shape) != (B, H, N, D):
        raise ValueError("q and k must have the same shape")
    lib = _lib.load()
    n = num_blocks(N, block)
    keep = keep_count(n, sparsity)
    if keep < 1:
        raise ValueError("sparsity must lie in [0, 1)")
    dev = q.device
    if out is None:
        mask = torch.empty((B, H, n, n), dtype=torch.uint8, device=dev)
        idx = torch.empty((B, H, n, keep), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    else:
        mask, idx, cnt = out
        for t, name, dt, shape in ((mask, "mask", torch.uint8, (B, H, n, n)), (idx, "idx", torch.int32, (B, H, n, keep)),
                                   (cnt, "cnt", torch.int32, (B, H, n))):
            _need(t, name, dt, None, dev)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}")
    score = torch.empty((B, H, n, n), dtype=torch.float32, device=dev) if return_score else None
    with _on(q):
        _check(lib.ba_att_select_noalloc(B, H, N, D, block, float(scale or 0.0), float(sparsity),
                                         q.data_ptr(), k.data_ptr(), mask.data_ptr(), idx.data_ptr(),
                                         cnt.data_ptr(), score.data_ptr() if score is not None else None,
                                         _stream(q)))
    if return_score:
        return mask, idx, cnt, score
    return mask, idx, cnt


def mask_to_index(mask: torch.Tensor, max_keep: int | None = None):
    """Block mask uint8 [B,H,n,n] -> (idx int32 [B,H,n,max_keep], cnt int32 [B,H,n])."""
    _need(mask, "mask", torch.uint8, 4)
    B, H, n, n2 = (int(x) for x in mask.shape)
    if n != n2:
        raise ValueError("mask must be square in its last two dimensions")
    max_keep = n if max_keep is None else int(max_keep)
    idx = torch.empty((B, H, n, max_keep), dtype=torch.int32, device=mask.device)
    cnt = torch.empty((B, H, n), dtype=torch.int32, device=mask.device)
    with _on(mask):
        _check(_lib.load().ba_att_mask_to_index(B, H, n, mask.data_ptr(), max_keep, idx.data_ptr(),
                                                cnt.data_ptr(), _stream(mask)))
    return idx, cnt


def _out(q, out_dtype, out, lse, return_lse):
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty((B, H, N, D), dtype=out_dtype, device=q.device)
    else:
        _need(out, "out", out_dtype, 4, q.device)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3, q.device)
        if tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be [B,H,N]")
    code = BA_F32 if out_dtype == torch.float32 else BA_BF16
    return out, lse, code


def forward(q, k, v, idx, cnt, block: int, scale: float | None = None,
            out_dtype: torch.dtype = torch.float32, out=None, lse=None, return_lse: bool = True):
    """Block-sparse attention over the listed key blocks; returns (O, LSE)."""
    B, H, N, D = _forward_args(q, k, v, idx, cnt, block)
    out, lse, code = _out(q, out_dtype, out, lse, return_lse)
    with _on(q):
        _check(_lib.load().ba_att_forward(B, H, N, D, block, float(scale or 0.0), q.data_ptr(),
                                          k.data_ptr(), v.data_ptr(), idx.data_ptr(), cnt.data_ptr(),
                                          int(idx.shape[3]), out.data_ptr(), code,
                                          lse.data_ptr() if lse is not None else None, _stream(q)))
    return out, lse


QUEUE_WORDS = 16  # BA_ATT_QUEUE_WORDS
_queues: dict = {}


def queue_for(device: torch.device, stream_handle: int) -> torch.Tensor:
    """The zeroed work queue kept for one (device, stream): the kernel leaves
    it zero at its end, so one queue serves every call on that stream."""
    key = (device.index, int(stream_handle))
    qt = _queues.get(key)
    if qt is None:
        qt = torch.zeros(QUEUE_WORDS, dtype=torch.int32, device=device)
        _queues[key] = qt
    return qt


def forward_queued(q, k, v, idx, cnt, block: int, scale: float | None = None,
                   out_dtype: torch.dtype = torch.float32, out=None, lse=None, return_lse: bool = True,
                   queue: torch.Tensor | None = None):
    """ba_att_forward_queued: the sparse forward with its tiles taken from a
    per-XCD work queue by a resident grid; same results as forward(), bit for
    bit.  queue: int32 [16] zeros (default: one kept per device and stream)."""
    B, H, N, D = _forward_args(q, k, v, idx, cnt, block)
    out, lse, code = _out(q, out_dtype, out, lse, return_lse)
    with _on(q):
        stream = _stream(q)
        if queue is None:
            queue = queue_for(q.device, stream or 0)
        else:
            _need(queue, "queue", torch.int32, 1, q.device)
            if queue.numel() < QUEUE_WORDS or queue.data_ptr() % 64:
                raise ValueError("queue must hold 16 int32 words, 64-byte aligned")
        _check(_lib.load().ba_att_forward_queued(B, H, N, D, block, float(scale or 0.0), q.data_ptr(),
                                                 k.data_ptr(), v.data_ptr(), idx.data_ptr(), cnt.data_ptr(),
                                                 int(idx.shape[3]), out.data_ptr(), code,
                                                 lse.data_ptr() if lse is not None else None,
                                                 queue.data_ptr(), stream))
    return out, lse


def _forward_args(q, k, v, idx, cnt, block):
    B, H, N, D = _qkv_shape(q)
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, 4, q.device)
        if tuple(t.shape) != (B, H, N, D):
            raise ValueError(f"{name} must have the shape of q")
    _need(idx, "idx", torch.int32, 4, q.device)
    _need(cnt, "cnt", torch.int32, 3, q.device)
    n = num_blocks(N, block)
    if tuple(idx.shape[:3]) != (B, H, n) or tuple(cnt.shape) != (B, H, n):
        raise ValueError("idx/cnt must be [B,H,n,max_keep] / [B,H,n]")
    return B, H, N, D


def forward_split_workspace_bytes(B: int, H: int, N: int, D: int, n_split: int) -> int:
    return int(_lib.load().ba_att_forward_split_workspace_bytes(B, H, N, D, n_split))


def forward_split(q, k, v, idx, cnt, block: int, n_split: int, scale: float | None = None,
                  out_dtype: torch.dtype = torch.float32, out=None, lse=None, return_lse: bool = True,
                  workspace: torch.Tensor | None = None):
    """Block-sparse attention with every row's block list cut into n_split
    parts attended separately and merged exactly; returns (O, LSE)."""
    B, H, N, D = _forward_args(q, k, v, idx, cnt, block)
    out, lse, code = _out(q, out_dtype, out, lse, return_lse)
    need = forward_split_workspace_bytes(B, H, N, D, n_split)
    if need == 0:
        raise ValueError("n_split must lie in [1, 64]")
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    with _on(q):
        _check(_lib.load().ba_att_forward_split(
            B, H, N, D, block, float(scale or 0.0), q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
            cnt.data_ptr(), int(idx.shape[3]), int(n_split), out.data_ptr(), code,
            lse.data_ptr() if lse is not None else None, workspace.data_ptr(), ws_bytes, _stream(q)))
    return out, lse


def forward_split_parts(B: int, H: int, N: int, block: int, max_keep: int) -> int:
    """n_split that fills the current device once (1: no split needed)."""
    parts = int(_lib.load().ba_att_forward_split_parts(B, H, N, block, max_keep))
    if parts < 1:
        raise ValueError("invalid shape, or the device cannot be queried")
    return parts


def forward_auto(q, k, v, idx, cnt, block: int, scale: float | None = None,
                 out_dtype: torch.dtype = torch.float32, out=None, lse=None, return_lse: bool = True):
    """ba_att_forward, or ba_att_forward_split with the suggested number of
    parts when the unsplit launch would leave the device partly idle."""
    B, H, N, D = _forward_args(q, k, v, idx, cnt, block)
    with _on(q):
        parts = forward_split_parts(B, H, N, block, int(idx.shape[3]))
    if parts == 1:
        return forward(q, k, v, idx, cnt, block, scale, out_dtype, out, lse, return_lse)
    return forward_split(q, k, v, idx, cnt, block, parts, scale, out_dtype, out, lse, return_lse)


def merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, out_dtype: torch.dtype = torch.float32,
          out=None, lse=None, return_lse: bool = True):
    """Exact log-space merge of attention results over disjoint key sets:
    o_parts fp32 [P,B,H,N,D], lse_parts fp32 [P,B,H,N] -> (O, LSE)."""
    _need(o_parts, "o_parts", torch.float32, 5)
    _need(lse_parts, "lse_parts", torch.float32, 4, o_parts.device)
    P, B, H, N, D = (int(x) for x in o_parts.shape)
    if tuple(lse_parts.shape) != (P, B, H, N):
        raise ValueError("lse_parts must be [P,B,H,N]")
    out, lse, code = _out(o_parts[0], out_dtype, out, lse, return_lse)
    with _on(o_parts):
        _check(_lib.load().ba_att_merge(B, H, N, D, P, o_parts.data_ptr(), lse_parts.data_ptr(),
                                        out.data_ptr(), code, lse.data_ptr() if lse is not None else None,
                                        _stream(o_parts)))
    return out, lse


def forward_ext(q, k, v, idx, cnt, block: int, o_ext: torch.Tensor, lse_ext: torch.Tensor,
                scale: float | None = None, out_dtype: torch.dtype = torch.float32, out=None, lse=None,
                return_lse: bool = True):
    """Block-sparse attention merged with an external attention result
    (o_ext fp32 [B,H,N,D], lse_ext fp32 [B,H,N]) over a disjoint key set."""
    B, H, N, D = _forward_args(q, k, v, idx, cnt, block)
    _need(o_ext, "o_ext", torch.float32, 4, q.device)
    _need(lse_ext, "lse_ext", torch.float32, 3, q.device)
    if tuple(o_ext.shape) != (B, H, N, D) or tuple(lse_ext.shape) != (B, H, N):
        raise ValueError("o_ext/lse_ext must be [B,H,N,D] / [B,H,N]")
    out, lse, code = _out(q, out_dtype, out, lse, return_lse)
    with _on(q):
        _check(_lib.load().ba_att_forward_ext(
            B, H, N, D, block, float(scale or 0.0), q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
            cnt.data_ptr(), int(idx.shape[3]), o_ext.data_ptr(), lse_ext.data_ptr(), out.data_ptr(), code,
            lse.data_ptr() if lse is not None else None, _stream(q)))
    return out, lse


def dense(q, k, v, scale: float | None = None, out_dtype: torch.dtype = torch.float32,
          out=None, lse=None, return_lse: bool = True):
    """Dense attention softmax(scale Q K^T) V; returns (O, LSE)."""
    B, H, N, D = _qkv_shape(q)
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, 4, q.device)
        if tuple(t.shape) != (B, H, N, D):
            raise ValueError(f"{name} must have the shape of q")
    out, lse, code = _out(q, out_dtype, out, lse, return_lse)
    with _on(q):
        _check(_lib.load().ba_att_dense(B, H, N, D, float(scale or 0.0), q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), out.data_ptr(), code,
                                        lse.data_ptr() if lse is not None else None, _stream(q)))
    return out, lse


def ba_attention(q, k, v, block: int, sparsity: float, scale: float | None = None,
                 out_dtype: torch.dtype = torch.bfloat16):
    """Both passes: selection then block-sparse attention; returns (O, LSE, mask)."""
    mask, idx, cnt = select(q, k, block, sparsity, scale)
    out, lse = forward(q, k, v, idx, cnt, block, scale, out_dtype=out_dtype)
    return out, lse, mask


def block_map(q, k, block: int, lse: torch.Tensor | None = None, scale: float | None = None):
    """Exact post-downsample maps of the full attention: M_lme fp32 [B,H,n,n]
    (block log-mean-exp of the logits) and, given the rows' natural-log LSE
    over all keys (fp32 [B,H,N], e.g. from dense), M_prob fp32 [B,H,n,n]
    (block mean of the softmax probabilities); M_prob is None without lse."""
    B, H, N, D = _qkv_shape(q)
    _need(k, "k", torch.bfloat16, 4, q.device)
    if tuple(k.shape) != (B, H, N, D):
        raise ValueError("k must have the shape of q")
    if lse is not None:
        _need(lse, "lse", torch.float32, 3, q.device)
        if tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be [B,H,N]")
    n = num_blocks(N, block)
    m_lme = torch.empty((B, H, n, n), dtype=torch.float32, device=q.device)
    m_prob = torch.empty_like(m_lme) if lse is not None else None
    with _on(q):
        _check(_lib.load().ba_att_block_map(
            B, H, N, D, block, float(scale or 0.0), q.data_ptr(), k.data_ptr(),
            lse.data_ptr() if lse is not None else None, m_lme.data_ptr(),
            m_prob.data_ptr() if m_prob is not None else None, _stream(q)))
    return m_lme, m_prob


def score_full_workspace_bytes(B: int, H: int, N: int, D: int, block: int) -> int:
    return int(_lib.load().ba_att_score_full_workspace_bytes(B, H, N, D, block))


def score_full(q, k, block: int, scale: float | None = None, workspace: torch.Tensor | None = None):
    """Block scores with full block covariances and without any correction:
    returns (S_full, S_mean), fp32 [B,H,n,n] each."""
    B, H, N, D = _qkv_shape(q)
    _need(k, "k", torch.bfloat16, 4, q.device)
    if tuple(k.shape) != (B, H, N, D):
        raise ValueError("k must have the shape of q")
    n = num_blocks(N, block)
    need = score_full_workspace_bytes(B, H, N, D, block)
    if need == 0:
        raise RuntimeError("BA-Att call failed: unsupported shape for the full-covariance score")
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    s_full = torch.empty((B, H, n, n), dtype=torch.float32, device=q.device)
    s_mean = torch.empty_like(s_full)
    with _on(q):
        _check(_lib.load().ba_att_score_full(
            B, H, N, D, block, float(scale or 0.0), q.data_ptr(), k.data_ptr(), s_full.data_ptr(),
            s_mean.data_ptr(), workspace.data_ptr(), ws_bytes, _stream(q)))
    return s_full, s_mean


def rank_agreement(x: torch.Tensor, r: torch.Tensor, keep: int):
    """Per row of two block maps fp32 [B,H,n,n]: (recall, rho) fp32 [B,H,n] --
    overlap of the kept sets (norm-sort rule) / keep, and Spearman's rho."""
    _need(x, "x", torch.float32, 4)
    _need(r, "r", torch.float32, 4, x.device)
    if x.shape != r.shape or x.shape[2] != x.shape[3]:
        raise ValueError("x and r must be the same [B,H,n,n] shape")
    B, H, n, _ = (int(v) for v in x.shape)
    recall = torch.empty((B, H, n), dtype=torch.float32, device=x.device)
    rho = torch.empty_like(recall)
    with _on(x):
        _check(_lib.load().ba_att_rank_agreement(B, H, n, int(keep), x.data_ptr(), r.data_ptr(),
                                                 recall.data_ptr(), rho.data_ptr(), _stream(x)))
    return recall, rho


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
