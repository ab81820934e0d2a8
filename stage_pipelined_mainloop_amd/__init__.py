"""Stage-pipelined half-precision TN GEMM for MI355X (gfx950).

    D = alpha * A @ B.T     A: (M, K) fp16, B: (N, K) fp16, D: (M, N) fp16

The work is done by hand-written HIP kernels in libstagegemm.so behind the
C-ABI declared in include/stagegemm.h.  `_lib` mirrors that ABI name for name
(pointers and sizes); `gemm` is a thin torch convenience that passes tensor
pointers and the current HIP stream.  PyTorch only provides device memory and
streams.  Importing this package loads nothing; the library is loaded on the
first call and a missing build raises.
"""
from __future__ import annotations

from ._lib import (SgConfig, SgConfigInfo, SgError, attention_fp16_fwd, attention_fp16_fwd_split,
                   attention_fp16_splits, attention_fp16_workspace_bytes, configs, gemm_fp16_tn,
                   gemm_fp16_tn_alpha,
                   gemm_fp16_tn_alpha_beta, gemm_fp16_tn_cfg, gemm_fp16_tn_splitk,
                   gemm_fp16_tn_splitk_noalloc,
                   gemm_fp16_tn_splitk_splits, gemm_fp16_tn_splitk_workspace_bytes, sg_get_config,
                   gemm_fp16_tn_remainder_quarters,
                   sg_minimum_stages, sg_num_configs,
                   sg_persistent_wait_count, sg_pipeline_wait_count, sg_query_config, sg_select_config,
                   sg_split_plan, sg_status_string, SgSplitInfo)

# Split-K workspaces kept per (device, stream) and reused: calls on one
# stream never overlap, calls on different streams get different buffers.
_split_workspaces: dict = {}


def split_workspace(device, stream, nbytes: int):
    """A device buffer of at least `nbytes` for split-K calls on `stream` (a
    torch.cuda.Stream), reused across calls.  Under HIP-graph capture a fresh
    buffer is allocated from the graph's pool each time."""
    import torch
    if torch.cuda.is_current_stream_capturing():
        with torch.cuda.stream(stream):
            return torch.empty(nbytes, dtype=torch.uint8, device=device)
    key = (torch.device(device).index, stream.cuda_stream)
    buf = _split_workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(stream):
            buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _split_workspaces[key] = buf
    return buf


def gemm(A, B, out=None, alpha: float | None = None, config=None, stream=None,
         beta: float | None = None, C=None, splits: int | None = None, workspace=None):
    """D = alpha * A @ B.T (+ beta * C) on the GPU for fp16 CUDA (HIP) tensors.

    A: (M, K), B: (N, K), out: (M, N) or None (allocated).  `config` picks a
    compiled variant (SgConfig or a 6-tuple) instead of the library's choice.
    With a non-zero `beta`, C is an (M, N) fp16 tensor (it may be `out`
    itself for an in-place update).  `stream` is a torch.cuda.Stream
    (default: the current stream).

    Without config or C, the call may split output tiles along K
    (gemm_fp16_tn_splitk): `splits` sets the count (default: the library's
    choice for the shape; 1 = never).  Its `workspace` (a device tensor of at
    least gemm_fp16_tn_splitk_workspace_bytes bytes) is allocated once per
    stream when not given."""
    import torch

    if A.dtype != torch.float16 or B.dtype != torch.float16:
        raise TypeError("A and B must be float16")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError(f"shapes {tuple(A.shape)} and {tuple(B.shape)} do not form A @ B.T")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be device tensors on the same device")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major)")
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    elif (out.dtype != torch.float16 or tuple(out.shape) != (M, N) or not out.is_contiguous()
          or out.device != A.device):
        raise ValueError("out must be a contiguous (M, N) float16 tensor on A's device")
    s = (stream if stream is not None else torch.cuda.current_stream(A.device)).cuda_stream
    a, b, d = A.data_ptr(), B.data_ptr(), out.data_ptr()
    if beta is not None and beta != 0.0:
        if config is not None:
            raise ValueError("beta is not available with an explicit config")
        if C is None or C.dtype != torch.float16 or tuple(C.shape) != (M, N) \
                or not C.is_contiguous() or C.device != A.device:
            raise ValueError("beta needs C: a contiguous (M, N) float16 tensor on A's device")
        gemm_fp16_tn_alpha_beta(M, N, K, 1.0 if alpha is None else float(alpha), float(beta),
                                a, b, C.data_ptr(), d, s)
    elif config is not None:
        gemm_fp16_tn_cfg(M, N, K, 1.0 if alpha is None else float(alpha), a, b, d, config, s)
    else:
        st = stream if stream is not None else torch.cuda.current_stream(A.device)
        need = 0
        if M > 0 and N > 0 and K > 0 and (splits is None or splits > 1):
            with torch.cuda.device(A.device):          # the library queries the current device
                if splits is None:
                    splits = max(gemm_fp16_tn_splitk_splits(M, N, K), 1)
                if splits > 1:
                    need = gemm_fp16_tn_splitk_workspace_bytes(M, N, K, splits)
        if need > 0:
            if workspace is None:
                workspace = split_workspace(A.device, st, need)
            elif (not workspace.is_cuda or workspace.device != A.device
                  or workspace.numel() * workspace.element_size() < need):
                raise ValueError(f"workspace must be a tensor of at least {need} bytes on A's device")
            with torch.cuda.device(A.device):
                gemm_fp16_tn_splitk(M, N, K, 1.0 if alpha is None else float(alpha), a, b, d, splits,
                                    workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), s)
        elif alpha is None:
            gemm_fp16_tn(M, N, K, a, b, d, s)
        else:
            gemm_fp16_tn_alpha(M, N, K, float(alpha), a, b, d, s)
    return out


def attention(Q, K, V, alpha: float | None = None, out=None, stream=None, splits: int | None = None,
              workspace=None):
    """O = softmax(alpha * Q K^T) V, softmax along each row, on the GPU.

    Q: (H, M, d) or (M, d); K, V: (H, N, d) or (N, d); fp16 CUDA (HIP)
    tensors, contiguous; d = 128.  alpha defaults to fp32(1 / sqrt(d)).
    `splits` cuts the keys into that many runs merged afterwards (default:
    the library's choice for the device, 1 when the heads already fill it);
    with more than one, `workspace` (a device tensor of at least
    attention_fp16_workspace_bytes bytes) is used, or one is allocated.
    Returns O shaped like Q."""
    import math

    import torch

    if Q.dtype != torch.float16 or K.dtype != torch.float16 or V.dtype != torch.float16:
        raise TypeError("Q, K and V must be float16")
    q3, k3, v3 = (x if x.dim() == 3 else x.unsqueeze(0) for x in (Q, K, V))
    if q3.dim() != 3 or k3.shape != v3.shape or q3.shape[0] != k3.shape[0] \
            or q3.shape[2] != k3.shape[2]:
        raise ValueError(f"shapes {tuple(Q.shape)}, {tuple(K.shape)}, {tuple(V.shape)} do not match")
    if not (Q.is_cuda and K.is_cuda and V.is_cuda) or not (Q.device == K.device == V.device):
        raise ValueError("Q, K and V must be device tensors on the same device")
    if not (Q.is_contiguous() and K.is_contiguous() and V.is_contiguous()):
        raise ValueError("Q, K and V must be contiguous")
    H, M, d = q3.shape
    N = k3.shape[1]
    if alpha is None:
        alpha = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty_like(Q)
    elif (out.shape != Q.shape or out.dtype != torch.float16 or not out.is_contiguous()
          or out.device != Q.device):
        raise ValueError("out must be a contiguous float16 tensor shaped like Q, on Q's device")
    st = stream if stream is not None else torch.cuda.current_stream(Q.device)
    if H == 0 or M == 0:
        splits = 1
    elif splits is None:
        with torch.cuda.device(Q.device):
            splits = attention_fp16_splits(H, M, N, d)
        # -1 (sizes the library refuses): the call below reports why
        splits = max(splits, 1)
    need = attention_fp16_workspace_bytes(H, M, N, d, splits) if splits > 1 else 0
    if need == 0:
        with torch.cuda.device(Q.device):              # the launcher queries the current device
            attention_fp16_fwd_split(H, M, N, d, float(alpha), Q.data_ptr(), K.data_ptr(),
                                     V.data_ptr(), out.data_ptr(), splits, 0, 0, st.cuda_stream)
        return out
    if workspace is None:
        with torch.cuda.stream(st):
            workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    elif (not workspace.is_cuda or workspace.device != Q.device
          or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace must be a tensor of at least {need} bytes on Q's device")
    with torch.cuda.device(Q.device):
        attention_fp16_fwd_split(H, M, N, d, float(alpha), Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                 out.data_ptr(), splits, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), st.cuda_stream)
    return out


__all__ = [
    "gemm", "attention", "attention_fp16_fwd", "attention_fp16_fwd_split", "attention_fp16_splits",
    "attention_fp16_workspace_bytes", "gemm_fp16_tn", "gemm_fp16_tn_alpha", "gemm_fp16_tn_alpha_beta", "gemm_fp16_tn_cfg",
    "gemm_fp16_tn_splitk", "gemm_fp16_tn_splitk_noalloc", "gemm_fp16_tn_splitk_splits",
    "gemm_fp16_tn_remainder_quarters",
    "gemm_fp16_tn_splitk_workspace_bytes",
    "split_workspace", "sg_split_plan", "SgSplitInfo",
    "sg_select_config",
    "sg_num_configs", "sg_get_config", "sg_query_config", "sg_minimum_stages",
    "sg_pipeline_wait_count", "sg_persistent_wait_count", "sg_status_string", "configs", "SgConfig", "SgConfigInfo",
    "SgError",
]
