"""ctypes binding of libabg.so (include/abg.h).

Argument marshalling only: tensors are torch CUDA tensors (device memory),
passed as raw pointers with the current stream; all arithmetic runs in the
library's HIP kernels.  If the library has not been built the calls raise
instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libabg.so")

ABG_F32 = 0
ABG_BF16 = 1

STATUS = {0: "ABG_OK", 1: "ABG_ERR_NULL", 2: "ABG_ERR_SHAPE", 3: "ABG_ERR_UNSUPPORTED",
          4: "ABG_ERR_ALIGN", 5: "ABG_ERR_VALUE", 6: "ABG_ERR_DEVICE", 7: "ABG_ERR_ALIAS"}

#: Every symbol include/abg.h declares.
EXPORTS = ("abg_abi_version", "abg_status_string", "abg_last_error",
           "abg_pair_bias_project", "abg_biased_mqa_fwd", "abg_biased_mqa_fwd_ex",
           "abg_biased_mqa_fwd_workspace_bytes", "abg_biased_mqa_fwd_ex_noalloc",
           "abg_pair_biased_mqa_fwd")

#: Device scratch that abg_biased_mqa_fwd_ex_noalloc holds per GPU
#: (ABG_NOALLOC_SCRATCH_BYTES in include/abg.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


class AbgError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libabg.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.abg_abi_version.restype = i32
    lib.abg_abi_version.argtypes = []
    lib.abg_status_string.restype = ctypes.c_char_p
    lib.abg_status_string.argtypes = [i32]
    lib.abg_last_error.restype = ctypes.c_char_p
    lib.abg_last_error.argtypes = []
    lib.abg_pair_bias_project.restype = i32
    lib.abg_pair_bias_project.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, vp]
    lib.abg_biased_mqa_fwd.restype = i32
    lib.abg_biased_mqa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                       i64, i64, f32, f32, i32, vp]
    lib.abg_biased_mqa_fwd_ex.restype = i32
    lib.abg_biased_mqa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                          i64, i64, i64, i64, i64, i64, f32, f32, i32, vp]
    lib.abg_biased_mqa_fwd_workspace_bytes.restype = i64
    lib.abg_biased_mqa_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.abg_biased_mqa_fwd_ex_noalloc.restype = i32
    lib.abg_biased_mqa_fwd_ex_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                  i64, i64, i64, i64, i64, f32, f32, i32, vp]
    lib.abg_pair_biased_mqa_fwd.restype = i32
    lib.abg_pair_biased_mqa_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                            i64, i64, i64, i64, i64, i64, i64, f32, f32, i32, vp]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load().abg_last_error().decode(errors="replace")
        raise AbgError(status, msg)


# ---------------------------------------------------------------------------
# Raw calls (pointers and sizes), as in include/abg.h
# ---------------------------------------------------------------------------
def raw_pair_bias_project(pair, weight, bias, Bp, P, C, H, dtype, stream=None) -> int:
    return load().abg_pair_bias_project(pair, weight, bias, Bp, P, C, H, dtype, stream)


def raw_biased_mqa_fwd(q, k, v, bias, out, B, S, Hq, Dk, Dv, bias_batch_stride,
                       bias_group, scale, softcap, dtype, stream=None) -> int:
    return load().abg_biased_mqa_fwd(q, k, v, bias, out, B, S, Hq, Dk, Dv,
                                     bias_batch_stride, bias_group, scale, softcap,
                                     dtype, stream)


def raw_biased_mqa_fwd_ex(q, k, v, bias, out, workspace, workspace_bytes, B, Sq, Sk, q_offset,
                          Hq, Dk, Dv, bias_batch_stride, bias_group, kv_splits, scale, softcap,
                          dtype, stream=None) -> int:
    return load().abg_biased_mqa_fwd_ex(q, k, v, bias, out, workspace, workspace_bytes, B, Sq,
                                        Sk, q_offset, Hq, Dk, Dv, bias_batch_stride,
                                        bias_group, kv_splits, scale, softcap, dtype, stream)


def raw_biased_mqa_fwd_ex_noalloc(q, k, v, bias, out, B, Sq, Sk, q_offset, Hq, Dk, Dv,
                                  bias_batch_stride, bias_group, kv_splits, scale, softcap, dtype,
                                  stream=None) -> int:
    return load().abg_biased_mqa_fwd_ex_noalloc(q, k, v, bias, out, B, Sq, Sk, q_offset, Hq, Dk,
                                                Dv, bias_batch_stride, bias_group, kv_splits,
                                                scale, softcap, dtype, stream)


def raw_pair_biased_mqa_fwd(q, k, v, pair, weight, out, workspace, workspace_bytes, B, Sq, Sk,
                            q_offset, Hq, Dk, Dv, C, pair_batch_stride, pair_group, kv_splits,
                            scale, softcap, dtype, stream=None) -> int:
    return load().abg_pair_biased_mqa_fwd(q, k, v, pair, weight, out, workspace, workspace_bytes,
                                          B, Sq, Sk, q_offset, Hq, Dk, Dv, C, pair_batch_stride,
                                          pair_group, kv_splits, scale, softcap, dtype, stream)


def workspace_bytes(B, Sq, Hq, Dv, kv_splits) -> int:
    """Device workspace that a call with ``kv_splits`` key ranges needs."""
    return int(load().abg_biased_mqa_fwd_workspace_bytes(B, Sq, Hq, Dv, kv_splits))


def auto_kv_splits(B, Sq, Sk, target_groups=256) -> int:
    """Fewest key ranges (a power of two dividing the ceil(Sk/64) key tiles,
    at most 64) that give at least ``target_groups`` workgroups (one per CU)."""
    tiles = -(-Sk // 64)
    blocks = -(-Sq // 32)
    z = 1
    while B * blocks * z < target_groups and z < 64 and tiles % (2 * z) == 0:
        z *= 2
    return z


# ---------------------------------------------------------------------------
# torch front end
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ABG_BF16
    if t.dtype == torch.float32:
        return ABG_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device) -> Optional[int]:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def pair_bias_project(pair, weight, out=None):
    """bias[b, h, p, r] = sum_c pair[b, p, r, c] * weight[c, h].

    ``pair`` [Bp, P, P, C] or [P, P, C] and ``weight`` [C, 8] of the same
    dtype (bfloat16 or float32); returns float32 [Bp, 8, P, P] (or [8, P, P]).
    """
    import torch
    _dev(pair, "pair")
    _dev(weight, "weight")
    squeeze = pair.dim() == 3
    p4 = pair.unsqueeze(0) if squeeze else pair
    if p4.dim() != 4 or p4.shape[1] != p4.shape[2]:
        raise ValueError(f"pair must be [Bp, P, P, C], got {tuple(pair.shape)}")
    Bp, P, _, C = p4.shape
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError(f"weight must be [C={C}, H], got {tuple(weight.shape)}")
    if weight.dtype != pair.dtype:
        raise TypeError("pair and weight must have the same dtype")
    H = weight.shape[1]
    if out is None:
        out = torch.empty((Bp, H, P, P), dtype=torch.float32, device=pair.device)
    _dev(out, "out")
    if out.dtype != torch.float32 or out.numel() != Bp * H * P * P:
        raise ValueError("out must be float32 [Bp, H, P, P]")
    _check(raw_pair_bias_project(p4.data_ptr(), weight.data_ptr(), out.data_ptr(), Bp, P, C, H,
                                 _dtype_code(pair), _stream(pair.device)))
    return out[0] if (squeeze and out.dim() == 4) else out


def _attn_args(q, k, v, bias, out, scale, bias_group):
    """Shapes, dtypes and strides of an attention call (checks only); returns
    (B, Sq, Sk, Hq, Dk, Dv, bias_stride, scale, out), with ``out`` a new
    tensor if None was given."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (bias, "bias")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, S, heads, D]")
    B, Sq, Hq, Dk = q.shape
    Sk = k.shape[1]
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, Sk, 1, Dk) or tuple(v.shape[:3]) != (B, Sk, 1):
        raise ValueError(f"k must be [B,Sk,1,Dk] and v [B,Sk,1,Dv]; got {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if bias.dtype != torch.float32:
        raise TypeError("bias must be float32")
    P = (Sk + 15) // 16  # compact bias cells per side
    if bias.dim() == 3:
        bias_stride = 0
        if tuple(bias.shape) != (Hq, P, P):
            raise ValueError(f"bias must be [{Hq},{P},{P}], got {tuple(bias.shape)}")
    elif bias.dim() == 4:
        if tuple(bias.shape[1:]) != (Hq, P, P):
            raise ValueError(f"bias must be [Bb,{Hq},{P},{P}], got {tuple(bias.shape)}")
        bias_stride = 0 if bias.shape[0] == 1 else Hq * P * P
        if bias.shape[0] > 1 and bias.shape[0] * bias_group < B:
            raise ValueError("bias has too few items for B and bias_group")
    else:
        raise ValueError("bias must be 3-D or 4-D")
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=q.dtype, device=q.device)
    _dev(out, "out")
    if out.dtype != q.dtype or tuple(out.shape) != (B, Sq, Hq, Dv):
        raise ValueError("out must match q's dtype and be [B, Sq, Hq, Dv]")
    return B, Sq, Sk, Hq, Dk, Dv, bias_stride, scale, out


def biased_mqa_fwd(q, k, v, bias, out=None, *, scale: Optional[float] = None,
                   softcap: float = 5.0, bias_group: int = 1, q_offset: int = 0,
                   kv_splits=1, workspace=None):
    """Biased, soft-capped multi-query attention forward on the GPU.

    ``q`` [B, Sq, 8, 128] holds positions q_offset .. q_offset + Sq - 1 of a
    sequence whose ``k`` [B, Sk, 1, 128] and ``v`` [B, Sk, 1, Dv] (bfloat16 or
    float32; Dv 128, or 192 for bf16 with the cap) cover all Sk positions;
    Sq == Sk and q_offset == 0 is the plain call.  ``bias`` float32 compact
    bias [8, P, P] (P = ceil(Sk/16)) shared by all items, or [Bb, 8, P, P]
    with item b reading block b // bias_group.  ``scale`` defaults to
    1/sqrt(128); ``softcap`` 0 disables the cap.  ``kv_splits`` > 1 (or
    "auto") computes key ranges in separate workgroups and merges them; the
    float32 workspace is ``workspace`` or a new device tensor.  Returns
    ``out`` [B, Sq, 8, Dv] in the input dtype.
    """
    import torch
    B, Sq, Sk, Hq, Dk, Dv, bias_stride, scale, out = _attn_args(q, k, v, bias, out, scale,
                                                                bias_group)
    if kv_splits == "auto":
        kv_splits = auto_kv_splits(B, Sq, Sk)
    kv_splits = int(kv_splits)
    if kv_splits == 1 and Sq == Sk and q_offset == 0 and workspace is None:
        _check(raw_biased_mqa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), bias.data_ptr(),
                                  out.data_ptr(), B, Sk, Hq, Dk, Dv, bias_stride, bias_group,
                                  float(scale), float(softcap), _dtype_code(q), _stream(q.device)))
        return out
    need = workspace_bytes(B, Sq, Hq, Dv, kv_splits) if kv_splits >= 1 else 0
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(raw_biased_mqa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), bias.data_ptr(),
                                 out.data_ptr(), ws_ptr, ws_bytes, B, Sq, Sk, int(q_offset), Hq,
                                 Dk, Dv, bias_stride, bias_group, kv_splits, float(scale),
                                 float(softcap), _dtype_code(q), _stream(q.device)))
    return out


def biased_mqa_fwd_ex_noalloc(q, k, v, bias, out, *, scale: Optional[float] = None,
                              softcap: float = 5.0, bias_group: int = 1, q_offset: int = 0,
                              kv_splits: int = 1):
    """``biased_mqa_fwd`` through abg_biased_mqa_fwd_ex_noalloc: the key
    ranges' partials go to the library's own per-GPU scratch array, so the
    call allocates nothing (``out`` must be given).  At most
    NOALLOC_SCRATCH_BYTES of partials; calls on one GPU must not overlap in
    time (they share that array)."""
    if out is None:
        raise ValueError("out must be given: this call allocates nothing")
    B, Sq, Sk, Hq, Dk, Dv, bias_stride, scale, out = _attn_args(q, k, v, bias, out, scale,
                                                                bias_group)
    _check(raw_biased_mqa_fwd_ex_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         bias.data_ptr(), out.data_ptr(), B, Sq, Sk,
                                         int(q_offset), Hq, Dk, Dv, bias_stride, bias_group,
                                         int(kv_splits), float(scale), float(softcap),
                                         _dtype_code(q), _stream(q.device)))
    return out


def pair_biased_mqa_fwd(q, k, v, pair, weight, out=None, *, scale: Optional[float] = None,
                        softcap: float = 5.0, pair_group: int = 1, q_offset: int = 0,
                        kv_splits=1, workspace=None):
    """``biased_mqa_fwd`` with the bias projected inside the attention kernel
    from ``pair`` [P, P, 128] or [Bp, P, P, 128] and ``weight`` [128, 8] (both
    bfloat16; P = ceil(Sk/16)), so that no bias tensor is ever written.  Item
    b reads pair block b // pair_group.  bfloat16 inputs with the cap, value
    width 128 or 192.  Returns ``out`` [B, Sq, 8, Dv].
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (pair, "pair"), (weight, "weight")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, S, heads, D]")
    B, Sq, Hq, Dk = q.shape
    Sk = k.shape[1]
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, Sk, 1, Dk) or tuple(v.shape[:3]) != (B, Sk, 1):
        raise ValueError(f"k must be [B,Sk,1,Dk] and v [B,Sk,1,Dv]; got {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype == pair.dtype == weight.dtype):
        raise TypeError("q, k, v, pair and weight must share a dtype")
    P = (Sk + 15) // 16
    p4 = pair.unsqueeze(0) if pair.dim() == 3 else pair
    if p4.dim() != 4 or tuple(p4.shape[1:3]) != (P, P):
        raise ValueError(f"pair must be [P, P, C] or [Bp, P, P, C] with P = {P}, got {tuple(pair.shape)}")
    C = p4.shape[3]
    if tuple(weight.shape) != (C, Hq):
        raise ValueError(f"weight must be [{C}, {Hq}], got {tuple(weight.shape)}")
    if p4.shape[0] > 1 and p4.shape[0] * pair_group < B:
        raise ValueError("pair has too few items for B and pair_group")
    pair_stride = 0 if p4.shape[0] == 1 else P * P * C
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=q.dtype, device=q.device)
    _dev(out, "out")
    if out.dtype != q.dtype or tuple(out.shape) != (B, Sq, Hq, Dv):
        raise ValueError("out must match q's dtype and be [B, Sq, Hq, Dv]")
    if kv_splits == "auto":
        kv_splits = auto_kv_splits(B, Sq, Sk)
    kv_splits = int(kv_splits)
    need = workspace_bytes(B, Sq, Hq, Dv, kv_splits) if kv_splits >= 1 else 0
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(raw_pair_biased_mqa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), p4.data_ptr(),
                                   weight.data_ptr(), out.data_ptr(), ws_ptr, ws_bytes, B, Sq, Sk,
                                   int(q_offset), Hq, Dk, Dv, C, pair_stride, pair_group, kv_splits,
                                   float(scale), float(softcap), _dtype_code(q), _stream(q.device)))
    return out
