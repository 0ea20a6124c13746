"""Thin PyTorch-facing binding of the ring-attention C ABI.

Only argument marshalling happens here: torch supplies device memory and the
current HIP stream; every step of the computation runs in libra.so's kernels.
Tensors are token-major [batch, tokens, heads, head_dim] with a contiguous
last axis; K/V rings are [world, batch, tokens, heads, head_dim].
"""
from __future__ import annotations

import ctypes as C
from contextlib import contextmanager
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import check, lib, ra_posmap, ra_problem, ra_seg, ra_tensor

LAYOUTS = tuple(_lib.LAYOUT_IDS)


def _torch():
    import torch
    return torch


def _dtype_id(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return _lib.DTYPE_BF16
    if dt == torch.float32:
        return _lib.DTYPE_F32
    raise TypeError(f"unsupported dtype {dt} (bf16 or fp32)")


def _layout_id(layout: str) -> int:
    try:
        return _lib.LAYOUT_IDS[layout]
    except KeyError:
        raise ValueError(f"unknown layout {layout!r}; expected one of {LAYOUTS}") from None


def _t4(x) -> ra_tensor:
    """ra_tensor for a [b, tokens, heads, dim] tensor (None -> empty)."""
    if x is None:
        return ra_tensor(None, 0, 0, 0)
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("expected a [batch, tokens, heads, head_dim] tensor with contiguous head_dim")
    if not x.is_cuda:
        raise ValueError("tensors must be device (HIP) tensors")
    return ra_tensor(x.data_ptr(), x.stride(0), x.stride(1), x.stride(2))


def _t5(x) -> Tuple[ra_tensor, int]:
    """ra_tensor of block 0 of a [world, b, tokens, heads, dim] ring, and its rank stride."""
    if x.dim() != 5 or x.stride(4) != 1:
        raise ValueError("expected a [world, batch, tokens, heads, head_dim] ring with contiguous head_dim")
    if not x.is_cuda:
        raise ValueError("tensors must be device (HIP) tensors")
    return ra_tensor(x.data_ptr(), x.stride(1), x.stride(2), x.stride(3)), x.stride(0)


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


class CuSeqlens:
    """cu_seqlens (int32 offsets [0, l0, l0+l1, ...]) held once on the host and once on
    ``device``.  The library takes both copies (the host one plans the ring steps and
    splits the per-sequence layouts; the kernels read the device one).  Given a plain
    list, array or tensor instead, every call makes the missing copy itself, and copying
    a device tensor to the host waits for the stream; build this once and pass it to
    every call that uses the same sequences."""

    def __init__(self, cu_seqlens, device):
        torch = _torch()
        if isinstance(cu_seqlens, CuSeqlens):
            cu_seqlens = cu_seqlens.host
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        self.host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        if self.host.ndim != 1 or self.host.size < 2:
            raise ValueError("cu_seqlens must hold at least two offsets")
        self.dev = torch.from_numpy(self.host.copy()).to(device)

    @property
    def num_seqs(self) -> int:
        return int(self.host.size) - 1


def _host_cu(cu_seqlens):
    """The host int32 array of any accepted cu_seqlens form."""
    if isinstance(cu_seqlens, CuSeqlens):
        return cu_seqlens.host
    return np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                                           dtype=np.int32))


class _Cu:
    """Keeps the device and host copies of cu_seqlens alive for a call."""

    def __init__(self, cu_seqlens, device):
        torch = _torch()
        self.dev = None
        self.host = None
        self.n = 0
        if cu_seqlens is None:
            return
        if isinstance(cu_seqlens, CuSeqlens):
            if cu_seqlens.dev.device != torch.device(device):
                raise ValueError("CuSeqlens was built for another device")
            self.host, self.dev, self.n = cu_seqlens.host, cu_seqlens.dev, cu_seqlens.num_seqs
            return
        if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
            # the host copy lets the library skip steps and split per-sequence layouts
            self.dev = cu_seqlens.to(torch.int32).contiguous()
            self.host = np.ascontiguousarray(self.dev.cpu().numpy())
        else:
            self.host = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
            self.dev = torch.from_numpy(self.host).to(device)
        self.n = int(self.dev.numel()) - 1

    def fill(self, p: ra_problem):
        if self.dev is None:
            p.cu_seqlens = None
            p.cu_seqlens_host = None
            p.num_seqs = 0
        else:
            p.cu_seqlens = self.dev.data_ptr()
            p.cu_seqlens_host = self.host.ctypes.data if self.host is not None else None
            p.num_seqs = self.n


def _problem(x, heads: int, head_dim: int, seq_len: int, causal: bool, scale: Optional[float], cu: _Cu) -> ra_problem:
    p = ra_problem()
    p.batch = x.shape[0] if x.dim() == 4 else x.shape[1]
    p.heads = heads
    p.head_dim = head_dim
    p.dtype = _dtype_id(x.dtype)
    p.softmax_scale = float(scale) if scale is not None else 0.0
    p.causal = 1 if causal else 0
    p.seq_len = int(seq_len)
    cu.fill(p)
    return p


# ---- layouts -------------------------------------------------------------------------------

def layout_positions(layout: str, seq_len: int, world: int, rank: int, cu_seqlens=None) -> np.ndarray:
    """Global positions of ``rank``'s local tokens (as the library lays them out).
    The per-sequence layouts (``zigzag_varlen``, ``stripe_varlen``) need ``cu_seqlens``."""
    out = np.empty(seq_len // max(world, 1), dtype=np.int64)
    if cu_seqlens is None:
        check(lib().ra_layout_positions(_layout_id(layout), seq_len, world, rank,
                                        out.ctypes.data_as(C.POINTER(C.c_int64))))
        return out
    cu = _host_cu(cu_seqlens)
    if int(cu[-1]) != seq_len:
        raise ValueError("cu_seqlens must end at seq_len")
    check(lib().ra_layout_positions_cu(_layout_id(layout), cu.ctypes.data_as(C.POINTER(C.c_int32)), len(cu) - 1,
                                       world, rank, out.ctypes.data_as(C.POINTER(C.c_int64))))
    return out


def layout_posmap(layout: str, seq_len: int, world: int, rank: int) -> ra_posmap:
    m = ra_posmap()
    check(lib().ra_layout_posmap(_layout_id(layout), seq_len, world, rank, C.byref(m)))
    return m


def posmap(segments: Sequence[Tuple[int, int, int]]) -> ra_posmap:
    """Posmap from up to two (begin, stride, len) runs in local order."""
    if not 1 <= len(segments) <= 2:
        raise ValueError("one or two segments")
    m = ra_posmap()
    m.nseg = len(segments)
    for i, (b, s, n) in enumerate(segments):
        m.seg[i] = ra_seg(int(b), int(s), int(n))
    return m


# ---- block level ---------------------------------------------------------------------------

def block_attn_fwd(q, k, v, qmap: ra_posmap, kmap: ra_posmap, *, seq_len: int, causal: bool = False,
                   cu_seqlens=None, scale: Optional[float] = None, out_b=None, lse_b=None):
    """One block step: returns (out_b fp32 [b, lq, h, d], lse_b fp32 [b, h, lq])."""
    torch = _torch()
    b, lq, h, d = q.shape
    lk = k.shape[1]
    if out_b is None:
        out_b = torch.empty((b, lq, h, d), device=q.device, dtype=torch.float32)
    if lse_b is None:
        lse_b = torch.empty((b, h, lq), device=q.device, dtype=torch.float32)
    cu = _Cu(cu_seqlens, q.device)
    p = _problem(q, h, d, seq_len, causal, scale, cu)
    check(lib().ra_block_attn_fwd(C.byref(p), _t4(q), lq, qmap, _t4(k), _t4(v), lk, kmap, _t4(out_b),
                                  lse_b.data_ptr(), _stream()))
    return out_b, lse_b


def lse_merge(out, lse, out_b, lse_b) -> None:
    """In place: (out, lse) <- merge((out, lse), (out_b, lse_b)); all fp32."""
    b, lq, h, d = out.shape
    p = ra_problem()
    p.batch, p.heads, p.head_dim, p.dtype = b, h, d, _lib.DTYPE_F32
    check(lib().ra_lse_merge(C.byref(p), lq, _t4(out), lse.data_ptr(), _t4(out_b), lse_b.data_ptr(), _stream()))


def bwd_preprocess(out, dout):
    """delta = rowsum(dout * out) as fp32 [b, h, lq]."""
    torch = _torch()
    b, lq, h, d = out.shape
    delta = torch.empty((b, h, lq), device=out.device, dtype=torch.float32)
    p = ra_problem()
    p.batch, p.heads, p.head_dim, p.dtype = b, h, d, _dtype_id(dout.dtype)
    check(lib().ra_bwd_preprocess(C.byref(p), lq, _t4(out), _t4(dout), delta.data_ptr(), _stream()))
    return delta


def block_attn_bwd(q, k, v, dout, lse, delta, qmap: ra_posmap, kmap: ra_posmap, dq_acc, dk_acc, dv_acc, *,
                   seq_len: int, causal: bool = False, cu_seqlens=None, scale: Optional[float] = None) -> None:
    """Accumulate one block step's gradients into dq_acc/dk_acc/dv_acc (fp32)."""
    b, lq, h, d = q.shape
    lk = k.shape[1]
    cu = _Cu(cu_seqlens, q.device)
    p = _problem(q, h, d, seq_len, causal, scale, cu)
    check(lib().ra_block_attn_bwd(C.byref(p), _t4(q), lq, qmap, _t4(k), _t4(v), lk, kmap, _t4(dout),
                                  lse.data_ptr(), delta.data_ptr(), _t4(dq_acc), _t4(dk_acc), _t4(dv_acc),
                                  _stream()))


# ---- virtual ring --------------------------------------------------------------------------

def ring_fwd(layout: str, world: int, rank: int, q_local, k_ring, v_ring, *, causal: bool = True,
             cu_seqlens=None, scale: Optional[float] = None, out=None, lse=None, want_lowp: bool = False,
             out_lowp=None):
    """Rank ``rank``'s share of the virtual ring.  Returns (out fp32, lse fp32, out_lowp or None)."""
    torch = _torch()
    b, L, h, d = q_local.shape
    S = L * world
    if out is None:
        out = torch.empty((b, L, h, d), device=q_local.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty((b, h, L), device=q_local.device, dtype=torch.float32)
    if want_lowp and out_lowp is None:
        out_lowp = torch.empty((b, L, h, d), device=q_local.device, dtype=q_local.dtype)
    cu = _Cu(cu_seqlens, q_local.device)
    p = _problem(q_local, h, d, S, causal, scale, cu)
    kt, srank = _t5(k_ring)
    vt, srank_v = _t5(v_ring)
    if srank != srank_v:
        raise ValueError("k_ring and v_ring must share the rank stride")
    check(lib().ra_ring_fwd(C.byref(p), _layout_id(layout), world, rank, _t4(q_local), kt, vt, srank,
                            _t4(out), lse.data_ptr(), _t4(out_lowp), _stream()))
    return out, lse, out_lowp


def ring_workspace_bytes(layout: str, world: int, q_local, causal: bool = True, minimal: bool = False,
                         cu_seqlens=None) -> int:
    """Workspace bytes ring_bwd uses: its fastest path (stored dS for bf16), or with
    ``minimal`` the least it accepts (dQ then recomputes S and dP)."""
    b, L, h, d = q_local.shape
    p = _problem(q_local, h, d, L * world, causal, None, _Cu(cu_seqlens, q_local.device))
    fn = lib().ra_ring_workspace_min_bytes if minimal else lib().ra_ring_workspace_bytes
    return int(fn(C.byref(p), _layout_id(layout), world))


def ring_bwd(layout: str, world: int, rank: int, q_local, k_ring, v_ring, out, lse, dout, *,
             causal: bool = True, cu_seqlens=None, scale: Optional[float] = None,
             dq=None, dk_ring=None, dv_ring=None, workspace=None, store_ds: bool = True):
    """Backward of rank ``rank``'s share.  dq is overwritten; dk_ring/dv_ring (fp32) are accumulated
    (allocated zeroed when not given).  ``workspace`` (uint8 device tensor) is allocated when not
    given: of ring_workspace_bytes() with ``store_ds`` (dQ from the stored dS), else of the
    minimal size (dQ recomputes S and dP).  Returns (dq, dk_ring, dv_ring)."""
    torch = _torch()
    b, L, h, d = q_local.shape
    S = L * world
    dev = q_local.device
    if dq is None:
        dq = torch.empty((b, L, h, d), device=dev, dtype=torch.float32)
    if dk_ring is None:
        dk_ring = torch.zeros((world, b, L, h, d), device=dev, dtype=torch.float32)
    if dv_ring is None:
        dv_ring = torch.zeros((world, b, L, h, d), device=dev, dtype=torch.float32)
    cu = _Cu(cu_seqlens, dev)
    p = _problem(q_local, h, d, S, causal, scale, cu)
    fn = lib().ra_ring_workspace_bytes if store_ds else lib().ra_ring_workspace_min_bytes
    need = int(fn(C.byref(p), _layout_id(layout), world))
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=dev, dtype=torch.uint8)
    kt, srank = _t5(k_ring)
    vt, _ = _t5(v_ring)
    dkt, sgrad = _t5(dk_ring)
    dvt, sgrad_v = _t5(dv_ring)
    if sgrad != sgrad_v:
        raise ValueError("dk_ring and dv_ring must share the rank stride")
    check(lib().ra_ring_bwd(C.byref(p), _layout_id(layout), world, rank, _t4(q_local), kt, vt, srank,
                            _t4(out), lse.data_ptr(), _t4(dout), _t4(dq), dkt, dvt, sgrad,
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()))
    return dq, dk_ring, dv_ring


def ring_bwd_noalloc(layout: str, world: int, rank: int, q_local, k_ring, v_ring, out, lse, dout, dq, dk_ring,
                     dv_ring, *, causal: bool = True, cu_seqlens=None, scale: Optional[float] = None):
    """ring_bwd for callers that cannot allocate: every buffer is the caller's, the
    library's scratch is its fixed per-GPU array (noalloc_scratch_bytes()).  dq is
    overwritten, dk_ring/dv_ring accumulated.  (cu_seqlens given as a device tensor is
    copied to the host here; pass a host array to keep the call free of copies.)"""
    b, L, h, d = q_local.shape
    cu = _Cu(cu_seqlens, q_local.device)
    p = _problem(q_local, h, d, L * world, causal, scale, cu)
    kt, srank = _t5(k_ring)
    vt, _ = _t5(v_ring)
    dkt, sgrad = _t5(dk_ring)
    dvt, sgrad_v = _t5(dv_ring)
    if sgrad != sgrad_v:
        raise ValueError("dk_ring and dv_ring must share the rank stride")
    check(lib().ra_ring_bwd_noalloc(C.byref(p), _layout_id(layout), world, rank, _t4(q_local), kt, vt, srank,
                                    _t4(out), lse.data_ptr(), _t4(dout), _t4(dq), dkt, dvt, sgrad, _stream()))
    return dq, dk_ring, dv_ring


def noalloc_scratch_bytes() -> int:
    return int(lib().ra_noalloc_scratch_bytes())


# ---- gathered K/V share (llama3-style) -----------------------------------------------------

def gathered_fwd(layout: str, world: int, rank: int, q_local, k_all, v_all, *, causal: bool = True,
                 cu_seqlens=None, scale: Optional[float] = None, out=None, lse=None, want_lowp: bool = False,
                 out_lowp=None):
    """Rank ``rank``'s share against the whole gathered K/V ([b, S, h, d], global order), one
    block step.  Returns (out fp32, lse fp32, out_lowp or None)."""
    torch = _torch()
    b, L, h, d = q_local.shape
    S = k_all.shape[1]
    if S != L * world:
        raise ValueError("k_all must hold world * local tokens")
    if out is None:
        out = torch.empty((b, L, h, d), device=q_local.device, dtype=torch.float32)
    if lse is None:
        lse = torch.empty((b, h, L), device=q_local.device, dtype=torch.float32)
    if want_lowp and out_lowp is None:
        out_lowp = torch.empty((b, L, h, d), device=q_local.device, dtype=q_local.dtype)
    cu = _Cu(cu_seqlens, q_local.device)
    p = _problem(q_local, h, d, S, causal, scale, cu)
    check(lib().ra_gathered_fwd(C.byref(p), _layout_id(layout), world, rank, _t4(q_local), _t4(k_all), _t4(v_all),
                                _t4(out), lse.data_ptr(), _t4(out_lowp), _stream()))
    return out, lse, out_lowp


def gathered_workspace_bytes(layout: str, world: int, rank: int, q_local, causal: bool = True,
                             minimal: bool = False, cu_seqlens=None) -> int:
    b, L, h, d = q_local.shape
    p = _problem(q_local, h, d, L * world, causal, None, _Cu(cu_seqlens, q_local.device))
    fn = lib().ra_gathered_workspace_min_bytes if minimal else lib().ra_gathered_workspace_bytes
    return int(fn(C.byref(p), _layout_id(layout), world, rank))


def gathered_bwd(layout: str, world: int, rank: int, q_local, k_all, v_all, out, lse, dout, *,
                 causal: bool = True, cu_seqlens=None, scale: Optional[float] = None, dq=None, dk_all=None,
                 dv_all=None, workspace=None, store_ds: bool = True):
    """Backward of gathered_fwd's share: dq overwritten, dk_all/dv_all (fp32, global order)
    accumulated (allocated zeroed when not given).  Returns (dq, dk_all, dv_all)."""
    torch = _torch()
    b, L, h, d = q_local.shape
    S = k_all.shape[1]
    dev = q_local.device
    if dq is None:
        dq = torch.empty((b, L, h, d), device=dev, dtype=torch.float32)
    if dk_all is None:
        dk_all = torch.zeros((b, S, h, d), device=dev, dtype=torch.float32)
    if dv_all is None:
        dv_all = torch.zeros((b, S, h, d), device=dev, dtype=torch.float32)
    cu = _Cu(cu_seqlens, dev)
    p = _problem(q_local, h, d, S, causal, scale, cu)
    fn = lib().ra_gathered_workspace_bytes if store_ds else lib().ra_gathered_workspace_min_bytes
    need = int(fn(C.byref(p), _layout_id(layout), world, rank))
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=dev, dtype=torch.uint8)
    check(lib().ra_gathered_bwd(C.byref(p), _layout_id(layout), world, rank, _t4(q_local), _t4(k_all), _t4(v_all),
                                _t4(out), lse.data_ptr(), _t4(dout), _t4(dq), _t4(dk_all), _t4(dv_all),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()))
    return dq, dk_all, dv_all


def cast_f32_to_bf16(x, out=None):
    """bf16 copy of a contiguous fp32 device tensor (round to nearest, ties to even)."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("expected a contiguous fp32 device tensor")
    if out is None:
        out = torch.empty(x.shape, device=x.device, dtype=torch.bfloat16)
    elif out.dtype != torch.bfloat16 or not out.is_contiguous() or out.numel() != x.numel():
        raise ValueError("out must be a contiguous bf16 tensor of the same size")
    check(lib().ra_cast_f32_to_bf16(x.data_ptr(), out.data_ptr(), x.numel(), _stream()))
    return out


# ---- kernel timing -------------------------------------------------------------------------

class KernelTimes:
    def __init__(self):
        self.launches: List[Tuple[str, int, float]] = []

    def by_kernel(self):
        agg = {}
        for name, _, ms in self.launches:
            n, t = agg.get(name, (0, 0.0))
            agg[name] = (n + 1, t + ms)
        return agg


@contextmanager
def kernel_timing(capacity: int = 4096):
    """Record HIP events around every library kernel launched inside the block."""
    res = KernelTimes()
    check(lib().ra_timing_begin(capacity))
    try:
        yield res
    finally:
        buf = (_lib.ra_launch_time * capacity)()
        n = C.c_int32(0)
        check(lib().ra_timing_end(buf, capacity, C.byref(n)))
        for i in range(n.value):
            res.launches.append((lib().ra_kernel_name(buf[i].kernel_id).decode(), buf[i].step, buf[i].ms))
