"""Torch-facing helpers over the C ABI: allocate device buffers with torch, pass their
addresses and the current stream to libtcq.  No arithmetic happens here."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib


def nwords(k: int, T: int) -> int:
    return (k * T + 31) // 32


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class Encoded:
    bitstream: torch.Tensor    # uint32 [blocks, nwords] (stored as int32)
    start_state: torch.Tensor  # uint32 [blocks] (stored as int32)
    cost: torch.Tensor         # float32 [blocks]
    recon: torch.Tensor | None  # float32 [M, N]


class Workspace:
    """Device workspace owned by torch's allocator."""

    def __init__(self, nbytes: int, device="cuda"):
        self.nbytes = int(nbytes)
        self.buf = torch.empty(max(self.nbytes, 1), dtype=torch.uint8, device=device)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()


def make_codebook(L: int, V: int, seed: int, device="cuda") -> torch.Tensor:
    host = _lib.tcq_make_codebook(L, V, seed)
    return torch.from_numpy(host).to(device)


def encode(W: torch.Tensor, d: torch.Tensor | None, codebook: torch.Tensor, L: int, k: int,
           V: int, T: int, recon: bool = False, workspace: Workspace | None = None,
           out: Encoded | None = None) -> Encoded:
    assert W.is_cuda and W.dtype == torch.float32 and W.dim() == 2 and W.stride(1) == 1
    M, N = W.shape
    assert codebook.is_cuda and codebook.dtype == torch.float32 and codebook.is_contiguous()
    if d is not None:
        assert d.is_cuda and d.dtype == torch.float32 and d.is_contiguous() and d.numel() == N
    nb = M * (N // T) if T > 0 else 0
    if out is None:
        dev = W.device
        out = Encoded(
            bitstream=torch.empty((nb, nwords(k, T)), dtype=torch.int32, device=dev),
            start_state=torch.empty(nb, dtype=torch.int32, device=dev),
            cost=torch.empty(nb, dtype=torch.float32, device=dev),
            recon=torch.empty((M, N), dtype=torch.float32, device=dev) if recon else None)
    if workspace is None:
        workspace = Workspace(_lib.tcq_encode_workspace_bytes(M, N, L, k, V, T), W.device)
    _lib.tcq_encode(W.data_ptr(), M, N, W.stride(0), None if d is None else d.data_ptr(),
                    codebook.data_ptr(), L, k, V, T, out.bitstream.data_ptr(),
                    out.start_state.data_ptr(), out.cost.data_ptr(),
                    None if out.recon is None else out.recon.data_ptr(),
                    N if out.recon is None else out.recon.stride(0), workspace.ptr,
                    workspace.nbytes, _stream())
    return out


def decode(bitstream: torch.Tensor, start_state: torch.Tensor, codebook: torch.Tensor, M: int,
           N: int, L: int, k: int, V: int, T: int) -> torch.Tensor:
    out = torch.empty((M, N), dtype=torch.float32, device=bitstream.device)
    _lib.tcq_decode(bitstream.data_ptr(), start_state.data_ptr(), codebook.data_ptr(), M, N,
                    L, k, V, T, out.data_ptr(), N, _stream())
    return out


def decode_gemv(bitstream: torch.Tensor, start_state: torch.Tensor, codebook: torch.Tensor,
                x: torch.Tensor, M: int, N: int, L: int, k: int, V: int, T: int) -> torch.Tensor:
    assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.numel() == N
    y = torch.empty(M, dtype=torch.float32, device=x.device)
    _lib.tcq_decode_gemv(bitstream.data_ptr(), start_state.data_ptr(), codebook.data_ptr(), M,
                         N, L, k, V, T, x.data_ptr(), y.data_ptr(), _stream())
    return y


@dataclass
class EncodedLdlq(Encoded):
    target: torch.Tensor | None = None  # float32 [M, N]


def encode_ldlq(W: torch.Tensor, U: torch.Tensor | None, d: torch.Tensor | None,
                codebook: torch.Tensor, L: int, k: int, V: int, T: int, recon: bool = True,
                target: bool = False, workspace: Workspace | None = None) -> EncodedLdlq:
    assert W.is_cuda and W.dtype == torch.float32 and W.dim() == 2 and W.stride(1) == 1
    M, N = W.shape
    if U is not None:
        assert U.is_cuda and U.dtype == torch.float32 and U.dim() == 2 and U.stride(1) == 1
    if d is not None:
        assert d.is_cuda and d.dtype == torch.float32 and d.is_contiguous() and d.numel() == N
    nb = M * (N // T)
    dev = W.device
    out = EncodedLdlq(
        bitstream=torch.empty((nb, nwords(k, T)), dtype=torch.int32, device=dev),
        start_state=torch.empty(nb, dtype=torch.int32, device=dev),
        cost=torch.empty(nb, dtype=torch.float32, device=dev),
        recon=torch.empty((M, N), dtype=torch.float32, device=dev) if recon else None,
        target=torch.empty((M, N), dtype=torch.float32, device=dev) if target else None)
    if workspace is None:
        workspace = Workspace(_lib.tcq_ldlq_workspace_bytes(M, N, L, k, V, T), dev)
    _lib.tcq_encode_ldlq(W.data_ptr(), M, N, W.stride(0),
                         None if U is None else U.data_ptr(), N if U is None else U.stride(0),
                         None if d is None else d.data_ptr(), codebook.data_ptr(), L, k, V, T,
                         out.bitstream.data_ptr(), out.start_state.data_ptr(),
                         out.cost.data_ptr(), None if out.recon is None else out.recon.data_ptr(),
                         N, None if out.target is None else out.target.data_ptr(), N,
                         workspace.ptr, workspace.nbytes, _stream())
    return out


def bcjr(W: torch.Tensor, d: torch.Tensor | None, codebook: torch.Tensor, L: int, k: int,
         V: int, T: int, tau: float, workspace: Workspace | None = None
         ) -> tuple[torch.Tensor, torch.Tensor]:
    """Soft codewords (float32 [M, N]) and log Z per block (float32 [M*N/T])."""
    assert W.is_cuda and W.dtype == torch.float32 and W.dim() == 2 and W.stride(1) == 1
    M, N = W.shape
    if d is not None:
        assert d.is_cuda and d.dtype == torch.float32 and d.is_contiguous() and d.numel() == N
    soft = torch.empty((M, N), dtype=torch.float32, device=W.device)
    logz = torch.empty(M * (N // T), dtype=torch.float32, device=W.device)
    if workspace is None:
        workspace = Workspace(_lib.tcq_bcjr_workspace_bytes(M, N, L, k, V, T), W.device)
    _lib.tcq_bcjr(W.data_ptr(), M, N, W.stride(0), None if d is None else d.data_ptr(),
                  codebook.data_ptr(), L, k, V, T, float(tau), soft.data_ptr(), N,
                  logz.data_ptr(), workspace.ptr, workspace.nbytes, _stream())
    return soft, logz


def hadamard(X: torch.Tensor, n: int, sigma: torch.Tensor | None = None, inverse: bool = False,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows of X rotated by R = H_n diag(sigma)/sqrt(n) in chunks of n (inverse: R^T)."""
    assert X.is_cuda and X.dtype == torch.float32 and X.dim() == 2 and X.stride(1) == 1
    rows, length = X.shape
    if sigma is not None:
        assert sigma.is_cuda and sigma.dtype == torch.float32 and sigma.is_contiguous()
    if out is None:
        out = torch.empty_like(X)
    _lib.tcq_hadamard(X.data_ptr(), rows, length, X.stride(0), n,
                      None if sigma is None else sigma.data_ptr(), inverse, out.data_ptr(),
                      out.stride(0), _stream())
    return out


def scale_field(W: torch.Tensor, normalized: bool = True
                ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor | None]:
    """(row_scale [M], col_scale [N], Wn [M, N] or None) with W = a_r b_c Wn_rc."""
    assert W.is_cuda and W.dtype == torch.float32 and W.dim() == 2 and W.stride(1) == 1
    M, N = W.shape
    a = torch.empty(M, dtype=torch.float32, device=W.device)
    b = torch.empty(N, dtype=torch.float32, device=W.device)
    Wn = torch.empty_like(W) if normalized else None
    ws = Workspace(_lib.tcq_scale_field_workspace_bytes(M, N), W.device)
    _lib.tcq_scale_field(W.data_ptr(), M, N, W.stride(0), a.data_ptr(), b.data_ptr(),
                         None if Wn is None else Wn.data_ptr(), N, ws.ptr, ws.nbytes, _stream())
    return a, b, Wn
