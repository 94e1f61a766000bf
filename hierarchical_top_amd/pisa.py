"""Python binding of libpisa (include/pisa.h): argument marshalling only.

Every step of the selection path runs in the library's HIP kernels; this module
turns torch tensors into pointers, sizes and the current HIP stream, and turns
negative status codes into exceptions. There is no fallback: if libpisa.so is
missing or no GPU is present, the calls raise.

Method: "Block Sparse Attention with Log-Linear Complexity" (PISA); the
library header cites the sections each call implements.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libpisa.so"
MAX_LEVELS = 32
F32, BF16 = 0, 1
TWO_STAGE, FUSED, LEVELS = 0, 1, 2
# size of the library-owned workspace of pisa_route_prefill_noalloc (PISA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
# block scores (pisa_score_kind): PISA's LSE, PISA-1 (mean), PISA-2 (mean + var / 2)
SCORE_KINDS = {"lse": 0, "mean": 1, "mean_var": 2}

c_i32, c_i64, c_p, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


class PisaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("libpisa status %d: %s" % (status, msg))
        self.status = status


class _PyramidDesc(ctypes.Structure):
    _fields_ = [
        ("B", c_i32), ("H_kv", c_i32), ("d", c_i32), ("C", c_i32), ("g", c_i32), ("L_cap", c_i32),
        ("N_cap", c_i64),
        ("M_cap", c_i64 * (MAX_LEVELS + 1)),
        ("off", c_i64 * (MAX_LEVELS + 1)),
        ("floats", c_i64),
        ("buf", c_p),
    ]


_lib = None


def lib():
    """Load libpisa.so (built by hierarchical_top_amd.build or __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError("libpisa.so is not built (run: python -m hierarchical_top_amd.build)")
        L = ctypes.CDLL(str(LIB_PATH))
        P = ctypes.POINTER(_PyramidDesc)
        sig = {
            "pisa_pyramid_plan": [P, c_i32, c_i32, c_i32, c_i32, c_i32, c_i64],
            "pisa_build_pyramid": [P, c_p, c_i32, c_i64, c_p],
            "pisa_pyramid_append": [P, c_p, c_i32, c_p, c_p],
            "pisa_route_prefill_workspace": [P, c_i64, c_i32, c_i32, c_i32, ctypes.POINTER(c_size)],
            "pisa_route_prefill": [P, c_p, c_p, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p,
                                   c_size, c_p],
            "pisa_route_prefill_scored": [P, c_p, c_p, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_p,
                                          c_p, c_p, c_size, c_p],
            "pisa_route_prefill_noalloc": [P, c_p, c_p, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p],
            "pisa_route_decode": [P, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_p, c_p, c_p],
            "pisa_route_decode_scored": [P, c_p, c_p, c_i32, c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p],
            "pisa_sparse_attn": [c_p, c_p, c_p, c_i32, c_i32, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_p,
                                 c_i32, c_i32, c_p, c_p, c_p, c_p],
            "pisa_sparse_attn_workspace": [c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32,
                                           ctypes.POINTER(c_size)],
            "pisa_sparse_attn_clustered": [c_p, c_p, c_p, c_i32, c_i32, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32,
                                           c_i32, c_p, c_i32, c_i32, c_p, c_p, c_p, c_p, c_size, c_p],
            "pisa_sparse_attn_bwd_workspace": [c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32,
                                               ctypes.POINTER(c_size)],
            "pisa_sparse_attn_bwd": [c_p, c_p, c_p, c_p, c_p, c_p, c_i32, c_i32, c_i64, c_i64, c_i64, c_i32, c_i32,
                                     c_i32, c_i32, c_p, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_size, c_p],
            "pisa_selection_quality_workspace": [c_i32, c_i64, c_i32, c_i32, ctypes.POINTER(c_size)],
            "pisa_selection_quality": [c_p, c_p, c_i32, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_p, c_i32, c_p,
                                       c_p, c_p, c_p, c_p, c_p, c_size, c_p],
            "pisa_bsa_select": [P, c_p, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p],
            "pisa_time_stage": [c_i32, c_p, c_p],
            "pisa_time_stage_pending": [c_i32],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.pisa_status_str.argtypes = [ctypes.c_int]
        L.pisa_status_str.restype = ctypes.c_char_p
        L.pisa_last_error.argtypes = []
        L.pisa_last_error.restype = ctypes.c_char_p
        L.pisa_abi_version.argtypes = []
        L.pisa_abi_version.restype = c_i32
        _lib = L
    return _lib


EXPORTS = ["pisa_pyramid_plan", "pisa_build_pyramid", "pisa_pyramid_append", "pisa_route_prefill_workspace",
           "pisa_route_prefill", "pisa_route_prefill_scored", "pisa_route_prefill_noalloc", "pisa_route_decode",
           "pisa_route_decode_scored", "pisa_sparse_attn", "pisa_sparse_attn_workspace",
           "pisa_sparse_attn_clustered", "pisa_sparse_attn_bwd_workspace", "pisa_sparse_attn_bwd",
           "pisa_selection_quality_workspace", "pisa_selection_quality", "pisa_bsa_select", "pisa_time_stage",
           "pisa_time_stage_pending",
           "pisa_status_str", "pisa_last_error", "pisa_abi_version"]

# Stage ids of pisa_time_stage (include/pisa.h, enum pisa_stage).
STAGES = {"build": 0, "append": 1, "route_fused": 2, "route_decode": 3, "upper": 4, "cluster": 5, "leaf": 6,
          "final": 7, "attn": 8, "bsa": 9, "attn_bwd": 10}


def _check(status: int):
    if status != 0:
        raise PisaError(status, lib().pisa_last_error().decode())


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise TypeError("libpisa takes float32 or bfloat16 tensors, got %s" % x.dtype)


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _dev(*xs):
    for x in xs:
        if x is not None and (not x.is_cuda or not x.is_contiguous()):
            raise ValueError("libpisa takes contiguous GPU tensors")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Pyramid:
    """Mean-pooled key pyramid for B sequences of up to N_cap tokens.

    Owns its float32 summary buffer (a torch tensor on `device`).
    """

    def __init__(self, B: int, H_kv: int, d: int, C: int, g: int, N_cap: int, device="cuda"):
        self.desc = _PyramidDesc()
        _check(lib().pisa_pyramid_plan(ctypes.byref(self.desc), B, H_kv, d, C, g, N_cap))
        self.buf = torch.empty(max(int(self.desc.floats), 1), dtype=torch.float32, device=device)
        self.desc.buf = self.buf.data_ptr()
        self.B, self.H_kv, self.d, self.C, self.g, self.N_cap = B, H_kv, d, C, g, N_cap

    @property
    def L_cap(self) -> int:
        return int(self.desc.L_cap)

    def level(self, l: int) -> torch.Tensor:
        """Level-l storage [B][H_kv][M_cap[l]][d] (a view of the buffer)."""
        o, M = int(self.desc.off[l]), int(self.desc.M_cap[l])
        n = self.B * self.H_kv * M * self.d
        return self.buf[o:o + n].view(self.B, self.H_kv, M, self.d)

    def build(self, K: torch.Tensor, N: int):
        """Build levels 1..L(N) from K [B][N_cap][H_kv][d]."""
        _dev(K)
        _check(lib().pisa_build_pyramid(ctypes.byref(self.desc), _ptr(K), _dt(K), N, _stream()))

    def append(self, K: torch.Tensor, seqlen: torch.Tensor):
        """Update the path of the newest token of each sequence (seqlen: int64 [B])."""
        _dev(K, seqlen)
        assert seqlen.dtype == torch.int64
        _check(lib().pisa_pyramid_append(ctypes.byref(self.desc), _ptr(K), _dt(K), _ptr(seqlen), _stream()))


def route_workspace_bytes(pyr: Pyramid, N: int, H_q: int, K_top: int, mode: int = TWO_STAGE) -> int:
    n = c_size(0)
    _check(lib().pisa_route_prefill_workspace(ctypes.byref(pyr.desc), N, H_q, K_top, mode, ctypes.byref(n)))
    return int(n.value)


def route_prefill(pyr: Pyramid, Q: torch.Tensor, K: torch.Tensor, N: int, K_top: int, causal: bool = True,
                  mode: int = TWO_STAGE, with_score: bool = False, workspace: torch.Tensor | None = None,
                  out: torch.Tensor | None = None, score_out: torch.Tensor | None = None,
                  score_kind: str = "lse"):
    """Route every position of Q [B][N][H_q][d]; returns idx [B][H_kv][N][K_top] (and scores).

    score_kind: "lse" (PISA), "mean" (PISA-1) or "mean_var" (PISA-2); the last two
    run on the level-synchronous and fused routers."""
    _dev(Q, K)
    B, Nq, H_q, d = Q.shape
    assert Nq == N and K.dtype == Q.dtype
    idx = out if out is not None else torch.empty(B, pyr.H_kv, N, K_top, dtype=torch.int32, device=Q.device)
    score = None
    if with_score:
        score = score_out if score_out is not None else torch.empty(B, pyr.H_kv, N, K_top, dtype=torch.float32,
                                                                    device=Q.device)
    need = route_workspace_bytes(pyr, N, H_q, K_top, mode)
    ws = workspace
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    _check(lib().pisa_route_prefill_scored(ctypes.byref(pyr.desc), _ptr(Q), _ptr(K), _dt(Q), N, H_q, K_top,
                                           1 if causal else 0, H_q // pyr.H_kv, mode, SCORE_KINDS[score_kind],
                                           _ptr(idx), _ptr(score), _ptr(ws) if need else None, need, _stream()))
    return (idx, score) if with_score else idx


def route_prefill_noalloc(pyr: Pyramid, Q: torch.Tensor, K: torch.Tensor, N: int, K_top: int, causal: bool = True,
                          out: torch.Tensor | None = None, score_out: torch.Tensor | None = None):
    """route_prefill with the level-synchronous router and the library's own scratch array as
    its workspace (pisa_route_prefill_noalloc): returns (idx, score) [B][H_kv][N][K_top]. Only
    the outputs are allocated here, and not at all when out / score_out are given."""
    _dev(Q, K)
    B, Nq, H_q, d = Q.shape
    assert Nq == N and K.dtype == Q.dtype
    idx = out if out is not None else torch.empty(B, pyr.H_kv, N, K_top, dtype=torch.int32, device=Q.device)
    score = score_out if score_out is not None else torch.empty(B, pyr.H_kv, N, K_top, dtype=torch.float32,
                                                                device=Q.device)
    _check(lib().pisa_route_prefill_noalloc(ctypes.byref(pyr.desc), _ptr(Q), _ptr(K), _dt(Q), N, H_q, K_top,
                                            1 if causal else 0, H_q // pyr.H_kv, _ptr(idx), _ptr(score), _stream()))
    return idx, score


def route_decode(pyr: Pyramid, q: torch.Tensor, K: torch.Tensor, seqlen: torch.Tensor, K_top: int,
                 with_score: bool = False, out: torch.Tensor | None = None, score_out: torch.Tensor | None = None,
                 score_kind: str = "lse"):
    """Route the newest token of each sequence: q [B][H_q][d]; returns idx [B][H_kv][K_top].
    score_kind: "lse" (PISA), "mean" (PISA-1) or "mean_var" (PISA-2)."""
    _dev(q, K, seqlen)
    B, H_q, d = q.shape
    idx = out if out is not None else torch.empty(B, pyr.H_kv, K_top, dtype=torch.int32, device=q.device)
    score = None
    if with_score:
        score = score_out if score_out is not None else torch.empty(B, pyr.H_kv, K_top, dtype=torch.float32,
                                                                    device=q.device)
    _check(lib().pisa_route_decode_scored(ctypes.byref(pyr.desc), _ptr(q), _ptr(K), _dt(q), _ptr(seqlen), H_q, K_top,
                                          H_q // pyr.H_kv, SCORE_KINDS[score_kind], _ptr(idx), _ptr(score),
                                          _stream()))
    return (idx, score) if with_score else idx


def sparse_attn(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, block_idx: torch.Tensor, C: int, N_kv: int,
                causal: bool = True, kv_len: torch.Tensor | None = None, with_lse: bool = False,
                out: torch.Tensor | None = None):
    """Block-sparse attention: Q [B][N_q][H_q][d], K/V [B][N_alloc][H_kv][d], block_idx [B][H_kv][N_q][K_top]."""
    _dev(Q, K, V, block_idx, kv_len)
    B, N_q, H_q, d = Q.shape
    N_alloc, H_kv = K.shape[1], K.shape[2]
    K_top = block_idx.shape[-1]
    O = out if out is not None else torch.empty_like(Q)
    lse = torch.empty(B, H_q, N_q, dtype=torch.float32, device=Q.device) if with_lse else None
    _check(lib().pisa_sparse_attn(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, N_q, N_kv, N_alloc, H_q, H_kv, d, C,
                                  _ptr(block_idx), K_top, 1 if causal else 0, _ptr(kv_len), _ptr(O), _ptr(lse),
                                  _stream()))
    return (O, lse) if with_lse else O


def sparse_attn_workspace_bytes(B: int, N_q: int, N_alloc: int, H_q: int, H_kv: int, d: int, C: int,
                                K_top: int) -> int:
    n = c_size(0)
    _check(lib().pisa_sparse_attn_workspace(B, N_q, N_alloc, H_q, H_kv, d, C, K_top, ctypes.byref(n)))
    return int(n.value)


def sparse_attn_clustered(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, block_idx: torch.Tensor, C: int,
                          N_kv: int, causal: bool = True, kv_len: torch.Tensor | None = None, with_lse: bool = False,
                          workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Block-sparse attention clustered by selected block (bf16); same results as sparse_attn."""
    _dev(Q, K, V, block_idx, kv_len)
    B, N_q, H_q, d = Q.shape
    N_alloc, H_kv = K.shape[1], K.shape[2]
    K_top = block_idx.shape[-1]
    need = sparse_attn_workspace_bytes(B, N_q, N_alloc, H_q, H_kv, d, C, K_top)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=Q.device)
    O = out if out is not None else torch.empty_like(Q)
    lse = torch.empty(B, H_q, N_q, dtype=torch.float32, device=Q.device) if with_lse else None
    _check(lib().pisa_sparse_attn_clustered(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, N_q, N_kv, N_alloc, H_q, H_kv, d,
                                            C, _ptr(block_idx), K_top, 1 if causal else 0, _ptr(kv_len), _ptr(O),
                                            _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return (O, lse) if with_lse else O


def sparse_attn_bwd_workspace_bytes(B: int, N_q: int, N_alloc: int, H_q: int, H_kv: int, d: int, C: int,
                                    K_top: int) -> int:
    n = c_size(0)
    _check(lib().pisa_sparse_attn_bwd_workspace(B, N_q, N_alloc, H_q, H_kv, d, C, K_top, ctypes.byref(n)))
    return int(n.value)


def sparse_attn_bwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor, dO: torch.Tensor,
                    lse: torch.Tensor, block_idx: torch.Tensor, C: int, N_kv: int, causal: bool = True,
                    kv_len: torch.Tensor | None = None, workspace: torch.Tensor | None = None, out=None):
    """Gradients of block-sparse attention (bf16 inputs): returns fp32 (dQ, dK, dV) shaped like Q, K, V.

    O and lse are the forward's output and log-normaliser [B][H_q][N_q]; out = (dQ, dK, dV) to reuse."""
    _dev(Q, K, V, O, dO, lse, block_idx, kv_len)
    B, N_q, H_q, d = Q.shape
    N_alloc, H_kv = K.shape[1], K.shape[2]
    K_top = block_idx.shape[-1]
    assert O.shape == Q.shape and dO.shape == Q.shape and lse.dtype == torch.float32
    need = sparse_attn_bwd_workspace_bytes(B, N_q, N_alloc, H_q, H_kv, d, C, K_top)
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        torch.empty(need, dtype=torch.uint8, device=Q.device)
    if out is None:
        out = (torch.empty(Q.shape, dtype=torch.float32, device=Q.device),
               torch.empty(K.shape, dtype=torch.float32, device=Q.device),
               torch.empty(V.shape, dtype=torch.float32, device=Q.device))
    dQ, dK, dV = out
    _check(lib().pisa_sparse_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(lse), _dt(Q), B, N_q, N_kv,
                                      N_alloc, H_q, H_kv, d, C, _ptr(block_idx), K_top, 1 if causal else 0,
                                      _ptr(kv_len), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream()))
    return dQ, dK, dV


def selection_quality(Q: torch.Tensor, K: torch.Tensor, sel: torch.Tensor, C: int, with_mass: bool = False,
                      with_ref: bool = False):
    """Quality of the causal selection sel [B][H_kv][N][K_top] against full attention (bf16 Q, K):
    returns dict(recall, captured, ratio [B][H_kv][N] fp32, mass [B][H_kv][N][M1] and ref
    [B][H_kv][N][K_top] when asked)."""
    _dev(Q, K, sel)
    B, N, H_q, d = Q.shape
    H_kv = K.shape[2]
    K_top = sel.shape[-1]
    M1 = -(-N // C)
    n = c_size(0)
    _check(lib().pisa_selection_quality_workspace(B, N, H_q, C, ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=Q.device)
    f = dict(device=Q.device, dtype=torch.float32)
    out = {k: torch.empty(B, H_kv, N, **f) for k in ("recall", "captured", "ratio")}
    out["mass"] = torch.empty(B, H_kv, N, M1, **f) if with_mass else None
    out["ref"] = torch.empty(B, H_kv, N, K_top, dtype=torch.int32, device=Q.device) if with_ref else None
    _check(lib().pisa_selection_quality(_ptr(Q), _ptr(K), _dt(Q), B, N, H_q, H_kv, d, C, _ptr(sel), K_top,
                                        _ptr(out["mass"]), _ptr(out["ref"]), _ptr(out["recall"]),
                                        _ptr(out["captured"]), _ptr(out["ratio"]), _ptr(ws), ws.numel(), _stream()))
    return out


def bsa_select(pyr: Pyramid, Q: torch.Tensor, N: int, K_top: int, causal: bool = True, with_score: bool = False,
               out: torch.Tensor | None = None, score_out: torch.Tensor | None = None):
    """Exhaustive single-level selection (comparison point); returns idx [B][H_kv][N][K_top]."""
    _dev(Q)
    B, Nq, H_q, d = Q.shape
    idx = out if out is not None else torch.empty(B, pyr.H_kv, N, K_top, dtype=torch.int32, device=Q.device)
    score = None
    if with_score:
        score = score_out if score_out is not None else torch.empty(B, pyr.H_kv, N, K_top, dtype=torch.float32,
                                                                    device=Q.device)
    _check(lib().pisa_bsa_select(ctypes.byref(pyr.desc), _ptr(Q), _dt(Q), N, H_q, K_top, 1 if causal else 0,
                                 H_q // pyr.H_kv, _ptr(idx), _ptr(score), _stream()))
    return (idx, score) if with_score else idx


def time_stage(stage: str, start: "torch.cuda.Event", stop: "torch.cuda.Event"):
    """Arm a pair of timing events for the next call (on this thread) that runs `stage`.

    The events must already exist as HIP events (record them once beforehand);
    afterwards ``start.elapsed_time(stop)`` is the stage's duration on its stream.
    """
    for ev in (start, stop):
        if not ev.cuda_event:
            raise ValueError("record the event once before arming it")
    _check(lib().pisa_time_stage(STAGES[stage], ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)))


def time_stage_pending(stage: str) -> int:
    """Armed event pairs of `stage` not consumed yet on this thread."""
    return int(lib().pisa_time_stage_pending(STAGES[stage]))


def time_stage_clear(stage: str):
    _check(lib().pisa_time_stage(STAGES[stage], None, None))
