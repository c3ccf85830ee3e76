"""Python binding of librlk.so, the fused deterministic selected-token
log-probability operator ("linear_logp") for MI355X / gfx950.

Only argument marshalling lives here: every step of the computation runs in
the HIP kernels behind the C ABI of ``include/rlk.h``.  PyTorch supplies
device memory, streams and autograd plumbing.  There is no fallback: if the
library is missing or the device is not gfx950, calls raise.

    logp = linear_logp(h, W, y)            # autograd-aware
    logp, lse = linear_logp_fwd(h, W, y)
    grad_h, grad_W = linear_logp_bwd(h, W, y, lse, g)
    part = lse_partial(h, W_shard, y, vocab_start, V_global)   # [T, 4] records
    logp, lse = lse_merge(torch.stack(parts), y)
    C = gemm_bf16_nt(A, B)                  # deterministic A @ B^T
    logp, lse, z = linear_logp_fwd_save(h, W, y)          # save-logits variant
    logp, lse, loss, g = linear_logp_fwd_rl(h, W, y, logp_old, adv)  # + RL objective
    grad_h, grad_W = linear_logp_bwd_saved(h, W, y, lse, g, z)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "IGNORE_INDEX", "RlkError", "lib", "library_path", "contract_version",
    "workspace_bytes", "linear_logp_fwd", "linear_logp_bwd", "lse_partial",
    "lse_merge", "linear_logp", "gemm_bf16_nt", "linear_logp_fwd_save", "linear_logp_bwd_saved",
    "saved_logits_ld", "rl_token_loss", "profile_begin", "profile_end",
    "linear_logp_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "linear_logp_fwd_rl",
]

IGNORE_INDEX = -100
OP_FWD, OP_BWD, OP_PARTIAL = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "librlk.so")

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_size = ctypes.c_size_t

_SIGNATURES = {
    "rlk_contract_version": (_i32, []),
    "rlk_status_string": (ctypes.c_char_p, [_i32]),
    "rlk_last_error_message": (ctypes.c_char_p, []),
    "rlk_workspace_bytes": (_size, [_i32, _i64, _i64, _i64]),
    "rlk_linear_logp_fwd": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i32,
                                   _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "rlk_linear_logp_bwd": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _i64, _i64, _i64, _i32, _c_void_p, _c_void_p,
                                   _c_void_p, _size, _c_void_p]),
    "rlk_lse_partial": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _i64,
                               _i32, _c_void_p, _c_void_p, _size, _c_void_p]),
    "rlk_lse_merge": (_i32, [_c_void_p, _i32, _c_void_p, _i64, _i32, _c_void_p, _c_void_p,
                             _c_void_p]),
    "rlk_gemm_bf16_nt": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _i32,
                                _c_void_p]),
    "rlk_saved_logits_ld": (_i64, [_i64]),
    "rlk_linear_logp_fwd_save": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i32,
                                        _c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _size,
                                        _c_void_p]),
    "rlk_linear_logp_bwd_saved": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_void_p, _i64, _i64, _i64, _i64, _i32, _c_void_p,
                                         _c_void_p, _c_void_p, _size, _c_void_p]),
    "rlk_rl_token_loss": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
                                 ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                 _c_void_p, _c_void_p, _c_void_p]),
    "rlk_linear_logp_fwd_noalloc": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i32,
                                           _c_void_p, _c_void_p, _c_void_p]),
    "rlk_linear_logp_fwd_rl": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i32,
                                      _c_void_p, _c_void_p, _c_void_p,
                                      ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                      _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size,
                                      _c_void_p]),
    # benchmark helpers (include/rlk_bench.h)
    "rlk_bench_mfma_ceiling": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _c_void_p]),
    "rlk_profile_begin": (_i32, []),
    "rlk_profile_end": (_i32, [_c_void_p, _i32, ctypes.POINTER(_i32)]),
}


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]

_LIB = None


class RlkError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        msg = L.rlk_status_string(status).decode()
        detail = L.rlk_last_error_message().decode()
        super().__init__(f"{where}: status {status} ({msg}){': ' + detail if detail else ''}")
        self.status = status


def lib():
    """The loaded librlk.so (ctypes), with argument types declared."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run `python -m selected_token_lm_amd.build`")
        L = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def contract_version() -> int:
    return int(lib().rlk_contract_version())


def workspace_bytes(op: int, T: int, H: int, V: int) -> int:
    return int(lib().rlk_workspace_bytes(op, T, H, V))


def _check(status: int, where: str):
    if status != 0:
        raise RlkError(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _prep(h, W, y):
    """Shapes and dtypes first, then the device, so that a malformed call
    fails in Python before any kernel can read past a short tensor."""
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("h and W must be bfloat16")
    if h.dim() != 2 or W.dim() != 2 or h.shape[1] != W.shape[1]:
        raise ValueError("h must be [T, H] and W [V, H]")
    if y.dim() != 1 or y.shape[0] != h.shape[0]:
        raise ValueError(f"y must be [T] = [{h.shape[0]}], got {list(y.shape)}")
    if y.dtype not in (torch.int32, torch.int64):
        raise TypeError("y must hold int32 or int64 target ids")
    if not (h.is_cuda and W.is_cuda and y.is_cuda):
        raise ValueError("h, W and y must be device tensors")
    if W.device != h.device or y.device != h.device:
        raise ValueError("h, W and y must be on one device")
    y = y.to(torch.int32) if y.dtype != torch.int32 else y
    return h.contiguous(), W.contiguous(), y.contiguous()


def _rows(T, device, **named):
    """Per-row tensors: each 1-D of length T (checked for all of them first),
    then each on `device`; returned contiguous, int32 for `y`, else float32.
    The kernels read element t for every row t < T, so a shorter tensor would
    be read out of bounds on the device."""
    for name, t in named.items():
        if t is None:
            raise ValueError(f"{name} is required")
        if t.dim() != 1 or t.shape[0] != T:
            raise ValueError(f"{name} must be 1-D of length T = {T}, got shape {list(t.shape)}")
    for name, t in named.items():
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be on {device}")
    return [t.to(torch.int32 if name == "y" else torch.float32).contiguous() for name, t in named.items()]


def _workspace(op, T, H, V, device):
    n = workspace_bytes(op, T, H, V)
    if n == 0:
        raise ValueError(f"invalid shape T={T} H={H} V={V}")
    return torch.empty(n, dtype=torch.uint8, device=device), n


def _given_workspace(ws, device):
    """A caller's workspace: a contiguous byte tensor on `device` (the
    library checks its size against rlk_workspace_bytes)."""
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"ws must be a contiguous uint8 tensor on {device}")
    return ws, ws.numel()


def linear_logp_fwd(h, W, y, ignore_index: int = IGNORE_INDEX, ws=None):
    """Selected-token log-probabilities and log-sum-exp, fp32 [T] each."""
    h, W, y = _prep(h, W, y)
    T, H = h.shape
    V = W.shape[0]
    logp = torch.empty(T, dtype=torch.float32, device=h.device)
    lse = torch.empty(T, dtype=torch.float32, device=h.device)
    if ws is None:
        ws, n = _workspace(OP_FWD, T, H, V, h.device)
    else:
        ws, n = _given_workspace(ws, h.device)
    _check(lib().rlk_linear_logp_fwd(_ptr(h), _ptr(W), _ptr(y), T, H, V, ignore_index,
                                     _ptr(logp), _ptr(lse), _ptr(ws), n, _stream()),
           "rlk_linear_logp_fwd")
    return logp, lse


# Size of the library's fixed device scratch (RLK_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def linear_logp_fwd_noalloc(h, W, y, ignore_index: int = IGNORE_INDEX, logp=None, lse=None):
    """linear_logp_fwd without a workspace: the library's fixed device scratch
    serves instead (nothing is allocated when logp and lse are given).  Calls
    on one GPU share that scratch and must not overlap."""
    h, W, y = _prep(h, W, y)
    T, H = h.shape
    V = W.shape[0]
    if logp is None:
        logp = torch.empty(T, dtype=torch.float32, device=h.device)
    if lse is None:
        lse = torch.empty(T, dtype=torch.float32, device=h.device)
    for name, t in (("logp", logp), ("lse", lse)):
        if t.dtype != torch.float32 or t.shape != (T,) or not t.is_contiguous() or t.device != h.device:
            raise ValueError(f"{name} must be a contiguous float32 [T] tensor on {h.device}")
    _check(lib().rlk_linear_logp_fwd_noalloc(_ptr(h), _ptr(W), _ptr(y), T, H, V, ignore_index,
                                             _ptr(logp), _ptr(lse), _stream()),
           "rlk_linear_logp_fwd_noalloc")
    return logp, lse


def linear_logp_bwd(h, W, y, lse, g, ignore_index: int = IGNORE_INDEX,
                    need_grad_h: bool = True, need_grad_W: bool = True, ws=None):
    """(grad_h bf16 [T,H] or None, grad_W fp32 [V,H] or None) of sum_t g_t logp_t."""
    h, W, y = _prep(h, W, y)
    T, H = h.shape
    V = W.shape[0]
    lse, g = _rows(T, h.device, lse=lse, g=g)
    grad_h = torch.empty((T, H), dtype=torch.bfloat16, device=h.device) if need_grad_h else None
    grad_W = torch.empty((V, H), dtype=torch.float32, device=h.device) if need_grad_W else None
    if ws is None:
        ws, n = _workspace(OP_BWD, T, H, V, h.device)
    else:
        ws, n = _given_workspace(ws, h.device)
    _check(lib().rlk_linear_logp_bwd(_ptr(h), _ptr(W), _ptr(y), _ptr(lse), _ptr(g), T, H, V,
                                     ignore_index, _ptr(grad_h), _ptr(grad_W), _ptr(ws), n,
                                     _stream()),
           "rlk_linear_logp_bwd")
    return grad_h, grad_W


def saved_logits_ld(V: int) -> int:
    """Row stride (floats) of the saved-logits buffer for a vocabulary of V rows."""
    return int(lib().rlk_saved_logits_ld(V))


def linear_logp_fwd_save(h, W, y, ignore_index: int = IGNORE_INDEX, ws=None, zsave=None):
    """Forward that also keeps the fp32 logits of the active rows.

    Returns (logp, lse, zsave) with zsave fp32 [T, saved_logits_ld(V)] in the
    split layout of include/rlk.h; logp and lse equal linear_logp_fwd's bits.
    """
    h, W, y = _prep(h, W, y)
    T, H = h.shape
    V = W.shape[0]
    ld = saved_logits_ld(V)
    logp = torch.empty(T, dtype=torch.float32, device=h.device)
    lse = torch.empty(T, dtype=torch.float32, device=h.device)
    if zsave is None:
        zsave = torch.empty((T, ld), dtype=torch.float32, device=h.device)
    if ws is None:
        ws, n = _workspace(OP_FWD, T, H, V, h.device)
    else:
        ws, n = _given_workspace(ws, h.device)
    _check(lib().rlk_linear_logp_fwd_save(_ptr(h), _ptr(W), _ptr(y), T, H, V, ignore_index,
                                          _ptr(logp), _ptr(lse), _ptr(zsave), zsave.stride(0),
                                          _ptr(ws), n, _stream()),
           "rlk_linear_logp_fwd_save")
    return logp, lse, zsave


def linear_logp_bwd_saved(h, W, y, lse, g, zsave, ignore_index: int = IGNORE_INDEX,
                          need_grad_h: bool = True, need_grad_W: bool = True, ws=None):
    """linear_logp_bwd from the logits saved by linear_logp_fwd_save (no recompute)."""
    h, W, y = _prep(h, W, y)
    T, H = h.shape
    V = W.shape[0]
    lse, g = _rows(T, h.device, lse=lse, g=g)
    if (zsave.dtype != torch.float32 or zsave.dim() != 2 or zsave.stride(1) != 1
            or zsave.shape[0] != T or zsave.stride(0) < saved_logits_ld(V) or zsave.device != h.device):
        raise ValueError("zsave must be the float32 [T, ld] buffer of linear_logp_fwd_save")
    grad_h = torch.empty((T, H), dtype=torch.bfloat16, device=h.device) if need_grad_h else None
    grad_W = torch.empty((V, H), dtype=torch.float32, device=h.device) if need_grad_W else None
    if ws is None:
        ws, n = _workspace(OP_BWD, T, H, V, h.device)
    else:
        ws, n = _given_workspace(ws, h.device)
    _check(lib().rlk_linear_logp_bwd_saved(_ptr(h), _ptr(W), _ptr(y), _ptr(lse), _ptr(g), _ptr(zsave),
                                           zsave.stride(0), T, H, V, ignore_index, _ptr(grad_h),
                                           _ptr(grad_W), _ptr(ws), n, _stream()),
           "rlk_linear_logp_bwd_saved")
    return grad_h, grad_W


def lse_partial(h, W_shard, y, vocab_start: int, V_global: int,
                ignore_index: int = IGNORE_INDEX, ws=None, out=None):
    """Per-row statistics of the range [vocab_start, vocab_start + len(W_shard)).

    Returns a float32 tensor [T, 4] holding (m, s, z_target, owned) per row;
    the last column holds uint32 bits (view it with ``.view(torch.int32)``).
    """
    h, W_shard, y = _prep(h, W_shard, y)
    T, H = h.shape
    n_rows = W_shard.shape[0]
    if out is None:
        out = torch.empty((T, 4), dtype=torch.float32, device=h.device)
    elif out.shape != (T, 4) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [T, 4] tensor")
    if ws is None:
        ws, n = _workspace(OP_PARTIAL, T, H, V_global, h.device)
    else:
        ws, n = _given_workspace(ws, h.device)
    _check(lib().rlk_lse_partial(_ptr(h), _ptr(W_shard), _ptr(y), T, H, vocab_start, n_rows,
                                 V_global, ignore_index, _ptr(out), _ptr(ws), n, _stream()),
           "rlk_lse_partial")
    return out


def lse_merge(parts, y, ignore_index: int = IGNORE_INDEX):
    """Merge [P, T, 4] range statistics (ascending vocabulary order) into (logp, lse)."""
    if parts.dim() != 3 or parts.shape[2] != 4 or parts.dtype != torch.float32:
        raise ValueError("parts must be float32 [P, T, 4]")
    if not parts.is_cuda:
        raise ValueError("parts must be a device tensor")
    parts = parts.contiguous()
    P, T = parts.shape[0], parts.shape[1]
    y, = _rows(T, parts.device, y=y)
    logp = torch.empty(T, dtype=torch.float32, device=parts.device)
    lse = torch.empty(T, dtype=torch.float32, device=parts.device)
    _check(lib().rlk_lse_merge(_ptr(parts), P, _ptr(y), T, ignore_index, _ptr(logp), _ptr(lse),
                               _stream()),
           "rlk_lse_merge")
    return logp, lse


def gemm_bf16_nt(A, B, out_dtype=torch.float32):
    """Deterministic, batch-invariant A @ B^T for bf16 A [M, K] and B [N, K].

    out_dtype torch.float32 or torch.bfloat16 (rounded once).  K % 64 == 0.
    """
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("A must be [M, K] and B [N, K]")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    A, B = A.contiguous(), B.contiguous()
    M, K = A.shape
    N = B.shape[0]
    ldc = (N + 3) // 4 * 4
    C = torch.empty((M, ldc), dtype=out_dtype, device=A.device)
    _check(lib().rlk_gemm_bf16_nt(_ptr(A), _ptr(B), M, N, K, _ptr(C), ldc,
                                  0 if out_dtype == torch.float32 else 1, _stream()),
           "rlk_gemm_bf16_nt")
    return C[:, :N] if ldc != N else C


def linear_logp_fwd_rl(h, W, y, logp_old, adv, eps_low: float = 0.2, eps_high: float = 0.2,
                       beta: float = 0.0, logp_ref=None, scale: float = 1.0,
                       ignore_index: int = IGNORE_INDEX, ws=None):
    """Forward with the per-token RL objective fused into its last kernel:
    (logp, lse, loss, g), each fp32 [T]; logp/lse equal linear_logp_fwd's
    bits and loss/g equal rl_token_loss's on that logp."""
    h, W, y = _prep(h, W, y)
    T, H = h.shape
    V = W.shape[0]
    if beta != 0.0 and logp_ref is None:
        raise ValueError("logp_ref is required when beta != 0")
    named = dict(logp_old=logp_old, adv=adv)
    if logp_ref is not None:
        named["logp_ref"] = logp_ref
    checked = dict(zip(named, _rows(T, h.device, **named)))
    out = [torch.empty(T, dtype=torch.float32, device=h.device) for _ in range(4)]
    if ws is None:
        ws, n = _workspace(OP_FWD, T, H, V, h.device)
    else:
        ws, n = _given_workspace(ws, h.device)
    _check(lib().rlk_linear_logp_fwd_rl(_ptr(h), _ptr(W), _ptr(y), T, H, V, ignore_index,
                                        _ptr(checked["logp_old"]), _ptr(checked["adv"]),
                                        _ptr(checked.get("logp_ref")), eps_low, eps_high, beta, scale,
                                        *(_ptr(t) for t in out), _ptr(ws), n, _stream()),
           "rlk_linear_logp_fwd_rl")
    return tuple(out)


def rl_token_loss(logp, logp_old, adv, y, eps_low: float = 0.2, eps_high: float = 0.2,
                  beta: float = 0.0, logp_ref=None, scale: float = 1.0,
                  ignore_index: int = IGNORE_INDEX):
    """Per-token clipped-surrogate + k3-KL loss and g = dloss/dlogp, fp32 [T] each."""
    if logp.dim() != 1:
        raise ValueError("logp must be 1-D")
    if beta != 0.0 and logp_ref is None:
        raise ValueError("logp_ref is required when beta != 0")
    T = logp.shape[0]
    named = dict(logp=logp, logp_old=logp_old, adv=adv, y=y)
    if logp_ref is not None:
        named["logp_ref"] = logp_ref
    checked = dict(zip(named, _rows(T, logp.device, **named)))
    logp, logp_old, adv, y = checked["logp"], checked["logp_old"], checked["adv"], checked["y"]
    ref = checked.get("logp_ref")
    if not logp.is_cuda:
        raise ValueError("inputs must be device tensors")
    loss = torch.empty(T, dtype=torch.float32, device=logp.device)
    g = torch.empty(T, dtype=torch.float32, device=logp.device)
    _check(lib().rlk_rl_token_loss(_ptr(logp), _ptr(logp_old), _ptr(adv), _ptr(ref), _ptr(y), T,
                                   ignore_index, eps_low, eps_high, beta, scale, _ptr(loss), _ptr(g),
                                   _stream()),
           "rlk_rl_token_loss")
    return loss, g


def bench_mfma_ceiling(blocks: int = 256, iters: int = 4096, repeats: int = 3):
    """Benchmark only: TFLOP/s of a pure loop of the tile engine's MFMA
    instruction (v_mfma_f32_16x16x32_bf16; v_mfma_f32_32x32x16_bf16 in a
    contract-1 build) on random operands (no memory traffic), eight waves per
    workgroup as in the eight-wave tile kernels, best and median of `repeats`
    timed launches.  2^23 FLOP per workgroup per iteration."""
    gen = torch.Generator(device="cuda").manual_seed(12345)
    src = torch.randn(24 * 512 * 8, device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    flops = float(2 ** 23) * iters * blocks
    times = []
    for r in range(repeats + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(lib().rlk_bench_mfma_ceiling(_ptr(src), _ptr(out), blocks, iters, _stream()),
               "rlk_bench_mfma_ceiling")
        e1.record()
        torch.cuda.synchronize()
        if r:  # the first launch warms up
            times.append(e0.elapsed_time(e1))
    times.sort()
    return {"best_tflops": flops / times[0] / 1e9, "median_tflops": flops / times[len(times) // 2] / 1e9,
            "launch_ms": times}


def profile_begin():
    """Start timing every kernel the library launches (HIP events on its stream)."""
    _check(lib().rlk_profile_begin(), "rlk_profile_begin")


def profile_end():
    """Stop timing; {kernel name: (launches, total ms)} since profile_begin()."""
    buf = (KernelTime * 64)()
    n = _i32(0)
    _check(lib().rlk_profile_end(buf, 64, ctypes.byref(n)), "rlk_profile_end")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(min(n.value, 64))}


class _LinearLogp(torch.autograd.Function):
    @staticmethod
    def forward(ctx, h, W, y, ignore_index):
        logp, lse = linear_logp_fwd(h, W, y, ignore_index)
        ctx.save_for_backward(h, W, y, lse)
        ctx.ignore_index = ignore_index
        return logp

    @staticmethod
    def backward(ctx, g):
        h, W, y, lse = ctx.saved_tensors
        gh, gW = linear_logp_bwd(h, W, y, lse, g, ctx.ignore_index,
                                 need_grad_h=ctx.needs_input_grad[0],
                                 need_grad_W=ctx.needs_input_grad[1])
        if gW is not None:
            gW = gW.to(W.dtype)
        return gh, gW, None, None


def linear_logp(h, W, y, ignore_index: int = IGNORE_INDEX):
    """log_softmax(h @ W^T)[t, y_t] per row (0 where y_t == ignore_index), autograd-aware.

    The weight gradient is computed in fp32 and cast to W's dtype for
    autograd; call ``linear_logp_bwd`` directly to keep it in fp32.
    """
    return _LinearLogp.apply(h, W, y, ignore_index)
