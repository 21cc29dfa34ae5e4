"""ctypes binding of liblvtv.so: argument marshalling only.

Every step of the verify and the loss runs in the library's HIP kernels;
this module checks tensor dtypes, devices and layouts, allocates outputs and
the workspace with torch on the tensors' device, and passes raw pointers and
torch's current HIP stream. There is no CPU fallback: if the library is not
built, or the tensors are not on a GPU, calls raise.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblvtv.so")

LVTV_F32 = 0
LVTV_BF16 = 1

STATUS_BAD_K = 1
STATUS_BAD_TOKEN = 2
STATUS_BAD_TEMPERATURE = 4
STATUS_NONFINITE = 8
STATUS_BAD_TRUNCATION = 16

EXPORTS = (
    "lvtv_version",
    "lvtv_strerror",
    "lvtv_workspace_reset",
    "spec_verify_workspace_bytes",
    "spec_verify",
    "spec_verify_packed_workspace_bytes",
    "spec_verify_packed",
    "spec_verify_topkp_workspace_bytes",
    "spec_verify_topkp",
    "e2e_tv_loss_workspace_bytes",
    "e2e_tv_loss_fwd_bwd",
    "draft_loss_workspace_bytes",
    "draft_loss_fwd_bwd",
    "draft_loss_logits_workspace_bytes",
    "draft_loss_logits_fwd_bwd",
    "dspark_schedule",
    "lvtv_debug_draft_loss",
    "spec_verify_noalloc",
)

NOALLOC_SCRATCH_BYTES = 16 << 20  # LVTV_NOALLOC_SCRATCH_BYTES

SCHED_MAX_ITEMS = 8192  # LVTV_SCHED_MAX_ITEMS

# Objectives of draft_loss_fwd_bwd (include/lvtv.h, LVTV_OBJ_*).
OBJECTIVES = {"e2e_tv": 0, "step_tv": 1, "ce": 2, "kl": 3}

# Paths of lvtv_debug_draft_loss (LVTV_PATH_*).
PATHS = {"auto": 0, "multi-pass": 2, "reread": 3}
SPIN_LIMIT = 1 << 16  # what the product calls use

_lib = None
_lock = threading.Lock()


class LvtvError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH):
    """Load liblvtv.so and declare its signatures (no HIP call is made)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise LvtvError(
                f"{path} is missing: build it with `python -m lossless_verify_tv_amd.build`")
        lib = ctypes.CDLL(path)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        lib.lvtv_version.restype = ctypes.c_int
        lib.lvtv_version.argtypes = []
        lib.lvtv_strerror.restype = ctypes.c_char_p
        lib.lvtv_strerror.argtypes = [ctypes.c_int]
        lib.lvtv_workspace_reset.restype = ctypes.c_int
        lib.lvtv_workspace_reset.argtypes = [vp, sz, vp]
        lib.spec_verify_workspace_bytes.restype = sz
        lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, ctypes.c_int]
        lib.spec_verify.restype = ctypes.c_int
        lib.spec_verify.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32,
                                    vp, vp, vp, vp, vp, sz, vp]
        lib.spec_verify_packed_workspace_bytes.restype = sz
        lib.spec_verify_packed_workspace_bytes.argtypes = [i32, i32, i32, ctypes.c_int]
        lib.spec_verify_packed.restype = ctypes.c_int
        lib.spec_verify_packed.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32,
                                           vp, vp, vp, vp, vp, sz, vp]
        lib.spec_verify_topkp_workspace_bytes.restype = sz
        lib.spec_verify_topkp_workspace_bytes.argtypes = [i32, i32, i32, ctypes.c_int]
        lib.spec_verify_topkp.restype = ctypes.c_int
        lib.spec_verify_topkp.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32,
                                          i32, vp, vp, vp, vp, vp, sz, vp]
        lib.e2e_tv_loss_workspace_bytes.restype = sz
        lib.e2e_tv_loss_workspace_bytes.argtypes = [i32, i32, i32]
        lib.e2e_tv_loss_fwd_bwd.restype = ctypes.c_int
        lib.e2e_tv_loss_fwd_bwd.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        lib.draft_loss_workspace_bytes.restype = sz
        lib.draft_loss_workspace_bytes.argtypes = [i32, i32, i32]
        lib.draft_loss_fwd_bwd.restype = ctypes.c_int
        lib.draft_loss_fwd_bwd.argtypes = [vp, vp, i32, i32, i32, ctypes.c_int, vp, vp, vp, vp,
                                           sz, vp]
        lib.draft_loss_logits_workspace_bytes.restype = sz
        lib.draft_loss_logits_workspace_bytes.argtypes = [i32, i32, i32]
        lib.draft_loss_logits_fwd_bwd.restype = ctypes.c_int
        lib.draft_loss_logits_fwd_bwd.argtypes = [vp, vp, ctypes.c_float, i32, i32, i32,
                                                  ctypes.c_int, vp, vp, vp, vp, sz, vp]
        lib.dspark_schedule.restype = ctypes.c_int
        lib.dspark_schedule.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        lib.spec_verify_noalloc.restype = ctypes.c_int
        lib.spec_verify_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, i32, i32, i32,
                                            vp, vp, vp, vp, vp]
        lib.lvtv_debug_draft_loss.restype = ctypes.c_int
        lib.lvtv_debug_draft_loss.argtypes = [vp, vp, vp, ctypes.c_float, i32, i32, i32,
                                              ctypes.c_int, ctypes.c_int, i32, vp, vp, vp, vp,
                                              vp, sz, vp]
        _lib = lib
        return lib


def strerror(code: int) -> str:
    return load_library().lvtv_strerror(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise LvtvError(f"{what} failed: {strerror(code)} (code {code})")


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return LVTV_BF16
    if t.dtype == torch.float32:
        return LVTV_F32
    raise ValueError("logits must be float32 or bfloat16")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


# Workspaces are cached per device and grown on demand. Calls on one device
# that share the cached workspace must run on one stream (torch's current
# stream); pass an explicit `workspace` otherwise.
_workspaces: dict = {}


def new_workspace(nbytes, device):
    """A workspace of at least `nbytes` bytes on `device`, zero-filled by the
    library's fill kernel (no call depends on the contents; zeros keep a
    fresh workspace deterministic to look at)."""
    ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    with torch.cuda.device(device):
        _check(load_library().lvtv_workspace_reset(_ptr(ws), ws.numel(), _stream(device)),
               "lvtv_workspace_reset")
    return ws


def _workspace(op, device, nbytes):
    key = (op, device.type, device.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(nbytes, device)
        _workspaces[key] = ws
    return ws


def spec_verify_workspace_bytes(B, Kmax, V, dtype=LVTV_BF16) -> int:
    return int(load_library().spec_verify_workspace_bytes(B, Kmax, V, dtype))


def spec_verify(target_logits, draft_logits, draft_tokens, k_per_req, temperature, seed,
                workspace=None, out=None, top_k=None, top_p=None):
    """Verify step for B requests (see include/lvtv.h for the contract).

    target_logits [B, Kmax+1, V] and draft_logits [B, Kmax, V]: float32 or
    bfloat16, contiguous, on one GPU. draft_tokens int32 [B, Kmax];
    k_per_req int32 [B]; temperature float32 [B]; seed int64/uint64 [B]
    (bit pattern used as the 64-bit Philox key). Returns (accepted_len
    int32 [B], out_tokens int32 [B, Kmax+1], alpha float32 [B, Kmax],
    status int32 [B]) on the device; no synchronisation.

    With ``top_k`` (int32 [B]) and ``top_p`` (float32 [B]) the call is
    spec_verify_topkp: p and q are truncated to each row's top-k, then top-p,
    tokens before the verify step.
    """
    lib = load_library()
    dev = target_logits.device
    trunc = top_k is not None or top_p is not None
    _require(top_k is not None and top_p is not None or not trunc,
             "top_k and top_p go together")
    _require(dev.type == "cuda", "spec_verify needs GPU tensors")
    _require(target_logits.dim() == 3 and draft_logits.dim() == 3, "logits must be 3-D")
    B, K1, V = target_logits.shape
    Kmax = K1 - 1
    _require(tuple(draft_logits.shape) == (B, Kmax, V), "draft_logits must be [B, Kmax, V]")
    _require(target_logits.dtype == draft_logits.dtype, "target and draft dtypes differ")
    if target_logits.dtype == torch.bfloat16:
        dtype = LVTV_BF16
    elif target_logits.dtype == torch.float32:
        dtype = LVTV_F32
    else:
        raise ValueError("logits must be float32 or bfloat16")
    for name, t, dt, shape in (("draft_tokens", draft_tokens, (torch.int32,), (B, Kmax)),
                               ("k_per_req", k_per_req, (torch.int32,), (B,)),
                               ("temperature", temperature, (torch.float32,), (B,)),
                               ("seed", seed, (torch.int64, torch.uint64), (B,))) + (
            (("top_k", top_k, (torch.int32,), (B,)),
             ("top_p", top_p, (torch.float32,), (B,))) if trunc else ()):
        _require(t.dtype in dt, f"{name} must be {dt}")
        _require(tuple(t.shape) == shape, f"{name} must have shape {shape}")
        _require(t.device == dev and t.is_contiguous(), f"{name} must be contiguous on {dev}")
    for t in (target_logits, draft_logits):
        _require(t.device == dev and t.is_contiguous(), "logits must be contiguous on one GPU")
    need = (lib.spec_verify_topkp_workspace_bytes if trunc else
            lib.spec_verify_workspace_bytes)(B, Kmax, V, dtype)
    _require(need > 0, f"sizes out of range: B={B} Kmax={Kmax} V={V}")
    ws = workspace if workspace is not None else _workspace("verify", dev, need)
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, Kmax + 1, dtype=torch.int32, device=dev)
        alpha = torch.empty(B, max(Kmax, 0), dtype=torch.float32, device=dev)
        status = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        acc, toks, alpha, status = out
    with torch.cuda.device(dev):
        if trunc:
            code = lib.spec_verify_topkp(_ptr(target_logits), _ptr(draft_logits), dtype,
                                         _ptr(draft_tokens), _ptr(k_per_req), _ptr(temperature),
                                         _ptr(seed), _ptr(top_k), _ptr(top_p), B, Kmax, V,
                                         _ptr(acc), _ptr(toks), _ptr(alpha), _ptr(status),
                                         _ptr(ws), ws.numel(), _stream(dev))
        else:
            code = lib.spec_verify(_ptr(target_logits), _ptr(draft_logits), dtype,
                                   _ptr(draft_tokens), _ptr(k_per_req), _ptr(temperature),
                                   _ptr(seed), B, Kmax, V, _ptr(acc), _ptr(toks), _ptr(alpha),
                                   _ptr(status), _ptr(ws), ws.numel(), _stream(dev))
    _check(code, "spec_verify_topkp" if trunc else "spec_verify")
    return acc, toks, alpha, status


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, k_per_req, temperature, seed,
                        out):
    """spec_verify through the entry point that allocates nothing (its
    scratch is the library's static per-GPU array). ``out`` = (accepted_len,
    out_tokens, alpha, status), preallocated by the caller; tensors as
    spec_verify. Returns ``out``."""
    lib = load_library()
    dev = target_logits.device
    _require(dev.type == "cuda", "spec_verify_noalloc needs GPU tensors")
    B, K1, V = target_logits.shape
    Kmax = K1 - 1
    _require(tuple(draft_logits.shape) == (B, Kmax, V), "draft_logits must be [B, Kmax, V]")
    _require(target_logits.dtype == draft_logits.dtype, "target and draft dtypes differ")
    dtype = _dtype_code(target_logits)
    acc, toks, alpha, status = out
    for t in (target_logits, draft_logits, draft_tokens, k_per_req, temperature, seed, acc, toks,
              alpha, status):
        _require(t.device == dev and t.is_contiguous(), "tensors must be contiguous on one GPU")
    with torch.cuda.device(dev):
        code = lib.spec_verify_noalloc(_ptr(target_logits), _ptr(draft_logits), dtype,
                                       _ptr(draft_tokens), _ptr(k_per_req), _ptr(temperature),
                                       _ptr(seed), B, Kmax, V, _ptr(acc), _ptr(toks),
                                       _ptr(alpha), _ptr(status), _stream(dev))
    _check(code, "spec_verify_noalloc")
    return out


def spec_verify_topkp_workspace_bytes(B, Kmax, V, dtype=LVTV_BF16) -> int:
    return int(load_library().spec_verify_topkp_workspace_bytes(B, Kmax, V, dtype))


def spec_verify_topkp(target_logits, draft_logits, draft_tokens, k_per_req, temperature, seed,
                      top_k, top_p, workspace=None, out=None):
    """spec_verify with per-request top-k (int32 [B]; <= 0 or >= V: off) and
    top-p (float32 [B]; >= 1: off, NaN or <= 0 faults the request with
    STATUS_BAD_TRUNCATION) applied to p and q first."""
    return spec_verify(target_logits, draft_logits, draft_tokens, k_per_req, temperature, seed,
                       workspace=workspace, out=out, top_k=top_k, top_p=top_p)


def e2e_tv_loss_workspace_bytes(N, W, V) -> int:
    return int(load_library().e2e_tv_loss_workspace_bytes(N, W, V))


def e2e_tv_loss_fwd_bwd(draft_logits, target_probs, workspace=None, out=None):
    """E2E-TV loss and gradient (see include/lvtv.h).

    draft_logits bfloat16 [N, W, V], target_probs float32 [N, W, V], both
    contiguous on one GPU. Returns (loss float32 [1], alpha float32 [N, W],
    dlogits bfloat16 [N, W, V]) on the device; no synchronisation.
    """
    lib = load_library()
    dev = draft_logits.device
    _require(dev.type == "cuda", "e2e_tv_loss_fwd_bwd needs GPU tensors")
    _require(draft_logits.dtype == torch.bfloat16, "draft_logits must be bfloat16")
    _require(target_probs.dtype == torch.float32, "target_probs must be float32")
    _require(draft_logits.dim() == 3 and tuple(target_probs.shape) == tuple(draft_logits.shape),
             "draft_logits and target_probs must both be [N, W, V]")
    for t in (draft_logits, target_probs):
        _require(t.device == dev and t.is_contiguous(), "inputs must be contiguous on one GPU")
    N, W, V = draft_logits.shape
    need = lib.e2e_tv_loss_workspace_bytes(N, W, V)
    _require(need > 0, f"sizes out of range: N={N} W={W} V={V}")
    ws = workspace if workspace is not None else _workspace("loss", dev, need)
    if out is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        alpha = torch.empty(N, W, dtype=torch.float32, device=dev)
        dlogits = torch.empty(N, W, V, dtype=torch.bfloat16, device=dev)
    else:
        loss, alpha, dlogits = out
    with torch.cuda.device(dev):
        code = lib.e2e_tv_loss_fwd_bwd(_ptr(draft_logits), _ptr(target_probs), N, W, V,
                                       _ptr(loss), _ptr(alpha), _ptr(dlogits), _ptr(ws),
                                       ws.numel(), _stream(dev))
    _check(code, "e2e_tv_loss_fwd_bwd")
    return loss, alpha, dlogits


def draft_loss_workspace_bytes(N, W, V) -> int:
    return int(load_library().draft_loss_workspace_bytes(N, W, V))


def draft_loss_fwd_bwd(draft_logits, target_probs, objective, workspace=None, out=None):
    """The E2E-TV loss or a per-position comparator (per-step TV, CE, KL) and
    its gradient (see include/lvtv.h). ``objective`` is a key of OBJECTIVES
    or its LVTV_OBJ_* value; otherwise as e2e_tv_loss_fwd_bwd."""
    lib = load_library()
    obj = OBJECTIVES.get(objective, objective)
    _require(isinstance(obj, int), f"unknown objective {objective!r}")
    dev = draft_logits.device
    _require(dev.type == "cuda", "draft_loss_fwd_bwd needs GPU tensors")
    _require(draft_logits.dtype == torch.bfloat16, "draft_logits must be bfloat16")
    _require(target_probs.dtype == torch.float32, "target_probs must be float32")
    _require(draft_logits.dim() == 3 and tuple(target_probs.shape) == tuple(draft_logits.shape),
             "draft_logits and target_probs must both be [N, W, V]")
    for t in (draft_logits, target_probs):
        _require(t.device == dev and t.is_contiguous(), "inputs must be contiguous on one GPU")
    N, W, V = draft_logits.shape
    need = lib.draft_loss_workspace_bytes(N, W, V)
    _require(need > 0, f"sizes out of range: N={N} W={W} V={V}")
    ws = workspace if workspace is not None else _workspace("loss", dev, need)
    if out is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        alpha = torch.empty(N, W, dtype=torch.float32, device=dev)
        dlogits = torch.empty(N, W, V, dtype=torch.bfloat16, device=dev)
    else:
        loss, alpha, dlogits = out
    with torch.cuda.device(dev):
        code = lib.draft_loss_fwd_bwd(_ptr(draft_logits), _ptr(target_probs), N, W, V, obj,
                                      _ptr(loss), _ptr(alpha), _ptr(dlogits), _ptr(ws),
                                      ws.numel(), _stream(dev))
    _check(code, "draft_loss_fwd_bwd")
    return loss, alpha, dlogits


def draft_loss_logits_workspace_bytes(N, W, V) -> int:
    return int(load_library().draft_loss_logits_workspace_bytes(N, W, V))


def draft_loss_logits_fwd_bwd(draft_logits, target_logits, temperature, objective="e2e_tv",
                              workspace=None, out=None):
    """draft_loss_fwd_bwd with the target given as bfloat16 logits and a
    temperature applied to both rows (see include/lvtv.h). ``temperature`` is
    a host float; otherwise as draft_loss_fwd_bwd."""
    lib = load_library()
    obj = OBJECTIVES.get(objective, objective)
    _require(isinstance(obj, int), f"unknown objective {objective!r}")
    dev = draft_logits.device
    _require(dev.type == "cuda", "draft_loss_logits_fwd_bwd needs GPU tensors")
    _require(draft_logits.dtype == torch.bfloat16, "draft_logits must be bfloat16")
    _require(target_logits.dtype == torch.bfloat16, "target_logits must be bfloat16")
    _require(draft_logits.dim() == 3 and tuple(target_logits.shape) == tuple(draft_logits.shape),
             "draft_logits and target_logits must both be [N, W, V]")
    for t in (draft_logits, target_logits):
        _require(t.device == dev and t.is_contiguous(), "inputs must be contiguous on one GPU")
    N, W, V = draft_logits.shape
    need = lib.draft_loss_logits_workspace_bytes(N, W, V)
    _require(need > 0, f"sizes out of range: N={N} W={W} V={V}")
    ws = workspace if workspace is not None else _workspace("loss", dev, need)
    if out is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        alpha = torch.empty(N, W, dtype=torch.float32, device=dev)
        dlogits = torch.empty(N, W, V, dtype=torch.bfloat16, device=dev)
    else:
        loss, alpha, dlogits = out
    with torch.cuda.device(dev):
        code = lib.draft_loss_logits_fwd_bwd(_ptr(draft_logits), _ptr(target_logits),
                                             float(temperature), N, W, V, obj, _ptr(loss),
                                             _ptr(alpha), _ptr(dlogits), _ptr(ws), ws.numel(),
                                             _stream(dev))
    _check(code, "draft_loss_logits_fwd_bwd")
    return loss, alpha, dlogits


def dspark_schedule(confidence, sps, out=None):
    """Confidence-scheduled verify lengths (see include/lvtv.h).

    confidence float32 [R, L] and sps float32 [R (L + 1) + 1], contiguous on
    one GPU. Returns (verify_len int32 [R], best float64 [2]: Theta at the
    optimum and its batch size) on the device; no synchronisation."""
    lib = load_library()
    dev = confidence.device
    _require(dev.type == "cuda", "dspark_schedule needs GPU tensors")
    _require(confidence.dtype == torch.float32 and sps.dtype == torch.float32,
             "confidence and sps must be float32")
    _require(confidence.dim() == 2, "confidence must be [R, L]")
    R, L = confidence.shape
    _require(sps.dim() == 1 and sps.numel() >= R * (L + 1) + 1,
             "sps needs R (L + 1) + 1 entries, indexed by batch size")
    for t in (confidence, sps):
        _require(t.device == dev and t.is_contiguous(), "inputs must be contiguous on one GPU")
    if out is None:
        lens = torch.empty(R, dtype=torch.int32, device=dev)
        best = torch.empty(2, dtype=torch.float64, device=dev)
    else:
        lens, best = out
    with torch.cuda.device(dev):
        code = lib.dspark_schedule(_ptr(confidence), _ptr(sps), R, L, _ptr(lens), _ptr(best),
                                   _stream(dev))
    _check(code, "dspark_schedule")
    return lens, best


def spec_verify_packed_workspace_bytes(B, total_rows, V, dtype=LVTV_BF16) -> int:
    return int(load_library().spec_verify_packed_workspace_bytes(B, total_rows, V, dtype))


def spec_verify_packed(target_logits, draft_logits, draft_tokens, row_offsets, temperature, seed,
                       workspace=None, out=None):
    """Verify step on the packed layout (see include/lvtv.h): target_logits
    [total_rows, V], draft_logits [total_rows - B, V] (same dtype, bf16 or
    fp32), draft_tokens int32 [total_rows - B], row_offsets int32 [B + 1],
    temperature float32 [B], seed int64/uint64 [B]. Returns (accepted_len
    [B], out_tokens [total_rows], alpha [total_rows - B], status [B])."""
    lib = load_library()
    dev = target_logits.device
    _require(dev.type == "cuda", "spec_verify_packed needs GPU tensors")
    dtype = _dtype_code(target_logits)
    _require(target_logits.dim() == 2, "target_logits must be [total_rows, V]")
    total_rows, V = target_logits.shape
    B = row_offsets.numel() - 1
    _require(B >= 1 and row_offsets.dtype == torch.int32, "row_offsets must be int32 [B + 1]")
    nd = total_rows - B
    _require(draft_logits.dtype == target_logits.dtype and draft_logits.dim() == 2 and
             tuple(draft_logits.shape) == (nd, V), "draft_logits must be [total_rows - B, V]")
    _require(draft_tokens.dtype == torch.int32 and draft_tokens.numel() == nd,
             "draft_tokens must be int32 [total_rows - B]")
    _require(temperature.dtype == torch.float32 and temperature.numel() == B,
             "temperature must be float32 [B]")
    _require(seed.dtype in (torch.int64, torch.uint64) and seed.numel() == B,
             "seed must be 64-bit [B]")
    for t in (target_logits, draft_logits, draft_tokens, row_offsets, temperature, seed):
        _require(t.device == dev and t.is_contiguous(), "inputs must be contiguous on one GPU")
    need = lib.spec_verify_packed_workspace_bytes(B, total_rows, V, dtype)
    _require(need > 0, f"sizes out of range: B={B} total_rows={total_rows} V={V}")
    ws = workspace if workspace is not None else _workspace("verify_packed", dev, need)
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(total_rows, dtype=torch.int32, device=dev)
        alpha = torch.empty(max(nd, 1), dtype=torch.float32, device=dev)[:nd]
        status = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        acc, toks, alpha, status = out
    with torch.cuda.device(dev):
        code = lib.spec_verify_packed(_ptr(target_logits), _ptr(draft_logits if nd else None),
                                      dtype, _ptr(draft_tokens if nd else None),
                                      _ptr(row_offsets), _ptr(temperature), _ptr(seed), B,
                                      total_rows, V, _ptr(acc), _ptr(toks),
                                      _ptr(alpha if nd else None), _ptr(status), _ptr(ws),
                                      ws.numel(), _stream(dev))
    _check(code, "spec_verify_packed")
    return acc, toks, alpha, status


def debug_draft_loss(draft_logits, target_probs=None, target_logits=None, temperature=1.0,
                     objective="e2e_tv", path="auto", spin_limit=SPIN_LIMIT, want_f32=False,
                     workspace=None):
    """Test and debugging hook (lvtv_debug_draft_loss): draft_loss_fwd_bwd
    (``target_probs``) or draft_loss_logits_fwd_bwd (``target_logits`` and
    ``temperature``) with the path forced ("auto" or "multi-pass"), the
    single-read kernel's spin limit set (0: every row takes the repair
    path) and, with ``want_f32``, the fp32 gradient before rounding.
    Returns (loss, alpha, dlogits, dlogits_f32 or None)."""
    lib = load_library()
    obj = OBJECTIVES.get(objective, objective)
    _require(isinstance(obj, int), f"unknown objective {objective!r}")
    _require(path in PATHS, f"unknown path {path!r}")
    _require((target_probs is None) != (target_logits is None),
             "give exactly one of target_probs and target_logits")
    target = target_probs if target_probs is not None else target_logits
    dev = draft_logits.device
    _require(dev.type == "cuda", "debug_draft_loss needs GPU tensors")
    _require(draft_logits.dtype == torch.bfloat16, "draft_logits must be bfloat16")
    _require(target.dtype == (torch.float32 if target_probs is not None else torch.bfloat16),
             "target_probs must be float32, target_logits bfloat16")
    _require(draft_logits.dim() == 3 and tuple(target.shape) == tuple(draft_logits.shape),
             "draft_logits and the target must both be [N, W, V]")
    for t in (draft_logits, target):
        _require(t.device == dev and t.is_contiguous(), "inputs must be contiguous on one GPU")
    N, W, V = draft_logits.shape
    need = lib.draft_loss_workspace_bytes(N, W, V)
    _require(need > 0, f"sizes out of range: N={N} W={W} V={V}")
    ws = workspace if workspace is not None else _workspace("loss", dev, need)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    alpha = torch.empty(N, W, dtype=torch.float32, device=dev)
    dlogits = torch.empty(N, W, V, dtype=torch.bfloat16, device=dev)
    d32 = torch.empty(N, W, V, dtype=torch.float32, device=dev) if want_f32 else None
    with torch.cuda.device(dev):
        code = lib.lvtv_debug_draft_loss(
            _ptr(draft_logits), _ptr(target_probs), _ptr(target_logits), float(temperature),
            N, W, V, obj, PATHS[path], int(spin_limit), _ptr(loss), _ptr(alpha), _ptr(dlogits),
            _ptr(d32), _ptr(ws), ws.numel(), _stream(dev))
    _check(code, "lvtv_debug_draft_loss")
    return loss, alpha, dlogits, d32
