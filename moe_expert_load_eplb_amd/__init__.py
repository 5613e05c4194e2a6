"""Python binding of libeplb (the EPLB hot path on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libeplb.so``; this module checks dtypes, devices and contiguity, passes raw
device pointers and the current HIP stream through the C ABI declared in
``include/eplb.h``, and raises :class:`EplbError` on a non-zero return code.
PyTorch supplies device memory and streams.

Importing this package loads the library; if it has not been built
(``python moe_expert_load_eplb_amd/build.py``) the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeplb.so")

EPLB_OK = 0
EPLB_E_ARG = 1
EPLB_E_DIV = 2
EPLB_E_REDUNDANCY = 3
EPLB_E_CAPACITY = 4
EPLB_E_LIMIT = 5
EPLB_E_RANGE = 6
EPLB_E_HIP = 7
EPLB_S_OK = 0
EPLB_S_BAD_LOAD = 16
EPLB_S_OVERFLOW = 17
EPLB_S_BAD_MAP = 18
EPLB_S_BAD_TOPOLOGY = 19

EXPORTS = ("eplb_load_hist", "eplb_rebalance", "eplb_redirect", "eplb_hist_redirect",
           "eplb_load_ema", "eplb_ema_redirect", "eplb_placement_load", "eplb_rearrange", "eplb_lp_solve", "eplb_lp_redirect",
           "eplb_lp_redirect_workspace_bytes", "eplb_status_string",
           "eplb_rebalance_lds_bytes", "eplb_rebalance_max_count", "eplb_lp_redirect_noalloc")


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python moe_expert_load_eplb_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    missing = [f for f in EXPORTS if not hasattr(lib, f)]
    if missing:
        raise ImportError(f"{_LIB_PATH} lacks {missing}: rebuild it with "
                          "`python moe_expert_load_eplb_amd/build.py`")
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.eplb_load_hist.argtypes = [p, i64, i64, i32, i32, p, i32, i64, p, p, p]
    lib.eplb_load_hist.restype = i32
    lib.eplb_rebalance.argtypes = [p, i64, i32, i32, i32, i32, i32, i32, p, p, p, p, p]
    lib.eplb_rebalance.restype = i32
    lib.eplb_redirect.argtypes = [p, i64, i64, i32, i32, p, p, i32, p, p]
    lib.eplb_redirect.restype = i32
    lib.eplb_hist_redirect.argtypes = [p, i64, i64, i32, i32, p, i32, i64, p, p, p, p, i32, p, p]
    lib.eplb_hist_redirect.restype = i32
    lib.eplb_load_ema.argtypes = [p, i64, i64, i32, i32, p, i32, p, p, p]
    lib.eplb_load_ema.restype = i32
    lib.eplb_ema_redirect.argtypes = [p, i64, i64, i32, i32, p, i32, p, p, p, p, i32, p, p]
    lib.eplb_ema_redirect.restype = i32
    lib.eplb_placement_load.argtypes = [p, p, p, i64, i32, i32, i32, p, p, p]
    lib.eplb_placement_load.restype = i32
    lib.eplb_rearrange.argtypes = [p, p, p, i64, i32, i32, i32, i32, i32, p, p, p, p, p, p]
    lib.eplb_rearrange.restype = i32
    lib.eplb_lp_solve.argtypes = [p, p, p, i64, i32, i32, i32, p, p, p, p, p]
    lib.eplb_lp_solve.restype = i32
    lib.eplb_lp_redirect.argtypes = [p, i64, i64, i32, i32, p, p, i32, i32, p, i64, p, p]
    lib.eplb_lp_redirect.restype = i32
    lib.eplb_lp_redirect_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.eplb_lp_redirect_workspace_bytes.restype = i64
    lib.eplb_status_string.argtypes = [i32]
    lib.eplb_status_string.restype = ctypes.c_char_p
    lib.eplb_rebalance_lds_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.eplb_rebalance_lds_bytes.restype = i64
    lib.eplb_rebalance_max_count.argtypes = [i32, i32, i32, i32]
    lib.eplb_rebalance_max_count.restype = i32
    lib.eplb_lp_redirect_noalloc.argtypes = [p, i64, i64, i32, i32, p, p, i32, i32, p, p]
    lib.eplb_lp_redirect_noalloc.restype = i32
    return lib


lib = _load()


class EplbError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {lib.eplb_status_string(code).decode()} (code {code})")


def status_string(code: int) -> str:
    return lib.eplb_status_string(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != EPLB_OK:
        raise EplbError(code, where)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def load_hist(idx: torch.Tensor, E: int, ring: torch.Tensor, step: int,
              load: torch.Tensor | None = None, n_invalid: torch.Tensor | None = None):
    """Count one step's routing ids into ring[step % W] and sum the window.

    idx [L, T, K] int32; ring [W, L, E] int32 (zeroed once by the caller).
    Returns (load [L, E] int64, n_invalid [L] int64).
    """
    if idx.dim() != 3:
        raise ValueError("idx must be [L, T, K]")
    L, T, K = idx.shape
    if ring.dim() != 3 or ring.shape[1] != L or ring.shape[2] != E:
        raise ValueError(f"ring must be [W, {L}, {E}], got {tuple(ring.shape)}")
    W = ring.shape[0]
    dev = idx.device
    if load is None:
        load = torch.empty((L, E), dtype=torch.int64, device=dev)
    if n_invalid is None:
        n_invalid = torch.empty((L,), dtype=torch.int64, device=dev)
    if tuple(load.shape) != (L, E) or tuple(n_invalid.shape) != (L,):
        raise ValueError("load must be [L, E] and n_invalid [L]")
    rc = lib.eplb_load_hist(_dev(idx, torch.int32, "idx"), L, T, K, E,
                            _dev(ring, torch.int32, "ring"), W, int(step),
                            _dev(load, torch.int64, "load"), _dev(n_invalid, torch.int64, "n_invalid"),
                            _stream(dev))
    _check(rc, "eplb_load_hist")
    return load, n_invalid


def max_count(E: int, P: int, G: int, N: int) -> int:
    """Largest replica count a placement can give one expert (the least
    log2phy width rebalance accepts), from eplb_rebalance_max_count."""
    n = lib.eplb_rebalance_max_count(int(E), int(P), int(G), int(N))
    if n < 0:
        raise EplbError(-n, "eplb_rebalance_max_count")
    return n


def rebalance(load: torch.Tensor, P: int, G: int, N: int, RK: int, X: int | None = None,
              out: tuple | None = None):
    """Replica placement for every row of ``load`` ([B, E] int64).

    Returns (phy2log [B, P], log2phy [B, E, X], logcnt [B, E], status [B]),
    all int32.  X defaults to the largest possible count.
    """
    if load.dim() != 2:
        raise ValueError("load must be [B, E]")
    B, E = load.shape
    if X is None:
        X = max_count(E, P, G, N)
    dev = load.device
    if out is None:
        out = (torch.empty((B, P), dtype=torch.int32, device=dev),
               torch.empty((B, E, X), dtype=torch.int32, device=dev),
               torch.empty((B, E), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    phy2log, log2phy, logcnt, status = out
    if (tuple(phy2log.shape) != (B, P) or tuple(log2phy.shape) != (B, E, X)
            or tuple(logcnt.shape) != (B, E) or tuple(status.shape) != (B,)):
        raise ValueError("output shapes must be [B, P], [B, E, X], [B, E], [B]")
    rc = lib.eplb_rebalance(_dev(load, torch.int64, "load"), B, E, P, G, N, RK, X,
                            _dev(phy2log, torch.int32, "phy2log"), _dev(log2phy, torch.int32, "log2phy"),
                            _dev(logcnt, torch.int32, "logcnt"), _dev(status, torch.int32, "status"),
                            _stream(dev))
    _check(rc, "eplb_rebalance")
    return phy2log, log2phy, logcnt, status


def rebalance_experts(weight: torch.Tensor, num_replicas: int, num_groups: int, num_nodes: int, num_gpus: int):
    """The pages' interface to the rebalance (EPLB README translation,
    «DualPipe и EPLB», Part 2, section "Интерфейс и пример"): the same
    arguments and the same three maps, for a caller switching from it.

    weight [layers, E]: token counts per logical expert, any integer dtype or
    a floating dtype holding whole numbers, on the GPU or the host (a host
    tensor is copied to the current GPU).  Returns int64 (phy2log [layers,
    num_replicas], log2phy [layers, E, max logcnt], logcnt [layers, E]) on
    weight's device; log2phy is as wide as the largest replica count, as the
    pages' function returns it, which costs one device-to-host read.  A load
    outside [0, 2^40] raises EplbError.
    """
    if weight.dim() != 2:
        raise ValueError("weight must be [layers, experts]")
    if weight.is_floating_point() and not bool(torch.equal(weight, torch.trunc(weight))):
        raise ValueError("weight must hold whole token counts")
    if weight.is_floating_point() and weight.numel() and float(weight.abs().max()) >= 2.0 ** 62:
        raise ValueError("weight holds values that do not convert to int64")
    dev = weight.device if weight.device.type == "cuda" else torch.device("cuda", torch.cuda.current_device())
    load = weight.to(device=dev, dtype=torch.int64).contiguous()
    phy2log, log2phy, logcnt, status = rebalance(load, num_replicas, num_groups, num_nodes, num_gpus)
    bad = status.ne(0).nonzero()
    if bad.numel():
        raise EplbError(int(status[bad[0, 0]]), f"eplb_rebalance (layer {int(bad[0, 0])})")
    width = int(logcnt.max()) if logcnt.numel() else 1
    out = (phy2log.long(), log2phy[:, :, :width].long(), logcnt.long())
    return tuple(t.to(weight.device) for t in out)


def redirect(idx: torch.Tensor, log2phy: torch.Tensor, logcnt: torch.Tensor,
             out: torch.Tensor | None = None) -> torch.Tensor:
    """Physical replica of every routed (token, k): [L, T, K] int32."""
    if idx.dim() != 3 or log2phy.dim() != 3 or logcnt.dim() != 2:
        raise ValueError("idx [L, T, K], log2phy [L, E, X], logcnt [L, E] expected")
    L, T, K = idx.shape
    _, E, X = log2phy.shape
    if log2phy.shape[0] != L or tuple(logcnt.shape) != (L, E):
        raise ValueError("log2phy / logcnt do not match idx's layers")
    if out is None:
        out = torch.empty_like(idx)
    if out.shape != idx.shape:
        raise ValueError("out must have idx's shape")
    rc = lib.eplb_redirect(_dev(idx, torch.int32, "idx"), L, T, K, E,
                           _dev(log2phy, torch.int32, "log2phy"), _dev(logcnt, torch.int32, "logcnt"), X,
                           _dev(out, torch.int32, "out"), _stream(idx.device))
    _check(rc, "eplb_redirect")
    return out


def hist_redirect(idx: torch.Tensor, E: int, ring: torch.Tensor, step: int,
                  log2phy: torch.Tensor, logcnt: torch.Tensor, load: torch.Tensor | None = None,
                  n_invalid: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """load_hist and redirect in one pass over idx (the placement given is the
    one in force for this step).  Returns (load, n_invalid, out)."""
    if idx.dim() != 3 or log2phy.dim() != 3 or logcnt.dim() != 2:
        raise ValueError("idx [L, T, K], log2phy [L, E, X], logcnt [L, E] expected")
    L, T, K = idx.shape
    if ring.dim() != 3 or ring.shape[1] != L or ring.shape[2] != E:
        raise ValueError(f"ring must be [W, {L}, {E}], got {tuple(ring.shape)}")
    if tuple(log2phy.shape[:2]) != (L, E) or tuple(logcnt.shape) != (L, E):
        raise ValueError("log2phy / logcnt do not match idx's layers and E")
    W, X = ring.shape[0], log2phy.shape[2]
    dev = idx.device
    if load is None:
        load = torch.empty((L, E), dtype=torch.int64, device=dev)
    if n_invalid is None:
        n_invalid = torch.empty((L,), dtype=torch.int64, device=dev)
    if out is None:
        out = torch.empty_like(idx)
    if tuple(load.shape) != (L, E) or tuple(n_invalid.shape) != (L,) or out.shape != idx.shape:
        raise ValueError("load [L, E], n_invalid [L], out like idx expected")
    rc = lib.eplb_hist_redirect(_dev(idx, torch.int32, "idx"), L, T, K, E, _dev(ring, torch.int32, "ring"), W,
                                int(step), _dev(load, torch.int64, "load"),
                                _dev(n_invalid, torch.int64, "n_invalid"), _dev(log2phy, torch.int32, "log2phy"),
                                _dev(logcnt, torch.int32, "logcnt"), X, _dev(out, torch.int32, "out"),
                                _stream(dev))
    _check(rc, "eplb_hist_redirect")
    return load, n_invalid, out


def load_ema(idx: torch.Tensor, E: int, ema: torch.Tensor, shift: int,
             count: torch.Tensor | None = None, n_invalid: torch.Tensor | None = None):
    """Count one step's routing ids and fold them into an integer moving
    average: ema <- ema - (ema >> shift) + count, in place.

    idx [L, T, K] int32; ema [L, E] int64 (zeroed once by the caller).
    Returns (ema, count [L, E] int32, n_invalid [L] int64).
    """
    if idx.dim() != 3:
        raise ValueError("idx must be [L, T, K]")
    L, T, K = idx.shape
    if tuple(ema.shape) != (L, E):
        raise ValueError(f"ema must be [{L}, {E}], got {tuple(ema.shape)}")
    dev = idx.device
    if count is None:
        count = torch.empty((L, E), dtype=torch.int32, device=dev)
    if n_invalid is None:
        n_invalid = torch.empty((L,), dtype=torch.int64, device=dev)
    if tuple(count.shape) != (L, E) or tuple(n_invalid.shape) != (L,):
        raise ValueError("count must be [L, E] and n_invalid [L]")
    rc = lib.eplb_load_ema(_dev(idx, torch.int32, "idx"), L, T, K, E, _dev(count, torch.int32, "count"),
                           int(shift), _dev(ema, torch.int64, "ema"), _dev(n_invalid, torch.int64, "n_invalid"),
                           _stream(dev))
    _check(rc, "eplb_load_ema")
    return ema, count, n_invalid


def ema_redirect(idx: torch.Tensor, E: int, ema: torch.Tensor, shift: int, log2phy: torch.Tensor,
                 logcnt: torch.Tensor, count: torch.Tensor | None = None, n_invalid: torch.Tensor | None = None,
                 out: torch.Tensor | None = None):
    """load_ema and redirect in one pass over idx (the placement given is the
    one in force for this step).  Returns (ema, count, n_invalid, out)."""
    if idx.dim() != 3 or log2phy.dim() != 3 or logcnt.dim() != 2:
        raise ValueError("idx [L, T, K], log2phy [L, E, X], logcnt [L, E] expected")
    L, T, K = idx.shape
    if tuple(ema.shape) != (L, E):
        raise ValueError(f"ema must be [{L}, {E}], got {tuple(ema.shape)}")
    if tuple(log2phy.shape[:2]) != (L, E) or tuple(logcnt.shape) != (L, E):
        raise ValueError("log2phy / logcnt do not match idx's layers and E")
    X = log2phy.shape[2]
    dev = idx.device
    if count is None:
        count = torch.empty((L, E), dtype=torch.int32, device=dev)
    if n_invalid is None:
        n_invalid = torch.empty((L,), dtype=torch.int64, device=dev)
    if out is None:
        out = torch.empty_like(idx)
    if tuple(count.shape) != (L, E) or tuple(n_invalid.shape) != (L,) or out.shape != idx.shape:
        raise ValueError("count [L, E], n_invalid [L], out like idx expected")
    rc = lib.eplb_ema_redirect(_dev(idx, torch.int32, "idx"), L, T, K, E, _dev(count, torch.int32, "count"),
                               int(shift), _dev(ema, torch.int64, "ema"), _dev(n_invalid, torch.int64, "n_invalid"),
                               _dev(log2phy, torch.int32, "log2phy"), _dev(logcnt, torch.int32, "logcnt"), X,
                               _dev(out, torch.int32, "out"), _stream(dev))
    _check(rc, "eplb_ema_redirect")
    return ema, count, n_invalid, out


def placement_load(load: torch.Tensor, phy2log: torch.Tensor, logcnt: torch.Tensor, RK: int,
                   out: tuple | None = None):
    """Load of every rank under a placement and its max / mean.

    load [B, E] int64, phy2log [B, P] int32, logcnt [B, E] int32.
    Returns (rank_load [B, RK] float64, imbalance [B] float64); NaN marks a
    problem with an invalid load or map.
    """
    if load.dim() != 2 or phy2log.dim() != 2 or logcnt.dim() != 2:
        raise ValueError("load [B, E], phy2log [B, P], logcnt [B, E] expected")
    B, E = load.shape
    P = phy2log.shape[1]
    if phy2log.shape[0] != B or tuple(logcnt.shape) != (B, E):
        raise ValueError("phy2log / logcnt do not match load")
    dev = load.device
    if out is None:
        out = (torch.empty((B, RK), dtype=torch.float64, device=dev),
               torch.empty((B,), dtype=torch.float64, device=dev))
    rank_load, imbalance = out
    if tuple(rank_load.shape) != (B, RK) or tuple(imbalance.shape) != (B,):
        raise ValueError("outputs must be [B, RK] and [B]")
    rc = lib.eplb_placement_load(_dev(load, torch.int64, "load"), _dev(phy2log, torch.int32, "phy2log"),
                                 _dev(logcnt, torch.int32, "logcnt"), B, E, P, int(RK),
                                 _dev(rank_load, torch.float64, "rank_load"),
                                 _dev(imbalance, torch.float64, "imbalance"), _stream(dev))
    _check(rc, "eplb_placement_load")
    return rank_load, imbalance


def rearrange(old_phy2log: torch.Tensor, new_phy2log: torch.Tensor, new_log2phy: torch.Tensor, RK: int, N: int,
              out: tuple | None = None):
    """Plan of weight copies from the placement in force to a new one.

    old_phy2log, new_phy2log [B, P] int32; new_log2phy [B, E, X] int32.
    Returns (phy2log [B, P], log2phy [B, E, X], src [B, P], moves [B, 3],
    status [B]), all int32: the new placement permuted within ranks so that
    every replica that can stay does, and for each changed slot the old slot
    to copy from (-1 where nothing moves).
    """
    if old_phy2log.dim() != 2 or new_phy2log.dim() != 2 or new_log2phy.dim() != 3:
        raise ValueError("old_phy2log [B, P], new_phy2log [B, P], new_log2phy [B, E, X] expected")
    B, P = new_phy2log.shape
    _, E, X = new_log2phy.shape
    if tuple(old_phy2log.shape) != (B, P) or new_log2phy.shape[0] != B:
        raise ValueError("the three maps must describe the same B problems and P slots")
    dev = new_phy2log.device
    if out is None:
        out = (torch.empty((B, P), dtype=torch.int32, device=dev),
               torch.empty((B, E, X), dtype=torch.int32, device=dev),
               torch.empty((B, P), dtype=torch.int32, device=dev),
               torch.empty((B, 3), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    phy2log, log2phy, src, moves, status = out
    if (tuple(phy2log.shape) != (B, P) or tuple(log2phy.shape) != (B, E, X) or tuple(src.shape) != (B, P)
            or tuple(moves.shape) != (B, 3) or tuple(status.shape) != (B,)):
        raise ValueError("output shapes must be [B, P], [B, E, X], [B, P], [B, 3], [B]")
    rc = lib.eplb_rearrange(_dev(old_phy2log, torch.int32, "old_phy2log"), _dev(new_phy2log, torch.int32, "new_phy2log"),
                            _dev(new_log2phy, torch.int32, "new_log2phy"), B, E, P, int(RK), int(N), X,
                            _dev(phy2log, torch.int32, "phy2log"), _dev(log2phy, torch.int32, "log2phy"),
                            _dev(src, torch.int32, "src"), _dev(moves, torch.int32, "moves"),
                            _dev(status, torch.int32, "status"), _stream(dev))
    _check(rc, "eplb_rearrange")
    return phy2log, log2phy, src, moves, status


def lp_solve(cnt: torch.Tensor, home: torch.Tensor, rep: torch.Tensor, out: tuple | None = None):
    """Per-batch redistribution of tokens over replica edges.

    cnt [B, E] int64 (tokens per expert in the batch), home [B, E] int32
    (rank of each expert's original), rep [B, RK, R] int32 (expert in each
    replica slot, or -1).  Returns (lam [B] int64, flow [B, RK, R] int64,
    rank_load [B, RK] int64, status [B] int32).
    """
    if cnt.dim() != 2 or home.dim() != 2 or rep.dim() != 3:
        raise ValueError("cnt [B, E], home [B, E], rep [B, RK, R] expected")
    B, E = cnt.shape
    _, RK, R = rep.shape
    if tuple(home.shape) != (B, E) or rep.shape[0] != B:
        raise ValueError("cnt, home and rep must describe the same B problems")
    dev = cnt.device
    if out is None:
        out = (torch.empty((B,), dtype=torch.int64, device=dev),
               torch.empty((B, RK, R), dtype=torch.int64, device=dev),
               torch.empty((B, RK), dtype=torch.int64, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    lam, flow, rank_load, status = out
    if (tuple(lam.shape) != (B,) or tuple(flow.shape) != (B, RK, R) or tuple(rank_load.shape) != (B, RK)
            or tuple(status.shape) != (B,)):
        raise ValueError("output shapes must be [B], [B, RK, R], [B, RK], [B]")
    rc = lib.eplb_lp_solve(_dev(cnt, torch.int64, "cnt"), _dev(home, torch.int32, "home"),
                           _dev(rep, torch.int32, "rep"), B, E, RK, R, _dev(lam, torch.int64, "lam"),
                           _dev(flow, torch.int64, "flow"), _dev(rank_load, torch.int64, "rank_load"),
                           _dev(status, torch.int32, "status"), _stream(dev))
    _check(rc, "eplb_lp_solve")
    return lam, flow, rank_load, status


def lp_redirect_workspace_bytes(L: int, T: int, K: int, E: int) -> int:
    n = lib.eplb_lp_redirect_workspace_bytes(L, T, K, E)
    if n < 0:
        raise EplbError(-n, "eplb_lp_redirect_workspace_bytes")
    return n


def lp_redirect(idx: torch.Tensor, E: int, rep: torch.Tensor, flow: torch.Tensor,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Physical expert of every (token, k) under the flows of lp_solve:
    [L, T, K] int32.  ``workspace`` (any dtype, contiguous, on the GPU) must
    hold lp_redirect_workspace_bytes(L, T, K, E) bytes; one is made if absent."""
    if idx.dim() != 3 or rep.dim() != 3 or flow.dim() != 3:
        raise ValueError("idx [L, T, K], rep [L, RK, R], flow [L, RK, R] expected")
    L, T, K = idx.shape
    _, RK, R = rep.shape
    if rep.shape[0] != L or tuple(flow.shape) != tuple(rep.shape):
        raise ValueError("rep and flow must be [L, RK, R] for idx's layers")
    need = lp_redirect_workspace_bytes(L, T, K, E)
    if workspace is None:
        workspace = torch.empty((max(need, 4),), dtype=torch.uint8, device=idx.device)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if out is None:
        out = torch.empty_like(idx)
    if out.shape != idx.shape:
        raise ValueError("out must have idx's shape")
    rc = lib.eplb_lp_redirect(_dev(idx, torch.int32, "idx"), L, T, K, E, _dev(rep, torch.int32, "rep"),
                              _dev(flow, torch.int64, "flow"), RK, R, workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), _dev(out, torch.int32, "out"),
                              _stream(idx.device))
    _check(rc, "eplb_lp_redirect")
    return out


NOALLOC_SCRATCH_BYTES = 4 * 1024 * 1024


def lp_redirect_noalloc(idx: torch.Tensor, E: int, rep: torch.Tensor, flow: torch.Tensor,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """lp_redirect without a workspace: the counts live in the library's
    fixed per-GPU array (NOALLOC_SCRATCH_BYTES).  Calls that overlap in time
    on one GPU race; calls on one stream are safe."""
    if idx.dim() != 3 or rep.dim() != 3 or flow.dim() != 3:
        raise ValueError("idx [L, T, K], rep [L, RK, R], flow [L, RK, R] expected")
    L, T, K = idx.shape
    _, RK, R = rep.shape
    if rep.shape[0] != L or tuple(flow.shape) != tuple(rep.shape):
        raise ValueError("rep and flow must be [L, RK, R] for idx's layers")
    if out is None:
        out = torch.empty_like(idx)
    if out.shape != idx.shape:
        raise ValueError("out must have idx's shape")
    rc = lib.eplb_lp_redirect_noalloc(_dev(idx, torch.int32, "idx"), L, T, K, E, _dev(rep, torch.int32, "rep"),
                                      _dev(flow, torch.int64, "flow"), RK, R, _dev(out, torch.int32, "out"),
                                      _stream(idx.device))
    _check(rc, "eplb_lp_redirect_noalloc")
    return out
