"""ctypes binding of libdbs.so (C ABI in include/dbs.h).

Argument marshalling only: every step of a pass runs in the HIP kernels of
libdbs.so.  Tensors must be float32, contiguous, on a CUDA (HIP) device, of
shape [n,n] or [batch,n,n]; calls enqueue on the tensor device's current
torch stream and return without synchronising.  There is no CPU fallback:
without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libdbs.so")

ALGO_AUTO, ALGO_PERK, ALGO_LDS, ALGO_BLOCKED = 0, 1, 2, 3
_ALGOS = {"auto": ALGO_AUTO, "perk": ALGO_PERK, "lds": ALGO_LDS, "blocked": ALGO_BLOCKED}

CHECK_FLAGS = {
    "asym": 1, "diag": 2, "nonfinite": 4, "l_gt_u": 8, "l_neg": 16,
    "unquant": 32, "range": 64, "negzero": 128,
}

DBS_OK, DBS_EINVAL, DBS_EDEVICE, DBS_ELAUNCH, DBS_EUNSUPPORTED = 0, -1, -2, -3, -4

EXPORTS = ("dbs_options_init", "dbs_smooth_opts", "dbs_smooth_packed_opts", "dbs_schedule",
           "dbs_schedule_packed",
           "dbs_smooth", "dbs_smooth_algo", "dbs_smooth_profiled", "dbs_rounds", "dbs_round",
           "dbs_check", "dbs_smooth_range", "dbs_block_rounds", "dbs_tightened", "dbs_bounds_from_restraints",
           "dbs_pack", "dbs_unpack", "dbs_smooth_packed", "dbs_smooth_packed_range",
           "dbs_check_packed", "dbs_smooth_directed", "dbs_smooth_directed_range",
           "dbs_smooth_packed_directed_range", "dbs_lookahead_bands", "dbs_step_blocks",
           "dbs_lds_max_n", "dbs_auto_algo", "dbs_strerror", "dbs_version")

AUTO = -1


class Options(ctypes.Structure):
    """struct dbs_options (include/dbs.h): per-call options of a pass."""
    _fields_ = [("algo", ctypes.c_int32), ("directed", ctypes.c_int32),
                ("lookahead", ctypes.c_int32), ("step_blocks", ctypes.c_int32),
                ("lead", ctypes.c_int32), ("infeasible", ctypes.c_void_p)]


# bits of the infeasibility words (include/dbs.h)
INFEASIBLE_EARLY = 1
INFEASIBLE_END = 2


RESTRAINT_FLAGS = {"index": 1, "value": 2}

PROF_KINDS = ("round", "small", "panel", "tiles", "mirror", "strip", "fill", "scatter")


class DbsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load libdbs.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise ImportError(f"{SO_PATH} is missing: build it first "
                              "(python -m distance_geometry_bound_amd.build)")
        L = ctypes.CDLL(SO_PATH)
        vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.dbs_smooth.argtypes = [vp, vp, i64, i64, vp]
        L.dbs_smooth_algo.argtypes = [vp, vp, i64, i64, vp, c_int]
        opp = ctypes.POINTER(Options)
        L.dbs_options_init.argtypes = [opp]
        L.dbs_options_init.restype = None
        L.dbs_smooth_opts.argtypes = [vp, vp, i64, i64, i64, i64, vp, opp]
        L.dbs_smooth_packed_opts.argtypes = [vp, i64, i64, i64, i64, vp, opp]
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.dbs_schedule.argtypes = [i64, i64, opp, i32p, i32p, i32p]
        L.dbs_schedule_packed.argtypes = [i64, i64, opp, i32p, i32p, i32p]
        L.dbs_smooth_profiled.argtypes = [vp, vp, i64, i64, vp, opp,
                                          ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
        L.dbs_rounds.argtypes = [vp, vp, i64, i64, i64, i64, vp]
        L.dbs_round.argtypes = [vp, vp, i64, i64, i64, vp]
        L.dbs_smooth_range.argtypes = [vp, vp, i64, i64, i64, i64, vp, c_int]
        L.dbs_tightened.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp]
        L.dbs_pack.argtypes = [vp, vp, vp, i64, i64, vp]
        L.dbs_unpack.argtypes = [vp, vp, vp, i64, i64, vp]
        L.dbs_smooth_packed.argtypes = [vp, i64, i64, vp]
        L.dbs_smooth_packed_range.argtypes = [vp, i64, i64, i64, i64, vp]
        L.dbs_bounds_from_restraints.argtypes = [vp, vp, i64, i64, ctypes.c_float,
                                                 ctypes.c_float, vp, vp, vp, vp, vp, i64, vp, vp]
        L.dbs_check.argtypes = [vp, vp, i64, i64, vp, vp]          # ..., stream, d_flags
        L.dbs_check_packed.argtypes = [vp, i64, i64, vp, vp]      # ..., stream, d_flags
        L.dbs_smooth_directed.argtypes = [vp, vp, i64, i64, vp]
        L.dbs_smooth_directed_range.argtypes = [vp, vp, i64, i64, i64, i64, vp, c_int]
        L.dbs_smooth_packed_directed_range.argtypes = [vp, i64, i64, i64, i64, vp]
        L.dbs_auto_algo.argtypes = [i64, i64]
        L.dbs_lookahead_bands.argtypes = [i64, i64]
        L.dbs_step_blocks.argtypes = [i64, i64]
        L.dbs_strerror.argtypes = [c_int]
        L.dbs_strerror.restype = ctypes.c_char_p
        for f in ("dbs_smooth", "dbs_smooth_algo", "dbs_smooth_profiled", "dbs_rounds", "dbs_round",
                  "dbs_check",
                  "dbs_smooth_range", "dbs_block_rounds", "dbs_tightened",
                  "dbs_bounds_from_restraints", "dbs_pack", "dbs_unpack", "dbs_smooth_packed",
                  "dbs_smooth_packed_range", "dbs_check_packed", "dbs_smooth_directed",
                  "dbs_smooth_directed_range", "dbs_smooth_packed_directed_range",
                  "dbs_lds_max_n", "dbs_auto_algo", "dbs_lookahead_bands", "dbs_step_blocks",
                  "dbs_version", "dbs_smooth_opts", "dbs_smooth_packed_opts", "dbs_schedule",
                  "dbs_schedule_packed"):
            getattr(L, f).restype = c_int
        _lib = L
    return _lib


def _raise(status: int):
    if status == DBS_OK:
        return
    msg = lib().dbs_strerror(status).decode()
    if status in (DBS_EINVAL, DBS_EUNSUPPORTED):
        raise ValueError(f"{msg} (status {status})")
    raise DbsError(status, msg)


def _shape(U, L):
    import torch

    for name, T in (("U", U), ("L", L)):
        if not isinstance(T, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if T.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
        if T.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU")
        if not T.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if U.shape != L.shape or U.dim() not in (2, 3) or U.shape[-1] != U.shape[-2]:
        raise ValueError(f"U and L must be [n,n] or [batch,n,n] and equal; got "
                         f"{tuple(U.shape)} and {tuple(L.shape)}")
    if U.device != L.device:
        raise ValueError("U and L must be on the same device")
    n = U.shape[-1]
    batch = 1 if U.dim() == 2 else U.shape[0]
    return n, batch


def _stream(T):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(T.device).cuda_stream)


def _call(T, fn, *args):
    import torch

    with torch.cuda.device(T.device):
        _raise(fn(*args))


def options(algo: str = "auto", directed: bool = False, lookahead=None, step_blocks=None,
            lead=None, infeasible=None):
    """struct dbs_options for a pass: `lookahead` (0, 1, 2), `step_blocks`
    (1 .. 4) and `lead` (False, True) force the blocked schedule, None keeps
    the automatic choice.  `infeasible`: None, or an int32 device tensor of
    one word per molecule that the pass ORs INFEASIBLE_* bits into."""
    if algo not in _ALGOS:
        raise ValueError(f"algo must be one of {sorted(_ALGOS)}")
    return Options(_ALGOS[algo], 1 if directed else 0,
                   AUTO if lookahead is None else int(lookahead),
                   AUTO if step_blocks is None else int(step_blocks),
                   AUTO if lead is None else int(lead),
                   None if infeasible is None else infeasible.data_ptr())


def _check_words(W, batch, device):
    """The infeasibility words of a pass: None, or a contiguous int32 tensor of
    at least `batch` elements on the pass's device."""
    import torch

    if W is None:
        return
    if not isinstance(W, torch.Tensor) or W.dtype != torch.int32 or not W.is_contiguous():
        raise ValueError("infeasible must be a contiguous int32 tensor")
    if W.device != device or W.numel() < batch:
        raise ValueError(f"infeasible must hold {batch} words on {device}")


def _pass(U, L, k_begin, k_end, **kw):
    n, batch = _shape(U, L)
    _check_words(kw.get("infeasible"), batch, U.device)
    o = options(**kw)
    if n == 0 or batch == 0:
        return
    k_end = n if k_end is None else int(k_end)
    _call(U, lib().dbs_smooth_opts, U.data_ptr(), L.data_ptr(), n, batch, int(k_begin), k_end,
          _stream(U), ctypes.byref(o))


def smooth(U, L, algo: str = "auto", check: bool = False, lookahead=None,
           step_blocks=None, lead=None, infeasible=None) -> None:
    """One full smoothing pass on U, L in place (enqueued on the current stream).

    check=True first tests the preconditions on the device (dbs_check; this
    synchronises) and raises ValueError naming the violated ones.  lookahead
    and step_blocks force the blocked schedule; infeasible takes the
    per-molecule words of the infeasibility test (see options())."""
    n, batch = _shape(U, L)
    options(algo, False, lookahead, step_blocks, lead)
    if n == 0 or batch == 0:
        return
    if check:
        bad = _check_flags(U, L)
        if bad:
            names = [k for k, v in CHECK_FLAGS.items() if bad & v]
            raise ValueError(f"bounds violate the preconditions: {', '.join(names)}")
    _pass(U, L, 0, None, algo=algo, lookahead=lookahead, step_blocks=step_blocks, lead=lead,
          infeasible=infeasible)


def smooth_profiled(U, L, algo: str = "auto", directed: bool = False, lookahead=None,
                    step_blocks=None, lead=None) -> dict:
    """smooth() with HIP events around every kernel launch; synchronises and
    returns {kind: (launches, total_ms)} for the kernel kinds in PROF_KINDS."""
    n, batch = _shape(U, L)
    o = options(algo, directed, lookahead, step_blocks, lead)
    counts = (ctypes.c_int64 * len(PROF_KINDS))()
    ms = (ctypes.c_double * len(PROF_KINDS))()
    if n > 0 and batch > 0:
        _call(U, lib().dbs_smooth_profiled, U.data_ptr(), L.data_ptr(), n, batch, _stream(U),
              ctypes.byref(o), counts, ms)
    return {k: (int(counts[i]), float(ms[i])) for i, k in enumerate(PROF_KINDS)}


def smooth_rounds(U, L, k_begin: int, k_end: int) -> None:
    """Rounds k_begin..k_end-1 of a pass, one launch per round, in place."""
    n, batch = _shape(U, L)
    if n == 0 or batch == 0:
        return
    _call(U, lib().dbs_rounds, U.data_ptr(), L.data_ptr(), n, batch, int(k_begin),
          int(k_end), _stream(U))


def smooth_round(U, L, k: int) -> None:
    """Round k only (dbs_round)."""
    n, batch = _shape(U, L)
    if n == 0 or batch == 0:
        return
    _call(U, lib().dbs_round, U.data_ptr(), L.data_ptr(), n, batch, int(k), _stream(U))


def smooth_range(U, L, k_begin: int, k_end: int, algo: str = "auto", lookahead=None,
                 step_blocks=None, lead=None, infeasible=None) -> None:
    """Rounds k_begin..k_end-1 of a pass, in place (see dbs_smooth_range)."""
    _pass(U, L, k_begin, k_end, algo=algo, lookahead=lookahead, step_blocks=step_blocks,
          lead=lead, infeasible=infeasible)


def smooth_directed_range(U, L, k_begin: int, k_end: int, algo: str = "auto", lookahead=None,
                          step_blocks=None, lead=None, infeasible=None) -> None:
    """smooth_range with directed rounding: sums of upper bounds rounded up,
    differences of lower bounds rounded down (see dbs_smooth_directed_range)."""
    _pass(U, L, k_begin, k_end, algo=algo, directed=True, lookahead=lookahead,
          step_blocks=step_blocks, lead=lead, infeasible=infeasible)


def smooth_directed(U, L, algo: str = "auto", lookahead=None, step_blocks=None,
                    lead=None, infeasible=None) -> None:
    """A full pass with directed rounding, in place."""
    _pass(U, L, 0, None, algo=algo, directed=True, lookahead=lookahead, step_blocks=step_blocks,
          lead=lead, infeasible=infeasible)


def tightened(U0, L0, U1, L1):
    """uint8 mask of the cells whose U or L differs between two states."""
    import torch

    n, batch = _shape(U0, L0)
    if _shape(U1, L1) != (n, batch) or U1.device != U0.device:
        raise ValueError("the two states must have the same shape and device")
    mask = torch.empty(U0.shape, dtype=torch.uint8, device=U0.device)
    if n and batch:
        _call(U0, lib().dbs_tightened, U0.data_ptr(), L0.data_ptr(), U1.data_ptr(),
              L1.data_ptr(), n, batch, mask.data_ptr(), _stream(U0))
    return mask


def bounds_from_restraints(n: int, ia, ja, lo, hi, unknown_L: float, unknown_U: float,
                           mol=None, batch: int = 1, out=None):
    """Dense [batch,n,n] (U, L) from a restraint list (see dbs_bounds_from_restraints).

    ia, ja, mol: int32 tensors, lo, hi: float32 tensors, all on one GPU.
    out: optional (U, L) to write into; else new tensors on that GPU.
    Returns (U, L, status) with status the DBS_RESTRAINT_* bits (synchronises).
    """
    import torch

    dev = ia.device
    for name, t, dt in (("ia", ia, torch.int32), ("ja", ja, torch.int32),
                        ("lo", lo, torch.float32), ("hi", hi, torch.float32)):
        if t.dtype != dt or t.device != dev or not t.is_contiguous() or t.dim() != 1:
            raise ValueError(f"{name} must be a contiguous 1-D {dt} tensor on {dev}")
    count = ia.numel()
    if not (ja.numel() == lo.numel() == hi.numel() == count):
        raise ValueError("restraint arrays differ in length")
    if mol is not None and (mol.dtype != torch.int32 or mol.device != dev or
                            not mol.is_contiguous() or mol.numel() != count):
        raise ValueError("mol must be a contiguous int32 tensor like ia")
    if out is None:
        U = torch.empty((batch, n, n), dtype=torch.float32, device=dev)
        L = torch.empty_like(U)
    else:
        U, L = out
    n_, b_ = _shape(U, L)
    if (n_, b_) != (n, batch):
        raise ValueError("out has the wrong shape")
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    _call(U, lib().dbs_bounds_from_restraints, U.data_ptr(), L.data_ptr(), n, batch,
          float(unknown_L), float(unknown_U), mol.data_ptr() if mol is not None else None,
          ia.data_ptr(), ja.data_ptr(), lo.data_ptr(), hi.data_ptr(), count, status.data_ptr(),
          _stream(U))
    return U, L, int(status.item()) & 0xFFFFFFFF


def _shape1(P):
    import torch

    if not isinstance(P, torch.Tensor) or P.dtype != torch.float32:
        raise TypeError("P must be a float32 torch.Tensor")
    if P.device.type != "cuda" or not P.is_contiguous():
        raise ValueError("P must be a contiguous GPU tensor")
    if P.dim() not in (2, 3) or P.shape[-1] != P.shape[-2]:
        raise ValueError(f"P must be [n,n] or [batch,n,n], got {tuple(P.shape)}")
    return P.shape[-1], 1 if P.dim() == 2 else P.shape[0]


def pack(U, L, out=None):
    """Packed one-buffer form of symmetric U, L (see dbs_pack)."""
    import torch

    n, batch = _shape(U, L)
    P = torch.empty_like(U) if out is None else out
    if _shape1(P) != (n, batch):
        raise ValueError("out has the wrong shape")
    if n and batch:
        _call(U, lib().dbs_pack, U.data_ptr(), L.data_ptr(), P.data_ptr(), n, batch, _stream(U))
    return P


def unpack(P):
    """(U, L) from the packed form (see dbs_unpack)."""
    import torch

    n, batch = _shape1(P)
    U, L = torch.empty_like(P), torch.empty_like(P)
    if n and batch:
        _call(P, lib().dbs_unpack, P.data_ptr(), U.data_ptr(), L.data_ptr(), n, batch, _stream(P))
    return U, L


def _packed_pass(P, k_begin, k_end, **kw):
    n, batch = _shape1(P)
    _check_words(kw.get("infeasible"), batch, P.device)
    o = options(**kw)
    if n == 0 or batch == 0:
        return
    k_end = n if k_end is None else int(k_end)
    _call(P, lib().dbs_smooth_packed_opts, P.data_ptr(), n, batch, int(k_begin), k_end,
          _stream(P), ctypes.byref(o))


def smooth_packed(P, k_begin: int = 0, k_end=None, algo: str = "auto", lookahead=None,
                  step_blocks=None, lead=None, infeasible=None) -> None:
    """Rounds k_begin..k_end-1 (default: a full pass) on the packed form, in place."""
    _packed_pass(P, k_begin, k_end, algo=algo, lookahead=lookahead, step_blocks=step_blocks,
                 lead=lead, infeasible=infeasible)


def smooth_packed_directed(P, k_begin: int = 0, k_end=None, algo: str = "auto", lookahead=None,
                           step_blocks=None, lead=None, infeasible=None) -> None:
    """smooth_packed with directed rounding, in place."""
    _packed_pass(P, k_begin, k_end, algo=algo, directed=True, lookahead=lookahead,
                 step_blocks=step_blocks, lead=lead, infeasible=infeasible)


def _check_flags(U, L) -> int:
    """Precondition flags (CHECK_FLAGS bits) of U, L; synchronises the stream."""
    import torch

    n, batch = _shape(U, L)
    flags = torch.zeros(1, dtype=torch.int32, device=U.device)
    if n == 0 or batch == 0:
        return 0
    _call(U, lib().dbs_check, U.data_ptr(), L.data_ptr(), n, batch, _stream(U),
          flags.data_ptr())
    return int(flags.item()) & 0xFFFFFFFF


def check(U, L) -> int:
    """Precondition flags (CHECK_FLAGS bits) of U, L; synchronises the stream."""
    return _check_flags(U, L)


def check_packed(P) -> int:
    """Precondition flags of the pair a packed buffer stands for; synchronises."""
    import torch

    n, batch = _shape1(P)
    flags = torch.zeros(1, dtype=torch.int32, device=P.device)
    if n == 0 or batch == 0:
        return 0
    _call(P, lib().dbs_check_packed, P.data_ptr(), n, batch, _stream(P), flags.data_ptr())
    return int(flags.item()) & 0xFFFFFFFF


def schedule(n: int, batch: int = 1, lookahead=None, step_blocks=None, lead=None,
             packed: bool = False):
    """(look-ahead depth, k-blocks per step, lead schedule 0/1) of a blocked
    pass of this shape on the dense (or packed) layout, with the given forced
    values (None: automatic); see dbs_schedule and dbs_schedule_packed."""
    o = options("auto", False, lookahead, step_blocks, lead)
    la, sb, ld = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    f = lib().dbs_schedule_packed if packed else lib().dbs_schedule
    _raise(f(int(n), int(batch), ctypes.byref(o), ctypes.byref(la), ctypes.byref(sb),
             ctypes.byref(ld)))
    return int(la.value), int(sb.value), int(ld.value)


def lookahead_bands(n: int, batch: int = 1) -> int:
    """Steps the blocked pass updates ahead on its second stream (0, 1, 2)."""
    return int(lib().dbs_lookahead_bands(int(n), int(batch)))


def step_blocks(n: int, batch: int = 1) -> int:
    """k-blocks per step of the blocked pass (1 .. 4)."""
    return int(lib().dbs_step_blocks(int(n), int(batch)))


def auto_algo(n: int, batch: int = 1) -> str:
    code = lib().dbs_auto_algo(n, batch)
    return {v: k for k, v in _ALGOS.items()}[code]
