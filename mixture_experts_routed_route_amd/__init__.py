"""
Python binding of the MI355X routed mixture-of-experts FFN layer.

A thin ctypes layer over ``libmoe_mi355x.so`` (C ABI in ``include/moe.h``):
it marshals torch tensors into pointers and sizes, takes the current HIP
stream, and allocates the caller-owned workspaces with ``torch.empty``.
Every step of the layer runs in the library's HIP kernels; there is no
fallback. If the library is not built, every call raises.

    plan = moe_plan_create(logits, k=8, capacity_factor=0.0)
    y = moe_forward(plan, x, w_gate, w_up, w_down)

or, with the router map in the same call (logits = x . w_router^T and the
routing statistics beside the plan):

    plan, logits, stats = moe_route(x, w_router, k=8)

Weights are torch tensors [E (+1 shared), F, D] / [E (+1), D, F] in x's dtype,
or, for 4-bit weights, ``(packed uint8 [.., N, K/2], params fp16)`` pairs:
params [.., N, K/32] are the block scales of the signed format, params
[.., N, K/G, 2] the (scale, bias) pairs of the affine format with groups of
G = 32 or 64 K values (the format follows from the params' shape).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_F16, MOE_Q4B32 = 0, 1, 2, 3
MOE_Q4A32, MOE_Q4A64 = 4, 5
MOE_OPT_PHASE_EVENTS = 1
MOE_OPT_BF16_PLAIN_H = 2
MOE_OPT_EXACT_ROUTES = 4
MOE_OPT_BF16_SPLIT_H = 8
MOE_OPT_ONE_STREAM = 16
MOE_OPT_TILED_DECODE = 32
MOE_OPT_PHASE_SHIFT = 16


def MOE_OPT_PHASE_ONLY(p: int) -> int:
    """Option bit: with MOE_OPT_PHASE_EVENTS, record phase p (see PHASES);
    any such bit set limits the recording to the phases selected."""
    v = 1 << (MOE_OPT_PHASE_SHIFT + p)
    return v - (1 << 32) if v >= (1 << 31) else v   # the int32 flags field
MOE_N_PHASES = 16
PHASES = ("classify", "dequant_once", "gateup_full", "gateup_thin16",
          "down_full", "down_thin16", "combine", "router_gemm", "route_plan",
          "router_stats", "bwd_recompute", "bwd_data", "bwd_weights",
          "bwd_routing", "gateup_thin64", "down_thin64")

STATUS_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EUNSUPPORTED",
                -3: "MOE_EWORKSPACE", -4: "MOE_EHIP"}

_TORCH_TO_MOE = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16,
                 torch.float16: MOE_F16}

EXPORTED = (
    "moe_plan_workspace_bytes", "moe_plan_create", "moe_plan_stats_get",
    "moe_plan_get_views", "moe_plan_destroy", "moe_options_default",
    "moe_forward_workspace_bytes", "moe_forward", "moe_dequant_q4",
    "moe_phase_times", "moe_last_error", "moe_version",
    "moe_route_workspace_bytes", "moe_route", "moe_dequant_weights",
    "moe_backward_workspace_bytes", "moe_backward", "moe_forward_get_views",
    "moe_forward_noalloc",
)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

ROUTE_STATS = ("kept_mass", "want_k", "z_loss", "balance", "aux")


class PlanDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("capacity_factor", ctypes.c_float)]


class Options(ctypes.Structure):
    _fields_ = [("swiglu_limit", ctypes.c_float),
                ("splitk_max_pairs", ctypes.c_float),
                ("fat_rows", ctypes.c_int32), ("flags", ctypes.c_int32)]


class Weight(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


class PlanStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "T", "E", "k", "n_shared", "limit", "pairs", "kept", "dropped",
        "touched", "max_rows", "nonfinite", "thin", "full", "fat")] + [
        ("drop_fraction", ctypes.c_double)]


class PlanViews(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_id", "topk_w", "slot", "tok2pair", "counts", "offsets",
        "pair_token", "pair_w", "stats")]


class ForwardViews(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("h_lo", ctypes.c_void_p),
                ("h_ld", ctypes.c_int64), ("ht", ctypes.c_void_p),
                ("ht_lo", ctypes.c_void_p), ("pairs_max", ctypes.c_int64),
                ("ypair", ctypes.c_void_p), ("ypair_dtype", ctypes.c_int32),
                ("fat_slot", ctypes.c_void_p),
                ("fat_copy", ctypes.c_void_p * 3),
                ("fat_slots", ctypes.c_int64)]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def library(path: str = LIB_PATH):
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with __graft_entry__.build() or "
            "python mixture_experts_routed_route_amd/build.py")
    L = ctypes.CDLL(path)
    vp, sz, i32, i64 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                        ctypes.c_int64)
    L.moe_plan_workspace_bytes.argtypes = [ctypes.POINTER(PlanDesc)]
    L.moe_plan_workspace_bytes.restype = sz
    L.moe_plan_create.argtypes = [ctypes.POINTER(PlanDesc), vp, vp, sz, vp,
                                  ctypes.POINTER(vp)]
    L.moe_plan_create.restype = i32
    L.moe_plan_stats_get.argtypes = [vp, ctypes.POINTER(Options),
                                     ctypes.POINTER(PlanStats), vp]
    L.moe_plan_stats_get.restype = i32
    L.moe_plan_get_views.argtypes = [vp, ctypes.POINTER(PlanViews)]
    L.moe_plan_get_views.restype = i32
    L.moe_plan_destroy.argtypes = [vp]
    L.moe_plan_destroy.restype = None
    L.moe_options_default.argtypes = [ctypes.POINTER(Options)]
    L.moe_options_default.restype = None
    L.moe_forward_workspace_bytes.argtypes = [vp, i32, i32, i32, i32,
                                              ctypes.POINTER(Options)]
    L.moe_forward_workspace_bytes.restype = sz
    L.moe_forward.argtypes = [vp, vp, i32, Weight, Weight, Weight, i32, i32,
                              vp, i32, vp, sz, ctypes.POINTER(Options), vp]
    L.moe_forward.restype = i32
    L.moe_forward_noalloc.argtypes = [vp, vp, i32, Weight, Weight, Weight, i32,
                                      i32, vp, i32, ctypes.POINTER(Options), vp]
    L.moe_forward_noalloc.restype = i32
    L.moe_forward_get_views.argtypes = [vp, i32, i32, i32, i32,
                                        ctypes.POINTER(Options), vp,
                                        ctypes.POINTER(ForwardViews)]
    L.moe_forward_get_views.restype = i32
    L.moe_dequant_q4.argtypes = [vp, vp, i64, i64, vp, vp]
    L.moe_dequant_q4.restype = i32
    L.moe_dequant_weights.argtypes = [i32, vp, vp, i64, i64, vp, vp]
    L.moe_dequant_weights.restype = i32
    L.moe_phase_times.argtypes = [ctypes.POINTER(ctypes.c_double), i32,
                                  ctypes.POINTER(i64), i32]
    L.moe_phase_times.restype = i32
    L.moe_route_workspace_bytes.argtypes = [ctypes.POINTER(PlanDesc), i32]
    L.moe_route_workspace_bytes.restype = sz
    L.moe_route.argtypes = [ctypes.POINTER(PlanDesc), vp, i32, vp, i32,
                            ctypes.c_float, vp, vp, vp, vp, sz, i32, vp,
                            ctypes.POINTER(vp)]
    L.moe_route.restype = i32
    L.moe_backward_workspace_bytes.argtypes = [vp, i32, i32, i32]
    L.moe_backward_workspace_bytes.restype = sz
    L.moe_backward.argtypes = [vp, vp, i32, Weight, Weight, Weight, i32, i32,
                               vp, vp, vp, vp, vp, vp, vp, vp, sz,
                               ctypes.POINTER(Options), vp]
    L.moe_backward.restype = i32
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_version.argtypes = []
    L.moe_version.restype = ctypes.c_char_p
    _lib = L
    return L


def moe_last_error() -> str:
    return library().moe_last_error().decode()


def moe_version() -> str:
    return library().moe_version().decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, moe_last_error())


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def moe_options_default() -> Options:
    o = Options()
    library().moe_options_default(ctypes.byref(o))
    return o


def make_options(swiglu_limit=None, splitk_max_pairs=None, fat_rows=None,
                 flags=None, exact_routes=False) -> Options:
    """Options with the defaults, except what is given. exact_routes sets
    MOE_OPT_EXACT_ROUTES (the S rule alone decides split-K vs full)."""
    o = moe_options_default()
    if swiglu_limit is not None:
        o.swiglu_limit = float(swiglu_limit)
    if splitk_max_pairs is not None:
        o.splitk_max_pairs = float(splitk_max_pairs)
    if fat_rows is not None:
        o.fat_rows = int(fat_rows)
    if flags is not None:
        o.flags = int(flags)
    if exact_routes:
        o.flags |= MOE_OPT_EXACT_ROUTES
    return o


class Plan:
    """A dispatch plan: host handle + its device workspace (kept alive)."""

    def __init__(self, handle, ws, logits, desc: PlanDesc):
        self.handle = handle
        self.ws = ws
        self.logits = logits
        self.desc = desc
        self.T, self.E, self.k = desc.T, desc.E, desc.k
        self.n_shared = desc.n_shared
        self.capacity_factor = desc.capacity_factor

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:
            _lib.moe_plan_destroy(h)


def moe_plan_workspace_bytes(T, E, k, capacity_factor=0.0, n_shared=0) -> int:
    d = PlanDesc(T, E, k, n_shared, capacity_factor)
    return int(library().moe_plan_workspace_bytes(ctypes.byref(d)))


def moe_plan_create(logits: torch.Tensor, k: int, capacity_factor: float = 0.0,
                    n_shared: int = 0,
                    workspace: torch.Tensor | None = None) -> Plan:
    """Route f32 logits [T, E] (device) and build the dispatch plan.

    Pass ``workspace`` (uint8, device) to reuse one buffer across plans."""
    L = library()
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a 2-D float32 tensor")
    logits = logits.contiguous()
    T, E = logits.shape
    d = PlanDesc(T, E, int(k), int(n_shared), float(capacity_factor))
    nbytes = L.moe_plan_workspace_bytes(ctypes.byref(d))
    if nbytes == 0:
        raise MoeError(MOE_EINVAL, moe_last_error())
    if workspace is not None and workspace.numel() >= nbytes:
        ws = workspace
    else:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=logits.device)
    h = ctypes.c_void_p()
    _check(L.moe_plan_create(ctypes.byref(d), logits.data_ptr(), ws.data_ptr(),
                             nbytes, _stream(logits.device), ctypes.byref(h)))
    return Plan(h, ws, logits, d)


def moe_route_workspace_bytes_for(T: int, E: int, k: int, D: int,
                                  capacity_factor: float = 0.0,
                                  n_shared: int = 0) -> int:
    d = PlanDesc(T, E, k, n_shared, capacity_factor)
    return int(library().moe_route_workspace_bytes(ctypes.byref(d), D))


def moe_route(x: torch.Tensor, w_router: torch.Tensor, k: int,
              capacity_factor: float = 0.0, n_shared: int = 0,
              z_weight: float = 1e-3, want_per_token: bool = False,
              workspace: torch.Tensor | None = None, flags: int = 0,
              logits: torch.Tensor | None = None,
              stats: torch.Tensor | None = None):
    """logits = x . w_router^T (f32 [T, E]), the plan over them, and the
    routing statistics as a device f32 tensor [8] (kept_mass, want_k, z_loss,
    balance, aux, 0, 0, 0). Returns (plan, logits, stats), plus the per-token
    wanted counts (int32 [T]) when ``want_per_token``."""
    L = library()
    if x.dtype not in _TORCH_TO_MOE or x.dim() != 2:
        raise ValueError("x must be a 2-D float32/bfloat16/float16 tensor")
    if w_router.dtype != x.dtype or w_router.dim() != 2 \
            or w_router.shape[1] != x.shape[1] or w_router.device != x.device:
        raise ValueError("w_router must be [E, D] in x's dtype, on x's device")
    x, w_router = x.contiguous(), w_router.contiguous()
    T, D = x.shape
    E = w_router.shape[0]
    d = PlanDesc(T, E, int(k), int(n_shared), float(capacity_factor))
    nbytes = L.moe_route_workspace_bytes(ctypes.byref(d), D)
    if nbytes == 0:
        raise MoeError(MOE_EINVAL, moe_last_error())
    if workspace is not None and workspace.numel() >= nbytes:
        ws = workspace
    else:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    if logits is None:
        logits = torch.empty(T, E, dtype=torch.float32, device=x.device)
    if logits.shape != (T, E) or logits.dtype != torch.float32 \
            or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous float32 [T, E] tensor")
    if stats is None:
        stats = torch.empty(8, dtype=torch.float32, device=x.device)
    want = (torch.empty(T, dtype=torch.int32, device=x.device)
            if want_per_token else None)
    h = ctypes.c_void_p()
    _check(L.moe_route(ctypes.byref(d), x.data_ptr(), _TORCH_TO_MOE[x.dtype],
                       w_router.data_ptr(), D, float(z_weight),
                       logits.data_ptr(), stats.data_ptr(),
                       None if want is None else want.data_ptr(),
                       ws.data_ptr(), nbytes, int(flags), _stream(x.device),
                       ctypes.byref(h)))
    plan = Plan(h, ws, logits, d)
    return (plan, logits, stats, want) if want_per_token else (plan, logits, stats)


def moe_plan_stats_get(plan: Plan, options: Options | None = None) -> dict:
    st = PlanStats()
    o = options or moe_options_default()
    _check(library().moe_plan_stats_get(plan.handle, ctypes.byref(o),
                                        ctypes.byref(st),
                                        _stream(plan.ws.device)))
    return {n: getattr(st, n) for n, _ in PlanStats._fields_}


def moe_plan_get_views(plan: Plan) -> dict:
    """torch views of the plan's device arrays (inside its workspace)."""
    v = PlanViews()
    _check(library().moe_plan_get_views(plan.handle, ctypes.byref(v)))
    base = plan.ws.data_ptr()
    T, k = plan.T, plan.k
    n_exp = plan.E + plan.n_shared

    def view(ptr, n, dtype):
        off = ptr - base
        size = torch.tensor([], dtype=dtype).element_size()
        return plan.ws[off:off + n * size].view(dtype)

    out = {
        "topk_id": view(v.topk_id, T * k, torch.int32).view(T, k),
        "topk_w": view(v.topk_w, T * k, torch.float32).view(T, k),
        "slot": view(v.slot, T * k, torch.int32).view(T, k),
        "tok2pair": view(v.tok2pair, T * k, torch.int32).view(T, k),
        "counts": view(v.counts, n_exp, torch.int32),
        "offsets": view(v.offsets, n_exp + 1, torch.int32),
        "stats": view(v.stats, 8, torch.int64),
    }
    P = int(out["offsets"][-1].item())
    out["pair_token"] = view(v.pair_token, P, torch.int32)
    out["pair_w"] = view(v.pair_w, P, torch.float32)
    return out


def q4_dtype(data: torch.Tensor, params: torch.Tensor) -> int:
    """The 4-bit format of a (packed, params) pair, from the params' shape:
    [.., N, K/32] scales -> MOE_Q4B32; [.., N, K/G, 2] (scale, bias) pairs
    -> MOE_Q4A32 or MOE_Q4A64 by G."""
    K = data.shape[-1] * 2
    if params.dim() == data.dim() and params.shape[-1] * 32 == K:
        return MOE_Q4B32
    if params.dim() == data.dim() + 1 and params.shape[-1] == 2:
        groups = params.shape[-2]
        if groups * 32 == K:
            return MOE_Q4A32
        if groups * 64 == K:
            return MOE_Q4A64
    raise ValueError(f"4-bit params of shape {tuple(params.shape)} do not "
                     f"match packed data of shape {tuple(data.shape)}")


def _weight(w, device) -> tuple:
    if isinstance(w, (tuple, list)):
        data, scales = w
        if data.dtype != torch.uint8 or scales.dtype != torch.float16:
            raise ValueError("4-bit weights are (uint8 data, float16 params)")
        if data.device != device or scales.device != device:
            raise ValueError("weights must be on the input's device")
        data, scales = data.contiguous(), scales.contiguous()
        return (Weight(q4_dtype(data, scales), data.data_ptr(), scales.data_ptr()),
                (data, scales))
    if w.dtype not in _TORCH_TO_MOE:
        raise ValueError(f"unsupported weight dtype {w.dtype}")
    if w.device != device:
        raise ValueError("weights must be on the input's device")
    w = w.contiguous()
    return Weight(_TORCH_TO_MOE[w.dtype], w.data_ptr(), None), (w,)


def _dims(w_gate):
    if isinstance(w_gate, (tuple, list)):
        data = w_gate[0]
        return data.shape[1], data.shape[2] * 2      # F, D
    return w_gate.shape[1], w_gate.shape[2]


def _check_weight_shapes(plan, w_gate, w_up, w_down, D: int, F: int):
    """W_gate, W_up [n, F, D] and W_down [n, D, F] (4-bit: packed [.., K/2]
    with matching params) with n >= E + n_shared experts, one format: a
    mismatched tensor would otherwise be read out of bounds on the device."""
    n_need = plan.E + plan.n_shared
    want = {"w_gate": (F, D), "w_up": (F, D), "w_down": (D, F)}
    fmt = None
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        N, K = want[name]
        if isinstance(w, (tuple, list)):
            data, params = w
            if data.dim() != 3 or tuple(data.shape[1:]) != (N, K // 2):
                raise ValueError(f"{name} packed data must be [n, {N}, {K // 2}], "
                                 f"got {tuple(data.shape)}")
            if tuple(params.shape[:2]) != tuple(data.shape[:2]):
                raise ValueError(f"{name} params {tuple(params.shape)} do not "
                                 f"match its data {tuple(data.shape)}")
            f = q4_dtype(data, params)
        else:
            if w.dim() != 3 or tuple(w.shape[1:]) != (N, K):
                raise ValueError(f"{name} must be [n, {N}, {K}], got {tuple(w.shape)}")
            data, f = w, w.dtype
        if data.shape[0] < n_need:
            raise ValueError(f"{name} holds {data.shape[0]} experts, the plan "
                             f"needs {n_need} (E + n_shared)")
        if fmt is not None and f != fmt:
            raise ValueError("w_gate, w_up and w_down must share one format")
        fmt = f


def moe_forward_workspace_bytes(plan: Plan, D: int, F: int, x_dtype: int,
                                w_dtype: int, options: Options | None = None) -> int:
    o = options or moe_options_default()
    return int(library().moe_forward_workspace_bytes(
        plan.handle, D, F, x_dtype, w_dtype, ctypes.byref(o)))


def moe_forward(plan: Plan, x: torch.Tensor, w_gate, w_up, w_down,
                options: Options | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None,
                y_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """y [T, D] in f32 (the residual stream's dtype) or in x's dtype.

    Pass ``workspace`` (and ``out``) to reuse buffers across calls."""
    L = library()
    if x.dtype not in _TORCH_TO_MOE or x.dim() != 2:
        raise ValueError("x must be a 2-D float32/bfloat16/float16 tensor")
    x = x.contiguous()
    T, D = x.shape
    if T != plan.T:
        raise ValueError(f"x has {T} tokens, the plan {plan.T}")
    F, Dw = _dims(w_gate)
    if Dw != D:
        raise ValueError(f"weights have d_model {Dw}, x has {D}")
    _check_weight_shapes(plan, w_gate, w_up, w_down, D, F)
    o = options or moe_options_default()
    wg, keep_g = _weight(w_gate, x.device)
    wu, keep_u = _weight(w_up, x.device)
    wd, keep_d = _weight(w_down, x.device)
    xdt = _TORCH_TO_MOE[x.dtype]
    nbytes = L.moe_forward_workspace_bytes(plan.handle, D, F, xdt, wg.dtype,
                                           ctypes.byref(o))
    if nbytes == 0:
        raise MoeError(MOE_EUNSUPPORTED, moe_last_error())
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty(T, D, dtype=y_dtype, device=x.device)
    if out.dtype not in (torch.float32, x.dtype) or out.shape != (T, D) \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, D] f32 or x-dtype tensor")
    _check(L.moe_forward(plan.handle, x.data_ptr(), xdt, wg, wu, wd, D, F,
                         out.data_ptr(), _TORCH_TO_MOE[out.dtype],
                         workspace.data_ptr(),
                         workspace.numel(), ctypes.byref(o),
                         _stream(x.device)))
    return out


def moe_forward_noalloc(plan: Plan, x: torch.Tensor, w_gate, w_up, w_down,
                        options: Options | None = None,
                        out: torch.Tensor | None = None,
                        y_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """moe_forward with the library's own per-GPU scratch as its workspace
    (no device allocation inside the call; pass ``out`` to allocate nothing
    here either). Calls that overlap on one GPU race on that scratch."""
    L = library()
    if x.dtype not in _TORCH_TO_MOE or x.dim() != 2:
        raise ValueError("x must be a 2-D float32/bfloat16/float16 tensor")
    x = x.contiguous()
    T, D = x.shape
    if T != plan.T:
        raise ValueError(f"x has {T} tokens, the plan {plan.T}")
    F, Dw = _dims(w_gate)
    if Dw != D:
        raise ValueError(f"weights have d_model {Dw}, x has {D}")
    _check_weight_shapes(plan, w_gate, w_up, w_down, D, F)
    o = options or moe_options_default()
    wg, keep_g = _weight(w_gate, x.device)
    wu, keep_u = _weight(w_up, x.device)
    wd, keep_d = _weight(w_down, x.device)
    if out is None:
        out = torch.empty(T, D, dtype=y_dtype, device=x.device)
    if out.dtype not in (torch.float32, x.dtype) or out.shape != (T, D) \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, D] f32 or x-dtype tensor")
    _check(L.moe_forward_noalloc(plan.handle, x.data_ptr(), _TORCH_TO_MOE[x.dtype],
                                 wg, wu, wd, D, F, out.data_ptr(),
                                 _TORCH_TO_MOE[out.dtype], ctypes.byref(o),
                                 _stream(x.device)))
    return out


def moe_forward_get_views(plan: Plan, workspace: torch.Tensor, D: int, F: int,
                          x_dtype: torch.dtype, w_dtype: int,
                          options: Options | None = None) -> dict:
    """torch views of a forward workspace after a moe_forward call with the
    same plan, sizes, dtypes and options: ``ypair`` [P, D] (unweighted
    per-pair outputs, rows in the plan's pair order), ``h`` [P, h_ld] (thin
    routes' SwiGLU output), ``ht`` [F/32, P, 32] (full tile's), and for 4-bit
    fat routes ``fat_slot`` [E + n_shared] and ``fat_copy`` (three uint16
    views [n_slots, K/32, N, 32] of the fp16 copies of W_gate, W_up,
    W_down)."""
    v = ForwardViews()
    o = options or moe_options_default()
    xdt = _TORCH_TO_MOE[x_dtype]
    _check(library().moe_forward_get_views(plan.handle, D, F, xdt, int(w_dtype),
                                           ctypes.byref(o),
                                           workspace.data_ptr(),
                                           ctypes.byref(v)))
    base = workspace.data_ptr()
    P = int(v.pairs_max)
    n_exp = plan.E + plan.n_shared

    def view(ptr, n, dtype):
        off = ptr - base
        size = torch.tensor([], dtype=dtype).element_size()
        return workspace[off:off + n * size].view(dtype)

    yd = torch.float16 if v.ypair_dtype == MOE_F16 else torch.float32
    out = {"ypair": view(v.ypair, P * D, yd).view(P, D),
           "h": view(v.h, P * int(v.h_ld), x_dtype).view(P, int(v.h_ld))}
    if v.h_lo:
        out["h_lo"] = view(v.h_lo, P * int(v.h_ld), x_dtype).view(P, int(v.h_ld))
    if v.ht:
        out["ht"] = view(v.ht, P * F, x_dtype).view(F // 32, P, 32)
    if v.ht_lo:
        out["ht_lo"] = view(v.ht_lo, P * F, x_dtype).view(F // 32, P, 32)
    if v.fat_slot:
        out["fat_slot"] = view(v.fat_slot, n_exp, torch.int32)
    if v.fat_copy[0]:
        dims = ((F, D), (F, D), (D, F))
        n_slots = int(v.fat_slots)
        copies = []
        for m in range(3):
            N, K = dims[m]
            copies.append(view(v.fat_copy[m], n_slots * N * K, torch.int16)
                          .view(n_slots, K // 32, N, 32))
        out["fat_copy"] = copies
    return out


def moe_backward(plan: Plan, x: torch.Tensor, w_gate, w_up, w_down,
                 dy: torch.Tensor, options: Options | None = None,
                 want_dtw: bool = False, want_dlogits: bool = False,
                 workspace: torch.Tensor | None = None) -> dict:
    """Gradients of sum(dy * y) for the layer moe_forward computes with the
    same plan, x and 16-bit weights: dx [T, D], dw_gate / dw_up [E(+1), F,
    D], dw_down [E(+1), D, F] (f32), and optionally d_topk_w [T, k] and
    d_logits [T, E]."""
    L = library()
    if x.dtype not in (torch.bfloat16, torch.float16) or x.dim() != 2:
        raise ValueError("backward takes a 2-D bfloat16/float16 x")
    x = x.contiguous()
    T, D = x.shape
    if T != plan.T:
        raise ValueError(f"x has {T} tokens, the plan {plan.T}")
    if isinstance(w_gate, (tuple, list)):
        raise ValueError("backward takes 16-bit weights (4-bit ones are frozen)")
    F = w_gate.shape[1]
    _check_weight_shapes(plan, w_gate, w_up, w_down, D, F)
    dy = dy.to(torch.float32).contiguous()
    if dy.shape != (T, D) or dy.device != x.device:
        raise ValueError("dy must be [T, D] on x's device")
    o = options or moe_options_default()
    wg, keep_g = _weight(w_gate, x.device)
    wu, keep_u = _weight(w_up, x.device)
    wd, keep_d = _weight(w_down, x.device)
    xdt = _TORCH_TO_MOE[x.dtype]
    nbytes = L.moe_backward_workspace_bytes(plan.handle, D, F, xdt)
    if nbytes == 0:
        raise MoeError(MOE_EUNSUPPORTED, moe_last_error())
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    n_exp = plan.E + plan.n_shared
    f32 = dict(dtype=torch.float32, device=x.device)
    out = dict(dx=torch.empty(T, D, **f32),
               dw_gate=torch.empty(n_exp, F, D, **f32),
               dw_up=torch.empty(n_exp, F, D, **f32),
               dw_down=torch.empty(n_exp, D, F, **f32))
    if want_dtw:
        out["d_topk_w"] = torch.empty(T, plan.k, **f32)
    if want_dlogits:
        out["d_logits"] = torch.empty(T, plan.E, **f32)
    ptr = lambda name: out[name].data_ptr() if name in out else None
    _check(L.moe_backward(plan.handle, x.data_ptr(), xdt, wg, wu, wd, D, F,
                          dy.data_ptr(), ptr("dx"), ptr("dw_gate"), ptr("dw_up"),
                          ptr("dw_down"), ptr("d_topk_w"), ptr("d_logits"),
                          workspace.data_ptr(), workspace.numel(),
                          ctypes.byref(o), _stream(x.device)))
    return out


def moe_dequant_q4(data: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """fp16_rne(q * s) of [.., N, K/2] 4-bit rows; returns [.., N, K] fp16."""
    if data.dtype != torch.uint8 or scales.dtype != torch.float16:
        raise ValueError("expects uint8 data and float16 scales")
    data, scales = data.contiguous(), scales.contiguous()
    K = data.shape[-1] * 2
    rows = data.numel() // data.shape[-1]
    out = torch.empty(*data.shape[:-1], K, dtype=torch.float16,
                      device=data.device)
    _check(library().moe_dequant_q4(data.data_ptr(), scales.data_ptr(), rows,
                                    K, out.data_ptr(), _stream(data.device)))
    return out


def moe_dequant_weights(data: torch.Tensor, params: torch.Tensor) -> torch.Tensor:
    """fp16 of [.., N, K/2] 4-bit rows in any format (the params' shape
    picks it): fp16_rne(q * s) or fp16_rne(q * s + b); returns [.., N, K]."""
    if data.dtype != torch.uint8 or params.dtype != torch.float16:
        raise ValueError("expects uint8 data and float16 params")
    data, params = data.contiguous(), params.contiguous()
    dt = q4_dtype(data, params)
    K = data.shape[-1] * 2
    rows = data.numel() // data.shape[-1]
    out = torch.empty(*data.shape[:-1], K, dtype=torch.float16,
                      device=data.device)
    _check(library().moe_dequant_weights(dt, data.data_ptr(), params.data_ptr(),
                                         rows, K, out.data_ptr(),
                                         _stream(data.device)))
    return out


def moe_phase_times(reset: bool = True) -> tuple:
    """(ms per phase summed over recorded calls, number of calls)."""
    ms = (ctypes.c_double * MOE_N_PHASES)()
    calls = ctypes.c_int64()
    _check(library().moe_phase_times(ms, MOE_N_PHASES, ctypes.byref(calls),
                                     1 if reset else 0))
    return dict(zip(PHASES, list(ms))), int(calls.value)


# short aliases
plan = moe_plan_create
forward = moe_forward
route = moe_route
backward = moe_backward
