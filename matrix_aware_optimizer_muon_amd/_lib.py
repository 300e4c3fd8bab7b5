"""ctypes binding of libmuon.so (include/muon.h).

Argument marshalling only: every step of the optimizer runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing the import of the binding
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARGUMENT = 1
MUON_ERR_UNSUPPORTED = 2
MUON_ERR_WORKSPACE_TOO_SMALL = 3
MUON_ERR_HIP = 4

MUON_F32 = 0
MUON_BF16 = 1

NOALLOC_WORKSPACE_BYTES = 64 << 20  # MUON_NOALLOC_WORKSPACE_BYTES

EXPORTED = ("muon_default_hparams", "muon_plan", "muon_plan_destroy", "muon_plan_workspace_size",
            "muon_plan_info", "muon_plan_bucket_info", "muon_step_batched",
            "muon_step_batched_noalloc", "rownorm_step", "muon_plan_set_profiling",
            "muon_plan_kernel_times", "muon_status_string")
KERNEL_CLASSES = ("prep", "norm", "syrk", "poly", "pqpg", "ph", "final", "rownorm", "colsum",
                  "colfinal", "colapply", "xcast", "xupd", "wupd")
FORMULATIONS = {"auto": 0, "gram": 1, "direct": 2}


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class Hparams(ctypes.Structure):
    _fields_ = [("momentum", ctypes.c_float), ("nesterov", ctypes.c_int),
                ("ns_steps", ctypes.c_int), ("a", ctypes.c_float), ("b", ctypes.c_float),
                ("c", ctypes.c_float), ("scale_coeff", ctypes.c_float),
                ("rownorm_eps", ctypes.c_float)]


class BucketHint(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("tile", ctypes.c_int),
                ("formulation", ctypes.c_int), ("group", ctypes.c_int), ("xcd_chunk", ctypes.c_int),
                ("waves", ctypes.c_int)]


class BucketInfo(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("count", ctypes.c_int64),
                ("chunks", ctypes.c_int64), ("tile", ctypes.c_int), ("formulation", ctypes.c_int),
                ("transposed", ctypes.c_int), ("fused_recursion", ctypes.c_int),
                ("operand_scales", ctypes.c_float * 5), ("group", ctypes.c_int),
                ("xcd_chunk", ctypes.c_int), ("waves", ctypes.c_int)]


class PlanDesc(ctypes.Structure):
    _fields_ = [("num_matrices", ctypes.c_int64), ("rows", ctypes.POINTER(ctypes.c_int64)),
                ("cols", ctypes.POINTER(ctypes.c_int64)), ("grad_dtype", ctypes.c_int),
                ("ns_dtype", ctypes.c_int), ("hp", Hparams),
                ("max_workspace_bytes", ctypes.c_int64), ("formulation", ctypes.c_int),
                ("hints", ctypes.POINTER(BucketHint)), ("num_hints", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libmuon.so from the package directory (built in place)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    # torch first: it brings the HIP runtime the process uses (its bundled
    # copy), which libmuon.so then binds to.  Loaded first, libmuon.so would
    # pull in the system copy as well, and one of the two runtimes then finds
    # no device (hipHostMalloc: "no ROCm-capable device is detected").
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.muon_default_hparams.argtypes = [ctypes.POINTER(Hparams)]
    lib.muon_plan.argtypes = [ctypes.POINTER(PlanDesc), ctypes.POINTER(P),
                              ctypes.POINTER(ctypes.c_size_t)]
    lib.muon_plan_destroy.argtypes = [P]
    lib.muon_plan_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.muon_plan_info.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.muon_plan_bucket_info.argtypes = [P, ctypes.c_int64, ctypes.POINTER(BucketInfo)]
    step_args = [P, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P), ctypes.c_float,
                 ctypes.c_float, P, ctypes.c_size_t, P, ctypes.POINTER(P)]
    lib.muon_step_batched.argtypes = step_args
    lib.rownorm_step.argtypes = step_args
    lib.muon_step_batched_noalloc.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(P),
                                              ctypes.POINTER(P), ctypes.c_float, ctypes.c_float,
                                              P, ctypes.POINTER(P)]
    lib.muon_plan_set_profiling.argtypes = [P, ctypes.c_int]
    D = ctypes.POINTER(ctypes.c_double)
    lib.muon_plan_kernel_times.argtypes = [P, D, ctypes.POINTER(ctypes.c_int64), D, D]
    lib.muon_status_string.argtypes = [ctypes.c_int]
    lib.muon_status_string.restype = ctypes.c_char_p
    for name in ("muon_default_hparams", "muon_plan", "muon_plan_destroy",
                 "muon_plan_workspace_size", "muon_plan_info", "muon_plan_bucket_info",
                 "muon_step_batched", "muon_step_batched_noalloc",
                 "rownorm_step", "muon_plan_set_profiling", "muon_plan_kernel_times"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().muon_status_string(int(status)).decode()


def default_hparams() -> Hparams:
    hp = Hparams()
    st = load().muon_default_hparams(ctypes.byref(hp))
    if st != MUON_OK:
        raise MuonError(st, "muon_default_hparams")
    return hp


def _ptr_array(ptrs: Sequence[Optional[int]]):
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = p if p else None
    return arr


class Plan:
    """A planned set of matrices (muon_plan).  `shapes` is a list of (m, n).

    grad_dtype / ns_dtype are "f32" or "bf16"; formulation is "auto", "gram"
    or "direct" (or the muon_formulation value).  `hints` maps a shape (m, n)
    to {"tile": 0|64|128|256, "formulation": "auto"|"gram"|"direct",
    "group": 0..64, "xcd_chunk": -1..65536, "waves": 0|4|8} (muon_bucket_hint;
    missing keys are 0, the planner's rule)."""

    def __init__(self, shapes: Sequence[tuple], grad_dtype: str = "f32", ns_dtype: str = "bf16",
                 hp: Optional[Hparams] = None, max_workspace_bytes: int = 0,
                 formulation: str = "auto", hints: Optional[dict] = None):
        lib = load()
        self._lib = lib
        self.shapes = [(int(m), int(n)) for m, n in shapes]
        n = len(self.shapes)
        rows = (ctypes.c_int64 * max(n, 1))(*[s[0] for s in self.shapes])
        cols = (ctypes.c_int64 * max(n, 1))(*[s[1] for s in self.shapes])
        desc = PlanDesc()
        desc.num_matrices = n
        desc.rows = ctypes.cast(rows, ctypes.POINTER(ctypes.c_int64))
        desc.cols = ctypes.cast(cols, ctypes.POINTER(ctypes.c_int64))
        desc.grad_dtype = {"f32": MUON_F32, "bf16": MUON_BF16}[grad_dtype]
        desc.ns_dtype = {"f32": MUON_F32, "bf16": MUON_BF16}[ns_dtype]
        desc.hp = hp if hp is not None else default_hparams()
        desc.max_workspace_bytes = int(max_workspace_bytes)
        desc.formulation = FORMULATIONS[formulation] if isinstance(formulation, str) else int(formulation)
        items = list((hints or {}).items())
        harr = (BucketHint * max(len(items), 1))()
        for i, ((m, n), h) in enumerate(items):
            f = h.get("formulation", "auto")
            harr[i] = BucketHint(int(m), int(n), int(h.get("tile", 0)),
                                 FORMULATIONS[f] if isinstance(f, str) else int(f),
                                 int(h.get("group", 0)), int(h.get("xcd_chunk", 0)),
                                 int(h.get("waves", 0)))
        desc.hints = ctypes.cast(harr, ctypes.POINTER(BucketHint)) if items else None
        desc.num_hints = len(items)
        self.hp = desc.hp
        self.grad_dtype, self.ns_dtype = grad_dtype, ns_dtype
        handle = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        st = lib.muon_plan(ctypes.byref(desc), ctypes.byref(handle), ctypes.byref(ws))
        if st != MUON_OK:
            raise MuonError(st, "muon_plan")
        self._handle = handle
        self.workspace_bytes = int(ws.value)

    def info(self) -> tuple[int, int]:
        nb, nc = ctypes.c_int64(), ctypes.c_int64()
        st = self._lib.muon_plan_info(self._handle, ctypes.byref(nb), ctypes.byref(nc))
        if st != MUON_OK:
            raise MuonError(st, "muon_plan_info")
        return int(nb.value), int(nc.value)

    def buckets(self) -> list:
        """The planner's decision per bucket (muon_plan_bucket_info)."""
        names = {v: k for k, v in FORMULATIONS.items()}
        out = []
        for i in range(self.info()[0]):
            b = BucketInfo()
            st = self._lib.muon_plan_bucket_info(self._handle, i, ctypes.byref(b))
            if st != MUON_OK:
                raise MuonError(st, "muon_plan_bucket_info")
            out.append({"shape": (int(b.rows), int(b.cols)), "count": int(b.count),
                        "chunks": int(b.chunks), "tile": int(b.tile),
                        "formulation": names[int(b.formulation)], "transposed": bool(b.transposed),
                        "fused": bool(b.fused_recursion),
                        "scales": tuple(float(x) for x in b.operand_scales),
                        "group": int(b.group), "xcd_chunk": int(b.xcd_chunk),
                        "waves": int(b.waves)})
        return out

    def _call(self, fn, name, W, M, G, lr, wd, workspace_ptr, workspace_bytes, stream, out):
        n = len(self.shapes)
        if not (len(W) == len(M) == len(G) == n):
            raise ValueError(f"expected {n} matrices")
        o_arr = _ptr_array(out) if out is not None else None
        st = fn(self._handle, _ptr_array(W), _ptr_array(M), _ptr_array(G), ctypes.c_float(lr),
                ctypes.c_float(wd), ctypes.c_void_p(workspace_ptr), ctypes.c_size_t(workspace_bytes),
                ctypes.c_void_p(stream or 0), o_arr)
        if st != MUON_OK:
            raise MuonError(st, name)

    def step_ptrs(self, W, M, G, lr, wd, workspace_ptr, workspace_bytes, stream=0, O_out=None):
        """muon_step_batched on raw device pointers."""
        self._call(self._lib.muon_step_batched, "muon_step_batched", W, M, G, lr, wd,
                   workspace_ptr, workspace_bytes, stream, O_out)

    def step_noalloc_ptrs(self, W, M, G, lr, wd, stream=0, O_out=None):
        """muon_step_batched_noalloc on raw device pointers (the library's own
        per-GPU scratch instead of a workspace)."""
        n = len(self.shapes)
        if not (len(W) == len(M) == len(G) == n):
            raise ValueError(f"expected {n} matrices")
        o_arr = _ptr_array(O_out) if O_out is not None else None
        st = self._lib.muon_step_batched_noalloc(
            self._handle, _ptr_array(W), _ptr_array(M), _ptr_array(G), ctypes.c_float(lr),
            ctypes.c_float(wd), ctypes.c_void_p(stream or 0), o_arr)
        if st != MUON_OK:
            raise MuonError(st, "muon_step_batched_noalloc")

    def rownorm_ptrs(self, W, M, G, lr, wd, workspace_ptr, workspace_bytes, stream=0, R_out=None):
        """rownorm_step on raw device pointers."""
        self._call(self._lib.rownorm_step, "rownorm_step", W, M, G, lr, wd, workspace_ptr,
                   workspace_bytes, stream, R_out)

    def set_profiling(self, enable: bool):
        st = self._lib.muon_plan_set_profiling(self._handle, 1 if enable else 0)
        if st != MUON_OK:
            raise MuonError(st, "muon_plan_set_profiling")

    def kernel_times(self) -> dict:
        """Per kernel class: total ms, launches, algorithmic flops and bytes
        accumulated since profiling was enabled (waits for the events)."""
        n = len(KERNEL_CLASSES)
        ms, fl, by = (ctypes.c_double * n)(), (ctypes.c_double * n)(), (ctypes.c_double * n)()
        la = (ctypes.c_int64 * n)()
        st = self._lib.muon_plan_kernel_times(self._handle, ms, la, fl, by)
        if st != MUON_OK:
            raise MuonError(st, "muon_plan_kernel_times")
        return {k: {"ms": ms[i], "launches": int(la[i]), "flops": fl[i], "bytes": by[i]}
                for i, k in enumerate(KERNEL_CLASSES) if la[i] > 0}

    def close(self):
        if getattr(self, "_handle", None):
            self._lib.muon_plan_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

