"""ctypes binding of libcefn.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  PyTorch supplies device memory and the stream.  Importing
this module fails loudly when the shared library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcefn.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_OOM, MOE_ERR_HIP = range(5)
DTYPE = {"f32": 0, "f16": 1, "bf16": 2}
RESID = {"none": 0, "f32": 1, "f16": 2, "int4_g32": 3}
ACT = {"gelu_tanh": 0, "swiglu": 1}


class moe_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "T_max", "d", "f", "G", "K", "top_groups", "top_experts", "r",
        "act", "x_dtype", "base_dtype", "resid")]


class moe_weights(C.Structure):
    _fields_ = [("W_grp", C.c_void_p), ("W_exp", C.c_void_p),
                ("group_bias", C.c_void_p), ("expert_bias", C.c_void_p),
                ("base", C.c_void_p * 3), ("A", C.c_void_p * 3), ("B", C.c_void_p * 3)]


class moe_route_out(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "idx", "w", "gidx", "counts", "offsets", "perm", "gcounts", "goffsets", "gperm")]


class moe_stats(C.Structure):
    _fields_ = [("stored_params", C.c_int64), ("stored_bytes", C.c_int64),
                ("dense_equiv_params", C.c_int64)]


class MoEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m compressed_expert_ffn_amd.build`")
    # PyTorch ships its own HIP runtime under the same soname as the system
    # one this library links.  Only one can live in a process; load torch's
    # first so the library and torch share it (the other order leaves torch
    # unable to see the GPU).
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    sig = {
        "moe_create": ([C.POINTER(moe_config), C.POINTER(moe_weights), P, C.POINTER(P)], C.c_int),
        "moe_route": ([P, P, C.c_int32, C.POINTER(moe_route_out), P], C.c_int),
        "moe_forward": ([P, P, C.c_int32, P, C.POINTER(moe_route_out), P], C.c_int),
        "moe_destroy": ([P], C.c_int),
        "moe_last_error": ([], C.c_char_p),
        "moe_config_stats": ([C.POINTER(moe_config), C.POINTER(moe_stats)], C.c_int),
        "moe_debug_residual": ([P, C.c_int32, C.c_int32, C.c_int32, P, P, P], C.c_int),
        "moe_profile_begin": ([P, C.c_int32, C.c_int32], C.c_int),
        "moe_profile_end": ([P, P, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                             C.c_char_p, C.c_int32], C.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def check(rc: int):
    if rc != MOE_OK:
        raise MoEError(rc, lib.moe_last_error().decode())


def make_config(T_max, d, f, G, K, top_groups, top_experts, r, act, x_dtype, base_dtype,
                resid) -> moe_config:
    return moe_config(T_max, d, f, G, K, top_groups, top_experts, r, ACT[act],
                      DTYPE[x_dtype], DTYPE[base_dtype], RESID[resid])


def config_from_workload(w, T_max=None) -> moe_config:
    return make_config(w.T if T_max is None else T_max, w.d, w.f, w.G, w.K, w.top_groups,
                       w.top_experts, w.r, w.act, w.x_dtype, w.base_dtype, w.resid)


def config_stats(cfg: moe_config) -> dict:
    st = moe_stats()
    check(lib.moe_config_stats(C.byref(cfg), C.byref(st)))
    return dict(stored_params=st.stored_params, stored_bytes=st.stored_bytes,
                dense_equiv_params=st.dense_equiv_params)


def _host_ptr(a, keep):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    keep.append(a)
    return a.ctypes.data


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


class Layer:
    """One created layer (a moe_handle) plus torch-side buffer marshalling.

    inputs: the host arrays of one layer (X is not needed), in the layout
    include/moe.h documents; fp16 arrays as numpy float16, bf16 as uint16 bits.
    """

    def __init__(self, cfg: moe_config, inputs: dict):
        keep = []
        w = moe_weights()
        w.W_grp = _host_ptr(np.asarray(inputs["W_grp"], dtype=np.float32), keep)
        w.W_exp = _host_ptr(None if inputs.get("W_exp") is None
                            else np.asarray(inputs["W_exp"], dtype=np.float32), keep)
        w.group_bias = _host_ptr(None if inputs.get("group_bias") is None
                                 else np.asarray(inputs["group_bias"], dtype=np.float32), keep)
        w.expert_bias = _host_ptr(None if inputs.get("expert_bias") is None
                                  else np.asarray(inputs["expert_bias"], dtype=np.float32), keep)
        for p, b in enumerate(inputs["base"]):
            w.base[p] = _host_ptr(b, keep)
        for p, a in enumerate(inputs.get("A") or []):
            w.A[p] = _host_ptr(a, keep)
        for p, b in enumerate(inputs.get("B") or []):
            w.B[p] = _host_ptr(b, keep)
        self.cfg = cfg
        self.E = cfg.G * cfg.K
        self.k = cfg.top_groups * cfg.top_experts
        h = C.c_void_p()
        check(lib.moe_create(C.byref(cfg), C.byref(w), None, C.byref(h)))
        self.h = h

    # ----------------------------------------------------------------------
    def _torch_x_dtype(self):
        import torch
        return {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[self.cfg.x_dtype]

    def route_buffers(self, T: int, device="cuda"):
        import torch
        i32 = dict(dtype=torch.int32, device=device)
        return dict(idx=torch.empty((T, self.k), **i32),
                    w=torch.empty((T, self.k), dtype=torch.float32, device=device),
                    gidx=torch.empty((T, self.cfg.top_groups), **i32),
                    counts=torch.empty(self.E, **i32), offsets=torch.empty(self.E + 1, **i32),
                    perm=torch.empty(T * self.k, **i32), gcounts=torch.empty(self.cfg.G, **i32),
                    goffsets=torch.empty(self.cfg.G + 1, **i32),
                    gperm=torch.empty(T * self.cfg.top_groups, **i32))

    @staticmethod
    def _route_struct(bufs):
        ro = moe_route_out()
        if bufs is not None:
            for name, _ in moe_route_out._fields_:
                t = bufs.get(name)
                setattr(ro, name, None if t is None else t.data_ptr())
        return ro

    def route(self, X, bufs=None, stream=None):
        T = X.shape[0]
        bufs = self.route_buffers(T, X.device) if bufs is None else bufs
        ro = self._route_struct(bufs)
        check(lib.moe_route(self.h, C.c_void_p(X.data_ptr()), T, C.byref(ro), _stream_ptr(stream)))
        return bufs

    def forward(self, X, Y=None, route_bufs=None, stream=None):
        import torch
        T = X.shape[0]
        if Y is None:
            Y = torch.empty((T, self.cfg.d), dtype=self._torch_x_dtype(), device=X.device)
        ro = self._route_struct(route_bufs)
        rop = C.byref(ro) if route_bufs is not None else None
        check(lib.moe_forward(self.h, C.c_void_p(X.data_ptr()), T, C.c_void_p(Y.data_ptr()),
                              rop, _stream_ptr(stream)))
        return Y

    def debug_residual(self, proj: int, which: int, expert: int):
        """(values float32 [n, r], q int8 [n, r], scale fp16 bits [n/32, r])."""
        d, f, r = self.cfg.d, self.cfg.f, self.cfg.r
        P = 3 if self.cfg.act == ACT["swiglu"] else 2
        din, dout = (d, f) if proj < P - 1 else (f, d)
        n = din if which == 0 else dout
        vals = np.zeros((n, r), dtype=np.float32)
        q = np.zeros((n, r), dtype=np.int8)
        sc = np.zeros((n // 32, r), dtype=np.uint16)
        check(lib.moe_debug_residual(self.h, proj, which, expert, vals.ctypes.data,
                                     q.ctypes.data, sc.ctypes.data))
        return vals, q, sc

    STAGES = ("router", "scatter", "ugemm", "gemm1", "vreduce", "gemm2", "combine")

    def profile_begin(self, max_calls: int, stages=None):
        mask = -1 if stages is None else sum(1 << self.STAGES.index(s) for s in stages)
        check(lib.moe_profile_begin(self.h, max_calls, mask))

    def profile_end(self) -> dict:
        ms = (C.c_float * 16)()
        ns, nc = C.c_int32(), C.c_int32()
        names = C.create_string_buffer(256)
        check(lib.moe_profile_end(self.h, ms, 16, C.byref(ns), C.byref(nc), names, 256))
        keys = names.value.decode().split(",")
        return dict(calls=nc.value, stage_ms={k: ms[i] for i, k in enumerate(keys[:ns.value])})

    def close(self):
        if getattr(self, "h", None):
            lib.moe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
