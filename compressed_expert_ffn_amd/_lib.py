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
                ("base", C.c_void_p * 3), ("A", C.c_void_p * 3), ("B", C.c_void_p * 3),
                ("on_device", C.c_int32)]


class moe_route_out(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "idx", "w", "gidx", "counts", "offsets", "perm", "gcounts", "goffsets", "gperm")]


class moe_stats(C.Structure):
    _fields_ = [("stored_params", C.c_int64), ("stored_bytes", C.c_int64),
                ("dense_equiv_params", C.c_int64)]


class moe_grads(C.Structure):
    _fields_ = [("dW_grp", C.c_void_p), ("dW_exp", C.c_void_p), ("d_group_bias", C.c_void_p),
                ("d_expert_bias", C.c_void_p), ("dbase", C.c_void_p * 3), ("dA", C.c_void_p * 3),
                ("dB", C.c_void_p * 3)]


class moe_offload_stats_t(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("calls", "group_loads", "group_hits", "prefetched", "bytes_h2d",
                                          "passes")]


class moe_cluster_config(C.Structure):
    _fields_ = [("E", C.c_int32), ("G", C.c_int32), ("d", C.c_int32), ("n_param", C.c_int64),
                ("alpha", C.c_double), ("beta", C.c_double), ("tau", C.c_double), ("eps", C.c_double),
                ("cache_life", C.c_int32)]


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
        "moe_forward_noalloc": ([P, P, C.c_int32, P, C.POINTER(moe_route_out), P], C.c_int),
        "moe_destroy": ([P], C.c_int),
        "moe_backward": ([P, P, C.c_int32, P, P, C.POINTER(moe_grads), P], C.c_int),
        "moe_offload_enable": ([P, C.c_int32], C.c_int),
        "moe_forward_offload": ([P, P, C.c_int32, P, C.POINTER(moe_route_out), P], C.c_int),
        "moe_offload_stats": ([P, C.POINTER(moe_offload_stats_t)], C.c_int),
        "moe_last_error": ([], C.c_char_p),
        "moe_config_stats": ([C.POINTER(moe_config), C.POINTER(moe_stats)], C.c_int),
        "moe_stats": ([P, C.POINTER(moe_stats)], C.c_int),
        "moe_debug_residual": ([P, C.c_int32, C.c_int32, C.c_int32, P, P, P], C.c_int),
        "moe_debug_dequant": ([P, C.c_int32, C.c_int32, C.c_int32, P], C.c_int),
        "moe_debug_q": ([P, C.c_int32, C.c_int32, C.c_int32, P, P], C.c_int),
        "moe_cluster_create": ([C.POINTER(moe_cluster_config), C.POINTER(P)], C.c_int),
        "moe_cluster_destroy": ([P], C.c_int),
        "moe_cluster_get_centroids": ([P, P], C.c_int),
        "moe_cluster_set_centroids": ([P, P], C.c_int),
        "moe_cluster_observe": ([P, P, C.c_int32, P, C.c_int32], C.c_int),
        "moe_cluster_regroup": ([P, P, P, P, P, P, P], C.c_int),
        "moe_compress_projection": ([C.c_int32, C.c_int32, P, C.c_int32, C.c_int32, C.c_int32, P, P, P, P, P,
                                     C.c_int32], C.c_int),
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


def _device_ptr(a, keep):
    """Copy a host array to a new device buffer (kept alive in ``keep``)."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.uint8).reshape(-1).copy()).cuda()
    keep.append(t)
    return t.data_ptr()


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


class Layer:
    """One created layer (a moe_handle) plus torch-side buffer marshalling.

    inputs: the host arrays of one layer (X is not needed), in the layout
    include/moe.h documents; fp16 arrays as numpy float16, bf16 as uint16 bits.
    on_device: hand the weights over as device buffers (copied there first).
    """

    def __init__(self, cfg: moe_config, inputs: dict, on_device: bool = False):
        keep = []
        ptr = _device_ptr if on_device else _host_ptr
        w = moe_weights()
        w.on_device = 1 if on_device else 0
        w.W_grp = ptr(np.asarray(inputs["W_grp"], dtype=np.float32), keep)
        w.W_exp = ptr(None if inputs.get("W_exp") is None
                      else np.asarray(inputs["W_exp"], dtype=np.float32), keep)
        w.group_bias = ptr(None if inputs.get("group_bias") is None
                           else np.asarray(inputs["group_bias"], dtype=np.float32), keep)
        w.expert_bias = ptr(None if inputs.get("expert_bias") is None
                            else np.asarray(inputs["expert_bias"], dtype=np.float32), keep)
        for p, b in enumerate(inputs["base"]):
            w.base[p] = ptr(b, keep)
        for p, a in enumerate(inputs.get("A") or []):
            w.A[p] = ptr(a, keep)
        for p, b in enumerate(inputs.get("B") or []):
            w.B[p] = ptr(b, keep)
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

    def offload_enable(self, slots: int):
        check(lib.moe_offload_enable(self.h, slots))

    def forward_offload(self, X, Y=None, route_bufs=None, stream=None):
        import torch
        T = X.shape[0]
        if Y is None:
            Y = torch.empty((T, self.cfg.d), dtype=self._torch_x_dtype(), device=X.device)
        ro = self._route_struct(route_bufs)
        rop = C.byref(ro) if route_bufs is not None else None
        check(lib.moe_forward_offload(self.h, C.c_void_p(X.data_ptr()), T, C.c_void_p(Y.data_ptr()), rop,
                                      _stream_ptr(stream)))
        return Y

    def offload_stats(self) -> dict:
        st = moe_offload_stats_t()
        check(lib.moe_offload_stats(self.h, C.byref(st)))
        return {n: getattr(st, n) for n, _ in moe_offload_stats_t._fields_}

    def backward(self, X, dY, stream=None) -> dict:
        """moe_backward: returns dX (x dtype) and float32 gradients of every
        weight, as torch tensors on the device."""
        import torch
        c = self.cfg
        T, d, f, G, K, r = X.shape[0], c.d, c.f, c.G, c.K, c.r
        P = 3 if c.act == ACT["swiglu"] else 2
        dev = X.device
        f32 = dict(dtype=torch.float32, device=dev)
        dims = [(d, f)] * (P - 1) + [(f, d)]
        out = dict(dX=torch.empty_like(X), dW_grp=torch.empty((d, G), **f32),
                   dW_exp=torch.empty((G, d, K), **f32), d_group_bias=torch.empty(G, **f32),
                   d_expert_bias=torch.empty(self.E, **f32),
                   dbase=[torch.empty((G, di, do), **f32) for di, do in dims],
                   dA=[torch.empty((self.E, di, r), **f32) for di, do in dims] if r else None,
                   dB=[torch.empty((self.E, do, r), **f32) for di, do in dims] if r else None)
        g = moe_grads()
        g.dW_grp = out["dW_grp"].data_ptr()
        g.dW_exp = out["dW_exp"].data_ptr()
        g.d_group_bias = out["d_group_bias"].data_ptr()
        g.d_expert_bias = out["d_expert_bias"].data_ptr()
        for p in range(P):
            g.dbase[p] = out["dbase"][p].data_ptr()
            if r:
                g.dA[p] = out["dA"][p].data_ptr()
                g.dB[p] = out["dB"][p].data_ptr()
        check(lib.moe_backward(self.h, C.c_void_p(X.data_ptr()), T, C.c_void_p(dY.data_ptr()),
                               C.c_void_p(out["dX"].data_ptr()), C.byref(g), _stream_ptr(stream)))
        return out

    def stats(self) -> dict:
        st = moe_stats()
        check(lib.moe_stats(self.h, C.byref(st)))
        return dict(stored_params=st.stored_params, stored_bytes=st.stored_bytes,
                    dense_equiv_params=st.dense_equiv_params)

    def _factor_rows(self, proj: int, which: int) -> int:
        d, f = self.cfg.d, self.cfg.f
        P = 3 if self.cfg.act == ACT["swiglu"] else 2
        din, dout = (d, f) if proj < P - 1 else (f, d)
        return din if which == 0 else dout

    def debug_dequant(self, proj: int, which: int, expert: int) -> np.ndarray:
        vals = np.zeros((self._factor_rows(proj, which), self.cfg.r), dtype=np.float32)
        check(lib.moe_debug_dequant(self.h, proj, which, expert, vals.ctypes.data))
        return vals

    def debug_q(self, proj: int, which: int, expert: int):
        n, r = self._factor_rows(proj, which), self.cfg.r
        q = np.zeros((n, r), dtype=np.int8)
        sc = np.zeros((n // 32, r), dtype=np.uint16)
        check(lib.moe_debug_q(self.h, proj, which, expert, q.ctypes.data, sc.ctypes.data))
        return q, sc

    def forward_noalloc(self, X, Y, route_bufs=None, stream=None):
        """moe_forward_noalloc: the workspace is the library's static device
        array; Y must be given (nothing is allocated on this path)."""
        ro = self._route_struct(route_bufs)
        rop = C.byref(ro) if route_bufs is not None else None
        check(lib.moe_forward_noalloc(self.h, C.c_void_p(X.data_ptr()), X.shape[0],
                                      C.c_void_p(Y.data_ptr()), rop, _stream_ptr(stream)))
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


# ---------------------------------------------- clustering and compression --
class Cluster:
    """The host clustering state of include/moe_cluster.h (marshalling only)."""

    def __init__(self, E, G, d, n_param, alpha=0.7, beta=0.05, tau=0.1, eps=1e-3, cache_life=4):
        self.cfg = moe_cluster_config(E, G, d, n_param, alpha, beta, tau, eps, cache_life)
        h = C.c_void_p()
        check(lib.moe_cluster_create(C.byref(self.cfg), C.byref(h)))
        self.h = h

    def observe(self, X, idx):
        X = np.ascontiguousarray(X, dtype=np.float32)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        check(lib.moe_cluster_observe(self.h, X.ctypes.data, X.shape[0], idx.ctypes.data, idx.shape[1]))

    def centroids(self) -> np.ndarray:
        mu = np.zeros((self.cfg.E, self.cfg.d), dtype=np.float64)
        check(lib.moe_cluster_get_centroids(self.h, mu.ctypes.data))
        return mu

    def set_centroids(self, mu):
        mu = np.ascontiguousarray(mu, dtype=np.float64)
        check(lib.moe_cluster_set_centroids(self.h, mu.ctypes.data))

    def regroup(self, vecs, u):
        """vecs: E float32 arrays of n_param values; u: G uniforms.
        Returns (group_of [E], members [G, K], S [E, E], fresh [E])."""
        E, G = self.cfg.E, self.cfg.G
        keep = [np.ascontiguousarray(v, dtype=np.float32).reshape(-1) for v in vecs]
        assert all(v.size == self.cfg.n_param for v in keep)
        ptrs = (C.c_void_p * E)(*[v.ctypes.data for v in keep])
        u = np.ascontiguousarray(u, dtype=np.float64)
        group_of = np.zeros(E, dtype=np.int32)
        members = np.zeros((G, E // G), dtype=np.int32)
        S = np.zeros((E, E), dtype=np.float64)
        fresh = np.zeros(E, dtype=np.int32)
        check(lib.moe_cluster_regroup(self.h, ptrs, u.ctypes.data, group_of.ctypes.data,
                                      members.ctypes.data, S.ctypes.data, fresh.ctypes.data))
        return group_of, members, S, fresh

    def close(self):
        if getattr(self, "h", None):
            lib.moe_cluster_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def compress_projection(W, members, r: int, n_threads: int = 0):
    """W: float32 [E, d_in, d_out] (or a list of E such arrays); members
    [G, K].  Returns base [G, d_in, d_out], A [E, d_in, r], B [E, d_out, r]
    (float32, regrouped order) and the relative errors [E] (float64)."""
    keep = [np.ascontiguousarray(w, dtype=np.float32) for w in W]
    E = len(keep)
    din, dout = keep[0].shape
    members = np.ascontiguousarray(members, dtype=np.int32)
    G = members.shape[0]
    ptrs = (C.c_void_p * E)(*[w.ctypes.data for w in keep])
    base = np.zeros((G, din, dout), dtype=np.float32)
    A = np.zeros((E, din, r), dtype=np.float32)
    B = np.zeros((E, dout, r), dtype=np.float32)
    err = np.zeros(E, dtype=np.float64)
    check(lib.moe_compress_projection(E, G, members.ctypes.data, din, dout, r, ptrs, base.ctypes.data,
                                      A.ctypes.data, B.ctypes.data, err.ctypes.data, n_threads))
    return base, A, B, err
