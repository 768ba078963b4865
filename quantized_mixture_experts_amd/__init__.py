"""Python binding of libmoeq (routed MoE layer over block-quantised experts, gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoeq.so.  torch provides device memory and the current stream.  There is no
fallback: importing works without the library, but every call raises if
libmoeq.so is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeq.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGNMENT, MOE_ERR_WORKSPACE, MOE_ERR_HIP = \
    0, -1, -2, -3, -4, -5
WFMT_MXFP4, WFMT_CB4, WFMT_MXFP4_PS, WFMT_AFF3 = 1, 2, 3, 4
DT_F32, DT_BF16 = 0, 1
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2

EXPORTED = ["moe_packed_bytes", "moe_workspace_bytes", "moe_router_topk", "moe_bucket", "moe_forward",
            "moe_forward_timed", "moe_dequant", "moe_dequant_grouped", "moe_rms_rescale", "moe_forward_rms",
            "moe_hbm_read_probe", "moe_forward_noalloc", "moe_status_str"]
STAGES = ["router", "topk", "bucket", "gateup", "down", "combine", "xquant"]


class MoeLayerC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("wfmt", ctypes.c_int32), ("has_shared", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p), ("gate_up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("codebook", ctypes.c_void_p), ("shared_gate_w", ctypes.c_void_p),
                ("omit_below", ctypes.c_float)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoeq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run quantized_mixture_experts_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_packed_bytes.argtypes, L.moe_packed_bytes.restype = [i32, i32, i32], sz
        L.moe_workspace_bytes.argtypes, L.moe_workspace_bytes.restype = [ctypes.POINTER(MoeLayerC), i32], sz
        L.moe_router_topk.argtypes = [ctypes.POINTER(MoeLayerC), vp, i32, i32, vp, vp, vp, sz, vp]
        L.moe_bucket.argtypes = [ctypes.POINTER(MoeLayerC), vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_forward.argtypes = [ctypes.POINTER(MoeLayerC), vp, i32, i32, vp, vp, sz, vp, i32, vp, vp, vp, vp, vp]
        L.moe_forward_timed.argtypes = [ctypes.POINTER(MoeLayerC), vp, i32, i32, vp, vp, sz, vp, i32, vp]
        L.moe_dequant.argtypes = [i32, vp, vp, i32, i32, vp, vp]
        L.moe_dequant_grouped.argtypes = [i32, vp, vp, i32, i32, vp, vp]
        L.moe_rms_rescale.argtypes = [vp, i32, i32, ctypes.c_float, vp, vp]
        L.moe_forward_rms.argtypes = [ctypes.POINTER(MoeLayerC), vp, ctypes.c_float, i32, i32, vp, vp, sz, vp, i32,
                                      vp]
        L.moe_hbm_read_probe.argtypes = [vp, sz, vp, i32, vp]
        L.moe_forward_noalloc.argtypes = [ctypes.POINTER(MoeLayerC), vp, i32, i32, vp, vp, i32]
        L.moe_status_str.argtypes, L.moe_status_str.restype = [ctypes.c_int], ctypes.c_char_p
        for f in ["moe_router_topk", "moe_bucket", "moe_forward", "moe_forward_timed", "moe_dequant",
                  "moe_dequant_grouped", "moe_rms_rescale", "moe_forward_rms", "moe_hbm_read_probe",
                  "moe_forward_noalloc"]:
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def packed_bytes(wfmt: int, rows: int, cols: int) -> int:
    return lib().moe_packed_bytes(wfmt, rows, cols)


class DeviceLayer:
    """A layer resident in device memory: router weights, one bank of packed experts
    (expert-major: gate_up then down of expert 0, then expert 1, ...), the device
    pointer tables and the descriptor the C ABI takes."""

    def __init__(self, hidden: int, inter: int, n_experts: int, top_k: int, wfmt: int, has_shared: int,
                 router_w, router_b, gate_up: Sequence[np.ndarray], down: Sequence[np.ndarray],
                 codebook=None, shared_gate_w=None, device="cuda", omit_below: float = 0.0):
        import torch
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self.wfmt, self.has_shared = wfmt, has_shared
        dev = torch.device(device)
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        self.router_w = f32(router_w)
        self.router_b = None if router_b is None else f32(router_b)
        self.shared_gate_w = None if shared_gate_w is None else f32(shared_gate_w)
        self.codebook = None if codebook is None else torch.from_numpy(
            np.ascontiguousarray(codebook, dtype=np.int8)).to(dev)
        n = n_experts + has_shared
        gu_b = packed_bytes(wfmt, 2 * inter, hidden)
        dn_b = packed_bytes(wfmt, hidden, inter)
        a_gu = (gu_b + 255) // 256 * 256
        a_dn = (dn_b + 255) // 256 * 256
        stride = a_gu + a_dn
        self.bank = torch.empty(n * stride, dtype=torch.uint8, device=dev)
        host = torch.empty(stride, dtype=torch.uint8, pin_memory=dev.type == "cuda")
        for e in range(n):
            host.zero_()
            if gate_up[e] is not None:
                host[:gu_b] = torch.from_numpy(np.asarray(gate_up[e], dtype=np.uint8))
                host[a_gu:a_gu + dn_b] = torch.from_numpy(np.asarray(down[e], dtype=np.uint8))
            self.bank[e * stride:(e + 1) * stride].copy_(host, non_blocking=False)
        base = self.bank.data_ptr()
        self.gate_up_ptrs = torch.tensor([base + e * stride for e in range(n)], dtype=torch.int64, device=dev)
        self.down_ptrs = torch.tensor([base + e * stride + a_gu for e in range(n)], dtype=torch.int64, device=dev)
        self.expert_stride, self.gu_offset, self.dn_offset = stride, 0, a_gu
        self.c = MoeLayerC(hidden, inter, n_experts, top_k, wfmt, has_shared, _ptr(self.router_w),
                           _ptr(self.router_b), _ptr(self.gate_up_ptrs), _ptr(self.down_ptrs), _ptr(self.codebook),
                           _ptr(self.shared_gate_w), omit_below)

    @property
    def omit_below(self) -> float:
        """Marginal-expert omission threshold of the descriptor (0: off)."""
        return self.c.omit_below

    @omit_below.setter
    def omit_below(self, tau: float):
        self.c.omit_below = tau

    @classmethod
    def from_layer(cls, layer, device="cuda", omit_below: float = 0.0):
        """From a host layer object with the generator's attribute names."""
        return cls(layer.hidden, layer.inter, layer.n_experts, layer.top_k, layer.wfmt, layer.has_shared,
                   layer.router_w, layer.router_b, layer.gate_up, layer.down, layer.codebook,
                   layer.shared_gate_w, device, omit_below)

    def workspace_bytes(self, T: int) -> int:
        return lib().moe_workspace_bytes(ctypes.byref(self.c), T)

    def workspace(self, T: int):
        """A zero-filled workspace for up to T tokens (its header must be zero before the
        first call; every call leaves it zero)."""
        import torch
        n = self.workspace_bytes(T)
        if n == 0 and T > 0:
            raise MoeError(MOE_ERR_INVALID_ARG, "moe_workspace_bytes")
        return torch.zeros(max(n, 1), dtype=torch.uint8, device=self.router_w.device)


def router_topk(L: DeviceLayer, x, x_dtype: int, ws=None, stream=None):
    import torch
    T = x.shape[0]
    ws = L.workspace(T) if ws is None else ws
    ids = torch.empty((T, L.top_k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, L.top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_topk(ctypes.byref(L.c), x.data_ptr(), x_dtype, T, ids.data_ptr(), w.data_ptr(),
                                 ws.data_ptr(), ws.numel(), _stream(stream)), "moe_router_topk")
    return ids, w


def bucket(L: DeviceLayer, ids, ws=None, stream=None):
    import torch
    T = ids.shape[0]
    ws = L.workspace(T) if ws is None else ws
    P = T * L.top_k + T * L.has_shared
    counts = torch.empty(L.n_experts + 1, dtype=torch.int32, device=ids.device)
    offsets = torch.empty(L.n_experts + 2, dtype=torch.int32, device=ids.device)
    perm = torch.empty(max(P, 1), dtype=torch.int32, device=ids.device)
    _check(lib().moe_bucket(ctypes.byref(L.c), ids.data_ptr(), T, counts.data_ptr(), offsets.data_ptr(),
                            perm.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)), "moe_bucket")
    return counts, offsets, perm[:P]


def forward(L: DeviceLayer, x, x_dtype: int, y=None, ws=None, path: int = PATH_AUTO, debug: bool = False,
            stream=None):
    """y [T][H] fp32.  With debug=True also returns the routing and bucketing used."""
    import torch
    T = x.shape[0]
    ws = L.workspace(T) if ws is None else ws
    y = torch.empty((T, L.hidden), dtype=torch.float32, device=x.device) if y is None else y
    dbg = None
    if debug:
        P = T * L.top_k + T * L.has_shared
        dbg = dict(ids=torch.empty((T, L.top_k), dtype=torch.int32, device=x.device),
                   gates=torch.empty((T, L.top_k), dtype=torch.float32, device=x.device),
                   counts=torch.empty(L.n_experts + 1, dtype=torch.int32, device=x.device),
                   offsets=torch.empty(L.n_experts + 2, dtype=torch.int32, device=x.device),
                   perm=torch.empty(max(P, 1), dtype=torch.int32, device=x.device))
    d = (lambda k: dbg[k].data_ptr()) if debug else (lambda k: None)
    _check(lib().moe_forward(ctypes.byref(L.c), x.data_ptr(), x_dtype, T, y.data_ptr(), ws.data_ptr(),
                             ws.numel(), _stream(stream), path, d("ids"), d("gates"), d("counts"),
                             d("offsets"), d("perm")), "moe_forward")
    if debug:
        dbg["perm"] = dbg["perm"][:T * L.top_k + T * L.has_shared]
        return y, dbg
    return y


def forward_noalloc(L: DeviceLayer, x, x_dtype: int, y=None, path: int = PATH_AUTO, stream=None):
    """moe_forward_noalloc: y [T][H] fp32, with the library's per-device scratch array as the
    workspace (no workspace argument; nothing is allocated by the library)."""
    import torch
    T = x.shape[0]
    y = torch.empty((T, L.hidden), dtype=torch.float32, device=x.device) if y is None else y
    _check(lib().moe_forward_noalloc(ctypes.byref(L.c), x.data_ptr(), x_dtype, T, y.data_ptr(), _stream(stream),
                                     path), "moe_forward_noalloc")
    return y


def forward_timed(L: DeviceLayer, x, x_dtype: int, y, ws, events, path: int = PATH_AUTO, stream=None):
    """moe_forward with per-stage kernel timestamps; `events` is a ctypes array of
    2 * len(STAGES) hipEvent_t handles (see HipEvents)."""
    T = x.shape[0]
    _check(lib().moe_forward_timed(ctypes.byref(L.c), x.data_ptr(), x_dtype, T, y.data_ptr(), ws.data_ptr(),
                                   ws.numel(), _stream(stream), path, events), "moe_forward_timed")
    return y


class HipEvents:
    """hipEvent_t handles from the HIP runtime (the library stamps them per stage)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = h
        self.n = n

    def slice(self, start: int, count: int):
        return ctypes.cast(ctypes.byref(self.handles, start * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self, i: int, j: int) -> Optional[float]:
        ms = ctypes.c_float()
        r = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j])
        if r != 0:  # a stage that launched nothing: clear the error the query left behind
            self.hip.hipGetLastError()
            return None
        return ms.value

    def __del__(self):
        try:
            for i in range(self.n):
                self.hip.hipEventDestroy(self.handles[i])
        except Exception:
            pass


def dequant(wfmt: int, packed, rows: int, cols: int, codebook=None, stream=None):
    import torch
    out = torch.empty((rows, cols), dtype=torch.float32, device=packed.device)
    _check(lib().moe_dequant(wfmt, packed.data_ptr(), _ptr(codebook), rows, cols, out.data_ptr(),
                             _stream(stream)), "moe_dequant")
    return out


def dequant_grouped(wfmt: int, packed, rows: int, cols: int, codebook=None, stream=None):
    """moe_dequant_grouped: the grouped (prefill) kernels' CB4 decode of one packed matrix."""
    import torch
    out = torch.empty((rows, cols), dtype=torch.float32, device=packed.device)
    _check(lib().moe_dequant_grouped(wfmt, packed.data_ptr(), _ptr(codebook), rows, cols, out.data_ptr(),
                                     _stream(stream)), "moe_dequant_grouped")
    return out


def forward_rms(L: DeviceLayer, y_prev, eps: float = 1e-6, y=None, ws=None, path: int = PATH_AUTO, events=None,
                residual: bool = False, stream=None):
    """moe_forward_rms: the layer on the bf16 RMS rescale of the previous layer's fp32
    output y_prev [T][H] (the values rms_rescale(y_prev, eps) gives); residual=True adds
    y_prev to the result.  `events`: None or 2 * len(STAGES) hipEvent_t handles (see
    HipEvents)."""
    import torch
    T = y_prev.shape[0]
    ws = L.workspace(T) if ws is None else ws
    y = torch.empty((T, L.hidden), dtype=torch.float32, device=y_prev.device) if y is None else y
    _check(lib().moe_forward_rms(ctypes.byref(L.c), y_prev.data_ptr(), eps, int(residual), T, y.data_ptr(),
                                 ws.data_ptr(), ws.numel(), _stream(stream), path, events), "moe_forward_rms")
    return y


def rms_rescale(y, eps: float = 1e-6, out=None, stream=None):
    import torch
    T, H = y.shape
    out = torch.empty((T, H), dtype=torch.int16, device=y.device) if out is None else out
    _check(lib().moe_rms_rescale(y.data_ptr(), T, H, eps, out.data_ptr(), _stream(stream)), "moe_rms_rescale")
    return out


def hbm_read_probe(buf, out, blocks: int, stream=None):
    """moe_hbm_read_probe: stream-read every byte of the device tensor buf (one word per
    block written to out, a device int32 tensor of at least `blocks` entries)."""
    _check(lib().moe_hbm_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(), blocks,
                                    _stream(stream)), "moe_hbm_read_probe")
