"""W4A16 mixture-of-experts expert layer for MI355X (gfx950).

Python binding of ``libmoe_w4a16.so`` (declared in include/moe_w4a16.h).
This module only marshals arguments: every step of the layer runs in the
library's HIP kernels. PyTorch supplies device memory and streams. There is
no CPU fallback: if the library is not built, every call raises.

Low-level names mirror the C ABI (``moe_prepare_weights``, ``moe_align``,
``moe_w4a16_indexed``, ...). ``PreparedWeights`` wraps a handle with
torch-tensor conveniences.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# the in-tree build of csrc/ (w4a16_int4_grouped_amd/build.py); no other library stands in for it
LIB_PATH = os.path.join(PKG_DIR, "libmoe_w4a16.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED_SCHEMA = 2
MOE_ERR_MODE_MISMATCH = 3
MOE_ERR_OVERRIDE_REJECTED = 4
MOE_ERR_WORKSPACE_TOO_SMALL = 5
MOE_ERR_HIP = 6
MOE_ERR_ROUTING_MISMATCH = 7

MOE_MODE_INDEXED = 0
MOE_MODE_CONTIGUOUS = 1
MOE_MODE_MASKED = 2
MODES = {"indexed": MOE_MODE_INDEXED, "contiguous": MOE_MODE_CONTIGUOUS, "masked": MOE_MODE_MASKED}

# bytes of the fixed device scratch array behind moe_w4a16_indexed_noalloc
NOALLOC_SCRATCH_BYTES = 128 << 20

MOE_SCALE_BF16 = 1
MOE_PACK_INT32_LOW_NIBBLE_FIRST_K = 1

EXPORTS = [
    "moe_abi_version", "moe_last_error", "moe_status_string", "moe_prepared_bytes",
    "moe_prepare_weights", "moe_release_weights", "moe_plan_create", "moe_routing_block", "moe_routing_bytes",
    "moe_routing_layout", "moe_align", "moe_align_ep", "moe_permute", "moe_workspace_bytes", "moe_w4a16_indexed",
    "moe_w4a16_indexed_noalloc", "moe_w4a16_contiguous", "moe_w4a16_masked", "moe_w4a16_gate_up", "moe_w4a16_down", "moe_swiglu",
    "moe_dequant_weights", "moe_describe",
    "moe_profile_enable", "moe_profile_reset", "moe_profile_read",
]


class WeightDesc(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("zero_point", ctypes.c_int32),
                ("scale_dtype", ctypes.c_int32), ("pack_order", ctypes.c_int32), ("mode", ctypes.c_int32)]


def make_desc(E, H, I, mode="indexed", bits=4, group_size=32, zero_point=8,
              scale_dtype=MOE_SCALE_BF16, pack_order=MOE_PACK_INT32_LOW_NIBBLE_FIRST_K) -> WeightDesc:
    return WeightDesc(E, H, I, bits, group_size, zero_point, scale_dtype, pack_order,
                      MODES[mode] if isinstance(mode, str) else int(mode))


class Tuning(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("dispatch", ctypes.c_int32), ("global_experts", ctypes.c_int32)]


class RoutingLayout(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("cap", ctypes.c_int32), ("nblocks", ctypes.c_int32),
                ("sentinel", ctypes.c_int32), ("off_header", ctypes.c_int64),
                ("off_counts", ctypes.c_int64), ("off_offsets", ctypes.c_int64),
                ("off_sorted", ctypes.c_int64), ("off_block_expert", ctypes.c_int64),
                ("off_slot_of", ctypes.c_int64), ("off_scratch", ctypes.c_int64), ("total_ints", ctypes.c_int64)]


class MoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED_SCHEMA",
           3: "MOE_ERR_MODE_MISMATCH", 4: "MOE_ERR_OVERRIDE_REJECTED",
           5: "MOE_ERR_WORKSPACE_TOO_SMALL", 6: "MOE_ERR_HIP", 7: "MOE_ERR_ROUTING_MISMATCH"}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m w4a16_int4_grouped_amd.build`"
                           " (there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    sig = {
        "moe_abi_version": (S, []),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_status_string": (ctypes.c_char_p, [S]),
        "moe_prepared_bytes": (SZ, [ctypes.POINTER(WeightDesc)]),
        "moe_prepare_weights": (S, [ctypes.POINTER(WeightDesc), P, P, P, P, P, SZ, P, ctypes.POINTER(P)]),
        "moe_release_weights": (None, [P]),
        "moe_plan_create": (P, [ctypes.POINTER(WeightDesc)]),
        "moe_routing_block": (I32, [P, I32, I32, ctypes.POINTER(Tuning)]),
        "moe_routing_bytes": (SZ, [P, I32, I32, ctypes.POINTER(Tuning)]),
        "moe_routing_layout": (S, [P, I32, I32, ctypes.POINTER(Tuning), ctypes.POINTER(RoutingLayout)]),
        "moe_align": (S, [P, P, I32, I32, ctypes.POINTER(Tuning), P, SZ, P]),
        "moe_align_ep": (S, [P, P, I32, I32, P, I32, ctypes.POINTER(Tuning), P, SZ, P]),
        "moe_permute": (S, [P, P, I32, I32, ctypes.POINTER(Tuning), P, P, P, P, P]),
        "moe_workspace_bytes": (SZ, [P, I32, I32, I32, I32, ctypes.POINTER(Tuning)]),
        "moe_w4a16_indexed": (S, [P, P, I32, I32, P, P, P, P, P, SZ, ctypes.POINTER(Tuning), P]),
        "moe_w4a16_indexed_noalloc": (S, [P, P, I32, I32, P, P, P, ctypes.POINTER(Tuning), P]),
        "moe_w4a16_contiguous": (S, [P, P, I32, P, P, P, I32, I32, P, P, SZ, ctypes.POINTER(Tuning), P]),
        "moe_w4a16_masked": (S, [P, P, I32, P, I32, P, P, SZ, ctypes.POINTER(Tuning), P]),
        "moe_w4a16_gate_up": (S, [P, P, I32, I32, P, P, ctypes.POINTER(Tuning), P]),
        "moe_w4a16_down": (S, [P, P, I32, I32, P, P, ctypes.POINTER(Tuning), P]),
        "moe_swiglu": (S, [P, I64, I32, P, P]),
        "moe_dequant_weights": (S, [P, I32, I32, P, P]),
        "moe_describe": (S, [P, I32, I32, I32, I32, ctypes.POINTER(Tuning), ctypes.c_char_p, SZ]),
        "moe_profile_enable": (S, [S]),
        "moe_profile_reset": (None, []),
        "moe_profile_read": (S, [ctypes.c_char_p, SZ]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return lib().moe_last_error().decode()


def check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, last_error())


# ---------------------------------------------------------------------------
# torch plumbing (device memory and streams only)
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _tuning(ovr):
    if ovr is None:
        return None
    if isinstance(ovr, Tuning):
        return ctypes.byref(ovr)
    return ctypes.byref(Tuning(int(ovr.get("block_m", 0)), int(ovr.get("schedule", 0)),
                               int(ovr.get("dispatch", 0)), int(ovr.get("global_experts", 0))))


def _empty(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


class PreparedWeights:
    """A prepared-weight handle plus the device buffer it lives in.

    w13_q int32 [E, 2I, H/8], w13_s bf16 [E, 2I, H/32], w2_q int32 [E, H, I/8],
    w2_s bf16 [E, H, I/32], all on one GPU.
    """

    def __init__(self, w13_q, w13_s, w2_q, w2_s, mode="indexed", stream=None):
        import torch
        E, N13, _ = w13_q.shape
        H = w2_q.shape[1]
        I = N13 // 2
        self.E, self.H, self.I = E, H, I
        self.mode = MODES[mode] if isinstance(mode, str) else int(mode)
        self.device = w13_q.device
        desc = make_desc(E, H, I, self.mode)
        L = lib()
        nbytes = L.moe_prepared_bytes(ctypes.byref(desc))
        if nbytes == 0:
            raise MoeError(MOE_ERR_UNSUPPORTED_SCHEMA, last_error())
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        check(L.moe_prepare_weights(ctypes.byref(desc), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s),
                                    _ptr(self.buffer), nbytes, _stream(stream), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.moe_release_weights(h)
            self.handle = None

    # -- routing ------------------------------------------------------------
    def routing_layout(self, T, topk, ovr=None) -> RoutingLayout:
        out = RoutingLayout()
        check(lib().moe_routing_layout(self.handle, T, topk, _tuning(ovr), ctypes.byref(out)))
        return out

    def align(self, topk_ids, ovr=None, routing=None, stream=None):
        import torch
        T, topk = topk_ids.shape
        nbytes = lib().moe_routing_bytes(self.handle, T, topk, _tuning(ovr))
        if nbytes == 0:
            check(MOE_ERR_INVALID_ARG)
        if routing is None:
            routing = torch.empty(nbytes // 4, dtype=torch.int32, device=self.device)
        check(lib().moe_align(self.handle, _ptr(topk_ids), T, topk, _tuning(ovr), _ptr(routing),
                              routing.numel() * routing.element_size(), _stream(stream)))
        return routing

    def align_ep(self, topk_ids, expert_map, num_global_experts, ovr=None, routing=None, stream=None):
        """Routing of this handle's share of num_global_experts experts:
        expert_map[global id] = local expert or -1."""
        import torch
        T, topk = topk_ids.shape
        nbytes = lib().moe_routing_bytes(self.handle, T, topk, _tuning(ovr))
        if nbytes == 0:
            check(MOE_ERR_INVALID_ARG)
        if routing is None:
            routing = torch.empty(nbytes // 4, dtype=torch.int32, device=self.device)
        check(lib().moe_align_ep(self.handle, _ptr(topk_ids), T, topk, _ptr(expert_map), num_global_experts,
                                 _tuning(ovr), _ptr(routing), routing.numel() * routing.element_size(),
                                 _stream(stream)))
        return routing

    def permute(self, x, topk, routing, ovr=None, stream=None, out=None):
        """Contiguous rows, m_indices and row_src of the routing; `out` may
        give the three buffers (routing capacity rows each)."""
        import torch
        T = x.shape[0]
        L = self.routing_layout(T, topk, ovr)
        if out is None:
            a = torch.empty((L.cap, self.H), dtype=torch.bfloat16, device=self.device)
            m = torch.empty(L.cap, dtype=torch.int32, device=self.device)
            r = torch.empty(L.cap, dtype=torch.int32, device=self.device)
        else:
            a, m, r = out
            if (a.dtype != torch.bfloat16 or m.dtype != torch.int32 or r.dtype != torch.int32
                    or not (a.is_contiguous() and m.is_contiguous() and r.is_contiguous())
                    or a.dim() != 2 or a.shape[0] < L.cap or a.shape[1] != self.H
                    or m.numel() < L.cap or r.numel() < L.cap):
                check(MOE_ERR_INVALID_ARG)
        check(lib().moe_permute(self.handle, _ptr(x), T, topk, _tuning(ovr), _ptr(routing), _ptr(a), _ptr(m),
                                _ptr(r), _stream(stream)))
        return a, m, r

    # -- the layer ------------------------------------------------------------
    def workspace_bytes(self, rows, topk=0, tokens=0, mode=None, ovr=None) -> int:
        m = self.mode if mode is None else mode
        return int(lib().moe_workspace_bytes(self.handle, m, rows, topk, tokens, _tuning(ovr)))

    def indexed(self, x, topk_ids, topk_w, routing=None, out=None, ws=None, ovr=None, stream=None):
        import torch
        T, topk = topk_ids.shape
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=self.device)
        if ws is None:
            ws = _empty(self.workspace_bytes(T, topk, T, ovr=ovr), self.device)
        check(lib().moe_w4a16_indexed(self.handle, _ptr(x), T, topk, _ptr(topk_ids), _ptr(topk_w),
                                      _ptr(routing), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                      _tuning(ovr), _stream(stream)))
        return out

    def indexed_noalloc(self, x, topk_ids, topk_w, out, ovr=None, stream=None):
        """The indexed layer on the library's fixed scratch array: allocates
        nothing, so `out` must be given."""
        T, topk = topk_ids.shape
        check(lib().moe_w4a16_indexed_noalloc(self.handle, _ptr(x), T, topk, _ptr(topk_ids), _ptr(topk_w),
                                              _ptr(out), _tuning(ovr), _stream(stream)))
        return out

    def contiguous(self, a, m_indices, row_src=None, topk_w=None, T=0, topk=0, out=None, ws=None,
                   ovr=None, stream=None):
        import torch
        M_pad = a.shape[0]
        if out is None:
            rows = T if row_src is not None else M_pad
            out = torch.empty((rows, self.H), dtype=torch.bfloat16, device=self.device)
        if ws is None:
            ws = _empty(self.workspace_bytes(M_pad, topk if row_src is not None else 0, T), self.device)
        check(lib().moe_w4a16_contiguous(self.handle, _ptr(a), M_pad, _ptr(m_indices), _ptr(row_src),
                                         _ptr(topk_w), T, topk, _ptr(out), _ptr(ws),
                                         ws.numel() * ws.element_size(), _tuning(ovr), _stream(stream)))
        return out

    def masked(self, a3, masked_m, expected_m, out=None, ws=None, ovr=None, stream=None):
        import torch
        E, max_m, H = a3.shape
        if out is None:
            out = torch.empty((E * max_m, self.H), dtype=torch.bfloat16, device=self.device)
        if ws is None:
            ws = _empty(self.workspace_bytes(max_m), self.device)
        check(lib().moe_w4a16_masked(self.handle, _ptr(a3), max_m, _ptr(masked_m), expected_m, _ptr(out),
                                     _ptr(ws), ws.numel() * ws.element_size(), _tuning(ovr), _stream(stream)))
        return out

    # -- unfused steps (indexed) ------------------------------------------------
    def gate_up(self, x, topk, routing, out=None, ovr=None, stream=None):
        """BF16 [cap, 2I] gate | up rows at the routing's slots."""
        import torch
        T = x.shape[0]
        if out is None:
            cap = self.routing_layout(T, topk, ovr).cap
            out = torch.empty((cap, 2 * self.I), dtype=torch.bfloat16, device=self.device)
        check(lib().moe_w4a16_gate_up(self.handle, _ptr(x), T, topk, _ptr(routing), _ptr(out), _tuning(ovr),
                                      _stream(stream)))
        return out

    def down(self, a, T, topk, routing, out=None, ovr=None, stream=None):
        """BF16 [cap, H] rows of the second GEMM at the routing's slots."""
        import torch
        if out is None:
            out = torch.empty((a.shape[0], self.H), dtype=torch.bfloat16, device=self.device)
        check(lib().moe_w4a16_down(self.handle, _ptr(a), T, topk, _ptr(routing), _ptr(out), _tuning(ovr),
                                   _stream(stream)))
        return out

    def dequant(self, which, expert, stream=None):
        import torch
        shape = (2 * self.I, self.H) if which == 13 else (self.H, self.I)
        out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        check(lib().moe_dequant_weights(self.handle, which, expert, _ptr(out), _stream(stream)))
        return out

    def describe(self, rows, topk=0, expected_m=0, ovr=None, mode=None) -> str:
        buf = ctypes.create_string_buffer(512)
        m = self.mode if mode is None else mode
        n = lib().moe_describe(self.handle, m, rows, topk, expected_m, _tuning(ovr), buf, 512)
        if n < 0:
            raise MoeError(MOE_ERR_INVALID_ARG, last_error())
        return buf.value.decode()


def swiglu(h, out=None, stream=None):
    """BF16 [rows, I] = silu(h[:, :I]) * h[:, I:] for BF16 h [rows, 2I]."""
    import torch
    rows, two_i = h.shape
    if out is None:
        out = torch.empty((rows, two_i // 2), dtype=torch.bfloat16, device=h.device)
    check(lib().moe_swiglu(_ptr(h), rows, two_i // 2, _ptr(out), _stream(stream)))
    return out


def profile_enable(on=True):
    check(lib().moe_profile_enable(1 if on else 0))


def profile_reset():
    lib().moe_profile_reset()


def profile_read() -> dict:
    """{kernel name: (launches, total_ms)} since the last reset (synchronises)."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().moe_profile_read(buf, 1 << 16)
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out
