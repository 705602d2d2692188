"""C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any HIP call.

Handle-level checks use moe_plan_create (a handle without weights), so no
GPU is needed; calls that pass validation then stop with INVALID_ARG because
the plan has no prepared weights.
"""
import ctypes
import os
import re

import pytest

import w4a16_int4_grouped_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")


@pytest.fixture(scope="session")
def L():
    if not os.path.exists(M.LIB_PATH):
        from w4a16_int4_grouped_amd import build
        build.build()
    return M.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)
    return sorted(set(n for n in names if not n.endswith("_t")))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ["moe_prepare_weights", "moe_align", "moe_w4a16_indexed", "moe_w4a16_contiguous",
                 "moe_w4a16_masked"]:
        assert name in fns
    assert set(fns) == set(M.EXPORTS), set(fns) ^ set(M.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 1


def desc(E=8, H=256, I=512, mode="indexed", **kw):
    return M.make_desc(E, H, I, mode, **kw)


@pytest.mark.parametrize("kw", [dict(bits=8), dict(group_size=64), dict(zero_point=0), dict(scale_dtype=2),
                                dict(pack_order=2), dict(H=100), dict(I=48)])
def test_unsupported_schema_fails_at_load(L, kw):
    d = desc(**{k: v for k, v in kw.items() if k in ("H", "I")},
             **{k: v for k, v in kw.items() if k not in ("H", "I")})
    assert L.moe_prepared_bytes(ctypes.byref(d)) == 0
    assert L.moe_plan_create(ctypes.byref(d)) is None
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 20)
    st = L.moe_prepare_weights(ctypes.byref(d), fake, fake, fake, fake, fake, 1 << 30, None, ctypes.byref(h))
    assert st == M.MOE_ERR_UNSUPPORTED_SCHEMA, M.last_error()
    assert "supported" in M.last_error() or "multiples of 32" in M.last_error()


@pytest.mark.parametrize("kw", [dict(E=0), dict(E=5000), dict(mode=7)])
def test_invalid_desc(L, kw):
    d = desc(**kw)
    assert L.moe_prepared_bytes(ctypes.byref(d)) == 0
    assert M.last_error()


def test_prepare_argument_checks(L):
    d = desc()
    need = L.moe_prepared_bytes(ctypes.byref(d))
    assert need > 0
    h = ctypes.c_void_p()
    good = ctypes.c_void_p(1 << 20)
    st = L.moe_prepare_weights(ctypes.byref(d), None, good, good, good, good, need, None, ctypes.byref(h))
    assert st == M.MOE_ERR_INVALID_ARG
    odd = ctypes.c_void_p((1 << 20) + 4)
    st = L.moe_prepare_weights(ctypes.byref(d), odd, good, good, good, good, need, None, ctypes.byref(h))
    assert st == M.MOE_ERR_INVALID_ARG and "align" in M.last_error()
    st = L.moe_prepare_weights(ctypes.byref(d), good, good, good, good, good, need - 1, None, ctypes.byref(h))
    assert st == M.MOE_ERR_WORKSPACE_TOO_SMALL
    st = L.moe_prepare_weights(ctypes.byref(d), good, good, good, good, good, need, None, None)
    assert st == M.MOE_ERR_INVALID_ARG


def test_prepared_bytes_matches_layout(L):
    E, H, I = 8, 256, 512
    d = desc(E, H, I)
    words = E * 2 * I * H // 2 + E * H * I // 2            # packed bytes, already tile-aligned here
    scales = (E * 2 * I * H // 32 + E * H * I // 32) * 2
    assert L.moe_prepared_bytes(ctypes.byref(d)) == words + scales + 256


class Plan:
    def __init__(self, L, mode, E=16, H=256, I=128):
        self.L = L
        self.d = desc(E, H, I, mode)
        self.h = L.moe_plan_create(ctypes.byref(self.d))
        assert self.h

    def __del__(self):
        self.L.moe_release_weights(self.h)


def test_routing_layout_arithmetic(L):
    p = Plan(L, "indexed", E=16)
    T, topk = 100, 4
    lay = M.RoutingLayout()
    assert L.moe_routing_layout(p.h, T, topk, None, ctypes.byref(lay)) == M.MOE_OK
    B = lay.block
    assert B in (16, 32, 64, 128)
    assert lay.cap == T * topk + 16 * (B - 1)
    assert lay.nblocks == -(-lay.cap // B)
    assert lay.sentinel == T * topk
    assert lay.off_counts >= 16 and lay.off_offsets >= lay.off_counts + 16
    assert lay.off_sorted >= lay.off_offsets + 17 and lay.off_block_expert >= lay.off_sorted + lay.cap
    assert lay.off_slot_of >= lay.off_block_expert + lay.nblocks
    assert lay.off_scratch >= lay.off_slot_of + T * topk
    assert L.moe_routing_bytes(p.h, T, topk, None) == lay.total_ints * 4
    t = M.Tuning(64, 0, 0, 0)
    assert L.moe_routing_block(p.h, T, topk, ctypes.byref(t)) == 64
    bad = M.Tuning(48, 0, 0, 0)
    assert L.moe_routing_block(p.h, T, topk, ctypes.byref(bad)) == 0
    assert L.moe_routing_block(p.h, T, 0, None) == 0            # topk < 1
    assert L.moe_routing_block(p.h, T, 17, None) == 0           # topk > E


def test_mode_is_recorded_and_checked(L):
    pi, pc, pm = Plan(L, "indexed"), Plan(L, "contiguous"), Plan(L, "masked")
    fake = ctypes.c_void_p(1 << 20)
    ws = 1 << 40
    st = L.moe_w4a16_indexed(pm.h, fake, 4, 2, fake, fake, None, fake, fake, ws, None, None)
    assert st == M.MOE_ERR_MODE_MISMATCH and "masked" in M.last_error()
    st = L.moe_w4a16_masked(pi.h, fake, 8, fake, 4, fake, fake, ws, None, None)
    assert st == M.MOE_ERR_MODE_MISMATCH
    st = L.moe_w4a16_contiguous(pm.h, fake, 128, fake, None, None, 0, 0, fake, fake, ws, None, None)
    assert st == M.MOE_ERR_MODE_MISMATCH
    st = L.moe_align(pc.h, fake, 4, 2, None, fake, ws, None)
    assert st == M.MOE_ERR_MODE_MISMATCH


def test_grouped_layouts_reject_overrides(L):
    pc, pm = Plan(L, "contiguous"), Plan(L, "masked")
    fake = ctypes.c_void_p(1 << 20)
    t = M.Tuning(64, 0, 0, 0)
    st = L.moe_w4a16_contiguous(pc.h, fake, 128, fake, None, None, 0, 0, fake, fake, 1 << 40,
                                ctypes.byref(t), None)
    assert st == M.MOE_ERR_OVERRIDE_REJECTED
    st = L.moe_w4a16_masked(pm.h, fake, 8, fake, 4, fake, fake, 1 << 40, ctypes.byref(t), None)
    assert st == M.MOE_ERR_OVERRIDE_REJECTED


def test_argument_errors(L):
    pi, pc, pm = Plan(L, "indexed"), Plan(L, "contiguous"), Plan(L, "masked")
    fake = ctypes.c_void_p(1 << 20)
    big = 1 << 40
    # masked: expected_m must be positive
    assert L.moe_w4a16_masked(pm.h, fake, 8, fake, 0, fake, fake, big, None, None) == M.MOE_ERR_INVALID_ARG
    assert "expected_m" in M.last_error()
    # contiguous: M_pad a multiple of 128
    assert L.moe_w4a16_contiguous(pc.h, fake, 100, fake, None, None, 0, 0, fake, fake, big, None,
                                  None) == M.MOE_ERR_INVALID_ARG
    # indexed: NULL x, bad topk, misaligned out
    assert L.moe_w4a16_indexed(pi.h, None, 4, 2, fake, fake, None, fake, fake, big, None,
                               None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_w4a16_indexed(pi.h, fake, 4, 0, fake, fake, None, fake, fake, big, None,
                               None) == M.MOE_ERR_INVALID_ARG
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.moe_w4a16_indexed(pi.h, fake, 4, 2, fake, fake, None, odd, fake, big, None,
                               None) == M.MOE_ERR_INVALID_ARG
    # workspace too small
    need = L.moe_workspace_bytes(pi.h, M.MOE_MODE_INDEXED, 4, 2, 4, None)
    assert need > 0
    assert L.moe_w4a16_indexed(pi.h, fake, 4, 2, fake, fake, None, fake, fake, need - 1, None,
                               None) == M.MOE_ERR_WORKSPACE_TOO_SMALL
    # valid arguments on a plan handle stop before any device work
    assert L.moe_w4a16_indexed(pi.h, fake, 4, 2, fake, fake, None, fake, fake, need, None,
                               None) == M.MOE_ERR_INVALID_ARG
    assert "plan" in M.last_error()
    # T = 0 is a valid empty call
    assert L.moe_w4a16_indexed(pi.h, None, 0, 2, None, None, None, None, None, 0, None, None) == M.MOE_OK
    # dequant argument checks
    assert L.moe_dequant_weights(pi.h, 7, 0, fake, None) == M.MOE_ERR_INVALID_ARG
    assert L.moe_dequant_weights(pi.h, 13, 99, fake, None) == M.MOE_ERR_INVALID_ARG


def test_workspace_sizes(L):
    E, H, I = 16, 256, 128
    pi, pc, pm = Plan(L, "indexed", E, H, I), Plan(L, "contiguous", E, H, I), Plan(L, "masked", E, H, I)
    T, topk = 50, 4
    lay = M.RoutingLayout()
    L.moe_routing_layout(pi.h, T, topk, None, ctypes.byref(lay))
    ws = L.moe_workspace_bytes(pi.h, M.MOE_MODE_INDEXED, T, topk, T, None)
    assert ws >= lay.cap * I * 2 + T * topk * H * 2 + lay.total_ints * 4   # a, 16-bit weighted rows, routing
    assert L.moe_workspace_bytes(pm.h, M.MOE_MODE_MASKED, 64, 0, 0, None) >= E * 64 * I * 2
    assert L.moe_workspace_bytes(pc.h, M.MOE_MODE_CONTIGUOUS, 256, 4, T, None) >= 256 * I * 2 + T * 4 * H * 2
    assert L.moe_workspace_bytes(pc.h, M.MOE_MODE_INDEXED, 256, 4, T, None) == 0   # wrong mode


def test_describe_reports_schedule(L):
    p = Plan(L, "indexed", E=384, H=7168, I=2048)
    buf = ctypes.create_string_buffer(512)
    n = L.moe_describe(p.h, M.MOE_MODE_INDEXED, 448, 8, 0, None, buf, 512)
    assert n > 0
    s = buf.value.decode()
    assert "rows_per_expert=10" in s and "schedule=" in s


def test_status_strings(L):
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(4) == b"MOE_ERR_OVERRIDE_REJECTED"


def test_schedule_choice_by_rows_per_expert(L):
    """Indexed: below 80 rows per expert small-M with 16-row alignment, at
    or above it large-M with 128-row blocks (tokens per expert, not total
    tokens, decide); an explicit large-M request the kernel cannot serve is
    rejected."""
    p = Plan(L, "indexed", E=16, H=256, I=128)
    assert L.moe_routing_block(p.h, 100, 4, None) == 16        # 25 rows / expert
    assert L.moe_routing_block(p.h, 320, 4, None) == 128       # 80 rows / expert
    small = M.Tuning(0, 1, 0, 0)
    assert L.moe_routing_block(p.h, 320, 4, ctypes.byref(small)) == 16
    large = M.Tuning(0, 2, 0, 0)
    assert L.moe_routing_block(p.h, 8, 2, ctypes.byref(large)) == 128
    large64 = M.Tuning(64, 2, 0, 0)
    assert L.moe_routing_block(p.h, 320, 4, ctypes.byref(large64)) == 0
    assert "large-M" in M.last_error()
    # persistent small-M dispatch: one routing block per weight pass
    assert L.moe_routing_block(p.h, 100, 4, ctypes.byref(M.Tuning(0, 0, 1, 0))) == 32
    assert L.moe_routing_block(p.h, 40, 4, ctypes.byref(M.Tuning(0, 0, 2, 0))) == 16
    assert L.moe_routing_block(p.h, 320, 4, ctypes.byref(M.Tuning(0, 0, 2, 0))) == 128   # large-M
    assert L.moe_routing_block(p.h, 100, 4, ctypes.byref(M.Tuning(0, 0, 3, 0))) == 32
    assert L.moe_routing_block(p.h, 100, 4, ctypes.byref(M.Tuning(0, 0, 4, 0))) == 0
    assert "dispatch" in M.last_error()
    tail = Plan(L, "indexed", E=16, H=160, I=96)               # K not whole 128-chunks
    assert L.moe_routing_block(tail.h, 320, 4, None) == 16
    assert L.moe_routing_block(tail.h, 320, 4, ctypes.byref(large)) == 0
    fake = ctypes.c_void_p(1 << 20)
    st = L.moe_w4a16_indexed(tail.h, fake, 320, 4, fake, fake, None, fake, fake, 1 << 40,
                             ctypes.byref(large), None)
    assert st == M.MOE_ERR_OVERRIDE_REJECTED


def test_noalloc_scratch_size_and_host_checks(L):
    """The fixed scratch array behind moe_w4a16_indexed_noalloc holds the
    Kimi decode shape's workspace; a call that needs more fails with
    WORKSPACE_TOO_SMALL on the host, before anything is enqueued."""
    text = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == M.NOALLOC_SCRATCH_BYTES
    d = desc(E=384, H=7168, I=2048)
    h = L.moe_plan_create(ctypes.byref(d))
    assert h
    try:
        need = L.moe_workspace_bytes(h, M.MOE_MODE_INDEXED, 448, 8, 448, None)
        assert 0 < need <= M.NOALLOC_SCRATCH_BYTES, need
        big = L.moe_workspace_bytes(h, M.MOE_MODE_INDEXED, 4096, 8, 4096, None)
        assert big > M.NOALLOC_SCRATCH_BYTES
        st = L.moe_w4a16_indexed_noalloc(h, 16, 4096, 8, 16, 16, 16, None, None)
        assert st == 5 and b"scratch" in L.moe_last_error()          # WORKSPACE_TOO_SMALL
        # fits: stops at the plan's missing weights, before any HIP call
        st = L.moe_w4a16_indexed_noalloc(h, 16, 448, 8, 16, 16, 16, None, None)
        assert st == 1 and b"no prepared weights" in L.moe_last_error()
        assert L.moe_w4a16_indexed_noalloc(h, 16, 448, 8, None, 16, 16, None, None) == 1   # NULL ids
        assert L.moe_w4a16_indexed_noalloc(h, 16, 0, 8, 16, 16, 16, None, None) == 0       # nothing to do
    finally:
        L.moe_release_weights(h)
