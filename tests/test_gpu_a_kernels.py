"""GPU parity of the bit-exact steps: alignment, permutation, dequantisation,
and the MFMA fragment mapping (one-hot weights), through the C ABI."""
import numpy as np
import pytest

import synth
from oracle import moe_oracle as O
from tests.gpu_util import (bf16_dev, bits_host, check_tol, f32_dev, i32_dev, log, prepare,
                            require_gpu)

pytestmark = pytest.mark.gpu


def tiny_weights(E, H, I, seed=0):
    r = np.random.default_rng(seed)
    w13_q = r.integers(0, 2**32, (E, 2 * I, H // 8), dtype=np.uint32).view(np.int32)
    w2_q = r.integers(0, 2**32, (E, H, I // 8), dtype=np.uint32).view(np.int32)
    w13_s = synth._to_bf16_bits((np.abs(r.standard_normal((E, 2 * I, H // 32))) * 0.02 + 1e-3).astype(np.float32))
    w2_s = synth._to_bf16_bits((np.abs(r.standard_normal((E, H, I // 32))) * 0.02 + 1e-3).astype(np.float32))
    return w13_q, w13_s, w2_q, w2_s


ROUTINGS = [
    # (name, E, T, topk, kind)
    ("cfg0", 8, 32, 2, "softmax"),
    ("cfg1", 384, 448, 8, "softmax"),
    ("cfg2-zipf", 384, 8192, 8, "zipf"),
    ("cfg4", 384, 4096, 8, "softmax"),
    ("one-token", 5, 1, 3, "softmax"),
    ("ragged", 7, 1001, 3, "softmax"),
    ("small-path-max", 64, 512, 8, "softmax"),   # 4096 rows: the one-workgroup path's limit
    ("chunked-path-min", 64, 513, 8, "zipf"),    # 4104 rows: the smallest multi-workgroup case
    ("experts-513", 513, 40, 4, "softmax"),      # above the one-workgroup path's 512 experts, few rows
    ("experts-max", 4096, 700, 8, "zipf"),       # the largest expert count a handle accepts
    ("topk-max", 96, 64, 64, "softmax"),         # the largest top-k (64): 4096 rows
    ("many-rows", 384, 16384, 8, "zipf"),        # 131072 rows in 128 chunks
    ("no-rows-chunked", 600, 0, 4, "softmax"),   # no rows above 512 experts: the scan alone writes the sentinels
]


def routing_ids(E, T, topk, kind, seed):
    if kind == "zipf":
        return synth.zipf_routing(seed, T, E, topk)[0]
    return synth.softmax_routing(seed, T, E, topk)[0]


@pytest.fixture(scope="module")
def handles():
    require_gpu()
    cache = {}

    def get(E):
        if E not in cache:
            cache[E] = prepare(tiny_weights(E, 64, 32), "indexed")
        return cache[E]
    return get


def read_routing(h, routing, T, topk, ovr=None):
    lay = h.routing_layout(T, topk, ovr)
    r = routing.cpu().numpy()
    E = h.E
    return dict(counts=r[lay.off_counts:lay.off_counts + E],
                offsets=r[lay.off_offsets:lay.off_offsets + E + 1],
                sorted_ids=r[lay.off_sorted:lay.off_sorted + lay.cap],
                block_expert=r[lay.off_block_expert:lay.off_block_expert + lay.nblocks],
                slot_of=r[lay.off_slot_of:lay.off_slot_of + lay.sentinel],
                total=int(r[7]), block=lay.block)


def slot_of_ref(al):
    """Inverse of the oracle's sorted_ids over flat rows (-1: routed nowhere)."""
    inv = np.full(al["sentinel"], -1, np.int32)
    sid = al["sorted_ids"]
    p = np.flatnonzero(sid < al["sentinel"])
    inv[sid[p]] = p
    return inv


@pytest.mark.parametrize("name,E,T,topk,kind", ROUTINGS)
@pytest.mark.parametrize("block_m", [0, 16, 64, 128])
def test_align_bit_exact(handles, name, E, T, topk, kind, block_m):
    h = handles(E)
    ids = routing_ids(E, T, topk, kind, seed=200 + T)
    if name == "ragged":
        ids[::17, 0] = -1          # dropped rows
        ids[5, 1] = E              # out of range
    ovr = {"block_m": block_m} if block_m else None
    ids_d = i32_dev(ids)
    first = None
    for rep in range(3):
        routing = h.align(ids_d, ovr=ovr)
        got = read_routing(h, routing, T, topk, ovr)
        if first is None:
            first = got
        else:
            for k in ("sorted_ids", "offsets"):
                assert np.array_equal(got[k], first[k]), f"nondeterministic {k}"
    ref = O.align(ids, E, got["block"])
    log(f"  align {name} B={got['block']} total={ref['total']} cap={ref['cap']}")
    for k in ("counts", "offsets", "sorted_ids", "block_expert"):
        assert np.array_equal(got[k], ref[k]), k
    assert np.array_equal(got["slot_of"], slot_of_ref(ref))
    assert got["total"] == ref["total"]


EP_CASES = [
    # (Eg, E_local, T, topk, placement, kind): one GPU's share of Eg experts
    (384, 48, 448, 8, "contiguous", "softmax"),      # EP8 share of the decode routing
    (384, 48, 448, 8, "round-robin", "softmax"),
    (384, 48, 6000, 8, "round-robin", "zipf"),       # multi-workgroup path (48000 rows)
    (16, 5, 37, 3, "contiguous", "softmax"),
]


def ep_map(Eg, E_local, placement, g=1):
    emap = np.full(Eg, -1, dtype=np.int32)
    if placement == "contiguous":
        mine = np.arange(g * E_local, (g + 1) * E_local)
    else:
        mine = np.arange(g, Eg, Eg // E_local)[:E_local]
    emap[mine] = np.arange(mine.size)
    return emap


@pytest.mark.parametrize("Eg,E,T,topk,placement,kind", EP_CASES)
@pytest.mark.parametrize("block_m", [0, 128])
def test_align_ep_bit_exact(handles, Eg, E, T, topk, placement, kind, block_m):
    """Expert-parallel alignment: global ids through the share's map."""
    h = handles(E)
    ids = routing_ids(Eg, T, topk, kind, seed=300 + T).copy()
    ids[::13, 0] = -1
    ids[3 % T, topk - 1] = Eg + 2
    emap = ep_map(Eg, E, placement)
    ovr = {"global_experts": Eg}
    if block_m:
        ovr["block_m"] = block_m
    routing = h.align_ep(i32_dev(ids), i32_dev(emap), Eg, ovr=ovr)
    got = read_routing(h, routing, T, topk, ovr)
    ref = O.align(O.ep_local_ids(ids, emap), E, got["block"])
    log(f"  align_ep Eg={Eg} E={E} T={T} {placement} B={got['block']} total={ref['total']}")
    for k in ("counts", "offsets", "sorted_ids", "block_expert"):
        assert np.array_equal(got[k], ref[k]), k
    assert np.array_equal(got["slot_of"], slot_of_ref(ref))
    assert got["total"] == ref["total"]


def test_align_empty(handles):
    import torch
    h = handles(8)
    ids = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    routing = h.align(ids)
    got = read_routing(h, routing, 0, 2)
    ref = O.align(np.zeros((0, 2), np.int32), 8, got["block"])
    for k in ("counts", "offsets", "sorted_ids", "block_expert"):
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("block_m", [16, 128])
def test_permute_bit_exact(handles, block_m):
    E, T, topk = 7, 300, 3
    h = handles(E)
    ids = routing_ids(E, T, topk, "softmax", 5)
    x = synth.activations(9, T, 64)
    ovr = {"block_m": block_m}
    routing = h.align(i32_dev(ids), ovr=ovr)
    a, m_idx, row_src = h.permute(bf16_dev(x), topk, routing, ovr=ovr)
    al = O.align(ids, E, block_m)
    # rows of a past the padded total lie outside the layout and are not written
    n = al["total"]
    assert int(routing[7].item()) == n
    assert np.array_equal(bits_host(a)[:n], O.permute(x, al, topk)[:n])
    ok = al["sorted_ids"] < al["sentinel"]
    m_ref = np.where(ok, np.repeat(al["block_expert"], block_m)[:al["cap"]], -1)
    assert np.array_equal(m_idx.cpu().numpy(), m_ref)
    assert np.array_equal(row_src.cpu().numpy(), np.where(ok, al["sorted_ids"], -1))


def test_permute_into_given_buffers(handles):
    """permute() into caller-given buffers (as the bench's routing step
    reuses them call after call) writes what a fresh call returns, twice in
    a row, and refuses buffers smaller than the routing's capacity."""
    import torch
    import w4a16_int4_grouped_amd as M
    E, T, topk = 7, 300, 3
    h = handles(E)
    ovr = {"block_m": 128}
    x = bf16_dev(synth.activations(9, T, 64))
    ids = i32_dev(routing_ids(E, T, topk, "softmax", 5))
    routing = h.align(ids, ovr=ovr)
    ref = [v.cpu() for v in h.permute(x, topk, routing, ovr=ovr)]
    cap, n = ref[0].shape[0], int(routing[7].item())
    assert 0 < n < cap
    bufs = (torch.full((cap, 64), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16),
            torch.full((cap,), 12345, dtype=torch.int32, device="cuda"),
            torch.full((cap,), 12345, dtype=torch.int32, device="cuda"))
    for _ in range(2):
        got = h.permute(x, topk, h.align(ids, ovr=ovr, routing=routing), ovr=ovr, out=bufs)
        assert all(g is b for g, b in zip(got, bufs))
        a = got[0].cpu().view(torch.int16)
        assert torch.equal(a[:n], ref[0].view(torch.int16)[:n])
        assert bool((a[n:] == -1).all()), "rows past the padded total must stay unwritten"
        assert torch.equal(got[1].cpu(), ref[1]) and torch.equal(got[2].cpu(), ref[2])
    short = (bufs[0][:cap - 1], bufs[1], bufs[2])
    with pytest.raises(M.MoeError, match="INVALID_ARG"):
        h.permute(x, topk, routing, ovr=ovr, out=short)


@pytest.mark.parametrize("E", [7, 600])
def test_permute_empty_routing(handles, E):
    """No tokens: every slot's m_indices and row_src become -1 and no row of
    a_out is written (the padded total is 0), on both alignment paths."""
    import torch
    h = handles(E)
    ids = i32_dev(np.zeros((0, 4), np.int32))
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    routing = h.align(ids)
    cap = h.routing_layout(0, 4).cap
    assert int(routing[7].item()) == 0 and cap > 0
    bufs = (torch.full((cap, 64), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16),
            torch.full((cap,), 12345, dtype=torch.int32, device="cuda"),
            torch.full((cap,), 12345, dtype=torch.int32, device="cuda"))
    a, m, r = h.permute(x, 4, routing, out=bufs)
    torch.cuda.synchronize()
    assert bool((m == -1).all()) and bool((r == -1).all())
    assert bool((a.view(torch.int16) == -1).all()), "a row past the padded total was written"


def test_dequant_exhaustive_all_scales():
    """Every finite BF16 scale below 2^117 in magnitude (plus zeros and
    subnormals) against all 16 codes, through the GEMMs' dequantisation
    routine (the inspection path adds only the sign of exactly-zero
    products, which an MFMA cannot observe)."""
    require_gpu()
    s_all = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    supported = (s_all & 0x7FFF) < 0x7A00
    s = s_all[supported]
    # one expert, W13 with N = 2I rows, K = H columns: N*(K/32) >= len(s)
    H, I = 1024, 1024
    N, G = 2 * I, H // 32
    assert N * G >= s.size
    scales = np.resize(s, N * G).reshape(N, G)
    # every group of 32 holds each of the 16 codes twice
    q = ((np.arange(H)[None, :] + np.arange(N)[:, None]) % 16).astype(np.uint32)
    words = np.zeros((N, H // 8), dtype=np.uint32)
    for i in range(8):
        words |= q[:, i::8] << np.uint32(4 * i)
    w13_q = words.view(np.int32)[None]
    w13_s = scales[None]
    w2 = tiny_weights(1, H, I, seed=3)
    h = prepare((w13_q, w13_s, w2[2], w2[3]), "indexed")
    got = bits_host(h.dequant(13, 0))
    ref = O.dequant(w13_q[0], w13_s[0])
    nan_ref = np.isnan(O.bf16_to_f64(ref))
    assert not nan_ref.any()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}: got {got[tuple(bad[0])]:#x} ref {ref[tuple(bad[0])]:#x}"
    got2 = bits_host(h.dequant(2, 0))
    assert np.array_equal(got2, O.dequant(w2[2][0], w2[3][0]))


def test_unsupported_scales_fail_at_load():
    require_gpu()
    import w4a16_int4_grouped_amd as M
    w = list(tiny_weights(2, 64, 32))
    for bad in (0x7F80, 0x7FC0, 0x7A00, 0xFE00):
        w13_s = w[1].copy()
        w13_s[1, 3, 1] = bad
        with pytest.raises(M.MoeError) as ei:
            prepare((w[0], w13_s, w[2], w[3]), "indexed")
        assert ei.value.status == M.MOE_ERR_UNSUPPORTED_SCHEMA


@pytest.mark.parametrize("cfg", [0, 4])
def test_dequant_config_weights_bit_exact(cfg):
    """The configs' own weights: every expert of config 0, sampled experts
    (first, middle, last) of the TP8 shard."""
    require_gpu()
    wl = synth.WORKLOADS[cfg]
    experts = list(range(wl.E)) if wl.E <= 8 else [0, wl.E // 2, wl.E - 1]
    w = synth.stacked_weights(wl)
    h = prepare(w, "indexed")
    for e in experts:
        assert np.array_equal(bits_host(h.dequant(13, e)), O.dequant(w[0][e], w[1][e])), (cfg, e, 13)
        assert np.array_equal(bits_host(h.dequant(2, e)), O.dequant(w[2][e], w[3][e])), (cfg, e, 2)


def onehot_weights(E, H, I):
    """Row n has its single nonzero at k = (3n + 1) mod K (not symmetric, so
    a transposed tile shows), and power-of-two scales that vary with the row,
    the scale group and the expert."""
    def mat(N, K, scale_bits):
        q = np.full((N, K), 8, dtype=np.uint32)
        q[np.arange(N), (3 * np.arange(N) + 1) % K] = 9
        words = np.zeros((N, K // 8), dtype=np.uint32)
        for i in range(8):
            words |= q[:, i::8] << np.uint32(4 * i)
        g = np.arange(K // 32)[None, :]
        n = np.arange(N)[:, None]
        s = (scale_bits + (((n + 3 * g) % 4) << 7)).astype(np.uint16)
        return words.view(np.int32), s
    w13 = [mat(2 * I, H, 0x3F80 - (e << 7)) for e in range(E)]
    w2 = [mat(H, I, 0x3F00 + (e << 7)) for e in range(E)]
    return (np.stack([a for a, _ in w13]), np.stack([b for _, b in w13]),
            np.stack([a for a, _ in w2]), np.stack([b for _, b in w2]))


def test_fragment_mapping_onehot():
    """One nonzero term per dot product: any row/column/k/scale-group or
    gate/up mix-up in the MFMA fragment layout is an O(1) error."""
    require_gpu()
    E, H, I, T, topk = 4, 256, 128, 19, 2
    w = onehot_weights(E, H, I)
    r = np.random.default_rng(4)
    x = synth.activations(3, T, H)
    ids = np.stack([r.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    tw = r.random((T, topk)).astype(np.float32)
    h = prepare(w, "indexed")
    out = h.indexed(bf16_dev(x), i32_dev(ids), f32_dev(tw))
    ref = O.moe_indexed(x, ids, tw, w, E=E)
    got = O.bf16_to_f64(bits_host(out))
    # exact up to BF16 output rounding and FP32 silu
    rms = float(np.sqrt(np.mean(ref ** 2)))
    np.testing.assert_allclose(got, ref, rtol=2 ** -7, atol=1e-2 * rms)
    check_tol(got, ref, "one-hot")
