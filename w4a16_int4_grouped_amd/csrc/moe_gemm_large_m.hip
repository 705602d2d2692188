// Grouped W4A16 GEMM, large-M schedule (many rows per expert).
//
// Above roughly 80 rows per expert the GEMM is a dense contraction and the
// tile follows each expert's padded rows (Chord page, "Indexed kernels",
// Fig. 2, and "H200 prefill and TP8": block_m sized to the padded rows).
//
// Work item: one 128-row token tile x 256 weight rows. The four waves each
// own one row group of 64 weight rows (4 MFMA tiles of 16 rows) and all 128
// tokens (8 MFMA tiles of 16 columns), so a wave holds 4 x 8 accumulator
// tiles. Weights stay on the A side of v_mfma_f32_16x16x32_bf16 as in the
// small-M kernel and use the same prepared layout: a lane's 32 k values of a
// tile share one scale group, so a dequantised A fragment (17 VALU
// instructions for 8 weights) feeds eight MFMAs, and VALU work stays near
// half of the MFMA time.
//
// Per K chunk of 128:
//   * the token tile (128 rows x 128 k of BF16, 32 KB) goes straight from
//     global memory to LDS (global_load_lds_dwordx4, no staging registers),
//     one chunk ahead, into the other of two buffers;
//   * each wave loads its 4 KB of packed weights and 512 B of scales one
//     chunk ahead into registers;
//   * both are issued at the top of the chunk, so the barrier at its end
//     (which waits for every outstanding load) finds them long arrived.
// The LDS layout of a buffer (swizzled 1 KB groups of 16 rows x 4 pieces)
// is described in moe_tile.h.
//
// Row sets: a 128-slot block of the indexed routing (block 128; rows via
// sorted_ids, pad slots hold the sentinel), a 128-row block of the
// contiguous layout, or an expert of the masked layout (tiles of 128 over
// its valid rows). Epilogues as in the small-M kernel.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_launch.h"
#include "moe_tile.h"

namespace moe {

namespace {

constexpr int kBM = 128;                       // token rows per tile
constexpr int kBufU4 = kBM * kKC * 2 / 16;     // 16-byte slots per LDS buffer (2048)

struct AFragL {
  u32x4_t A[kMT];
  u32x2_t S;
};

__device__ __forceinline__ void load_a_l(AFragL& f, const u32x4_t* __restrict__ wq,
                                         const u32x2_t* __restrict__ ws, int lane) {
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) f.A[mt] = __builtin_nontemporal_load(wq + mt * 64 + lane);
  f.S = __builtin_nontemporal_load(ws + lane);
}

// One K chunk: 4 MFMA steps g of 32 k over the first NTE token tiles. The
// token fragments of a step stay in registers while the wave's 4 weight
// tiles pass one at a time; each tile's MFMAs carry the dequantisation of
// the next tile (17 VALU instructions) and, on the last tile of a step, the
// LDS reads of the next step's token fragments. HINTS: interleave them in a
// fixed issue order (each MFMA followed by its share of the vector work),
// which pays in the K loop, where global loads and a barrier share the
// chunk; the barrier-free resident form runs faster with the compiler's own
// order (measured: down projection of the TP8 shard 362 -> 325 us).
template <int NTE, bool HINTS>
__device__ __forceinline__ void mma_chunk_l(const AFragL& f, const u32x4_t* lds_buf, int rd0,
                                            f32x4_t (&acc)[kMT][NTE], uint32_t mlo, uint32_t mhi) {
  constexpr int kValuPerMfma = NTE >= 8 ? 2 : (17 + NTE - 1) / NTE;
  GroupScale gs[kMT];
  {
    const float sc[4] = {bf16_lo(f.S[0]), bf16_hi(f.S[0]), bf16_lo(f.S[1]), bf16_hi(f.S[1])};
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) gs[mt] = group_scale(sc[mt]);
  }
  u32x4_t b[NTE];
#pragma unroll
  for (int nt = 0; nt < NTE; ++nt) b[nt] = lds_buf[rd0 + nt * 256];
  u32x4_t a = dq8(f.A[0][0], gs[0], mlo, mhi);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const bool last = (mt == kMT - 1);
      const int ng = last ? g + 1 : g, nmt = last ? 0 : mt + 1;
      u32x4_t an = a;
      if (ng < 4) an = dq8(f.A[nmt][ng], gs[nmt], mlo, mhi);
#pragma unroll
      for (int nt = 0; nt < NTE; ++nt) {
        acc[mt][nt] = mfma16(a, b[nt], acc[mt][nt]);
        // the step's last use of b[nt]: its register takes the next step's
        if (last && g < 3) b[nt] = lds_buf[(rd0 ^ (g + 1)) + nt * 256];
      }
      if constexpr (HINTS) {
        // issue order within the region: each MFMA followed by its share of
        // the vector work (and of the next step's LDS reads)
#pragma unroll
        for (int i = 0; i < NTE; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
          if (last && g < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);         // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      a = an;
    }
  }
}

// The K loop of one tile over its first NTE token tiles: chunk c+1's token
// tile (only the waves whose rows are read load theirs) and weights are
// fetched while chunk c is computed.
template <int NTE>
__device__ __forceinline__ void k_loop(u32x4_t (&lds)[2][kBufU4], const char* src0, const char* src1,
                                       int wave, int lane, const u32x4_t* __restrict__ wq,
                                       const u32x2_t* __restrict__ ws, int Kc, int rd0,
                                       f32x4_t (&acc)[kMT][NTE]) {
  const bool loader = 2 * wave < NTE;   // this wave's 32 rows are read
  const uint32_t mlo = kF16MagicLo, mhi = kF16MagicHi;
  AFragL fa, fb;
  __syncthreads();   // the previous tile's readers are done with buffer 0
  if (loader) dma_tile(lds[0], src0, src1, 0, wave);
  load_a_l(fa, wq, ws, lane);
  __syncthreads();

  // step: compute chunk c from (CUR, buffer BUF); chunk c+1 is fetched into
  // (NXT, the other buffer) first.
#define MOE_LARGE_M_STEP(BUF, CUR, NXT, C)                                                    \
  if ((C) < Kc) {                                                                             \
    if ((C) + 1 < Kc) {                                                                       \
      if (loader) dma_tile(lds[(BUF) ^ 1], src0, src1, (C) + 1, wave);                        \
      load_a_l(NXT, wq + (size_t)((C) + 1) * (kMT * 64), ws + (size_t)((C) + 1) * 64, lane);  \
    }                                                                                         \
    mma_chunk_l<NTE, true>(CUR, lds[BUF], rd0, acc, mlo, mhi);                                      \
    __syncthreads();                                                                          \
  }
  for (int kc = 0; kc < Kc; kc += 2) {
    MOE_LARGE_M_STEP(0, fa, fb, kc)
    MOE_LARGE_M_STEP(1, fb, fa, kc + 1)
  }
#undef MOE_LARGE_M_STEP
}

// Per-workgroup state of one row set.
struct TileCtx {
  const u32x4_t* wq;
  const u32x2_t* ws;
  int lane, wave, rg, e, slot0, count, rd0;
  bool active;
};

// This lane's two DMA source rows of token tile tb (row 32*wave + 16*ql +
// lane/4 of the tile), each advanced to its swizzled 16-byte piece.
template <int SET, int EPI>
__device__ __forceinline__ void tile_sources(const GemmParams& p, const TileCtx& c, int tb,
                                             const char* (&src)[2]) {
  // rows of x gathered through the routing (W13 of the indexed layout)
  const bool gather = SET == SET_ROUTED && p.gather;
  const int lane = c.lane;
  const int piece = dma_piece(lane);
#pragma unroll
  for (int ql = 0; ql < 2; ++ql) {
    const int r = tb + 32 * c.wave + 16 * ql + (lane >> 2);   // tile row
    int row;
    if constexpr (SET == SET_ROUTED) {
      if (gather) {
        const int f = p.sorted_ids[c.slot0 + r];
        row = (f >= 0 && f < p.sentinel) ? f / p.topk : 0;   // pad slots read row 0
      } else {
        row = c.slot0 + r;
      }
    } else if constexpr (SET == SET_MASKED) {
      row = c.slot0 + min(r, c.count - 1);   // pad rows repeat a valid row
    } else {
      row = c.slot0 + r;
    }
    src[ql] = reinterpret_cast<const char*>(p.src + (size_t)row * p.src_ld) + piece;
  }
}

// Writes the accumulators of row group rg for token rows tb .. tb + rows.
// The rows' routing data (slot contents, source row, routing weight) is
// loaded for all NTE token tiles before any tile is written, so those loads
// are in flight together: two dependent round trips per tile instead of two
// per token tile (measured on the prefill down projection: the epilogue took
// 16 % of the wave time with a round trip per tile).
template <int SET, int EPI, int NTE>
__device__ __forceinline__ void epilogue(const GemmParams& p, const TileCtx& c, int tb, int rows,
                                         int rg, const f32x4_t (&acc)[kMT][NTE]) {
  const int lane = c.lane;
  // what each row writes: ROUTED the flat index at its slot; BLOCKS with
  // COMBINE the flat index its row_src gives; otherwise >= 0. -1: nothing.
  int fv[NTE];
#pragma unroll
  for (int nt = 0; nt < NTE; ++nt) {
    const int r = tb + nt * 16 + (lane & 15);
    const bool in = r < c.count && r - tb < rows;
    const int slot = c.slot0 + (in ? r : tb);   // a row of the tile: always readable
    if constexpr (SET == SET_ROUTED) {
      fv[nt] = in ? p.sorted_ids[slot] : -1;
    } else if constexpr (EPI == EPI_COMBINE) {
      fv[nt] = in ? p.m_indices[slot] : -1;
    } else {
      fv[nt] = in ? 0 : -1;
    }
  }
  if constexpr (SET != SET_ROUTED && EPI == EPI_COMBINE) {
    int src[NTE];   // loaded for every row (a load under a branch would wait alone)
#pragma unroll
    for (int nt = 0; nt < NTE; ++nt) {
      const int r = min(tb + nt * 16 + (lane & 15), c.count - 1);
      src[nt] = p.row_src[c.slot0 + r];
    }
#pragma unroll
    for (int nt = 0; nt < NTE; ++nt) fv[nt] = fv[nt] == c.e ? src[nt] : -1;
  }
  if constexpr (SET == SET_ROUTED || EPI == EPI_COMBINE) {
#pragma unroll
    for (int nt = 0; nt < NTE; ++nt)
      if (fv[nt] >= p.sentinel) fv[nt] = -1;   // pad slot (ROUTED), out-of-range source (COMBINE)
  }
  float wv[NTE];
  if constexpr (EPI == EPI_COMBINE) {
#pragma unroll
    for (int nt = 0; nt < NTE; ++nt) wv[nt] = p.topk_w[fv[nt] >= 0 ? fv[nt] : 0];
  }
#pragma unroll
  for (int nt = 0; nt < NTE; ++nt) {
    if (fv[nt] < 0) continue;
    const int slot = c.slot0 + tb + nt * 16 + (lane & 15);
    if constexpr (EPI == EPI_SWIGLU) {
      uint16_t* dst = p.a_out + (size_t)slot * p.a_ld + rg * 32 + (lane >> 4) * 4;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const f32x4_t g = acc[2 * pp][nt], u = acc[2 * pp + 1][nt];
        u32x2_t v;
        v[0] = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
        v[1] = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
        *reinterpret_cast<u32x2_t*>(dst + pp * 16) = v;
      }
    } else if constexpr (EPI == EPI_COMBINE) {
      if (rg * kRowsRG < p.N) {   // the row group's 64 features, lane-contiguous (store_y16)
        f32x4_t v[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) v[mt] = acc[mt][nt];
        store_y16<kMT>(p.yq, (size_t)fv[nt] * p.yrows_ld + rg * kRowsRG + (lane >> 4) * 16, wv[nt], v);
      }
    } else {
      uint16_t* dst = p.out + (size_t)slot * p.out_ld;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int n = store_col(p.N, p.gate_up_I, rg, mt, lane);
        if (n >= 0) {
          u32x2_t v;
          v[0] = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
          v[1] = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
          *reinterpret_cast<u32x2_t*>(dst + n) = v;
        }
      }
    }
  }
}

// Row metadata of a resident tile, built once in LDS: for each tile row
// the flat index f it feeds (-1: nothing to write) and its routing weight.
struct RowMeta {
  int32_t f[kBM];
  float w[kBM];
};

template <int SET, int EPI>
__device__ __forceinline__ void build_meta(const GemmParams& p, const TileCtx& c, RowMeta& m) {
  for (int r = threadIdx.x; r < kBM; r += 256) {
    const int slot = c.slot0 + r;
    int f;
    if constexpr (SET == SET_ROUTED) {
      f = p.sorted_ids[slot];
    } else if constexpr (EPI == EPI_COMBINE) {
      f = (p.m_indices[slot] == c.e) ? p.row_src[slot] : -1;
    } else {
      f = 0;   // contiguous rows are written by slot
    }
    const bool ok = f >= 0 && (SET != SET_ROUTED && EPI != EPI_COMBINE ? true : f < p.sentinel);
    m.f[r] = ok ? f : -1;
    m.w[r] = (EPI == EPI_COMBINE && ok) ? p.topk_w[f] : 0.f;
  }
}

// The epilogue of the resident form: row validity and weights from LDS.
template <int SET, int EPI, int NTE>
__device__ __forceinline__ void epilogue_meta(const GemmParams& p, const TileCtx& c, int rows, int rg,
                                              const RowMeta& m, const f32x4_t (&acc)[kMT][NTE]) {
  const int lane = c.lane;
#pragma unroll
  for (int nt = 0; nt < NTE; ++nt) {
    const int r = nt * 16 + (lane & 15);
    if (r >= rows) continue;
    const int f = m.f[r];
    if (f < 0) continue;
    const int slot = c.slot0 + r;
    if constexpr (EPI == EPI_SWIGLU) {
      uint16_t* dst = p.a_out + (size_t)slot * p.a_ld + rg * 32 + (lane >> 4) * 4;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const f32x4_t g = acc[2 * pp][nt], u = acc[2 * pp + 1][nt];
        u32x2_t v;
        v[0] = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
        v[1] = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
        *reinterpret_cast<u32x2_t*>(dst + pp * 16) = v;
      }
    } else if constexpr (EPI == EPI_COMBINE) {
      const float w = m.w[r];
      if (rg * kRowsRG < p.N) {   // the row group's 64 features, lane-contiguous (store_y16)
        f32x4_t v[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) v[mt] = acc[mt][nt];
        store_y16<kMT>(p.yq, (size_t)f * p.yrows_ld + rg * kRowsRG + (lane >> 4) * 16, w, v);
      }
    } else {
      uint16_t* dst = p.out + (size_t)slot * p.out_ld;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int n = store_col(p.N, p.gate_up_I, rg, mt, lane);
        if (n >= 0) {
          u32x2_t v;
          v[0] = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
          v[1] = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
          *reinterpret_cast<u32x2_t*>(dst + n) = v;
        }
      }
    }
  }
}

// One token tile (rows tb .. tb + 128 of the set, `rows` of them worth
// computing): source rows, the K loop over the first NTE token tiles, and
// the epilogue. Each NTE is a complete body, so no accumulator is live
// across the choice.
template <int SET, int EPI, int NTE>
__device__ __forceinline__ void run_tile(const GemmParams& p, const TileCtx& c,
                                         u32x4_t (&lds)[2][kBufU4], int tb, int rows) {
  const char* src[2];
  tile_sources<SET, EPI>(p, c, tb, src);
  f32x4_t acc[kMT][NTE];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTE; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  k_loop<NTE>(lds, src[0], src[1], c.wave, c.lane, c.wq, c.ws, p.Kc, c.rd0, acc);
  if (c.active) epilogue<SET, EPI, NTE>(p, c, 0 + tb, rows, c.rg, acc);
}

// K-resident form for K <= 256 (KCR = K / 128 chunks): the token tile is
// loaded into LDS once (chunk c in buffer c) and the workgroup walks row
// group quads q0 .. q1 of the output, each wave streaming its weights one
// chunk ahead across quad boundaries. The tile is read-only after the first
// barrier, so the loop has no barrier at all; a short-K GEMM with many
// output rows (the down projection of a TP8 shard) no longer pays a
// workgroup start and a tile load per 256 output rows.
template <int SET, int EPI, int NTE, int KCR>
__device__ __forceinline__ void run_tile_res(const GemmParams& p, const TileCtx& c,
                                             u32x4_t (&lds)[2][kBufU4], RowMeta& meta, int rows,
                                             int q0, int q1) {
  const int lane = c.lane, wave = c.wave;
  const uint32_t mlo = kF16MagicLo, mhi = kF16MagicHi;
  const char* src[2];
  tile_sources<SET, EPI>(p, c, 0, src);
  if (2 * wave < NTE) {   // this wave's 32 rows are read
#pragma unroll
    for (int kc = 0; kc < KCR; ++kc) dma_tile(lds[kc], src[0], src[1], kc, wave);
  }
  // weights of (quad q, chunk kc) for this wave (row group clamped: waves
  // past the last row group stream a valid one and skip the epilogue)
  auto wq_of = [&](int q) {
    const int rg = min(q * 4 + wave, p.RG - 1);
    return ((size_t)c.e * p.RG + rg) * KCR;
  };
  const u32x4_t* __restrict__ wq0 = reinterpret_cast<const u32x4_t*>(p.wq);
  const u32x2_t* __restrict__ ws0 = reinterpret_cast<const u32x2_t*>(p.wsc);
  AFragL fa, fb;
  {
    const size_t t0 = wq_of(q0);
    load_a_l(fa, wq0 + t0 * (kMT * 64), ws0 + t0 * 64, lane);
    if constexpr (KCR == 2) load_a_l(fb, wq0 + (t0 + 1) * (kMT * 64), ws0 + (t0 + 1) * 64, lane);
  }
  build_meta<SET, EPI>(p, c, meta);
  __syncthreads();   // the token tile and the row metadata are in LDS
  for (int q = q0; q < q1; ++q) {
    // keep the epilogue's LDS reads inside the loop: hoisted, they would hold
    // registers across the whole quad loop
    asm volatile("" ::: "memory");
    const int rg = q * 4 + wave;
    const size_t tn = wq_of(q + 1 < q1 ? q + 1 : q);   // past the last quad: a valid repeat
    f32x4_t acc[kMT][NTE];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTE; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (KCR == 2) {
      // both chunks of the next quad are requested before this quad's
      // epilogue: vmcnt counts stores and loads in one in-order counter, so
      // a weight load issued after the epilogue's stores could only be
      // waited for together with them (measured on the TP8 shard's down
      // projection: the stores then added to the compute time instead of
      // draining under the next quad's MFMAs)
      mma_chunk_l<NTE, false>(fa, lds[0], c.rd0, acc, mlo, mhi);
      load_a_l(fa, wq0 + tn * (kMT * 64), ws0 + tn * 64, lane);
      mma_chunk_l<NTE, false>(fb, lds[1], c.rd0, acc, mlo, mhi);
      load_a_l(fb, wq0 + (tn + 1) * (kMT * 64), ws0 + (tn + 1) * 64, lane);
    } else {
      load_a_l(fb, wq0 + tn * (kMT * 64), ws0 + tn * 64, lane);
      mma_chunk_l<NTE, false>(fa, lds[0], c.rd0, acc, mlo, mhi);
      fa = fb;
    }
    if (rg < p.RG) epilogue_meta<SET, EPI, NTE>(p, c, rows, rg, meta, acc);
  }
}

// Calls f(std::integral_constant<int, NTE>) with NTE = ceil(rows / 16), the
// 16-row token tiles a tile of `rows` rows (1 .. 128) computes: each count
// is a complete body, and a tile pays at most 15 padding rows of MFMAs.
template <typename F>
__device__ __forceinline__ void with_token_tiles(int rows, F&& f) {
  switch ((rows + 15) >> 4) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 5: f(std::integral_constant<int, 5>{}); break;
    case 6: f(std::integral_constant<int, 6>{}); break;
    case 7: f(std::integral_constant<int, 7>{}); break;
    default: f(std::integral_constant<int, 8>{}); break;
  }
}

// KCR = 0: K-loop form, one quad of row groups per workgroup. KCR = 1 or 2
// (K = 128 * KCR): K-resident form, p.qpw quads per workgroup.
template <int SET, int EPI, int KCR>
__global__ __launch_bounds__(256, 2) void gemm_large_m(const GemmParams p) {
  __shared__ u32x4_t lds[2][kBufU4];
  __shared__ RowMeta meta;   // resident form only (1 KB; unused and dropped otherwise)
  TileCtx c;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = c.lane;
  int logical;
  if constexpr (SET == SET_ROUTED) {
    // the grid covers the routing's capacity; only the blocks up to its
    // padded total hold rows
    const int32_t* hdr = p.routing_hdr;
    if (hdr[HDR_MAGIC] != kRoutingMagic || hdr[HDR_BLOCK] != p.block || hdr[HDR_E] != p.E ||
        hdr[HDR_T] * hdr[HDR_TOPK] != p.sentinel)
      return;   // routing made for other shapes: compute nothing
    const int nact = min(max(hdr[HDR_TOTAL], 0) / kBM, p.nsets);
    if (KCR == 0 && p.xcd_deal) {
      logical = xcd_deal_blocks(blockIdx.x, nact, p.wg_per_set, p.xcd_deal);
    } else {
      logical = xcd_remap_active(blockIdx.x, nact * p.wg_per_set);
    }
    if (logical < 0) return;
  } else if (KCR == 0 && SET == SET_BLOCKS && p.xcd_deal) {
    logical = xcd_deal_blocks(blockIdx.x, p.nsets, p.wg_per_set, p.xcd_deal);
    if (logical < 0) return;
  } else {
    logical = xcd_remap(blockIdx.x, p.total_wg);
  }
  const int set = logical / p.wg_per_set;
  const int wgi = logical - set * p.wg_per_set;
  const int rg_raw = (KCR == 0 ? wgi : wgi * p.qpw) * 4 + c.wave;
  c.active = rg_raw < p.RG;
  c.rg = c.active ? rg_raw : p.RG - 1;

  // ---- the row set (uniform over the workgroup). n_eff: one past the last
  // valid row of the (single) tile of a routing or contiguous block; token
  // tiles past it are neither loaded nor computed.
  int n_eff = kBM;
  if constexpr (SET == SET_ROUTED) {
    c.e = p.block_expert[set];
    c.slot0 = set * kBM;
    c.count = kBM;
    if (c.e < 0 || c.e >= p.E) return;
    int last = 0;
#pragma unroll
    for (int r = lane; r < kBM; r += 64) {
      const int f = p.sorted_ids[c.slot0 + r];
      if (f >= 0 && f < p.sentinel) last = r + 1;
    }
    n_eff = __builtin_amdgcn_readfirstlane(wave_max(last));
  } else if constexpr (SET == SET_MASKED) {
    c.e = set;
    c.slot0 = c.e * p.max_m;
    c.count = min(max(p.masked_m[c.e], 0), p.max_m);
  } else {   // contiguous blocks are one 128-row tile (block_rows == kBM)
    c.slot0 = set * kBM;
    c.count = kBM;
    int m[2];
    int mx = -1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      m[i] = p.m_indices[c.slot0 + lane + 64 * i];
      if (m[i] >= 0 && m[i] < p.E) mx = max(mx, m[i]);
    }
    c.e = wave_max(mx);
    int last = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (m[i] == c.e) last = lane + 64 * i + 1;
    n_eff = __builtin_amdgcn_readfirstlane(wave_max(last));
  }
  if (c.count <= 0 || c.e < 0 || c.e >= p.E || n_eff <= 0) return;

  const size_t tile0 = ((size_t)c.e * p.RG + c.rg) * p.Kc;
  c.wq = reinterpret_cast<const u32x4_t*>(p.wq) + tile0 * (kMT * 64);
  c.ws = reinterpret_cast<const u32x2_t*>(p.wsc) + tile0 * 64;
  c.rd0 = frag_rd0(lane);

  if constexpr (KCR > 0) {   // one tile (routing or contiguous block), quads q0 .. q1
    const int q0 = wgi * p.qpw, q1 = min(q0 + p.qpw, (p.RG + 3) / 4);
    if (q0 >= q1) return;
    const int rows = n_eff;
    with_token_tiles(rows, [&](auto nte) {
      run_tile_res<SET, EPI, decltype(nte)::value, KCR>(p, c, lds, meta, rows, q0, q1);
    });
  } else {
    for (int tb = 0; tb < c.count; tb += kBM) {
      const int rows = SET == SET_MASKED ? min(c.count - tb, kBM) : n_eff;   // uniform
      with_token_tiles(rows, [&](auto nte) { run_tile<SET, EPI, decltype(nte)::value>(p, c, lds, tb, rows); });
    }
  }
}

}  // namespace

hipError_t launch_gemm_large_m(const GemmParams& p, int set, int epi, hipStream_t s) {
  if (p.total_wg <= 0) return hipSuccess;
  if (p.K % kKC) return hipErrorInvalidValue;   // whole chunks only
  if (set == SET_BLOCKS && p.block_rows != kBM) return hipErrorInvalidValue;
  if (set == SET_ROUTED && p.block != kBM) return hipErrorInvalidValue;
  const dim3 grid(p.total_wg), block(256);
  if (p.qpw > 0) {   // K-resident form: K of 1 or 2 chunks, one tile per row set
    if (p.Kc < 1 || p.Kc > 2 || set == SET_MASKED) return hipErrorInvalidValue;
#define MOE_GEMM_RES(SET_, EPI_)                                                                   \
  if (set == SET_ && epi == EPI_) {                                                                \
    if (p.Kc == 1) hipLaunchKernelGGL((gemm_large_m<SET_, EPI_, 1>), grid, block, 0, s, p);       \
    else hipLaunchKernelGGL((gemm_large_m<SET_, EPI_, 2>), grid, block, 0, s, p);                 \
    return hipGetLastError();                                                                      \
  }
    MOE_GEMM_RES(SET_ROUTED, EPI_SWIGLU)
    MOE_GEMM_RES(SET_ROUTED, EPI_COMBINE)
    MOE_GEMM_RES(SET_ROUTED, EPI_STORE)
    MOE_GEMM_RES(SET_BLOCKS, EPI_SWIGLU)
    MOE_GEMM_RES(SET_BLOCKS, EPI_COMBINE)
    MOE_GEMM_RES(SET_BLOCKS, EPI_STORE)
#undef MOE_GEMM_RES
    return hipErrorInvalidValue;
  }
#define MOE_GEMM_CASE(SET_, EPI_)                                                  \
  if (set == SET_ && epi == EPI_) {                                                \
    hipLaunchKernelGGL((gemm_large_m<SET_, EPI_, 0>), grid, block, 0, s, p);      \
    return hipGetLastError();                                                      \
  }
  MOE_GEMM_CASE(SET_ROUTED, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_ROUTED, EPI_COMBINE)
  MOE_GEMM_CASE(SET_ROUTED, EPI_STORE)
  MOE_GEMM_CASE(SET_MASKED, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_MASKED, EPI_STORE)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_COMBINE)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_STORE)
#undef MOE_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
