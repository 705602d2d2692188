// Grouped W4A16 GEMM, large-M schedule with 256-row token tiles.
//
// At prefill sizes the large-M kernel is bound by its instruction stream:
// each dequantised weight fragment (17 VALU instructions per 8 weights)
// feeds one MFMA per 16-token tile, so the token rows a fragment serves set
// the VALU share. This form doubles them: a workgroup takes two consecutive
// 128-row blocks of one expert (256 token rows) x 256 weight rows, with
// eight waves of 32 weight rows (2 MFMA tiles) x all 256 tokens (16 MFMA
// tiles), so one dequantised fragment feeds 16 MFMAs (Chord page, "H200
// prefill and TP8": block_m follows the rows an expert holds).
//
// One workgroup per CU (2 waves per SIMD). Nothing else on the CU covers a
// wait at a barrier, so the token tile streams through a 4-slot LDS ring of
// half chunks (2 MFMA steps = 64 k each, 32 KB), copied straight from
// global memory into LDS (global_load_lds) two stages ahead, at the end of
// each stage's MFMAs. Before a stage, each wave waits only for its own copy
// of that stage (an explicit vmcnt counting the loads issued since), then
// s_barrier; never for the later stage in flight. Every stage issues the
// same loads (past the end: stage 0's again, into a free slot), the loop
// body has no guard (K is a whole number of chunk pairs) and a scheduling
// barrier closes each stage: with a branch or guard around the loads, or
// with work moved across stages, the compiler falls back to waiting for all
// outstanding loads. Weights: one chunk ahead in registers.
//
// Measured against the 128-row kernel (its default): 5 % faster on W13
// when every tile is a full pair (an EP share at 512 rows per expert),
// slower where most tiles are single blocks (a Zipf prefill: one workgroup
// of 8 waves per CU then serves 128 rows). A copy with the in-loop token
// copies removed ran 22 % faster than the 128-row kernel, so the copies and
// their barriers, not the MFMAs, bound this form.
//
// The half-chunk stage layout and its copies are described in moe_tile.h.
//
// Row sets: routing blocks (indexed, block 128) or 128-row contiguous
// blocks, paired as (2i, 2i+1); a pair whose blocks belong to two experts is
// run as two 128-row tiles. Epilogues as in the 128-row kernel.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_launch.h"
#include "moe_tile.h"

namespace moe {

namespace {

constexpr int kBM1 = 128;                      // rows of one block
constexpr int kStages = 4;
constexpr int kStageU4 = 256 * 64 * 2 / 16;    // 16-byte slots per stage (2048, 32 KB)

// The LDS ring: four separate arrays, so that alias analysis tells a slot
// being filled from the slot being read (it then inserts no wait for the
// fill before the reads).
struct Ring {
  u32x4_t* s[kStages];
};

struct WFrag {
  u32x4_t A[2];   // the wave's 2 weight tiles of one chunk (words = MFMA steps)
  uint32_t S;     // their 2 BF16 scales
};

__device__ __forceinline__ void load_w(WFrag& f, const u32x4_t* __restrict__ wq, const uint32_t* __restrict__ ws,
                                       int lane) {
  f.A[0] = __builtin_nontemporal_load(wq + lane);
  f.A[1] = __builtin_nontemporal_load(wq + 64 + lane);
  f.S = __builtin_nontemporal_load(ws + 2 * lane);
}

// Keeps a loaded value where it is used: the empty asm "changes" it, and
// volatile asm keeps its place among the barriers, so no consumer of the
// value is hoisted above the wait that covers its load.
__device__ __forceinline__ void pin(WFrag& f) {
  asm volatile("" : "+v"(f.A[0]), "+v"(f.A[1]), "+v"(f.S));
}

// Two MFMA steps (one stage) over the first NT token tiles.
template <int NT>
__device__ __forceinline__ void mma_stage(const WFrag& f, const u32x4_t* stage, int h, int rd,
                                          f32x4_t (&acc)[2][NT], const GroupScale (&gs)[2]) {
  const uint32_t mlo = kF16MagicLo, mhi = kF16MagicHi;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int g = 2 * h + j;
    const u32x4_t a0 = dq8(f.A[0][g], gs[0], mlo, mhi);
    const u32x4_t a1 = dq8(f.A[1][g], gs[1], mlo, mhi);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4_t b = stage[nt * 128 + (rd ^ j)];
      acc[0][nt] = mfma16(a0, b, acc[0][nt]);
      acc[1][nt] = mfma16(a1, b, acc[1][nt]);
    }
  }
}

struct WideCtx {
  int lane, wave, rg, mt0, e, slot0, rd;
  bool active;
  const u32x4_t* wq;    // chunk 0 of this wave's 2 tiles
  const uint32_t* ws;   // chunk 0 of this wave's scale pair
};

// Epilogue of rows r < rows of a tile starting at set slot0. The rows'
// routing data (flat index, routing weight) is loaded for all NT token tiles
// first, so the loads are in flight together instead of one round trip per
// tile.
template <int SET, int EPI, int NT>
__device__ __forceinline__ void wide_epilogue(const GemmParams& p, const WideCtx& c, int rows,
                                              const f32x4_t (&acc)[2][NT]) {
  const int lane = c.lane;
  int fv[NT];   // flat row index (combine), or >= 0 for a row to write; -1: skip
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + (lane & 15);
    const int slot = c.slot0 + min(r, rows - 1);
    if constexpr (SET == SET_ROUTED) {
      fv[nt] = p.sorted_ids[slot];
    } else {
      fv[nt] = p.m_indices[slot];
    }
  }
  if constexpr (SET != SET_ROUTED && EPI == EPI_COMBINE) {
    int src[NT];   // loaded for every row (a load under a branch would wait alone)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) src[nt] = p.row_src[c.slot0 + min(nt * 16 + (lane & 15), rows - 1)];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) fv[nt] = fv[nt] == c.e ? src[nt] : -1;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + (lane & 15);
    bool ok;
    if constexpr (SET == SET_ROUTED || EPI == EPI_COMBINE)
      ok = fv[nt] >= 0 && fv[nt] < p.sentinel;
    else
      ok = fv[nt] == c.e;   // not a pad row (or another expert's)
    if (r >= rows) ok = false;
    if (!ok) fv[nt] = -1;
  }
  float wv[NT];
  if constexpr (EPI == EPI_COMBINE) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wv[nt] = p.topk_w[fv[nt] >= 0 ? fv[nt] : 0];
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (fv[nt] < 0) continue;
    const int slot = c.slot0 + nt * 16 + (lane & 15);
    if constexpr (EPI == EPI_SWIGLU) {
      // tiles mt0 (gate) and mt0 + 1 (up) of row group rg
      uint16_t* dst = p.a_out + (size_t)slot * p.a_ld + c.rg * 32 + (c.mt0 >> 1) * 16 + (lane >> 4) * 4;
      const f32x4_t g = acc[0][nt], u = acc[1][nt];
      u32x2_t v;
      v[0] = pack_bf16x2(swiglu(g[0], u[0]), swiglu(g[1], u[1]));
      v[1] = pack_bf16x2(swiglu(g[2], u[2]), swiglu(g[3], u[3]));
      *reinterpret_cast<u32x2_t*>(dst) = v;
    } else if constexpr (EPI == EPI_COMBINE) {
      if (c.rg * kRowsRG < p.N) {   // tiles mt0, mt0 + 1 of the row group, lane-contiguous (store_y16)
        const f32x4_t v[2] = {acc[0][nt], acc[1][nt]};
        const size_t idx = (size_t)fv[nt] * p.yrows_ld + c.rg * kRowsRG + (lane >> 4) * 16 + c.mt0 * 4;
        store_y16<2>(p.yq, idx, wv[nt], v);
      }
    } else {
      uint16_t* dst = p.out + (size_t)slot * p.out_ld;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int n = store_col(p.N, p.gate_up_I, c.rg, c.mt0 + t, lane);
        if (n >= 0) {
          u32x2_t v;
          v[0] = pack_bf16x2(acc[t][nt][0], acc[t][nt][1]);
          v[1] = pack_bf16x2(acc[t][nt][2], acc[t][nt][3]);
          *reinterpret_cast<u32x2_t*>(dst + n) = v;
        }
      }
    }
  }
}

// One tile of `tile_rows` (128 or 256) rows from slot0, `rows` of them worth
// computing (NT = ceil(rows / 16) token tiles, rounded up to the variant).
template <int SET, int EPI, int NT>
__device__ __forceinline__ void wide_tile(const GemmParams& p, const WideCtx& c,
                                          const Ring& lds, int rows) {
  const int lane = c.lane, wave = c.wave;
  // token rows of this lane's two DMA row blocks; rows past `rows` repeat the
  // last one (every wave loads its share unconditionally: a branch around the
  // loads would make the compiler wait for all of them before the LDS reads)
  const bool gather = SET == SET_ROUTED && p.gather;
  uint32_t rowb[2];   // byte offsets of the rows in the token matrix
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = stage_row(wave, i, lane);
    const int slot = c.slot0 + min(r, rows - 1);
    int row = slot;
    if (gather) {
      const int f = p.sorted_ids[slot];
      row = (f >= 0 && f < p.sentinel) ? f / p.topk : 0;   // pad slots read row 0
    }
    rowb[i] = (uint32_t)row * (uint32_t)p.src_ld * 2u;
  }
  const StageSrc src = stage_src(p.src, rowb[0], rowb[1], lane);
  const int NS = 2 * p.Kc;   // stages
  f32x4_t acc[2][NT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4_t* wq_dummy = reinterpret_cast<const u32x4_t*>(p.wq);
  const uint32_t* ws_dummy = reinterpret_cast<const uint32_t*>(p.wsc);
  auto wq_at = [&](int kc) { return kc < p.Kc ? c.wq + (size_t)kc * (kMT * 64) : wq_dummy; };
  auto ws_at = [&](int kc) { return kc < p.Kc ? c.ws + (size_t)kc * 128 : ws_dummy; };

  // stage t goes straight to ring slot t % 4, two stages ahead (issued at
  // the end of iteration t-2, waited for at the top of iteration t)
  WFrag fw[2];
  stage_barrier();   // the previous tile's readers are done with the ring
  // issued in this order (the waits below count on it)
  dma_stage(lds.s[0], src, 0, wave);
  __builtin_amdgcn_sched_barrier(0);
  load_w(fw[0], wq_at(0), ws_at(0), lane);
  __builtin_amdgcn_sched_barrier(0);
  dma_stage(lds.s[1], src, 1, wave);
  __builtin_amdgcn_sched_barrier(0);

  // Loads issued after those iteration s needs: s even (needs DMA(s), W(c)):
  // DMA(s+1); s odd (needs DMA(s)): W(c+1), DMA(s+1).
  // NS is a multiple of 4 (K a whole number of chunk pairs): no guard in
  // the body, whose every iteration then issues the same loads
#define MOE_WIDE_ITER(SS, CUR, NXT)                                                           \
  {                                                                                           \
    const int s = s0 + (SS);                                                                  \
    {                                                                                         \
      if ((SS) % 2 == 0) wait_vm<4>();                                                        \
      else wait_vm<7>();                                                                      \
      stage_barrier();                                                                        \
      if ((SS) % 2 == 0) load_w(fw[NXT], wq_at((s >> 1) + 1), ws_at((s >> 1) + 1), lane);    \
      pin(fw[CUR]);                                                                           \
      GroupScale gs[2] = {group_scale(bf16_lo(fw[CUR].S)), group_scale(bf16_hi(fw[CUR].S))};  \
      mma_stage<NT>(fw[CUR], lds.s[(SS) & 3], (SS) & 1, c.rd, acc, gs);                      \
      dma_stage(lds.s[((SS) + 2) & 3], src, s + 2 < NS ? s + 2 : 0, wave);                    \
      __builtin_amdgcn_sched_barrier(0);   /* no work moves across stages */                  \
    }                                                                                         \
  }
  // a do-while: with a branch around the loop the compiler sinks the
  // weight loads above into it, past the copies the waits count on
  int s0 = 0;
  do {
    MOE_WIDE_ITER(0, 0, 1)
    MOE_WIDE_ITER(1, 0, 1)
    MOE_WIDE_ITER(2, 1, 0)
    MOE_WIDE_ITER(3, 1, 0)
    s0 += 4;
  } while (s0 < NS);
#undef MOE_WIDE_ITER
  wait_vm<0>();   // the loads past the end land before their registers are dropped
  if (c.active) wide_epilogue<SET, EPI, NT>(p, c, rows, acc);
}

template <int SET, int EPI>
__device__ __forceinline__ void wide_tile_any(const GemmParams& p, const WideCtx& c,
                                              const Ring& lds, int rows) {
  if (rows <= 64)
    wide_tile<SET, EPI, 4>(p, c, lds, rows);
  else if (rows <= 128)
    wide_tile<SET, EPI, 8>(p, c, lds, rows);
  else if (rows <= 192)
    wide_tile<SET, EPI, 12>(p, c, lds, rows);
  else
    wide_tile<SET, EPI, 16>(p, c, lds, rows);
}

// Expert and one-past-last-row of block b (uniform over the wave; -1 / 0
// for a block past the set, an empty block or a block of no expert).
template <int SET>
__device__ __forceinline__ void block_info(const GemmParams& p, int b, int nblocks, int lane, int& e,
                                           int& n_eff) {
  e = -1;
  n_eff = 0;
  if (b >= nblocks) return;
  const int slot0 = b * kBM1;
  if constexpr (SET == SET_ROUTED) {
    e = p.block_expert[b];
    int last = 0;
#pragma unroll
    for (int r = lane; r < kBM1; r += 64) {
      const int f = p.sorted_ids[slot0 + r];
      if (f >= 0 && f < p.sentinel) last = r + 1;
    }
    n_eff = wave_max(last);
  } else {
    int m[2], mx = -1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      m[i] = p.m_indices[slot0 + lane + 64 * i];
      if (m[i] >= 0 && m[i] < p.E) mx = max(mx, m[i]);
    }
    e = wave_max(mx);
    int last = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (m[i] == e && e >= 0) last = lane + 64 * i + 1;
    n_eff = wave_max(last);
  }
  if (e < 0 || e >= p.E) {
    e = -1;
    n_eff = 0;
  }
  e = __builtin_amdgcn_readfirstlane(e);
  n_eff = __builtin_amdgcn_readfirstlane(n_eff);
}

template <int SET, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_wide(const GemmParams p) {
  __shared__ u32x4_t lds0[kStageU4], lds1[kStageU4], lds2[kStageU4], lds3[kStageU4];
  const Ring lds = {{lds0, lds1, lds2, lds3}};
  WideCtx c;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = c.lane;
  int nblocks, logical;
  if constexpr (SET == SET_ROUTED) {
    const int32_t* hdr = p.routing_hdr;
    if (hdr[HDR_MAGIC] != kRoutingMagic || hdr[HDR_BLOCK] != p.block || hdr[HDR_E] != p.E ||
        hdr[HDR_T] * hdr[HDR_TOPK] != p.sentinel)
      return;   // routing made for other shapes: compute nothing
    nblocks = min(max(hdr[HDR_TOTAL], 0) / kBM1, p.nsets);
    logical = xcd_remap_active(blockIdx.x, (nblocks + 1) / 2 * p.wg_per_set);
    if (logical < 0) return;
  } else {
    nblocks = p.nsets;
    logical = xcd_remap(blockIdx.x, p.total_wg);
  }
  const int pair = logical / p.wg_per_set;
  const int quad = logical - pair * p.wg_per_set;
  const int rg_raw = quad * 4 + (c.wave >> 1);
  c.active = rg_raw < p.RG;
  c.rg = c.active ? rg_raw : p.RG - 1;
  c.mt0 = 2 * (c.wave & 1);
  c.rd = stage_rd(lane);

  int e0, n0, e1, n1;
  block_info<SET>(p, 2 * pair, nblocks, lane, e0, n0);
  block_info<SET>(p, 2 * pair + 1, nblocks, lane, e1, n1);
  auto bind = [&](int e) {
    c.e = e;
    const size_t tile0 = ((size_t)e * p.RG + c.rg) * p.Kc;
    c.wq = reinterpret_cast<const u32x4_t*>(p.wq) + tile0 * (kMT * 64) + c.mt0 * 64;
    c.ws = reinterpret_cast<const uint32_t*>(p.wsc) + tile0 * 128 + (c.mt0 >> 1);
  };
  if (e0 >= 0 && e1 == e0 && n0 == kBM1 && n1 > 0) {   // one 256-row tile
    bind(e0);
    c.slot0 = 2 * pair * kBM1;
    wide_tile_any<SET, EPI>(p, c, lds, kBM1 + n1);
  } else {
    if (e0 >= 0 && n0 > 0) {
      bind(e0);
      c.slot0 = 2 * pair * kBM1;
      wide_tile_any<SET, EPI>(p, c, lds, n0);
    }
    if (e1 >= 0 && n1 > 0) {
      bind(e1);
      c.slot0 = (2 * pair + 1) * kBM1;
      wide_tile_any<SET, EPI>(p, c, lds, n1);
    }
  }
}

}  // namespace

hipError_t launch_gemm_wide(const GemmParams& p, int set, int epi, hipStream_t s) {
  if (p.total_wg <= 0) return hipSuccess;
  if (p.K % (2 * kKC)) return hipErrorInvalidValue;   // whole chunk pairs only
  if (!src_fits_u32(p, set)) return hipErrorInvalidValue;
  if (set == SET_BLOCKS && p.block_rows != kBM1) return hipErrorInvalidValue;
  if (set == SET_ROUTED && p.block != kBM1) return hipErrorInvalidValue;
  const dim3 grid(p.total_wg), block(512);
#define MOE_WIDE_CASE(SET_, EPI_)                                                \
  if (set == SET_ && epi == EPI_) {                                              \
    hipLaunchKernelGGL((gemm_wide<SET_, EPI_>), grid, block, 0, s, p);           \
    return hipGetLastError();                                                    \
  }
  MOE_WIDE_CASE(SET_ROUTED, EPI_SWIGLU)
  MOE_WIDE_CASE(SET_ROUTED, EPI_COMBINE)
  MOE_WIDE_CASE(SET_ROUTED, EPI_STORE)
  MOE_WIDE_CASE(SET_BLOCKS, EPI_SWIGLU)
  MOE_WIDE_CASE(SET_BLOCKS, EPI_COMBINE)
  MOE_WIDE_CASE(SET_BLOCKS, EPI_STORE)
#undef MOE_WIDE_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
