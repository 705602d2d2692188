// Grouped W4A16 GEMM, small-M schedule (few rows per expert).
//
// At a few routed rows per expert a GEMM is a weight stream, so the
// dequantised weights take the wide MFMA operand: they are the 16-row A side
// of v_mfma_f32_16x16x32_bf16 and the tokens are the 16-column B side, padded
// to 16 (Chord page, "H200 and Blackwell indexed decode": the decode
// configuration swaps the MMA operands so dequantised weights fill MMA-M).
//
// Work item: one row set (an expert, or a 128-row block of the contiguous
// layout) x 256 weight rows. Each of the 4 waves owns one row group of 64
// weight rows (4 MFMA tiles) over the whole K, and the workgroup loops over
// the set's rows 16*NT at a time, so an expert's weights are streamed once
// whenever its rows fit in 16*NT. The grid is fixed from host-known sizes and
// each workgroup reads its row count on the device (a semi-static token-tile
// schedule, the variant the Chord page measured faster than a fully dynamic
// one in "H200 and Blackwell indexed decode").
//
// Per K chunk of 128:
//   * each wave streams 4 KB of its packed weights (one coalesced 1 KB load
//     per tile) and 512 B of scales, two chunks ahead of the math, in three
//     rotating register buffers (about 9 KB in flight per wave, enough to
//     keep HBM busy at four waves per SIMD);
//   * the workgroup loads the token tile (16*NT rows x 128 k of BF16) once,
//     one chunk ahead, through registers into one of three LDS buffers
//     (rows padded to 272 B so the fragment reads hit 64 distinct banks);
//   * every lane's 32 k values of a tile share one scale group, so each
//     (lane, tile, chunk) needs one scale.
// Loads past the last chunk go to a valid dummy address, so every load in
// the loop is unconditional and each wait covers exactly the buffer in use.
//
// Epilogues: SwiGLU into the BF16 intermediate (W13, gate/up tiles
// interleaved so both halves of a column sit in the same lane and register),
// the routing-weighted FP32 row w*y stored at its flat index for the combine
// kernel (W2, indexed / contiguous with row_src), or a BF16 store (W2,
// masked / contiguous without row_src).
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kBRow = 136;   // LDS token row: 128 BF16 + 8 pad (272 B)

struct AFrag {
  u32x4_t A[kMT];
  u32x2_t S;
};

template <int NT>
struct TileLds {
  uint16_t b[3][NT][16][kBRow];
};

// wq / ws: the wave's chunk base (wave-uniform, kept in SGPRs); lane: the
// per-lane element offset.
__device__ __forceinline__ void load_a(AFrag& f, const u32x4_t* __restrict__ wq,
                                       const u32x2_t* __restrict__ ws, int lane) {
  // weights and scales are streamed once: nontemporal loads keep them from
  // displacing activation rows in L2
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) f.A[mt] = __builtin_nontemporal_load(wq + mt * 64 + lane);
  f.S = __builtin_nontemporal_load(ws + lane);
}

template <int NT>
__device__ __forceinline__ void load_b(u32x4_t (&st)[NT], const uint16_t* const (&lrow)[NT], int kc,
                                       int kmax) {
  // this thread's 16-byte piece of each token row; k past K reads zero (the
  // substitute address is the row's first element, always valid)
  const int lpiece = (threadIdx.x & 15) * 8;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bool ok = kc * kKC < kmax;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lrow[nt] + (ok ? kc * kKC : -lpiece));
    const u32x4_t z = {0u, 0u, 0u, 0u};
    st[nt] = ok ? v : z;
  }
}

template <int NT>
__device__ __forceinline__ void store_b(TileLds<NT>& lds, int buf, const u32x4_t (&st)[NT]) {
  const int r = threadIdx.x >> 4, piece = threadIdx.x & 15;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    *reinterpret_cast<u32x4_t*>(&lds.b[buf][nt][r][piece * 8]) = st[nt];
}

// One K chunk. NT = 1 (decode, 4 waves/SIMD at <= 128 registers): weight
// tile outer, the single token fragment re-read from LDS per step. NT >= 2:
// step outer; the step's NT token fragments stay in registers across the 4
// weight tiles (one LDS read per token tile and step instead of four), and
// each tile's MFMAs carry the next tile's dequantisation and, on the last
// tile, the next step's LDS reads (issue order set by sched_group_barrier).
template <int NT>
__device__ __forceinline__ void mma_chunk(const AFrag& f, const TileLds<NT>& lds, int buf,
                                          f32x4_t (&acc)[kMT][NT], uint32_t mlo,
                                          uint32_t mhi) {
  const int lane = threadIdx.x & 63;
  const uint16_t* brow = &lds.b[buf][0][lane & 15][(lane >> 4) * 32];
  const float sc[4] = {bf16_lo(f.S[0]), bf16_hi(f.S[0]), bf16_lo(f.S[1]), bf16_hi(f.S[1])};
  if constexpr (NT == 1) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const GroupScale gs = group_scale(sc[mt]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4_t bf = *reinterpret_cast<const u32x4_t*>(brow + g * 8);
        const u32x4_t a = dq8(f.A[mt][g], gs, mlo, mhi);
        acc[mt][0] = mfma16(a, bf, acc[mt][0]);
      }
    }
  } else {
    constexpr int kValu = (17 + NT - 1) / NT;
    GroupScale gs[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) gs[mt] = group_scale(sc[mt]);
    u32x4_t bf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bf[nt] = *reinterpret_cast<const u32x4_t*>(brow + nt * (16 * kBRow));
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
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt] = mfma16(a, bf[nt], acc[mt][nt]);
          if (last && g < 3)
            bf[nt] = *reinterpret_cast<const u32x4_t*>(brow + nt * (16 * kBRow) + (g + 1) * 8);
        }
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
          if (last && g < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);                // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        a = an;
      }
    }
  }
}

// Occupancy target per token-tile count: 4 workgroups (4 waves per SIMD) fit
// NT = 1 in 128 registers without spilling; wider tiles need more registers.
template <int NT>
constexpr int kSmallMBlocksPerCU = NT == 1 ? 4 : (NT == 2 ? 3 : 2);

template <int NT, int SET, int EPI>
__global__ __launch_bounds__(256, kSmallMBlocksPerCU<NT>) void gemm_small_m(const GemmParams p) {
  constexpr bool kGather = (SET == SET_INDEXED && EPI == EPI_SWIGLU);
  __shared__ TileLds<NT> lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int logical = xcd_remap(blockIdx.x, p.total_wg);
  const int set = logical / p.wg_per_set;
  const int rg_raw = (logical - set * p.wg_per_set) * 4 + wave;
  const bool active = rg_raw < p.RG;          // waves past the last row group still load tiles
  const int rg = active ? rg_raw : p.RG - 1;

  // ---- the row set (uniform over the workgroup)
  int e, slot0, count;
  if constexpr (SET == SET_INDEXED) {
    const int32_t* hdr = p.routing_hdr;
    if (hdr[HDR_MAGIC] != kRoutingMagic || hdr[HDR_BLOCK] != p.block || hdr[HDR_E] != p.E ||
        hdr[HDR_T] * hdr[HDR_TOPK] != p.sentinel)
      return;   // routing made for other shapes: compute nothing
    e = set;
    slot0 = p.offsets[e];
    count = p.counts[e];
  } else if constexpr (SET == SET_MASKED) {
    e = set;
    slot0 = e * p.max_m;
    count = min(max(p.masked_m[e], 0), p.max_m);
  } else {
    slot0 = set * p.block_rows;
    count = p.block_rows;
    int m = -1;
    for (int r = lane; r < p.block_rows; r += 64) {
      const int v = p.m_indices[slot0 + r];
      if (v >= 0 && v < p.E) m = max(m, v);
    }
    e = wave_max(m);
  }
  if (count <= 0 || e < 0) return;

  const size_t tile0 = ((size_t)e * p.RG + rg) * p.Kc;
  const size_t cstride = 1;   // tiles between consecutive chunks of a row group
  const u32x4_t* __restrict__ wq = reinterpret_cast<const u32x4_t*>(p.wq) + tile0 * (kMT * 64);
  const u32x2_t* __restrict__ ws = reinterpret_cast<const u32x2_t*>(p.wsc) + tile0 * 64;
  // dummy source for prefetches past the last chunk (valid, quickly cached)
  const u32x4_t* __restrict__ wq_dummy = reinterpret_cast<const u32x4_t*>(p.wq);
  const u32x2_t* __restrict__ ws_dummy = reinterpret_cast<const u32x2_t*>(p.wsc);
  const int Kc = p.Kc;
  const uint32_t mlo = kF16MagicLo, mhi = kF16MagicHi;
  const int lr = threadIdx.x >> 4;             // token row this thread loads into LDS
  const int lpiece = (threadIdx.x & 15) * 8;   // its k offset within a chunk
  const int kmax = p.K - lpiece;               // chunk kc is readable if kc*128 < kmax

  for (int tb = 0; tb < count; tb += 16 * NT) {
    const uint16_t* lrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = min(tb + nt * 16 + lr, count - 1);   // pad columns repeat a valid row
      const int slot = slot0 + r;
      const int row = kGather ? p.sorted_ids[slot] / p.topk : slot;
      lrow[nt] = p.src + (size_t)row * p.src_ld + lpiece;
    }
    f32x4_t acc[kMT][NT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // prologue: weights of chunks 0 and 1, token tile of chunk 0
    AFrag fr0, fr1, fr2;
    u32x4_t st[NT];
    load_b<NT>(st, lrow, 0, kmax);
    load_a(fr0, wq, ws, lane);
    load_a(fr1, Kc > 1 ? wq + cstride * (kMT * 64) : wq_dummy, Kc > 1 ? ws + cstride * 64 : ws_dummy,
           lane);
    __syncthreads();   // the previous pass's readers are done with the LDS tiles
    store_b<NT>(lds, 0, st);
    __syncthreads();

    // step J computes chunk c from register buffer J and LDS buffer J, and
    // prefetches chunk c+2 into register buffer (J+2)%3 and the token tile of
    // chunk c+1 into LDS buffer (J+1)%3.
#define MOE_SMALL_M_STEP(J, CUR, NXT2)                                                           \
  {                                                                                              \
    const int c = kc + J;                                                                        \
    load_b<NT>(st, lrow, min(c + 1, Kc - 1), kmax);                                              \
    const bool more = c + 2 < Kc;                                                                \
    load_a(NXT2, more ? wq + (size_t)(c + 2) * cstride * (kMT * 64) : wq_dummy,                  \
           more ? ws + (size_t)(c + 2) * cstride * 64 : ws_dummy, lane);                         \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    if (c < Kc) mma_chunk<NT>(CUR, lds, J, acc, mlo, mhi);                                          \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    store_b<NT>(lds, (J + 1) % 3, st);                                                           \
    __syncthreads();                                                                             \
  }
    for (int kc = 0; kc < Kc; kc += 3) {
      MOE_SMALL_M_STEP(0, fr0, fr2)
      MOE_SMALL_M_STEP(1, fr1, fr0)
      MOE_SMALL_M_STEP(2, fr2, fr1)
    }
#undef MOE_SMALL_M_STEP
    if (!active) continue;

    // ---- epilogue
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = tb + nt * 16 + (lane & 15);
      if (r >= count) continue;
      const int slot = slot0 + r;
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
        int f;
        if constexpr (SET == SET_INDEXED) {
          f = p.sorted_ids[slot];
        } else {
          f = (p.m_indices[slot] == e) ? p.row_src[slot] : -1;
        }
        if (f < 0 || f >= p.sentinel) continue;
        const float w = p.topk_w[f];
        float* dst = p.yrows + (size_t)f * p.yrows_ld;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const int n = rg * kRowsRG + mt * 16 + (lane >> 4) * 4;
          if (n < p.N) *reinterpret_cast<f32x4_t*>(dst + n) = w * acc[mt][nt];
        }
      } else {
        uint16_t* dst = p.out + (size_t)slot * p.out_ld;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const int n = rg * kRowsRG + mt * 16 + (lane >> 4) * 4;
          if (n < p.N) {
            u32x2_t v;
            v[0] = pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]);
            v[1] = pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3]);
            *reinterpret_cast<u32x2_t*>(dst + n) = v;
          }
        }
      }
    }
  }
}

template <int NT>
hipError_t launch_nt(const GemmParams& p, int set, int epi, hipStream_t s) {
  const dim3 grid(p.total_wg), block(256);
#define MOE_GEMM_CASE(SET_, EPI_)                                                  \
  if (set == SET_ && epi == EPI_) {                                                \
    hipLaunchKernelGGL((gemm_small_m<NT, SET_, EPI_>), grid, block, 0, s, p);     \
    return hipGetLastError();                                                      \
  }
  MOE_GEMM_CASE(SET_INDEXED, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_INDEXED, EPI_COMBINE)
  MOE_GEMM_CASE(SET_MASKED, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_MASKED, EPI_STORE)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_SWIGLU)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_COMBINE)
  MOE_GEMM_CASE(SET_BLOCKS, EPI_STORE)
#undef MOE_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_small_m(const GemmParams& p, int set, int epi, int nt, hipStream_t s) {
  if (p.total_wg <= 0) return hipSuccess;
  switch (nt) {
    case 1: return launch_nt<1>(p, set, epi, s);
    case 2: return launch_nt<2>(p, set, epi, s);
    case 4: return launch_nt<4>(p, set, epi, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
