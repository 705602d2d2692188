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
// weight rows (4 MFMA tiles) over the whole K, and loops over the set's rows
// 16*NT at a time, so an expert's weights are streamed once whenever its
// rows fit in 16*NT. The grid is fixed from host-known sizes and each
// workgroup reads its row count on the device (a semi-static token-tile
// schedule, the variant the Chord page measured faster than a fully dynamic
// one in "H200 and Blackwell indexed decode").
//
// Per K chunk of 128, lane l loads 16 contiguous bytes of each of its 4
// tiles (one coalesced 1 KB wave load per tile), one dword pair of scales
// and 64 contiguous bytes of each token row it feeds; all of lane l's 32 k
// values of a tile share one scale group. Loads of chunk kc+1 are issued
// before the dequantisation and MFMAs of chunk kc.
//
// Epilogues: SwiGLU into the BF16 intermediate (W13, gate/up tiles
// interleaved so both halves of a column sit in the same lane and register),
// FP32 top-k-weighted scatter-add (W2, indexed / contiguous with row_src), or
// a BF16 store (W2, masked / contiguous without row_src).
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

template <int NT>
struct Frags {
  u32x4_t A[kMT];
  u32x2_t S;
  u32x4_t B[NT][4];
};

template <int NT, bool TAIL>
__device__ __forceinline__ void load_chunk(Frags<NT>& f, const u32x4_t* __restrict__ wq,
                                           const u32x2_t* __restrict__ ws,
                                           const uint16_t* const (&brow)[NT], int kc, int klim,
                                           int kq) {
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) f.A[mt] = wq[(kc * kMT + mt) * 64];
  f.S = ws[kc * 64];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (!TAIL) {
        f.B[nt][g] = *reinterpret_cast<const u32x4_t*>(brow[nt] + kc * kKC + g * 8);
      } else {
        // k past K: zero the activation (the prepared weights there are 0)
        // (the substitute address is the row's first element, always valid)
        const bool ok = g * 8 < klim;
        const uint16_t* src = ok ? brow[nt] + kc * kKC + g * 8 : brow[nt] - kq;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src);
        const u32x4_t z = {0u, 0u, 0u, 0u};
        f.B[nt][g] = ok ? v : z;
      }
    }
  }
}

template <int NT>
__device__ __forceinline__ void mma_chunk(const Frags<NT>& f, f32x4_t (&acc)[kMT][NT]) {
  const float s16[4] = {bf16_lo(f.S[0]), bf16_hi(f.S[0]), bf16_lo(f.S[1]), bf16_hi(f.S[1])};
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4_t a = dq8(f.A[mt][g], s16[mt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16(a, f.B[nt][g], acc[mt][nt]);
    }
  }
}

template <int NT, int SET, int EPI>
__global__ __launch_bounds__(256) void gemm_small_m(const GemmParams p) {
  constexpr bool kGather = (SET == SET_INDEXED && EPI == EPI_SWIGLU);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int logical = xcd_remap(blockIdx.x, p.total_wg);
  const int set = logical / p.wg_per_set;
  const int rg = (logical - set * p.wg_per_set) * 4 + wave;
  if (rg >= p.RG) return;

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
    if (e < 0) return;   // all padding
  }
  if (count <= 0) return;

  const size_t tile0 = ((size_t)e * p.RG + rg) * p.Kc;
  const u32x4_t* __restrict__ wq = reinterpret_cast<const u32x4_t*>(p.wq) + tile0 * (kMT * 64) + lane;
  const u32x2_t* __restrict__ ws = reinterpret_cast<const u32x2_t*>(p.wsc) + tile0 * 64 + lane;
  const int kq = (lane >> 4) * 32;            // this lane's k offset inside a chunk
  const int kfull = p.K / kKC;                // chunks without a K tail
  const int tail_lim = p.K - kfull * kKC - kq; // valid k of this lane in the tail chunk

  for (int tb = 0; tb < count; tb += 16 * NT) {
    const uint16_t* brow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = min(tb + nt * 16 + (lane & 15), count - 1);   // pad columns repeat a valid row
      const int slot = slot0 + r;
      const int row = kGather ? p.sorted_ids[slot] / p.topk : slot;
      brow[nt] = p.src + (size_t)row * p.src_ld + kq;
    }
    f32x4_t acc[kMT][NT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    Frags<NT> cur, nxt;
    if (kfull > 0) load_chunk<NT, false>(cur, wq, ws, brow, 0, 0, kq);
    else load_chunk<NT, true>(cur, wq, ws, brow, 0, tail_lim, kq);
    for (int kc = 0; kc < p.Kc; ++kc) {
      if (kc + 1 < kfull) load_chunk<NT, false>(nxt, wq, ws, brow, kc + 1, 0, kq);
      else if (kc + 1 < p.Kc) load_chunk<NT, true>(nxt, wq, ws, brow, kc + 1, tail_lim, kq);
      mma_chunk<NT>(cur, acc);
      cur = nxt;
    }

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
        float* dst = p.acc_out + (size_t)(f / p.topk) * p.acc_ld;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const int n = rg * kRowsRG + mt * 16 + (lane >> 4) * 4;
          if (n < p.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + n + i, w * acc[mt][nt][i]);
          }
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
