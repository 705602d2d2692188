// Internal layouts of the prepared weights, the routing buffer and the
// workspace. Shared by the host dispatcher and the kernels (not part of the
// public ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMT = 4;        // 16-row MFMA tiles per row group
constexpr int kRowsRG = 64;   // weight rows per row group (one wave)
constexpr int kKC = 128;      // K per chunk: 4 scale groups of 32
constexpr int kAlign = 256;   // byte alignment of every sub-buffer

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Prepared layout of one weight matrix (W13 or W2) of all experts.
//
// Rows are cut into 16-row MFMA tiles and tiles into row groups of kMT = 4
// (64 rows). For W13 the tiles alternate gate / up: prepared tile 2j is gate
// rows [16j, 16j+16) and tile 2j+1 is up rows I + [16j, 16j+16), so one wave
// holds both halves of 32 intermediate columns. K is cut into chunks of 128.
//
// Words: u32x4[E][RG][Kc][kMT][64]. Lane l of tile mt holds row 16*mt + l%16
// of the group and the four canonical words covering
// k = 128*kc + 32*(l/16) + [0, 32): word g is the MFMA A fragment of step g
// of the chunk, and all 32 values share one scale group.
// Scales: u16[E][RG][Kc][64][kMT]: lane l's scale for tile mt.
// Words and scales keep their canonical values. Rows past N and k past K are
// padding: words 0x88888888 (q = 8, weight 0) and scale 0.
struct MatLayout {
  int E = 0, N = 0, K = 0;   // true shape
  int RG = 0, Kc = 0;        // row groups, k chunks
  int interleave_I = 0;      // I for W13 (gate/up interleave), 0 for W2
  size_t words_bytes = 0, scales_bytes = 0;
  size_t off_words = 0, off_scales = 0;  // from the prepared buffer start

  void init(int e, int n, int k, int inter) {
    E = e; N = n; K = k; interleave_I = inter;
    RG = (N + kRowsRG - 1) / kRowsRG;
    Kc = (K + kKC - 1) / kKC;
    words_bytes = (size_t)E * RG * Kc * kMT * 64 * 16;
    scales_bytes = (size_t)E * RG * Kc * 64 * kMT * 2;
  }
};

struct PreparedLayout {
  MatLayout w13, w2;
  size_t total = 0;
  void init(int E, int H, int I) {
    w13.init(E, 2 * I, H, I);
    w2.init(E, H, I, 0);
    size_t o = 0;
    w13.off_words = o; o = round_up(o + w13.words_bytes, kAlign);
    w13.off_scales = o; o = round_up(o + w13.scales_bytes, kAlign);
    w2.off_words = o; o = round_up(o + w2.words_bytes, kAlign);
    w2.off_scales = o; o = round_up(o + w2.scales_bytes, kAlign);
    total = o;
  }
};

// Canonical row of prepared tile jt (= 4*rg + mt), row-in-tile r.
__host__ __device__ inline int canon_row(int jt, int r, int interleave_I) {
  if (interleave_I) return ((jt & 1) ? interleave_I : 0) + 16 * (jt >> 1) + r;
  return 16 * jt + r;
}

// Routing buffer (int32 elements).
constexpr int kAlignChunk = 1024;   // flat rows per alignment chunk
constexpr int kHdrInts = 16;
enum RoutingHdr { HDR_MAGIC = 0, HDR_BLOCK = 1, HDR_E = 2, HDR_T = 3, HDR_TOPK = 4,
                  HDR_CAP = 5, HDR_NBLOCKS = 6, HDR_TOTAL = 7, HDR_NCHUNKS = 8 };
constexpr int32_t kRoutingMagic = 0x31414F4D;

struct RoutingLayout {
  int32_t block = 0, cap = 0, nblocks = 0, sentinel = 0, nchunks = 0;
  int64_t off_header = 0, off_counts = 0, off_offsets = 0, off_sorted = 0,
          off_block_expert = 0, off_slot_of = 0, off_scratch = 0, total_ints = 0;
  void init(int E, int T, int topk, int B) {
    block = B;
    sentinel = T * topk;
    cap = T * topk + E * (B - 1);
    nblocks = (cap + B - 1) / B;
    nchunks = (T * topk + kAlignChunk - 1) / kAlignChunk;
    auto r64 = [](int64_t v) { return (v + 63) / 64 * 64; };   // 256-byte steps
    off_header = 0;
    off_counts = r64(kHdrInts);
    off_offsets = r64(off_counts + E);
    off_sorted = r64(off_offsets + E + 1);
    off_block_expert = r64(off_sorted + cap);
    off_slot_of = r64(off_block_expert + nblocks);
    off_scratch = r64(off_slot_of + sentinel);
    total_ints = r64(off_scratch + (int64_t)(nchunks > 0 ? nchunks : 1) * E);
  }
};

}  // namespace moe
