// Device-side building blocks shared by the attention kernels of this library
// (forward: fa_fwd.hip; backward: fa_bwd.hip): vector types, the gfx950 MFMA
// operand layouts used by both, LDS swizzles, the asynchronous global -> LDS
// tile copy, the S tile product and the XCD-aware grid decode.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64): A operand -- lane l holds
// A[l % 32][8 * (l / 32) + e], e = 0..7; B operand -- lane l holds
// B[8 * (l / 32) + e][l % 32]; accumulator -- lane l, register r holds
// C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32].  A lane therefore owns one
// column of C.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// The kernels take the score multiplier as c = scale * log2(e) and work with
// |c|.  A negative c stands for a negative scale: the kernel negates one
// operand of the score product (the sign bits of a register fragment, an
// exact operation), so scale * q.k = |scale| * (-q).k.  A zero scale arrives
// as kZeroScaleC: every visible key then gets the weight exp2(s * c - m * c)
// = 1 exactly (the argument is below 2^-24 for any finite score), and masked
// keys (score -inf) keep weight 0; -inf * 0 would give NaN instead.
constexpr float kZeroScaleC = 0x1p-100f;
__device__ __forceinline__ uint32_t sign_flip_mask(float c) { return c < 0.0f ? 0x80008000u : 0u; }

constexpr int kRowsPerWave = 32;  // query (or key) rows per wavefront

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float other_half(float x) {
  // value held by lane l ^ 32 (the other 32-lane half of the wavefront)
  return __shfl_xor(x, 32);
}

// Logical workgroup index from the hardware one: workgroup i is dispatched to
// XCD i % 8; give each XCD a contiguous range of logical indices.
__device__ __forceinline__ int xcd_logical_index(int i, int n) {
  const int x = i & 7, s = i >> 3;
  const int base = n >> 3, rem = n & 7;
  return x * base + (x < rem ? x : rem) + s;
}

// Logical index -> (bh, query tile).  Heads are taken in groups of
// `group_heads`.  Causal: inside a group the tiles of its heads are
// interleaved, heaviest (last) query tiles first, so that every round of
// workgroups holds a mix of long and short ones.  Without the mask all tiles
// are equally long and the group is walked head by head.
template <bool CAUSAL>
__device__ __forceinline__ void decode_tile(int L, int nq, int bh_total, int group_heads,
                                            int& bh, int& qt) {
  const int gsize = group_heads * nq;
  const int grp = L / gsize;
  const int r = L - grp * gsize;
  const int left = bh_total - grp * group_heads;
  const int hin = left < group_heads ? left : group_heads;
  if (CAUSAL) {
    bh = grp * group_heads + r % hin;
    qt = nq - 1 - r / hin;
  } else {
    // equal-length tiles: head-major, so that the workgroups running at the
    // same time on an XCD stream the same head's K/V through its L2
    bh = grp * group_heads + r / nq;
    qt = r % nq;
  }
}

// ----------------------------------------------------------------------------
// bf16 kernel
// ----------------------------------------------------------------------------

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// D = 256, one-wave ring kernel (a study build): a row's reference max is
// only raised when a tile's max exceeds it by more than this many powers of
// two, so softmax weights stay <= 2^24 (their float32 sums and the O
// accumulator stay far from overflow, and a bf16 weight keeps its relative
// precision at any magnitude).  A large margin keeps the raises rare even for
// rows whose scores spread widely.
constexpr float kRescaleThreshold = 24.0f;
// Largest sum of one lane's softmax weights in a tile that the D <= 128
// kernels accept without moving the row's reference max.
constexpr float kRowSumLimit = 4096.0f;
// The same limit for the D = 256 wave-pair kernel: 2^kRescaleThreshold, so
// that no weight exceeds 2^24 (a sum within it bounds each of its terms).
constexpr float kPairSumLimit = 16777216.0f;

template <int D_, int BC_, int WAVES_>
struct BfCfg {
  static constexpr int D = D_;
  static constexpr int BC = BC_;                       // keys per tile
  static constexpr int WAVES = WAVES_;                 // wavefronts per workgroup
  static constexpr int BR = kRowsPerWave * WAVES;      // query rows per workgroup
  static constexpr int KCH = D / 16;                   // MFMA k-steps of Q*K^T
  static constexpr int KB = BC / 32;                   // 32-key blocks per tile
  static constexpr int DB = D / 32;                    // 32-row blocks of O^T
  static constexpr int PCH = BC / 16;                  // MFMA k-steps of P*V
  static constexpr int ROW_BYTES = D * 2;              // one K or V row in LDS
  static constexpr int TILE_BYTES = BC * ROW_BYTES;    // K tile or V tile
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;     // 2 K + 2 V buffers
  static constexpr int RC = D / 8;                     // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 64 / RC;        // rows per 1 KiB wave load
  // Waves that issue the tile copies: all of a 4-wave workgroup; in an 8-wave
  // workgroup four of them, one per SIMD.
  static constexpr int COPY_WAVES = WAVES == 8 ? 4 : WAVES;
  static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / COPY_WAVES;  // per tensor
  // VALU instructions the schedule places after each MFMA of a tile.
  static constexpr int VALU_PER_MFMA = WAVES == 8 ? 4 : 5;
  // LDS bank geometry: 64 banks of 4 bytes, i.e. 256-byte bank lines.
  static constexpr int ROWS_PER_LINE = 256 / ROW_BYTES > 1 ? 256 / ROW_BYTES : 1;
  static constexpr int CH_PER_LINE = 16;               // 16-byte chunks per bank line
  static constexpr int NKOFF = KCH < 8 ? KCH : 8;      // distinct K read offsets
  static constexpr int NVOFF = DB < 4 ? DB : 4;        // distinct V read offsets
  static_assert(TILE_BYTES % (1024 * COPY_WAVES) == 0, "tile must split into 1 KiB wave loads");
  static_assert(COPY_WAVES * LOADS_PER_WAVE * 1024 == TILE_BYTES, "copy shares cover the tile");
  static_assert(COPY_WAVES * LOADS_PER_WAVE * ROWS_PER_LOAD == BC, "copy rows stay in the tile");
  static_assert(D % 32 == 0 && BC % 32 == 0 && D >= 64 && RC <= 64, "tile shape");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// 16-byte chunk swizzles (physical chunk = logical chunk ^ swizzle(row)), for
// an LDS of 64 four-byte banks (a 16-lane group of 16-byte reads, or a
// 32-lane group of 8-byte reads, is served per pass).
// K: a 16-lane group reads one chunk column of 16 different rows of a 32-row
// block -> the 16 rows of a bank line's worth must land in 16 distinct chunk
// slots: XOR with the row index among the rows that share a line position.
template <class C>
__device__ __forceinline__ int kswz(int r) {
  return (r / C::ROWS_PER_LINE) & (C::CH_PER_LINE / C::ROWS_PER_LINE - 1);
}
// V: a 32-lane pass of the transposing read covers 4 consecutive rows x 64
// bytes (4 chunks): shift each row's 4-chunk group to its own slot.
template <class C>
__device__ __forceinline__ int vswz(int r) {
  constexpr int groups = (C::CH_PER_LINE / C::ROWS_PER_LINE) / 4;  // 4-chunk slots per row
  return ((r / C::ROWS_PER_LINE) & (groups - 1)) << 2;
}

// MFMA row m of a 32-key block reads key row perm(m): bits 2 and 3 swapped.
__device__ __forceinline__ int key_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// The value held by lane l ^ 32, through the gfx950 lane-half swap.
__device__ __forceinline__ float swap_halves(float x, int hh) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, hh ? r[0] : r[1]);
}

// Per-lane element offsets (within one head, tile starting at key 0) of the
// 16-byte pieces this lane copies; row r of the tile lands in LDS row r with
// its chunks swizzled.
template <class C, bool IS_V>
__device__ __forceinline__ void tile_offsets(int* off, int* row, int part, int lane) {
#pragma unroll
  for (int u = 0; u < C::LOADS_PER_WAVE; ++u) {
    const int n = part * C::LOADS_PER_WAVE + u;
    const int r = n * C::ROWS_PER_LOAD + lane / C::RC;
    const int lch = (lane % C::RC) ^ (IS_V ? vswz<C>(r) : kswz<C>(r));
    row[u] = r;
    off[u] = r * C::D + lch * 8;
  }
}

// Buffer-resource word 3 for raw (untyped) buffer loads on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;

// Asynchronous global -> LDS copy of BYTES per lane: lane l's bytes at
// base + boff land in LDS at dst + BYTES * l.  Issued as a buffer load with
// the LDS bit: it is tracked by the vector-memory counter only, so the
// compiler keeps exact LDS-counter waits for the operand reads that run while
// copies are in flight.  (For the global-segment form of the same copy the
// compiler assumes it may be pending on the LDS counter too and turns every
// such wait into a wait for all outstanding LDS operations.)  `base` is made
// wave-uniform (scalar registers); `boff` is the per-lane byte offset.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* base, uint32_t boff, lds_u8* dst,
                                        int soff = 0) {
  const uint64_t b64 = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  void* p = (void*)(((uint64_t)hi << 32) | lo);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(p, (short)0, -1, kRawBufferWord3);
  auto* d = (__attribute__((address_space(3))) void*)dst;
  static_assert(BYTES == 16 || BYTES == 4, "copy size per lane");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, boff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 4, boff, soff, 0, 0);
}

// Asynchronous global -> LDS copy of one K or V tile.  Share `part` of the
// copy, issued by one wave, is LOADS_PER_WAVE transfers of 1 KiB, lane l
// filling bytes 16l .. 16l+15 (a wave-uniform base address plus a per-lane
// 32-bit offset).  In the last (partial) tile, rows past the sequence end are
// clamped to the last row: finite data whose keys are masked.
template <class C>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ head_src, lds_u8* dst,
                                           int k0, int S, int part, const int* off,
                                           const int* row) {
  // The tile's base address is wave-uniform: keep it in scalar registers so
  // each copy is issued as scalar base + 32-bit lane offset.
  const uint64_t b64 = (uint64_t)(head_src + (size_t)k0 * C::D);
  const uint32_t b_lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t b_hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  const char* base = (const char*)(((uint64_t)b_hi << 32) | b_lo);
  lds_u8* lds = dst + part * (C::LOADS_PER_WAVE * 1024);
  if (k0 + C::BC <= S) {
#pragma unroll
    for (int u = 0; u < C::LOADS_PER_WAVE; ++u)
      lds_dma<16>(base, (uint32_t)(off[u] * 2), lds + u * 1024);
  } else {
#pragma unroll
    for (int u = 0; u < C::LOADS_PER_WAVE; ++u) {
      const int o = off[u] - (row[u] - min(row[u], S - 1 - k0)) * C::D;
      lds_dma<16>(base, (uint32_t)(o * 2), lds + u * 1024);
    }
  }
}

// Compact per-lane state of the tile copies (D = 64 and 128, where a tile
// row is at most 256 bytes).  This lane's 16 bytes of piece 0 of the wave's
// share sit in tile row row0; piece u holds rows row0 + u * ROWS_PER_LOAD,
// 1 KiB further on in both memories.  Those rows have row0's V swizzle, and a
// K swizzle that differs from row0's by an XOR of 4u, so a piece's offsets
// follow from piece 0's with a scalar offset (and, for K, one XOR).
struct CopyLanes {
  int krow;   // K: byte offset of row row0 in the tile
  int kch;    // K: byte offset, within the row, of this lane's chunk in piece 0
  int vbyte;  // V: byte offset of this lane's 16 bytes in piece 0
};

template <class C>
__device__ __forceinline__ CopyLanes copy_lanes(int part, int lane) {
  // kswz(r) = (r / ROWS_PER_LINE) mod P, P = CH_PER_LINE / ROWS_PER_LINE: the
  // share's first row is a multiple of P lines, a lane's row within piece 0
  // adds < 4 lines, and piece u adds 4u lines with 4u + 3 < P.
  constexpr int P = C::CH_PER_LINE / C::ROWS_PER_LINE;
  // (With one piece per wave nothing is assumed about later pieces.)
  static_assert(C::ROW_BYTES <= 256 &&
                    (C::LOADS_PER_WAVE == 1 ||
                     (C::ROWS_PER_LOAD == 4 * C::ROWS_PER_LINE &&
                      (C::LOADS_PER_WAVE * C::ROWS_PER_LOAD / C::ROWS_PER_LINE) % P == 0 &&
                      4 * C::LOADS_PER_WAVE <= P)),
                "piece u's K swizzle must be piece 0's XOR 4u");
  const int row0 = part * C::LOADS_PER_WAVE * C::ROWS_PER_LOAD + lane / C::RC;
  CopyLanes cl;
  cl.krow = row0 * C::ROW_BYTES;
  cl.kch = ((lane % C::RC) ^ kswz<C>(row0)) << 4;
  cl.vbyte = row0 * C::ROW_BYTES + (((lane % C::RC) ^ vswz<C>(row0)) << 4);
  return cl;
}

// Asynchronous global -> LDS copy of one K (IS_V false) or V tile with the
// compact lane state: share `part`, LOADS_PER_WAVE pieces of 1 KiB.  In the
// last (partial) tile, rows past the sequence end are clamped to the last
// row: finite data whose keys are masked.
template <class C, bool IS_V>
__device__ __forceinline__ void copy_tile(const uint16_t* __restrict__ head_src, lds_u8* dst,
                                          int k0, int S, int part, int lane,
                                          const CopyLanes& cl) {
  const uint64_t b64 = (uint64_t)(head_src + (size_t)k0 * C::D);
  const uint32_t b_lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t b_hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  const char* base = (const char*)(((uint64_t)b_hi << 32) | b_lo);
  lds_u8* lds = dst + part * (C::LOADS_PER_WAVE * 1024);
  if (k0 + C::BC <= S) {
#pragma unroll
    for (int u = 0; u < C::LOADS_PER_WAVE; ++u) {
      const int o = IS_V ? cl.vbyte : cl.krow + (cl.kch ^ (64 * u));
      lds_dma<16>(base, (uint32_t)o, lds + u * 1024, 1024 * u);
    }
  } else {
    const int row0 = part * C::LOADS_PER_WAVE * C::ROWS_PER_LOAD + lane / C::RC;
    const int chunk = IS_V ? cl.vbyte - cl.krow : cl.kch;  // piece 0's chunk byte offset
#pragma unroll
    for (int u = 0; u < C::LOADS_PER_WAVE; ++u) {
      const int r = row0 + u * C::ROWS_PER_LOAD;
      const int src_row = min(r, S - 1 - k0);
      const int o = src_row * C::ROW_BYTES + (IS_V ? chunk : (chunk ^ (64 * u)));
      lds_dma<16>(base, (uint32_t)o, lds + u * 1024);
    }
  }
}

// S^T (keys x queries) for one tile: s[kb] = K[kb*32 + perm(m)][:] . Q[my_q][:]
template <class C>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[C::KB], const lds_u8* Ks,
                                        const bf16x8 (&qf)[C::KCH], const int (&k_off)[C::NKOFF]) {
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
    for (int ch = 0; ch < C::KCH; ++ch) {
      const bf16x8 kf = *(const lds_bf16x8*)(Ks + kb * 32 * C::ROW_BYTES +
                                              (ch / C::NKOFF) * 256 + k_off[ch % C::NKOFF]);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ch], ch == 0 ? f32x16{} : s[kb], 0,
                                                      0, 0);
    }
  }
}

// K tile stored as two planes, one per half of the head dimension (the
// head-dim split copy of the pipelining study; D = 128, 64-key tiles): plane
// h holds dims [64h, 64h + 64) of the tile's rows, 128 bytes per row, with the
// 16-byte chunks of row r swizzled by (r / 2) mod 8 (a 16-lane pass of 16-byte
// reads then meets each bank once).
__device__ __forceinline__ int planar_kswz(int r) { return (r >> 1) & 7; }

// Asynchronous copy of plane h of a K tile (D = 128, BC = 64): 8 pieces of
// 1 KiB, piece n = rows 8n .. 8n+7; share `part` of COPY_WAVES issues pieces
// part * per .. part * per + per - 1.  Rows past the sequence end are clamped
// to the last row (finite data whose keys are masked).
template <class C>
__device__ __forceinline__ void copy_k_plane(const uint16_t* __restrict__ head_src, lds_u8* dst,
                                             int k0, int S, int part, int lane, int h) {
  static_assert(C::D == 128 && C::BC == 64, "planar K tiles: D = 128, 64-key tiles");
  constexpr int per = 8 / C::COPY_WAVES;  // pieces of a plane per copy wave
  const uint64_t b64 = (uint64_t)(head_src + (size_t)k0 * C::D);
  const uint32_t b_lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t b_hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  const char* base = (const char*)(((uint64_t)b_hi << 32) | b_lo);
#pragma unroll
  for (int u = 0; u < per; ++u) {
    const int n = part * per + u;
    const int r = 8 * n + (lane >> 3);
    const int cc = (lane & 7) ^ planar_kswz(r);
    const int src_row = min(r, S - 1 - k0);
    lds_dma<16>(base, (uint32_t)(src_row * C::ROW_BYTES + h * 128 + cc * 16),
                dst + h * 8192 + n * 1024);
  }
}

// Row max of a tile's raw scores for the lane's query (both lane halves).
template <class C>
__device__ __forceinline__ float row_max(const f32x16 (&s)[C::KB], int hh) {
  float x = s[0][0];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) x = fmaxf(x, s[kb][r]);
  return fmaxf(x, swap_halves(x, hh));
}

}  // namespace
