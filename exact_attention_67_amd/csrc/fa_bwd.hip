// Attention backward for MI355X (gfx950): dq, dk, dv of the fused forward.
//
// The pages ("Profiling in PyTorch (Part 3): Attention is all you profile",
// the "FlashAttention-2" blog) only say that the fused kernels serve training
// too; the computation here is the gradient of the forward definition
// (matmul, scale, causal mask, softmax, matmul), the same steps the
// FlashAttention-2 blog's fused forward avoids materialising:
//
//   P     = exp(scale * q k^T - LSE)      (recomputed from q, k and the saved LSE)
//   dv    = P^T dO
//   dP    = dO v^T
//   Delta = rowsum(dO * O)
//   dS    = P * (dP - Delta)
//   dq    = scale * dS k,   dk = scale * dS^T q
//
// Two kernels, dQ first:
//  * fa_bwd_dkdv_pair_kernel: one workgroup of 8 wavefronts per (block of
//    128 keys, head, batch).  Waves w and w + 4 share a SIMD and own the same
//    32 keys; the P wave forms S = q K^T, the weights P and dV, and hands P
//    to the dS wave through LDS, which forms dP = dO V^T, dS and dK one tile
//    later.  S and dP come out with one key per lane (the forward's
//    S^T = K Q^T with the roles of queries and keys exchanged), so P and dS
//    are per-lane columns; dV += P^T dO and dK += dS^T q read dO and q with
//    the transposing LDS read.  Each query tile of q and dO is copied once,
//    in a swizzle that serves both the row reads and the transposing reads.
//    Query tiles are 64 rows (32 at D = 256).
//  * fa_bwd_dq_kernel: one workgroup of 8 wavefronts per (block of 256
//    queries, head, batch), two wavefronts per SIMD as in the forward; waves
//    0-3 issue the tile copies.  (D = 256: 4 wavefronts, 32-key tiles.)  The forward's layout (one query per lane):
//    S^T = K q^T, dP^T = V dO^T, dS^T, then dq^T += K^T dS^T with K read
//    transposed.  K and V tiles are stored in one swizzle that serves both the
//    row reads and the transposing reads, so each K tile is copied once.
//    Before its loop it forms Delta for its rows from the dO fragments it
//    holds and O loaded the same way, and stores it for dK/dV.
// No atomics and no workspace beyond the caller's Delta buffer: dq is
// accumulated by the workgroup that owns the query tile.  fa_bwd_noalloc
// keeps Delta in a fixed device array of the library instead (scratch below).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "fa.h"
#include "fa_device.h"

namespace {

// Copy of 64 floats (one per query row of a tile) into LDS: lane l copies
// src[min(row0 + l, S - 1)].
__device__ __forceinline__ void issue_rowvec(const float* __restrict__ src, lds_u8* dst, int row0,
                                             int S, int lane) {
  lds_dma<4>(src, (uint32_t)min(row0 + lane, S - 1) * 4u, dst);
}

typedef __attribute__((address_space(3))) float lds_f32;

// bf16 O^T-layout accumulator column (lane = row `row` of the output, 16
// registers per 32-wide block) scaled and stored to out[row][0..D).
template <int DB>
__device__ __forceinline__ void store_col(uint16_t* __restrict__ out_row, const f32x16 (&acc)[DB],
                                          float mul, int hh) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 pk;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const __bf16 lo = (__bf16)(acc[db][gq * 4 + 2 * t] * mul);
        const __bf16 hi = (__bf16)(acc[db][gq * 4 + 2 * t + 1] * mul);
        pk[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<u32x2*>(out_row + db * 32 + gq * 8 + hh * 4) = pk;
    }
}

// One swizzle for tiles read both row-wise (16 rows of one chunk column per
// pass) and with the transposing read (4 consecutive rows x 4 chunks per
// pass), conflict-free for both: a bijection of the 16 rows of a pass onto
// chunk slots that also sends 4 consecutive rows to distinct 64-byte groups.
template <class C>
__device__ __forceinline__ int uswz(int r) {
  static_assert(C::ROW_BYTES == 512 || C::ROW_BYTES == 256 || C::ROW_BYTES == 128,
                "unified swizzle: D = 64, 128 or 256");
  // (512-byte rows: two bank lines per row; the XOR stays within a line)
  if constexpr (C::ROW_BYTES >= 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Copy offsets and operand-read offsets for the unified swizzle.
template <class C>
__device__ __forceinline__ void tile_offsets_u(int* off, int* row, int part, int lane) {
#pragma unroll
  for (int u = 0; u < C::LOADS_PER_WAVE; ++u) {
    const int n = part * C::LOADS_PER_WAVE + u;
    const int r = n * C::ROWS_PER_LOAD + lane / C::RC;
    row[u] = r;
    off[u] = r * C::D + ((lane % C::RC) ^ uswz<C>(r)) * 8;
  }
}
// (v_off: the transposing read's first half, rows R; v_hi: second half, rows
// R + 4, whose swizzle differs.)
template <class C>
__device__ __forceinline__ void operand_offsets_u(int lane, int (&k_off)[C::NKOFF],
                                                  int (&v_off)[C::NVOFF], int (&v_hi)[C::NVOFF]) {
  const int m = lane & 31, hh = lane >> 5;
  const int pm = key_perm(m);
  const int ksw = uswz<C>(pm);
#pragma unroll
  for (int b = 0; b < C::NKOFF; ++b) k_off[b] = pm * C::ROW_BYTES + (((2 * b + hh) ^ ksw) << 4);
  const int g = lane >> 4, j4 = (lane >> 2) & 3, t4 = lane & 3;
  const int vx = 2 * (g & 1) + (t4 >> 1);
  const int vsw = uswz<C>(hh * 8 + j4), vsw4 = uswz<C>(hh * 8 + j4 + 4);
  const int v_row = (hh * 8 + j4) * C::ROW_BYTES + (t4 & 1) * 8;
#pragma unroll
  for (int d4 = 0; d4 < C::NVOFF; ++d4) {
    v_off[d4] = v_row + (((4 * d4 + vx) ^ vsw) << 4);
    v_hi[d4] = v_row + 4 * C::ROW_BYTES + (((4 * d4 + vx) ^ vsw4) << 4);
  }
}

// Fragments of one row (lane's row `row` of a [S, D] matrix) as the B operand
// of qk_tile: lane holds X[row][ch*16 + hh*8 .. +8], its sign bits XORed with
// `flip` (negated for a negative scale); zero past the end.
template <class C>
__device__ __forceinline__ void row_fragments(bf16x8 (&f)[C::KCH], const uint16_t* __restrict__ X,
                                              int row, int S, int hh, uint32_t flip = 0u) {
#pragma unroll
  for (int ch = 0; ch < C::KCH; ++ch) {
    u32x4 raw = u32x4{0u, 0u, 0u, 0u};
    if (row < S) raw = *reinterpret_cast<const u32x4*>(X + (size_t)row * C::D + ch * 16 + hh * 8);
    f[ch] = __builtin_bit_cast(bf16x8, raw ^ flip);
  }
}

// One 32-row block of S = X * frag^T (rows of the tile X, read in the
// permuted order, against the lane's own fragment): s = X[kb*32 + perm(m)] . frag.
template <class C>
__device__ __forceinline__ void qk_block(f32x16& s, const lds_u8* X, const bf16x8 (&f)[C::KCH],
                                         const int (&k_off)[C::NKOFF], int kb) {
#pragma unroll
  for (int ch = 0; ch < C::KCH; ++ch) {
    const bf16x8 xf = *(const lds_bf16x8*)(X + kb * 32 * C::ROW_BYTES + (ch / C::NKOFF) * 256 +
                                           k_off[ch % C::NKOFF]);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, f[ch], ch == 0 ? f32x16{} : s, 0, 0, 0);
  }
}

// acc[hb] += A^T * bf for the 16 contraction rows of chunk pc (A read
// transposed from a tile in the unified swizzle), for NB 32-wide head-dim
// blocks starting at block part * NB.
template <class C, int NB>
__device__ __forceinline__ void tr_chunk(f32x16 (&acc)[NB], const lds_u8* tile,
                                         const bf16x8& bf, const int (&v_off)[C::NVOFF],
                                         const int (&v_hi)[C::NVOFF], int pc, int part) {
  static_assert(NB % C::NVOFF == 0, "a head-dim part spans whole offset groups");
  const lds_u8* t = tile + pc * 16 * C::ROW_BYTES + part * (NB / C::NVOFF) * 256;
#pragma unroll
  for (int db = 0; db < NB; ++db) {
    const lds_u8* b = t + (db / C::NVOFF) * 256;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + v_off[db % C::NVOFF]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + v_hi[db % C::NVOFF]));
    const bf16x8 af =
        __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[db], 0, 0, 0);
  }
}

// ----------------------------------------------------------------------------
// dK, dV with wave pairs: one workgroup of 8 wavefronts per (block of 128
// keys, head, batch)
// ----------------------------------------------------------------------------
// Waves w and w + 4 run on the same SIMD and own the same 32 keys; they split
// the work on each 64-query tile.  The P wave computes S = q K^T, the weights
// P and dV += P^T dO, and leaves P (bf16, the operand of its dV product) in
// LDS.  The dS wave computes dP = dO V^T, and one tile later, with that P,
// dS = P (dP - Delta) and dK += dS^T q.  Each wave holds about half the state
// of a wave doing both (its fragments, its accumulators, one score tile), so
// two of them fit on a SIMD and keep its matrix core busy while the other
// waits on LDS or forms weights.
//
// Tiles: q(t), LSE(t), Delta(t) in stage (t - t_first) mod 3, dO(t) in stage
// (t - t_first) mod 2 (nothing reads dO(t-1) during step t).  Step t copies
// tile t+1 into the next stages; the P wave reads q(t) by rows and dO(t)
// transposed, the dS wave dO(t) by rows and q(t-1) transposed.  P(t) goes to
// exchange buffer (t - t_first) mod 2.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_bwd_dkdv_pair_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int S, int nk, int bh_total, int group_heads, float c,
    float scale) {
  // Query tiles of 64 rows, 32 at D = 256 (registers: the key fragment and
  // the accumulator alone take 192 of a wave's 256 there).
  constexpr int BQ = D == 256 ? 32 : 64;
  using C = BfCfg<D, BQ, 4>;        // tile geometry; each role copies its tensor in 4 parts
  constexpr int XB = C::PCH * 1024;  // P of one pair and tile: PCH chunks x 64 lanes x 16 B
  static_assert(C::PCH == 2 * C::KB, "two 16-query chunks per 32-query block");
  __shared__ __attribute__((aligned(1024))) uint8_t q0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t q1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t q2_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t d0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t d1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t x0_raw[4 * XB];
  __shared__ __attribute__((aligned(1024))) uint8_t x1_raw[4 * XB];
  __shared__ __attribute__((aligned(256))) uint8_t l0_raw[256];
  __shared__ __attribute__((aligned(256))) uint8_t l1_raw[256];
  __shared__ __attribute__((aligned(256))) uint8_t l2_raw[256];
  __shared__ __attribute__((aligned(256))) uint8_t e0_raw[256];
  __shared__ __attribute__((aligned(256))) uint8_t e1_raw[256];
  __shared__ __attribute__((aligned(256))) uint8_t e2_raw[256];
  lds_u8* q0s = (lds_u8*)q0_raw;
  lds_u8* q1s = (lds_u8*)q1_raw;
  lds_u8* q2s = (lds_u8*)q2_raw;
  lds_u8* d0s = (lds_u8*)d0_raw;
  lds_u8* d1s = (lds_u8*)d1_raw;
  lds_u8* x0s = (lds_u8*)x0_raw;
  lds_u8* x1s = (lds_u8*)x1_raw;
  lds_u8* l0s = (lds_u8*)l0_raw;
  lds_u8* l1s = (lds_u8*)l1_raw;
  lds_u8* l2s = (lds_u8*)l2_raw;
  lds_u8* e0s = (lds_u8*)e0_raw;
  lds_u8* e1s = (lds_u8*)e1_raw;
  lds_u8* e2s = (lds_u8*)e2_raw;

  // Heaviest key blocks (the first ones, seen by most query tiles) first.
  int bh, kt;
  decode_tile<CAUSAL>(xcd_logical_index(blockIdx.x, nk * bh_total), nk, bh_total, group_heads,
                      bh, kt);
  if (CAUSAL) kt = nk - 1 - kt;

  const size_t head = (size_t)bh * (size_t)S * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* dOh = dO + head;
  const float* LSEh = LSE + (size_t)bh * S;
  const float* Dh = Delta + (size_t)bh * S;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = wave & 3;        // pair: keys kw0 .. kw0 + 31
  const bool p_wave = wave < 4;   // role (wave-uniform)
  const int m = lane & 31;
  const int hh = lane >> 5;
  const int k0 = kt * 128;
  const int kw0 = k0 + pr * kRowsPerWave;
  const int my_k = kw0 + m;

  // Query tiles this workgroup visits: causal -- those with a query >= k0.
  // A pair takes part in tile t when some query of the tile sees one of its
  // keys (with the causal mask this holds for every tile after its first).
  const int nt = (S + BQ - 1) / BQ;
  const int t_first = CAUSAL ? k0 / BQ : 0;
  auto live = [&](int t) { return kw0 < S && (!CAUSAL || t * BQ + BQ - 1 >= kw0); };

  // Copies: the P waves copy q, the dS waves dO (each wave a quarter), wave 0
  // LSE and wave 4 Delta.
  // (offsets recomputed at each copy rather than held through the loop)
  auto copy_tile = [&](int t, lds_u8* qd, lds_u8* dd, lds_u8* ld, lds_u8* ed) {
    const int q0 = t * BQ;
    int off[C::LOADS_PER_WAVE], row[C::LOADS_PER_WAVE];
    tile_offsets_u<C>(off, row, pr, lane);
    if (p_wave) {
      issue_tile<C>(Qh, qd, q0, S, pr, off, row);
      if (wave == 0) issue_rowvec(LSEh, ld, q0, S, lane);
    } else {
      issue_tile<C>(dOh, dd, q0, S, pr, off, row);
      if (wave == 4) issue_rowvec(Dh, ed, q0, S, lane);
    }
  };

  // The lane's key fragment: K for the P wave (S), V for the dS wave (dP).
  bf16x8 kf[C::KCH];
  // (negative scale: the P wave's S from -K with |c|, see kZeroScaleC; dK
  // uses q as it is)
  row_fragments<C>(kf, (p_wave ? K : V) + head, my_k, S, hh, p_wave ? sign_flip_mask(c) : 0u);
  c = fabsf(c);
  int k_off[C::NKOFF], v_off[C::NVOFF], v_hi[C::NVOFF];
  operand_offsets_u<C>(lane, k_off, v_off, v_hi);

  f32x16 acc[C::DB];  // dV (P wave) or dK (dS wave), transposed
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  // P wave, tile t: S from q(t), mask, weights, P to the exchange buffer,
  // dV += P^T dO(t).
  auto p_step = [&](const int t, const lds_u8* qs, const lds_u8* dsn, const lds_u8* ls,
                    lds_u8* xs) {
    if (!live(t)) return;
    f32x16 s[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) qk_block<C>(s[kb], qs, kf, k_off, kb);
    const int q0 = t * BQ;
    if ((CAUSAL && q0 < kw0 + 31) || (q0 + BQ > S)) {
#pragma unroll
      for (int qb = 0; qb < C::KB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // register r of block qb holds query row 32*qb + 16*(r/8) + 8*hh + r%8
          const int q = q0 + 32 * qb + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (q >= S || (CAUSAL && my_k > q)) s[qb][r] = -INFINITY;
        }
    }
    lds_u8* xw = xs + pr * XB + lane * 16;
#pragma unroll
    for (int pc = 0; pc < C::PCH; ++pc) {
      const int qb = pc >> 1, half = pc & 1;
      const int rb = 32 * qb + 16 * half + 8 * hh;
      bf16x8 pq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float lse2 = reinterpret_cast<const lds_f32*>(ls)[rb + e] * kLog2e;
        pq[e] = (__bf16)fast_exp2(fmaf(s[qb][8 * half + e], c, -lse2));
      }
      *(lds_bf16x8*)(xw + pc * 1024) = pq;
      tr_chunk<C, C::DB>(acc, dsn, pq, v_off, v_hi, pc, 0);  // dV^T += dO^T P
    }
    // compiler MFMA/LDS interleave strategy 1 (measured: 1 % faster here, and
    // 2.5 % slower in the dS wave, which keeps the default order)
    __builtin_amdgcn_iglp_opt(1);
  };
  // dS wave, step t: dP(t) from dO(t) into dp_out (d_dp); dS(t-1) from
  // P(t-1) (xs), dP(t-1) (dp_in) and Delta(t-1), dK += dS^T q(t-1) (d_ds).
  auto d_dp = [&](const int t, const lds_u8* dsr, f32x16 (&dp_out)[C::KB]) {
    if (!live(t)) return;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) qk_block<C>(dp_out[kb], dsr, kf, k_off, kb);
  };
  auto d_ds = [&](const int tp, const lds_u8* qprev, const lds_u8* eprev, const lds_u8* xs,
                  const f32x16 (&dp_in)[C::KB]) {
    if (!live(tp)) return;
    const lds_u8* xr = xs + pr * XB + lane * 16;
#pragma unroll
    for (int pc = 0; pc < C::PCH; ++pc) {
      const int qb = pc >> 1, half = pc & 1;
      const int rb = 32 * qb + 16 * half + 8 * hh;
      const bf16x8 pq = *(const lds_bf16x8*)(xr + pc * 1024);
      bf16x8 dsq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float del = reinterpret_cast<const lds_f32*>(eprev)[rb + e];
        dsq[e] = (__bf16)((float)pq[e] * (dp_in[qb][8 * half + e] - del));
      }
      tr_chunk<C, C::DB>(acc, qprev, dsq, v_off, v_hi, pc, 0);  // dK^T += q^T dS
    }
  };
  auto d_step = [&](const int t, const lds_u8* dsr, const lds_u8* qprev, const lds_u8* eprev,
                    const lds_u8* xs, f32x16 (&dp_out)[C::KB], const f32x16 (&dp_in)[C::KB]) {
    if constexpr (D == 256) {
      // one dP set: dS(t-1) consumes it before dP(t) overwrites it
      if (t > t_first) d_ds(t - 1, qprev, eprev, xs, dp_in);
      if (t < nt) d_dp(t, dsr, dp_out);
    } else {
      if (t < nt) d_dp(t, dsr, dp_out);
      if (t > t_first) d_ds(t - 1, qprev, eprev, xs, dp_in);
    }
  };

  if (t_first < nt) copy_tile(t_first, q0s, d0s, l0s, e0s);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Each role runs its own loop (so neither holds the other's registers);
  // both take one barrier per step, the same steps, so the workgroup's
  // barriers stay matched.  Six steps per pass (three q stages; two dO
  // stages, exchange buffers and dP sets), every buffer named at compile
  // time.  Step: copy tile t+1 into the next stages, the role's work, wait
  // for the copies, barrier.
#define FA_PAIR_COPY(QN, DN, LN, EN) \
  if (t + 1 < nt) copy_tile(t + 1, QN, DN, LN, EN);
#define FA_PAIR_END                    \
  __builtin_amdgcn_s_waitcnt(0);       \
  __syncthreads();
  if (p_wave) {
    if (t_first < nt) {
      for (int t = t_first;;) {
        FA_PAIR_COPY(q1s, d1s, l1s, e1s) p_step(t, q0s, d0s, l0s, x0s); FA_PAIR_END
        if (++t >= nt) break;
        FA_PAIR_COPY(q2s, d0s, l2s, e2s) p_step(t, q1s, d1s, l1s, x1s); FA_PAIR_END
        if (++t >= nt) break;
        FA_PAIR_COPY(q0s, d1s, l0s, e0s) p_step(t, q2s, d0s, l2s, x0s); FA_PAIR_END
        if (++t >= nt) break;
        FA_PAIR_COPY(q1s, d0s, l1s, e1s) p_step(t, q0s, d1s, l0s, x1s); FA_PAIR_END
        if (++t >= nt) break;
        FA_PAIR_COPY(q2s, d1s, l2s, e2s) p_step(t, q1s, d0s, l1s, x0s); FA_PAIR_END
        if (++t >= nt) break;
        FA_PAIR_COPY(q0s, d0s, l0s, e0s) p_step(t, q2s, d1s, l2s, x1s); FA_PAIR_END
        if (++t >= nt) break;
      }
    }
    if (my_k < S) store_col<C::DB>(dV + head + (size_t)my_k * D, acc, 1.0f, hh);
    return;
  }
  // dS wave: one step more than the P wave (t = nt: the final tile's dS and
  // dK only, with no copy and no barrier).
#define FA_PAIR_DEND            \
  if (t < nt) {                 \
    FA_PAIR_END                 \
  }
  // dP of the current and the previous tile (at D = 256 one set serves both)
  f32x16 dp_a[C::KB], dp_x[C::KB];
  f32x16(&dp_b)[C::KB] = [&]() -> f32x16(&)[C::KB] {
    if constexpr (D == 256) return dp_a;
    else return dp_x;
  }();
  if (t_first < nt) {
    for (int t = t_first;;) {
      FA_PAIR_COPY(q1s, d1s, l1s, e1s) d_step(t, d0s, q2s, e2s, x1s, dp_a, dp_b); FA_PAIR_DEND
      if (++t > nt) break;
      FA_PAIR_COPY(q2s, d0s, l2s, e2s) d_step(t, d1s, q0s, e0s, x0s, dp_b, dp_a); FA_PAIR_DEND
      if (++t > nt) break;
      FA_PAIR_COPY(q0s, d1s, l0s, e0s) d_step(t, d0s, q1s, e1s, x1s, dp_a, dp_b); FA_PAIR_DEND
      if (++t > nt) break;
      FA_PAIR_COPY(q1s, d0s, l1s, e1s) d_step(t, d1s, q2s, e2s, x0s, dp_b, dp_a); FA_PAIR_DEND
      if (++t > nt) break;
      FA_PAIR_COPY(q2s, d1s, l2s, e2s) d_step(t, d0s, q0s, e0s, x1s, dp_a, dp_b); FA_PAIR_DEND
      if (++t > nt) break;
      FA_PAIR_COPY(q0s, d0s, l0s, e0s) d_step(t, d1s, q1s, e1s, x0s, dp_b, dp_a); FA_PAIR_DEND
      if (++t > nt) break;
    }
  }
#undef FA_PAIR_DEND
#undef FA_PAIR_COPY
#undef FA_PAIR_END
  if (my_k < S) store_col<C::DB>(dK + head + (size_t)my_k * D, acc, scale, hh);
}

// acc[db] += A^T * bf, A read transposed from a tile in the unified swizzle.
template <class C>
__device__ __forceinline__ void tr_product_u(f32x16 (&acc)[C::DB], const lds_u8* tile,
                                             const bf16x8 (&bf)[C::PCH],
                                             const int (&v_off)[C::NVOFF],
                                             const int (&v_hi)[C::NVOFF]) {
#pragma unroll
  for (int pc = 0; pc < C::PCH; ++pc)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const lds_u8* b = tile + pc * 16 * C::ROW_BYTES + (db / C::NVOFF) * 256;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + v_off[db % C::NVOFF]));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + v_hi[db % C::NVOFF]));
      const bf16x8 af =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[pc], acc[db], 0, 0, 0);
    }
}

// ----------------------------------------------------------------------------
// dQ: one workgroup per (256 queries, head, batch)
// ----------------------------------------------------------------------------
template <int D, int BC, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(64 * WAVES, WAVES == 8 ? 2 : 1) void fa_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ Delta,
    uint16_t* __restrict__ dQ, int S, int nq, int bh_total, int group_heads, float c,
    float scale) {
  using C = BfCfg<D, BC, WAVES>;  // key tiles of BC; waves of 32 queries
  // K tile in two layouts (row reads for S^T, transposed reads for dq), V
  // tile row-wise (for dP^T); two stages.
  __shared__ __attribute__((aligned(1024))) uint8_t kr0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kr1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vr0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vr1_raw[C::TILE_BYTES];
  lds_u8* kr0 = (lds_u8*)kr0_raw;
  lds_u8* kr1 = (lds_u8*)kr1_raw;
  lds_u8* vr0 = (lds_u8*)vr0_raw;
  lds_u8* vr1 = (lds_u8*)vr1_raw;

  int bh, qt;
  decode_tile<CAUSAL>(xcd_logical_index(blockIdx.x, nq * bh_total), nq, bh_total, group_heads,
                      bh, qt);
  const size_t head = (size_t)bh * (size_t)S * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const uint16_t* dOh = dO + head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * C::BR;
  const int qw0 = q0 + wave * kRowsPerWave;
  const int my_q = qw0 + m;

  const int kend = CAUSAL ? min(S, q0 + C::BR) : S;
  const int ntiles = (kend + BC - 1) / BC;
  const int wave_klast = CAUSAL ? min(qw0 + kRowsPerWave - 1, S - 1) : (S - 1);
  const int wave_ntiles = qw0 < S ? min(ntiles, wave_klast / BC + 1) : 0;

  const bool copier = wave < C::COPY_WAVES;
  const int cw = copier ? wave : 0;  // this wave's share of each tile copy
  // The copy offsets are recomputed at each copy (a few instructions, copier
  // waves only) rather than held in registers through the loop.
  auto copies = [&](int j, lds_u8* kr, lds_u8* vr) {
    if (!copier) return;
    int off[C::LOADS_PER_WAVE], row[C::LOADS_PER_WAVE];
    const int k0 = j * BC;
    tile_offsets_u<C>(off, row, cw, lane);
    issue_tile<C>(Kh, kr, k0, S, cw, off, row);
    issue_tile<C>(Vh, vr, k0, S, cw, off, row);
  };

  bf16x8 qf[C::KCH], df[C::KCH];
  // negative scale: S^T from -q with |c| (see kZeroScaleC); dq uses K as it is
  row_fragments<C>(qf, Qh, my_q, S, hh, sign_flip_mask(c));
  row_fragments<C>(df, dOh, my_q, S, hh);
  c = fabsf(c);
  int k_off[C::NKOFF], v_off[C::NVOFF], v_hi[C::NVOFF];
  operand_offsets_u<C>(lane, k_off, v_off, v_hi);
  const float lse2 = my_q < S ? LSE[(size_t)bh * S + my_q] * kLog2e : 0.0f;
  // Delta of the wave's rows, from the dO fragments and O loaded the same
  // way (each lane half holds half of a row's entries); stored for dK/dV.
  float delta;
  {
    bf16x8 of[C::KCH];
    row_fragments<C>(of, O + head, my_q, S, hh);
    float part = 0.0f;
#pragma unroll
    for (int ch = 0; ch < C::KCH; ++ch)
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)df[ch][e], (float)of[ch][e], part);
    delta = part + __shfl_xor(part, 32);
    if (hh == 0 && my_q < S) Delta[(size_t)bh * S + my_q] = delta;
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  if (ntiles > 0) copies(0, kr0, vr0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto step = [&](const int j, const lds_u8* kr, const lds_u8* vr, lds_u8* nkr, lds_u8* nvr) {
    if (j + 1 < ntiles) copies(j + 1, nkr, nvr);
    if (j < wave_ntiles) {
      const int k0 = j * BC;
      f32x16 s[C::KB], dp[C::KB];
      qk_tile<C>(s, kr, qf, k_off);   // S^T[key][q]
      qk_tile<C>(dp, vr, df, k_off);  // dP^T[key][q]
      const bool masked = (CAUSAL && (k0 + BC - 1 > qw0)) || (k0 + BC > S);
      const int lim = (CAUSAL ? min(my_q, S - 1) : (S - 1)) - k0 - hh * 8;
      bf16x8 dsf[C::PCH];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // register r of block kb holds key kb*32 + (r>>3)*16 + hh*8 + (r&7)
          float p = fast_exp2(fmaf(s[kb][r], c, -lse2));
          if (masked && kb * 32 + (r >> 3) * 16 + (r & 7) > lim) p = 0.0f;
          dsf[2 * kb + (r >> 3)][r & 7] = (__bf16)(p * (dp[kb][r] - delta));
        }
      tr_product_u<C>(acc, kr, dsf, v_off, v_hi);  // dq^T += K^T dS^T
      // compiler MFMA/LDS interleave strategy 1 (measured: 0.5-2 % faster)
      __builtin_amdgcn_iglp_opt(1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    step(j, kr0, vr0, kr1, vr1);
    step(j + 1, kr1, vr1, kr0, vr0);
  }
  if (j < ntiles) step(j, kr0, vr0, kr1, vr1);

  if (my_q >= S) return;
  store_col<C::DB>(dQ + head + (size_t)my_q * D, acc, scale, hh);
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

template <class KernelT, class... Args>
int launch_k(KernelT kernel, unsigned grid, unsigned threads, hipStream_t stream,
             Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid),
                                       dim3(threads), argv, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D>
int run_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
            const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
            float* delta, int bh, int S, bool causal, float scale, hipStream_t s) {
  const float c = scale == 0.0f ? kZeroScaleC : scale * kLog2e;  // sign: see kZeroScaleC
  const int group_heads = bh >= 8 ? bh / 8 : 1;
  // dQ first: it also forms Delta, which dK/dV reads.  dQ: 8 waves and
  // 64-key tiles; D = 256: 4 waves and 32-key tiles (registers and LDS).
  constexpr int BT = D == 256 ? 32 : 64;
  constexpr int QW = D == 256 ? 4 : 8;
  const int nq = (S + 32 * QW - 1) / (32 * QW);
  const unsigned gq = (unsigned)nq * (unsigned)bh;
  int st;
  if (causal)
    st = launch_k(fa_bwd_dq_kernel<D, BT, QW, true>, gq, 64 * QW, s, q, k, v, dout, o,
                  (const float*)lse, delta, dq, S, nq, bh, group_heads, c, scale);
  else
    st = launch_k(fa_bwd_dq_kernel<D, BT, QW, false>, gq, 64 * QW, s, q, k, v, dout, o,
                  (const float*)lse, delta, dq, S, nq, bh, group_heads, c, scale);
  if (st != FA_OK) return st;
  const int nk = (S + 127) / 128;
  const unsigned grid = (unsigned)nk * (unsigned)bh;
  if (causal)
    return launch_k(fa_bwd_dkdv_pair_kernel<D, true>, grid, 512, s, q, k, v, dout,
                    (const float*)lse, (const float*)delta, dk, dv, S, nk, bh, group_heads, c,
                    scale);
  return launch_k(fa_bwd_dkdv_pair_kernel<D, false>, grid, 512, s, q, k, v, dout,
                  (const float*)lse, (const float*)delta, dk, dv, S, nk, bh, group_heads, c,
                  scale);
}

}  // namespace

// Argument checks shared by fa_bwd and fa_bwd_noalloc.  delta is the caller's
// Delta buffer, or NULL when the library's scratch array holds Delta.
int validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, bool own_delta,
                 int B, int H, int S, int D, int causal, float scale) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || (!own_delta && !delta))
    return FA_ERR_NULL;
  if (B < 1 || H < 1 || S < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const int64_t bh = (int64_t)B * H;
  const int64_t nk = ((int64_t)S + 127) / 128;
  if (bh > INT32_MAX || (int64_t)S * D > INT32_MAX || 2 * nk * bh > INT32_MAX ||
      (uint64_t)(bh * S * D) > (uint64_t)(SIZE_MAX / 4))
    return FA_ERR_SHAPE;
  const uintptr_t a16 = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o |
                        (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv;
  if ((a16 & 15u) || (((uintptr_t)lse | (uintptr_t)delta) & 3u)) return FA_ERR_ALIGN;
  const size_t tb = (size_t)(bh * S * D) * 2, lb = (size_t)(bh * S) * sizeof(float);
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t in_b[6] = {tb, tb, tb, tb, tb, lb};
  void* outs[4] = {dq, dk, dv, delta};
  const size_t out_b[4] = {tb, tb, tb, lb};
  const int nout = own_delta ? 3 : 4;
  for (int a = 0; a < nout; ++a) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[a], out_b[a], ins[i], in_b[i])) return FA_ERR_ALIAS;
    for (int b = a + 1; b < nout; ++b)
      if (overlap(outs[a], out_b[a], outs[b], out_b[b])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

int bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
        const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int S,
        int D, int causal, float scale, void* stream) {
  const int64_t bh = (int64_t)B * H;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* Q = static_cast<const uint16_t*>(q);
  const auto* Kp = static_cast<const uint16_t*>(k);
  const auto* Vp = static_cast<const uint16_t*>(v);
  const auto* O = static_cast<const uint16_t*>(o);
  const auto* dO = static_cast<const uint16_t*>(dout);
  auto* dQ = static_cast<uint16_t*>(dq);
  auto* dK = static_cast<uint16_t*>(dk);
  auto* dV = static_cast<uint16_t*>(dv);
  if (D == 64)
    return run_bwd<64>(Q, Kp, Vp, O, dO, lse, dQ, dK, dV, delta, (int)bh, S, causal != 0, scale, s);
  if (D == 128)
    return run_bwd<128>(Q, Kp, Vp, O, dO, lse, dQ, dK, dV, delta, (int)bh, S, causal != 0, scale, s);
  return run_bwd<256>(Q, Kp, Vp, O, dO, lse, dQ, dK, dV, delta, (int)bh, S, causal != 0, scale, s);
}

// Delta of fa_bwd_noalloc: one float per query row, at most FA_BWD_SCRATCH_ROWS
// rows per call.  Every row a call uses is written by the call's dQ kernel
// before its dK/dV kernel reads it, so nothing needs clearing.
// Each GPU holds its own copy of the array, at its own address, for the life
// of the process; host code uses that address (scratch_address), never the
// array's name, which on the host only stands in for the device symbol.
static __device__ __align__(256) float scratch[FA_BWD_SCRATCH_ROWS];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];  // device address of scratch, per device

// Address of scratch on the device `stream` runs on, looked up once per
// device with that device current.
int scratch_address(hipStream_t stream, float** out) {
  int dev = -1;
  const hipError_t ge = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (ge != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (e != hipSuccess || !addr) return FA_ERR_LAUNCH;
    p = static_cast<float*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FA_OK;
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* delta, int B, int H, int S, int D, int causal, float scale,
                      void* stream) {
  const int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, false, B, H, S, D,
                              causal, scale);
  if (st != FA_OK) return st;
  return bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, S, D, causal, scale, stream);
}

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int S, int D, int causal, float scale,
                              void* stream) {
  int st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, true, B, H, S, D, causal,
                        scale);
  if (st != FA_OK) return st;
  if ((int64_t)B * H * S > (int64_t)FA_BWD_SCRATCH_ROWS) return FA_ERR_SCRATCH;
  float* delta = nullptr;
  st = scratch_address(static_cast<hipStream_t>(stream), &delta);
  if (st != FA_OK) return st;
  return bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, S, D, causal, scale, stream);
}
