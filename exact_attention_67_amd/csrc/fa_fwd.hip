// Fused, tiled, exact attention forward for MI355X (gfx950, CDNA4).
//
// One workgroup of 4 or 8 wavefronts owns one (query tile of 128 or 256 rows,
// head, batch); each wavefront owns 32 query rows (at D = 256 a pair of
// wavefronts on one SIMD shares them, one forming the softmax weights, the
// other the P*V product).  Key/value tiles are
// streamed through LDS with a running (online) softmax, so the seq x seq score
// matrix only ever exists in registers -- the method of "Profiling in PyTorch
// (Part 3): Attention is all you profile", section "Why flash attention
// exists", with the FlashAttention-2 choices listed in the "FlashAttention-2"
// blog, section "FlashAttention-2 Optimizations": causal tiles that are fully
// masked are skipped, the grid runs over sequence blocks as well as batch and
// heads, and the work is split between waves by query rows so that no
// cross-wave reduction is needed.  The "Pipelining GmemCopy on kHeadDim" issue
// discusses overlapping the global-memory copy of the next key block with the
// math on the current one; here whole K/V tiles are copied one to two tiles
// ahead, straight from global memory into LDS (no register staging), into
// double-buffered (four buffers each at D = 256) LDS buffers.
//
// gfx950 mapping (bf16 path):
//  * Both contractions run on v_mfma_f32_32x32x16_bf16 in transposed form:
//    S^T = K * Q^T and O^T = V^T * P^T.  In the 32x32 accumulator layout a lane
//    holds one column (= one query) and 16 rows (= keys or head-dim entries),
//    so a query's row max / row sum is an in-lane reduction plus one exchange
//    between lane l and lane l^32, and the per-query rescale factor multiplies
//    the lane's own O^T column.
//  * The 32 K rows fed to one MFMA are read in a permuted order (bits 2 and 3
//    of the row index swapped).  With that order a lane's accumulator
//    registers hold runs of 8 consecutive keys, so after the softmax they are
//    directly the B operand of the P*V MFMA.
//  * V stays row-major in LDS; the V^T operand is read with the transposing
//    LDS read (two ds_read_b64_tr_b16 per MFMA).
//  * LDS rows are XOR-swizzled in 16-byte units so the MFMA operand reads are
//    free of bank conflicts on the 64-bank LDS.
//  * exp2 with the scale folded into one FMA per score.  A row's reference
//    max is raised only when the weights of a tile would grow too large (D <=
//    128: a lane's sum of weights in the tile above 2^12, found after the
//    weights are formed, with P*V deferred by one tile so that it only ever
//    sees checked weights; D = 256: the same check against 2^24, the O wave
//    rescaling O when the reference that comes with the weights moved), so
//    the rescale of the O accumulator (wave-uniform) runs on few tiles.  O is
//    normalised by the sum of
//    the bf16 weights that multiplied V (for D <= 128 formed on the matrix
//    cores by a 16x16x32 product with a 0/1 operand).
//  * The 1-D grid is decoded XCD-aware (the 8 XCDs receive workgroups round-
//    robin; consecutive logical tiles of the same heads are kept on one XCD so
//    they share its L2) and, when causal, heaviest query tiles first.
//  * Queries against a longer or shorter key sequence (Sq != Sk, causal mask
//    aligned bottom-right) run through the same kernels; rows with no visible
//    key give O = 0 and LSE = -inf.  A single query row of few heads
//    (decode) has a kernel of its own that streams K/V rows into registers
//    (fa_decode_kernel).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"
#include "fa_device.h"

namespace {

constexpr int kWaves = 4;                   // float32 kernel: wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = kRowsPerWave * kWaves;  // float32 kernel: query rows per workgroup
#ifndef FA_MFMA_SUM
#define FA_MFMA_SUM 1
#endif
constexpr bool kMfmaSum = FA_MFMA_SUM != 0;  // bf16-weight sums on the matrix cores

// s_waitcnt immediate: at most n vector-memory operations outstanding, all
// LDS operations done (expcnt untouched).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// How fa_fwd_bf16_kernel moves K/V tiles into LDS.  The library's fa_fwd uses
// kPipeOverlap; the other modes exist for the pipelining study of the
// "Pipelining GmemCopy on kHeadDim" issue (whole-tile prefetch against none,
// and deeper buffering) and are compiled only into separate study libraries
// (FA_PIPE at build time).
enum PipeMode : int {
  kPipeOverlap = 0,     // a tile is copied during the step before it is read; two buffers each
  kPipeNoPrefetch = 1,  // each step copies the tiles it reads, waits for them, then computes
  kPipeKSplit = 2,      // as kPipeNoPrefetch, with K copied in two head-dim halves: the
                        // products over dims 0-63 start once the first half has landed
                        // (D = 128; other head dimensions run kPipeNoPrefetch)
  kPipeRing3 = 3,       // three buffers each; a tile is copied two steps before it is read
  kPipeRing4 = 4,       // four buffers each; a tile is copied three steps before it is read
  kPipeMfmaOnly = 5,    // no copies, no exponentials, no weight check: the products and
                        // their LDS operand reads alone (a timing probe; results are void)
  kPipeD256Ring = 6,    // D = 256 on fa_fwd_bf16_ring_kernel (one wave per SIMD) in place
                        // of the wave-pair kernel; D <= 128 as kPipeOverlap
};
template <int PIPE>
struct PipeCfg {
  static constexpr int R = PIPE == kPipeRing3 ? 3 : PIPE == kPipeRing4 ? 4 : 2;  // buffers each
  static constexpr int U = R == 3 ? 6 : R;  // steps per unrolled group: buffer slots and S parity
  static constexpr bool kPrefetch = PIPE != kPipeNoPrefetch && PIPE != kPipeKSplit;
  static constexpr bool kCopies = PIPE != kPipeMfmaOnly;
  static constexpr bool kSoftmax = PIPE != kPipeMfmaOnly;
};
#ifndef FA_PIPE
#define FA_PIPE 0
#endif
constexpr int kPipe = FA_PIPE;
static_assert(kPipe == kPipeOverlap || kPipe == kPipeNoPrefetch || kPipe == kPipeKSplit ||
                  kPipe == kPipeRing3 || kPipe == kPipeRing4 || kPipe == kPipeMfmaOnly ||
                  kPipe == kPipeD256Ring,
              "FA_PIPE");

// sched_group_barrier with a compile-time count; nothing when the count is 0.
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}

// Fixed instruction order of one full tile step of fa_fwd_bf16_kernel (product
// I of the step is the I-th MFMA in program order: the bf16-weight sums when
// MFMA_SUM, then the P*V products, then the S products).  Each product is
// followed by the operand reads of the product kLead places later (two
// transposing V reads for a P*V product, one K read for an S product) and by
// its share of the step's FMAs, adds and bf16 packs.  The exponentials are
// left to the compiler's placement: pinning one to every product (a group of
// transcendental instructions per product) measured about 2 % slower, since
// it shortens how far ahead the operand reads are waited for.
template <class C, bool MFMA_SUM, int N>
struct StepOrder {
  static constexpr int kLead = 3;
  static constexpr int kSum = MFMA_SUM ? C::PCH : 0;
  static constexpr int kPV = C::DB * C::PCH;
  // an FMA and an add per score, a bf16 pack per pair, and the dot products
  // of the bf16 sums when they are not on the matrix cores
  static constexpr int kValu = C::KB * 16 * 2 + C::KB * 8 + (MFMA_SUM ? 0 : C::PCH * 4);
  // operand reads issued after product i: those of product i + kLead (the
  // bf16-weight sums read no operands)
  static constexpr int reads_of(int j) { return j < 0 ? 0 : j < kPV ? 2 : j < N - kSum ? 1 : 0; }
  static constexpr int reads(int i) { return reads_of(i + kLead - kSum); }
  // reads of the products that start before any product has issued
  static constexpr int first_reads() {
    int n = 0;
    for (int j = 0; j < kLead - kSum; ++j) n += reads_of(j);
    return n;
  }
  // product i's share of `total` instructions, spread evenly over the products
  static constexpr int share(int i, int total) { return ((i + 1) * total) / N - (i * total) / N; }
};

template <class C, bool MFMA_SUM, int... I>
__device__ __forceinline__ void step_schedule(std::integer_sequence<int, I...>) {
  using O = StepOrder<C, MFMA_SUM, (int)sizeof...(I)>;
  sched_group<0x100, O::first_reads()>();
  ((sched_group<0x008, 1>(), sched_group<0x100, O::reads(I)>(),
    sched_group<0x002, O::share(I, O::kValu)>()),
   ...);
}

// Two waves per SIMD (two 4-wave or one 8-wave workgroup per CU; D <= 128).
//
// Tile step t (one 64-key tile; one workgroup barrier per step):
//  * the weights of tile t are formed from S(t), computed in step t-1:
//    p = 2^(s*c - m*c) against the row's reference max m, rounded to bf16;
//  * O += P(t-1) V(t-1) and the row sums of the bf16 weights of tile t-1 on
//    the matrix cores (the weights were checked at the end of step t-1);
//  * S(t+1) = Q K(t+1)^T on the matrix cores.
// The vector work of the step (one FMA, one exponential, one add per score and
// one bf16 pack per pair) runs beside the step's 36 matrix instructions.  The
// row max is not taken per tile: after the weights of tile t are formed, a
// lane whose sum of weights exceeds kRowSumLimit (or is not finite) sends the
// wave through a rare path that raises the reference to the tile's max and
// rescales (weights stay <= kRowSumLimit, so nothing overflows).  The
// reference is set from the true max of tile 0 before the first step, and it
// only moves up, so the largest weight of a row is >= 1.
template <int D, int BC, int WAVES, bool CAUSAL, bool MFMA_SUM, int PIPE>
__global__ __launch_bounds__(64 * WAVES, 2) void fa_fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Sq, int Sk, int nq, int bh_total, int group_heads, float c) {
  using C = BfCfg<D, BC, WAVES>;
  // negative scale: S from -Q with |c| (see kZeroScaleC)
  const uint32_t qflip = sign_flip_mask(c);
  c = fabsf(c);
  using PC = PipeCfg<PIPE>;
  constexpr int R = PC::R, U = PC::U;
  // Separate buffers (R for K, R for V) rather than one array indexed by tile
  // number: every access below names its buffer statically (the step code is
  // unrolled over U consecutive steps), so the compiler can tell that an
  // asynchronous copy into one buffer never aliases reads of another and does
  // not make those reads wait for the copy.
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf2_raw[R > 2 ? C::TILE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf3_raw[R > 3 ? C::TILE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf2_raw[R > 2 ? C::TILE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf3_raw[R > 3 ? C::TILE_BYTES : 16];
  // buffer of K (V) tile u, for a compile-time u (only its residue mod R matters)
  const auto kslot = [&](auto u) -> lds_u8* {
    constexpr int i = decltype(u)::value % R;
    if constexpr (i == 0) return (lds_u8*)kbuf0_raw;
    else if constexpr (i == 1) return (lds_u8*)kbuf1_raw;
    else if constexpr (i == 2) return (lds_u8*)kbuf2_raw;
    else return (lds_u8*)kbuf3_raw;
  };
  const auto vslot = [&](auto u) -> lds_u8* {
    constexpr int i = decltype(u)::value % R;
    if constexpr (i == 0) return (lds_u8*)vbuf0_raw;
    else if constexpr (i == 1) return (lds_u8*)vbuf1_raw;
    else if constexpr (i == 2) return (lds_u8*)vbuf2_raw;
    else return (lds_u8*)vbuf3_raw;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  int bh, qt;
  decode_tile<CAUSAL>(xcd_logical_index(blockIdx.x, nq * bh_total), nq, bh_total,
                      group_heads, bh, qt);

  const size_t qhead = (size_t)bh * (size_t)Sq * D;  // q and o of this head
  const size_t khead = (size_t)bh * (size_t)Sk * D;  // k and v of this head
  const uint16_t* Qh = Q + qhead;
  const uint16_t* Kh = K + khead;
  const uint16_t* Vh = V + khead;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;   // column of the 32x32 accumulator = query
  const int hh = lane >> 5;  // lane half
  const int q0 = qt * C::BR;
  const int qw0 = q0 + wave * kRowsPerWave;
  const int my_q = qw0 + m;

  // Key tiles this workgroup visits, and how many of them this wave needs.
  // The queries are the last Sq positions of the Sk keys' sequence: with the
  // causal mask, query row i sees keys j <= i + kshift (bottom-right
  // alignment; kshift = 0 for self-attention).  Rows before the first key see
  // nothing (possible when Sq > Sk).  Every row that sees a key sees key 0.
  const int kshift = Sk - Sq;
  const int kend = CAUSAL ? max(0, min(Sk, q0 + C::BR + kshift)) : Sk;
  const int ntiles = (kend + BC - 1) / BC;
  const int wave_klast = CAUSAL ? min(qw0 + kRowsPerWave - 1 + kshift, Sk - 1) : (Sk - 1);
  const int wave_ntiles = (qw0 < Sq && wave_klast >= 0) ? min(ntiles, wave_klast / BC + 1) : 0;

  // Copy waves: the first COPY_WAVES waves (all of a 4-wave workgroup; waves
  // 0..3, one per SIMD, of an 8-wave one).  Those are the older wave of each
  // SIMD pair, which the matrix core serves first.
  const bool copier = wave < C::COPY_WAVES;
  const int cw = copier ? wave : 0;  // this wave's share of each copy
  const CopyLanes cl = copy_lanes<C>(cw, lane);

  // With prefetch: K(0) .. K(R-1) and V(0) .. V(R-3) now; step t copies
  // K(t+R) and V(t+R-2) (so K(t+2) and V(t) with two buffers).  Without:
  // K(0) now; step t copies K(t+1) and V(t-1).
  const auto copy_k = [&](int u, lds_u8* dst) { copy_tile<C, false>(Kh, dst, u * BC, Sk, cw, lane, cl); };
  const auto copy_v = [&](int u, lds_u8* dst) { copy_tile<C, true>(Vh, dst, u * BC, Sk, cw, lane, cl); };
  if constexpr (PIPE == kPipeKSplit) {
    if (copier && ntiles > 0) {
      copy_k_plane<C>(Kh, kslot(I0{}), 0, Sk, cw, lane, 0);
      copy_k_plane<C>(Kh, kslot(I0{}), 0, Sk, cw, lane, 1);
    }
  } else if constexpr (PC::kCopies) {
    if (copier && ntiles > 0) {
      copy_k(0, kslot(I0{}));
      if constexpr (PC::kPrefetch) {
        if (ntiles > 1) copy_k(1, kslot(I1{}));
        if constexpr (R > 2) {
          if (ntiles > 2) copy_k(2, kslot(I2{}));
          copy_v(0, vslot(I0{}));
        }
        if constexpr (R > 3) {
          if (ntiles > 3) copy_k(3, kslot(I3{}));
          if (ntiles > 1) copy_v(1, vslot(I1{}));
        }
      }
    }
  }

  // Q fragments (B operand of S^T = K * Q^T): lane holds Q[my_q][ch*16 + hh*8 .. +8].
  bf16x8 qf[C::KCH];
#pragma unroll
  for (int ch = 0; ch < C::KCH; ++ch) {
    u32x4 raw = u32x4{0u, 0u, 0u, 0u};
    if (my_q < Sq) raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)my_q * D + ch * 16 + hh * 8);
    qf[ch] = __builtin_bit_cast(bf16x8, raw ^ qflip);
  }

  // Per-lane byte offsets of the operand reads inside a buffer.
  // K (A operand of S^T): row perm(m), logical chunk 2*ch + hh; chunk bits
  // above the swizzle go into the immediate offset.
  const int pm = key_perm(m);
  const int ksw = kswz<C>(pm);
  int k_off[C::NKOFF];
#pragma unroll
  for (int b = 0; b < C::NKOFF; ++b) k_off[b] = pm * C::ROW_BYTES + (((2 * b + hh) ^ ksw) << 4);
  // V (A operand of O^T, via the transposing read): inside each 16-lane group,
  // source lane 4j+t points at V[key base + hh*8 + j][d base + 16*(g&1) + 4t],
  // i.e. logical chunk 4*db + 2*(g&1) + t/2 of row (hh*8 + j) + 16*pc (+ 4).
  const int g = lane >> 4, j4 = (lane >> 2) & 3, t4 = lane & 3;
  const int vx = 2 * (g & 1) + (t4 >> 1);
  const int vsw = vswz<C>(hh * 8 + j4);  // same for the +4 and +16*pc rows
  const int v_row = (hh * 8 + j4) * C::ROW_BYTES + (t4 & 1) * 8;
  int v_off[C::NVOFF];
#pragma unroll
  for (int d4 = 0; d4 < C::NVOFF; ++d4) v_off[d4] = v_row + (((4 * d4 + vx) ^ vsw) << 4);

  // Row sums of the bf16 weights on the matrix cores: one 16x16x32 product per
  // 16-key chunk with the weights' B operand as it stands and a 0/1 A operand
  // that picks, for output rows 0-3 and 8-11, the chunk's keys of query n and,
  // for rows 4-7 and 12-15, those of query n + 16.  Then every accumulator
  // register of lane l holds the sum for query l % 32 (both lane halves).
  bf16x8 sel;
  {
    const __bf16 one = (__bf16)((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 1.0f : 0.0f);
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = one;
  }

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  f32x4 l_mfma = f32x4{};   // sum of bf16(p) on the matrix cores (MFMA_SUM)
  float l_round = 0.0f;     // this lane's share of sum(bf16(p)) (otherwise)
  float m_run = -INFINITY;  // reference max of the raw (unscaled) scores
  float l_exact = 0.0f;     // this lane's share of sum(p) with float32 weights
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pf[C::PCH];        // bf16 weights of the tile whose P*V is pending

  const auto needs_mask = [&](int k0) {
    return (CAUSAL && (k0 + BC - 1 > qw0 + kshift)) || (k0 + BC > Sk);
  };
  const auto apply_mask = [&](f32x16 (&s)[C::KB], int k0) {
    const int lim = (CAUSAL ? min(my_q + kshift, Sk - 1) : (Sk - 1)) - k0 - hh * 8;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + (r >> 3) * 16 + (r & 7);
        s[kb][r] = key > lim ? -INFINITY : s[kb][r];
      }
  };
  // Weights of 16-key chunk pc of a tile (this lane's 8 keys): bf16 B operand.
  const auto weights = [&](const f32x16 (&s)[C::KB], int pc, float mc, float& rs) {
    bf16x8 w;
    // two scores at a time, so that no exponential is followed at once by
    // its use
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float p0, p1;
      if constexpr (PC::kSoftmax) {
        const float x0 = fmaf(s[pc >> 1][(pc & 1) * 8 + e], c, -mc);
        const float x1 = fmaf(s[pc >> 1][(pc & 1) * 8 + e + 1], c, -mc);
        p0 = fast_exp2(x0);
        p1 = fast_exp2(x1);
      } else {
        p0 = s[pc >> 1][(pc & 1) * 8 + e];
        p1 = s[pc >> 1][(pc & 1) * 8 + e + 1];
      }
      rs += p0;
      rs += p1;
      w[e] = (__bf16)p0;
      w[e + 1] = (__bf16)p1;
    }
    return w;
  };
  // A row that has seen no key keeps m_run = -inf; its weights are
  // exp2(-inf - 0) = 0.
  const auto ref_mc = [&]() { return m_run == -INFINITY ? 0.0f : m_run * c; };
  // Sums of the bf16 weights of a tile (before its P*V, i.e. after its check).
  const auto weight_sums = [&]() {
    if constexpr (MFMA_SUM) {
#pragma unroll
      for (int pc = 0; pc < C::PCH; ++pc)
        l_mfma = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pf[pc], l_mfma, 0, 0, 0);
    } else {
#pragma unroll
      for (int pc = 0; pc < C::PCH; ++pc)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x2 two = {pf[pc][2 * t], pf[pc][2 * t + 1]};
          l_round = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l_round, false);
        }
    }
  };
  const auto pv_chunk = [&](const lds_u8* v_cur, int pc) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const lds_u8* p = v_cur + pc * 16 * C::ROW_BYTES + (db / C::NVOFF) * 256 +
                        v_off[db % C::NVOFF];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
      const s16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * C::ROW_BYTES));
      const bf16x8 vf =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[pc], acc[db], 0, 0, 0);
    }
  };
  // The rare path: some weight of tile s (masked, with the reference mc) was
  // above the limit.  Raise the reference to the row max seen so far, rescale
  // what was accumulated (tiles up to the previous one), and form the tile's
  // weights again.
  const auto raise_reference = [&](const f32x16 (&s)[C::KB], float& rs) {
    // (The weights formed before are replaced; this use keeps their
    // computation where the instruction order put it.)
#pragma unroll
    for (int pc = 0; pc < C::PCH; ++pc) asm volatile("" ::"v"(pf[pc]));
    const float mt = row_max<C>(s, hh);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = m_new == m_run ? 1.0f : fast_exp2((m_run - m_new) * c);
    m_run = m_new;
    l_exact *= alpha;
    l_round *= alpha;
    l_mfma *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
    const float mc = ref_mc();
    rs = 0.0f;
#pragma unroll
    for (int pc = 0; pc < C::PCH; ++pc) pf[pc] = weights(s, pc, mc, rs);
  };

  // Planar K (kPipeKSplit): the lane's chunk of products ch and ch + 4 (dims
  // 16 ch + 8 hh .. +8 in planes 0 and 1) for ch = 0..3.
  int kp_off[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) kp_off[b] = pm * 128 + (((2 * b + hh) ^ planar_kswz(pm)) << 4);
  // products over dims [64 h, 64 h + 64) of S(tile in ks) into s (the first
  // half starts the accumulation)
  const auto qk_half = [&](f32x16 (&s)[C::KB], const lds_u8* ks, auto half_tag) {
    constexpr int h = decltype(half_tag)::value;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bf16x8 kf = *(const lds_bf16x8*)(ks + h * 8192 + kb * 4096 + kp_off[b]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[4 * h + b],
                                                        h == 0 && b == 0 ? f32x16{} : s[kb], 0, 0, 0);
      }
  };

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // S tiles in two named buffers used alternately (no copy between tiles).
  f32x16 s_a[C::KB], s_b[C::KB];
  if (wave_ntiles > 0) {
    // S(0) and the reference max from it: every row that sees any key sees
    // key 0, so only rows that see nothing keep -inf.
    if constexpr (PIPE == kPipeKSplit) {
      qk_half(s_a, kslot(I0{}), I0{});
      qk_half(s_a, kslot(I0{}), I1{});
    } else {
      qk_tile<C>(s_a, kslot(I0{}), qf, k_off);
    }
    if (needs_mask(0)) apply_mask(s_a, 0);
    m_run = row_max<C>(s_a, hh);
  }
  __syncthreads();  // every wave is done with K(0) before a copy overwrites it

  // Step t: reads K(t+1) from k_next and V(t-1) from v_prev, and copies
  // tiles as the pipeline mode says.  S(t) is in s_in; S(t+1) goes to s_out.
  // Three kinds of step:
  //  kFirst (t = 0):    weights of tile 0, S(1) if the wave needs tile 1;
  //  kFull  (1 <= t, t + 1 < wave_ntiles): P*V of t-1, weights of t, S(t+1),
  //                     under a fixed instruction order;
  //  kTail  (the wave's last steps): P*V of t-1 if the wave has it, weights
  //                     of t if the wave has tile t, no S.
  // Every path gives the weights and S buffers defined values, so that their
  // previous contents are not kept alive across a step.  The step's position
  // in a group of U steps (PH = t mod U) names its buffers.
  const auto pick = [](auto first_tag, auto& a, auto& b) -> auto& {
    if constexpr (decltype(first_tag)::value) return a;
    else return b;
  };
  if constexpr (PIPE == kPipeKSplit) {
    // Step t: copy V(t-1), then K(t+1) in its two head-dim planes; wait for V
    // and the first plane; P*V of t-1, the weights of t and the products of
    // S(t+1) over dims 0-63; wait for the second plane; the products over
    // dims 64-127.  (Unpinned code: a study of the copy split, not of the
    // schedule.)
    const auto ks_step = [&](auto ph_tag, const int t) {
      constexpr int PH = decltype(ph_tag)::value;
      lds_u8* k_next = kslot(std::integral_constant<int, PH + 1>{});
      const lds_u8* v_prev = vslot(std::integral_constant<int, PH + 1>{});
      const std::integral_constant<bool, PH % 2 == 0> even{};
      f32x16(&s_in)[C::KB] = pick(even, s_a, s_b);
      f32x16(&s_out)[C::KB] = pick(even, s_b, s_a);
      const bool k_copy = t + 1 < ntiles;
      if (copier) {
        if (t >= 1 && t - 1 < ntiles) copy_v(t - 1, vslot(std::integral_constant<int, PH + 1>{}));
        if (k_copy) {
          copy_k_plane<C>(Kh, k_next, (t + 1) * BC, Sk, cw, lane, 0);
          copy_k_plane<C>(Kh, k_next, (t + 1) * BC, Sk, cw, lane, 1);
        }
      }
      // V and plane 0 have landed, for every wave (plane 1 may be in flight)
      if (k_copy) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8 / C::COPY_WAVES));
      else __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const bool do_sm = t < wave_ntiles;
      if (t >= 1 && do_sm && needs_mask(t * BC)) apply_mask(s_in, t * BC);
      const float mc = ref_mc();
      float rs = 0.0f;
      if (t >= 1 && t - 1 < wave_ntiles) {
        weight_sums();
#pragma unroll
        for (int pc = 0; pc < C::PCH; ++pc) pv_chunk(v_prev, pc);
      }
#pragma unroll
      for (int pc = 0; pc < C::PCH; ++pc) pf[pc] = do_sm ? weights(s_in, pc, mc, rs) : bf16x8{};
      const bool s_next = t + 1 < wave_ntiles;
      if (s_next) qk_half(s_out, k_next, I0{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (s_next) {
        qk_half(s_out, k_next, I1{});
      } else {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) s_out[kb] = f32x16{};
      }
      if (do_sm) {
        if (__any(!(rs <= kRowSumLimit))) raise_reference(s_in, rs);
        l_exact += rs;
      }
    };
    int t = 0;
    for (; t + 1 <= ntiles; t += 2) {
      ks_step(I0{}, t);
      ks_step(I1{}, t + 1);
    }
    if (t <= ntiles) ks_step(I0{}, t);
  } else {
  constexpr int kFirst = 0, kFull = 1, kTail = 2;
  auto step = [&](auto kind_tag, auto ph_tag, const int t) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr int PH = decltype(ph_tag)::value;
    const lds_u8* k_next = kslot(std::integral_constant<int, PH + 1>{});
    const lds_u8* v_prev = vslot(std::integral_constant<int, PH + U - 1>{});
    // (chosen at compile time, so that both stay in registers)
    const std::integral_constant<bool, PH % 2 == 0> even{};
    f32x16(&s_in)[C::KB] = pick(even, s_a, s_b);
    f32x16(&s_out)[C::KB] = pick(even, s_b, s_a);
    if constexpr (PC::kCopies) {
      if constexpr (PC::kPrefetch) {
        if (copier) {
          if constexpr (R == 2) {
            if (t + 2 < ntiles) copy_k(t + 2, kslot(std::integral_constant<int, PH>{}));
            if (t < ntiles) copy_v(t, vslot(std::integral_constant<int, PH>{}));
          } else if (ntiles > 0) {
            // a fixed number of copies per step (the step-end wait counts
            // them): past the last tile the last tile is copied again, into
            // a buffer that no later step reads
            copy_k(min(t + R, ntiles - 1), kslot(std::integral_constant<int, PH>{}));
            copy_v(min(t + R - 2, ntiles - 1), vslot(std::integral_constant<int, PH + U - 2>{}));
          }
        }
      } else {
        if (copier) {
          if (t + 1 < ntiles) copy_k(t + 1, kslot(std::integral_constant<int, PH + 1>{}));
          if (t >= 1 && t - 1 < ntiles) copy_v(t - 1, vslot(std::integral_constant<int, PH + U - 1>{}));
        }
        // the tiles this step reads have landed, for every wave
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
    const bool do_sm = KIND == kFull || t < wave_ntiles;
    if (KIND != kFirst && do_sm && needs_mask(t * BC)) apply_mask(s_in, t * BC);
    const float mc = ref_mc();
    float rs = 0.0f;
    if constexpr (KIND == kFull) {
      // Operand reads in the order they are issued: each pair of products
      // has its second product's reads first, so that the wait for the first
      // product's operands covers the second's as well.
      bf16x8 vf[C::PCH * C::DB], kf[C::KB * C::KCH];
#pragma unroll
      for (int f = 0; f < C::PCH * C::DB; ++f) {
        const int g = f ^ 1;
        const lds_u8* p = v_prev + (g / C::DB) * 16 * C::ROW_BYTES +
                          ((g % C::DB) / C::NVOFF) * 256 + v_off[(g % C::DB) % C::NVOFF];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * C::ROW_BYTES));
        vf[g] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int f = 0; f < C::KB * C::KCH; ++f) {
        const int g = f ^ 1;
        const int kb = g % C::KB, ch = g / C::KB;
        kf[g] = *(const lds_bf16x8*)(k_next + kb * 32 * C::ROW_BYTES + (ch / C::NKOFF) * 256 +
                                      k_off[ch % C::NKOFF]);
      }
      weight_sums();
#pragma unroll
      for (int f = 0; f < C::PCH * C::DB; ++f)
        acc[f % C::DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f], pf[f / C::DB],
                                                                 acc[f % C::DB], 0, 0, 0);
#pragma unroll
      for (int pc = 0; pc < C::PCH; ++pc) pf[pc] = weights(s_in, pc, mc, rs);
#pragma unroll
      for (int f = 0; f < C::KB * C::KCH; ++f) {
        const int kb = f % C::KB, ch = f / C::KB;
        s_out[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[f], qf[ch],
                                                            ch == 0 ? f32x16{} : s_out[kb], 0, 0, 0);
      }
      // Instruction order: the bf16-weight sums, then P(t-1)*V(t-1) chunk by
      // chunk (two transposing reads per product), then S(t+1) (one read per
      // product; the key blocks alternate, so consecutive products share
      // their Q fragment: +0.3-0.6 %, same results); operand reads run three
      // products ahead; the vector work of tile t is spread evenly over the
      // products.
      step_schedule<C, MFMA_SUM>(std::make_integer_sequence<int, (MFMA_SUM ? C::PCH : 0) +
                                                                 C::DB * C::PCH + C::KB * C::KCH>{});
    } else {
      if (KIND == kTail && t - 1 < wave_ntiles) {
        weight_sums();
#pragma unroll
        for (int pc = 0; pc < C::PCH; ++pc) pv_chunk(v_prev, pc);
      }
      if (do_sm) {
#pragma unroll
        for (int pc = 0; pc < C::PCH; ++pc) pf[pc] = weights(s_in, pc, mc, rs);
      } else {
#pragma unroll
        for (int pc = 0; pc < C::PCH; ++pc) pf[pc] = bf16x8{};
      }
      if (KIND == kFirst && t + 1 < wave_ntiles) {
        qk_tile<C>(s_out, k_next, qf, k_off);
      } else {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) s_out[kb] = f32x16{};
      }
    }
    if constexpr (PC::kSoftmax) {
      if (do_sm) {
        // The reference moves only if some weight of this tile is too large
        // (or not finite); for a row that sees no key all weights are 0.
        if (__any(!(rs <= kRowSumLimit))) raise_reference(s_in, rs);
        l_exact += rs;
      }
    }
    if constexpr (PC::kPrefetch) {
      // With R buffers the copies of the last R - 2 steps may stay in flight
      // (the steps after the next one read them); the others have landed.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(PC::kCopies ? (R - 2) * 2 * C::LOADS_PER_WAVE : 0));
      __syncthreads();
    }
  };
  const std::integral_constant<int, kFirst> first{};
  const std::integral_constant<int, kFull> full{};
  const std::integral_constant<int, kTail> tail{};
  // Steps 0 .. ntiles (the last one only finishes P*V of the last tile).  The
  // full steps run in groups of U (static buffers and S parity); the wave's
  // remaining full steps and its last steps follow.  Every wave takes
  // ntiles + 1 steps (barriers).
  step(first, I0{}, 0);
  int t = 1;
  const int t_tail = max(1, wave_ntiles - 1);  // first step that is not full
  for (; t + U <= t_tail; t += U) {
    step(full, I1{}, t);
    step(full, std::integral_constant<int, 2 % U>{}, t + 1);
    if constexpr (U > 2) {
      step(full, std::integral_constant<int, 3 % U>{}, t + 2);
      step(full, std::integral_constant<int, 4 % U>{}, t + 3);
    }
    if constexpr (U > 4) {
      step(full, std::integral_constant<int, 5 % U>{}, t + 4);
      step(full, std::integral_constant<int, 6 % U>{}, t + 5);
    }
  }
  if constexpr (U == 2) {
    // at most one full step left (t is odd here); tail steps in pairs
    if (t < t_tail) {
      step(full, I1{}, t);
      ++t;
    }
    if (!(t & 1) && t <= ntiles) {
      step(tail, I0{}, t);
      ++t;
    }
    for (; t + 1 <= ntiles; t += 2) {
      step(tail, I1{}, t);
      step(tail, I0{}, t + 1);
    }
    if (t <= ntiles) step(tail, I1{}, t);
  } else {
    // t = 1 (mod U) here: the remaining full steps (fewer than U) keep static
    // buffers; then S(t) is moved to s_a and the wave's last steps (no S,
    // buffers chosen at run time; they are few) follow.
    const auto one_full = [&](auto ph_tag) -> bool {
      if (t >= t_tail) return false;
      step(full, ph_tag, t);
      ++t;
      return true;
    };
    if constexpr (U == 4) {
      (void)(one_full(I1{}) && one_full(I2{}) && one_full(I3{}));
    } else {
      (void)(one_full(I1{}) && one_full(I2{}) && one_full(I3{}) &&
             one_full(std::integral_constant<int, 4>{}) && one_full(std::integral_constant<int, 5>{}));
    }
    if (t & 1) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) s_a[kb] = s_b[kb];
    }
    const auto kslot_rt = [&](int i) -> lds_u8* {
      return i == 0 ? (lds_u8*)kbuf0_raw : i == 1 ? (lds_u8*)kbuf1_raw
             : i == 2 ? (lds_u8*)kbuf2_raw : (lds_u8*)kbuf3_raw;
    };
    const auto vslot_rt = [&](int i) -> lds_u8* {
      return i == 0 ? (lds_u8*)vbuf0_raw : i == 1 ? (lds_u8*)vbuf1_raw
             : i == 2 ? (lds_u8*)vbuf2_raw : (lds_u8*)vbuf3_raw;
    };
    for (; t <= ntiles; ++t) {
      if (copier && ntiles > 0) {
        copy_k(min(t + R, ntiles - 1), kslot_rt(t % R));
        copy_v(min(t + R - 2, ntiles - 1), vslot_rt((t + R - 2) % R));
      }
      const bool do_sm = t < wave_ntiles;
      if (do_sm && needs_mask(t * BC)) apply_mask(s_a, t * BC);
      const float mc = ref_mc();
      float rs = 0.0f;
      if (t - 1 < wave_ntiles) {
        weight_sums();
        const lds_u8* v_prev = vslot_rt((t - 1) % R);
#pragma unroll
        for (int pc = 0; pc < C::PCH; ++pc) pv_chunk(v_prev, pc);
      }
      if (do_sm) {
#pragma unroll
        for (int pc = 0; pc < C::PCH; ++pc) pf[pc] = weights(s_a, pc, mc, rs);
        if (__any(!(rs <= kRowSumLimit))) raise_reference(s_a, rs);
        l_exact += rs;
      } else {
#pragma unroll
        for (int pc = 0; pc < C::PCH; ++pc) pf[pc] = bf16x8{};
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((R - 2) * 2 * C::LOADS_PER_WAVE));
      __syncthreads();
    }
    // no copy into this workgroup's LDS is still in flight when it ends
    __builtin_amdgcn_s_waitcnt(0);
  }

  }  // pipeline modes

  const float le = l_exact + swap_halves(l_exact, hh);
  const float lr = MFMA_SUM ? l_mfma[0] : l_round + swap_halves(l_round, hh);
  if (my_q >= Sq) return;
  // O is normalised by the sum of the bf16 weights that multiplied V, so the
  // weights applied to V sum to one exactly (up to float32 rounding); the
  // log-sum-exp uses the float32 weights.
  const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
  uint16_t* Orow = O + qhead + (size_t)my_q * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      // registers gq*4 .. gq*4+3 hold head-dim entries db*32 + gq*8 + hh*4 + 0..3
      u32x2 pk;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const __bf16 lo = (__bf16)(acc[db][gq * 4 + 2 * tt] * inv);
        const __bf16 hi = (__bf16)(acc[db][gq * 4 + 2 * tt + 1] * inv);
        pk[tt] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<u32x2*>(Orow + db * 32 + gq * 8 + hh * 4) = pk;
    }
  // A row that saw no key keeps m_run = -inf and le = 0: O = 0, LSE = -inf.
  if (hh == 0) LSE[(size_t)bh * Sq + my_q] = (m_run * c + fast_log2(le)) * kLn2;
}

// Byte offsets (per lane) of the copies of the tile starting at key k0: in
// the last (partial) tile, rows past the sequence end are clamped to the last
// row (finite data whose keys are masked).
template <class C>
__device__ __forceinline__ void tile_src(const uint16_t* __restrict__ head_src, int k0, int S,
                                         const int* off, const int* row, const char*& base,
                                         int* boff) {
  const uint64_t b64 = (uint64_t)(head_src + (size_t)k0 * C::D);
  const uint32_t b_lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t b_hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  base = (const char*)(((uint64_t)b_hi << 32) | b_lo);
  if (k0 + C::BC <= S) {
#pragma unroll
    for (int u = 0; u < C::LOADS_PER_WAVE; ++u) boff[u] = off[u] * 2;
  } else {
#pragma unroll
    for (int u = 0; u < C::LOADS_PER_WAVE; ++u)
      boff[u] = (off[u] - (row[u] - min(row[u], S - 1 - k0)) * C::D) * 2;
  }
}

// One 1 KiB piece (16 bytes per lane) of a tile copy into LDS.
__device__ __forceinline__ void copy_piece(const char* base, int boff, lds_u8* dst) {
  lds_dma<16>(base, (uint32_t)boff, dst);
}

// A workgroup barrier that waits for nothing by itself (copies in flight stay
// in flight); no instruction moves across it.
__device__ __forceinline__ void plain_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ----------------------------------------------------------------------------
// bf16 kernel with a four-deep K/V ring (D = 256, one wave per SIMD; the
// ring256 study build runs it in place of the wave-pair kernel below)
// ----------------------------------------------------------------------------
// At D = 256 a wave needs the whole register file, so each SIMD runs a single
// wave and nothing hides the start-of-tile copy issue or the wait for copies.
// This variant keeps four K and four V buffers, issues each tile's copies in
// the middle of the matrix-core work two tiles ahead of use, and at the end of
// a tile waits only for the copies of the previous tile.  Same arithmetic,
// tiling and masking as fa_fwd_bf16_kernel.  The softmax sets each row's
// reference max from tile 0 and raises it only when a tile's max exceeds it
// by more than kRescaleThreshold powers of two; that check comes first in a
// tile, and the rescale runs between two stretches of tile steps (see the
// loop below), not inside them.
template <int D, int BC, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(64 * WAVES, D <= 128 ? 2 : 1) void fa_fwd_bf16_ring_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Sq, int Sk, int nq, int bh_total, int group_heads, float c) {
  using C = BfCfg<D, BC, WAVES>;
  // negative scale: S from -Q with |c| (see kZeroScaleC)
  const uint32_t qflip = sign_flip_mask(c);
  c = fabsf(c);
  // Every wave copies its share (wave w fills bytes [w, w+1) * NL KiB of a
  // buffer): the copy split must cover exactly the waves of the workgroup.
  static_assert(C::COPY_WAVES == WAVES, "ring kernel: every wave issues tile copies");
  constexpr int NL = C::LOADS_PER_WAVE;  // copy pieces per tensor per wave
  // Rings of four K and four V buffers, each a separate array so that every
  // access names its buffer statically.  Step j reads K(j+1) and V(j) and
  // copies K(j+3) and V(j+2), each into the buffer whose last reader was step
  // j-2; the copies of step j are waited for at the end of step j+1.
  __shared__ __attribute__((aligned(1024))) uint8_t kb0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb2_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb3_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb2_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb3_raw[C::TILE_BYTES];
  lds_u8* kb0 = (lds_u8*)kb0_raw;
  lds_u8* kb1 = (lds_u8*)kb1_raw;
  lds_u8* kb2 = (lds_u8*)kb2_raw;
  lds_u8* kb3 = (lds_u8*)kb3_raw;
  lds_u8* vb0 = (lds_u8*)vb0_raw;
  lds_u8* vb1 = (lds_u8*)vb1_raw;
  lds_u8* vb2 = (lds_u8*)vb2_raw;
  lds_u8* vb3 = (lds_u8*)vb3_raw;

  int bh, qt;
  decode_tile<CAUSAL>(xcd_logical_index(blockIdx.x, nq * bh_total), nq, bh_total,
                      group_heads, bh, qt);

  const size_t qhead = (size_t)bh * (size_t)Sq * D;  // q and o of this head
  const size_t khead = (size_t)bh * (size_t)Sk * D;  // k and v of this head
  const uint16_t* Qh = Q + qhead;
  const uint16_t* Kh = K + khead;
  const uint16_t* Vh = V + khead;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * C::BR;
  const int qw0 = q0 + wave * kRowsPerWave;
  const int my_q = qw0 + m;

  // The queries are the last Sq positions of the Sk keys' sequence: with the
  // causal mask, query row i sees keys j <= i + kshift (bottom-right
  // alignment; kshift = 0 for self-attention).  Rows before the first key see
  // nothing (possible when Sq > Sk).
  const int kshift = Sk - Sq;
  const int kend = CAUSAL ? max(0, min(Sk, q0 + C::BR + kshift)) : Sk;
  const int ntiles = (kend + BC - 1) / BC;
  const int wave_klast = CAUSAL ? min(qw0 + kRowsPerWave - 1 + kshift, Sk - 1) : (Sk - 1);
  const int wave_ntiles = (qw0 < Sq && wave_klast >= 0) ? min(ntiles, wave_klast / BC + 1) : 0;

  int koff[NL], krow[NL], voff[NL], vrow[NL];
  tile_offsets<C, false>(koff, krow, wave, lane);
  tile_offsets<C, true>(voff, vrow, wave, lane);
  const int wslot = wave * (NL * 1024);  // this wave's share of a buffer

  // Prologue copies: K(0..2), V(0..1) (tiles past the end: the last tile).
  if (ntiles > 0) {
    const char* b;
    int bo[NL];
    lds_u8* kdst[3] = {kb0, kb1, kb2};
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      tile_src<C>(Kh, min(t, ntiles - 1) * BC, Sk, koff, krow, b, bo);
#pragma unroll
      for (int u = 0; u < NL; ++u) copy_piece(b, bo[u], kdst[t] + wslot + u * 1024);
    }
    lds_u8* vdst[2] = {vb0, vb1};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      tile_src<C>(Vh, min(t, ntiles - 1) * BC, Sk, voff, vrow, b, bo);
#pragma unroll
      for (int u = 0; u < NL; ++u) copy_piece(b, bo[u], vdst[t] + wslot + u * 1024);
    }
  }

  bf16x8 qf[C::KCH];
#pragma unroll
  for (int ch = 0; ch < C::KCH; ++ch) {
    u32x4 raw = u32x4{0u, 0u, 0u, 0u};
    if (my_q < Sq) raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)my_q * D + ch * 16 + hh * 8);
    qf[ch] = __builtin_bit_cast(bf16x8, raw ^ qflip);
  }

  const int pm = key_perm(m);
  const int ksw = kswz<C>(pm);
  int k_off[C::NKOFF];
#pragma unroll
  for (int b = 0; b < C::NKOFF; ++b) k_off[b] = pm * C::ROW_BYTES + (((2 * b + hh) ^ ksw) << 4);
  const int g = lane >> 4, j4 = (lane >> 2) & 3, t4 = lane & 3;
  const int vx = 2 * (g & 1) + (t4 >> 1);
  const int vsw = vswz<C>(hh * 8 + j4);
  const int v_row = (hh * 8 + j4) * C::ROW_BYTES + (t4 & 1) * 8;
  int v_off[C::NVOFF];
#pragma unroll
  for (int d4 = 0; d4 < C::NVOFF; ++d4) v_off[d4] = v_row + (((4 * d4 + vx) ^ vsw) << 4);

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_exact = 0.0f;
  float l_round0 = 0.0f, l_round1 = 0.0f;  // two chains of the bf16-weight sum
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 s_a[C::KB], s_b[C::KB];
  float mt_a = 0.0f, mt_b = 0.0f;
  // S(0) and the reference max from it (masked): every row that sees any key
  // sees key 0, so only rows that see nothing keep -inf.
  const auto mask_tile = [&](f32x16 (&s)[C::KB], int k0) {
    const int lim = (CAUSAL ? min(my_q + kshift, Sk - 1) : (Sk - 1)) - k0 - hh * 8;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + (r >> 3) * 16 + (r & 7);
        s[kb][r] = key > lim ? -INFINITY : s[kb][r];
      }
  };
  if (wave_ntiles > 0) {
    qk_tile<C>(s_a, kb0, qf, k_off);
    if ((CAUSAL && (BC - 1 > qw0 + kshift)) || (BC > Sk)) mask_tile(s_a, 0);
    mt_a = row_max<C>(s_a, hh);
    m_run = mt_a;
  }

  // Step j.  When the row's reference max has to move for tile j, the step
  // leaves at once, having done nothing but mask S(j), with the tile's max in
  // mt_move, and returns false; the caller rescales and runs step j again.
  // (The rescale sits outside the loops of steps: inside them the compiler
  // would keep a copy of the O accumulator in the vector registers at every
  // step.)
  float mt_move = 0.0f;
  auto step = [&](const int j, const lds_u8* k_next, lds_u8* k_load, const lds_u8* v_cur,
                  lds_u8* v_load, f32x16 (&s_in)[C::KB], f32x16 (&s_out)[C::KB], float& mt_in,
                  float& mt_out) -> bool {
    // Sources of this step's copies (a valid tile even past the end, so that
    // every step issues the same number of copies).
    const char* kbase;
    const char* vbase;
    int kbo[NL], vbo[NL];
    tile_src<C>(Kh, min(j + 3, ntiles - 1) * BC, Sk, koff, krow, kbase, kbo);
    tile_src<C>(Vh, min(j + 2, ntiles - 1) * BC, Sk, voff, vrow, vbase, vbo);
    lds_u8* kdst = k_load + wslot;
    lds_u8* vdst = v_load + wslot;
    if (j < wave_ntiles) {
      const int k0 = j * BC;
      float mt = mt_in;
      if ((CAUSAL && (k0 + BC - 1 > qw0 + kshift)) || (k0 + BC > Sk)) {
        mask_tile(s_in, k0);
        mt = row_max<C>(s_in, hh);
      }
      if (__any((mt - m_run) * c > kRescaleThreshold)) {
        mt_move = mt;
        return false;
      }
      const float mc = m_run == -INFINITY ? 0.0f : m_run * c;

      qk_tile<C>(s_out, k_next, qf, k_off);

      float rs = 0.0f;
      bf16x8 pf[C::PCH];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s_in[kb][r], c, -mc));
          rs += p;
          pf[2 * kb + (r >> 3)][r & 7] = (__bf16)p;
        }

#pragma unroll
      for (int u = 0; u < NL; ++u) copy_piece(kbase, kbo[u], kdst + u * 1024);
#pragma unroll
      for (int u = 0; u < NL; ++u) copy_piece(vbase, vbo[u], vdst + u * 1024);

#pragma unroll
      for (int pc = 0; pc < C::PCH; ++pc)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const lds_u8* p = v_cur + pc * 16 * C::ROW_BYTES + (db / C::NVOFF) * 256 +
                            v_off[db % C::NVOFF];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * C::ROW_BYTES));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[pc], acc[db], 0, 0, 0);
        }
      l_exact += rs;
#pragma unroll
      for (int pc = 0; pc < C::PCH; ++pc)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x2 two = {pf[pc][2 * t], pf[pc][2 * t + 1]};
          if (pc & 1) l_round1 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l_round1, false);
          else l_round0 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l_round0, false);
        }
      mt_out = row_max<C>(s_out, hh);

      // Instruction order: each MFMA is followed by its share of the vector
      // work and of the operand reads (kLead MFMAs ahead); the copies spread
      // over the region, one every 32 / (2 * NL) MFMAs.
      constexpr int kLead = 3;
      constexpr int kNM = C::KB * C::KCH + C::DB * C::PCH;  // MFMAs in the region
      constexpr int kEvery = kNM / (2 * NL);
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
      for (int i = 0; i < C::KB * C::KCH; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        if (i % kEvery == kEvery / 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLead, 0);
#pragma unroll
      for (int i = 0; i < C::DB * C::PCH; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        if (i % kEvery == kEvery / 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NL; ++u) copy_piece(kbase, kbo[u], kdst + u * 1024);
#pragma unroll
      for (int u = 0; u < NL; ++u) copy_piece(vbase, vbo[u], vdst + u * 1024);
    }
    // The previous step's copies have landed (this step's stay in flight);
    // this wave's LDS reads are done.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * NL));
    plain_barrier();
    return true;
  };
  // Unrolled by four (ring position and S parity static); the remaining
  // tiles run after the loop so that the back edge always follows step 3.
  // Step j with the buffers of ring position j mod 4 (static, as is the S
  // parity, in each call below).
#define FA_RING_STEP(J, POS)                                                       \
  ((POS) == 0   ? step(J, kb1, kb3, vb0, vb2, s_a, s_b, mt_a, mt_b)               \
   : (POS) == 1 ? step(J, kb2, kb0, vb1, vb3, s_b, s_a, mt_b, mt_a)               \
   : (POS) == 2 ? step(J, kb3, kb1, vb2, vb0, s_a, s_b, mt_a, mt_b)               \
                : step(J, kb0, kb2, vb3, vb1, s_b, s_a, mt_b, mt_a))
  // Stretches of steps, each until the last tile or until step j needs a
  // higher reference (need: step j has not run), then the rescale.
  int j = 0;
  for (;;) {
    bool need = false;
    // up to the next multiple of four, then groups of four
    switch (j & 3) {
      case 1:
        if (j < ntiles) {
          if (!FA_RING_STEP(j, 1)) { need = true; break; }
          ++j;
        }
        [[fallthrough]];
      case 2:
        if (j < ntiles) {
          if (!FA_RING_STEP(j, 2)) { need = true; break; }
          ++j;
        }
        [[fallthrough]];
      case 3:
        if (j < ntiles) {
          if (!FA_RING_STEP(j, 3)) { need = true; break; }
          ++j;
        }
        [[fallthrough]];
      default:
        break;
    }
    if (!need) {
      for (; j < ntiles; j += 4) {
        if (!FA_RING_STEP(j, 0)) { need = true; break; }
        if (j + 1 < ntiles && !FA_RING_STEP(j + 1, 1)) { j += 1; need = true; break; }
        if (j + 2 < ntiles && !FA_RING_STEP(j + 2, 2)) { j += 2; need = true; break; }
        if (j + 3 < ntiles && !FA_RING_STEP(j + 3, 3)) { j += 3; need = true; break; }
      }
    }
    if (!need) break;
    // Raise the reference to the masked max of tile j and rescale what was
    // accumulated over tiles 0 .. j-1; step j then runs with it.
    const float m_new = fmaxf(m_run, mt_move);
    const float alpha = m_new == m_run ? 1.0f : fast_exp2((m_run - m_new) * c);
    m_run = m_new;
    l_exact *= alpha;
    l_round0 *= alpha;
    l_round1 *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
  }
#undef FA_RING_STEP
  __builtin_amdgcn_s_waitcnt(0);

  const float l_round = l_round0 + l_round1;
  const float lr = l_round + swap_halves(l_round, hh);
  const float le = l_exact + swap_halves(l_exact, hh);
  if (my_q >= Sq) return;
  const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
  uint16_t* Orow = O + qhead + (size_t)my_q * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 pk;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const __bf16 lo = (__bf16)(acc[db][gq * 4 + 2 * t] * inv);
        const __bf16 hi = (__bf16)(acc[db][gq * 4 + 2 * t + 1] * inv);
        pk[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<u32x2*>(Orow + db * 32 + gq * 8 + hh * 4) = pk;
    }
  // A row that saw no key keeps m_run = -inf and le = 0: O = 0, LSE = -inf.
  if (hh == 0) LSE[(size_t)bh * Sq + my_q] = (m_run * c + fast_log2(le)) * kLn2;
}

// ----------------------------------------------------------------------------
// bf16 kernel on wave pairs (D = 256)
// ----------------------------------------------------------------------------
// At D = 256 a wave that held a 32-row slice's whole state (Q, S, O) would
// need the full register file, one wave per SIMD, and could not hide its own
// latencies.  Here eight waves, two per SIMD, form four pairs; pair p owns
// query rows [32p, 32p + 32) of the workgroup's 128.  The S wave of a pair
// (waves 0-3) holds Q and forms the scores, the softmax weights and their
// float32 row sum (for the LSE); the O wave (waves 4-7, on the same SIMD as
// its S wave) holds O, accumulates it from the weights and V, keeps the
// bf16-weight row sum (the normalisation) and issues every K/V tile copy.
// Each does 16 of the 32 matrix-core products of a 32-key tile, so neither
// repeats work, and the S wave's exponentials overlap the O wave's products
// on the SIMD.  The weights P(t) of tile t (bf16, the B operand of the P.V
// product exactly as the S wave holds it) pass through LDS with the
// reference max they were taken against; the O wave rescales O (and its sum)
// when that reference moved.
//
// Step j (one workgroup barrier each): the S wave forms S(j+3) from K(j+3)
// and the weights P(j+2) of S(j+2); the O wave adds V(j) P(j), with P(j) in
// registers since step j-1, and reads P(j+1) for the next step, so that no
// LDS wait sits between the barrier and its first product.  It also issues
// the copies of K(j+5) and V(j+3), each waited for at the end of step j+1.
// K and V each have four LDS buffers.  Softmax: the reference max comes from
// tile 0 and is raised, to the row max seen so far, only when a lane's sum of
// a tile's weights exceeds kPairSumLimit (no weight above 2^24).
template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_fwd_bf16_pair_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int Sq, int Sk, int nq, int bh_total, int group_heads, float c) {
  using C = BfCfg<256, 32, 4>;  // tile geometry: 128 query rows, 32-key tiles
  constexpr int D = C::D, BC = C::BC;
  constexpr int NL = C::LOADS_PER_WAVE;  // copy pieces per tensor per O wave
  static_assert(C::BR == 4 * kRowsPerWave && C::COPY_WAVES == 4 && C::KB == 1 && C::PCH == 2,
                "pair kernel: four pairs of 32 rows, one 32-key block per tile");
  // negative scale: S from -Q with |c| (see kZeroScaleC)
  const uint32_t qflip = sign_flip_mask(c);
  c = fabsf(c);
  __shared__ __attribute__((aligned(1024))) uint8_t kb0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb2_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb3_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb2_raw[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb3_raw[C::TILE_BYTES];
  // P(t) of the four pairs for t even / odd: 2 KiB per pair, chunk pc of lane
  // l at pc * 1024 + 16 l (no bank conflict on either side).
  __shared__ __attribute__((aligned(1024))) uint8_t xp0_raw[4 * 2048];
  __shared__ __attribute__((aligned(1024))) uint8_t xp1_raw[4 * 2048];
  // the reference max of P(t) per row (t even / odd)
  __shared__ float xm0[C::BR], xm1[C::BR];
  lds_u8* kb0 = (lds_u8*)kb0_raw;
  lds_u8* kb1 = (lds_u8*)kb1_raw;
  lds_u8* kb2 = (lds_u8*)kb2_raw;
  lds_u8* kb3 = (lds_u8*)kb3_raw;
  lds_u8* vb0 = (lds_u8*)vb0_raw;
  lds_u8* vb1 = (lds_u8*)vb1_raw;
  lds_u8* vb2 = (lds_u8*)vb2_raw;
  lds_u8* vb3 = (lds_u8*)vb3_raw;
  lds_u8* xp0 = (lds_u8*)xp0_raw;
  lds_u8* xp1 = (lds_u8*)xp1_raw;

  int bh, qt;
  decode_tile<CAUSAL>(xcd_logical_index(blockIdx.x, nq * bh_total), nq, bh_total,
                      group_heads, bh, qt);
  const size_t qhead = (size_t)bh * (size_t)Sq * D;
  const size_t khead = (size_t)bh * (size_t)Sk * D;
  const uint16_t* Qh = Q + qhead;
  const uint16_t* Kh = K + khead;
  const uint16_t* Vh = V + khead;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const int m = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * C::BR;
  const int qw0 = q0 + pair * kRowsPerWave;
  const int my_q = qw0 + m;
  // bottom-right causal alignment, as in the other kernels
  const int kshift = Sk - Sq;
  const int kend = CAUSAL ? max(0, min(Sk, q0 + C::BR + kshift)) : Sk;
  const int ntiles = (kend + BC - 1) / BC;
  const int pair_klast = CAUSAL ? min(qw0 + kRowsPerWave - 1 + kshift, Sk - 1) : (Sk - 1);
  const int wnt = (qw0 < Sq && pair_klast >= 0) ? min(ntiles, pair_klast / BC + 1) : 0;
  const int xoff = pair * 2048 + lane * 16;  // this lane's P chunk 0
  const int moff = pair * kRowsPerWave + m;  // this lane's row in xm

  // The O wave of pair p issues share p of every K and V tile copy.
  int koff[NL], krow[NL], voff[NL], vrow[NL];
  tile_offsets<C, false>(koff, krow, pair, lane);
  tile_offsets<C, true>(voff, vrow, pair, lane);
  const int wslot = pair * (NL * 1024);  // this wave's share of a buffer
  // Copy of tile t (the last tile past the end, so that every step issues
  // the same number of copies).
  const auto copy = [&](const uint16_t* src, int t, const int* off, const int* row,
                        lds_u8* dst) {
    const char* b;
    int bo[NL];
    tile_src<C>(src, min(t, ntiles - 1) * BC, Sk, off, row, b, bo);
#pragma unroll
    for (int u = 0; u < NL; ++u) copy_piece(b, bo[u], dst + wslot + u * 1024);
  };
  const auto prologue_copies = [&]() {
    if (ntiles > 0) {
      copy(Kh, 0, koff, krow, kb0);
      copy(Kh, 1, koff, krow, kb1);
      copy(Kh, 2, koff, krow, kb2);
      copy(Kh, 3, koff, krow, kb3);
      copy(Vh, 0, voff, vrow, vb0);
      copy(Vh, 1, voff, vrow, vb1);
    }
  };

  if (wave < 4) {
    // ---------------- S wave: scores, weights, row sums, LSE ----------------
    bf16x8 qf[C::KCH];
#pragma unroll
    for (int ch = 0; ch < C::KCH; ++ch) {
      u32x4 raw = u32x4{0u, 0u, 0u, 0u};
      if (my_q < Sq)
        raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)my_q * D + ch * 16 + hh * 8);
      qf[ch] = __builtin_bit_cast(bf16x8, raw ^ qflip);
    }
    const int pm = key_perm(m);
    const int ksw = kswz<C>(pm);
    int k_off[C::NKOFF];
#pragma unroll
    for (int b = 0; b < C::NKOFF; ++b)
      k_off[b] = pm * C::ROW_BYTES + (((2 * b + hh) ^ ksw) << 4);

    float m_run = -INFINITY;
    float l_exact = 0.0f;  // float32 sum of the weights (for the LSE)
    f32x16 s_a[1], s_b[1];

    const auto needs_mask = [&](int t) {
      const int k0 = t * BC;
      return (CAUSAL && (k0 + BC - 1 > qw0 + kshift)) || (k0 + BC > Sk);
    };
    const auto mask_tile = [&](f32x16 (&s)[1], int k0) {
      const int lim = (CAUSAL ? min(my_q + kshift, Sk - 1) : (Sk - 1)) - k0 - hh * 8;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 3) * 16 + (r & 7);
        s[0][r] = key > lim ? -INFINITY : s[0][r];
      }
    };
    // Weights of the tile in s against m_run (bf16, in the layout of the B
    // operand of the P.V product) and their float32 sum.
    const auto weights = [&](const f32x16 (&s)[1], bf16x8 (&pf)[2], float& rs) {
      const float mc = m_run == -INFINITY ? 0.0f : m_run * c;
      rs = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[0][r], c, -mc));
        rs += p;
        pf[r >> 3][r & 7] = (__bf16)p;
      }
    };
    // The rare path: a lane's weights sum past kPairSumLimit (or not to a
    // finite value).  Raise the reference to the row max seen so far and form
    // the tile's weights again (the O wave rescales O when it sees the new
    // reference next to them).
    const auto raise = [&](const f32x16 (&s)[1], bf16x8 (&pf)[2], float& rs) {
      // (the weights formed before are replaced; this use keeps their
      // computation where the instruction order put it, and the pass of the
      // scores through it keeps this path's work out of the common one)
      f32x16 sr[1] = {s[0]};
      asm volatile("" : "+v"(sr[0]) : "v"(pf[0]), "v"(pf[1]));
      const float mt = row_max<C>(sr, hh);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_new == m_run ? 1.0f : fast_exp2((m_run - m_new) * c);
      m_run = m_new;
      l_exact *= alpha;
      weights(sr, pf, rs);
    };
    // Weights of tile t for the O wave: P and its reference to LDS.
    const auto publish = [&](const f32x16 (&s)[1], lds_u8* xp, float* xm) {
      bf16x8 pf[2];
      float rs;
      weights(s, pf, rs);
      if (__any(!(rs <= kPairSumLimit))) raise(s, pf, rs);
      *(lds_bf16x8*)(xp + xoff) = pf[0];
      *(lds_bf16x8*)(xp + xoff + 1024) = pf[1];
      xm[moff] = m_run;
      l_exact += rs;
    };

    __syncthreads();  // K(0..3), V(0..1) are in LDS
    // P(0), P(1) and S(2).  The reference max comes from S(0) (masked): every
    // row that sees any key sees key 0, so only rows that see nothing keep
    // -inf.
    if (wnt > 0) {
      qk_tile<C>(s_b, kb0, qf, k_off);
      if (needs_mask(0)) mask_tile(s_b, 0);
      m_run = row_max<C>(s_b, hh);
      publish(s_b, xp0, xm0);
      if (wnt > 1) {
        qk_tile<C>(s_b, kb1, qf, k_off);
        if (needs_mask(1)) mask_tile(s_b, BC);
        publish(s_b, xp1, xm1);
      }
      if (wnt > 2) qk_tile<C>(s_a, kb2, qf, k_off);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    plain_barrier();
    plain_barrier();  // the O waves have read P(0): its buffer takes P(2)

    // step j: S(j+3) into s_out, the weights of S(j+2) (in s_in) to xp
    const auto s_step = [&](const int j, const lds_u8* k_rd, f32x16 (&s_in)[1],
                            f32x16 (&s_out)[1], lds_u8* xp, float* xm) {
      const int t = j + 2;  // the tile whose weights this step forms
      if (t + 1 < wnt && !needs_mask(t)) {
        qk_tile<C>(s_out, k_rd, qf, k_off);
        publish(s_in, xp, xm);
        // each product followed by one K read (kLead ahead) and 4 VALU
        constexpr int kLead = 3;
        __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      } else if (t < wnt) {  // a masked tile, or the pair's last
        if (needs_mask(t)) mask_tile(s_in, t * BC);
        if (t + 1 < wnt) qk_tile<C>(s_out, k_rd, qf, k_off);
        publish(s_in, xp, xm);
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
      plain_barrier();
    };
    // S(t) lives in s_a for t even, s_b for t odd; K(t) in kb(t mod 4); P(t)
    // in xp(t mod 2).
#define FA_S_STEP(J, POS)                                              \
  ((POS) == 0   ? s_step(J, kb3, s_a, s_b, xp0, xm0)                   \
   : (POS) == 1 ? s_step(J, kb0, s_b, s_a, xp1, xm1)                   \
   : (POS) == 2 ? s_step(J, kb1, s_a, s_b, xp0, xm0)                   \
                : s_step(J, kb2, s_b, s_a, xp1, xm1))
    int j = 0;
    for (; j + 4 <= ntiles; j += 4) {
      FA_S_STEP(j, 0);
      FA_S_STEP(j + 1, 1);
      FA_S_STEP(j + 2, 2);
      FA_S_STEP(j + 3, 3);
    }
    if (j < ntiles) FA_S_STEP(j, 0);
    if (j + 1 < ntiles) FA_S_STEP(j + 1, 1);
    if (j + 2 < ntiles) FA_S_STEP(j + 2, 2);
#undef FA_S_STEP

    const float le = l_exact + swap_halves(l_exact, hh);
    // A row that saw no key keeps m_run = -inf and le = 0: LSE = -inf.
    if (my_q < Sq && hh == 0) LSE[(size_t)bh * Sq + my_q] = (m_run * c + fast_log2(le)) * kLn2;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    plain_barrier();
    return;
  }

  // ---------------- O wave: O += V P, the tile copies ----------------
  // The O wave's instructions win the SIMD's issue arbitration over its S
  // wave's: its step is the longer one (the S wave waits at the barrier).
  __builtin_amdgcn_s_setprio(1);
  prologue_copies();
  const int g = lane >> 4, j4 = (lane >> 2) & 3, t4 = lane & 3;
  const int vx = 2 * (g & 1) + (t4 >> 1);
  const int vsw = vswz<C>(hh * 8 + j4);
  const int v_row = (hh * 8 + j4) * C::ROW_BYTES + (t4 & 1) * 8;
  int v_off[C::NVOFF];
#pragma unroll
  for (int d4 = 0; d4 < C::NVOFF; ++d4) v_off[d4] = v_row + (((4 * d4 + vx) ^ vsw) << 4);
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // K(0..3), V(0..1) are in LDS
  if (ntiles > 0) copy(Vh, 2, voff, vrow, vb2);
  plain_barrier();  // P(0), P(1) and their references are in LDS
  if (ntiles > 0) copy(Kh, 4, koff, krow, kb0);
  // the weights for this step and the reference they were taken against
  bf16x8 pf[2];
  float m_p = -INFINITY;
  if (wnt > 0) {
    pf[0] = *(const lds_bf16x8*)(xp0 + xoff);
    pf[1] = *(const lds_bf16x8*)(xp0 + xoff + 1024);
    m_p = xm0[moff];
  }
  float m_b = m_p;  // the reference O is scaled to
  // sum of the bf16 weights (two chains), the normalisation of O
  float l_round0 = 0.0f, l_round1 = 0.0f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
  plain_barrier();  // P(0) is read: step 0 of the S waves overwrites it

  const auto o_step = [&](const int j, const lds_u8* v_rd, lds_u8* k_wr, lds_u8* v_wr,
                          const lds_u8* xp_next, const float* xm_next) {
    if (j < wnt) {
      if (__any(m_p != m_b)) {
        const float alpha = m_p == m_b ? 1.0f : fast_exp2((m_b - m_p) * c);
        m_b = m_p;
        l_round0 *= alpha;
        l_round1 *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
      }
#pragma unroll
      for (int pc = 0; pc < 2; ++pc)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x2 two = {pf[pc][2 * t], pf[pc][2 * t + 1]};
          if (pc & 1) l_round1 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l_round1, false);
          else l_round0 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l_round0, false);
        }
      // P(j+1) for the next step (written during step j-1)
      bf16x8 pn[2];
      float mn = m_p;
      if (j + 1 < wnt) {
        pn[0] = *(const lds_bf16x8*)(xp_next + xoff);
        pn[1] = *(const lds_bf16x8*)(xp_next + xoff + 1024);
        mn = xm_next[moff];
      }
      copy(Kh, j + 5, koff, krow, k_wr);
      copy(Vh, j + 3, voff, vrow, v_wr);
#pragma unroll
      for (int pc = 0; pc < C::PCH; ++pc)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const lds_u8* p = v_rd + pc * 16 * C::ROW_BYTES + (db / C::NVOFF) * 256 +
                            v_off[db % C::NVOFF];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * C::ROW_BYTES));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[pc], acc[db], 0, 0, 0);
        }
      // each product's two V reads issued kLead products ahead, one copy
      // after every second product
      constexpr int kLead = 3;
      constexpr int kNM = C::DB * C::PCH;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLead, 0);
#pragma unroll
      for (int i = 0; i < kNM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kLead < kNM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (i & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if (j + 1 < wnt) {
        pf[0] = pn[0];
        pf[1] = pn[1];
        m_p = mn;
      }
    } else {
      copy(Kh, j + 5, koff, krow, k_wr);
      copy(Vh, j + 3, voff, vrow, v_wr);
    }
    // The previous step's copies have landed (this step's stay in flight).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * NL));
    plain_barrier();
  };
  // V(t) in vb(t mod 4), K(t) in kb(t mod 4), P(t) in xp(t mod 2)
#define FA_O_STEP(J, POS)                                          \
  ((POS) == 0   ? o_step(J, vb0, kb1, vb3, xp1, xm1)               \
   : (POS) == 1 ? o_step(J, vb1, kb2, vb0, xp0, xm0)               \
   : (POS) == 2 ? o_step(J, vb2, kb3, vb1, xp1, xm1)               \
                : o_step(J, vb3, kb0, vb2, xp0, xm0))
  int j = 0;
  for (; j + 4 <= ntiles; j += 4) {
    FA_O_STEP(j, 0);
    FA_O_STEP(j + 1, 1);
    FA_O_STEP(j + 2, 2);
    FA_O_STEP(j + 3, 3);
  }
  if (j < ntiles) FA_O_STEP(j, 0);
  if (j + 1 < ntiles) FA_O_STEP(j + 1, 1);
  if (j + 2 < ntiles) FA_O_STEP(j + 2, 2);
#undef FA_O_STEP
  __builtin_amdgcn_s_waitcnt(0);  // no copy may land after the workgroup ends
  plain_barrier();                // the S waves' last barrier
  const float l_round = l_round0 + l_round1;
  const float lr = l_round + swap_halves(l_round, hh);
  if (my_q >= Sq) return;
  const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
  uint16_t* Orow = O + qhead + (size_t)my_q * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 pk;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const __bf16 lo = (__bf16)(acc[db][gq * 4 + 2 * t] * inv);
        const __bf16 hi = (__bf16)(acc[db][gq * 4 + 2 * t + 1] * inv);
        pk[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<u32x2*>(Orow + db * 32 + gq * 8 + hh * 4) = pk;
    }
}

// ----------------------------------------------------------------------------
// float32 kernel (v_mfma_f32_32x32x2_f32): same tiling and softmax, float32
// operands and float32 softmax weights.  Single-buffered LDS, 32-key tiles.
// ----------------------------------------------------------------------------

template <int D>
struct F32Cfg {
  static constexpr int BC = 32;
  static constexpr int KST = D + 1;  // padded K/V row stride (floats)
  static constexpr int ELEMS = 2 * BC * KST;
  static constexpr int DB = D / 32;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int S, int nq, int bh_total,
    int group_heads, float c) {
  using C = F32Cfg<D>;
  // negative scale: S from -Q with |c| (see kZeroScaleC)
  const float qsign = c < 0.0f ? -1.0f : 1.0f;
  c = fabsf(c);
  constexpr int BC = C::BC;
  __shared__ float smem[C::ELEMS];
  float* Ks = smem;
  float* Vs = smem + BC * C::KST;

  int bh, qt;
  decode_tile<CAUSAL>(xcd_logical_index(blockIdx.x, nq * bh_total), nq, bh_total,
                      group_heads, bh, qt);
  const size_t head = (size_t)bh * (size_t)S * D;
  const float* Qh = Q + head;
  const float* Kh = K + head;
  const float* Vh = V + head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * kRowsPerWave;
  const int my_q = qw0 + m;
  const bool wave_active = qw0 < S;
  const int kend = CAUSAL ? min(S, q0 + kBr) : S;
  const int ntiles = (kend + BC - 1) / BC;
  const int wave_klast = CAUSAL ? min(qw0 + kRowsPerWave - 1, S - 1) : (S - 1);

  // B operand of S^T = K * Q^T: lane holds Q[my_q][2*ch + hh].
  float qf[D / 2];
#pragma unroll
  for (int ch = 0; ch < D / 2; ++ch) qf[ch] = (my_q < S) ? qsign * Qh[(size_t)my_q * D + 2 * ch + hh] : 0.0f;

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = -INFINITY;
  float l_part = 0.0f;

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * BC;
    __syncthreads();  // previous tile fully consumed
    for (int e = tid; e < BC * D; e += kThreads) {
      const int row = e / D, col = e % D;
      const int key = k0 + row;
      const bool ok = key < S;
      Ks[row * C::KST + col] = ok ? Kh[(size_t)key * D + col] : 0.0f;
      Vs[row * C::KST + col] = ok ? Vh[(size_t)key * D + col] : 0.0f;
    }
    __syncthreads();
    if (!(wave_active && k0 <= wave_klast)) continue;

    // S^T: A = K rows (identity order), lane holds K[k0 + m][2*ch + hh].
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
    for (int ch = 0; ch < D / 2; ++ch)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[m * C::KST + 2 * ch + hh], qf[ch], s, 0, 0, 0);
    // Register r holds key k0 + (r/4)*8 + hh*4 + r%4.

    const bool need_mask = (CAUSAL && (k0 + BC - 1 > qw0)) || (k0 + BC > S);
    if (need_mask) {
      const int lim = CAUSAL ? min(my_q, S - 1) : (S - 1);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + (r >> 2) * 8 + hh * 4 + (r & 3);
        if (key > lim) s[r] = -INFINITY;
      }
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = fmaxf(mt, other_half(mt));
    const bool grow = mt > m_run;
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2((m_run - m_new) * c);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    const float mc = (m_run == -INFINITY) ? 0.0f : m_run * c;
    float rs = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(fmaf(s[r], c, -mc));
      s[r] = p;
      rs += p;
    }
    l_part += rs;

    // O^T += V^T * P^T in 16 steps of 2 keys: step r pairs register r of the
    // two lane halves, i.e. keys (r/4)*8 + hh*4 + r%4.
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + hh * 4 + (r & 3);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * C::KST + db * 32 + m], s[r],
                                                       acc[db], 0, 0, 0);
      }
  }

  if (!wave_active) return;
  const float l_tot = l_part + other_half(l_part);
  if (my_q >= S) return;
  const float inv = 1.0f / l_tot;
  float* Orow = O + head + (size_t)my_q * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) Orow[db * 32 + (r >> 2) * 8 + hh * 4 + (r & 3)] = acc[db][r] * inv;
  if (hh == 0) LSE[(size_t)bh * S + my_q] = (m_run * c + fast_log2(l_tot)) * kLn2;
}

// ----------------------------------------------------------------------------
// Host side: validation and launch
// ----------------------------------------------------------------------------

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

struct Plan {
  int bh_total;
  int group_heads;
  float c;
};

// Shape checks shared by the entry points and the plan query: Sq query rows
// against Sk keys per (batch, head).
int validate_shape(int B, int H, int Sq, int Sk, int D, int causal, size_t elem) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return FA_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  const int64_t bh = (int64_t)B * H;
  // every configuration uses query tiles of at least 128 rows
  const int64_t nq_max = ((int64_t)Sq + 127) / 128;
  if (bh > INT32_MAX || (int64_t)Sq * D > INT32_MAX || (int64_t)Sk * D > INT32_MAX ||
      nq_max * bh > INT32_MAX)
    return FA_ERR_SHAPE;
  const int64_t n = bh * (int64_t)(Sq > Sk ? Sq : Sk) * D;
  if ((uint64_t)n > (uint64_t)(SIZE_MAX / elem) / 2) return FA_ERR_SHAPE;
  return FA_OK;
}

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int B, int H, int Sq, int Sk, int D, int causal, float scale, size_t elem,
             Plan* plan) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  const int st = validate_shape(B, H, Sq, Sk, D, causal, elem);
  if (st != FA_OK) return st;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const int64_t bh = (int64_t)B * H;
  const uintptr_t a16 = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o;
  if ((a16 & 15u) || ((uintptr_t)lse & 3u)) return FA_ERR_ALIGN;
  const size_t qb = (size_t)(bh * Sq * D) * elem;   // q and o
  const size_t kb = (size_t)(bh * Sk * D) * elem;   // k and v
  const size_t lb = (size_t)(bh * Sq) * sizeof(float);
  if (ranges_overlap(o, qb, q, qb) || ranges_overlap(o, qb, k, kb) ||
      ranges_overlap(o, qb, v, kb) || ranges_overlap(lse, lb, q, qb) ||
      ranges_overlap(lse, lb, k, kb) || ranges_overlap(lse, lb, v, kb) ||
      ranges_overlap(lse, lb, o, qb))
    return FA_ERR_ALIAS;
  plan->bh_total = (int)bh;
  plan->group_heads = bh >= 8 ? (int)(bh / 8) : 1;
  plan->c = scale == 0.0f ? kZeroScaleC : scale * kLog2e;  // sign: see kZeroScaleC
  return FA_OK;
}

template <class KernelT, class... Args>
int launch(KernelT kernel, unsigned grid, unsigned threads, hipStream_t stream, Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid),
                                       dim3(threads), argv, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ----------------------------------------------------------------------------
// bf16 decode kernel: one query row per (batch, head)
// ----------------------------------------------------------------------------
// With a single query row the products are matrix-vector ones and the launch
// is bound by reading K and V from memory.  One workgroup per (batch, head);
// its WAVES waves take contiguous ranges of the keys and stream them straight
// from global memory into registers (no LDS staging, so the bytes in flight
// are bounded by registers, not by LDS buffers).  Per block of KPI keys, lane
// l holds head-dim entries [32 (l mod LPK), +32) of key l / LPK (LPK = D / 32
// lanes per key): 64 contiguous bytes of K and of V per lane, and one
// contiguous range of KPI rows per wave.  The next block's loads are in
// flight while the current one is used.  Score: bf16 dot products with
// float32 accumulation, summed over the key's LPK lanes.  Softmax as in the
// D = 256 wave-pair kernel: the wave's reference max comes from its first
// block and is raised (to the max of the block) only when a weight would
// exceed 2^24.  O accumulates the float32 weights (not rounded) times V in
// float32 and is normalised by the float32 sum of the same weights.  The
// waves' partial results (reference, sum, O) are then combined through LDS,
// each weighted by 2^((m_w - m) c) against the largest reference m.  A row
// always sees every key (the causal mask with one query aligned bottom-right
// keeps all of them).
constexpr int kDecodeWaves = 8;

template <int D>
struct DecCfg {
  static constexpr int LPK = D / 32;      // lanes per key
  static constexpr int KPI = 64 / LPK;    // keys per block (one per lane group)
};

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void fa_decode_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int Sk,
    int chunk, float c) {
  using C = DecCfg<D>;
  constexpr int LPK = C::LPK, KPI = C::KPI;
  static_assert(WAVES <= 16 && KPI * LPK == 64, "decode: lane layout");
  // negative scale: S from -Q with |c| (see kZeroScaleC)
  const uint32_t qflip = sign_flip_mask(c);
  c = fabsf(c);
  __shared__ float wm[WAVES], wl[WAVES];
  __shared__ float wo[WAVES][D];

  const int bh = blockIdx.x;
  const uint16_t* Kh = K + (size_t)bh * (size_t)Sk * D;
  const uint16_t* Vh = V + (size_t)bh * (size_t)Sk * D;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = lane / LPK;  // the lane's key within a block
  const int dg = lane % LPK;  // the lane's 32 head-dim entries
  const int k_begin = min(Sk, wave * chunk);
  const int k_end = min(Sk, k_begin + chunk);
  const int nblk = (k_end - k_begin + KPI - 1) / KPI;

  // the lane's 32 entries of q as bf16 pairs
  u32x4 qv[4];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(Q + (size_t)bh * D + dg * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = qp[i] ^ qflip;
  }
  // loads of block b: the lane's 64 bytes of K and of V (key clamped to the
  // range; keys past it are masked)
  const auto load = [&](int b, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
    const int key = min(k_begin + b * KPI + kg, k_end - 1);
    const u32x4* kp = reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + dg * 32);
    const u32x4* vp = reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + dg * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = kp[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = vp[i];
  };
  // sum over the lanes of a key, max over the keys of the block
  const auto key_sum = [&](float x) {
#pragma unroll
    for (int msk = 1; msk < LPK; msk <<= 1) x += __shfl_xor(x, msk);
    return x;
  };
  const auto block_max = [&](float x) {
#pragma unroll
    for (int msk = LPK; msk < 64; msk <<= 1) x = fmaxf(x, __shfl_xor(x, msk));
    return x;
  };

  float o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = 0.0f;
  float l = 0.0f;          // the lane's key weights summed (each key once per lane)
  float m_ref = -INFINITY;  // the wave's reference max (raw scores)

  const auto block = [&](int b, const u32x4 (&kr)[4], const u32x4 (&vr)[4]) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // (element copies first: a bit cast of a vector element would read element 0)
        const uint32_t kk = kr[i][e], qq = qv[i][e];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kk),
                                            __builtin_bit_cast(bf16x2, qq), s, false);
      }
    s = key_sum(s);
    if (k_begin + b * KPI + kg >= k_end) s = -INFINITY;
    if (b == 0) m_ref = block_max(s);  // finite: the block holds key k_begin
    float p = fast_exp2(fmaf(s, c, -m_ref * c));
    if (__any(!(p <= kPairSumLimit))) {
      const float m_new = fmaxf(m_ref, block_max(s));
      const float alpha = fast_exp2((m_ref - m_new) * c);
      m_ref = m_new;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] *= alpha;
      p = fast_exp2(fmaf(s, c, -m_ref * c));
    }
    l += p;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = vr[i][e];
        o[8 * i + 2 * e] = fmaf(p, __builtin_bit_cast(float, w << 16), o[8 * i + 2 * e]);
        o[8 * i + 2 * e + 1] =
            fmaf(p, __builtin_bit_cast(float, w & 0xffff0000u), o[8 * i + 2 * e + 1]);
      }
  };

  if (nblk > 0) {
    // loads are unconditional (a key past the range reads the range's last
    // row again); only the blocks' arithmetic stops at nblk
    u32x4 k0[4], v0[4], k1[4], v1[4];
    load(0, k0, v0);
    for (int b = 0; b < nblk; b += 2) {
      load(b + 1, k1, v1);
      block(b, k0, v0);
      load(b + 2, k0, v0);
      if (b + 1 < nblk) block(b + 1, k1, v1);
    }
    // the wave's totals: O over the keys of the block (lanes of equal dg), l
#pragma unroll
    for (int i = 0; i < 32; ++i)
#pragma unroll
      for (int msk = LPK; msk < 64; msk <<= 1) o[i] += __shfl_xor(o[i], msk);
#pragma unroll
    for (int msk = LPK; msk < 64; msk <<= 1) l += __shfl_xor(l, msk);
  }
  if (lane == 0) {
    wm[wave] = m_ref;
    wl[wave] = l;
  }
  if (kg == 0) {
#pragma unroll
    for (int i = 0; i < 32; ++i) wo[wave][dg * 32 + i] = o[i];
  }
  __syncthreads();
  if (wave != 0) return;
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) m = fmaxf(m, wm[w]);
  float lt = 0.0f;
  float f[WAVES];
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    f[w] = wm[w] == -INFINITY ? 0.0f : fast_exp2((wm[w] - m) * c);
    lt += wl[w] * f[w];
  }
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  constexpr int DPL = D / 64;  // output entries per lane
  uint16_t* Orow = O + (size_t)bh * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int d = lane * DPL + i;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) acc = fmaf(wo[w][d], f[w], acc);
    Orow[d] = __builtin_bit_cast(uint16_t, (__bf16)(acc * inv));
  }
  if (lane == 0) LSE[bh] = (m * c + fast_log2(lt)) * kLn2;
}

// Launch shape of the bf16 kernel for one call.
struct LaunchCfg {
  int waves;     // wavefronts per workgroup
  int rows;      // query rows per workgroup (32 per wave; at D = 256 per pair of waves)
  int bc;        // keys per K/V tile
  int nq;        // query tiles per head
  unsigned grid; // workgroups
  bool decode;   // fa_decode_kernel: one query row, one workgroup per head
};

// Tile sizes: 64-key tiles up to D = 128, 32-key tiles at D = 256 (LDS and
// registers).  Workgroup size: an 8-wave workgroup (256 query rows) shares
// each staged K/V tile among twice as many rows as a 4-wave one, halving the
// global->LDS copy volume per flop.  At D = 128 that pays when the grid still
// holds enough workgroups to balance: one per CU when the workgroups are of
// about equal length (no mask, or queries behind a key prefix at least as
// long as themselves, so the longest query tile's keys exceed the mean by at
// most a third), two per CU otherwise (the causal mask over a square
// sequence: lengths 1..n).  At D = 64 the exponentials, not the copies,
// dominate.  D = 256 runs four pairs of waves on 128 rows (two waves per
// SIMD).  A single query row against the keys of at most one head per CU
// (D <= 128) goes to fa_decode_kernel: with so few workgroups the tiled
// kernel's one staged tile per wave keeps too few bytes in flight per CU,
// while the decode kernel's eight waves each hold two blocks of K/V rows in
// registers.  With more heads the two read at about the same rate.
LaunchCfg bf16_config(int Sq, int Sk, int D, bool causal, int bh_total) {
  constexpr int64_t kCUs = 256;
  LaunchCfg cfg;
  cfg.decode = Sq == 1 && D <= 128 && bh_total <= kCUs;
  if (cfg.decode) {
    cfg.waves = kDecodeWaves;
    cfg.rows = 1;
    cfg.bc = 2048 / D;  // keys per block of the decode kernel
    cfg.nq = 1;
    cfg.grid = (unsigned)bh_total;
    return cfg;
  }
  cfg.bc = D == 256 ? 32 : 64;
  cfg.waves = 4;
  const bool even = !causal || (int64_t)Sk - Sq >= Sq;
  // (With at most 128 queries the upper half of a 256-row tile would stay
  // empty: decode and short chunks keep 128-row workgroups, two per CU.)
  if (D == 128 && Sq > 128 && (int64_t)((Sq + 255) / 256) * bh_total >= (even ? 1 : 2) * kCUs)
    cfg.waves = 8;
  cfg.rows = kRowsPerWave * cfg.waves;
  if (D == 256) {
    cfg.waves = kPipe == kPipeD256Ring ? 4 : 8;
    cfg.rows = 128;
  }
  const int br = cfg.rows;
  cfg.nq = (Sq + br - 1) / br;
  cfg.grid = (unsigned)cfg.nq * (unsigned)bh_total;
  return cfg;
}

template <int D, int BC, int WAVES>
int run_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int Sq, int Sk,
             bool causal, const Plan& p, const LaunchCfg& cfg, hipStream_t stream) {
  static_assert(BfCfg<D, BC, WAVES>::BR == kRowsPerWave * WAVES, "rows per workgroup");
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* K = static_cast<const uint16_t*>(k);
  const uint16_t* V = static_cast<const uint16_t*>(v);
  uint16_t* Out = static_cast<uint16_t*>(o);
  // the head-dim split copy exists for D = 128 only; the D = 256 study mode
  // leaves D <= 128 as the library runs it
  constexpr int P = kPipe == kPipeKSplit && D != 128 ? kPipeNoPrefetch
                    : kPipe == kPipeD256Ring         ? kPipeOverlap
                                                     : kPipe;
  if constexpr (D == 256 && kPipe == kPipeD256Ring) {
    if (causal)
      return launch(fa_fwd_bf16_ring_kernel<D, BC, WAVES, true>, cfg.grid, 64 * cfg.waves, stream,
                    Q, K, V, Out, lse, Sq, Sk, cfg.nq, p.bh_total, p.group_heads, p.c);
    return launch(fa_fwd_bf16_ring_kernel<D, BC, WAVES, false>, cfg.grid, 64 * cfg.waves, stream,
                  Q, K, V, Out, lse, Sq, Sk, cfg.nq, p.bh_total, p.group_heads, p.c);
  } else if constexpr (D == 256) {
    if (causal)
      return launch(fa_fwd_bf16_pair_kernel<true>, cfg.grid, 64 * cfg.waves, stream, Q, K, V, Out,
                    lse, Sq, Sk, cfg.nq, p.bh_total, p.group_heads, p.c);
    return launch(fa_fwd_bf16_pair_kernel<false>, cfg.grid, 64 * cfg.waves, stream, Q, K, V, Out,
                  lse, Sq, Sk, cfg.nq, p.bh_total, p.group_heads, p.c);
  } else {
    if (causal)
      return launch(fa_fwd_bf16_kernel<D, BC, WAVES, true, kMfmaSum, P>, cfg.grid, 64 * WAVES, stream,
                    Q, K, V, Out, lse, Sq, Sk, cfg.nq, p.bh_total, p.group_heads, p.c);
    return launch(fa_fwd_bf16_kernel<D, BC, WAVES, false, kMfmaSum, P>, cfg.grid, 64 * WAVES, stream,
                  Q, K, V, Out, lse, Sq, Sk, cfg.nq, p.bh_total, p.group_heads, p.c);
  }
}

template <int D>
int run_decode(const void* q, const void* k, const void* v, void* o, float* lse, int Sk,
               const Plan& p, const LaunchCfg& cfg, hipStream_t stream) {
  constexpr int KPI = DecCfg<D>::KPI;
  // contiguous key ranges of whole blocks, one per wave
  const int chunk = (int)(((int64_t)Sk + kDecodeWaves * KPI - 1) / (kDecodeWaves * KPI) * KPI);
  return launch(fa_decode_kernel<D, kDecodeWaves>, cfg.grid, 64 * kDecodeWaves, stream,
                static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, Sk, chunk, p.c);
}

template <int D>
int run_f32(const float* q, const float* k, const float* v, float* o, float* lse, int S,
            bool causal, const Plan& p, hipStream_t stream) {
  const int nq = (S + kBr - 1) / kBr;
  const unsigned grid = (unsigned)nq * (unsigned)p.bh_total;
  if (causal)
    return launch(fa_fwd_f32_kernel<D, true>, grid, kThreads, stream, q, k, v, o, lse, S, nq,
                  p.bh_total, p.group_heads, p.c);
  return launch(fa_fwd_f32_kernel<D, false>, grid, kThreads, stream, q, k, v, o, lse, S, nq,
                p.bh_total, p.group_heads, p.c);
}

int fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Sq, int Sk, int D, int causal, float scale, void* stream) {
  Plan p;
  const int st = validate(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, 2, &p);
  if (st != FA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const LaunchCfg cfg = bf16_config(Sq, Sk, D, causal, p.bh_total);
  if (cfg.decode)
    return D == 64 ? run_decode<64>(q, k, v, o, lse, Sk, p, cfg, s)
                   : run_decode<128>(q, k, v, o, lse, Sk, p, cfg, s);
  switch (D) {
    case 64: return run_bf16<64, 64, 4>(q, k, v, o, lse, Sq, Sk, causal, p, cfg, s);
    case 128:
      if (cfg.waves == 8) return run_bf16<128, 64, 8>(q, k, v, o, lse, Sq, Sk, causal, p, cfg, s);
      return run_bf16<128, 64, 4>(q, k, v, o, lse, Sq, Sk, causal, p, cfg, s);
    default: return run_bf16<256, 32, 4>(q, k, v, o, lse, Sq, Sk, causal, p, cfg, s);
  }
}

// ----------------------------------------------------------------------------
// Merge of results computed over disjoint key sets
// ----------------------------------------------------------------------------
// LSE = log sum_g exp(LSE_g), O = sum_g exp(LSE_g - LSE) O_g, per output row.
// One thread per 16 bytes (8 bf16) of an output row: 16-byte loads of each
// part's O (for up to 16 parts all issued before any is used), float32
// weights and sums, one bf16 (round to nearest even) store.
// A part whose weight is 0 (LSE_g = -inf, or underflow) is skipped and its O
// is not read.  A row with no visible key in any part: O = 0, LSE = -inf.
template <int D, int GU>  // GU > 0: G <= GU parts, unrolled; GU = 0: any G
__global__ __launch_bounds__(256) void fa_merge_kernel(const uint16_t* __restrict__ Op,
                                                       const float* __restrict__ Lp, int G,
                                                       int64_t rows, uint16_t* __restrict__ O,
                                                       float* __restrict__ L) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * CPR) return;
  const int64_t r = t / CPR;
  const int ch = (int)(t % CPR);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  auto add = [&](const u32x4 raw, const float w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += w * __builtin_bit_cast(float, raw[e] << 16);
      acc[2 * e + 1] += w * __builtin_bit_cast(float, raw[e] & 0xFFFF0000u);
    }
  };
  if constexpr (GU > 0) {
    // All parts' LSEs, then all parts' 16-byte loads in flight together.
    float lg[GU];
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < GU; ++g) {
      const float x = Lp[(g < G ? g : G - 1) * rows + r];  // index kept in range
      lg[g] = g < G ? x : -INFINITY;
      m = fmaxf(m, lg[g]);
    }
    if (m != -INFINITY) {
      float sum = 0.0f;
#pragma unroll
      for (int g = 0; g < GU; ++g) sum += fast_exp2((lg[g] - m) * kLog2e);
      lse = m + fast_log2(sum) * kLn2;
      float w[GU];
      u32x4 raw[GU];
#pragma unroll
      for (int g = 0; g < GU; ++g) {
        w[g] = fast_exp2((lg[g] - lse) * kLog2e);
        raw[g] = u32x4{0u, 0u, 0u, 0u};
        if (w[g] != 0.0f)
          raw[g] = *reinterpret_cast<const u32x4*>(Op + ((g < G ? g : G - 1) * rows + r) * D +
                                                    ch * 8);
      }
#pragma unroll
      for (int g = 0; g < GU; ++g)
        if (w[g] != 0.0f) add(raw[g], w[g]);
    }
  } else {
    float m = -INFINITY;
    for (int g = 0; g < G; ++g) m = fmaxf(m, Lp[g * rows + r]);
    if (m != -INFINITY) {
      float sum = 0.0f;
      for (int g = 0; g < G; ++g) sum += fast_exp2((Lp[g * rows + r] - m) * kLog2e);
      lse = m + fast_log2(sum) * kLn2;
      for (int g = 0; g < G; ++g) {
        const float w = fast_exp2((Lp[g * rows + r] - lse) * kLog2e);
        if (w == 0.0f) continue;
        add(*reinterpret_cast<const u32x4*>(Op + (g * rows + r) * D + ch * 8), w);
      }
    }
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    out[e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2 * e]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2 * e + 1]) << 16);
  *reinterpret_cast<u32x4*>(O + r * D + ch * 8) = out;
  if (ch == 0) L[r] = lse;
}

template <int D>
int run_merge(const uint16_t* Op, const float* Lp, int G, int64_t rows, uint16_t* O, float* L,
              hipStream_t s) {
  const unsigned grid = (unsigned)((rows * (D / 8) + 255) / 256);
  if (G <= 4) return launch(fa_merge_kernel<D, 4>, grid, 256, s, Op, Lp, G, rows, O, L);
  if (G <= 8) return launch(fa_merge_kernel<D, 8>, grid, 256, s, Op, Lp, G, rows, O, L);
  if (G <= 16) return launch(fa_merge_kernel<D, 16>, grid, 256, s, Op, Lp, G, rows, O, L);
  return launch(fa_merge_kernel<D, 0>, grid, 256, s, Op, Lp, G, rows, O, L);
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int S, int D, int causal, float scale, void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, S, S, D, causal, scale, stream);
}

extern "C" int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Sq, int Sk, int D, int causal, float scale, void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, stream);
}

extern "C" int fa_merge(const void* o_parts, const float* lse_parts, int G, int B, int H, int S,
                        int D, void* o, float* lse, void* stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (G < 1 || B < 1 || H < 1 || S < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return FA_ERR_HEADDIM;
  const int64_t rows = (int64_t)B * H * S;
  if (rows > INT32_MAX || (uint64_t)G * (uint64_t)rows * D > (uint64_t)(SIZE_MAX / 4) ||
      (uint64_t)(rows * (D / 8) + 255) / 256 > (uint64_t)UINT32_MAX)
    return FA_ERR_SHAPE;
  if ((((uintptr_t)o_parts | (uintptr_t)o) & 15u) ||
      (((uintptr_t)lse_parts | (uintptr_t)lse) & 3u))
    return FA_ERR_ALIGN;
  const size_t ob = (size_t)rows * D * 2, lb = (size_t)rows * sizeof(float);
  if (ranges_overlap(o, ob, o_parts, ob * G) || ranges_overlap(o, ob, lse_parts, lb * G) ||
      ranges_overlap(lse, lb, o_parts, ob * G) || ranges_overlap(lse, lb, lse_parts, lb * G) ||
      ranges_overlap(o, ob, lse, lb))
    return FA_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* Op = static_cast<const uint16_t*>(o_parts);
  uint16_t* Out = static_cast<uint16_t*>(o);
  switch (D) {
    case 64: return run_merge<64>(Op, lse_parts, G, rows, Out, lse, s);
    case 128: return run_merge<128>(Op, lse_parts, G, rows, Out, lse, s);
    default: return run_merge<256>(Op, lse_parts, G, rows, Out, lse, s);
  }
}

extern "C" int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int S, int D, int causal, float scale, void* stream) {
  Plan p;
  const int st = validate(q, k, v, o, lse, B, H, S, S, D, causal, scale, 4, &p);
  if (st != FA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (D) {
    case 64: return run_f32<64>(q, k, v, o, lse, S, causal, p, s);
    case 128: return run_f32<128>(q, k, v, o, lse, S, causal, p, s);
    default: return run_f32<256>(q, k, v, o, lse, S, causal, p, s);
  }
}

extern "C" const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a tensor pointer is NULL";
    case FA_ERR_SHAPE: return "a size (B, H, S, Sq, Sk or G) is < 1, or a size overflows";
    case FA_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_CAUSAL: return "causal must be 0 or 1";
    case FA_ERR_ALIGN: return "q/k/v/o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "o or lse overlaps an input or each other";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_SCRATCH: return "B*H*S exceeds the library's backward scratch array";
    default: return "unknown status";
  }
}

extern "C" int fa_fwd_plan(int B, int H, int S, int D, int causal, int elem_bytes,
                           int* rows_per_group, int* keys_per_tile, int* threads, int* groups) {
  if (elem_bytes != 2 && elem_bytes != 4) return FA_ERR_SHAPE;
  const int st = validate_shape(B, H, S, S, D, causal, (size_t)elem_bytes);
  if (st != FA_OK) return st;
  const int bh = B * H;
  int rows, keys, thr, grid;
  if (elem_bytes == 2) {
    const LaunchCfg cfg = bf16_config(S, S, D, causal != 0, bh);
    rows = cfg.rows;
    keys = cfg.bc;
    thr = 64 * cfg.waves;
    grid = (int)cfg.grid;
  } else {
    rows = kBr;
    keys = F32Cfg<64>::BC;
    thr = kThreads;
    grid = ((S + kBr - 1) / kBr) * bh;
  }
  if (rows_per_group) *rows_per_group = rows;
  if (keys_per_tile) *keys_per_tile = keys;
  if (threads) *threads = thr;
  if (groups) *groups = grid;
  return FA_OK;
}

extern "C" int fa_fwd_kv_plan(int B, int H, int Sq, int Sk, int D, int causal,
                              int* rows_per_group, int* keys_per_tile, int* threads,
                              int* groups) {
  const int st = validate_shape(B, H, Sq, Sk, D, causal, 2);
  if (st != FA_OK) return st;
  const LaunchCfg cfg = bf16_config(Sq, Sk, D, causal != 0, B * H);
  if (rows_per_group) *rows_per_group = cfg.rows;
  if (keys_per_tile) *keys_per_tile = cfg.bc;
  if (threads) *threads = 64 * cfg.waves;
  if (groups) *groups = (int)cfg.grid;
  return FA_OK;
}

extern "C" int fa_abi_version(void) { return 1; }
