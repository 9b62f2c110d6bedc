// Back-to-back GEMM for gfx950, exact shapes: O = F(alpha * A.B0 + bias) . B1
// with K and N in {64, 128} and L a multiple of 64 (bf16 operands).
//
// Method: ComFuse review (pith.science review of arXiv 2608.03537), Referee
// Report major comment 2 (paper Sec. IV-A, Eqs. (2)-(5)) and Fig. 5: S = A.B0 is
// transformed tile by tile and consumed by the second GEMM from on-chip
// storage, the contraction over L accumulated segment by segment. One
// workgroup owns 128 or 256 rows of A (4 waves x 32 or 64) and walks all of L in 64-wide
// segments; O stays in registers. The segment arithmetic (operand swap, P
// packed from the GEMM1 accumulators in the permuted l order, power-of-two
// online-softmax stabiliser) is the one of the general kernel in b2b.hip.
//
// What differs from the general kernel, for speed:
//  * the B0 and B1 segments go from memory straight into an LDS ring of
//    kStages segments (buffer_load_dwordx4 ... lds), refilled one segment per
//    iteration with explicit vmcnt waits; no VGPR staging, no transposes;
//  * B1 stays [l][n] in LDS and GEMM2 reads B1^T with ds_read_b64_tr_b16;
//    B0 given [K][L] likewise stays [k][l] and GEMM1 reads it transposed;
//  * at most 256 registers per lane, so two workgroups share a CU and one
//    wave's softmax (VALU, exp) overlaps the other's MFMAs;
//  * with per-batch B0/B1 (attention heads) the row tiles of one batch entry
//    run on one XCD, so its B0/B1 segments are fetched into that XCD's L2 once;
//  * B0/B1 shared by the whole batch and no longer than the ring stay
//    resident in LDS for all the tiles a workgroup processes.
#include "cf_device.hpp"
#include "cf_launch.h"

namespace cf {
namespace {

constexpr int kTLC = 64;      // L segment
constexpr int kTThreads = 256;

// MB: row blocks of 32 per wave. Two (only where registers allow, K = N = 64)
// give each wave four independent accumulator chains and let every B0/B1
// fragment read from LDS feed two MFMAs; one keeps tiles small when there
// are few rows.
// kBiasEsz: bytes per bias element (0: no bias). A stage then ends with a
// 256-byte block holding the segment's kTLC bias values.
template <int KS, int NB, int MB_, int kBiasEsz = 0>
struct TCfg {
  static constexpr int K = 16 * KS, N = 32 * NB;
  static constexpr int MB = MB_;
  static constexpr int BM = 128 * MB;                            // rows per tile
  static constexpr int kB0Bytes = kTLC * K * 2;
  static constexpr int kB1Bytes = kTLC * N * 2;
  static constexpr int kBiasOff = kB0Bytes + kB1Bytes;
  static constexpr int kStage = kBiasOff + (kBiasEsz ? 256 : 0);
  static constexpr int kStages = 4 * kStage <= 80 * 1024 ? 4 : 3 * kStage <= 80 * 1024 ? 3 : 2;
  static constexpr int kLds = kStages * kStage;
  static constexpr int kB0Blocks = kB0Bytes / 1024;              // 1 KiB DMA blocks
  static constexpr int kLoads = kBiasOff / (kTThreads * 16);     // B0/B1 DMA loads per thread per segment
  static constexpr int kLoadsAll = kLoads + (kBiasEsz ? 1 : 0);  // with the bias load
  static constexpr int kBiasLanes = kTLC * kBiasEsz / 4;         // lanes of the (4-byte) bias load that carry data
};

// XOR swizzles of the 16-byte chunks of an LDS row (physical = logical ^ f):
// conflict free for the access patterns below whether the LDS serves 128 or
// 256 bytes per cycle.
__device__ inline int swz_rows128(int r) { return (r & 7) ^ ((r >> 3) & 1); }   // 16-B row reads, 128-B rows
__device__ inline int swz_rows256(int r) { return r & 15; }                     // 16-B row reads, 256-B rows
__device__ inline int swz_tr128(int r) { return 2 * (r & 3); }                  // transposed reads, 128-B rows
__device__ inline int swz_tr256(int r) { return (2 * (r & 3)) ^ (4 * (r & 3)); }  // transposed reads, 256-B rows

// Per-lane LDS read offsets within a stage (B0 segment, then B1 segment):
//  b0_rd: GEMM1's operand B0^T, rows l = lb*32 + (lane & 31), k-slots 8h..8h+7
//         of step ks; one offset per ks for B0 given [L][K] (16-byte row
//         reads), one per lb for B0 given [K][L] (transposed reads);
//  b1_rd: GEMM2's operand B1^T, rows n = nb*32 + (lane & 31), k-slots = l in
//         the permuted order: half 0 reads rows c16*16 + 4h + 0..3, half 1 rows +8.
template <int KS, int NB, bool kB0LK>
__device__ inline void stage_read_offsets(int lane, uint32_t (&b0_rd)[kB0LK ? KS : 2], uint32_t (&b1_rd)[NB]) {
  constexpr int K = 16 * KS, N = 32 * NB, kB0Bytes = kTLC * K * 2;
  const int h = lane >> 5, r32 = lane & 31;
  if constexpr (kB0LK) {
    constexpr int RB = K * 2;
    const int f = K == 64 ? swz_rows128(r32) : swz_rows256(r32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b0_rd[ks] = (uint32_t)(r32 * RB + 16 * ((2 * ks + h) ^ f));
  } else {
    // [k][l]: lane 16g + i reads row ks*16 + 8(g>>1) + 4 half + i/4, columns
    // lb*32 + 16(g&1) + 4(i&3) .. +3; one base per lb
    const int g = lane >> 4, i = lane & 15;
    const int f = swz_tr128(i >> 2);
    const int c = 2 * (g & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
      b0_rd[lb] = (uint32_t)((8 * (g >> 1) + (i >> 2)) * 128 + 16 * ((4 * lb + c) ^ f) + 8 * (i & 1));
  }
  constexpr int RB = N * 2;
  const int g = lane >> 4, i = lane & 15;
  const int f = N == 64 ? swz_tr128(i >> 2) : swz_tr256(i >> 2);
  const int c = 2 * (g & 1) + ((i & 3) >> 1);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    b1_rd[nb] = (uint32_t)(kB0Bytes + (4 * (g >> 1) + (i >> 2)) * RB + 16 * ((4 * nb + c) ^ f) + 8 * (i & 1));
}

// Global byte offset, within B0 or B1, of the 16 bytes that lane `lane` of
// wave `wave` loads into 1 KiB block q = kWaves*i + wave of the stage holding
// segment s (B0 blocks first, then B1), in the swizzled layouts that
// stage_read_offsets reads.
template <int KS, int NB, bool kB0LK, int kWaves>
__device__ inline uint32_t seg_load_off(const B2bParams& p, int wave, int lane, int i, int s) {
  constexpr int K = 16 * KS, N = 32 * NB, kB0Blocks = kTLC * K * 2 / 1024;
  const int q = kWaves * i + wave;
  if (q < kB0Blocks) {
    if constexpr (kB0LK) {             // rows l of K * 2 bytes
      constexpr int cpr = K / 8, rpb = 1024 / (K * 2);
      const int row = q * rpb + lane / cpr, ph = lane % cpr;
      const int lg = ph ^ (K == 64 ? swz_rows128(row) : swz_rows256(row));
      return ((uint32_t)(row + s * kTLC) * p.ldb0 + (uint32_t)(8 * lg)) * 2u;
    } else {                           // rows k of 64 l (128 bytes)
      const int row = q * 8 + lane / 8, ph = lane % 8;
      const int lg = ph ^ swz_tr128(row);
      return ((uint32_t)row * p.ldb0 + (uint32_t)(8 * lg + s * kTLC)) * 2u;
    }
  }
  constexpr int cpr = N / 8, rpb = 1024 / (N * 2);   // B1 rows l of N * 2 bytes
  const int qb = q - kB0Blocks;
  const int row = qb * rpb + lane / cpr, ph = lane % cpr;
  const int lg = ph ^ (N == 64 ? swz_tr128(row) : swz_tr256(row));
  return ((uint32_t)(row + s * kTLC) * p.ldb1 + (uint32_t)(8 * lg)) * 2u;
}

// Softmax of one 32-row block whose S^T accumulators s[lb] hold l = lb*32 +
// 8(r >> 2) + 4h + (r & 3) of row m = lane & 31. Full form: the row extreme
// of S (max for alpha >= 0, min otherwise, so that it is the extreme of
// alpha*S), and the integer stabiliser cs raised to cover it with an exact
// power-of-two rescale of what was accumulated (o and the lane's row-sum part
// ls).
template <int NB>
__device__ inline void sm_full_rb(const f32x16_t (&s)[2], f32x16_t (&o)[NB], float& cs, float& ls, float scale) {
  float mx;
  if (scale >= 0.0f) {
    mx = -INFINITY;
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[lb][r]);
    mx = max_halves(mx);
  } else {
    mx = INFINITY;
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fminf(mx, s[lb][r]);
    mx = min_halves(mx);
  }
  const float cn = fmaxf(cs, ceilf(mx * scale));
  if (cn > cs && cs != -INFINITY) {
    const int sh = (int)(cs - cn);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nb][r] = __builtin_amdgcn_ldexpf(o[nb][r], sh);
    ls = __builtin_amdgcn_ldexpf(ls, sh);
  }
  cs = cn;
}
// The terms 2^(scale*s - cs) of one row block, added to the lane's row-sum part
// unrounded, and packed to bf16 as the GEMM2 operand (k-slot order of the
// accumulator registers). cs = -inf only while a causal row has seen no key;
// every term is 0 then.
template <bool kCausal>
__device__ inline void sm_terms_rb(const f32x16_t (&s)[2], u32x4_t (&pfr)[4], float cs, float& ls, float scale) {
  const float c0 = (kCausal && cs == -INFINITY) ? 0.0f : cs;
#pragma unroll
  for (int lb = 0; lb < 2; ++lb) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = fast_exp2(__builtin_fmaf(s[lb][r], scale, -c0));
      ls += e[r];
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) pfr[2 * lb + c][q] = pack_bf16x2(e[8 * c + 2 * q], e[8 * c + 2 * q + 1]);
  }
}

}  // namespace

// kCausal (softmax only): key l is visible to row m iff l <= m + p.coff; the
// segments past the last key a tile's rows see are not computed, the segment
// on the diagonal is masked per element, and row tiles that see more keys are
// scheduled first.
// kBias (elementwise F only): S gets a bias per column l, 1 bf16 or 2 fp32.
// Each wave streams the segment's bias into the stage's bias block with the
// ring, 4 bytes per lane (all four waves write the same bytes), so every wave
// issues the same number of ring loads; the bias base must be 4-byte aligned.
template <int KS, int NB, int MB_, bool kSoftmax, bool kB0LK, bool kCausal = false, int kBias = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(kTThreads, kTThreads), amdgpu_waves_per_eu(2, 2)))
void b2b_stream_kernel(B2bParams p) {
  using C = TCfg<KS, NB, MB_, kBias == 2 ? 4 : kBias == 1 ? 2 : 0>;
  constexpr int NS = C::kStages;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::kLds];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  constexpr int MB = C::MB;
  const int mtiles = (p.M + C::BM - 1) / C::BM;
  const int nchunks = p.L / kTLC;
  const float scale = kSoftmax ? p.alpha * kLog2e : p.alpha;
  const float floor_v = p.act == 1 ? 0.0f : -INFINITY;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;

  // ---- DMA plan: load i of wave w fills 1 KiB block q = 4 i + w of a stage
  // (B0 blocks first); per load the global byte offset at segment 0 (batch
  // entry base excluded) and the per-segment step, uniform over the wave
  uint32_t goff[C::kLoads], gstep[C::kLoads];
  bool is_b0[C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    is_b0[i] = (kTThreads / 64) * i + wave < C::kB0Blocks;
    goff[i] = seg_load_off<KS, NB, kB0LK, kTThreads / 64>(p, wave, lane, i, 0);
    gstep[i] = is_b0[i] ? (kB0LK ? (uint32_t)kTLC * p.ldb0 * 2u : kTLC * 2u) : (uint32_t)kTLC * p.ldb1 * 2u;
  }

  // ---- LDS read offsets (within a stage)
  uint32_t b0_rd[kB0LK ? KS : 2], b1_rd[NB];
  stage_read_offsets<KS, NB, kB0LK>(lane, b0_rd, b1_rd);

  const u32x4_t rsb = rsrc_words(p.bias, (uint32_t)p.L * (kBias == 2 ? 4u : 2u));
  auto issue = [&](int s, int nseg, const u32x4_t& rs0, const u32x4_t& rs1) {
    const uint32_t sb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + (uint32_t)((s % NS) * C::kStage)));
    const uint32_t st = sb + (uint32_t)(wave * 1024);
    const bool ok = s < nseg;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
      lds_dma16(st + i * 4096, is_b0[i] ? rs0 : rs1, ok ? goff[i] + (uint32_t)s * gstep[i] : kOutOfRange);
    if constexpr (kBias != 0)
      lds_dma4(sb + C::kBiasOff, rsb,
               ok && lane < C::kBiasLanes ? (uint32_t)(s * C::kBiasLanes + lane) * 4u : kOutOfRange);
  };

  // one segment: GEMM1, F, GEMM2 on stage buffer st; row block rb of the wave.
  // wrow0: first row of this wave (causal masking)
  auto segment = [&](const uint8_t* st, int lc, const u32x4_t (&af)[MB][KS], f32x16_t (&oacc)[MB][NB],
                     float (&cst)[MB], float (&lsum)[MB], int wrow0) {
    f32x16_t sacc[MB][2];
    // GEMM1 (S of the segment) and, for causal rows, the hiding of the keys a
    // row may not see (their extreme-side infinity drops out of the row
    // extreme and gives exp2(-inf) = 0)
    // The MFMA blocks run at raised wave priority: the SIMD's other wave (of
    // the CU's other workgroup) is then the one that waits while its softmax
    // fills the issue slots the MFMAs leave free.
    auto gemm1 = [&]() {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) sacc[rb][lb] = f32x16_t{0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          u32x4_t bf;
          if constexpr (kB0LK) {
            bf = *(const u32x4_t*)(st + b0_rd[ks] + lb * 32 * C::K * 2);
          } else {
            const u32x2_t lo = lds_read_tr16(st + b0_rd[lb] + ks * 16 * 128);
            const u32x2_t hi = lds_read_tr16(st + b0_rd[lb] + ks * 16 * 128 + 4 * 128);
            bf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          }
#pragma unroll
          for (int rb = 0; rb < MB; ++rb)
            sacc[rb][lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bf),
                                                                    __builtin_bit_cast(bf16x8_t, af[rb][ks]), sacc[rb][lb], 0, 0, 0);
        }
      __builtin_amdgcn_s_setprio(0);
      // register r of block lb holds l = lc*64 + lb*32 + 8(r>>2) + 4h + (r&3)
      if constexpr (kCausal) {
        if (lc * kTLC + kTLC - 1 > wrow0 + p.coff) {   // the segment crosses the diagonal for this wave
          const float hide = scale >= 0.0f ? -INFINITY : INFINITY;
#pragma unroll
          for (int rb = 0; rb < MB; ++rb) {
            const int lim = wrow0 + rb * 32 + r32 + p.coff - (lc * kTLC + 4 * h);   // visible iff l - base <= lim
#pragma unroll
            for (int lb = 0; lb < 2; ++lb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (lb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[rb][lb][r] = hide;
          }
        }
      }
    };
    u32x4_t pf[MB][4];
    // softmax of row block rb: full form (row extreme, stabiliser raised with
    // an exact rescale) and the terms with the current stabiliser
    auto softmax_full = [&](int rb) { sm_full_rb<NB>(sacc[rb], oacc[rb], cst[rb], lsum[rb], scale); };
    auto softmax_terms = [&](int rb) { sm_terms_rb<kCausal>(sacc[rb], pf[rb], cst[rb], lsum[rb], scale); };
    if constexpr (kSoftmax) {
      // Any integer stabiliser gives the same quotient (rounding commutes with
      // scaling by a power of two), so the row extreme is taken only while a
      // row has none yet, and when a segment's own terms add up past 2^32; that
      // segment is then redone from a recomputed S (cheaper than keeping S
      // live). Otherwise the current stabiliser is kept.
      bool fresh = false;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) fresh |= cst[rb] == -INFINITY;
      bool full = __builtin_amdgcn_ballot_w64(fresh) != 0;
#pragma nounroll
      for (;;) {
        gemm1();
        float lprev[MB];
        bool big = false;
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          if (full) softmax_full(rb);
          lprev[rb] = lsum[rb];
          softmax_terms(rb);
          big |= !(lsum[rb] - lprev[rb] <= 0x1p32f);
        }
        if (full || __builtin_amdgcn_ballot_w64(big) == 0) break;
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) lsum[rb] = lprev[rb];
        full = true;
      }
    } else {
      gemm1();
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) {
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          float x[16];
          if constexpr (kBias != 0) {
            // the lane's columns: four runs j of four l from lb*32 + 4h + 8j
            uint32_t bwd[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int l0 = lb * 32 + 4 * h + 8 * j;
              if constexpr (kBias == 2) {
                const u32x4_t v = *(const u32x4_t*)(st + C::kBiasOff + l0 * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) bwd[4 * j + e] = v[e];
              } else {
                const u32x2_t v = *(const u32x2_t*)(st + C::kBiasOff + l0 * 2);
                bwd[4 * j] = v[0] << 16;
                bwd[4 * j + 1] = v[0] & 0xffff0000u;
                bwd[4 * j + 2] = v[1] << 16;
                bwd[4 * j + 3] = v[1] & 0xffff0000u;
              }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float bv = __uint_as_float(bwd[r]);
              x[r] = fmaxf(__builtin_fmaf(sacc[rb][lb][r], scale, bv), floor_v);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = fmaxf(sacc[rb][lb][r] * scale, floor_v);
          }
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) pf[rb][2 * lb + c][q] = pack_bf16x2(x[8 * c + 2 * q], x[8 * c + 2 * q + 1]);
        }
      }
    }
    // GEMM2 over the four 16-wide slices of the segment
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x2_t lo = lds_read_tr16(st + b1_rd[nb] + c * 16 * C::N * 2);
        const u32x2_t hi = lds_read_tr16(st + b1_rd[nb] + c * 16 * C::N * 2 + 8 * C::N * 2);
        const u32x4_t vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
          oacc[rb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf),
                                                                  __builtin_bit_cast(bf16x8_t, pf[rb][c]), oacc[rb][nb], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- B0/B1 shared by the batch and no longer than the ring: load once
  const bool shared = p.batch == 1 || (p.sb0 == 0 && p.sb1 == 0);
  const bool resident = shared && nchunks <= NS;
  if (resident) {
    const u32x4_t rs0 = rsrc_words(p.B0, (uint32_t)((size_t)(kB0LK ? p.L : C::K) * p.ldb0 * 2));
    const u32x4_t rs1 = rsrc_words(p.B1, (uint32_t)((size_t)p.L * p.ldb1 * 2));
#pragma unroll
    for (int s = 0; s < NS; ++s) issue(s, nchunks, rs0, rs1);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // ---- tile schedule: with per-batch B0/B1 and a batch that is a multiple of
  // 8, batch entry b is handled by the workgroups of XCD b % 8 (workgroup w
  // runs on XCD w % 8); otherwise tiles go round robin
  const int G = (int)gridDim.x;
  const bool by_xcd = !shared && mtiles > 1 && (p.batch & 7) == 0 && (G & 7) == 0;
  const int x = (int)blockIdx.x & 7;
  const int per_x = by_xcd ? (x < p.batch ? (p.batch - x + 7) / 8 : 0) * mtiles : p.batch * mtiles;
  const int e0 = by_xcd ? (int)blockIdx.x >> 3 : (int)blockIdx.x;
  const int estep = by_xcd ? G >> 3 : G;

  for (int e = e0; e < per_x; e += estep) {
    int b, mt;
    if (by_xcd) {
      b = x + 8 * (e / mtiles);
      mt = e % mtiles;
    } else {
      b = e / mtiles;
      mt = e % mtiles;
    }
    if constexpr (kCausal) {
      // causal work grows with the row tile: when the stride is a multiple of
      // the tiles per batch entry, rotate the row tile by the round so that
      // every workgroup gets each row position once (the tiles of one entry
      // still run in the same round); tiles that see the most keys first
      if (estep % mtiles == 0) mt = (mt + e / estep) % mtiles;
      mt = mtiles - 1 - mt;
    }
    const int m0 = mt * C::BM;
    int nseg = nchunks;
    if constexpr (kCausal) {
      const int last = min(m0 + C::BM - 1, p.M - 1) + p.coff;
      nseg = last < 0 ? 0 : min(nchunks, last / kTLC + 1);
    }
    const uint16_t* Ab = (const uint16_t*)p.A + (size_t)b * p.sa;
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(Ab, (uint32_t)((size_t)p.M * p.lda * 2));
    const u32x4_t rs0 = rsrc_words((const uint16_t*)p.B0 + (size_t)b * p.sb0,
                                   (uint32_t)((size_t)(kB0LK ? p.L : C::K) * p.ldb0 * 2));
    const u32x4_t rs1 = rsrc_words((const uint16_t*)p.B1 + (size_t)b * p.sb1, (uint32_t)((size_t)p.L * p.ldb1 * 2));

    if (!resident) {
#pragma unroll
      for (int s = 0; s < NS - 1; ++s) issue(s, nseg, rs0, rs1);
    }
    // A fragments of this wave's rows (rows >= M read as zero)
    u32x4_t af[MB][KS];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      const uint32_t row = (uint32_t)(m0 + (wave * MB + rb) * 32 + r32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) af[rb][ks] = buf_load_b128(rsA, (row * p.lda + (uint32_t)(ks * 16 + 8 * h)) * 2);
    }
    // One full wait, on every path, for the A fragments (and the first
    // segments): a wait the compiler placed for the fragments would sit in
    // the segment loop, run every iteration and also drain the ring loads
    // issued just before it. The empty asm keeps the fragment loads above it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    f32x16_t oacc[MB][NB];
    float cst[MB], lsum[MB];   // softmax: integer stabiliser of the row, this lane's part of the unrounded row sum
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[rb][nb] = f32x16_t{0};
      cst[rb] = -INFINITY;
      lsum[rb] = 0.0f;
    }

    const int wrow0 = m0 + wave * MB * 32;
    for (int lc = 0; lc < nseg; ++lc) {
      if (!resident) {
        // segment lc complete in every thread, all reads of segment lc - 1 done
        asm volatile("" ::: "memory");
        wait_vm_lgkm0<(NS - 2) * C::kLoadsAll>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(lc + NS - 1, nseg, rs0, rs1);   // into the buffer of segment lc - 1
      }
      // causal: a wave whose rows see none of the segment skips its arithmetic
      // (it still takes part in the workgroup's barriers and loads)
      if (!kCausal || lc * kTLC <= wrow0 + MB * 32 - 1 + p.coff)
        segment(smem + (lc % NS) * C::kStage, lc, af, oacc, cst, lsum, wrow0);
    }
    if (!resident) {
      // the next tile's first segments reuse the ring
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }

    // ---- normalise and store: oacc[rb][nb][4q + e] is O[m][nb*32 + 8q + 4h + e]
    const uint32_t es = p.out_f32 ? 4u : 2u;
    const __amdgpu_buffer_rsrc_t rsO = make_rsrc((uint8_t*)p.O + (size_t)b * p.so * es,
                                                 (uint32_t)((size_t)p.M * p.ldo * es));
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      float inv = 1.0f;
      const uint32_t row = (uint32_t)(m0 + (wave * MB + rb) * 32 + r32);
      if constexpr (kSoftmax) {
        const float ls = sum_halves(lsum[rb]);
        inv = ls > 0.0f ? 1.0f / ls : 0.0f;   // 0 only for a causal row that sees no key
        // log-sum-exp of the row: sum exp(alpha s) = 2^c * ls
        if (p.row_stats != nullptr && h == 0 && row < (uint32_t)p.M)
          p.row_stats[(size_t)b * p.M + row] = ls > 0.0f ? (cst[rb] + log2f(ls)) * kLn2 : -INFINITY;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb * 32 + 8 * q + 4 * h;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = oacc[rb][nb][4 * q + e] * inv;
          if (p.out_f32) {
            if (p.o_vec) {
              const u32x4_t v = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
              buf_store_b128(v, rsO, (row * p.ldo + (uint32_t)n) * 4);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) buf_store_b32(__float_as_uint(y[e]), rsO, (row * p.ldo + (uint32_t)(n + e)) * 4);
            }
          } else {
            if (p.o_vec) {
              const u32x2_t v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
              buf_store_b64(v, rsO, (row * p.ldo + (uint32_t)n) * 2);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) buf_store_b16((uint16_t)f32_to_bf16(y[e]), rsO, (row * p.ldo + (uint32_t)(n + e)) * 2);
            }
          }
        }
    }
  }
}

typedef short i16x2_t __attribute__((ext_vector_type(2)));

// ---- elementwise F with B0 and B1 resident in LDS (the MLP form)
//
// B0 and B1 are shared by the batch and exactly as long as the ring (L = 256
// for K = N = 64, 192 with one width 128, 128 with both), F is elementwise
// without bias. The weights are loaded once per workgroup; then each wave
// runs its own 32-row blocks with no further barrier:
//  * the first tile's A rows are requested together with the weights, and
//    each tile requests the next tile's rows before its own arithmetic;
//  * the segments are software-pipelined inside the wave: GEMM1 of segment
//    j + 1 is issued between the vector instructions that transform segment j
//    into GEMM2's operand, so the matrix core runs while the wave packs.
// The arithmetic and its order are those of b2b_stream_kernel, except that F
// is applied after the bf16 rounding: kRelu takes the ReLU of the rounded
// pair as a 16-bit signed max with 0 (rounding keeps the sign, so this is the
// rounding of the ReLU; a negative value or -0 becomes +0, a NaN keeps its
// sign's side), and kUnit (alpha = 1) skips the scaling. Built with four
// waves (two workgroups per CU); one eight-wave workgroup per CU, which loads
// the weights into LDS once per CU instead of twice, measured slower.
template <int KS, int NB, bool kB0LK, int kWaves, bool kUnit, bool kRelu>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves), amdgpu_waves_per_eu(2, 2)))
void b2b_mlp_kernel(B2bParams p) {
  using C = TCfg<KS, NB, 1>;
  constexpr int NS = C::kStages;            // segments of L (the host checks L == NS * kTLC)
  constexpr int BM = 32 * kWaves;           // rows per tile, 32 per wave
  constexpr int kThreads = 64 * kWaves;
  constexpr int kLoads = C::kStage / (kThreads * 16);
  static_assert(kLoads * kThreads * 16 == C::kStage, "whole 1 KiB blocks per wave");
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::kLds];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r32 = lane & 31;
  const int mtiles = (p.M + BM - 1) / BM;
  const int ntile = p.batch * mtiles;
  const float scale = p.alpha;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;

  // ---- the weights: load i of wave w fills 1 KiB block q = kWaves i + w of
  // stage s (B0 blocks first), the layouts and swizzles of b2b_stream_kernel
  {
    const u32x4_t rs0 = rsrc_words(p.B0, (uint32_t)((size_t)(kB0LK ? p.L : C::K) * p.ldb0 * 2));
    const u32x4_t rs1 = rsrc_words(p.B1, (uint32_t)((size_t)p.L * p.ldb1 * 2));
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t st = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + (uint32_t)(s * C::kStage))) +
                          (uint32_t)(wave * 1024);
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        lds_dma16(st + i * kWaves * 1024, kWaves * i + wave < C::kB0Blocks ? rs0 : rs1,
                  seg_load_off<KS, NB, kB0LK, kWaves>(p, wave, lane, i, s));
    }
  }

  // ---- fragment read offsets within a stage
  uint32_t b0_rd[kB0LK ? KS : 2], b1_rd[NB];
  stage_read_offsets<KS, NB, kB0LK>(lane, b0_rd, b1_rd);

  // A fragments of tile e for this wave's 32 rows (zero when !ok or past M)
  auto a_load = [&](int e, bool ok, u32x4_t (&af)[KS]) {
    const int b = e / mtiles, mt = e - b * mtiles;
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc((const uint16_t*)p.A + (size_t)b * p.sa,
                                                 (uint32_t)((size_t)p.M * p.lda * 2));
    const uint32_t row = (uint32_t)(mt * BM + wave * 32 + r32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      af[ks] = buf_load_b128(rsA, ok ? (row * p.lda + (uint32_t)(ks * 16 + 8 * h)) * 2 : kOutOfRange);
  };
  u32x4_t af[KS];
  const int G = (int)gridDim.x;
  int e = (int)blockIdx.x;
  a_load(e, e < ntile, af);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // GEMM1 of segment sg (B0 fragments from stage sg) into sx
  auto g1 = [&](int sg, f32x16_t (&sx)[2]) {
    const uint8_t* st = smem + sg * C::kStage;
    u32x4_t bf[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int lb = 0; lb < 2; ++lb) {
        if constexpr (kB0LK) {
          bf[ks][lb] = *(const u32x4_t*)(st + b0_rd[ks] + lb * 32 * C::K * 2);
        } else {
          const u32x2_t lo = lds_read_tr16(st + b0_rd[lb] + ks * 16 * 128);
          const u32x2_t hi = lds_read_tr16(st + b0_rd[lb] + ks * 16 * 128 + 4 * 128);
          bf[ks][lb] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
    for (int lb = 0; lb < 2; ++lb) sx[lb] = f32x16_t{0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int lb = 0; lb < 2; ++lb)
        sx[lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bf[ks][lb]),
                                                         __builtin_bit_cast(bf16x8_t, af[ks]), sx[lb], 0, 0, 0);
  };
  // F of one segment packed as GEMM2's operand: register r of block lb holds
  // l = lb*32 + 8(r>>2) + 4h + (r&3), packed in the k-slot order of GEMM2
  auto tf = [&](const f32x16_t (&sx)[2], u32x4_t (&pf)[4]) {
#pragma unroll
    for (int lb = 0; lb < 2; ++lb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x0 = sx[lb][8 * c + 2 * q], x1 = sx[lb][8 * c + 2 * q + 1];
          uint32_t v = kUnit ? pack_bf16x2(x0, x1) : pack_bf16x2(x0 * scale, x1 * scale);
          if constexpr (kRelu)
            v = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2_t, v), i16x2_t{0, 0}));
          pf[2 * lb + c][q] = v;
        }
  };
  constexpr int kTfValu = (kUnit ? 0 : 32) + 16 + (kRelu ? 16 : 0);   // vector instructions of tf
  // GEMM2 of segment sg (B1 fragments from stage sg) into o
  auto g2 = [&](int sg, const u32x4_t (&pf)[4], f32x16_t (&o)[NB]) {
    const uint8_t* st = smem + sg * C::kStage;
    u32x4_t vf[4][NB];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x2_t lo = lds_read_tr16(st + b1_rd[nb] + c * 16 * C::N * 2);
        const u32x2_t hi = lds_read_tr16(st + b1_rd[nb] + c * 16 * C::N * 2 + 8 * C::N * 2);
        vf[c][nb] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[c][nb]),
                                                        __builtin_bit_cast(bf16x8_t, pf[c]), o[nb], 0, 0, 0);
  };

  for (; e < ntile; e += G) {
    const int en = e + G;
    u32x4_t an[KS];
    a_load(en < ntile ? en : e, en < ntile, an);
    f32x16_t oacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{0};
    f32x16_t s0[2], s1[2];
    u32x4_t pf[4];
    g1(0, s0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      f32x16_t (&cur)[2] = (j & 1) ? s1 : s0;
      f32x16_t (&nxt)[2] = (j & 1) ? s0 : s1;
      if (j + 1 < NS) {
        g1(j + 1, nxt);
        tf(cur, pf);
        // GEMM1's fragment reads first, then its MFMAs one at a time between
        // the transform's vector instructions
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS * (kB0LK ? 1 : 2), 0);
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (kTfValu + 2 * KS - 1) / (2 * KS), 0);
        }
      } else {
        tf(cur, pf);
      }
      g2(j, pf, oacc);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- store: oacc[nb][4q + k] is O[row][nb*32 + 8q + 4h + k] (rows past M
    // are dropped by the range check)
    const int b = e / mtiles, mt = e - b * mtiles;
    const uint32_t es = p.out_f32 ? 4u : 2u;
    const __amdgpu_buffer_rsrc_t rsO = make_rsrc((uint8_t*)p.O + (size_t)b * p.so * es,
                                                 (uint32_t)((size_t)p.M * p.ldo * es));
    const uint32_t row = (uint32_t)(mt * BM + wave * 32 + r32);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nb * 32 + 8 * q + 4 * h;
        const f32x4_t y = {oacc[nb][4 * q], oacc[nb][4 * q + 1], oacc[nb][4 * q + 2], oacc[nb][4 * q + 3]};
        if (p.out_f32) {
          if (p.o_vec) {
            buf_store_b128(__builtin_bit_cast(u32x4_t, y), rsO, (row * p.ldo + (uint32_t)n) * 4);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) buf_store_b32(__float_as_uint(y[k]), rsO, (row * p.ldo + (uint32_t)(n + k)) * 4);
          }
        } else {
          if (p.o_vec) {
            buf_store_b64(u32x2_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])}, rsO, (row * p.ldo + (uint32_t)n) * 2);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) buf_store_b16((uint16_t)f32_to_bf16(y[k]), rsO, (row * p.ldo + (uint32_t)(n + k)) * 2);
          }
        }
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) af[ks] = an[ks];
  }
}

// ---- ping-pong schedule (softmax, no mask, no bias; selected by cf_set_b2b_pingpong)
//
// The softmax of a segment is vector ALU work (an exp per score, slower to
// issue than other vector instructions) about as long as the segment's MFMAs,
// and one wave can only start it once its GEMM1 MFMAs have drained. Here a
// workgroup
// of eight waves runs as two groups of four, waves w and w + 4 sharing a SIMD,
// and every wave alternates an MFMA phase (GEMM2 of the previous segment,
// GEMM1 of this one) and a vector phase (the softmax terms). Group 1 runs one
// phase behind group 0 and a workgroup barrier closes every phase, so on each
// SIMD one wave feeds the matrix core while the other computes exponentials
// (the alternating MFMA/vector wave groups of the method's ping-pong pipeline,
// ComFuse review, "Assumptions & free parameters", Sec. III-C). One workgroup
// fills a CU: 512 rows per tile (64 per wave); the tile's A rows sit in LDS
// (in registers they spilled) beside the ring of B0/B1 segments, which both
// groups share and which streams the segments of the workgroup's successive
// tiles as one sequence.
constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;

template <int KS, int NB, bool kB0LK>
__global__ __attribute__((amdgpu_flat_work_group_size(kPThreads, kPThreads), amdgpu_waves_per_eu(2, 2)))
void b2b_pp_kernel(B2bParams p) {
  constexpr int K = 16 * KS, N = 32 * NB;
  constexpr int MB = 2, BM = kPWaves * MB * 32;
  constexpr int kB0Bytes = kTLC * K * 2, kB1Bytes = kTLC * N * 2;
  constexpr int kStage = kB0Bytes + kB1Bytes;
  constexpr int kB0Blocks = kB0Bytes / 1024;
  constexpr int kLoads = kStage / (kPThreads * 16);        // ring loads per thread per segment
  static_assert(kLoads * kPThreads * 16 == kStage, "whole 1 KiB blocks per wave");
  // LDS: the ring of NS segments, then the tile's A rows (K * 2 bytes each,
  // 16-byte chunks XOR-swizzled by row like B0 given [L][K])
  constexpr int kABytes = BM * K * 2;
  constexpr int kAOff = 160 * 1024 - kABytes;
  constexpr int NS = kAOff / kStage < 8 ? kAOff / kStage : 8;
  static_assert(NS >= 4, "ring of at least four segments");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * kStage + kABytes];
  constexpr int kA = NS * kStage;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int h = lane >> 5, r32 = lane & 31;
  const int mtiles = (p.M + BM - 1) / BM;
  const int nchunks = p.L / kTLC;
  const float scale = p.alpha * kLog2e;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;

  // ring plan: load i of wave w fills 1 KiB block q = 8 i + w of a stage (B0
  // blocks first); the global offsets are recomputed at every issue (a few
  // integer instructions) rather than held in registers across the loop
  auto ring_off = [&](int i, int s) { return seg_load_off<KS, NB, kB0LK, kPWaves>(p, wave, lane, i, s); };
  // segment s (ok: it exists) into ring buffer slot `slot`
  auto issue = [&](int slot, int s, bool ok, const u32x4_t& rs0, const u32x4_t& rs1) {
    const uint32_t sb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + (uint32_t)(slot * kStage)));
    const uint32_t st = sb + (uint32_t)(wave * 1024);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      lds_dma16(st + i * kPWaves * 1024, kPWaves * i + wave < kB0Blocks ? rs0 : rs1, ok ? ring_off(i, s) : kOutOfRange);
  };

  // fragment read offsets within a stage
  uint32_t b0_rd[kB0LK ? KS : 2], b1_rd[NB];
  stage_read_offsets<KS, NB, kB0LK>(lane, b0_rd, b1_rd);
  // A fragment of row block rb, k step ks: row wave*64 + rb*32 + (lane & 31),
  // 8 k from ks*16 + 8h
  uint32_t a_rd[KS];
  {
    const int f = K == 64 ? swz_rows128(r32) : swz_rows256(r32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a_rd[ks] = (uint32_t)(kA + (wave * MB * 32 + r32) * K * 2 + 16 * ((2 * ks + h) ^ f));
  }
  auto afrag = [&](int rb, int ks) -> u32x4_t { return *(const u32x4_t*)(smem + a_rd[ks] + rb * 32 * K * 2); };
  auto b0frag = [&](const uint8_t* st, int ks, int lb) -> u32x4_t {
    if constexpr (kB0LK) {
      return *(const u32x4_t*)(st + b0_rd[ks] + lb * 32 * K * 2);
    } else {
      const u32x2_t lo = lds_read_tr16(st + b0_rd[lb] + ks * 16 * 128);
      const u32x2_t hi = lds_read_tr16(st + b0_rd[lb] + ks * 16 * 128 + 4 * 128);
      return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  auto b1frag = [&](const uint8_t* st, int c, int nb) -> u32x4_t {
    const u32x2_t lo = lds_read_tr16(st + b1_rd[nb] + c * 16 * N * 2);
    const u32x2_t hi = lds_read_tr16(st + b1_rd[nb] + c * 16 * N * 2 + 8 * N * 2);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  };
  auto mfma = [](const u32x4_t& b, const u32x4_t& a, const f32x16_t& acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                    __builtin_bit_cast(bf16x8_t, a), acc, 0, 0, 0);
  };

  // ---- B0/B1 shared by the batch and no longer than the ring: load once
  const bool shared = p.batch == 1 || (p.sb0 == 0 && p.sb1 == 0);
  const bool resident = shared && nchunks <= NS;
  if (resident) {
    const u32x4_t rs0 = rsrc_words(p.B0, (uint32_t)((size_t)(kB0LK ? p.L : K) * p.ldb0 * 2));
    const u32x4_t rs1 = rsrc_words(p.B1, (uint32_t)((size_t)p.L * p.ldb1 * 2));
#pragma unroll
    for (int s = 0; s < NS; ++s) issue(s, s, s < nchunks, rs0, rs1);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // ---- tile schedule (as in b2b_stream_kernel)
  const int G = (int)gridDim.x;
  const bool by_xcd = !shared && mtiles > 1 && (p.batch & 7) == 0 && (G & 7) == 0;
  const int x = (int)blockIdx.x & 7;
  const int per_x = by_xcd ? (x < p.batch ? (p.batch - x + 7) / 8 : 0) * mtiles : p.batch * mtiles;
  const int e0 = by_xcd ? (int)blockIdx.x >> 3 : (int)blockIdx.x;
  const int estep = by_xcd ? G >> 3 : G;

  const int ntiles = per_x > e0 ? (per_x - e0 + estep - 1) / estep : 0;   // tiles of this workgroup
  const int nseg = nchunks;
  auto tile_b = [&](int t) { const int e = e0 + t * estep; return by_xcd ? x + 8 * (e / mtiles) : e / mtiles; };
  auto tile_m0 = [&](int t) { return (e0 + t * estep) % mtiles * BM; };
  // The ring streams the segments of all this workgroup's tiles as one
  // sequence: segment s of tile t is element t * nseg + s, in slot (t * nseg +
  // s) % NS, so the next tile's first segments arrive during the current
  // tile's last phases. (it, is): tile and segment of the next element to issue.
  int it = 0, is = 0, gnext = 0;
  auto issue_next = [&]() {
    const bool ok = it < ntiles;
    const int b = ok ? tile_b(it) : 0;
    const u32x4_t rs0 = rsrc_words((const uint16_t*)p.B0 + (size_t)b * p.sb0,
                                   (uint32_t)((size_t)(kB0LK ? p.L : K) * p.ldb0 * 2));
    const u32x4_t rs1 = rsrc_words((const uint16_t*)p.B1 + (size_t)b * p.sb1, (uint32_t)((size_t)p.L * p.ldb1 * 2));
    issue(gnext % NS, is, ok, rs0, rs1);
    ++gnext;
    if (++is == nseg) { is = 0; ++it; }
  };
  // this wave's MB*32 rows of A of tile t into LDS, 1 KiB (K == 64: 8 rows)
  // per load; rows past M read as zero
  auto load_a = [&](int t) {
    const uint16_t* Ab = (const uint16_t*)p.A + (size_t)tile_b(t) * p.sa;
    const int m0 = tile_m0(t);
    const u32x4_t rsAw = rsrc_words(Ab, (uint32_t)((size_t)p.M * p.lda * 2));
    constexpr int cpr = K / 8, rpl = 64 / cpr, nld = MB * 32 / rpl;
    const uint32_t ab = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + kA + wave * MB * 32 * K * 2));
#pragma unroll
    for (int i = 0; i < nld; ++i) {
      const int rl = i * rpl + lane / cpr, ph = lane % cpr;   // row within the wave's rows
      const int lg = ph ^ (K == 64 ? swz_rows128(rl) : swz_rows256(rl));
      const int row = m0 + wave * MB * 32 + rl;
      lds_dma16(ab + i * 1024, rsAw, row < p.M ? ((uint32_t)row * p.lda + (uint32_t)(8 * lg)) * 2u : kOutOfRange);
    }
  };
  if (ntiles > 0) {
    if (!resident) {
      for (int s = 0; s < NS - 2; ++s) issue_next();
    }
    load_a(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int b = tile_b(t);
    const int m0 = tile_m0(t);
    const int sbase = resident ? 0 : t * nseg;   // ring element of the tile's segment 0
    f32x16_t oacc[MB][NB];
    f32x16_t sacc[MB][2];
    u32x4_t pf[MB][4];
    float cst[MB], lsum[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[rb][nb] = f32x16_t{0};
      cst[rb] = -INFINITY;
      lsum[rb] = 0.0f;
    }

    // Phases: group 0 runs GEMM1(0), softmax(0), GEMM2(0)+GEMM1(1), ...,
    // softmax(nseg-1), GEMM2(nseg-1) in phases 0 .. 2 nseg, group 1 the same
    // one phase later; a workgroup barrier opens every phase (2 nseg + 2 of
    // them, each wave passes all). Stage s is read in phases 2s .. 2s + 3, so
    // at the start of phase 2i (i >= 0) segment i has to be in and the stage
    // of segment i - 2 is refilled with segment i + NS - 2.
    auto phase = [&](int k) {
      asm volatile("" ::: "memory");
      if (!resident && (k & 1) == 0 && k < 2 * nseg) {
        wait_vm_lgkm0<(NS - 3) * kLoads>();   // segment k / 2 landed in this wave's share
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_next();                         // element sbase + k / 2 + NS - 2
      } else {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    };
    // The MFMA phase: GEMM2 of segment j2 (if j2 >= 0) and GEMM1 of segment j1
    // (if j1 >= 0), at raised wave priority. The B1 fragments are read first;
    // each GEMM2 MFMA is then followed by one of GEMM1's LDS reads, so that
    // GEMM1's operands are in when its MFMAs start.
    auto mphase = [&](int j2, int j1) {
      __builtin_amdgcn_s_setprio(1);
      u32x4_t vf[4][NB], bf[KS][2], fa[MB][KS];
      if (j2 >= 0) {
        const uint8_t* st = smem + ((sbase + j2) % NS) * kStage;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) vf[c][nb] = b1frag(st, c, nb);
      }
      if (j1 >= 0) {
        const uint8_t* st = smem + ((sbase + j1) % NS) * kStage;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int lb = 0; lb < 2; ++lb) bf[ks][lb] = b0frag(st, ks, lb);
#pragma unroll
          for (int rb = 0; rb < MB; ++rb) fa[rb][ks] = afrag(rb, ks);
        }
      }
      if (j2 >= 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) oacc[rb][nb] = mfma(vf[c][nb], pf[rb][c], oacc[rb][nb]);
      }
      if (j1 >= 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int lb = 0; lb < 2; ++lb)
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
              sacc[rb][lb] = mfma(bf[ks][lb], fa[rb][ks], ks == 0 ? f32x16_t{0} : sacc[rb][lb]);
      }
      if (j2 >= 0 && j1 >= 0) {
        // 16 LDS reads (B1), then 16 x (GEMM2 MFMA, one GEMM1 read), then GEMM1
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // softmax of a segment: the row extreme only while a row has no
    // stabiliser yet, or when the segment's terms add up past 2^32 (the block
    // is then redone with it; S is still in registers)
    auto softmax = [&]() {
      bool fresh = false;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) fresh |= cst[rb] == -INFINITY;
      const bool full = __builtin_amdgcn_ballot_w64(fresh) != 0;
      float lprev[MB];
      bool big = false;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) {
        if (full) sm_full_rb<NB>(sacc[rb], oacc[rb], cst[rb], lsum[rb], scale);
        lprev[rb] = lsum[rb];
        sm_terms_rb<false>(sacc[rb], pf[rb], cst[rb], lsum[rb], scale);
        big |= !(lsum[rb] - lprev[rb] <= 0x1p32f);
      }
      if (!full && __builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
          lsum[rb] = lprev[rb];
          sm_full_rb<NB>(sacc[rb], oacc[rb], cst[rb], lsum[rb], scale);
          sm_terms_rb<false>(sacc[rb], pf[rb], cst[rb], lsum[rb], scale);
        }
      }
    };
    if (grp == 1) phase(0);
    phase(grp);
    mphase(-1, 0);
    for (int j = 1; j < nseg; ++j) {
      phase(2 * j - 1 + grp);
      softmax();
      phase(2 * j + grp);
      mphase(j - 1, j);
    }
    phase(2 * nseg - 1 + grp);
    if (t + 1 < ntiles) load_a(t + 1);   // this wave's last GEMM1 of the tile is done
    softmax();
    phase(2 * nseg + grp);
    mphase(nseg - 1, -1);
    if (grp == 0) phase(2 * nseg + 1);

    // ---- normalise and store: oacc[rb][nb][4q + e] is O[m][nb*32 + 8q + 4h + e]
    const uint32_t es = p.out_f32 ? 4u : 2u;
    const __amdgpu_buffer_rsrc_t rsO = make_rsrc((uint8_t*)p.O + (size_t)b * p.so * es,
                                                 (uint32_t)((size_t)p.M * p.ldo * es));
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      const uint32_t row = (uint32_t)(m0 + (wave * MB + rb) * 32 + r32);
      const float ls = sum_halves(lsum[rb]);
      const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
      if (p.row_stats != nullptr && h == 0 && row < (uint32_t)p.M)
        p.row_stats[(size_t)b * p.M + row] = ls > 0.0f ? (cst[rb] + log2f(ls)) * kLn2 : -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb * 32 + 8 * q + 4 * h;
          float y[4];
#pragma unroll
          for (int ee = 0; ee < 4; ++ee) y[ee] = oacc[rb][nb][4 * q + ee] * inv;
          if (p.out_f32) {
            if (p.o_vec) {
              const u32x4_t v = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
              buf_store_b128(v, rsO, (row * p.ldo + (uint32_t)n) * 4);
            } else {
#pragma unroll
              for (int ee = 0; ee < 4; ++ee) buf_store_b32(__float_as_uint(y[ee]), rsO, (row * p.ldo + (uint32_t)(n + ee)) * 4);
            }
          } else {
            if (p.o_vec) {
              const u32x2_t v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
              buf_store_b64(v, rsO, (row * p.ldo + (uint32_t)n) * 2);
            } else {
#pragma unroll
              for (int ee = 0; ee < 4; ++ee) buf_store_b16((uint16_t)f32_to_bf16(y[ee]), rsO, (row * p.ldo + (uint32_t)(n + ee)) * 2);
            }
          }
        }
    }
    // the next tile's A rows in (its first phase's barrier follows)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// ---- dispatch
namespace {
template <bool kSoftmax, bool kB0LK, bool kCausal = false, int kBias = 0>
const void* pick_stream_kn(int K, int N, bool two_blocks) {
  if (K == 64 && N == 64) {
    // two row blocks per wave: never with a bias or the causal mask
    if constexpr (kBias == 0 && !kCausal)
      if (two_blocks) return (const void*)&b2b_stream_kernel<4, 2, 2, kSoftmax, kB0LK, kCausal>;
    return (const void*)&b2b_stream_kernel<4, 2, 1, kSoftmax, kB0LK, kCausal, kBias>;
  }
  if (K == 64 && N == 128) return (const void*)&b2b_stream_kernel<4, 4, 1, kSoftmax, kB0LK, kCausal, kBias>;
  if (K == 128 && N == 64) return (const void*)&b2b_stream_kernel<8, 2, 1, kSoftmax, kB0LK, kCausal, kBias>;
  if (K == 128 && N == 128) return (const void*)&b2b_stream_kernel<8, 4, 1, kSoftmax, kB0LK, kCausal, kBias>;
  // the wider GEMM1 (the DLRM widths): A's fragments for all of K stay in
  // registers (64 or 128 VGPRs a wave, so one wave per SIMD at K = 512) and
  // the ring holds two segments
  if (K == 256 && N == 64) return (const void*)&b2b_stream_kernel<16, 2, 1, kSoftmax, kB0LK, kCausal, kBias>;
  if (K == 256 && N == 128) return (const void*)&b2b_stream_kernel<16, 4, 1, kSoftmax, kB0LK, kCausal, kBias>;
  if (K == 512 && N == 64) return (const void*)&b2b_stream_kernel<32, 2, 1, kSoftmax, kB0LK, kCausal, kBias>;
  // N = 256 where two stages fit the LDS (K = 64 keeps the general kernel: its
  // softmax instantiations spill at two waves per SIMD)
  if (K == 128 && N == 256) return (const void*)&b2b_stream_kernel<8, 8, 1, kSoftmax, kB0LK, kCausal, kBias>;
  if (K == 256 && N == 256) return (const void*)&b2b_stream_kernel<16, 8, 1, kSoftmax, kB0LK, kCausal, kBias>;
  if constexpr (kBias == 0)   // two 80 KiB stages fill the LDS; no room for a bias block
    if (K == 512 && N == 128) return (const void*)&b2b_stream_kernel<32, 4, 1, kSoftmax, kB0LK, kCausal, kBias>;
  return nullptr;
}

template <int KS, int NB, bool kUnit, bool kRelu>
const void* pick_mlp_f(const B2bParams& p) {
  return p.b0_lk ? (const void*)&b2b_mlp_kernel<KS, NB, true, 4, kUnit, kRelu>
                 : (const void*)&b2b_mlp_kernel<KS, NB, false, 4, kUnit, kRelu>;
}
template <int KS, int NB>
const void* pick_mlp_kn(const B2bParams& p, int* rows_per_tile, int* threads) {
  if (p.L != TCfg<KS, NB, 1>::kStages * kTLC) return nullptr;
  if (rows_per_tile) *rows_per_tile = 128;
  if (threads) *threads = kTThreads;
  const bool unit = p.alpha == 1.0f, relu = p.act == 1;
  if (unit) return relu ? pick_mlp_f<KS, NB, true, true>(p) : pick_mlp_f<KS, NB, true, false>(p);
  return relu ? pick_mlp_f<KS, NB, false, true>(p) : pick_mlp_f<KS, NB, false, false>(p);
}
const void* pick_mlp(const B2bParams& p, int* rows_per_tile, int* threads) {
  if (p.K == 64 && p.N == 64) return pick_mlp_kn<4, 2>(p, rows_per_tile, threads);
  if (p.K == 64 && p.N == 128) return pick_mlp_kn<4, 4>(p, rows_per_tile, threads);
  if (p.K == 128 && p.N == 64) return pick_mlp_kn<8, 2>(p, rows_per_tile, threads);
  if (p.K == 128 && p.N == 128) return pick_mlp_kn<8, 4>(p, rows_per_tile, threads);
  return nullptr;
}
}  // namespace

const void* b2b_stream_pick(const B2bParams& p, int cus, int* rows_per_tile, int* threads) {
  if (p.L % kTLC != 0 || p.L < kTLC) return nullptr;
  // a bias the ring loads cannot read takes the general kernel
  if (p.bias && !p.bias_vec) return nullptr;
  if (threads) *threads = kTThreads;
  // the ping-pong schedule (when selected): softmax without mask, K = N = 64,
  // and 512-row tiles enough for one workgroup on every CU
  if (p.pingpong && p.row_op == 1 && !p.causal && !p.bias && p.K == 64 && p.N == 64 &&
      (long)p.batch * ((p.M + 511) / 512) >= cus) {
    if (rows_per_tile) *rows_per_tile = 512;
    if (threads) *threads = kPThreads;
    return p.b0_lk ? (const void*)&b2b_pp_kernel<4, 2, true> : (const void*)&b2b_pp_kernel<4, 2, false>;
  }
  // elementwise F without bias, B0/B1 shared by the batch and exactly one ring
  // long: the MLP kernel (128-row tiles)
  if (p.row_op == 0 && !p.causal && !p.bias && (p.batch == 1 || (p.sb0 == 0 && p.sb1 == 0))) {
    const void* k = pick_mlp(p, rows_per_tile, threads);
    if (k) return k;
  }
  // 256-row tiles only when they still give every CU two workgroups, not
  // with a bias (whose registers they have no room for), and not with the
  // causal mask (128-row tiles skip more of the masked work: fewer of their
  // waves sit out a segment on the diagonal, measured about 4 % faster on the
  // attention workload)
  const bool two = !p.bias && !p.causal && p.K == 64 && p.N == 64 && (long)p.batch * ((p.M + 255) / 256) >= 2L * cus;
  const bool sm = p.row_op == 1;
  const void* k;
  if (p.causal)   // keys stored [L, K] (attention); other layouts take the general kernel
    k = p.b0_lk ? pick_stream_kn<true, true, true>(p.K, p.N, two) : nullptr;
  else if (p.bias && p.bias_f32)   // elementwise F only (the softmax takes no bias)
    k = p.b0_lk ? pick_stream_kn<false, true, false, 2>(p.K, p.N, false)
                : pick_stream_kn<false, false, false, 2>(p.K, p.N, false);
  else if (p.bias)
    k = p.b0_lk ? pick_stream_kn<false, true, false, 1>(p.K, p.N, false)
                : pick_stream_kn<false, false, false, 1>(p.K, p.N, false);
  else
    k = sm ? (p.b0_lk ? pick_stream_kn<true, true>(p.K, p.N, two) : pick_stream_kn<true, false>(p.K, p.N, two))
           : (p.b0_lk ? pick_stream_kn<false, true>(p.K, p.N, two) : pick_stream_kn<false, false>(p.K, p.N, two));
  if (k && rows_per_tile) *rows_per_tile = two ? 256 : 128;
  return k;
}

}  // namespace cf
