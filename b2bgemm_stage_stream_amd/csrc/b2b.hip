// Back-to-back GEMM kernels for gfx950: O = F(alpha * A.B0 + bias) . B1.
//
// Method: ComFuse review (pith.science review of arXiv 2608.03537), Referee
// Report major comment 2 (paper Sec. IV-A, Eqs. (2)-(5)) and Fig. 5: the
// intermediate S = A.B0 is transformed tile by tile and consumed by the second
// GEMM from on-chip storage, the second GEMM's contraction over L being
// accumulated segment by segment. The pages spread the segments over a cluster
// of co-scheduled CTAs and merge them through distributed shared memory;
// gfx950 has no clusters, so here one workgroup owns a block of 128 rows of A
// and walks all of L itself in segments of 64, accumulating O in registers.
// That is the same segmented sum, evaluated sequentially, with no exchange
// between workgroups at all.
//
// Any K and N: GEMM1 runs over K in blocks of 16*KS (one pipeline step per
// (segment, k-block), the A fragments of a block reloaded per step when there
// is more than one), and O is split into column blocks of 32*NB, each its own
// workgroup tile; a tile recomputes S and F for its column block (the softmax
// evaluates the same online sequence in every block, so the blocks agree).
//
// Per wave (32 rows m):
//   GEMM1: S^T[l][m] = sum_k B0^T[l][k] A^T[k][m] with v_mfma_f32_32x32x16_bf16
//          (src0 = B0 chunk rows l, src1 = A rows m), so every accumulator
//          register of a lane belongs to row m = lane & 31;
//   F:     alpha, bias[l], ReLU; or the row softmax, evaluated online with an
//          integer (power-of-two) stabiliser c: p = 2^(t - c), t = log2(e) *
//          alpha * S, and every rescale of O and of the row sum by 2^(c_old -
//          c_new) is exact;
//   GEMM2: O^T[n][m] += sum_l B1^T[n][l] P^T[l][m]: the bf16 operand P is
//          packed straight from the GEMM1 accumulators. A lane's registers hold
//          l = 8q + 4h + e (h = lane >> 5) of each 32-block, so the MFMA
//          k-slot j of lane half h stands for l' = 8(j >> 2) + 4h + (j & 3)
//          within a 16-chunk; B1^T is stored in LDS in that permuted order so
//          each lane reads its 8 values with one 16-byte load.
// S and P are never written to memory.
#include <type_traits>

#include "cf_device.hpp"
#include "cf_launch.h"

namespace cf {
namespace {

constexpr int kBM = 128;      // rows of A per workgroup tile (4 waves x 32)
constexpr int kLC = 64;       // L segment (chunk) per pipeline step
constexpr int kThreads = 256;

// Byte offset of 16-byte chunk `c` of row `row` in a row-major LDS tile with
// `cpr` (power of two) chunks per row, XOR-swizzled by the low row bits.
__device__ inline uint32_t swz(int row, int c, int cpr) {
  return (uint32_t)(row * cpr * 16 + ((c ^ (row & (cpr - 1))) << 4));
}


template <int KS, int NB, bool kSoftmax, bool kB0LK>
struct B2bCfg {
  static constexpr int kKpad = 16 * KS;                       // padded K
  static constexpr int kB0Cpr = 2 * KS;                       // 16-B chunks per B0 row (l)
  static constexpr int kB0Bytes = kLC * kKpad * 2;            // B0 chunk [64 l][Kpad]
  static constexpr int kB1Bytes = NB * 32 * kLC * 2;          // B1^T chunk [NB*32 n][64 l]
  static constexpr int kStage = kB0Bytes + kB1Bytes;
  static constexpr int kLds = 2 * kStage;
};

}  // namespace

// kExact: K == 16*KS, N == 32*NB and L a multiple of 64 (no column masks, one
// k-block, one column block).
template <int KS, int NB, bool kSoftmax, bool kB0LK, bool kExact>
__global__ __launch_bounds__(kThreads) void b2b_kernel(B2bParams p) {
  using Cfg = B2bCfg<KS, NB, kSoftmax, kB0LK>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::kLds];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r32 = lane & 31;
  const int mtiles = (p.M + kBM - 1) / kBM;
  const int nblocks = kExact ? 1 : (p.N + 32 * NB - 1) / (32 * NB);   // column blocks of O
  const int tiles = p.batch * mtiles * nblocks;
  const int nchunks = (p.L + kLC - 1) / kLC;
  const int nkb = kExact ? 1 : (p.K + 16 * KS - 1) / (16 * KS);       // k-blocks of GEMM1
  const float scale = kSoftmax ? p.alpha * kLog2e : p.alpha;
  const float floor_v = p.act == 1 ? 0.0f : -INFINITY;

  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int nbk = tile % nblocks, rest = tile / nblocks;
    const int b = rest / mtiles;
    // causal: work grows with the row tile; rotate it by the round when the
    // grid is a multiple of the tiles per batch entry (every workgroup then
    // gets each row position once) and take the tiles that see the most keys
    // first
    int mt = rest - b * mtiles;
    if (p.causal) {
      if (nblocks == 1 && gridDim.x % mtiles == 0) mt = (mt + tile / (int)gridDim.x) % mtiles;
      mt = mtiles - 1 - mt;
    }
    const int m0 = mt * kBM;
    const int n0 = nbk * 32 * NB;   // first column of O in this tile
    // causal: segments past the last key any row of the tile sees are skipped
    int nch = nchunks;
    if (p.causal) {
      const int last = min(m0 + kBM - 1, p.M - 1) + p.coff;
      nch = last < 0 ? 0 : min(nchunks, last / kLC + 1);
    }
    const uint16_t* Ab = (const uint16_t*)p.A + (size_t)b * p.sa;
    const uint16_t* B0b = (const uint16_t*)p.B0 + (size_t)b * p.sb0;
    const uint16_t* B1b = (const uint16_t*)p.B1 + (size_t)b * p.sb1;
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(Ab, (uint32_t)((size_t)p.M * p.lda * 2));
    const __amdgpu_buffer_rsrc_t rsB0 =
        make_rsrc(B0b, (uint32_t)((size_t)(kB0LK ? p.L : p.K) * p.ldb0 * 2));
    const __amdgpu_buffer_rsrc_t rsB1 = make_rsrc(B1b, (uint32_t)((size_t)p.L * p.ldb1 * 2));

    // ---- A fragments of this wave's 32 rows in k-block kb (rows >= M read as
    // zero, k >= K masked)
    u32x4_t af[KS];
    auto load_a = [&](int kb) {
      const uint32_t row = (uint32_t)(m0 + wave * 32 + r32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int k = kb * 16 * KS + ks * 16 + 8 * h;
        if (kExact || k + 8 <= p.K) {
          af[ks] = buf_load_b128(rsA, (row * p.lda + (uint32_t)k) * 2);
        } else {
          u32x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (k + 2 * e < p.K) ? buf_load_b16(rsA, (row * p.lda + (uint32_t)(k + 2 * e)) * 2) : 0u;
            const uint32_t hi = (k + 2 * e + 1 < p.K) ? buf_load_b16(rsA, (row * p.lda + (uint32_t)(k + 2 * e + 1)) * 2) : 0u;
            v[e] = lo | (hi << 16);
          }
          af[ks] = v;
        }
      }
    };
    load_a(0);

    // ---- chunk staging: global -> registers -> LDS (B0 chunk as [l][k], B1^T as [n][perm l])
    // B0 [L][K] (lk): 64 x 2KS chunks of 16 B, thread t takes chunks t + 256 i.
    // B0 [K][L] (kl) and B1 [L][N]: 4x8 blocks (4 rows, 8 contiguous columns)
    // transposed through registers and written as 8-byte pieces.
    constexpr int kB0Chunks = kLC * 2 * KS;                         // lk: 16-B chunks
    constexpr int kB0Blocks = (16 * KS / 4) * (kLC / 8);            // kl: 4 k x 8 l blocks
    constexpr int kB0Regs = kB0LK ? (kB0Chunks + kThreads - 1) / kThreads : 4 * ((kB0Blocks + kThreads - 1) / kThreads);
    constexpr int kB1Blocks = (kLC / 4) * (NB * 4);                  // 4 l x 8 n blocks
    constexpr int kB1Regs = 4 * ((kB1Blocks + kThreads - 1) / kThreads);
    u32x4_t r0[kB0Regs], r1[kB1Regs];

    // one 16-byte row piece of 8 bf16 at element (row, col) of a [rows][ld]
    // matrix; columns >= ncols and (via the range check) rows past the end read
    // as zero
    auto piece = [&](__amdgpu_buffer_rsrc_t rs, int row, int col, uint32_t ld, int ncols) {
      if (kExact || col + 8 <= ncols) return buf_load_b128(rs, ((uint32_t)row * ld + (uint32_t)col) * 2);
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (col + 2 * e < ncols) ? buf_load_b16(rs, ((uint32_t)row * ld + (uint32_t)(col + 2 * e)) * 2) : 0u;
        const uint32_t hi = (col + 2 * e + 1 < ncols) ? buf_load_b16(rs, ((uint32_t)row * ld + (uint32_t)(col + 2 * e + 1)) * 2) : 0u;
        v[e] = lo | (hi << 16);
      }
      return v;
    };

    // pipeline step st = (segment st / nkb, k-block st % nkb): the B0 block of
    // that segment and k-block, and with the last k-block the B1 segment
    auto load_chunk = [&](int st) {
      const int lc = st / nkb, kb = st - lc * nkb;
      const int l0 = lc * kLC, k0 = kb * 16 * KS;
      if constexpr (kB0LK) {
#pragma unroll
        for (int i = 0; i < kB0Regs; ++i) {
          const int id = tid + kThreads * i;
          r0[i] = (id < kB0Chunks) ? piece(rsB0, l0 + id / (2 * KS), k0 + (id % (2 * KS)) * 8, p.ldb0, p.K)
                                   : u32x4_t{0u, 0u, 0u, 0u};
        }
      } else {
#pragma unroll
        for (int bi = 0; bi < kB0Regs / 4; ++bi) {
          const int blk = tid + kThreads * bi;
          const int kq = blk / (kLC / 8), lg = blk % (kLC / 8);
#pragma unroll
          for (int i = 0; i < 4; ++i)   // rows k >= K read as zero (range check)
            r0[4 * bi + i] = (blk < kB0Blocks) ? piece(rsB0, k0 + kq * 4 + i, l0 + lg * 8, p.ldb0, p.L)
                                               : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
      if (kb == nkb - 1) {
#pragma unroll
        for (int bi = 0; bi < kB1Regs / 4; ++bi) {
          const int blk = tid + kThreads * bi;
          const int lq = blk / (NB * 4), ng = blk % (NB * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i)   // rows l >= L read as zero (range check), columns >= N as zero
            r1[4 * bi + i] = (blk < kB1Blocks) ? piece(rsB1, l0 + lq * 4 + i, n0 + ng * 8, p.ldb1, p.N)
                                               : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };

    // column j (0..7) of a 4x8 block held in 4 registers (row i in regs[i], two
    // columns per dword) as 4 consecutive bf16 = one 8-byte piece
    auto column4 = [](const u32x4_t* regs, int j) {
      const int d = j >> 1;
      u32x2_t o;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t a = regs[2 * q][d], c = regs[2 * q + 1][d];
        o[q] = (j & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      return o;
    };

    auto store_chunk = [&](int buf, int st) {
      const bool with_b1 = st % nkb == nkb - 1;
      uint8_t* s0 = smem + buf * Cfg::kStage;
      uint8_t* s1 = s0 + Cfg::kB0Bytes;
      if constexpr (kB0LK) {
#pragma unroll
        for (int i = 0; i < kB0Regs; ++i) {
          const int id = tid + kThreads * i;
          if (id < kB0Chunks)
            *(u32x4_t*)(s0 + swz(id / (2 * KS), id % (2 * KS), Cfg::kB0Cpr)) = r0[i];
        }
      } else {
#pragma unroll
        for (int bi = 0; bi < kB0Regs / 4; ++bi) {
          const int blk = tid + kThreads * bi;
          if (blk < kB0Blocks) {
            const int kq = blk / (kLC / 8), lg = blk % (kLC / 8);
            // row l = 8lg + j of the B0 tile gets k = 4kq .. 4kq+3: half (kq & 1) of chunk kq/2
#pragma unroll
            for (int j = 0; j < 8; ++j)
              *(u32x2_t*)(s0 + swz(lg * 8 + j, kq >> 1, Cfg::kB0Cpr) + 8 * (kq & 1)) = column4(&r0[4 * bi], j);
          }
        }
      }
#pragma unroll
      for (int bi = 0; bi < kB1Regs / 4; ++bi) {
        const int blk = tid + kThreads * bi;
        if (with_b1 && blk < kB1Blocks) {
          const int lq = blk / (NB * 4), ng = blk % (NB * 4);
          // The block holds l' = 4 sub + i (i = 0..3) of 16-chunk c16. Position of
          // l' in the permuted order: 8 ((l' >> 2) & 1) + 4 (l' >> 3) + (l' & 3)
          // = 8 (sub & 1) + 4 (sub >> 1) + i, i.e. 16-B chunk 2 c16 + (sub & 1),
          // byte 8 (sub >> 1).
          const int c16 = lq >> 2, sub = lq & 3;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            *(u32x2_t*)(s1 + swz(ng * 8 + j, 2 * c16 + (sub & 1), 8) + 8 * (sub >> 1)) = column4(&r1[4 * bi], j);
        }
      }
    };

    // ---- accumulators and row state
    f32x16_t oacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x16_t{0};
    float cst = -INFINITY;   // softmax: integer stabiliser of this row (same in both lane halves)
    float lsum = 0.0f;       // softmax: this lane's part of the unrounded row sum

    const int nsteps = nch * nkb;
    if (nsteps > 0) {
      load_chunk(0);
      store_chunk(0, 0);
      if (nsteps > 1) load_chunk(1);
    }
    __syncthreads();

    const int my_row = m0 + wave * 32 + r32;
    f32x16_t sacc[2];
    for (int stp = 0; stp < nsteps; ++stp) {
      const int lc = stp / nkb, kb = stp - lc * nkb;
      const uint8_t* s0 = smem + (stp & 1) * Cfg::kStage;
      const uint8_t* s1 = s0 + Cfg::kB0Bytes;
      if (nkb > 1 && stp > 0) load_a(kb);
      // GEMM1: two 32-blocks of l, accumulated over the k-blocks
#pragma unroll
      for (int lb = 0; lb < 2; ++lb) {
        if (kb == 0) sacc[lb] = f32x16_t{0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4_t bf = *(const u32x4_t*)(s0 + swz(lb * 32 + r32, 2 * ks + h, Cfg::kB0Cpr));
          sacc[lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bf),
                                                              __builtin_bit_cast(bf16x8_t, af[ks]), sacc[lb], 0, 0, 0);
        }
      }
      // the next step's blocks go to the other LDS buffer while this one is consumed
      if (stp + 1 < nsteps) store_chunk((stp + 1) & 1, stp + 1);
      if (stp + 2 < nsteps) load_chunk(stp + 2);
      if (kb != nkb - 1) {
        __syncthreads();
        continue;
      }

      // F on registers; l of register r of block lb: lc*64 + lb*32 + 8(r>>2) + 4h + (r&3)
      const int lbase = lc * kLC + 4 * h;
      u32x4_t pf[4];   // bf16 operand, one u32x4 per 16-chunk of l
      if constexpr (kSoftmax) {
        float mx = -INFINITY;
#pragma unroll
        for (int lb = 0; lb < 2; ++lb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int l = lbase + lb * 32 + 8 * (r >> 2) + (r & 3);
            const bool vis = (kExact || l < p.L) && (!p.causal || l <= my_row + p.coff);
            const float t = vis ? sacc[lb][r] * scale : -INFINITY;
            sacc[lb][r] = t;
            mx = fmaxf(mx, t);
          }
        mx = max_halves(mx);
        const float cn = fmaxf(cst, ceilf(mx));   // -inf only while every l so far is masked
        if (cn > cst && cst != -INFINITY) {
          const int sh = (int)(cst - cn);          // exact power-of-two rescale
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[nb][r] = __builtin_amdgcn_ldexpf(oacc[nb][r], sh);
          lsum = __builtin_amdgcn_ldexpf(lsum, sh);
        }
        cst = cn;
        const float cs = (cst == -INFINITY) ? 0.0f : cst;
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          float e[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            e[r] = fast_exp2(sacc[lb][r] - cs);
            lsum += e[r];
          }
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) pf[2 * lb + c][q] = pack_bf16x2(e[8 * c + 2 * q], e[8 * c + 2 * q + 1]);
        }
      } else {
#pragma unroll
        for (int lb = 0; lb < 2; ++lb) {
          float x[16];
          if (p.bias) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int l = lbase + lb * 32 + 8 * (r >> 2) + (r & 3);
              float bv = 0.0f;
              if (kExact || l < p.L)
                bv = p.bias_f32 ? ((const float*)p.bias)[l] : bf16_to_f32(((const uint16_t*)p.bias)[l]);
              x[r] = fmaxf(__builtin_fmaf(sacc[lb][r], scale, bv), floor_v);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = fmaxf(sacc[lb][r] * scale, floor_v);
          }
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) pf[2 * lb + c][q] = pack_bf16x2(x[8 * c + 2 * q], x[8 * c + 2 * q + 1]);
        }
      }

      // GEMM2: O^T += B1^T P^T over the four 16-chunks of this L segment
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4_t vf = *(const u32x4_t*)(s1 + swz(nb * 32 + r32, 2 * c + h, 8));
          oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf),
                                                              __builtin_bit_cast(bf16x8_t, pf[c]), oacc[nb], 0, 0, 0);
        }
      __syncthreads();
    }

    // ---- normalise and store: oacc[nb][4q + e] is O[m][nb*32 + 8q + 4h + e]
    float inv = 1.0f;
    const uint32_t row = (uint32_t)(m0 + wave * 32 + r32);
    if constexpr (kSoftmax) {
      const float ls = sum_halves(lsum);
      inv = ls > 0.0f ? 1.0f / ls : 0.0f;   // 0 only for a causal row that sees no key
      // log-sum-exp of the row: sum exp(alpha s) = 2^c * ls
      if (p.row_stats != nullptr && nbk == 0 && h == 0 && row < (uint32_t)p.M)
        p.row_stats[(size_t)b * p.M + row] = ls > 0.0f ? (cst + log2f(ls)) * kLn2 : -INFINITY;
    }
    const __amdgpu_buffer_rsrc_t rsO = make_rsrc((uint8_t*)p.O + (size_t)b * p.so * (p.out_f32 ? 4 : 2),
                                                 (uint32_t)((size_t)p.M * p.ldo * (p.out_f32 ? 4 : 2)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + nb * 32 + 8 * q + 4 * h;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = oacc[nb][4 * q + e] * inv;
        if (p.out_f32) {
          if (p.o_vec && n + 4 <= p.N) {
            const u32x4_t v = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
            buf_store_b128(v, rsO, (row * p.ldo + (uint32_t)n) * 4);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              buf_store_b32(__float_as_uint(y[e]), rsO, (n + e < p.N) ? (row * p.ldo + (uint32_t)(n + e)) * 4 : kOutOfRange);
          }
        } else {
          if (p.o_vec && n + 4 <= p.N) {
            const u32x2_t v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            buf_store_b64(v, rsO, (row * p.ldo + (uint32_t)n) * 2);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              buf_store_b16((uint16_t)f32_to_bf16(y[e]), rsO, (n + e < p.N) ? (row * p.ldo + (uint32_t)(n + e)) * 2 : kOutOfRange);
          }
        }
      }
  }
}

namespace {

// Instantiations: KS (K padded to 16*KS) in {1, 2, 4, 8}, NB (N padded to 32*NB)
// in {1, 2, 4}; exact-shape variants for K in {64, 128}, N in {64, 128}.
template <bool kSoftmax, bool kB0LK>
const void* pick_kn(int KS, int NB, bool exact) {
#define CF_B2B_CASE(ks, nb) \
  if (KS == ks && NB == nb) return (const void*)&b2b_kernel<ks, nb, kSoftmax, kB0LK, false>;
#define CF_B2B_EXACT(ks, nb) \
  if (exact && KS == ks && NB == nb) return (const void*)&b2b_kernel<ks, nb, kSoftmax, kB0LK, true>;
  CF_B2B_EXACT(4, 2) CF_B2B_EXACT(4, 4) CF_B2B_EXACT(8, 2) CF_B2B_EXACT(8, 4)
  CF_B2B_CASE(1, 1) CF_B2B_CASE(1, 2) CF_B2B_CASE(1, 4)
  CF_B2B_CASE(2, 1) CF_B2B_CASE(2, 2) CF_B2B_CASE(2, 4)
  CF_B2B_CASE(4, 1) CF_B2B_CASE(4, 2) CF_B2B_CASE(4, 4)
  CF_B2B_CASE(8, 1) CF_B2B_CASE(8, 2) CF_B2B_CASE(8, 4)
#undef CF_B2B_CASE
#undef CF_B2B_EXACT
  return nullptr;
}

// K above 128 runs in k-blocks of 128, N above 128 in column blocks of 128
int ks_of(int K) { return K <= 16 ? 1 : K <= 32 ? 2 : K <= 64 ? 4 : 8; }
int nb_of(int N) { return N <= 32 ? 1 : N <= 64 ? 2 : 4; }

const void* pick(const B2bParams& p) {
  const int KS = ks_of(p.K), NB = nb_of(p.N);
  if (!KS || !NB) return nullptr;
  const bool sm = p.row_op == 1;
  const bool exact = p.K == 16 * KS && p.N == 32 * NB && p.L % kLC == 0;
  if (sm) return p.b0_lk ? pick_kn<true, true>(KS, NB, exact) : pick_kn<true, false>(KS, NB, exact);
  return p.b0_lk ? pick_kn<false, true>(KS, NB, exact) : pick_kn<false, false>(KS, NB, exact);
}

}  // namespace

bool b2b_supported(const B2bParams& p) {
  if (p.row_op != 0 && p.row_op != 1) return false;
  if (p.K < 1 || p.L < 1 || p.N < 1) return false;
  // 32-bit buffer offsets within one batch
  const uint64_t lim = 1ull << 31;
  if ((uint64_t)(p.M + kBM) * p.lda * 2 >= lim) return false;
  if ((uint64_t)(p.b0_lk ? p.L + kLC : p.K + 128) * p.ldb0 * 2 >= lim) return false;
  if ((uint64_t)(p.L + kLC) * p.ldb1 * 2 >= lim) return false;
  if ((uint64_t)(p.M + kBM) * p.ldo * 4 >= lim) return false;
  return pick(p) != nullptr;
}

hipError_t launch_b2b(const B2bParams& p, hipStream_t stream) {
  int cus = 0, per_cu = 0;
  hipError_t e;
  if ((e = device_cus_cached(&cus)) != hipSuccess) return e;
  int bm = kBM, threads = kThreads;
  const void* ks = b2b_stream_pick(p, cus, &bm, &threads);
  const void* k = ks ? ks : pick(p);
  if (!k) return hipErrorNotSupported;
  if ((e = blocks_per_cu_cached(k, threads, &per_cu)) != hipSuccess) return e;
  // the general kernel's tiles also run over the column blocks of O
  const long nblocks = ks ? 1 : (p.N + 32 * nb_of(p.N) - 1) / (32 * nb_of(p.N));
  const long tiles = (long)p.batch * ((p.M + bm - 1) / bm) * nblocks;
  const long cap = (long)(per_cu > 0 ? per_cu : 1) * cus;
  long g = tiles < cap ? tiles : cap;
  if (ks && g >= 8) g -= g % 8;   // the streamed kernel maps workgroups to XCDs in groups of 8
  const int grid = (int)g;
  void* args[] = {(void*)&p};
  return hipLaunchKernel(k, dim3(grid), dim3(threads), args, 0, stream);
}

}  // namespace cf
