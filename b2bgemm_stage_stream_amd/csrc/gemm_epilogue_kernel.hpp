// Persistent GEMM + epilogue kernel for gfx950 (Stage-Stream execution).
// Template definitions; instantiated by gemm_epilogue_inst.hip.
//
// Method: ComFuse review (pith.science review of arXiv 2608.03537), "What
// carries the argument" and Fig. 3/Fig. 4: the accumulator tiles of P = A.B
// stream through the elementwise epilogue nodes while still on chip; a row
// reduction is a stage boundary resolved by a three-level aggregation. By the
// review's reading of Eq. (1) (Referee Report, major comment 1) a reduction
// over the columns of row m only needs the tiles T_{m,n} that share m.
//
// MI355X design:
//  * one workgroup (4 waves) owns a 256x256 output tile; each wave a 128x128
//    quarter held as 4x4 fp32 32x32 MFMA accumulators (256 AGPRs per lane);
//  * operands go HBM -> VGPR -> LDS (double buffered, 2 x 64 KiB), B is
//    transposed on the way in when stored [K, N], and the tiles use an XOR
//    swizzle of their 16-byte chunks; MFMA src0 is the B tile and src1 the A
//    tile, so each lane's accumulator registers all belong to one output row m
//    (lane & 31) and the row reduction is mostly in-lane;
//  * reduction level 1: in-lane over 64 registers, then across the two lane
//    halves with v_permlane32_swap; level 2: the two waves that share rows
//    merge through LDS; level 3: the workgroups of one row strip exchange
//    per-row partial statistics through an epoch-tagged workspace in device
//    memory (the pages use distributed shared memory inside a thread block
//    cluster; gfx950 has no clusters, so this goes through L2/MALL);
//  * the grid is persistent and never larger than the number of co-resident
//    workgroups, and it is a multiple of the strip width, so every strip is
//    processed by simultaneously resident workgroups in one round;
//  * the partial statistics are merged in a fixed order, so all workgroups of
//    a strip compute bit-identical row statistics and results are
//    deterministic.
// P itself is never written to memory.
#pragma once

#include "cf_device.hpp"
#include "cf_launch.h"

#include <type_traits>

namespace cf {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;                   // one LDS tile row: 8 chunks of 16 bytes
constexpr int kTileBytes = kGemmBM * kRowBytes;  // 32 KiB per operand tile (BM == BN)

template <bool kF32> struct In;
template <> struct In<false> { static constexpr int kChunk = 8; static constexpr int kSize = 2; };
template <> struct In<true>  { static constexpr int kChunk = 4; static constexpr int kSize = 4; };

__device__ inline uint32_t swz(int row, int chunk) { return (uint32_t)(row * kRowBytes + ((chunk ^ (row & 7)) << 4)); }

// ----------------------------------------------------------------------------- operand loads
// Global -> registers for one k-tile (BK = 8 chunks of 16 bytes) of a [rows][k]
// operand (A, or B stored [N, K]). Thread t covers chunk (t & 7) of rows
// (t >> 3) + 32 i. `off` is this thread's byte offset of row (t >> 3), chunk
// (t & 7) at k-tile start; rows past the end of the buffer read as zero (buffer
// range check); chunks past K are zeroed here (only in the last k-tile).
template <bool kF32, bool kVec>
__device__ inline void load_rowmajor(u32x4_t (&regs)[8], __amdgpu_buffer_rsrc_t rs, uint32_t off,
                                     uint32_t row_step, int kc, int K, uint32_t ld, uint32_t row0, int tid) {
  if constexpr (kVec) {
#pragma unroll
    for (int i = 0; i < 8; ++i) regs[i] = buf_load_b128(rs, off + (uint32_t)i * row_step);
    if (kc >= K) {
#pragma unroll
      for (int i = 0; i < 8; ++i) regs[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  } else {
    constexpr int S = In<kF32>::kSize;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t row = row0 + (uint32_t)((tid >> 3) + 32 * i);
      u32x4_t v;
      if constexpr (kF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = buf_load_b32(rs, (row * ld + (uint32_t)(kc + e)) * S);
          v[e] = (kc + e < K) ? x : 0u;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = buf_load_b16(rs, (row * ld + (uint32_t)(kc + 2 * e)) * S);
          const uint32_t hi = buf_load_b16(rs, (row * ld + (uint32_t)(kc + 2 * e + 1)) * S);
          v[e] = ((kc + 2 * e < K) ? lo : 0u) | ((kc + 2 * e + 1 < K) ? (hi << 16) : 0u);
        }
      }
      regs[i] = v;
    }
  }
}

__device__ inline void store_rowmajor(const u32x4_t (&regs)[8], uint8_t* tile, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *(u32x4_t*)(tile + swz((tid >> 3) + 32 * i, tid & 7)) = regs[i];
}

// B stored [K, N]: load a k-tile x 256 columns, to be transposed into the LDS
// tile [n][k]. bf16: thread t owns the 8x8 block (k: 8*(t&7) + i, n: 8*(t>>3) + j),
// so the 8 lanes that share an LDS row write its 8 distinct 16-byte chunks.
// fp32: thread t owns two 4x4 blocks (k: 4*((t&3) + 4*b) + i, n: 4*(t>>2) + j).
// `off` is the byte offset of (k-tile start + first k of the thread, first n of
// the thread). Rows k >= K read as zero (range check); columns >= N hold
// values of other columns and only reach output columns that are never stored
// and are excluded from the row statistics.
template <bool kF32, bool kVec>
__device__ inline void load_kn(u32x4_t (&regs)[8], __amdgpu_buffer_rsrc_t rs, uint32_t off,
                               uint32_t ldbytes, int n, int N) {
  constexpr int S = In<kF32>::kSize;
  if constexpr (kVec) {
    if constexpr (!kF32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) regs[i] = buf_load_b128(rs, off + (uint32_t)i * ldbytes);
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) regs[4 * b + i] = buf_load_b128(rs, off + (uint32_t)(16 * b + i) * ldbytes);
    }
  } else {
    constexpr int R = kF32 ? 4 : 8;      // k rows per block
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ro = off + (uint32_t)((kF32 ? 16 * (i / 4) + (i % 4) : i)) * ldbytes;
      u32x4_t v;
      if constexpr (kF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = buf_load_b32(rs, ro + (uint32_t)e * S);
          v[e] = (n + e < N) ? x : 0u;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = buf_load_b16(rs, ro + (uint32_t)(2 * e) * S);
          const uint32_t hi = buf_load_b16(rs, ro + (uint32_t)(2 * e + 1) * S);
          v[e] = ((n + 2 * e < N) ? lo : 0u) | ((n + 2 * e + 1 < N) ? (hi << 16) : 0u);
        }
      }
      regs[i] = v;
      (void)R;
    }
  }
}

template <bool kF32>
__device__ inline void store_kn(const u32x4_t (&regs)[8], uint8_t* tile, int tid) {
  if constexpr (!kF32) {
    const int ng = tid >> 3, kg = tid & 7;
    // regs[i] holds k = 8kg + i, columns n = 8ng + 2d, 8ng + 2d + 1 in dword d.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = j >> 1;
      u32x4_t o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = regs[2 * p][d], b = regs[2 * p + 1][d];
        o[p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      *(u32x4_t*)(tile + swz(ng * 8 + j, kg)) = o;
    }
  } else {
    const int ng = tid >> 2;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int kg = (tid & 3) + 4 * b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t o;
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = regs[4 * b + p][j];
        *(u32x4_t*)(tile + swz(ng * 4 + j, kg)) = o;
      }
    }
  }
}

template <bool kF32>
__device__ inline void mfma(f32x16_t& acc, const u32x4_t& src0, const u32x4_t& src1) {
  if constexpr (!kF32) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, src0),
                                                  __builtin_bit_cast(bf16x8_t, src1), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(src0[j]), __uint_as_float(src1[j]),
                                                 acc, 0, 0, 0);
  }
}

// ----------------------------------------------------------------------------- bf16 streaming main loop
// bf16 operands, whole 16-byte accesses and K a multiple of 32: the operands go
// straight from memory into LDS (buffer_load_dwordx4 ... lds, no VGPR staging)
// through a ring of kStages stages of 32 k each; the loads of a stage are
// issued between kStages - 2 and kStages - 1 iterations before the MFMAs
// consume it.
//
// Stage layout (32 KiB): A [256 m][64 B] then B. B given [N, K] is stored like
// A ([256 n][64 B]); B given [K, N] stays [32 k][512 B] and the MFMA operand is
// read with ds_read_b64_tr_b16, which hands lane i of each 16-lane group the
// column i of the 4 x 16 block whose 8-byte row pieces the group addressed.
//
// One load instruction of a wave fills 1 KiB of LDS contiguously (lane l at
// +16 l), so the bank swizzle is applied on the global side: lane l loads the
// logical 16-byte chunk that belongs at its physical position.
//  * 64-byte rows: physical chunk = logical ^ swz64(row); conflict free for the
//    MFMA reads whether the LDS serves 8 or 16 lanes of a 16-byte read per cycle.
//  * 512-byte B rows: physical chunk = logical ^ swz512(k); the 4 rows a 16-lane
//    transposed read touches land in distinct banks.
constexpr int kStageK = 32;
constexpr int kStages = 4;
constexpr int kStageBytes = 2 * kGemmBM * kStageK * 2;   // A + B, 32 KiB
constexpr int kStageB = kGemmBM * kStageK * 2;           // offset of B in a stage
static_assert(kStages * kStageBytes <= 160 * 1024, "LDS ring exceeds 160 KiB");

__device__ inline int swz64(int row) { return (((row >> 1) ^ (row >> 3)) & 1) | ((row >> 1) & 2); }
__device__ inline int swz512(int k) { const int j = k & 3; return (2 * j) ^ (4 * j); }

// `tid` is threadIdx.x passed through an opaque copy made per output tile, so
// that the per-lane offsets below are computed per tile instead of being
// hoisted out of the persistent loop (where they would be spilled and reloaded
// inside the k loop).
//
// Schedule of iteration kt (stage kt in LDS, 32 k = two k16 steps):
//   phase A: 16 MFMAs of step 0, the fragment reads of step 1, and the four A
//            loads of stage kt + kStages - 1 (one per 4 MFMAs);
//   wait until stage kt + 1 has landed, barrier;
//   phase B: 16 MFMAs of step 1, the fragment reads of step 0 of stage kt + 1,
//            and the four B loads of stage kt + kStages - 1.
// Stage kt + kStages - 1 goes into the buffer of stage kt - 1, whose last reads
// finished before the previous barrier, so the refill of a stage spreads over a
// whole iteration. Loads of stages past the end use an out-of-range offset
// (nothing is fetched) so that every iteration issues the same number of loads
// and the vmcnt thresholds stay constant.
template <bool kBnk>
__device__ inline void mainloop_stream(f32x16_t (&acc)[4][4], const GemmEpilogueParams& p, uint8_t* smem,
                                        int m0, int n0, int tid) {
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r32 = lane & 31;
  const int KT = p.K / kStageK;
  const u32x4_t rsA = rsrc_words(p.A, p.a_bytes), rsB = rsrc_words(p.B, p.b_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)smem;
  uint32_t ga[4], gb[4];
  {
    const int ra = lane >> 2, ca = (lane & 3) ^ swz64(lane >> 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * (4 * wave + i) + ra;
      ga[i] = ((uint32_t)(m0 + row) * p.lda + (uint32_t)(8 * ca)) * 2u;
      if constexpr (kBnk) {
        gb[i] = ((uint32_t)(n0 + row) * p.ldb + (uint32_t)(8 * ca)) * 2u;
      } else {
        const int kr = 2 * (4 * wave + i) + (lane >> 5);
        const int cb = (lane & 31) ^ swz512(kr);
        gb[i] = ((uint32_t)kr * p.ldb + (uint32_t)(n0 + 8 * cb)) * 2u;
      }
    }
  }
  const uint32_t a_step = kStageK * 2u;
  const uint32_t b_step = kBnk ? kStageK * 2u : (uint32_t)kStageK * p.ldb * 2u;
  // load j (0..3 A, 4..7 B) of stage s; stages past the end read out of range
  auto dma = [&](int s, int j) {
    const uint32_t st = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds0 + (uint32_t)((s % kStages) * kStageBytes + wave * 4096)));
    const bool ok = s < KT;
    if (j < 4) lds_dma16(st + j * 1024, rsA, ok ? ga[j] + (uint32_t)s * a_step : kOutOfRange);
    else lds_dma16(st + kStageB + (j - 4) * 1024, rsB, ok ? gb[j - 4] + (uint32_t)s * b_step : kOutOfRange);
  };
  const int sa = swz64(r32);
  const uint32_t a_rd[2] = {(uint32_t)((wm * 128 + r32) * 64 + 16 * ((0 + h) ^ sa)),
                            (uint32_t)((wm * 128 + r32) * 64 + 16 * ((2 + h) ^ sa))};
  const uint32_t bn_rd[2] = {(uint32_t)(kStageB + (wn * 128 + r32) * 64 + 16 * ((0 + h) ^ sa)),
                             (uint32_t)(kStageB + (wn * 128 + r32) * 64 + 16 * ((2 + h) ^ sa))};
  uint32_t bt_rd[4];
  {
    const int g = lane >> 4, i = lane & 15;
    const int f = swz512(i >> 2);
    const int c = 2 * (g & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int phys = wn * 16 + ((nb * 4 + c) ^ f);
      bt_rd[nb] = (uint32_t)(kStageB + (8 * (g >> 1) + (i >> 2)) * 512 + 16 * phys + 8 * (i & 1));
    }
  }
  // fragment reads of one k16 step as a sequence of ops, B first:
  //  !kBnk: ops 0..7 B halves (nb = op/2), 8..11 A;  kBnk: 0..3 B, 4..7 A
  constexpr int kOps = kBnk ? 8 : 12;
  struct Frags { u32x4_t a[4]; u32x2_t blo[4], bhi[4]; u32x4_t b[4]; };
  auto read_op = [&](Frags& f, const uint8_t* st, int kk, int op) {
    if constexpr (kBnk) {
      if (op < 4) f.b[op] = *(const u32x4_t*)(st + bn_rd[kk] + op * 32 * 64);
      else f.a[op - 4] = *(const u32x4_t*)(st + a_rd[kk] + (op - 4) * 32 * 64);
    } else {
      if (op < 8) {
        const int nb = op >> 1;
        const uint8_t* q = st + bt_rd[nb] + kk * 16 * 512 + (op & 1) * 4 * 512;
        if (op & 1) f.bhi[nb] = lds_read_tr16(q); else f.blo[nb] = lds_read_tr16(q);
      } else {
        f.a[op - 8] = *(const u32x4_t*)(st + a_rd[kk] + (op - 8) * 32 * 64);
      }
    }
  };
  auto bfrag = [&](const Frags& f, int nb) -> u32x4_t {
    if constexpr (kBnk) return f.b[nb];
    else return u32x4_t{f.blo[nb][0], f.blo[nb][1], f.bhi[nb][0], f.bhi[nb][1]};
  };
  // one phase: 16 MFMAs on `use`, the kOps reads of `nxt` (if st_rd) and 4 DMAs
  auto phase = [&](auto rd, const Frags& use, Frags& nxt, const uint8_t* st_rd, int kk_rd, int s_dma, int j0) {
    constexpr bool kRead = decltype(rd)::value;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      dma(s_dma, j0 + g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        mfma<false>(acc[g][nb], bfrag(use, nb), use.a[g]);
        constexpr int per = kOps / 4;
        if (kRead && nb < per) read_op(nxt, st_rd, kk_rd, g * per + nb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (KT == 0) return;
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) dma(s, j);
  wait_vm_lgkm0<(kStages - 2) * 8>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  Frags f0, f1;
#pragma unroll
  for (int op = 0; op < kOps; ++op) read_op(f0, smem, 0, op);
  for (int kt = 0; kt + 1 < KT; ++kt) {
    // phase A: MFMAs of (kt, k16 step 0); reads of (kt, step 1); A loads of stage kt + kStages - 1
    phase(std::true_type{}, f0, f1, smem + (kt % kStages) * kStageBytes, 1, kt + kStages - 1, 0);
    asm volatile("" ::: "memory");
    wait_vm_lgkm0<(kStages - 3) * 8 + 4>();     // stage kt + 1 complete
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // phase B: MFMAs of (kt, step 1); reads of (kt + 1, step 0); B loads of stage kt + kStages - 1
    phase(std::true_type{}, f1, f0, smem + ((kt + 1) % kStages) * kStageBytes, 0, kt + kStages - 1, 4);
  }
  {
    const int kt = KT - 1;
    phase(std::true_type{}, f0, f1, smem + (kt % kStages) * kStageBytes, 1, kt + kStages - 1, 0);
    phase(std::false_type{}, f1, f0, smem, 0, kt + kStages - 1, 4);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// ----------------------------------------------------------------------------- epilogue helpers
__device__ inline float load_vec(const void* p, int n, int is_f32) {
  return is_f32 ? ((const float*)p)[n] : bf16_to_f32(((const uint16_t*)p)[n]);
}

// Strip exchange word: low 32 bits value, high 32 bits epoch tag. Agent-scope
// atomics make each word visible across XCDs without an L2-wide flush, and the
// tag in the same word makes every value self-validating.
__device__ inline void publish(uint64_t* slot, float v, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
  __hip_atomic_store(slot, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// ----------------------------------------------------------------------------- epilogue
// Accumulator layout: acc[mb][nb][4q + e] of a lane belongs to output element
//   (m0 + ml, n0 + nl + e),  ml = wm*128 + mb*32 + (lane & 31),
//   nl = wn*128 + nb*32 + 8q + 4h,  h = lane >> 5.
// All 16 accumulator registers a lane holds in one column block nb of one
// row block mb belong to the same output row, so the row reduction is in-lane
// (64 values per row block), then across the two lane halves.
//
// The epilogue streams over the accumulators (which stay in AGPRs) once per
// pass, recomputing the elementwise stage x = act(alpha * P + bias + R) each
// time instead of writing it back. Each group of 4 accumulators is read with
// an asm v_accvgpr_read whose extra input is a value computed from the
// previous group; this keeps the reads in stream order so that only a few
// accumulators live in VGPRs at a time.
//
// LDS use after the main loop (the operand tiles are dead by then):
// the small arrays come first so that every per-group access is a base
// register plus an immediate offset below 64 KiB
constexpr int kOffVec = 0;                       // bias, gamma, beta: [3][256] f32
constexpr int kOffWpart = kOffVec + 3 * 1024;    // [2][256] float2: partial per wave column
constexpr int kOffRstat = kOffWpart + 4096;      // [256] float2: final row statistics
constexpr int kOffRes = kOffRstat + 2048;        // staged residual tile
constexpr int kResStride = 528;                  // bytes per staged residual row (256 bf16 + 16 B pad)
constexpr int kLdsEpilogue = kOffRes + 256 * kResStride;
// second row stage (two-stage instantiations only): gamma2, beta2 [2][256]
// f32, then its row statistics [256] float2
constexpr int kOffTwo = kLdsEpilogue;
constexpr int kLdsTwo = kOffTwo + 2 * 1024 + 2048;

// Four accumulators of block `blk`, registers 4q..4q+3, read into VGPRs after
// `tok` is available.
template <int Q>
__device__ inline void acc_read4(const f32x16_t& blk, float tok, float (&v)[4]) {
  asm("v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\t"
      "v_accvgpr_read_b32 %2, %6\n\tv_accvgpr_read_b32 %3, %7"
      : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3])
      : "a"(blk[4 * Q]), "a"(blk[4 * Q + 1]), "a"(blk[4 * Q + 2]), "a"(blk[4 * Q + 3]), "v"(tok));
}

// Top-k lists: L (value, column) pairs sorted by value descending, equal
// values by column ascending (L = 8, or 4 when k <= 4). An empty entry is
// (-inf, kNoColumn); it ranks below every real entry, -inf included. NaN is
// mapped to -inf by the caller.
constexpr int kNoColumn = 0x7fffffff;

// Inserts a candidate whose column is larger than every column the list holds
// (a lane visits its columns in increasing order), so an equal value never
// moves ahead. Every position is updated at once from the old list: g[j] says
// the candidate ranks before entry j (monotone in j), entry j becomes the
// candidate where g[j] first holds and entry j-1 after that; its value is the
// median of (old j, candidate, old j-1), which is that choice for a sorted
// list. kMaybeEmpty: the list may still hold empty entries, which any
// candidate with a column displaces. No branches and no chain through the
// positions.
template <bool kMaybeEmpty, int L>
__device__ inline void topk_insert_next(float (&tv)[L], int (&tc)[L], float cv, int cc) {
  bool g[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    g[j] = cv > tv[j];
    if constexpr (kMaybeEmpty) g[j] = g[j] | (tc[j] == kNoColumn);
  }
#pragma unroll
  for (int j = L - 1; j > 0; --j) {
    tc[j] = g[j] ? (g[j - 1] ? tc[j - 1] : cc) : tc[j];
    tv[j] = __builtin_amdgcn_fmed3f(tv[j], cv, tv[j - 1]);
  }
  tc[0] = g[0] ? cc : tc[0];
  tv[0] = fmaxf(tv[0], cv);
}

// (va, ca) ranks before (vb, cb): larger value, or equal value and smaller column.
__device__ inline bool topk_before(float va, int ca, float vb, int cb) {
  return (va > vb) | ((va == vb) & (ca < cb));
}

// Merges list (bv, bc) into (tv, tc), keeping the L best of the union: the
// elementwise better of a[i] and b[L-1-i] is the union's best L as a bitonic
// sequence, which log2(L) half-cleaner stages sort.
template <int L>
__device__ inline void topk_merge(float (&tv)[L], int (&tc)[L], const float (&bv)[L], const int (&bc)[L]) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool b = topk_before(bv[L - 1 - i], bc[L - 1 - i], tv[i], tc[i]);
    tv[i] = b ? bv[L - 1 - i] : tv[i];
    tc[i] = b ? bc[L - 1 - i] : tc[i];
  }
#pragma unroll
  for (int d = L / 2; d > 0; d >>= 1) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if ((i & d) == 0) {
        const bool sw = topk_before(tv[i + d], tc[i + d], tv[i], tc[i]);
        const float v0 = tv[i], v1 = tv[i + d];
        const int c0 = tc[i], c1 = tc[i + d];
        tv[i] = sw ? v1 : v0;
        tc[i] = sw ? c1 : c0;
        tv[i + d] = sw ? v0 : v1;
        tc[i + d] = sw ? c0 : c1;
      }
    }
  }
}

// (n, mean, M2) merge of two partial statistics (Chan et al.'s pairwise update).
__device__ inline void chan_merge(float& n, float& mean, float& m2, float nb, float meanb, float m2b) {
  const float nn = n + nb;
  if (nn > 0.0f) {
    const float d = meanb - mean;
    mean = mean + d * (nb / nn);
    m2 = m2 + m2b + d * d * (n * nb / nn);
  }
  n = nn;
}

// Lane l receives the value of lane l ^ X of its own 32-lane half
// (ds_swizzle in bit-mask mode: and 0x1f, or 0, xor X).
template <int X>
__device__ inline float xor_lanes(float v) {
  static_assert(X > 0 && X < 32, "xor within a 32-lane half");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (X << 10)));
}

// Values of the two lane halves: .x from lane (l & 31), .y from lane (l | 32).
__device__ inline float2 halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ROW: 0 none, 1 softmax, 2 LayerNorm, 3 RMSNorm, 4 argmax, 5 top-k (cf_row_op); 6 top-k with k <= 4.
// kFast: 16-byte accesses are allowed, N is a multiple of 8 and the residual
// (if any) is bf16; otherwise every column is masked against N, element by
// element.
// kRagged (with kFast): the column tile extends past N; the row statistics
// skip the columns >= N and the 16-byte stores of those columns are dropped
// (N a multiple of 8: a 4- or 8-column group is valid or invalid as a whole).
// kPre: a bias or a residual is present.
// kId: alpha == 1 and no activation, so the elementwise stage is P (+ bias + R).
// ROW2 (with ROW 1-3): a second row stage (1 softmax, 2 LayerNorm, 3 RMSNorm;
// 0 none) acts on the first stage's output y over the same row, with its own
// statistics pass over y and its own strip exchange (slots p.ws_slots2).
// Every choice inside the per-group code is a compile-time one: run-time
// conditions there cost scalar registers that the epilogue does not have.
template <int ROW, bool kFast, bool kPre, bool kId, bool kRagged = false, int ROW2 = 0>
__device__ inline __attribute__((always_inline)) void epilogue(const f32x16_t (&acc)[4][4], const GemmEpilogueParams& p, uint8_t* smem,
                                int strip, int tn, uint32_t tag, bool& timed_out, int tid) {
  // top-k (ROW 5: lists of 8; ROW 6: lists of 4, for k <= 4)
  constexpr bool kTop = ROW == 5 || ROW == 6;
  constexpr int kL = ROW == 6 ? 4 : 8;
  // column reductions (ROW 7, 8, 9: softmax, LayerNorm, RMSNorm over the rows
  // m of each column n): the statistics are per column, and the exchange runs
  // over the tiles of the tile column (the complementary strip)
  constexpr bool kCol = ROW >= 7 && ROW <= 9;
  constexpr int R = kCol ? ROW - 6 : ROW;   // the reduction's operation (1-3 as for rows)
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int m0 = strip * kGemmBM, n0 = tn * kGemmBN;
  const __amdgpu_buffer_rsrc_t rsC = make_rsrc(p.C, p.c_bytes);

  float* vbias = (float*)(smem + kOffVec);
  float* vgamma = vbias + 256;
  float* vbeta = vgamma + 256;
  float2* wpart = (float2*)(smem + kOffWpart);
  float2* rstat = (float2*)(smem + kOffRstat);
  {
    const int n = n0 + tid;
    const bool ok = n < p.N;
    vbias[tid] = (p.bias && ok) ? load_vec(p.bias, n, p.vec_f32) : 0.0f;
    vgamma[tid] = (p.gamma && ok) ? load_vec(p.gamma, n, p.vec_f32) : 1.0f;
    vbeta[tid] = (p.beta && ok) ? load_vec(p.beta, n, p.vec_f32) : 0.0f;
  }
  // top-k takes no residual (its lists use the residual staging area)
  const bool has_res = !kTop && p.residual != nullptr;
  const __amdgpu_buffer_rsrc_t rsR = make_rsrc(p.residual, has_res ? p.r_bytes : 0u);
  if (kFast && has_res) {
    // stage the bf16 residual tile [256][256] in LDS with coalesced 16-byte loads;
    // rows >= M read as zero
    const int c = tid & 31;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      u32x4_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 5) + 8 * (8 * b + i);
        v[i] = buf_load_b128(rsR, ((uint32_t)(m0 + row) * p.ldr + (uint32_t)(n0 + c * 8)) * 2);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 5) + 8 * (8 * b + i);
        *(u32x4_t*)(smem + kOffRes + row * kResStride + c * 16) = v[i];
      }
    }
  }
  __syncthreads();

  const float alpha = p.alpha;
  const float floor_v = p.act == 1 ? 0.0f : -INFINITY;   // ReLU as max with a floor
  const int ncol = p.N - (n0 + wn * 128 + 4 * h);          // element (c = nb*32 + 8q + e) valid iff c < ncol
  // Per-lane LDS bases: every per-group access below is one of these plus a
  // compile-time offset (below 64 KiB, so it folds into the instruction).
  const float* vb_lane = vbias + wn * 128 + 4 * h;
  const float* vg_lane = vgamma + wn * 128 + 4 * h;
  const float* ve_lane = vbeta + wn * 128 + 4 * h;
  uint8_t* res_lane = smem + kOffRes + (wm * 128 + r32) * kResStride + (wn * 128 + 4 * h) * 2;

  // x for the 4 columns of group (mb, nb, q); tok orders the accumulator reads
  // bias of the 4 columns of group (nb, q)
  auto bias4 = [&](int nb, int q) -> f32x4_t {
    if constexpr (kPre) return *(const f32x4_t*)(vb_lane + nb * 32 + 8 * q);
    else return f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  auto xgroup = [&](int mb, int nb, auto qc, const f32x4_t& bv, float tok, float (&x)[4]) {
    constexpr int q = decltype(qc)::value;
    const int nl = wn * 128 + nb * 32 + 8 * q + 4 * h;
    float rv[4] = {0.f, 0.f, 0.f, 0.f};
    if (kPre && has_res) {
      const int ml = wm * 128 + mb * 32 + r32;
      if constexpr (kFast) {
        const u32x2_t w = *(const u32x2_t*)(res_lane + mb * 32 * kResStride + (nb * 32 + 8 * q) * 2);
        rv[0] = bf16lo(w[0]); rv[1] = bf16hi(w[0]); rv[2] = bf16lo(w[1]); rv[3] = bf16hi(w[1]);
      } else {
        const uint32_t rs = p.res_f32 ? 4 : 2;
        const uint32_t base = ((uint32_t)(m0 + ml) * p.ldr + (uint32_t)(n0 + nl)) * rs;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = (nb * 32 + 8 * q + e < ncol) ? base + (uint32_t)e * rs : kOutOfRange;
          rv[e] = p.res_f32 ? __uint_as_float(buf_load_b32(rsR, off)) : bf16_to_f32(buf_load_b16(rsR, off));
        }
      }
    }
    float v[4];
    acc_read4<q>(acc[mb][nb], tok, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (kId && kPre) x[e] = (v[e] + bv[e]) + rv[e];
      else if constexpr (kId) x[e] = v[e];
      else if constexpr (kPre) x[e] = fmaxf(__builtin_fmaf(alpha, v[e], bv[e]) + rv[e], floor_v);
      else x[e] = fmaxf(alpha * v[e], floor_v);
    }
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  // visit the 16 groups of row block mb in order: f(nb, qc, ...)
  auto for_groups = [&](auto&& f) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) { f(nb, Q0{}); f(nb, Q1{}); f(nb, Q2{}); f(nb, Q3{}); }
  };
  auto valid = [&](int nb, int q, int e) { return (kFast && !kRagged) || (nb * 32 + 8 * q + e < ncol); };

  float tok = 0.0f;
  if constexpr (ROW != 0) {
    const int cnt_w = min(max(p.N - (n0 + wn * 128), 0), 128);
    if constexpr (kCol) {
      // ---- column reduction, levels 1 and 2: over the 4 rows a lane holds
      // of each of its columns (one per row block), then over the 32 lanes of
      // its half (xor butterfly; the two halves hold different columns), then,
      // below, over the two waves that share the columns (wm 0 and 1). Rows
      // >= M are left out. Partial per column: softmax (max, sum exp(x -
      // max)); LayerNorm (mean, M2), from sums shifted by a value K of the
      // column (the half's first row) so that the lane merges are plain sums;
      // RMSNorm sum x^2.
      bool rok[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) rok[mb] = m0 + wm * 128 + mb * 32 + r32 < p.M;
      // merge of (a, b, n) with a partner's (oa, ob, on)
      auto merge = [&](float& a, float& b, float& n, float oa, float ob, float on) {
        if constexpr (R == 1) {
          const float mx = fmaxf(a, oa);
          const float sa = a == -INFINITY ? 0.0f : b * fast_exp2((a - mx) * kLog2e);
          const float sb = oa == -INFINITY ? 0.0f : ob * fast_exp2((oa - mx) * kLog2e);
          a = mx;
          b = sa + sb;
        } else if constexpr (R == 2) {
          a += oa;
          b += ob;
          n += on;
        } else {
          a += oa;
        }
      };
      auto butterfly = [&](float& a, float& b, float& n) {
        auto step = [&](auto xc) {
          constexpr int X = decltype(xc)::value;
          const float oa = xor_lanes<X>(a);
          const float ob = R == 3 ? 0.0f : xor_lanes<X>(b);
          const float on = R == 2 ? xor_lanes<X>(n) : 0.0f;
          merge(a, b, n, oa, ob, on);
        };
        step(std::integral_constant<int, 16>{});
        step(std::integral_constant<int, 8>{});
        step(std::integral_constant<int, 4>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 1>{});
      };
      for_groups([&](int nb, auto qc) {
        constexpr int q = decltype(qc)::value;
        const f32x4_t bv = bias4(nb, q);
        float xv[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          xgroup(mb, nb, qc, bv, tok, xv[mb]);
          tok = xv[mb][3];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float a = 0.0f, b = 0.0f, n = 0.0f;
          if constexpr (R == 1) {
            a = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) a = rok[mb] ? fmaxf(a, xv[mb][e]) : a;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) b += rok[mb] ? fast_exp2((xv[mb][e] - a) * kLog2e) : 0.0f;
          } else if constexpr (R == 2) {
            // K: the column's value in the half's lane 0 (row m0 + wm*128, valid)
            const float K = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(xv[0][e]), 0));
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
              const float d = rok[mb] ? xv[mb][e] - K : 0.0f;
              n += rok[mb] ? 1.0f : 0.0f;
              a += d;
              b = __builtin_fmaf(d, d, b);
            }
            butterfly(a, b, n);
            // (mean, M2) of the column's rows in this wave
            const float mean = n > 0.0f ? K + a / n : 0.0f;
            b = n > 0.0f ? fmaxf(b - a * (a / n), 0.0f) : 0.0f;
            a = mean;
          } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) a = rok[mb] ? __builtin_fmaf(xv[mb][e], xv[mb][e], a) : a;
          }
          if constexpr (R != 2) butterfly(a, b, n);
          tok = a;
          if (r32 == 0) wpart[wm * 256 + wn * 128 + nb * 32 + 8 * q + 4 * h + e] = make_float2(a, b);
        }
      });
    } else {
    // ---- reduction levels 1 and 2 (in-lane, lane halves, then the two waves sharing rows)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      float a = 0.0f, b = 0.0f;
      if constexpr (ROW == 1) {
        float mx = -INFINITY;
        for_groups([&](int nb, auto qc) {
          float x[4];
          xgroup(mb, nb, qc, bias4(nb, decltype(qc)::value), tok, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = valid(nb, decltype(qc)::value, e) ? fmaxf(mx, x[e]) : mx;
          tok = mx;
        });
        mx = max_halves(mx);
        const float mxs = (mx == -INFINITY) ? 0.0f : mx * kLog2e;
        float s = 0.0f;
        for_groups([&](int nb, auto qc) {
          float x[4];
          xgroup(mb, nb, qc, bias4(nb, decltype(qc)::value), tok, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ex = fast_exp2(__builtin_fmaf(x[e], kLog2e, -mxs));
            s += valid(nb, decltype(qc)::value, e) ? ex : 0.0f;
          }
          tok = s;
        });
        a = mx;
        b = sum_halves(s);
      } else if constexpr (ROW == 2) {
        // shifted sums about K (a value of this lane's row), then Chan merges
        float K = 0.0f, s1 = 0.0f, s2 = 0.0f, cnt = 0.0f;
        bool first = true;
        for_groups([&](int nb, auto qc) {
          float x[4];
          xgroup(mb, nb, qc, bias4(nb, decltype(qc)::value), tok, x);
          if (first) { K = valid(nb, 0, 0) ? x[0] : 0.0f; first = false; }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = valid(nb, decltype(qc)::value, e);
            const float d = ok ? x[e] - K : 0.0f;
            s1 += d;
            s2 = __builtin_fmaf(d, d, s2);
            if constexpr (!kFast || kRagged) cnt += ok ? 1.0f : 0.0f;
          }
          tok = s2;
        });
        if constexpr (kFast && !kRagged) cnt = 64.0f;
        float mean = cnt > 0.0f ? K + s1 / cnt : 0.0f;
        float m2 = cnt > 0.0f ? fmaxf(s2 - s1 * (s1 / cnt), 0.0f) : 0.0f;
        const float2 hn = halves(cnt), hm = halves(mean), hq = halves(m2);
        float n = hn.x, mm = hm.x, q2 = hq.x;
        chan_merge(n, mm, q2, hn.y, hm.y, hq.y);
        a = mm;
        b = q2;
        (void)cnt_w;
      } else if constexpr (ROW == 3) {
        float s2 = 0.0f;
        for_groups([&](int nb, auto qc) {
          float x[4];
          xgroup(mb, nb, qc, bias4(nb, decltype(qc)::value), tok, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xx = valid(nb, decltype(qc)::value, e) ? x[e] : 0.0f;
            s2 = __builtin_fmaf(xx, xx, s2);
          }
          tok = s2;
        });
        a = sum_halves(s2);
      } else if constexpr (kTop) {
        // top-k: a lane inserts its columns, in increasing order, into a sorted
        // list of kL, which goes to LDS (the residual staging area: top-k
        // takes no residual)
        float tv[kL];
        int tc[kL];
#pragma unroll
        for (int j = 0; j < kL; ++j) {
          tv[j] = -INFINITY;
          tc[j] = kNoColumn;
        }
        for_groups([&](int nb, auto qc) {
          constexpr int q = decltype(qc)::value;
          float x[4];
          xgroup(mb, nb, qc, bias4(nb, q), tok, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = valid(nb, q, e);
            // NaN ranks as -inf; a column past N stays out
            const float cv = ok ? fmaxf(x[e], -INFINITY) : -INFINITY;
            const int cc = ok ? n0 + wn * 128 + nb * 32 + 8 * q + 4 * h + e : kNoColumn;
            // empty entries remain only among the first kL candidates (past
            // those, only columns beyond N, which come last, leave entries empty)
            if (nb * 16 + q * 4 + e < kL) topk_insert_next<true>(tv, tc, cv, cc);
            else topk_insert_next<false>(tv, tc, cv, cc);
          }
          tok = tv[kL - 1];
        });
        {
          // lists of [wn][h][row]: the per-row merge below reads all four
          const int row = wm * 128 + mb * 32 + r32;
          float* lv = (float*)(smem + kOffRes) + ((wn * 2 + h) * 256 + row) * kL;
          int* lc = (int*)(smem + kOffRes + 4 * 256 * kL * 4) + ((wn * 2 + h) * 256 + row) * kL;
#pragma unroll
          for (int j = 0; j < kL; ++j) {
            lv[j] = tv[j];
            lc[j] = tc[j];
          }
        }
      } else {
        // argmax: a lane visits its columns in increasing order, so a strict >
        // keeps the first of equal values; its first column is taken whatever
        // its value (NaN ranks as -inf), so a row of -inf still names a column.
        // The lane halves interleave and are merged with the column as
        // tie-break (b holds the column's bits)
        float mx = -INFINITY;
        int ix = kNoColumn;
        for_groups([&](int nb, auto qc) {
          constexpr int q = decltype(qc)::value;
          float x[4];
          xgroup(mb, nb, qc, bias4(nb, q), tok, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xv = fmaxf(x[e], -INFINITY);
            const int c = n0 + wn * 128 + nb * 32 + 8 * q + 4 * h + e;
            if (nb == 0 && q == 0 && e == 0) {   // columns past N come last
              mx = valid(nb, q, e) ? xv : -INFINITY;
              ix = valid(nb, q, e) ? c : kNoColumn;
            } else if (valid(nb, q, e) && xv > mx) {
              mx = xv;
              ix = c;
            }
          }
          tok = mx;
        });
        const float2 hm = halves(mx), hi = halves(__int_as_float(ix));
        const int i0 = __float_as_int(hi.x), i1 = __float_as_int(hi.y);
        const bool take1 = hm.y > hm.x || (hm.y == hm.x && i1 < i0);
        a = take1 ? hm.y : hm.x;
        b = __int_as_float(take1 ? i1 : i0);
      }
      if constexpr (!kTop)
        if (h == 0) wpart[wn * 256 + wm * 128 + mb * 32 + r32] = make_float2(a, b);
    }
    }   // row reductions
    __syncthreads();

    // ---- one thread per row: merge the two wave partials, then (reduction
    // level 3) exchange with the other column tiles of the strip and merge all
    // of them in tile order
    if constexpr (kTop) {
      // top-k: merge the four lists of the tile (two lane halves of two
      // waves), then the strip's: column tile 0 stores the result, so the
      // other tiles publish their lists (2 kL tagged words per row) and go on,
      // and tile 0 merges them all
      const int ml = tid;
      const bool row_ok = m0 + ml < p.M;
      const float* lv = (const float*)(smem + kOffRes);
      const int* lc = (const int*)(smem + kOffRes + 4 * 256 * kL * 4);
      float tv[kL];
      int tc[kL];
#pragma unroll
      for (int j = 0; j < kL; ++j) {
        tv[j] = lv[ml * kL + j];
        tc[j] = lc[ml * kL + j];
      }
      for (int l = 1; l < 4; ++l) {
        float bv[kL];
        int bc[kL];
#pragma unroll
        for (int j = 0; j < kL; ++j) {
          bv[j] = lv[(l * 256 + ml) * kL + j];
          bc[j] = lc[(l * 256 + ml) * kL + j];
        }
        topk_merge(tv, tc, bv, bc);
      }
      if (p.ws_hdr != nullptr && row_ok) {
        // word j of row ml of tile t at t * (256 * 2 kL) + j * 256 + ml: each
        // store instruction writes whole contiguous lines
        uint64_t* slots = p.ws_slots + (size_t)strip * p.tiles_n * (256 * 2 * kL) + (size_t)ml;
        if (tn != 0) {
#pragma unroll
          for (int j = 0; j < kL; ++j) {
            publish(slots + (size_t)tn * (256 * 2 * kL) + j * 256, tv[j], tag);
            publish(slots + (size_t)tn * (256 * 2 * kL) + (kL + j) * 256, __int_as_float(tc[j]), tag);
          }
        } else {
          // the peers' lists, kPeers tiles at a time with all their loads in
          // flight together, merged in tile order
          constexpr int kPeers = 2;
          const uint64_t t0 = wall_clock64();
          bool lost = false;   // a peer's list never arrived: the row's results become NaN (index -1)
          for (int tb = 1; tb < p.tiles_n; tb += kPeers) {
            uint64_t w[kPeers][2 * kL];
            uint32_t need = 0;
#pragma unroll
            for (int i = 0; i < kPeers; ++i)
              if (tb + i < p.tiles_n) need |= 1u << i;
            const uint32_t have = need;
            while (need) {
#pragma unroll
              for (int i = 0; i < kPeers; ++i) {
                if (need & (1u << i)) {
                  const uint64_t* ps = slots + (size_t)(tb + i) * (256 * 2 * kL);
#pragma unroll
                  for (int j = 0; j < 2 * kL; ++j)
                    w[i][j] = __hip_atomic_load(ps + j * 256, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
              }
#pragma unroll
              for (int i = 0; i < kPeers; ++i) {
                bool all = true;
#pragma unroll
                for (int j = 0; j < 2 * kL; ++j) all = all & ((uint32_t)(w[i][j] >> 32) == tag);
                if (all) need &= ~(1u << i);
              }
              if (!need) break;
              if (timed_out || wall_clock64() - t0 > p.spin_ticks) {   // recorded in the workspace header
                timed_out = true;
                lost = true;
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
#pragma unroll
            for (int i = 0; i < kPeers; ++i) {
              if (have & (1u << i)) {
                float pv[kL];
                int pc[kL];
#pragma unroll
                for (int j = 0; j < kL; ++j) {
                  pv[j] = __uint_as_float((uint32_t)w[i][j]);
                  pc[j] = (int)(uint32_t)w[i][kL + j];
                }
                topk_merge(tv, tc, pv, pc);
              }
            }
          }
          if (lost) {
#pragma unroll
            for (int j = 0; j < kL; ++j) {
              tv[j] = __int_as_float(0x7fc00000);
              tc[j] = -1;
            }
          }
        }
      }
      // the row's k largest, stored once per strip (column tile 0)
      if (tn == 0 && row_ok) {
        const int m = m0 + ml;
#pragma unroll
        for (int j = 0; j < kL; ++j) {
          if (j < p.topk) {
            p.row_index[(size_t)m * p.topk + j] = tc[j];
            if (p.row_stats != nullptr) p.row_stats[(size_t)m * p.topk + j] = tv[j];
          }
        }
      }
    } else {
      // thread ml: row ml of the tile (row reductions) or its column ml
      // (column reductions). The exchange group: the tiles of the row strip,
      // or of the tile column; G members, this tile is member `me` of group
      // `gi`, and a statistic covers `total` elements
      const int ml = tid;
      const bool row_ok = kCol ? n0 + ml < p.N : m0 + ml < p.M;
      const float2 w0 = wpart[ml], w1 = wpart[256 + ml];
      const int ext = kCol ? p.M - m0 : p.N - n0;
      const int c0 = min(max(ext, 0), 128), c1 = min(max(ext - 128, 0), 128);
      const int G = kCol ? p.strips : p.tiles_n;
      const int me = kCol ? strip : tn, gi = kCol ? tn : strip;
      const int total = kCol ? p.M : p.N;
      float a, b;
      if constexpr (R == 1) {
        a = fmaxf(w0.x, w1.x);
        b = w0.y * fast_exp2((w0.x - a) * kLog2e) + (c1 > 0 ? w1.y * fast_exp2((w1.x - a) * kLog2e) : 0.0f);
      } else if constexpr (R == 2) {
        float n = (float)c0;
        a = w0.x;
        b = w0.y;
        chan_merge(n, a, b, (float)c1, w1.x, w1.y);
      } else if constexpr (R == 3) {
        a = w0.x + w1.x;
        b = 0.0f;
      } else {   // argmax: the first column half holds the smaller columns
        const bool take1 = c1 > 0 && w1.x > w0.x;
        a = take1 ? w1.x : w0.x;
        b = take1 ? w1.y : w0.y;
      }
      // Leader-follower mode (strips of at least p.lf_tiles tiles): column
      // tile 0 merges every partial and publishes the merged statistics in its
      // own slot; the other tiles publish their partials and read only that.
      // Peer-to-peer mode: every tile reads every partial. Both merge in tile
      // order, so the statistics are bit-identical either way.
      const bool lf = p.lf_tiles > 0 && G >= p.lf_tiles;
      if (p.ws_hdr != nullptr && row_ok && lf && me != 0) {
        uint64_t* slots = p.ws_slots + (size_t)gi * G * 512 + ml;
        publish(slots + (size_t)me * 512, a, tag);
        if constexpr (R != 3) publish(slots + (size_t)me * 512 + 256, b, tag);
        const uint64_t t0 = wall_clock64();
        bool lost = false;
        for (;;) {
          const uint64_t wa = __hip_atomic_load(slots, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          uint64_t wb = 0;
          if constexpr (R != 3) wb = __hip_atomic_load(slots + 256, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((uint32_t)(wa >> 32) == tag && (R == 3 || (uint32_t)(wb >> 32) == tag)) {
            a = __uint_as_float((uint32_t)wa);
            b = __uint_as_float((uint32_t)wb);
            break;
          }
          if (timed_out || wall_clock64() - t0 > p.spin_ticks) {   // recorded in the workspace header
            timed_out = true;
            lost = true;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (lost) {
          a = __int_as_float(0x7fc00000);
          b = ROW == 4 ? __int_as_float(-1) : __int_as_float(0x7fc00000);
        }
      } else if (p.ws_hdr != nullptr && row_ok) {
        // word w (0: a, 1: b) of row ml of tile t at t * 512 + w * 256 + ml, so
        // that each store instruction writes whole contiguous lines
        uint64_t* slots = p.ws_slots + (size_t)gi * G * 512 + ml;
        if (!lf) {   // the leader's own slot carries the merged result instead
          publish(slots + (size_t)me * 512, a, tag);
          if constexpr (R != 3) publish(slots + (size_t)me * 512 + 256, b, tag);
        }
        const uint64_t t0 = wall_clock64();
        // The peers' words are fetched 8 column tiles at a time with all loads
        // in flight together, and the words not yet published are polled again
        // together. The merge then runs in tile order, so every workgroup of
        // the strip computes bit-identical statistics.
        float ra = 0.0f, rb = 0.0f, rn = 0.0f;
        if constexpr (R == 1 || ROW == 4) ra = -INFINITY;
        if constexpr (ROW == 4) rb = __int_as_float(0x7fffffff);
        bool lost = false;   // a peer's partial never arrived: the row's results become NaN (index -1)
        for (int tb = 0; tb < G; tb += 8) {
          float va[8], vb[8];
          uint32_t need = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            va[j] = a;
            vb[j] = b;
            if (tb + j < G && tb + j != me) need |= 1u << j;
          }
          while (need) {
            uint64_t wa[8], wb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              wa[j] = wb[j] = 0;
              if (need & (1u << j)) {
                wa[j] = __hip_atomic_load(slots + (size_t)(tb + j) * 512, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if constexpr (R != 3)
                  wb[j] = __hip_atomic_load(slots + (size_t)(tb + j) * 512 + 256, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
              }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const bool ok = (uint32_t)(wa[j] >> 32) == tag && (R == 3 || (uint32_t)(wb[j] >> 32) == tag);
              if ((need & (1u << j)) && ok) {
                va[j] = __uint_as_float((uint32_t)wa[j]);
                vb[j] = __uint_as_float((uint32_t)wb[j]);
                need &= ~(1u << j);
              }
            }
            if (!need) break;
            if (timed_out || wall_clock64() - t0 > p.spin_ticks) {   // recorded in the workspace header
              timed_out = true;
              lost = true;
#pragma unroll
              for (int j = 0; j < 8; ++j)
                if (need & (1u << j)) va[j] = vb[j] = 0.0f;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int tt = tb + j;
            if (tt >= G) break;
            if constexpr (R == 1) {
              const float Mn = fmaxf(ra, va[j]);
              rb = rb * fast_exp2((ra - Mn) * kLog2e) + vb[j] * fast_exp2((va[j] - Mn) * kLog2e);
              ra = Mn;
            } else if constexpr (R == 2) {
              chan_merge(rn, ra, rb, (float)min(kGemmBN, total - tt * kGemmBN), va[j], vb[j]);
            } else if constexpr (R == 3) {
              ra += va[j];
            } else if (tt == 0 || va[j] > ra) {   // argmax: tiles in column order, so ties keep the smaller column
              ra = va[j];
              rb = vb[j];
            }
          }
        }
        a = ra;
        b = rb;
        if (lost) {
          a = __int_as_float(0x7fc00000);
          b = ROW == 4 ? __int_as_float(-1) : __int_as_float(0x7fc00000);
        }
        if (lf) {   // the leader (me == 0) hands the merged statistics to its followers
          publish(slots, a, tag);
          if constexpr (R != 3) publish(slots + 256, b, tag);
        }
      }
      float2 st;
      if constexpr (R == 1) st = make_float2(a * kLog2e, 1.0f / b);
      else if constexpr (R == 2) st = make_float2(a, rsqrtf(b / (float)total + p.eps));
      else if constexpr (R == 3) st = make_float2(rsqrtf(a / (float)total + p.eps), 0.0f);
      else st = make_float2(a, b);
      rstat[ml] = st;
      // the reduction's own per-row (per-column) result, stored once per
      // exchange group (by its member 0)
      if (me == 0 && row_ok) {
        const int m = kCol ? n0 + ml : m0 + ml;
        if constexpr (ROW == 4) p.row_index[m] = __float_as_int(b);
        if (p.row_stats != nullptr) {
          if constexpr (R == 1) p.row_stats[m] = a + logf(b);   // log-sum-exp: max + ln sum exp(x - max)
          else if constexpr (R == 2) { p.row_stats[2 * m] = a; p.row_stats[2 * m + 1] = st.y; }
          else if constexpr (R == 3) p.row_stats[m] = st.x;
          else p.row_stats[m] = a;
        }
      }
    }
    __syncthreads();
  }

  constexpr bool kTwo = ROW2 != 0;
  // ---- second row stage (ROW2): statistics of y = stage1(x) per row, a
  // second strip exchange, then z = stage2(y) in the store pass below
  float* vg2 = (float*)(smem + kOffTwo);
  float* vb2 = vg2 + 256;
  float2* rstat2 = (float2*)(smem + kOffTwo + 2048);
  const float* vg2_lane = vg2 + wn * 128 + 4 * h;
  const float* vb2_lane = vb2 + wn * 128 + 4 * h;
  // stage 1 of one element: softmax st = (max * log2 e, 1 / sum); LayerNorm
  // (mean, 1 / sqrt(var + eps)); RMSNorm (1 / sqrt(ms + eps), -)
  auto stage1 = [&](float x, float2 st1, float g, float be) -> float {
    if constexpr (ROW == 2) return __builtin_fmaf((x - st1.x) * st1.y, g, be);
    else if constexpr (ROW == 3) return x * st1.x * g;
    else if constexpr (ROW == 1) return fast_exp2(__builtin_fmaf(x, kLog2e, -st1.x)) * st1.y;
    else return x;
  };
  if constexpr (kTwo && ROW >= 1 && ROW <= 3) {
    {
      const int n = n0 + tid;
      const bool ok = n < p.N;
      vg2[tid] = (p.gamma2 && ok) ? load_vec(p.gamma2, n, p.vec_f32) : 1.0f;
      vb2[tid] = (p.beta2 && ok) ? load_vec(p.beta2, n, p.vec_f32) : 0.0f;
    }
    float2 s1[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) s1[mb] = rstat[wm * 128 + mb * 32 + r32];
    auto ygroup = [&](int mb, int nb, auto qc, float (&y)[4]) {
      constexpr int q = decltype(qc)::value;
      const int c = nb * 32 + 8 * q;
      float x[4];
      xgroup(mb, nb, qc, bias4(nb, q), tok, x);
      f32x4_t g = {1.f, 1.f, 1.f, 1.f}, be = {0.f, 0.f, 0.f, 0.f};
      if constexpr (ROW == 2 || ROW == 3) g = *(const f32x4_t*)(vg_lane + c);
      if constexpr (ROW == 2) be = *(const f32x4_t*)(ve_lane + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = stage1(x[e], s1[mb], g[e], be[e]);
    };
    auto stage2 = [&](auto r2c) {
      constexpr int R2 = decltype(r2c)::value;
      // levels 1 and 2 over y, as for the first stage over x
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        float a = 0.0f, b = 0.0f;
        if constexpr (R2 == 1) {
          float mx = -INFINITY;
          for_groups([&](int nb, auto qc) {
            float y[4];
            ygroup(mb, nb, qc, y);
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = valid(nb, decltype(qc)::value, e) ? fmaxf(mx, y[e]) : mx;
            tok = mx;
          });
          mx = max_halves(mx);
          const float mxs = (mx == -INFINITY) ? 0.0f : mx * kLog2e;
          float sm = 0.0f;
          for_groups([&](int nb, auto qc) {
            float y[4];
            ygroup(mb, nb, qc, y);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float ex = fast_exp2(__builtin_fmaf(y[e], kLog2e, -mxs));
              sm += valid(nb, decltype(qc)::value, e) ? ex : 0.0f;
            }
            tok = sm;
          });
          a = mx;
          b = sum_halves(sm);
        } else if constexpr (R2 == 2) {
          float K = 0.0f, s1s = 0.0f, s2s = 0.0f, cnt = 0.0f;
          bool first = true;
          for_groups([&](int nb, auto qc) {
            float y[4];
            ygroup(mb, nb, qc, y);
            if (first) { K = valid(nb, 0, 0) ? y[0] : 0.0f; first = false; }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool ok = valid(nb, decltype(qc)::value, e);
              const float d = ok ? y[e] - K : 0.0f;
              s1s += d;
              s2s = __builtin_fmaf(d, d, s2s);
              cnt += ok ? 1.0f : 0.0f;
            }
            tok = s2s;
          });
          const float mean = cnt > 0.0f ? K + s1s / cnt : 0.0f;
          const float m2 = cnt > 0.0f ? fmaxf(s2s - s1s * (s1s / cnt), 0.0f) : 0.0f;
          const float2 hn = halves(cnt), hm = halves(mean), hq = halves(m2);
          float nn = hn.x, mm = hm.x, q2 = hq.x;
          chan_merge(nn, mm, q2, hn.y, hm.y, hq.y);
          a = mm;
          b = q2;
        } else {
          float sq = 0.0f;
          for_groups([&](int nb, auto qc) {
            float y[4];
            ygroup(mb, nb, qc, y);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float yy = valid(nb, decltype(qc)::value, e) ? y[e] : 0.0f;
              sq = __builtin_fmaf(yy, yy, sq);
            }
            tok = sq;
          });
          a = sum_halves(sq);
        }
        if (h == 0) wpart[wn * 256 + wm * 128 + mb * 32 + r32] = make_float2(a, b);
      }
      __syncthreads();
      // level 3 over the strip (slots p.ws_slots2), merged in tile order
      {
        const int ml = tid;
        const bool row_ok = m0 + ml < p.M;
        const float2 w0 = wpart[ml], w1 = wpart[256 + ml];
        const int c0 = min(max(p.N - n0, 0), 128), c1 = min(max(p.N - n0 - 128, 0), 128);
        float a, b;
        if constexpr (R2 == 1) {
          a = fmaxf(w0.x, w1.x);
          b = w0.y * fast_exp2((w0.x - a) * kLog2e) + (c1 > 0 ? w1.y * fast_exp2((w1.x - a) * kLog2e) : 0.0f);
        } else if constexpr (R2 == 2) {
          float nn = (float)c0;
          a = w0.x;
          b = w0.y;
          chan_merge(nn, a, b, (float)c1, w1.x, w1.y);
        } else {
          a = w0.x + w1.x;
          b = 0.0f;
        }
        if (p.ws_hdr != nullptr && row_ok) {
          uint64_t* slots = p.ws_slots2 + (size_t)strip * p.tiles_n * 512 + ml;   // layout as in stage 1
          publish(slots + (size_t)tn * 512, a, tag);
          if constexpr (R2 != 3) publish(slots + (size_t)tn * 512 + 256, b, tag);
          const uint64_t t0 = wall_clock64();
          float ra = R2 == 1 ? -INFINITY : 0.0f, rb = 0.0f, rn = 0.0f;
          bool lost = false;   // a peer's partial never arrived: the row's results become NaN
          for (int tb = 0; tb < p.tiles_n; tb += 8) {
            float va[8], vb[8];
            uint32_t need = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              va[j] = a;
              vb[j] = b;
              if (tb + j < p.tiles_n && tb + j != tn) need |= 1u << j;
            }
            while (need) {
              uint64_t wa[8], wb[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                wa[j] = wb[j] = 0;
                if (need & (1u << j)) {
                  wa[j] = __hip_atomic_load(slots + (size_t)(tb + j) * 512, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                  if constexpr (R2 != 3)
                    wb[j] = __hip_atomic_load(slots + (size_t)(tb + j) * 512 + 256, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                }
              }
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const bool ok = (uint32_t)(wa[j] >> 32) == tag && (R2 == 3 || (uint32_t)(wb[j] >> 32) == tag);
                if ((need & (1u << j)) && ok) {
                  va[j] = __uint_as_float((uint32_t)wa[j]);
                  vb[j] = __uint_as_float((uint32_t)wb[j]);
                  need &= ~(1u << j);
                }
              }
              if (!need) break;
              if (timed_out || wall_clock64() - t0 > p.spin_ticks) {   // recorded in the workspace header
                timed_out = true;
                lost = true;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                  if (need & (1u << j)) va[j] = vb[j] = 0.0f;
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int tt = tb + j;
              if (tt >= p.tiles_n) break;
              if constexpr (R2 == 1) {
                const float Mn = fmaxf(ra, va[j]);
                rb = rb * fast_exp2((ra - Mn) * kLog2e) + vb[j] * fast_exp2((va[j] - Mn) * kLog2e);
                ra = Mn;
              } else if constexpr (R2 == 2) {
                chan_merge(rn, ra, rb, (float)min(kGemmBN, p.N - tt * kGemmBN), va[j], vb[j]);
              } else {
                ra += va[j];
              }
            }
          }
          a = ra;
          b = rb;
          if (lost) a = b = __int_as_float(0x7fc00000);
        }
        if constexpr (R2 == 1) rstat2[ml] = make_float2(a * kLog2e, 1.0f / b);
        else if constexpr (R2 == 2) rstat2[ml] = make_float2(a, rsqrtf(b / (float)p.N + p.eps2));
        else rstat2[ml] = make_float2(rsqrtf(a / (float)p.N + p.eps2), 0.0f);
      }
      __syncthreads();
    };
    stage2(std::integral_constant<int, ROW2>{});
  }

  // ---- stage 2: normalise, affine, cast, store
  // Column group outer, row block inner: the per-column vectors are read
  // from LDS once per group and reused by the 4 row blocks.
  // kX: the second output X (x before the row operation) is 0 absent, 1 bf16,
  // 2 fp32, 3 decided at run time (general path, one instantiation); it is
  // stored straight from the registers that hold x
  const __amdgpu_buffer_rsrc_t rsX = make_rsrc(p.X, p.X ? p.x_bytes : 0u);
  auto store_pass = [&](auto f32c, auto xc) {
    constexpr bool kOutF32 = decltype(f32c)::value;
    constexpr int kX = decltype(xc)::value;
    constexpr uint32_t es = kOutF32 ? 4u : 2u;
    const uint32_t xes = kX == 2 ? 4u : kX == 1 ? 2u : (p.x_f32 ? 4u : 2u);
    float2 st[4], st2[4];
    uint32_t rowoff[4], xrowoff[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int ml = wm * 128 + mb * 32 + r32;
      st[mb] = (ROW != 0 && !kCol) ? rstat[ml] : make_float2(0.f, 0.f);
      st2[mb] = kTwo ? rstat2[ml] : make_float2(0.f, 0.f);
      rowoff[mb] = ((uint32_t)(m0 + ml) * p.ldc + (uint32_t)(n0 + wn * 128 + 4 * h)) * es;
      if constexpr (kX != 0) xrowoff[mb] = ((uint32_t)(m0 + ml) * p.ldx + (uint32_t)(n0 + wn * 128 + 4 * h)) * xes;
    }
    for_groups([&](int nb, auto qc) {
      constexpr int q = decltype(qc)::value;
      const int c = nb * 32 + 8 * q;
      const f32x4_t bv = bias4(nb, q);
      f32x4_t g = {1.f, 1.f, 1.f, 1.f}, be = {0.f, 0.f, 0.f, 0.f};
      if constexpr (R == 2 || R == 3) g = *(const f32x4_t*)(vg_lane + c);
      if constexpr (R == 2) be = *(const f32x4_t*)(ve_lane + c);
      // column reductions: the statistics of the group's 4 columns
      f32x4_t csx = {0.f, 0.f, 0.f, 0.f}, csy = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kCol) {
        const float* rs_lane = (const float*)rstat + 2 * (wn * 128 + 4 * h);
        const f32x4_t s01 = *(const f32x4_t*)(rs_lane + 2 * c);
        const f32x4_t s23 = *(const f32x4_t*)(rs_lane + 2 * c + 4);
        csx = f32x4_t{s01[0], s01[2], s23[0], s23[2]};
        csy = f32x4_t{s01[1], s01[3], s23[1], s23[3]};
      }
      f32x4_t g2 = {1.f, 1.f, 1.f, 1.f}, b2 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kTwo) {
        g2 = *(const f32x4_t*)(vg2_lane + c);
        b2 = *(const f32x4_t*)(vb2_lane + c);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        float x[4], y[4];
        xgroup(mb, nb, qc, bv, tok, x);
        // ragged tile: the group's 4 columns are valid or invalid together
        const uint32_t gok = (!kRagged || c < ncol) ? 0u : kOutOfRange;
        if constexpr (kX == 2) {
          if constexpr (kFast) {
            const u32x4_t v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
            buf_store_b128(v, rsX, (xrowoff[mb] + (uint32_t)c * 4) | gok);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              buf_store_b32(__float_as_uint(x[e]), rsX, (c + e < ncol) ? xrowoff[mb] + (uint32_t)(c + e) * 4 : kOutOfRange);
          }
        } else if constexpr (kX == 1) {
          if constexpr (kFast) {
            const u32x2_t v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
            buf_store_b64(v, rsX, (xrowoff[mb] + (uint32_t)c * 2) | gok);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              buf_store_b16((uint16_t)f32_to_bf16(x[e]), rsX, (c + e < ncol) ? xrowoff[mb] + (uint32_t)(c + e) * 2 : kOutOfRange);
          }
        } else if constexpr (kX == 3) {
          if (p.X) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t off = (c + e < ncol) ? xrowoff[mb] + (uint32_t)(c + e) * xes : kOutOfRange;
              if (p.x_f32) buf_store_b32(__float_as_uint(x[e]), rsX, off);
              else buf_store_b16((uint16_t)f32_to_bf16(x[e]), rsX, off);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (kCol && R == 2) y[e] = __builtin_fmaf((x[e] - csx[e]) * csy[e], g[e], be[e]);
          else if constexpr (kCol && R == 3) y[e] = x[e] * csx[e] * g[e];
          else if constexpr (kCol) y[e] = fast_exp2(__builtin_fmaf(x[e], kLog2e, -csx[e])) * csy[e];
          else if constexpr (ROW == 2) y[e] = __builtin_fmaf((x[e] - st[mb].x) * st[mb].y, g[e], be[e]);
          else if constexpr (ROW == 3) y[e] = x[e] * st[mb].x * g[e];
          else if constexpr (ROW == 1) y[e] = fast_exp2(__builtin_fmaf(x[e], kLog2e, -st[mb].x)) * st[mb].y;
          else y[e] = x[e];
        }
        if constexpr (kTwo) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (ROW2 == 2) y[e] = __builtin_fmaf((y[e] - st2[mb].x) * st2[mb].y, g2[e], b2[e]);
            else if constexpr (ROW2 == 3) y[e] = y[e] * st2[mb].x * g2[e];
            else y[e] = fast_exp2(__builtin_fmaf(y[e], kLog2e, -st2[mb].x)) * st2[mb].y;
          }
        }
        tok = y[3];
        if constexpr (kOutF32) {
          if constexpr (kFast) {
            const u32x4_t v = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
            buf_store_b128(v, rsC, (rowoff[mb] + (uint32_t)c * 4) | gok);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              buf_store_b32(__float_as_uint(y[e]), rsC, (c + e < ncol) ? rowoff[mb] + (uint32_t)(c + e) * 4 : kOutOfRange);
          }
        } else {
          if constexpr (kFast) {
            // staged in LDS (over this element's staged residual, which this
            // lane has just read) and written out by whole rows below
            const u32x2_t v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            *(u32x2_t*)(res_lane + mb * 32 * kResStride + c * 2) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              buf_store_b16((uint16_t)f32_to_bf16(y[e]), rsC, (c + e < ncol) ? rowoff[mb] + (uint32_t)(c + e) * 2 : kOutOfRange);
          }
        }
      }
    });
  };
  // argmax / top-k without a matrix output (the logits are never written)
  if constexpr (ROW == 4 || kTop) {
    if (p.C == nullptr && p.X == nullptr) return;
  }
  using X0 = std::integral_constant<int, 0>;
  using X1 = std::integral_constant<int, 1>;
  using X2 = std::integral_constant<int, 2>;
  using XR = std::integral_constant<int, 3>;
  // (the general path takes X's dtype at run time)
  if (p.c_f32) {
    if constexpr (!kFast) store_pass(std::true_type{}, XR{});
    else if (!p.X) store_pass(std::true_type{}, X0{});
    else if (p.x_f32) store_pass(std::true_type{}, X2{});
    else store_pass(std::true_type{}, X1{});
  } else {
    if constexpr (!kFast) store_pass(std::false_type{}, XR{});
    else if (!p.X) store_pass(std::false_type{}, X0{});
    else if (p.x_f32) store_pass(std::false_type{}, X2{});
    else store_pass(std::false_type{}, X1{});
    if constexpr (kFast) {
      // bf16 tile [256][256] from LDS to C: each wave store covers two whole
      // 512-byte row segments; rows >= M fall outside the buffer and are dropped
      __syncthreads();
      const int c = tid & 31;
#pragma unroll 8
      for (int i = 0; i < 32; ++i) {
        const int row = (tid >> 5) + 8 * i;
        const u32x4_t v = *(const u32x4_t*)(smem + kOffRes + row * kResStride + c * 16);
        const uint32_t cok = (!kRagged || n0 + c * 8 < p.N) ? 0u : kOutOfRange;
        buf_store_b128(v, rsC, (((uint32_t)(m0 + row) * p.ldc + (uint32_t)(n0 + c * 8)) * 2u) | cok);
      }
    }
  }
}

// kVec (fast path): vector loads, N a multiple of 8, bf16 or no residual; the
// epilogue of whole column tiles is then specialised on kRow (cf_row_op) and
// kPre (bias/residual present). The general path (kVec false) is specialised
// on kRow only and masks every access element by element.
// kRow2 (with kVec and kRow 1-3): the second row stage, see epilogue's ROW2.
template <bool kF32, bool kBnk, bool kVec, int kRow, bool kPre, int kRow2 = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_epilogue_kernel(GemmEpilogueParams p) {
  constexpr int kLdsMain = 4 * kTileBytes > kStages * kStageBytes ? 4 * kTileBytes : kStages * kStageBytes;
  constexpr int kLdsEpi = kRow2 != 0 ? kLdsTwo : kLdsEpilogue;
  constexpr int kLdsBytes = kLdsMain > kLdsEpi ? kLdsMain : kLdsEpi;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
  constexpr int BK = 8 * In<kF32>::kChunk;
  constexpr int S = In<kF32>::kSize;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(p.B, p.b_bytes);

  const bool exchange = p.ws_hdr != nullptr;
  uint32_t tag = 0;
  if (exchange) tag = __hip_atomic_load(p.ws_hdr + kHdrEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  bool timed_out = false;

  const int KT = (p.K + BK - 1) / BK;

  for (int base = 0; base < p.tiles; base += gridDim.x) {
    // Tile of this round. Workgroups are dispatched round-robin over the 8
    // XCDs (workgroup w on XCD w % 8); in a full round each XCD takes an
    // xcd_a x xcd_b rectangle of (strip, column) tiles so that its workgroups
    // share A strips and B panels in that XCD's L2.
    const int tile = round_tile(base, (int)blockIdx.x, (int)gridDim.x, p.tiles, p.group, p.xcd_a, p.xcd_b);
    if (tile >= p.tiles) break;
    // tiles are numbered group by group: strip-major for row reductions (a
    // group is a row strip), column-major for column reductions (a group is
    // a tile column)
    const int grp = tile / p.group, mbr = tile - grp * p.group;
    const int strip = p.col ? mbr : grp, tn = p.col ? grp : mbr;
    const int m0 = strip * kGemmBM, n0 = tn * kGemmBN;

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{0};

    // ------------------------------------------------------------------ main loop
    // threadIdx.x through an opaque copy per tile: per-lane offsets derived
    // from it are recomputed per tile rather than hoisted out of the
    // persistent loop and spilled
    int tid_t;
    asm volatile("" : "=v"(tid_t) : "0"((int)threadIdx.x));
    bool streamed = false;
    if constexpr (!kF32 && kVec) {
      if (p.K % kStageK == 0) {
        mainloop_stream<kBnk>(acc, p, smem, m0, n0, tid_t);
        __syncthreads();   // the epilogue reuses the LDS ring
        streamed = true;
      }
    }
    if (!streamed) {
    // the register-staged loop's lane offsets also come from the per-tile
    // copy, so that they are not computed once before the tile loop and kept
    // (spilled) through the streamed path
    const int tid = tid_t, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, r32 = lane & 31;
    u32x4_t ra[8], rb[8];
    // per-thread byte offsets at k = 0 and the per-k-tile steps
    const uint32_t a_off0 = ((uint32_t)(m0 + (tid >> 3)) * p.lda + (uint32_t)((tid & 7) * In<kF32>::kChunk)) * S;
    const uint32_t a_rstep = 32u * p.lda * S;
    uint32_t b_off0, b_rstep, b_kstep;
    int b_n = 0;
    if constexpr (kBnk) {
      b_off0 = ((uint32_t)(n0 + (tid >> 3)) * p.ldb + (uint32_t)((tid & 7) * In<kF32>::kChunk)) * S;
      b_rstep = 32u * p.ldb * S;
      b_kstep = BK * S;
    } else {
      b_n = n0 + (kF32 ? (tid >> 2) * 4 : (tid >> 3) * 8);
      const int kr = kF32 ? (tid & 3) * 4 : (tid & 7) * 8;
      b_off0 = ((uint32_t)kr * p.ldb + (uint32_t)b_n) * S;
      b_rstep = p.ldb * S;
      b_kstep = (uint32_t)BK * p.ldb * S;
    }
    auto load_tile = [&](int kt) {
      const int k0 = kt * BK;
      const int kc = k0 + (tid & 7) * In<kF32>::kChunk;
      load_rowmajor<kF32, kVec>(ra, rsA, a_off0 + (uint32_t)k0 * S, a_rstep, kc, p.K, p.lda, (uint32_t)m0, tid);
      if constexpr (kBnk) load_rowmajor<kF32, kVec>(rb, rsB, b_off0 + (uint32_t)k0 * S, b_rstep, kc, p.K, p.ldb, (uint32_t)n0, tid);
      else load_kn<kF32, kVec>(rb, rsB, b_off0 + (uint32_t)kt * b_kstep, b_rstep, b_n, p.N);
    };
    auto store_tile = [&](int buf) {
      uint8_t* ta = smem + buf * kTileBytes;
      store_rowmajor(ra, ta, tid);
      if constexpr (kBnk) store_rowmajor(rb, ta + 2 * kTileBytes, tid);
      else store_kn<kF32>(rb, ta + 2 * kTileBytes, tid);
    };

    // Software pipeline over k-tiles: while the MFMAs consume tile kt from one
    // LDS buffer, tile kt+1 (already in registers) is written to the other
    // buffer and tile kt+2 is fetched from memory into registers.
    if (KT > 0) {
      load_tile(0);
      store_tile(0);
      if (KT > 1) load_tile(1);
      __syncthreads();
    }
    // LDS layout: A0 @0, A1 @32K, B0 @64K, B1 @96K
    const uint32_t a_rd = (uint32_t)((wm * 128 + r32) * kRowBytes);
    const uint32_t b_rd = (uint32_t)(2 * kTileBytes + (wn * 128 + r32) * kRowBytes);
    auto read_frags = [&](u32x4_t (&af)[4], u32x4_t (&bfr)[4], uint32_t bufoff, int kk) {
      const uint32_t coff = (uint32_t)((((2 * kk + h) ^ (lane & 7))) << 4) + bufoff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bfr[i] = *(const u32x4_t*)(smem + b_rd + coff + i * 32 * kRowBytes);
        af[i] = *(const u32x4_t*)(smem + a_rd + coff + i * 32 * kRowBytes);
      }
    };
    for (int kt = 0; kt < KT; ++kt) {
      const uint32_t bufoff = (uint32_t)(kt & 1) * kTileBytes;
      u32x4_t af[2][4], bfr[2][4];
      read_frags(af[0], bfr[0], bufoff, 0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) read_frags(af[(kk + 1) & 1], bfr[(kk + 1) & 1], bufoff, kk + 1);
        if (kk == 1 && kt + 1 < KT) store_tile((kt + 1) & 1);
        if (kk == 2 && kt + 2 < KT) load_tile(kt + 2);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) mfma<kF32>(acc[mb][nb], bfr[kk & 1][nb], af[kk & 1][mb]);
      }
      __syncthreads();
    }
    }

    // ------------------------------------------------------------------ epilogue
    if constexpr (kRow2 != 0) {
      // fast path only (the launcher routes nothing else here); the
      // column-masked epilogue serves whole and ragged tiles
      if (p.alpha == 1.0f && p.act == 0) epilogue<kRow, true, kPre, true, true, kRow2>(acc, p, smem, strip, tn, tag, timed_out, tid_t);
      else epilogue<kRow, true, kPre, false, true, kRow2>(acc, p, smem, strip, tn, tag, timed_out, tid_t);
    } else if constexpr (kVec) {
      // the last column tile of a strip may be ragged (N a multiple of 8, not
      // of 256): its epilogue masks columns against N; the main loop's
      // accumulators of columns >= N hold whatever the B loads read there,
      // and the masked epilogue only ever selects them away
      if (n0 + kGemmBN > p.N) epilogue<kRow, true, kPre, false, true>(acc, p, smem, strip, tn, tag, timed_out, tid_t);
      else if (p.alpha == 1.0f && p.act == 0) epilogue<kRow, true, kPre, true>(acc, p, smem, strip, tn, tag, timed_out, tid_t);
      else epilogue<kRow, true, kPre, false>(acc, p, smem, strip, tn, tag, timed_out, tid_t);
    } else {
      epilogue<kRow, false, true, false>(acc, p, smem, strip, tn, tag, timed_out, tid_t);
    }
    __syncthreads();   // the next tile's operand stores reuse this LDS
  }

  if (exchange) {
    if (timed_out) __hip_atomic_fetch_or(p.ws_hdr + kHdrError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(p.ws_hdr + kHdrDone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == gridDim.x - 1) {
        __hip_atomic_store(p.ws_hdr + kHdrDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ws_hdr + kHdrEpoch, tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace cf
