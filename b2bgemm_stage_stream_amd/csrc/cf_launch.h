// Kernel parameter blocks and launchers (host <-> kernel interface, internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cf_plan.h"

namespace cf {

// Workspace header words (uint32 index into the header); the header is
// kWsHeaderBytes long and followed by the partial-statistics slots.
enum : int { kHdrEpoch = 0, kHdrDone = 32, kHdrError = 64 };

// Output tile of one workgroup in the GEMM + epilogue kernel.
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;

struct GemmEpilogueParams {
  const void* A;
  const void* B;
  void* C;
  const void* bias;
  const void* residual;
  const void* gamma;
  const void* beta;
  uint32_t lda, ldb, ldc, ldr;   // elements
  uint32_t a_bytes, b_bytes, c_bytes, r_bytes;   // extents for the buffer range checks
  int M, N, K;
  int tiles_n;       // column tiles per row strip
  int tiles;         // total output tiles
  int xcd_a, xcd_b;  // per-XCD rectangle of a round (strips x columns); 0: plain order
  float alpha, eps;
  int act;           // cf_act
  int row_op;        // cf_row_op
  int c_f32;         // 1: fp32 output, 0: bf16
  int vec_f32;       // dtype of bias/gamma/beta: 1 fp32, 0 bf16
  int res_f32;       // dtype of residual
  void* X;           // optional second output: x before the row operation
  uint32_t ldx, x_bytes;
  int x_f32;         // dtype of X: 1 fp32, 0 bf16
  float* row_stats;  // optional per-row statistics of the row operation
  int32_t* row_index;   // row argmax / top-k: column(s) of each row's maximum (k largest)
  int row_op2;       // second row stage on the first one's output (0: none)
  const void* gamma2;
  const void* beta2;
  float eps2;
  uint32_t* ws_hdr;  // workspace header (NULL when tiles_n == 1 or no row op)
  uint64_t* ws_slots;
  uint64_t* ws_slots2;   // the second stage's exchange slots
  uint64_t spin_ticks;   // wall-clock ticks a strip wait may take
  int topk;          // top-k: k (1..8)
  int lf_tiles;      // leader-follower exchange for groups of at least this many tiles (0: never)
  int col;           // the row op reduces over the rows m of each column (column reduction)
  int group;         // tiles per exchange group: tiles_n (row strips) or strips (tile columns)
  int strips;        // row strips
};

// Launches the persistent kernel. in_f32: fp32 inputs (else bf16); b_nk: B
// stored [N, K]; vec (fast path): 16-byte accesses allowed, N a multiple of
// 8 and the residual (if any) bf16. p.row_op2 != 0 selects the two-stage
// instantiations.
hipError_t launch_gemm_epilogue(const GemmEpilogueParams& p, bool in_f32, bool b_nk, bool vec,
                                int grid, hipStream_t stream);

// Workgroups of `kernel` with `threads` threads that fit on one compute unit
// of the current device, and the device's compute units; both cached.
hipError_t blocks_per_cu_cached(const void* kernel, int threads, int* n);
hipError_t device_cus_cached(int* cus);

// Workgroups of the GEMM + epilogue kernel that fit on one compute unit.
int gemm_epilogue_blocks_per_cu(const GemmEpilogueParams& p, bool in_f32, bool b_nk, bool vec);

hipError_t launch_workspace_clear(void* ws, size_t bytes, hipStream_t stream);

struct B2bParams {
  const void* A;
  const void* B0;
  const void* B1;
  void* O;
  const void* bias;     // [L] or NULL
  uint32_t lda, ldb0, ldb1, ldo;
  uint64_t sa, sb0, sb1, so;   // batch strides, elements
  int batch, M, K, L, N;
  float alpha;
  int act;
  int row_op;
  int out_f32;
  int bias_f32;
  int bias_vec;      // bias 4-byte aligned: streamed with the B0/B1 segments
  int b0_lk;
  int o_vec;     // O base, ldo and batch stride allow 4-element vector stores
  int causal;    // softmax only: key l visible to row m iff l <= m + coff
  int coff;      // L - M
  float* row_stats;   // softmax only, optional: log-sum-exp of each row, [batch][M]
  int pingpong;        // softmax: the ping-pong schedule where it applies (cf_set_b2b_pingpong)
};

hipError_t launch_b2b(const B2bParams& p, hipStream_t stream);
// Streamed kernel for exact shapes (K, N in {64, 128}, L a multiple of 64), or
// null; *rows_per_tile receives its tile height and *threads its workgroup
// size.
const void* b2b_stream_pick(const B2bParams& p, int cus, int* rows_per_tile, int* threads);
// Returns false when (K, N, row_op, ...) has no kernel instantiation.
bool b2b_supported(const B2bParams& p);

}  // namespace cf
