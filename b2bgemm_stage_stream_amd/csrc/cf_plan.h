// Host-side planning of the GEMM + epilogue launch: argument checks, the
// per-strip workspace layout, the persistent grid and the tile each
// workgroup takes in a round. Plain C++ over the C ABI's types: no HIP call
// and no HIP header, so the same code also builds for the CPU tests (which
// define CF_HD as empty before including it).
//
// Method: ComFuse review, Referee Report major comment 1 (Sec. III, Eq. (1)):
// a row reduction needs only the tiles that share the row index, i.e. one
// row strip. Its workgroups exchange per-row partial statistics, so a strip's
// tiles must be processed by workgroups that are resident at the same time
// (the review's co-scheduling requirement, "Load-bearing premise").
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <cmath>
#include <cstring>

#include "cf.h"

#ifndef CF_HD
#define CF_HD __host__ __device__
#endif

namespace cf {

constexpr int64_t kPlanTile = 256;        // output tile edge (rows and columns)
constexpr size_t kWsHeaderBytes = 512;    // workspace header, then the exchange slots

// The integer a caller stored in an enum field of the C ABI. C callers may
// store any int there; reading it as its integer representation keeps the
// checks defined for values that are not enumerators.
template <class E>
inline int ev(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C ABI enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

inline bool plan_is_dtype(int d) { return d == CF_F32 || d == CF_BF16; }
inline size_t plan_dsize(int d) { return d == CF_F32 ? 4 : 2; }
inline bool plan_aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Bytes spanned by `rows` rows of leading dimension ld (elements of size es),
// padded by `pad_rows` rows so that out-of-range tile rows stay below 2^31.
inline bool fits31(int64_t rows, int64_t pad_rows, int64_t ld, size_t es) {
  const long double b = (long double)(rows + pad_rows) * (long double)ld * (long double)es;
  return b < 2147483648.0L;
}

struct GemmPlan {
  int64_t tiles_n = 0, strips = 0, tiles = 0;
  bool col = false;        // a column reduction: groups are tile columns
  int64_t group = 0;       // tiles per exchange group (tiles_n, or strips for a column reduction)
  bool exchange = false;
  size_t slot_bytes = 0;   // one stage's exchange slots
  size_t ws_bytes = 0;
};

// Tiles of the problem and the workspace its strip exchange needs.
inline GemmPlan plan_gemm(int64_t M, int64_t N, const cf_epilogue* epi) {
  GemmPlan g;
  g.tiles_n = (N + kPlanTile - 1) / kPlanTile;
  g.strips = (M + kPlanTile - 1) / kPlanTile;
  g.tiles = g.tiles_n * g.strips;
  g.col = epi && ev(epi->axis) == CF_AXIS_COLUMN;
  g.group = g.col ? g.strips : g.tiles_n;
  g.exchange = epi && ev(epi->row_op) != CF_ROW_NONE && g.group > 1;
  if (g.exchange) {
    // one slot set per reduction stage; top-k publishes up to 8 (value, column) pairs per row
    const size_t words = ev(epi->row_op) == CF_ROW_TOPK ? 16 : 2;
    const size_t slots = (size_t)g.strips * (size_t)g.tiles_n * (size_t)kPlanTile * words * sizeof(uint64_t);
    g.slot_bytes = ((slots + 255) / 256) * 256;
    g.ws_bytes = kWsHeaderBytes + g.slot_bytes * (ev(epi->row_op2) != CF_ROW_NONE ? 2 : 1);
  }
  return g;
}

// The epilogue descriptor's own consistency (both entry points).
inline cf_status check_epilogue(const cf_epilogue* epi, int64_t N, bool allow_row_ops_norm, bool allow_residual) {
  if (!epi) return CF_OK;
  if (epi->struct_size != sizeof(cf_epilogue)) return CF_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(epi->alpha) || !std::isfinite(epi->eps) || epi->eps < 0.0f) return CF_ERR_INVALID_ARGUMENT;
  if (ev(epi->act) != CF_ACT_NONE && ev(epi->act) != CF_ACT_RELU) return CF_ERR_INVALID_ARGUMENT;
  if (ev(epi->row_op) < CF_ROW_NONE || ev(epi->row_op) > CF_ROW_TOPK) return CF_ERR_INVALID_ARGUMENT;
  if (ev(epi->row_op) == CF_ROW_ARGMAX || ev(epi->row_op) == CF_ROW_TOPK) {
    if (!epi->row_index || !plan_aligned(epi->row_index, 4) || epi->gamma || epi->beta) return CF_ERR_INVALID_ARGUMENT;
    if (!allow_residual) return CF_ERR_UNSUPPORTED;
  } else if (epi->row_index) {
    return CF_ERR_INVALID_ARGUMENT;
  }
  if (ev(epi->row_op) == CF_ROW_TOPK) {
    if (epi->topk < 1 || epi->topk > 8 || epi->topk > N) return CF_ERR_INVALID_ARGUMENT;
    if (epi->residual) return CF_ERR_UNSUPPORTED;   // its LDS staging area holds the lists
  } else if (epi->topk != 0) {
    return CF_ERR_INVALID_ARGUMENT;
  }
  if (!plan_is_dtype(ev(epi->vec_dtype)) || !plan_is_dtype(ev(epi->residual_dtype))) return CF_ERR_INVALID_ARGUMENT;
  const size_t vs = plan_dsize(ev(epi->vec_dtype));
  if ((epi->bias && !plan_aligned(epi->bias, vs)) || (epi->gamma && !plan_aligned(epi->gamma, vs)) ||
      (epi->beta && !plan_aligned(epi->beta, vs)))
    return CF_ERR_INVALID_ARGUMENT;
  if (epi->residual) {
    if (!allow_residual) return CF_ERR_UNSUPPORTED;
    if (epi->ld_residual < N || epi->ld_residual < 1) return CF_ERR_INVALID_ARGUMENT;
    if (!plan_aligned(epi->residual, plan_dsize(ev(epi->residual_dtype)))) return CF_ERR_INVALID_ARGUMENT;
  }
  if (epi->row_stats && (ev(epi->row_op) == CF_ROW_NONE || !plan_aligned(epi->row_stats, 4))) return CF_ERR_INVALID_ARGUMENT;
  if (ev(epi->mask) != CF_MASK_NONE && ev(epi->mask) != CF_MASK_CAUSAL) return CF_ERR_INVALID_ARGUMENT;
  if (ev(epi->mask) != CF_MASK_NONE && (allow_residual || ev(epi->row_op) != CF_ROW_SOFTMAX)) return CF_ERR_UNSUPPORTED;
  if (epi->x_out) {
    if (!allow_residual) return CF_ERR_UNSUPPORTED;
    if (ev(epi->x_out_dtype) != CF_BF16 && ev(epi->x_out_dtype) != CF_F32) return CF_ERR_INVALID_ARGUMENT;
    if (epi->ld_x_out < N || epi->ld_x_out < 1) return CF_ERR_INVALID_ARGUMENT;
    if (!plan_aligned(epi->x_out, plan_dsize(ev(epi->x_out_dtype)))) return CF_ERR_INVALID_ARGUMENT;
  }
  if (!allow_row_ops_norm) {
    if (ev(epi->row_op) == CF_ROW_LAYERNORM || ev(epi->row_op) == CF_ROW_RMSNORM) return CF_ERR_UNSUPPORTED;
    if (epi->gamma || epi->beta) return CF_ERR_UNSUPPORTED;
  }
  // reduction axis: a column reduction takes softmax, LayerNorm or RMSNorm
  // alone (one stage), in cf_gemm_epilogue only
  const int axis = ev(epi->axis);
  if (axis != CF_AXIS_ROW && axis != CF_AXIS_COLUMN) return CF_ERR_INVALID_ARGUMENT;
  if (axis == CF_AXIS_COLUMN) {
    const int op = ev(epi->row_op);
    if (op == CF_ROW_NONE) return CF_ERR_INVALID_ARGUMENT;
    if (!allow_residual) return CF_ERR_UNSUPPORTED;
    if (op != CF_ROW_SOFTMAX && op != CF_ROW_LAYERNORM && op != CF_ROW_RMSNORM) return CF_ERR_UNSUPPORTED;
    if (ev(epi->row_op2) != CF_ROW_NONE) return CF_ERR_UNSUPPORTED;
  }
  // second row stage: softmax / LayerNorm / RMSNorm after one of those three
  if (ev(epi->row_op2) < CF_ROW_NONE || ev(epi->row_op2) > CF_ROW_ARGMAX) return CF_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(epi->eps2) || epi->eps2 < 0.0f) return CF_ERR_INVALID_ARGUMENT;
  if (ev(epi->row_op2) == CF_ROW_NONE) {
    if (epi->gamma2 || epi->beta2 || epi->eps2 != 0.0f) return CF_ERR_INVALID_ARGUMENT;
  } else {
    if (!allow_residual) return CF_ERR_UNSUPPORTED;
    const bool norm1 = ev(epi->row_op) == CF_ROW_SOFTMAX || ev(epi->row_op) == CF_ROW_LAYERNORM || ev(epi->row_op) == CF_ROW_RMSNORM;
    if (!norm1 || ev(epi->row_op2) == CF_ROW_ARGMAX) return CF_ERR_INVALID_ARGUMENT;
    if (epi->beta2 && ev(epi->row_op2) != CF_ROW_LAYERNORM) return CF_ERR_INVALID_ARGUMENT;
    if ((epi->gamma2 && !plan_aligned(epi->gamma2, vs)) || (epi->beta2 && !plan_aligned(epi->beta2, vs)))
      return CF_ERR_INVALID_ARGUMENT;
  }
  return CF_OK;
}

// What the argument checks of cf_gemm_epilogue derive for the launch.
struct GemmChecked {
  GemmPlan plan;
  int row_op = 0;      // the row op run (top-1 runs as the argmax)
  bool vec = false;    // fast path: 16-byte accesses everywhere
  bool empty = false;  // M or N is 0: nothing to launch
};

// Every argument check of cf_gemm_epilogue, in order, without touching the
// device. ws_limit: the largest workspace the call can use (the caller's
// ws_bytes, or the static scratch size); ws is the caller's workspace or
// NULL when the library provides it (need_ws_ptr false).
inline cf_status check_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, int b_is_nk, int ab_dtype, const void* C, int64_t ldc,
                            int c_dtype, const cf_epilogue* epi, const void* ws, size_t ws_limit,
                            bool need_ws_ptr, GemmChecked* out) {
  if (M < 0 || N < 0 || K < 0) return CF_ERR_INVALID_ARGUMENT;
  if (!plan_is_dtype(ab_dtype) || !plan_is_dtype(c_dtype)) return CF_ERR_INVALID_ARGUMENT;
  if (b_is_nk != 0 && b_is_nk != 1) return CF_ERR_INVALID_ARGUMENT;
  cf_status st = check_epilogue(epi, N, true, true);
  if (st != CF_OK) return st;
  if (M == 0 || N == 0) {
    out->empty = true;
    return CF_OK;
  }
  const size_t es = plan_dsize(ab_dtype), cs = plan_dsize(c_dtype);
  const bool argmax = epi && (ev(epi->row_op) == CF_ROW_ARGMAX || ev(epi->row_op) == CF_ROW_TOPK);
  if (C ? ldc < N : !argmax) return CF_ERR_INVALID_ARGUMENT;
  if (K > 0) {
    if (!A || !B || lda < K) return CF_ERR_INVALID_ARGUMENT;
    if (ldb < (b_is_nk ? K : N)) return CF_ERR_INVALID_ARGUMENT;
    if (!plan_aligned(A, es) || !plan_aligned(B, es)) return CF_ERR_INVALID_ARGUMENT;
  }
  if (C && !plan_aligned(C, cs)) return CF_ERR_INVALID_ARGUMENT;
  if (M > INT32_MAX - kPlanTile || N > INT32_MAX - kPlanTile || K > INT32_MAX - kPlanTile) return CF_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: every operand (plus one tile of padding) below 2 GiB
  if (C && !fits31(M, kPlanTile, ldc, cs)) return CF_ERR_UNSUPPORTED;
  if (K > 0) {
    if (!fits31(M, kPlanTile, lda, es)) return CF_ERR_UNSUPPORTED;
    if (b_is_nk ? !fits31(N, kPlanTile, ldb, es) : !fits31(K, 64, ldb, es)) return CF_ERR_UNSUPPORTED;
  }
  const int rdt = (epi && epi->residual) ? ev(epi->residual_dtype) : (int)CF_BF16;
  if (epi && epi->residual && !fits31(M, kPlanTile, epi->ld_residual, plan_dsize(rdt))) return CF_ERR_UNSUPPORTED;
  const void* const X = epi ? epi->x_out : nullptr;
  const size_t xs = X ? plan_dsize(ev(epi->x_out_dtype)) : 2;
  if (X && !fits31(M, kPlanTile, epi->ld_x_out, xs)) return CF_ERR_UNSUPPORTED;
  // top-1 is the row argmax (same order, ties and NaN ranking, same outputs)
  const int row_op = (epi && ev(epi->row_op) == CF_ROW_TOPK && epi->topk == 1) ? (int)CF_ROW_ARGMAX
                     : epi ? (int)ev(epi->row_op) : 0;
  const GemmPlan plan = plan_gemm(M, N, epi);
  // an exchange group is at most 256 tiles (a row strip of N, or a tile column of M)
  if (row_op != CF_ROW_NONE && (plan.col ? M : N) > 65536) return CF_ERR_UNSUPPORTED;
  if (plan.exchange) {
    if (plan.ws_bytes > ws_limit) return CF_ERR_WORKSPACE;
    if (need_ws_ptr && (!ws || !plan_aligned(ws, 256))) return CF_ERR_WORKSPACE;
  }

  // fast path: 16-byte accesses everywhere, bf16 (or no) residual; a ragged
  // last column tile (N a multiple of 8) takes the masked epilogue
  const int64_t ce = ab_dtype == CF_F32 ? 4 : 8;
  bool vec = (N % 8 == 0) && (K % ce == 0) && (lda % ce == 0) && (ldb % ce == 0) &&
             (!C || (ldc % 8 == 0 && plan_aligned(C, 16))) && plan_aligned(A, 16) && plan_aligned(B, 16);
  if (epi && epi->residual)
    vec = vec && ev(epi->residual_dtype) == CF_BF16 && epi->ld_residual % 8 == 0 && plan_aligned(epi->residual, 16);
  if (X) vec = vec && epi->ld_x_out % 8 == 0 && plan_aligned(X, 16);
  // two row stages and top-k (k > 1): fast-path layouts and bf16 inputs only;
  // column reductions: fast-path layouts
  if (epi && (ev(epi->row_op2) != CF_ROW_NONE || row_op == CF_ROW_TOPK) && (!vec || ab_dtype != CF_BF16))
    return CF_ERR_UNSUPPORTED;
  if (plan.col && !vec) return CF_ERR_UNSUPPORTED;
  out->plan = plan;
  out->row_op = row_op;
  out->vec = vec;
  out->empty = false;
  return CF_OK;
}

// The persistent grid and its XCD rectangles.
struct GridPlan {
  int64_t grid = 0;
  int xcd_a = 0, xcd_b = 0;   // per-XCD rectangle of a full round (strips x columns); 0: plain order
};

// per_cu workgroups of the kernel fit on each of `cus` compute units. With an
// exchange, a round of the persistent grid is a whole number of exchange
// groups (row strips, or tile columns for a column reduction), all resident
// at once, so every group's tiles run together: a group wider than the
// resident capacity is refused. Workgroup w runs on XCD w % 8; a full round
// of `grid` tiles is cut into 8 equal a x b rectangles (a groups by b members,
// a + b smallest), one per XCD, so that an XCD's workgroups share A strips
// and B column panels in its L2.
inline cf_status plan_grid(const GemmPlan& g, int64_t per_cu, int64_t cus, GridPlan* out) {
  if (per_cu <= 0 || cus <= 0) return CF_ERR_UNSUPPORTED;
  const int64_t cap = per_cu * cus;
  GridPlan r;
  if (g.exchange) {
    if (g.group > cap) return CF_ERR_UNSUPPORTED;
    r.grid = g.tiles < (cap / g.group) * g.group ? g.tiles : (cap / g.group) * g.group;
  } else {
    r.grid = g.tiles < cap ? g.tiles : cap;
  }
  if (r.grid % 8 == 0 && r.grid % g.group == 0) {
    const int64_t S = r.grid / g.group, per = r.grid / 8;
    int64_t best = 0;
    for (int64_t a = 1; a <= S; ++a) {
      if (S % a || per % a) continue;
      const int64_t b = per / a;
      if (g.group % b || (S / a) * (g.group / b) != 8) continue;
      if (!best || a + b < best + per / best) best = a;
    }
    if (best) {
      r.xcd_a = (int)best;
      r.xcd_b = (int)(per / best);
    }
  }
  *out = r;
  return CF_OK;
}

// Tile of workgroup `bid` in the round that starts at tile `base`, tiles
// numbered group by group (tile = group * tiles_n + member; tiles_n here is
// the group width: column tiles per row strip, or row strips per tile column
// for a column reduction). A full round with XCD rectangles gives XCD x =
// bid % 8 the rectangle (rx, ry) of the round's groups x members; otherwise
// tiles go in plain order. A result >= tiles means the workgroup has no tile
// left.
CF_HD inline int round_tile(int base, int bid, int grid, int tiles, int tiles_n, int xcd_a, int xcd_b) {
  if (xcd_a > 0 && base + grid <= tiles) {
    const int x = bid & 7, i = bid >> 3;
    const int rects_n = tiles_n / xcd_b;
    const int rx = x / rects_n, ry = x - rx * rects_n;
    return (base / tiles_n + rx * xcd_a + i / xcd_b) * tiles_n + ry * xcd_b + i % xcd_b;
  }
  return base + bid;
}

}  // namespace cf
