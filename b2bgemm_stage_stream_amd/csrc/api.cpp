// C ABI of the library (declared in include/cf.h): argument validation, launch
// planning and dispatch. Every argument check runs before the first HIP call.
#include "cf.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "cf_launch.h"
#include "cf_plan.h"

namespace {

thread_local int g_last_hip_error = 0;
std::atomic<uint64_t> g_timeout_us{2000000};
// strips of at least this many column tiles exchange leader-follower (0: never)
std::atomic<int> g_lf_tiles{CF_DEFAULT_LEADER_TILES};
std::atomic<int> g_b2b_pingpong{0};

struct DeviceInfo {
  bool valid = false;
  int cus = 0;
  int wallclock_khz = 0;
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

cf_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return CF_ERR_HIP;
}

// Current device and its properties; CF_ERR_NO_DEVICE when none is visible.
cf_status current_device(int* dev_out, DeviceInfo* info) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return CF_ERR_NO_DEVICE;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return CF_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_dev[dev].valid) {
    DeviceInfo d;
    if ((e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return hip_fail(e);
    if ((e = hipDeviceGetAttribute(&d.wallclock_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return hip_fail(e);
    if (d.wallclock_khz <= 0) d.wallclock_khz = 100000;
    d.valid = true;
    g_dev[dev] = d;
  }
  *dev_out = dev;
  *info = g_dev[dev];
  return CF_OK;
}

using cf::check_epilogue;
using cf::GemmPlan;
using cf::plan_gemm;

bool aligned(const void* p, size_t a) { return cf::plan_aligned(p, a); }
bool is_dtype(int d) { return cf::plan_is_dtype(d); }
size_t dsize(cf_dtype d) { return cf::plan_dsize(d); }

}  // namespace

extern "C" {

void cf_epilogue_init(cf_epilogue* epi) {
  if (!epi) return;
  std::memset(epi, 0, sizeof(*epi));
  epi->struct_size = sizeof(cf_epilogue);
  epi->alpha = 1.0f;
  epi->residual_dtype = CF_BF16;
  epi->vec_dtype = CF_BF16;
  epi->act = CF_ACT_NONE;
  epi->row_op = CF_ROW_NONE;
  epi->eps = 0.0f;
}

size_t cf_gemm_epilogue_workspace_size(int64_t M, int64_t N, int64_t K, const cf_epilogue* epi) {
  (void)K;
  if (M <= 0 || N <= 0) return 0;
  return plan_gemm(M, N, epi).ws_bytes;
}

cf_status cf_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned(ws, 256) || ws_bytes < cf::kWsHeaderBytes) return CF_ERR_WORKSPACE;
  int dev;
  DeviceInfo info;
  cf_status st = current_device(&dev, &info);
  if (st != CF_OK) return st;
  hipError_t e = cf::launch_workspace_clear(ws, ws_bytes & ~(size_t)3, (hipStream_t)stream);
  return e == hipSuccess ? CF_OK : hip_fail(e);
}

cf_status cf_workspace_status(const void* ws, void* stream) {
  if (!ws || !aligned(ws, 256)) return CF_ERR_WORKSPACE;
  int dev;
  DeviceInfo info;
  cf_status st = current_device(&dev, &info);
  if (st != CF_OK) return st;
  uint32_t err = 0;
  hipError_t e = hipMemcpyAsync(&err, (const uint32_t*)ws + cf::kHdrError, sizeof(err), hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  if ((e = hipStreamSynchronize((hipStream_t)stream)) != hipSuccess) return hip_fail(e);
  return err ? CF_ERR_DEVICE_TIMEOUT : CF_OK;
}

}  // extern "C"

// Scratch of the allocation-free entry point: one static device array per GPU
// the library runs on, held until the process ends. Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per device.
static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

struct ScratchDevice {
  void* ptr = nullptr;    // device address of `scratch` on this device
  bool cleared = false;   // the clear kernel has been enqueued once
};
std::mutex g_scratch_mu;
ScratchDevice g_scratch[64];

// The current device's scratch address; its first use on a device enqueues a
// clear of the whole array on `stream` (the exchange protocol needs a zeroed
// epoch word and zeroed slots once).
cf_status scratch_of_device(int dev, hipStream_t stream, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchDevice& sd = g_scratch[dev];
  if (sd.ptr == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (ptr == nullptr || !aligned(ptr, 256)) return CF_ERR_WORKSPACE;
    sd.ptr = ptr;
  }
  if (!sd.cleared) {
    const hipError_t e = cf::launch_workspace_clear(sd.ptr, kScratchBytes, stream);
    if (e != hipSuccess) return hip_fail(e);
    sd.cleared = true;
  }
  *out = sd.ptr;
  return CF_OK;
}

// cf_gemm_epilogue, with the caller's workspace (use_scratch false) or the
// library's static scratch (use_scratch true; ws and ws_bytes are ignored).
cf_status gemm_epilogue_run(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                            int64_t ldb, int b_is_nk, cf_dtype ab_dtype, void* C, int64_t ldc, cf_dtype c_dtype,
                            const cf_epilogue* epi, void* ws, size_t ws_bytes, void* stream, bool use_scratch) {
  // ---- argument checks (no HIP calls)
  cf::GemmChecked chk;
  cf_status st = cf::check_gemm(M, N, K, A, lda, B, ldb, b_is_nk, cf::ev(ab_dtype), C, ldc, cf::ev(c_dtype), epi, ws,
                                use_scratch ? kScratchBytes : ws_bytes, !use_scratch, &chk);
  if (st != CF_OK || chk.empty) return st;
  const GemmPlan& plan = chk.plan;
  const int row_op = chk.row_op;
  const bool vec = chk.vec;
  const size_t es = dsize(ab_dtype), cs = dsize(c_dtype);
  const cf_dtype rdt = (epi && epi->residual) ? epi->residual_dtype : CF_BF16;
  void* const X = epi ? epi->x_out : nullptr;
  const size_t xs = X ? dsize(epi->x_out_dtype) : 2;

  // ---- device
  int dev;
  DeviceInfo info;
  if ((st = current_device(&dev, &info)) != CF_OK) return st;
  if (use_scratch && plan.exchange) {
    if ((st = scratch_of_device(dev, (hipStream_t)stream, &ws)) != CF_OK) return st;
    ws_bytes = kScratchBytes;
  }

  cf::GemmEpilogueParams p;
  std::memset(&p, 0, sizeof(p));
  p.A = A;
  p.B = B;
  p.C = C;
  p.bias = epi ? epi->bias : nullptr;
  p.residual = epi ? epi->residual : nullptr;
  p.gamma = epi ? epi->gamma : nullptr;
  p.beta = epi ? epi->beta : nullptr;
  p.lda = (uint32_t)(K > 0 ? lda : 0);
  p.ldb = (uint32_t)(K > 0 ? ldb : 0);
  p.ldc = (uint32_t)(C ? ldc : 0);
  p.ldr = (uint32_t)(p.residual ? epi->ld_residual : 0);
  p.a_bytes = (uint32_t)(K > 0 ? (uint64_t)M * lda * es : 0);
  p.b_bytes = (uint32_t)(K > 0 ? (uint64_t)(b_is_nk ? N : K) * ldb * es : 0);
  p.c_bytes = (uint32_t)(C ? (uint64_t)M * ldc * cs : 0);
  p.r_bytes = (uint32_t)(p.residual ? (uint64_t)M * epi->ld_residual * dsize(rdt) : 0);
  p.X = X;
  p.ldx = (uint32_t)(X ? epi->ld_x_out : 0);
  p.x_bytes = (uint32_t)(X ? (uint64_t)M * epi->ld_x_out * xs : 0);
  p.x_f32 = X && epi->x_out_dtype == CF_F32;
  p.row_stats = epi ? epi->row_stats : nullptr;
  p.row_index = epi ? epi->row_index : nullptr;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tiles_n = (int)plan.tiles_n;
  p.tiles = (int)plan.tiles;
  p.col = plan.col ? 1 : 0;
  p.group = (int)plan.group;
  p.strips = (int)plan.strips;
  p.alpha = epi ? epi->alpha : 1.0f;
  p.eps = epi ? epi->eps : 0.0f;
  p.act = epi ? (int)epi->act : 0;
  p.row_op = row_op;
  p.c_f32 = c_dtype == CF_F32;
  p.vec_f32 = epi ? epi->vec_dtype == CF_F32 : 0;
  p.res_f32 = rdt == CF_F32;
  p.topk = epi ? epi->topk : 0;
  p.row_op2 = epi ? (int)epi->row_op2 : 0;
  p.gamma2 = epi ? epi->gamma2 : nullptr;
  p.beta2 = epi ? epi->beta2 : nullptr;
  p.eps2 = epi ? epi->eps2 : 0.0f;
  if (plan.exchange) {
    p.ws_hdr = (uint32_t*)ws;
    p.ws_slots = (uint64_t*)((char*)ws + cf::kWsHeaderBytes);
    if (p.row_op2 != 0) p.ws_slots2 = (uint64_t*)((char*)ws + cf::kWsHeaderBytes + plan.slot_bytes);
  }
  p.spin_ticks = g_timeout_us.load() * (uint64_t)info.wallclock_khz / 1000u;
  p.lf_tiles = g_lf_tiles.load();

  const bool in_f32 = ab_dtype == CF_F32;
  const int per_cu = cf::gemm_epilogue_blocks_per_cu(p, in_f32, b_is_nk != 0, vec);
  if (per_cu <= 0) return hip_fail(hipGetLastError());
  cf::GridPlan gp;
  if ((st = cf::plan_grid(plan, per_cu, info.cus, &gp)) != CF_OK) return st;
  const int64_t grid = gp.grid;
  p.xcd_a = gp.xcd_a;
  p.xcd_b = gp.xcd_b;
  hipError_t e = cf::launch_gemm_epilogue(p, in_f32, b_is_nk != 0, vec, (int)grid, (hipStream_t)stream);
  return e == hipSuccess ? CF_OK : hip_fail(e);
}

}  // namespace

extern "C" {

cf_status cf_gemm_epilogue(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                           int64_t ldb, int b_is_nk, cf_dtype ab_dtype, void* C, int64_t ldc, cf_dtype c_dtype,
                           const cf_epilogue* epi, void* ws, size_t ws_bytes, void* stream) {
  return gemm_epilogue_run(M, N, K, A, lda, B, ldb, b_is_nk, ab_dtype, C, ldc, c_dtype, epi, ws, ws_bytes, stream,
                           false);
}

cf_status cf_gemm_epilogue_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                                   int64_t ldb, int b_is_nk, cf_dtype ab_dtype, void* C, int64_t ldc,
                                   cf_dtype c_dtype, const cf_epilogue* epi, void* stream) {
  return gemm_epilogue_run(M, N, K, A, lda, B, ldb, b_is_nk, ab_dtype, C, ldc, c_dtype, epi, nullptr, 0, stream,
                           true);
}

cf_status cf_b2bgemm(int64_t batch, int64_t M, int64_t K, int64_t L, int64_t N, const void* A, int64_t lda,
                     int64_t sa, const void* B0, int64_t ldb0, int64_t sb0, int b0_is_lk, const void* B1,
                     int64_t ldb1, int64_t sb1, void* O, int64_t ldo, int64_t so, cf_dtype in_dtype,
                     cf_dtype out_dtype, const cf_epilogue* mid, void* stream) {
  if (batch < 0 || M < 0 || K < 0 || L < 0 || N < 0) return CF_ERR_INVALID_ARGUMENT;
  if (!is_dtype(cf::ev(in_dtype)) || !is_dtype(cf::ev(out_dtype))) return CF_ERR_INVALID_ARGUMENT;
  if (b0_is_lk != 0 && b0_is_lk != 1) return CF_ERR_INVALID_ARGUMENT;
  if (sa < 0 || sb0 < 0 || sb1 < 0 || so < 0) return CF_ERR_INVALID_ARGUMENT;
  cf_status st = check_epilogue(mid, L, false, false);
  if (st != CF_OK) return st;
  if (batch == 0 || M == 0 || N == 0) return CF_OK;
  if (!A || !B0 || !B1 || !O) return CF_ERR_INVALID_ARGUMENT;
  if (lda < K || ldb0 < (b0_is_lk ? K : L) || ldb1 < N || ldo < N) return CF_ERR_INVALID_ARGUMENT;
  if (in_dtype != CF_BF16) return CF_ERR_UNSUPPORTED;
  const size_t os = dsize(out_dtype);
  if (!aligned(A, 16) || !aligned(B0, 16) || !aligned(B1, 16) || !aligned(O, os)) return CF_ERR_UNSUPPORTED;
  if (lda % 8 || ldb0 % 8 || ldb1 % 8 || sa % 8 || sb0 % 8 || sb1 % 8) return CF_ERR_UNSUPPORTED;
  if (mid && mid->bias && mid->vec_dtype != CF_BF16 && mid->vec_dtype != CF_F32) return CF_ERR_INVALID_ARGUMENT;
  // the softmax kernels take the scores alpha * S as they are
  if (mid && mid->row_op == CF_ROW_SOFTMAX && (mid->bias || mid->act != CF_ACT_NONE)) return CF_ERR_UNSUPPORTED;
  if (batch > INT32_MAX || M > INT32_MAX || L > INT32_MAX || K > INT32_MAX || N > INT32_MAX) return CF_ERR_UNSUPPORTED;

  cf::B2bParams p;
  std::memset(&p, 0, sizeof(p));
  p.A = A;
  p.B0 = B0;
  p.B1 = B1;
  p.O = O;
  p.bias = mid ? mid->bias : nullptr;
  p.lda = (uint32_t)lda;
  p.ldb0 = (uint32_t)ldb0;
  p.ldb1 = (uint32_t)ldb1;
  p.ldo = (uint32_t)ldo;
  p.sa = (uint64_t)sa;
  p.sb0 = (uint64_t)sb0;
  p.sb1 = (uint64_t)sb1;
  p.so = (uint64_t)so;
  p.batch = (int)batch;
  p.M = (int)M;
  p.K = (int)K;
  p.L = (int)L;
  p.N = (int)N;
  p.alpha = mid ? mid->alpha : 1.0f;
  p.act = mid ? (int)mid->act : 0;
  p.row_op = mid ? (int)mid->row_op : 0;
  p.out_f32 = out_dtype == CF_F32;
  p.bias_f32 = (mid && mid->vec_dtype == CF_F32) ? 1 : 0;
  p.bias_vec = p.bias && aligned(p.bias, 4);
  p.b0_lk = b0_is_lk;
  p.o_vec = aligned(O, 16) && ldo % 4 == 0 && so % 4 == 0;
  p.causal = mid && mid->mask == CF_MASK_CAUSAL;
  p.row_stats = mid ? mid->row_stats : nullptr;
  p.coff = (int)(L - M);
  p.pingpong = g_b2b_pingpong.load();
  if (!cf::b2b_supported(p)) return CF_ERR_UNSUPPORTED;

  int dev;
  DeviceInfo info;
  if ((st = current_device(&dev, &info)) != CF_OK) return st;
  hipError_t e = cf::launch_b2b(p, (hipStream_t)stream);
  return e == hipSuccess ? CF_OK : hip_fail(e);
}

const char* cf_status_string(cf_status s) {
  switch (s) {
    case CF_OK: return "CF_OK";
    case CF_ERR_INVALID_ARGUMENT: return "CF_ERR_INVALID_ARGUMENT";
    case CF_ERR_UNSUPPORTED: return "CF_ERR_UNSUPPORTED";
    case CF_ERR_WORKSPACE: return "CF_ERR_WORKSPACE";
    case CF_ERR_NO_DEVICE: return "CF_ERR_NO_DEVICE";
    case CF_ERR_HIP: return "CF_ERR_HIP";
    case CF_ERR_DEVICE_TIMEOUT: return "CF_ERR_DEVICE_TIMEOUT";
  }
  return "CF_ERR_UNKNOWN";
}

int cf_last_hip_error(void) { return g_last_hip_error; }

const char* cf_version(void) { return "cf 0.1.0 (gfx950)"; }

uint64_t cf_set_exchange_timeout_us(uint64_t us) { return g_timeout_us.exchange(us); }

int cf_set_exchange_leader_tiles(int min_tiles) {
  return min_tiles < 0 ? g_lf_tiles.load() : g_lf_tiles.exchange(min_tiles);
}

int cf_set_b2b_pingpong(int on) {
  return on < 0 ? g_b2b_pingpong.load() : g_b2b_pingpong.exchange(on ? 1 : 0);
}

}  // extern "C"
