// C ABI of split-KV decode attention and the logsumexp merge (declared in
// include/fa_split.h): argument checks, split plan, launches.  No
// allocation and no synchronisation.  fa_fwd_split_noalloc keeps its partials
// in the file-scope device array `scratch` (one copy per GPU, held until the
// process ends) and caches each device's address of it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <climits>
#include <cmath>
#include <cstdint>

#include "fa_split.h"
#include "fa_split_kernel.hpp"
#include "fa_host.hpp"

// Partials of fa_fwd_split_noalloc: a fixed device array instead of a
// caller's workspace.  The split kernel writes every element of the partials a
// call uses before the merge reads it, so no call needs it cleared.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

namespace {

using fa::MergeParams;
using fa::SplitParams;

// Each device's address of `scratch` (the host-side name is only a stand-in
// for it), looked up with that device current on its first call there.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Keys per tile per head dim: one wave per workgroup, 32 KiB of K/V ring at
// d = 64 and 128, so that five workgroups share a CU and keep enough of the
// K/V stream in flight.  d = 256 takes the smallest tile the 32 x 32 MFMA
// allows (32 keys), a 64 KiB ring and two workgroups per CU.  fp8 takes
// 64-key tiles at every d (its P V MFMA consumes 64 keys), which at one byte
// per element gives the same ring sizes (16, 32 and 64 KiB).
constexpr int split_bc_of(int d, bool fp8) { return fp8 || d == 64 ? 64 : 32; }
int split_bc(int64_t d, int dtype) { return split_bc_of((int)d, dtype == FA_FP8_E4M3); }
constexpr int kSplitNW = 1;
constexpr int kRowsPerBlock = 32 * kSplitNW;

struct Plan {
  int64_t rows_per_head;   // G * N_q
  int64_t nrb;             // row blocks per K/V head
  int64_t splits;
  int64_t chunk;           // keys per split
  int64_t workspace_bytes;
};

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return cus;
}

fa_status check_split_shape(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, int dtype) {
  if (dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || N_q < 1 || N_k < N_q) return FA_ERR_SHAPE;
  if (B > INT_MAX / H) return FA_ERR_SHAPE;
  if (N_k > (int64_t)INT_MAX / (2 * d) || N_q > (int64_t)INT_MAX / (2 * d)) return FA_ERR_SHAPE;
  if (B * H > INT64_MAX / (N_k * d * 4)) return FA_ERR_SHAPE;
  if ((H / H_kv) * N_q > INT_MAX / 2) return FA_ERR_SHAPE;
  return FA_OK;
}

// The split plan: num_splits > 0 asks for that many (fewer when the tiles run
// out); 0 picks enough splits for about two workgroups per CU (the best of 2
// to 32 splits on every decode shape measured on MI355X: B = 8, H_kv = 8,
// N_k = 32K takes 8; B = 4, H = 32, N_k = 16K takes 4), each split keeping at
// least four tiles.
fa_status make_plan(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, int num_splits,
                    int dtype, int cus, Plan* out) {
  if (num_splits < 0) return FA_ERR_SHAPE;
  const int64_t bc = split_bc(d, dtype);
  Plan pl{};
  pl.rows_per_head = (H / H_kv) * N_q;
  pl.nrb = (pl.rows_per_head + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t base = B * H_kv * pl.nrb;
  const int64_t tiles = (N_k + bc - 1) / bc;
  int64_t want = num_splits;
  if (want == 0) {
    want = (2 * (int64_t)cus + base - 1) / base;
    want = std::max<int64_t>(1, std::min(want, tiles / 4));
  }
  want = std::min(want, tiles);
  const int64_t chunk_tiles = (tiles + want - 1) / want;
  pl.chunk = chunk_tiles * bc;
  pl.splits = (tiles + chunk_tiles - 1) / chunk_tiles;
  if (pl.splits * base > INT_MAX) return FA_ERR_SHAPE;
  const int64_t rows_total = B * H * N_q;
  if (rows_total > INT64_MAX / (pl.splits * (d + 1) * 4)) return FA_ERR_SHAPE;
  pl.workspace_bytes = pl.splits * rows_total * (d + 1) * 4;
  *out = pl;
  return FA_OK;
}

// K/V ring depth.  Measured on MI355X at 2 to 5 stages with plain loads:
// 5.5-5.8 TB/s whatever the depth (a 1 GiB device copy reaches 5.2).  With
// the streaming loads a third stage is slower (GQA decode 155.8 -> 162.6 us,
// fp8 80.9 -> 83.5 us), so the plain double buffer is kept.
constexpr int kSplitNS = 2;

template <int D, bool CAUSAL, int MODE>
hipError_t launch_split(const SplitParams& p, int grid, hipStream_t stream) {
  constexpr int BC = split_bc_of(D, MODE == fa::MODE_FP8);
  void (*kern)(SplitParams) = &fa::fa_split_kernel<D, BC, kSplitNW, kSplitNS, CAUSAL, MODE>;
  SplitParams args = p;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(grid), dim3(64 * kSplitNW), kargs, 0, stream);
}

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int64_t S, int64_t rows, int64_t d, void* o,
                        float* lse, bool out_bf16, hipStream_t stream) {
  MergeParams mp{};
  mp.o_part = o_parts;
  mp.lse_part = lse_parts;
  mp.o = o;
  mp.lse = lse;
  mp.rows = rows;
  mp.S = (int)S;
  mp.d = (int)d;
  mp.out_bf16 = out_bf16 ? 1 : 0;
  void* kargs[] = {&mp};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_merge_kernel), dim3((unsigned)((rows + 3) / 4)),
                         dim3(256), kargs, 0, stream);
}

}  // namespace

extern "C" {

fa_status fa_fwd_split_plan(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, int num_splits,
                            int dtype, int* splits, int64_t* workspace_bytes) {
  fa_status st = check_split_shape(B, H, H_kv, N_q, N_k, d, dtype);
  if (st != FA_OK) return st;
  Plan pl;
  st = make_plan(B, H, H_kv, N_q, N_k, d, num_splits, dtype, num_splits == 0 ? device_cus() : 256, &pl);
  if (st != FA_OK) return st;
  if (splits) *splits = (int)pl.splits;
  if (workspace_bytes) *workspace_bytes = pl.workspace_bytes;
  return FA_OK;
}

}  // extern "C"

namespace {

template <int MODE>
hipError_t launch_split_mode(const SplitParams& p, int64_t d, bool causal, int grid, hipStream_t s) {
  if (d == 64) return causal ? launch_split<64, true, MODE>(p, grid, s) : launch_split<64, false, MODE>(p, grid, s);
  if (d == 128) return causal ? launch_split<128, true, MODE>(p, grid, s) : launch_split<128, false, MODE>(p, grid, s);
  return causal ? launch_split<256, true, MODE>(p, grid, s) : launch_split<256, false, MODE>(p, grid, s);
}

// fa_fwd_split (and fa_fwd_split_fp8, dtype FA_FP8_E4M3 with the three
// descales) with the partials either in the caller's workspace or, when
// workspace is NULL, in `scratch` (fa_fwd_split_noalloc)
fa_status run_split(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace, int64_t B,
                    int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, float scale, int causal,
                    int num_splits, int dtype, void* stream, float dq = 1.f, float dk = 1.f, float dv = 1.f) {
  const bool use_scratch = workspace == nullptr;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_split_shape(B, H, H_kv, N_q, N_k, d, dtype);
  if (st != FA_OK) return st;
  for (const void* ptr : {q, k, v, (const void*)o, (const void*)lse})
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  if (!use_scratch && !aligned16(workspace)) return FA_ERR_ALIGN;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  for (float ds : {dq, dk, dv})
    if (!std::isfinite(ds) || !(ds > 0.f)) return FA_ERR_SCALE;
  const bool fp8 = dtype == FA_FP8_E4M3;
  const double c2 = std::fabs((double)scale) * (double)dq * (double)dk * 1.4426950408889634;
  if (!std::isfinite((float)c2)) return FA_ERR_SCALE;
  Plan pl;
  st = make_plan(B, H, H_kv, N_q, N_k, d, num_splits, dtype, num_splits == 0 ? device_cus() : 256, &pl);
  if (st != FA_OK) return st;
  if (use_scratch) {
    if (pl.workspace_bytes > kScratchBytes) return FA_ERR_SCRATCH;
    workspace = scratch_on_current_device();
    if (!workspace) return FA_ERR_HIP;
  }

  const int64_t rows_total = B * H * N_q;
  SplitParams p{};
  p.q = q; p.k = k; p.v = v;
  p.o_part = static_cast<float*>(workspace);
  p.lse_part = p.o_part + pl.splits * rows_total * d;
  p.BHkv = (int)(B * H_kv);
  p.G = (int)(H / H_kv);
  p.N_q = (int)N_q;
  p.N_k = (int)N_k;
  p.rows = (int)pl.rows_per_head;
  p.nrb = (int)pl.nrb;
  p.S = (int)pl.splits;
  p.chunk = (int)pl.chunk;
  // masked scores are -inf and rely on c2 > 0 (see fa_api.hip); a negative scale flips Q's sign bits
  p.c2 = std::max((float)c2, 1e-30f);
  p.out_mul = fp8 ? dv : 1.f;
  p.qsign = scale < 0.f ? (fp8 ? 0x80808080u : 0x80008000u) : 0u;
  const int grid = (int)(pl.splits * pl.nrb * B * H_kv);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e0 = fp8 ? launch_split_mode<fa::MODE_FP8>(p, d, causal != 0, grid, s)
                            : launch_split_mode<fa::MODE_BF16>(p, d, causal != 0, grid, s);
  if (e0 != hipSuccess) return FA_ERR_HIP;
  const hipError_t e = launch_merge(p.o_part, p.lse_part, pl.splits, rows_total, d, o, lse, true, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace, int64_t B,
                       int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, float scale, int causal,
                       int num_splits, int dtype, void* stream) {
  if (!workspace) return FA_ERR_NULL;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  return run_split(q, k, v, o, lse, workspace, B, H, H_kv, N_q, N_k, d, scale, causal, num_splits, dtype, stream);
}

fa_status fa_fwd_split_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse, void* workspace,
                           int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, float scale,
                           float q_descale, float k_descale, float v_descale, int causal, int num_splits,
                           void* stream) {
  if (!workspace) return FA_ERR_NULL;
  return run_split(q8, k8, v8, o_bf16, lse, workspace, B, H, H_kv, N_q, N_k, d, scale, causal, num_splits,
                   FA_FP8_E4M3, stream, q_descale, k_descale, v_descale);
}

fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                               int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, float scale, int causal,
                               int num_splits, int dtype, void* stream) {
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  return run_split(q, k, v, o, lse, nullptr, B, H, H_kv, N_q, N_k, d, scale, causal, num_splits, dtype, stream);
}

int64_t fa_split_scratch_bytes(void) { return kScratchBytes; }

fa_status fa_lse_merge(const float* o_parts, const float* lse_parts, int64_t num_parts, int64_t rows, int64_t d,
                       void* o, float* lse, int out_dtype, void* stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (out_dtype != FA_BF16 && out_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (num_parts < 1 || num_parts > INT_MAX || rows < 1 || d < 1 || d > 4096) return FA_ERR_SHAPE;
  if ((rows + 3) / 4 > INT_MAX || rows > INT64_MAX / (num_parts * d * 4)) return FA_ERR_SHAPE;
  for (const void* ptr : {(const void*)o_parts, (const void*)lse_parts, (const void*)o, (const void*)lse})
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  const hipError_t e = launch_merge(o_parts, lse_parts, num_parts, rows, d, o, lse, out_dtype == FA_BF16,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
