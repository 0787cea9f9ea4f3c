// Issue-rate microbenchmarks behind the design of the forward kernels: how
// much softmax-type work (fp32 FMAs, exponentials, LDS operand reads) a SIMD
// can run beside 32x32x16 bf16 MFMAs, when one wave issues both kinds and when
// different waves do.  A diagnostic library of its own (libfa_probe.so, built
// by `python -m exact_io_aware_48_amd.build --probes`), not part of the
// product library; `python bench.py --issue-probes` runs it.
//
// Every kernel runs one workgroup per CU (grid = the device's CU count) for a
// fixed number of iterations and writes one float per thread to `out` (so
// that no work is dead); the host times `reps` back-to-back launches with HIP
// events after `reps / 2 + 1` warm-up launches.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 96 * 1024;   // one workgroup per CU

// Mixed waves: NT threads (256: one wave per SIMD, 512: two), each wave
// issuing per iteration 8 groups of [one MFMA (if MF), NL ds_read_b128 whose
// results feed later MFMAs, NV independent FMAs, NE exponentials], in that
// order (pinned with sched_group_barrier).
template <int NT, bool MF, int NV, int NE, int NL>
__global__ __launch_bounds__(NT) void probe_mixed(float* out, int iters, float seed) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += NT) reinterpret_cast<float*>(lds)[i] = 1e-3f * (i & 7);
  __syncthreads();
  bf16x8 op[8], b;
  for (int i = 0; i < 8; ++i) {
    b[i] = (__bf16)(seed + i);
    for (int j = 0; j < 8; ++j) op[j][i] = (__bf16)(seed * (lane + i + (j & 3)));
  }
  f32x16 c[8];
  for (int j = 0; j < 8; ++j) c[j] = f32x16{};
  float x[32], y[32];
  for (int i = 0; i < 32; ++i) {
    x[i] = seed * (threadIdx.x + i);
    y[i] = seed * (i - lane);
  }
  // reads stay inside the first (8 * NL) KiB of the 96 KiB array
  const char* lp = lds + lane * 16;
  static_assert(8 * NL * 1024 <= kLdsBytes, "LDS reads in bounds");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if constexpr (MF) c[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], b, c[m], 0, 0, 0);
#pragma unroll
      for (int l = 0; l < NL; ++l)
        op[(m + 4 + l) & 7] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(lp + (m * NL + l) * 1024));
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int r = (m * NV + v) & 31;
        x[r] = __builtin_fmaf(x[r], 0.999f, 0.001f);
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int r = (m * NE + e) & 31;
        y[r] = __builtin_amdgcn_exp2f(-__builtin_fabsf(y[r]));
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if constexpr (MF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (NL > 0) __builtin_amdgcn_sched_group_barrier(0x100, NL, 0);
      if constexpr (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
      if constexpr (NE > 0) __builtin_amdgcn_sched_group_barrier(0x400, NE, 0);
    }
  }
  float acc = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int i = 0; i < 16; ++i) acc += c[j][i];
  for (int j = 0; j < 8; ++j)
    for (int i = 0; i < 8; ++i) acc += (float)op[j][i];
  for (int i = 0; i < 32; ++i) acc += x[i] + y[i];
  out[(int64_t)blockIdx.x * NT + threadIdx.x] = acc;
}

// Split roles: 512 threads, waves 0-3 (one per SIMD) issue 8 MFMAs per
// iteration when ROLE & 1; waves 4-7 (one per SIMD) issue 64 FMAs per
// iteration when ROLE & 2, or 64 exponentials when ROLE & 4 as well.
template <int ROLE>
__global__ __launch_bounds__(512) void probe_roles(float* out, int iters, float seed) {
  // the mixed kernels' LDS footprint, so that one workgroup runs per CU here too
  __shared__ float lds[kLdsBytes / 4];
  if (threadIdx.x == 0) lds[kLdsBytes / 4 - 1] = 0.f;
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float acc = lds[kLdsBytes / 4 - 1];
  if (wave < 4) {
    if constexpr ((ROLE & 1) != 0) {
      bf16x8 a, b;
      for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (threadIdx.x + i));
        b[i] = (__bf16)(seed + i);
      }
      f32x16 c[8];
      for (int j = 0; j < 8; ++j) c[j] = f32x16{};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
      }
      for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 16; ++i) acc += c[j][i];
    }
  } else if constexpr ((ROLE & 2) != 0) {
    float x[16];
    for (int i = 0; i < 16; ++i) x[i] = seed * (threadIdx.x + i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr ((ROLE & 4) != 0) x[i] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[i]));
          else x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
        }
    }
    for (int i = 0; i < 16; ++i) acc += x[i];
  }
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = acc;
}

int launch(void (*kern)(float*, int, float), int cus, int threads, float* out, int iters) {
  float seed = 1e-3f;
  void* args[] = {&out, &iters, &seed};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(cus), dim3(threads), args, 0, nullptr) == hipSuccess
             ? 0 : 6;
}

int time_kernel(void (*kern)(float*, int, float), int threads, float* out, int iters, int reps, float* ms) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 6;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 6;
  int st = 0;
  for (int r = 0; r < reps / 2 + 1 && st == 0; ++r) st = launch(kern, cus, threads, out, iters);
  if (st == 0 && hipEventRecord(e0, nullptr) != hipSuccess) st = 6;
  for (int r = 0; r < reps && st == 0; ++r) st = launch(kern, cus, threads, out, iters);
  if (st == 0 && (hipEventRecord(e1, nullptr) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)) st = 6;
  float t = 0.f;
  if (st == 0 && hipEventElapsedTime(&t, e0, e1) != hipSuccess) st = 6;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st == 0) *ms = t / reps;
  return st;
}

}  // namespace

extern "C" {

// The mixed-wave configurations, by index; fa_probe_mixed_name gives each one's
// label.  Returns 0, 2 for an unknown index or a short out buffer (it needs
// 512 floats per CU), 6 for a HIP error.
int fa_probe_mixed_count(void) { return 12; }

const char* fa_probe_mixed_name(int i) {
  static const char* names[] = {
      "2 waves/SIMD: 8 MFMA",                 "2 waves/SIMD: 64 FMA",
      "2 waves/SIMD: 32 exp",                 "2 waves/SIMD: 8 MFMA + 64 FMA",
      "2 waves/SIMD: 8 MFMA + 32 exp",        "2 waves/SIMD: 8 MFMA + 24 FMA + 8 exp",
      "2 waves/SIMD: 8 MFMA + 8 ds_read_b128", "2 waves/SIMD: 8 MFMA + 24 FMA + 8 exp + 8 ds_read_b128",
      "1 wave/SIMD: 8 MFMA",                  "1 wave/SIMD: 64 FMA",
      "1 wave/SIMD: 8 MFMA + 64 FMA",         "1 wave/SIMD: 8 MFMA + 24 FMA + 8 exp"};
  return i >= 0 && i < 12 ? names[i] : "";
}

// per-wave and per-iteration work of configuration i: {waves per SIMD, MFMAs, FMAs, exps, LDS reads}
int fa_probe_mixed_work(int i, int* work5) {
  static const int w[12][5] = {{2, 8, 0, 0, 0},  {2, 0, 64, 0, 0}, {2, 0, 0, 32, 0}, {2, 8, 64, 0, 0},
                               {2, 8, 0, 32, 0}, {2, 8, 24, 8, 0}, {2, 8, 0, 0, 8},  {2, 8, 24, 8, 8},
                               {1, 8, 0, 0, 0},  {1, 0, 64, 0, 0}, {1, 8, 64, 0, 0}, {1, 8, 24, 8, 0}};
  if (i < 0 || i >= 12 || !work5) return 2;
  for (int k = 0; k < 5; ++k) work5[k] = w[i][k];
  return 0;
}

int fa_probe_mixed(int i, float* out, int64_t out_floats, int iters, int reps, float* ms) {
  int cus = 0, dev = 0;
  if (!out || !ms || iters < 1 || reps < 1) return 2;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 6;
  if (out_floats < (int64_t)cus * 512) return 2;
  switch (i) {
    case 0: return time_kernel(probe_mixed<512, true, 0, 0, 0>, 512, out, iters, reps, ms);
    case 1: return time_kernel(probe_mixed<512, false, 8, 0, 0>, 512, out, iters, reps, ms);
    case 2: return time_kernel(probe_mixed<512, false, 0, 4, 0>, 512, out, iters, reps, ms);
    case 3: return time_kernel(probe_mixed<512, true, 8, 0, 0>, 512, out, iters, reps, ms);
    case 4: return time_kernel(probe_mixed<512, true, 0, 4, 0>, 512, out, iters, reps, ms);
    case 5: return time_kernel(probe_mixed<512, true, 3, 1, 0>, 512, out, iters, reps, ms);
    case 6: return time_kernel(probe_mixed<512, true, 0, 0, 1>, 512, out, iters, reps, ms);
    case 7: return time_kernel(probe_mixed<512, true, 3, 1, 1>, 512, out, iters, reps, ms);
    case 8: return time_kernel(probe_mixed<256, true, 0, 0, 0>, 256, out, iters, reps, ms);
    case 9: return time_kernel(probe_mixed<256, false, 8, 0, 0>, 256, out, iters, reps, ms);
    case 10: return time_kernel(probe_mixed<256, true, 8, 0, 0>, 256, out, iters, reps, ms);
    case 11: return time_kernel(probe_mixed<256, true, 3, 1, 0>, 256, out, iters, reps, ms);
    default: return 2;
  }
}

// Split roles, role = bit 0 MFMA waves, bit 1 VALU waves, bit 2 exponentials
// in place of the FMAs (1, 2, 3, 6, 7 are the meaningful ones).
int fa_probe_roles(int role, float* out, int64_t out_floats, int iters, int reps, float* ms) {
  int cus = 0, dev = 0;
  if (!out || !ms || iters < 1 || reps < 1) return 2;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 6;
  if (out_floats < (int64_t)cus * 512) return 2;
  switch (role) {
    case 1: return time_kernel(probe_roles<1>, 512, out, iters, reps, ms);
    case 2: return time_kernel(probe_roles<2>, 512, out, iters, reps, ms);
    case 3: return time_kernel(probe_roles<3>, 512, out, iters, reps, ms);
    case 6: return time_kernel(probe_roles<6>, 512, out, iters, reps, ms);
    case 7: return time_kernel(probe_roles<7>, 512, out, iters, reps, ms);
    default: return 2;
  }
}

}  // extern "C"
