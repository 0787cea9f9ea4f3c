// C ABI of the FlashAttention backward (declared in include/fa_bwd.h):
// argument checks, kernel instances, grids and the three launches.  No
// allocation, no synchronisation; the only state is the per-device residency
// cache (fa_host.hpp); the caller provides the
// statistics workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa_bwd.h"
#include "fa_bwd_kernel.hpp"
#include "fa_host.hpp"

namespace {

using fa::BwdParams;

// Shapes per head dim.  dK/dV: NW waves of 32 keys, each holding K and the
// two fp32 accumulators in VGPRs.  At d = 128 the main shape stages V in LDS
// (K, V and the accumulators would not fit the 256 VGPRs of two waves per
// SIMD) and gives a workgroup 256 keys; the small shape (128 keys, one wave
// per SIMD with K and V in VGPRs) serves small causal grids (launch_dkdv).
// At d = 64 V stays in VGPRs.
// dQ: NW waves of 32 queries, B_c-key K/V tiles.
template <int NW_, int WPE_, bool VLDS_, int KW_ = 32> struct KvShape {
  static constexpr int NW = NW_, WPE = WPE_, KW = KW_;   // KW: keys per wave
  static constexpr bool VLDS = VLDS_;
};
template <int D> struct BwdCfg;
template <> struct BwdCfg<64> {
  using KV = KvShape<4, 2, false>;
  using KV_SMALL = KV;
  static constexpr int Q_BC = 64, Q_NW = 4, Q_WPE = 2;
};
template <> struct BwdCfg<128> {
  using KV = KvShape<8, 2, true>;
  using KV_SMALL = KvShape<4, 1, false>;
  static constexpr int Q_BC = 64, Q_NW = 8, Q_WPE = 2;
};
// d = 256: a wave's dK and dV accumulators alone take 256 registers, so both
// kernels run one wave per SIMD (the 512-register file), four waves per
// workgroup; K and V stay in VGPRs (V in LDS would not fit beside the
// 2 x 64 KiB Q/dO ring).
template <> struct BwdCfg<256> {
  using KV = KvShape<4, 1, false, 16>;
  using KV_SMALL = KV;
  static constexpr int Q_BC = 32, Q_NW = 4, Q_WPE = 1;
};

int64_t stat_tiles(int64_t N) { return (N + fa::kStatRows - 1) / fa::kStatRows; }

// workspace: the statistics tiles, then (grouped query heads only) room for
// dK and dV partials of up to G parts per K/V head
int64_t stats_bytes(int64_t BH, int64_t N) { return BH * stat_tiles(N) * (2 * fa::kStatRows) * (int64_t)sizeof(float); }
int64_t partial_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d) {
  return H > H_kv ? 2 * B * H * N * d * (int64_t)sizeof(float) : 0;
}

// A causal grid's workgroups are dealt zig-zag over the CUs when the whole
// grid is resident at once (see map_block).
template <bool CAUSAL>
void set_balance(BwdParams& p, const void* kern, int threads, int grid, std::atomic<int>* cache) {
  if constexpr (CAUSAL) {
    const Residency r = residency(kern, threads, cache);
    p.cus_per_xcd = r.cus_per_xcd;
    p.zigzag = r.cus_per_xcd > 0 && grid <= r.resident ? 1 : 0;
  } else {
    (void)kern; (void)threads; (void)grid; (void)cache;
  }
}

template <int D, bool CAUSAL, class S>
hipError_t launch_dkdv_shape(const BwdParams& base, int64_t BHkv, int parts, hipStream_t stream) {
  BwdParams p = base;
  constexpr int BK = S::KW * S::NW;
  p.BH = (int)(BHkv * parts);                // (K/V head, part) pairs
  p.parts = parts;
  p.nrb = (base.N + BK - 1) / BK;
  p.G = 1;
  p.xcd_heads = p.BH % 8 == 0 ? 1 : 0;
  void (*kern)(BwdParams) = &fa::fa_bwd_dkdv_kernel<D, S::NW, S::WPE, CAUSAL, S::VLDS, S::KW>;
  const int grid = p.nrb * p.BH;
  static std::atomic<int> cache[kMaxDevices];
  set_balance<CAUSAL>(p, reinterpret_cast<const void*>(kern), 64 * S::NW, grid, cache);
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(grid), dim3(64 * S::NW), args, 0, stream);
  if (e != hipSuccess || parts == 1) return e;
  const int64_t n4 = BHkv * base.N * D / 4;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
  void* rargs[] = {&p, const_cast<int64_t*>(&n4)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_bwd_reduce_kernel), dim3((unsigned)blocks), dim3(256),
                         rargs, 0, stream);
}

// Shape and split of the dK/dV launch.  A grid of main-shape workgroups that
// fills fewer than two rounds of resident workgroups (one round without the
// causal mask, whose blocks are equal) is dominated by its heaviest blocks:
// grouped query heads are then split over up to G workgroups per key block
// (partials summed afterwards); with one query head per K/V head a causal
// grid takes the small shape instead.
template <int D, bool CAUSAL, class BIG, class SMALL>
hipError_t launch_dkdv(const BwdParams& base, int64_t BHkv, int G, hipStream_t stream) {
  constexpr int BK = BIG::KW * BIG::NW;
  static std::atomic<int> cache[kMaxDevices];
  const Residency r = residency(reinterpret_cast<const void*>(&fa::fa_bwd_dkdv_kernel<D, BIG::NW, BIG::WPE, CAUSAL,
                                                                                      BIG::VLDS, BIG::KW>),
                                64 * BIG::NW, cache);
  const int64_t grid = (base.N + BK - 1) / BK * BHkv;
  const int64_t target = (CAUSAL ? 2 : 1) * (int64_t)r.resident;
  if (r.resident > 0 && grid < target) {
    if (G > 1) {
      const int parts = (int)std::min<int64_t>(G, (target + grid - 1) / grid);
      return launch_dkdv_shape<D, CAUSAL, BIG>(base, BHkv, parts, stream);
    }
    if constexpr (CAUSAL && !std::is_same<BIG, SMALL>::value) return launch_dkdv_shape<D, CAUSAL, SMALL>(base, BHkv, 1, stream);
  }
  return launch_dkdv_shape<D, CAUSAL, BIG>(base, BHkv, 1, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdParams& base, int64_t B, int64_t H, int64_t H_kv, hipStream_t stream) {
  using C = BwdCfg<D>;
  const int N = base.N;

  // 1. dQ, forming the statistics of its rows on the way: one workgroup per
  //    32*Q_NW queries of a query head
  {
    BwdParams p = base;
    constexpr int BR = 32 * C::Q_NW;
    p.BH = (int)(B * H);
    p.nrb = (N + BR - 1) / BR;
    p.G = base.qg;
    p.xcd_heads = (p.BH / p.G) % 8 == 0 ? 1 : 0;
    void (*kern)(BwdParams) = &fa::fa_bwd_dq_kernel<D, C::Q_BC, C::Q_NW, C::Q_WPE, CAUSAL>;
    const int grid = p.nrb * p.BH;
    static std::atomic<int> cache[kMaxDevices];
    set_balance<CAUSAL>(p, reinterpret_cast<const void*>(kern), 64 * C::Q_NW, grid, cache);
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(grid), dim3(64 * C::Q_NW), args, 0,
                                   stream);
    if (e != hipSuccess) return e;
  }
  // 2. dK, dV: one workgroup per 32*NW keys of a K/V head, reading the statistics
  return launch_dkdv<D, CAUSAL, typename C::KV, typename C::KV_SMALL>(base, B * H_kv, (int)(H / H_kv), stream);
}

fa_status check_bwd_shape(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int dtype) {
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 1 || H_kv < 1 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (B > INT_MAX / H) return FA_ERR_SHAPE;                    // B*H fits an int
  if (N > (int64_t)INT_MAX / (2 * d)) return FA_ERR_SHAPE;     // one head's bytes fit an int
  const int64_t bh = B * H;
  if (bh > INT64_MAX / (N * d * 4)) return FA_ERR_SHAPE;       // byte sizes fit int64
  // grids: statistics tiles, key blocks and query blocks (at least 64 rows each)
  if (bh * stat_tiles(N) > INT_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd_workspace_size(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int64_t* bytes) {
  if (!bytes) return FA_ERR_NULL;
  const fa_status st = check_bwd_shape(B, H, H_kv, N, d, FA_BF16);
  if (st != FA_OK) return st;
  *bytes = stats_bytes(B * H, N) + partial_bytes(B, H, H_kv, N, d);
  return FA_OK;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* workspace, float* dq, float* dk, float* dv, int64_t B, int64_t H, int64_t H_kv, int64_t N,
                 int64_t d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !workspace || !dq || !dk || !dv) return FA_ERR_NULL;
  const fa_status st = check_bwd_shape(B, H, H_kv, N, d, dtype);
  if (st != FA_OK) return st;
  for (const void* ptr : {q, k, v, o, dout, (const void*)lse, (const void*)workspace, (const void*)dq,
                          (const void*)dk, (const void*)dv})
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  const float c2 = scale * 1.4426950408889634f;
  if (!std::isfinite(scale) || !std::isfinite(c2)) return FA_ERR_SCALE;

  BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.ws = static_cast<float*>(workspace);
  p.part_out = p.ws + stats_bytes(B * H, N) / (int64_t)sizeof(float);
  p.parts = 1;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.N = (int)N;
  p.qg = (int)(H / H_kv);
  p.T = (int)stat_tiles(N);
  p.c2 = c2;
  p.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d == 64) e = causal ? launch_bwd<64, true>(p, B, H, H_kv, s) : launch_bwd<64, false>(p, B, H, H_kv, s);
  else if (d == 128) e = causal ? launch_bwd<128, true>(p, B, H, H_kv, s) : launch_bwd<128, false>(p, B, H, H_kv, s);
  else e = causal ? launch_bwd<256, true>(p, B, H, H_kv, s) : launch_bwd<256, false>(p, B, H, H_kv, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
