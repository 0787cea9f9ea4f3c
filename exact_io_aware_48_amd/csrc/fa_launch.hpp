// Host-side launch table of the forward: the kernel instance and tile shape
// per (mode, head dim, variant), and the launch itself.  Shared by the plain
// entry points (fa_api.hip) and the mask variants (fa_var_api.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "fa_fwd_kernel.hpp"
#include "fa_pipe_kernel.hpp"
#include "fa_host.hpp"

namespace {

using fa::Params;

// A launch plan: tile shape and LDS footprint of the kernel instance used.
struct Tile {
  int bc;      // keys per K/V tile
  int nw;      // waves per workgroup, 32 query rows each
  int lds;     // LDS bytes per workgroup
  int br() const { return 32 * nw; }
};

// Shape per (mode, d), chosen by measurement on MI355X.  Eight waves per
// workgroup (256 query rows) halve the K/V traffic per FLOP for the large
// heads; d = 64 keeps four waves so that the short causal rows spread over
// more workgroups.  d = 256 with 16-bit tiles uses 32-key tiles to stay
// within 256 VGPRs at two waves per SIMD.  PRIO: raised wave priority
// outside the MFMA blocks (bf16 d = 256; fp8 d = 128 and 256, where it beat
// ping-pong by 2.1% and 1.4%).  PP: ping-pong wave groups (the upper half of
// the waves runs P V one tile late); the kernel keeps the option, no shape
// uses it since.
// PIPE: the software-pipelined kernel (fa_pipe_kernel.hpp), whose waves weave
// each tile's softmax into the neighbouring tiles' MFMAs (bf16, d = 128).
// RP: issue priority by the key tiles a workgroup has left (fa_fwd_kernel),
// for the non-causal bf16 d = 64 instance: there four equal workgroups share
// a CU, and the oldest waves' precedence otherwise has them finish one after
// another (the last alone on the CU).  Measured: BERT-large 22.5 -> 21.1 us;
// for causal rows, which differ in length, it cost 2%.
template <int MODE, int D> struct Cfg;
template <int BC_, int NW_, bool PP_, bool PRIO_ = false, bool PIPE_ = false, int RP_ = 0> struct Shape {
  static constexpr int BC = BC_, NW = NW_;
  static constexpr bool PP = PP_, PRIO = PRIO_, PIPE = PIPE_;
  static constexpr int RP = RP_;
};
template <> struct Cfg<fa::MODE_BF16, 64> : Shape<64, 4, false, false, false, 2> {};
template <> struct Cfg<fa::MODE_BF16, 128> : Shape<64, 8, false, false, true> {};
template <> struct Cfg<fa::MODE_BF16, 256> : Shape<32, 8, false, true> {};
template <> struct Cfg<fa::MODE_FP8, 64> : Shape<64, 4, false> {};
template <> struct Cfg<fa::MODE_FP8, 128> : Shape<64, 8, false, true> {};
template <> struct Cfg<fa::MODE_FP8, 256> : Shape<64, 8, false, true> {};
template <> struct Cfg<fa::MODE_F32, 64> : Shape<64, 4, false> {};
template <> struct Cfg<fa::MODE_F32, 128> : Shape<64, 4, false> {};
template <> struct Cfg<fa::MODE_F32, 256> : Shape<32, 4, false> {};
// The ALiBi and block-sparse variants are instances of fa_fwd_kernel with
// the plain shape's row block (so the grid is the same): bf16 d = 128 keeps
// the 128-key tiles measured for it before the pipelined kernel; raised
// priority is for the plain kernel only.
template <int MODE, int D> struct VarCfg : Cfg<MODE, D> {};
template <> struct VarCfg<fa::MODE_BF16, 128> : Shape<128, 8, false> {};

template <int MODE, int D>
Tile tile_for() {
  using C = Cfg<MODE, D>;
  // the pipelined kernel, and some plain instances, also stage the Q tile in LDS
  return Tile{C::BC, C::NW,
              fa::Geo<D, C::BC, C::NW, MODE, C::PP>::LDSB +
                  (C::PIPE ? 32 * C::NW * D * 2 : fa::q_region_bytes<D, C::BC, C::NW, MODE, C::PP>())};
}

Tile lookup_tile(int mode, int d) {
  switch (mode) {
    case fa::MODE_BF16:
      return d == 64 ? tile_for<fa::MODE_BF16, 64>() : d == 128 ? tile_for<fa::MODE_BF16, 128>()
                                                                 : tile_for<fa::MODE_BF16, 256>();
    case fa::MODE_FP8:
      return d == 64 ? tile_for<fa::MODE_FP8, 64>() : d == 128 ? tile_for<fa::MODE_FP8, 128>()
                                                                : tile_for<fa::MODE_FP8, 256>();
    default:
      return d == 64 ? tile_for<fa::MODE_F32, 64>() : d == 128 ? tile_for<fa::MODE_F32, 128>()
                                                                : tile_for<fa::MODE_F32, 256>();
  }
}

template <int MODE, int D, bool CAUSAL, int VAR = fa::VAR_NONE>
hipError_t launch(const Params& p, int grid, hipStream_t stream) {
  using C = typename std::conditional<VAR == fa::VAR_NONE, Cfg<MODE, D>, VarCfg<MODE, D>>::type;
  constexpr int BC = C::BC, NW = C::NW;
  static_assert(NW == Cfg<MODE, D>::NW, "variants and the plain kernel share the row-block size");
  void (*kern)(Params);
  if constexpr (VAR == fa::VAR_NONE && C::PIPE)
    kern = &fa::fa_fwd_pipe_kernel<D, BC, NW, CAUSAL>;
  else
    kern = &fa::fa_fwd_kernel<D, BC, NW, MODE, CAUSAL, C::PP, VAR, VAR == fa::VAR_NONE && C::PRIO,
                              VAR == fa::VAR_NONE && !CAUSAL ? C::RP : 0>;
  Params args = p;
  if constexpr (CAUSAL) {
    static std::atomic<int> cache[kMaxDevices];   // one per kernel
    const Residency r = residency(reinterpret_cast<const void*>(kern), NW * 64, cache);
    args.cus_per_xcd = r.cus_per_xcd;
    args.zigzag = r.cus_per_xcd > 0 && grid <= r.resident ? 1 : 0;
  }
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(grid), dim3(NW * 64), kargs, 0, stream);
}

}  // namespace

// ALiBi and block-sparse forward (fa_var_api.hip): every mode and head dim.
hipError_t fa_dispatch_variant(int var, int mode, const fa::Params& p, int d, bool causal, int grid,
                               hipStream_t stream);
