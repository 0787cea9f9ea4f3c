// The ALiBi and block-sparse forward instances (every mode and head dim),
// kept in their own translation unit so that they compile beside the plain
// kernels.  Called from fa_api.hip after its argument checks.
#include <hip/hip_runtime.h>

#include "fa_launch.hpp"

namespace {

// fp32 inputs at d = 256 have no variant instance (fa_api.hip rejects them
// first): it needs more registers than a wave holds, and its spilled form got
// rows of the ragged causal diagonal tile wrong.
template <int MODE, int VAR>
hipError_t dispatch_mode(const Params& p, int d, bool causal, int grid, hipStream_t s) {
  if (d == 64) return causal ? launch<MODE, 64, true, VAR>(p, grid, s) : launch<MODE, 64, false, VAR>(p, grid, s);
  if (d == 128)
    return causal ? launch<MODE, 128, true, VAR>(p, grid, s) : launch<MODE, 128, false, VAR>(p, grid, s);
  if constexpr (MODE == fa::MODE_F32)
    return hipErrorNotSupported;
  else
    return causal ? launch<MODE, 256, true, VAR>(p, grid, s) : launch<MODE, 256, false, VAR>(p, grid, s);
}

template <int VAR>
hipError_t dispatch_var(int mode, const Params& p, int d, bool causal, int grid, hipStream_t s) {
  switch (mode) {
    case fa::MODE_BF16: return dispatch_mode<fa::MODE_BF16, VAR>(p, d, causal, grid, s);
    case fa::MODE_FP8: return dispatch_mode<fa::MODE_FP8, VAR>(p, d, causal, grid, s);
    default: return dispatch_mode<fa::MODE_F32, VAR>(p, d, causal, grid, s);
  }
}

}  // namespace

hipError_t fa_dispatch_variant(int var, int mode, const fa::Params& p, int d, bool causal, int grid,
                               hipStream_t stream) {
  if (var == fa::VAR_ALIBI) return dispatch_var<fa::VAR_ALIBI>(mode, p, d, causal, grid, stream);
  return dispatch_var<fa::VAR_BLOCKSPARSE>(mode, p, d, causal, grid, stream);
}
