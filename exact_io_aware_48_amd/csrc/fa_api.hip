// C ABI of the FlashAttention forward library (declared in include/fa_fwd.h):
// argument checks, choice of kernel instance, grid, launch.  No allocation,
// no synchronisation; the only state is the per-device residency cache (fa_host.hpp).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <climits>
#include <atomic>
#include <type_traits>

#include "fa_fwd.h"
#include "fa_launch.hpp"

namespace {

using fa::Params;

template <int MODE>
hipError_t dispatch_d(const Params& p, int d, bool causal, int grid, hipStream_t s) {
  if (d == 64) return causal ? launch<MODE, 64, true>(p, grid, s) : launch<MODE, 64, false>(p, grid, s);
  if (d == 128) return causal ? launch<MODE, 128, true>(p, grid, s) : launch<MODE, 128, false>(p, grid, s);
  return causal ? launch<MODE, 256, true>(p, grid, s) : launch<MODE, 256, false>(p, grid, s);
}

// What a variant entry point adds to the plain forward.
struct Variant {
  int kind = fa::VAR_NONE;
  const float* slopes = nullptr;     // ALiBi
  const uint8_t* bmask = nullptr;    // block-sparse
  int64_t sb = 0, sh = 0;
};

int mode_of(int dtype) {
  return dtype == FA_BF16 ? fa::MODE_BF16 : dtype == FA_FP8_E4M3 ? fa::MODE_FP8 : fa::MODE_F32;
}

// shape and dtype checks shared by every entry point
fa_status check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (B > INT_MAX / H) return FA_ERR_SHAPE;                 // B*H fits an int
  if (N > (int64_t)INT_MAX / d) return FA_ERR_SHAPE;        // one head's elements fit an int
  const int64_t bh = B * H;
  if (bh > INT64_MAX / (N * d * 4)) return FA_ERR_SHAPE;    // byte sizes fit int64
  const Tile t = lookup_tile(mode_of(dtype), (int)d);
  const int64_t nrb = (N + t.br() - 1) / t.br();
  if (nrb * bh > INT_MAX) return FA_ERR_SHAPE;              // grid size
  return FA_OK;
}

fa_status run(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
              int64_t H_kv, int64_t N, int64_t d, float scale, float dq, float dk, float dv, int causal,
              int dtype, void* stream, const Variant& var = Variant{}) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (var.kind == fa::VAR_ALIBI && !var.slopes) return FA_ERR_NULL;
  if (var.kind == fa::VAR_BLOCKSPARSE && !var.bmask) return FA_ERR_NULL;
  fa_status st = check_shape(B, H, N, d, dtype);
  if (st == FA_OK && (H_kv < 1 || H % H_kv != 0)) st = FA_ERR_SHAPE;
  if (st == FA_OK && var.kind != fa::VAR_NONE && dtype == FA_F32 && d == 256) st = FA_ERR_UNSUPPORTED;
  if (st == FA_OK && var.kind == fa::VAR_BLOCKSPARSE && (var.sb < 0 || var.sh < 0)) st = FA_ERR_SHAPE;
  if (st != FA_OK) return st;
  if (var.kind == fa::VAR_ALIBI && (reinterpret_cast<uintptr_t>(var.slopes) & 3u)) return FA_ERR_ALIGN;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  if (!(std::isfinite(dq) && dq > 0.f && std::isfinite(dk) && dk > 0.f && std::isfinite(dv) && dv > 0.f))
    return FA_ERR_SCALE;
  const int mode = mode_of(dtype);
  const Tile t = lookup_tile(mode, (int)d);
  const int br = t.br();

  Params p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.BH = (int)(B * H);
  p.N = (int)N;
  p.nrb = (int)((N + br - 1) / br);
  p.G = (int)(H / H_kv);
  p.xcd_heads = ((p.BH / p.G) % 8 == 0) ? 1 : 0;   // whole groups of heads per XCD
  const double c2 = std::fabs((double)scale) * (double)dq * (double)dk * 1.4426950408889634;
  if (!std::isfinite((float)c2)) return FA_ERR_SCALE;
  // The kernel masks scores with -inf and relies on c2 > 0 to keep their
  // exponentials at exactly 0.  For |scale| this small every product
  // |score| * c2 is far below one fp32 ulp of 1, so flooring it changes nothing.
  p.c2 = std::max((float)c2, 1e-30f);
  p.out_mul = mode == fa::MODE_FP8 ? dv : 1.f;
  p.qsign = 0;
  if (scale < 0.f) p.qsign = mode == fa::MODE_BF16 ? 0x80008000u : mode == fa::MODE_FP8 ? 0x80808080u : 1u;

  p.H = (int)H;
  p.slopes = var.slopes;
  p.alibi_mul = -1.4426950408889634f / p.c2;     // c2 * alibi_mul = -log2(e)
  p.bmask = var.bmask;
  p.bm_sb = var.sb;
  p.bm_sh = var.sh;
  p.nb = (int)((N + fa::kMaskBlock - 1) / fa::kMaskBlock);

  const int grid = p.nrb * p.BH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (var.kind != fa::VAR_NONE) {
    e = fa_dispatch_variant(var.kind, mode, p, (int)d, causal != 0, grid, s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  switch (mode) {
    case fa::MODE_BF16: e = dispatch_d<fa::MODE_BF16>(p, (int)d, causal != 0, grid, s); break;
    case fa::MODE_FP8: e = dispatch_d<fa::MODE_FP8>(p, (int)d, causal != 0, grid, s); break;
    default: e = dispatch_d<fa::MODE_F32>(p, (int)d, causal != 0, grid, s); break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                 int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  return run(q, k, v, o, lse, B, H, H, N, d, scale, 1.f, 1.f, 1.f, causal, dtype, stream);
}

fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse, int64_t B,
                     int64_t H, int64_t N, int64_t d, float scale, float q_descale, float k_descale,
                     float v_descale, int causal, void* stream) {
  return run(q8, k8, v8, o_bf16, lse, B, H, H, N, d, scale, q_descale, k_descale, v_descale, causal,
             FA_FP8_E4M3, stream);
}

fa_status fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t H_kv, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  return run(q, k, v, o, lse, B, H, H_kv, N, d, scale, 1.f, 1.f, 1.f, causal, dtype, stream);
}

fa_status fa_fwd_gqa_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse, int64_t B,
                         int64_t H, int64_t H_kv, int64_t N, int64_t d, float scale, float q_descale,
                         float k_descale, float v_descale, int causal, void* stream) {
  return run(q8, k8, v8, o_bf16, lse, B, H, H_kv, N, d, scale, q_descale, k_descale, v_descale, causal,
             FA_FP8_E4M3, stream);
}

fa_status fa_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse, const float* slopes,
                       int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  Variant var;
  var.kind = fa::VAR_ALIBI;
  var.slopes = slopes;
  return run(q, k, v, o, lse, B, H, H, N, d, scale, 1.f, 1.f, 1.f, causal, dtype, stream, var);
}

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             const uint8_t* block_mask, int64_t mask_stride_b, int64_t mask_stride_h, int64_t B,
                             int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype, void* stream) {
  Variant var;
  var.kind = fa::VAR_BLOCKSPARSE;
  var.bmask = block_mask;
  var.sb = mask_stride_b;
  var.sh = mask_stride_h;
  return run(q, k, v, o, lse, B, H, H, N, d, scale, 1.f, 1.f, 1.f, causal, dtype, stream, var);
}

fa_status fa_fwd_alibi_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse,
                           const float* slopes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                           float q_descale, float k_descale, float v_descale, int causal, void* stream) {
  Variant var;
  var.kind = fa::VAR_ALIBI;
  var.slopes = slopes;
  return run(q8, k8, v8, o_bf16, lse, B, H, H, N, d, scale, q_descale, k_descale, v_descale, causal, FA_FP8_E4M3,
             stream, var);
}

fa_status fa_fwd_blocksparse_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse,
                                 const uint8_t* block_mask, int64_t mask_stride_b, int64_t mask_stride_h, int64_t B,
                                 int64_t H, int64_t N, int64_t d, float scale, float q_descale, float k_descale,
                                 float v_descale, int causal, void* stream) {
  Variant var;
  var.kind = fa::VAR_BLOCKSPARSE;
  var.bmask = block_mask;
  var.sb = mask_stride_b;
  var.sh = mask_stride_h;
  return run(q8, k8, v8, o_bf16, lse, B, H, H, N, d, scale, q_descale, k_descale, v_descale, causal, FA_FP8_E4M3,
             stream, var);
}

fa_status fa_plan(int64_t B, int64_t H, int64_t N, int64_t d, int causal, int dtype, int* block_rows,
                  int* block_cols, int64_t* workgroups, int* threads, int* lds_bytes, int64_t* kv_tiles) {
  fa_status st = check_shape(B, H, N, d, dtype);
  if (st != FA_OK) return st;
  const Tile t = lookup_tile(mode_of(dtype), (int)d);
  const int64_t br = t.br(), bc = t.bc;
  const int64_t nrb = (N + br - 1) / br, tiles_all = (N + bc - 1) / bc;
  int64_t tiles = 0;
  if (causal) {
    for (int64_t rb = 0; rb < nrb; ++rb) {
      const int64_t need = (rb * br + br - 1) / bc + 1;
      tiles += need < tiles_all ? need : tiles_all;
    }
  } else {
    tiles = nrb * tiles_all;
  }
  if (block_rows) *block_rows = (int)br;
  if (block_cols) *block_cols = (int)bc;
  if (workgroups) *workgroups = nrb * B * H;
  if (threads) *threads = 64 * t.nw;
  if (lds_bytes) *lds_bytes = t.lds;
  if (kv_tiles) *kv_tiles = tiles * B * H;
  return FA_OK;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "FA_ERR_SHAPE: B, H, N (and H_kv) must be >= 1, H a multiple of H_kv, and sizes must fit the index types";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: d must be 64, 128 or 256 and dtype a fa_dtype value";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: every pointer must be 16-byte aligned";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and descales finite and > 0";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected the launch";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the call needs more partials than fa_fwd_split_noalloc's fixed scratch holds";
    default: return "unknown fa_status";
  }
}

int fa_version(void) { return 100; }

fa_status fa_timeline_read(void* dst, int64_t bytes) {
#ifdef FA_TIMELINE
  if (!dst) return FA_ERR_NULL;
  if (bytes < 0 || bytes > (int64_t)sizeof(unsigned long long) * fa::kTimelineWords) return FA_ERR_SHAPE;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(fa::fa_timeline_buf), (size_t)bytes, 0, hipMemcpyDeviceToHost) == hipSuccess
             ? FA_OK
             : FA_ERR_HIP;
#else
  (void)dst;
  (void)bytes;
  return FA_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
