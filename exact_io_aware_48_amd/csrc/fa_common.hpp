// Shared pieces of the gfx950 attention kernels: parameter block, vector
// types, LDS tile geometry and swizzles, MFMA/LDS wrappers, grid mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum { MODE_BF16 = 0, MODE_FP8 = 1, MODE_F32 = 2 };

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;          // batch * heads
  int N;           // sequence length (queries = keys)
  int nrb;         // row blocks per head = ceil(N / B_r)
  int xcd_heads;   // 1: heads are spread over XCDs head-major (BH % 8 == 0)
  float c2;        // |scale| * descale_q * descale_k * log2(e)
  float out_mul;   // factor applied to O before dividing by l (fp8: descale_v / 256)
  uint32_t qsign;  // XOR mask on Q's sign bits (negative scale)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- tile geometry
template <int D, int BC, int NW, int MODE, int STAGES = 2>
struct Geo {
  static constexpr int EB = MODE == MODE_FP8 ? 1 : 2;      // bytes per element in LDS
  static constexpr int PLANES = MODE == MODE_F32 ? 2 : 1;  // hi/lo planes for the fp32 split
  static constexpr int ROWB = D * EB;                      // bytes per LDS tile row
  static constexpr int CPR = ROWB / 16;                    // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;                  // one plane of one tensor
  static constexpr int STAGEB = 2 * PLANES * TILEB;        // K and V planes of one stage
  static constexpr int LDSB = STAGES * STAGEB;             // ring of STAGES tiles
  static constexpr int NT = NW * 64;                       // threads
  static constexpr int UNITS = TILEB / 16;                 // 16-byte LDS chunks per plane
  static constexpr int UPT = UNITS / NT;                   // chunks per thread per tensor
  static constexpr int BR = 32 * NW;                       // query rows per workgroup
  // rows that share one 256-byte span of LDS banks
  static constexpr int RPP = CPR >= 16 ? 1 : 16 / CPR;
  static_assert(UNITS % NT == 0, "tile must split evenly over the threads");
  static_assert(BC % 32 == 0, "B_c is a multiple of 32");
  static_assert(MODE != MODE_FP8 || BC % 64 == 0, "fp8 P.V consumes 64 keys per MFMA");
  static_assert(LDSB <= 160 * 1024, "LDS budget");
  static_assert(STAGES == 2 || (STAGES == 3 && MODE != MODE_F32), "fp32 staging is double buffered");
};

// XOR swizzles of the 16-byte chunk index.  K tiles are read 32 rows at a
// time at one logical chunk (MFMA A operand); V tiles are read with the
// transpose loads, a few rows by a few adjacent chunks at a time.
// CPR = 16-byte chunks per tile row; rows sharing one 256-byte bank span: RPP.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) {
  constexpr int RPP = CPR >= 16 ? 1 : 16 / CPR;
  constexpr int span = CPR < 16 ? CPR : 16;
  return (row / RPP) % span;
}
template <int CPR, int MODE>
__device__ __forceinline__ int swz_v(int row) {
  constexpr int RPP = CPR >= 16 ? 1 : 16 / CPR;
  if constexpr (MODE == MODE_FP8) {
    // transposed byte reads touch rows {r%4, (r/8)%2} x 2 chunks
    if constexpr (CPR >= 16) return 2 * ((row & 3) + 4 * ((row >> 3) & 1));
    else if constexpr (CPR == 8) return 2 * (((row & 3) >> 1) + 2 * ((row >> 3) & 1));
    else return 2 * ((row >> 3) & 1);
  } else {
    // transposed 16-bit reads touch 4 consecutive rows x 4 chunks
    constexpr int groups = CPR >= 16 ? 4 : CPR / 4;
    return 4 * ((row / RPP) % groups);
  }
}

// ---------------------------------------------------------------- small helpers
__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ i32x4 lds_read16(const char FA_LDS* p) {
  return *reinterpret_cast<const i32x4 FA_LDS*>(p);
}
__device__ __forceinline__ void lds_write16(char FA_LDS* p, i32x4 v) {
  *reinterpret_cast<i32x4 FA_LDS*>(p) = v;
}
// One 16-byte-per-lane HBM -> LDS load (global_load_lds_dwordx4): lane l's
// 16 bytes land at LDS byte lds + 16*l.  Issued from asm so that the
// compiler's wait insertion does not treat it as aliasing every later LDS read
// (it cannot tell the stages apart); completion is awaited explicitly with
// s_waitcnt vmcnt(0) before the workgroup barrier that publishes the tile.
__device__ __forceinline__ void dma16(const void* gsrc, const char FA_LDS* lds) {
  const uint32_t m0v = (uint32_t)(uintptr_t)lds;
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0v) : "memory");
}
// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order, so the older ones are then done).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ i16x4 lds_tr16(const char FA_LDS* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<i16x4 FA_LDS*>(const_cast<char FA_LDS*>(p)));
}
__device__ __forceinline__ i32x2 lds_tr8(const char FA_LDS* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<i32x2 FA_LDS*>(const_cast<char FA_LDS*>(p)));
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format codes 0/0 = e4m3 for both operands; E8M0 scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// round-to-nearest-even float -> bf16 bits (the hardware conversion)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));   // v_cvt_pk_bf16_f32
}
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// split 8 fp32 values into bf16 hi and lo parts (x ~= hi + lo)
__device__ __forceinline__ void split8(const float* x, i32x4& hi, i32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    float r0 = x[2 * i] - bf16_lo_to_f32(h);
    float r1 = x[2 * i + 1] - bf16_hi_to_f32(h);
    hi[i] = (int)h;
    lo[i] = (int)pack_bf16x2(r0, r1);
  }
}

// map a workgroup id to (head, row block); heaviest causal row blocks first
template <bool CAUSAL>
__device__ __forceinline__ void map_block(const Params& p, int id, int& bh, int& rb) {
  if (p.xcd_heads) {
    const int xcd = id & 7, slot = id >> 3;
    bh = xcd + 8 * (slot / p.nrb);
    rb = slot % p.nrb;
  } else {
    bh = id % p.BH;
    rb = id / p.BH;
  }
  if (CAUSAL) rb = p.nrb - 1 - rb;
}

}  // namespace fa
