// Shared pieces of the gfx950 attention kernels: parameter block, vector
// types, LDS tile geometry and swizzles, MFMA/LDS wrappers, grid mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
  int G;           // query heads per K/V head (grouped-query attention; 1 = one K/V head per head)
  int xcd_heads;   // 1: K/V heads are spread over XCDs, with their query heads ((BH / G) % 8 == 0)
  int cus_per_xcd; // compute units per XCD (0: unknown)
  int zigzag;      // causal grid fully resident: deal row blocks to CUs zig-zag (see map_block)
  float c2;        // |scale| * descale_q * descale_k * log2(e)
  float out_mul;   // factor applied to O before dividing by l (fp8: descale_v)
  uint32_t qsign;  // XOR mask on Q's sign bits (negative scale)
  // variants (VAR_ALIBI, VAR_BLOCKSPARSE); unused otherwise
  int H;                   // query heads per batch (head index = bh % H)
  const float* slopes;     // ALiBi: [H] slopes
  float alibi_mul;         // ALiBi: -1 / |scale| (the bias is added to the unscaled score)
  const uint8_t* bmask;    // block-sparse: mask bytes, nonzero = block computed
  int64_t bm_sb, bm_sh;    // block-sparse: strides of batch and head, in bytes (0 broadcasts)
  int nb;                  // block-sparse: blocks per side, ceil(N / kMaskBlock)
};

// ---------------------------------------------------------------- timeline
// Diagnostic builds (-DFA_TIMELINE, python -m exact_io_aware_48_amd.build
// --timeline) stamp each forward workgroup's phases with the 100 MHz
// s_memrealtime clock: entry, Q and first tiles in, main loop done, O
// stored (after a workgroup barrier).  Thread 0 writes six words per
// workgroup (the four stamps, XCC_ID << 32 | HW_ID, row block << 32 | head)
// with plain vector stores; fa_timeline_read copies them out.  Product builds
// compile all of it away.
#ifdef FA_TIMELINE
constexpr bool kTimeline = true;
constexpr int kTimelineWords = 1 << 18;
static __device__ unsigned long long fa_timeline_buf[kTimelineWords];
#else
constexpr bool kTimeline = false;
#endif
__device__ __forceinline__ unsigned long long timeline_clock() {
  if constexpr (kTimeline) return __builtin_amdgcn_s_memrealtime();
  return 0;
}
__device__ __forceinline__ void timeline_record(unsigned long long t0, unsigned long long t1, unsigned long long t2,
                                                int bh, int rb) {
#ifdef FA_TIMELINE
  __syncthreads();
  const unsigned long long t3 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0 && (blockIdx.x + 1) * 6 <= (unsigned)kTimelineWords) {
    unsigned long long* w = fa_timeline_buf + blockIdx.x * 6;
    const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID
    const unsigned xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
    w[0] = t0; w[1] = t1; w[2] = t2; w[3] = t3;
    w[4] = ((unsigned long long)xcc << 32) | hw;
    w[5] = ((unsigned long long)(unsigned)rb << 32) | (unsigned)bh;
  }
#else
  (void)t0; (void)t1; (void)t2; (void)bh; (void)rb;
#endif
}

enum { VAR_NONE = 0, VAR_ALIBI = 1, VAR_BLOCKSPARSE = 2 };
constexpr int kMaskBlock = 128;   // block-sparse mask granularity (queries x keys)

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
template <int D, int BC, int NW, int MODE, bool PP = false>
struct Geo {
  static constexpr int EB = MODE == MODE_FP8 ? 1 : 2;      // bytes per element in LDS
  static constexpr int PLANES = MODE == MODE_F32 ? 2 : 1;  // hi/lo planes for the fp32 split
  static constexpr int ROWB = D * EB;                      // bytes per LDS tile row
  static constexpr int CPR = ROWB / 16;                    // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;                  // one plane of one tensor
  static constexpr int SLOTB = PLANES * TILEB;             // one ring slot (all planes of one tile)
  static constexpr int KST = 2;                            // K ring: tile j in use, tile j+1 in flight
  static constexpr int VST = PP ? 3 : 2;                   // V ring: the ping-pong group also keeps tile j-1
  static constexpr int LDSB = (KST + VST) * SLOTB;
  static constexpr int NT = NW * 64;                       // threads
  static constexpr int UNITS = TILEB / 16;                 // 16-byte LDS chunks per plane
  // a tile smaller than one chunk per thread is staged by its first LOADERS waves
  static constexpr int UPT = UNITS >= NT ? UNITS / NT : 1; // chunks per loading thread per tensor
  static constexpr int LOADERS = UNITS >= NT ? NW : UNITS / 64;
  static constexpr int BR = 32 * NW;                       // query rows per workgroup
  // rows that share one 256-byte span of LDS banks
  static constexpr int RPP = CPR >= 16 ? 1 : 16 / CPR;
  static_assert(UNITS >= NT ? UNITS % NT == 0 : UNITS % 64 == 0, "tile must split evenly over the loading waves");
  static_assert(BC % 32 == 0, "B_c is a multiple of 32");
  static_assert(MODE != MODE_FP8 || BC % 64 == 0, "fp8 P.V consumes 64 keys per MFMA");
  static_assert(LDSB <= 160 * 1024, "LDS budget");
  static_assert(!PP || (MODE != MODE_F32 && NW % 2 == 0), "ping-pong needs DMA staging and an even wave count");
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
  // v_maximum_f32: no NaN canonicalisation of the inputs (fmaxf costs two)
  return __builtin_elementwise_maximum(__int_as_float(r[0]), __int_as_float(r[1]));
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
// The same load addressed as a wave-uniform 64-bit base (SGPRs) plus a
// per-lane 32-bit byte offset.  NT: with the non-temporal (streaming) cache
// hint, for data each workgroup reads once and no other one reads again
// (split-KV decoding's K/V stream: 11-15% faster on MI355X).  Kernels whose
// workgroups share K/V through the L2 keep it off (it cost them 4-16%).
template <bool NT = false>
__device__ __forceinline__ void dma16_s(const char* sbase, int voff, const char FA_LDS* lds) {
  const uint32_t m0v = (uint32_t)(uintptr_t)lds;
  if constexpr (NT)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(m0v) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0v) : "memory");
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

// A block of NI independent-operand MFMA items whose A operands come from
// LDS: read(i) returns item i's operand (R LDS reads), mma(i, a) issues its
// MFMA.  The reads run DEPTH items ahead of the MFMAs, in a fixed order given
// to the scheduler with sched_group_barrier (LLVM AMDGPU masks: 0x008 MFMA,
// 0x100 LDS read): the first DEPTH items' reads, then one MFMA and the reads
// of the item DEPTH ahead, then the last DEPTH MFMAs.  Without it the
// compiler keeps as few operand buffers as registers force, and each MFMA
// waits for the LDS read issued just before it.
template <int NI, int DEPTH, int R, class Op, class Read, class Mma>
__device__ __forceinline__ void mfma_pipeline(Read&& read, Mma&& mma) {
  constexpr int AHEAD = NI < DEPTH ? NI : DEPTH;
  Op a[AHEAD];
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) a[i] = read(i);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    mma(i, a[i % AHEAD]);
    if (i + AHEAD < NI) a[i % AHEAD] = read(i + AHEAD);
  }
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kDsRead, R * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < NI - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, AHEAD, 0);
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

// Map a workgroup id to (head, row block).
// The hardware deals workgroup ids to the 8 XCDs round-robin (XCD = id % 8)
// and, within an XCD, slots s = id / 8 to its CUs round-robin (CU s % C for
// C CUs per XCD), so slots s, s + C, s + 2C ... share a CU.
//   * xcd_heads: all row blocks of all query heads that share a K/V head
//     stay on one XCD (that K/V stream stays in the XCD's L2): K/V head
//     xcd + 8*j, and the XCD-local query head hl is query head G*(xcd + 8*(hl/G)) + hl%G.
//   * causal: row blocks differ in work (row block i has i+1 key tiles of
//     B_r), so the XCD's work list is ordered heaviest first.  When the whole
//     grid is resident at once (zigzag), consecutive passes of C slots take
//     that list forward, backward, forward ... so every CU's workgroups add up
//     to about the same number of tiles; otherwise heaviest-first order lets
//     CUs that free up early take the next-heaviest block.
__device__ __forceinline__ int zigzag_slot(int s, int total, int C) {
  const int r = s / C, pos = s - r * C, base = r * C;
  const int R = min(C, total - base);          // slots in this pass
  return base + ((r & 1) ? R - 1 - pos : pos);
}
// P: any parameter block with the fields BH, nrb, G, xcd_heads, zigzag and cus_per_xcd.
template <class P>
__device__ __forceinline__ int xcd_head(const P& p, int xcd, int hl) {
  return p.G * (xcd + 8 * (hl / p.G)) + hl % p.G;
}
template <bool CAUSAL, class P>
__device__ __forceinline__ void map_block(const P& p, int id, int& bh, int& rb) {
  const int nrb = p.nrb;
  if constexpr (!CAUSAL) {
    if (p.xcd_heads) {
      const int xcd = id & 7, s = id >> 3;
      bh = xcd_head(p, xcd, s / nrb);
      rb = s % nrb;
    } else {
      bh = id % p.BH;
      rb = id / p.BH;
    }
  } else {
    if (p.xcd_heads) {
      const int xcd = id & 7, s = id >> 3, hpx = p.BH >> 3;
      const int k = p.zigzag ? zigzag_slot(s, hpx * nrb, p.cus_per_xcd) : s;
      bh = xcd_head(p, xcd, k % hpx);
      rb = nrb - 1 - k / hpx;
    } else {
      const int k = p.zigzag ? zigzag_slot(id, p.BH * nrb, 8 * p.cus_per_xcd) : id;
      bh = k % p.BH;
      rb = nrb - 1 - k / p.BH;
    }
  }
}

}  // namespace fa
