// Per-wave building blocks shared by the attention kernels: the wave's Q
// fragment, S^T = K_j Q^T over one LDS tile, masking, the online-softmax
// exponentials with P packed as an MFMA operand, O^T += V_j^T P^T, the output
// epilogue, and the HBM -> LDS staging of a K or V tile.
//
// Register layouts (v_mfma_f32_32x32x16_bf16 on a wave64; lane = 32*hf + n):
//   S^T accumulator (32 keys x 32 queries): lane holds query n, element i is
//     key 8*(i/4) + 4*hf + i%4 of the 32-key block.
//   O^T accumulator (32 dims x 32 queries): lane holds query n, element i is
//     dim 8*(i/4) + 4*hf + i%4 of the 32-dim block.
// Because the sum over the MFMA's k dimension does not care about the order
// of k, P^T is fed from the S^T registers as they are, and the V^T operand is
// read in the same key order with the LDS transpose loads.
#pragma once

#include <type_traits>

#include "fa_common.hpp"

namespace fa {

template <int D, int BC, int NW, int MODE>
struct Tile {
  using G = Geo<D, BC, NW, MODE>;
  static constexpr int KB = BC / 32;                                // 32-key blocks per tile
  static constexpr int NDB = D / 32;                                // 32-wide blocks of the head dim
  static constexpr int QK_STEPS = MODE == MODE_FP8 ? D / 64 : D / 16;   // MFMA k-steps over d
  static constexpr int PV_STEPS = MODE == MODE_FP8 ? BC / 64 : BC / 16; // MFMA k-steps over keys
  // Lazy-rescale threshold (log2 units): the exponent base may lag a row's
  // running max by up to TAU, so P <= 2^TAU.  fp8 stores P as e4m3 of
  // 2^EXP_SHIFT * P <= 2^8 (e4m3 holds up to 448); the pre-scale keeps small
  // probabilities out of e4m3's subnormal range (normal down to P = 2^-12).
  // A lag of 2 instead of 0 removes most of the O rescales (128 multiplies
  // each at d = 256), which fp8's short MFMA time does not hide.  The factor
  // is taken into the exponent base, so the exponentials produce the scaled P
  // directly and l sums it as well; O is unchanged (the factor cancels in
  // O / l) and L subtracts it back.
  static constexpr float TAU = MODE == MODE_FP8 ? 2.f : 8.f;
  static constexpr float EXP_SHIFT = MODE == MODE_FP8 ? 8.f - TAU : 0.f;

  // the wave's 32 queries as the B operand of S^T = K Q^T
  struct QFrag {
    bf16x8 a[MODE == MODE_FP8 ? 1 : QK_STEPS];   // bf16 values (fp32 mode: hi parts)
    bf16x8 l[MODE == MODE_F32 ? QK_STEPS : 1];   // fp32 mode: lo parts
    i32x8 f8[MODE == MODE_FP8 ? QK_STEPS : 1];   // fp8 bytes
  };
  // P of one tile as the B operand of O^T += V^T P^T
  //   bf16/fp32: element i of step s <- key 16*s + 8*(i/4) + 4*hf + i%4 (hi parts; lo in l)
  //   fp8:       byte 16*kb' + i of step g <- key 64*g + 32*kb' + 8*(i/4) + 4*hf + i%4, x 2^EXP_SHIFT
  struct PFrag {
    i32x4 h[MODE == MODE_FP8 ? 1 : PV_STEPS];    // bf16 pairs
    i32x4 l[MODE == MODE_F32 ? PV_STEPS : 1];
    i32x8 f8[MODE == MODE_FP8 ? PV_STEPS : 1];
  };
  // bf16: the operand reads of both products run PDEPTH MFMAs ahead
  // (qk_pipe, pv_pipe).  Left to itself the compiler keeps one or two
  // operand buffers when registers are short (d = 256: one, so every MFMA
  // waited for the LDS read issued just before it).  The read addresses are
  // kept as a few per-lane bases plus instruction immediates, which frees the
  // registers the deeper pipeline needs.  Depths 2 and 4 measured the same as 3.
  // fp8 (operands of 8 registers, two or four reads each) pipelines two
  // deep with the plain addressing, which fits its register budget.
  static constexpr bool PIPE = MODE != MODE_F32;
  static constexpr bool PIPE_ADDR = MODE == MODE_BF16;
  static constexpr int PDEPTH = MODE == MODE_FP8 ? 2 : 3;
  struct Lane {
    int n, hf;                  // query column, lane half
    int v_row, v_col;           // per-lane parts of the V^T transpose-read address
    int ka[PIPE_ADDR ? 8 : 1];  // bf16: K-read offsets of d-steps c < 8 (step c + 8: +256 bytes)
    int va[PIPE_ADDR ? 4 : 1];  // bf16: V^T-read offsets of d-blocks db < 4 (db + 4: +256 bytes)
    int kf[MODE == MODE_FP8 ? 2 * QK_STEPS : 1];  // fp8: K-read offsets of d-step c, halves 0 and 1
    int vf[MODE == MODE_FP8 ? NDB : 1];           // fp8: V^T-read offsets of d-block db
  };

  static __device__ __forceinline__ Lane lane_info(int lane) {
    Lane ln;
    ln.n = lane & 31;
    ln.hf = lane >> 5;
    const int grp = lane >> 4;  // 16-lane group
    if constexpr (MODE == MODE_FP8) {
      const int isrc = (lane & 15) >> 1;  // which of the 8 returned bytes this lane sources
      ln.v_row = 8 * (isrc >> 2) + 4 * ln.hf + (isrc & 3);
      ln.v_col = 16 * (grp & 1) + 8 * (lane & 1);
    } else {
      ln.v_row = 4 * ln.hf + ((lane >> 2) & 3);
      ln.v_col = 2 * (16 * (grp & 1) + 4 * (lane & 3));
    }
    if constexpr (MODE == MODE_FP8) {
      // Whole per-lane offsets, formed once: K row n (+ 32 kb), chunk
      // (4c + 2hf + j) ^ swz_k(n) in kf[2c + j]; V^T rows v_row (+ 16 t + 64 s), byte
      // column 32 db + v_col.  Both swizzles repeat every 16 rows, so the
      // row steps are instruction immediates.  The empty asm hides how an
      // offset was formed: otherwise the compiler keeps the row and column
      // parts apart and adds them again before every read (12 VALU
      // instructions per tile at d = 256).
#pragma unroll
      for (int i = 0; i < 2 * QK_STEPS; ++i) {
        ln.kf[i] = ln.n * G::ROWB + (((4 * (i >> 1) + 2 * ln.hf + (i & 1)) ^ swz_k<G::CPR>(ln.n)) << 4);
        asm volatile("" : "+v"(ln.kf[i]));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + ln.v_col;
        ln.vf[db] = ln.v_row * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(ln.v_row)) << 4) | (col & 15));
        asm volatile("" : "+v"(ln.vf[db]));
      }
    }
    if constexpr (PIPE_ADDR) {
      // K row n (+ 32 kb), chunk (2c + hf) ^ (n % 16): the swizzle leaves bit 4
      // of the chunk index alone, so steps c and c + 8 are 256 bytes apart.
      // V^T rows v_row (+ 8, + 16 s) share the swizzle 4 * (v_row % 4), which
      // leaves bit 4 alone too, so d-blocks db and db + 4 are 256 bytes apart.
      // (Rows 32 kb + n and v_row + 16 s + 8 keep the same swizzle for every
      // tile width used: 8, 16 or 32 chunks per row.)
      static_assert(G::CPR == 8 || G::CPR == 16 || G::CPR == 32, "PIPE addressing: 128- to 512-byte tile rows");
#pragma unroll
      for (int c = 0; c < 8; ++c)
        ln.ka[c] = ln.n * G::ROWB + (((2 * c + ln.hf) ^ swz_k<G::CPR>(ln.n)) << 4);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int col = 64 * db + ln.v_col;
        ln.va[db] = ln.v_row * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(ln.v_row)) << 4) | (col & 15));
      }
    }
    return ln;
  }

  // Q slice of query my_q (zeros past the end) -> registers; qsign flips the
  // sign bits when the softmax scale is negative.
  static __device__ __forceinline__ void load_q(const Params& p, int64_t head_off, int my_q, const Lane& ln, QFrag& q) {
    const bool valid = my_q < p.N;
    const int sgn = (int)p.qsign;
    if constexpr (MODE == MODE_BF16) {
      const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.q) + head_off + (int64_t)my_q * D);
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        i32x4 w = valid ? src[2 * c + ln.hf] : i32x4{0, 0, 0, 0};
        w ^= i32x4{sgn, sgn, sgn, sgn};
        q.a[c] = __builtin_bit_cast(bf16x8, w);
      }
    } else if constexpr (MODE == MODE_FP8) {
      const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint8_t*>(p.q) + head_off + (int64_t)my_q * D);
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        i32x4 w0 = valid ? src[4 * c + 2 * ln.hf] : i32x4{0, 0, 0, 0};
        i32x4 w1 = valid ? src[4 * c + 2 * ln.hf + 1] : i32x4{0, 0, 0, 0};
        w0 ^= i32x4{sgn, sgn, sgn, sgn};
        w1 ^= i32x4{sgn, sgn, sgn, sgn};
        q.f8[c] = i32x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      }
    } else {
      const float* src = static_cast<const float*>(p.q) + head_off + (int64_t)my_q * D;
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        float x[8];
        if (valid) {
          f32x4 a = *reinterpret_cast<const f32x4*>(src + 16 * c + 8 * ln.hf);
          f32x4 b = *reinterpret_cast<const f32x4*>(src + 16 * c + 8 * ln.hf + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
        if (p.qsign) {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = -x[i];
        }
        i32x4 hi, lo;
        split8(x, hi, lo);
        q.a[c] = __builtin_bit_cast(bf16x8, hi);
        q.l[c] = __builtin_bit_cast(bf16x8, lo);
      }
    }
  }

  // ---- Q and O through LDS (bf16 and fp8 inputs, bf16 output).  A wave's
  // direct loads of its Q slice touch 32 rows of 16 or 32 bytes per
  // instruction, and so do the stores of O^T from the accumulator layout.
  // Staged through LDS, every HBM access is a run of whole rows (1 KiB per
  // wave instruction); the LDS tile uses the K swizzle (16-byte chunk c of
  // row r at chunk c ^ swz_k(r)).
  static constexpr int QROWB = D * (MODE == MODE_FP8 ? 1 : 2);   // bytes per Q row
  static constexpr int QCPR = QROWB / 16;

  // the workgroup's BR = 32 NW rows starting at gsrc (rows_valid of them
  // exist; later ones re-read the last, whose scores stay in their own
  // rows, which are never stored) -> LDS, one DMA per 1 KiB block: blocks
  // below SPLIT to dst_a + 1024 b, the others to dst_b + 1024 (b - SPLIT)
  // (two free ring slots can hold the tile)
  template <int SPLIT>
  static __device__ __forceinline__ void dma_q(const char* gsrc, int rows_valid, char FA_LDS* dst_a, char FA_LDS* dst_b,
                                               int wave, int lane) {
    static_assert(MODE != MODE_F32, "16-bit or 8-bit rows");
    constexpr int PER = 32 * NW * QCPR / (NW * 64);   // chunks per thread
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = i * NW + wave;
      const int u = blk * 64 + lane;
      const int r = u / QCPR, pc = u % QCPR;
      const int off = min(r, rows_valid - 1) * QROWB + ((pc ^ swz_k<QCPR>(r)) << 4);
      dma16_s(gsrc, off, blk < SPLIT ? dst_a + blk * 1024 : dst_b + (blk - SPLIT) * 1024);
    }
  }
  // this wave's Q slice from its 32 staged rows at wave_rows (the row
  // swizzle repeats every 16 rows) -- qsign flips the sign bits when the
  // softmax scale is negative
  static __device__ __forceinline__ void load_q_lds(const char FA_LDS* wave_rows, const Lane& ln, uint32_t qsign,
                                                    QFrag& q) {
    static_assert(MODE != MODE_F32 && QROWB == G::ROWB, "K-tile addressing");
    const int sgn = (int)qsign;
    if constexpr (MODE == MODE_BF16) {
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        i32x4 w = lds_read16(wave_rows + ln.ka[c & 7] + ((c >> 3) << 8));
        w ^= i32x4{sgn, sgn, sgn, sgn};
        q.a[c] = __builtin_bit_cast(bf16x8, w);
      }
    } else {
      // step c: chunks 4c + 2 hf and 4c + 2 hf + 1 of row n (as k_operand)
      const char FA_LDS* rp = wave_rows + ln.n * QROWB;
      const int sw = swz_k<QCPR>(ln.n);
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        i32x4 w0 = lds_read16(rp + (((4 * c + 2 * ln.hf) ^ sw) << 4));
        i32x4 w1 = lds_read16(rp + (((4 * c + 2 * ln.hf + 1) ^ sw) << 4));
        w0 ^= i32x4{sgn, sgn, sgn, sgn};
        w1 ^= i32x4{sgn, sgn, sgn, sgn};
        q.f8[c] = i32x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      }
    }
  }
  // O = out_mul * O / l for the wave's 32 queries through the wave's own
  // LDS region (no other wave touches it), then whole row segments to HBM;
  // L = ln2 * (m + log2 l) as in store().  GDB d-blocks (64 bytes of each
  // row) per pass: the region holds 32 rows of 64 GDB bytes.
  template <int GDB>
  static __device__ __forceinline__ void store_lds(const Params& p, int64_t head_off, int bh, int qw0, int my_q,
                                                   const Lane& ln, const f32x16 (&oacc)[NDB], float m_run, float l_run,
                                                   char FA_LDS* region, int lane) {
    static_assert(MODE != MODE_F32 && NDB % GDB == 0, "bf16 output in whole passes");
    constexpr int RB = 64 * GDB, CPRR = RB / 16;    // region row bytes, 16-byte chunks per region row
    constexpr int RPI = 1024 / RB;                  // rows per wave instruction
    const float l_tot = swap_halves_sum(l_run);
    const bool seen = l_tot > 0.f;
    const float inv = seen ? p.out_mul / l_tot : 0.f;
    if (my_q < p.N && ln.hf == 0)
      p.lse[(int64_t)bh * p.N + my_q] = seen ? (m_run - EXP_SHIFT + __log2f(l_tot)) * kLn2 : -INFINITY;
    char FA_LDS* const rowp = region + ln.n * RB;
    const int sw = swz_k<CPRR>(ln.n);
    const int rr = lane / CPRR, lc = lane % CPRR;
#pragma unroll
    for (int pass = 0; pass < NDB / GDB; ++pass) {
      // lane (n, hf): dims 32 db + 8 g + 4 hf .. + 3 of row n = 8 bytes of chunk 4 (db - GDB pass) + g
#pragma unroll
      for (int b = 0; b < GDB; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int db = GDB * pass + b;
          const float x0 = oacc[db][4 * g] * inv, x1 = oacc[db][4 * g + 1] * inv;
          const float x2 = oacc[db][4 * g + 2] * inv, x3 = oacc[db][4 * g + 3] * inv;
          *reinterpret_cast<i32x2 FA_LDS*>(rowp + (((4 * b + g) ^ sw) << 4) + 8 * ln.hf) =
              i32x2{(int)pack_bf16x2(x0, x1), (int)pack_bf16x2(x2, x3)};
        }
      // the reads below fetch other lanes' writes: wait for them (the next
      // pass's writes come after this pass's reads have returned: their data
      // feeds the stores)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + rr;
        const i32x4 v = lds_read16(region + r * RB + ((lc ^ swz_k<CPRR>(r)) << 4));
        // non-temporal: O is not read again here, and streaming it out leaves
        // less to write back when the kernel ends (GPT-2-small 21.5 -> 20.1 us,
        // BERT-large 23.3 -> 22.3 us; the long workloads unchanged)
        if (qw0 + r < p.N)
          __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(static_cast<uint16_t*>(p.o) + head_off +
                                                                 (int64_t)(qw0 + r) * D + 32 * GDB * pass + 8 * lc));
      }
      asm volatile("" ::: "memory");
    }
  }

  // ---- single MFMA items.  A QK item (c, kb) adds d-step c of key block kb
  // to S^T; a PV item (s, db) adds key-step s to d-block db of O^T.  Each
  // item's A operand is one LDS read (fp8: two, or four transposed reads).
  using Op = typename std::conditional<MODE == MODE_FP8, i32x8, bf16x8>::type;

  static __device__ __forceinline__ Op k_operand(const char FA_LDS* kbase, int c, int kb, const Lane& ln) {
    if constexpr (MODE == MODE_FP8) {
      const char FA_LDS* rp = kbase + 32 * kb * G::ROWB;
      i32x4 a0 = lds_read16(rp + ln.kf[2 * c]);
      i32x4 a1 = lds_read16(rp + ln.kf[2 * c + 1]);
      return i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    } else {
      const int row = 32 * kb + ln.n;
      return __builtin_bit_cast(bf16x8, lds_read16(kbase + row * G::ROWB + (((2 * c + ln.hf) ^ swz_k<G::CPR>(row)) << 4)));
    }
  }
  static __device__ __forceinline__ void qk_mma(f32x16 (&st)[KB], int c, int kb, const Op& a, const QFrag& q) {
    if constexpr (MODE == MODE_FP8) st[kb] = mfma_fp8(a, q.f8[c], st[kb]);
    else st[kb] = mfma_bf16(a, q.a[c], st[kb]);
  }
  static __device__ __forceinline__ Op v_operand(const char FA_LDS* vbase, int s, int db, const Lane& ln) {
    if constexpr (MODE == MODE_FP8) {               // 64 keys per step
      int va[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        i32x2 r = lds_tr8(vbase + (64 * s + 16 * t) * G::ROWB + ln.vf[db]);
        va[2 * t] = r[0];
        va[2 * t + 1] = r[1];
      }
      return i32x8{va[0], va[1], va[2], va[3], va[4], va[5], va[6], va[7]};
    } else {                                        // 16 keys per step
      const int row = 16 * s + ln.v_row;
      const int col = 32 * db * 2 + ln.v_col;        // bytes
      const int off0 = row * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(row)) << 4) | (col & 15));
      const int off1 = (row + 8) * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(row + 8)) << 4) | (col & 15));
      i16x4 lo = lds_tr16(vbase + off0), hi = lds_tr16(vbase + off1);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  static __device__ __forceinline__ void pv_mma(f32x16 (&oacc)[NDB], int s, int db, const Op& a, const PFrag& pf) {
    if constexpr (MODE == MODE_FP8) oacc[db] = mfma_fp8(a, pf.f8[s], oacc[db]);
    else oacc[db] = mfma_bf16(a, __builtin_bit_cast(bf16x8, pf.h[s]), oacc[db]);
  }

  // PIPE: the K operand of item i = (d-step c = i / KB, key block kb = i % KB)
  static __device__ __forceinline__ Op k_operand_pipe(const char FA_LDS* kbase, int i, const Lane& ln) {
    const int c = i / KB, kb = i % KB;
    if constexpr (PIPE_ADDR)
      return __builtin_bit_cast(bf16x8, lds_read16(kbase + ln.ka[c & 7] + ((c >> 3) << 8) + kb * 32 * G::ROWB));
    else
      return k_operand(kbase, c, kb, ln);
  }
  // PIPE: the V^T operand of item i = (key step s = i / NDB, d-block db = i % NDB)
  static __device__ __forceinline__ Op v_operand_pipe(const char FA_LDS* vbase, int i, const Lane& ln) {
    const int s = i / NDB, db = i % NDB;
    if constexpr (PIPE_ADDR) {
      const char FA_LDS* p = vbase + ln.va[db & 3] + ((db >> 2) << 8) + 16 * s * G::ROWB;
      i16x4 lo = lds_tr16(p), hi = lds_tr16(p + 8 * G::ROWB);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return v_operand(vbase, s, db, ln);
    }
  }
  // LDS reads per operand
  static constexpr int K_READS = MODE == MODE_FP8 ? 2 : 1, V_READS = MODE == MODE_FP8 ? 4 : 2;
  static __device__ __forceinline__ void qk_pipe(f32x16 (&st)[KB], const char FA_LDS* kbase, const QFrag& q, const Lane& ln) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) st[kb] = f32x16{};
    mfma_pipeline<QK_STEPS * KB, PDEPTH, K_READS, Op>(
        [&](int i) __attribute__((always_inline)) { return k_operand_pipe(kbase, i, ln); },
        [&](int i, const Op& a) __attribute__((always_inline)) { qk_mma(st, i / KB, i % KB, a, q); });
  }
  static __device__ __forceinline__ void pv_pipe(f32x16 (&oacc)[NDB], const char FA_LDS* vbase, const PFrag& pf, const Lane& ln) {
    mfma_pipeline<PV_STEPS * NDB, PDEPTH, V_READS, Op>(
        [&](int i) __attribute__((always_inline)) { return v_operand_pipe(vbase, i, ln); },
        [&](int i, const Op& a) __attribute__((always_inline)) { pv_mma(oacc, i / NDB, i % NDB, a, pf); });
  }

  // st = K Q^T for the tile at kbase (rows: keys, columns: this wave's queries)
  static __device__ __forceinline__ void qk(f32x16 (&st)[KB], const char FA_LDS* kbase, const QFrag& q, const Lane& ln) {
    if constexpr (PIPE) {
      qk_pipe(st, kbase, q, ln);
      return;
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) st[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < QK_STEPS; ++c) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (MODE == MODE_F32) {
          const int row = 32 * kb + ln.n;
          const int off = row * G::ROWB + (((2 * c + ln.hf) ^ swz_k<G::CPR>(row)) << 4);
          bf16x8 a = __builtin_bit_cast(bf16x8, lds_read16(kbase + off));
          bf16x8 al = __builtin_bit_cast(bf16x8, lds_read16(kbase + G::TILEB + off));
          st[kb] = mfma_bf16(a, q.a[c], st[kb]);
          st[kb] = mfma_bf16(a, q.l[c], st[kb]);
          st[kb] = mfma_bf16(al, q.a[c], st[kb]);
        } else {
          qk_mma(st, c, kb, k_operand(kbase, c, kb, ln), q);
        }
      }
    }
  }

  // scores of keys past lim (relative to the tile start and to 4*hf) -> -inf.
  // Callers branch around it: only diagonal and ragged tiles need it, and
  // the compiler would otherwise speculate it into every tile.
  static __device__ __forceinline__ void mask(f32x16 (&st)[KB], int lim) {
    asm volatile("" ::: "memory");   // keeps the caller's branch a real branch
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        st[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3)) > lim ? -INFINITY : st[kb][i];
  }

  // ALiBi: st += mul * |dq - key offset|, dq = the lane's query minus the
  // tile's first key minus 4*hf (|i - j| is exact in fp32 below 2^24)
  static __device__ __forceinline__ void alibi(f32x16 (&st)[KB], float dq, float mul) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        st[kb][i] = __builtin_fmaf(__builtin_fabsf(dq - (float)(32 * kb + 8 * (i >> 2) + (i & 3))), mul, st[kb][i]);
  }

  // ---- the online-softmax step of one score tile, as a sequence of slices
  // (a caller may run other work between them).  In order:
  //   NMAX slices   partial maxima over 8 scores each
  //   1 slice       the row max (both lane halves), the new running max,
  //                 alpha = 2^(m_old - m_new) and the exponent base in use
  //   NEXP slices   P = 2^(c2 * s - m) for 4 scores each (masked scores are
  //                 -inf and c2 > 0, so their P is exactly 0)
  //   NPACK slices  4 probabilities packed into the P operand and added, in
  //                 fp32 and before rounding, to this lane half's row sum
  // Rescaling: only when some row's maximum grew by more than TAU (log2
  // units) over the base in use, which keeps exponents <= 2^TAU; O and l
  // always share one base, so the result is the same.
  static constexpr int NMAX = 2 * KB, NEXP = 4 * KB, NPACK = 4 * KB;
  static constexpr int NSLICES = NMAX + 1 + NEXP + NPACK;
  struct Softmax {
    float mpart[NMAX];
    float alpha;     // factor for O and l (1 when the base is kept)
    bool grow;       // this lane's base changed
    float m_use;     // exponent base (0 while nothing is seen yet)
    float psum[2];
  };

  template <int SL>
  static __device__ __forceinline__ void softmax_slice(f32x16 (&st)[KB], Softmax& sm, float& m_run, float c2, PFrag& pf) {
    if constexpr (SL < NMAX) {
      const int kb = SL / 2, i0 = 8 * (SL % 2);
      // v_maximum3_f32: no NaN canonicalisation of the inputs, -inf handled as usual
      float m = st[kb][i0];
#pragma unroll
      for (int i = 1; i < 8; ++i) m = __builtin_elementwise_maximum(m, st[kb][i0 + i]);
      sm.mpart[SL] = m;
    } else if constexpr (SL == NMAX) {
      float m = sm.mpart[0];
#pragma unroll
      for (int i = 1; i < NMAX; ++i) m = __builtin_elementwise_maximum(m, sm.mpart[i]);
      const float m_tile = swap_halves_max(m) * c2;
      sm.grow = m_tile > m_run + TAU;
      sm.alpha = sm.grow ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.f;
      m_run = sm.grow ? m_tile : m_run;
      sm.m_use = m_run == -INFINITY ? 0.f : m_run - EXP_SHIFT;
    } else if constexpr (SL < NMAX + 1 + NEXP) {
      constexpr int g = SL - NMAX - 1;
      const int kb = g / 4, i0 = 4 * (g % 4);
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = st[kb][i0 + i];
        x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c2, -sm.m_use));
        st[kb][i0 + i] = x[i];
      }
    } else {
      constexpr int g = SL - NMAX - 1 - NEXP;
      const int kb = g / 4, i0 = 4 * (g % 4);
      float x0 = st[kb][i0], x1 = st[kb][i0 + 1], x2 = st[kb][i0 + 2], x3 = st[kb][i0 + 3];
      if constexpr (MODE == MODE_FP8) {
        // step g/8, word g%8 <- scores 4g .. 4g+3 of the tile.  The two
        // conversions write both halves of the word, so it starts undefined
        // (a zero start cost a v_mov per word).
        int word;
        asm volatile("" : "=v"(word));
        word = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, word, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, word, true);
        pf.f8[g / 8][g % 8] = word;
      } else {
        // step g/2, words 2*(g%2) and 2*(g%2)+1 <- scores 4g .. 4g+3 of the tile
        int h0 = (int)pack_bf16x2(x0, x1), h1 = (int)pack_bf16x2(x2, x3);
        pf.h[g / 2][2 * (g % 2)] = h0;
        pf.h[g / 2][2 * (g % 2) + 1] = h1;
        if constexpr (MODE == MODE_F32) {
          int l0 = (int)pack_bf16x2(x0 - bf16_lo_to_f32(h0), x1 - bf16_hi_to_f32(h0));
          int l1 = (int)pack_bf16x2(x2 - bf16_lo_to_f32(h1), x3 - bf16_hi_to_f32(h1));
          pf.l[g / 2][2 * (g % 2)] = l0;
          pf.l[g / 2][2 * (g % 2) + 1] = l1;
        }
      }
      const float part = (x0 + x1) + (x2 + x3);
      sm.psum[g & 1] = g < 2 ? part : sm.psum[g & 1] + part;
    }
  }
  template <int A, int B>
  static __device__ __forceinline__ void softmax_slices(f32x16 (&st)[KB], Softmax& sm, float& m_run, float c2, PFrag& pf) {
    if constexpr (A < B) {
      softmax_slice<A>(st, sm, m_run, c2, pf);
      softmax_slices<A + 1, B>(st, sm, m_run, c2, pf);
    }
  }

  // ---- the online-softmax step with the row max taken only when needed
  // (bf16).  Once every row of the wave has a finite running max, a tile's
  // exponentials are taken against the base already in use, without the
  // tile's row max.  Every P is >= 0, so a lane sum of at most 2^TAU bounds
  // each of the lane's probabilities by 2^TAU: the base could stay, which is
  // what the lazy rule decides from the max.  A larger sum (or a NaN) sends
  // the wave through the max-first order (rebase): the row max of the
  // exponents, a new base where a row grew by more than TAU, the tile's
  // exponentials again, and O and l rescaled.  Bases, probabilities and
  // rescales are those of the max-first order; what is saved is the max of
  // every other tile.  (fp8, whose lag of 2 under a 2^6 pre-scale leaves
  // no such margin, measured slower with a 448 bound and exact rebases:
  // 1.88 -> 1.91 ms at d = 256, 0.338 -> 0.391 ms long causal d = 128.)
  static constexpr bool SPEC = MODE == MODE_BF16;
  static constexpr float SPEC_LIMIT = 256.f;   // 2^TAU
  static constexpr float RTAU = TAU;

  // the exponent base of a row with running max m_run (0 before any key)
  static __device__ __forceinline__ float m_use(float m_run) {
    return m_run == -INFINITY ? 0.f : m_run - EXP_SHIFT;
  }
  // the row max of st over both lane halves
  static __device__ __forceinline__ float row_max(const f32x16 (&st)[KB]) {
    float m[2 * KB];
#pragma unroll
    for (int h = 0; h < 2 * KB; ++h) {
      const int kb = h / 2, i0 = 8 * (h % 2);
      m[h] = st[kb][i0];
#pragma unroll
      for (int i = 1; i < 8; ++i) m[h] = __builtin_elementwise_maximum(m[h], st[kb][i0 + i]);
    }
#pragma unroll
    for (int h = 1; h < 2 * KB; ++h) m[0] = __builtin_elementwise_maximum(m[0], m[h]);
    return swap_halves_max(m[0]);
  }
  // st <- c2 * st - m_use (scores to exponents, log2 units)
  static __device__ __forceinline__ void to_exponents(f32x16 (&st)[KB], float c2, float m_use) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kb][i] = __builtin_fmaf(st[kb][i], c2, -m_use);
  }
  // P = 2^x packed as the P.V operand (x is kept); returns this lane's sum
  // of the fp32 probabilities
  static __device__ __forceinline__ float probs(const f32x16 (&x)[KB], PFrag& pf) {
    static_assert(MODE == MODE_BF16, "bf16 P operand");
    float sum[2];
#pragma unroll
    for (int g = 0; g < 4 * KB; ++g) {
      const int kb = g / 4, i0 = 4 * (g % 4);
      const float e0 = __builtin_amdgcn_exp2f(x[kb][i0]), e1 = __builtin_amdgcn_exp2f(x[kb][i0 + 1]);
      const float e2 = __builtin_amdgcn_exp2f(x[kb][i0 + 2]), e3 = __builtin_amdgcn_exp2f(x[kb][i0 + 3]);
      // step g/2, words 2*(g%2) and 2*(g%2)+1 <- scores 4g .. 4g+3 of the tile
      pf.h[g / 2][2 * (g % 2)] = (int)pack_bf16x2(e0, e1);
      pf.h[g / 2][2 * (g % 2) + 1] = (int)pack_bf16x2(e2, e3);
      const float part = (e0 + e1) + (e2 + e3);
      sum[g & 1] = g < 2 ? part : sum[g & 1] + part;
    }
    return sum[0] + sum[1];
  }
  // the max-first order for a tile whose exponents x were taken against
  // the base m_use(m_run) and whose lane sums passed SPEC_LIMIT: a row whose
  // max passed the base by more than RTAU (a row without a base: that saw
  // any key) moves its base to that max and its exponents with it.  Returns
  // alpha = 2^(m_old - m_new) for O and l (1: base kept or new).
  static __device__ __forceinline__ float rebase(f32x16 (&x)[KB], float& m_run) {
    const float mx = row_max(x);
    const bool fresh = m_run == -INFINITY;
    const bool grow = fresh ? mx > -INFINITY : mx > RTAU;
    const float delta = grow ? mx : 0.f;
    m_run = fresh ? (grow ? mx : m_run) : m_run + delta;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) x[kb] -= delta;
    // (a row without a base has O = 0 and l = 0: its factor stays 1)
    return grow && !fresh ? __builtin_amdgcn_exp2f(-delta) : 1.f;
  }

  // oacc += V^T P^T for the tile at vbase
  static __device__ __forceinline__ void pv(f32x16 (&oacc)[NDB], const char FA_LDS* vbase, const PFrag& pf, const Lane& ln) {
    if constexpr (PIPE) {
      pv_pipe(oacc, vbase, pf, ln);
      return;
    }
#pragma unroll
    for (int s = 0; s < PV_STEPS; ++s) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (MODE == MODE_F32) {
          const int row = 16 * s + ln.v_row;
          const int col = 32 * db * 2 + ln.v_col;      // bytes
          const int off0 = row * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(row)) << 4) | (col & 15));
          const int off1 = (row + 8) * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(row + 8)) << 4) | (col & 15));
          i16x4 lo = lds_tr16(vbase + off0), hi = lds_tr16(vbase + off1);
          i16x4 lo2 = lds_tr16(vbase + G::TILEB + off0), hi2 = lds_tr16(vbase + G::TILEB + off1);
          bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          bf16x8 al = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8 ph = __builtin_bit_cast(bf16x8, pf.h[s]), pl = __builtin_bit_cast(bf16x8, pf.l[s]);
          oacc[db] = mfma_bf16(a, ph, oacc[db]);
          oacc[db] = mfma_bf16(a, pl, oacc[db]);
          oacc[db] = mfma_bf16(al, ph, oacc[db]);
        } else {
          pv_mma(oacc, s, db, v_operand(vbase, s, db, ln), pf);
        }
      }
    }
  }

  // O = out_mul * O / l and L = ln2 * (m + log2 l) for query my_q (a row
  // that saw no key, possible only under a block-sparse mask: O = 0, L = -inf)
  static __device__ __forceinline__ void store(const Params& p, int64_t head_off, int bh, int my_q, const Lane& ln,
                                               const f32x16 (&oacc)[NDB], float m_run, float l_run) {
    const float l_tot = swap_halves_sum(l_run);
    const bool seen = l_tot > 0.f;
    const float inv = seen ? p.out_mul / l_tot : 0.f;
    if (my_q >= p.N) return;
    if (ln.hf == 0)
      p.lse[(int64_t)bh * p.N + my_q] = seen ? (m_run - EXP_SHIFT + __log2f(l_tot)) * kLn2 : -INFINITY;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * ln.hf;
        const float x0 = oacc[db][4 * g] * inv, x1 = oacc[db][4 * g + 1] * inv;
        const float x2 = oacc[db][4 * g + 2] * inv, x3 = oacc[db][4 * g + 3] * inv;
        if constexpr (MODE == MODE_F32) {
          float* dst = static_cast<float*>(p.o) + head_off + (int64_t)my_q * D + col;
          *reinterpret_cast<f32x4*>(dst) = f32x4{x0, x1, x2, x3};
        } else {
          uint16_t* dst = static_cast<uint16_t*>(p.o) + head_off + (int64_t)my_q * D + col;
          *reinterpret_cast<i32x2*>(dst) = i32x2{(int)pack_bf16x2(x0, x1), (int)pack_bf16x2(x2, x3)};
        }
      }
  }
};

// HBM -> LDS staging of one K or V tile with global_load_lds_dwordx4 (bf16 and
// fp8 tiles).  One wave instruction fills 1 KiB of LDS, lane l at byte 16*l;
// the XOR swizzle is applied by choosing which global chunk each lane
// fetches.  The per-lane byte offsets inside a full tile do not depend on the
// tile, so they are computed once; the tile's base address is wave-uniform
// and travels in SGPRs.  Rows past the end of the sequence re-read row N-1:
// their scores are masked, so they only ever meet P = 0.  NT: streaming
// loads (dma16_s), for a K/V stream no other workgroup reads.
template <int D, int BC, int NW, int MODE, bool IS_V, bool NT = false>
struct Stager {
  using G = Geo<D, BC, NW, MODE>;
  // Chunk i of a thread lies NW * 1024 bytes (ADV rows) after chunk 0.  When
  // ADV is a multiple of the swizzle period (16 rows for every K and V
  // swizzle here), chunk i has chunk 0's swizzle: its offset is chunk 0's
  // plus a constant, and one register holds them all.
  static constexpr int ADV = NW * 1024 / G::ROWB;
  static constexpr bool AFFINE = NW * 1024 % G::ROWB == 0 && ADV % 16 == 0;
  int ofs[AFFINE ? 1 : G::UPT];
  int row0_, swz0_;   // AFFINE: chunk 0's row and swizzled byte column

  static __device__ __forceinline__ int swz(int row) {
    if constexpr (IS_V) return swz_v<G::CPR, MODE>(row);
    else return swz_k<G::CPR>(row);
  }
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < (AFFINE ? 1 : G::UPT); ++i) {
      const int off = (i * NW + wave) * 1024 + lane * 16;
      const int row = off / G::ROWB, pc = (off % G::ROWB) >> 4;
      ofs[i] = row * G::ROWB + ((pc ^ swz(row)) << 4);
      if (i == 0) {
        row0_ = row;
        swz0_ = (pc ^ swz(row)) << 4;
      }
    }
  }
  // tile j of the head at glob -> LDS at dst
  __device__ __forceinline__ void issue(const char* glob, int j, int N, char FA_LDS* dst, int wave, int lane) const {
    if (G::LOADERS < NW && wave >= G::LOADERS) return;
    const int row0 = j * BC;
    const char* base = glob + (int64_t)row0 * G::ROWB;
    if (row0 + BC <= N) {
#pragma unroll
      for (int i = 0; i < G::UPT; ++i)
        dma16_s<NT>(base, AFFINE ? ofs[0] + i * NW * 1024 : ofs[i], dst + (i * NW + wave) * 1024);
    } else {
      const int last = N - 1 - row0;
#pragma unroll
      for (int i = 0; i < G::UPT; ++i) {
        if constexpr (AFFINE) {
          dma16_s<NT>(base, min(row0_ + i * ADV, last) * G::ROWB + swz0_, dst + (i * NW + wave) * 1024);
        } else {
          const int off = (i * NW + wave) * 1024 + lane * 16;
          const int row = off / G::ROWB, pc = (off % G::ROWB) >> 4;
          dma16_s<NT>(base, min(row, last) * G::ROWB + ((pc ^ swz(row)) << 4), dst + (i * NW + wave) * 1024);
        }
      }
    }
  }
};

}  // namespace fa
