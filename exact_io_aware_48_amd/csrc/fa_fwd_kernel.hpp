// FlashAttention forward for gfx950 (CDNA4): one fused kernel per (d, dtype, mask).
//
// What it computes (per batch b, head h):  O = softmax(scale * Q K^T) V and the
// per-row logsumexp L, optionally under the causal mask -- the formula of the
// systems-analysis.info page "FlashAttention (PL)" ("Problematyka standardowego
// mechanizmu uwagi") and the chipfoundryservices glossary "Flash Attention".
//
// How (the glossary's "Tiling Algorithm", steps 1-6, restated for CDNA4):
//   * A workgroup owns B_r = 32 * NW query rows of one head (step 1).  Each of
//     its NW wave64s owns 32 of those rows; the wave's Q slice is loaded from
//     HBM once, straight into VGPRs in MFMA operand layout (step 2's "load the
//     Q block once", robocikowo.com page).
//   * K and V stream through LDS in tiles of B_c keys, double-buffered: while a
//     tile is consumed, the next one is already in flight from HBM/L2 (the
//     overlap of loads and matrix work the pages credit FlashAttention-3 with).
//   * S^T = K_j Q_i^T is computed on MFMA (step 3) -- transposed so that one
//     query's scores sit in one lane column of the 32x32 accumulator: the row
//     max and row sum of the online softmax become in-lane reductions plus a
//     single exchange between the two 32-lane halves (v_permlane32_swap).
//   * Online softmax (step 4; systems-analysis "Obliczanie Softmax w trybie
//     online"): running max m and sum l in fp32, in log2 units so that
//     v_exp_f32 (2^x) does the exponentials; when m grows the output
//     accumulator is multiplied by 2^(m_old - m_new) (robocikowo's
//     rescale(O_prev, m_old, m_new)).
//   * O^T += V_j^T P^T on MFMA (step 5).  P^T comes straight from the S^T
//     accumulator registers; the matching V^T operand is read from the
//     row-major V tile with the LDS transpose reads ds_read_b64_tr_b16/_b8.
//   * After the last tile, O is divided by l once and L = ln2 * (m + log2 l)
//     is written (step 6; FlashAttention-2's fewer non-matmul operations,
//     glossary "Flash Attention 2 Improvements").
//   * Under the causal mask, tiles entirely above the diagonal are never
//     loaded or computed; row blocks are dispatched heaviest first.
//   * The grid is mapped so that all row blocks of a head run on one XCD
//     (workgroups are dealt to the 8 XCDs round-robin), keeping that head's
//     K/V stream in one L2.
//
// Numeric modes:
//   MODE_BF16 : bf16 in/out, v_mfma_f32_32x32x16_bf16 for both products.
//   MODE_FP8  : OCP e4m3fn in (per-tensor descales), bf16 out,
//               v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales) for both
//               products; P is scaled by 256 before rounding to e4m3.
//   MODE_F32  : fp32 in/out; each operand x is split as hi = bf16(x),
//               lo = bf16(x - hi) and each product uses hi*hi + hi*lo + lo*hi.
#pragma once

#include "fa_common.hpp"

namespace fa {

// ---------------------------------------------------------------- the kernel
template <int D, int BC, int NW, int MODE, bool CAUSAL, int STAGES = 2>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_kernel(Params p) {
  using G = Geo<D, BC, NW, MODE, STAGES>;
  constexpr int KB = BC / 32;                       // 32-key blocks per tile
  constexpr int NDB = D / 32;                       // 32-wide blocks of the head dim
  constexpr int QK_STEPS = MODE == MODE_FP8 ? D / 64 : D / 16;   // MFMA k-steps over d
  constexpr int PV_STEPS = MODE == MODE_FP8 ? BC / 64 : BC / 16; // MFMA k-steps over keys
  // lazy-rescale threshold (log2 units); fp8 keeps P <= 1 so that 256 * P fits e4m3
  constexpr float TAU = MODE == MODE_FP8 ? 0.f : 8.f;

  __shared__ __attribute__((aligned(16))) char smem_raw[G::LDSB];
  char FA_LDS* const smem = (char FA_LDS*)(smem_raw);  // generic -> LDS address space

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;     // query column of this lane in the 32x32 accumulators
  const int hf = lane >> 5;    // lane half

  int bh, rb;
  map_block<CAUSAL>(p, blockIdx.x, bh, rb);
  const int N = p.N;
  const int64_t head_off = (int64_t)bh * N * D;    // element offset of this head
  const int q_row0 = rb * G::BR;                   // first query of the workgroup
  const int qw0 = q_row0 + 32 * wave;              // first query of this wave
  const int my_q = qw0 + n;

  const int tiles_all = (N + BC - 1) / BC;
  const int n_tiles = CAUSAL ? min(tiles_all, (q_row0 + G::BR - 1) / BC + 1) : tiles_all;
  const int wave_tiles = CAUSAL ? min(tiles_all, (qw0 + 31) / BC + 1) : tiles_all;

  // ---------------- Q slice -> registers (B operand of S^T = K Q^T)
  bf16x8 qa[QK_STEPS];        // bf16 mode: the bf16 values; f32 mode: hi parts
  bf16x8 ql[MODE == MODE_F32 ? QK_STEPS : 1];
  i32x8 q8[MODE == MODE_FP8 ? QK_STEPS : 1];
  {
    const bool valid = my_q < N;
    if constexpr (MODE == MODE_BF16) {
      const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.q) + head_off + (int64_t)my_q * D);
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        i32x4 w = valid ? src[2 * c + hf] : i32x4{0, 0, 0, 0};
        const int sgn = (int)p.qsign;
        w ^= i32x4{sgn, sgn, sgn, sgn};
        qa[c] = __builtin_bit_cast(bf16x8, w);
      }
    } else if constexpr (MODE == MODE_FP8) {
      const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint8_t*>(p.q) + head_off + (int64_t)my_q * D);
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        i32x4 w0 = valid ? src[4 * c + 2 * hf] : i32x4{0, 0, 0, 0};
        i32x4 w1 = valid ? src[4 * c + 2 * hf + 1] : i32x4{0, 0, 0, 0};
        const int sgn = (int)p.qsign;
        w0 ^= i32x4{sgn, sgn, sgn, sgn};
        w1 ^= i32x4{sgn, sgn, sgn, sgn};
        q8[c] = i32x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      }
    } else {
      const float* src = static_cast<const float*>(p.q) + head_off + (int64_t)my_q * D;
#pragma unroll
      for (int c = 0; c < QK_STEPS; ++c) {
        float x[8];
        if (valid) {
          f32x4 a = *reinterpret_cast<const f32x4*>(src + 16 * c + 8 * hf);
          f32x4 b = *reinterpret_cast<const f32x4*>(src + 16 * c + 8 * hf + 4);
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
        qa[c] = __builtin_bit_cast(bf16x8, hi);
        ql[c] = __builtin_bit_cast(bf16x8, lo);
      }
    }
  }

  // ---------------- K/V tile staging
  // bf16/fp8: direct HBM -> LDS loads (global_load_lds_dwordx4).  One wave
  // instruction fills 1 KiB of LDS, lane l at byte 16*l; the XOR swizzle is
  // applied by choosing which global chunk each lane fetches.  Rows past the
  // end of the sequence re-read row N-1: their scores are masked, so they
  // only ever meet P = 0.
  // fp32: HBM -> registers -> hi/lo split -> LDS, thread t moving the 16-byte
  // LDS chunks u = t + i * NT of each plane.
  constexpr bool DMA = MODE != MODE_F32;
  constexpr int SRC_VEC = 2;                          // fp32: 16-byte global loads per LDS chunk
  i32x4 kst[DMA ? 1 : G::UPT * SRC_VEC], vst[DMA ? 1 : G::UPT * SRC_VEC];
  const char* kglob = static_cast<const char*>(p.k) + head_off * G::EB;
  const char* vglob = static_cast<const char*>(p.v) + head_off * G::EB;

  auto issue_tile = [&](int j, char FA_LDS* kdst) __attribute__((always_inline)) {  // DMA modes
    const int row0 = j * BC;
    char FA_LDS* vdst = kdst + G::TILEB;
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
      const int blk = (i * NW + wave) * 1024;         // this wave instruction's LDS block
      const int off = blk + lane * 16;
      const int row = off / G::ROWB, pc = (off % G::ROWB) >> 4;
      const int64_t grow = (int64_t)min(row0 + row, N - 1) * G::ROWB;
      const char* ks = kglob + grow + ((pc ^ swz_k<G::CPR>(row)) << 4);
      const char* vs = vglob + grow + ((pc ^ swz_v<G::CPR, MODE>(row)) << 4);
      dma16(ks, kdst + blk);
      dma16(vs, vdst + blk);
    }
  };
  auto load_tile = [&](int j) __attribute__((always_inline)) {                      // fp32 mode
    const int row0 = j * BC;
#pragma unroll
    for (int i = 0; i < (DMA ? 0 : G::UPT); ++i) {
      const int u = tid + i * G::NT;
      const int row = u / G::CPR, ch = u % G::CPR;
      const bool ok = row0 + row < N;
      const float* kb = static_cast<const float*>(p.k) + head_off + (int64_t)(row0 + row) * D + ch * 8;
      const float* vb = static_cast<const float*>(p.v) + head_off + (int64_t)(row0 + row) * D + ch * 8;
      kst[2 * i] = ok ? *reinterpret_cast<const i32x4*>(kb) : i32x4{0, 0, 0, 0};
      kst[2 * i + 1] = ok ? *reinterpret_cast<const i32x4*>(kb + 4) : i32x4{0, 0, 0, 0};
      vst[2 * i] = ok ? *reinterpret_cast<const i32x4*>(vb) : i32x4{0, 0, 0, 0};
      vst[2 * i + 1] = ok ? *reinterpret_cast<const i32x4*>(vb + 4) : i32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](char FA_LDS* kbase) __attribute__((always_inline)) {        // fp32 mode
    char FA_LDS* vbase = kbase + G::PLANES * G::TILEB;
#pragma unroll
    for (int i = 0; i < (DMA ? 0 : G::UPT); ++i) {
      const int u = tid + i * G::NT;
      const int row = u / G::CPR, ch = u % G::CPR;
      const int koff = row * G::ROWB + ((ch ^ swz_k<G::CPR>(row)) << 4);
      const int voff = row * G::ROWB + ((ch ^ swz_v<G::CPR, MODE>(row)) << 4);
      float kx[8], vx[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kx[e] = __int_as_float(kst[2 * i][e]); kx[4 + e] = __int_as_float(kst[2 * i + 1][e]);
        vx[e] = __int_as_float(vst[2 * i][e]); vx[4 + e] = __int_as_float(vst[2 * i + 1][e]);
      }
      i32x4 kh, kl, vh, vl;
      split8(kx, kh, kl);
      split8(vx, vh, vl);
      lds_write16(kbase + koff, kh);
      lds_write16(kbase + G::TILEB + koff, kl);
      lds_write16(vbase + voff, vh);
      lds_write16(vbase + G::TILEB + voff, vl);
    }
  };
  constexpr int TILE_LOADS = 2 * G::UPT;               // DMA instructions per thread per tile
  auto wait_loads = [&]() __attribute__((always_inline)) {
    if constexpr (DMA) wait_vmcnt<0>();
  };

  // ---------------- running state
  f32x16 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;   // running max of scaled scores, log2 units (same in both lane halves)
  float l_run = 0.f;         // this lane half's part of the running sum
  const float c2 = p.c2;     // > 0 (the host keeps it at least 1e-30)
  // causal: the last key this lane's query sees, relative to 4*hf; ragged: the last key
  const int last_key = (CAUSAL ? min(N - 1, my_q) : N - 1) - 4 * hf;

  // per-lane pieces of the V^T transpose-read addresses (see the PV step)
  const int grp = lane >> 4;              // 16-lane group
  int v_row_part, v_col_part;             // key row offset, byte column offset
  if constexpr (MODE == MODE_FP8) {
    const int isrc = (lane & 15) >> 1;    // which of the 8 returned bytes this lane sources
    v_row_part = 8 * (isrc >> 2) + 4 * hf + (isrc & 3);
    v_col_part = 16 * (grp & 1) + 8 * (lane & 1);
  } else {
    v_row_part = 4 * hf + ((lane >> 2) & 3);
    v_col_part = 2 * (16 * (grp & 1) + 4 * (lane & 3));
  }

  auto compute_tile = [&](int j, const char FA_LDS* kbase) __attribute__((always_inline)) {
    const char FA_LDS* vbase = kbase + G::PLANES * G::TILEB;

    // ---- S^T = K_j Q^T   (rows: keys, columns: this wave's 32 queries)
    f32x16 st[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) st[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < QK_STEPS; ++c) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = 32 * kb + n;
        if constexpr (MODE == MODE_FP8) {
          const int sw = swz_k<G::CPR>(row);
          const char FA_LDS* rp = kbase + row * G::ROWB;
          i32x4 a0 = lds_read16(rp + (((4 * c + 2 * hf) ^ sw) << 4));
          i32x4 a1 = lds_read16(rp + (((4 * c + 2 * hf + 1) ^ sw) << 4));
          i32x8 a = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          st[kb] = mfma_fp8(a, q8[c], st[kb]);
        } else {
          const int off = row * G::ROWB + (((2 * c + hf) ^ swz_k<G::CPR>(row)) << 4);
          bf16x8 a = __builtin_bit_cast(bf16x8, lds_read16(kbase + off));
          st[kb] = mfma_bf16(a, qa[c], st[kb]);
          if constexpr (MODE == MODE_F32) {
            bf16x8 al = __builtin_bit_cast(bf16x8, lds_read16(kbase + G::TILEB + off));
            st[kb] = mfma_bf16(a, ql[c], st[kb]);
            st[kb] = mfma_bf16(al, qa[c], st[kb]);
          }
        }
      }
    }

    // ---- online softmax (log2 domain)
    // accumulator element i of block kb holds key key0 + 32*kb + 8*(i/4) + 4*hf + i%4
    const int key0 = j * BC;
    if ((key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qw0)) {
      const int lim = last_key - key0;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          st[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3)) > lim ? -INFINITY : st[kb][i];
    }
    float mraw = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, st[kb][i]);
    mraw = swap_halves_max(mraw);
    // Rescale only when some row's maximum grew by more than TAU (log2
    // units) over the base in use: exponents are then <= 2^TAU, and since O
    // and l always share one base the result is the same.
    const float m_tile = mraw * c2;
    const bool grow = m_tile > m_run + TAU;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      asm volatile("" ::: "memory");   // keep this a real (rarely taken) branch, not a select
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.f;
      m_run = grow ? m_tile : m_run;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b) oacc[b] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;

    // masked scores are -inf and c2 > 0, so their exponentials are exactly 0
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][i], c2, -m_use));
        st[kb][i] = e;
        psum += e;
      }
    l_run += psum;

    // ---- O^T += V_j^T P^T
    if constexpr (MODE == MODE_FP8) {
#pragma unroll
      for (int g = 0; g < PV_STEPS; ++g) {              // 64 keys per step
        // B operand byte 16*kb' + i <- P of key 64g + 32*kb' + 8*(i/4) + 4*hf + i%4
        i32x8 pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb = 2 * g + (w >> 2);
          const int i0 = 4 * (w & 3);
          int word = 0;
          word = __builtin_amdgcn_cvt_pk_fp8_f32(st[kb][i0] * 256.f, st[kb][i0 + 1] * 256.f, word, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(st[kb][i0 + 2] * 256.f, st[kb][i0 + 3] * 256.f, word, true);
          pb[w] = word;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          int va[8];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int row = 64 * g + 16 * t + v_row_part;
            const int col = 32 * db + v_col_part;        // bytes
            const int off = row * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(row)) << 4) | (col & 15));
            i32x2 r = lds_tr8(vbase + off);
            va[2 * t] = r[0];
            va[2 * t + 1] = r[1];
          }
          i32x8 a = i32x8{va[0], va[1], va[2], va[3], va[4], va[5], va[6], va[7]};
          oacc[db] = mfma_fp8(a, pb, oacc[db]);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < PV_STEPS; ++s) {              // 16 keys per step
        const int kb = s >> 1, cp = s & 1;
        // B operand element i <- P of key 32*kb + 16*cp + 8*(i/4) + 4*hf + i%4
        i32x4 ph, pl;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float x0 = st[kb][8 * cp + 2 * w], x1 = st[kb][8 * cp + 2 * w + 1];
          const uint32_t h = pack_bf16x2(x0, x1);
          ph[w] = (int)h;
          if constexpr (MODE == MODE_F32)
            pl[w] = (int)pack_bf16x2(x0 - bf16_lo_to_f32(h), x1 - bf16_hi_to_f32(h));
        }
        const bf16x8 pbh = __builtin_bit_cast(bf16x8, ph);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int row = 32 * kb + 16 * cp + v_row_part;
          const int col = 32 * db * 2 + v_col_part;      // bytes
          const int off0 = row * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(row)) << 4) | (col & 15));
          const int off1 = (row + 8) * G::ROWB + ((((col >> 4) ^ swz_v<G::CPR, MODE>(row + 8)) << 4) | (col & 15));
          i16x4 lo = lds_tr16(vbase + off0), hi = lds_tr16(vbase + off1);
          bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = mfma_bf16(a, pbh, oacc[db]);
          if constexpr (MODE == MODE_F32) {
            i16x4 lo2 = lds_tr16(vbase + G::TILEB + off0), hi2 = lds_tr16(vbase + G::TILEB + off1);
            bf16x8 al = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = mfma_bf16(a, __builtin_bit_cast(bf16x8, pl), oacc[db]);
            oacc[db] = mfma_bf16(al, pbh, oacc[db]);
          }
        }
      }
    }
  };

  if constexpr (STAGES == 2) {
    if constexpr (DMA) {
      issue_tile(0, smem);
    } else {
      load_tile(0);
      store_tile(smem);
    }
    wait_loads();
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
      char FA_LDS* const cur = smem + (j & 1) * G::STAGEB;
      char FA_LDS* const next = smem + ((j & 1) ^ 1) * G::STAGEB;
      const bool more = j + 1 < n_tiles;
      if (more) {                       // start fetching tile j+1 into the other stage
        if constexpr (DMA) issue_tile(j + 1, next);
        else load_tile(j + 1);
      }
      if (j < wave_tiles) compute_tile(j, cur);
      if constexpr (!DMA) {
        if (more) store_tile(next);
      }
      wait_loads();
      __syncthreads();
    }
  } else {
    // three-stage ring: tile j+2 is in flight while tile j is consumed; the
    // wait at the end of iteration j covers tile j+1 only
    issue_tile(0, smem);
    if (n_tiles > 1) {
      issue_tile(1, smem + G::STAGEB);
      wait_vmcnt<TILE_LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    int cur_s = 0;                      // stage of tile j
    for (int j = 0; j < n_tiles; ++j) {
      const int ahead_s = cur_s == 0 ? 2 : cur_s - 1;   // (j + 2) % 3
      const bool ahead = j + 2 < n_tiles;
      if (ahead) issue_tile(j + 2, smem + ahead_s * G::STAGEB);
      if (j < wave_tiles) compute_tile(j, smem + cur_s * G::STAGEB);
      if (ahead) wait_vmcnt<TILE_LOADS>();
      else wait_vmcnt<0>();
      __syncthreads();
      cur_s = cur_s == 2 ? 0 : cur_s + 1;
    }
  }

  // ---------------- epilogue: O = O / l, L = ln2 * (m + log2 l)
  const float l_tot = swap_halves_sum(l_run);
  const float inv = p.out_mul / l_tot;
  if (my_q < N) {
    if (hf == 0) p.lse[(int64_t)bh * N + my_q] = (m_run + __log2f(l_tot)) * kLn2;
    // accumulator element i of d-block db holds dim 32*db + 8*(i/4) + 4*hf + i%4
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * hf;
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
}

}  // namespace fa
