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
//   * Ping-pong (PP): with eight waves in a workgroup, the two waves sharing a
//     SIMD would otherwise run in lock step (both in softmax, matrix core
//     idle).  The upper half of the waves therefore runs each tile's P V one
//     iteration late -- [P V_{j-1}] [S_j, softmax_j] against the lower half's
//     [S_j, softmax_j] [P V_j] -- so one wave's softmax overlaps the other's
//     MFMAs.  The V ring keeps one extra tile for the late group.  (An
//     option: raised wave priority outside the MFMA blocks measured faster
//     on every shape, so no instance uses ping-pong now.)
//   * The grid is mapped so that all row blocks of a head run on one XCD
//     (workgroups are dealt to the 8 XCDs round-robin), keeping that head's
//     K/V stream in one L2.
//
// Variants (every mode, PP off):
//   VAR_ALIBI       : the score of query i and key j gets -slope_h * |i - j|
//                     after scaling (added to the unscaled score as
//                     -slope_h / |scale| * |i - j| before the softmax).
//   VAR_BLOCKSPARSE : a byte mask over 128 x 128 (query block, key block)
//                     pairs; the workgroup walks only the key tiles some
//                     wave's block allows (the others are never loaded), and
//                     each wave skips the tiles its own block does not allow.
//
// Numeric modes:
//   MODE_BF16 : bf16 in/out, v_mfma_f32_32x32x16_bf16 for both products.
//   MODE_FP8  : OCP e4m3fn in (per-tensor descales), bf16 out,
//               v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales) for both
//               products; P is rounded to e4m3 as 2^6 * P, at most 2^8
//               with the rescale lag of 2 (the exponentials produce it
//               directly: the factor is in their base).
//   MODE_F32  : fp32 in/out; each operand x is split as hi = bf16(x),
//               lo = bf16(x - hi) and each product uses hi*hi + hi*lo + lo*hi.
#pragma once

#include "fa_tile.hpp"

namespace fa {

// ---------------------------------------------------------------- the kernel
// PRIO: a wave runs at raised priority except while it issues its MFMA
// blocks, so that a wave leaving its matrix work gets its softmax through
// ahead of the other wave's MFMA issue (measured at d = 256: +1% to +6%
// depending on the GPU session; none or a loss at d = 64 and 128).
// RP > 0: each step, a wave takes an issue priority that grows with the key
// tiles its workgroup still has to stream (above 4 RP: 3, 2 RP: 2, RP: 1,
// else 0).  Workgroups sharing a CU then advance together, and the one with
// the most work left goes first, instead of the oldest waves finishing early
// and leaving the last workgroup alone on the CU.
template <int RP>
__device__ __forceinline__ void prio_by_remaining(int rem) {
  if (rem > 4 * RP) __builtin_amdgcn_s_setprio(3);
  else if (rem > 2 * RP) __builtin_amdgcn_s_setprio(2);
  else if (rem > RP) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// How the kernel brings in its Q tile (bf16 and fp8): 1 = through the second
// K and V ring slots, which tile 0 leaves free (the tile fits them: rows
// 0 .. BR/2 - 1 in K slot 1, the rest in V slot 1); 2 = through an LDS region
// of its own (eight-wave workgroups, which run one per CU at their register
// counts, when it fits the LDS); 0 = each wave loads its slice directly.
template <int D, int BC, int NW, int MODE, bool PP>
constexpr int q_stage_mode() {
  if (MODE == MODE_F32 || PP) return 0;
  using G = Geo<D, BC, NW, MODE, PP>;
  constexpr int qtile = 32 * NW * D * (MODE == MODE_FP8 ? 1 : 2);
  if (qtile <= 2 * G::SLOTB) return 1;
  if (NW == 8 && G::LDSB + qtile <= 160 * 1024) return 2;
  return 0;
}
template <int D, int BC, int NW, int MODE, bool PP>
constexpr int q_region_bytes() {
  return q_stage_mode<D, BC, NW, MODE, PP>() == 2 ? 32 * NW * D * (MODE == MODE_FP8 ? 1 : 2) : 0;
}

template <int D, int BC, int NW, int MODE, bool CAUSAL, bool PP = false, int VAR = VAR_NONE, bool PRIO = false,
          int RP = 0>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_kernel(Params p) {
  static_assert(!(PRIO && RP), "one priority scheme");
  const unsigned long long t_entry = timeline_clock();
  static_assert(VAR == VAR_NONE || !PP, "variants: no ping-pong");
  static_assert(VAR != VAR_BLOCKSPARSE || ((32 * NW) % kMaskBlock == 0 && kMaskBlock % BC == 0),
                "row blocks and key tiles nest in the mask blocks");
  using G = Geo<D, BC, NW, MODE, PP>;
  using T = Tile<D, BC, NW, MODE>;
  constexpr int NDB = T::NDB;
  constexpr bool DMA = MODE != MODE_F32;

  // (the ALiBi fp8 instances keep direct Q loads: a region costs them spills)
  constexpr int QMODE0 = q_stage_mode<D, BC, NW, MODE, PP>();
  constexpr int QMODE = QMODE0 == 2 && VAR == VAR_ALIBI && MODE == MODE_FP8 ? 0 : QMODE0;
  __shared__ __attribute__((aligned(16))) char smem_raw[G::LDSB + (QMODE == 2 ? q_region_bytes<D, BC, NW, MODE, PP>() : 0)];
  char FA_LDS* const smem = (char FA_LDS*)(smem_raw);  // generic -> LDS address space
  // K ring slots first, then V ring slots
  auto kslot = [&](int s) __attribute__((always_inline)) { return smem + s * G::SLOTB; };
  auto vslot = [&](int s) __attribute__((always_inline)) { return smem + (G::KST + s) * G::SLOTB; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform in an SGPR, so that LDS and DMA addresses stay scalar (not
  // with ping-pong, whose fp8 d = 256 instance then spills)
  const int wave = PP ? tid >> 6 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const typename T::Lane ln = T::lane_info(lane);
  const bool late = PP && wave >= NW / 2;   // ping-pong: this wave runs P V one tile late

  int bh, rb;
  map_block<CAUSAL>(p, blockIdx.x, bh, rb);
  const int N = p.N;
  const int64_t head_off = (int64_t)bh * N * D;    // element offset of this head in Q and O
  const int64_t kv_off = (int64_t)(bh / p.G) * N * D;   // ... and of its K/V head
  const int q_row0 = rb * G::BR;                   // first query of the workgroup
  const int qw0 = q_row0 + 32 * wave;              // first query of this wave
  const int my_q = qw0 + ln.n;

  const int tiles_all = (N + BC - 1) / BC;
  const int n_tiles = CAUSAL ? min(tiles_all, (q_row0 + G::BR - 1) / BC + 1) : tiles_all;
  const int wave_tiles = CAUSAL ? min(tiles_all, (qw0 + 31) / BC + 1) : tiles_all;

  // Q through LDS in whole rows with tile 0 (q_stage_mode), or each wave's
  // slice directly
  typename T::QFrag q;
  if constexpr (QMODE == 0) T::load_q(p, head_off, my_q, ln, q);
  const char* const qglob = static_cast<const char*>(p.q) + head_off * T::QROWB / D + (int64_t)q_row0 * T::QROWB;
  auto stage_q = [&]() __attribute__((always_inline)) {
    if constexpr (QMODE == 1)
      T::template dma_q<NW * 32 * T::QROWB / 2048>(qglob, N - q_row0, kslot(1), vslot(1), wave, lane);
    else if constexpr (QMODE == 2)
      T::template dma_q<1 << 30>(qglob, N - q_row0, smem + G::LDSB, smem + G::LDSB, wave, lane);
  };
  // after the barrier that publishes tile 0 (and Q); in the ring slots, a
  // second barrier frees them for tile 1
  auto take_q = [&]() __attribute__((always_inline)) {
    if constexpr (QMODE == 1) {
      const char FA_LDS* rows = wave < NW / 2 ? kslot(1) + wave * 32 * T::QROWB : vslot(1) + (wave - NW / 2) * 32 * T::QROWB;
      T::load_q_lds(rows, ln, p.qsign, q);
      __syncthreads();
    } else if constexpr (QMODE == 2) {
      T::load_q_lds(smem + G::LDSB + wave * 32 * T::QROWB, ln, p.qsign, q);
    }
  };

  // ---------------- K/V tile staging
  // bf16/fp8: direct HBM -> LDS loads.  fp32: HBM -> registers -> hi/lo
  // split -> LDS, thread t moving the 16-byte LDS chunks u = t + i * NT of
  // each plane (rows past the end are zero-filled; they are masked anyway).
  Stager<D, BC, NW, MODE, false> kstage;
  Stager<D, BC, NW, MODE, true> vstage;
  if constexpr (DMA) {
    kstage.init(wave, lane);
    vstage.init(wave, lane);
  }
  const char* kglob = static_cast<const char*>(p.k) + kv_off * G::EB;
  const char* vglob = static_cast<const char*>(p.v) + kv_off * G::EB;
  auto issue_tile = [&](int j, char FA_LDS* kdst, char FA_LDS* vdst) __attribute__((always_inline)) {
    kstage.issue(kglob, j, N, kdst, wave, lane);
    vstage.issue(vglob, j, N, vdst, wave, lane);
  };
  constexpr int SRC_VEC = 2;                          // fp32: 16-byte global loads per LDS chunk
  i32x4 kst[DMA ? 1 : G::UPT * SRC_VEC], vst[DMA ? 1 : G::UPT * SRC_VEC];
  auto load_tile = [&](int j) __attribute__((always_inline)) {                      // fp32 mode
    const int row0 = j * BC;
#pragma unroll
    for (int i = 0; i < (DMA ? 0 : G::UPT); ++i) {
      const int u = tid + i * G::NT;
      const int row = u / G::CPR, ch = u % G::CPR;
      const bool ok = row0 + row < N;
      const float* kb = static_cast<const float*>(p.k) + kv_off + (int64_t)(row0 + row) * D + ch * 8;
      const float* vb = static_cast<const float*>(p.v) + kv_off + (int64_t)(row0 + row) * D + ch * 8;
      kst[2 * i] = ok ? *reinterpret_cast<const i32x4*>(kb) : i32x4{0, 0, 0, 0};
      kst[2 * i + 1] = ok ? *reinterpret_cast<const i32x4*>(kb + 4) : i32x4{0, 0, 0, 0};
      vst[2 * i] = ok ? *reinterpret_cast<const i32x4*>(vb) : i32x4{0, 0, 0, 0};
      vst[2 * i + 1] = ok ? *reinterpret_cast<const i32x4*>(vb + 4) : i32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](char FA_LDS* kbase, char FA_LDS* vbase) __attribute__((always_inline)) {  // fp32 mode
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

  // ---------------- running state
  f32x16 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;   // running max of scaled scores, log2 units (same in both lane halves)
  float l_run = 0.f;         // this lane half's part of the running sum
  const float c2 = p.c2;     // > 0 (the host keeps it at least 1e-30)
  // causal: the last key this lane's query sees, relative to 4*hf; ragged: the last key
  const int last_key = (CAUSAL ? min(N - 1, my_q) : N - 1) - 4 * ln.hf;
  typename T::PFrag pf;      // P of the current tile

  // ALiBi: this head's -slope / |scale|
  float alibi_a = 0.f;
  if constexpr (VAR == VAR_ALIBI) alibi_a = p.slopes[bh % p.H] * p.alibi_mul;

  // S_j = K_j Q^T (+ ALiBi bias, masks) into st
  auto scores = [&](int j, const char FA_LDS* kbase, f32x16 (&st)[T::KB]) __attribute__((always_inline)) {
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    T::qk(st, kbase, q, ln);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    const int key0 = j * BC;
    if constexpr (VAR == VAR_ALIBI) T::alibi(st, (float)(my_q - key0 - 4 * ln.hf), alibi_a);
    if ((key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qw0)) T::mask(st, last_key - key0);
  };
  // the max-first online-softmax update of st (raw scores), P packed into pf
  auto softmax_max_first = [&](f32x16 (&st)[T::KB]) __attribute__((always_inline)) {
    typename T::Softmax sm;
    T::template softmax_slices<0, T::NMAX + 1>(st, sm, m_run, c2, pf);
    if (__builtin_amdgcn_ballot_w64(sm.grow)) {
      asm volatile("" ::: "memory");   // keep this a real (rarely taken) branch, not a select
      l_run *= sm.alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b) oacc[b] *= sm.alpha;
    }
    T::template softmax_slices<T::NMAX + 1, T::NSLICES>(st, sm, m_run, c2, pf);
    l_run += sm.psum[0] + sm.psum[1];
  };
  // S_j, online-softmax update, P_j packed into pf
  auto qk_softmax = [&](int j, const char FA_LDS* kbase) __attribute__((always_inline)) {
    f32x16 st[T::KB];
    scores(j, kbase, st);
    if constexpr (T::SPEC && VAR == VAR_NONE) {
      // Once every row of the wave has a base, the exponentials are taken
      // against it without the row max (Tile::SPEC).  The max-first order
      // (Tile::rebase) runs for a wave with a row that has no base yet, and
      // again for a tile whose lane sum passed 2^TAU, with its scores
      // recomputed from the K tile (in LDS until the barrier ending the step).
      bool max_first = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
      float alpha = 1.f, psum;
      for (;;) {
        T::to_exponents(st, c2, T::m_use(m_run));
        if (max_first) alpha = T::rebase(st, m_run);
        psum = T::probs(st, pf);
        if (max_first || !__builtin_amdgcn_ballot_w64(!(psum <= T::SPEC_LIMIT))) break;
        asm volatile("" ::: "memory");   // a real (rarely taken) branch
        max_first = true;
        scores(j, kbase, st);
      }
      if (max_first) {
        asm volatile("" ::: "memory");
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < NDB; ++b) oacc[b] *= alpha;
      }
      l_run += psum;
    } else {
      softmax_max_first(st);
    }
  };
  auto pv = [&](const char FA_LDS* vbase) __attribute__((always_inline)) {
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    T::pv(oacc, vbase, pf, ln);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
  };

  unsigned long long t_pro = 0;
  if constexpr (VAR == VAR_BLOCKSPARSE) {
    // ---------------- block-sparse: only the tiles some wave's block allows
    const uint8_t* mrow = p.bmask + (int64_t)(bh / p.H) * p.bm_sb + (int64_t)(bh % p.H) * p.bm_sh;
    constexpr int RBLK = (32 * NW) / kMaskBlock;       // mask row blocks per workgroup
    const int rblk0 = q_row0 / kMaskBlock;
    const int wblk = qw0 / kMaskBlock;                 // this wave's mask row block
    auto allows = [&](int rblk, int j) __attribute__((always_inline)) {
      return rblk < p.nb && mrow[(int64_t)rblk * p.nb + (j * BC) / kMaskBlock] != 0;
    };
    auto needed = [&](int j) __attribute__((always_inline)) {
      bool any = false;
#pragma unroll
      for (int r = 0; r < RBLK; ++r) any = any || allows(rblk0 + r, j);
      return any;
    };
    auto next_needed = [&](int j) __attribute__((always_inline)) {
      while (j < n_tiles && !needed(j)) ++j;
      return j;
    };
    int j = next_needed(0);
    stage_q();
    if (j < n_tiles) {
      if constexpr (DMA) {
        issue_tile(j, kslot(0), vslot(0));
      } else {
        load_tile(j);
        store_tile(kslot(0), vslot(0));
      }
    }
    if constexpr (DMA) wait_vmcnt<0>();
    __syncthreads();
    take_q();
    t_pro = timeline_clock();
    int cur = 0;
    while (j < n_tiles) {
      const int jn = next_needed(j + 1);
      if (jn < n_tiles) {
        if constexpr (DMA) issue_tile(jn, kslot(cur ^ 1), vslot(cur ^ 1));
        else load_tile(jn);
      }
      if (j < wave_tiles && allows(wblk, j)) {
        qk_softmax(j, kslot(cur));
        pv(vslot(cur));
      }
      if constexpr (DMA) {
        wait_vmcnt<0>();
      } else {
        if (jn < n_tiles) store_tile(kslot(cur ^ 1), vslot(cur ^ 1));
      }
      __syncthreads();
      cur ^= 1;
      j = jn;
    }
  } else {
    // ---------------- main loop: one barrier per tile; tile j+1 is in flight
    // while tile j is used.  The slots refilled in step j held K_{j-1} and
    // V_{j-1} (V_{j-2} with ping-pong), whose last readers finished before the
    // barrier that ended step j-1.
    stage_q();
    if constexpr (DMA) {
      issue_tile(0, kslot(0), vslot(0));
      wait_vmcnt<0>();
    } else {
      load_tile(0);
      store_tile(kslot(0), vslot(0));
    }
    __syncthreads();
    take_q();
    t_pro = timeline_clock();

    if constexpr (!PP) {
      // two-slot ring: step j uses slot j % 2 and fills the other; unrolled
      // by two so that the slot offsets are constants of the LDS instructions
      auto step = [&](int j, int sl) __attribute__((always_inline)) {
        if constexpr (RP > 0) prio_by_remaining<RP>(n_tiles - j);
        const bool more = j + 1 < n_tiles;
        if (more) {                     // start fetching tile j+1 into the free slots
          if constexpr (DMA) issue_tile(j + 1, kslot(sl ^ 1), vslot(sl ^ 1));
          else load_tile(j + 1);
        }
        if (j < wave_tiles) {
          qk_softmax(j, kslot(sl));
          pv(vslot(sl));
        }
        if constexpr (DMA) {
          wait_vmcnt<0>();              // tile j+1 has landed
        } else {
          if (more) store_tile(kslot(sl ^ 1), vslot(sl ^ 1));
        }
        __syncthreads();
      };
      int j = 0;
      for (; j + 1 < n_tiles; j += 2) {
        step(j, 0);
        step(j + 1, 1);
      }
      if (j < n_tiles) step(j, 0);
    } else {
      int ks_cur = 0, vs_cur = 0, vs_prev = G::VST - 1;  // ring slots of tile j (K, V) and of V_{j-1}
      for (int j = 0; j < n_tiles; ++j) {
        const int ks_next = ks_cur ^ 1;
        const int vs_next = vs_cur + 1 == G::VST ? 0 : vs_cur + 1;
        const bool more = j + 1 < n_tiles;
        if (more) {                       // start fetching tile j+1 into the free slots
          if constexpr (DMA) issue_tile(j + 1, kslot(ks_next), vslot(vs_next));
          else load_tile(j + 1);
        }
        if (late) {                       // [P V_{j-1}] [S_j, softmax_j]
          if (j >= 1 && j - 1 < wave_tiles) pv(vslot(vs_prev));
          if (j < wave_tiles) qk_softmax(j, kslot(ks_cur));
        } else {                          // [S_j, softmax_j] [P V_j]
          if (j < wave_tiles) {
            qk_softmax(j, kslot(ks_cur));
            pv(vslot(vs_cur));
          }
        }
        if constexpr (DMA) {
          wait_vmcnt<0>();                // tile j+1 has landed
        } else {
          if (more) store_tile(kslot(ks_next), vslot(vs_next));
        }
        __syncthreads();
        vs_prev = vs_cur;
        ks_cur = ks_next;
        vs_cur = vs_next;
      }
      if (late && wave_tiles == n_tiles) pv(vslot(vs_prev));   // the late group's last P V
    }
  }

  const unsigned long long t_loop = timeline_clock();
  // (not at d = 256 for the block-sparse bf16 instances and the causal or
  // variant fp8 ones, where it costs spills)
  constexpr bool O_STAGE = MODE != MODE_F32 && !(D == 256 && ((MODE == MODE_BF16 && VAR == VAR_BLOCKSPARSE) ||
                                                              (MODE == MODE_FP8 && (CAUSAL || VAR != VAR_NONE))));
  if constexpr (O_STAGE) {
    // every loop above ends with a barrier: the rings are free for O, whose
    // rows leave in whole segments (as many d-blocks per pass as a wave's
    // share of the rings holds)
    constexpr int GDB0 = G::LDSB / (NW * 2048);
    constexpr int GDB = GDB0 >= NDB ? NDB : GDB0;
    T::template store_lds<GDB>(p, head_off, bh, qw0, my_q, ln, oacc, m_run, l_run, smem + wave * 32 * 64 * GDB, lane);
  } else {
    T::store(p, head_off, bh, my_q, ln, oacc, m_run, l_run);
  }
  timeline_record(t_entry, t_pro, t_loop, bh, rb);
}

}  // namespace fa
