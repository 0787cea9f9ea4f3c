// FlashAttention forward for gfx950, bf16, software-pipelined across key tiles.
//
// Same computation as fa_fwd_kernel (the glossary's "Tiling Algorithm" steps
// 1-6 with the online softmax of systems-analysis.info "FlashAttention (PL)",
// "Obliczanie Softmax w trybie online"; the causal mask and the logsumexp L of
// the robocikowo.com "Flash Attention" page), with a different order of work
// inside each wave.
//
// Why.  On a CDNA4 SIMD the matrix core runs an MFMA for 32 cycles while the
// issuing wave is free to issue other instructions.  When the softmax of a
// tile is a phase of its own, between the QK^T and the P V products, the
// matrix core idles through it (both waves of a SIMD tend to reach it
// together, held in step by the tile barrier).  Measured on MI355X, a wave
// that issues three VALU instructions, one exponential and one or two LDS
// reads between consecutive MFMAs loses only 10-15% of MFMA throughput.  So
// each wave carries two score tiles and overlaps the softmax of one with the
// matrix products of its neighbours.  (On the long causal d = 128 workload
// this takes fewer cycles per tile than the plain loop, but the chip's power
// limit then lowers the clock by about as much: the two run within 1% of each
// other on the same GPU.  The energy per tile -- LDS reads, VALU work, MFMA
// operand toggling -- is what sets this kernel's speed.)
//
//   iteration j:  stage A  S_{j+1} = K_{j+1} Q^T        (16 MFMAs at d=128)
//                          with the exponentials, bf16 packing and row sums
//                          of tile j woven in (exp2(x), x = c2*s - m, the
//                          exponent base already subtracted)
//                 [if some lane's sum of tile j's probabilities passed
//                  2^TAU: tile j's row max, new bases where a row grew by
//                  more than TAU, tile j's probabilities again, O and l
//                  *= alpha -- rare once the bases have settled]
//                 stage B  O^T += V_j^T P_j^T            (16 MFMAs at d=128)
//                          with x = c2*s - m for tile j+1 woven in, against
//                          the base in use (no row max: see Tile::SPEC)
//
// The order inside each stage (one MFMA, its LDS operand reads run three
// items ahead, then a fixed number of VALU and transcendental instructions)
// is pinned with sched_group_barrier.  Dependencies stay exact: tile j's
// exponentials use the base in use when its exponents were formed (stage B
// of iteration j-1); a base that moves for tile j moves before P_j V_j is
// added, with O and l rescaled first.  Tile 0's base is its row max.  Bases,
// probabilities and rescales are those of taking every tile's row max first
// under the lazy rule; the result is the same as fa_fwd_kernel's up to the
// order of floating-point additions.
//
// K/V stream: 64-key tiles through two-slot K and V rings in LDS
// (global_load_lds_dwordx4, XOR-swizzled as in fa_tile.hpp).  Iteration j
// reads K_{j+1} and V_j and fetches K_{j+2} and V_{j+1} into the slots that
// held K_j and V_{j-1}; one workgroup barrier per tile publishes them.  Under
// the causal mask tiles above the diagonal are never fetched, and each wave
// stops computing after its own last tile (it keeps fetching for the others).
#pragma once

#include <type_traits>

#include "fa_tile.hpp"

namespace fa {

// NI LDS-fed MFMA items with other work woven in, one fenced slot per item:
// slot i issues MFMA i, the operand reads of item i + DEPTH (so every read
// has DEPTH MFMAs to land) and work(i), a fixed slice of independent VALU
// work; sched_barrier(0) between slots keeps the scheduler from regrouping
// them.  (Left free, it chains MFMAs on one accumulator and moves each read
// next to its consumer, and clusters the slices' transcendentals.)
template <int I, int NI, int AHEAD, class Op, class Read, class Mma, class Work>
__device__ __forceinline__ void woven_slot(Op (&a)[AHEAD], Read& read, Mma& mma, Work& work) {
  if constexpr (I < NI) {
    mma(I, a[I % AHEAD]);
    if constexpr (I + AHEAD < NI) a[I % AHEAD] = read(I + AHEAD);
    work(std::integral_constant<int, I>{});
    __builtin_amdgcn_sched_barrier(0);
    woven_slot<I + 1, NI, AHEAD>(a, read, mma, work);
  }
}
template <int NI, int DEPTH, class Op, class Read, class Mma, class Work>
__device__ __forceinline__ void mfma_pipeline_woven(Read&& read, Mma&& mma, Work&& work) {
  constexpr int AHEAD = NI < DEPTH ? NI : DEPTH;
  Op a[AHEAD];
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) a[i] = read(i);
  woven_slot<0, NI, AHEAD>(a, read, mma, work);
}

template <int D, int BC, int NW>
struct PipeWave {
  using T = Tile<D, BC, NW, MODE_BF16>;
  static constexpr int KB = T::KB;                 // 32-key blocks per tile
  static constexpr int NDB = T::NDB;               // 32-wide blocks of d
  static constexpr int QK_NI = T::QK_STEPS * KB;   // MFMAs of S = K Q^T per tile
  static constexpr int PV_NI = T::PV_STEPS * NDB;  // MFMAs of O += P V per tile
  static constexpr int NS = 16 * KB;               // scores per lane per tile
  static constexpr float TAU = T::TAU;
  using Op = typename T::Op;

  // ---- stage A work: tile j's exponentials (x already holds c2*s - m), P_j
  // packed as the MFMA B operand, and this lane half's sum of the fp32
  // probabilities, in QK_NI slices of NS / 2 / QK_NI score pairs each (per
  // pair: two exponentials, one pack, two adds into two running sums)
  static constexpr int PAIRS_PER_SLOT = NS / 2 / QK_NI;
  static_assert(PAIRS_PER_SLOT * QK_NI * 2 == NS, "score pairs split evenly over the QK MFMAs");
  struct ProbState {
    float sum0, sum1;
  };
  static __device__ __forceinline__ void prob_pair(int pr, f32x16 (&x)[KB], typename T::PFrag& pf, ProbState& ps) {
    const int kb = pr / 8, i0 = 2 * (pr % 8);      // scores i0, i0 + 1 of block kb
    const float e0 = __builtin_amdgcn_exp2f(x[kb][i0]);
    const float e1 = __builtin_amdgcn_exp2f(x[kb][i0 + 1]);
    // score i of block kb is element 4 (g % 2) + i % 4 of key step 2 kb + g / 2, g = i / 4
    const int g = i0 / 4;
    pf.h[2 * kb + g / 2][2 * (g % 2) + (i0 % 4) / 2] = (int)pack_bf16x2(e0, e1);
    ps.sum0 = pr == 0 ? e0 : ps.sum0 + e0;
    ps.sum1 = pr == 0 ? e1 : ps.sum1 + e1;
  }
  template <int SL>
  static __device__ __forceinline__ void prob_slice(f32x16 (&x)[KB], typename T::PFrag& pf, ProbState& ps) {
#pragma unroll
    for (int k = 0; k < PAIRS_PER_SLOT; ++k) prob_pair(SL * PAIRS_PER_SLOT + k, x, pf, ps);
  }
  // the whole tile at once (outside the pipeline)
  static __device__ __forceinline__ void probs(f32x16 (&x)[KB], typename T::PFrag& pf, float& psum) {
    ProbState ps;
#pragma unroll
    for (int pr = 0; pr < NS / 2; ++pr) prob_pair(pr, x, pf, ps);
    psum = ps.sum0 + ps.sum1;
  }

  // Empty asm uses keep a stage's results in the stage's own block: without
  // them the compiler moves tile j's exponentials past the diagonal-mask
  // branch into stage B (sched_barrier does not stop pure arithmetic from
  // moving between blocks).
  static __device__ __forceinline__ void anchor_p(const typename T::PFrag& pf, float psum) {
    if constexpr (T::PV_STEPS == 4)
      asm volatile("" ::"v"(pf.h[0]), "v"(pf.h[1]), "v"(pf.h[2]), "v"(pf.h[3]), "v"(psum));
    else
      asm volatile("" ::"v"(pf.h[0]), "v"(pf.h[1]), "v"(psum));
  }
  static __device__ __forceinline__ void anchor_s(const f32x16 (&s)[KB]) {
    static_assert(KB == 2, "two 32-key blocks per tile");
    asm volatile("" ::"v"(s[0]), "v"(s[1]));
  }

  static __device__ __forceinline__ Op k_read(const char FA_LDS* kbase, int i, const typename T::Lane& ln) {
    return T::k_operand_pipe(kbase, i, ln);
  }
  static __device__ __forceinline__ Op v_read(const char FA_LDS* vbase, int i, const typename T::Lane& ln) {
    return T::v_operand_pipe(vbase, i, ln);
  }

  // stage A: nxt = K Q^T over the tile at kbase, with cur's probabilities woven in
  static __device__ __forceinline__ void stage_a(f32x16 (&nxt)[KB], const char FA_LDS* kbase,
                                                 const typename T::QFrag& q, const typename T::Lane& ln,
                                                 f32x16 (&cur)[KB], typename T::PFrag& pf, float& psum) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) nxt[kb] = f32x16{};
    ProbState ps;
    mfma_pipeline_woven<QK_NI, T::PDEPTH, Op>(
        [&](int i) __attribute__((always_inline)) { return k_read(kbase, i, ln); },
        [&](int i, const Op& a) __attribute__((always_inline)) { T::qk_mma(nxt, i / KB, i % KB, a, q); },
        [&](auto sl) __attribute__((always_inline)) { prob_slice<decltype(sl)::value>(cur, pf, ps); });
    psum = ps.sum0 + ps.sum1;
    anchor_p(pf, psum);
  }

  // stage B: O^T += V^T P^T over the tile at vbase, with nxt's exponents
  // x = c2 * s - m_run woven in (against the base in use: no row max)
  static constexpr int X_PER_SLOT = NS / PV_NI;
  static_assert(X_PER_SLOT * PV_NI == NS, "scores split evenly over the P V MFMAs");
  static __device__ __forceinline__ void stage_b(f32x16 (&oacc)[NDB], const char FA_LDS* vbase,
                                                 const typename T::PFrag& pf, const typename T::Lane& ln,
                                                 f32x16 (&nxt)[KB], float c2, float m_use) {
    mfma_pipeline_woven<PV_NI, T::PDEPTH, Op>(
        [&](int i) __attribute__((always_inline)) { return v_read(vbase, i, ln); },
        [&](int i, const Op& a) __attribute__((always_inline)) { T::pv_mma(oacc, i / NDB, i % NDB, a, pf); },
        [&](auto sl) __attribute__((always_inline)) {
          constexpr int v0 = decltype(sl)::value * X_PER_SLOT;
#pragma unroll
          for (int v = v0; v < v0 + X_PER_SLOT; ++v)
            nxt[v / 16][v % 16] = __builtin_fmaf(nxt[v / 16][v % 16], c2, -m_use);
        });
    anchor_s(nxt);
  }
};

template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_pipe_kernel(Params p) {
  using G = Geo<D, BC, NW, MODE_BF16>;
  using T = Tile<D, BC, NW, MODE_BF16>;
  using W = PipeWave<D, BC, NW>;
  constexpr int KB = W::KB, NDB = W::NDB;
  static_assert(G::KST == 2 && G::VST == 2, "two-slot K and V rings");
  const unsigned long long t_entry = timeline_clock();

  // K and V rings, then the Q tile (prologue); the O tile reuses the rings
  constexpr int QTILEB = G::BR * T::QROWB;
  __shared__ __attribute__((aligned(16))) char smem_raw[G::LDSB + QTILEB];
  char FA_LDS* const smem = (char FA_LDS*)(smem_raw);
  auto kslot = [&](int s) __attribute__((always_inline)) { return smem + s * G::SLOTB; };
  auto vslot = [&](int s) __attribute__((always_inline)) { return smem + (G::KST + s) * G::SLOTB; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const typename T::Lane ln = T::lane_info(lane);

  int bh, rb;
  map_block<CAUSAL>(p, blockIdx.x, bh, rb);
  const int N = p.N;
  const int64_t head_off = (int64_t)bh * N * D;
  const int64_t kv_off = (int64_t)(bh / p.G) * N * D;
  const int q_row0 = rb * G::BR;
  const int qw0 = q_row0 + 32 * wave;
  const int my_q = qw0 + ln.n;

  const int tiles_all = (N + BC - 1) / BC;
  const int n_tiles = CAUSAL ? min(tiles_all, (q_row0 + G::BR - 1) / BC + 1) : tiles_all;
  const int wave_tiles = CAUSAL ? min(tiles_all, (qw0 + 31) / BC + 1) : tiles_all;

  // the Q tile goes to LDS with the first K/V tiles (whole rows per DMA)
  char FA_LDS* const qtile = smem + G::LDSB;
  T::template dma_q<1 << 30>(static_cast<const char*>(p.q) + head_off * 2 + (int64_t)q_row0 * T::QROWB, N - q_row0, qtile,
                             qtile, wave, lane);

  Stager<D, BC, NW, MODE_BF16, false> kstage;
  Stager<D, BC, NW, MODE_BF16, true> vstage;
  kstage.init(wave, lane);
  vstage.init(wave, lane);
  const char* kglob = static_cast<const char*>(p.k) + kv_off * G::EB;
  const char* vglob = static_cast<const char*>(p.v) + kv_off * G::EB;

  f32x16 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = p.c2;
  const int last_key = (CAUSAL ? min(N - 1, my_q) : N - 1) - 4 * ln.hf;
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    const int key0 = j * BC;
    return (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qw0);
  };

  f32x16 sa[KB], sb[KB];        // score tiles j and j+1, alternating by the parity of j
  typename T::PFrag pf;

  // ---- prologue: K_0, V_0, K_1 in flight; S_0 and its exponents
  kstage.issue(kglob, 0, N, kslot(0), wave, lane);
  vstage.issue(vglob, 0, N, vslot(0), wave, lane);
  if (1 < n_tiles) kstage.issue(kglob, 1, N, kslot(1), wave, lane);
  wait_vmcnt<0>();
  __syncthreads();
  typename T::QFrag q;
  T::load_q_lds(qtile + wave * 32 * T::QROWB, ln, p.qsign, q);
  {
    T::qk(sa, kslot(0), q, ln);
    if (needs_mask(0)) T::mask(sa, last_key);
    // the first base is tile 0's row max (every row sees key 0, so it is
    // finite); O and l are still 0, so nothing is rescaled
    m_run = T::row_max(sa) * c2;
    T::to_exponents(sa, c2, m_run);
  }
  __syncthreads();                                // every wave is done with K_0's slot
  const unsigned long long t_pro = timeline_clock();

  // ---- main loop, unrolled by two so that ring slots and score buffers are fixed
  // iteration j: K_{j+1} in kslot((j+1)%2), V_j in vslot(j%2); fetch K_{j+2}
  // into kslot(j%2) and V_{j+1} into vslot((j+1)%2).  A wave computes while
  // j < wave_tiles and only fetches after that.  On its last tile (j + 1 =
  // wave_tiles) stage A still runs its QK^T, on whatever the K slot it reads
  // holds (no fetch writes that slot in this iteration), and the result is
  // thrown away: one code path keeps O in one set of registers.
  auto step = [&](int j, f32x16 (&cur)[KB], f32x16 (&nxt)[KB], const int par) __attribute__((always_inline)) {
    char FA_LDS* const k_use = kslot(par ^ 1);
    char FA_LDS* const v_use = vslot(par);
    if (j + 2 < n_tiles) kstage.issue(kglob, j + 2, N, kslot(par), wave, lane);
    if (j + 1 < n_tiles) vstage.issue(vglob, j + 1, N, vslot(par ^ 1), wave, lane);
    if (j < wave_tiles) {
      const bool real = j + 1 < wave_tiles;     // tile j+1 is one of this wave's tiles
      float psum;
      W::stage_a(nxt, k_use, q, ln, cur, pf, psum);
      // tile j's exponents were taken against the base in use without its
      // row max; a lane sum above 2^TAU (or a NaN) means some probability
      // passed 2^TAU: take the row max, move the bases that grew by more than
      // TAU, redo the tile's probabilities and rescale O and l (before P_j V_j)
      if (__builtin_amdgcn_ballot_w64(!(psum <= T::SPEC_LIMIT))) {
        asm volatile("" ::: "memory");   // a real (rarely taken) branch, not a select
        const float alpha = T::rebase(cur, m_run);
        W::probs(cur, pf, psum);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < NDB; ++b) oacc[b] *= alpha;
      }
      l_run += psum;
      if (real && needs_mask(j + 1)) T::mask(nxt, last_key - (j + 1) * BC);
      W::stage_b(oacc, v_use, pf, ln, nxt, c2, m_run);
    }
    wait_vmcnt<0>();      // K_{j+2} and V_{j+1} have landed
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    step(j, sa, sb, 0);
    step(j + 1, sb, sa, 1);
  }
  if (j < n_tiles) step(j, sa, sb, 0);

  const unsigned long long t_loop = timeline_clock();
  // the last step ended with a barrier: the rings are free for the O tile
  T::template store_lds<NDB>(p, head_off, bh, qw0, my_q, ln, oacc, m_run, l_run, smem + wave * 32 * T::QROWB, lane);
  timeline_record(t_entry, t_pro, t_loop, bh, rb);
}

}  // namespace fa
