// Split-KV attention for decode shapes on gfx950, and the logsumexp merge.
//
// What it computes: for N_q queries that are the last N_q positions of an
// N_k-key sequence (query i sees keys j <= N_k - N_q + i under the causal
// mask), O = softmax(scale * Q K^T) V and L = logsumexp, for grouped K/V
// heads.  The pages name sequence parallelism among FlashAttention-2's
// changes (systems-analysis.info "FlashAttention (PL)", section
// "FlashAttention-2 (2023)") and list decoding work (FlashDecoding++) in its
// literature; the split over keys with a logsumexp merge is that idea for a
// sequence too short in queries to fill the GPU.
//
// How:
//   1. fa_split_kernel (bf16, or fp8 with per-tensor descales: the forward's
//      fp8 pieces, e4m3 operands on the fp8 MFMA, P pre-scaled to e4m3):
//      a workgroup owns one key range (a split) of one K/V
//      head and up to 32*NW of its rows, a row being (query head of the
//      group, query): decode has G * N_q rows per K/V head, so the query
//      heads that share a K/V stream share one pass over it.  The range's
//      K/V tiles stream through an LDS ring with the forward's staging and
//      per-wave pieces (S^T = K Q^T, online softmax, O^T += V^T P^T); the
//      workgroup writes its partial O_s (normalised over its range, fp32)
//      and L_s.  A row that sees no key of the range writes O_s = 0,
//      L_s = -inf.
//   2. fa_merge_kernel: L = logsumexp_s L_s and O = sum_s exp(L_s - L) O_s per
//      row, one wave per row.
#pragma once

#include "fa_tile.hpp"

namespace fa {

struct SplitParams {
  const void* q;      // bf16 or e4m3 [B][H][N_q][D]
  const void* k;      // bf16 or e4m3 [B][H_kv][N_k][D]
  const void* v;
  float* o_part;      // [S][B*H*N_q][D]
  float* lse_part;    // [S][B*H*N_q]
  int BHkv;           // B * H_kv
  int G;              // query heads per K/V head
  int N_q, N_k;
  int rows;           // G * N_q rows per K/V head
  int nrb;            // row blocks per K/V head
  int S;              // splits
  int chunk;          // keys per split, a multiple of the tile
  float c2;           // |scale| * log2(e) (fp8: times the q and k descales)
  uint32_t qsign;     // XOR mask on Q's sign bits (negative scale)
  float out_mul;      // fp8: the v descale (unused for bf16)
};

// Wait until the oldest tile in flight has landed, `more` being how many
// tiles after it are still to be waited for (at most NS - 2 of them are in
// flight behind it; loads complete in issue order).
template <int NS, int LOADS>
__device__ __forceinline__ void wait_tile(int more) {
  if constexpr (NS >= 4) {
    if (more >= 2) { wait_vmcnt<(NS >= 4 ? 2 : 0) * LOADS>(); return; }
  }
  if constexpr (NS >= 3) {
    if (more >= 1) { wait_vmcnt<(NS >= 3 ? 1 : 0) * LOADS>(); return; }
  }
  wait_vmcnt<0>();
}

// NS: depth of the K/V ring (tiles j+1 .. j+NS-1 in flight while tile j is used).
template <int D, int BC, int NW, int NS, bool CAUSAL, int MODE = MODE_BF16>
__global__ __launch_bounds__(NW * 64) void fa_split_kernel(SplitParams p) {
  static_assert(MODE == MODE_BF16 || MODE == MODE_FP8, "bf16 or fp8 inputs");
  using G = Geo<D, BC, NW, MODE>;
  using T = Tile<D, BC, NW, MODE>;
  constexpr int NDB = T::NDB;
  constexpr int SLOT = 2 * G::SLOTB;                      // K tile then V tile
  constexpr int LOADS = 2 * G::UPT;                       // DMA instructions per tile per wave
  static_assert(NS >= 2 && NS * SLOT <= 160 * 1024, "LDS budget");
  static_assert((NS - 2) * LOADS <= 63, "outstanding loads fit the wait counter");

  __shared__ __attribute__((aligned(16))) char smem_raw[NS * SLOT];
  char FA_LDS* const smem = (char FA_LDS*)(smem_raw);
  auto kslot = [&](int s) __attribute__((always_inline)) { return smem + s * SLOT; };
  auto vslot = [&](int s) __attribute__((always_inline)) { return smem + s * SLOT + G::SLOTB; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const typename T::Lane ln = T::lane_info(lane);

  const int id = blockIdx.x;
  const int s = id % p.S;
  const int rb = (id / p.S) % p.nrb;
  const int bhk = id / (p.S * p.nrb);
  const int N_k = p.N_k;
  const int64_t kv_off = (int64_t)bhk * N_k * D;

  // this lane's row: (query head hh of the group, query i)
  const int r = rb * G::BR + 32 * wave + ln.n;
  const bool row_ok = r < p.rows;
  const int hh = row_ok ? r / p.N_q : 0, qi = row_ok ? r - hh * p.N_q : 0;
  const int64_t row_g = (int64_t)bhk * p.rows + r;              // = (bhk*G + hh)*N_q + qi
  // the row's Q slice as the B operand (bf16: dims 16c + 8hf .. +7 of step c;
  // fp8: bytes 64c + 32hf .. +31)
  typename T::QFrag q;
  {
    const int sgn = (int)p.qsign;
    const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const char*>(p.q) + row_g * G::ROWB);
    const i32x4 sg{sgn, sgn, sgn, sgn}, zero{0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < T::QK_STEPS; ++c) {
      if constexpr (MODE == MODE_FP8) {
        const i32x4 w0 = (row_ok ? src[4 * c + 2 * ln.hf] : zero) ^ sg;
        const i32x4 w1 = (row_ok ? src[4 * c + 2 * ln.hf + 1] : zero) ^ sg;
        q.f8[c] = i32x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      } else {
        q.a[c] = __builtin_bit_cast(bf16x8, (row_ok ? src[2 * c + ln.hf] : zero) ^ sg);
      }
    }
  }

  // key range of this split, and the last key this lane's row sees
  const int k_lo = s * p.chunk, k_hi = min(N_k, k_lo + p.chunk);
  const int row_last = CAUSAL ? N_k - p.N_q + qi : N_k - 1;
  const int last_key = min(row_last, k_hi - 1) - 4 * ln.hf;
  const int j0 = k_lo / BC, j1 = (k_hi + BC - 1) / BC;
  const int first_row_last = CAUSAL ? N_k - p.N_q : N_k - 1;   // the smallest limit of any row

  // each K/V byte is read by this workgroup alone: streaming loads
  Stager<D, BC, NW, MODE, false, true> kstage;
  Stager<D, BC, NW, MODE, true, true> vstage;
  kstage.init(wave, lane);
  vstage.init(wave, lane);
  const char* kglob = static_cast<const char*>(p.k) + kv_off * G::EB;
  const char* vglob = static_cast<const char*>(p.v) + kv_off * G::EB;

  f32x16 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.c2;
  typename T::PFrag pf;

  // Tile t of the range is tile j0 + (t + rot) % nt: every workgroup starts at
  // a different place in its range, so that workgroups whose ranges lie a
  // power of two apart do not stream the same HBM channels in lock step.  The
  // online softmax does not depend on the order of the tiles beyond rounding.
  const int nt = j1 - j0;
  const int rot = nt > 0 ? (s + bhk) % nt : 0;
  auto tile_of = [&](int t) __attribute__((always_inline)) {
    const int u = t + rot;
    return j0 + (u >= nt ? u - nt : u);
  };

  // prologue: tiles 0 .. NS-2 of the range in flight, the first one landed
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nt) {
      kstage.issue(kglob, tile_of(t), N_k, kslot(t), wave, lane);
      vstage.issue(vglob, tile_of(t), N_k, vslot(t), wave, lane);
    }
  wait_tile<NS, LOADS>(nt - 1);
  __syncthreads();
  int cur = 0;
  for (int t = 0; t < nt; ++t) {
    // refill the slot tile t-1 used (its readers passed the last barrier)
    if (t + NS - 1 < nt) {
      const int slot = cur == 0 ? NS - 1 : cur - 1;
      kstage.issue(kglob, tile_of(t + NS - 1), N_k, kslot(slot), wave, lane);
      vstage.issue(vglob, tile_of(t + NS - 1), N_k, vslot(slot), wave, lane);
    }
    {
      f32x16 st[T::KB];
      T::qk(st, kslot(cur), q, ln);
      const int key0 = tile_of(t) * BC;
      if ((key0 + BC > k_hi) || (CAUSAL && key0 + BC - 1 > first_row_last)) T::mask(st, last_key - key0);
      typename T::Softmax sm;
      T::template softmax_slices<0, T::NMAX + 1>(st, sm, m_run, c2, pf);
      if (__builtin_amdgcn_ballot_w64(sm.grow)) {
        asm volatile("" ::: "memory");
        l_run *= sm.alpha;
#pragma unroll
        for (int b = 0; b < NDB; ++b) oacc[b] *= sm.alpha;
      }
      T::template softmax_slices<T::NMAX + 1, T::NSLICES>(st, sm, m_run, c2, pf);
      l_run += sm.psum[0] + sm.psum[1];
      T::pv(oacc, vslot(cur), pf, ln);
    }
    wait_tile<NS, LOADS>(nt - t - 2);                     // tile t+1 has landed
    __syncthreads();
    cur = cur + 1 == NS ? 0 : cur + 1;
  }

  const float l_tot = swap_halves_sum(l_run);
  if (!row_ok) return;
  const int64_t prow = (int64_t)s * p.BHkv * p.rows + row_g;   // row of this split's partial
  const bool seen = l_tot > 0.f;
  // fp8: l and O carry the pre-scale 2^EXP_SHIFT of P, which cancels in O / l
  // and leaves L through the base
  const float inv = seen ? (MODE == MODE_FP8 ? p.out_mul : 1.f) / l_tot : 0.f;
  if (ln.hf == 0) p.lse_part[prow] = seen ? (m_run - T::EXP_SHIFT + __log2f(l_tot)) * kLn2 : -INFINITY;
  float* dst = p.o_part + prow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * db + 8 * g + 4 * ln.hf;
      *reinterpret_cast<f32x4*>(dst + col) = f32x4{oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                                   oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
    }
}

struct MergeParams {
  const float* o_part;   // [S][rows][d]
  const float* lse_part; // [S][rows]
  void* o;               // [rows][d], bf16 or fp32
  float* lse;            // [rows]
  int64_t rows;
  int S, d;
  int out_bf16;
};

// One wave per row.  The splits' L_s are read all at once (lane s holds split
// s, 64 splits per pass) and reduced across the wave; O column c = lane + 64 j
// sums exp(L_s - max) O_s over the splits in order, with the O_s loads issued
// eight at a time (a loop that waited for each load in turn made the merge a
// chain of 4 S + d/64 * S load latencies).
__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
// a butterfly: every lane adds the same two values at every step, so all
// lanes end with the same sum
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(256) void fa_merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;                       // the whole wave: one row per wave
  const int S = p.S;
  auto lse_of = [&](int s) __attribute__((always_inline)) { return p.lse_part[(int64_t)s * p.rows + row]; };
  const float l_lane = lane < S ? lse_of(lane) : -INFINITY;   // splits 0..63, kept
  float m = l_lane;
  for (int s0 = 64; s0 < S; s0 += 64) m = fmaxf(m, s0 + lane < S ? lse_of(s0 + lane) : -INFINITY);
  m = wave_max64(m);
  const float m_use = m == -INFINITY ? 0.f : m;
  const float w_lane = __expf(l_lane - m_use);                 // the weight of split `lane` (0 past S)
  float part = w_lane;
  for (int s0 = 64; s0 < S; s0 += 64) part += s0 + lane < S ? __expf(lse_of(s0 + lane) - m_use) : 0.f;
  const float tot = wave_sum64(part);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (lane == 0) p.lse[row] = tot > 0.f ? m_use + __logf(tot) : -INFINITY;
  const int64_t stride = (int64_t)p.rows * p.d;   // between splits
  auto columns = [&](auto weight) __attribute__((always_inline)) {
    for (int c = lane; c < p.d; c += 64) {
      const float* src = p.o_part + row * p.d + c;
      float acc = 0.f;
      int s = 0;
      for (; s + 8 <= S; s += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[(s + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = __builtin_fmaf(weight(s + u), v[u], acc);
      }
      for (; s < S; ++s) acc = __builtin_fmaf(weight(s), src[s * stride], acc);
      const float x = acc * inv;
      if (p.out_bf16) {
        static_cast<uint16_t*>(p.o)[row * p.d + c] = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
      } else {
        static_cast<float*>(p.o)[row * p.d + c] = x;
      }
    }
  };
  // the weight of split s: lane s's w_lane (at most 64 splits), else formed again
  if (S <= 64)
    columns([&](int s) __attribute__((always_inline)) {
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), s));
    });
  else
    columns([&](int s) __attribute__((always_inline)) { return __expf(lse_of(s) - m_use); });
}

}  // namespace fa
