// FlashAttention forward for small heads with 16 queries per wave (bf16).
//
// Same operation and online softmax as fa_fwd_kernel (see there), laid out
// on v_mfma_f32_16x16x32_bf16 so that a wave owns 16 query rows instead of
// 32: at d = 64 the softmax arithmetic per score is as large as the matrix
// work, and twice the waves per SIMD give the scheduler twice the chance to
// overlap one wave's exponentials with another's MFMAs.
//
// Lane = 16*g + m.  S^T = K Q^T in 16-key x 16-query blocks: lane holds query
// m, element j of block kb is key 16*kb + 4g + j.  The row statistics reduce
// over the lane's own elements and then across the four lane groups g.  P^T
// feeds O^T += V^T P^T straight from the accumulators (k-slot (g, i) of a
// 32-key step is key 16*(i/4) + 4g + i%4), with V^T read by the LDS
// transpose loads.  K and V tiles use the swz16 swizzle (row reads of 16 rows
// at one chunk for K, transposed reads of 8 rows x 2 chunks for V).
#pragma once

#include "fa_bwd_kernel.hpp"

namespace fa {

// x reduced over the four lanes 16 apart that hold one query
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(a[0]) + __int_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fa_fwd16_kernel(Params p) {
  constexpr int BR = 16 * NW;
  constexpr int ROWB = 2 * D, CPR = ROWB / 16;
  constexpr int TILEB = BC * ROWB;
  constexpr int STAGEB = 2 * TILEB;          // K tile, V tile
  constexpr int NC = D / 32;                 // 32-dim k-steps of S
  constexpr int KB = BC / 16;                // 16-key blocks per tile
  constexpr int NS = BC / 32;                // 32-key k-steps of P V
  constexpr int NDB = D / 16;                // 16-dim blocks of O
  constexpr float TAU = 8.f;
  static_assert(2 * STAGEB <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * STAGEB];
  char FA_LDS* const smem = (char FA_LDS*)(smem_raw);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;

  int bh, rb;
  map_block<CAUSAL>(p, blockIdx.x, bh, rb);
  const int N = p.N;
  const int64_t head_off = (int64_t)bh * N * D;
  const int64_t kv_off = (int64_t)(bh / p.G) * N * D;
  const int q_row0 = rb * BR, qw0 = q_row0 + 16 * wave, my_q = qw0 + m;

  // Q rows as B operands: step c holds dims 32c + 8g .. +7 of query my_q
  bf16x8 qf[NC];
  {
    const bool ok = my_q < N;
    const int sgn = (int)p.qsign;
    const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.q) + head_off + (int64_t)my_q * D);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      i32x4 w = ok ? src[4 * c + g] : i32x4{0, 0, 0, 0};
      w ^= i32x4{sgn, sgn, sgn, sgn};
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int tiles_all = (N + BC - 1) / BC;
  const int n_tiles = CAUSAL ? min(tiles_all, (q_row0 + BR - 1) / BC + 1) : tiles_all;
  const int wave_tiles = CAUSAL ? min(tiles_all, (qw0 + 15) / BC + 1) : tiles_all;
  const int last_key = (CAUSAL ? min(N - 1, my_q) : N - 1) - 4 * g;

  Stager16<D, BC, NW> stage;
  const char* kglob = static_cast<const char*>(p.k) + kv_off * 2;
  const char* vglob = static_cast<const char*>(p.v) + kv_off * 2;
  auto slot = [&](int s) __attribute__((always_inline)) { return smem + s * STAGEB; };
  auto issue = [&](int j, char FA_LDS* dst) __attribute__((always_inline)) {
    stage.issue(kglob, j * BC, N, dst, wave, lane);
    stage.issue(vglob, j * BC, N, dst + TILEB, wave, lane);
  };
  auto row_a = [&](const char FA_LDS* base, int kb, int c) __attribute__((always_inline)) {
    const int row = 16 * kb + m;
    return __builtin_bit_cast(bf16x8, lds_read16(base + row * ROWB + (((4 * c + g) ^ swz16<CPR>(row)) << 4)));
  };
  auto tr_a = [&](const char FA_LDS* base, int s, int db) __attribute__((always_inline)) {
    const int row = 32 * s + 4 * g + ((lane >> 2) & 3);
    const int col = 32 * db + 8 * (lane & 3);
    const int off0 = row * ROWB + ((((col >> 4) ^ swz16<CPR>(row)) << 4) | (col & 15));
    const int off1 = (row + 16) * ROWB + ((((col >> 4) ^ swz16<CPR>(row + 16)) << 4) | (col & 15));
    const i16x4 lo = lds_tr16(base + off0), hi = lds_tr16(base + off1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x4 oacc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) oacc[b] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.c2;

  auto tile = [&](int j, const char FA_LDS* ks) __attribute__((always_inline)) {
    const char FA_LDS* vs = ks + TILEB;
    f32x4 st[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) st[kb] = f32x4{};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) st[kb] = mfma16(row_a(ks, kb, c), qf[c], st[kb]);
    const int key0 = j * BC;
    if ((key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qw0)) {
      asm volatile("" ::: "memory");
      const int lim = last_key - key0;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[kb][e] = (16 * kb + e) > lim ? -INFINITY : st[kb][e];
    }
    float mx = st[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = __builtin_elementwise_maximum(mx, st[kb][e]);
    const float m_tile = quad_max(mx) * c2;
    const bool grow = m_tile > m_run + TAU;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      asm volatile("" ::: "memory");
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b) oacc[b] *= alpha;
      m_run = grow ? m_tile : m_run;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    i32x4 pp[NS];
    float ps = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[2 * s + h][e], c2, -m_use));
        ps += (x[0] + x[1]) + (x[2] + x[3]);
        pp[s][2 * h] = (int)pack_bf16x2(x[0], x[1]);
        pp[s][2 * h + 1] = (int)pack_bf16x2(x[2], x[3]);
      }
    l_run += ps;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma16(tr_a(vs, s, db), __builtin_bit_cast(bf16x8, pp[s]), oacc[db]);
  };

  issue(0, slot(0));
  wait_vmcnt<0>();
  __syncthreads();
  int cur = 0;
  for (int j = 0; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) issue(j + 1, slot(cur ^ 1));
    if (j < wave_tiles) tile(j, slot(cur));
    wait_vmcnt<0>();
    __syncthreads();
    cur ^= 1;
  }

  const float l_tot = quad_sum(l_run);
  if (my_q >= N) return;
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.f / l_tot : 0.f;
  if (g == 0) p.lse[(int64_t)bh * N + my_q] = seen ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  uint16_t* dst = static_cast<uint16_t*>(p.o) + head_off + (int64_t)my_q * D + 4 * g;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<i32x2*>(dst + 16 * db) =
        i32x2{(int)pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv), (int)pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv)};
}

}  // namespace fa
