// FlashAttention backward for gfx950 (CDNA4): gradients by recomputation.
//
// What it computes (per batch b, query head h, K/V head g = h / G): for the
// loss sum(dO * O) of the forward O = softmax(scale * Q K^T) V,
//     P  = exp(scale * Q K^T - L)          (L: the forward's per-row logsumexp)
//     dV = P^T dO                          (summed over the G query heads of g)
//     dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D)
//     dQ = scale * dS K,  dK = scale * dS^T Q   (dK summed like dV)
// The robocikowo.com "Flash Attention" page says the backward pass does not
// store the N x N matrix but rebuilds it from O and L; the formulas above are
// the chain rule of the forward definition (systems-analysis.info
// "FlashAttention (PL)", "Problematyka standardowego mechanizmu uwagi").
//
// How (two launches, no atomics, bitwise reproducible):
//   1. statistics: D = rowsum(dO * O) and L2 = L * log2(e) per query, written
//      to a caller workspace in 64-query tiles [L2 x 64][D x 64]; rows past N
//      get L2 = +inf and D = 0, so their P is exactly 0 downstream.  The dQ
//      kernel (3.) forms them for its own rows as it starts, and runs first.
//   2. dK/dV: a workgroup owns 32*NW keys of one K/V head; each wave keeps its
//      32 keys' K and V rows in VGPRs (MFMA B operands) and its dK^T, dV^T
//      accumulators in VGPRs, and streams the Q and dO tiles of all G query
//      heads through a double-buffered LDS ring.  Per 32-query block:
//        S = Q K^T and dP = dO V^T  (lane = key, elements over queries),
//        P and dS in fp32, packed to bf16 straight from the accumulators,
//        dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read by the LDS
//        transpose loads (ds_read_b64_tr_b16).
//      Under the causal mask the query tiles before the key block are never
//      loaded; key blocks are dispatched earliest (heaviest) first.
//   3. dQ: a workgroup owns 32*NW queries; each wave keeps Q and dO in
//      VGPRs and streams K and V tiles, as the forward does:
//        S^T = K Q^T and dP^T = V dO^T (lane = query),
//        dQ^T += K^T dS^T with K^T read by the transpose loads.
//   Tiles that are read both row-wise (ds_read_b128) and transposed share one
//   XOR swizzle of the 16-byte chunk index that keeps both access patterns
//   free of LDS bank conflicts (swz_u below).
//
// Inputs are bf16; the three gradients are written as fp32.
#pragma once

#include "fa_common.hpp"

namespace fa {

struct BwdParams {
  const void* q;       // bf16 [B][H][N][D]
  const void* k;       // bf16 [B][H_kv][N][D]
  const void* v;
  const void* o;       // bf16 [B][H][N][D] (the forward's output)
  const void* dout;    // bf16 [B][H][N][D]
  const float* lse;    // [B][H][N], natural log
  float* ws;           // [B*H][T][2][64]: L2 then D per 64-query tile
  float* dq;           // fp32 [B][H][N][D]
  float* dk;           // fp32 [B][H_kv][N][D]
  float* dv;
  int BH;              // heads of this launch's grid (B*H for dQ, B*H_kv times the parts for dK/dV)
  int N;
  int nrb;             // row blocks per head in this launch's grid
  int G;               // grid mapping: query heads grouped per XCD (dQ: H/H_kv; dK/dV: 1)
  int qg;              // query heads per K/V head
  int xcd_heads;
  int cus_per_xcd;
  int zigzag;
  int T;               // 64-query statistics tiles per head (ceil(N / 64))
  float c2;            // scale * log2(e), signed
  float scale;
  // dK/dV with the query heads of a group split over `parts` workgroups per
  // key block: part hp takes heads hp, hp + parts, ... and writes its share
  // of dK and dV to part_out ([2][parts][B*H_kv][N][D], dK first); a reduction
  // sums the parts.  parts = 1 writes dk and dv directly.
  int parts;
  float* part_out;
};

constexpr int kStatRows = 64;   // queries per statistics tile

// vmcnt(0), written as inline asm (ordered with the DMA asm around it) and
// again as the builtin, which the compiler's own wait insertion sees: it
// does not see waits in inline asm, so registers loaded before a loop would
// otherwise get a fresh vmcnt(0) at their first use inside it, one that also
// waits for the prefetch DMA in flight.  Builtin immediate (gfx9 encoding):
// vmcnt 0, expcnt 7 and lgkmcnt 15 (no wait on those).
__device__ __forceinline__ void wait_vmcnt0_seen() {
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Chunk swizzle for tiles read both row-wise (16 lanes x 16 rows at one
// logical chunk, ds_read_b128) and transposed (32 lanes x 4 rows x 4 adjacent
// chunks, ds_read_b64_tr_b16).  With RPP rows per 256-byte bank span and
// rr = row / RPP, the chunk is XORed with 4 * (rr % (CPR/4)) + (rr / (CPR/4)) % 4:
// the low field differs across any 4 consecutive rows of one bank phase (no
// two transposed rows collide in a group of 4 chunks) and the whole value
// is a bijection on 16 consecutive rows of one phase (row reads collide never).
// Rows of 512 bytes (d = 256) span two bank spans; the XOR then acts on the
// 16 chunk positions of one span exactly as for 256-byte rows.
template <int CPR>
__device__ __forceinline__ int swz_u(int row) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "tile rows of 128, 256 or 512 bytes");
  constexpr int RPP = CPR >= 16 ? 1 : 16 / CPR;
  constexpr int A = CPR >= 16 ? 4 : CPR / 4;
  const int rr = row / RPP;
  return 4 * (rr % A) + (rr / A) % 4;
}

// Per-lane geometry of the operand reads (lane = 32*hf + n).
struct BwdLane {
  int n, hf;
  int t_row, t_col;   // transpose reads: row within a 16-row step, byte column within a 64-byte block
};
__device__ __forceinline__ BwdLane bwd_lane(int lane) {
  BwdLane ln;
  ln.n = lane & 31;
  ln.hf = lane >> 5;
  ln.t_row = 4 * ln.hf + ((lane >> 2) & 3);
  ln.t_col = 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  return ln;
}

// A operand rows 32*blk + n of a swizzled bf16 tile, d-step c (dims 16c + 8hf .. +7).
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char FA_LDS* base, int blk, int c, const BwdLane& ln) {
  constexpr int ROWB = 2 * D, CPR = ROWB / 16;
  const int row = 32 * blk + ln.n;
  return __builtin_bit_cast(bf16x8, lds_read16(base + row * ROWB + (((2 * c + ln.hf) ^ swz_u<CPR>(row)) << 4)));
}
// A operand X^T (dims 32*db .. +31 as rows) over tile rows
// 16*s + 8*(i/4) + 4*hf + i%4 of a swizzled bf16 tile (transpose reads).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char FA_LDS* base, int s, int db, const BwdLane& ln) {
  constexpr int ROWB = 2 * D, CPR = ROWB / 16;
  const int row = 16 * s + ln.t_row;
  const int col = 64 * db + ln.t_col;   // bytes
  const int off0 = row * ROWB + ((((col >> 4) ^ swz_u<CPR>(row)) << 4) | (col & 15));
  const int off1 = (row + 8) * ROWB + ((((col >> 4) ^ swz_u<CPR>(row + 8)) << 4) | (col & 15));
  const i16x4 lo = lds_tr16(base + off0), hi = lds_tr16(base + off1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 32 rows x D of a bf16 head (row r0 + n; zeros past N) as MFMA B operand
// fragments: step c holds dims 16c + 8hf .. +7.
template <int D>
__device__ __forceinline__ void load_frag(const void* base, int64_t head_off, int row, int N, const BwdLane& ln,
                                          bf16x8 (&f)[D / 16]) {
  const bool ok = row < N;
  const i32x4* src = reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(base) + head_off + (int64_t)row * D);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) f[c] = __builtin_bit_cast(bf16x8, ok ? src[2 * c + ln.hf] : i32x4{0, 0, 0, 0});
}

// HBM -> LDS staging of a ROWS x D bf16 tile with the swz_u swizzle, by all NW
// waves.  Rows past N re-read row N-1 (their contributions are zeroed by the
// caller's statistics or mask).
template <int D, int ROWS, int NW>
struct UStager {
  static constexpr int ROWB = 2 * D, CPR = ROWB / 16;
  static constexpr int UNITS = ROWS * ROWB / 16;
  static constexpr int UPT = UNITS / (NW * 64);
  static_assert(UNITS % (NW * 64) == 0, "tile splits evenly over the waves");
  int ofs[UPT];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int off = (i * NW + wave) * 1024 + lane * 16;
      const int row = off / ROWB, pc = (off % ROWB) >> 4;
      ofs[i] = row * ROWB + ((pc ^ swz_u<CPR>(row)) << 4);
    }
  }
  // rows row0 .. row0+ROWS-1 of the head at glob (bytes) -> LDS at dst
  __device__ __forceinline__ void issue(const char* glob, int row0, int N, char FA_LDS* dst, int wave, int lane) const {
    const char* base = glob + (int64_t)row0 * ROWB;
    if (row0 + ROWS <= N) {
#pragma unroll
      for (int i = 0; i < UPT; ++i) dma16_s(base, ofs[i], dst + (i * NW + wave) * 1024);
    } else {
      const int last = N - 1 - row0;
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int off = (i * NW + wave) * 1024 + lane * 16;
        const int row = off / ROWB, pc = (off % ROWB) >> 4;
        dma16_s(base, min(row, last) * ROWB + ((pc ^ swz_u<CPR>(row)) << 4), dst + (i * NW + wave) * 1024);
      }
    }
  }
};

// ---------------------------------------------------------------- 2. dK / dV
// v_mfma_f32_16x16x32_bf16 on a wave64, lane = 16*g + m:
//   A (16 x 32): lane holds row m, k-slots 8g .. 8g+7
//   B (32 x 16): lane holds column m, the same k-slots
//   C (16 x 16): lane holds column m, rows 4g .. 4g+3
// S and dP are 16-query x 16-key blocks with the key in the lane (column)
// and the queries along the elements, so P and dS feed dV^T += dO^T P and
// dK^T += Q^T dS as B operands straight from the accumulators: k-slot
// (g, i) of a 32-query step is query 16*(i/4) + 4g + i%4 of that step, and
// the matching dO^T / Q^T operand is two transpose reads of rows 4g .. 4g+3
// and 16 + 4g .. 16 + 4g+3.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Chunk swizzle of the tiles the dK/dV kernel reads row-wise (16 rows at one
// logical chunk) and transposed (8 consecutive rows x 2 adjacent chunks per
// 32 lanes): with rr = row / RPP, XOR with 2 * (rr % (CPR/2)) + (rr / (CPR/2)) % 2,
// a bijection on 16 consecutive rows of one bank phase whose upper bits
// differ across 8 consecutive rows (4 per phase when two rows share a span;
// 512-byte rows XOR within the 16 positions of one span, as 256-byte rows do).
template <int CPR>
__device__ __forceinline__ int swz16(int row) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "tile rows of 128, 256 or 512 bytes");
  constexpr int RPP = CPR >= 16 ? 1 : 16 / CPR;
  constexpr int A = CPR >= 16 ? 8 : CPR / 2;
  const int rr = row / RPP;
  return 2 * (rr % A) + (rr / A) % 2;
}

// HBM -> LDS staging of ROWS x D bf16 rows with swz16, by all NW waves
// (rows past N re-read row N-1).
template <int D, int ROWS, int NW>
struct Stager16 {
  static constexpr int ROWB = 2 * D, CPR = ROWB / 16;
  static constexpr int UNITS = ROWS * ROWB / 16;
  static constexpr int UPT = UNITS / (NW * 64);
  static_assert(UNITS % (NW * 64) == 0, "tile splits evenly over the waves");
  __device__ __forceinline__ void issue(const char* glob, int row0, int N, char FA_LDS* dst, int wave, int lane) const {
    const char* base = glob + (int64_t)row0 * ROWB;
    const int last = N - 1 - row0;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int off = (i * NW + wave) * 1024 + lane * 16;
      const int row = off / ROWB, pc = (off % ROWB) >> 4;
      dma16_s(base, min(row, last) * ROWB + ((pc ^ swz16<CPR>(row)) << 4), dst + (i * NW + wave) * 1024);
    }
  }
};

// A workgroup owns BK = KW*NW keys of one K/V head; wave w owns keys
// KW*w .. KW*w + KW-1 as KW/16 blocks of 16 keys (KW = 32, or 16 at d = 256
// to halve the registers K, V and the accumulators take).  K stays in VGPRs
// as B operands; V (VLDS) is staged once into LDS and read as B operands, or
// kept in VGPRs.
template <int D, int NW, int WPE, bool CAUSAL, bool VLDS, int KW = 32>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void fa_bwd_dkdv_kernel(BwdParams p) {
  static_assert(KW == 16 || KW == 32, "one or two 16-key blocks per wave");
  constexpr int KBW = KW / 16;              // 16-key blocks per wave
  constexpr int BQ = kStatRows;             // queries per tile
  constexpr int BK = KW * NW;               // keys per workgroup
  constexpr int ROWB = 2 * D, CPR = ROWB / 16;
  constexpr int TILEB = BQ * ROWB;
  constexpr int STATB = 1024;               // L2 and D of the tile (512 B), then a copy
  constexpr int STAGEB = 2 * TILEB + STATB;
  constexpr int VBYTES = VLDS ? BK * ROWB : 0;
  constexpr int NC = D / 32;                // 32-dim k-steps of S and dP
  constexpr int NDB = D / 16;               // 16-dim blocks of dK^T and dV^T
  static_assert(2 * STAGEB + VBYTES <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * STAGEB + (VLDS ? VBYTES : 16)];
  char FA_LDS* const smem = (char FA_LDS*)(smem_raw);
  char FA_LDS* const vsm = smem + 2 * STAGEB;

  // wave index in an SGPR, so that LDS and DMA addresses stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;

  int vh, rb;
  map_block<CAUSAL>(p, blockIdx.x, vh, rb);   // vh: (K/V head, part of its query heads)
  const int bhk = vh / p.parts, hp = vh - bhk * p.parts;
  const int kblk = p.nrb - 1 - rb;          // causal: earliest key blocks (most query tiles) first
  const int N = p.N;
  const int k0 = kblk * BK, kw0 = k0 + KW * wave;
  const int64_t kv_off = (int64_t)bhk * N * D;

  // K (and V) rows kw0 + 16*kb + m: chunk 4c + g of each row (zeros past N)
  bf16x8 kf[KBW][NC], vf[KBW][VLDS ? 1 : NC];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    const int key = kw0 + 16 * kb + m;
    const bool ok = key < N;
    const i32x4* ks = reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.k) + kv_off + (int64_t)key * D);
    const i32x4* vs = reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.v) + kv_off + (int64_t)key * D);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[kb][c] = __builtin_bit_cast(bf16x8, ok ? ks[4 * c + g] : i32x4{0, 0, 0, 0});
      if constexpr (!VLDS) vf[kb][c] = __builtin_bit_cast(bf16x8, ok ? vs[4 * c + g] : i32x4{0, 0, 0, 0});
    }
  }

  f32x4 dk[KBW][NDB], dv[KBW][NDB];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
    for (int b = 0; b < NDB; ++b) dk[kb][b] = dv[kb][b] = f32x4{};

  const int T = p.T;
  const int t0 = CAUSAL ? k0 / BQ : 0;      // earlier query tiles see none of these keys
  const int nt = T - t0;
  const int nh = (p.qg - hp + p.parts - 1) / p.parts;   // query heads of this part
  const int n_iter = nh * nt;               // (query head, query tile) pairs

  Stager16<D, BQ, NW> stage;
  auto issue = [&](int it, char FA_LDS* dst) __attribute__((always_inline)) {
    const int ih = it / nt, t = t0 + it - ih * nt;
    const int64_t bhq = (int64_t)bhk * p.qg + hp + (int64_t)ih * p.parts;
    stage.issue(static_cast<const char*>(p.q) + bhq * N * ROWB, t * BQ, N, dst, wave, lane);
    stage.issue(static_cast<const char*>(p.dout) + bhq * N * ROWB, t * BQ, N, dst + TILEB, wave, lane);
    if (wave == 0)
      dma16_s(reinterpret_cast<const char*>(p.ws + (bhq * T + t) * (2 * kStatRows)), 16 * (lane & 31), dst + 2 * TILEB);
  };

  // Per-lane LDS offsets of the operand reads.  swz16 depends on row % 16
  // only, and the chunk bits a read varies (4c in chunk 4c + g, 2db in chunk
  // 2db + (lane & 3) / 2) are disjoint from the lane's own, so every offset
  // is a lane base XOR a chunk term plus a constant row offset:
  //   row_a, v_b: ra ^ (c << 6) + 16 * ROWB * (row block)
  //   tr_a:       ta ^ (db << 5) + ROWB * (32 s, + 16 for the upper rows)
  // The bases are re-laundered per tile (at its top), so the XORs are formed
  // where they are used rather than kept live across the loop, where they
  // spilled and every reload waited for the prefetch DMA in flight.
  int ra = m * ROWB + ((g ^ swz16<CPR>(m)) << 4);
  int ta;
  {
    const int r0 = 4 * g + ((lane >> 2) & 3);
    ta = r0 * ROWB + (((((lane & 3) >> 1) ^ swz16<CPR>(r0)) << 4) | (8 * (lane & 1)));
  }
  // A operand: rows 16*qb + m of a Q or dO tile, dims 32c + 8g .. +7
  auto row_a = [&](const char FA_LDS* base, int qb, int c) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, lds_read16(base + 16 * qb * ROWB + (ra ^ (c << 6))));
  };
  // A operand X^T: dims 16*db + m over the queries of 32-query step s in k-slot order
  auto tr_a = [&](const char FA_LDS* base, int s, int db) __attribute__((always_inline)) {
    const char FA_LDS* b = base + 32 * s * ROWB + (ta ^ (db << 5));
    const i16x4 lo = lds_tr16(b), hi = lds_tr16(b + 16 * ROWB);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // B operand V^T: keys KW*wave + 16*kb + m, dims 32c + 8g .. +7
  auto v_b = [&](int kb, int c) __attribute__((always_inline)) {
    if constexpr (VLDS) {
      return __builtin_bit_cast(bf16x8, lds_read16(vsm + (KW * wave + 16 * kb) * ROWB + (ra ^ (c << 6))));
    } else {
      return vf[kb][c];
    }
  };

  const float c2 = p.c2;
  auto tile = [&](int it, const char FA_LDS* qs) __attribute__((always_inline)) {
    const int ih = it / nt, t = t0 + it - ih * nt;
    const int qt0 = t * BQ;
    if (CAUSAL && qt0 + BQ - 1 < kw0) return;          // every query of the tile precedes every key of the wave
    asm volatile("" : "+v"(ra), "+v"(ta));
    const char FA_LDS* dos = qs + TILEB;
    const char FA_LDS* st = qs + 2 * TILEB;
    const bool diag = CAUSAL && qt0 < kw0 + KW - 1;
    const int lim = kw0 + m - qt0 - 4 * g;              // keep element iff its (query - key) offset >= lim
#pragma unroll
    for (int s = 0; s < BQ / 32; ++s) {
      i32x4 pp[KBW], dsp[KBW];                          // B operands of this 32-query step, per key block
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qb = 2 * s + h;
        f32x4 sc[KBW], dp[KBW];
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) sc[kb] = dp[kb] = f32x4{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 aq = row_a(qs, qb, c);
          const bf16x8 ao = row_a(dos, qb, c);
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) {
            sc[kb] = mfma16(aq, kf[kb][c], sc[kb]);
            dp[kb] = mfma16(ao, v_b(kb, c), dp[kb]);
          }
        }
        const f32x4 l2 = *reinterpret_cast<const f32x4 FA_LDS*>(st + 4 * (16 * qb + 4 * g));
        const f32x4 dd = *reinterpret_cast<const f32x4 FA_LDS*>(st + 4 * (kStatRows + 16 * qb + 4 * g));
        float pr[KBW][4];
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) pr[kb][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][j], c2, -l2[j]));
        if (diag) {
          asm volatile("" ::: "memory");                // keep this a branch: only diagonal tiles mask
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[kb][j] = (16 * qb + j - 16 * kb) >= lim ? pr[kb][j] : 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          float ds[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) ds[j] = pr[kb][j] * (dp[kb][j] - dd[j]);
          pp[kb][2 * h] = (int)pack_bf16x2(pr[kb][0], pr[kb][1]);
          pp[kb][2 * h + 1] = (int)pack_bf16x2(pr[kb][2], pr[kb][3]);
          dsp[kb][2 * h] = (int)pack_bf16x2(ds[0], ds[1]);
          dsp[kb][2 * h + 1] = (int)pack_bf16x2(ds[2], ds[3]);
        }
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 ao = tr_a(dos, s, db);
        const bf16x8 aq = tr_a(qs, s, db);
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          dv[kb][db] = mfma16(ao, __builtin_bit_cast(bf16x8, pp[kb]), dv[kb][db]);
          dk[kb][db] = mfma16(aq, __builtin_bit_cast(bf16x8, dsp[kb]), dk[kb][db]);
        }
      }
    }
  };

  auto slot = [&](int s) __attribute__((always_inline)) { return smem + s * STAGEB; };
  if constexpr (VLDS) {
    Stager16<D, BK, NW> vstage;
    vstage.issue(static_cast<const char*>(p.v) + kv_off * 2, k0, N, vsm, wave, lane);
  }
  issue(0, slot(0));
  wait_vmcnt0_seen();   // K and V registers, Q/dO tile 0
  __syncthreads();
  if constexpr (CAUSAL) {
    // two-slot ring, unrolled by two so that the slot offsets are constants
    // (not without the mask: those instances then need more registers)
    auto step = [&](int it, int sl) __attribute__((always_inline)) {
      if (it + 1 < n_iter) issue(it + 1, slot(sl ^ 1));
      tile(it, slot(sl));
      wait_vmcnt<0>();
      __syncthreads();
    };
    int it = 0;
    for (; it + 1 < n_iter; it += 2) {
      step(it, 0);
      step(it + 1, 1);
    }
    if (it < n_iter) step(it, 0);
  } else {
    int cur = 0;
    for (int it = 0; it < n_iter; ++it) {
      if (it + 1 < n_iter) issue(it + 1, slot(cur ^ 1));
      tile(it, slot(cur));
      wait_vmcnt<0>();
      __syncthreads();
      cur ^= 1;
    }
  }

  const float sc = p.scale;
  float* dk_base = p.dk;
  float* dv_base = p.dv;
  if (p.parts > 1) {
    const int64_t slab = (int64_t)p.BH / p.parts * N * D;   // one part's [B*H_kv][N][D]
    dk_base = p.part_out + hp * slab;
    dv_base = p.part_out + (p.parts + hp) * slab;
  }
  // dK^T and dV^T leave through LDS as whole fp32 rows (one tensor per
  // pass): each wave writes its KW rows into its own region of the Q/dO ring
  // and V area, free since the last barrier, and reads them back a full row
  // segment per lane group, so every store instruction covers whole rows.
  // The 16-byte chunk of a row is XORed with row % 16, so that the 16 rows a
  // write instruction touches at one logical chunk fall in distinct banks.
  // (Stored from the accumulator layout, 16 rows x 64 bytes per instruction,
  // these stores bounded GPT-2-small's backward at 5.1 of 67.5 us.)
  constexpr int OROWB = 4 * D, OCPR = OROWB / 16;   // fp32 row bytes, chunks per row
  constexpr int WREG = KW * OROWB;                   // one wave's rows of one tensor
  constexpr int RPI = 1024 / OROWB;                  // rows per wave instruction
  static_assert(NW * WREG <= (int)sizeof(smem_raw) && OCPR >= 16 && KW % RPI == 0, "dK/dV staging fits");
  char FA_LDS* const wreg = smem + wave * WREG;
  auto stage_out = [&](const f32x4 (&acc)[KBW][NDB], float mul, float* base) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int row = 16 * kb + m;                  // dims 16 db + 4 g .. + 3 of key kw0 + row
        *reinterpret_cast<f32x4 FA_LDS*>(wreg + row * OROWB + (((4 * db + g) ^ (row & 15)) << 4)) = acc[kb][db] * mul;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the reads below fetch other lanes' writes
    const int rr = lane / OCPR, lc = lane % OCPR;
#pragma unroll
    for (int i = 0; i < KW / RPI; ++i) {
      const int row = i * RPI + rr;
      const f32x4 v = *reinterpret_cast<const f32x4 FA_LDS*>(wreg + row * OROWB + ((lc ^ (row & 15)) << 4));
      if (kw0 + row < N)
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(base + kv_off + (int64_t)(kw0 + row) * D + 4 * lc));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read out before the next tensor's writes
  };
  stage_out(dk, sc, dk_base);
  stage_out(dv, 1.f, dv_base);
}

// dk = sum of the parts' dK, dv likewise (four floats per thread)
__global__ __launch_bounds__(256) void fa_bwd_reduce_kernel(BwdParams p, int64_t n4) {
  const int64_t slab4 = n4;                 // float4s per part per tensor
  const f32x4* src = reinterpret_cast<const f32x4*>(p.part_out);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 a = src[i], b = src[p.parts * slab4 + i];
    for (int hp = 1; hp < p.parts; ++hp) {
      a += src[hp * slab4 + i];
      b += src[(p.parts + hp) * slab4 + i];
    }
    reinterpret_cast<f32x4*>(p.dk)[i] = a;
    reinterpret_cast<f32x4*>(p.dv)[i] = b;
  }
}

// ---------------------------------------------------------------- 3. dQ
// The dQ workgroup also forms its rows of the statistics workspace, which
// the dK/dV launch that follows reads.
template <int D, int BC, int NW, int WPE, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int BR = 32 * NW;
  constexpr int ROWB = 2 * D;
  constexpr int TILEB = BC * ROWB;
  constexpr int STAGEB = 2 * TILEB;          // K tile, V tile
  constexpr int NSTEP = D / 16, NDB = D / 32, KB = BC / 32;
  static_assert(2 * STAGEB <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem_raw[2 * STAGEB];
  char FA_LDS* const smem = (char FA_LDS*)(smem_raw);

  // wave index in an SGPR, so that LDS and DMA addresses stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const BwdLane ln = bwd_lane(lane);

  int bh, rb;
  map_block<CAUSAL>(p, blockIdx.x, bh, rb);
  const int N = p.N;
  const int q_row0 = rb * BR, qw0 = q_row0 + 32 * wave, my_q = qw0 + ln.n;
  const int64_t head_off = (int64_t)bh * N * D;
  const int64_t kv_off = (int64_t)(bh / p.qg) * N * D;

  bf16x8 qf[NSTEP], of[NSTEP];
  load_frag<D>(p.q, head_off, my_q, N, ln, qf);
  load_frag<D>(p.dout, head_off, my_q, N, ln, of);
  // this query's statistics: D = rowsum(dO * O) (each lane half sums its
  // half of the dims) and L2 = L * log2(e); queries past N get +inf and 0, so
  // their P is 0.  They are also written to the workspace for the dK/dV
  // launch that follows.
  float l2 = INFINITY, dd = 0.f;
  {
    bf16x8 of_o[NSTEP];
    load_frag<D>(p.o, head_off, my_q, N, ln, of_o);
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < NSTEP; ++c) {
      const i32x4 a = __builtin_bit_cast(i32x4, of_o[c]), b = __builtin_bit_cast(i32x4, of[c]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        part = __builtin_fmaf(bf16_lo_to_f32(a[j]), bf16_lo_to_f32(b[j]), part);
        part = __builtin_fmaf(bf16_hi_to_f32(a[j]), bf16_hi_to_f32(b[j]), part);
      }
    }
    const float dsum = swap_halves_sum(part);
    if (my_q < N) {
      l2 = p.lse[(int64_t)bh * N + my_q] * kLog2e;
      dd = dsum;
    }
    if (ln.hf == 0 && my_q < p.T * kStatRows) {
      float* w = p.ws + ((int64_t)bh * p.T + my_q / kStatRows) * (2 * kStatRows) + my_q % kStatRows;
      w[0] = l2;
      w[kStatRows] = dd;
    }
  }

  f32x16 dq[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) dq[b] = f32x16{};

  const int tiles_all = (N + BC - 1) / BC;
  const int n_tiles = CAUSAL ? min(tiles_all, (q_row0 + BR - 1) / BC + 1) : tiles_all;
  const int wave_tiles = CAUSAL ? min(tiles_all, (qw0 + 31) / BC + 1) : tiles_all;
  const int last_key = (CAUSAL ? min(N - 1, my_q) : N - 1) - 4 * ln.hf;

  UStager<D, BC, NW> stage;
  stage.init(wave, lane);
  const char* kglob = static_cast<const char*>(p.k) + kv_off * 2;
  const char* vglob = static_cast<const char*>(p.v) + kv_off * 2;
  auto slot = [&](int s) __attribute__((always_inline)) { return smem + s * STAGEB; };
  auto issue = [&](int j, char FA_LDS* dst) __attribute__((always_inline)) {
    stage.issue(kglob, j * BC, N, dst, wave, lane);
    stage.issue(vglob, j * BC, N, dst + TILEB, wave, lane);
  };

  const float c2 = p.c2;
  auto tile = [&](int j, const char FA_LDS* ks) __attribute__((always_inline)) {
    const char FA_LDS* vs = ks + TILEB;
    const int key0 = j * BC;
    const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > qw0);
    const int lim = last_key - key0;
    // per 32-key block: S^T, dP^T, dS^T, then that block's share of dQ^T
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 s{}, dp{};
      // items 2c (S^T, K rows) and 2c + 1 (dP^T, V rows), operand reads three ahead
      mfma_pipeline<2 * NSTEP, 3, 1, bf16x8>(
          [&](int i) __attribute__((always_inline)) { return row_operand<D>((i & 1) ? vs : ks, kb, i >> 1, ln); },
          [&](int i, const bf16x8& a) __attribute__((always_inline)) {
            if (i & 1) dp = mfma_bf16(a, of[i >> 1], dp);
            else s = mfma_bf16(a, qf[i >> 1], s);
          });
      float pr[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -l2));
      if (need_mask) {
        asm volatile("" ::: "memory");                 // keep this a branch: only diagonal and ragged tiles mask
#pragma unroll
        for (int i = 0; i < 16; ++i) pr[i] = (32 * kb + 8 * (i >> 2) + (i & 3)) > lim ? 0.f : pr[i];
      }
      i32x4 dsp[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int i0 = 8 * u + 2 * w;
          dsp[u][w] = (int)pack_bf16x2(pr[i0] * (dp[i0] - dd), pr[i0 + 1] * (dp[i0 + 1] - dd));
        }
      // items u * NDB + db: key step u of the block into d-block db
      mfma_pipeline<2 * NDB, 3, 2, bf16x8>(
          [&](int i) __attribute__((always_inline)) { return tr_operand<D>(ks, 2 * kb + i / NDB, i % NDB, ln); },
          [&](int i, const bf16x8& a) __attribute__((always_inline)) {
            dq[i % NDB] = mfma_bf16(a, __builtin_bit_cast(bf16x8, dsp[i / NDB]), dq[i % NDB]);
          });
    }
  };

  issue(0, slot(0));
  wait_vmcnt<0>();
  __syncthreads();
  // two-slot ring, unrolled by two so that the slot offsets are constants
  auto step = [&](int j, int sl) __attribute__((always_inline)) {
    if (j + 1 < n_tiles) issue(j + 1, slot(sl ^ 1));
    if (j < wave_tiles) tile(j, slot(sl));
    wait_vmcnt<0>();
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    step(j, 0);
    step(j + 1, 1);
  }
  if (j < n_tiles) step(j, 0);

  // dQ leaves through LDS as whole row segments, as dK and dV do in their
  // kernel: the K/V ring (free since the last barrier) holds NW x 32 rows of
  // D / NPASS dims per pass, chunk XOR (row % 16) against bank conflicts,
  // and the stores are non-temporal (dQ is not read again here).
  constexpr int NPASS = NW * 32 * 4 * D <= 2 * STAGEB ? 1 : NW * 32 * 4 * D <= 4 * STAGEB ? 2 : 4;
  constexpr int RB = 4 * D / NPASS, CPRR = RB / 16;   // region row bytes, 16-byte chunks per region row
  constexpr int DBP = NDB / NPASS;                    // 32-wide d-blocks per pass
  constexpr int RPI = 1024 / RB;                      // rows per wave instruction
  static_assert(NW * 32 * RB <= 2 * STAGEB && CPRR >= 16 && NDB % NPASS == 0, "dQ staging fits");
  char FA_LDS* const wreg = smem + wave * 32 * RB;
  const float sc = p.scale;
  const int rr = lane / CPRR, lc = lane % CPRR;
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    // lane (n, hf): dims 32 db + 8 g + 4 hf .. + 3 of query row n
#pragma unroll
    for (int b = 0; b < DBP; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int db = DBP * pass + b, c = 8 * b + 2 * g + ln.hf;
        *reinterpret_cast<f32x4 FA_LDS*>(wreg + ln.n * RB + ((c ^ (ln.n & 15)) << 4)) =
            f32x4{dq[db][4 * g] * sc, dq[db][4 * g + 1] * sc, dq[db][4 * g + 2] * sc, dq[db][4 * g + 3] * sc};
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the reads below fetch other lanes' writes
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + rr;
      const f32x4 v = *reinterpret_cast<const f32x4 FA_LDS*>(wreg + row * RB + ((lc ^ (row & 15)) << 4));
      if (qw0 + row < N)
        __builtin_nontemporal_store(
            v, reinterpret_cast<f32x4*>(p.dq + head_off + (int64_t)(qw0 + row) * D + pass * (D / NPASS) + 4 * lc));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read out before the next pass's writes
  }
}

}  // namespace fa
