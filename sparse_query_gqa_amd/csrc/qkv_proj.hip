// Query/key/value projections with token-compacted queries.
//
// GQE review (paper.oopus.info), section 二: only the selected query heads
// take part in attention and the rest are skipped, so only their query rows
// are projected; the shared head is projected for every token. GQA tutorial
// (zone.ci), 4.3: queries carry N heads, keys and values G heads. Every
// projection is linear without bias: q_{i,h} = W_Q[h] x_i with W_Q[h] the d
// rows h*d .. h*d+d-1 of W_Q (block N is the shared head), k_{i,g} =
// W_K[g] x_i, v_{i,g} = W_V[g] x_i.
//
// Work is split into tiles of output columns by a set of token rows. A
// routed query head takes only the tokens whose top-k holds it, compacted in
// token order (the order of the router's expert-major token lists), so no
// row of an unselected head is ever computed; the shared head, K and V take
// every token. Tile kinds:
//   * prefill: supersteps of a few hundred tokens, each with 256 x 256 tiles
//     over the key and value columns and one tile per query head holding
//     the superstep's tokens that selected it, on v_mfma_f32_32x32x16_bf16;
//     x and weight rows go straight into LDS by LDS-DMA, k in steps of 32
//     through a ring of stages;
//   * decode (few tokens, bound by reading the weights): 32-row tiles whose
//     routed rows are found by scanning the tokens' top-k, the model width
//     split over the four wavefronts, fragments loaded from global memory,
//     partial sums reduced in LDS. Keys and values go to cache row
//     kv_len[b] - q_len + t.
//   * fp32: plain VALU code, one thread per output value.
#include "gqe_internal.h"

namespace gqe {

namespace {

constexpr int kDRows = 32;   // token rows per decode tile

// Output row of token ft for head slot `which` (0..N query heads, then K
// heads g = 0..G-1, then V heads): the element offset of column 0, or -1
// for a cache row outside 0..S_max-1 (a kv_len that breaks the caller's
// contract: that row is not written, so nothing outside the cache is).
__device__ __forceinline__ int64_t out_row(const ProjParams& p, int which, int ft, int& kind) {
  if (which <= p.N) {
    kind = 0;
    return ((int64_t)ft * (p.N + 1) + which) * p.d;
  }
  const int kv = which - p.N - 1;  // 0..2G-1
  kind = kv < p.G ? 1 : 2;
  const int g = kv < p.G ? kv : kv - p.G;
  const int b = ft / p.L, t = ft - b * p.L;
  const int pos = p.kv_len ? p.kv_len[b] - p.L + t : t;
  if (pos < 0 || pos >= p.Smax) return -1;
  return (((int64_t)b * p.G + g) * p.Smax + pos) * p.d;
}

__device__ __forceinline__ const __bf16* head_weights(const ProjParams& p, int which) {
  if (which <= p.N) return (const __bf16*)p.w_q + (int64_t)which * p.d * p.D;
  const int kv = which - p.N - 1;
  return kv < p.G ? (const __bf16*)p.w_k + (int64_t)kv * p.d * p.D
                  : (const __bf16*)p.w_v + (int64_t)(kv - p.G) * p.d * p.D;
}

__device__ __forceinline__ void* out_base(const ProjParams& p, int kind) {
  return kind == 0 ? p.q : (kind == 1 ? p.k : p.v);
}

// ---------------------------------------------------------------------------
// Prefill tiles. Tokens (flat index b*S + s) are taken in supersteps of U
// consecutive tokens. A superstep's tiles are consecutive logical tiles, and
// consecutive logical tiles run on one XCD (block i on XCD i % 8, logical
// tile (i % 8) * per + i / 8), so its x rows come from HBM once and then from
// that XCD's L2; while they run, each tile also loads a slice of the next
// superstep's x rows into L2, so that its first reader does not wait on HBM.
// A superstep has
//   * dense tiles: 256 tokens x 256 columns of [G key heads | G value heads],
//     U / 256 windows of them, every token a row;
//   * one head tile per query head h = 0..N (N is the shared head): the
//     superstep's tokens whose top-k holds h (every token for the shared
//     head), compacted in token order by a ballot, which is the order of the
//     expert-major token lists, and taken 512 rows per pass.
// U = 256 * clamp(floor(3M / 2k), 1, 6) keeps a routed head's expected row
// count U k / M near 384, so that one pass almost always takes it.
// Products: v_mfma_f32_32x32x16_bf16, weight rows as the A operand and x rows
// as B, 512 threads. Operands reach LDS by raw-buffer LDS-DMA (rows past a
// tensor's end read zeros). The dense tiles and the d = 64 head tiles take k
// in steps of 32 through a ring of four buffers, so that three stages of x
// rows are in flight (k64 stages in two buffers left one in flight, and the
// loads' latency exposed); the d = 128 head tiles use a ring of three (four
// would not fit beside the row list) and the d = 32 head tiles k64 stages in
// two buffers. The next stage's loads go out between the products of the
// current one, so each stage costs one barrier. The tile goes back to HBM
// through LDS in 16-byte pieces.
// ---------------------------------------------------------------------------
constexpr int kDT = 256;     // dense tile: tokens and columns
constexpr int kHR = 512;     // head tile: rows per pass
constexpr int kUMax = 1536;  // superstep tokens, at most

int superstep_tokens(int M, int k) {
  const int f = (3 * M) / (2 * k);
  return 256 * (f < 1 ? 1 : (f > 6 ? 6 : f));
}

// Stage layouts. k32: rows of 64 bytes, 16-byte piece c of row r at
// position c ^ ((r >> 2) & 3); a 1 KiB DMA chunk holds 16 rows, lane l
// writing row l / 4 at position l % 4. k64: rows of 128 bytes, piece c at
// c ^ ((r >> 1) & 7); a chunk holds 8 rows, lane l writing row l / 8 at
// position l % 8. Either way the 16 rows of a fragment read fall on distinct
// bank groups, and lane l loads the logical piece its position holds.
__device__ __forceinline__ uint32_t piece_off4(int row, int lane) {
  return 16u * (uint32_t)((lane & 3) ^ ((row >> 2) & 3));
}
__device__ __forceinline__ uint32_t piece_off8(int row, int lane) {
  return 16u * (uint32_t)((lane & 7) ^ ((row >> 1) & 7));
}

// Fragment byte offsets in a stage of R x rows followed by the weight rows,
// KP pieces per row: x row xr0 + 32 rb + l32 and weight row wc0 + 32 cb + l32,
// logical piece 2 kk + half.
template <int R, int RB, int CB, int KP>
__device__ __forceinline__ void frag_offsets(int xr0, int wc0, int (&xo)[KP / 2][RB], int (&wo)[KP / 2][CB]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  auto pos = [](int r, int c) { return KP == 4 ? (c ^ ((r >> 2) & 3)) : (c ^ ((r >> 1) & 7)); };
#pragma unroll
  for (int kk = 0; kk < KP / 2; ++kk) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = xr0 + 32 * rb + l32;
      xo[kk][rb] = r * 16 * KP + 16 * pos(r, 2 * kk + half);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = wc0 + 32 * cb + l32;
      wo[kk][cb] = R * 16 * KP + c * 16 * KP + 16 * pos(c, 2 * kk + half);
    }
  }
}

// The products of one tile over the model width: nk stages of k64 in two
// LDS buffers of SB bytes. The wavefront's tile is RB x 32 x rows by CB x 32
// weight rows (offsets from frag_offsets); with `on` false it skips its
// products but still issues its loads and takes every barrier.
// dma.one(kt, st, i) issues this wavefront's i-th of NL loads of stage kt (a
// stage past the last re-loads the last one) into buffer st; pf() issues PF
// loads whose data nobody reads (they warm L2). The loads of stage kt+1 go
// out between the products of stage kt; one barrier per stage then publishes
// stage kt+1 and frees the buffer of stage kt. acc[cb][rb], lane (half,
// l32), element e: x row xr0 + 32 rb + l32, weight row wc0 + 32 cb +
// 8 (e / 4) + 4 half + e % 4.
template <int R, int RB, int CB, int SB, int NL, int PF, typename Dma, typename Pf>
__device__ __forceinline__ void gemm_k64(char* lds, int nk, int xr0, int wc0, bool on, const Dma& dma, const Pf& pf,
                                         f32x16 (&acc)[CB][RB]) {
  int xo[4][RB], wo[4][CB];
  frag_offsets<R, RB, CB, 8>(xr0, wc0, xo, wo);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[cb][rb][e] = 0.f;
  bf16x8 wf[2][CB], xf[2][RB];
  auto read_frags = [&](const char* sb, const int kk, const int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) wf[slot][cb] = *(const bf16x8*)(sb + wo[kk][cb]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) xf[slot][rb] = *(const bf16x8*)(sb + xo[kk][rb]);
  };
  for (int i = 0; i < NL; ++i) dma.one(0, 0, i);
  pf();
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(PF) : "memory");  // stage 0 complete
  __syncthreads();
  constexpr int NM = CB * RB;
  for (int kt = 0; kt < nk; ++kt) {
    const char* sb = lds + (kt & 1) * SB;
    if (on) {
      read_frags(sb, 0, 0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk + 1 < 4) read_frags(sb, kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int q = 0; q < NM; ++q) {
#pragma unroll
          for (int i = 0; i < NL; ++i)
            if ((i * 4 * NM) / NL == kk * NM + q) dma.one(kt + 1, (kt + 1) & 1, i);
          // the loads stay where they are among the products
          __builtin_amdgcn_sched_barrier(0);
          const int cb = q / RB, rb = q % RB;
          acc[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk & 1][cb], xf[kk & 1][rb], acc[cb][rb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      for (int i = 0; i < NL; ++i) dma.one(kt + 1, (kt + 1) & 1, i);
    }
    // this wavefront's loads of stage kt+1 (and the warming ones) have
    // landed; after the barrier so have everyone's, and stage kt is free
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// The same with k32 stages in a ring of NS >= 3 buffers: the second half of
// stage kt's fragments is read, and its first-half products run, before the
// barrier that publishes stage kt+1 (at most NS-3 later stages and, in the
// first step, the PF warming loads still in flight); then stage kt+NS-1's
// loads go out between stage kt's second-half products.
template <int R, int RB, int CB, int SB, int NS, int NL, int PF, typename Dma, typename Pf>
__device__ __forceinline__ void gemm_k32(char* lds, int nk, int xr0, int wc0, bool on, const Dma& dma, const Pf& pf,
                                         f32x16 (&acc)[CB][RB]) {
  static_assert(NS >= 3, "ring");
  int xo[2][RB], wo[2][CB];
  frag_offsets<R, RB, CB, 4>(xr0, wc0, xo, wo);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[cb][rb][e] = 0.f;
  bf16x8 wf[2][CB], xf[2][RB];
  auto read_frags = [&](const int kt, const int kk) __attribute__((always_inline)) {
    const char* sb = lds + (kt % NS) * SB;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) wf[kk][cb] = *(const bf16x8*)(sb + wo[kk][cb]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) xf[kk][rb] = *(const bf16x8*)(sb + xo[kk][rb]);
  };
  for (int s = 0; s < NS - 1; ++s)
    for (int i = 0; i < NL; ++i) dma.one(s, s, i);
  pf();
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(NL * (NS - 2) + PF) : "memory");  // stage 0 complete
  __syncthreads();
  if (on) read_frags(0, 0);
  constexpr int NM = CB * RB;
  for (int kt = 0; kt < nk; ++kt) {
    if (on) {
      read_frags(kt, 1);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0][cb], xf[0][rb], acc[cb][rb], 0, 0, 0);
    }
    if (kt == 0) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(NL * (NS - 3) + PF) : "memory");
    else __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(NL * (NS - 3)) : "memory");
    __syncthreads();
    if (on) {
#pragma unroll
      for (int q = 0; q < NM; ++q) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
          if ((i * NM) / NL == q) dma.one(kt + NS - 1, (kt + NS - 1) % NS, i);
        __builtin_amdgcn_sched_barrier(0);
        const int cb = q / RB, rb = q % RB;
        acc[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1][cb], xf[1][rb], acc[cb][rb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kt + 1 < nk) read_frags(kt + 1, 0);
    } else {
      for (int i = 0; i < NL; ++i) dma.one(kt + NS - 1, (kt + NS - 1) % NS, i);
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA may outlive the ring
  __syncthreads();
}

// acc into the LDS staging tile ys (row stride YP elements), rows xr0 + ...,
// columns wc0 + ...
template <int RB, int CB, int YP>
__device__ __forceinline__ void stage_out(__bf16* ys, int xr0, int wc0, const f32x16 (&acc)[CB][RB]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = xr0 + 32 * rb + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = f2bf(acc[cb][rb][4 * q + e]);
        *(bf16x4*)&ys[row * YP + wc0 + 32 * cb + 8 * q + 4 * half] = o4;
      }
    }
}

// Loads of one tile stage, lane by lane: loads 0 .. NX-1 are x chunks from
// `rx` (chunk `xc0 + i` of the stage), loads NX .. NX+NW-1 weight chunks from
// `rw` (chunk `wc0 + i` of the weight region at byte wbase), or into the
// sink when `wreal` is false. Offsets advance by `kb` bytes per stage. With
// `skip` (only where every wait is vmcnt(0) or counts the warming loads
// alone, as in gemm_k64), x chunks from `xlive` on, whose rows all lie past
// the pass's row count, and weight loads into the sink are not issued.
template <int NX, int NW>
struct TileLoads {
  char* lds;
  int nk, sb, kb, xc0, wc0, wbase, sink;
  bool wreal;
  i32x4 rx, rw;
  uint32_t xoff[NX], woff[NW];
  bool skip = false;
  int xlive = NX;
  __device__ __forceinline__ void one(const int kt, const int st, const int i) const {
    const uint32_t k2 = (uint32_t)min(kt, nk - 1) * (uint32_t)kb;
    char* base = lds + st * sb;
    if (i < NX) {
      if (!skip || i < xlive) lds_dma16_b(rx, xoff[i] + k2, base + (xc0 + i) * 1024);
    } else if (!skip || wreal) {
      lds_dma16_b(rw, woff[i - NX] + k2, wreal ? base + wbase + (wc0 + i - NX) * 1024 : lds + sink);
    }
  }
};

template <int D>
__global__ __launch_bounds__(512, 1) void proj_tile_kernel(ProjParams p, int U, int per_super, int n_kv, int per) {
  constexpr bool H64 = D <= 32;            // head tiles in k64 stages
  constexpr int RBH = D == 128 ? 4 : 2;    // head tile: wavefront rows / 32
  constexpr int CBH = D == 32 ? 1 : 2;     // head tile: wavefront columns / 32
  constexpr int SBD = 2 * kDT * 64;        // dense stage: 256 x rows + 256 weight rows, k32
  constexpr int NSD = 4;                   // dense stages in the ring
  constexpr int SBH = H64 ? (kHR + D) * 128 : (kHR + D) * 64;  // head stage
  constexpr int NSH = H64 ? 2 : (D == 64 ? 4 : 3);
  constexpr int YPD = kDT + 8, YPH = D + 8;  // staging row strides (elements)
  constexpr int SINK = NSD * SBD > NSH * SBH ? NSD * SBD : NSH * SBH;  // 1 KiB for loads kept nowhere
  constexpr int L1 = kDT * YPD * 2 > kHR * YPH * 2 ? kDT * YPD * 2 : kHR * YPH * 2;
  constexpr int LDSB = SINK + 1024 > L1 ? SINK + 1024 : L1;
  static_assert(LDSB + kUMax * 4 + 64 <= 163840, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[LDSB];
  __shared__ int rows_s[kUMax];
  __shared__ int wcnt[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t j = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  const int64_t u = j / per_super;
  const int r = (int)(j - u * per_super);
  const int64_t t_base = u * U;
  if (t_base >= p.T) return;
  const int nu = (int)min<int64_t>(U, p.T - t_base);  // tokens of this superstep
  const int n_dense = (U / kDT) * n_kv;
  const __bf16* x = (const __bf16*)p.x;
  const uint32_t rowb = (uint32_t)p.D * 2u;  // bytes of a row of x or of a weight
  // the next superstep's x rows, loaded into L2 in 8 KiB pieces (one lane
  // per 128-byte line): pieces 16 r .. 16 r + 15 of it, two per wavefront
  const int64_t tn = t_base + U;
  const i32x4 rpf = buf_rsrc(x + (tn < p.T ? tn : t_base) * p.D,
                             tn < p.T ? (uint32_t)min<int64_t>(U, p.T - tn) * rowb : 0u);
  const uint32_t pfoff = (uint32_t)(r * 16 + wave * 2) * 8192u + (uint32_t)lane * 128u;

  if (r < n_dense) {
    const int win = r / n_kv, ct = r - win * n_kv;
    const int64_t t0 = t_base + (int64_t)win * kDT;
    if (t0 >= p.T) return;
    const int nv = (int)min<int64_t>(kDT, p.T - t0);
    const int gd = p.G * D, ncols = 2 * gd;
    const int n0 = ct * kDT;
    // x chunks 2 wave + i (rows 32 wave + 16 i + lane / 4); weight rows
    // n0 + 32 wave .. +31 of [W_K | W_V], all key or all value rows (32
    // divides G*d)
    const int nw = n0 + 32 * wave;
    const __bf16* wb = nw >= ncols ? (const __bf16*)p.w_k
                       : nw < gd   ? (const __bf16*)p.w_k + (int64_t)nw * p.D
                                   : (const __bf16*)p.w_v + (int64_t)(nw - gd) * p.D;
    TileLoads<2, 2> ld{lds, p.D / 32, SBD, 64, 2 * wave, 2 * wave, kDT * 64, SINK, true,
                       buf_rsrc(x + t0 * p.D, (uint32_t)nv * rowb), buf_rsrc(wb, nw < ncols ? 32u * rowb : 0u), {}, {}};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 32 * wave + 16 * i + (lane >> 2);
      ld.xoff[i] = (uint32_t)row * rowb + piece_off4(row, lane);
      ld.woff[i] = (uint32_t)(16 * i + (lane >> 2)) * rowb + piece_off4(row, lane);
    }
    auto pf = [&]() __attribute__((always_inline)) {
      lds_dma16_b(rpf, pfoff, lds + SINK);
      lds_dma16_b(rpf, pfoff + 8192u, lds + SINK);
    };
    const int wm = wave & 1, wn = wave >> 1;  // 128 tokens x 64 columns each
    f32x16 acc[2][4];
    gemm_k32<kDT, 4, 2, SBD, NSD, 4, 2>(lds, p.D / 32, 128 * wm, 64 * wn, 128 * wm < nv && n0 + 64 * wn < ncols, ld,
                                        pf, acc);
    __bf16* ys = (__bf16*)lds;
    stage_out<4, 2, YPD>(ys, 128 * wm, 64 * wn, acc);
    __syncthreads();
    for (int it = tid; it < kDT * (kDT / 8); it += 512) {
      const int row = it >> 5, c8 = (it & 31) * 8;
      const int n = n0 + c8;
      if (row >= nv || n >= ncols) continue;
      const int t = (int)(t0 + row);
      const int b = t / p.L, s = t - b * p.L;
      const bool isv = n >= gd;
      const int nn = isv ? n - gd : n;
      const int g = nn / D;
      __bf16* dst = (__bf16*)(isv ? p.v : p.k) + (((int64_t)b * p.G + g) * p.Smax + s) * D + (nn - g * D);
      *(bf16x8*)dst = *(const bf16x8*)&ys[row * YPD + c8];
    }
    return;
  }

  // head tile: compact the superstep's tokens that selected head h
  const int h = r - n_dense;  // 0..N; N is the shared head
  const int g = h < p.N ? h / p.M : 0, m = h < p.N ? h - g * p.M : 0;
  int count = 0;
  for (int q0 = 0; q0 < nu; q0 += 512) {
    const int lt = q0 + tid;
    bool keep = lt < nu;
    if (keep && h < p.N) {
      const int32_t* tk = p.topk + ((t_base + lt) * p.G + g) * p.K;
      bool chose = false;
      for (int s = 0; s < p.K; ++s) chose |= tk[s] == m;
      keep = chose;
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
    if (lane == 0) wcnt[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int before = count, total = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = wcnt[i];
      before += i < wave ? c : 0;
      total += c;
    }
    if (keep) rows_s[before + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] = lt;
    count += total;
    __syncthreads();  // wcnt is rewritten by the next round
  }
  if (count == 0) return;  // uniform: no token of the superstep picked this head

  const uint32_t xend = (uint32_t)nu * rowb;
  const i32x4 rx = buf_rsrc(x + t_base * p.D, xend);
  const i32x4 rnone = buf_rsrc(x, 0u);
  constexpr int WR = RBH * 32;  // rows per wavefront
  const int wm = D == 128 ? (wave & 3) : wave;
  const int wn = D == 128 ? (wave >> 2) : 0;
  // weight chunk `wave` of the head (k64: rows 8 wave .. +7; k32: rows
  // 16 wave .. +15) when the head has it; other wavefronts load into the sink
  constexpr int WCR = H64 ? 8 : 16;
  const bool wreal = wave < D / WCR;
  const i32x4 rw = buf_rsrc((const __bf16*)p.w_q + ((int64_t)h * D + (wreal ? WCR * wave : 0)) * p.D,
                            wreal ? (uint32_t)WCR * rowb : 0u);
  for (int c0 = 0; c0 < count; c0 += kHR) {
    if (c0 > 0) __syncthreads();  // the previous pass is done with the staging tile
    const int nr = min(kHR, count - c0);
    const i32x4 rp = c0 == 0 ? rpf : rnone;  // L2 warming in the first pass only
    auto pf = [&]() __attribute__((always_inline)) {
      lds_dma16_b(rp, pfoff, lds + SINK);
      lds_dma16_b(rp, pfoff + 8192u, lds + SINK);
    };
    f32x16 acc[CBH][RBH];
    if constexpr (H64) {
      // x chunks 8 wave + i: rows 64 wave + 8 i + lane / 8 of the pass
      TileLoads<8, 1> ld{lds, p.D / 64, SBH, 128, 8 * wave, wave, kHR * 128, SINK, wreal, rx, rw, {}, {}};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 64 * wave + 8 * i + (lane >> 3);
        ld.xoff[i] = row < nr ? (uint32_t)rows_s[c0 + row] * rowb + piece_off8(row, lane) : xend;
      }
      ld.woff[0] = (uint32_t)(lane >> 3) * rowb + piece_off8(8 * wave + (lane >> 3), lane);
      // chunks past the pass's rows carry nothing (a quarter of them at an
      // expected 384 of 512 rows): gemm_k64 waits for everything, so they go
      ld.skip = true;
      ld.xlive = __builtin_amdgcn_readfirstlane(min(8, max(0, (nr - 64 * wave + 7) / 8)));
      gemm_k64<kHR, RBH, CBH, SBH, 9, 2>(lds, p.D / 64, WR * wm, 64 * wn, WR * wm < nr, ld, pf, acc);
    } else {
      // x chunks 4 wave + i: rows 64 wave + 16 i + lane / 4 of the pass
      TileLoads<4, 1> ld{lds, p.D / 32, SBH, 64, 4 * wave, wave, kHR * 64, SINK, wreal, rx, rw, {}, {}};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 64 * wave + 16 * i + (lane >> 2);
        ld.xoff[i] = row < nr ? (uint32_t)rows_s[c0 + row] * rowb + piece_off4(row, lane) : xend;
      }
      ld.woff[0] = (uint32_t)(lane >> 2) * rowb + piece_off4(16 * wave + (lane >> 2), lane);
      gemm_k32<kHR, RBH, CBH, SBH, NSH, 5, 2>(lds, p.D / 32, WR * wm, 64 * wn, WR * wm < nr, ld, pf, acc);
    }
    __bf16* ys = (__bf16*)lds;
    stage_out<RBH, CBH, YPH>(ys, WR * wm, 64 * wn, acc);
    __syncthreads();
    for (int it = tid; it < nr * (D / 8); it += 512) {
      const int row = it / (D / 8), c8 = (it % (D / 8)) * 8;
      const int64_t t = t_base + rows_s[c0 + row];
      *(bf16x8*)((__bf16*)p.q + (t * (p.N + 1) + h) * D + c8) = *(const bf16x8*)&ys[row * YPH + c8];
    }
  }
}

// fp32: one thread per (token, column) of one head slot (blockIdx.y); a
// routed query head computes only the tokens whose top-k holds it.
__global__ __launch_bounds__(256) void proj_f32_kernel(ProjParams p) {
  const int which = blockIdx.y;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)p.T * p.d) return;
  const int ft = (int)(e / p.d), c = (int)(e - (int64_t)ft * p.d);
  if (which < p.N) {
    const int g = which / p.M, m = which - g * p.M;
    bool chose = false;
    for (int s = 0; s < p.K; ++s) chose |= p.topk[((int64_t)ft * p.G + g) * p.K + s] == m;
    if (!chose) return;
  }
  const float* xr = (const float*)p.x + (int64_t)ft * p.D;
  const float* wr;
  if (which <= p.N) wr = (const float*)p.w_q + ((int64_t)which * p.d + c) * p.D;
  else {
    const int kv = which - p.N - 1;
    wr = (kv < p.G ? (const float*)p.w_k + ((int64_t)kv * p.d + c) * p.D
                   : (const float*)p.w_v + ((int64_t)(kv - p.G) * p.d + c) * p.D);
  }
  float s = 0.f;
  for (int i = 0; i < p.D; ++i) s = fmaf(xr[i], wr[i], s);
  int kind;
  const int64_t o = out_row(p, which, ft, kind);
  if (o < 0) return;
  ((float*)out_base(p, kind))[o + c] = s;
}

// Decode tiles: head slot blockIdx.y, 32-column block blockIdx.z of that
// head, chunk blockIdx.x of 32 tokens (flat index b*q_len + t). A routed head
// keeps the chunk's tokens whose top-k holds it (a ballot, in token order);
// other slots keep every token. Splitting the head's columns over blocks
// spreads the weight reads, which bound this shape, over more CUs. The four
// wavefronts each take a quarter of the model width; fragments come straight
// from global memory (the weights are read once, x stays in L2), and the
// partial tiles are summed in LDS in a fixed order.
__global__ __launch_bounds__(256) void proj_decode_kernel(ProjParams p) {
  constexpr int CB = 1;
  constexpr int U = 8;  // k-steps of loads in flight per wavefront
  __shared__ int rows[kDRows];
  __shared__ int nrows_s;
  __shared__ float red[4][CB][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int which = blockIdx.y;
  if (wave == 0) {
    const int ft = blockIdx.x * kDRows + lane;
    bool keep = lane < kDRows && ft < p.T;
    if (keep && which < p.N) {
      const int g = which / p.M, m = which - g * p.M;
      bool chose = false;
      for (int s = 0; s < p.K; ++s) chose |= p.topk[((int64_t)ft * p.G + g) * p.K + s] == m;
      keep = chose;
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
    if (keep) rows[__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] = ft;
    if (lane == 0) nrows_s = __builtin_popcountll(bal);
  }
  __syncthreads();
  const int nrows = nrows_s;
  if (nrows == 0) return;

  const __bf16* xr = (const __bf16*)p.x + (int64_t)rows[min(l32, nrows - 1)] * p.D + 8 * half;
  const int col0 = 32 * blockIdx.z;  // first column of this block within the head
  const __bf16* wh = head_weights(p, which) + (int64_t)(col0 + l32) * p.D + 8 * half;
  const int kq = p.D / 4;  // model-width quarter of this wavefront
  const int k0 = wave * kq;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[cb][e] = 0.f;
  int k = k0;
  for (; k + 16 * U <= k0 + kq; k += 16 * U) {
    bf16x8 xf[U], wf[U][CB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xf[u] = *(const bf16x8*)(xr + k + 16 * u);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) wf[u][cb] = *(const bf16x8*)(wh + (int64_t)32 * cb * p.D + k + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[u][cb], xf[u], acc[cb], 0, 0, 0);
  }
  for (; k < k0 + kq; k += 16) {  // quarter widths that are not a multiple of 64
    const bf16x8 xf = *(const bf16x8*)(xr + k);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(wh + (int64_t)32 * cb * p.D + k), xf,
                                                        acc[cb], 0, 0, 0);
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave][cb][e][lane] = acc[cb][e];
  __syncthreads();
  // wavefront w sums and stores the 32-column blocks cb = w, w+4, ...
  for (int cb = wave; cb < CB; cb += 4) {
    if (l32 >= nrows) continue;
    int kind;
    const int64_t o = out_row(p, which, rows[l32], kind);
    if (o < 0) continue;
    __bf16* out = (__bf16*)out_base(p, kind) + o + col0;
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * jq + e;
        o4[e] = f2bf(((red[0][cb][i][lane] + red[1][cb][i][lane]) + red[2][cb][i][lane]) + red[3][cb][i][lane]);
      }
      *(bf16x4*)(out + 32 * cb + 8 * jq + 4 * half) = o4;
    }
  }
}

}  // namespace

hipError_t launch_proj(const ProjParams& p, bool bf16, hipStream_t s) {
  const int heads = p.N + 1 + 2 * p.G;
  if (!bf16) {
    const unsigned nx = (unsigned)(((int64_t)p.T * p.d + 255) / 256);
    hipLaunchKernelGGL(proj_f32_kernel, dim3(nx, heads), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  if (p.kv_len) {  // decode: few tokens, (chunk of 32 tokens) x head slot
    const dim3 grid((unsigned)((p.T + kDRows - 1) / kDRows), (unsigned)heads, (unsigned)(p.d / 32));
    hipLaunchKernelGGL(proj_decode_kernel, grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
  const int U = superstep_tokens(p.M, p.K);
  const int n_kv = (2 * p.G * p.d + kDT - 1) / kDT;
  const int per_super = (U / kDT) * n_kv + p.N + 1;
  const int64_t total = (int64_t)((p.T + U - 1) / U) * per_super;
  const int per = (int)((total + 7) / 8);
  const unsigned nblk = (unsigned)(8 * per);
  switch (p.d) {
    case 32: hipLaunchKernelGGL(proj_tile_kernel<32>, dim3(nblk), dim3(512), 0, s, p, U, per_super, n_kv, per); break;
    case 64: hipLaunchKernelGGL(proj_tile_kernel<64>, dim3(nblk), dim3(512), 0, s, p, U, per_super, n_kv, per); break;
    case 128: hipLaunchKernelGGL(proj_tile_kernel<128>, dim3(nblk), dim3(512), 0, s, p, U, per_super, n_kv, per); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqe
