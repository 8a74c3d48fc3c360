// Backward pass of the sparse-query causal prefill attention.
//
// For a query row q with visible keys j <= pos, s_j = q.k_j / sqrt(d),
// P = softmax(s) and o = sum_j P_j v_j (GQA tutorial, 技术深化: scaled
// dot-product attention with an additive causal mask). Given dO:
//   dv_j += P_j dO,   dP_j = dO.v_j,   dS_j = P_j (dP_j - dO.o),
//   dq = sum_j dS_j k_j / sqrt(d),   dk_j += dS_j q / sqrt(d).
// A KV head's dK and dV are sums over every query row that reads it: the
// selected heads of its group and, for KV head 0, the shared head (GQA-zone
// page, 训练与部署: keys and values shared by several query heads collect
// the sum of their gradients). The forward's per-row log-sum-exp rebuilds P
// without a running max: P_j = exp(s_j - lse).
//
// Passes, all on the forward's row packing (rows of (b, v) token-major, k per
// token for a routed group, one for the shared head v = G):
//  1. prep: per row, copy q (bf16: times scale*log2(e), so that q.k comes
//     out of the MFMA as an exp2 argument) and dO into contiguous packed rows
//     and store the lse offset and -dO.O (rows past the end of a packed
//     block are zero);
//  2. dK/dV: a workgroup per (sequence, virtual group, 32-key block) keeps
//     the block's K and V in LDS and streams every row that can see the
//     block; each of its four wavefronts takes every fourth 32-row tile
//     through its own LDS ring, and the four partial sums are added through
//     LDS at the end;
//  3. dQ: the forward's 256-row tiles (one KV head each), with K and V
//     blocks streamed through LDS as in the forward;
//  4. KV head 0 receives two sums (routed group 0 and the shared head); both
//     go to an fp32 workspace and the last pass adds them.
// bf16 products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the
// fp32 path is plain VALU arithmetic.
#include <type_traits>

#include "prefill_tiles.h"

namespace gqe {

constexpr int kBwdChunk = 32;  // consecutive key blocks of one (b, v) given to one XCD

// ---------------------------------------------------------------------------
// 1. prep
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int EPT = 16 / (int)sizeof(T);  // elements per thread (16 bytes)
  constexpr int TPR = D / EPT;              // threads per row (divides 64)
  constexpr int RPB = 256 / TPR;
  const PrefillParams& f = p.f;
  const int seg = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int64_t nrows = (int64_t)f.B * (f.G + 1) * p.Rp;
  if (row >= nrows) return;  // (whole TPR groups leave together)
  const int64_t bv = row / p.Rp;
  const int r = (int)(row - bv * p.Rp);
  const int b = (int)(bv / (f.G + 1)), v = (int)(bv - (int64_t)b * (f.G + 1));
  const int R = (v == f.G) ? f.S : f.S * f.K;
  uint4* qd = (uint4*)((T*)p.qp + row * D) + seg;
  uint4* dd = (uint4*)((T*)p.dop + row * D) + seg;
  if (r >= R) {
    *qd = make_uint4(0u, 0u, 0u, 0u);
    *dd = make_uint4(0u, 0u, 0u, 0u);
    if (seg == 0) {
      p.nlse[row] = 0.f;
      p.ndel[row] = 0.f;
    }
    return;
  }
  int pos, slot, head;
  row_info(f, b, v, r, pos, slot, head);
  const int64_t tok = (int64_t)b * f.S + pos;
  const int64_t orow = (v == f.G) ? tok : (tok * f.G + v) * f.K + slot;
  const uint4 qv = ((const uint4*)((const T*)f.q + (tok * (f.N + 1) + head) * D))[seg];
  const uint4 ov = ((const uint4*)((const T*)(v == f.G ? f.o_s : f.o_r) + orow * D))[seg];
  const uint4 gv = ((const uint4*)((const T*)(v == f.G ? p.do_s : p.do_r) + orow * D))[seg];
  if constexpr (sizeof(T) == 2) {
    // bf16: q * scale * log2(e), rounded once (as the forward's scores are)
    uint4 qs = qv;
    const __bf16* qe = (const __bf16*)&qv;
    __bf16* qo = (__bf16*)&qs;
#pragma unroll
    for (int i = 0; i < EPT; ++i) qo[i] = f2bf((float)qe[i] * (f.scale * 1.44269504088896340736f));
    *qd = qs;
  } else {
    *qd = qv;
  }
  *dd = gv;
  const T* oe = (const T*)&ov;
  const T* ge = (const T*)&gv;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) acc = fmaf((float)oe[i], (float)ge[i], acc);
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (seg == 0) {
    const float lse = (v == f.G) ? f.lse_s[tok] : f.lse_r[orow];
    // bf16: -lse*log2(e), the exp2 argument's offset for prescaled q;
    // fp32: -lse*sqrt(d), the offset of the raw product q.k
    p.nlse[row] = sizeof(T) == 2 ? -lse * 1.44269504088896340736f : -lse / f.scale;
    p.ndel[row] = -acc;
  }
}

// LDS tile layout shared by the bf16 kernels: row r of a tile at r*ROWB, its
// 16-byte chunk c at chunk position c ^ swz(r) (the forward's layout: plain
// 16-byte row reads and transposing 8-byte reads are both free of bank
// conflicts). Row offsets that are multiples of 16 leave swz unchanged.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  return (((r >> 1) & 7) ^ ((r & 2) << 1)) & (D / 8 - 1);
}

// Transposing read of a 16-row step of a tile: lane (half, l32) receives
// column d = 32 db + l32 of rows 8 (e/4) + 4 half + e%4, e = 0..7, i.e. the
// contraction slots of an MFMA operand whose other side is an S-layout
// fragment. off[tt][db] is tr_offsets' result.
template <int D>
struct TrOffsets {
  int off[2][D / 32];
  __device__ __forceinline__ TrOffsets(int lane) {
    constexpr int ROWB = 2 * D;
    const int half = lane >> 5;
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        off[tt][db] = (8 * tt + tr_row) * ROWB + 16 * ((4 * db + (tr_d >> 3)) ^ tile_swz<D>(8 * tt + tr_row)) +
                      2 * (tr_d & 7);
  }
  __device__ __forceinline__ bf16x8 read(const char* base, int st, int db) const {
    u32x4 w;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const char* a = base + 16 * st * 2 * D + off[tt][db];
      const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a);
      const u32x2 y = __builtin_bit_cast(u32x2, x);
      w[2 * tt] = y[0];
      w[2 * tt + 1] = y[1];
    }
    return __builtin_bit_cast(bf16x8, w);
  }
};

// ---------------------------------------------------------------------------
// 2. dK / dV (bf16)
// ---------------------------------------------------------------------------
// Workgroup (b, v, kb): keys key0 = kb*32 .. +31 of KV head (v == G ? 0 :
// v); the rows that can see key0 start at row key0*kk (kk rows per token).
// With q' = q * scale * log2(e) (packed) and per-row offsets -lse*log2(e)
// and -delta as the MFMAs' initial accumulators, per 32-row tile a
// wavefront computes
//   S  = Q' K^T - lse*log2(e),  P = exp2(S)   (= exp(q.k/sqrt(d) - lse))
//   dPm = dO V^T - delta,  dS = P * dPm,
//   dV += P^T dO,  dK += dS^T Q'   (times ln 2 at the end: scale/(scale*log2 e))
// In the S layout lane (half, l32) holds key l32 and rows 8(t/4) + 4 half +
// t%4, which is exactly the A operand P^T / dS^T of the dV / dK products
// (contraction over rows), so P and dS never leave registers; the B operands
// dO and Q' come from transposing LDS reads, K and V from the block's copy
// in LDS.
//
// Registers decide the shape: one 32-key block per workgroup keeps a
// wavefront's working set (dK and dV accumulators, S and dP, the tile's
// fragments) within 256 VGPRs, so that the MFMAs write VGPRs (the VALU reads
// S and dP without copies out of AGPRs) and, for d <= 64, two workgroups
// share a CU. A 64-key block halves the LDS reads per MFMA but needs AGPR
// accumulators and one workgroup per CU: it ran 25% slower.
//
// Grid: chunks of kBwdChunk consecutive key blocks of one (b, v), longest
// rows first (chunk index c = kb-chunk * U + u); chunk c runs on XCD c % 8,
// so the workgroups an XCD runs at once stream the same rows through its L2.
template <int D>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void bwd_dkdv_kernel(BwdParams p, int nkb) {
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
  constexpr int NH = 1;  // 32-key halves per workgroup (one: see the note on registers above)
  constexpr int KB = 32 * NH;
  constexpr int KS = D / 16, DB = D / 32, ROWB = 2 * D;
  constexpr int TB = 32 * ROWB;       // one 32-row tile of Q or dO
  constexpr int NQ = TB / 1024;       // 1 KiB LDS-DMA chunks per tile
  constexpr int RPC = 1024 / ROWB;    // rows per chunk
  constexpr int BUFB = 2 * TB + 256;  // Q tile, dO tile, lse offsets[32], -delta[32]
  constexpr int NBUF = 2;
  constexpr int NDMA = 2 * NQ + 1;    // LDS-DMA instructions per tile
  __shared__ __attribute__((aligned(1024))) char lds[4][NBUF][BUFB];
  __shared__ __attribute__((aligned(1024))) char kvl[2][KB * ROWB];  // the block's K and V rows
  static_assert(sizeof(lds) >= 4 * KB * D * sizeof(float), "reduction space");

  const PrefillParams& f = p.f;
  const int U = f.B * (f.G + 1);
  const int nkbc = (nkb + kBwdChunk - 1) / kBwdChunk;
  const int x = blockIdx.x % 8, jj = blockIdx.x / 8;
  const int c = x + 8 * (jj / kBwdChunk);
  if (c >= nkbc * U) return;
  const int kb = (c / U) * kBwdChunk + jj % kBwdChunk;
  if (kb >= nkb) return;
  const int u = c % U;
  const int b = u / (f.G + 1), v = u - b * (f.G + 1);
  const int kvh = (v == f.G) ? 0 : v;
  const int kk = (v == f.G) ? 1 : f.K;
  const int R = f.S * kk;
  const int key0 = kb * KB;
  const int row0 = key0 * kk;  // a multiple of 32
  const int ntiles = (R - row0 + 31) / 32;
  const int64_t pbase = (int64_t)u * p.Rp;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // The block's K and V rows (keys past the end repeat the last key) go to
  // LDS once, in the tile layout; each tile reads its B operands of Q' K^T
  // and dO V^T from there (lane (half, l32): key 32h + l32, d 16s + 8 half),
  // which keeps them out of the register budget.
  {
    const int64_t hb = ((int64_t)b * f.G + kvh) * (int64_t)f.S * D;
    constexpr int CPR = D / 8;
    for (int ch = tid; ch < KB * CPR; ch += 256) {
      const int r = ch / CPR, cc = ch % CPR;
      const int key = min(key0 + r, f.S - 1);
      const int off = r * ROWB + 16 * (cc ^ tile_swz<D>(r));
      *(uint4*)(kvl[0] + off) = *(const uint4*)((const __bf16*)f.k + hb + (int64_t)key * D + 8 * cc);
      *(uint4*)(kvl[1] + off) = *(const uint4*)((const __bf16*)f.v + hb + (int64_t)key * D + 8 * cc);
    }
    __syncthreads();
  }

  // this wavefront's tiles: wave, wave + 4, ...
  const int ntw = ntiles > wave ? (ntiles - wave + 3) / 4 : 0;
  const int dma_r = (16 * lane) / ROWB;
  const int dma_p = ((16 * lane) % ROWB) / 16;
  uint32_t dma_off[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    const int rb = n * RPC + dma_r;
    dma_off[n] = rb * ROWB + 16 * (dma_p ^ tile_swz<D>(rb));
  }
  // Tile i of this wavefront into buffer bf (past the last tile it re-loads
  // the last one, so that every pass issues the same number of loads).
  auto dma = [&](const int i, const int bf) __attribute__((always_inline)) {
    const int tr0 = row0 + 32 * (wave + 4 * min(i, ntw - 1));
    const __bf16* qs = (const __bf16*)p.qp + (pbase + tr0) * D;
    const __bf16* gs = (const __bf16*)p.dop + (pbase + tr0) * D;
    char* dst = lds[wave][bf];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      lds_dma16_s(qs, dma_off[n], dst + n * 1024);
      lds_dma16_s(gs, dma_off[n], dst + TB + n * 1024);
    }
    if (lane < 16) lds_dma16((lane < 8 ? p.nlse : p.ndel) + pbase + tr0 + 4 * (lane & 7), dst + 2 * TB);
  };

  int k_off[KS];  // row l32, chunk 2s + half
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = l32 * ROWB + 16 * ((2 * s + half) ^ tile_swz<D>(l32));
  const TrOffsets<D> tr(lane);
  // For d <= 64 the block's K and V fragments (the same for every tile) stay
  // in registers: LDS read bandwidth, not the MFMAs, bounds this kernel, and
  // they were a quarter of each tile's LDS reads.
  bf16x8 kreg[D <= 64 ? KS : 1], vreg[D <= 64 ? KS : 1];
  if constexpr (D <= 64) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kreg[s] = *(const bf16x8*)(kvl[0] + k_off[s]);
      vreg[s] = *(const bf16x8*)(kvl[1] + k_off[s]);
    }
  }

  f32x16 dk[NH][DB], dv[NH][DB];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 16; ++t) dk[h][db][t] = dv[h][db][t] = 0.f;

  auto tile = [&](const int bf, const int tr0, const bool masked) __attribute__((always_inline)) {
    const char* qt = lds[wave][bf];
    const char* gt = qt + TB;
    const float* ld = (const float*)(qt + 2 * TB);
    bf16x8 qa[KS], ga[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qa[s] = *(const bf16x8*)(qt + k_off[s]);
      ga[s] = *(const bf16x8*)(gt + k_off[s]);
    }
    f32x16 nl, nd;  // element t <-> row 8(t/4) + 4 half + t%4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 a = *(const f32x4*)(ld + 8 * j + 4 * half);
      const f32x4 e = *(const f32x4*)(ld + 32 + 8 * j + 4 * half);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nl[4 * j + i] = a[i];
        nd[4 * j + i] = e[i];
      }
    }
    f32x16 sc[NH], dp[NH];
    bf16x8 pa[NH][2], sa[NH][2];
    bf16x8 gtr[2][DB], qtr[2][DB];
    auto sdp = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bf16x8 kf, vf;
        if constexpr (D <= 64) {
          kf = kreg[s];
          vf = vreg[s];
        } else {
          kf = *(const bf16x8*)(kvl[0] + 32 * h * ROWB + k_off[s]);
          vf = *(const bf16x8*)(kvl[1] + 32 * h * ROWB + k_off[s]);
        }
        sc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kf, s ? sc[h] : nl, 0, 0, 0);
        dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[s], vf, s ? dp[h] : nd, 0, 0, 0);
      }
    };
    // The mask is a real branch taken on the tiles that need it (one path
    // through the loop body: two copies made the compiler copy the dK and
    // dV accumulators between them on every tile).
    auto mask = [&](const int h) __attribute__((always_inline)) {
      if (masked) {
        __asm__ volatile("" ::: "memory");  // keep this a branch
        const int lim = (key0 + 32 * h + l32) * kk;  // rows below this cannot see the lane's key
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int r = tr0 + 8 * (t >> 2) + 4 * half + (t & 3);
          if (r >= R || r < lim) sc[h][t] = -INFINITY;
        }
      }
    };
    auto soft = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 16; t += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sc[h][t]), p1 = __builtin_amdgcn_exp2f(sc[h][t + 1]);
        pa[h][t >> 3][t & 7] = f2bf(p0);
        pa[h][t >> 3][(t & 7) + 1] = f2bf(p1);
        sa[h][t >> 3][t & 7] = f2bf(p0 * dp[h][t]);
        sa[h][t >> 3][(t & 7) + 1] = f2bf(p1 * dp[h][t + 1]);
      }
    };
    auto reads_tr = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          gtr[st][db] = tr.read(gt, st, db);
          qtr[st][db] = tr.read(qt, st, db);
        }
    };
    auto dvdk = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[h][st], gtr[st][db], dv[h][db], 0, 0, 0);
          dk[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[h][st], qtr[st][db], dk[h][db], 0, 0, 0);
        }
    };
    // (d = 128 reads the transposed fragments after S and dP: 64 more live
    // registers during those products would not fit)
    if constexpr (D <= 64) reads_tr();
    sdp(0);
    if constexpr (D > 64) reads_tr();
    mask(0);
    soft(0);
    dvdk(0);
  };

  if (ntw > 0) {
    dma(0, 0);
    dma(1, 1);
    for (int i = 0; i < ntw; ++i) {
      const int bf = i & 1;
      const int tr0 = row0 + 32 * (wave + 4 * i);
      // tile i is complete once only tile i+1's loads remain in flight; a
      // wavefront reads only what its own loads wrote
      __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory");
      // rows below (last key)*kk, or past the end, need the mask
      tile(bf, tr0, tr0 < (key0 + KB - 1) * kk || tr0 + 32 > R);
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of bf done before it is refilled
      dma(i + 2, bf);
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA may outlive the rings
  }

  // Sum the four wavefronts' partials through LDS and store.
  float* red = (float*)&lds[0][0][0];
  auto reduce_store = [&](f32x16(&acc)[NH][DB], const int which, const float mul) __attribute__((always_inline)) {
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t)
          red[(wave * KB + 32 * h + 8 * (t >> 2) + 4 * half + (t & 3)) * D + 32 * db + l32] = acc[h][db][t];
    __syncthreads();
    for (int e = tid; e < KB * D / 4; e += 256) {
      f32x4 sum = *(const f32x4*)(red + 4 * e);
#pragma unroll
      for (int w = 1; w < 4; ++w) sum += *(const f32x4*)(red + w * KB * D + 4 * e);
      sum *= mul;
      const int j = key0 + (4 * e) / D, col = (4 * e) % D;
      if (j >= f.S) continue;
      if (v == 0 || v == f.G) {
        float* dst = p.part + ((((int64_t)which * 2 + (v == f.G)) * f.B + b) * f.S + j) * D + col;
        *(f32x4*)dst = sum;
      } else {
        __bf16* dst = (__bf16*)(which ? p.dv : p.dk) + (((int64_t)b * f.G + v) * f.S + j) * D + col;
        const bf16x4 o = {f2bf(sum[0]), f2bf(sum[1]), f2bf(sum[2]), f2bf(sum[3])};
        *(bf16x4*)dst = o;
      }
    }
  };
  reduce_store(dk, 0, 0.69314718055994531f);  // dS^T Q' carries scale*log2(e); dK needs scale
  reduce_store(dv, 1, 1.f);
}

// ---------------------------------------------------------------------------
// 3. dQ (bf16)
// ---------------------------------------------------------------------------
// The forward's tiles: 256 rows of one (b, v), RH 32-row halves per
// wavefront. Per 64-key block (in LDS) and 32-key half sb:
//   S^T = K Q'^T - lse*log2(e),  dP^T = V dO^T - delta   (lane (half, l32)
//   holds row l32, so both offsets are per-lane initial accumulators)
//   P = exp2(S^T),  dS^T = P dP^T,  dQ^T += K^T dS^T   (K^T from
//   transposing LDS reads)
// A wavefront owns 32 rows (eight wavefronts) so that its working set fits
// 128 VGPRs (d = 64) and four wavefronts share a SIMD; d = 32 takes two
// 32-row halves per wavefront (four wavefronts: its K/V blocks are too small
// to split over eight), which then run as four phases: S^T, dP^T of half 0 |
// S^T, dP^T of half 1 beside half 0's exponentials | dQ of half 0 beside
// half 1's exponentials | dQ of half 1.
template <int D>
__global__ __launch_bounds__(D == 32 ? 256 : 512) void bwd_dq_kernel(BwdParams p, int tiles_r, int tiles_s) {
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
  constexpr int RH = D == 32 ? 2 : 1;  // 32-row halves per wavefront
  constexpr int NW = 8 / RH;           // wavefronts: 256 rows per workgroup
  constexpr int KS = D / 16, DB = D / 32, ROWB = 2 * D;
  constexpr int MATB = kKeyBlock * ROWB;  // one K or V block
  constexpr int NPW = MATB / 1024 / NW;   // 1 KiB LDS-DMA chunks per wavefront per matrix
  static_assert(NPW >= 1, "block too small for the LDS-DMA split");
  constexpr int RPC = 1024 / ROWB;
  constexpr int NBUF = 4;
  __shared__ __attribute__((aligned(1024))) char lds[NBUF][2][MATB];  // [buffer][K, V]

  const PrefillParams& f = p.f;
  const TileCoord tc = tile_of_block(f, tiles_r, tiles_s);
  if (!tc.valid) return;
  const int b = tc.b, v = tc.v;
  const int kvh = (v == f.G) ? 0 : v;
  const int nrows = (v == f.G) ? f.S : f.S * f.K;
  const int r0 = tc.tile * 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int last_r = min(r0 + 256, nrows) - 1;
  int pos_last, pos_first, s_, h_;
  row_info(f, b, v, last_r, pos_last, s_, h_);
  row_info(f, b, v, r0, pos_first, s_, h_);
  const int64_t pbase = ((int64_t)b * (f.G + 1) + v) * p.Rp;

  // Q' and dO rows (B operands): lane (half, l32) holds row l32 of half h,
  // d 16s + 8 half .. +7; the row's offsets as pinned 16-register tuples
  // (the MFMAs' initial accumulators).
  // (d = 128 keeps the offsets as scalars and adds them in the softmax: its
  // register budget has no room for the tuples)
  constexpr bool TUPLES = RH == 2;
  int pos[RH], slot[RH], head[RH];
  bool row_ok[RH];
  bf16x8 qf[RH][KS], gf[RH][KS];
  f32x16 bl[RH] = {}, bd[RH] = {};
  float nls[RH], nds[RH];
#pragma unroll
  for (int h = 0; h < RH; ++h) {
    const int r = r0 + wave * 32 * RH + h * 32 + l32;
    row_ok[h] = r < nrows;
    const int rr = row_ok[h] ? r : last_r;
    row_info(f, b, v, rr, pos[h], slot[h], head[h]);
    const __bf16* qrow = (const __bf16*)p.qp + (pbase + rr) * D;
    const __bf16* grow = (const __bf16*)p.dop + (pbase + rr) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[h][s] = *(const bf16x8*)(qrow + 16 * s + 8 * half);
      gf[h][s] = *(const bf16x8*)(grow + 16 * s + 8 * half);
    }
    nls[h] = p.nlse[pbase + rr];
    nds[h] = p.ndel[pbase + rr];
    if constexpr (TUPLES) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        __asm__("v_mov_b32 %0, %1" : "+v"(bl[h][j]) : "v"(nls[h]));
        __asm__("v_mov_b32 %0, %1" : "+v"(bd[h][j]) : "v"(nds[h]));
      }
    }
  }
  // wait for these loads before the LDS-DMA loop (see the dK/dV kernel)
#pragma unroll
  for (int h = 0; h < RH; ++h) {
#pragma unroll
    for (int s = 0; s < KS; ++s) __asm__ volatile("" ::"v"(qf[h][s]), "v"(gf[h][s]));
    __asm__ volatile("" ::"v"(pos[h]), "v"(head[h]), "v"(nls[h]), "v"(nds[h]));
  }

  const __bf16* kbase = (const __bf16*)f.k + ((int64_t)b * f.G + kvh) * (int64_t)f.S * D;
  const __bf16* vbase = (const __bf16*)f.v + ((int64_t)b * f.G + kvh) * (int64_t)f.S * D;
  const int nblocks = pos_last / kKeyBlock + 1;
  const int dma_r = (16 * lane) / ROWB;
  const int dma_p = ((16 * lane) % ROWB) / 16;
  uint32_t dma_off[NPW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int rb = (wave * NPW + i) * RPC + dma_r;
    dma_off[i] = rb * ROWB + 16 * (dma_p ^ tile_swz<D>(rb));
  }
  auto dma = [&](const int kb, const int bf) __attribute__((always_inline)) {
    if ((kb + 1) * kKeyBlock <= f.S) {
      const __bf16* kblk = kbase + (int64_t)kb * kKeyBlock * D;
      const __bf16* vblk = vbase + (int64_t)kb * kKeyBlock * D;
#pragma unroll
      for (int i = 0; i < NPW; ++i) {
        const int n = wave * NPW + i;
        lds_dma16_s(kblk, dma_off[i], lds[bf][0] + n * 1024);
        lds_dma16_s(vblk, dma_off[i], lds[bf][1] + n * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPW; ++i) {
        const int n = wave * NPW + i;
        const int rb = n * RPC + dma_r;
        const int row = min(kb * kKeyBlock + rb, f.S - 1);  // keys past the end re-read the last (masked)
        const int64_t g = (int64_t)row * D + 8 * (dma_p ^ tile_swz<D>(rb));
        lds_dma16(kbase + g, lds[bf][0] + n * 1024);
        lds_dma16(vbase + g, lds[bf][1] + n * 1024);
      }
    }
  };

  int k_off[KS];  // key row l32, chunk 2s + half
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = l32 * ROWB + 16 * ((2 * s + half) ^ tile_swz<D>(l32));
  const TrOffsets<D> tr(lane);

  f32x16 dq[RH][DB];
#pragma unroll
  for (int h = 0; h < RH; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 16; ++t) dq[h][db][t] = 0.f;

  // The mask is a real branch taken on the blocks that need it (one path
  // through the loop body, as in the dK/dV kernel).
  auto block = [&](const int j, const int buf, const bool masked) __attribute__((always_inline)) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const char* kt = lds[buf][0] + sb * 32 * ROWB;
      const char* vt = lds[buf][1] + sb * 32 * ROWB;
      bf16x8 ka[KS], va[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[s] = *(const bf16x8*)(kt + k_off[s]);
        va[s] = *(const bf16x8*)(vt + k_off[s]);
      }
      f32x16 sc[RH], dp[RH];
      bf16x8 ds16[RH][2];
      bf16x8 ktr[2][DB];
      auto sdp = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const f32x16 zero16 = {};
          sc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qf[h][s], s ? sc[h] : (TUPLES ? bl[h] : zero16), 0,
                                                          0, 0);
          dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[s], gf[h][s], s ? dp[h] : (TUPLES ? bd[h] : zero16), 0,
                                                          0, 0);
        }
      };
      auto mask = [&](const int h) __attribute__((always_inline)) {
        if (masked) {
          __asm__ volatile("" ::: "memory");  // keep this a branch
          // element t <-> key j*64 + sb*32 + 8(t/4) + 4 half + t%4
          const int lim = pos[h] - j * kKeyBlock - sb * 32 - 4 * half;
#pragma unroll
          for (int t = 0; t < 16; ++t)
            if (8 * (t >> 2) + (t & 3) > lim) sc[h][t] = -INFINITY;
        }
      };
      auto soft = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 16; t += 2) {
          float s0 = sc[h][t], s1 = sc[h][t + 1], d0 = dp[h][t], d1 = dp[h][t + 1];
          if constexpr (!TUPLES) {  // (x + 0 is not folded away, so only add when needed)
            s0 += nls[h];
            s1 += nls[h];
            d0 += nds[h];
            d1 += nds[h];
          }
          const float p0 = __builtin_amdgcn_exp2f(s0), p1 = __builtin_amdgcn_exp2f(s1);
          ds16[h][t >> 3][t & 7] = f2bf(p0 * d0);
          ds16[h][t >> 3][(t & 7) + 1] = f2bf(p1 * d1);
        }
      };
      auto reads_tr = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < DB; ++db) ktr[st][db] = tr.read(kt, st, db);
      };
      auto dq_mfma = [&](const int h) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dq[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktr[st][db], ds16[h][st], dq[h][db], 0, 0, 0);
      };
      if constexpr (RH == 2) {
        sdp(0);
        mask(0);
        __builtin_amdgcn_sched_barrier(0);
        sdp(1);
        soft(0);
        reads_tr();
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mask(1);
        dq_mfma(0);
        soft(1);
#pragma unroll
        for (int i = 0; i < 2 * DB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        dq_mfma(1);
      } else {
        sdp(0);
        mask(0);
        soft(0);
        reads_tr();
        dq_mfma(0);
      }
    }
  };

  dma(0, 0);
  dma(min(1, nblocks - 1), 1);
  dma(min(2, nblocks - 1), 2);
  const int nfull = min((pos_first + 1) / kKeyBlock, nblocks);  // blocks no row of the tile needs masked
  for (int j = 0; j < nblocks; ++j) {
    // blocks j+1 and j+2 stay in flight; the barrier publishes block j and
    // tells that every wavefront has left block j-1, whose buffer block j+3
    // then takes (past the last block it re-loads that one)
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * NPW) : "memory");
    __syncthreads();
    dma(min(j + 3, nblocks - 1), (j + 3) % NBUF);
    block(j, j % NBUF, j >= nfull);
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int h = 0; h < RH; ++h) {
    if (!row_ok[h]) continue;
    __bf16* out = (__bf16*)p.dq + (((int64_t)b * f.S + pos[h]) * (f.N + 1) + head[h]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = f2bf(dq[h][db][4 * jq + i] * f.scale);
        *(bf16x4*)(out + db * 32 + 8 * jq + 4 * half) = o4;
      }
  }
}

// ---------------------------------------------------------------------------
// 4. KV head 0: routed group 0 plus shared head
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdParams p, int D) {
  const PrefillParams& f = p.f;
  const int64_t per = (int64_t)f.S * D, n4 = (int64_t)f.B * per / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const int64_t e = 4 * i, b = e / per, rest = e - b * per;
  const int64_t plane = (int64_t)f.B * per;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const f32x4 a = *(const f32x4*)(p.part + (2 * which) * plane + e);
    const f32x4 s = *(const f32x4*)(p.part + (2 * which + 1) * plane + e);
    const f32x4 t = a + s;
    __bf16* dst = (__bf16*)(which ? p.dv : p.dk) + b * f.G * per + rest;
    const bf16x4 o = {f2bf(t[0]), f2bf(t[1]), f2bf(t[2]), f2bf(t[3])};
    *(bf16x4*)dst = o;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: plain VALU arithmetic on the packed rows
// ---------------------------------------------------------------------------
// dQ: one wavefront per row; lanes over keys for s, dP and dS, lanes over d
// for the sum of dS_j k_j.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(BwdParams p) {
  const PrefillParams& f = p.f;
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows_r = (int64_t)f.S * f.K, per_b = f.G * rows_r + f.S;
  if (grow >= f.B * per_b) return;
  const int b = (int)(grow / per_b);
  const int64_t rem = grow - b * per_b;
  const int v = rem < f.G * rows_r ? (int)(rem / rows_r) : f.G;
  const int r = (int)(v == f.G ? rem - f.G * rows_r : rem - v * rows_r);
  int pos, slot, head;
  row_info(f, b, v, r, pos, slot, head);
  const int kvh = (v == f.G) ? 0 : v;
  const int64_t prow = ((int64_t)b * (f.G + 1) + v) * p.Rp + r;
  const float* q = (const float*)p.qp + prow * D;
  const float* g = (const float*)p.dop + prow * D;
  const float nl = p.nlse[prow], nd = p.ndel[prow];
  const float* K = (const float*)f.k + ((int64_t)b * f.G + kvh) * (int64_t)f.S * D;
  const float* V = (const float*)f.v + ((int64_t)b * f.G + kvh) * (int64_t)f.S * D;
  constexpr int DL = (D + 63) / 64;
  float dq[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) dq[i] = 0.f;
  for (int j0 = 0; j0 <= pos; j0 += 64) {
    const int j = j0 + lane;
    float ds = 0.f;
    if (j <= pos) {
      float sacc = 0.f, dpacc = 0.f;
      for (int e = 0; e < D; ++e) {
        sacc = fmaf(q[e], K[(int64_t)j * D + e], sacc);
        dpacc = fmaf(g[e], V[(int64_t)j * D + e], dpacc);
      }
      const float pj = expf((sacc + nl) * f.scale);  // exp(s - lse)
      ds = pj * (dpacc + nd);
    }
    const int nk = min(64, pos + 1 - j0);
    for (int t = 0; t < nk; ++t) {
      const float dst = __shfl(ds, t, 64);
#pragma unroll
      for (int i = 0; i < DL; ++i) {
        const int e = lane + 64 * i;
        if (e < D) dq[i] = fmaf(dst, K[(int64_t)(j0 + t) * D + e], dq[i]);
      }
    }
  }
  float* out = (float*)p.dq + (((int64_t)b * f.S + pos) * (f.N + 1) + head) * D;
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    const int e = lane + 64 * i;
    if (e < D) out[e] = dq[i] * f.scale;
  }
}

// dK, dV: one wavefront per key j of KV head g; lanes over rows (the routed
// rows of group g from row j*k on and, for g = 0, the shared rows from j on),
// then lanes over d for the sums over rows.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(BwdParams p) {
  const PrefillParams& f = p.f;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= (int64_t)f.B * f.G * f.S) return;
  const int j = (int)(gw % f.S);
  const int g = (int)((gw / f.S) % f.G);
  const int b = (int)(gw / ((int64_t)f.S * f.G));
  const int64_t kvrow = (((int64_t)b * f.G + g) * f.S + j) * D;
  const float* kj = (const float*)f.k + kvrow;
  const float* vj = (const float*)f.v + kvrow;
  constexpr int DL = (D + 63) / 64;
  float dk[DL], dv[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) dk[i] = dv[i] = 0.f;
  auto rows = [&](const int v, const int rstart, const int R) {
    const int64_t pb = ((int64_t)b * (f.G + 1) + v) * p.Rp;
    const float* Q = (const float*)p.qp + pb * D;
    const float* Gd = (const float*)p.dop + pb * D;
    for (int r0 = rstart; r0 < R; r0 += 64) {
      const int r = r0 + lane;
      float pj = 0.f, ds = 0.f;
      if (r < R) {
        float sacc = 0.f, dpacc = 0.f;
        for (int e = 0; e < D; ++e) {
          sacc = fmaf(Q[(int64_t)r * D + e], kj[e], sacc);
          dpacc = fmaf(Gd[(int64_t)r * D + e], vj[e], dpacc);
        }
        pj = expf((sacc + p.nlse[pb + r]) * f.scale);
        ds = pj * (dpacc + p.ndel[pb + r]);
      }
      const int nr = min(64, R - r0);
      for (int t = 0; t < nr; ++t) {
        const float pt = __shfl(pj, t, 64), dst = __shfl(ds, t, 64);
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          const int e = lane + 64 * i;
          if (e < D) {
            dk[i] = fmaf(dst, Q[(int64_t)(r0 + t) * D + e], dk[i]);
            dv[i] = fmaf(pt, Gd[(int64_t)(r0 + t) * D + e], dv[i]);
          }
        }
      }
    }
  };
  rows(g, j * f.K, f.S * f.K);
  if (g == 0) rows(f.G, j, f.S);
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    const int e = lane + 64 * i;
    if (e < D) {
      ((float*)p.dk)[kvrow + e] = dk[i] * f.scale;
      ((float*)p.dv)[kvrow + e] = dv[i];
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D>
static void launch_prep(const BwdParams& p, hipStream_t s) {
  constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
  const int64_t rows = (int64_t)p.f.B * (p.f.G + 1) * p.Rp;
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
}

template <int D>
static void launch_bf16(const BwdParams& p, hipStream_t s) {
  const PrefillParams& f = p.f;
  launch_prep<__bf16, D>(p, s);
  constexpr int KB = 32;
  const int nkb = (f.S + KB - 1) / KB;
  const int nchunks = ((nkb + kBwdChunk - 1) / kBwdChunk) * f.B * (f.G + 1);
  const unsigned ng = 8u * kBwdChunk * (unsigned)((nchunks + 7) / 8);
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(ng), dim3(256), 0, s, p, nkb);
  const int tiles_r = (f.S * f.K + 255) / 256, tiles_s = (f.S + 255) / 256;
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(tile_grid_blocks(f, tiles_s)), dim3(D == 32 ? 256 : 512), 0, s, p,
                     tiles_r, tiles_s);
  const int64_t n4 = (int64_t)f.B * f.S * D / 4;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, p, D);
}

template <int D>
static void launch_f32(const BwdParams& p, hipStream_t s) {
  const PrefillParams& f = p.f;
  launch_prep<float, D>(p, s);
  const int64_t rows = (int64_t)f.B * ((int64_t)f.G * f.S * f.K + f.S);
  hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
  const int64_t keys = (int64_t)f.B * f.G * f.S;
  hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, dim3((unsigned)((keys + 3) / 4)), dim3(256), 0, s, p);
}

hipError_t launch_prefill_bwd(const BwdParams& p, int d, bool bf16, hipStream_t s) {
  switch (d) {
    case 32: bf16 ? launch_bf16<32>(p, s) : launch_f32<32>(p, s); break;
    case 64: bf16 ? launch_bf16<64>(p, s) : launch_f32<64>(p, s); break;
    case 128: bf16 ? launch_bf16<128>(p, s) : launch_f32<128>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqe
