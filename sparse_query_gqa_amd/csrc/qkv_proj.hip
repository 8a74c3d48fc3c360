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
// Work is split into tiles of one head's d output columns by a set of token
// rows. A routed query head takes its rows from the token list of its
// (sequence, group, expert), which the router builds, so no row of an
// unselected head is ever computed; the shared head, K and V take
// contiguous token ranges. Tile kinds:
//   * prefill (large T): 256-row tiles on v_mfma_f32_32x32x16_bf16, x rows
//     gathered straight into LDS by LDS-DMA, k in steps of 32 through a
//     four-stage ring;
//   * decode (few tokens, bound by reading the weights): 32-row tiles whose
//     routed rows are found by scanning the tokens' top-k, the model width
//     split over the four wavefronts, fragments loaded from global memory,
//     partial sums reduced in LDS. Keys and values go to cache row
//     kv_len[b] - q_len + t.
//   * fp32: plain VALU code, one thread per output value.
#include "gqe_internal.h"

namespace gqe {

namespace {

constexpr int kPRows = 256;  // token rows per prefill tile (4 wavefronts x 64)
constexpr int kPK = 32;      // k per stage
constexpr int kPStages = 4;
constexpr int kDRows = 32;   // token rows per decode tile

// Output row of token ft for head slot `which` (0..N query heads, then K
// heads g = 0..G-1, then V heads): the element offset of column 0.
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
// Prefill tiles. Blocks are laid out per XCD (block i runs on XCD i % 8):
// logical tile j = (i % 8) * per + i / 8, so consecutive logical tiles share
// an XCD and its L2. Logical tiles are the contiguous-row tiles first, the
// 2G+1 heads of one token range next to each other (x read once into that
// L2), then the routed-query tiles, per (sequence, group) an upper bound of
// ceil(k*S/256) + M tiles of which the tiles past the lists' real count exit.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void proj_prefill_kernel(ProjParams p, int n_row_tiles,
                                                                            int e_per_bg, int per) {
  constexpr int CB = D / 32;              // 32-column blocks of the head
  constexpr int XB = kPRows * kPK * 2;    // x stage: 256 rows x 64 bytes
  constexpr int WB = D * kPK * 2;         // W stage: d rows x 64 bytes
  constexpr int SB = XB + WB;
  constexpr int XCH = XB / 1024 / 4;      // 1 KiB x chunks per wavefront per stage
  constexpr int WCH = WB / 1024;          // 1 KiB W chunks per stage (2, 4 or 8)
  constexpr int WPW = WCH >= 4 ? WCH / 4 : 1;  // W chunks per wavefront (re-loaded when WCH < 4)
  __shared__ __attribute__((aligned(1024))) char lds[kPStages * SB];
  __shared__ int rows[kPRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int j = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const int heads_r = 2 * p.G + 1;  // shared query head, G key heads, G value heads
  int which, nrows;
  if (j < n_row_tiles * heads_r) {
    const int rt = j / heads_r, hs = j - rt * heads_r;
    which = hs == 0 ? p.N : p.N + hs;
    const int t0 = rt * kPRows;
    nrows = min(kPRows, p.T - t0);
    rows[tid] = t0 + min(tid, nrows - 1);
  } else {
    const int e = j - n_row_tiles * heads_r;
    const int bg = e / e_per_bg;
    if (bg >= p.B * p.G) return;
    int r = e - bg * e_per_bg;
    const int b = bg / p.G, g = bg - b * p.G;
    const int32_t* off = p.list_off + (int64_t)bg * (p.M + 1);
    int m = 0, n = 0;
    for (; m < p.M; ++m) {
      n = off[m + 1] - off[m];
      const int tiles = (n + kPRows - 1) / kPRows;
      if (r < tiles) break;
      r -= tiles;
    }
    if (m == p.M) return;  // past this (sequence, group)'s real tile count
    which = g * p.M + m;
    nrows = min(kPRows, n - r * kPRows);
    const int32_t* lt = p.list_tok + (int64_t)bg * p.K * p.L + off[m] + r * kPRows;
    rows[tid] = b * p.L + lt[min(tid, nrows - 1)];
  }
  __syncthreads();

  const __bf16* xg = (const __bf16*)p.x;
  const __bf16* wh = head_weights(p, which);
  // LDS layout per stage: row r at r*64 bytes, 16-byte chunk c at position
  // c ^ ((r >> 2) & 3), so the 16 rows of a 16-byte fragment read fall on
  // distinct bank groups. DMA: lane l of a 1 KiB chunk writes row l/4,
  // position l%4, loading the chunk the swizzle puts there.
  const int dr = lane >> 2, dp = lane & 3;
  const __bf16* xsrc[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int r = (wave * XCH + i) * 16 + dr;
    xsrc[i] = xg + (int64_t)rows[r] * p.D + 8 * (dp ^ ((r >> 2) & 3));
  }
  uint32_t woff[WPW];
#pragma unroll
  for (int i = 0; i < WPW; ++i) {
    const int n = (wave * WPW + i) % WCH;
    const int r = n * 16 + dr;
    woff[i] = (uint32_t)(r * p.D + 8 * (dp ^ ((r >> 2) & 3))) * 2;
  }
  const int nk = p.D / kPK;
  auto dma = [&](const int ks, const int st) __attribute__((always_inline)) {
    const int kk = min(ks, nk - 1) * kPK;  // past the end: re-load the last stage (not read)
    char* sb = lds + st * SB;
#pragma unroll
    for (int i = 0; i < XCH; ++i) lds_dma16(xsrc[i] + kk, sb + (wave * XCH + i) * 1024);
#pragma unroll
    for (int i = 0; i < WPW; ++i) lds_dma16_s(wh + kk, woff[i], sb + XB + ((wave * WPW + i) % WCH) * 1024);
  };

  // fragments: W rows 32*cb + l32 (A operand), x rows 64*wave + 32*rb + l32
  // (B operand), chunk 2*ks + half of the stage
  int w_off[2], x_off[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    w_off[ks] = l32 * 64 + 16 * ((2 * ks + half) ^ ((l32 >> 2) & 3));
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = 64 * wave + 32 * rb + l32;
      x_off[rb][ks] = r * 64 + 16 * ((2 * ks + half) ^ ((r >> 2) & 3));
    }
  }
  f32x16 acc[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[cb][rb][e] = 0.f;

#pragma unroll
  for (int s = 0; s < kPStages - 1; ++s) dma(s, s);
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks % kPStages;
    // stage ks is complete when at most the two later stages' loads are
    // outstanding; the barrier publishes it and frees the stage read in step
    // ks-1 for step ks+3
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (XCH + WPW)) : "memory");
    __syncthreads();
    dma(ks + kPStages - 1, (ks + kPStages - 1) % kPStages);
    const char* sb = lds + st * SB;
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      bf16x8 wf[CB], xf[2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) wf[cb] = *(const bf16x8*)(sb + XB + cb * 32 * 64 + w_off[kq]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) xf[rb] = *(const bf16x8*)(sb + x_off[rb][kq]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb], xf[rb], acc[cb][rb], 0, 0, 0);
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA may outlive the workgroup

  // lane (half, l32) of tile (cb, rb) holds token row 64*wave + 32*rb + l32
  // and columns 32*cb + 8*(e/4) + 4*half + e%4
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 64 * wave + 32 * rb + l32;
    if (r >= nrows) continue;
    int kind;
    const int64_t o = out_row(p, which, rows[r], kind);
    __bf16* out = (__bf16*)out_base(p, kind) + o;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = f2bf(acc[cb][rb][4 * jq + e]);
        *(bf16x4*)(out + 32 * cb + 8 * jq + 4 * half) = o4;
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
  ((float*)out_base(p, kind))[o + c] = s;
}

// Decode tiles: head slot blockIdx.y, chunk blockIdx.x of 32 tokens (flat
// index b*q_len + t). A routed head keeps the chunk's tokens whose top-k
// holds it (a ballot, in token order); other slots keep every token. The
// four wavefronts each take a quarter of the model width; fragments come
// straight from global memory (the weights are read once, x stays in L2),
// and the partial tiles are summed in LDS in a fixed order.
template <int D>
__global__ __launch_bounds__(256) void proj_decode_kernel(ProjParams p) {
  constexpr int CB = D / 32;
  constexpr int U = 4;  // k-steps of loads in flight per wavefront
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
  const __bf16* wh = head_weights(p, which) + (int64_t)l32 * p.D + 8 * half;
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
    __bf16* out = (__bf16*)out_base(p, kind) + o;
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
    const dim3 grid((unsigned)((p.T + kDRows - 1) / kDRows), (unsigned)heads);
    switch (p.d) {
      case 32: hipLaunchKernelGGL(proj_decode_kernel<32>, grid, dim3(256), 0, s, p); break;
      case 64: hipLaunchKernelGGL(proj_decode_kernel<64>, grid, dim3(256), 0, s, p); break;
      case 128: hipLaunchKernelGGL(proj_decode_kernel<128>, grid, dim3(256), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int n_row_tiles = (p.T + kPRows - 1) / kPRows;
  const int e_per_bg = (p.K * p.L + kPRows - 1) / kPRows + p.M;
  const int64_t total = (int64_t)n_row_tiles * (2 * p.G + 1) + (int64_t)p.B * p.G * e_per_bg;
  const int per = (int)((total + 7) / 8);
  const unsigned nblk = (unsigned)(8 * per);
  switch (p.d) {
    case 32: hipLaunchKernelGGL(proj_prefill_kernel<32>, dim3(nblk), dim3(256), 0, s, p, n_row_tiles, e_per_bg, per); break;
    case 64: hipLaunchKernelGGL(proj_prefill_kernel<64>, dim3(nblk), dim3(256), 0, s, p, n_row_tiles, e_per_bg, per); break;
    case 128: hipLaunchKernelGGL(proj_prefill_kernel<128>, dim3(nblk), dim3(256), 0, s, p, n_row_tiles, e_per_bg, per); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqe
