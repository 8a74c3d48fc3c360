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
//   * prefill (large T): windows of 256 tokens, each with 128-column dense
//     tiles and one routed tile per query head, on v_mfma_f32_32x32x16_bf16;
//     x rows go straight into LDS by LDS-DMA, k in steps of 32 through a
//     three-stage ring;
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
constexpr int kPStages = 3;
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
// Prefill tiles, by window of 256 consecutive tokens (flat index b*S + s).
// A window has ceil((2G+1)*d / 128) dense tiles over the columns [shared
// query head | G key heads | G value heads], 128 columns each, and N routed
// tiles, one per query head h = g*M + m, whose rows are the window's tokens
// with m in their group-g top-k: a ballot over the window in token order,
// which is the order of the expert-major token lists. Wavefronts skip the
// 32-row blocks past a routed tile's row count, so the work follows the
// selected rows. The tiles of a window are consecutive logical tiles, and
// consecutive logical tiles run on one XCD (block i on XCD i % 8, logical
// tile (i % 8) * per + i / 8), so the window's x rows come from HBM once and
// then from that XCD's L2.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void proj_prefill_kernel(ProjParams p, int tiles_pw, int n_dense, int per) {
  constexpr int TC = 128;                 // columns of a dense tile
  constexpr int CB = TC / 32;             // 32-column blocks (a routed tile uses D / 32)
  constexpr int XB = kPRows * kPK * 2;    // x stage: 256 rows x 64 bytes
  constexpr int WB = TC * kPK * 2;        // W stage: 128 rows x 64 bytes
  constexpr int SB = XB + WB;
  constexpr int XCH = XB / 1024 / 4;      // 1 KiB x chunks per wavefront per stage
  constexpr int WCH = WB / 1024 / 4;      // 1 KiB W chunks per wavefront per stage
  __shared__ __attribute__((aligned(1024))) char lds[kPStages * SB];
  __shared__ int rows[kPRows];
  __shared__ int wcount[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int j = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const int win = j / tiles_pw, kt = j - win * tiles_pw;
  const int t0 = win * kPRows;
  if (t0 >= p.T) return;
  const int nwin = min(kPRows, p.T - t0);
  const int ncols = (2 * p.G + 1) * D;  // dense columns
  int c0 = 0, qhead = -1, ncb, nrows;
  if (kt < n_dense) {
    c0 = kt * TC;
    ncb = min(CB, (ncols - c0) / 32);
    nrows = nwin;
    rows[tid] = t0 + min(tid, nwin - 1);
  } else {
    qhead = kt - n_dense;
    ncb = D / 32;
    const int g = qhead / p.M, m = qhead - g * p.M;
    const int ft = t0 + tid;
    bool keep = tid < nwin;
    if (keep) {
      bool chose = false;
      for (int s = 0; s < p.K; ++s) chose |= p.topk[((int64_t)ft * p.G + g) * p.K + s] == m;
      keep = chose;
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
    if (lane == 0) wcount[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wave; ++i) base += wcount[i];
    nrows = wcount[0] + wcount[1] + wcount[2] + wcount[3];
    if (keep) rows[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] = ft;
    if (nrows == 0) return;  // uniform: no token of the window picked this head
  }
  __syncthreads();

  // LDS layout per stage: row r at r*64 bytes, 16-byte chunk c at position
  // c ^ ((r >> 2) & 3), so the 16 rows of a 16-byte fragment read fall on
  // distinct bank groups. DMA: lane l of a 1 KiB chunk writes row l/4,
  // position l%4, loading the chunk the swizzle puts there. Rows past the
  // tile's count re-load its last row (not stored); so do W rows past the
  // tile's columns.
  const int dr = lane >> 2, dp = lane & 3;
  const __bf16* xsrc[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int r = (wave * XCH + i) * 16 + dr;
    xsrc[i] = (const __bf16*)p.x + (int64_t)rows[min(r, nrows - 1)] * p.D + 8 * (dp ^ ((r >> 2) & 3));
  }
  const __bf16* wsrc[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int r = (wave * WCH + i) * 16 + dr;
    const int chunk = 8 * (dp ^ ((r >> 2) & 3));
    const __bf16* row;
    if (qhead >= 0) {
      row = (const __bf16*)p.w_q + ((int64_t)qhead * D + min(r, D - 1)) * p.D;
    } else {
      const int c = min(c0 + r, ncols - 1);
      if (c < D) row = (const __bf16*)p.w_q + ((int64_t)p.N * D + c) * p.D;
      else if (c < D + p.G * D) row = (const __bf16*)p.w_k + (int64_t)(c - D) * p.D;
      else row = (const __bf16*)p.w_v + (int64_t)(c - D - p.G * D) * p.D;
    }
    wsrc[i] = row + chunk;
  }
  const int nk = p.D / kPK;
  auto dma = [&](const int ks, const int st) __attribute__((always_inline)) {
    const int kk = min(ks, nk - 1) * kPK;  // past the end: re-load the last stage (not read)
    char* sb = lds + st * SB;
#pragma unroll
    for (int i = 0; i < XCH; ++i) lds_dma16(xsrc[i] + kk, sb + (wave * XCH + i) * 1024);
#pragma unroll
    for (int i = 0; i < WCH; ++i) lds_dma16(wsrc[i] + kk, sb + XB + (wave * WCH + i) * 1024);
  };

  // fragments: W rows 32*cb + l32 (A operand), x rows 32*(wave + 4*rb) + l32
  // (B operand: row blocks interleaved over the wavefronts, so a routed tile
  // that is half full still keeps all four busy), chunk 2*kq + half
  const int sw = (l32 >> 2) & 3;
  int w_off[2], x_off[2][2];
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    w_off[kq] = l32 * 64 + 16 * ((2 * kq + half) ^ sw);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) x_off[rb][kq] = (32 * (wave + 4 * rb) + l32) * 64 + 16 * ((2 * kq + half) ^ sw);
  }
  // 32-row blocks of this wavefront that hold selected rows (uniform)
  const bool rb_on0 = 32 * wave < nrows, rb_on1 = 32 * (wave + 4) < nrows;
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
    // stage ks is complete when at most the next stage's loads are
    // outstanding; the barrier publishes it and frees the stage read in step
    // ks-1 for step ks+2
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(XCH + WCH) : "memory");
    __syncthreads();
    dma(ks + kPStages - 1, (ks + kPStages - 1) % kPStages);
    if (!rb_on0) continue;
    const char* sb = lds + st * SB;
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      bf16x8 wf[CB], xf[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) xf[rb] = *(const bf16x8*)(sb + x_off[rb][kq]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (cb >= ncb) break;
        wf[cb] = *(const bf16x8*)(sb + XB + cb * 32 * 64 + w_off[kq]);
        acc[cb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb], xf[0], acc[cb][0], 0, 0, 0);
        if (rb_on1) acc[cb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb], xf[1], acc[cb][1], 0, 0, 0);
      }
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA may outlive the workgroup

  // lane (half, l32) of tile (cb, rb) holds token row 32*(wave + 4*rb) + l32
  // and columns 32*cb + 8*(e/4) + 4*half + e%4
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 32 * (wave + 4 * rb) + l32;
    if (r >= nrows) continue;
    const int ft = rows[r];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if (cb >= ncb) break;
      int which, col;
      if (qhead >= 0) {
        which = qhead;
        col = 32 * cb;
      } else {
        const int c = c0 + 32 * cb;
        which = c < D ? p.N : p.N + 1 + (c - D) / D;
        col = c < D ? c : (c - D) % D;
      }
      int kind;
      const int64_t o = out_row(p, which, ft, kind);  // (prefill: always a valid row)
      __bf16* out = (__bf16*)out_base(p, kind) + o + col;
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = f2bf(acc[cb][rb][4 * jq + e]);
        *(bf16x4*)(out + 8 * jq + 4 * half) = o4;
      }
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
  const int n_dense = ((2 * p.G + 1) * p.d + 127) / 128;
  const int tiles_pw = n_dense + p.N;
  const int64_t total = (int64_t)((p.T + kPRows - 1) / kPRows) * tiles_pw;
  const int per = (int)((total + 7) / 8);
  const unsigned nblk = (unsigned)(8 * per);
  switch (p.d) {
    case 32: hipLaunchKernelGGL(proj_prefill_kernel<32>, dim3(nblk), dim3(256), 0, s, p, tiles_pw, n_dense, per); break;
    case 64: hipLaunchKernelGGL(proj_prefill_kernel<64>, dim3(nblk), dim3(256), 0, s, p, tiles_pw, n_dense, per); break;
    case 128: hipLaunchKernelGGL(proj_prefill_kernel<128>, dim3(nblk), dim3(256), 0, s, p, tiles_pw, n_dense, per); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqe
