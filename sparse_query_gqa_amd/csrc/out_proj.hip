// Slot assembly + output projection: y_t = Concat(O_t, obar_t, s_t) W_O.
//
// GQE review (paper.oopus.info), section 二 输出怎么拼起来: the hard slots are
// the selected heads' outputs concatenated; obar_t = sum over groups and
// selected experts of w * o (the renormalised weighted-sum slot); s_t is the
// shared head's output. The slot vector A_t is never materialised: the GEMM
// A-tile loader reads it straight from the attention outputs. Columns
// [0, G*k*d) are o_routed[t] as stored (group-major, slots ascending);
// columns [G*k*d, G*k*d + d) are obar computed in fp32 from the G*k stored
// slots and the fp32 weights; the last d columns are o_shared[t].
//
// Two further slot layouts serve the ablation variants (GQE review, section
// 四, Table 2): hard slots only, [O_t, s_t], and weighted concatenation,
// [w * O_t, s_t], where each hard slot is scaled by its renormalised weight;
// neither has the obar slot, and W_O has (G*k+1)*d rows.
//
// Two bf16 kernels: a pipelined GEMM for T >= 256 (below) and, for fewer
// tokens, a plain 128x128-tile kernel: four wavefronts of 64x64 each on
// v_mfma_f32_32x32x16_bf16, W_O's tile transposed into LDS to give the B
// operand k-contiguous lanes.
#include "gqe_internal.h"

namespace gqe {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 32, kPadK = 8;

__device__ __forceinline__ bf16x8 scale8(bf16x8 v, float s) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = f2bf((float)v[i] * s);
  return v;
}

template <typename T>
__device__ __forceinline__ float slot_value(const OutProjParams& p, int64_t t, int col) {
  const int hard = p.Gk * p.d;
  if (col < hard) {
    const float v = (float)((const T*)p.o_r)[t * hard + col];
    return p.weighted ? v * p.w[t * p.Gk + col / p.d] : v;
  }
  if (col < hard + p.nob) {
    const int e = col - hard;
    float s = 0.f;
    for (int j = 0; j < p.Gk; ++j)
      s = fmaf(p.w[t * p.Gk + j], (float)((const T*)p.o_r)[t * hard + j * p.d + e], s);
    return s;
  }
  return (float)((const T*)p.o_s)[t * p.d + (col - hard - p.nob)];
}

__global__ __launch_bounds__(256) void out_proj_bf16_kernel(OutProjParams p) {
  __shared__ __bf16 As[kBM][kBK + kPadK];
  __shared__ __bf16 Bt[kBN][kBK + kPadK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * kBM;
  const int n0 = blockIdx.y * kBN;
  const int hard = p.Gk * p.d;
  const int Kd = hard + p.nob + p.d;
  const __bf16* orr = (const __bf16*)p.o_r;
  const __bf16* os = (const __bf16*)p.o_s;
  const __bf16* wo = (const __bf16*)p.w_o;
  const bf16x8 zero8 = {};

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // A loader: thread -> (row = tid/2, 16 columns at (tid%2)*16) ... as two 8-wide pieces
  const int a_row = tid >> 1, a_col = (tid & 1) * 16;
  const int64_t at = m0 + a_row;
  const bool a_ok = at < p.T;
  // B loader: thread -> (k = tid/8, 16 output columns at (tid%8)*16)
  const int b_k = tid >> 3, b_n = (tid & 7) * 16;

  for (int k0 = 0; k0 < Kd; k0 += kBK) {
    bf16x8 a[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = k0 + a_col + 8 * h;
      if (!a_ok) {
        a[h] = zero8;
      } else if (col < hard) {
        a[h] = *(const bf16x8*)(orr + at * hard + col);
        if (p.weighted) a[h] = scale8(a[h], p.w[at * p.Gk + col / p.d]);
      } else if (col < hard + p.nob) {
        const int e = col - hard;
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < p.Gk; ++j) {
          const float wj = p.w[at * p.Gk + j];
          const bf16x8 ov = *(const bf16x8*)(orr + at * hard + j * p.d + e);
#pragma unroll
          for (int i = 0; i < 8; ++i) s[i] = fmaf(wj, (float)ov[i], s[i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) a[h][i] = f2bf(s[i]);
      } else {
        a[h] = *(const bf16x8*)(os + at * p.d + (col - hard - p.nob));
      }
    }
    bf16x8 bw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = n0 + b_n + 8 * h;
      bw[h] = (n < p.Dout) ? *(const bf16x8*)(wo + (int64_t)(k0 + b_k) * p.Dout + n) : zero8;
    }
    __syncthreads();
    *(bf16x8*)&As[a_row][a_col] = a[0];
    *(bf16x8*)&As[a_row][a_col + 8] = a[1];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) Bt[b_n + 8 * h + i][b_k] = bw[h][i];
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8*)&As[wm * 64 + i * 32 + l32][ks * 16 + 8 * half];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *(const bf16x8*)&Bt[wn * 64 + j * 32 + l32][ks * 16 + 8 * half];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }
  // C layout: lane holds column l32, rows 8*(r/4) + 4*half + r%4
  __bf16* y = (__bf16*)p.y;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
      if (n >= p.Dout) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (t < p.T) y[t * p.Dout + n] = f2bf(acc[i][j][r]);
      }
    }
}

// bf16 GEMM form. Computed as y^T = W_O^T A^T with v_mfma_f32_32x32x16_bf16:
// the W_O tile sits in LDS row-major ([k][n], as stored) and its fragments
// come from ds_read_b64_tr_b16 (four consecutive k of one n per lane); the A
// tile sits token-major ([t][k]) and is read with 16-byte loads. Each lane
// then holds four consecutive output columns of one token. A workgroup of 8
// wavefronts computes 128 tokens x 256 columns (64 x 64 per wavefront), k in
// steps of 32 through a four-stage LDS ring filled by LDS-DMA
// (global_load_lds_dwordx4): the hard-slot and shared-head columns of A come
// straight from o_routed / o_shared, obar is computed once per tile into its
// own LDS region at the start. Every step issues the same three DMA loads
// per thread (dummies for obar steps and past the end), so one fixed vmcnt
// wait before the barrier makes the current step's tile complete. The output
// tile is staged through LDS and written as whole rows.
constexpr int kGT = 128;      // tokens per tile
constexpr int kGN = 256;      // output columns per tile
constexpr int kGK = 32;       // k per step
constexpr int kGStages = 4;

template <int DH, int MODE>  // MODE: 0 [O, obar, s], 1 [O, s], 2 [w*O, s]
__global__ __launch_bounds__(512, 1) void out_proj_gemm_kernel(OutProjParams p) {
  constexpr int AB = kGT * kGK * 2;  // A tile: 128 token rows x 64 bytes
  constexpr int BB = kGK * kGN * 2;  // W_O tile: 32 k rows x 512 bytes
  constexpr int SB = AB + BB;
  constexpr int OPAD = DH + 8;       // obar row stride: 16 bytes of padding keep 16 rows on distinct banks
  constexpr int YPAD = kGN + 8;      // output staging row stride
  static_assert(kGT * YPAD * 2 <= kGStages * SB, "output staging must fit the stage ring");
  __shared__ __attribute__((aligned(1024))) char lds[kGStages * SB];
  __shared__ __attribute__((aligned(16))) __bf16 obar[kGT][OPAD];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;  // token half, column quarter
  const int64_t m0 = (int64_t)blockIdx.x * kGT;
  const int n0 = blockIdx.y * kGN;
  const int hard = p.Gk * DH;
  constexpr int nob = MODE == 0 ? DH : 0;
  constexpr bool weighted = MODE == 2;
  const int nk = (hard + nob + DH) / kGK;
  const __bf16* orr = (const __bf16*)p.o_r;
  const __bf16* os = (const __bf16*)p.o_s;
  const __bf16* wo = (const __bf16*)p.w_o;
  const int64_t tmax = p.T - 1;


  // LDS-DMA of step kt into stage st. A: chunk `wave` = token rows
  // 16*wave + lane/4, 16-byte chunk position lane%4, holding logical chunk
  // position ^ ((row >> 2) & 3). W_O: chunks 2*wave + i = k rows 2n + lane/32,
  // position lane%32 holding logical chunk position ^ ((row & 3) << 2).
  const int a_row = 16 * wave + (lane >> 2);
  const int a_c = (lane & 3) ^ ((a_row >> 2) & 3);
  const int64_t a_t = min(m0 + a_row, tmax);
  auto dma = [&](const int kt, const int st) __attribute__((always_inline)) {
    const int k0 = min(kt, nk - 1) * kGK;
    char* sbase = lds + st * SB;
    const __bf16* asrc;
    if (k0 < hard) asrc = orr + a_t * hard + k0 + 8 * a_c;
    else if (k0 >= hard + nob) asrc = os + a_t * DH + (k0 - hard - nob) + 8 * a_c;
    else asrc = orr + a_t * hard + 8 * a_c;  // obar step: a dummy load, the tile is not read
    lds_dma16(asrc, sbase + wave * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = 2 * wave + i;
      const int row = 2 * n + (lane >> 5);
      const int c = (lane & 31) ^ ((row & 3) << 2);
      const int col = min(n0 + 8 * c, p.Dout - 8);
      lds_dma16(wo + (int64_t)(k0 + row) * p.Dout + col, sbase + AB + n * 1024);
    }
  };

  // fragment addresses. A^T (B operand): token row t = wm*64 + tb*32 + l32,
  // chunk 2*kk + half. W^T (A operand): transposing read; in a 16-lane group
  // source lane i points at k row K0 + i/4, column N0 + 4*(i%4), and output
  // lane i receives k rows K0..K0+3 of column N0 + i.
  int a_off[2][2];  // [tb][kk]
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int t = wm * 64 + tb * 32 + l32;
      a_off[tb][kk] = t * 64 + 16 * ((2 * kk + half) ^ ((t >> 2) & 3));
    }
  const int tr_row = 8 * half + ((lane & 15) >> 2);  // + 16*kk + 4*tt
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + wn*64 + nb*32
  int w_off[2][2];  // [nb][tt] at kk = 0; kk adds 16 rows (same swizzle)
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = tr_row + 4 * tt;
      const int col = wn * 64 + nb * 32 + tr_col;
      w_off[nb][tt] = row * 512 + 16 * ((col >> 3) ^ ((row & 3) << 2)) + 2 * (col & 7);
    }

  f32x16 acc[2][2];  // [nb][tb]: 32 columns x 32 tokens
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int kt = 0; kt < kGStages - 1; ++kt) dma(kt, kt);
  // obar = sum over the G*k slots of w * o, in fp32, rounded to bf16; one
  // 8-column piece of one token per work item. Computed after the first
  // stages' LDS-DMA is issued, so that those loads are in flight meanwhile
  // (waiting on these loads also drains the earlier DMA: the counter is in
  // order); the main loop's first barrier publishes obar.
  for (int it = tid; nob && it < kGT * (DH / 8); it += 512) {
    const int row = it / (DH / 8), e = (it % (DH / 8)) * 8;
    const int64_t t = min(m0 + row, tmax);
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.Gk; ++j) {
      const float wj = p.w[t * p.Gk + j];
      const bf16x8 ov = *(const bf16x8*)(orr + t * hard + j * DH + e);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = fmaf(wj, (float)ov[i], s[i]);
    }
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = f2bf(s[i]);
    *(bf16x8*)&obar[row][e] = r;
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % kGStages;
    // step kt's tile is complete when at most the two later tiles' loads are
    // outstanding; the barrier makes it (and obar) visible and frees the
    // stage read in step kt-1 for step kt+3
    __asm__ volatile("s_waitcnt vmcnt(6)" ::: "memory");
    __syncthreads();
    dma(kt + kGStages - 1, (kt + kGStages - 1) % kGStages);
    const char* sbase = lds + st * SB;
    const int k0 = kt * kGK;
    const bool ob = k0 >= hard && k0 < hard + nob;
    // weighted concatenation: this step's hard slot k0 / DH, one weight per token
    float wsc[2] = {1.f, 1.f};
    if (weighted && k0 < hard) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        wsc[tb] = p.w[min(m0 + wm * 64 + tb * 32 + l32, tmax) * p.Gk + k0 / DH];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[2], wf[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if (ob) {
          const int t = wm * 64 + tb * 32 + l32;
          af[tb] = *(const bf16x8*)&obar[t][k0 - hard + 16 * kk + 8 * half];
        } else {
          af[tb] = *(const bf16x8*)(sbase + a_off[tb][kk]);
          if (weighted && k0 < hard) af[tb] = scale8(af[tb], wsc[tb]);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        u32x4 w4;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const char* a = sbase + AB + kk * 16 * 512 + w_off[nb][tt];
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a);
          const u32x2 w2 = __builtin_bit_cast(u32x2, x);
          w4[2 * tt] = w2[0];
          w4[2 * tt + 1] = w2[1];
        }
        wf[nb] = __builtin_bit_cast(bf16x8, w4);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], af[tb], acc[nb][tb], 0, 0, 0);
    }
  }

  // output tile through LDS: lane (half, l32) of tile (nb, tb) holds token
  // wm*64 + tb*32 + l32 and columns wn*64 + nb*32 + 8*(r/4) + 4*half + r%4
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __bf16* ys = (__bf16*)lds;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = wm * 64 + tb * 32 + l32;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = f2bf(acc[nb][tb][4 * rq + i]);
        *(bf16x4*)&ys[t * YPAD + wn * 64 + nb * 32 + 8 * rq + 4 * half] = o4;
      }
    }
  __syncthreads();
  __bf16* y = (__bf16*)p.y;
  for (int it = tid; it < kGT * (kGN / 8); it += 512) {
    const int row = it / (kGN / 8), c8 = (it % (kGN / 8)) * 8;
    const int64_t t = m0 + row;
    const int n = n0 + c8;
    if (t < p.T && n < p.Dout) *(bf16x8*)(y + t * p.Dout + n) = *(const bf16x8*)&ys[row * YPAD + c8];
  }
}

// Few-token form (T <= 16, decode): y^T = W_O^T A^T on v_mfma_f32_16x16x32_bf16
// with 16 output columns per workgroup, so that the W_O stream is spread over
// Dout/16 workgroups. The 8 wavefronts split K; each copies its K slice of
// the 16 columns (32 k rows x 32 bytes per step) into a private LDS region by
// LDS-DMA and reads the W_O^T fragments from it with ds_read_b64_tr_b16. The
// A^T operand needs no transpose: lane l takes token l%16 and 8 consecutive
// k, which are contiguous in o_routed / o_shared; obar is computed once for
// the 16 tokens into LDS. A pass first issues all its loads, then its MFMAs.
// The partial 16x16 tiles of the 8 wavefronts are added in LDS in a fixed
// order.
constexpr int kSmallT = 16;
constexpr int kSmallSteps = 16;  // 32-k steps per wavefront per pass (16 KiB of LDS)

template <int DH>
__global__ __launch_bounds__(512, 1) void out_proj_small_kernel(OutProjParams p) {
  __shared__ __attribute__((aligned(1024))) char wl[8][kSmallSteps][1024];
  __shared__ float part[8][16][17];
  __shared__ __attribute__((aligned(16))) __bf16 obar_s[16][DH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups go round-robin to the 8 XCDs. Four 16-column slices share each
  // 128-byte line of a W_O row, so when the slice count allows, the four
  // slices of a line are given to consecutive workgroups of one XCD: the line
  // then comes from HBM once, into that XCD's L2.
  int slice = blockIdx.x;
  if (gridDim.x % 32 == 0) {
    const int x = blockIdx.x % 8, i = blockIdx.x / 8;
    slice = (i / 4) * 32 + x * 4 + i % 4;
  }
  const int n0 = slice * 16;
  const int hard = p.Gk * DH;
  const int nob = p.nob;
  const int nsteps = (hard + nob + DH) / 32;
  const int s_lo = wave * nsteps / 8, s_hi = (wave + 1) * nsteps / 8;
  const __bf16* orr = (const __bf16*)p.o_r;
  const __bf16* os = (const __bf16*)p.o_s;
  const __bf16* wo = (const __bf16*)p.w_o;

  // obar of the 16 tokens (tokens past T repeat token T-1), fp32 sums rounded to bf16
  for (int it = tid; nob && it < 16 * (DH / 8); it += 512) {
    const int t = min(it / (DH / 8), (int)p.T - 1), e = (it % (DH / 8)) * 8;
    float sacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
    for (int j = 0; j < p.Gk; ++j) {
      const float wj = p.w[(int64_t)t * p.Gk + j];
      const bf16x8 ov = *(const bf16x8*)(orr + (int64_t)t * hard + j * DH + e);
#pragma unroll
      for (int i = 0; i < 8; ++i) sacc[i] = fmaf(wj, (float)ov[i], sacc[i]);
    }
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = f2bf(sacc[i]);
    *(bf16x8*)&obar_s[it / (DH / 8)][e] = r;
  }
  __syncthreads();

  // B operand: token t = lane%16 (tokens past T read token T-1; their
  // outputs are not stored), k = 8*(lane/16) + 0..7 of the step
  const int bt = min(lane & 15, (int)p.T - 1), bk = 8 * (lane >> 4);
  // W_O DMA: lane l copies k row l/2, columns 8*(l%2) + 0..7 (clamped to the
  // last full 8 columns past Dout; those outputs are not stored)
  const int d_row = lane >> 1, d_col = min(n0 + 8 * (lane & 1), p.Dout - 8);
  // transposing read: source lane i of a 16-lane group points at k row
  // K0 + i/4, column 4*(i%4); output lane i gets k rows K0..K0+3 of column i
  const int tr_off = (((lane & 15) >> 2) + 8 * (lane >> 4)) * 32 + 8 * (lane & 3);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_lo; s0 < s_hi; s0 += kSmallSteps) {
    const int ns = min(kSmallSteps, s_hi - s0);
    bf16x8 bq[kSmallSteps];
#pragma unroll
    for (int i = 0; i < kSmallSteps; ++i) {
      if (i < ns) {
        __builtin_amdgcn_global_load_lds(wo + (int64_t)((s0 + i) * 32 + d_row) * p.Dout + d_col,
                                         (__attribute__((address_space(3))) void*)wl[wave][i], 16, 0, 0);
        const int k = (s0 + i) * 32 + bk;
        if (k < hard) {
          bq[i] = *(const bf16x8*)(orr + (int64_t)bt * hard + k);
          if (p.weighted) bq[i] = scale8(bq[i], p.w[(int64_t)bt * p.Gk + k / DH]);
        } else if (k < hard + nob) {
          bq[i] = *(const bf16x8*)&obar_s[lane & 15][k - hard];
        } else {
          bq[i] = *(const bf16x8*)(os + (int64_t)bt * DH + (k - hard - nob));
        }
      }
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < kSmallSteps; ++i) {
      if (i < ns) {
        u32x4 w4;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(wl[wave][i] + tr_off + tt * 4 * 32));
          const u32x2 w2 = __builtin_bit_cast(u32x2, x);
          w4[2 * tt] = w2[0];
          w4[2 * tt + 1] = w2[1];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w4), bq[i], acc, 0, 0, 0);
      }
    }
  }
  // lane l holds columns 4*(l/16) + 0..3 of token l%16
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][lane & 15][4 * (lane >> 4) + i] = acc[i];
  __syncthreads();
  if (tid < 256) {
    const int t = tid >> 4, c = tid & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += part[w][t][c];
    if (t < p.T && n0 + c < p.Dout) ((__bf16*)p.y)[(int64_t)t * p.Dout + n0 + c] = f2bf(sum);
  }
}

// fp32: one thread per output element, sequential fp32 accumulation.
__global__ __launch_bounds__(256) void out_proj_f32_kernel(OutProjParams p) {
  const int n = blockIdx.y * 64 + (threadIdx.x & 63);
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= p.Dout || t >= p.T) return;
  const int Kd = p.Gk * p.d + p.nob + p.d;
  const float* wo = (const float*)p.w_o;
  float acc = 0.f;
  for (int col = 0; col < Kd; ++col)
    acc = fmaf(slot_value<float>(p, t, col), wo[(int64_t)col * p.Dout + n], acc);
  ((float*)p.y)[t * p.Dout + n] = acc;
}

hipError_t launch_out_proj(const OutProjParams& p, bool bf16, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (bf16 && p.T >= kGT * 2) {
    const dim3 grid((unsigned)((p.T + kGT - 1) / kGT), (p.Dout + kGN - 1) / kGN);
    const int mode = p.nob ? 0 : (p.weighted ? 2 : 1);
#define GQE_OUT_PROJ_GEMM(DH)                                                                    \
  if (mode == 0) hipLaunchKernelGGL((out_proj_gemm_kernel<DH, 0>), grid, dim3(512), 0, s, p);    \
  else if (mode == 1) hipLaunchKernelGGL((out_proj_gemm_kernel<DH, 1>), grid, dim3(512), 0, s, p); \
  else hipLaunchKernelGGL((out_proj_gemm_kernel<DH, 2>), grid, dim3(512), 0, s, p);
    switch (p.d) {
      case 32: GQE_OUT_PROJ_GEMM(32) break;
      case 64: GQE_OUT_PROJ_GEMM(64) break;
      case 128: GQE_OUT_PROJ_GEMM(128) break;
      default: return hipErrorInvalidValue;
    }
#undef GQE_OUT_PROJ_GEMM
  } else if (bf16 && p.T <= kSmallT) {
    const dim3 grid((p.Dout + 15) / 16);
    switch (p.d) {
      case 32: hipLaunchKernelGGL(out_proj_small_kernel<32>, grid, dim3(512), 0, s, p); break;
      case 64: hipLaunchKernelGGL(out_proj_small_kernel<64>, grid, dim3(512), 0, s, p); break;
      case 128: hipLaunchKernelGGL(out_proj_small_kernel<128>, grid, dim3(512), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
  } else if (bf16) {
    const dim3 grid((unsigned)((p.T + kBM - 1) / kBM), (p.Dout + kBN - 1) / kBN);
    hipLaunchKernelGGL(out_proj_bf16_kernel, grid, dim3(256), 0, s, p);
  } else {
    const dim3 grid((unsigned)((p.T + 3) / 4), (p.Dout + 63) / 64);
    hipLaunchKernelGGL(out_proj_f32_kernel, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gqe
