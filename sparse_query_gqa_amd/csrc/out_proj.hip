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
// Two further slot layouts serve the ablation rows of GQE review, section
// 四, Table 2, which keep the hard slots only: A_t = O_t (hard
// concatenation), and A_t = p * O_t (weighted concatenation without the
// renormalised slot), each hard slot scaled by its router probability p,
// which the caller passes in place of w. Neither has the obar slot or the
// shared head, and W_O has G*k*d rows.
//
// Three bf16 kernels: a tiled GEMM for T >= 256, a GEMV-shaped one for
// T <= 16 (decode), and for the tokens between a plain 128x128-tile kernel:
// four wavefronts of 64x64 each on v_mfma_f32_32x32x16_bf16, W_O's tile
// transposed into LDS to give the B operand k-contiguous lanes.
#include <algorithm>

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
  const int Kd = hard + p.nob + p.nsh;
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

// Tiled form (T >= 256). Computed as y^T = W_O^T A^T with
// v_mfma_f32_32x32x16_bf16: the W_O tile sits in LDS as stored ([k][n]) and
// its fragments come from ds_read_b64_tr_b16 (four consecutive k of one n per
// lane); the A tile sits token-major ([t][k]) and is read with 16-byte loads,
// so each lane holds four consecutive output columns of one token. The
// hard-slot and shared-head columns of A come straight from o_routed /
// o_shared; obar is computed once per tile (its loads issued eight slots at
// a time, so their latencies overlap). At d = 32 it sits in its own LDS
// region; at d >= 64 each thread keeps its d/16 pieces in registers and
// writes them into the ring's A region when an obar step is staged (its two
// A loads then repeat the step's W_O loads), so the 32 or 64 KiB obar would
// take go to a fifth stage instead. A
// workgroup of eight wavefronts computes 256 tokens x 256 columns (128
// tokens x 64 columns each). The tile is large so that the
// bytes staged per FLOP are few: a CU then keeps the loads of NS - 1 steps in
// flight against the latency of L2 and the memory-side cache. k goes in
// steps of 32 through an NS-stage LDS ring filled by LDS-DMA from raw buffer
// resources (a step moves with scalar resource words; rows past T read
// zeros); every step issues the same four loads per thread (a dummy load
// on obar steps), so one fixed vmcnt wait makes a stage complete. With four
// or more stages the ring advances in the middle of a step and the next step's first
// fragments are read while the current step's second MFMA half runs.
// Workgroup i runs on XCD i % 8; XCD x takes token tiles x, x + 8, ... and
// for each all column tiles in turn, so a token tile's slot rows come from
// HBM once and W_O stays in each XCD's L2.
constexpr int kPT = 256;  // tokens per tile
constexpr int kPN = 256;  // output columns per tile
constexpr int kPK = 32;   // k per step

template <int DH, int MODE, int NS>
__global__ __launch_bounds__(512, 1) void out_proj_tile_kernel(OutProjParams p, int cpw) {
  constexpr int AB = kPT * kPK * 2;  // A stage: 256 token rows x 64 bytes
  constexpr int WB = kPK * kPN * 2;  // W_O stage: 32 k rows x 512 bytes
  constexpr int SB = AB + WB;
  constexpr int nob = MODE == 0 ? DH : 0;
  constexpr int nsh = MODE == 0 ? DH : 0;
  constexpr bool weighted = MODE == 2;
  // d >= 64: obar stays in registers (DH bytes per thread) and is written
  // into the A region of its k steps, which frees its LDS for more stages
  constexpr bool OBR = MODE == 0 && DH >= 64;
  constexpr int NIT = DH / 16;  // obar items (8-column pieces) per thread
  constexpr int OB = MODE == 0 && !OBR ? kPT * DH * 2 : 0;  // obar tile (unpadded)
  constexpr int YPAD = kPN + 8;                     // output staging row stride
  static_assert((kPT / 2) * YPAD * 2 <= NS * SB, "half-tile staging fits in the ring");
  constexpr int LDSB = NS * SB + OB;
  // weighted layout: the token tile's slot weights of the first WSL slots,
  // [slot][token], loaded once (a global load inside the k loop would make its
  // vmcnt wait drain the LDS-DMA ring, whose loads were issued before it)
  constexpr int WSL = weighted ? 32 : 0;
  static_assert(LDSB + kPT * WSL * 4 <= 163840, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[LDSB];
  __shared__ float wlds[weighted ? kPT * WSL : 1];
  __bf16* obar = (__bf16*)(lds + NS * SB);  // [kPT][DH], 16-byte chunks swizzled per row
  // obar chunk c of token row t sits at chunk position c ^ oswz(t), so that the
  // fragment reads (32 consecutive rows, one chunk each) hit distinct banks
  auto oswz = [](int t) { return DH == 32 ? ((t >> 2) & 3) : DH == 64 ? ((t >> 1) & 7) : (t & 15); };

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;  // token half, column quarter
  // token tile ttile and column tiles c_lo .. c_hi-1 (cpw of them): obar is
  // formed once and serves every column tile of the workgroup
  const int ncol = (p.Dout + kPN - 1) / kPN;
  const int ngrp = (ncol + cpw - 1) / cpw;
  const int64_t ntok = (p.T + kPT - 1) / kPT;
  const int xcd = blockIdx.x % 8, jj = blockIdx.x / 8;
  const int64_t ttile = xcd + 8 * (int64_t)(jj / ngrp);
  if (ttile >= ntok) return;
  const int64_t m0 = ttile * kPT;
  const int c_lo = (jj % ngrp) * cpw, c_hi = min(ncol, c_lo + cpw);
  int n0 = c_lo * kPN;
  const int hard = p.Gk * DH;
  const int nk = (hard + nob + nsh) / kPK;
  const __bf16* orr = (const __bf16*)p.o_r;
  const __bf16* os = (const __bf16*)p.o_s;
  const __bf16* wo = (const __bf16*)p.w_o;
  const int64_t tmax = p.T - 1;
  const uint32_t rows = (uint32_t)min<int64_t>(p.T - m0, kPT);  // valid token rows of this tile

  // LDS-DMA lane geometry. A: 1 KiB chunk c = 2*wave + i holds token rows
  // 16c + lane/4, 16-byte piece lane%4 holding the row's logical piece
  // (lane%4) ^ ((row >> 2) & 3). W_O: chunk c holds k rows 2c + lane/32,
  // piece lane%32 holding logical column chunk (lane%32) ^ ((row & 3) << 2).
  uint32_t a_off_r[2], a_off_s[2], w_off_d[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = 2 * wave + i;
    const int row = 16 * c + (lane >> 2);
    const int lp = (lane & 3) ^ ((row >> 2) & 3);
    a_off_r[i] = (uint32_t)(row * hard * 2 + lp * 16);
    a_off_s[i] = (uint32_t)(row * DH * 2 + lp * 16);
    const int kr = 2 * c + (lane >> 5);
    const int lc = (lane & 31) ^ ((kr & 3) << 2);
    w_off_d[i] = (uint32_t)kr * (uint32_t)p.Dout * 2u + (uint32_t)lc * 16u;
  }
  // OBR: this thread's obar pieces: token rows tid / (DH/8) + (4096/DH) b,
  // columns 8 (tid % (DH/8)) .. +7
  bf16x8 obr[NIT];
  auto dma = [&](const int kt, const int st) __attribute__((always_inline)) {
    const int k0 = min(kt, nk - 1) * kPK;
    char* sbase = lds + st * SB;
    if (OBR && k0 >= hard && k0 < hard + nob) {
      // obar columns k0 - hard .. +31 from registers into the A region; the
      // step's two A loads become a second copy of its W_O loads (same bytes
      // to the same place), so every step still issues four loads
      if (((tid % (DH / 8)) >> 2) == (k0 - hard) / kPK) {
#pragma unroll
        for (int b = 0; b < NIT; ++b) {
          const int row = tid / (DH / 8) + (4096 / DH) * b;
          *(bf16x8*)(sbase + row * 64 + 16 * ((tid & 3) ^ ((row >> 2) & 3))) = obr[b];
        }
      }
      const i32x4 rw = buf_rsrc(wo + (int64_t)k0 * p.Dout + n0, (uint32_t)kPK * (uint32_t)p.Dout * 2u - (uint32_t)n0 * 2u);
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16_b(rw, w_off_d[i & 1], sbase + AB + (2 * wave + (i & 1)) * 1024);
      return;
    }
    // the step's source; the branch selects scalars, the resource is built once
    const __bf16* abase = orr + m0 * hard;  // obar step: a dummy load of the first slot columns
    uint32_t anum = rows * (uint32_t)hard * 2u;
    bool shared_slot = false;
    if (k0 < hard) {
      abase = orr + m0 * hard + k0;
      anum = rows * (uint32_t)hard * 2u - (uint32_t)k0 * 2u;
    } else if (k0 >= hard + nob) {
      const int ks = k0 - hard - nob;
      abase = os + m0 * DH + ks;
      anum = rows * (uint32_t)DH * 2u - (uint32_t)ks * 2u;
      shared_slot = true;
    }
    const i32x4 ra = buf_rsrc(abase, anum);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      lds_dma16_b(ra, shared_slot ? a_off_s[i] : a_off_r[i], sbase + (2 * wave + i) * 1024);
    const i32x4 rw = buf_rsrc(wo + (int64_t)k0 * p.Dout + n0, (uint32_t)kPK * (uint32_t)p.Dout * 2u - (uint32_t)n0 * 2u);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16_b(rw, w_off_d[i], sbase + AB + (2 * wave + i) * 1024);
  };

  // Fragment addresses. A^T (B operand): token t = wm*128 + tb*32 + l32,
  // chunk 2*kk + half. W^T (A operand): transposing read; in a 16-lane group
  // source lane i points at k row K0 + i/4, column N0 + 4*(i%4), and output
  // lane i receives k rows K0..K0+3 of column N0 + i.
  int a_frag[4][2];  // [tb][kk]
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int t = wm * 128 + tb * 32 + l32;
      a_frag[tb][kk] = t * 64 + 16 * ((2 * kk + half) ^ ((t >> 2) & 3));
    }
  const int tr_row = 8 * half + ((lane & 15) >> 2);              // + 16*kk + 4*tt
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);    // + wn*64 + nb*32
  int w_frag[2][2];  // [nb][tt] at kk = 0; kk adds 16 rows (same swizzle)
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = tr_row + 4 * tt;
      const int col = wn * 64 + nb * 32 + tr_col;
      w_frag[nb][tt] = row * 512 + 16 * ((col >> 3) ^ ((row & 3) << 2)) + 2 * (col & 7);
    }

  f32x16 acc[2][4];  // [nb][tb]: 32 columns x 32 tokens

  if constexpr (weighted) {
    const int nsl = min(p.Gk, WSL);
    for (int i = tid; i < kPT * nsl; i += 512) {
      const int j = i / kPT, t = i % kPT;
      wlds[j * kPT + t] = p.w[min(m0 + t, tmax) * p.Gk + j];
    }
  }
  // the first column tile's first stages load while obar is formed (unless
  // one of them is an obar step that takes obar from registers)
  const bool ob_early = OBR && hard / kPK < NS - 1;
  if (!ob_early) {
#pragma unroll
    for (int kt = 0; kt < NS - 1; ++kt) dma(kt, kt);
  }
  // obar = sum over the G*k slots of w * o, in fp32, rounded to bf16; one
  // 8-column piece of one token per work item, DH/16 items per thread. The
  // loads of up to four items (eight slots each) are issued together before
  // their products, beside the first stages' loads (the MFMA accumulators are
  // not live yet, so the registers are there): with a runtime slot count the
  // compiler would otherwise serialise their latencies.
  constexpr int IB = NIT < 4 ? NIT : 4;  // items per batch
  for (int b0 = 0; nob && b0 < NIT; b0 += IB) {
    int row[IB], e[IB];
    int64_t t[IB];
    float sacc[IB][8];
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      const int it = tid + 512 * (b0 + b);
      row[b] = it / (DH / 8);
      e[b] = (it % (DH / 8)) * 8;
      t[b] = min(m0 + row[b], tmax);
#pragma unroll
      for (int i = 0; i < 8; ++i) sacc[b][i] = 0.f;
    }
    for (int j0 = 0; j0 < p.Gk; j0 += 8) {
      bf16x8 ov[IB][8];
      float wj[IB][8];
#pragma unroll
      for (int b = 0; b < IB; ++b)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(j0 + u, p.Gk - 1);
          ov[b][u] = *(const bf16x8*)(orr + t[b] * hard + j * DH + e[b]);
          wj[b][u] = j0 + u < p.Gk ? p.w[t[b] * p.Gk + j] : 0.f;
        }
      // slots in order, as one item at a time would add them
#pragma unroll
      for (int b = 0; b < IB; ++b)
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) sacc[b][i] = fmaf(wj[b][u], (float)ov[b][u][i], sacc[b][i]);
    }
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      bf16x8 r;
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = f2bf(sacc[b][i]);
      if constexpr (OBR) obr[b0 + b] = r;
      else *(bf16x8*)&obar[row[b] * DH + 8 * ((e[b] >> 3) ^ oswz(row[b]))] = r;
    }
  }
  if (ob_early) {
#pragma unroll
    for (int kt = 0; kt < NS - 1; ++kt) dma(kt, kt);
  }

  bf16x8 af[4][2], wf[2][2];  // [tb or nb][kk]
  auto read_frags = [&](const int kt, const int kk) __attribute__((always_inline)) {
    const char* sbase = lds + (kt % NS) * SB;
    const int k0 = kt * kPK;
    const bool ob = !OBR && k0 >= hard && k0 < hard + nob;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if (ob) {
        const int t = wm * 128 + tb * 32 + l32;
        af[tb][kk] = *(const bf16x8*)&obar[t * DH + 8 * ((((k0 - hard) >> 3) + 2 * kk + half) ^ oswz(t))];
      } else {
        af[tb][kk] = *(const bf16x8*)(sbase + a_frag[tb][kk]);
      }
      if (weighted && k0 < hard) {
        const int tl = wm * 128 + tb * 32 + l32, slot = k0 / DH;
        const float wsc = slot < WSL ? wlds[slot * kPT + tl] : p.w[min(m0 + tl, tmax) * p.Gk + slot];
#pragma unroll
        for (int i = 0; i < 8; ++i) af[tb][kk][i] = f2bf((float)af[tb][kk][i] * wsc);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      u32x4 w4;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const char* a = sbase + AB + kk * 16 * 512 + w_frag[nb][tt];
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a);
        const u32x2 w2 = __builtin_bit_cast(u32x2, x);
        w4[2 * tt] = w2[0];
        w4[2 * tt + 1] = w2[1];
      }
      wf[nb][kk] = __builtin_bit_cast(bf16x8, w4);
    }
  };
  auto mfmas = [&](const int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb][kk], af[tb][kk], acc[nb][tb], 0, 0, 0);
  };

  // Output staging sits at the ring's end, so that the stages below it (E of
  // them) can take the next column tile's first loads before this one's
  // second-half output stores: each wavefront issues exactly SST of those
  // (stores count in vmcnt beside the LDS-DMA, in issue order), and the next
  // tile's first waits count them instead of waiting for them.
  constexpr int STG = (kPT / 2) * YPAD * 2;
  constexpr int E = NS >= 4 ? (NS * SB - STG) / SB : 0;
  constexpr int SST = (kPT / 2) * (kPN / 8) / 512;  // stores of the second half
  static_assert(E < NS, "staging");
  for (int c = c_lo; c < c_hi; ++c) {
  const int n_st = c * kPN;  // this column tile's first column
  if (c > c_lo) {
    // the previous column tile is stored (the barrier ending its epilogue):
    // the ring takes this one's first stages, stages 0 .. E-1 already issued
    n0 = c * kPN;
#pragma unroll
    for (int kt = E; kt < NS - 1; ++kt) dma(kt, kt);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if constexpr (NS >= 4) {
    // stage 0 complete (stages 1 .. NS-2 may be in flight, and after a
    // previous column tile its SST output stores, issued after stage E-1);
    // the barrier also publishes obar
    if (c > c_lo && E > 0) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (NS - 2) + SST) : "memory");
    else __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (NS - 2)) : "memory");
    __syncthreads();
    read_frags(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      read_frags(kt, 1);
      mfmas(0);
      // stage kt+1 complete, later ones in flight; after the barrier every
      // wavefront has finished its reads of stage kt-1, whose buffer takes
      // stage kt+NS-1
      if (kt == 0 && c > c_lo && E > 1) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (NS - 3) + SST) : "memory");
      else __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (NS - 3)) : "memory");
      __syncthreads();
      dma(kt + NS - 1, (kt + NS - 1) % NS);
      if (kt + 1 < nk) read_frags(kt + 1, 0);
      mfmas(1);
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt complete (kt+1 .. kt+NS-2 in flight); after the barrier the
      // buffer of stage kt-1 takes stage kt+NS-1 (and obar is published)
      __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * (NS - 2)) : "memory");
      __syncthreads();
      dma(kt + NS - 1, (kt + NS - 1) % NS);
      read_frags(kt, 0);
      read_frags(kt, 1);
      mfmas(0);
      mfmas(1);
    }
  }

  // output tile through the top of the ring's LDS (obar stays for the next
  // column tile), 128 token rows at a time: lane (half, l32) of tile (nb, tb) holds
  // token wm*128 + tb*32 + l32 and columns wn*64 + nb*32 + 8*(r/4) + 4*half + r%4
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __bf16* ys = (__bf16*)(lds + NS * SB - STG);
  // rows past T and columns past Dout go to an offset past the buffer's end,
  // where the store is dropped: every lane issues every store
  const uint32_t ynum = rows * (uint32_t)p.Dout * 2u;
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc((__bf16*)p.y + m0 * p.Dout, 0, (int)ynum, 0x00020000);
  for (int hh = 0; hh < 2; ++hh) {
    if (wm == hh) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int t = tb * 32 + l32;
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            bf16x4 o4;
#pragma unroll
            for (int i = 0; i < 4; ++i) o4[i] = f2bf(acc[nb][tb][4 * rq + i]);
            *(bf16x4*)&ys[t * YPAD + wn * 64 + nb * 32 + 8 * rq + 4 * half] = o4;
          }
        }
    }
    __syncthreads();
    if (hh == 1 && c + 1 < c_hi) {
      // the accumulators are staged: the next column tile's first E stages
      // go out before this half's stores
      n0 = (c + 1) * kPN;
#pragma unroll
      for (int kt = 0; kt < E; ++kt) dma(kt, kt);
    }
#pragma unroll 1
    for (int j = 0; j < SST; ++j) {
      const int it = tid + 512 * j;
      const int row = it / (kPN / 8), c8 = (it % (kPN / 8)) * 8;
      const int n = n_st + c8;
      const uint32_t off = n < p.Dout ? ((uint32_t)(hh * (kPT / 2) + row) * (uint32_t)p.Dout + (uint32_t)n) * 2u : ynum;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, *(const bf16x8*)&ys[row * YPAD + c8]), yr, off, 0, 0);
    }
    __syncthreads();  // ys is rewritten next (the other half, or the next column tile's ring)
  }
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
  const int nsteps = (hard + nob + p.nsh) / 32;
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
  const int Kd = p.Gk * p.d + p.nob + p.nsh;
  const float* wo = (const float*)p.w_o;
  float acc = 0.f;
  for (int col = 0; col < Kd; ++col)
    acc = fmaf(slot_value<float>(p, t, col), wo[(int64_t)col * p.Dout + n], acc);
  ((float*)p.y)[t * p.Dout + n] = acc;
}

hipError_t launch_out_proj(const OutProjParams& p, bool bf16, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (bf16 && p.T >= 256) {
    const int64_t ntok = (p.T + kPT - 1) / kPT;
    const int ncol = (p.Dout + kPN - 1) / kPN;
    const int mode = p.nob ? 0 : (p.weighted ? 2 : 1);
    // With obar (mode 0), a workgroup takes several column tiles of its token
    // tile, so that obar is formed once for them, as long as every CU still
    // gets a workgroup (one runs per CU); otherwise one column tile each.
    int cpw = 1;
    if (mode == 0) {
      const int64_t want = (int64_t)device_cus();
      cpw = (int)std::max<int64_t>(1, std::min<int64_t>(ncol, ntok * ncol / want));
    }
    const int ngrp = (ncol + cpw - 1) / cpw;
    const dim3 grid((unsigned)(8 * ((ntok + 7) / 8) * ngrp));
#define GQE_OUT_PROJ_GEMM(DH)                                                                                    \
  if (mode == 0) hipLaunchKernelGGL((out_proj_tile_kernel<DH, 0, DH >= 64 ? 5 : 4>), grid, dim3(512), 0, s, p, cpw); \
  else if (mode == 1) hipLaunchKernelGGL((out_proj_tile_kernel<DH, 1, 4>), grid, dim3(512), 0, s, p, cpw);          \
  else hipLaunchKernelGGL((out_proj_tile_kernel<DH, 2, 4>), grid, dim3(512), 0, s, p, cpw);
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
