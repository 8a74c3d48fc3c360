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
// bf16: 128x128 output tile per 256-thread workgroup, K step 32, four
// wavefronts of 64x64 each on v_mfma_f32_32x32x16_bf16. W_O is row-major
// [K, D] (the natural y = A W_O layout), so its tile is transposed into LDS
// to give the B operand k-contiguous lanes.
#include "gqe_internal.h"

namespace gqe {

constexpr int kBM = 128, kBN = 128, kBK = 32, kPadK = 8;

template <typename T>
__device__ __forceinline__ float slot_value(const OutProjParams& p, int64_t t, int col) {
  const int hard = p.Gk * p.d;
  if (col < hard) return (float)((const T*)p.o_r)[t * hard + col];
  if (col < hard + p.d) {
    const int e = col - hard;
    float s = 0.f;
    for (int j = 0; j < p.Gk; ++j)
      s = fmaf(p.w[t * p.Gk + j], (float)((const T*)p.o_r)[t * hard + j * p.d + e], s);
    return s;
  }
  return (float)((const T*)p.o_s)[t * p.d + (col - hard - p.d)];
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
  const int Kd = hard + 2 * p.d;
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
      } else if (col < hard + p.d) {
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
        a[h] = *(const bf16x8*)(os + at * p.d + (col - hard - p.d));
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

// fp32: one thread per output element, sequential fp32 accumulation.
__global__ __launch_bounds__(256) void out_proj_f32_kernel(OutProjParams p) {
  const int n = blockIdx.y * 64 + (threadIdx.x & 63);
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= p.Dout || t >= p.T) return;
  const int Kd = p.Gk * p.d + 2 * p.d;
  const float* wo = (const float*)p.w_o;
  float acc = 0.f;
  for (int col = 0; col < Kd; ++col)
    acc = fmaf(slot_value<float>(p, t, col), wo[(int64_t)col * p.Dout + n], acc);
  ((float*)p.y)[t * p.Dout + n] = acc;
}

hipError_t launch_out_proj(const OutProjParams& p, bool bf16, hipStream_t s) {
  if (bf16) {
    const dim3 grid((unsigned)((p.T + kBM - 1) / kBM), (p.Dout + kBN - 1) / kBN);
    hipLaunchKernelGGL(out_proj_bf16_kernel, grid, dim3(256), 0, s, p);
  } else {
    const dim3 grid((unsigned)((p.T + 3) / 4), (p.Dout + 63) / 64);
    hipLaunchKernelGGL(out_proj_f32_kernel, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace gqe
