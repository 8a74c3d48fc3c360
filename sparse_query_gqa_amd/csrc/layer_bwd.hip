// Backward of the output projection and of the router.
//
// Output projection (GQE review, section 二: y = Concat(O, obar, s) W_O with
// obar = sum over groups and selected experts of w * o): with A the slot
// vector, dW_O = A^T dy and dA = dy W_O^T. dA splits into the hard slots,
// the obar slot and the shared slot; obar feeds back into every hard slot
// (w * dobar) and into the routing weights (dw = o . dobar), which is the
// path that gives the router a gradient. The ablation layouts (A = O and
// A = p * O, section 四, Table 2) hold the hard slots only; the weighted one
// scales each hard slot's gradient by its weight p and gives dp = o . dslot,
// and in both the shared head's gradient is zero.
//
// Router: p = softmax(z) per group, w = p_sel / sum p_sel on the selected
// experts (the renormalised weight). dp_sel = (dw - sum dw w) / sum p_sel,
// 0 on the others, or dp_sel = dw when the weights were the selected p
// themselves (the weighted-concatenation layout); the balance loss (coef * M * mean_g sum_m f P, f the share
// of selections, P the mean probability; section 二 names the standard MoE
// balance loss) adds coef * M * f / (T * G) to dp of every expert;
// dz = p (dp - p . dp); dW_r = dz^T x, db_r = sum_t dz, dx = dz W_r.
//
// The four products (dA, dW_O, dW_r, dx) run on one bf16 MFMA GEMM kernel
// with fp32 accumulation whose operands are read either row-major along the
// contraction (16-byte LDS reads) or transposed (ds_read_b64_tr_b16), and
// whose long-contraction forms are split into fp32 partials added in a
// fixed order (deterministic). The fp32 path uses plain VALU kernels.
#include "gqe_internal.h"

namespace gqe {

typedef uint32_t u32x2b __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4b __attribute__((ext_vector_type(4)));
typedef short s16x4b __attribute__((ext_vector_type(4)));

void gemm_split(int64_t K, int tiles, int& nsplit, int& kchunk) {
  const int64_t want = (512 + tiles - 1) / tiles;
  const int64_t most = (K + 255) / 256;
  int64_t ns = want < most ? want : most;
  if (ns < 1) ns = 1;
  const int64_t kc = ((K + ns - 1) / ns + 31) / 32 * 32;
  kchunk = (int)(kc > 0 ? kc : 32);
  nsplit = (int)((K + kchunk - 1) / kchunk);
  if (nsplit < 1) nsplit = 1;
}

// ---------------------------------------------------------------------------
// GEMM: C[m][n] = sum_k A'[m][k] B'[k][n] (+ split partials)
// ---------------------------------------------------------------------------
// A' is A stored [M][K] (row-major along k) or, with A_TR, A stored [K][M];
// B' is B stored [N][K] or, with B_TR, B stored [K][N]. Loads past the
// stored extents (rows x cols) are zero, so ragged edges need no special
// case; every stored row stride and column extent is a multiple of 8.
struct Gemm {
  const void* a;
  const void* b;
  void* c;
  int64_t lda, ldb, ldc, c_split;  // element strides; c_split between split partials
  int M, N, K;                     // C extent; contraction extent
  int a_rows, a_cols, b_rows, b_cols;
  int kchunk;                      // contraction per split (multiple of 32)
  int out_bf16;                    // C stored as bf16 (no split) instead of fp32
  float alpha;
};

template <bool A_TR, bool B_TR>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(Gemm p) {
  constexpr int NTS = 80;   // bytes per row of a [128][32] tile (conflict-free 16-byte reads)
  constexpr int TRS = 288;  // bytes per row of a [32][128] tile (conflict-free transposing reads)
  constexpr int AB = A_TR ? 32 * TRS : 128 * NTS;
  constexpr int BB = B_TR ? 32 * TRS : 128 * NTS;
  __shared__ __attribute__((aligned(16))) char lds[2][AB + BB];

  const int n0 = blockIdx.x * 128, m0 = blockIdx.y * 128, z = blockIdx.z;
  const int kb = z * p.kchunk, ke = min(p.K, kb + p.kchunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;

  auto load = [&](const void* base, int64_t ld, int rows, int cols, bool tr, int r0, int k0, uint4 (&r)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i;
      int gr, gc;
      if (!tr) {
        gr = r0 + (ch >> 2);
        gc = k0 + 8 * (ch & 3);
      } else {
        gr = k0 + (ch >> 4);
        gc = r0 + 8 * (ch & 15);
      }
      r[i] = (gr < rows && gc + 8 <= cols) ? *(const uint4*)((const __bf16*)base + (int64_t)gr * ld + gc)
                                           : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store = [&](char* dst, bool tr, const uint4 (&r)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i;
      const int off = tr ? (ch >> 4) * TRS + (ch & 15) * 16 : (ch >> 2) * NTS + (ch & 3) * 16;
      *(uint4*)(dst + off) = r[i];
    }
  };
  // transposing fragment: lane (half, l32) gets column c0 + l32, k = 16s + 8 half + 0..7
  auto tr_frag = [&](const char* t, int s, int c0) __attribute__((always_inline)) {
    u32x4b w;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = 16 * s + 8 * half + 4 * tt + ((lane & 15) >> 2);
      const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const s16x4b x =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4b*)(t + row * TRS + 2 * col));
      const u32x2b y = __builtin_bit_cast(u32x2b, x);
      w[2 * tt] = y[0];
      w[2 * tt + 1] = y[1];
    }
    return __builtin_bit_cast(bf16x8, w);
  };
  auto frag = [&](const char* t, bool tr, int s, int c0) __attribute__((always_inline)) {
    if (tr) return tr_frag(t, s, c0);
    return *(const bf16x8*)(t + (c0 + l32) * NTS + 32 * s + 16 * half);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[i][j][t] = 0.f;

  uint4 ra[2], rb[2];
  if (kb < ke) {
    load(p.a, p.lda, p.a_rows, p.a_cols, A_TR, m0, kb, ra);
    load(p.b, p.ldb, p.b_rows, p.b_cols, B_TR, n0, kb, rb);
    store(lds[0], A_TR, ra);
    store(lds[0] + AB, B_TR, rb);
  }
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += 32) {
    const bool more = k0 + 32 < ke;
    if (more) {
      load(p.a, p.lda, p.a_rows, p.a_cols, A_TR, m0, k0 + 32, ra);
      load(p.b, p.ldb, p.b_rows, p.b_cols, B_TR, n0, k0 + 32, rb);
    }
    const char* ta = lds[buf];
    const char* tb = lds[buf] + AB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = frag(ta, A_TR, s, wm + 32 * i);
        fb[i] = frag(tb, B_TR, s, wn + 32 * i);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store(lds[buf ^ 1], A_TR, ra);
      store(lds[buf ^ 1] + AB, B_TR, rb);
    }
    __syncthreads();
    buf ^= 1;
  }

  // lane (half, l32) holds rows 8(t/4) + 4 half + t%4 of column l32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int m = m0 + wm + 32 * i + 8 * (t >> 2) + 4 * half + (t & 3);
        if (m >= p.M) continue;
        const float v = acc[i][j][t] * p.alpha;
        if (p.out_bf16)
          ((__bf16*)p.c)[(int64_t)m * p.ldc + n] = f2bf(v);
        else
          ((float*)p.c)[(int64_t)z * p.c_split + (int64_t)m * p.ldc + n] = v;
      }
    }
}

// fp32: one thread per output element, sequential fp32 accumulation.
template <bool A_TR, bool B_TR>
__global__ __launch_bounds__(256) void gemm_f32_kernel(Gemm p) {
  const int n = blockIdx.x * 16 + (threadIdx.x & 15);
  const int m = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int z = blockIdx.z;
  if (m >= p.M || n >= p.N) return;
  const int kb = z * p.kchunk, ke = min(p.K, kb + p.kchunk);
  const float* A = (const float*)p.a;
  const float* B = (const float*)p.b;
  float acc = 0.f;
  for (int k = kb; k < ke; ++k) {
    const float a = A_TR ? (k < p.a_rows && m < p.a_cols ? A[(int64_t)k * p.lda + m] : 0.f)
                         : (m < p.a_rows && k < p.a_cols ? A[(int64_t)m * p.lda + k] : 0.f);
    const float b = B_TR ? (k < p.b_rows && n < p.b_cols ? B[(int64_t)k * p.ldb + n] : 0.f)
                         : (n < p.b_rows && k < p.b_cols ? B[(int64_t)n * p.ldb + k] : 0.f);
    acc = fmaf(a, b, acc);
  }
  ((float*)p.c)[(int64_t)z * p.c_split + (int64_t)m * p.ldc + n] = acc * p.alpha;
}

// Sum of nsplit fp32 partials, in split order.
__global__ __launch_bounds__(256) void split_sum_kernel(const float* part, float* out, int64_t n, int nsplit) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < nsplit; ++z) s += part[(int64_t)z * n + i];
  out[i] = s;
}

template <bool A_TR, bool B_TR>
static void run_gemm(Gemm g, int nsplit, float* out, bool bf16, hipStream_t s) {
  // with nsplit > 1, g.c is the partial buffer and out receives the sum
  if (bf16) {
    const dim3 grid((g.N + 127) / 128, (g.M + 127) / 128, nsplit);
    hipLaunchKernelGGL((gemm_bf16_kernel<A_TR, B_TR>), grid, dim3(256), 0, s, g);
  } else {
    const dim3 grid((g.N + 15) / 16, (g.M + 15) / 16, nsplit);
    hipLaunchKernelGGL((gemm_f32_kernel<A_TR, B_TR>), grid, dim3(256), 0, s, g);
  }
  if (nsplit > 1) {
    const int64_t n = (int64_t)g.M * g.N;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)g.c, out,
                       n, nsplit);
  }
}

// ---------------------------------------------------------------------------
// Output projection backward
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return (float)((const T*)p)[i];
}
template <typename T>
__device__ __forceinline__ void st(void* p, int64_t i, float v) {
  ((T*)p)[i] = (T)v;
}

// A group of d/4 lanes per (token, slot j), four elements per lane: j < G*k
// a hard slot (dO_r row and dw), j == G*k the shared slot (dO_s row).
template <typename T>
__device__ __forceinline__ f32x4 ld4(const void* p, int64_t i) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 v = *(const bf16x4*)((const __bf16*)p + i);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return *(const f32x4*)((const float*)p + i);
  }
}
template <typename T>
__device__ __forceinline__ void st4(void* p, int64_t i, const f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 o = {f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
    *(bf16x4*)((__bf16*)p + i) = o;
  } else {
    *(f32x4*)((float*)p + i) = v;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void slot_bwd_kernel(OutProjBwdParams p) {
  const int L = p.d / 4;  // lanes per (token, slot): 8, 16 or 32
  const int64_t g = ((int64_t)blockIdx.x * 256 + threadIdx.x) / L;
  const int e = 4 * (threadIdx.x % L);
  const int64_t per = p.Gk + 1;
  if (g >= p.T * per) return;  // (whole lane groups leave together)
  const int64_t t = g / per;
  const int j = (int)(g - t * per);
  const float* da = p.da + t * p.Kd;
  const int hard = p.Gk * p.d;
  if (j == p.Gk) {  // the shared slot; without one (ablation layouts) its gradient is 0
    if (p.do_s)
      st4<T>(p.do_s, t * p.d + e, p.nsh ? *(const f32x4*)(da + hard + p.nob + e) : f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  const float w = (p.nob || p.weighted) ? p.w[t * p.Gk + j] : 0.f;
  const f32x4 o = ld4<T>(p.o_r, (t * p.Gk + j) * p.d + e);
  const f32x4 dslot = *(const f32x4*)(da + j * p.d + e);
  f32x4 gr;
  float dwacc = 0.f;
  if (p.nob) {  // [O, obar, s]
    const f32x4 dob = *(const f32x4*)(da + hard + e);
    gr = dslot + w * dob;
    for (int i = 0; i < 4; ++i) dwacc = fmaf(o[i], dob[i], dwacc);
  } else if (p.weighted) {  // [p O]
    gr = w * dslot;
    for (int i = 0; i < 4; ++i) dwacc = fmaf(o[i], dslot[i], dwacc);
  } else {  // [O]
    gr = dslot;
  }
  st4<T>(p.do_r, (t * p.Gk + j) * p.d + e, gr);
  for (int m = L / 2; m > 0; m >>= 1) dwacc += __shfl_xor(dwacc, m, 64);
  if (e == 0) p.dw[t * p.Gk + j] = dwacc;
}

// The slot vector A_t (what the forward GEMM multiplies by W_O), stored in
// the storage dtype: hard slots (scaled by w when weighted), obar in fp32
// then rounded, shared slot. Four consecutive columns per thread (d is a
// multiple of 4, so the four never straddle two slots).
template <typename T>
__global__ __launch_bounds__(256) void assemble_kernel(OutProjBwdParams p) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= p.T * p.Kd) return;
  const int64_t t = i4 / p.Kd;
  const int c = (int)(i4 - t * p.Kd);
  const int hard = p.Gk * p.d;
  f32x4 v;
  if (c < hard) {
    v = ld4<T>(p.o_r, t * hard + c);
    if (p.weighted) v *= p.w[t * p.Gk + c / p.d];
  } else if (c < hard + p.nob) {
    const int e = c - hard;
    v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.Gk; ++j) {
      const float w = p.w[t * p.Gk + j];
      const f32x4 o = ld4<T>(p.o_r, (t * p.Gk + j) * p.d + e);
      for (int q = 0; q < 4; ++q) v[q] = fmaf(w, o[q], v[q]);
    }
  } else {
    v = ld4<T>(p.o_s, t * p.d + (c - hard - p.nob));
  }
  st4<T>(p.a, i4, v);
}

template <typename T>
static void out_proj_bwd_typed(const OutProjBwdParams& p, bool bf16, hipStream_t s) {
  // dA = dy W_O^T: A' = dy [T][Dout], B' = W_O [Kd][Dout] (both along the contraction)
  Gemm g{};
  g.a = p.dy;
  g.b = p.w_o;
  g.c = p.da;
  g.lda = p.Dout;
  g.ldb = p.Dout;
  g.ldc = p.Kd;
  g.M = (int)p.T;
  g.N = p.Kd;
  g.K = p.Dout;
  g.a_rows = (int)p.T;
  g.a_cols = p.Dout;
  g.b_rows = p.Kd;
  g.b_cols = p.Dout;
  g.kchunk = (p.Dout + 31) / 32 * 32;
  g.alpha = 1.f;
  run_gemm<false, false>(g, 1, nullptr, bf16, s);
  const int64_t lanes = p.T * (p.Gk + 1) * (p.d / 4);
  hipLaunchKernelGGL(slot_bwd_kernel<T>, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, p);
  const int64_t n4 = p.T * p.Kd / 4;
  hipLaunchKernelGGL(assemble_kernel<T>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, p);
  // dW_O = A^T dy: A stored [T][Kd] and dy [T][Dout], both transposed
  Gemm h{};
  h.a = p.a;
  h.b = p.dy;
  h.c = p.nsplit > 1 ? (void*)p.part : (void*)p.dw_o;
  h.lda = p.Kd;
  h.ldb = p.Dout;
  h.ldc = p.Dout;
  h.c_split = (int64_t)p.Kd * p.Dout;
  h.M = p.Kd;
  h.N = p.Dout;
  h.K = (int)p.T;
  h.a_rows = (int)p.T;
  h.a_cols = p.Kd;
  h.b_rows = (int)p.T;
  h.b_cols = p.Dout;
  h.kchunk = p.kchunk;
  h.alpha = 1.f;
  run_gemm<true, true>(h, p.nsplit, p.dw_o, bf16, s);
}

hipError_t launch_out_proj_bwd(const OutProjBwdParams& p, bool bf16, hipStream_t s) {
  if (bf16)
    out_proj_bwd_typed<__bf16>(p, true, s);
  else
    out_proj_bwd_typed<float>(p, false, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router backward
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// selections per (group, expert): LDS histogram per block, then integer adds
__global__ __launch_bounds__(256) void count_kernel(RouteBwdParams p) {
  __shared__ int32_t h[kMaxRouterCols];
  const int GM = p.G * p.M;
  for (int i = threadIdx.x; i < GM; i += 256) h[i] = 0;
  __syncthreads();
  const int64_t n = p.T * p.G * p.K;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int g = (int)((i / p.K) % p.G);
    atomicAdd(&h[g * p.M + min(max(p.topk[i], 0), p.M - 1)], 1);  // (clamped: stays inside h)
  }
  __syncthreads();
  for (int i = threadIdx.x; i < GM; i += 256)
    if (h[i]) atomicAdd(&p.counts[i], h[i]);
}

// One thread per (token, group): dz of the renormalised weights or of the
// selected probabilities (and of the balance loss).
template <typename T>
__global__ __launch_bounds__(256) void dz_kernel(RouteBwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.T * p.G) return;
  const int64_t t = i / p.G;
  const int g = (int)(i - t * p.G);
  const float* zr = p.z + i * p.M;
  float pr[kMaxExperts], dp[kMaxExperts];
  float mx = -INFINITY;
  for (int m = 0; m < p.M; ++m) mx = fmaxf(mx, zr[m]);
  float sum = 0.f;
  for (int m = 0; m < p.M; ++m) {
    pr[m] = expf(zr[m] - mx);
    sum += pr[m];
  }
  const float inv = 1.f / sum;
  for (int m = 0; m < p.M; ++m) {
    pr[m] *= inv;
    dp[m] = 0.f;
  }
  int sel[kMaxExperts];  // (indices clamped to 0..M-1, as everywhere else)
  for (int j = 0; j < p.K; ++j) sel[j] = min(max(p.topk[i * p.K + j], 0), p.M - 1);
  const float* dw = p.dw + i * p.K;
  float ps = 0.f;
  for (int j = 0; j < p.K; ++j) ps += pr[sel[j]];
  float dww = 0.f;
  for (int j = 0; j < p.K; ++j) dww = fmaf(dw[j], pr[sel[j]] / ps, dww);
  for (int j = 0; j < p.K; ++j) dp[sel[j]] = p.wprob ? dw[j] : (dw[j] - dww) / ps;
  if (p.aux_coef != 0.f) {
    const float c = p.aux_coef * p.M / ((float)p.T * p.G) / ((float)p.T * p.K);
    for (int m = 0; m < p.M; ++m) dp[m] += c * (float)p.counts[g * p.M + m];
  }
  float pdp = 0.f;
  for (int m = 0; m < p.M; ++m) pdp = fmaf(pr[m], dp[m], pdp);
  const int GM = p.G * p.M;
  for (int m = 0; m < p.M; ++m) {
    const float d = pr[m] * (dp[m] - pdp);
    p.dz[t * GM + g * p.M + m] = d;
    st<T>(p.dzb, t * p.GMp + g * p.M + m, d);
    if (p.pbuf) p.pbuf[t * GM + g * p.M + m] = pr[m];
  }
  if (g == 0)
    for (int c = GM; c < p.GMp; ++c) st<T>(p.dzb, t * p.GMp + c, 0.f);
}

// Column sums over tokens, two levels (partials of kColChunk tokens, then
// their sum in chunk order): which = 0 sums dz into db_r, 1 sums p. In a
// block, thread (r, c) with c = tid % GM sums column c over the chunk's
// tokens r, r + R, ... (R = 256 / GM rows of threads, reads coalesced along
// the columns); the R partials are then added in LDS in row order.
__global__ __launch_bounds__(256) void colsum_kernel(RouteBwdParams p, int which) {
  __shared__ float red[256];
  const int GM = p.G * p.M;
  const int R = 256 / GM;
  const int c = threadIdx.x % GM, r = threadIdx.x / GM;
  const float* src = which ? p.pbuf : p.dz;
  const int64_t t0 = (int64_t)blockIdx.x * kColChunk, t1 = min(p.T, t0 + kColChunk);
  float s = 0.f;
  if (r < R)
    for (int64_t t = t0 + r; t < t1; t += R) s += src[t * GM + c];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < GM) {
    float tot = 0.f;
    for (int k = 0; k < R; ++k) tot += red[k * GM + threadIdx.x];
    p.colpart[((int64_t)which * p.nchunk + blockIdx.x) * GM + threadIdx.x] = tot;
  }
}

__global__ __launch_bounds__(256) void colsum_final_kernel(RouteBwdParams p) {
  const int GM = p.G * p.M;
  const int c = threadIdx.x;
  __shared__ float fP[kMaxRouterCols];
  float s = 0.f, P = 0.f;
  if (c < GM) {
    for (int k = 0; k < p.nchunk; ++k) s += p.colpart[(int64_t)k * GM + c];
    p.db_r[c] = s;
    if (p.aux_loss) {
      for (int k = 0; k < p.nchunk; ++k) P += p.colpart[((int64_t)p.nchunk + k) * GM + c];
      // f * P with f = count / (T k) and P = sum p / T
      fP[c] = ((float)p.counts[c] / ((float)p.T * p.K)) * (P / (float)p.T);
    }
  }
  if (!p.aux_loss) return;
  __syncthreads();
  if (c == 0) {
    float tot = 0.f;
    for (int i = 0; i < GM; ++i) tot += fP[i];
    *p.aux_loss = p.aux_coef * p.M * tot / p.G;
  }
}

template <typename T>
static void route_bwd_typed(const RouteBwdParams& p, bool bf16, hipStream_t s) {
  const int GM = p.G * p.M;
  const bool counts = p.aux_coef != 0.f || p.aux_loss;
  if (counts) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3((GM + 255) / 256), dim3(256), 0, s, p.counts, GM);
    const int64_t n = p.T * p.G * p.K;
    const unsigned nb = (unsigned)min((int64_t)1024, (n + 255) / 256);
    hipLaunchKernelGGL(count_kernel, dim3(nb), dim3(256), 0, s, p);
  }
  hipLaunchKernelGGL(dz_kernel<T>, dim3((unsigned)((p.T * p.G + 255) / 256)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(colsum_kernel, dim3(p.nchunk), dim3(256), 0, s, p, 0);
  if (p.aux_loss) hipLaunchKernelGGL(colsum_kernel, dim3(p.nchunk), dim3(256), 0, s, p, 1);
  hipLaunchKernelGGL(colsum_final_kernel, dim3(1), dim3(256), 0, s, p);
  // dW_r = dz^T x: dz stored [T][GMp], x [T][D], both transposed
  Gemm h{};
  h.a = p.dzb;
  h.b = p.x;
  h.c = p.nsplit > 1 ? (void*)p.part : (void*)p.dw_r;
  h.lda = p.GMp;
  h.ldb = p.D;
  h.ldc = p.D;
  h.c_split = (int64_t)GM * p.D;
  h.M = GM;
  h.N = p.D;
  h.K = (int)p.T;
  h.a_rows = (int)p.T;
  h.a_cols = p.GMp;
  h.b_rows = (int)p.T;
  h.b_cols = p.D;
  h.kchunk = p.kchunk;
  h.alpha = 1.f;
  run_gemm<true, true>(h, p.nsplit, p.dw_r, bf16, s);
  // dx = dz W_r: dz along the contraction, W_r stored [GM][D] (transposed)
  Gemm g{};
  g.a = p.dzb;
  g.b = p.w;
  g.c = p.dx;
  g.lda = p.GMp;
  g.ldb = p.D;
  g.ldc = p.D;
  g.M = (int)p.T;
  g.N = p.D;
  g.K = p.GMp;
  g.a_rows = (int)p.T;
  g.a_cols = p.GMp;
  g.b_rows = GM;
  g.b_cols = p.D;
  g.kchunk = p.GMp;
  g.out_bf16 = bf16 ? 1 : 0;
  g.alpha = 1.f;
  run_gemm<false, true>(g, 1, nullptr, bf16, s);
}

hipError_t launch_route_bwd(const RouteBwdParams& p, bool bf16, hipStream_t s) {
  if (bf16)
    route_bwd_typed<__bf16>(p, true, s);
  else
    route_bwd_typed<float>(p, false, s);
  return hipGetLastError();
}

}  // namespace gqe
