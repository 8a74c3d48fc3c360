// Router, top-k selection and per-(group, expert) token lists.
//
// GQE review (paper.oopus.info), section 二 路由器: per token i and group g,
// z = r_g(x_i) in R^M, p = softmax(z), K_g = TopK(p, k), and the renormalised
// weights w_m = p_m / sum_{m' in K_g} p_{m'}.
//
// Router scores are a skinny product z[T, G*M] = x[T, D] W_r^T. For bf16 it
// runs on MFMA (16x16x32 bf16 -> fp32): a workgroup owns 64 tokens (16 when
// there are at most 16) and all G*M experts, its wavefronts splitting the
// features, streaming x once from
// HBM with 16-byte loads; W_r (at most 256 x D bf16) stays hot in L2. The
// fp32 path is a plain VALU dot product.
// The reduction order is fixed, so the emitted logits - and therefore the
// selection, which is a pure function of them - are deterministic.
#include "gqe_internal.h"

namespace gqe {

constexpr int kRouteTok = 16;  // tokens per workgroup (fp32)

// Selection epilogue: z for kRouteTok tokens in LDS ([tok][G*M], bias
// included). One thread per (token, group): TopK by repeated first-maximum
// scans (strictly greater wins, so ties keep the lower index), indices
// written ascending, weights exp(z_m - zmax) / sum over the selected set and,
// when asked for, the probabilities exp(z_m - zmax) / sum over all M.
__device__ void route_select_store(const float* zs, int ntok, int64_t tok0,
                                   const RouteParams& p) {
  const int GM = p.G * p.M;
  for (int e = threadIdx.x; e < ntok * p.G; e += blockDim.x) {
    const int t = e / p.G, g = e % p.G;
    const float* z = zs + t * GM + g * p.M;
    const int64_t tok = tok0 + t;
    if (p.logits) {
      for (int m = 0; m < p.M; ++m) p.logits[(tok * p.G + g) * p.M + m] = z[m];
    }
    uint32_t chosen = 0;
    float zmax = -INFINITY;
    for (int r = 0; r < p.k; ++r) {
      int best = -1;
      float bv = 0.f;
      for (int m = 0; m < p.M; ++m) {
        if ((chosen >> m) & 1u) continue;
        if (best < 0 || z[m] > bv) { best = m; bv = z[m]; }
      }
      chosen |= 1u << best;
      if (r == 0) zmax = bv;  // the first pick is the maximum
    }
    float den = 0.f, all = 0.f;
    for (int m = 0; m < p.M; ++m) {
      const float e = expf(z[m] - zmax);
      all += e;
      if ((chosen >> m) & 1u) den += e;
    }
    int j = 0;
    const int64_t o = (tok * p.G + g) * p.k;
    for (int m = 0; m < p.M; ++m) {
      if ((chosen >> m) & 1u) {
        const float e = expf(z[m] - zmax);
        p.topk_idx[o + j] = m;
        p.topk_w[o + j] = e / den;
        if (p.topk_p) p.topk_p[o + j] = e / all;
        ++j;
      }
    }
  }
}

// bf16 router scores on MFMA. A block takes TT 16-token tiles (four; one
// when there are at most 16 tokens, as in decode, so that the LDS partials
// leave room for up to 16 wavefronts) and all G*M experts; its W wavefronts
// split the 32-wide feature steps, and the W partial score tiles are summed
// in LDS in wavefront order (fixed, so the logits are deterministic). Each
// wavefront loads a batch of SB steps - x fragments of its TT token tiles and
// W_r fragments of its NT expert tiles - before the batch's MFMAs, so the
// loads of a batch are in flight together; each W_r fragment feeds TT MFMAs.
// 16x16x32 operand layout: lane l holds A[l%16][8*(l/16) .. +8] (token row,
// 8 consecutive features) and B[8*(l/16) .. +8][l%16] (expert column); the
// result D[4*(l/16)+i][l%16] lands in register i.

template <int NT, int SB, int MAXW, int TT>
__global__ __launch_bounds__(64 * MAXW) void route_bf16_kernel(RouteParams p) {
  constexpr int BT = 16 * TT;  // tokens per block
  extern __shared__ float zpart[];  // [W][64][GM]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, W = blockDim.x >> 6;
  const int64_t tok0 = (int64_t)blockIdx.x * BT;
  const int ntok = (int)((p.T - tok0) < BT ? (p.T - tok0) : BT);
  const int GM = p.G * p.M;
  const int D = p.D;
  const __bf16* x = (const __bf16*)p.x;
  const __bf16* wr = (const __bf16*)p.w;

  const int row = lane & 15;
  const int kof = 8 * (lane >> 4);
  // token rows past T read row T-1; their scores are not used
  const __bf16* xrow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
    xrow[tt] = x + min(tok0 + tt * 16 + row, p.T - 1) * (int64_t)D;
  // expert rows past G*M read row G*M-1; their scores are not stored
  const __bf16* wrow[NT];
#pragma unroll
  for (int e = 0; e < NT; ++e) wrow[e] = wr + (int64_t)min(e * 16 + row, GM - 1) * D;
  const int nsteps = (D + 31) / 32;
  const int st0 = (int)((int64_t)w * nsteps / W), st1 = (int)((int64_t)(w + 1) * nsteps / W);

  f32x4 acc[TT][NT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int e = 0; e < NT; ++e) acc[tt][e] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bf16x8 zero8 = {};
  for (int sb = st0; sb < st1; sb += SB) {
    bf16x8 a[SB][TT], bw[SB][NT];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      // D is a multiple of 8; a 32-wide step may run past D only in its tail
      const int c = (sb + i) * 32 + kof;
      const bool ok = sb + i < st1 && c < D;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) a[i][tt] = ok ? *(const bf16x8*)(xrow[tt] + c) : zero8;
#pragma unroll
      for (int e = 0; e < NT; ++e) bw[i][e] = ok ? *(const bf16x8*)(wrow[e] + c) : zero8;
    }
#pragma unroll
    for (int i = 0; i < SB; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int e = 0; e < NT; ++e)
          acc[tt][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][tt], bw[i][e], acc[tt][e], 0, 0, 0);
  }
  float* zw = zpart + (size_t)w * BT * GM;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int e = 0; e < NT; ++e) {
      const int ex = e * 16 + row;  // output column = expert
      if (ex < GM) {
#pragma unroll
        for (int i = 0; i < 4; ++i) zw[(tt * 16 + 4 * (lane >> 4) + i) * GM + ex] = acc[tt][e][i];
      }
    }
  __syncthreads();
  // sum the wavefront partials in order, add the bias; result in slice 0
  for (int idx = threadIdx.x; idx < BT * GM; idx += blockDim.x) {
    float z = zpart[idx];
    for (int ww = 1; ww < W; ++ww) z += zpart[(size_t)ww * BT * GM + idx];
    zpart[idx] = z + (p.bias ? p.bias[idx % GM] : 0.f);
  }
  __syncthreads();
  route_select_store(zpart, ntok, tok0, p);
}

// fp32 router scores: one thread per (token, expert), sequential fp32 FMAs.
__global__ __launch_bounds__(64) void route_f32_kernel(RouteParams p) {
  __shared__ float zs[kRouteTok * kMaxRouterCols];
  const int64_t tok0 = (int64_t)blockIdx.x * kRouteTok;
  const int ntok = (int)((p.T - tok0) < kRouteTok ? (p.T - tok0) : kRouteTok);
  const int GM = p.G * p.M;
  const float* x = (const float*)p.x;
  const float* w = (const float*)p.w;
  for (int e = threadIdx.x; e < ntok * GM; e += blockDim.x) {
    const int t = e / GM, ex = e % GM;
    const float* xr = x + (tok0 + t) * (int64_t)p.D;
    const float* wr = w + (int64_t)ex * p.D;
    float s = 0.f;
    for (int c = 0; c < p.D; ++c) s = fmaf(xr[c], wr[c], s);
    zs[t * GM + ex] = s + (p.bias ? p.bias[ex] : 0.f);
  }
  __syncthreads();
  route_select_store(zs, ntok, tok0, p);
}

// ---------------------------------------------------------------------------
// Token lists: count (per 64-token chunk) -> exclusive scan -> scatter. Ranks
// inside a chunk come from wavefront ballots, so the lists are ascending and
// deterministic without atomics.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t selected_mask(const ListParams& p, int b, int t, int g) {
  if (t >= p.S) return 0u;
  const int32_t* s = p.topk_idx + (((int64_t)b * p.S + t) * p.G + g) * p.k;
  uint32_t m = 0;
  for (int j = 0; j < p.k; ++j) m |= 1u << s[j];
  return m;
}

__global__ __launch_bounds__(64) void list_count_kernel(ListParams p) {
  const int chunk = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int t = chunk * kListChunk + lane;
  for (int g = 0; g < p.G; ++g) {
    const uint32_t sel = selected_mask(p, b, t, g);
    for (int m = 0; m < p.M; ++m) {
      const uint64_t bal = __ballot((sel >> m) & 1u);
      if (lane == 0)
        p.counts[(((int64_t)b * p.G + g) * p.M + m) * p.nchunk + chunk] = __popcll(bal);
    }
  }
}

// One block per (b, g): exclusive scan of the chunk counts of each expert,
// in place, and the list offsets.
__global__ __launch_bounds__(256) void list_scan_kernel(ListParams p) {
  __shared__ int wave_tot[4];
  __shared__ int carry_s;
  const int bg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int running = 0;  // identical in every thread
  for (int m = 0; m < p.M; ++m) {
    if (tid == 0) p.list_off[(int64_t)bg * (p.M + 1) + m] = running;
    int32_t* cnt = p.counts + ((int64_t)bg * p.M + m) * p.nchunk;
    int carry = 0;
    for (int c0 = 0; c0 < p.nchunk; c0 += 256) {
      const int c = c0 + tid;
      const int v = c < p.nchunk ? cnt[c] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      if (lane == 63) wave_tot[wv] = incl;
      __syncthreads();
      int before = 0, tot = 0;
      for (int i = 0; i < 4; ++i) {
        if (i < wv) before += wave_tot[i];
        tot += wave_tot[i];
      }
      if (c < p.nchunk) cnt[c] = running + carry + before + incl - v;
      carry += tot;
      __syncthreads();
    }
    running += carry;
  }
  if (tid == 0) p.list_off[(int64_t)bg * (p.M + 1) + p.M] = running;
  (void)carry_s;
}

__global__ __launch_bounds__(64) void list_scatter_kernel(ListParams p) {
  const int chunk = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int t = chunk * kListChunk + lane;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g = 0; g < p.G; ++g) {
    const uint32_t sel = selected_mask(p, b, t, g);
    const int64_t bg = (int64_t)b * p.G + g;
    for (int m = 0; m < p.M; ++m) {
      const bool mine = (sel >> m) & 1u;
      const uint64_t bal = __ballot(mine);
      if (mine) {
        const int pos = p.counts[(bg * p.M + m) * p.nchunk + chunk] + __popcll(bal & below);
        p.list_tok[bg * ((int64_t)p.k * p.S) + pos] = t;
      }
    }
  }
}

template <int NT, int SB, int MAXW, int TT>
static void launch_route_bf16(const RouteParams& p, hipStream_t s) {
  // wavefronts per block: about 256 features each, at most MAXW, and the
  // [W][16*TT][G*M] fp32 partials within 64 KB of LDS
  constexpr int BT = 16 * TT;
  const int GM = p.G * p.M;
  int W = 1;
  while (W < MAXW && W * 2 * 256 <= p.D && W * 2 * BT * GM * 4 <= 65536) W *= 2;
  const size_t lds = (size_t)W * BT * GM * sizeof(float);
  const unsigned nblk = (unsigned)((p.T + BT - 1) / BT);
  hipLaunchKernelGGL((route_bf16_kernel<NT, SB, MAXW, TT>), dim3(nblk), dim3(64 * W), lds, s, p);
}

hipError_t launch_route(const RouteParams& p, bool bf16, hipStream_t s) {
  if (bf16) {
    const int nt = (p.G * p.M + 15) / 16;  // 16-expert tiles
    // batch size and block size keep the fragments and accumulators within
    // the register budget of the block size
    if (p.T <= 16) {
      // a few tokens (decode): one token tile per block, so that the partials
      // leave room for more wavefronts over the features
      if (nt <= 1) launch_route_bf16<1, 4, 16, 1>(p, s);
      else if (nt <= 2) launch_route_bf16<2, 4, 16, 1>(p, s);
      else if (nt <= 4) launch_route_bf16<4, 2, 16, 1>(p, s);
      else if (nt <= 8) launch_route_bf16<8, 1, 16, 1>(p, s);
      else launch_route_bf16<16, 1, 8, 1>(p, s);
    } else if (nt <= 1) launch_route_bf16<1, 4, 16, 4>(p, s);
    else if (nt <= 2) launch_route_bf16<2, 2, 16, 4>(p, s);
    else if (nt <= 4) launch_route_bf16<4, 1, 16, 4>(p, s);
    else if (nt <= 8) launch_route_bf16<8, 1, 4, 4>(p, s);
    else launch_route_bf16<16, 1, 4, 4>(p, s);
  } else {
    const unsigned nblk = (unsigned)((p.T + kRouteTok - 1) / kRouteTok);
    hipLaunchKernelGGL(route_f32_kernel, dim3(nblk), dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_lists(const ListParams& p, hipStream_t s) {
  hipLaunchKernelGGL(list_count_kernel, dim3(p.nchunk, p.B), dim3(64), 0, s, p);
  hipLaunchKernelGGL(list_scan_kernel, dim3(p.B * p.G), dim3(256), 0, s, p);
  hipLaunchKernelGGL(list_scatter_kernel, dim3(p.nchunk, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace gqe
