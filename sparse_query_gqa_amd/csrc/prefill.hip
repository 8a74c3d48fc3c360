// Sparse-query causal prefill attention.
//
// GQE review (paper.oopus.info), section 二: only the k selected query heads
// of each group (plus the always-on shared head) attend; the group's KV head
// stays dense. GQA tutorial (zone.ci), 技术深化: head h reads KV head
// floor(h/M), never a repeated copy; scores q.k/sqrt(d), additive causal mask.
//
// Work decomposition ("position-major" packing). For sequence b and virtual
// group v in 0..G (v == G is the shared head, which reads KV head 0) the rows
// are the selected (token, slot) pairs, token-major: row r of a routed group
// is token r/k, slot r%k; row r of the shared group is token r. A workgroup
// owns 128 consecutive rows, so every tile holds exactly k rows per token
// whatever the routing skew, and all of them read the same KV head: each
// K/V tile is staged once in LDS and used by every selected head of the
// group.
//
// bf16 path: 4 wavefronts x 32 rows. Per 64-key block each wavefront computes
// S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, so that every
// lane owns one query row in both products (row max, row sum and rescale are
// per-lane scalars; the two lane halves are combined with one exchange).
// Online softmax in fp32 with exp2 and scale*log2(e) folded into one FMA.
#include "gqe_internal.h"

namespace gqe {

constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;
constexpr int kTileRows = kRowsPerWave * kWaves;  // 128
constexpr int kKeyBlock = 64;
constexpr int kKPad = 8;  // bf16 elements of padding per K row in LDS
constexpr int kVPad = 8;  // per V^T row

struct TileCoord {
  int b, v, tile;  // tile index within (b, v): rows [tile*128, tile*128+128)
  bool valid;
};

// Block -> tile. Blocks are spread round-robin over the 8 XCDs, so block w
// is re-mapped to a logical tile index such that each XCD walks a contiguous
// range of the (b, v, tile) order: its concurrently running workgroups read
// the same KV head and share it in that XCD's L2. Within a (b, v) tiles run
// from the longest causal extent to the shortest.
__device__ __forceinline__ TileCoord tile_of_block(const PrefillParams& p, int tiles_r,
                                                  int tiles_s) {
  const int per_b = p.G * tiles_r + tiles_s;
  const int total = p.B * per_b;
  const int nblk = gridDim.x;
  const int per_xcd = nblk / 8;
  const int w = blockIdx.x;
  const int logical = (w % 8) * per_xcd + (w / 8);
  TileCoord c;
  c.valid = logical < total;
  int rem = c.valid ? logical : 0;
  // order: v-major over (v, b) so groups sharing a KV head sit together
  // (the shared head, v == G, reads KV head 0 and follows group 0).
  int vslot = rem / (p.B * tiles_r);
  if (vslot < 1) {  // group 0
    c.v = 0;
    c.b = rem / tiles_r;
    c.tile = tiles_r - 1 - rem % tiles_r;
  } else {
    rem -= p.B * tiles_r;
    if (rem < p.B * tiles_s) {  // shared head next to group 0
      c.v = p.G;
      c.b = rem / tiles_s;
      c.tile = tiles_s - 1 - rem % tiles_s;
    } else {
      rem -= p.B * tiles_s;
      const int vv = 1 + rem / (p.B * tiles_r);
      rem %= (p.B * tiles_r);
      c.v = vv;
      c.b = rem / tiles_r;
      c.tile = tiles_r - 1 - rem % tiles_r;
    }
  }
  return c;
}

// Row r of (b, v) -> token position, slot, query head.
__device__ __forceinline__ void row_info(const PrefillParams& p, int b, int v, int r, int& pos,
                                         int& slot, int& head) {
  if (v == p.G) {
    pos = r;
    slot = 0;
    head = p.N;
  } else {
    pos = r / p.K;
    slot = r - pos * p.K;
    head = v * p.M + p.topk[(((int64_t)b * p.S + pos) * p.G + v) * p.K + slot];
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillParams p, int tiles_r,
                                                              int tiles_s) {
  static_assert(D == 32 || D == 64 || D == 128, "head dim");
  constexpr int KS = D / 16;                       // MFMA k-steps over d
  constexpr int DB = D / 32;                       // 32-wide d blocks of O^T
  constexpr int LD_PASSES = kKeyBlock * D / (256 * 8);  // 16-byte loads per thread
  __shared__ __bf16 Ks[kKeyBlock][D + kKPad];
  __shared__ __bf16 Vt[D][kKeyBlock + kVPad];

  const TileCoord tc = tile_of_block(p, tiles_r, tiles_s);
  if (!tc.valid) return;
  const int b = tc.b, v = tc.v;
  const int kvh = (v == p.G) ? 0 : v;
  const int nrows = (v == p.G) ? p.S : p.S * p.K;
  const int r0 = tc.tile * kTileRows;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  // this lane's query row
  const int my_r = r0 + wave * kRowsPerWave + l32;
  const int last_r = min(r0 + kTileRows, nrows) - 1;
  const bool row_ok = my_r < nrows;
  int pos, slot, head;
  row_info(p, b, v, row_ok ? my_r : last_r, pos, slot, head);
  int pos_last, s_, h_;
  row_info(p, b, v, last_r, pos_last, s_, h_);
  int pos_first;
  row_info(p, b, v, r0, pos_first, s_, h_);

  // Q^T fragments (B operand of S^T = K Q^T): d = 16*s + 8*half + [0,8)
  const __bf16* qrow = (const __bf16*)p.q + (((int64_t)b * p.S + pos) * (p.N + 1) + head) * D;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(qrow + 16 * s + 8 * half);

  const __bf16* kbase = (const __bf16*)p.k + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;
  const __bf16* vbase = (const __bf16*)p.v + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale * 1.44269504088896340736f;  // scale * log2(e)

  const int nblocks = pos_last / kKeyBlock + 1;
  bf16x8 kreg[LD_PASSES], vreg[LD_PASSES];
  const bf16x8 zero8 = {};

  auto gload = [&](int kb) {
#pragma unroll
    for (int ps = 0; ps < LD_PASSES; ++ps) {
      const int e = (ps * 256 + tid) * 8;
      const int key = e / D, col = e % D;
      const int gk = kb * kKeyBlock + key;
      if (gk < p.S) {
        kreg[ps] = *(const bf16x8*)(kbase + (int64_t)gk * D + col);
        vreg[ps] = *(const bf16x8*)(vbase + (int64_t)gk * D + col);
      } else {
        kreg[ps] = zero8;
        vreg[ps] = zero8;
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int ps = 0; ps < LD_PASSES; ++ps) {
      const int e = (ps * 256 + tid) * 8;
      const int key = e / D, col = e % D;
      *(bf16x8*)&Ks[key][col] = kreg[ps];
#pragma unroll
      for (int i = 0; i < 8; ++i) Vt[col + i][key] = vreg[ps][i];
    }
  };

  gload(0);
  lstore();
  __syncthreads();

  for (int kb = 0; kb < nblocks; ++kb) {
    if (kb + 1 < nblocks) gload(kb + 1);

    // S^T for two 32-key halves of the block
    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[sb][j] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = *(const bf16x8*)&Ks[sb * 32 + l32][16 * s + 8 * half];
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[sb], 0, 0, 0);
      }
    }
    // causal mask only on blocks that reach past the tile's first position
    if (kb * kKeyBlock + kKeyBlock - 1 > pos_first) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb * kKeyBlock + sb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
          if (key > pos) sacc[sb][j] = -INFINITY;
        }
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 16; ++j) bmax = fmaxf(bmax, sacc[sb][j]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(m_run, bmax);  // finite: key 0 is visible to every row
    const float alpha = exp2f((m_run - m_new) * c);
    const float mc = m_new * c;
    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = exp2f(fmaf(sacc[sb][j], c, -mc));
        psum += e;
        pf[sb][j >> 3][j & 7] = f2bf(e);
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[i][j] *= alpha;

    // O^T += V^T P^T. Contraction index of step st of key half sb, lane half h,
    // element t <-> key sb*32 + 16*st + 8*(t/4) + 4*h + t%4 (the S^T layout).
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kc = sb * 32 + 16 * st + 4 * half;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const __bf16* vr = &Vt[db * 32 + l32][kc];
          const bf16x4 lo = *(const bf16x4*)vr;
          const bf16x4 hi = *(const bf16x4*)(vr + 8);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[sb][st], oacc[db], 0, 0, 0);
        }
      }

    if (kb + 1 < nblocks) {
      __syncthreads();
      lstore();
      __syncthreads();
    }
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  __bf16* out = (v == p.G)
                    ? (__bf16*)p.o_s + ((int64_t)b * p.S + pos) * D
                    : (__bf16*)p.o_r + ((((int64_t)b * p.S + pos) * p.G + v) * p.K + slot) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      bf16x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = f2bf(oacc[db][4 * jq + i] * inv);
      *(bf16x4*)(out + db * 32 + 8 * jq + 4 * half) = o4;
    }
}

// fp32 path: one wavefront per query row; lanes over keys for the scores,
// lanes over d for P V. Plain fp32 arithmetic throughout.
template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows_r = (int64_t)p.S * p.K, per_b = p.G * rows_r + p.S;
  if (grow >= p.B * per_b) return;
  const int b = (int)(grow / per_b);
  int64_t rem = grow - b * per_b;
  const int v = rem < p.G * rows_r ? (int)(rem / rows_r) : p.G;
  const int r = (int)(v == p.G ? rem - p.G * rows_r : rem - v * rows_r);
  int pos, slot, head;
  row_info(p, b, v, r, pos, slot, head);
  const int kvh = (v == p.G) ? 0 : v;
  const float* q = (const float*)p.q + (((int64_t)b * p.S + pos) * (p.N + 1) + head) * D;
  const float* K = (const float*)p.k + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;
  const float* V = (const float*)p.v + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;
  constexpr int DL = (D + 63) / 64;
  float o[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 <= pos; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j <= pos) {
      float acc = 0.f;
      for (int e = 0; e < D; ++e) acc = fmaf(q[e], K[(int64_t)j * D + e], acc);
      s = acc * p.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = expf(m - mn);
    const float pj = (j <= pos) ? expf(s - mn) : 0.f;
    l = l * alpha + wave_sum(pj);
    const int nk = min(64, pos + 1 - j0);
#pragma unroll
    for (int i = 0; i < DL; ++i) o[i] *= alpha;
    for (int t = 0; t < nk; ++t) {
      const float pt = __shfl(pj, t, 64);
#pragma unroll
      for (int i = 0; i < DL; ++i) {
        const int e = lane + 64 * i;
        if (e < D) o[i] = fmaf(pt, V[(int64_t)(j0 + t) * D + e], o[i]);
      }
    }
    m = mn;
  }
  float* out = (v == p.G) ? (float*)p.o_s + ((int64_t)b * p.S + pos) * D
                          : (float*)p.o_r + ((((int64_t)b * p.S + pos) * p.G + v) * p.K + slot) * D;
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    const int e = lane + 64 * i;
    if (e < D) out[e] = o[i] / l;
  }
}

hipError_t launch_prefill(const PrefillParams& p, int d, bool bf16, hipStream_t s) {
  if (bf16) {
    const int tiles_r = (p.S * p.K + kTileRows - 1) / kTileRows;
    const int tiles_s = (p.S + kTileRows - 1) / kTileRows;
    const int total = p.B * (p.G * tiles_r + tiles_s);
    const int nblk = ((total + 7) / 8) * 8;
    switch (d) {
      case 32: hipLaunchKernelGGL(prefill_bf16_kernel<32>, dim3(nblk), dim3(256), 0, s, p, tiles_r, tiles_s); break;
      case 64: hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(nblk), dim3(256), 0, s, p, tiles_r, tiles_s); break;
      case 128: hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(nblk), dim3(256), 0, s, p, tiles_r, tiles_s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    const int64_t rows = (int64_t)p.B * ((int64_t)p.G * p.S * p.K + p.S);
    const unsigned nblk = (unsigned)((rows + 3) / 4);
    switch (d) {
      case 32: hipLaunchKernelGGL(prefill_f32_kernel<32>, dim3(nblk), dim3(256), 0, s, p); break;
      case 64: hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3(nblk), dim3(256), 0, s, p); break;
      case 128: hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3(nblk), dim3(256), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace gqe
