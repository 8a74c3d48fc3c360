// Sparse-query decode attention against a [B, G, S_max, d] KV cache.
//
// GQA tutorial (zone.ci), 技术深化 and 工程实操: in decode the queries are few
// and the keys are the whole history; the causal mask uses each query's
// absolute position (kv_len - q_len + t), never a top-left triangle. Decode
// is bound by reading the KV cache (GQA deep-dive, §1.1), so the kernel is
// built around streaming K and V once per (sequence, group): every selected
// head of the group (and the shared head, on group 0) is served from the
// same bytes (the KV head is never repeated).
//
// Split-sequence: block (split c, group g, sequence b) reads keys
// [c*chunk, min((c+1)*chunk, kv_len)) with coalesced 16-byte loads (a key row
// is spread over d*elem/16 lanes), keeps an fp32 running (max, sum, o) per
// row, and writes one partial per row. A combine kernel merges the partials.
#include "gqe_internal.h"

namespace gqe {

DecodeSplit decode_split(int B, int G, int Smax, int k, int q_len) {
  DecodeSplit s;
  s.rows = (k + 1) * q_len;
  const int bg = B * G > 0 ? B * G : 1;
  int target = (8192 + bg - 1) / bg;  // aim for ~8k blocks in total
  if (target < 1) target = 1;
  int chunk = (Smax + target - 1) / target;
  chunk = ((chunk + 255) / 256) * 256;  // whole unrolled iterations
  if (chunk < 256) chunk = 256;
  s.chunk = chunk;
  s.nsplit = (Smax + chunk - 1) / chunk;
  if (s.nsplit < 1) s.nsplit = 1;
  return s;
}

template <typename T>
struct Vec16;
template <>
struct Vec16<__bf16> {
  typedef bf16x8 type;
  static constexpr int n = 8;
};
template <>
struct Vec16<float> {
  typedef f32x4 type;
  static constexpr int n = 4;
};

// Merge running softmax state (m, l, o) with another one; m in raw score
// units, exponentials exp2((s - m) * c).
__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float m2, float l2,
                                            const float* o2, int n, float c) {
  const float mn = fmaxf(m, m2);
  const float a1 = (m == -INFINITY) ? 0.f : exp2f((m - mn) * c);
  const float a2 = (m2 == -INFINITY) ? 0.f : exp2f((m2 - mn) * c);
  l = l * a1 + l2 * a2;
  for (int i = 0; i < n; ++i) o[i] = o[i] * a1 + o2[i] * a2;
  m = mn;
}

template <typename T, int D, int RM>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  using V = typename Vec16<T>::type;
  constexpr int VEC = Vec16<T>::n;   // elements per lane per key
  constexpr int TPK = D / VEC;       // lanes per key row
  constexpr int KPB = 256 / TPK;     // keys per block-wide pass
  constexpr int U = 4;               // passes in flight
  static_assert(TPK <= 64 && (64 % TPK) == 0, "key row must fit a wavefront");

  const int c_split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int kvl = p.kv_len[b];
  const int k_begin = c_split * p.chunk;
  if (k_begin >= kvl) return;  // the combine reads only the splits below kv_len
  const int k_end = min(k_begin + p.chunk, kvl);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = tid % TPK;        // which VEC-slice of d
  const int kl = tid / TPK;          // key lane within a pass
  const float c = p.scale * 1.44269504088896340736f;

  // rows of (b, g): K*L routed rows (token t = r / K, slot r % K), then L
  // shared rows on group 0
  const int nrows = p.K * p.L + (g == 0 ? p.L : 0);
  float q[RM][VEC];
  int rpos[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    rpos[r] = -1;
#pragma unroll
    for (int i = 0; i < VEC; ++i) q[r][i] = 0.f;
    if (r < nrows) {
      int t, head;
      if (r < p.K * p.L) {
        t = r / p.K;
        head = g * p.M + p.topk[(((int64_t)b * p.L + t) * p.G + g) * p.K + (r % p.K)];
      } else {
        t = r - p.K * p.L;
        head = p.N;
      }
      rpos[r] = kvl - p.L + t;
      const T* qp = (const T*)p.q + (((int64_t)b * p.L + t) * (p.N + 1) + head) * D + part * VEC;
      const V qv = *(const V*)qp;
#pragma unroll
      for (int i = 0; i < VEC; ++i) q[r][i] = (float)qv[i];
    }
  }

  float m[RM], l[RM], o[RM][VEC];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[r][i] = 0.f;
  }

  const T* kb = (const T*)p.k + ((int64_t)b * p.G + g) * (int64_t)p.Smax * D + part * VEC;
  const T* vb = (const T*)p.v + ((int64_t)b * p.G + g) * (int64_t)p.Smax * D + part * VEC;

  for (int j0 = k_begin; j0 < k_end; j0 += U * KPB) {
    V kv[U], vv[U];
    int key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      key[u] = j0 + u * KPB + kl;
      if (key[u] < k_end) {
        kv[u] = *(const V*)(kb + (int64_t)key[u] * D);
        vv[u] = *(const V*)(vb + (int64_t)key[u] * D);
      }
    }
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r < nrows) {
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float acc = 0.f;
          if (key[u] < k_end) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc = fmaf(q[r][i], (float)kv[u][i], acc);
          }
#pragma unroll
          for (int o2 = 1; o2 < TPK; o2 <<= 1) acc += __shfl_xor(acc, o2, 64);
          s[u] = (key[u] < k_end && key[u] <= rpos[r]) ? acc : -INFINITY;
        }
        float mx = m[r];
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u]);
        if (mx != -INFINITY) {  // else nothing visible yet for this row here
          const float alpha = (m[r] == -INFINITY) ? 0.f : exp2f((m[r] - mx) * c);
          l[r] *= alpha;
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[r][i] *= alpha;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float e = (s[u] == -INFINITY) ? 0.f : exp2f((s[u] - mx) * c);
            l[r] += e;
#pragma unroll
            for (int i = 0; i < VEC; ++i) o[r][i] = fmaf(e, (key[u] < k_end) ? (float)vv[u][i] : 0.f, o[r][i]);
          }
          m[r] = mx;
        }
      }
    }
  }

  // merge key lanes inside the wavefront (lanes with equal `part`)
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    if (r < nrows) {
#pragma unroll
      for (int off = TPK; off < 64; off <<= 1) {
        const float m2 = __shfl_xor(m[r], off, 64);
        const float l2 = __shfl_xor(l[r], off, 64);
        float o2[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) o2[i] = __shfl_xor(o[r][i], off, 64);
        merge_state(m[r], l[r], o[r], m2, l2, o2, VEC, c);
      }
    }
  }
  // merge the 4 wavefronts through LDS
  __shared__ float sm[4][RM][2];
  __shared__ float so[4][RM][D];
  if (lane < TPK) {
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r < nrows) {
        sm[wave][r][0] = m[r];
        sm[wave][r][1] = l[r];
#pragma unroll
        for (int i = 0; i < VEC; ++i) so[wave][r][part * VEC + i] = o[r][i];
      }
    }
  }
  __syncthreads();
  // thread (r, e) finalises row r, element e of this split's partial
  const int64_t rec = (((int64_t)b * p.G + g) * p.nsplit + c_split) * p.R;
  for (int idx = tid; idx < nrows * D; idx += 256) {
    const int r = idx / D, e = idx % D;
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float m2 = sm[w][r][0], l2 = sm[w][r][1], o2 = so[w][r][e];
      merge_state(mm, ll, &oo, m2, l2, &o2, 1, c);
    }
    p.ws_o[(rec + r) * D + e] = oo;
    if (e == 0) {
      p.ws_ml[(rec + r) * 2 + 0] = mm;
      p.ws_ml[(rec + r) * 2 + 1] = ll;
    }
  }
}

// Combine the partials of the splits below kv_len: one block per (g, b).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int kvl = p.kv_len[b];
  const int ns = min(p.nsplit, (kvl + p.chunk - 1) / p.chunk);
  const int nrows = p.K * p.L + (g == 0 ? p.L : 0);
  const float c = p.scale * 1.44269504088896340736f;
  const int64_t rec0 = ((int64_t)b * p.G + g) * p.nsplit;
  for (int idx = threadIdx.x; idx < nrows * D; idx += blockDim.x) {
    const int r = idx / D, e = idx % D;
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
    for (int cs = 0; cs < ns; ++cs) {
      const int64_t rr = (rec0 + cs) * p.R + r;
      const float m2 = p.ws_ml[rr * 2 + 0], l2 = p.ws_ml[rr * 2 + 1];
      const float o2 = p.ws_o[rr * D + e];
      merge_state(mm, ll, &oo, m2, l2, &o2, 1, c);
    }
    const float val = oo / ll;
    T* out;
    if (r < p.K * p.L) {
      const int t = r / p.K, slot = r % p.K;
      out = (T*)p.o_r + ((((int64_t)b * p.L + t) * p.G + g) * p.K + slot) * D;
    } else {
      const int t = r - p.K * p.L;
      out = (T*)p.o_s + ((int64_t)b * p.L + t) * D;
    }
    out[e] = (T)val;
  }
}

template <typename T, int D>
static void launch_decode_t(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(p.nsplit, p.G, p.B);
  if (p.R <= 4)
    hipLaunchKernelGGL((decode_split_kernel<T, D, 4>), grid, dim3(256), 0, s, p);
  else if (p.R <= 8)
    hipLaunchKernelGGL((decode_split_kernel<T, D, 8>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, kMaxDecodeRows>), grid, dim3(256), 0, s, p);
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.G, p.B), dim3(256), 0, s, p);
}

hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s) {
  if (bf16) {
    switch (d) {
      case 32: launch_decode_t<__bf16, 32>(p, s); break;
      case 64: launch_decode_t<__bf16, 64>(p, s); break;
      case 128: launch_decode_t<__bf16, 128>(p, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (d) {
      case 32: launch_decode_t<float, 32>(p, s); break;
      case 64: launch_decode_t<float, 64>(p, s); break;
      case 128: launch_decode_t<float, 128>(p, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace gqe
