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
// is spread over d*elem/16 lanes; a wavefront load covers whole rows), keeps
// an fp32 running (max, sum, o) per row, and writes one partial per row. The
// inner loop is branch-free per lane: q.k uses v_dot2_f32_bf16 on packed
// pairs, the row reduction uses DPP lane permutes, keys past the split are
// loaded clamped and masked. K and V are read with non-temporal loads (each
// byte is used once per call; measured 6.9 vs 6.2 TB/s for a plain
// contiguous stream on this chip). A combine kernel merges the partials.
#include "gqe_internal.h"

namespace gqe {

DecodeSplit decode_split(int B, int G, int Smax, int k, int q_len) {
  DecodeSplit s;
  s.rows = (k + 1) * q_len;
  const int bg = B * G > 0 ? B * G : 1;
  // aim for ~2k blocks in total: at 16 x 8 heads x 64k keys, 2k blocks of
  // 4096 keys ran 1.5% faster than 4k blocks of 2048 (and 8k, 16k slower)
  int target = (2048 + bg - 1) / bg;
  if (target < 1) target = 1;
  int chunk = (Smax + target - 1) / target;
  chunk = ((chunk + 511) / 512) * 512;  // whole unrolled iterations (at most 512 keys)
  if (chunk < 512) chunk = 512;
  s.chunk = chunk;
  s.nsplit = (Smax + chunk - 1) / chunk;
  if (s.nsplit < 1) s.nsplit = 1;
  return s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Merge running softmax state (m, l, o) with another one; m is in log2 units
// (scores already multiplied by scale*log2(e)).
__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float m2, float l2,
                                            const float* o2, int n) {
  const float mn = fmaxf(m, m2);
  const float a1 = (m == -INFINITY) ? 0.f : exp2f(m - mn);
  const float a2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mn);
  l = l * a1 + l2 * a2;
  for (int i = 0; i < n; ++i) o[i] = o[i] * a1 + o2[i] * a2;
  m = mn;
}

// Sum over each aligned group of TPK lanes, left in every lane of the group:
// quad permutes (xor 1, xor 2), then the half-row and row mirrors, all as
// DPP moves (no LDS traffic); groups wider than a 16-lane row add shuffles.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int x = __builtin_bit_cast(int, v), y;
  switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true); break;   // quad_perm [1,0,3,2]
    case 1: y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); break;   // quad_perm [2,3,0,1]
    case 2: y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true); break;  // row_half_mirror
    default: y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true); break; // row_mirror
  }
  return v + __builtin_bit_cast(float, y);
}
template <int TPK>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (TPK >= 2) v = dpp_add(v, 0);
  if constexpr (TPK >= 4) v = dpp_add(v, 1);
  if constexpr (TPK >= 8) v = dpp_add(v, 2);
  if constexpr (TPK >= 16) v = dpp_add(v, 3);
  if constexpr (TPK >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (TPK >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Element i of a 4-dword vector, reinterpreted. The element is copied to a
// scalar first: bit-casting a vector subscript directly reads element 0 with
// this compiler.
__device__ __forceinline__ bf16x2 pair_at(const u32x4& v, int i) {
  const uint32_t w = v[i];
  return __builtin_bit_cast(bf16x2, w);
}
__device__ __forceinline__ float f32_at(const u32x4& v, int i) {
  const uint32_t w = v[i];
  return __builtin_bit_cast(float, w);
}

// Unpack a 16-byte key/value slice to fp32.
template <typename T>
__device__ __forceinline__ void to_f32(const u32x4& w, float* f);
template <>
__device__ __forceinline__ void to_f32<__bf16>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i];
    f[2 * i] = __builtin_bit_cast(float, x << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, x & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void to_f32<float>(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = f32_at(w, i);
}

// Partial q.k over this lane's 16-byte slice: bf16 pairs through
// v_dot2_f32_bf16 (exact products, fp32 sums), fp32 through FMAs.
template <typename T>
__device__ __forceinline__ float slice_dot(const u32x4& q, const u32x4& k);
template <>
__device__ __forceinline__ float slice_dot<__bf16>(const u32x4& q, const u32x4& k) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(pair_at(q, i), pair_at(k, i), acc, false);
  return acc;
}
template <>
__device__ __forceinline__ float slice_dot<float>(const u32x4& q, const u32x4& k) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = fmaf(f32_at(q, i), f32_at(k, i), acc);
  return acc;
}

constexpr float kDecodeRescaleLog2 = 8.0f;

template <typename T, int D, int RM, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  constexpr int VEC = 16 / (int)sizeof(T);  // elements per lane per key row
  constexpr int TPK = D / VEC;              // lanes per key row
  constexpr int KPB = 256 / TPK;            // keys per block-wide pass
  constexpr int U = RM <= 4 ? 8 : 4;        // passes per iteration (loads in flight)
  static_assert(TPK <= 64 && (64 % TPK) == 0, "key row must fit a wavefront");

  const int c_split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  // (a kv_len outside 0..S_max breaks the caller's contract; clamping keeps
  // every read inside the sequence's cache, the outputs are then unspecified)
  const int kvl = min(max(p.kv_len[b], 0), p.Smax);
  const int k_begin = c_split * p.chunk;
  if (k_begin >= kvl) return;  // the combine reads only the splits below kv_len
  const int k_end = min(k_begin + p.chunk, kvl);
  const int k_lo = p.kv_start ? p.kv_start[b] : 0;  // keys below are padding
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = tid % TPK;  // which 16-byte slice of the row
  const int kl = tid / TPK;    // key lane within a pass
  const float c = p.scale * 1.44269504088896340736f;

  // rows of (b, g): K*L routed rows (token t = r / K, slot r % K), then L
  // shared rows on group 0
  const int nrows = p.K * p.L + (g == 0 ? p.L : 0);
  u32x4 q[RM];
  int rpos[RM];
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    rpos[r] = -1;
    q[r] = u32x4{0u, 0u, 0u, 0u};
    if (r < nrows) {
      int t, head;
      if (r < p.K * p.L) {
        t = r / p.K;
        // (clamped as in the prefill: an out-of-range index reads inside q)
        head = g * p.M + min(max(p.topk[(((int64_t)b * p.L + t) * p.G + g) * p.K + (r % p.K)], 0), p.M - 1);
      } else {
        t = r - p.K * p.L;
        head = p.N;
      }
      rpos[r] = kvl - p.L + t;
      q[r] = *(const u32x4*)((const T*)p.q + (((int64_t)b * p.L + t) * (p.N + 1) + head) * D + part * VEC);
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

  // contiguous: the (b, g) slice of the cache; paged: the pool (the page
  // offset locates the row)
  const int64_t slice = PAGED ? 0 : ((int64_t)b * p.G + g) * (int64_t)p.Smax * D;
  const T* kb = (const T*)p.k + slice + part * VEC;
  const T* vb = (const T*)p.v + slice + part * VEC;
  // Paged: a pass covers KPB <= 64 consecutive keys and pages hold a power of
  // two >= 64 of them, so a pass lies in one page (one block-table entry per
  // pass); lanes clamped to the split's last key use that key's page.
  const int32_t* bt = PAGED ? p.block_table + (int64_t)b * p.max_pages : nullptr;
  const int pmask = (1 << p.page_shift) - 1;
  const int64_t pstride = (int64_t)p.G << p.page_shift;  // rows per page across the G heads
  const int64_t goff = (int64_t)g << p.page_shift;
  int64_t last_row = 0;
  if constexpr (PAGED) last_row = ((int64_t)bt[(k_end - 1) >> p.page_shift] * pstride + goff + ((k_end - 1) & pmask)) * D;

  for (int j0 = k_begin; j0 < k_end; j0 += U * KPB) {
    // keys past the split are loaded from its last key (always valid) and masked
    u32x4 kw[U], vw[U];
    int key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      key[u] = j0 + u * KPB + kl;
      int64_t off;
      if constexpr (PAGED) {
        const int key0 = min(j0 + u * KPB, k_end - 1);  // uniform: first key of the pass
        const int64_t page = bt[key0 >> p.page_shift];
        off = key[u] < k_end ? (page * pstride + goff + (key[u] & pmask)) * D : last_row;
      } else {
        off = (int64_t)min(key[u], k_end - 1) * D;
      }
      // the cache is read once per call: non-temporal loads stream it
      kw[u] = __builtin_nontemporal_load((const u32x4*)(kb + off));
      vw[u] = __builtin_nontemporal_load((const u32x4*)(vb + off));
    }
    float vf[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) to_f32<T>(vw[u], vf[u]);
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r < nrows) {  // uniform
        float s[U];
        float bm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float dot = group_sum<TPK>(slice_dot<T>(q[r], kw[u]));
          s[u] = (key[u] < k_end && key[u] <= rpos[r] && key[u] >= k_lo) ? dot * c : -INFINITY;
          bm = fmaxf(bm, s[u]);
        }
        // lazy rescale: move the reference max only when it grows by more
        // than 2^8 (or is still -inf), so most iterations skip the rescale
        const float mn = fmaxf(m[r], bm);
        const bool move = mn - m[r] > kDecodeRescaleLog2;  // NaN (both -inf) -> false
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          const float alpha = move ? ((m[r] == -INFINITY) ? 0.f : exp2f(m[r] - mn)) : 1.f;
          if (move) m[r] = mn;
          l[r] *= alpha;
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[r][i] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          // s finite implies m finite (it moved to at least s - 2^8)
          const float e = (s[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[u] - m[r]);
          l[r] += e;
#pragma unroll
          for (int i = 0; i < VEC; ++i) o[r][i] = fmaf(e, vf[u][i], o[r][i]);
        }
      }
    }
  }

  // merge the key lanes of the wavefront (lanes with equal `part`)
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
        merge_state(m[r], l[r], o[r], m2, l2, o2, VEC);
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
      merge_state(mm, ll, &oo, m2, l2, &o2, 1);
    }
    p.ws_o[(rec + r) * D + e] = oo;
    if (e == 0) {
      p.ws_ml[(rec + r) * 2 + 0] = mm;
      p.ws_ml[(rec + r) * 2 + 1] = ll;
    }
  }
}

// Combine the partials of the splits below kv_len: one block per (row, group,
// sequence), one thread per element; the largest split max first, then the
// rescaled sums, 8 splits per step.
template <typename T, int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeParams p) {
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z, e = threadIdx.x;
  const int nrows = p.K * p.L + (g == 0 ? p.L : 0);
  if (r >= nrows) return;
  const int kvl = min(max(p.kv_len[b], 0), p.Smax);  // as in the split kernel
  const int ns = min(p.nsplit, (kvl + p.chunk - 1) / p.chunk);
  const int64_t rec0 = ((int64_t)b * p.G + g) * p.nsplit;
  float mm = -INFINITY;
  for (int cs = 0; cs < ns; ++cs) mm = fmaxf(mm, p.ws_ml[((rec0 + cs) * p.R + r) * 2]);
  float ll = 0.f, oo = 0.f;
  int cs = 0;
  for (; cs + 8 <= ns; cs += 8) {
    float m8[8], l8[8], o8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t rr = (rec0 + cs + u) * p.R + r;
      m8[u] = p.ws_ml[rr * 2 + 0];
      l8[u] = p.ws_ml[rr * 2 + 1];
      o8[u] = p.ws_o[rr * D + e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float a = (m8[u] == -INFINITY) ? 0.f : exp2f(m8[u] - mm);
      ll = fmaf(l8[u], a, ll);
      oo = fmaf(o8[u], a, oo);
    }
  }
  for (; cs < ns; ++cs) {
    const int64_t rr = (rec0 + cs) * p.R + r;
    const float m2 = p.ws_ml[rr * 2 + 0];
    const float a = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mm);
    ll = fmaf(p.ws_ml[rr * 2 + 1], a, ll);
    oo = fmaf(p.ws_o[rr * D + e], a, oo);
  }
  T* out;
  if (r < p.K * p.L) {
    const int t = r / p.K, slot = r % p.K;
    out = (T*)p.o_r + ((((int64_t)b * p.L + t) * p.G + g) * p.K + slot) * D;
  } else {
    const int t = r - p.K * p.L;
    out = (T*)p.o_s + ((int64_t)b * p.L + t) * D;
  }
  out[e] = (T)(oo / ll);
}

template <typename T, int D>
static void launch_decode_t(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(p.nsplit, p.G, p.B);
  const bool paged = p.block_table != nullptr;
  if (p.R <= 4) {
    if (paged) hipLaunchKernelGGL((decode_split_kernel<T, D, 4, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_split_kernel<T, D, 4, false>), grid, dim3(256), 0, s, p);
  } else if (p.R <= 8) {
    if (paged) hipLaunchKernelGGL((decode_split_kernel<T, D, 8, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_split_kernel<T, D, 8, false>), grid, dim3(256), 0, s, p);
  } else {
    if (paged) hipLaunchKernelGGL((decode_split_kernel<T, D, kMaxDecodeRows, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_split_kernel<T, D, kMaxDecodeRows, false>), grid, dim3(256), 0, s, p);
  }
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.R, p.G, p.B), dim3(D), 0, s, p);
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
