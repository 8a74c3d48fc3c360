// Internal declarations shared by the HIP kernels and the C ABI layer.
// Nothing here is part of the public interface (include/gqe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Router limits (checked by the ABI layer).
constexpr int kMaxExperts = 32;      // M
constexpr int kMaxRouterCols = 256;  // G*M
// Decode: rows per (sequence, group) kept in registers.
constexpr int kMaxDecodeRows = 16;   // (k+1)*q_len
// Token chunk of the list builder (one wavefront).
constexpr int kListChunk = 64;

struct RouteParams {
  const void* x;         // [T, D]
  const void* w;         // [GM, D]
  const float* bias;     // [GM] or null
  float* logits;         // [T, G, M] or null
  int32_t* topk_idx;     // [T, G, k]
  float* topk_w;         // [T, G, k]
  float* topk_p;         // [T, G, k] or null: p of the selected experts
  int64_t T;
  int D, G, M, k;
};

struct ListParams {
  const int32_t* topk_idx;  // [B*S, G, k]
  int32_t* list_off;        // [B, G, M+1]
  int32_t* list_tok;        // [B, G, k*S]
  int32_t* counts;          // workspace [B, G, M, nchunk]
  int B, S, G, M, k, nchunk;
};

struct PrefillParams {
  const void* q;          // [B, S, N+1, d]
  const void* k;          // [B, G, S, d]
  const void* v;          // [B, G, S, d]
  const int32_t* topk;    // [B*S, G, k]
  void* o_r;              // [B, S, G, k, d]
  void* o_s;              // [B, S, d]
  int B, S, N, G, M, K;
  float scale;            // 1/sqrt(d)
  // optional (training): per row ln sum_j exp(q.k_j / sqrt(d)), the softmax
  // normaliser the backward pass recomputes P with; null = not written
  float* lse_r;           // [B, S, G, k]
  float* lse_s;           // [B, S]
};

struct BwdParams {
  PrefillParams f;        // forward inputs and outputs (o_r, o_s) and the row lse
  const void* do_r;       // [B, S, G, k, d]
  const void* do_s;       // [B, S, d]
  void* dq;               // [B, S, N+1, d] (rows of unselected heads untouched)
  void* dk;               // [B, G, S, d]
  void* dv;               // [B, G, S, d]
  // workspace: rows packed per (b, v), row r of (b, v) at (b*(G+1) + v)*Rp + r
  void* qp;               // [B, G+1, Rp, d] q of the row
  void* dop;              // [B, G+1, Rp, d] dO of the row
  float* nlse;            // [B, G+1, Rp] -lse*sqrt(d)
  float* ndel;            // [B, G+1, Rp] -dO.O
  float* part;            // [2 (dK, dV), 2 (group 0, shared head), B, S, d] (bf16 path)
  int Rp;                 // S*k rounded up to a multiple of 32
};

// Output projection backward (slot layouts as in OutProjParams).
struct OutProjBwdParams {
  const void* o_r;        // [T, G*k*d]
  const float* w;         // [T, G*k]
  const void* o_s;        // [T, d]
  const void* w_o;        // [Kd, Dout]
  const void* dy;         // [T, Dout]
  void* do_r;             // [T, G*k*d] out
  float* dw;              // [T, G*k] out
  void* do_s;             // [T, d] out
  float* dw_o;            // [Kd, Dout] out (fp32)
  float* da;              // workspace [T, Kd] fp32: dy W_O^T
  void* a;                // workspace [T, Kd] dtype: the slot vectors
  float* part;            // workspace [nsplit, Kd, Dout] fp32 (nsplit > 1)
  int64_t T;
  int Gk, d, Dout, Kd, nob, nsh, weighted, nsplit, kchunk;
};

// Router backward.
struct RouteBwdParams {
  const void* x;          // [T, D]
  const void* w;          // [GM, D]
  const float* z;         // [T, G, M] logits
  const int32_t* topk;    // [T, G, k]
  const float* dw;        // [T, G, k]
  float* dz;              // [T, GM] out (workspace when the caller wants none)
  void* dzb;              // workspace [T, GMp] dtype, zero past GM
  float* pbuf;            // workspace [T, GM] softmax (balance loss only)
  int32_t* counts;        // workspace [G*M]
  float* colpart;         // workspace [2, nchunk, GM]
  void* dx;               // [T, D] out
  float* dw_r;            // [GM, D] out
  float* db_r;            // [GM] out
  float* aux_loss;        // [1] out or null
  float* part;            // workspace [nsplit, GM, D] (nsplit > 1)
  float aux_coef;
  int wprob;              // 1: dw is the gradient of the selected p, 0: of the renormalised w
  int64_t T;
  int D, G, M, K, GMp, nchunk, nsplit, kchunk;
};

struct DecodeParams {
  const void* q;          // [B, L, N+1, d]
  const void* k;          // [B, G, Smax, d]
  const void* v;
  const int32_t* kv_len;  // [B]
  const int32_t* topk;    // [B*L, G, k]
  void* o_r;              // [B, L, G, k, d]
  void* o_s;              // [B, L, d]
  float* ws_o;            // [B, G, nsplit, R, d]
  float* ws_ml;           // [B, G, nsplit, R, 2]
  int B, L, Smax, N, G, M, K, R, nsplit, chunk;
  float scale;
  // paged cache (block_table non-null): k, v are page pools [n_pages, G, P, d]
  // with P = 1 << page_shift; key j of sequence b is row j % P of page
  // block_table[b * max_pages + j / P]
  const int32_t* block_table;
  int page_shift, max_pages;
  const int32_t* kv_start;  // [B] first valid key (left padding) or null
};

struct OutProjParams {
  const void* o_r;        // [T, G*k*d]
  const float* w;         // [T, G*k]
  const void* o_s;        // [T, d]
  const void* w_o;        // [Kd, Dout]
  void* y;                // [T, Dout]
  int64_t T;
  int Gk, d, Dout;
  // slot layout: [hard slots | obar (nob = d columns, or 0) | shared (nsh =
  // d columns, or 0)]; with `weighted` each hard slot is scaled by its weight
  // in w (the router probability p in the weighted-concatenation layout)
  int nob, nsh, weighted;
};

struct ProjParams {
  const void* x;           // [T, D], T = B*L
  const void* w_q;         // [(N+1)*d, D]
  const void* w_k;         // [G*d, D]
  const void* w_v;         // [G*d, D]
  const int32_t* topk;     // [T, G, k]
  const int32_t* kv_len;   // [B] (decode) or null (prefill)
  void* q;                 // [T, N+1, d]
  void* k;                 // [B, G, Smax, d]
  void* v;                 // [B, G, Smax, d]
  int T, B, L, D, N, G, M, K, d, Smax;
};

// Decode split geometry shared by the workspace query and the launcher.
struct DecodeSplit {
  int rows;    // (k+1)*q_len
  int chunk;   // keys per split
  int nsplit;  // ceil(Smax / chunk)
};
DecodeSplit decode_split(int B, int G, int Smax, int k, int q_len);

// Compute units of the current device (launch shapes that must fill the chip).
int device_cus();

hipError_t launch_route(const RouteParams& p, bool bf16, hipStream_t s);
hipError_t launch_lists(const ListParams& p, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int d, bool bf16, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s);
hipError_t launch_out_proj(const OutProjParams& p, bool bf16, hipStream_t s);
hipError_t launch_proj(const ProjParams& p, bool bf16, hipStream_t s);
hipError_t launch_prefill_bwd(const BwdParams& p, int d, bool bf16, hipStream_t s);
hipError_t launch_out_proj_bwd(const OutProjBwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_route_bwd(const RouteBwdParams& p, bool bf16, hipStream_t s);
// split of a long contraction for the weight-gradient products: kchunk is a
// multiple of 32, nsplit * kchunk >= K
void gemm_split(int64_t K, int tiles, int& nsplit, int& kchunk);
constexpr int kColChunk = 1024;  // tokens per partial of the router's column sums

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(__bf16 h) { return (float)h; }
__device__ __forceinline__ __bf16 f2bf(float f) { return (__bf16)f; }  // round to nearest even

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l writes LDS bytes [lds + 16 l, +16), lds a
// wavefront-uniform LDS byte address, which the instruction takes from m0. It
// is issued from asm so that the compiler does not track it as a pending LDS
// store: it would otherwise wait for every such load (vmcnt(0)) before any
// LDS read it cannot prove disjoint, the transposing reads among them, which
// leaves no load in flight across a step. The caller waits on vmcnt itself
// before the barrier that publishes the data. The instruction writes no
// register; the nop is the wait state an m0 write needs before it.
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds);
}
__device__ __forceinline__ void lds_dma16(const void* gptr, const void* lds) {
  __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_addr(lds)) : "memory");
}

// The same with a wavefront-uniform base address and a 32-bit per-lane byte
// offset (the saddr form): moving the base to the next block is scalar work.
// Five wait states cover a base that a VALU op (readfirstlane) wrote.
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t off, const void* lds) {
  __asm__ volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_addr(lds))
                   : "memory");
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): a load at an offset at or
// past `bytes` returns zeros (the range check of a raw buffer), so a block
// that runs past the end of a tensor needs no clamped addresses. Word 3
// selects 32-bit data, as a raw buffer of the gfx9 family needs; the words
// are made wavefront-uniform (SGPRs).
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from a buffer (this lane's byte offset `off`) straight
// into LDS bytes [lds + 16 l, +16), as lds_dma16; lanes past the buffer's end
// write zeros. Five wait states cover resource words a VALU op
// (readfirstlane) wrote.
__device__ __forceinline__ void lds_dma16_b(i32x4 rsrc, uint32_t off, const void* lds) {
  __asm__ volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc),
                   "{m0}"(lds_addr(lds))
                   : "memory");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace gqe
