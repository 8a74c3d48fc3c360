// C ABI of the GQE layer: argument validation and launch geometry.
//
// Every check runs before anything is enqueued, so a rejected call writes
// nothing. Unsupported head layouts are rejected rather than mapped
// (GQA tutorial, zone.ci, 扩展验证组合). Nothing here allocates, frees or
// synchronises; all work goes onto the caller's stream.
#include <math.h>
#include <stdlib.h>
#include <stdio.h>

#include <mutex>

#include "../../include/gqe.h"
#include "gqe_internal.h"

using namespace gqe;

// Scratch memory of gqe_attn_decode_noalloc: the split partials live in this
// file-scope device array instead of a caller workspace. Every GPU the library
// runs on holds its own copy until the process ends. In host code the name
// stands for a host-side shadow, not a device address: the device address is
// looked up once per device with hipGetSymbolAddress and only that pointer is
// ever handed to kernels.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up on the first
// call on that device. Returns GQE_OK and the address, or GQE_ERR_HIP.
int scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQE_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GQE_ERR_HIP;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return GQE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool trace_on() {
  static int on = -1;
  if (on < 0) {
    const char* e = getenv("GQE_TRACE");
    on = (e && *e && *e != '0') ? 1 : 0;
  }
  return on == 1;
}

// Shape checks common to every entry point. Empty (B or S == 0) is valid.
int check_dims(const gqe_dims* d, bool need_D = true) {
  if (!d) return GQE_ERR_INVALID_ARG;
  if (d->B < 0 || d->S < 0 || d->D <= 0 || d->N <= 0 || d->G <= 0 || d->k <= 0 || d->d <= 0)
    return GQE_ERR_INVALID_ARG;
  if (d->dtype != GQE_BF16 && d->dtype != GQE_F32) return GQE_ERR_UNSUPPORTED;
  if (d->N % d->G != 0) return GQE_ERR_UNSUPPORTED;
  const int M = d->N / d->G;
  if (d->k > M) return GQE_ERR_UNSUPPORTED;
  if (M > kMaxExperts || d->G * M > kMaxRouterCols) return GQE_ERR_UNSUPPORTED;
  if (d->d != 32 && d->d != 64 && d->d != 128) return GQE_ERR_UNSUPPORTED;
  if (need_D && d->D % 8 != 0) return GQE_ERR_UNSUPPORTED;
  // every element offset must fit the 64-bit arithmetic used by the kernels
  // and the int32 token positions
  if ((int64_t)d->B * d->S > (int64_t)INT32_MAX) return GQE_ERR_UNSUPPORTED;
  return GQE_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return GQE_OK;
  if (trace_on()) fprintf(stderr, "[gqe] HIP error: %s\n", hipGetErrorString(e));
  return GQE_ERR_HIP;
}

int prefill_common(const gqe_dims* d, const void* q, const void* k, const void* v,
                   const int32_t* topk_idx, void* o_routed, void* o_shared, float* lse_r,
                   float* lse_s, void* stream) {
  int st = check_dims(d, false);
  if (st) return st;
  // one KV head's keys are read through a raw buffer of S*d*2 bytes (32-bit size)
  if ((int64_t)d->S * d->d * 2 > (int64_t)UINT32_MAX) return GQE_ERR_UNSUPPORTED;
  if (!q || !k || !v || !topk_idx || !o_routed || !o_shared) return GQE_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, topk_idx, o_routed, o_shared, lse_r, lse_s};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQE_ERR_ALIGNMENT;
  // rows per (sequence, group) and tile counts must stay in int32
  if ((int64_t)d->S * d->k > (int64_t)INT32_MAX / 2) return GQE_ERR_UNSUPPORTED;
  if (d->B == 0 || d->S == 0) return GQE_OK;
  PrefillParams pp{q, k, v, topk_idx, o_routed, o_shared, d->B, d->S, d->N, d->G, d->N / d->G,
                   d->k, (float)(1.0 / sqrt((double)d->d)), lse_r, lse_s};
  if (trace_on())
    fprintf(stderr, "[gqe] prefill B=%d S=%d N=%d G=%d k=%d d=%d dtype=%d lse=%d\n", d->B, d->S,
            d->N, d->G, d->k, d->d, d->dtype, lse_r != nullptr);
  return hip_status(launch_prefill(pp, d->d, d->dtype == GQE_BF16, (hipStream_t)stream));
}

// Backward workspace: packed q and dO rows, -lse*sqrt(d) and -dO.O per row,
// and (bf16) the two fp32 partial sums of KV head 0's dK and dV.
struct BwdLayout {
  int Rp;
  size_t qp, dop, nlse, ndel, part, part_bytes, total;
};
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
BwdLayout bwd_layout(const gqe_dims* d) {
  BwdLayout L{};
  L.Rp = (int)((((int64_t)d->S * d->k) + 31) / 32 * 32);
  const size_t rows = (size_t)d->B * (d->G + 1) * (size_t)L.Rp;
  const size_t esz = d->dtype == GQE_BF16 ? 2 : 4;
  size_t off = 0;
  L.qp = off;
  off += round256(rows * d->d * esz);
  L.dop = off;
  off += round256(rows * d->d * esz);
  L.nlse = off;
  off += round256(rows * 4);
  L.ndel = off;
  off += round256(rows * 4);
  L.part = off;
  L.part_bytes = d->dtype == GQE_BF16 ? round256((size_t)4 * d->B * d->S * d->d * 4) : 0;
  off += L.part_bytes;
  L.total = off;
  return L;
}

// Output-projection backward workspace: dA (fp32), the slot vectors
// (dtype) and the split partials of dW_O.
struct OutProjBwdLayout {
  int Kd, nsplit, kchunk;
  size_t da, a, part, total;
};
OutProjBwdLayout out_proj_bwd_layout(const gqe_dims* d, int32_t mode, int64_t T) {
  OutProjBwdLayout L{};
  L.Kd = d->G * d->k * d->d + (mode == GQE_SLOTS_FULL ? 2 * d->d : 0);
  const int tiles = ((L.Kd + 127) / 128) * ((d->D + 127) / 128);
  gemm_split(T, tiles, L.nsplit, L.kchunk);
  const size_t esz = d->dtype == GQE_BF16 ? 2 : 4;
  size_t off = 0;
  L.da = off;
  off += round256((size_t)T * L.Kd * 4);
  L.a = off;
  off += round256((size_t)T * L.Kd * esz);
  L.part = off;
  if (L.nsplit > 1) off += round256((size_t)L.nsplit * L.Kd * d->D * 4);
  L.total = off;
  return L;
}

// Router backward workspace: dz (fp32, when the caller takes none), dz in
// the storage dtype padded to GMp columns, the softmax (balance loss), the
// selection counts, the column-sum partials and the split partials of dW_r.
struct RouteBwdLayout {
  int GM, GMp, nchunk, nsplit, kchunk;
  size_t dz, dzb, pbuf, counts, colpart, part, total;
};
RouteBwdLayout route_bwd_layout(const gqe_dims* d) {
  RouteBwdLayout L{};
  const int64_t T = (int64_t)d->B * d->S;
  L.GM = d->N;
  L.GMp = (L.GM + 31) / 32 * 32;
  L.nchunk = (int)((T + kColChunk - 1) / kColChunk);
  const int tiles = ((L.GM + 127) / 128) * ((d->D + 127) / 128);
  gemm_split(T, tiles, L.nsplit, L.kchunk);
  const size_t esz = d->dtype == GQE_BF16 ? 2 : 4;
  size_t off = 0;
  L.dz = off;
  off += round256((size_t)T * L.GM * 4);
  L.dzb = off;
  off += round256((size_t)T * L.GMp * esz);
  L.pbuf = off;
  off += round256((size_t)T * L.GM * 4);
  L.counts = off;
  off += round256((size_t)L.GM * 4);
  L.colpart = off;
  off += round256((size_t)2 * L.nchunk * L.GM * 4);
  L.part = off;
  if (L.nsplit > 1) off += round256((size_t)L.nsplit * L.GM * d->D * 4);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* gqe_status_string(int status) {
  switch (status) {
    case GQE_OK: return "GQE_OK";
    case GQE_ERR_INVALID_ARG: return "GQE_ERR_INVALID_ARG: null pointer or inconsistent size";
    case GQE_ERR_UNSUPPORTED: return "GQE_ERR_UNSUPPORTED: head layout, head_dim, top-k or dtype not supported";
    case GQE_ERR_ALIGNMENT: return "GQE_ERR_ALIGNMENT: device pointer not 16-byte aligned";
    case GQE_ERR_WORKSPACE: return "GQE_ERR_WORKSPACE: workspace missing or too small";
    case GQE_ERR_HIP: return "GQE_ERR_HIP: the HIP runtime refused a launch";
    case GQE_ERR_SCRATCH: return "GQE_ERR_SCRATCH: the call needs more than the library's static scratch";
    default: return "unknown gqe status";
  }
}

int gqe_version(void) { return 10000; }

size_t gqe_route_workspace_bytes(const gqe_dims* d) {
  if (check_dims(d) != GQE_OK) return 0;
  const int64_t nchunk = (d->S + kListChunk - 1) / kListChunk;
  return (size_t)d->B * d->G * (d->N / d->G) * nchunk * sizeof(int32_t);
}

int gqe_route(const gqe_dims* d, const void* x, const void* w_router, const float* b_router,
              float* logits, int32_t* topk_idx, float* topk_w, float* topk_p,
              int32_t* list_off, int32_t* list_tok, void* workspace, size_t ws_bytes,
              void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (!x || !w_router || !topk_idx || !topk_w) return GQE_ERR_INVALID_ARG;
  if ((list_off == nullptr) != (list_tok == nullptr)) return GQE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w_router, b_router, logits, topk_idx, topk_w, topk_p, list_off, list_tok};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GQE_ERR_ALIGNMENT;
  const bool lists = list_off != nullptr;
  if (lists) {
    const size_t need = gqe_route_workspace_bytes(d);
    if (need > 0 && (!workspace || ws_bytes < need)) return GQE_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return GQE_ERR_ALIGNMENT;
  }
  const int64_t T = (int64_t)d->B * d->S;
  if (T == 0) return GQE_OK;
  hipStream_t s = (hipStream_t)stream;
  RouteParams rp{x, w_router, b_router, logits, topk_idx, topk_w, topk_p, T, d->D, d->G, d->N / d->G, d->k};
  if (trace_on())
    fprintf(stderr, "[gqe] route T=%lld D=%d G=%d M=%d k=%d lists=%d\n", (long long)T, d->D, d->G,
            d->N / d->G, d->k, (int)lists);
  st = hip_status(launch_route(rp, d->dtype == GQE_BF16, s));
  if (st || !lists) return st;
  ListParams lp{topk_idx, list_off, list_tok, (int32_t*)workspace, d->B, d->S, d->G, d->N / d->G,
                d->k, (d->S + kListChunk - 1) / kListChunk};
  return hip_status(launch_lists(lp, s));
}

int gqe_attn_prefill(const gqe_dims* d, const void* q, const void* k, const void* v,
                     const int32_t* topk_idx, void* o_routed, void* o_shared, void* stream) {
  return prefill_common(d, q, k, v, topk_idx, o_routed, o_shared, nullptr, nullptr, stream);
}

int gqe_attn_prefill_train(const gqe_dims* d, const void* q, const void* k, const void* v,
                           const int32_t* topk_idx, void* o_routed, void* o_shared,
                           float* lse_routed, float* lse_shared, void* stream) {
  if (!lse_routed || !lse_shared) return GQE_ERR_INVALID_ARG;
  return prefill_common(d, q, k, v, topk_idx, o_routed, o_shared, lse_routed, lse_shared, stream);
}

size_t gqe_attn_prefill_bwd_workspace_bytes(const gqe_dims* d) {
  if (check_dims(d, false) != GQE_OK) return 0;
  if ((int64_t)d->S * d->k > (int64_t)INT32_MAX / 2) return 0;
  return bwd_layout(d).total;
}

int gqe_attn_prefill_bwd(const gqe_dims* d, const void* q, const void* k, const void* v,
                         const int32_t* topk_idx, const void* o_routed, const void* o_shared,
                         const float* lse_routed, const float* lse_shared, const void* do_routed,
                         const void* do_shared, void* dq, void* dk, void* dv, void* workspace,
                         size_t ws_bytes, void* stream) {
  int st = check_dims(d, false);
  if (st) return st;
  if (!q || !k || !v || !topk_idx || !o_routed || !o_shared || !lse_routed || !lse_shared ||
      !do_routed || !do_shared || !dq || !dk || !dv)
    return GQE_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, topk_idx, o_routed, o_shared, lse_routed, lse_shared,
                        do_routed, do_shared, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQE_ERR_ALIGNMENT;
  if ((int64_t)d->S * d->k > (int64_t)INT32_MAX / 2) return GQE_ERR_UNSUPPORTED;
  if (d->B == 0 || d->S == 0) return GQE_OK;
  const BwdLayout L = bwd_layout(d);
  if (!workspace || ws_bytes < L.total) return GQE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GQE_ERR_ALIGNMENT;
  char* ws = (char*)workspace;
  BwdParams bp{};
  bp.f = PrefillParams{q, k, v, topk_idx, const_cast<void*>(o_routed), const_cast<void*>(o_shared),
                       d->B, d->S, d->N, d->G, d->N / d->G, d->k, (float)(1.0 / sqrt((double)d->d)),
                       const_cast<float*>(lse_routed), const_cast<float*>(lse_shared)};
  bp.do_r = do_routed;
  bp.do_s = do_shared;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.qp = ws + L.qp;
  bp.dop = ws + L.dop;
  bp.nlse = (float*)(ws + L.nlse);
  bp.ndel = (float*)(ws + L.ndel);
  bp.part = L.part_bytes ? (float*)(ws + L.part) : nullptr;
  bp.Rp = L.Rp;
  if (trace_on())
    fprintf(stderr, "[gqe] prefill_bwd B=%d S=%d N=%d G=%d k=%d d=%d dtype=%d Rp=%d\n", d->B, d->S,
            d->N, d->G, d->k, d->d, d->dtype, L.Rp);
  return hip_status(launch_prefill_bwd(bp, d->d, d->dtype == GQE_BF16, (hipStream_t)stream));
}

size_t gqe_decode_workspace_bytes(const gqe_dims* d, int32_t q_len) {
  if (check_dims(d, false) != GQE_OK || q_len <= 0) return 0;
  const DecodeSplit sp = decode_split(d->B, d->G, d->S, d->k, q_len);
  const size_t recs = (size_t)d->B * d->G * sp.nsplit * sp.rows;
  const size_t o_bytes = recs * d->d * sizeof(float);
  return o_bytes + recs * 2 * sizeof(float);
}

// Argument checks of gqe_attn_decode and gqe_attn_decode_noalloc, everything
// but the workspace. Returns GQE_OK (with *empty set for a call with nothing
// to do) or the error.
static int decode_check(const gqe_dims* d, int32_t q_len, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* kv_len, const int32_t* topk_idx,
                        void* o_routed, void* o_shared, bool* empty) {
  int st = check_dims(d, false);
  if (st) return st;
  if (q_len < 0) return GQE_ERR_INVALID_ARG;
  if (!q || !k_cache || !v_cache || !kv_len || !topk_idx || !o_routed || !o_shared)
    return GQE_ERR_INVALID_ARG;
  if (q_len > d->S && d->B > 0) return GQE_ERR_INVALID_ARG;  // kv_len <= S_max cannot hold
  if ((int64_t)(d->k + 1) * q_len > kMaxDecodeRows) return GQE_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQE_ERR_ALIGNMENT;
  *empty = d->B == 0 || q_len == 0;
  return GQE_OK;
}

// Launch of a checked decode call with its split partials at `workspace`
// (at least gqe_decode_workspace_bytes(d, q_len) bytes, 16-byte aligned).
static int decode_launch(const gqe_dims* d, int32_t q_len, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* kv_len, const int32_t* topk_idx,
                         void* o_routed, void* o_shared, void* workspace, void* stream) {
  const DecodeSplit sp = decode_split(d->B, d->G, d->S, d->k, q_len);
  const size_t recs = (size_t)d->B * d->G * sp.nsplit * sp.rows;
  float* ws_o = (float*)workspace;
  float* ws_ml = ws_o + recs * d->d;
  DecodeParams dp{q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared, ws_o, ws_ml,
                  d->B, q_len, d->S, d->N, d->G, d->N / d->G, d->k, sp.rows, sp.nsplit, sp.chunk,
                  (float)(1.0 / sqrt((double)d->d))};
  if (trace_on())
    fprintf(stderr, "[gqe] decode B=%d L=%d Smax=%d G=%d k=%d d=%d nsplit=%d chunk=%d\n", d->B,
            q_len, d->S, d->G, d->k, d->d, sp.nsplit, sp.chunk);
  return hip_status(launch_decode(dp, d->d, d->dtype == GQE_BF16, (hipStream_t)stream));
}

int gqe_attn_decode(const gqe_dims* d, int32_t q_len, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* kv_len, const int32_t* topk_idx,
                    void* o_routed, void* o_shared, void* workspace, size_t ws_bytes,
                    void* stream) {
  bool empty = false;
  int st = decode_check(d, q_len, q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared, &empty);
  if (st || empty) return st;
  const size_t need = gqe_decode_workspace_bytes(d, q_len);
  if (!workspace || ws_bytes < need) return GQE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GQE_ERR_ALIGNMENT;
  return decode_launch(d, q_len, q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared, workspace,
                       stream);
}

size_t gqe_decode_scratch_bytes(void) { return kDecodeScratchBytes; }

int gqe_attn_decode_noalloc(const gqe_dims* d, int32_t q_len, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* kv_len, const int32_t* topk_idx,
                            void* o_routed, void* o_shared, void* stream) {
  bool empty = false;
  int st = decode_check(d, q_len, q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared, &empty);
  if (st || empty) return st;
  if (gqe_decode_workspace_bytes(d, q_len) > kDecodeScratchBytes) return GQE_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st) return st;
  // nothing in the scratch needs clearing: the split pass writes every
  // partial that the combine pass reads
  return decode_launch(d, q_len, q, k_cache, v_cache, kv_len, topk_idx, o_routed, o_shared, ws, stream);
}

int gqe_attn_decode_paged(const gqe_dims* d, int32_t q_len, const void* q, const void* k_pages,
                          const void* v_pages, const int32_t* block_table, int32_t page_size,
                          const int32_t* kv_start, const int32_t* kv_len, const int32_t* topk_idx,
                          void* o_routed, void* o_shared, void* workspace, size_t ws_bytes,
                          void* stream) {
  int st = check_dims(d, false);
  if (st) return st;
  if (q_len < 0) return GQE_ERR_INVALID_ARG;
  if (!q || !k_pages || !v_pages || !block_table || !kv_len || !topk_idx || !o_routed || !o_shared)
    return GQE_ERR_INVALID_ARG;
  if (page_size < 64 || (page_size & (page_size - 1)) != 0) return GQE_ERR_UNSUPPORTED;
  if (d->S % page_size != 0) return GQE_ERR_INVALID_ARG;
  if (q_len > d->S && d->B > 0) return GQE_ERR_INVALID_ARG;
  if ((int64_t)(d->k + 1) * q_len > kMaxDecodeRows) return GQE_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k_pages, v_pages, block_table, kv_len, topk_idx, o_routed, o_shared};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQE_ERR_ALIGNMENT;
  if (kv_start && !aligned16(kv_start)) return GQE_ERR_ALIGNMENT;
  if (d->B == 0 || q_len == 0) return GQE_OK;
  const size_t need = gqe_decode_workspace_bytes(d, q_len);
  if (!workspace || ws_bytes < need) return GQE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GQE_ERR_ALIGNMENT;
  const DecodeSplit sp = decode_split(d->B, d->G, d->S, d->k, q_len);
  const size_t recs = (size_t)d->B * d->G * sp.nsplit * sp.rows;
  float* ws_o = (float*)workspace;
  float* ws_ml = ws_o + recs * d->d;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  DecodeParams dp{q, k_pages, v_pages, kv_len, topk_idx, o_routed, o_shared, ws_o, ws_ml,
                  d->B, q_len, d->S, d->N, d->G, d->N / d->G, d->k, sp.rows, sp.nsplit, sp.chunk,
                  (float)(1.0 / sqrt((double)d->d)), block_table, shift, d->S / page_size, kv_start};
  if (trace_on())
    fprintf(stderr, "[gqe] decode_paged B=%d L=%d Smax=%d page=%d G=%d k=%d d=%d nsplit=%d\n", d->B,
            q_len, d->S, page_size, d->G, d->k, d->d, sp.nsplit);
  return hip_status(launch_decode(dp, d->d, d->dtype == GQE_BF16, (hipStream_t)stream));
}

static int out_proj_mode(const gqe_dims* d, int32_t mode, int64_t T, const void* o_routed,
                         const float* topk_w, const void* o_shared, const void* w_o, void* y,
                         void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (T < 0) return GQE_ERR_INVALID_ARG;
  if (mode != GQE_SLOTS_FULL && mode != GQE_SLOTS_HARD && mode != GQE_SLOTS_WEIGHTED)
    return GQE_ERR_UNSUPPORTED;
  // the ablation layouts read no shared output, the hard one no weights
  const bool full = mode == GQE_SLOTS_FULL;
  if (!o_routed || (!topk_w && mode != GQE_SLOTS_HARD) || (!o_shared && full) || !w_o || !y)
    return GQE_ERR_INVALID_ARG;
  const void* ptrs[] = {o_routed, topk_w, o_shared, w_o, y};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GQE_ERR_ALIGNMENT;
  if ((T + 127) / 128 > (int64_t)UINT32_MAX) return GQE_ERR_UNSUPPORTED;
  // a 256-token output tile is stored through a raw buffer of 256*D*2 bytes
  if (d->D >= (1 << 23)) return GQE_ERR_UNSUPPORTED;
  if (T == 0) return GQE_OK;
  OutProjParams op{o_routed, topk_w, o_shared, w_o, y, T, d->G * d->k, d->d, d->D};
  op.nob = full ? d->d : 0;
  op.nsh = full ? d->d : 0;
  op.weighted = mode == GQE_SLOTS_WEIGHTED ? 1 : 0;
  if (trace_on())
    fprintf(stderr, "[gqe] out_proj mode=%d T=%lld K=%d D=%d\n", mode, (long long)T,
            d->G * d->k * d->d + op.nob + op.nsh, d->D);
  return hip_status(launch_out_proj(op, d->dtype == GQE_BF16, (hipStream_t)stream));
}

int gqe_out_proj(const gqe_dims* d, int64_t T, const void* o_routed, const float* topk_w,
                 const void* o_shared, const void* w_o, void* y, void* stream) {
  return out_proj_mode(d, GQE_SLOTS_FULL, T, o_routed, topk_w, o_shared, w_o, y, stream);
}

int gqe_out_proj_variant(const gqe_dims* d, int32_t mode, int64_t T, const void* o_routed,
                         const float* topk_w, const void* o_shared, const void* w_o, void* y,
                         void* stream) {
  return out_proj_mode(d, mode, T, o_routed, topk_w, o_shared, w_o, y, stream);
}

int gqe_qkv_proj(const gqe_dims* d, const void* x, const void* w_q, const void* w_k,
                 const void* w_v, const int32_t* topk_idx, void* q, void* k, void* v,
                 void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (!x || !w_q || !w_k || !w_v || !topk_idx || !q || !k || !v) return GQE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w_q, w_k, w_v, topk_idx, q, k, v};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQE_ERR_ALIGNMENT;
  if (d->dtype == GQE_BF16 && d->D % 64 != 0) return GQE_ERR_UNSUPPORTED;
  if ((int64_t)d->S * d->k > (int64_t)INT32_MAX / 2) return GQE_ERR_UNSUPPORTED;
  if (d->B == 0 || d->S == 0) return GQE_OK;
  ProjParams pp{x, w_q, w_k, w_v, topk_idx, nullptr, q, k, v,
                d->B * d->S, d->B, d->S, d->D, d->N, d->G, d->N / d->G, d->k, d->d, d->S};
  if (trace_on())
    fprintf(stderr, "[gqe] qkv_proj B=%d S=%d D=%d N=%d G=%d k=%d d=%d\n", d->B, d->S, d->D, d->N,
            d->G, d->k, d->d);
  return hip_status(launch_proj(pp, d->dtype == GQE_BF16, (hipStream_t)stream));
}

int gqe_qkv_proj_decode(const gqe_dims* d, int32_t q_len, const void* x, const void* w_q,
                        const void* w_k, const void* w_v, const int32_t* topk_idx,
                        const int32_t* kv_len, void* q, void* k_cache, void* v_cache,
                        void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (q_len < 0) return GQE_ERR_INVALID_ARG;
  if (!x || !w_q || !w_k || !w_v || !topk_idx || !kv_len || !q || !k_cache || !v_cache)
    return GQE_ERR_INVALID_ARG;
  if (q_len > d->S && d->B > 0) return GQE_ERR_INVALID_ARG;  // kv_len <= S_max cannot hold
  const void* ptrs[] = {x, w_q, w_k, w_v, topk_idx, kv_len, q, k_cache, v_cache};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQE_ERR_ALIGNMENT;
  if (d->dtype == GQE_BF16 && d->D % 64 != 0) return GQE_ERR_UNSUPPORTED;
  if ((int64_t)d->B * q_len > (int64_t)INT32_MAX / 2) return GQE_ERR_UNSUPPORTED;
  if (d->B == 0 || q_len == 0) return GQE_OK;
  ProjParams pp{x, w_q, w_k, w_v, topk_idx, kv_len, q, k_cache, v_cache,
                d->B * q_len, d->B, q_len, d->D, d->N, d->G, d->N / d->G, d->k, d->d, d->S};
  if (trace_on())
    fprintf(stderr, "[gqe] qkv_proj_decode B=%d L=%d Smax=%d D=%d N=%d G=%d k=%d d=%d\n", d->B,
            q_len, d->S, d->D, d->N, d->G, d->k, d->d);
  return hip_status(launch_proj(pp, d->dtype == GQE_BF16, (hipStream_t)stream));
}


size_t gqe_out_proj_bwd_workspace_bytes(const gqe_dims* d, int32_t mode, int64_t T) {
  if (check_dims(d) != GQE_OK || T < 0 || T > (int64_t)INT32_MAX) return 0;
  if (mode != GQE_SLOTS_FULL && mode != GQE_SLOTS_HARD && mode != GQE_SLOTS_WEIGHTED) return 0;
  return out_proj_bwd_layout(d, mode, T).total;
}

int gqe_out_proj_bwd(const gqe_dims* d, int32_t mode, int64_t T, const void* o_routed,
                     const float* topk_w, const void* o_shared, const void* w_o, const void* dy,
                     void* do_routed, float* dw, void* do_shared, float* dw_o, void* workspace,
                     size_t ws_bytes, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (T < 0) return GQE_ERR_INVALID_ARG;
  if (mode != GQE_SLOTS_FULL && mode != GQE_SLOTS_HARD && mode != GQE_SLOTS_WEIGHTED)
    return GQE_ERR_UNSUPPORTED;
  const bool full = mode == GQE_SLOTS_FULL;
  if (!o_routed || (!topk_w && mode != GQE_SLOTS_HARD) || (!o_shared && full) || !w_o || !dy ||
      !do_routed || !dw || (!do_shared && full) || !dw_o)
    return GQE_ERR_INVALID_ARG;
  const void* ptrs[] = {o_routed, topk_w, o_shared, w_o, dy, do_routed, dw, do_shared, dw_o};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GQE_ERR_ALIGNMENT;
  if (T > (int64_t)INT32_MAX) return GQE_ERR_UNSUPPORTED;
  if (T == 0) return GQE_OK;
  const OutProjBwdLayout L = out_proj_bwd_layout(d, mode, T);
  if (!workspace || ws_bytes < L.total) return GQE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GQE_ERR_ALIGNMENT;
  char* ws = (char*)workspace;
  OutProjBwdParams bp{};
  bp.o_r = o_routed;
  bp.w = topk_w;
  bp.o_s = o_shared;
  bp.w_o = w_o;
  bp.dy = dy;
  bp.do_r = do_routed;
  bp.dw = dw;
  bp.do_s = do_shared;
  bp.dw_o = dw_o;
  bp.da = (float*)(ws + L.da);
  bp.a = ws + L.a;
  bp.part = (float*)(ws + L.part);
  bp.T = T;
  bp.Gk = d->G * d->k;
  bp.d = d->d;
  bp.Dout = d->D;
  bp.Kd = L.Kd;
  bp.nob = full ? d->d : 0;
  bp.nsh = full ? d->d : 0;
  bp.weighted = mode == GQE_SLOTS_WEIGHTED ? 1 : 0;
  bp.nsplit = L.nsplit;
  bp.kchunk = L.kchunk;
  if (trace_on())
    fprintf(stderr, "[gqe] out_proj_bwd mode=%d T=%lld Kd=%d D=%d nsplit=%d\n", mode, (long long)T,
            L.Kd, d->D, L.nsplit);
  return hip_status(launch_out_proj_bwd(bp, d->dtype == GQE_BF16, (hipStream_t)stream));
}

size_t gqe_route_bwd_workspace_bytes(const gqe_dims* d) {
  if (check_dims(d) != GQE_OK) return 0;
  return route_bwd_layout(d).total;
}

int gqe_route_bwd(const gqe_dims* d, const void* x, const void* w_router, const float* logits,
                  const int32_t* topk_idx, const float* dw, int32_t weights, float aux_coef,
                  float* dz_or_null, void* dx, float* dw_router, float* db_router,
                  float* aux_loss_or_null, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (!x || !w_router || !logits || !topk_idx || !dw || !dx || !dw_router || !db_router)
    return GQE_ERR_INVALID_ARG;
  if (weights != GQE_WEIGHTS_RENORM && weights != GQE_WEIGHTS_PROB) return GQE_ERR_UNSUPPORTED;
  if (!(aux_coef >= 0.f) || aux_coef > 1e30f) return GQE_ERR_INVALID_ARG;  // rejects NaN too
  const void* ptrs[] = {x, w_router, logits, topk_idx, dw, dz_or_null, dx, dw_router, db_router,
                        aux_loss_or_null};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GQE_ERR_ALIGNMENT;
  const int64_t T = (int64_t)d->B * d->S;
  if (T == 0) return GQE_OK;
  const RouteBwdLayout L = route_bwd_layout(d);
  if (!workspace || ws_bytes < L.total) return GQE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GQE_ERR_ALIGNMENT;
  char* ws = (char*)workspace;
  RouteBwdParams rp{};
  rp.x = x;
  rp.w = w_router;
  rp.z = logits;
  rp.topk = topk_idx;
  rp.dw = dw;
  rp.dz = dz_or_null ? dz_or_null : (float*)(ws + L.dz);
  rp.dzb = ws + L.dzb;
  rp.pbuf = aux_loss_or_null ? (float*)(ws + L.pbuf) : nullptr;
  rp.counts = (int32_t*)(ws + L.counts);
  rp.colpart = (float*)(ws + L.colpart);
  rp.dx = dx;
  rp.dw_r = dw_router;
  rp.db_r = db_router;
  rp.aux_loss = aux_loss_or_null;
  rp.part = (float*)(ws + L.part);
  rp.aux_coef = aux_coef;
  rp.wprob = weights == GQE_WEIGHTS_PROB ? 1 : 0;
  rp.T = T;
  rp.D = d->D;
  rp.G = d->G;
  rp.M = d->N / d->G;
  rp.K = d->k;
  rp.GMp = L.GMp;
  rp.nchunk = L.nchunk;
  rp.nsplit = L.nsplit;
  rp.kchunk = L.kchunk;
  if (trace_on())
    fprintf(stderr, "[gqe] route_bwd T=%lld D=%d G=%d M=%d k=%d aux=%g nsplit=%d\n", (long long)T,
            d->D, d->G, rp.M, d->k, (double)aux_coef, L.nsplit);
  return hip_status(launch_route_bwd(rp, d->dtype == GQE_BF16, (hipStream_t)stream));
}

}  // extern "C"
