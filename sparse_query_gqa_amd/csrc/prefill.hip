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
// owns a tile of 256 consecutive rows, so every tile holds exactly k rows per
// token whatever the routing skew, and all of them read the same KV head:
// each K/V block is staged once in LDS and used by every selected head of the
// group.
//
// bf16 path. Per 64-key block a wavefront computes S^T = K Q^T and
// O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, so that every lane owns one
// query row in both products (row max, row sum and rescale are per-lane
// scalars; the two lane halves are combined with one exchange). Q is taken
// pre-scaled by scale*log2(e) and the row's reference max enters as the S^T
// MFMA's initial accumulator, so the scores come out of the MFMA as exp2
// arguments. The online softmax (fp32, exp2) moves the reference lazily: 2^64
// of headroom, checked through the row sums, so most blocks need no max at
// all. The causal mask only runs on the tile's diagonal blocks. Two kernels:
// 64 rows per wavefront for d <= 64 and 32 rows per wavefront for d = 128,
// both software-pipelined so that MFMAs and the softmax of neighbouring
// 32x32 score tiles overlap.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "prefill_tiles.h"

namespace gqe {

// The reference max used for the exponentials is only moved when a row's
// partial sum in a block reaches this value (no element can then exceed it),
// which keeps the fp32 accumulators far from overflow while most key blocks
// skip both the block max and the rescale of the output accumulators.
constexpr float kSumLimit = 18446744073709551616.0f;  // 2^64

// Quarter-pipelined form (d <= 64). A wavefront owns 64 query rows (two
// 32-row halves h) and each 64-key block splits into two 32-key halves sb,
// so a block is four 32x32 quarters, taken in the order (sb, h) = (0,0),
// (0,1), (1,0), (1,1). Quarter t goes through S^T (KS MFMAs), softmax (VALU)
// and P V (2*DB MFMAs). The steps are software-pipelined across quarters and
// key blocks: step t issues the S^T MFMAs of quarter t+1, the softmax of
// quarter t and the P V MFMAs of quarter t-1, so every MFMA has a share of
// the exponentials beside it. The S^T MFMAs go first, so that the scores the
// next step exponentiates are complete long before it starts; nothing reads
// the P V results until the step after. Consecutive quarters belong to different row
// halves, so a softmax that moves its half's reference only has to rescale
// an accumulator whose P V products are all issued.
//
// K/V blocks go from HBM straight into LDS (global_load_lds_dwordx4, no
// staging registers), row-major with the 16-byte chunks of each row
// XOR-swizzled so that neither read pattern has bank conflicts. K fragments
// are plain 16-byte reads; V^T fragments come from
// ds_read_b64_tr_b16, which hands each lane one d column of four keys. Blocks
// rotate through four buffers: block j+3 is loaded while blocks j+2 and j+1
// are in flight and block j is read, with one barrier per block.
//
// Key-split form (SPLIT, launches with fewer tiles than two per CU). There
// the kernel is bound by the longest tile, not by the total work. Eight
// wavefronts take one tile: group
// 0 (wavefronts 0..3) runs the first half of its key blocks, group 1 the
// second half, each through its own LDS ring and with the same rows. Both
// groups pass the same number of barriers (group 1's blocks past the last
// are fully masked). At the end group 1 leaves its unnormalised O, reference
// and row sums in LDS and group 0 merges them into its own and stores the
// rows. A row that sees no key of group 1's range takes group 0's result
// alone.
template <int D, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 512 : 256, SPLIT ? 1 : 2) void prefill_qp_kernel(PrefillParams p, int tiles_r,
                                                                                       int tiles_s) {
  static_assert(D == 32 || D == 64, "head dim");
  constexpr int NGRP = SPLIT ? 2 : 1;  // key-range groups of four wavefronts
  constexpr int kTileRows = 256;
  constexpr int KS = D / 16;   // MFMA k-steps over d
  constexpr int DB = D / 32;   // 32-wide d blocks of O^T
  constexpr int CPR = D / 8;   // 16-byte chunks per key row
  constexpr int ROWB = 2 * D;  // bytes per key row
  constexpr int MATB = kKeyBlock * ROWB;  // bytes of one K or V block
  constexpr int NPW = MATB / 1024 / 4;    // 1 KiB LDS-DMA chunks per wavefront per matrix
  static_assert(NPW >= 1, "block too small for the LDS-DMA split");
  constexpr int NBUF = 4;
  __shared__ __attribute__((aligned(1024))) char lds_all[NGRP][NBUF][2][MATB];  // [group][buffer][K, V]

  const TileCoord tc = tile_of_block(p, tiles_r, tiles_s);
  if (!tc.valid) return;
  const int b = tc.b, v = tc.v;
  const int kvh = (v == p.G) ? 0 : v;
  const int nrows = (v == p.G) ? p.S : p.S * p.K;
  const int r0 = tc.tile * kTileRows;
  const int tid = threadIdx.x, lane = tid & 63, wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = SPLIT ? (wave_id >> 2) : 0;
  const int wave = SPLIT ? (wave_id & 3) : wave_id;  // wavefront within its group: rows and DMA share
  auto& lds = lds_all[grp];
  const int half = lane >> 5, l32 = lane & 31;
  const int last_r = min(r0 + kTileRows, nrows) - 1;
  int pos_last, pos_first, s_, h_;
  row_info(p, b, v, last_r, pos_last, s_, h_);
  row_info(p, b, v, r0, pos_first, s_, h_);

  // Q^T fragments (B operand of S^T = K Q^T), pre-scaled by scale*log2(e) and
  // rounded to bf16, so that S^T comes out in log2 units.
  const float c = p.scale * 1.44269504088896340736f;
  int pos[2], slot[2];
  bool row_ok[2];
  bf16x8 qf[2][KS];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + wave * 64 + h * 32 + l32;
    row_ok[h] = r < nrows;
    int head;
    row_info(p, b, v, row_ok[h] ? r : last_r, pos[h], slot[h], head);
    const __bf16* qrow = (const __bf16*)p.q + (((int64_t)b * p.S + pos[h]) * (p.N + 1) + head) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[h][s] = *(const bf16x8*)(qrow + 16 * s + 8 * half);
#pragma unroll
      for (int t = 0; t < 8; ++t) qf[h][s][t] = f2bf((float)qf[h][s][t] * c);
    }
  }
  const __bf16* kbase = (const __bf16*)p.k + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;
  const __bf16* vbase = (const __bf16*)p.v + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;

  f32x16 oacc[2][DB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[h][i][j] = 0.f;
  // per row: running sum of P and the reference (log2 units) the scores are taken against
  float l_run[2] = {0.f, 0.f}, mr[2] = {0.f, 0.f};
  // -mr of each half as a 16-register MFMA accumulator, kept for its S^T
  // MFMAs; the moves are asm so that the compiler keeps the tuples instead of
  // re-creating them (16 moves) before every S^T product. They change only
  // when the reference moves.
  f32x16 bias[2] = {};
  auto set_bias = [&](const int h) __attribute__((always_inline)) {
    const float nm = -mr[h];
#pragma unroll
    for (int j = 0; j < 16; ++j) __asm__("v_mov_b32 %0, %1" : "+v"(bias[h][j]) : "v"(nm));
  };
  const int nblocks = pos_last / kKeyBlock + 1;

  // Layout of a block in LDS: key row r at r*ROWB, its 16-byte chunk c at
  // chunk position c ^ swz(r). With 64 four-byte banks two 128-byte rows
  // share a bank cycle, so swz takes row bits 1..3: the 16 rows of a 16-byte
  // K read land on distinct (row parity, chunk) pairs, and the 8 rows x 64
  // bytes of a transposing V read fill each bank exactly twice (bit 1 of the
  // row flips the 64-byte half). Row offsets that are multiples of 16 leave
  // swz unchanged, so they fold into instruction offsets.
  //
  // Block kb of K and V into buffer bf: lane l of 1 KiB chunk n writes LDS
  // bytes [1024 n + 16 l, +16), i.e. row 1024 n / ROWB + (16 l) / ROWB,
  // chunk position (16 l % ROWB) / 16; it loads the source chunk the swizzle
  // puts there. That lane offset is the same in every block, so a whole block
  // moves with the scalar words of a raw buffer resource that starts at the
  // block and ends at the head's last key: rows of a block that runs past the
  // sequence read zeros (and are masked).
  auto swz = [](int r) { return (((r >> 1) & 7) ^ ((r & 2) << 1)) & (CPR - 1); };
  constexpr int RPC = 1024 / ROWB;  // key rows per 1 KiB chunk
  const int dma_r = (16 * lane) / ROWB;
  const int dma_p = ((16 * lane) % ROWB) / 16;  // chunk position
  uint32_t dma_off[NPW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int rb = (wave * NPW + i) * RPC + dma_r;  // row in the block
    dma_off[i] = rb * ROWB + 16 * (dma_p ^ swz(rb));
  }
  // Block kb through raw buffers over the rest of this head's keys: rows past
  // the sequence read zeros (and are masked).
  const uint32_t head_bytes = (uint32_t)p.S * ROWB;
  auto dma = [&](const int kb, const int bf) __attribute__((always_inline)) {
    const uint32_t skip = (uint32_t)kb * MATB;
    const uint32_t rem = head_bytes > skip ? head_bytes - skip : 0u;
    const i32x4 rk = buf_rsrc((const char*)kbase + skip, rem);
    const i32x4 rv = buf_rsrc((const char*)vbase + skip, rem);
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int n = wave * NPW + i;
      lds_dma16_b(rk, dma_off[i], lds[bf][0] + n * 1024);
      lds_dma16_b(rv, dma_off[i], lds[bf][1] + n * 1024);
    }
  };

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16 sh[4];        // S^T per quarter (log2 units, relative to mr of its half)
  u32x4 ph[4][2];      // bf16 P^T fragments per quarter, one per 16-key step
  float ls[4];         // row sums of the bf16 P per quarter
  bf16x8 kf[2][KS];    // K fragments by key half
  bf16x8 vf[2][2][DB]; // V^T fragments by key half, 16-key step and d block

  // K fragment s of key half sb: row sb*32 + l32, chunk 2s + half
  int k_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = l32 * ROWB + 16 * ((2 * s + half) ^ swz(l32));
  auto read_k = [&](const int buf, const int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[sb][s] = *(const bf16x8*)(lds[buf][0] + sb * 32 * ROWB + k_off[s]);
  };
  // V^T fragment for key half sb, step st, d block db: lane (half, l32) holds
  // d = db*32 + l32 and contraction element t <-> key sb*32 + 16*st + 8*(t/4) +
  // 4*half + t%4, the S^T output layout. In a 16-lane group of the transposing
  // read, source lane i points at key K0 + i/4, d D0 + 4*(i%4), and output
  // lane i receives keys K0..K0+3 of d D0 + i.
  const int tr_key = 4 * half + ((lane & 15) >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int v_off[2][DB];  // by the 8-key step tt (it changes row bit 3) and d block
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_off[tt][db] = (8 * tt + tr_key) * ROWB + 16 * ((4 * db + (tr_d >> 3)) ^ swz(8 * tt + tr_key)) + 2 * (tr_d & 7);
  auto read_v = [&](const int buf, const int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x4 vw;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const char* a = lds[buf][1] + (sb * 32 + 16 * st) * ROWB + v_off[tt][db];
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a);
          const u32x2 w = __builtin_bit_cast(u32x2, x);
          vw[2 * tt] = w[0];
          vw[2 * tt + 1] = w[1];
        }
        vf[sb][st][db] = __builtin_bit_cast(bf16x8, vw);
      }
  };
  // S^T of quarter q: the accumulator starts at -mr of the quarter's half
  // (0 for the first block, which sets the reference).
  auto s_mfma = [&](const int q, auto first_tag) __attribute__((always_inline)) {
    const int sb = q >> 1, h = q & 1;
    const f32x16 zero16 = {};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sh[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          kf[sb][s], qf[h][s], s == 0 ? (decltype(first_tag)::value ? zero16 : bias[h]) : sh[q],
          0, 0, 0);
  };
  auto pv_mfma = [&](const int q) __attribute__((always_inline)) {
    const int sb = q >> 1, h = q & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[sb][st][db], __builtin_bit_cast(bf16x8, ph[q][st]),
                                                              oacc[h][db], 0, 0, 0);
  };
  auto exps = [&](const int q) __attribute__((always_inline)) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const bf16x2 pr = {f2bf(__builtin_amdgcn_exp2f(sh[q][j])), f2bf(__builtin_amdgcn_exp2f(sh[q][j + 1]))};
      ph[q][j >> 3][(j & 7) >> 1] = __builtin_bit_cast(uint32_t, pr);
      acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);  // row sum of the bf16 P used in P V
    }
    ls[q] = acc;
  };
  // Exact path: move the half's reference up to this quarter's max (the first
  // block sets it), rescale O and l of that half, recompute P.
  auto exact = [&](const int q, auto first_tag) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    const int h = q & 1;
    float bmax = sh[q][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) bmax = fmaxf(bmax, sh[q][j]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    // key 0 is visible to every row, so bmax is finite in the first block of
    // the whole range; in the key-split form a row may see nothing of group
    // 1's first block (its result is then not used), and the reference stays 0
    const float delta = FIRST ? (bmax == -INFINITY ? 0.f : bmax) : fmaxf(bmax, 0.f);
    mr[h] += delta;
    set_bias(h);
    if constexpr (!FIRST) {
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      l_run[h] *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[h][i][j] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) sh[q][j] -= delta;
    exps(q);
  };
  // Causal mask of quarter q of block kb, only on the tile's diagonal blocks
  // (a uniform branch kept out of the interleaved region).
  auto mask = [&](const int q, const int kb, const bool on) __attribute__((always_inline)) {
    if (on) {
      __asm__ volatile("" ::: "memory");  // keep this a real branch
      // key kb*64 + sb*32 + 8*(j/4) + 4*half + j%4 is visible iff key <= pos
      const int lim = pos[q & 1] - kb * kKeyBlock - (q >> 1) * 32 - 4 * half;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + (j & 3) > lim) sh[q][j] = -INFINITY;
    }
  };
  auto softmax = [&](const int q, auto first_tag) __attribute__((always_inline)) {
    if constexpr (decltype(first_tag)::value) exact(q, first_tag);
    else exps(q);
  };
  // Overflow check of a lazy softmax, then the half's row sum. Ends the step.
  auto settle = [&](const int q, auto first_tag) __attribute__((always_inline)) {
    if constexpr (!decltype(first_tag)::value) {
      if (__builtin_amdgcn_ballot_w64(ls[q] > kSumLimit) != 0) {
        __asm__ volatile("" ::: "memory");  // keep this a real branch
        exact(q, first_tag);
      }
    }
    l_run[q & 1] += ls[q];
  };
  // MFMA / VALU interleave of one step's region: the LDS reads for the next
  // step spread two per MFMA, and up to five VALU ops beside each MFMA (a
  // step has 34 to 42 of them for its 8 MFMAs; four per MFMA left the rest
  // after the last MFMA and was about 1% slower at 128k tokens).
  auto interleave = [&](auto n_mfma) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < decltype(n_mfma)::value; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
  };
  using kNo = std::integral_constant<bool, false>;
  using kYes = std::integral_constant<bool, true>;
  using kNS = std::integral_constant<int, KS>;
  using kNSPV = std::integral_constant<int, KS + 2 * DB>;

  // One key block j (in LDS buffer buf; its quarter 0 S^T is already in sh[0]
  // and its K fragments of key half 0 in kf[0]). Fragments are read one step
  // before their first use, into registers whose previous contents died a
  // step earlier.
  auto iteration = [&](const int j, const int buf, const int nbuf, const bool masked, auto first_tag,
                       auto prev_tag) __attribute__((always_inline)) {
    // step 0: P V(q3 of block j-1) | S^T(q1) | softmax(q0)
    mask(0, j, masked);
    read_k(buf, 1);
    read_v(buf, 0);
    s_mfma(1, first_tag);
    if constexpr (decltype(prev_tag)::value) pv_mfma(3);
    softmax(0, first_tag);
    if constexpr (decltype(prev_tag)::value) interleave(kNSPV());
    else interleave(kNS());
    settle(0, first_tag);
    // step 1: P V(q0) | S^T(q2) | softmax(q1)
    mask(1, j, masked);
    s_mfma(2, kNo());
    pv_mfma(0);
    softmax(1, first_tag);
    interleave(kNSPV());
    settle(1, first_tag);
    // step 2: P V(q1) | S^T(q3) | softmax(q2)
    mask(2, j, masked);
    read_v(buf, 1);
    s_mfma(3, kNo());
    pv_mfma(1);
    softmax(2, kNo());
    interleave(kNSPV());
    settle(2, kNo());
    // block j+1 (loaded two blocks ago) is complete and visible after the
    // wait, which leaves block j+2's loads in flight, and the barrier; block
    // j+3 then goes into the buffer of block j-1, whose last reads were
    // issued in its step 2. Every block issues the same loads (past the last
    // block it re-loads that one), so the wait count is fixed.
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NPW) : "memory");
    __syncthreads();
    dma(min(j + 3, nblocks - 1), (buf + 3) % NBUF);
    read_k(nbuf, 0);  // past the last block this reads a stale buffer; the result is unused
    // step 3: P V(q2) | S^T(q0 of block j+1) | softmax(q3)
    mask(3, j, masked);
    s_mfma(0, kNo());
    pv_mfma(2);
    softmax(3, kNo());
    interleave(kNSPV());
    settle(3, kNo());
  };

  // This group's key blocks: all of them, or in the key-split form the
  // group's half, [j0, j0 + nit) (blocks past the last re-load the last one
  // and are fully masked).
  const int nhalf = (nblocks + 1) / 2;
  const int j0 = SPLIT ? grp * nhalf : 0;
  const int nit = SPLIT ? nhalf : nblocks;
  dma(min(j0, nblocks - 1), 0);
  dma(min(j0 + 1, nblocks - 1), 1);
  dma(min(j0 + 2, nblocks - 1), 2);
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * NPW) : "memory");
  __syncthreads();
  read_k(0, 0);
  s_mfma(0, kYes());
  // Blocks at or below the tile's first position need no mask. The first
  // block sets the references. Block j0 + i sits in buffer i % 4.
  const int nfull = min((pos_first + 1) / kKeyBlock, nblocks);
  iteration(j0, 0, 1, j0 >= nfull, kYes(), kNo());
  for (int i = 1, buf = 1; i < nit; ++i) {
    const int nbuf = (buf + 1) % NBUF;
    iteration(j0 + i, buf, nbuf, j0 + i >= nfull, kNo(), kYes());
    buf = nbuf;
  }
  pv_mfma(3);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA may outlive the workgroup

  if constexpr (SPLIT) {
    // Merge group 1's partial rows into group 0's, lane by lane (the lanes
    // of wavefronts w and w+4 hold the same rows and key columns).
    constexpr int NO = 4 * 2 * DB * 16 * 64;  // O partials: [wave][h][db][j][lane]
    static_assert((NO + 2 * 4 * 2 * 64) * 4 <= (int)sizeof(lds_all), "merge space");
    float* xo = (float*)&lds_all[0][0][0][0];
    float* xm = xo + NO;             // references [wave][h][lane]
    float* xl = xm + 4 * 2 * 64;     // row sums
    __syncthreads();  // both rings are free
    if (grp == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) xo[(((wave * 2 + h) * DB + db) * 16 + j) * 64 + lane] = oacc[h][db][j];
        xm[(wave * 2 + h) * 64 + lane] = mr[h];
        xl[(wave * 2 + h) * 64 + lane] = l_run[h];
      }
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (pos[h] < nhalf * kKeyBlock) continue;  // the row sees no key of group 1's range
      const float m1 = xm[(wave * 2 + h) * 64 + lane];
      const float mm = fmaxf(mr[h], m1);
      const float a0 = __builtin_amdgcn_exp2f(mr[h] - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          oacc[h][db][j] = oacc[h][db][j] * a0 + xo[(((wave * 2 + h) * DB + db) * 16 + j) * 64 + lane] * a1;
      l_run[h] = l_run[h] * a0 + xl[(wave * 2 + h) * 64 + lane] * a1;
      mr[h] = mm;
    }
  }

#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float l_tot = l_run[h] + __shfl_xor(l_run[h], 32, 64);
    if (!row_ok[h]) continue;
    const float inv = 1.f / l_tot;
    if (p.lse_r && half == 0) {  // ln of the normaliser: (reference + log2 l) * ln 2
      const float lse = (mr[h] + __log2f(l_tot)) * 0.69314718055994531f;
      if (v == p.G) p.lse_s[(int64_t)b * p.S + pos[h]] = lse;
      else p.lse_r[(((int64_t)b * p.S + pos[h]) * p.G + v) * p.K + slot[h]] = lse;
    }
    __bf16* out = (v == p.G)
                      ? (__bf16*)p.o_s + ((int64_t)b * p.S + pos[h]) * D
                      : (__bf16*)p.o_r + ((((int64_t)b * p.S + pos[h]) * p.G + v) * p.K + slot[h]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = f2bf(oacc[h][db][4 * jq + i] * inv);
        *(bf16x4*)(out + db * 32 + 8 * jq + 4 * half) = o4;
      }
  }
}

// Head dim 128. A wavefront owns 32 query rows and a workgroup of 8
// wavefronts owns a 256-row tile. Each 64-key block is two 32-key halves;
// half t (block t/2, key half t%2) goes through S^T (8 MFMAs), softmax and
// P V (8 MFMAs), pipelined as in the quarter form: step t issues the P V
// MFMAs of half t-1, the S^T MFMAs of half t+1 and the softmax of half t.
// Consecutive halves belong to the same rows, so a reference move in step t
// also shifts the S^T of half t+1, which that step already computed.
//
// K/V go through LDS-DMA into four 16 KiB K buffers followed by four 16 KiB
// V buffers (one workgroup per CU). Rows are 256 bytes, so every row covers
// all 64 banks; the chunk swizzle swaps the two 2-bit fields of the row's low
// 4 bits, which makes a 16-byte K read over 16 rows and a transposing V read
// over 8 rows x 64 bytes both conflict-free. The block loop is unrolled over
// the four buffers, so that every fragment read is a per-lane register plus
// an immediate offset (no address arithmetic in the loop).
template <int D>
__global__ __launch_bounds__(512, 1) void prefill_d128_kernel(PrefillParams p, int tiles_r, int tiles_s) {
  static_assert(D == 128, "head dim");
  constexpr int kWaves8 = 8;
  constexpr int kTileRows = 32 * kWaves8;
  constexpr int KS = D / 16;   // MFMA k-steps over d
  constexpr int DB = D / 32;   // 32-wide d blocks of O^T
  constexpr int ROWB = 2 * D;  // bytes per key row
  constexpr int MATB = kKeyBlock * ROWB;        // bytes of one K or V block
  constexpr int NPW = MATB / 1024 / kWaves8;    // 1 KiB LDS-DMA chunks per wavefront per matrix
  static_assert(NPW >= 1, "block too small for the LDS-DMA split");
  constexpr int NBUF = 4;
  __shared__ __attribute__((aligned(1024))) char lds[2][NBUF][MATB];  // [K, V][buffer]

  const TileCoord tc = tile_of_block(p, tiles_r, tiles_s);
  if (!tc.valid) return;
  const int b = tc.b, v = tc.v;
  const int kvh = (v == p.G) ? 0 : v;
  const int nrows = (v == p.G) ? p.S : p.S * p.K;
  const int r0 = tc.tile * kTileRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int last_r = min(r0 + kTileRows, nrows) - 1;
  int pos_last, pos_first, s_, h_;
  row_info(p, b, v, last_r, pos_last, s_, h_);
  row_info(p, b, v, r0, pos_first, s_, h_);

  // Q^T fragments, pre-scaled by scale*log2(e) and rounded to bf16
  const float c = p.scale * 1.44269504088896340736f;
  int pos, slot, head;
  const int r = r0 + wave * 32 + l32;
  const bool row_ok = r < nrows;
  row_info(p, b, v, row_ok ? r : last_r, pos, slot, head);
  bf16x8 qf[KS];
  {
    const __bf16* qrow = (const __bf16*)p.q + (((int64_t)b * p.S + pos) * (p.N + 1) + head) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = *(const bf16x8*)(qrow + 16 * s + 8 * half);
#pragma unroll
      for (int t = 0; t < 8; ++t) qf[s][t] = f2bf((float)qf[s][t] * c);
    }
  }
  const __bf16* kbase = (const __bf16*)p.k + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;
  const __bf16* vbase = (const __bf16*)p.v + ((int64_t)b * p.G + kvh) * (int64_t)p.S * D;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
  float l_run = 0.f, mr = 0.f;  // running sum of P and the reference (log2 units)
  const int nblocks = pos_last / kKeyBlock + 1;

  // chunk position of 16-byte chunk c in row r is c ^ swz(r)
  auto swz = [](int rr) { return ((rr & 3) << 2) | ((rr >> 2) & 3); };
  constexpr int RPC = 1024 / ROWB;  // key rows per 1 KiB chunk
  const int dma_r = (16 * lane) / ROWB;
  const int dma_p = ((16 * lane) % ROWB) / 16;
  // as in the d <= 64 form: a fixed per-lane offset and a raw buffer resource
  // per block, which reads zeros past the sequence
  uint32_t dma_off[NPW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int rb = (wave * NPW + i) * RPC + dma_r;
    dma_off[i] = rb * ROWB + 16 * (dma_p ^ swz(rb));
  }
  // Block kb through raw buffers over the rest of this head's keys: rows past
  // the sequence read zeros (and are masked).
  const uint32_t head_bytes = (uint32_t)p.S * ROWB;
  auto dma = [&](const int kb, const int bf) __attribute__((always_inline)) {
    const uint32_t skip = (uint32_t)kb * MATB;
    const uint32_t rem = head_bytes > skip ? head_bytes - skip : 0u;
    const i32x4 rk = buf_rsrc((const char*)kbase + skip, rem);
    const i32x4 rv = buf_rsrc((const char*)vbase + skip, rem);
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int n = wave * NPW + i;
      lds_dma16_b(rk, dma_off[i], lds[0][bf] + n * 1024);
      lds_dma16_b(rv, dma_off[i], lds[1][bf] + n * 1024);
    }
  };

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16 sh[2];      // S^T of the current and the next key half (log2 units, relative to mr)
  u32x4 ph[2][2];    // bf16 P^T fragments of a key half, one per 16-key step
  float ls[2];       // row sums of the bf16 P of a key half
  bf16x8 kf[KS];     // K fragments of one key half
  bf16x8 vf[2][DB];  // V^T fragments of one key half, by 16-key step and d block

  // K fragment s of key half sb: row sb*32 + l32, chunk 2s + half
  int k_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = (l32 * ROWB + 16 * ((2 * s + half) ^ swz(l32))) & 0xffff;
  auto read_k = [&](const int buf, const int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = *(const bf16x8*)(lds[0][buf] + sb * 32 * ROWB + k_off[s]);
  };
  // V^T fragments: as in the quarter form (lane (half, l32) holds d = db*32 +
  // l32, contraction element t <-> key sb*32 + 16*st + 8*(t/4) + 4*half + t%4)
  const int tr_key = 4 * half + ((lane & 15) >> 2);
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int v_off[2][DB];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_off[tt][db] = ((8 * tt + tr_key) * ROWB + 16 * ((4 * db + (tr_d >> 3)) ^ swz(8 * tt + tr_key)) + 2 * (tr_d & 7)) & 0xffff;
  // Per-lane base addresses of the V reads in the first V buffer, kept opaque
  // (so that the compiler does not fold the V region's 64 KiB start back into
  // each read) and masked to 17 bits (so that it may add a non-negative
  // constant in the instruction's 16-bit offset field): with the buffer index
  // a constant in every unrolled copy of the block loop, each LDS read is a
  // register plus an immediate, with no address arithmetic in the loop. The K
  // offsets are masked to 16 bits for the same reason.
  uint32_t v_base[2][DB];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds[1][0] + v_off[tt][db];
      __asm__("" : "+v"(a));
      v_base[tt][db] = a & 0x1ffff;
    }
  auto read_v = [&](const int buf, const int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x4 vw;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const uint32_t a = v_base[tt][db] + buf * MATB + (sb * 32 + 16 * st) * ROWB;
          const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)a);
          const u32x2 w = __builtin_bit_cast(u32x2, x);
          vw[2 * tt] = w[0];
          vw[2 * tt + 1] = w[1];
        }
        vf[st][db] = __builtin_bit_cast(bf16x8, vw);
      }
  };
  // S^T of a key half into slot i; the accumulator starts at -mr (0 in the
  // first block, which sets the reference)
  // -mr as a kept 16-register MFMA accumulator, rewritten (asm moves tied to
  // the old value, so it stays in place) only when the reference moves
  f32x16 bias = {};
  auto set_bias = [&]() __attribute__((always_inline)) {
    const float nm = -mr;
#pragma unroll
    for (int j = 0; j < 16; ++j) __asm__("v_mov_b32 %0, %1" : "+v"(bias[j]) : "v"(nm));
  };
  auto s_mfma = [&](const int i, auto first_tag) __attribute__((always_inline)) {
    const f32x16 zero16 = {};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sh[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          kf[s], qf[s], s == 0 ? (decltype(first_tag)::value ? zero16 : bias) : sh[i], 0, 0, 0);
  };
  auto pv_mfma = [&](const int i) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st][db], __builtin_bit_cast(bf16x8, ph[i][st]),
                                                           oacc[db], 0, 0, 0);
  };
  auto exps = [&](const int i) __attribute__((always_inline)) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const bf16x2 pr = {f2bf(__builtin_amdgcn_exp2f(sh[i][j])), f2bf(__builtin_amdgcn_exp2f(sh[i][j + 1]))};
      ph[i][j >> 3][(j & 7) >> 1] = __builtin_bit_cast(uint32_t, pr);
      acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);  // row sum of the bf16 P used in P V
    }
    ls[i] = acc;
  };
  // Exact path: move the reference up to this half's max (the first block
  // sets it), rescale O and l, shift the next half's S^T, recompute P.
  auto exact = [&](const int i, auto first_tag) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    float bmax = sh[i][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) bmax = fmaxf(bmax, sh[i][j]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    // key 0 is visible to every row, so bmax is finite in the first block
    const float delta = FIRST ? bmax : fmaxf(bmax, 0.f);
    mr += delta;
    set_bias();
    if constexpr (!FIRST) {
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sh[i][j] -= delta;
      sh[i ^ 1][j] -= delta;
    }
    exps(i);
  };
  auto mask = [&](const int i, const int kb, const bool on) __attribute__((always_inline)) {
    if (on) {
      __asm__ volatile("" ::: "memory");  // keep this a real branch
      // key kb*64 + sb*32 + 8*(j/4) + 4*half + j%4 is visible iff key <= pos
      const int lim = pos - kb * kKeyBlock - i * 32 - 4 * half;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + (j & 3) > lim) sh[i][j] = -INFINITY;
    }
  };
  auto settle = [&](const int i, auto first_tag) __attribute__((always_inline)) {
    if constexpr (decltype(first_tag)::value) {
      exact(i, first_tag);
    } else if (__builtin_amdgcn_ballot_w64(ls[i] > kSumLimit) != 0) {
      __asm__ volatile("" ::: "memory");  // keep this a real branch
      exact(i, first_tag);
    }
    l_run += ls[i];
  };
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KS + 2 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  };
  using kNo = std::integral_constant<bool, false>;
  using kYes = std::integral_constant<bool, true>;

  // One key block j in buffer buf. On entry sh[0] holds S^T of its key half
  // 0, kf its K fragments of key half 1 and vf block j-1's V^T fragments of
  // key half 1. Fragments are read at the end of a step, after the last MFMA
  // that uses the ones they replace.
  auto iteration = [&](const int j, const int buf, const int nbuf, const bool masked, auto first_tag,
                       auto prev_tag) __attribute__((always_inline)) {
    // step 0: S^T(key half 1) | P V(key half 1 of block j-1) | softmax(key half 0)
    mask(0, j, masked);
    s_mfma(1, first_tag);
    if constexpr (decltype(prev_tag)::value) pv_mfma(1);
    if constexpr (!decltype(first_tag)::value) exps(0);
    interleave();
    settle(0, first_tag);
    read_v(buf, 0);
    // block j+1 (loaded two blocks ago) is complete and visible after the
    // wait, which leaves block j+2's loads in flight, and the barrier; block
    // j+3 then goes into the buffer of block j-1, whose last reads were
    // issued in its step 1. Every block issues the same loads (past the last
    // block it re-loads that one), so the wait count is fixed.
    __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NPW) : "memory");
    __syncthreads();
    dma(min(j + 3, nblocks - 1), (buf + 3) % NBUF);
    read_k(nbuf, 0);  // past the last block this reads a stale buffer; the result is unused
    // step 1: S^T(key half 0 of block j+1) | P V(key half 0) | softmax(key half 1)
    mask(1, j, masked);
    s_mfma(0, kNo());
    pv_mfma(0);
    exps(1);
    interleave();
    settle(1, kNo());
    read_v(buf, 1);
    read_k(nbuf, 1);
  };

  dma(0, 0);
  dma(min(1, nblocks - 1), 1);
  dma(min(2, nblocks - 1), 2);
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * NPW) : "memory");
  __syncthreads();
  read_k(0, 0);
  s_mfma(0, kYes());
  read_k(0, 1);
  // Blocks at or below the tile's first position need no mask. The first
  // block sets the reference (and shifts its key half 1 to it).
  const int nfull = min((pos_first + 1) / kKeyBlock, nblocks);
  iteration(0, 0, 1, nfull < 1, kYes(), kNo());
  // Block j sits in buffer j % 4. The loop is unrolled over the four buffers
  // so that every LDS address is a per-lane register plus an immediate.
  static_assert(NBUF == 4, "unrolled over four buffers");
  int j = 1;
  for (; j + 4 <= nblocks; j += 4) {
    iteration(j, 1, 2, j >= nfull, kNo(), kYes());
    iteration(j + 1, 2, 3, j + 1 >= nfull, kNo(), kYes());
    iteration(j + 2, 3, 0, j + 2 >= nfull, kNo(), kYes());
    iteration(j + 3, 0, 1, j + 3 >= nfull, kNo(), kYes());
  }
  if (j < nblocks) {
    iteration(j, 1, 2, j >= nfull, kNo(), kYes());
    if (j + 1 < nblocks) {
      iteration(j + 1, 2, 3, j + 1 >= nfull, kNo(), kYes());
      if (j + 2 < nblocks) iteration(j + 2, 3, 0, j + 2 >= nfull, kNo(), kYes());
    }
  }
  pv_mfma(1);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS-DMA may outlive the workgroup

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  const float inv = 1.f / l_tot;
  if (p.lse_r && half == 0) {  // ln of the normaliser: (reference + log2 l) * ln 2
    const float lse = (mr + __log2f(l_tot)) * 0.69314718055994531f;
    if (v == p.G) p.lse_s[(int64_t)b * p.S + pos] = lse;
    else p.lse_r[(((int64_t)b * p.S + pos) * p.G + v) * p.K + slot] = lse;
  }
  __bf16* out = (v == p.G) ? (__bf16*)p.o_s + ((int64_t)b * p.S + pos) * D
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
  if (p.lse_r && lane == 0) {
    const float lse = m + logf(l);
    if (v == p.G) p.lse_s[(int64_t)b * p.S + pos] = lse;
    else p.lse_r[(((int64_t)b * p.S + pos) * p.G + v) * p.K + slot] = lse;
  }
}

// Compute units of the current device (cached per device; a race between
// two first calls only stores the same value twice).
int device_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    c = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

// Form of the d <= 64 kernel: GQE_PREFILL_FORM=plain or split forces one
// (both compute the same outputs; tests run every case through both), any
// other value or none picks by tile count. Read at every launch.
static int prefill_form_override() {
  const char* f = getenv("GQE_PREFILL_FORM");
  if (!f) return -1;
  if (!strcmp(f, "plain")) return 0;
  if (!strcmp(f, "split")) return 1;
  return -1;
}

template <int D>
static void launch_prefill_bf16(const PrefillParams& p, hipStream_t s) {
  constexpr int TR = 256;  // rows per tile (workgroup)
  const int tiles_r = (p.S * p.K + TR - 1) / TR;
  const int tiles_s = (p.S + TR - 1) / TR;
  const int nblk = tile_grid_blocks(p, tiles_s);
  if constexpr (D <= 64) {
    // Fewer tiles than the two workgroups per CU the plain form runs: the
    // longest tile sets the time, and the key-split form halves it (measured:
    // 11-21% faster with 72-288 tiles, 25% slower with 576 tiles on 256 CUs).
    const int64_t ntiles = (int64_t)p.B * ((int64_t)p.G * tiles_r + tiles_s);
    const int forced = prefill_form_override();
    if (forced == 1 || (forced < 0 && ntiles < 2 * (int64_t)device_cus()))
      hipLaunchKernelGGL((prefill_qp_kernel<D, true>), dim3(nblk), dim3(512), 0, s, p, tiles_r, tiles_s);
    else
      hipLaunchKernelGGL((prefill_qp_kernel<D, false>), dim3(nblk), dim3(256), 0, s, p, tiles_r, tiles_s);
  } else
    hipLaunchKernelGGL(prefill_d128_kernel<D>, dim3(nblk), dim3(512), 0, s, p, tiles_r, tiles_s);
}

hipError_t launch_prefill(const PrefillParams& p, int d, bool bf16, hipStream_t s) {
  if (bf16) {
    switch (d) {
      case 32: launch_prefill_bf16<32>(p, s); break;
      case 64: launch_prefill_bf16<64>(p, s); break;
      case 128: launch_prefill_bf16<128>(p, s); break;
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
