// Merged self + cross attention, bf16 kernel (instantiated by attn.hip).
//
// One softmax over the concatenation of the decoder's causal self-attention
// KV and the cross KV of the cached pooled passage ("KaLM-Reranker-V1-Nano --
// MLX (Apple Silicon)", What this is: a single fused scaled-dot-product
// attention over [self KV ; cross KV]).  The bf16 kernel walks the self keys
// and then the cross keys in 32-key tiles with ONE online-softmax state
// (running max m, running sum l, fp32 accumulator) that is carried across the
// self/cross boundary -- a single pass, no second reduction.
//
// Work unit (one workgroup of NW = 4 waves by default, or 8): one pair, one
// KV head and NW slots of 32 decoder rows x one query head -- the query heads
// that share the KV head packed with row blocks (4 heads x 32 rows for 4:1
// grouping with 4 waves) -- so every K/V tile staged in LDS serves 32 * NW
// query vectors.  Each wave keeps its Q fragments (32 rows x 256 dims) and its
// fp32 O accumulator in registers (about 250 VGPRs, two waves per SIMD).  K
// and V tiles move global -> LDS with direct-to-LDS loads through a ring of 2
// (4 waves, 64 KB: two workgroups per CU, whose phases interleave on the
// SIMDs and hide each other's prologue and epilogue) or 3 (8 waves, 96 KB).

// MFMA mapping (v_mfma_f32_32x32x16_bf16, 64-wide waves):
//   S^T[key, row]  = K . Q^T     A = K tile rows from LDS, B = Q fragments
//   O^T[dim, row] += V^T . P^T   A = V^T from LDS (transposing reads), B = P
// Computing the transposed products puts one decoder row in each lane
// (lane & 31), so the softmax row max needs a single exchange with lane ^ 32,
// the rescale is one scalar per lane, and the S accumulator can be fed
// straight back as the B operand of the PV product: the K rows are read in
// the order "swap bits 2 and 3 of the slot index", which makes the 16 logits a
// lane holds exactly the 16 keys its PV fragments need.  Rescaling of the
// accumulator is lazy: the running max only moves when a tile's max exceeds
// it by more than 8 (log2 units), which keeps every exponent <= 2^8 and skips
// most rescales.
#pragma once
#include <math.h>

#include "kalm_common.h"

namespace {

constexpr int HD = 256;          // head dim of the bf16 path
constexpr int BKV = 32;          // keys per tile
constexpr float LAZY = 8.0f;     // lazy-rescale threshold, log2 units
// Streaming (non-temporal) hints for the Q loads and for the O stores, off by
// default: at the Small shape the hinted Q loads took the kernel from 1.66 to
// 1.98 ms, and the hinted O stores changed nothing measurable.
#ifndef ATTN_STREAM_Q
#define ATTN_STREAM_Q 0
#endif
#ifndef ATTN_STREAM_O
#define ATTN_STREAM_O 0
#endif
#if ATTN_STREAM_Q
#define ATTN_LD_Q(p) __builtin_nontemporal_load(p)
#else
#define ATTN_LD_Q(p) (*(p))
#endif
#if ATTN_STREAM_O
#define ATTN_ST_O(v, p) __builtin_nontemporal_store(v, p)
#else
#define ATTN_ST_O(v, p) (*(p) = (v))
#endif
#ifndef ATTN_WAVES
#define ATTN_WAVES 4             // waves per workgroup (4 or 8)
#endif


// Physical 16-byte chunk of logical chunk c (0..31) in a K row (512 bytes).
// The S product reads 16 keys at one logical chunk per 16-lane phase over 64
// banks (256 bytes): XOR with key & 15 spreads them over 16 chunk columns.
__device__ __forceinline__ int k_swz(int key, int c) { return c ^ (key & 15); }
// Same for a V row.  V is read with ds_read_b64_tr_b16: 32 lanes take 8 bytes
// from each of 4 consecutive keys at 4 consecutive chunks; XOR with 4*(key & 3)
// puts the 4 keys on 16 distinct chunk columns.
__device__ __forceinline__ int v_swz(int key, int c) { return c ^ ((key & 3) << 2); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Transposing LDS read at a byte address (gfx950 ds_read_b64_tr_b16).  In
// each 16-lane group, lane i receives halfword (i & 3) of the 8-byte pieces
// addressed by lanes (i >> 2) + 4k, k = 0..3 (in that order).
__device__ __forceinline__ u32x2_t lds_tr_at(uint32_t addr) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(size_t)addr);
  return __builtin_bit_cast(u32x2_t, v);
}

// The two halves of a wave exchanged (gfx950 v_permlane32_swap): for every
// lane, {a, b} holds the value of lane l and of lane l ^ 32, in some order --
// enough for a symmetric combination such as a max or a sum, without the LDS
// crossbar a general lane shuffle goes through.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// 16-byte LDS read at a byte address.
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
__device__ __forceinline__ bf16x8_t lds_read16(uint32_t addr) { return *(const lds_bf16x8_t*)(size_t)addr; }
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
__device__ __forceinline__ u32x4_t lds_read16u(uint32_t addr) { return *(const lds_u32x4_t*)(size_t)addr; }
__device__ __forceinline__ void lds_write8(uint32_t addr, u32x2_t v) { *(lds_u32x2_t*)(size_t)addr = v; }

// Row spaces of one pair.  The pair's self keys are Lq = cu_q[p+1] - cu_q[p]
// decoder positions; the query rows handled are positions pos0 .. pos0+nrow-1.
//   mode 0 (all rows):   Q, self K/V and O rows start at cu_q[p];
//   mode 1 (final row):  one query row per pair, position Lq-1; Q and O row p
//                        (self K/V rows still start at cu_q[p]);
//   mode 2 (shared):     Q and self K/V are the rows of the pair's query
//                        (p / D), shared by all its D passages, at cu_q[qD]/D;
//                        O rows start at cu_q[p];
//   mode 3 (shared final row): the final position only, of the shared rows:
//                        Q row cu_q[qD]/D + Lq-1, self K/V rows as mode 2,
//                        O row p.
// A pair whose rows fall outside the given row counts is skipped (no access).
struct PairRows {
  int64_t kv0, q0, o0;
  int Lq, nrow, pos0;
  bool ok;
};
__device__ __forceinline__ PairRows pair_rows(const int32_t* __restrict__ cu_q, int p, int D, int mode,
                                              int64_t q_rows, int64_t kv_rows, int64_t o_rows) {
  PairRows pr;
  const int64_t c0 = cu_q[p];
  pr.Lq = (int)((int64_t)cu_q[p + 1] - c0);
  pr.kv0 = pr.q0 = pr.o0 = c0;
  const bool fin = mode == 1 || mode == 3;
  if (mode == 2 || mode == 3) {
    const int64_t qs = (int64_t)cu_q[(int64_t)(p / D) * D] / D;
    pr.kv0 = pr.q0 = qs;
    if (mode == 3) {
      pr.q0 = qs + pr.Lq - 1;
      pr.o0 = p;
    }
  } else if (mode == 1) {
    pr.q0 = pr.o0 = p;
  }
  pr.nrow = fin ? (pr.Lq > 0 ? 1 : 0) : pr.Lq;
  pr.pos0 = fin ? pr.Lq - 1 : 0;
  pr.ok = c0 >= 0 && pr.Lq >= 0 && pr.kv0 >= 0 && pr.kv0 + pr.Lq <= kv_rows && pr.q0 >= 0 &&
          pr.q0 + pr.nrow <= q_rows && pr.o0 >= 0 && pr.o0 + pr.nrow <= o_rows;
  return pr;
}

// One workgroup = NW waves; wave w holds RT row tiles of 32 decoder rows of
// one query head (NH heads x WPH row blocks per workgroup), so every K/V tile
// staged in LDS is shared by 32 * RT * NW (row, head) query vectors, and with
// RT = 2 every K and V fragment read from LDS feeds two MFMAs (two
// independent accumulation chains).
//
// PART selects which keys the softmax walks (the merged softmax split at the
// self/cross boundary and put back together by log-sum-exp weights):
//   0  self then cross keys: the merged attention, bf16 output;
//   1  the causal self keys only (plain causal self-attention): fp32 output
//      O and its lse -- a self partial;
//   2  the cross keys only, starting from a self partial (oi, lsei) read at
//      the Q row: the online state begins at m = lse, l = 1, acc = o, which is
//      the state the walk over the self keys would have left; bf16 output;
//   3  one share of the cross keys (split-KV): block row y of the grid walks
//      cross tiles [y T, y T + T), T = ceil(tiles / gridDim.y), from an empty
//      state and writes an fp32 partial (o, lse) to slice y of Ov / lse (slice
//      stride o_rows rows); a share with no visible key writes o = 0,
//      lse = -inf.  The shares are combined by the log-sum-exp merge.
template <int NH, int NW, int RT, int MODE, int PART>
__global__ __launch_bounds__(NW * 64, RT == 1 ? 2 : 1) void merged_attn_bf16_kernel(
    const bf16_t* __restrict__ Q, int64_t q_ld, const bf16_t* __restrict__ Ks,
    const bf16_t* __restrict__ Vs, int64_t kv_ld, const int32_t* __restrict__ cu_q, int P,
    int64_t q_rows, int64_t kv_rows, int64_t o_rows, int nqb, const bf16_t* __restrict__ Kc,
    const bf16_t* __restrict__ Vc, int64_t c_ld, const uint8_t* __restrict__ cmask,
    const int32_t* __restrict__ doc_of_pair, int D, int Cmax, int nq, int nkv, float scale_log2,
    void* __restrict__ Ov, int64_t o_ld, float* __restrict__ lse, const float* __restrict__ oi, int64_t oi_ld,
    const float* __restrict__ lsei) {
  constexpr int WPH = NW / NH;            // row blocks per head
  constexpr int RB = 32 * RT * WPH;       // decoder rows per block
  // K and V rings: 2 deep for RT = 1 with 4 waves (two workgroups per CU,
  // 64 KB each), 3 deep with 8 waves; for RT = 2 (one workgroup per CU)
  // ATTN_RT2_RING deep.  A 3-deep K ring beside a 2-deep V ring (80 KB) was
  // measured slower at the Small shape (2.40 vs 2.25 ms).
#ifndef ATTN_RT2_RING
#define ATTN_RT2_RING 3
#endif
  constexpr int KR = RT == 2 ? ATTN_RT2_RING : (NW == 8 ? 3 : 2), VR = KR;
  constexpr int RPW = BKV / NW;           // key rows each wave copies per tile
  constexpr int TILE_B = BKV * HD * 2;    // bytes of one K (or V) tile
  // K tiles (k_swz) in slots 0..KR-1, then V tiles (v_swz) in VR slots
  __shared__ __attribute__((aligned(1024))) uint8_t kv_lds[(KR + VR) * TILE_B];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, g = lane >> 5;
  const int G = nq / nkv, HG = G / NH;

  // Work order for L2 reuse: the pair's head groups and row blocks
  // consecutive (they share the pair's self K/V and the passage's cross K/V);
  // passage-major -- every query's pair with passage 0, then with passage 1,
  // ... (pair p = q D + passage in the layout of kalm_pair_layout), so one
  // passage's cross K/V stays in L2 across the queries -- and each XCD (block
  // b runs on XCD b % 8) walks a contiguous range.
  // (32-bit unsigned arithmetic: the host keeps the number of work items
  // below 2^31, and 64-bit divisions by run-time values cost the scalar unit
  // hundreds of instructions)
  const uint32_t per_pair = (uint32_t)nkv * (uint32_t)HG * (uint32_t)nqb;
  const uint32_t total = (uint32_t)P * per_pair;
  const uint32_t b = blockIdx.x;
  const uint32_t xper = total / 8;
  const uint32_t t = (b < xper * 8) ? (b % 8) * xper + b / 8 : b;
  const uint32_t pi = t / per_pair;  // pair in walk order
  int p = (int)pi;
  if (D > 0 && P % D == 0) {
    const uint32_t nQ = (uint32_t)P / (uint32_t)D;
    const uint32_t q = pi % nQ;
    p = (int)(q * (uint32_t)D + (pi - q) / nQ);
  }
  const uint32_t rem = t - pi * per_pair;
  const uint32_t hgu = rem / (uint32_t)nqb;
  const int qb = (int)(rem - hgu * (uint32_t)nqb);
  const int hgi = (int)hgu;
  const int kvh = hgi / HG, hg = hgi % HG;

  const PairRows pr = pair_rows(cu_q, p, D, MODE, q_rows, kv_rows, o_rows);
  if (!pr.ok) {
    if (threadIdx.x == 0) KALM_DBG(KALM_DBG_PAIR_ROWS);
    return;
  }
  if (qb * RB >= pr.nrow) return;
  const int Lq = pr.Lq, nrow = pr.nrow, pos0 = pr.pos0;

  const int doc = PART == 1 ? 0 : doc_of_pair[p];  // a self partial reads no passage
  const bool bad_doc = PART != 1 && (doc < 0 || doc >= D);
  if (bad_doc && threadIdx.x == 0) KALM_DBG(KALM_DBG_DOC);

  // cross-tile validity words, kept in registers by every wave: lane l holds
  // the words of tiles l and l + 64 (one ballot per 64 chunks); word t is
  // read back with a scalar readlane
  const int n_ct_all = (PART == 1 || bad_doc) ? 0 : (Cmax + BKV - 1) / BKV;
  const int nc = min(n_ct_all * BKV, Cmax);  // chunks whose mask bytes are read
  const uint8_t* cmd = cmask + (int64_t)(bad_doc ? 0 : doc) * Cmax;
  // The first 256 chunks' mask bytes, loaded together from clamped in-range
  // addresses and before the Q loads: taking them then waits for these four
  // loads only (the vector memory counter completes in issue order), and the
  // Q loads' latency runs on under the ballots below.
  uint32_t pre[4] = {0, 0, 0, 0};
  if (nc > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pre[i] = cmd[min(64 * i + lane, nc - 1)];
  }
  asm volatile("" ::: "memory");  // the Q loads below stay after these

  const int h = kvh * G + hg * NH + wave / WPH;
  const int qr0 = qb * RB + (wave % WPH) * 32 * RT;  // first handled query row of this wave
  // row tile u of this wave: rows qr0 + 32u + (0..31); lane r holds one row
  int pos[RT], tile_first[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    pos[u] = pos0 + min(qr0 + 32 * u + r, nrow - 1);  // its self position: sees self keys 0..pos
    tile_first[u] = pos0 + qr0 + 32 * u;
  }
  const int wave_last = pos0 + min(qr0 + 32 * RT - 1, nrow - 1);

  // Q fragments (MFMA B operand of S^T = K Q^T): 16 k-steps of 16 dims per
  // row tile.
  bf16x8_t qf[RT][HD / 16];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const bf16_t* qp = Q + (pr.q0 + min(qr0 + 32 * u + r, nrow - 1)) * q_ld + (int64_t)h * HD + 8 * g;
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) qf[u][s] = ATTN_LD_Q((const bf16x8_t*)(qp + 16 * s));
  }
  // the mask bytes are taken only here, after the Q loads have gone out
  asm volatile("" : "+v"(pre[0]), "+v"(pre[1]), "+v"(pre[2]), "+v"(pre[3])::"memory");

  uint32_t cmw0 = 0, cmw1 = 0;
  {
    // word pair of one 64-chunk ballot: tile index w = base / 32 and w + 1
    auto put = [&](int base, uint64_t bits) {
      const int w = base >> 5;  // tile index of the low word
      if (lane == (w & 63)) {
        if (w < 64) cmw0 = (uint32_t)bits; else cmw1 = (uint32_t)bits;
      }
      if (lane == ((w + 1) & 63)) {
        if (w + 1 < 64) cmw0 = (uint32_t)(bits >> 32); else cmw1 = (uint32_t)(bits >> 32);
      }
    };
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (64 * i < nc) put(64 * i, __ballot(64 * i + lane < nc && pre[i] != 0));
    for (int base = 256; base < nc; base += 64) put(base, __ballot(base + lane < nc && cmd[base + lane] != 0));
  }
  auto cm_word = [&](int t) -> uint32_t {  // t is wave-uniform
    return t < 64 ? __builtin_amdgcn_readlane(cmw0, t) : __builtin_amdgcn_readlane(cmw1, t - 64);
  };
  const uint64_t nz0 = __ballot(cmw0 != 0), nz1 = __ballot(cmw1 != 0);
  int n_ct = nz1 ? 64 + 64 - __builtin_clzll(nz1) : (nz0 ? 64 - __builtin_clzll(nz0) : 0);
  // opaque: a self partial (no cross tile) keeps the loop the merged kernel
  // has -- with the tile kind known the compiler reorders it into spills
  asm volatile("" : "+s"(n_ct));
  int donor = 0;  // a valid chunk: masked chunk rows are fetched from it
  if (n_ct) {
    const int t = nz0 ? __builtin_ctzll(nz0) : 64 + __builtin_ctzll(nz1);
    donor = t * BKV + __builtin_ctz(cm_word(t));
  }
  // this block's share of the cross tiles (split-KV); all of them otherwise
  int ct0 = 0;
  if constexpr (PART == 3) {
    const int tps = (n_ct_all + (int)gridDim.y - 1) / (int)gridDim.y;
    ct0 = (int)blockIdx.y * tps;
    n_ct = max(0, min(n_ct, ct0 + tps) - ct0);
  }

  f32x16_t oacc[RT][HD / 32];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) {
#pragma unroll
    for (int i = 0; i < HD / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[u][i][e] = 0.f;
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
  }
  if constexpr (PART == 2) {
    // resume from the self partial of each row: its normalised output in the
    // accumulator layout (dims 32 db + 8 q + 4 g + 0..3 of row r), m = its lse
    // in log2 units, l = 1 (held by the g = 0 half; the halves are summed at
    // the end)
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int64_t row = pr.q0 + min(qr0 + 32 * u + r, nrow - 1);
      const float* op = oi + row * oi_ld + (int64_t)h * HD + 4 * g;
#pragma unroll
      for (int i = 0; i < HD / 32; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4_t t = *(const f32x4_t*)(op + 32 * i + 8 * q4);
#pragma unroll
          for (int j = 0; j < 4; ++j) oacc[u][i][4 * q4 + j] = t[j];
        }
      m_run[u] = lsei[row * nq + h] * 1.4426950408889634f;
      l_run[u] = g == 0 ? 1.f : 0.f;
    }
  }

  const int n_self = min(Lq, pos0 + min(nrow, qb * RB + RB));  // causal keys the block needs
  const int n_st = (PART == 2 || PART == 3) ? 0 : (n_self + BKV - 1) / BKV;
  const int n_tiles = n_st + n_ct;
  // byte addresses of key 0 of this pair (self) / chunk 0 of this passage (cross), head kvh
  const uint64_t ks_base = (uint64_t)(uintptr_t)(Ks + pr.kv0 * kv_ld + (int64_t)kvh * HD);
  const uint64_t vs_base = (uint64_t)(uintptr_t)(Vs + pr.kv0 * kv_ld + (int64_t)kvh * HD);
  const int64_t cdoc = (int64_t)(bad_doc ? 0 : doc) * Cmax * c_ld + (int64_t)kvh * HD;
  const uint64_t kc_base = (uint64_t)(uintptr_t)(Kc + cdoc);
  const uint64_t vc_base = (uint64_t)(uintptr_t)(Vc + cdoc);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(kv_lds));
  const uint32_t klds0 = lds0, vlds0 = lds0 + KR * TILE_B;
  const uint32_t kv_ld2 = (uint32_t)kv_ld * 2u, c_ld2 = (uint32_t)c_ld * 2u;

  // DMA plan: wave w copies key rows RPW*w .. RPW*w + RPW-1 of a tile, two
  // rows (1 KB) per instruction; in instruction j lane l writes physical
  // chunk l & 31 of key row RPW*w + 2j + (l >> 5), i.e. logical chunk
  // (l & 31) ^ swizzle(key) of that row
  const int dkey0 = RPW * wave + (lane >> 5);
  const uint32_t dslab = __builtin_amdgcn_readfirstlane(wave * RPW * (HD * 2));

  // copy the K and V rows of tile v into ring slot v % KR.  Key rows that do
  // not exist (past the pair / the passage) or are masked are fetched from a
  // valid row instead: their logits are masked to -inf, so p = 0 multiplies a
  // finite value.
  static_assert(KR == VR, "K and V tiles are copied together");
  auto issue_kv = [&](int v) {
    const bool self = v < n_st;
    const uint32_t so = klds0 + (uint32_t)((v % KR) * TILE_B) + dslab;  // the V slab is KR tiles further
    if constexpr (RPW == 8) {
      // the eight copies of a wave (4-wave workgroups), branch-free on full
      // tiles: copy j takes key row key0 + 2j, whose swizzled chunk is, with
      // key0 = 8 wave + g (bits 1..2 clear), ck0 ^ 32 j in K and cv0 ^ 128 (j & 1)
      // in V; one M0 save/restore for the eight
      int key0 = dkey0;
      asm volatile("" : "+v"(key0));  // recompute the per-lane parts here instead of holding them
      const uint32_t c4 = (uint32_t)(__lane_id() & 31) << 4;
      const uint32_t ck0 = c4 ^ ((uint32_t)(key0 & 15) << 4), cv0 = c4 ^ ((uint32_t)(key0 & 3) << 6);
      uint32_t row[4];
      uint64_t kb, vb;
      if (self) {
        kb = ks_base;
        vb = vs_base;
        const uint32_t r0 = (uint32_t)(v * BKV + key0) * kv_ld2;
        if (v * BKV + BKV <= Lq) {
#pragma unroll
          for (int j = 0; j < 4; ++j) row[j] = r0 + (uint32_t)(2 * j) * kv_ld2;
        } else {  // the ragged last self tile: rows past the pair clamped to its last key
          const uint32_t rmax = (uint32_t)(Lq - 1) * kv_ld2;
#pragma unroll
          for (int j = 0; j < 4; ++j) row[j] = min(r0 + (uint32_t)(2 * j) * kv_ld2, rmax);
        }
      } else {
        kb = kc_base;
        vb = vc_base;
        const int t = v - n_st + ct0;
        const uint32_t bits = cm_word(t);
        const uint32_t r0 = (uint32_t)(t * BKV + key0) * c_ld2;
        if (bits == 0xffffffffu) {
#pragma unroll
          for (int j = 0; j < 4; ++j) row[j] = r0 + (uint32_t)(2 * j) * c_ld2;
        } else {  // masked chunk rows fetched from the donor chunk
          const uint32_t rd = (uint32_t)donor * c_ld2, bl = bits >> key0;
#pragma unroll
          for (int j = 0; j < 4; ++j) row[j] = ((bl >> (2 * j)) & 1u) ? r0 + (uint32_t)(2 * j) * c_ld2 : rd;
        }
      }
      dma16x8<(uint32_t)(KR * TILE_B)>(kb, row[0] + ck0, row[1] + (ck0 ^ 32u), row[2] + (ck0 ^ 64u),
                                       row[3] + (ck0 ^ 96u), vb, row[0] + cv0, row[1] + (cv0 ^ 128u), row[2] + cv0,
                                       row[3] + (cv0 ^ 128u), so);
      return;
    }
    const int kb = self ? v * BKV : (v - n_st + ct0) * BKV;
    const uint32_t ld2 = self ? kv_ld2 : c_ld2;
    const uint32_t bits = self ? 0u : cm_word(v - n_st + ct0);
    int key0 = dkey0;
    asm volatile("" : "+v"(key0));  // recompute the per-row offsets here instead of holding them
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const uint64_t base = uniform64(kv == 0 ? (self ? ks_base : kc_base) : (self ? vs_base : vc_base));
#pragma unroll
      for (int j = 0; j < RPW / 2; ++j) {
        const int key = key0 + 2 * j;
        int row;
        if (self) row = min(kb + key, Lq - 1);
        else row = ((bits >> key) & 1u) ? kb + key : donor;
        const uint32_t ro = (uint32_t)row * ld2;
        const int c = __lane_id() & 31;
        dma16(base, ro + (uint32_t)((kv == 0 ? k_swz(key, c) : v_swz(key, c)) << 4),
              so + (uint32_t)(kv * KR * TILE_B) + j * 1024);
      }
    }
  };

  // K fragment reads.  Lane (r, g) reads key row krow (r with bits 2 and 3
  // swapped) at logical chunk 2s + g of k-step s; physical chunk (2s + g) ^
  // (krow & 15) = 2s ^ (g ^ (krow & 15)), so the byte address of k-step s is
  // kx ^ 32s with one per-lane base kx (the XOR only touches bits 4..8, below
  // the 512-byte row and tile offsets).
  const int krow = (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1);
  const uint32_t kx = klds0 + krow * (HD * 2) + ((g ^ (krow & 15)) << 4);
  // V^T fragment reads (transposing, 8 bytes per lane): in 16-lane group
  // G = lane >> 4, lane i addresses key 8 * (G >> 1) + (i >> 2) (+4 for the
  // second read, +16 per k-step) at dims 16 * (G & 1) + 4 * (i & 3) of each
  // 32-dim block db.  Physical chunk 4 (db ^ (key & 3)) + c0, so the byte
  // address of block db is vx ^ 64 db.
  const int vg = lane >> 4, vi = lane & 15;
  const int vkey = 8 * (vg >> 1) + (vi >> 2);
  const int vdim0 = 16 * (vg & 1) + 4 * (vi & 3);
  const uint32_t vx = vlds0 + vkey * (HD * 2) + 64 * (vkey & 3) + 16 * (vdim0 >> 3) +
                      2 * (vdim0 & 7);

  // Copy schedule (per wave): tiles 0 .. KR-2 before the loop, then at tile
  // v the K and V rows of tile v + KR - 1.  When tile v starts, the copies
  // still allowed in flight are those of the tiles issued after it.
  constexpr int CPT = RPW / 2;  // copy instructions per wave per K (or V) tile
  for (int v = 0; v < KR - 1 && v < n_tiles; ++v) issue_kv(v);
  // Make the Q loads complete here, visibly to the compiler: its wait-count
  // pass does not see the asm copies, and would otherwise keep waiting for
  // "the Q loads" inside the tile loop with vmcnt values that, on the
  // hardware counter, also cover the next tile's copies -- serialising every
  // tile's copy with its compute.
#pragma unroll
  for (int u = 0; u < RT; ++u) {
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) asm volatile("" ::"v"(qf[u][s]));
    if constexpr (PART == 2) {
#pragma unroll
      for (int i = 0; i < HD / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) asm volatile("" ::"v"(oacc[u][i][e]));  // scalar operands: valid for the host pass too
      asm volatile("" ::"v"(m_run[u]));
    }
  }
  for (int v = 0; v < n_tiles; ++v) {
    wait_dma_ktile<2 * CPT>(min(n_tiles - 1 - v, KR - 2));
    __syncthreads();  // tile v visible; the slots of tile v-1 are free
    if (v + KR - 1 < n_tiles) issue_kv(v + KR - 1);
    const bool self = v < n_st;
    const int kb = self ? v * BKV : (v - n_st + ct0) * BKV;
    // nothing to do: no valid rows in this wave, or a causal tile entirely
    // above its rows (the wave still joins every barrier and copy); a share
    // of the cross keys also skips tiles with no visible chunk, so that its
    // first walked tile sets a finite running max
    if (qr0 >= nrow || (self && kb > wave_last)) continue;
    if (PART == 3 && cm_word(v - n_st + ct0) == 0u) continue;
    uint32_t kt = kx + (uint32_t)((v % KR) * TILE_B), vt = vx + (uint32_t)((v % VR) * TILE_B);
    // opaque per tile: keeps the compiler from hoisting 24 precomputed
    // fragment addresses out of the loop (one XOR per read is cheaper than
    // the registers they would hold)
    asm volatile("" : "+v"(kt), "+v"(vt));
    f32x16_t sacc[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[u][e] = 0.f;
    // K fragments in groups of KG k-steps, the next group read while the
    // current one multiplies (bounds the registers held by K fragments)
#ifndef ATTN_KG
#define ATTN_KG 4
#endif
    constexpr int KG = RT == 2 ? 2 : ATTN_KG;
    bf16x8_t kf[HD / 16];
#pragma unroll
    for (int j = 0; j < KG; ++j) kf[j] = lds_read16(kt ^ (32u * j));
#pragma unroll
    for (int s0 = 0; s0 < HD / 16; s0 += KG) {
      if (s0 + KG < HD / 16) {
#pragma unroll
        for (int j = 0; j < KG; ++j) kf[s0 + KG + j] = lds_read16(kt ^ (32u * (s0 + KG + j)));
      }
#pragma unroll
      for (int j = 0; j < KG; ++j)
#pragma unroll
        for (int u = 0; u < RT; ++u)
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s0 + j], qf[u][s0 + j], sacc[u], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // masking only for the causal diagonal / ragged self tiles and partial cross tiles
    const uint32_t bits = self ? 0u : cm_word(v - n_st + ct0);
    bf16x8_t pf[RT][2];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const bool full = self ? (kb + BKV - 1 <= tile_first[u] && kb + BKV <= Lq) : (bits == 0xffffffffu);
      if (!full) {
        if (self) {
          const int kmax = pos[u] - kb - 8 * g;  // slot key offsets are 8g + const
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int c = e < 8 ? e : e + 8;
            if (c > kmax) sacc[u][e] = -INFINITY;
          }
        } else {
          const uint32_t mb = bits >> (8 * g);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int c = e < 8 ? e : e + 8;
            if (!((mb >> c) & 1u)) sacc[u][e] = -INFINITY;
          }
        }
      }
      float tmax = sacc[u][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sacc[u][e]);
      tmax = max_xor32(tmax) * scale_log2;  // the row's two halves; scale > 0 commutes with max
      // lazy rescale: the running max moves only when some row's tile max
      // exceeds it by more than LAZY (log2 units); the first tile (m_run =
      // -inf, accumulator 0) always takes this branch and only sets m.  Tile 0
      // holds key 0, visible to every row, so tmax is finite there (a resumed
      // walk starts from a finite m).  (A row tile whose rows all lie above a
      // causal tile sees only -inf: no change.)
      if (__ballot(tmax > m_run[u] + LAZY)) {
        const float m_new = fmaxf(m_run[u], tmax);
        // before the first tile every row has m = -inf and a zero state: nothing to scale
        if (__ballot(m_run[u] != -INFINITY)) {
          const float alpha = __builtin_amdgcn_exp2f(m_run[u] - m_new);  // exp2(-inf) = 0
          l_run[u] *= alpha;
#pragma unroll
          for (int i = 0; i < HD / 32; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[u][i][e] *= alpha;
        }
        m_run[u] = m_new;
      }
      const float nm = -m_run[u];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[u][e], scale_log2, nm));  // exp2(-inf) = 0
        l_run[u] += pv;
        if (e < 8) pf[u][0][e] = to_bf16(pv);
        else pf[u][1][e - 8] = to_bf16(pv);
      }
    }
    // V^T fragments of 32 dims: keys 8g..8g+7 (k-step 0) and 16+8g..16+8g+7
    // (k-step 1), 4 keys per transposing read; block db+1 is read while block
    // db multiplies
    auto vread = [&](int db, u32x4_t& a0, u32x4_t& a1) {
      const uint32_t base = vt ^ (64u * db);
      const u32x2_t t0 = lds_tr_at(base), t1 = lds_tr_at(base + 4 * HD * 2);
      const u32x2_t t2 = lds_tr_at(base + 16 * HD * 2), t3 = lds_tr_at(base + 20 * HD * 2);
      a0 = u32x4_t{t0[0], t0[1], t1[0], t1[1]};
      a1 = u32x4_t{t2[0], t2[1], t3[0], t3[1]};
    };
    u32x4_t vf[HD / 32][2];
    vread(0, vf[0][0], vf[0][1]);
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
      if (db + 1 < HD / 32) vread(db + 1, vf[db + 1][0], vf[db + 1][1]);
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        oacc[u][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[db][0]), pf[u][0],
                                                              oacc[u][db], 0, 0, 0);
        oacc[u][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[db][1]), pf[u][1],
                                                              oacc[u][db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- normalise and store.  The accumulator holds, per lane (r, g), dims
  // 32 db + 8 q + 4 g + (0..3) of row r; it is staged through LDS (now free)
  // so that the global stores write whole rows, 16 bytes per lane.
  // split-KV: this block's slice of the partial outputs
  if constexpr (PART == 3) {
    Ov = (float*)Ov + (int64_t)blockIdx.y * o_rows * o_ld;
    lse += (int64_t)blockIdx.y * o_rows * nq;
  }
#pragma unroll
  for (int u = 0; u < RT; ++u) {
    const float l_tot = sum_xor32(l_run[u]);
    // an empty share of the cross keys (PART 3 only: every other walk has a
    // visible key) is the zero partial o = 0, lse = -inf
    const float inv = bad_doc ? __builtin_nanf("") : (PART == 3 && l_tot == 0.f) ? 0.f : 1.f / l_tot;
    l_run[u] = inv;  // keep the reciprocal for the stores below
    const int jl = qr0 + 32 * u + r;
    if (lse && g == 0 && jl < nrow)
      lse[(pr.o0 + jl) * nq + h] = bad_doc                        ? __builtin_nanf("")
                                   : (PART == 3 && l_tot == 0.f) ? -INFINITY
                                       : (m_run[u] + __builtin_log2f(l_tot)) * 0.69314718055994531f;
  }
  if constexpr (PART == 1 || PART == 3) {
    // fp32 partial: 16-byte stores straight from the accumulator (lanes g = 0
    // and 1 together write 32 contiguous bytes of a row)
    float* Of = (float*)Ov;
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int jl = qr0 + 32 * u + r;
      if (jl >= nrow) continue;
      float* op = Of + (pr.o0 + jl) * o_ld + (int64_t)h * HD + 4 * g;
#pragma unroll
      for (int i = 0; i < HD / 32; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16_t& a = oacc[u][i];
          const float inv = l_run[u];
          *(f32x4_t*)(op + 32 * i + 8 * q4) =
              f32x4_t{a[4 * q4] * inv, a[4 * q4 + 1] * inv, a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv};
        }
    }
    return;
  }
  bf16_t* O = (bf16_t*)Ov;
  __syncthreads();  // every wave is done with the K/V ring
  constexpr int RING_B = (KR + VR) * TILE_B;
  // dims per pass: a wave stages 32 RT rows x DPP bf16; all NW waves must fit the ring
  constexpr int DPP = NW * 32 * RT * HD * 2 <= RING_B ? HD : (NW * 32 * RT * (HD / 2) * 2 <= RING_B ? HD / 2 : HD / 4);
  constexpr int CPR = DPP / 8;                // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPR;               // rows per read-back instruction
  const uint32_t ebase = lds0 + wave * (32 * RT * DPP * 2);
  bf16_t* orow0 = O + (pr.o0 + qr0) * o_ld + (int64_t)h * HD;
#pragma unroll
  for (int pass = 0; pass < HD / DPP; ++pass) {
#pragma unroll
    for (int u = 0; u < RT; ++u)
#pragma unroll
      for (int db = 0; db < DPP / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16_t& a = oacc[u][pass * (DPP / 32) + db];
          const float inv = l_run[u];
          u32x2_t o;
          o[0] = pack_bf16x2(a[4 * q4 + 0] * inv, a[4 * q4 + 1] * inv);
          o[1] = pack_bf16x2(a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv);
          const int row = 32 * u + r;
          const int c = (4 * db + q4) ^ (row & (CPR - 1));
          lds_write8(ebase + row * (DPP * 2) + c * 16 + 8 * g, o);
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 32 * RT / RPI; ++i) {
      const int rr = RPI * i + lane / CPR, c = lane % CPR;
      const u32x4_t val = lds_read16u(ebase + rr * (DPP * 2) + ((c ^ (rr & (CPR - 1))) << 4));
      if (qr0 + rr < nrow) ATTN_ST_O(val, (u32x4_t*)(orow0 + rr * o_ld + pass * DPP + 8 * c));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

typedef void (*bf16_kernel_t)(const bf16_t*, int64_t, const bf16_t*, const bf16_t*, int64_t, const int32_t*, int,
                              int64_t, int64_t, int64_t, int, const bf16_t*, const bf16_t*, int64_t, const uint8_t*,
                              const int32_t*, int, int, int, int, float, void*, int64_t, float*, const float*, int64_t,
                              const float*);
template <int NH, int NW, int RT>
bf16_kernel_t pick_bf16_kernel(int sel) {
  switch (sel) {
    case 0: return merged_attn_bf16_kernel<NH, NW, RT, 0, 1>;
    case 1: return merged_attn_bf16_kernel<NH, NW, RT, 0, 0>;
    case 2: return merged_attn_bf16_kernel<NH, NW, RT, 1, 0>;
    case 3: return merged_attn_bf16_kernel<NH, NW, RT, 2, 0>;
    case 4: return merged_attn_bf16_kernel<NH, NW, RT, 3, 0>;
    case 5: return merged_attn_bf16_kernel<NH, NW, RT, 0, 2>;
    case 6: return merged_attn_bf16_kernel<NH, NW, RT, 1, 2>;
    case 7: return merged_attn_bf16_kernel<NH, NW, RT, 2, 2>;
    case 8: return merged_attn_bf16_kernel<NH, NW, RT, 3, 2>;
    case 9: return merged_attn_bf16_kernel<NH, NW, RT, 0, 3>;
    case 10: return merged_attn_bf16_kernel<NH, NW, RT, 1, 3>;
    case 11: return merged_attn_bf16_kernel<NH, NW, RT, 2, 3>;
    default: return merged_attn_bf16_kernel<NH, NW, RT, 3, 3>;
  }
}

// Launch of the bf16 kernel for NW waves and RT row tiles per wave.
template <int NW, int RT>
void launch_bf16(const bf16_t* Q, int64_t q_ld, const bf16_t* Ks, const bf16_t* Vs, int64_t kv_ld,
                 const int32_t* cu_q, int P, int64_t q_rows, int64_t kv_rows, int64_t o_rows, int mode, int max_lq,
                 const bf16_t* Kc, const bf16_t* Vc, int64_t c_ld, const uint8_t* cmask,
                 const int32_t* doc_of_pair, int D, int Cmax, int nq, int nkv, float scale, void* O, int64_t o_ld,
                 float* lse, int part, const float* oi, int64_t oi_ld, const float* lsei, int n_split,
                 hipStream_t s) {
  const int G = nq / nkv;
  const int NH = G >= 4 ? 4 : G;  // heads per block (G is 1, 2 or a multiple of 4)
  const int RB = 32 * RT * (NW / NH);
  const int max_rows = (mode == 1 || mode == 3) ? 1 : max_lq;  // query rows per pair
  const int nqb = (max_rows + RB - 1) / RB;
  const int64_t blocks = (int64_t)P * nkv * (G / NH) * nqb;
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)blocks, part == 3 ? (unsigned)n_split : 1u), block(NW * 64);
  if (blocks == 0) return;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, Q, q_ld, Ks, Vs, kv_ld, cu_q, P, q_rows, kv_rows, o_rows, nqb, Kc, Vc,
                       c_ld, cmask, doc_of_pair, D, Cmax, nq, nkv, sl2, O, o_ld, lse, oi, oi_ld, lsei);
  };
  // one instantiation per (heads per block, row mode, part); a self partial
  // (part 1) runs on all rows of its sequences (mode 0) only
  // 0 self partial | 1..4 merged | 5..8 resumed | 9..12 split shares (by row mode)
  const int sel = part == 1 ? 0 : 1 + 4 * (part >= 2) + 4 * (part == 3) + mode;
  if (NH == 4) go(pick_bf16_kernel<4, NW, RT>(sel));
  else if (NH == 2) go(pick_bf16_kernel<2, NW, RT>(sel));
  else go(pick_bf16_kernel<1, NW, RT>(sel));
}

}  // namespace
