// a3 -- merged self + cross attention.
//
// One softmax over the concatenation of the decoder's causal self-attention
// KV and the cross KV of the cached pooled passage ("KaLM-Reranker-V1-Nano --
// MLX (Apple Silicon)", What this is: a single fused scaled-dot-product
// attention over [self KV ; cross KV]).  The bf16 kernel walks the self keys
// and then the cross keys in 32-key tiles with ONE online-softmax state
// (running max m, running sum l, fp32 accumulator) that is carried across the
// self/cross boundary -- a single pass, no second reduction.
//
// Work unit (one 256-thread workgroup): one pair, one KV head and 128 "rows",
// the query heads that share that KV head packed with 32-row blocks of decoder
// rows (4 heads x 32 rows for 4:1 grouping, 2 x 64 for 2:1, 1 x 128 for 1:1),
// so every K/V tile staged in LDS serves all heads of the group.  Each wave
// owns 32 rows of one head and keeps its Q fragments (32 rows x 256) in
// registers.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, 64-wide waves):
//   S^T[key, row]  = K . Q^T     A = K tile rows from LDS, B = Q fragments
//   O^T[dim, row] += V^T . P^T   A = V^T rows from LDS,    B = P from registers
// Computing the transposed products puts one decoder row in each lane
// (lane & 31), so the softmax row max needs a single exchange with lane ^ 32,
// the rescale is one scalar per lane, and the S accumulator can be fed
// straight back as the B operand of the PV product: the K rows are loaded in
// the order "swap bits 2 and 3 of the slot index", which makes the 16 logits a
// lane holds exactly the 16 keys its PV fragments need.  V is transposed once
// per tile while it is written to LDS (8-byte stores of 4 keys), so the PV
// fragment reads are 16-byte vectors.  Rescaling of the accumulator is lazy:
// the running max only moves when a tile's max exceeds it by more than 8
// (log2 units), which keeps every exponent <= 2^8 and skips most rescales.
#include <math.h>

#include "kalm_common.h"

namespace {

constexpr int HD = 256;        // head dim of the bf16 path
constexpr int BKV = 32;        // keys per tile
constexpr int VT_LD = BKV + 8; // bf16 per transposed-V row in LDS (80 bytes)
constexpr float LAZY = 8.0f;   // lazy-rescale threshold, log2 units
constexpr int MAX_CTILES = 128;  // cross tiles per passage (Cmax <= 4096)

__device__ __forceinline__ int key_of_slot(int v, int g) {  // key a lane's v-th logit belongs to
  return v < 8 ? 8 * g + v : 16 + 8 * g + (v - 8);
}
// Physical 16-byte chunk of logical chunk c (0..31) in K row `key` (512-byte
// rows).  A ds_read_b128 is served 16 lanes at a time over 64 banks (256 bytes);
// lanes 0-15 read keys 0-15 (in the bit-2/3 swapped order) at one logical
// chunk, so XOR with key & 15 spreads them over 16 distinct chunk columns.
__device__ __forceinline__ int k_swz(int key, int c) { return c ^ (key & 15); }

template <int NH>
__global__ __launch_bounds__(256, 1) void merged_attn_bf16_kernel(
    const bf16_t* __restrict__ Q, int64_t q_ld, const bf16_t* __restrict__ Ks,
    const bf16_t* __restrict__ Vs, int64_t kv_ld, const int32_t* __restrict__ cu_q, int P,
    int64_t rows, int nqb, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    int64_t c_ld, const uint8_t* __restrict__ cmask, const int32_t* __restrict__ doc_of_pair,
    int D, int Cmax, int nq, int nkv, float scale_log2, bf16_t* __restrict__ O, int64_t o_ld,
    float* __restrict__ lse) {
  constexpr int WPH = 4 / NH;   // waves per head
  constexpr int RB = 32 * WPH;  // decoder rows per block
  // two ring slots of (K tile [32 keys][256], swizzled) and (V^T tile [256][32+8])
  __shared__ __attribute__((aligned(1024))) bf16_t k_lds[2][BKV * HD];
  __shared__ __attribute__((aligned(16))) bf16_t vt_lds[2][HD * VT_LD];
  __shared__ __attribute__((aligned(1024))) bf16_t q_lds[4][32 * HD];  // each wave's 32 query rows (swizzled)
  __shared__ uint32_t cm_bits[MAX_CTILES];  // valid-chunk bits of each cross tile
  __shared__ int n_ctiles_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, g = lane >> 5;
  const int G = nq / nkv, HG = G / NH;

  // heaviest row blocks first (later rows see more causal keys)
  const int64_t per_level = (int64_t)P * nkv * HG;
  const int64_t b = blockIdx.x;
  const int qb = nqb - 1 - (int)(b / per_level);
  const int64_t rem = b % per_level;
  const int p = (int)(rem % P);
  const int hgi = (int)(rem / P);
  const int kvh = hgi / HG, hg = hgi % HG;

  const int64_t row0 = cu_q[p];
  int Lq = cu_q[p + 1] - (int)row0;
  if (row0 < 0 || row0 >= rows || Lq < 0) Lq = 0;
  else if (row0 + Lq > rows) Lq = (int)(rows - row0);
  if (qb * RB >= Lq) return;
  const int doc = doc_of_pair[p];
  const bool bad_doc = doc < 0 || doc >= D;

  // cross-tile validity bits; tiles past the last valid chunk are dropped
  const int n_ct_all = bad_doc ? 0 : (Cmax + BKV - 1) / BKV;
  if (tid < BKV) {
    const uint8_t* cmd = cmask + (int64_t)(bad_doc ? 0 : doc) * Cmax;
    for (int ct = 0; ct < n_ct_all; ++ct) {
      const int c = ct * BKV + tid;
      const bool v = c < Cmax && cmd[c] != 0;
      const uint64_t bits = __ballot(v);
      if (tid == 0) cm_bits[ct] = (uint32_t)bits;
    }
    if (tid == 0) {
      int last = 0;
      for (int ct = 0; ct < n_ct_all; ++ct)
        if (cm_bits[ct]) last = ct + 1;
      n_ctiles_s = last;
    }
  }
  __syncthreads();
  const int n_ct = n_ctiles_s;

  const int h = kvh * G + hg * NH + wave / WPH;
  const int qr0 = qb * RB + (wave % WPH) * 32;  // first decoder row of this wave
  const int i_loc = qr0 + r;                     // this lane's decoder row (pair-local)
  const int i_ld = min(i_loc, Lq - 1);
  const int wave_last = min(qr0 + 31, Lq - 1);

  // this wave's 32 query rows -> LDS by DMA (16 instructions of 2 rows x 512 bytes);
  // lane l writes physical chunk l & 31 of row 2j + (l >> 5); chunks XOR-swizzled
  // with row & 15 like K, so the B-operand reads of 16 rows are conflict free
  {
    const uint64_t qbase = uniform64((uint64_t)(uintptr_t)(Q + row0 * q_ld + (int64_t)h * HD));
    const uint32_t qlds = __builtin_amdgcn_readfirstlane(lds_addr(&q_lds[wave][0]));
    const uint32_t q_ld2 = (uint32_t)q_ld * 2u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int qrow = 2 * j + (lane >> 5);
      const int src_row = min(qr0 + qrow, Lq - 1);
      dma16(qbase, (uint32_t)src_row * q_ld2 + (uint32_t)(k_swz(qrow, lane & 31) * 16), qlds + j * 1024);
    }
  }

  f32x16_t oacc[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_self = min(Lq, qb * RB + RB);  // causal keys the block needs
  const int n_st = (n_self + BKV - 1) / BKV;
  const int n_tiles = n_st + n_ct;
  // byte addresses of key 0 of this pair (self) / chunk 0 of this passage (cross), head kvh
  const uint64_t ks_base = (uint64_t)(uintptr_t)(Ks + row0 * kv_ld + (int64_t)kvh * HD);
  const uint64_t vs_base = (uint64_t)(uintptr_t)(Vs + row0 * kv_ld + (int64_t)kvh * HD);
  const int64_t cdoc = (int64_t)(bad_doc ? 0 : doc) * Cmax * c_ld + (int64_t)kvh * HD;
  const uint64_t kc_base = (uint64_t)(uintptr_t)(Kc + cdoc);
  const uint64_t vc_base = (uint64_t)(uintptr_t)(Vc + cdoc);
  const uint32_t klds0 = __builtin_amdgcn_readfirstlane(lds_addr(&k_lds[0][0]));
  const uint32_t kv_ld2 = (uint32_t)kv_ld * 2u, c_ld2 = (uint32_t)c_ld * 2u;

  // Per-lane pieces of the copy addresses, fixed for the whole block.
  // K (LDS DMA): wave instruction j fills key rows kj, kj+1 (1 KB); lane l writes
  // physical chunk l & 31 of key row kj + (l >> 5).
  int kkey[4], klc16[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kkey[j] = 2 * (wave * 4 + j) + (lane >> 5);
    klc16[j] = k_swz(kkey[j], lane & 31) * 16;
  }
  const uint32_t kslab = __builtin_amdgcn_readfirstlane(wave * 4 * 1024);
  // V (registers): thread holds keys 4*vkg .. 4*vkg+3, dims 8*vdc .. 8*vdc+7
  const int vkg = tid & 7, vdc = tid >> 3;

  auto tile_src = [&](int v, uint64_t& kb_addr, uint64_t& vb_addr, uint32_t& ld2, int& lim, int& kb) {
    const bool self = v < n_st;
    kb = self ? v * BKV : (v - n_st) * BKV;
    ld2 = self ? kv_ld2 : c_ld2;
    lim = self ? Lq : Cmax;  // key rows at or past it are clamped
    kb_addr = (self ? ks_base : kc_base) + (uint64_t)kb * ld2;
    vb_addr = (self ? vs_base : vc_base) + (uint64_t)kb * ld2;
  };

  u32x4_t vr[4];
  // issue the copies of tile v: K straight to LDS slot v & 1, V into registers
  auto fetch = [&](int v) {
    uint64_t kba, vba;
    uint32_t ld2;
    int lim, kb;
    tile_src(v, kba, vba, ld2, lim, kb);
    const int nrow = lim - kb;  // rows of this tile that exist (>= 1)
    const uint32_t slot = klds0 + (uint32_t)((v & 1) * BKV * HD * 2) + kslab;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = min(kkey[j], nrow - 1);
      dma16(kba, (uint32_t)row * ld2 + klc16[j], slot + j * 1024);
    }
    const uint8_t* vb = (const uint8_t*)(uintptr_t)vba;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int row = min(4 * vkg + pp, nrow - 1);
      vr[pp] = *(const u32x4_t*)(vb + ((uint32_t)row * ld2 + vdc * 16));
    }
  };
  // zero the V rows of keys that do not exist or are masked, then write V^T
  auto store_vt = [&](int v) {
    const bool self = v < n_st;
    const int kb = self ? v * BKV : (v - n_st) * BKV;
    const uint32_t valid = self ? (Lq - kb >= BKV ? 0xffffffffu : ((1u << (Lq - kb)) - 1u)) : cm_bits[v - n_st];
    if (valid != 0xffffffffu) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
        if (!((valid >> (4 * vkg + pp)) & 1u)) vr[pp] = u32x4_t{0, 0, 0, 0};
    }
    bf16_t* vt = &vt_lds[v & 1][0] + (vdc * 8) * VT_LD + 4 * vkg;
#pragma unroll
    for (int m = 0; m < 4; ++m) {  // dims 2m (low halves) and 2m+1 (high halves)
      const uint32_t lo01 = __builtin_amdgcn_perm(vr[1][m], vr[0][m], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vr[3][m], vr[2][m], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vr[1][m], vr[0][m], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vr[3][m], vr[2][m], 0x07060302u);
      *(u32x2_t*)(vt + (2 * m) * VT_LD) = u32x2_t{lo01, lo23};
      *(u32x2_t*)(vt + (2 * m + 1) * VT_LD) = u32x2_t{hi01, hi23};
    }
  };

  const int krow = (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1);  // swap bits 2 and 3
  const bf16_t* kfrag0 = &k_lds[0][0] + krow * HD;
  const bf16_t* qfrag = &q_lds[wave][0] + r * HD;
  const bf16_t* vfrag0 = &vt_lds[0][0] + r * VT_LD + 8 * g;
  // consume tile v from ring slot v & 1
  auto consume = [&](int v) {
    const bool self = v < n_st;
    const int kb = self ? v * BKV : (v - n_st) * BKV;
    const bf16_t* kt = kfrag0 + (v & 1) * (BKV * HD);
    const bf16_t* vt = vfrag0 + (v & 1) * (HD * VT_LD);
    f32x16_t sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      const bf16x8_t kf = *(const bf16x8_t*)(kt + (k_swz(krow, 2 * s + g) << 3));
      const bf16x8_t qf = *(const bf16x8_t*)(qfrag + (k_swz(r, 2 * s + g) << 3));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, sacc, 0, 0, 0);
    }
    // masking only for the causal diagonal / ragged self tiles and partial cross tiles
    const uint32_t bits = self ? 0u : cm_bits[v - n_st];
    const bool full = self ? (kb + BKV - 1 <= qr0 && kb + BKV <= Lq) : (bits == 0xffffffffu);
    if (!full) {
      if (self) {
        const int kmax = min(i_loc, Lq - 1) - kb - 8 * g;  // slot key offsets are 8g + const
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = e < 8 ? e : e + 8;
          if (c > kmax) sacc[e] = -INFINITY;
        }
      } else {
        const uint32_t mb = bits >> (8 * g);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = e < 8 ? e : e + 8;
          if (!((mb >> c) & 1u)) sacc[e] = -INFINITY;
        }
      }
    }
    float tmax = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, sacc[e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * scale_log2;  // scale > 0 commutes with max
    if (v == 0) {
      m_run = tmax;  // first tile (causal tile 0: key 0 is visible to every row); accumulator still 0
    } else if (__ballot(tmax > m_run + LAZY)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < HD / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
    }
    const float nm = -m_run;
    bf16x8_t pf0, pf1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[e], scale_log2, nm));  // exp2(-inf) = 0
      l_run += pv;
      if (e < 8) pf0[e] = to_bf16(pv);
      else pf1[e - 8] = to_bf16(pv);
    }
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
      const bf16x8_t vf0 = *(const bf16x8_t*)(vt + db * 32 * VT_LD);
      const bf16x8_t vf1 = *(const bf16x8_t*)(vt + db * 32 * VT_LD + 16);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf0, pf0, oacc[db], 0, 0, 0);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf1, pf1, oacc[db], 0, 0, 0);
    }
  };

  // software pipeline: tile v+1's K copy and V loads are in flight while tile v
  // is consumed; one barrier per tile publishes the next slot
  fetch(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  store_vt(0);
  __syncthreads();
  for (int v = 0; v < n_tiles; ++v) {
    const bool more = v + 1 < n_tiles;
    if (more) fetch(v + 1);
    if (v >= n_st || v * BKV <= wave_last) consume(v);  // a wave skips causal tiles entirely above its rows
    if (more) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      store_vt(v + 1);
    }
    __syncthreads();
  }

  // ---- normalise and store
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (i_loc < Lq) {
    const float inv = bad_doc ? __builtin_nanf("") : 1.f / l_tot;
    bf16_t* op = O + (row0 + i_loc) * o_ld + (int64_t)h * HD + 4 * g;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16_t& a = oacc[db];
        u32x2_t o;
        o[0] = pack_bf16x2(a[4 * q4 + 0] * inv, a[4 * q4 + 1] * inv);
        o[1] = pack_bf16x2(a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv);
        *(u32x2_t*)(op + db * 32 + 8 * q4) = o;
      }
    if (lse && g == 0)
      lse[(row0 + i_loc) * nq + h] =
          bad_doc ? __builtin_nanf("") : (m_run + __builtin_log2f(l_tot)) * 0.69314718055994531f;
  }
}

// fp32 path (the small fp32 workload): one wavefront per (pair, head, row),
// lanes split the head dim, one online-softmax state per row walking the
// causal self keys and then the valid cross keys.
__global__ __launch_bounds__(256) void merged_attn_f32_kernel(
    const float* __restrict__ Q, int64_t q_ld, const float* __restrict__ Ks,
    const float* __restrict__ Vs, int64_t kv_ld, const int32_t* __restrict__ cu_q, int64_t rows,
    const float* __restrict__ Kc, const float* __restrict__ Vc, int64_t c_ld,
    const uint8_t* __restrict__ cmask, const int32_t* __restrict__ doc_of_pair, int D, int Cmax,
    int nq, int nkv, int d, float scale, float* __restrict__ O, int64_t o_ld,
    float* __restrict__ lse, int nrb) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = blockIdx.x;
  const int i = (int)(blk % nrb) * 4 + (threadIdx.x >> 6);
  const int h = (int)((blk / nrb) % nq);
  const int p = (int)(blk / ((int64_t)nrb * nq));
  const int64_t row0 = cu_q[p];
  int Lq = cu_q[p + 1] - (int)row0;
  if (row0 < 0 || row0 >= rows || Lq < 0) Lq = 0;
  else if (row0 + Lq > rows) Lq = (int)(rows - row0);
  if (i >= Lq) return;
  const int kvh = h / (nq / nkv);
  const int doc = doc_of_pair[p];
  const bool bad_doc = doc < 0 || doc >= D;
  constexpr int MAXJ = 4;  // d <= 256
  const int nj = (d + 63) / 64;
  float q[MAXJ], acc[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int e = lane + 64 * j;
    q[j] = (j < nj && e < d) ? Q[(row0 + i) * q_ld + (int64_t)h * d + e] : 0.f;
    acc[j] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const float* krow, const float* vrow) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int e = lane + 64 * j;
      if (j < nj && e < d) part = fmaf(q[j], krow[e], part);
    }
    const float s = wave_sum(part) * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float pw = expf(s - m_new);
    l = l * alpha + pw;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int e = lane + 64 * j;
      const float vv = (j < nj && e < d) ? vrow[e] : 0.f;
      acc[j] = acc[j] * alpha + pw * vv;
    }
    m = m_new;
  };
  for (int jk = 0; jk <= i; ++jk)
    visit(Ks + (row0 + jk) * kv_ld + (int64_t)kvh * d, Vs + (row0 + jk) * kv_ld + (int64_t)kvh * d);
  if (!bad_doc)
    for (int c = 0; c < Cmax; ++c)
      if (cmask[(int64_t)doc * Cmax + c])
        visit(Kc + ((int64_t)doc * Cmax + c) * c_ld + (int64_t)kvh * d,
              Vc + ((int64_t)doc * Cmax + c) * c_ld + (int64_t)kvh * d);
  const float inv = bad_doc ? __builtin_nanf("") : 1.f / l;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int e = lane + 64 * j;
    if (j < nj && e < d) O[(row0 + i) * o_ld + (int64_t)h * d + e] = acc[j] * inv;
  }
  if (lse && lane == 0) lse[(row0 + i) * nq + h] = bad_doc ? __builtin_nanf("") : m + logf(l);
}

}  // namespace

namespace kalm {

void launch_merged_attn_bf16(const bf16_t* Q, int64_t q_ld, const bf16_t* Ks, const bf16_t* Vs,
                             int64_t kv_ld, const int32_t* cu_q, int P, int64_t rows, int max_lq,
                             const bf16_t* Kc, const bf16_t* Vc, int64_t c_ld, const uint8_t* cmask,
                             const int32_t* doc_of_pair, int D, int Cmax, int nq, int nkv, float scale,
                             bf16_t* O, int64_t o_ld, float* lse, hipStream_t s) {
  const int G = nq / nkv;
  const int NH = G >= 4 ? 4 : G;  // heads per block (G is 1, 2 or a multiple of 4)
  const int RB = 32 * (4 / NH);
  const int nqb = (max_lq + RB - 1) / RB;
  const int64_t blocks = (int64_t)P * nkv * (G / NH) * nqb;
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)blocks), block(256);
  if (blocks == 0) return;
  if (NH == 4)
    hipLaunchKernelGGL(merged_attn_bf16_kernel<4>, grid, block, 0, s, Q, q_ld, Ks, Vs, kv_ld, cu_q, P, rows, nqb,
                       Kc, Vc, c_ld, cmask, doc_of_pair, D, Cmax, nq, nkv, sl2, O, o_ld, lse);
  else if (NH == 2)
    hipLaunchKernelGGL(merged_attn_bf16_kernel<2>, grid, block, 0, s, Q, q_ld, Ks, Vs, kv_ld, cu_q, P, rows, nqb,
                       Kc, Vc, c_ld, cmask, doc_of_pair, D, Cmax, nq, nkv, sl2, O, o_ld, lse);
  else
    hipLaunchKernelGGL(merged_attn_bf16_kernel<1>, grid, block, 0, s, Q, q_ld, Ks, Vs, kv_ld, cu_q, P, rows, nqb,
                       Kc, Vc, c_ld, cmask, doc_of_pair, D, Cmax, nq, nkv, sl2, O, o_ld, lse);
}

void launch_merged_attn_f32(const float* Q, int64_t q_ld, const float* Ks, const float* Vs,
                            int64_t kv_ld, const int32_t* cu_q, int P, int64_t rows, int max_lq,
                            const float* Kc, const float* Vc, int64_t c_ld, const uint8_t* cmask,
                            const int32_t* doc_of_pair, int D, int Cmax, int nq, int nkv, int d,
                            float scale, float* O, int64_t o_ld, float* lse, hipStream_t s) {
  if (P == 0 || max_lq == 0) return;
  const int nrb = (max_lq + 3) / 4;  // 4 rows (one per wave) per block
  const dim3 grid((unsigned)((int64_t)nrb * nq * P)), block(256);
  hipLaunchKernelGGL(merged_attn_f32_kernel, grid, block, 0, s, Q, q_ld, Ks, Vs, kv_ld, cu_q, rows, Kc, Vc,
                     c_ld, cmask, doc_of_pair, D, Cmax, nq, nkv, d, scale, O, o_ld, lse, nrb);
}

}  // namespace kalm
