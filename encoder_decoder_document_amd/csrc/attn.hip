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

__device__ __forceinline__ int key_of_slot(int v, int g) {  // key a lane's v-th logit belongs to
  return v < 8 ? 8 * g + v : 16 + 8 * g + (v - 8);
}
__device__ __forceinline__ int k_swz(int row) {  // LDS chunk swizzle of K row `row`
  return ((row >> 1) & 4) | (row & 3);
}

template <int NH>
__global__ __launch_bounds__(256, 2) void merged_attn_bf16_kernel(
    const bf16_t* __restrict__ Q, int64_t q_ld, const bf16_t* __restrict__ Ks,
    const bf16_t* __restrict__ Vs, int64_t kv_ld, const int32_t* __restrict__ cu_q, int P,
    int64_t rows, int nqb, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    int64_t c_ld, const uint8_t* __restrict__ cmask, const int32_t* __restrict__ doc_of_pair,
    int D, int Cmax, int nq, int nkv, float scale_log2, bf16_t* __restrict__ O, int64_t o_ld,
    float* __restrict__ lse) {
  constexpr int WPH = 4 / NH;   // waves per head
  constexpr int RB = 32 * WPH;  // decoder rows per block
  __shared__ __attribute__((aligned(16))) bf16_t k_lds[BKV * HD];
  __shared__ __attribute__((aligned(16))) bf16_t vt_lds[HD * VT_LD];
  __shared__ uint8_t cm_lds[BKV];

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

  const int h = kvh * G + hg * NH + wave / WPH;
  const int i_loc = qb * RB + (wave % WPH) * 32 + r;  // this lane's decoder row (pair-local)
  const int i_ld = min(i_loc, Lq - 1);
  const int wave_last = min(qb * RB + (wave % WPH) * 32 + 31, Lq - 1);

  bf16x8_t qf[HD / 16];
  {
    const bf16_t* qp = Q + (row0 + i_ld) * q_ld + (int64_t)h * HD + 8 * g;
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) qf[s] = *(const bf16x8_t*)(qp + 16 * s);
  }

  f32x16_t oacc[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // stage one 32-key tile of K (row-major, swizzled) and V (transposed) in LDS.
  // Rows whose `ok` test fails are zero-filled and never read from memory.
  auto stage = [&](const bf16_t* kbase, const bf16_t* vbase, int64_t ld, auto row_ok) {
    // K: 1024 16-byte chunks, 4 per thread
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int c = tid + 256 * pass;
      const int key = c >> 5, dc = c & 31;
      u32x4_t v = {0, 0, 0, 0};
      if (row_ok(key)) v = *(const u32x4_t*)(kbase + key * ld + dc * 8);
      *(u32x4_t*)(k_lds + key * HD + ((dc ^ k_swz(key)) << 3)) = v;
    }
    // V: thread holds 4 consecutive keys x 8 dims, writes 8 dims x 4 keys
    const int kg = tid & 7, dc = tid >> 3;
    u32x4_t vr[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int key = 4 * kg + pp;
      vr[pp] = u32x4_t{0, 0, 0, 0};
      if (row_ok(key)) vr[pp] = *(const u32x4_t*)(vbase + key * ld + dc * 8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t a0 = (vr[0][e >> 1] >> sh) & 0xffffu, a1 = (vr[1][e >> 1] >> sh) & 0xffffu;
      const uint32_t a2 = (vr[2][e >> 1] >> sh) & 0xffffu, a3 = (vr[3][e >> 1] >> sh) & 0xffffu;
      *(u32x2_t*)(vt_lds + (dc * 8 + e) * VT_LD + 4 * kg) = u32x2_t{a0 | (a1 << 16), a2 | (a3 << 16)};
    }
  };

  // consume the staged tile: kbase = index of the tile's first key
  auto consume = [&](int kbase, bool is_self) {
    f32x16_t sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
    const int krow = (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1);  // swap bits 2 and 3
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      const int kc = 2 * s + g;
      const bf16x8_t kf = *(const bf16x8_t*)(k_lds + krow * HD + ((kc ^ k_swz(krow)) << 3));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kk = key_of_slot(v, g);
      const bool ok = is_self ? (kbase + kk <= i_loc) && (kbase + kk < Lq) : (cm_lds[kk] != 0);
      const float s = ok ? sacc[v] * scale_log2 : -INFINITY;
      sacc[v] = s;
      tmax = fmaxf(tmax, s);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool need = tmax > m_run + LAZY;
    if (__ballot(need)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < HD / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
    }
    bf16x8_t pf0, pf1;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pv = (sacc[v] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sacc[v] - m_run);
      l_run += pv;
      if (v < 8) pf0[v] = to_bf16(pv);
      else pf1[v - 8] = to_bf16(pv);
    }
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
      const bf16_t* vrow = vt_lds + (db * 32 + r) * VT_LD + 8 * g;
      const bf16x8_t vf0 = *(const bf16x8_t*)(vrow);
      const bf16x8_t vf1 = *(const bf16x8_t*)(vrow + 16);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf0, pf0, oacc[db], 0, 0, 0);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf1, pf1, oacc[db], 0, 0, 0);
    }
  };

  // ---- self keys: causal, the block needs keys [0, min(Lq, last row + 1))
  const int n_self = min(Lq, qb * RB + RB);
  const bf16_t* ks_base = Ks + row0 * kv_ld + (int64_t)kvh * HD;
  const bf16_t* vs_base = Vs + row0 * kv_ld + (int64_t)kvh * HD;
  for (int kb = 0; kb < n_self; kb += BKV) {
    __syncthreads();  // previous tile consumed
    stage(ks_base + (int64_t)kb * kv_ld, vs_base + (int64_t)kb * kv_ld, kv_ld,
          [&](int key) { return kb + key < Lq; });
    __syncthreads();
    if (kb <= wave_last) consume(kb, true);
  }

  // ---- cross keys: the pooled passage chunks with chunk_mask = 1
  if (!bad_doc) {
    const uint8_t* cmd = cmask + (int64_t)doc * Cmax;
    const bf16_t* kc_base = Kc + (int64_t)doc * Cmax * c_ld + (int64_t)kvh * HD;
    const bf16_t* vc_base = Vc + (int64_t)doc * Cmax * c_ld + (int64_t)kvh * HD;
    for (int cb = 0; cb < Cmax; cb += BKV) {
      int mine = 0;
      if (tid < BKV) {
        mine = (cb + tid < Cmax) ? (cmd[cb + tid] != 0) : 0;
      }
      __syncthreads();  // previous tile consumed before cm_lds is overwritten
      if (tid < BKV) cm_lds[tid] = (uint8_t)mine;
      if (!__syncthreads_or(mine)) continue;  // no valid chunk in this tile
      stage(kc_base + (int64_t)cb * c_ld, vc_base + (int64_t)cb * c_ld, c_ld,
            [&](int key) { return cm_lds[key] != 0; });
      __syncthreads();
      consume(cb, false);
    }
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
