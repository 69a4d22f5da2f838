// a3 -- merged self + cross attention: the fp32 kernel and the launchers.
// The bf16 kernel lives in attn_bf16.h; it is instantiated here with one row
// tile of 32 decoder rows per wave (MFMA accumulators in VGPRs).  Two row
// tiles per wave (256 query vectors per K/V tile, accumulators in AGPRs) did
// not fit the 512 registers of a lane without spilling.
#include "attn_bf16.h"

namespace {

// fp32 path (the small fp32 workload): one wavefront per (pair, head, row),
// lanes split the head dim, one online-softmax state per row walking the
// causal self keys and then the valid cross keys.  part 1 walks the self keys
// only (a self partial); part 2 walks the cross keys only, starting from the
// self partial (oi, lsei) of the Q row: m = lse, l = 1, acc = o.
__global__ __launch_bounds__(256) void merged_attn_f32_kernel(
    const float* __restrict__ Q, int64_t q_ld, const float* __restrict__ Ks,
    const float* __restrict__ Vs, int64_t kv_ld, const int32_t* __restrict__ cu_q, int64_t q_rows,
    int64_t kv_rows, int64_t o_rows, int mode, const float* __restrict__ Kc, const float* __restrict__ Vc, int64_t c_ld,
    const uint8_t* __restrict__ cmask, const int32_t* __restrict__ doc_of_pair, int D, int Cmax,
    int nq, int nkv, int d, float scale, float* __restrict__ O, int64_t o_ld,
    float* __restrict__ lse, int nrb, int part, const float* __restrict__ oi, int64_t oi_ld,
    const float* __restrict__ lsei) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = blockIdx.x;
  const int i = (int)(blk % nrb) * 4 + (threadIdx.x >> 6);
  const int h = (int)((blk / nrb) % nq);
  const int p = (int)(blk / ((int64_t)nrb * nq));
  const PairRows pr = pair_rows(cu_q, p, D, mode, q_rows, kv_rows, o_rows);
  if (!pr.ok) {
    if (lane == 0) KALM_DBG(KALM_DBG_PAIR_ROWS);
    return;
  }
  if (i >= pr.nrow) return;
  const int pos = pr.pos0 + i;  // self position of this query row
  const int kvh = h / (nq / nkv);
  const int doc = part == 1 ? 0 : doc_of_pair[p];
  const bool bad_doc = part != 1 && (doc < 0 || doc >= D);
  if (bad_doc && lane == 0) KALM_DBG(KALM_DBG_DOC);
  constexpr int MAXJ = 4;  // d <= 256
  const int nj = (d + 63) / 64;
  float q[MAXJ], acc[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int e = lane + 64 * j;
    q[j] = (j < nj && e < d) ? Q[(pr.q0 + i) * q_ld + (int64_t)h * d + e] : 0.f;
    acc[j] = (part == 2 && j < nj && e < d) ? oi[(pr.q0 + i) * oi_ld + (int64_t)h * d + e] : 0.f;
  }
  float m = -INFINITY, l = 0.f;
  if (part == 2) {
    m = lsei[(pr.q0 + i) * nq + h];
    l = 1.f;
  }
  auto visit = [&](const float* krow, const float* vrow) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int e = lane + 64 * j;
      if (j < nj && e < d) part = fmaf(q[j], krow[e], part);
    }
    const float s = wave_sum(part) * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);  // expf(-inf) = 0 on the first key
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
  if (part != 2)
    for (int jk = 0; jk <= pos; ++jk)
      visit(Ks + (pr.kv0 + jk) * kv_ld + (int64_t)kvh * d, Vs + (pr.kv0 + jk) * kv_ld + (int64_t)kvh * d);
  if (part != 1 && !bad_doc)
    for (int c = 0; c < Cmax; ++c)
      if (cmask[(int64_t)doc * Cmax + c])
        visit(Kc + ((int64_t)doc * Cmax + c) * c_ld + (int64_t)kvh * d,
              Vc + ((int64_t)doc * Cmax + c) * c_ld + (int64_t)kvh * d);
  const float inv = bad_doc ? __builtin_nanf("") : 1.f / l;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int e = lane + 64 * j;
    if (j < nj && e < d) O[(pr.o0 + i) * o_ld + (int64_t)h * d + e] = acc[j] * inv;
  }
  if (lse && lane == 0) lse[(pr.o0 + i) * nq + h] = bad_doc ? __builtin_nanf("") : m + logf(l);
}

// Log-sum-exp merge of split-KV shares: the self partial (oi, lsei at the Q
// row) and n_split partials over disjoint shares of the cross keys (slices of
// ws_o / ws_l at the O row) combine into the softmax over all of them:
//   M = max lse_i,  w_i = e^(lse_i - M),  O = sum w_i o_i / sum w_i,
//   lse = M + log sum w_i.
// One block per (pair, query head); wave w takes rows w, w + 4, ...; each
// lane four of the 256 dims.
__global__ __launch_bounds__(256) void split_merge_kernel(
    const int32_t* __restrict__ cu_q, int D, int mode, int64_t q_rows, int64_t o_rows,
    const float* __restrict__ oi, int64_t oi_ld, const float* __restrict__ lsei, const float* __restrict__ ws_o,
    const float* __restrict__ ws_l, int S, int nq, bf16_t* __restrict__ O, int64_t o_ld,
    float* __restrict__ lse) {
  const int p = blockIdx.x, h = blockIdx.y;
  const PairRows pr = pair_rows(cu_q, p, D, mode, q_rows, INT64_MAX, o_rows);
  if (!pr.ok) {
    if (threadIdx.x == 0) KALM_DBG(KALM_DBG_PAIR_ROWS);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t dim0 = (int64_t)h * HD + 4 * lane;
  for (int i = wave; i < pr.nrow; i += 4) {
    const int64_t qrow = pr.q0 + i, orow = pr.o0 + i;
    const float ls = lsei[qrow * nq + h];
    float M = ls;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ws_l[((int64_t)s * o_rows + orow) * nq + h]);
    float w = expf(ls - M), sum = w;
    const f32x4_t os = *(const f32x4_t*)(oi + qrow * oi_ld + dim0);
    f32x4_t acc = os * w;
    for (int s = 0; s < S; ++s) {
      const float wl = expf(ws_l[((int64_t)s * o_rows + orow) * nq + h] - M);  // e^-inf = 0: empty share
      sum += wl;
      if (wl != 0.f) acc += *(const f32x4_t*)(ws_o + ((int64_t)s * o_rows + orow) * nq * HD + dim0) * wl;
    }
    const float inv = 1.f / sum;
    u32x2_t o;
    o[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    o[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *(u32x2_t*)(O + orow * o_ld + dim0) = o;
    if (lse && lane == 0) lse[orow * nq + h] = M + logf(sum);
  }
}

}  // namespace

KALM_DBG_TAKE_DEFINE(dbg_take_attn)

namespace kalm {

void launch_merged_attn_bf16(const bf16_t* Q, int64_t q_ld, const bf16_t* Ks, const bf16_t* Vs,
                             int64_t kv_ld, const int32_t* cu_q, int P, int64_t q_rows, int64_t kv_rows,
                             int64_t o_rows, int mode, int max_lq, const bf16_t* Kc, const bf16_t* Vc,
                             int64_t c_ld, const uint8_t* cmask, const int32_t* doc_of_pair, int D, int Cmax,
                             int nq, int nkv, float scale, void* O, int64_t o_ld, float* lse, int part,
                             const float* oi, int64_t oi_ld, const float* lsei, hipStream_t s) {
  launch_bf16<ATTN_WAVES, 1>(Q, q_ld, Ks, Vs, kv_ld, cu_q, P, q_rows, kv_rows, o_rows, mode, max_lq, Kc, Vc, c_ld,
                             cmask, doc_of_pair, D, Cmax, nq, nkv, scale, O, o_ld, lse, part, oi, oi_ld, lsei, 1, s);
}

void launch_merged_attn_split(const bf16_t* Q, int64_t q_ld, const int32_t* cu_q, int P, int64_t q_rows,
                              int64_t o_rows, int mode, int max_lq, const bf16_t* Kc, const bf16_t* Vc, int64_t c_ld,
                              const uint8_t* cmask, const int32_t* doc_of_pair, int D, int Cmax, int nq, int nkv,
                              float scale, const float* oi, int64_t oi_ld, const float* lsei, int n_split,
                              float* ws, bf16_t* O, int64_t o_ld, float* lse, hipStream_t s) {
  float* ws_o = ws;
  float* ws_l = ws + (int64_t)n_split * o_rows * nq * HD;
  launch_bf16<ATTN_WAVES, 1>(Q, q_ld, nullptr, nullptr, 0, cu_q, P, q_rows, INT64_MAX, o_rows, mode, max_lq, Kc, Vc,
                             c_ld, cmask, doc_of_pair, D, Cmax, nq, nkv, scale, ws_o, (int64_t)nq * HD, ws_l, 3,
                             nullptr, 0, nullptr, n_split, s);
  if (P == 0) return;
  hipLaunchKernelGGL(split_merge_kernel, dim3((unsigned)P, (unsigned)nq), dim3(256), 0, s, cu_q, D, mode, q_rows,
                     o_rows, oi, oi_ld, lsei, ws_o, ws_l, n_split, nq, O, o_ld, lse);
}

void launch_merged_attn_f32(const float* Q, int64_t q_ld, const float* Ks, const float* Vs,
                            int64_t kv_ld, const int32_t* cu_q, int P, int64_t q_rows, int64_t kv_rows,
                            int64_t o_rows, int mode, int max_lq, const float* Kc, const float* Vc, int64_t c_ld,
                            const uint8_t* cmask, const int32_t* doc_of_pair, int D, int Cmax, int nq, int nkv,
                            int d, float scale, float* O, int64_t o_ld, float* lse, int part, const float* oi,
                            int64_t oi_ld, const float* lsei, hipStream_t s) {
  const int max_rows = (mode == 1 || mode == 3) ? 1 : max_lq;
  if (P == 0 || max_rows == 0) return;
  const int nrb = (max_rows + 3) / 4;  // 4 rows (one per wave) per block
  const dim3 grid((unsigned)((int64_t)nrb * nq * P)), block(256);
  hipLaunchKernelGGL(merged_attn_f32_kernel, grid, block, 0, s, Q, q_ld, Ks, Vs, kv_ld, cu_q, q_rows, kv_rows,
                     o_rows, mode, Kc, Vc, c_ld, cmask, doc_of_pair, D, Cmax, nq, nkv, d, scale, O, o_ld, lse, nrb, part,
                     oi, oi_ld, lsei);
}

}  // namespace kalm
