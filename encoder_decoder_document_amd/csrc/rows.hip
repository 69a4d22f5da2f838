// a0 -- ragged pair layout, a4 -- yes/no readout, a5 -- residual-stream start,
// and the ranking of each query's passages by score.
//
// Pair layout: every query reranks the same set of passages ("KaLM-Reranker-V1
// -Nano -- MLX (Apple Silicon)", Speed), so pair p = (query p / D, doc p % D)
// and all D pairs of a query have its length; their decoder rows are packed
// back to back.  Yes/no readout: score = softmax([yes, no])[yes] =
// sigmoid(yes - no) at the final position (same page, What this is;
// "KaLM-Reranker-V1-Small Q4_K_M GGUF", Score a pair).
#include "kalm_common.h"

namespace {

// One block.  Running exclusive prefix over the query lengths, 1024 queries
// per step; the step's starts and lengths go to LDS and all threads then write
// the entries of its queries' pairs (pair-major, so consecutive threads write
// consecutive entries).  The
// prefix is taken in int64: a pair whose rows would end past INT32_MAX gets
// cu_q = final_row = h0_final = -1 (and cu_q[P] = -1 when the total overflows),
// which the attention kernels skip and the readout turns into NaN, so an
// oversized batch can never wrap row offsets into valid-looking rows.
__global__ __launch_bounds__(1024) void pair_layout_kernel(const int32_t* __restrict__ lq, int nQ,
                                                           int nD, int32_t* __restrict__ cu_q,
                                                           int32_t* __restrict__ doc_of_pair,
                                                           int32_t* __restrict__ final_row,
                                                           int32_t* __restrict__ h0_final,
                                                           int32_t* __restrict__ cu_u) {
  constexpr int64_t LIM = 0x7fffffffLL;
  __shared__ int64_t scan[1024];
  __shared__ int64_t qstart[1024], qlen[1024];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nQ; base += 1024) {
    const int q = base + threadIdx.x;
    const int64_t len = q < nQ ? (int64_t)lq[q] : 0;
    scan[threadIdx.x] = len;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
      const int64_t v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    const int64_t start = carry + scan[threadIdx.x] - len;  // exclusive prefix of query rows
    qstart[threadIdx.x] = start;
    qlen[threadIdx.x] = len;
    if (q < nQ && cu_u) cu_u[q] = start + len <= LIM ? (int32_t)start : -1;
    __syncthreads();
    // the entries of this step's pairs: pair p = q nD + dd, in pair order
    // (32-bit: the host keeps nQ nD below 2^31)
    const int nq_step = min(1024, nQ - base);
    const uint32_t n_ent = (uint32_t)nq_step * (uint32_t)nD;
    for (uint32_t e = threadIdx.x; e < n_ent; e += 1024) {
      const int ql = (int)(e / (uint32_t)nD), dd = (int)(e - (uint32_t)ql * (uint32_t)nD);
      const int64_t st = qstart[ql], ln = qlen[ql];
      const int64_t p = (int64_t)base * nD + e;
      const int64_t r0 = (int64_t)nD * st + (int64_t)dd * ln;
      const bool ok = r0 + ln <= LIM;
      if (!ok) KALM_DBG(KALM_DBG_LAYOUT);
      cu_q[p] = ok ? (int32_t)r0 : -1;
      doc_of_pair[p] = dd;
      final_row[p] = ok ? (int32_t)(r0 + ln - 1) : -1;
      if (h0_final) h0_final[p] = ok ? (int32_t)(st + ln - 1) : -1;
    }
    __syncthreads();
    if (threadIdx.x == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int64_t total = (int64_t)nD * carry;
    cu_q[(int64_t)nQ * nD] = total <= LIM ? (int32_t)total : -1;
    if (cu_u) cu_u[nQ] = carry <= LIM ? (int32_t)carry : -1;
  }
}

// One block per pair: h0_row[cu_q[p] + r] = (first row of the pair's query) + r.
__global__ __launch_bounds__(256) void h0_row_kernel(const int32_t* __restrict__ cu_q, int nD,
                                                     int32_t* __restrict__ h0_row, int64_t rows) {
  const int64_t p = blockIdx.x;
  const int64_t q = p / nD;
  const int32_t base = cu_q[p];
  const int32_t n = cu_q[p + 1] - base;
  const int32_t qstart = cu_q[q * nD] / nD;
  if (base < 0) return;
  for (int r = threadIdx.x; r < n; r += blockDim.x)
    if ((int64_t)base + r < rows) h0_row[base + r] = qstart + r;
}

template <bool HB, bool WB>
__global__ __launch_bounds__(256) void yesno_kernel(const void* __restrict__ h, int64_t h_ld,
                                                    int64_t rows, const int32_t* __restrict__ final_row,
                                                    int P, int H, const void* __restrict__ w,
                                                    float* __restrict__ yes, float* __restrict__ no,
                                                    float* __restrict__ margin,
                                                    float* __restrict__ score) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= P) return;
  const int64_t row = final_row[p];
  const bool ok = row >= 0 && row < rows;
  float sy = 0.f, sn = 0.f;
  for (int i = lane; ok && i < H; i += 64) {
    const float hv = HB ? from_bf16(((const bf16_t*)h)[row * h_ld + i]) : ((const float*)h)[row * h_ld + i];
    const float wy = WB ? from_bf16(((const bf16_t*)w)[i]) : ((const float*)w)[i];
    const float wn = WB ? from_bf16(((const bf16_t*)w)[H + i]) : ((const float*)w)[H + i];
    sy = fmaf(hv, wy, sy);
    sn = fmaf(hv, wn, sn);
  }
  sy = wave_sum(sy);
  sn = wave_sum(sn);
  if (!ok) sy = sn = __builtin_nanf("");
  if (!ok && lane == 0) KALM_DBG(KALM_DBG_FINAL_ROW);
  if (lane == 0) {
    const float m = sy - sn;
    const float e = expf(-fabsf(m));  // never overflows
    yes[p] = sy;
    no[p] = sn;
    if (margin) margin[p] = m;
    score[p] = m >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
  }
}

// One wavefront per destination row; 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const float* __restrict__ src,
                                                          const int32_t* __restrict__ idx, int64_t M,
                                                          int H, int64_t n_src,
                                                          float* __restrict__ dst,
                                                          bf16_t* __restrict__ dst_bf16) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int64_t s = idx[m];
  const bool ok = s >= 0 && s < n_src;
  if (!ok && lane == 0) KALM_DBG(KALM_DBG_GATHER);
  const float qnan = __builtin_nanf("");
  for (int h = lane * 4; h < H; h += 256) {
    f32x4_t v = ok ? *(const f32x4_t*)(src + s * H + h) : f32x4_t{qnan, qnan, qnan, qnan};
    *(f32x4_t*)(dst + m * H + h) = v;
    if (dst_bf16) {
      u32x2_t b;
      b[0] = pack_bf16x2(v[0], v[1]);
      b[1] = pack_bf16x2(v[2], v[3]);
      *(u32x2_t*)(dst_bf16 + m * H + h) = b;
    }
  }
}

// One workgroup per query: the rank of passage i is the number of passages
// that come before it in the order "higher score first, lower index first on
// equal scores, NaN scores last (by index)" -- a total order, so the ranks are
// a permutation and each passage writes itself to its rank if it is in the
// top n.  Scores are staged in LDS; D <= 4096.
constexpr int RANK_MAX_D = 4096;
__global__ __launch_bounds__(256) void rank_topn_kernel(const float* __restrict__ score, int D, int top_n,
                                                        int32_t* __restrict__ out_index,
                                                        float* __restrict__ out_score) {
  __shared__ float sc[RANK_MAX_D];
  const int64_t q = blockIdx.x;
  const float* s = score + q * D;
  for (int i = threadIdx.x; i < D; i += blockDim.x) sc[i] = s[i];
  __syncthreads();
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    const float si = sc[i];
    const bool ni = si != si;
    int rank = 0;
    for (int j = 0; j < D; ++j) {
      const float sj = sc[j];
      const bool nj = sj != sj;
      bool before;
      if (ni != nj) before = ni;                 // a number precedes every NaN
      else if (ni) before = j < i;               // NaNs by index
      else before = sj > si || (sj == si && j < i);
      rank += before ? 1 : 0;
    }
    if (rank < top_n) {
      out_index[q * top_n + rank] = i;
      out_score[q * top_n + rank] = si;
    }
  }
}

}  // namespace

KALM_DBG_TAKE_DEFINE(dbg_take_rows)

namespace kalm {

void launch_rank_topn(const float* score, int n_queries, int D, int top_n, int32_t* out_index, float* out_score,
                      hipStream_t s) {
  hipLaunchKernelGGL(rank_topn_kernel, dim3((unsigned)n_queries), dim3(256), 0, s, score, D, top_n, out_index,
                     out_score);
}


void launch_pair_layout(const int32_t* lq, int nQ, int nD, int32_t* cu_q, int32_t* doc_of_pair,
                        int32_t* final_row, int32_t* h0_row, int64_t rows, int32_t* h0_final, int32_t* cu_u,
                        hipStream_t s) {
  hipLaunchKernelGGL(pair_layout_kernel, dim3(1), dim3(1024), 0, s, lq, nQ, nD, cu_q, doc_of_pair, final_row,
                     h0_final, cu_u);
  if (h0_row && (int64_t)nQ * nD > 0)
    hipLaunchKernelGGL(h0_row_kernel, dim3((unsigned)((int64_t)nQ * nD)), dim3(256), 0, s, cu_q, nD, h0_row, rows);
}

void launch_yesno(const void* h, bool h_bf16, int64_t h_ld, int64_t rows, const int32_t* final_row, int P,
                  int H, const void* w, bool w_bf16, float* yes, float* no, float* margin, float* score,
                  hipStream_t s) {
  const dim3 grid((P + 3) / 4), block(256);
  if (h_bf16 && w_bf16)
    hipLaunchKernelGGL((yesno_kernel<true, true>), grid, block, 0, s, h, h_ld, rows, final_row, P, H, w, yes, no, margin, score);
  else if (h_bf16)
    hipLaunchKernelGGL((yesno_kernel<true, false>), grid, block, 0, s, h, h_ld, rows, final_row, P, H, w, yes, no, margin, score);
  else if (w_bf16)
    hipLaunchKernelGGL((yesno_kernel<false, true>), grid, block, 0, s, h, h_ld, rows, final_row, P, H, w, yes, no, margin, score);
  else
    hipLaunchKernelGGL((yesno_kernel<false, false>), grid, block, 0, s, h, h_ld, rows, final_row, P, H, w, yes, no, margin, score);
}

void launch_gather_rows(const float* src, const int32_t* idx, int64_t M, int H, int64_t n_src,
                        float* dst, bf16_t* dst_bf16, hipStream_t s) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, src, idx, M, H, n_src, dst, dst_bf16);
}

}  // namespace kalm
