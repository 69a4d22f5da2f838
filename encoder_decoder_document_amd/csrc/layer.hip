// Decoder-layer completion around the merged attention: RMSNorm, rotary
// position embedding and the gated-GELU activation of a gated MLP.
//
// The pages say the forward pass reads every dim, head count, layer count and
// RoPE parameter from the model's config and that the RoPE inverse-frequency
// tables are computed from it ("KaLM-Reranker-V1-Nano -- MLX (Apple
// Silicon)", What this is / Derivation); they give no other layer internals.
// These kernels implement the standard forms (the readings are stated with
// each); all three are elementwise or row-wise and bound by HBM bandwidth.
#include <math.h>

#include "kalm_common.h"

namespace {

// Four consecutive elements as floats / from floats (16-byte or 8-byte accesses).
template <typename T>
__device__ __forceinline__ f32x4_t ld4(const T* p);
template <>
__device__ __forceinline__ f32x4_t ld4<float>(const float* p) { return *(const f32x4_t*)p; }
template <>
__device__ __forceinline__ f32x4_t ld4<bf16_t>(const bf16_t* p) {
  const u32x2_t w = *(const u32x2_t*)p;
  return f32x4_t{bf16lo(w[0]), bf16hi(w[0]), bf16lo(w[1]), bf16hi(w[1])};
}
template <typename T>
__device__ __forceinline__ void st4(T* p, f32x4_t v);
template <>
__device__ __forceinline__ void st4<float>(float* p, f32x4_t v) { *(f32x4_t*)p = v; }
template <>
__device__ __forceinline__ void st4<bf16_t>(bf16_t* p, f32x4_t v) {
  *(u32x2_t*)p = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// RMSNorm, one wave per row: y = x / sqrt(mean(x^2) + eps) * w (fp32 sum of
// squares, one IEEE square root and division, one rounding to the output).
template <typename XT, typename WT, typename YT>
__global__ __launch_bounds__(256) void rms_norm_kernel(const XT* __restrict__ x, int64_t x_ld, int64_t M, int H,
                                                       const WT* __restrict__ w, float eps, YT* __restrict__ y,
                                                       int64_t y_ld) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const XT* xr = x + row * x_ld;
  float ss = 0.f;
  for (int c = 4 * lane; c < H; c += 256) {
    const f32x4_t v = ld4(xr + c);
    ss = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], ss))));
  }
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)H + eps);
  YT* yr = y + row * y_ld;
  for (int c = 4 * lane; c < H; c += 256) {
    const f32x4_t v = ld4(xr + c);
    const f32x4_t g = ld4(w + c);
    st4(yr + c, f32x4_t{v[0] * inv * g[0], v[1] * inv * g[1], v[2] * inv * g[2], v[3] * inv * g[3]});
  }
}

// Rotary embedding in place, "rotate half" pairing: for head dims i < d/2,
// (x_i, x_{i+d/2}) at position t turns by the angle t * theta^(-2i/d).
// Row mode 0: the rows of sequence s are cu[s] .. cu[s+1]-1 at positions
// 0, 1, ...; row mode 1: one row per sequence, row s, at position
// cu[s+1]-cu[s]-1 (its final position).  Each thread turns 4 dim pairs of one
// head of one row; blockIdx.x is the sequence, blockIdx.y a chunk of its rows.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ X, int64_t ld, int64_t rows, int col0, int nh,
                                                   int d, const int32_t* __restrict__ cu, int mode,
                                                   float log2_theta) {
  const int s = blockIdx.x;
  const int64_t c0 = cu[s];
  const int len = (int)((int64_t)cu[s + 1] - c0);
  const int per_row = nh * (d / 8);  // threads per row: 4 pairs each
  const int64_t t = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  const int64_t r = t / per_row;  // row within the sequence
  const int rem = (int)(t % per_row);
  const int head = rem / (d / 8), i0 = 4 * (rem % (d / 8));
  int64_t row;
  int pos;
  if (mode == 0) {
    if (r >= len) return;
    row = c0 + r;
    pos = (int)r;
  } else {
    if (r >= 1 || len <= 0) return;
    row = s;
    pos = len - 1;
  }
  if (row < 0 || row >= rows) {
    KALM_DBG(KALM_DBG_ROPE_ROW);
    return;
  }
  T* base = X + row * ld + col0 + (int64_t)head * d;
  const f32x4_t a = ld4(base + i0), b = ld4(base + i0 + d / 2);
  f32x4_t oa, ob;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float inv_freq = exp2f(-(float)(2 * (i0 + k)) / (float)d * log2_theta);
    float sn, cs;
    sincosf((float)pos * inv_freq, &sn, &cs);
    oa[k] = a[k] * cs - b[k] * sn;
    ob[k] = b[k] * cs + a[k] * sn;
  }
  st4(base + i0, oa);
  st4(base + i0 + d / 2, ob);
}

// Gated GELU: A[m, j] = gelu(Y[m, j]) * Y[m, I + j], gelu in its tanh form
// 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); four columns per thread.
template <typename T>
__global__ __launch_bounds__(256) void gated_gelu_kernel(const T* __restrict__ Y, int64_t y_ld, int64_t M, int I,
                                                         T* __restrict__ A, int64_t a_ld) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = I / 4;
  const int64_t m = t / per_row;
  if (m >= M) return;
  const int j = 4 * (int)(t % per_row);
  const f32x4_t g = ld4(Y + m * y_ld + j), u = ld4(Y + m * y_ld + I + j);
  f32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = gated_gelu_tanh(g[k], u[k]);
  }
  st4(A + m * a_ld + j, o);
}

}  // namespace

KALM_DBG_TAKE_DEFINE(dbg_take_layer)

namespace kalm {

void launch_rms_norm(const void* x, bool x_bf16, int64_t x_ld, int64_t M, int H, const void* w, bool w_bf16, float eps,
                     void* y, bool y_bf16, int64_t y_ld, hipStream_t s) {
  if (M == 0) return;
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
#define KALM_RMS(XT, WT, YT)                                                                                      \
  hipLaunchKernelGGL((rms_norm_kernel<XT, WT, YT>), grid, block, 0, s, (const XT*)x, x_ld, M, H, (const WT*)w, eps, \
                     (YT*)y, y_ld)
  if (!x_bf16 && !w_bf16 && !y_bf16) KALM_RMS(float, float, float);
  else if (!x_bf16 && !w_bf16 && y_bf16) KALM_RMS(float, float, bf16_t);
  else if (!x_bf16 && w_bf16 && !y_bf16) KALM_RMS(float, bf16_t, float);
  else if (!x_bf16 && w_bf16 && y_bf16) KALM_RMS(float, bf16_t, bf16_t);
  else if (x_bf16 && !w_bf16 && !y_bf16) KALM_RMS(bf16_t, float, float);
  else if (x_bf16 && !w_bf16 && y_bf16) KALM_RMS(bf16_t, float, bf16_t);
  else if (x_bf16 && w_bf16 && !y_bf16) KALM_RMS(bf16_t, bf16_t, float);
  else KALM_RMS(bf16_t, bf16_t, bf16_t);
#undef KALM_RMS
}

void launch_rope(void* X, bool bf16, int64_t ld, int64_t rows, int col0, int nh, int d, const int32_t* cu, int n_seq,
                 int max_len, int mode, float theta, hipStream_t s) {
  if (n_seq == 0 || nh == 0) return;
  const int64_t threads = (int64_t)(mode == 0 ? max_len : 1) * nh * (d / 8);
  if (threads == 0) return;
  const dim3 grid((unsigned)n_seq, (unsigned)((threads + 255) / 256)), block(256);
  const float l2t = log2f(theta);
  if (bf16)
    hipLaunchKernelGGL(rope_kernel<bf16_t>, grid, block, 0, s, (bf16_t*)X, ld, rows, col0, nh, d, cu, mode, l2t);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, block, 0, s, (float*)X, ld, rows, col0, nh, d, cu, mode, l2t);
}

void launch_gated_gelu(const void* Y, bool bf16, int64_t y_ld, int64_t M, int I, void* A, int64_t a_ld,
                       hipStream_t s) {
  const int64_t threads = M * (I / 4);
  if (threads == 0) return;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (bf16)
    hipLaunchKernelGGL(gated_gelu_kernel<bf16_t>, grid, block, 0, s, (const bf16_t*)Y, y_ld, M, I, (bf16_t*)A, a_ld);
  else
    hipLaunchKernelGGL(gated_gelu_kernel<float>, grid, block, 0, s, (const float*)Y, y_ld, M, I, (float*)A, a_ld);
}

}  // namespace kalm
