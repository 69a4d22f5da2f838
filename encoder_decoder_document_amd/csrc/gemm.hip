// a2 / a5 -- bf16 MFMA GEMM  Y[M,N] = X[M,K] . W[N,K]^T  (fp32 accumulation).
//
// Serves the cross K/V projection of the pooled passage vectors ("KaLM-Reranker
// -V1-Nano -- MLX (Apple Silicon)", What this is) and the linear layers of the
// decoder-stack glue.  Both operands are K-contiguous ([rows, K]), which is the
// layout the gfx950 v_mfma_f32_32x32x16_bf16 fragments want: every lane reads 8
// consecutive k values of one row.
//
// Block tile BM x BN x 64 with 256 threads (4 waves), each wave a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 MFMA blocks.  The MFMA "A"
// operand is the weight tile and the "B" operand the activation tile, so each
// lane's accumulator holds 4 consecutive output columns of one output row and
// the epilogue writes 8-byte (bf16) or 16-byte (fp32) vectors.  Global tiles
// are register-staged and double-buffered in LDS; 16-byte k-chunks are stored
// XOR-swizzled by (row & 7) so the fragment reads of 32 consecutive rows are
// bank-conflict free.  Workgroups are remapped so that each XCD walks a
// contiguous range of output tiles (the tiles sharing activation rows stay in
// one L2).
#include "kalm_common.h"

namespace {

enum Epi { EPI_BF16 = 0, EPI_F32 = 1, EPI_F32_ACC = 2 };

constexpr int BK = 64;

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, int M, int K, int N,
    void* __restrict__ Y, int epi, bf16_t* __restrict__ Ybf, const uint8_t* __restrict__ rmask) {
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int LA = BM / 32, LB = BN / 32;  // 16-byte loads per thread per k-tile

  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * BK];
  bf16_t* As = smem;                 // [2][BM][BK]
  bf16_t* Bs = smem + 2 * BM * BK;   // [2][BN][BK]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a
  // contiguous run of tiles, output columns fastest.
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = (M + BM - 1) / BM;
  const int total = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int per = total / 8;
  const int t = (b < per * 8) ? (b % 8) * per + (b / 8) : b;
  const int tm = t / tiles_n, tn = t % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  // skip tiles whose rows are all masked out (padded chunks of the cross projection)
  bool tile_live = true;
  if (rmask) {
    int any = 0;
    for (int rr = tid; rr < BM; rr += 256)
      if (m0 + rr < M && rmask[m0 + rr]) any = 1;
    tile_live = __syncthreads_or(any) != 0;
  }

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int lrow = tid >> 3, lkc = tid & 7;  // staging: row within 32-row slab, 16B k-chunk
  u32x4_t ra[LA], rb[LB];
  auto gload = [&](int k0) {
    const int kk = k0 + lkc * 8;
    const bool kin = kk < K;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int gm = min(m0 + lrow + 32 * i, M - 1);
      ra[i] = kin ? *(const u32x4_t*)(X + (int64_t)gm * K + kk) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int gn = min(n0 + lrow + 32 * i, N - 1);
      rb[i] = kin ? *(const u32x4_t*)(W + (int64_t)gn * K + kk) : u32x4_t{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
    bf16_t* a = As + buf * BM * BK;
    bf16_t* bb = Bs + buf * BN * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = lrow + 32 * i;
      *(u32x4_t*)(a + row * BK + ((lkc ^ (row & 7)) << 3)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int row = lrow + 32 * i;
      *(u32x4_t*)(bb + row * BK + ((lkc ^ (row & 7)) << 3)) = rb[i];
    }
  };

  const int nk = tile_live ? (K + BK - 1) / BK : 0;
  const int r = lane & 31, g = lane >> 5;
  if (nk > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const bf16_t* a = As + cur * BM * BK;
    const bf16_t* bb = Bs + cur * BN * BK;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int kc = 2 * s + g;
      bf16x8_t xf[FM], wf[FN];
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = wm * WTM + j * 32 + r;
        xf[j] = *(const bf16x8_t*)(a + row * BK + ((kc ^ (row & 7)) << 3));
      }
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int row = wn * WTN + i * 32 + r;
        wf[i] = *(const bf16x8_t*)(bb + row * BK + ((kc ^ (row & 7)) << 3));
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds Y[m][n .. n+3] for m = .. + (lane & 31), n = .. + 8*q + 4*g
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = m0 + wm * WTM + j * 32 + r;
    if (m >= M) continue;
    const bool row_ok = rmask ? rmask[m] != 0 : true;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WTN + i * 32 + 8 * q + 4 * g;
        if (n >= N) continue;
        float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
        float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (!row_ok) v0 = v1 = v2 = v3 = 0.f;
        const int64_t off = (int64_t)m * N + n;
        if (epi == EPI_BF16) {
          u32x2_t o;
          o[0] = pack_bf16x2(v0, v1);
          o[1] = pack_bf16x2(v2, v3);
          *(u32x2_t*)((bf16_t*)Y + off) = o;
        } else {
          float* yp = (float*)Y + off;
          if (epi == EPI_F32_ACC) {
            const f32x4_t old = *(const f32x4_t*)yp;
            v0 += old[0];
            v1 += old[1];
            v2 += old[2];
            v3 += old[3];
          }
          *(f32x4_t*)yp = f32x4_t{v0, v1, v2, v3};
          if (Ybf) {
            u32x2_t o;
            o[0] = pack_bf16x2(v0, v1);
            o[1] = pack_bf16x2(v2, v3);
            *(u32x2_t*)(Ybf + off) = o;
          }
        }
      }
    }
  }
}

// fp32 path (the small fp32 sanity workload): 64x64 tiles, 4x4 outputs per thread.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W, int M, int K,
                                                       int N, float* __restrict__ Y, int accumulate,
                                                       const uint8_t* __restrict__ rmask) {
  __shared__ float Xs[16][64 + 1];
  __shared__ float Ws[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int rr = e >> 4, kk = e & 15;
      const int gm = m0 + rr, gn = n0 + rr, gk = k0 + kk;
      Xs[kk][rr] = (gm < M && gk < K) ? X[(int64_t)gm * K + gk] : 0.f;
      Ws[kk][rr] = (gn < N && gk < K) ? W[(int64_t)gn * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float xv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = Xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = Ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    const bool row_ok = rmask ? rmask[m] != 0 : true;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = row_ok ? acc[i][j] : 0.f;
      float* yp = Y + (int64_t)m * N + n;
      if (accumulate) v += *yp;
      *yp = v;
    }
  }
}

}  // namespace

namespace kalm {

void launch_linear_bf16(const bf16_t* X, const bf16_t* W, int M, int K, int N, void* Y, bool y_f32,
                        bool accumulate, bf16_t* Y_bf16, const uint8_t* rmask, hipStream_t s) {
  const int epi = !y_f32 ? EPI_BF16 : (accumulate ? EPI_F32_ACC : EPI_F32);
  constexpr int BM = 256, BN = 256;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 2, 2>), dim3(tiles), dim3(256), 0, s, X, W, M, K, N, Y,
                     epi, Y_bf16, rmask);
}

void launch_linear_f32(const float* X, const float* W, int M, int K, int N, float* Y, bool accumulate,
                       const uint8_t* rmask, hipStream_t s) {
  const dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, X, W, M, K, N, Y, accumulate ? 1 : 0, rmask);
}

}  // namespace kalm
