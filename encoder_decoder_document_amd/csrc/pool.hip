// a1 -- chunk pooling of passage encoder states.
//
// Masked mean over consecutive groups of `chunk` tokens ("KaLM-Reranker-V1-Large
// Q8_0 GGUF", Frozen inference contract; "KaLM-Reranker-V1-Nano -- MLX (Apple
// Silicon)", What this is).  HBM-bound segmented reduction: one wavefront owns
// one output row (doc d, chunk c); the chunk's validity bits come from a wave
// ballot over the token mask, each lane streams 16-byte vectors of the chunk's
// valid token rows (masked tokens are never loaded, so NaN padding cannot
// leak), sums them in fp32, divides once by the valid count (IEEE division) and
// rounds once to the storage type.  Non-temporal loads and stores: every token
// row is read once and every pooled row written once.  The chunk-0 wave of each doc also counts
// the doc's valid chunks, so no atomics and no second pass are needed.
#include "kalm_common.h"

namespace {

template <bool BF16>
struct PoolVec;

template <>
struct PoolVec<true> {  // 8 bf16 per 16-byte vector
  static constexpr int N = 8;
  __device__ static void add(float* acc, const u32x4_t& r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16lo(r[i]);
      acc[2 * i + 1] += bf16hi(r[i]);
    }
  }
  __device__ static u32x4_t pack(const float* v) {
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    return o;
  }
};

template <>
struct PoolVec<false> {  // 4 fp32 per 16-byte vector
  static constexpr int N = 4;
  __device__ static void add(float* acc, const u32x4_t& r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = r[i];  // copy out first: bit-casting a vector-element lvalue reads element 0
      acc[i] += __builtin_bit_cast(float, u);
    }
  }
  __device__ static u32x4_t pack(const float* v) {
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_bit_cast(uint32_t, v[i]);
    return o;
  }
};

// CH > 0: compile-time chunk size (all loads of a vector issued together);
// CH == 0: any chunk size up to 64, valid tokens visited one by one.
template <bool BF16, int CH>
__global__ __launch_bounds__(256) void chunk_pool_kernel(const uint8_t* __restrict__ x,
                                                         const uint8_t* __restrict__ mask, int D,
                                                         int T, int H, int chunk, int Cmax,
                                                         uint8_t* __restrict__ pooled,
                                                         uint8_t* __restrict__ cmask,
                                                         int32_t* __restrict__ n_chunks) {
  using V = PoolVec<BF16>;
  constexpr int ESZ = BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  // 32-bit row index (the host keeps D * Cmax below 2^26): a 64-bit division
  // by the run-time Cmax costs the scalar unit hundreds of instructions
  const uint32_t id = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (id >= (uint32_t)D * (uint32_t)Cmax) return;
  const int d = (int)(id / (uint32_t)Cmax), c = (int)(id - (uint32_t)d * (uint32_t)Cmax);
  const int csz = CH > 0 ? CH : chunk;
  const uint8_t* m = mask + (int64_t)d * T;
  const int t0 = c * csz;

  bool v = false;
  if (lane < csz) {
    const int t = t0 + lane;
    v = (t < T) && (m[t] != 0);
  }
  const uint64_t bits = __ballot(v);
  const int cnt = __popcll(bits);
  if (lane == 0) cmask[id] = cnt > 0 ? 1 : 0;

  if (c == 0) {  // count this doc's valid chunks
    int n = 0;
    for (int cc = lane; cc < Cmax; cc += 64) {
      int any = 0;
      for (int j = 0; j < csz; ++j) {
        const int t = cc * csz + j;
        if (t < T && m[t]) { any = 1; break; }
      }
      n += any;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
    if (lane == 0) n_chunks[d] = n;
  }

  const int64_t row_bytes = (int64_t)H * ESZ;
  const uint8_t* xrow = x + ((int64_t)d * T + t0) * row_bytes;
  uint8_t* orow = pooled + (int64_t)id * row_bytes;
  const float fcnt = (float)cnt;
  // The token rows are read once: non-temporal loads and stores keep them
  // from displacing reused lines in L2 (about 15% faster at 100 x 1024 x 2560).
  if constexpr (CH > 0) {
    // U 16-byte vectors of the row per lane per step, and every token load of
    // a step issued before any is summed (U = 5 covers a 2560-wide row)
    constexpr int U = 5;
    for (int h0 = lane * V::N; h0 < H; h0 += U * 64 * V::N) {
      u32x4_t r[U][CH];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int h = h0 + u * 64 * V::N;
#pragma unroll
        for (int j = 0; j < CH; ++j)
          if (h < H && ((bits >> j) & 1))
            r[u][j] = __builtin_nontemporal_load((const u32x4_t*)(xrow + j * row_bytes + (int64_t)h * ESZ));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int h = h0 + u * 64 * V::N;
        if (h >= H) continue;
        float acc[V::N];
#pragma unroll
        for (int i = 0; i < V::N; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < CH; ++j)
          if ((bits >> j) & 1) V::add(acc, r[u][j]);
        float out[V::N];
#pragma unroll
        for (int i = 0; i < V::N; ++i) out[i] = cnt > 0 ? acc[i] / fcnt : 0.f;
        __builtin_nontemporal_store(V::pack(out), (u32x4_t*)(orow + (int64_t)h * ESZ));
      }
    }
  } else {
    for (int h = lane * V::N; h < H; h += 64 * V::N) {
      float acc[V::N];
#pragma unroll
      for (int i = 0; i < V::N; ++i) acc[i] = 0.f;
      uint64_t b = bits;
      while (b) {
        const int j = __builtin_ctzll(b);
        b &= b - 1;
        V::add(acc, __builtin_nontemporal_load((const u32x4_t*)(xrow + j * row_bytes + (int64_t)h * ESZ)));
      }
      float out[V::N];
#pragma unroll
      for (int i = 0; i < V::N; ++i) out[i] = cnt > 0 ? acc[i] / fcnt : 0.f;
      __builtin_nontemporal_store(V::pack(out), (u32x4_t*)(orow + (int64_t)h * ESZ));
    }
  }
}

}  // namespace

namespace kalm {

void launch_chunk_pool(const void* x, const uint8_t* mask, int D, int T, int H, int chunk, int Cmax,
                       kalm_dtype dt, void* pooled, uint8_t* cmask, int32_t* n_chunks, hipStream_t s) {
  const int64_t rows = (int64_t)D * Cmax;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const uint8_t* xb = (const uint8_t*)x;
  uint8_t* pb = (uint8_t*)pooled;
  if (dt == KALM_BF16) {
    if (chunk == 4)
      hipLaunchKernelGGL((chunk_pool_kernel<true, 4>), grid, block, 0, s, xb, mask, D, T, H, chunk, Cmax, pb, cmask, n_chunks);
    else
      hipLaunchKernelGGL((chunk_pool_kernel<true, 0>), grid, block, 0, s, xb, mask, D, T, H, chunk, Cmax, pb, cmask, n_chunks);
  } else {
    if (chunk == 4)
      hipLaunchKernelGGL((chunk_pool_kernel<false, 4>), grid, block, 0, s, xb, mask, D, T, H, chunk, Cmax, pb, cmask, n_chunks);
    else
      hipLaunchKernelGGL((chunk_pool_kernel<false, 0>), grid, block, 0, s, xb, mask, D, T, H, chunk, Cmax, pb, cmask, n_chunks);
  }
}

}  // namespace kalm
