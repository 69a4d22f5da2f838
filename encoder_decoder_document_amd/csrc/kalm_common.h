// Shared device helpers and host-side error plumbing of libkalm (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kalm.h"

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define KALM_WAVE 64

// float -> bf16, round to nearest even (the hardware v_cvt_pk_bf16_f32 path on gfx950).
__device__ __forceinline__ bf16_t to_bf16(float f) { return (bf16_t)f; }

// GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), times
// the gate's partner value u (the activation of a gated MLP).  Evaluated as
// x / (1 + exp(-2 y)) with y the tanh argument -- the same function, since
// (1 + tanh y) / 2 is the logistic function of 2 y -- with one hardware
// exp2 and one reciprocal: large |y| give exp2(+inf) = inf (-> 0) or 0 (-> x).
__device__ __forceinline__ float gated_gelu_tanh(float x, float u) {
  const float y = 0.7978845608028654f * fmaf(0.044715f * x * x, x, x);
  const float e = __builtin_amdgcn_exp2f(-2.f * 1.4426950408889634f * y);
  return x * __builtin_amdgcn_rcpf(1.f + e) * u;
}
__device__ __forceinline__ float from_bf16(bf16_t b) { return (float)b; }

// Pack two floats into one dword of two bf16 (lo = a, hi = b).
// Two floats -> two bf16 in one word (a in the low half), round to nearest
// even: a two-element vector conversion, which is one v_cvt_pk_bf16_f32
// (converting the halves one by one costs two conversions, a shift and an or).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, KALM_WAVE);
  return v;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane i of the wave writes LDS bytes [16 i, 16 i + 16) after the wave-uniform
// base held in M0.  Issued from asm: the compiler's wait-count pass treats every
// LDS-DMA as aliasing every LDS access and would otherwise wait for each copy
// before the next one is issued.  The instruction has no register results; the
// kernel waits for its copies explicitly (vmcnt) before the barrier that
// publishes a tile.
// A wave-uniform 64-bit value the compiler cannot prove uniform, moved to SGPRs.
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_t*)p;
}
// NT = true marks the data as streaming (non-temporal: the L2 evicts such
// lines first), for operands read once per kernel so that they do not push
// out data that is re-read, such as a GEMM's weight tiles.
template <bool NT = false>
__device__ __forceinline__ void dma16(uint64_t sbase, uint32_t voff, uint32_t lds_wave_base) {
  uint32_t saved;  // M0 is a compiler-reserved register: restore it after the copy is issued
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds_wave_base)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds_wave_base)
        : "memory");
}

// Four direct-to-LDS copies into LDS bases lds, lds + 1024, lds + 2048 and
// lds + 3072 (16 bytes per lane each), with one save and restore of M0.
__device__ __forceinline__ void dma16x4(uint64_t sbase, uint32_t o0, uint32_t o1, uint32_t o2, uint32_t o3,
                                        uint32_t lds) {
  uint32_t saved;
  const uint32_t l1 = lds + 1024u, l2 = lds + 2048u, l3 = lds + 3072u;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "global_load_lds_dwordx4 %1, %9\n\t"
      "s_mov_b32 m0, %6\n\t"
      "global_load_lds_dwordx4 %2, %9\n\t"
      "s_mov_b32 m0, %7\n\t"
      "global_load_lds_dwordx4 %3, %9\n\t"
      "s_mov_b32 m0, %8\n\t"
      "global_load_lds_dwordx4 %4, %9\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(lds), "s"(l1), "s"(l2), "s"(l3), "s"(sbase)
      : "memory");
}

// Eight direct-to-LDS copies with one save and restore of M0: four from
// sa + a0..a3 into LDS bases lds + 1024 j and four from sb + b0..b3 into
// lds + BOFS + 1024 j (16 bytes per lane each).
template <uint32_t BOFS>
__device__ __forceinline__ void dma16x8(uint64_t sa, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint64_t sb,
                                        uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %9\n\t"
      "global_load_lds_dwordx4 %1, %10\n\t"
      "s_add_u32 m0, %9, 0x400\n\t"
      "global_load_lds_dwordx4 %2, %10\n\t"
      "s_add_u32 m0, %9, 0x800\n\t"
      "global_load_lds_dwordx4 %3, %10\n\t"
      "s_add_u32 m0, %9, 0xc00\n\t"
      "global_load_lds_dwordx4 %4, %10\n\t"
      "s_add_u32 m0, %9, %12\n\t"
      "global_load_lds_dwordx4 %5, %11\n\t"
      "s_add_u32 m0, %9, %13\n\t"
      "global_load_lds_dwordx4 %6, %11\n\t"
      "s_add_u32 m0, %9, %14\n\t"
      "global_load_lds_dwordx4 %7, %11\n\t"
      "s_add_u32 m0, %9, %15\n\t"
      "global_load_lds_dwordx4 %8, %11\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1), "v"(b2), "v"(b3), "s"(lds), "s"(sa), "s"(sb),
        "n"(BOFS), "n"(BOFS + 1024u), "n"(BOFS + 2048u), "n"(BOFS + 3072u)
      : "memory", "scc");
}

// Wait until the copies of the oldest in-flight k-tile are done: at most
// `later` k-tiles (CPS copies each) issued after it may still be outstanding.
template <int CPS>
__device__ __forceinline__ void wait_dma_ktile(int later) {
  if (later >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * CPS) : "memory");
  else if (later == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CPS) : "memory");
  else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPS) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------ debug-build guards
// The kernels' own guards on data-dependent indexes -- a pair whose rows fall
// outside the given row counts, a passage index outside [0, D), a residual
// source row, gathered row or final row outside its array, a RoPE row outside
// X, a pair layout past INT32_MAX -- keep every access in bounds in every
// build (the work is skipped or its outputs are NaN).  Built with -DKALM_DEBUG
// (libkalm_debug.so), a guard that fires also sets its bit in a device word of
// its translation unit; every entry point of that build then synchronises its
// stream and turns a set bit into KALM_ERR_BOUNDS.  Release builds compile the
// reports out, so their kernels are unchanged.
enum : uint32_t {
  KALM_DBG_PAIR_ROWS = 1u,   // a pair's Q, K/V or O rows outside the row counts
  KALM_DBG_DOC = 2u,         // doc_of_pair outside [0, D)
  KALM_DBG_SRC_ROW = 4u,     // residual source row outside [0, r_rows)
  KALM_DBG_GATHER = 8u,      // gather index outside [0, n_src)
  KALM_DBG_FINAL_ROW = 16u,  // final row outside [0, rows)
  KALM_DBG_ROPE_ROW = 32u,   // RoPE row outside [0, rows)
  KALM_DBG_LAYOUT = 64u,     // pair layout offset past INT32_MAX
};
#ifdef KALM_DEBUG
static __device__ uint32_t kalm_dbg_word;
#define KALM_DBG(bit) atomicOr(&kalm_dbg_word, (uint32_t)(bit))
// Host: this translation unit's guard word on the current device, read and
// cleared (the caller has synchronised the stream that ran the kernels).
#define KALM_DBG_TAKE_DEFINE(name)                                                        \
  namespace kalm {                                                                        \
  uint32_t name() {                                                                       \
    uint32_t v = 0, z = 0;                                                                \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(kalm_dbg_word), sizeof(v)) != hipSuccess ||   \
        hipMemcpyToSymbol(HIP_SYMBOL(kalm_dbg_word), &z, sizeof(z)) != hipSuccess) {      \
      (void)hipGetLastError();                                                            \
      return 0x80000000u;                                                                 \
    }                                                                                     \
    return v;                                                                             \
  }                                                                                       \
  }
namespace kalm {
uint32_t dbg_take_rows();
uint32_t dbg_take_gemm();
uint32_t dbg_take_attn();
uint32_t dbg_take_layer();
}  // namespace kalm
#else
#define KALM_DBG(bit) ((void)0)
#define KALM_DBG_TAKE_DEFINE(name)
#endif

// ---------------------------------------------------------------- host side
namespace kalm {

kalm_status set_error(kalm_status st, const char* fmt, ...);
kalm_status check_device();
// After the launches of entry point `what` on `stream`: a launch error is
// KALM_ERR_LAUNCH; in the debug build the stream is also synchronised (a
// kernel fault is reported against `what`) and a fired guard is KALM_ERR_BOUNDS.
kalm_status check_launch(const char* what, void* stream);

}  // namespace kalm

#define KALM_REQUIRE(cond, status, ...)                     \
  do {                                                      \
    if (!(cond)) return ::kalm::set_error(status, __VA_ARGS__); \
  } while (0)

#define KALM_DEVICE_OR_RETURN()                        \
  do {                                                 \
    kalm_status _s = ::kalm::check_device();           \
    if (_s != KALM_OK) return _s;                      \
  } while (0)

// Launchers implemented in the kernel translation units.  The attention
// launchers' part: 0 merged self + cross softmax; 1 causal self keys only, fp32
// O and lse (a self partial); 2 cross keys only, resumed from the self partial
// (oi, lsei) at each Q row.
namespace kalm {
void launch_chunk_pool(const void* x, const uint8_t* mask, int D, int T, int H, int chunk, int Cmax,
                       kalm_dtype dt, void* pooled, uint8_t* cmask, int32_t* n_chunks, hipStream_t s);
void launch_pair_layout(const int32_t* lq, int nQ, int nD, int32_t* cu_q, int32_t* doc_of_pair,
                        int32_t* final_row, int32_t* h0_row, int64_t rows, int32_t* h0_final, int32_t* cu_u,
                        hipStream_t s);
// Linear layers.  With accumulate, Y (fp32) += X W^T, or -- given Rsrc -- Y = R + X W^T where row m of R is
// Rsrc[Rrow[m]] (Rsrc[m] when Rrow is null), an index outside [0, Rrows) giving NaN.
void launch_linear_bf16(const bf16_t* X, const bf16_t* W, int M, int K, int N, void* Y, bool y_f32,
                        bool accumulate, bf16_t* Y_bf16, const uint8_t* row_mask, hipStream_t s,
                        const float* Rsrc = nullptr, const int32_t* Rrow = nullptr, int64_t Rrows = 0);
void launch_linear_f32(const float* X, const float* W, int M, int K, int N, float* Y, bool accumulate,
                       const uint8_t* row_mask, hipStream_t s, const float* Rsrc = nullptr,
                       const int32_t* Rrow = nullptr, int64_t Rrows = 0);
void launch_merged_attn_bf16(const bf16_t* Q, int64_t q_ld, const bf16_t* Ks, const bf16_t* Vs,
                             int64_t kv_ld, const int32_t* cu_q, int P, int64_t q_rows, int64_t kv_rows,
                             int64_t o_rows, int mode, int max_lq, const bf16_t* Kc, const bf16_t* Vc,
                             int64_t c_ld, const uint8_t* cmask, const int32_t* doc_of_pair, int D, int Cmax,
                             int nq, int nkv, float scale, void* O, int64_t o_ld, float* lse, int part,
                             const float* oi, int64_t oi_ld, const float* lsei, hipStream_t s);
// Split-KV over the cross keys: n_split shares (part 3) into the workspace ws
// (fp32 partials: n_split * o_rows * nq * 256 outputs, then n_split * o_rows *
// nq lse values), merged with the self partial (oi, lsei) into O and lse.
void launch_merged_attn_split(const bf16_t* Q, int64_t q_ld, const int32_t* cu_q, int P, int64_t q_rows,
                              int64_t o_rows, int mode, int max_lq, const bf16_t* Kc, const bf16_t* Vc, int64_t c_ld,
                              const uint8_t* cmask, const int32_t* doc_of_pair, int D, int Cmax, int nq, int nkv,
                              float scale, const float* oi, int64_t oi_ld, const float* lsei, int n_split,
                              float* ws, bf16_t* O, int64_t o_ld, float* lse, hipStream_t s);
void launch_merged_attn_f32(const float* Q, int64_t q_ld, const float* Ks, const float* Vs,
                            int64_t kv_ld, const int32_t* cu_q, int P, int64_t q_rows, int64_t kv_rows,
                            int64_t o_rows, int mode, int max_lq, const float* Kc, const float* Vc, int64_t c_ld,
                            const uint8_t* cmask, const int32_t* doc_of_pair, int D, int Cmax, int nq, int nkv,
                            int d, float scale, float* O, int64_t o_ld, float* lse, int part, const float* oi,
                            int64_t oi_ld, const float* lsei, hipStream_t s);
void launch_yesno(const void* h, bool h_bf16, int64_t h_ld, int64_t rows, const int32_t* final_row, int P,
                  int H, const void* w, bool w_bf16, float* yes, float* no, float* margin, float* score,
                  hipStream_t s);
void launch_rank_topn(const float* score, int n_queries, int D, int top_n, int32_t* out_index, float* out_score,
                      hipStream_t s);
void launch_rms_norm(const void* x, bool x_bf16, int64_t x_ld, int64_t M, int H, const void* w, bool w_bf16, float eps,
                     void* y, bool y_bf16, int64_t y_ld, hipStream_t s);
void launch_rope(void* X, bool bf16, int64_t ld, int64_t rows, int col0, int nh, int d, const int32_t* cu, int n_seq,
                 int max_len, int mode, float theta, hipStream_t s);
void launch_linear_gelu_bf16(const bf16_t* X, const bf16_t* Wg, const bf16_t* Wu, int M, int K, int I, bf16_t* A,
                             hipStream_t s);
void launch_gated_gelu(const void* Y, bool bf16, int64_t y_ld, int64_t M, int I, void* A, int64_t a_ld,
                       hipStream_t s);
void launch_gather_rows(const float* src, const int32_t* idx, int64_t M, int H, int64_t n_src,
                        float* dst, bf16_t* dst_bf16, hipStream_t s);
}  // namespace kalm
