// C ABI entry points of libkalm: host-side argument validation and dispatch.
// Every check runs before anything is enqueued; there is no CPU fallback.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kalm_common.h"

// Device scratch of kalm_merged_attn_split_noalloc: the split-KV partials
// (o, lse of every share) live here instead of in a caller workspace.  Each
// GPU the library runs on holds its own copy from module load until the
// process ends; in host code `scratch` names a host-side stand-in, never
// the device memory -- kernels get the address from hipGetSymbolAddress.
#define KALM_NOALLOC_SCRATCH_BYTES (16u << 20)
static __device__ __align__(256) uint8_t scratch[KALM_NOALLOC_SCRATCH_BYTES];

namespace kalm {

static thread_local char g_err[512];

kalm_status set_error(kalm_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kalm_status check_device() {
  static std::atomic<int> ok{0};  // 1 = a gfx950 device was found once
  if (ok.load(std::memory_order_relaxed)) return KALM_OK;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return set_error(KALM_ERR_NO_DEVICE, "no HIP device visible (libkalm never falls back to the CPU)");
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return set_error(KALM_ERR_NO_DEVICE, "cannot query the current HIP device");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return set_error(KALM_ERR_NO_DEVICE, "device %d is %s; libkalm is built for gfx950 only", dev,
                     prop.gcnArchName);
  ok.store(1, std::memory_order_relaxed);
  return KALM_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU has its own copy at its own
// address) and kept; KALM_ERR_NO_DEVICE / KALM_ERR_LAUNCH with a message if
// there is no current device or the lookup fails.
static kalm_status noalloc_scratch(void** out) {
  constexpr int MAXDEV = 64;
  static std::mutex mu;
  static void* addr[MAXDEV] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV) {
    (void)hipGetLastError();
    return set_error(KALM_ERR_NO_DEVICE, "kalm_merged_attn_split_noalloc: no current HIP device below %d", MAXDEV);
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return set_error(KALM_ERR_LAUNCH, "kalm_merged_attn_split_noalloc: scratch address lookup failed: %s",
                       hipGetErrorString(e));
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return KALM_OK;
}

kalm_status check_launch(const char* what, void* stream) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(KALM_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
#ifdef KALM_DEBUG
  const hipError_t se = hipStreamSynchronize((hipStream_t)stream);
  if (se != hipSuccess) {
    (void)hipGetLastError();
    return set_error(KALM_ERR_LAUNCH, "%s: kernel failed: %s", what, hipGetErrorString(se));
  }
  const uint32_t w = dbg_take_rows() | dbg_take_gemm() | dbg_take_attn() | dbg_take_layer();
  if (w) {
    static const char* const names[] = {"pair rows outside the row counts", "passage index outside [0, D)",
                                        "residual source row outside [0, r_rows)", "gather index outside [0, n_src)",
                                        "final row outside [0, rows)", "RoPE row outside [0, rows)",
                                        "pair layout past INT32_MAX"};
    char buf[320];
    size_t n = 0;
    buf[0] = 0;
    for (int b = 0; b < 7; ++b)
      if ((w >> b) & 1u) n += snprintf(buf + n, sizeof(buf) - n, "%s%s", n ? "; " : "", names[b]);
    if (w & 0x80000000u) snprintf(buf + n, sizeof(buf) - n, "%sguard word unreadable", n ? "; " : "");
    return set_error(KALM_ERR_BOUNDS, "%s: bounds guard fired: %s", what, buf);
  }
#else
  (void)stream;
#endif
  return KALM_OK;
}

}  // namespace kalm

#define ALIGNED16(p) ((((uintptr_t)(p)) & 15u) == 0)

extern "C" {

int32_t kalm_version(void) { return 400; }

int32_t kalm_debug_build(void) {
#ifdef KALM_DEBUG
  return 1;
#else
  return 0;
#endif
}

const char* kalm_last_error(void) { return kalm::g_err; }

kalm_status kalm_device_check(void) { return kalm::check_device(); }

kalm_status kalm_pair_layout(const int32_t* lq, int32_t n_queries, int32_t n_docs, int32_t* cu_q,
                             int32_t* doc_of_pair, int32_t* final_row, int32_t* h0_row, int64_t rows,
                             int32_t* h0_final, int32_t* cu_u, void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(n_queries >= 0 && n_docs >= 0, KALM_ERR_INVALID_ARG, "kalm_pair_layout: negative sizes");
  KALM_REQUIRE((int64_t)n_queries * n_docs < (1LL << 31), KALM_ERR_UNSUPPORTED, "kalm_pair_layout: too many pairs");
  KALM_REQUIRE(cu_q && (n_queries == 0 || (lq && doc_of_pair && final_row)), KALM_ERR_INVALID_ARG,
               "kalm_pair_layout: null pointer");
  KALM_REQUIRE(rows >= 0 && rows < (1LL << 31), KALM_ERR_INVALID_ARG, "kalm_pair_layout: rows out of range");
  KALM_DEVICE_OR_RETURN();
  kalm::launch_pair_layout(lq, n_queries, n_docs, cu_q, doc_of_pair, final_row, h0_row, rows, h0_final, cu_u,
                           (hipStream_t)stream);
  return kalm::check_launch("kalm_pair_layout", stream);
}

kalm_status kalm_chunk_pool(const void* x, const uint8_t* token_mask, int32_t D, int32_t T, int32_t H,
                            int32_t chunk, kalm_dtype dt, void* pooled, uint8_t* chunk_mask,
                            int32_t* n_chunks, void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(dt == KALM_F32 || dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "kalm_chunk_pool: dtype %d", (int)dt);
  KALM_REQUIRE(D >= 0 && T >= 1 && H >= 1, KALM_ERR_INVALID_ARG, "kalm_chunk_pool: bad sizes D=%d T=%d H=%d", D, T, H);
  KALM_REQUIRE(chunk >= 1 && chunk <= 64, KALM_ERR_INVALID_ARG, "kalm_chunk_pool: chunk=%d not in 1..64", chunk);
  KALM_REQUIRE(H % (dt == KALM_BF16 ? 8 : 4) == 0, KALM_ERR_UNSUPPORTED, "kalm_chunk_pool: H=%d not a multiple of the 16-byte vector", H);
  KALM_REQUIRE(D == 0 || (x && token_mask && pooled && chunk_mask && n_chunks), KALM_ERR_INVALID_ARG,
               "kalm_chunk_pool: null pointer");
  KALM_REQUIRE(ALIGNED16(x) && ALIGNED16(pooled), KALM_ERR_INVALID_ARG, "kalm_chunk_pool: x/pooled not 16-byte aligned");
  KALM_REQUIRE((int64_t)D * ((T + chunk - 1) / chunk) < (1LL << 26), KALM_ERR_UNSUPPORTED,
               "kalm_chunk_pool: D * ceil(T / chunk) must stay below 2^26 pooled rows");
  KALM_DEVICE_OR_RETURN();
  if (D == 0) return KALM_OK;
  const int Cmax = (T + chunk - 1) / chunk;
  kalm::launch_chunk_pool(x, token_mask, D, T, H, chunk, Cmax, dt, pooled, chunk_mask, n_chunks, (hipStream_t)stream);
  return kalm::check_launch("kalm_chunk_pool", stream);
}

static kalm_status linear_impl(const char* fn, const void* X, const void* W, int32_t M, int32_t K, int32_t N,
                               kalm_dtype dt, void* Y, kalm_dtype y_dt, int32_t accumulate, void* Y_bf16,
                               void* stream, const float* R = nullptr, const int32_t* r_row = nullptr,
                               int64_t r_rows = 0);

kalm_status kalm_linear(const void* X, const void* W, int32_t M, int32_t K, int32_t N, kalm_dtype dt,
                        void* Y, kalm_dtype y_dt, int32_t accumulate, void* Y_bf16, void* stream) {
  return linear_impl("kalm_linear", X, W, M, K, N, dt, Y, y_dt, accumulate, Y_bf16, stream);
}

kalm_status kalm_linear_residual(const void* X, const void* W, int32_t M, int32_t K, int32_t N, kalm_dtype dt,
                                 const float* R, const int32_t* r_row, int64_t r_rows, float* Y, void* Y_bf16,
                                 void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(M == 0 || R, KALM_ERR_INVALID_ARG, "kalm_linear_residual: null residual source");
  KALM_REQUIRE(r_rows >= 0 && (r_row || r_rows >= M), KALM_ERR_INVALID_ARG,
               "kalm_linear_residual: without r_row the source needs M rows");
  KALM_REQUIRE(ALIGNED16(R), KALM_ERR_INVALID_ARG, "kalm_linear_residual: R must be 16-byte aligned");
  return linear_impl("kalm_linear_residual", X, W, M, K, N, dt, Y, KALM_F32, 1, Y_bf16, stream, R, r_row,
                     r_row ? r_rows : M);
}

static kalm_status linear_impl(const char* fn, const void* X, const void* W, int32_t M, int32_t K, int32_t N,
                               kalm_dtype dt, void* Y, kalm_dtype y_dt, int32_t accumulate, void* Y_bf16,
                               void* stream, const float* R, const int32_t* r_row, int64_t r_rows) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(dt == KALM_F32 || dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dt);
  KALM_REQUIRE(y_dt == KALM_F32 || y_dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "%s: y dtype %d", fn, (int)y_dt);
  KALM_REQUIRE(M >= 0 && K >= 1 && N >= 1, KALM_ERR_INVALID_ARG, "%s: bad sizes M=%d K=%d N=%d", fn, M, K, N);
  KALM_REQUIRE(M == 0 || (X && W && Y), KALM_ERR_INVALID_ARG, "%s: null pointer", fn);
  KALM_REQUIRE(!accumulate || y_dt == KALM_F32, KALM_ERR_UNSUPPORTED, "%s: accumulate needs an F32 Y", fn);
  KALM_REQUIRE(!Y_bf16 || y_dt == KALM_F32, KALM_ERR_UNSUPPORTED, "%s: Y_bf16 copy needs an F32 Y", fn);
  KALM_REQUIRE(ALIGNED16(X) && ALIGNED16(W) && ALIGNED16(Y) && ALIGNED16(Y_bf16), KALM_ERR_INVALID_ARG,
               "%s: pointers must be 16-byte aligned", fn);
  if (dt == KALM_BF16) {
    KALM_REQUIRE(K % 8 == 0 && N % 8 == 0, KALM_ERR_UNSUPPORTED, "%s: bf16 needs K%%8==0 and N%%8==0 (K=%d N=%d)", fn, K, N);
  } else {
    KALM_REQUIRE(y_dt == KALM_F32 && !Y_bf16, KALM_ERR_UNSUPPORTED, "%s: F32 inputs need an F32 Y and no bf16 copy", fn);
    KALM_REQUIRE(K % 4 == 0 && N % 4 == 0, KALM_ERR_UNSUPPORTED, "%s: f32 needs K%%4==0 and N%%4==0", fn);
  }
  KALM_DEVICE_OR_RETURN();
  if (M == 0) return KALM_OK;
  if (dt == KALM_BF16)
    kalm::launch_linear_bf16((const bf16_t*)X, (const bf16_t*)W, M, K, N, Y, y_dt == KALM_F32, accumulate != 0,
                             (bf16_t*)Y_bf16, nullptr, (hipStream_t)stream, R, r_row, r_rows);
  else
    kalm::launch_linear_f32((const float*)X, (const float*)W, M, K, N, (float*)Y, accumulate != 0, nullptr,
                            (hipStream_t)stream, R, r_row, r_rows);
  return kalm::check_launch(fn, stream);
}

static kalm_status cross_kv_impl(const char* fn, const void* pooled, const uint8_t* chunk_mask, int32_t D,
                                 int32_t Cmax, int32_t H, const void* Wkv, int32_t kv_dim, int32_t n_layers,
                                 kalm_dtype dt, void* KVc, void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(dt == KALM_F32 || dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dt);
  KALM_REQUIRE(D >= 0 && Cmax >= 1 && H >= 1 && kv_dim >= 1 && n_layers >= 1, KALM_ERR_INVALID_ARG,
               "%s: bad sizes", fn);
  KALM_REQUIRE((int64_t)D * Cmax < (1LL << 31), KALM_ERR_UNSUPPORTED, "%s: too many rows", fn);
  KALM_REQUIRE((int64_t)2 * kv_dim * n_layers < (1LL << 31), KALM_ERR_UNSUPPORTED, "%s: too many columns", fn);
  KALM_REQUIRE(D == 0 || (pooled && Wkv && KVc), KALM_ERR_INVALID_ARG, "%s: null pointer", fn);
  KALM_REQUIRE(ALIGNED16(pooled) && ALIGNED16(Wkv) && ALIGNED16(KVc), KALM_ERR_INVALID_ARG,
               "%s: pointers must be 16-byte aligned", fn);
  KALM_REQUIRE(H % (dt == KALM_BF16 ? 8 : 4) == 0 && kv_dim % 4 == 0, KALM_ERR_UNSUPPORTED,
               "%s: H=%d / kv_dim=%d not aligned to the vector width", fn, H, kv_dim);
  KALM_DEVICE_OR_RETURN();
  if (D == 0) return KALM_OK;
  // one GEMM over every layer's stacked weights: output row r holds, per layer,
  // that layer's keys then values of pooled row r
  const int M = D * Cmax, N = 2 * kv_dim * n_layers;
  if (dt == KALM_BF16)
    kalm::launch_linear_bf16((const bf16_t*)pooled, (const bf16_t*)Wkv, M, H, N, KVc, false, false, nullptr,
                             chunk_mask, (hipStream_t)stream);
  else
    kalm::launch_linear_f32((const float*)pooled, (const float*)Wkv, M, H, N, (float*)KVc, false, chunk_mask,
                            (hipStream_t)stream);
  return kalm::check_launch(fn, stream);
}

kalm_status kalm_cross_kv(const void* pooled, const uint8_t* chunk_mask, int32_t D, int32_t Cmax, int32_t H,
                          const void* Wkv, int32_t kv_dim, kalm_dtype dt, void* KVc, void* stream) {
  return cross_kv_impl("kalm_cross_kv", pooled, chunk_mask, D, Cmax, H, Wkv, kv_dim, 1, dt, KVc, stream);
}

kalm_status kalm_cross_kv_layers(const void* pooled, const uint8_t* chunk_mask, int32_t D, int32_t Cmax, int32_t H,
                                 const void* Wkv, int32_t kv_dim, int32_t n_layers, kalm_dtype dt, void* KVc,
                                 void* stream) {
  return cross_kv_impl("kalm_cross_kv_layers", pooled, chunk_mask, D, Cmax, H, Wkv, kv_dim, n_layers, dt, KVc,
                       stream);
}

static kalm_status merged_attn_impl(const char* fn, const void* Q, int64_t q_ld, int64_t q_rows, const void* Ks,
                                    const void* Vs, int64_t kv_ld, int64_t kv_rows, const int32_t* cu_q, int32_t P,
                                    int32_t max_lq, const void* Kc, const void* Vc, int64_t c_ld,
                                    const uint8_t* chunk_mask, const int32_t* doc_of_pair, int32_t D, int32_t Cmax,
                                    int32_t nq, int32_t nkv, int32_t d, float scale, kalm_dtype dt, void* O,
                                    int64_t o_ld, int64_t o_rows, float* lse, int32_t row_mode, void* stream,
                                    int part = 0, const float* oi = nullptr, int64_t oi_ld = 0,
                                    const float* lsei = nullptr, int32_t n_split = 1, void* ws = nullptr,
                                    int64_t ws_bytes = 0) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(dt == KALM_F32 || dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dt);
  // part 3: the cross keys in n_split shares merged with a self partial (bf16 path)
  const bool split = part == 3;
  if (split) {
    KALM_REQUIRE(dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "%s: split-KV is implemented for bf16 only", fn);
    KALM_REQUIRE(n_split >= 1 && n_split <= 64, KALM_ERR_INVALID_ARG, "%s: n_split %d not in 1..64", fn, n_split);
    KALM_REQUIRE(o_rows >= 0 && ws_bytes >= (int64_t)n_split * o_rows * nq * (d + 1) * 4, KALM_ERR_INVALID_ARG,
                 "%s: workspace of %lld bytes is smaller than n_split * o_rows * nq * (d + 1) * 4", fn,
                 (long long)ws_bytes);
    KALM_REQUIRE(P == 0 || o_rows == 0 || (ws && ALIGNED16(ws)), KALM_ERR_INVALID_ARG,
                 "%s: workspace missing or not 16-byte aligned", fn);
    part = 2;  // the checks below are those of a resumed pass
  }
  KALM_REQUIRE(row_mode >= 0 && row_mode <= 3, KALM_ERR_INVALID_ARG, "%s: row_mode %d not in 0..3", fn, row_mode);
  KALM_REQUIRE(P >= 0 && q_rows >= 0 && kv_rows >= 0 && o_rows >= 0 && max_lq >= 0 && D >= 0 && Cmax >= 0,
               KALM_ERR_INVALID_ARG, "%s: negative sizes", fn);
  KALM_REQUIRE(row_mode < 2 || P == 0 || D >= 1, KALM_ERR_INVALID_ARG, "%s: row_mode %d needs D >= 1", fn,
               row_mode);
  KALM_REQUIRE(nq >= 1 && nkv >= 1 && nq % nkv == 0, KALM_ERR_INVALID_ARG, "%s: nq=%d nkv=%d", fn, nq, nkv);
  KALM_REQUIRE(scale > 0.f, KALM_ERR_INVALID_ARG, "%s: scale must be positive", fn);
  // part 1 reads no cross keys and no passage index; part 2 reads no self keys
  KALM_REQUIRE(P == 0 || (Q && cu_q && O && (part == 2 || (Ks && Vs)) && (part == 1 || doc_of_pair)),
               KALM_ERR_INVALID_ARG, "%s: null pointer", fn);
  KALM_REQUIRE(part == 1 || Cmax == 0 || D == 0 || (Kc && Vc && chunk_mask), KALM_ERR_INVALID_ARG,
               "%s: null cross pointer", fn);
  KALM_REQUIRE(part != 1 || P == 0 || lse, KALM_ERR_INVALID_ARG, "%s: a self partial needs its lse output", fn);
  KALM_REQUIRE(part != 2 || P == 0 || (oi && lsei), KALM_ERR_INVALID_ARG, "%s: null self-partial pointer", fn);
  KALM_REQUIRE(q_ld >= (int64_t)nq * d && (part == 2 || kv_ld >= (int64_t)nkv * d) && o_ld >= (int64_t)nq * d &&
                   (part != 2 || oi_ld >= (int64_t)nq * d) && (part == 1 || Cmax == 0 || c_ld >= (int64_t)nkv * d),
               KALM_ERR_INVALID_ARG, "%s: leading dimension smaller than the heads", fn);
  if (dt == KALM_BF16) {
    KALM_REQUIRE(d == 256, KALM_ERR_UNSUPPORTED, "%s: bf16 path needs head_dim 256 (got %d)", fn, d);
    const int G = nq / nkv;
    KALM_REQUIRE(G == 1 || G == 2 || G % 4 == 0, KALM_ERR_UNSUPPORTED,
                 "%s: query heads per KV head must be 1, 2 or a multiple of 4 (got %d)", fn, G);
    KALM_REQUIRE(Cmax <= 4096, KALM_ERR_UNSUPPORTED, "%s: bf16 path supports Cmax <= 4096 (got %d)", fn, Cmax);
    // one workgroup per (pair, KV head, head group, block of >= 32 rows): at
    // most P * nq * ceil(rows / 32) of them, which must stay below 2^31
    const int64_t rows_per_pair = (row_mode == 1 || row_mode == 3) ? 1 : max_lq;
    KALM_REQUIRE((int64_t)P * nq * ((rows_per_pair + 31) / 32) < (1LL << 31), KALM_ERR_UNSUPPORTED,
                 "%s: too many attention work items (P=%d, nq=%d, max_lq=%d)", fn, P, nq, max_lq);
    KALM_REQUIRE((part == 2 || (int64_t)max_lq * kv_ld * 2 < (1LL << 31)) &&
                     (part == 1 || (int64_t)Cmax * c_ld * 2 < (1LL << 31)),
                 KALM_ERR_UNSUPPORTED, "%s: per-pair K block exceeds 2 GiB", fn);
    KALM_REQUIRE(q_ld % 8 == 0 && kv_ld % 8 == 0 && o_ld % 8 == 0 && c_ld % 8 == 0 && oi_ld % 4 == 0,
                 KALM_ERR_UNSUPPORTED, "%s: bf16 leading dimensions must be multiples of 8 (fp32 ones of 4)", fn);
    KALM_REQUIRE(ALIGNED16(Q) && ALIGNED16(Ks) && ALIGNED16(Vs) && ALIGNED16(O) && ALIGNED16(Kc) && ALIGNED16(Vc) &&
                     ALIGNED16(oi),
                 KALM_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
  } else {
    KALM_REQUIRE(d >= 1 && d <= 256, KALM_ERR_UNSUPPORTED, "%s: f32 path needs head_dim <= 256", fn);
  }
  KALM_DEVICE_OR_RETURN();
  if (P == 0 || o_rows == 0) return KALM_OK;
  if (split)
    kalm::launch_merged_attn_split((const bf16_t*)Q, q_ld, cu_q, P, q_rows, o_rows, row_mode, max_lq,
                                   (const bf16_t*)Kc, (const bf16_t*)Vc, c_ld, chunk_mask, doc_of_pair, D, Cmax, nq,
                                   nkv, scale, oi, oi_ld, lsei, n_split, (float*)ws, (bf16_t*)O, o_ld, lse,
                                   (hipStream_t)stream);
  else if (dt == KALM_BF16)
    kalm::launch_merged_attn_bf16((const bf16_t*)Q, q_ld, (const bf16_t*)Ks, (const bf16_t*)Vs, kv_ld, cu_q, P,
                                  q_rows, kv_rows, o_rows, row_mode, max_lq, (const bf16_t*)Kc, (const bf16_t*)Vc,
                                  c_ld, chunk_mask, doc_of_pair, D, Cmax, nq, nkv, scale, O, o_ld, lse, part, oi,
                                  oi_ld, lsei, (hipStream_t)stream);
  else
    kalm::launch_merged_attn_f32((const float*)Q, q_ld, (const float*)Ks, (const float*)Vs, kv_ld, cu_q, P, q_rows,
                                 kv_rows, o_rows, row_mode, max_lq, (const float*)Kc, (const float*)Vc, c_ld,
                                 chunk_mask, doc_of_pair, D, Cmax, nq, nkv, d, scale, (float*)O, o_ld, lse, part,
                                 oi, oi_ld, lsei, (hipStream_t)stream);
  return kalm::check_launch(fn, stream);
}

kalm_status kalm_merged_attn(const void* Q, int64_t q_ld, const void* Ks, const void* Vs, int64_t kv_ld,
                             const int32_t* cu_q, int32_t P, int64_t rows, int32_t max_lq, const void* Kc,
                             const void* Vc, int64_t c_ld, const uint8_t* chunk_mask,
                             const int32_t* doc_of_pair, int32_t D, int32_t Cmax, int32_t nq, int32_t nkv,
                             int32_t d, float scale, kalm_dtype dt, void* O, int64_t o_ld, float* lse,
                             void* stream) {
  return merged_attn_impl("kalm_merged_attn", Q, q_ld, rows, Ks, Vs, kv_ld, rows, cu_q, P, max_lq, Kc, Vc, c_ld,
                          chunk_mask, doc_of_pair, D, Cmax, nq, nkv, d, scale, dt, O, o_ld, rows, lse, 0, stream);
}

kalm_status kalm_merged_attn_rows(const void* Q, int64_t q_ld, int64_t q_rows, const void* Ks, const void* Vs,
                                  int64_t kv_ld, int64_t kv_rows, const int32_t* cu_q, int32_t P, int32_t max_lq,
                                  const void* Kc, const void* Vc, int64_t c_ld, const uint8_t* chunk_mask,
                                  const int32_t* doc_of_pair, int32_t D, int32_t Cmax, int32_t nq, int32_t nkv,
                                  int32_t d, float scale, kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows,
                                  float* lse, int32_t row_mode, void* stream) {
  return merged_attn_impl("kalm_merged_attn_rows", Q, q_ld, q_rows, Ks, Vs, kv_ld, kv_rows, cu_q, P, max_lq, Kc,
                          Vc, c_ld, chunk_mask, doc_of_pair, D, Cmax, nq, nkv, d, scale, dt, O, o_ld, o_rows, lse,
                          row_mode, stream);
}

kalm_status kalm_self_attn_partial(const void* Q, int64_t q_ld, const void* Ks, const void* Vs, int64_t kv_ld,
                                   int64_t rows, const int32_t* cu_s, int32_t n_seq, int32_t max_len, int32_t nq,
                                   int32_t nkv, int32_t d, float scale, kalm_dtype dt, float* O, int64_t o_ld,
                                   float* lse, void* stream) {
  return merged_attn_impl("kalm_self_attn_partial", Q, q_ld, rows, Ks, Vs, kv_ld, rows, cu_s, n_seq, max_len,
                          nullptr, nullptr, 0, nullptr, nullptr, 0, 0, nq, nkv, d, scale, dt, O, o_ld, rows, lse, 0,
                          stream, 1);
}

kalm_status kalm_merged_attn_resume(const void* Q, int64_t q_ld, int64_t q_rows, const float* o_self, int64_t s_ld,
                                    const float* lse_self, const int32_t* cu_q, int32_t P, int32_t max_lq,
                                    const void* Kc, const void* Vc, int64_t c_ld, const uint8_t* chunk_mask,
                                    const int32_t* doc_of_pair, int32_t D, int32_t Cmax, int32_t nq, int32_t nkv,
                                    int32_t d, float scale, kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows,
                                    float* lse, int32_t row_mode, void* stream) {
  // no self keys are read: the self-row bound is the Q-row one
  return merged_attn_impl("kalm_merged_attn_resume", Q, q_ld, q_rows, nullptr, nullptr, 0, INT64_MAX, cu_q, P,
                          max_lq, Kc, Vc, c_ld, chunk_mask, doc_of_pair, D, Cmax, nq, nkv, d, scale, dt, O, o_ld,
                          o_rows, lse, row_mode, stream, 2, o_self, s_ld, lse_self);
}

kalm_status kalm_merged_attn_split(const void* Q, int64_t q_ld, int64_t q_rows, const float* o_self, int64_t s_ld,
                                   const float* lse_self, const int32_t* cu_q, int32_t P, int32_t max_lq,
                                   const void* Kc, const void* Vc, int64_t c_ld, const uint8_t* chunk_mask,
                                   const int32_t* doc_of_pair, int32_t D, int32_t Cmax, int32_t nq, int32_t nkv,
                                   int32_t d, float scale, kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows,
                                   float* lse, int32_t row_mode, int32_t n_split, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  return merged_attn_impl("kalm_merged_attn_split", Q, q_ld, q_rows, nullptr, nullptr, 0, INT64_MAX, cu_q, P,
                          max_lq, Kc, Vc, c_ld, chunk_mask, doc_of_pair, D, Cmax, nq, nkv, d, scale, dt, O, o_ld,
                          o_rows, lse, row_mode, stream, 3, o_self, s_ld, lse_self, n_split, workspace,
                          workspace_bytes);
}

kalm_status kalm_merged_attn_split_noalloc(const void* Q, int64_t q_ld, int64_t q_rows, const float* o_self,
                                           int64_t s_ld, const float* lse_self, const int32_t* cu_q, int32_t P,
                                           int32_t max_lq, const void* Kc, const void* Vc, int64_t c_ld,
                                           const uint8_t* chunk_mask, const int32_t* doc_of_pair, int32_t D,
                                           int32_t Cmax, int32_t nq, int32_t nkv, int32_t d, float scale,
                                           kalm_dtype dt, void* O, int64_t o_ld, int64_t o_rows, float* lse,
                                           int32_t row_mode, int32_t n_split, void* stream) {
  const char* fn = "kalm_merged_attn_split_noalloc";
  kalm::g_err[0] = 0;
  KALM_REQUIRE(n_split >= 1 && n_split <= 64 && o_rows >= 0 && nq >= 1 && d >= 1, KALM_ERR_INVALID_ARG,
               "%s: bad n_split / o_rows / nq / d", fn);
  const int64_t need = (int64_t)n_split * o_rows * nq * (d + 1) * 4;
  KALM_REQUIRE(need <= (int64_t)KALM_NOALLOC_SCRATCH_BYTES, KALM_ERR_INVALID_ARG,
               "%s: the split partials need %lld bytes, more than the %u-byte static scratch (lower n_split or "
               "split the batch)", fn, (long long)need, (unsigned)KALM_NOALLOC_SCRATCH_BYTES);
  KALM_DEVICE_OR_RETURN();
  void* ws = nullptr;
  const kalm_status st = kalm::noalloc_scratch(&ws);
  if (st != KALM_OK) return st;
  return merged_attn_impl(fn, Q, q_ld, q_rows, nullptr, nullptr, 0, INT64_MAX, cu_q, P, max_lq, Kc, Vc, c_ld,
                          chunk_mask, doc_of_pair, D, Cmax, nq, nkv, d, scale, dt, O, o_ld, o_rows, lse, row_mode,
                          stream, 3, o_self, s_ld, lse_self, n_split, ws, (int64_t)KALM_NOALLOC_SCRATCH_BYTES);
}

kalm_status kalm_rms_norm(const void* x, kalm_dtype x_dt, int64_t x_ld, int64_t M, int32_t H, const void* w,
                          kalm_dtype w_dt, float eps, void* y, kalm_dtype y_dt, int64_t y_ld, void* stream) {
  kalm::g_err[0] = 0;
  const bool dts_ok = (x_dt == KALM_F32 || x_dt == KALM_BF16) && (w_dt == KALM_F32 || w_dt == KALM_BF16) &&
                      (y_dt == KALM_F32 || y_dt == KALM_BF16);
  KALM_REQUIRE(dts_ok, KALM_ERR_UNSUPPORTED, "kalm_rms_norm: dtype");
  KALM_REQUIRE(M >= 0 && H >= 4 && H % 4 == 0, KALM_ERR_INVALID_ARG, "kalm_rms_norm: H must be a positive multiple of 4");
  KALM_REQUIRE(x_ld >= H && y_ld >= H && x_ld % 4 == 0 && y_ld % 4 == 0, KALM_ERR_INVALID_ARG,
               "kalm_rms_norm: leading dimensions must be >= H and multiples of 4");
  KALM_REQUIRE(eps >= 0.f, KALM_ERR_INVALID_ARG, "kalm_rms_norm: eps must be >= 0");
  KALM_REQUIRE(M == 0 || (x && w && y), KALM_ERR_INVALID_ARG, "kalm_rms_norm: null pointer");
  KALM_REQUIRE(ALIGNED16(x) && ALIGNED16(w) && ALIGNED16(y), KALM_ERR_INVALID_ARG,
               "kalm_rms_norm: pointers must be 16-byte aligned");
  KALM_DEVICE_OR_RETURN();
  kalm::launch_rms_norm(x, x_dt == KALM_BF16, x_ld, M, H, w, w_dt == KALM_BF16, eps, y, y_dt == KALM_BF16, y_ld,
                        (hipStream_t)stream);
  return kalm::check_launch("kalm_rms_norm", stream);
}

kalm_status kalm_rope(void* X, kalm_dtype dt, int64_t ld, int64_t rows, int32_t col0, int32_t n_heads, int32_t d,
                      const int32_t* cu, int32_t n_seq, int32_t max_len, int32_t row_mode, float theta,
                      void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(dt == KALM_F32 || dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "kalm_rope: dtype");
  KALM_REQUIRE(row_mode == 0 || row_mode == 1, KALM_ERR_INVALID_ARG, "kalm_rope: row_mode %d not in 0..1", row_mode);
  KALM_REQUIRE(rows >= 0 && n_seq >= 0 && n_heads >= 0 && max_len >= 0 && col0 >= 0, KALM_ERR_INVALID_ARG,
               "kalm_rope: negative sizes");
  KALM_REQUIRE(d >= 8 && d % 8 == 0 && col0 % 4 == 0 && ld % 4 == 0 && ld >= col0 + (int64_t)n_heads * d,
               KALM_ERR_INVALID_ARG, "kalm_rope: d must be a multiple of 8, col0 and ld multiples of 4 covering the heads");
  KALM_REQUIRE(theta > 1.f, KALM_ERR_INVALID_ARG, "kalm_rope: theta must be > 1");
  KALM_REQUIRE((int64_t)max_len * n_heads * (d / 8) < (int64_t)65535 * 256, KALM_ERR_UNSUPPORTED,
               "kalm_rope: too many rows per sequence");
  KALM_REQUIRE(n_seq == 0 || (X && cu), KALM_ERR_INVALID_ARG, "kalm_rope: null pointer");
  KALM_REQUIRE(ALIGNED16(X), KALM_ERR_INVALID_ARG, "kalm_rope: X must be 16-byte aligned");
  KALM_DEVICE_OR_RETURN();
  kalm::launch_rope(X, dt == KALM_BF16, ld, rows, col0, n_heads, d, cu, n_seq, max_len, row_mode, theta,
                    (hipStream_t)stream);
  return kalm::check_launch("kalm_rope", stream);
}

kalm_status kalm_gated_gelu(const void* Y, kalm_dtype dt, int64_t y_ld, int64_t M, int32_t I, void* A, int64_t a_ld,
                            void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(dt == KALM_F32 || dt == KALM_BF16, KALM_ERR_UNSUPPORTED, "kalm_gated_gelu: dtype");
  KALM_REQUIRE(M >= 0 && I >= 4 && I % 4 == 0, KALM_ERR_INVALID_ARG, "kalm_gated_gelu: I must be a positive multiple of 4");
  KALM_REQUIRE(y_ld >= 2 * (int64_t)I && a_ld >= I && y_ld % 4 == 0 && a_ld % 4 == 0, KALM_ERR_INVALID_ARG,
               "kalm_gated_gelu: leading dimensions must cover the columns and be multiples of 4");
  KALM_REQUIRE(M == 0 || (Y && A), KALM_ERR_INVALID_ARG, "kalm_gated_gelu: null pointer");
  KALM_REQUIRE(ALIGNED16(Y) && ALIGNED16(A), KALM_ERR_INVALID_ARG, "kalm_gated_gelu: pointers must be 16-byte aligned");
  KALM_DEVICE_OR_RETURN();
  kalm::launch_gated_gelu(Y, dt == KALM_BF16, y_ld, M, I, A, a_ld, (hipStream_t)stream);
  return kalm::check_launch("kalm_gated_gelu", stream);
}

kalm_status kalm_linear_gated_gelu(const void* X, const void* Wg, const void* Wu, int32_t M, int32_t K, int32_t I,
                                   void* A, void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(M >= 0 && K >= 1 && I >= 1, KALM_ERR_INVALID_ARG, "kalm_linear_gated_gelu: bad sizes M=%d K=%d I=%d",
               M, K, I);
  KALM_REQUIRE(K % 8 == 0 && I % 128 == 0, KALM_ERR_UNSUPPORTED,
               "kalm_linear_gated_gelu: needs K %% 8 == 0 and I %% 128 == 0 (K=%d I=%d)", K, I);
  KALM_REQUIRE((int64_t)I * K < (1LL << 30), KALM_ERR_UNSUPPORTED, "kalm_linear_gated_gelu: weights too large");
  KALM_REQUIRE(M == 0 || (X && Wg && Wu && A), KALM_ERR_INVALID_ARG, "kalm_linear_gated_gelu: null pointer");
  KALM_REQUIRE(ALIGNED16(X) && ALIGNED16(Wg) && ALIGNED16(Wu) && ALIGNED16(A), KALM_ERR_INVALID_ARG,
               "kalm_linear_gated_gelu: pointers must be 16-byte aligned");
  KALM_DEVICE_OR_RETURN();
  kalm::launch_linear_gelu_bf16((const bf16_t*)X, (const bf16_t*)Wg, (const bf16_t*)Wu, M, K, I, (bf16_t*)A,
                                (hipStream_t)stream);
  return kalm::check_launch("kalm_linear_gated_gelu", stream);
}

kalm_status kalm_yesno_score(const void* h, kalm_dtype h_dt, int64_t h_ld, int64_t rows, const int32_t* final_row,
                             int32_t P, int32_t H, const void* w_yesno, kalm_dtype w_dt, float* yes, float* no,
                             float* margin, float* score, void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE((h_dt == KALM_F32 || h_dt == KALM_BF16) && (w_dt == KALM_F32 || w_dt == KALM_BF16),
               KALM_ERR_UNSUPPORTED, "kalm_yesno_score: dtype");
  KALM_REQUIRE(P >= 0 && H >= 1 && h_ld >= H && rows >= 0, KALM_ERR_INVALID_ARG, "kalm_yesno_score: bad sizes");
  KALM_REQUIRE(P == 0 || (h && final_row && w_yesno && yes && no && score), KALM_ERR_INVALID_ARG,
               "kalm_yesno_score: null pointer");
  KALM_DEVICE_OR_RETURN();
  if (P == 0) return KALM_OK;
  kalm::launch_yesno(h, h_dt == KALM_BF16, h_ld, rows, final_row, P, H, w_yesno, w_dt == KALM_BF16, yes, no, margin,
                     score, (hipStream_t)stream);
  return kalm::check_launch("kalm_yesno_score", stream);
}

kalm_status kalm_gather_rows(const float* src, const int32_t* idx, int64_t M, int32_t H, int64_t n_src, float* dst,
                             void* dst_bf16, void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(M >= 0 && H >= 1 && n_src >= 0, KALM_ERR_INVALID_ARG, "kalm_gather_rows: bad sizes");
  KALM_REQUIRE(H % 4 == 0, KALM_ERR_UNSUPPORTED, "kalm_gather_rows: H %% 4 != 0");
  KALM_REQUIRE(M == 0 || (src && idx && dst), KALM_ERR_INVALID_ARG, "kalm_gather_rows: null pointer");
  KALM_REQUIRE(ALIGNED16(src) && ALIGNED16(dst) && ALIGNED16(dst_bf16), KALM_ERR_INVALID_ARG,
               "kalm_gather_rows: pointers must be 16-byte aligned");
  KALM_DEVICE_OR_RETURN();
  if (M == 0) return KALM_OK;
  kalm::launch_gather_rows(src, idx, M, H, n_src, dst, (bf16_t*)dst_bf16, (hipStream_t)stream);
  return kalm::check_launch("kalm_gather_rows", stream);
}

kalm_status kalm_rank_topn(const float* score, int32_t n_queries, int32_t n_docs, int32_t top_n,
                           int32_t* out_index, float* out_score, void* stream) {
  kalm::g_err[0] = 0;
  KALM_REQUIRE(n_queries >= 0 && n_docs >= 0 && top_n >= 0, KALM_ERR_INVALID_ARG, "kalm_rank_topn: negative sizes");
  KALM_REQUIRE(top_n <= n_docs, KALM_ERR_INVALID_ARG, "kalm_rank_topn: top_n=%d > n_docs=%d", top_n, n_docs);
  KALM_REQUIRE(n_docs <= 4096, KALM_ERR_UNSUPPORTED, "kalm_rank_topn: n_docs=%d > 4096", n_docs);
  KALM_REQUIRE(n_queries == 0 || top_n == 0 || (score && out_index && out_score), KALM_ERR_INVALID_ARG,
               "kalm_rank_topn: null pointer");
  KALM_DEVICE_OR_RETURN();
  if (n_queries == 0 || top_n == 0) return KALM_OK;
  kalm::launch_rank_topn(score, n_queries, n_docs, top_n, out_index, out_score, (hipStream_t)stream);
  return kalm::check_launch("kalm_rank_topn", stream);
}

}  // extern "C"
