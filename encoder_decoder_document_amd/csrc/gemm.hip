// a2 / a5 -- bf16 MFMA GEMM  Y[M,N] = X[M,K] . W[N,K]^T  (fp32 accumulation).
//
// Serves the cross K/V projection of the pooled passage vectors ("KaLM-Reranker
// -V1-Nano -- MLX (Apple Silicon)", What this is) and the linear layers of the
// decoder-stack glue.  Both operands are K-contiguous ([rows, K]), which is the
// layout the gfx950 v_mfma_f32_32x32x16_bf16 fragments want: every lane reads 8
// consecutive k values of one row.
//
// Block tile BM x BN, k in steps of BK (32 or 64), 512 threads (8 waves),
// each wave a (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks.  The MFMA "A" operand is
// the weight tile and the "B" operand the activation tile, so each lane's
// accumulator holds 4 consecutive output columns of one output row and the
// epilogue writes 8-byte (bf16) or 16-byte (fp32) vectors.  Tiles move from
// global memory straight into LDS with the gfx950 global_load_lds_dwordx4 copy
// (no staging registers) through an LDS ring of STAGES k-tiles, one barrier
// per k-tile.  With BK = 64 every copied row is one whole 128-byte line, which
// halves the L1 -> L2 requests per byte.  The k-loop is bound by that per-k-tile
// rendezvous -- every wave waits for the slowest copy of the workgroup -- more
// than by L2 bandwidth or by the ring's depth.  16-byte k-chunks are stored XOR-swizzled
// (see swz), chosen through the address each lane fetches, so the fragment
// reads of 32 consecutive rows are bank-conflict free.  Workgroups are
// remapped so that each XCD walks a contiguous range of output tiles (the
// tiles sharing activation rows stay in one L2).  The persistent kernel also
// serves a gated MLP's gate/up projection fused with its activation (GELU).
#include "kalm_common.h"

namespace {

enum Epi { EPI_BF16 = 0, EPI_F32 = 1, EPI_F32_ACC = 2 };

// Streaming (non-temporal) hints: on the outputs (written once; the fp32
// residual read once) they help; on the activation tiles they were measured
// to hurt (the column-tile siblings re-read them through L2), so off.
#ifndef GEMM_STREAM_X
#define GEMM_STREAM_X false
#endif
// Explicit scheduling hints: the next k-step's fragment reads interleaved
// with the current k-step's MFMAs (measured within run-to-run noise of ~3%).
#ifndef GEMM_SCHED
#define GEMM_SCHED 1
#endif
#ifndef GEMM_PF_DIST
#define GEMM_PF_DIST 1  // k-tiles before the last at whose start the fp32 stream is loaded
#endif
#ifndef GEMM_PF_Y
#define GEMM_PF_Y true
#endif
// Activation slots of the residual update's ring (beside 2 weight slots):
// 3 puts each activation k-tile in flight one k-tile earlier than its weight
// k-tile -- the activations come from HBM, the weights from L2 -- and the
// ring (80 KB) still lets two workgroups share a CU.  Measured at the Small
// shape (A/B on one box): 3.11-3.13 ms against 3.20 ms per launch with 2.
#ifndef GEMM_RES_ASTG
#define GEMM_RES_ASTG 3
#endif
#ifndef GEMM_PERSIST
#define GEMM_PERSIST 1
#endif
// shortest k-loop at which a plain residual update takes the persistent kernel
#ifndef GEMM_RES_PERSIST_MINK
#define GEMM_RES_PERSIST_MINK 2048
#endif
#ifndef GEMM_PKREV
#define GEMM_PKREV 1
#endif
#ifndef GEMM_KREV
#define GEMM_KREV 1
#endif
#ifndef GEMM_STREAM_Y
#define GEMM_STREAM_Y true
#endif

// Physical 16-byte chunk of logical chunk c in row `row` of a k-tile whose
// rows are BK bf16 (64 or 128 bytes).  The gfx950 LDS serves a ds_read_b128
// 16 lanes at a time across 64 banks (256 bytes); the fragment reads of 16
// consecutive rows at one logical chunk must hit 16 distinct 16-byte bank
// groups.  BK = 32: 4 rows share 256 bytes, XOR with (row >> 2) & 3; BK = 64:
// 2 rows share 256 bytes, XOR with (row >> 1) & 7.
template <int BK>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (BK == 32) return c ^ ((row >> 2) & 3);
  else return c ^ ((row >> 1) & 7);
}

// Copy plan of one ROWS x BK k-tile of a [rows_total, K] bf16 matrix into LDS
// (16-byte chunk c of a row stored at swz(row, c)).  Each wave instruction
// fills 1 KB = 1024 / (2 BK) tile rows; lane l writes physical chunk l % CPR of
// row l / CPR (CPR = chunks per row), so it fetches the logical chunk that
// belongs there -- the XOR swizzle is applied through the global address, and
// with BK = 64 every row is one whole 128-byte line.  Addresses are a scalar
// 64-bit tile base plus a 32-bit per-lane byte offset; rows past the matrix
// end are clamped to its last row (their products are discarded).
template <int ROWS, int NWAVES, int BK, bool NT>
struct DmaPlan {
  static constexpr int CPR = BK / 8;                    // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                  // rows per instruction
  static constexpr int PER = ROWS / RPI / NWAVES;       // instructions per wave per stage
  uint64_t base;                                        // byte address of the tile's first row (uniform)
  uint32_t row_off[PER];                                // byte offset of this lane's source rows
  uint32_t slab[PER];                                   // LDS byte offset of each 1 KB slab (uniform)
  int lc8[PER];                                         // k offset of this lane's chunk in a k-tile

  __device__ __forceinline__ void init(const bf16_t* G, int rows_total, int K, int r0, int wave, int lane) {
    const int rr = lane / CPR;
    base = (uint64_t)(uintptr_t)(G + (int64_t)r0 * K);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int R0 = RPI * (wave * PER + j);
      const int row = min(r0 + R0 + rr, rows_total - 1) - r0;
      lc8[j] = swz<BK>(R0 + rr, lane % CPR) * 8;  // the swizzle is an involution
      row_off[j] = (uint32_t)row * (uint32_t)K * 2u;
      slab[j] = (uint32_t)__builtin_amdgcn_readfirstlane(R0 * BK * 2);
    }
  }
  // k-tile starting at k0 into the tile at LDS byte address tile_lds
  __device__ __forceinline__ void issue(uint32_t tile_lds, int k0, int K) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      int kk = k0 + lc8[j];
      if (kk >= K) kk = 0;  // in-bounds dummy; zeroed in LDS by zero_k_tail
      dma16<NT>(base, row_off[j] + (uint32_t)kk * 2u, tile_lds + slab[j]);
    }
  }
};

template <typename T>
__device__ __forceinline__ void st_out(T* p, T v) {
  if constexpr (GEMM_STREAM_Y) __builtin_nontemporal_store(v, p);
  else *p = v;
}
template <typename T>
__device__ __forceinline__ T ld_out(const T* p) {
  if constexpr (GEMM_STREAM_Y) return __builtin_nontemporal_load(p);
  else return *p;
}

// Zero the 16-byte chunks of a staged tile that lie beyond K (last k-tile only).
template <int ROWS, int BK>
__device__ __forceinline__ void zero_k_tail(bf16_t* tile, int k0, int K, int tid, int nthreads) {
  constexpr int CPR = BK / 8;
  for (int e = tid; e < ROWS * CPR; e += nthreads) {
    const int row = e / CPR, pc = e % CPR, lc = swz<BK>(row, pc);
    if (k0 + lc * 8 >= K) *(u32x4_t*)(tile + row * BK + pc * 8) = u32x4_t{0, 0, 0, 0};
  }
}

// WM x WN waves split the block tile BM x BN; k advances BK per stage and
// STAGES k-tiles live in the LDS ring (STAGES - 1 in flight while one feeds
// the MFMAs); OCC = waves per SIMD it is built for (bounds the registers).
// ASTG = 3 (with STAGES = 2) gives the activation operand a third slot of its
// own: its copies are issued one k-tile ahead of the weights' copies.
// PF_Y (residual update only): the fp32 values the epilogue adds to are loaded
// into registers while the last k-tile is copied and multiplied, so their
// memory latency is hidden instead of being paid after the k-loop.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int OCC, bool PF_Y = false,
          bool STREAM_X = GEMM_STREAM_X, bool RES = false, int ASTG = STAGES>
__global__ __launch_bounds__(WM * WN * 64, OCC) void gemm_bf16_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, int M, int K, int N,
    void* __restrict__ Y, int epi, bf16_t* __restrict__ Ybf, const uint8_t* __restrict__ rmask,
    const float* __restrict__ Rsrc, const int32_t* __restrict__ Rrow, int64_t Rrows) {
  constexpr int NW = WM * WN;
  constexpr int CPS = DmaPlan<BM, NW, BK, true>::PER + DmaPlan<BN, NW, BK, false>::PER;  // copies per thread per k-tile
  static_assert(STAGES >= 2 && STAGES <= 5, "wait_dma_ktile handles at most three later k-tiles in flight");
  constexpr int NT = NW * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int STAGE_ELEMS = (BM + BN) * BK;
  // SPLIT: ASTG activation slots beside STAGES weight slots; the activation
  // copies run one k-tile further ahead than the weight copies
  constexpr bool SPLIT = ASTG != STAGES;
  static_assert(!SPLIT || (STAGES == 2 && ASTG == 3), "split ring: 3 activation and 2 weight slots");
  constexpr int RING_ELEMS = SPLIT ? ASTG * BM * BK + STAGES * BN * BK : STAGES * STAGE_ELEMS;
  constexpr int PA = DmaPlan<BM, NW, BK, true>::PER;  // activation copies per thread per k-tile

  __shared__ __attribute__((aligned(1024))) bf16_t smem[RING_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

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
    // block-wide OR through the (not yet used) ring, so the kernel needs no
    // LDS beyond the ring
    int* flag = (int*)smem;
    if (tid == 0) *flag = 0;
    __syncthreads();
    for (int rr = tid; rr < BM; rr += NT)
      if (m0 + rr < M && rmask[m0 + rr]) *flag = 1;
    __syncthreads();
    tile_live = *flag != 0;
    __syncthreads();  // read before the first copies overwrite it
  }

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = tile_live ? (K + BK - 1) / BK : 0;
  const bool k_tail = (K % BK) != 0;
  DmaPlan<BM, NW, BK, STREAM_X> planA;
  DmaPlan<BN, NW, BK, false> planB;
  planA.init(X, M, K, m0, wave, lane);
  planB.init(W, N, K, n0, wave, lane);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  // k order: each round of co-resident workgroups (256 per CU slot) walks k
  // in the opposite direction to the previous round, so the weight k-tiles it
  // needs first are the ones the previous round used last (still in L2).
  const bool krev = GEMM_KREV && ((blockIdx.x / (256 * (OCC >= 4 ? OCC / 2 : 1))) & 1);
  auto kidx = [&](int i) { return krev ? nk - 1 - i : i; };
  auto issue = [&](int i) {  // the i-th k-tile in walk order into ring slot i % STAGES
    const uint32_t b = lds_base + (uint32_t)((i % STAGES) * STAGE_ELEMS * 2);
    planA.issue(b, kidx(i) * BK, K);
    planB.issue(b + BM * BK * 2, kidx(i) * BK, K);
  };
  auto a_slot = [&](int i) { return SPLIT ? smem + (i % ASTG) * (BM * BK) : smem + (i % STAGES) * STAGE_ELEMS; };
  auto b_slot = [&](int i) {
    return SPLIT ? smem + ASTG * (BM * BK) + (i % STAGES) * (BN * BK) : smem + (i % STAGES) * STAGE_ELEMS + BM * BK;
  };
  auto issue_a = [&](int i) { planA.issue(lds_base + (uint32_t)((i % ASTG) * BM * BK * 2), kidx(i) * BK, K); };
  auto issue_b = [&](int i) {
    planB.issue(lds_base + (uint32_t)((ASTG * BM * BK + (i % STAGES) * BN * BK) * 2), kidx(i) * BK, K);
  };

  const int r = lane & 31, g = lane >> 5;
  // epilogue geometry: a wave's accumulator leaves in row segments of WTN
  // columns, LPR lanes per row, RPI rows per instruction
  constexpr int LPR = WTN / 4;
  constexpr int RPI = 64 / LPR;
  constexpr int NY = FM * (32 / RPI);  // 16-byte pieces of the fp32 stream per lane (PF_Y)
  const int prow = lane / LPR, pcol = (lane % LPR) * 4;
  // the fp32 values the accumulate epilogue adds to: Y itself, or row Rrow[m]
  // (row m when Rrow is null) of a separate [Rrows, N] source -- the residual
  // stream started from a gathered row; an index outside [0, Rrows) gives NaN
  // (RES: a separate instantiation, so the plain update keeps its loads unconditional)
  auto res_at = [&](int m, int n) -> f32x4_t {
    if constexpr (!RES) {
      return ld_out((const f32x4_t*)((const float*)Y + (int64_t)m * N + n));
    } else {
      const int64_t src = Rrow ? (int64_t)Rrow[m] : (int64_t)m;
      if (src < 0 || src >= Rrows) {
        KALM_DBG(KALM_DBG_SRC_ROW);
        return f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      }
      return *(const f32x4_t*)(Rsrc + src * N + n);
    }
  };
  // PF_Y: piece i = j (32 / RPI) + rr / RPI of this lane's share of the fp32
  // stream is row m0 + wm WTM + 32 j + rr + prow, columns n .. n + 3.  All NY
  // pieces are loaded unconditionally, from the clamped in-range row and column
  // (pieces outside the output are loaded but never stored), so that exactly NY
  // vector loads follow the last k-tile's copies -- the wait at the last k-tile
  // counts on that -- and no branch around them makes the compiler drain the
  // copies first.  RES: each piece's source row is read in the prologue (the
  // first k-tile's wait completes it), so the pieces' loads do not wait for an
  // index load inside the k-loop; a source row outside [0, Rrows) is loaded
  // from Y's own row instead and replaced by NaN in the epilogue (bit i of sbad).
  f32x4_t yold[PF_Y ? NY : 1];
  int32_t srow[PF_Y && RES ? NY : 1];
  uint32_t sbad = 0;
  auto piece_row = [&](int i) { return m0 + wm * WTM + (i / (32 / RPI)) * 32 + (i % (32 / RPI)) * RPI + prow; };
  if constexpr (PF_Y && RES) {
    if (Rrow) {
#pragma unroll
      for (int i = 0; i < NY; ++i) srow[i] = Rrow[min(piece_row(i), M - 1)];
    } else {
#pragma unroll
      for (int i = 0; i < NY; ++i) srow[i] = min(piece_row(i), M - 1);
    }
  }
  auto load_yold = [&]() {
    const int nc = min(n0 + wn * WTN + pcol, N - 4);
#pragma unroll
    for (int i = 0; i < NY; ++i) {
      const int mc = min(piece_row(i), M - 1);
      const float* yrow = (const float*)Y + (int64_t)mc * N + nc;
      if constexpr (!RES) {
        yold[i] = ld_out((const f32x4_t*)yrow);
      } else {
        const int64_t src = srow[i];
        const bool bad = src < 0 || src >= Rrows;
        sbad |= (uint32_t)bad << i;
        // streaming load, like the plain update's: the gathered rows (re-read
        // once per passage) are kept from displacing the k-loop's operand tiles
        // in L2 (first layer at the Small shape: 3.62 -> 3.40-3.45 ms, A/B)
        yold[i] = ld_out((const f32x4_t*)(bad ? yrow : Rsrc + src * N + nc));
      }
    }
  };
  if constexpr (SPLIT) {
    // copy order: A0 B0 A1, then per k-tile kt: B(kt+1) A(kt+2) -- so when
    // k-tile kt starts, only A(kt+1) (issued last) may still be in flight
    if (nk > 0) {
      issue_a(0);
      issue_b(0);
    }
    if (nk > 1) issue_a(1);
  } else {
    for (int kt = 0; kt < STAGES - 1 && kt < nk; ++kt) issue(kt);
  }
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's copies of k-tile kt are done once at most those of the
    // (up to two) later k-tiles already issued are outstanding -- and, at the
    // last k-tile with PF_Y, the NY loads of the fp32 stream issued after them
    if (PF_Y && kt == nk - GEMM_PF_DIST && kt >= 1 && STAGES == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NY) : "memory");  // the copy is older than the NY loads
    else if (SPLIT && kt + 1 < nk)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PA) : "memory");  // A(kt + 1) may stay in flight
    else wait_dma_ktile<CPS>(SPLIT ? 0 : min(nk - 1 - kt, STAGES - 2));
    __syncthreads();  // k-tile kt visible to all waves; slot of k-tile kt-1 free
    bf16_t* cur = a_slot(kt);
    bf16_t* curb = b_slot(kt);
    if (k_tail && kidx(kt) == nk - 1) {
      zero_k_tail<BM, BK>(cur, kidx(kt) * BK, K, tid, NT);
      zero_k_tail<BN, BK>(curb, kidx(kt) * BK, K, tid, NT);
      __syncthreads();
    }
    if constexpr (PF_Y && RES) {
      // the source rows (read in the prologue) are complete at the first
      // k-tile's wait: take them here, before more copies are in flight
      if (kt == 0) {
#pragma unroll
        for (int i = 0; i < NY; ++i) asm volatile("" ::"v"(srow[i]));
      }
    }
    if constexpr (SPLIT) {
      if (kt + 1 < nk) issue_b(kt + 1);
      if (kt + 2 < nk) issue_a(kt + 2);
    } else {
      if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    }
    if (PF_Y && kt == max(nk - 1 - GEMM_PF_DIST, 0)) load_yold();
    const bf16_t* a = cur;
    const bf16_t* bb = curb;
    // fragments of k-step s + 1 are read from LDS while the MFMAs of k-step s run
    constexpr int KS = BK / 16;
    bf16x8_t xf[KS][FM], wf[KS][FN];
    auto ld = [&](int s) {
      const int kc = 2 * s + g;
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int row = wm * WTM + j * 32 + r;
        xf[s][j] = *(const bf16x8_t*)(a + row * BK + (swz<BK>(row, kc) << 3));
      }
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int row = wn * WTN + i * 32 + r;
        wf[s][i] = *(const bf16x8_t*)(bb + row * BK + (swz<BK>(row, kc) << 3));
      }
    };
    ld(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) ld(s + 1);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s][i], xf[s][j], acc[i][j], 0, 0, 0);
      if (GEMM_SCHED && s + 1 < KS) {
        constexpr int NR = FM + FN, NM = FM * FN, PER_R = NM / NR > 0 ? NM / NR : 1;
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, PER_R, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM - PER_R * NR > 0 ? NM - PER_R * NR : 0, 0);
      }
    }
  }

  if (PF_Y && nk == 0) load_yold();  // a tile with no k-step (all rows masked) still adds to the stream
  if (RES && PF_Y && sbad) KALM_DBG(KALM_DBG_SRC_ROW);

  // Epilogue through LDS: each wave parks 32 rows x WTN columns of its fp32
  // accumulator at a time (row stride padded by 16 bytes: conflict-free for
  // both the column-wise writes and the row-wise reads), then streams them out
  // row-wise so every global access covers whole 16-byte-aligned row segments
  // (WTN * 4 bytes per row for fp32, WTN * 2 for bf16) instead of 32 short
  // pieces per instruction.
  constexpr int EP_LD = WTN + 4;  // fp32 per parked row
  // waves take turns when all of their parking areas do not fit the ring at once
  constexpr int EP_ROUNDS = (NW * 32 * EP_LD * 4 + RING_ELEMS * 2 - 1) / (RING_ELEMS * 2);
  static_assert(EP_ROUNDS <= 2 && NW % EP_ROUNDS == 0, "epilogue staging fits the ring in two rounds");
  __syncthreads();  // every wave is done reading the ring
  float* park = (float*)smem + (wave / EP_ROUNDS) * (32 * EP_LD);
#pragma unroll
  for (int round = 0; round < EP_ROUNDS; ++round) {
  if (EP_ROUNDS > 1 && round > 0) __syncthreads();  // the previous round's waves are done with the area
  if (wave % EP_ROUNDS != round) continue;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4_t*)(park + r * EP_LD + i * 32 + 8 * q + 4 * g) =
            f32x4_t{acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    const int n = n0 + wn * WTN + pcol;
#pragma unroll
    for (int rr = 0; rr < 32; rr += RPI) {
      const int m = m0 + wm * WTM + j * 32 + rr + prow;
      f32x4_t v = *(const f32x4_t*)(park + (rr + prow) * EP_LD + pcol);
      if (m < M && n < N) {
        if (rmask && !rmask[m]) v = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int64_t off = (int64_t)m * N + n;
        // outputs are written once (and the fp32 stream read once): non-temporal
        if (epi == EPI_BF16) {
          st_out((u32x2_t*)((bf16_t*)Y + off), u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
        } else {
          f32x4_t* yp = (f32x4_t*)((float*)Y + off);
          if (epi == EPI_F32_ACC) {
            if constexpr (PF_Y) {
              const int i = j * (32 / RPI) + rr / RPI;
              v += yold[i];
              if (RES && ((sbad >> i) & 1u))
                v = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            } else {
              v += res_at(m, n);
            }
          }
          st_out(yp, v);
          if (Ybf) st_out((u32x2_t*)(Ybf + off), u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
        }
      }
    }
  }
  }
}

// Persistent variant for large problems: a grid of (256 x workgroups per CU)
// workgroups, each walking its output tiles in rounds (round k: every XCD
// holds 32 consecutive tiles, so tiles that share activation rows run side by
// side).  The LDS ring continues across tiles: the first k-tile of the next
// tile is copied while the current tile's epilogue runs, so no tile starts
// on a cold pipeline.  The epilogue parks each wave's fp32 accumulator in the
// ring slot just consumed (32 rows x WTN, 16-byte chunks XOR-swizzled by row),
// which the in-flight copy does not touch.
//
// GELU (gated MLP): W holds the gate rows and Wu the up rows of an MLP of width
// I = N / 2.  Output tile t covers BN / 2 gate columns and the BN / 2 up
// columns of the same units (the first half of the tile's weight rows come
// from W, the second from Wu), so the epilogue pairs each gate value with its
// up value and writes A[m, j] = gelu(x_m . wg_j) * (x_m . wu_j) as bf16 into Y
// ([M, I]); the fp32 products never leave the CU.
template <int BM, int BN, int WM, int WN, int BK, int OCC, bool GELU = false>
__global__ __launch_bounds__(WM * WN * 64, OCC) void gemm_bf16_persistent(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, int M, int K, int N, void* __restrict__ Y, int epi,
    bf16_t* __restrict__ Ybf, const bf16_t* __restrict__ Wu = nullptr) {
  constexpr int STAGES = 2;
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int STAGE_ELEMS = (BM + BN) * BK;
  constexpr int CPR = BK / 8, RPI_D = 64 / CPR;   // copy plan: chunks per row, rows per instruction
  constexpr int PER_A = BM / RPI_D / NW, PER_B = BN / RPI_D / NW;
  constexpr int CPS = PER_A + PER_B;             // copies per thread per k-tile
  static_assert(NW * 32 * WTN * 4 <= STAGE_ELEMS * 2, "a wave's parked rows fit one ring slot");
  static_assert(WTN % 64 == 0, "park swizzle: rows of 16 or 32 chunks");
  static_assert(!GELU || (WN % 2 == 0 && (BN / 2) % WTN == 0), "GELU: gate and up halves of a tile on separate waves");

  __shared__ __attribute__((aligned(1024))) bf16_t smem[STAGES * STAGE_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int r = lane & 31, g = lane >> 5;

  const int tiles_n = (N + BN - 1) / BN;
  const int tiles_m = (M + BM - 1) / BM;
  const int total = tiles_m * tiles_n;
  const int grid = gridDim.x;                    // a multiple of 8
  const int per = total / 8;
  auto tile_of = [&](int vb) { return (vb < per * 8) ? (vb % 8) * per + vb / 8 : vb; };
  const int nk = (K + BK - 1) / BK;
  const bool k_tail = (K % BK) != 0;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  // copy the k-tile of index kk (k0 = kk * BK) of output tile t into ring slot `slot`
  auto issue = [&](int t, int kk, int slot) {
    const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
    const uint32_t b = lds_base + (uint32_t)(slot * STAGE_ELEMS * 2);
    const int rr = lane / CPR;
    const int k0 = kk * BK;
    const uint64_t xa = uniform64((uint64_t)(uintptr_t)(X + (int64_t)m0 * K));
    // GELU: rows [0, BN/2) of the weight tile are gate units n0/2.., rows [BN/2, BN) the same up units
    const int g0 = n0 / 2, nu = N / 2;
    const uint64_t wa = uniform64((uint64_t)(uintptr_t)(W + (int64_t)(GELU ? g0 : n0) * K));
    const uint64_t wua = GELU ? uniform64((uint64_t)(uintptr_t)(Wu + (int64_t)g0 * K)) : 0;
#pragma unroll
    for (int j = 0; j < PER_A + PER_B; ++j) {
      const bool isA = j < PER_A;
      const int jj = isA ? j : j - PER_A;
      const int R0 = RPI_D * (wave * (isA ? PER_A : PER_B) + jj);
      const bool up = GELU && !isA && R0 >= BN / 2;  // wave-uniform
      const int row = isA ? min(m0 + R0 + rr, M - 1) - m0
                          : (GELU ? min(g0 + (up ? R0 - BN / 2 : R0) + rr, nu - 1) - g0 : min(n0 + R0 + rr, N - 1) - n0);
      int kk8 = k0 + swz<BK>(R0 + rr, lane % CPR) * 8;
      if (kk8 >= K) kk8 = 0;  // in-bounds dummy; zeroed in LDS by zero_k_tail
      const uint32_t off = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)kk8 * 2u;
      const uint32_t dst = b + (isA ? 0u : (uint32_t)(BM * BK * 2)) + (uint32_t)__builtin_amdgcn_readfirstlane(R0 * BK * 2);
      dma16(GELU && !isA ? uniform64(up ? wua : wa) : (isA ? xa : wa), off, dst);
    }
  };

  int vb = blockIdx.x;
  if (vb >= total) return;
  int gk = 0;  // k-tiles consumed by this workgroup (ring position)
  for (int kt = 0; kt < STAGES - 1 && kt < nk; ++kt) issue(tile_of(vb), kt, kt % STAGES);
  // k order: odd rounds walk k downwards, so a round starts on the weight
  // k-tiles the previous round used last (still in its XCD's L2)
  for (int rnd = 0; vb < total; vb += grid, ++rnd) {
    const bool rev = GEMM_PKREV && (rnd & 1);
    const bool rev_next = GEMM_PKREV && !(rnd & 1);
    auto kix = [&](int kt) { return rev ? nk - 1 - kt : kt; };
    const int t = tile_of(vb);
    const int m0 = (t / tiles_n) * BM, n0 = (t % tiles_n) * BN;
    const int vb_next = vb + grid;
    const bool has_next = vb_next < total;
    f32x16_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    for (int kt = 0; kt < nk; ++kt, ++gk) {
      // this k-tile's copies (issued one step earlier) are complete; vmcnt also
      // counts the previous tile's epilogue stores, which are waited for here
      wait_dma_ktile<CPS>(0);
      __syncthreads();  // k-tile visible to all waves; the other slot is free
      bf16_t* cur = smem + (gk % STAGES) * STAGE_ELEMS;
      if (k_tail && kix(kt) == nk - 1) {
        zero_k_tail<BM, BK>(cur, kix(kt) * BK, K, tid, NT);
        zero_k_tail<BN, BK>(cur + BM * BK, kix(kt) * BK, K, tid, NT);
        __syncthreads();
      }
      if (kt + 1 < nk) issue(t, kix(kt + 1), (gk + 1) % STAGES);
      else if (has_next) issue(tile_of(vb_next), rev_next ? nk - 1 : 0, (gk + 1) % STAGES);
      const bf16_t* a = cur;
      const bf16_t* bb = cur + BM * BK;
      // fragments of k-step s + 1 are read from LDS while the MFMAs of k-step s run
      constexpr int KS = BK / 16;
      bf16x8_t xf[KS][FM], wf[KS][FN];
      auto ld = [&](int s) {
        const int kc = 2 * s + g;
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int row = wm * WTM + j * 32 + r;
          xf[s][j] = *(const bf16x8_t*)(a + row * BK + (swz<BK>(row, kc) << 3));
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int row = wn * WTN + i * 32 + r;
          wf[s][i] = *(const bf16x8_t*)(bb + row * BK + (swz<BK>(row, kc) << 3));
        }
      };
      ld(0);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + 1 < KS) ld(s + 1);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s][i], xf[s][j], acc[i][j], 0, 0, 0);
        if (GEMM_SCHED && s + 1 < KS) {
          // interleave the FM + FN fragment reads of the next step among this step's MFMAs
          constexpr int NR = FM + FN, NM = FM * FN, PER_R = NM / NR > 0 ? NM / NR : 1;
#pragma unroll
          for (int q = 0; q < NR; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, PER_R, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, NM - PER_R * NR > 0 ? NM - PER_R * NR : 0, 0);
        }
      }
    }
    // ---- epilogue: park in the slot just consumed ((gk - 1) % STAGES); the
    // copy in flight targets the other slot
    __syncthreads();  // every wave is done reading the consumed slot
    float* park = (float*)(smem + ((gk - 1) % STAGES) * STAGE_ELEMS) + wave * (32 * WTN);
    constexpr int LPR = WTN / 4;  // lanes per row (16 bytes of fp32 each) = 16 chunks
    constexpr int RPI = 64 / LPR;
    const int prow = lane / LPR, pch = lane % LPR;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = (8 * i + 2 * q + g) ^ (r & 15);
          *(f32x4_t*)(park + r * WTN + ch * 4) =
              f32x4_t{acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
      if constexpr (GELU) {
        // a gate wave (wn < WN/2) and its up partner (wave + WM WN/2) park the
        // same units; each of the two writes the activation of half of them
        // (the gate wave the first WTN/2 columns); parks are reused next round
        __syncthreads();
        constexpr int HL = WTN / 8;  // lanes per row over half the columns
        const bool is_up = wn >= WN / 2;
        const float* pg = is_up ? park - (WN / 2) * WM * (32 * WTN) : park;
        const float* pu = pg + (WN / 2) * WM * (32 * WTN);
        const int c = (is_up ? HL : 0) + lane % HL;  // 16-byte chunk of the 64-column block
        const int nu = N / 2, n = n0 / 2 + (wn % (WN / 2)) * WTN + c * 4;
#pragma unroll
        for (int rr = 0; rr < 32; rr += 64 / HL) {
          const int prr = rr + lane / HL;
          const int m = m0 + wm * WTM + j * 32 + prr;
          const int o = prr * WTN + ((c ^ (prr & 15)) * 4);
          const f32x4_t gv = *(const f32x4_t*)(pg + o), uv = *(const f32x4_t*)(pu + o);
          if (m < M && n < nu)
            st_out((u32x2_t*)((bf16_t*)Y + (int64_t)m * nu + n),
                   u32x2_t{pack_bf16x2(gated_gelu_tanh(gv[0], uv[0]), gated_gelu_tanh(gv[1], uv[1])),
                           pack_bf16x2(gated_gelu_tanh(gv[2], uv[2]), gated_gelu_tanh(gv[3], uv[3]))});
        }
        __syncthreads();
        continue;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int n = n0 + wn * WTN + pch * 4;
#pragma unroll
      for (int rr = 0; rr < 32; rr += RPI) {
        const int prr = rr + prow;
        const int m = m0 + wm * WTM + j * 32 + prr;
        f32x4_t v = *(const f32x4_t*)(park + prr * WTN + ((pch ^ (prr & 15)) * 4));
        if (m < M && n < N) {
          const int64_t off = (int64_t)m * N + n;
          if (epi == EPI_BF16) {
            st_out((u32x2_t*)((bf16_t*)Y + off), u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
          } else {
            f32x4_t* yp = (f32x4_t*)((float*)Y + off);
            if (epi == EPI_F32_ACC) v += ld_out(yp);
            st_out(yp, v);
            if (Ybf) st_out((u32x2_t*)(Ybf + off), u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// fp32 path (the small fp32 sanity workload): 64x64 tiles, 4x4 outputs per thread.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W, int M, int K,
                                                       int N, float* __restrict__ Y, int accumulate,
                                                       const uint8_t* __restrict__ rmask,
                                                       const float* __restrict__ Rsrc,
                                                       const int32_t* __restrict__ Rrow, int64_t Rrows) {
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
    const int64_t src = Rrow ? (int64_t)Rrow[m] : (int64_t)m;
    const bool src_ok = !Rsrc || (src >= 0 && src < Rrows);
    if (accumulate && !src_ok && tx == 0) KALM_DBG(KALM_DBG_SRC_ROW);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = row_ok ? acc[i][j] : 0.f;
      float* yp = Y + (int64_t)m * N + n;
      if (accumulate) v += !Rsrc ? *yp : (src_ok ? Rsrc[src * N + n] : __builtin_nanf(""));
      *yp = v;
    }
  }
}

}  // namespace

KALM_DBG_TAKE_DEFINE(dbg_take_gemm)

namespace kalm {

void launch_linear_bf16(const bf16_t* X, const bf16_t* W, int M, int K, int N, void* Y, bool y_f32,
                        bool accumulate, bf16_t* Y_bf16, const uint8_t* rmask, hipStream_t s, const float* Rsrc,
                        const int32_t* Rrow, int64_t Rrows) {
  const int epi = !y_f32 ? EPI_BF16 : (accumulate ? EPI_F32_ACC : EPI_F32);
  const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  // A plain residual update (no gathered rows) with a long k-loop goes to the
  // persistent 256 x 256 kernel: its tiles need half the operand bytes per
  // output of the 128 x 128 ones, which outweighs an epilogue it cannot hide
  // behind a second workgroup.  Measured: at K = 2048, H = 2560 (the Long/wide
  // stack) 39.7 against 45.6 ms per launch; at K = 1024 (Small) 3.78 against 3.12.
  const bool res_persist = GEMM_PERSIST && !Rsrc && !rmask && K >= GEMM_RES_PERSIST_MINK;
  if (big_tiles >= 512 && epi == EPI_F32_ACC && !res_persist) {
    // residual update (reads and writes the fp32 stream): 128 x 128 tiles,
    // two workgroups per CU, so one's epilogue traffic overlaps the other's k-loop
    const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (Rsrc)
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 4, 64, 2, 4, GEMM_PF_Y, GEMM_STREAM_X, true, GEMM_RES_ASTG>), dim3(tiles),
                         dim3(512), 0, s, X, W, M, K, N, Y, epi, Y_bf16, rmask, Rsrc, Rrow, Rrows);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 4, 64, 2, 4, GEMM_PF_Y, GEMM_STREAM_X, false, GEMM_RES_ASTG>), dim3(tiles), dim3(512), 0, s, X, W,
                         M, K, N, Y, epi, Y_bf16, rmask, Rsrc, Rrow, Rrows);
  } else if (big_tiles >= 512 && rmask) {
    // rows with a zero mask byte (padded chunks of the cross projection) are
    // written as 0: 128 x 128 tiles, a tile whose rows are all masked skips its
    // k-loop (the persistent kernel below takes no mask)
    const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 4, 64, 2, 4>), dim3(tiles), dim3(512), 0, s, X, W, M, K, N, Y,
                       epi, Y_bf16, rmask, Rsrc, Rrow, Rrows);
  } else if (big_tiles >= 512 && GEMM_PERSIST) {  // never masked or gathered rows
    // persistent 256 x 256 tiles, one workgroup per CU
    const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
    const int grid = tiles < 256 ? ((tiles + 7) / 8) * 8 : 256;
    hipLaunchKernelGGL((gemm_bf16_persistent<256, 256, 2, 4, 64, 1>), dim3(grid), dim3(512), 0, s, X, W, M, K, N, Y,
                       epi, Y_bf16);
  } else if (big_tiles >= 512) {
    // 256 x 256 tiles, k-tiles of 64 (every copied row a whole 128-byte line), two-slot ring
    const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
#ifdef GEMM_W16
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 4, 4, 64, 2, 4>), dim3(tiles), dim3(1024), 0, s, X, W, M, K, N,
                       Y, epi, Y_bf16, rmask, Rsrc, Rrow, Rrows);
#else
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, 2, 4, 64, 2, 1>), dim3(tiles), dim3(512), 0, s, X, W, M, K, N, Y,
                       epi, Y_bf16, rmask, Rsrc, Rrow, Rrows);
#endif
  } else {  // small problems: more, smaller tiles to fill the 256 CUs
    const int tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (Rsrc)
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 4, 32, 4, 1, false, GEMM_STREAM_X, true>), dim3(tiles),
                         dim3(512), 0, s, X, W, M, K, N, Y, epi, Y_bf16, rmask, Rsrc, Rrow, Rrows);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 4, 32, 4, 1>), dim3(tiles), dim3(512), 0, s, X, W, M, K, N, Y,
                         epi, Y_bf16, rmask, Rsrc, Rrow, Rrows);
  }
}

void launch_linear_gelu_bf16(const bf16_t* X, const bf16_t* Wg, const bf16_t* Wu, int M, int K, int I, bf16_t* A,
                             hipStream_t s) {
  // output tiles of 128 gate + 128 up units (I % 128 == 0, checked by the caller)
  const int tiles = ((M + 255) / 256) * ((2 * I) / 256);
  if (tiles == 0) return;
  const int grid = tiles < 256 ? ((tiles + 7) / 8) * 8 : 256;
  hipLaunchKernelGGL((gemm_bf16_persistent<256, 256, 2, 4, 64, 1, true>), dim3(grid), dim3(512), 0, s, X, Wg, M, K,
                     2 * I, (void*)A, (int)EPI_BF16, (bf16_t*)nullptr, Wu);
}

void launch_linear_f32(const float* X, const float* W, int M, int K, int N, float* Y, bool accumulate,
                       const uint8_t* rmask, hipStream_t s, const float* Rsrc, const int32_t* Rrow, int64_t Rrows) {
  const dim3 grid((N + 63) / 64, (M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, X, W, M, K, N, Y, accumulate ? 1 : 0, rmask, Rsrc, Rrow,
                     Rrows);
}

}  // namespace kalm
