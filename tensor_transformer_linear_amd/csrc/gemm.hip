// K1: bf16 NT GEMM on gfx950 matrix cores with a fused output stage.
//
// C[M,N] = A[M,K] * B[N,K]^T where A is the activation and B a weight shard as
// stored ([out_features, in_features], K contiguous) - the per-rank matmul of a
// column- or row-parallel linear ([deepspeed] SubParamLinearLayer.forward,
// [nanotron] "MLP Module").
//
// A workgroup owns a BM x BN output tile and walks K; each wave owns a WM x WN
// sub-tile of 32x32 blocks computed with v_mfma_f32_32x32x16_bf16 from 16-byte
// LDS reads. Two main loops feed the LDS:
// * direct-to-LDS (the default when K % 32 == 0 and A needs no transform): each
//   32-wide K step goes global -> LDS into a ring of stages, several in flight,
//   through buffer_load_dwordx4 ... lds where a wave's blocks of a stage are
//   contiguous (one M0 and one scalar K offset serve them all), through
//   global_load_lds_dwordx4 otherwise. The 256x256, 256x128, 128x256 and 128x128
//   tiles run eight waves in two groups that ping-pong (one group multiplies while
//   the other reads its next fragments and issues the next loads) and stage two K
//   steps per 128-byte LDS row when K holds whole pairs, so every row fetch is one
//   full cache line. The other tiles double-buffer the operand
//   fragments in registers so the LDS reads of one half-step overlap the MFMAs of
//   the other;
// * register staging (any K % 8 == 0, and the fused RMSNorm): 64-wide K steps
//   go global -> registers -> LDS through two stages; the A slab can be
//   RMS-normalised on its way into LDS.
// The output stage adds the bias, applies GELU, rounds once and stores bf16
// or f32 at the (possibly remapped) output column, or adds into f32.
//
// A per-head row map lets a launch read a slice of every head's weight rows (the
// query columns of a fused q_wi weight), and the SwiGLU mode pairs each output
// column's gate and value rows in one tile: the output stage then stores
// bf16(swish(gate) * value) at a per-head output column ([palm] the q_wi and
// SwiGLU steps). Both are compiled only into the MAPPED instantiations.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int BK = 64;
constexpr int ROW_BYTES = BK * 2;

// LDS byte offset of 16-byte chunk kc (0..7) of tile row `row`. The LDS serves a wave's
// ds_read_b128 sixteen lanes at a time across 64 four-byte banks (256 bytes); the 16 lanes
// read 16 consecutive rows at one logical chunk. Rows are 128 bytes, so row parity picks the
// half of the 256-byte bank window and (row / 2) % 8 permutes the chunk within the half:
// the 16 reads land on 16 distinct bank groups. The 8 lanes that write one row also cover 8
// distinct chunks.
__device__ __forceinline__ int lds_off(int row, int kc) { return row * ROW_BYTES + ((kc ^ ((row >> 1) & 7)) << 4); }

// bf16(bf16(a * r) * t) (or bf16(a * r) without a scale) on eight packed values.
__device__ __forceinline__ u32x4_t rms_apply(u32x4_t a, float r, u32x4_t t, bool has_t) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = bf16_lo(a[i]) * r;
    float hi = bf16_hi(a[i]) * r;
    uint32_t n = pack_bf16x2(lo, hi);
    if (has_t) n = pack_bf16x2(bf16_lo(n) * bf16_lo(t[i]), bf16_hi(n) * bf16_hi(t[i]));
    o[i] = n;
  }
  return o;
}

// Logical output column fed by tile-local B row r of a tile whose first output column is n0.
// A SwiGLU tile covers BN / 2 output columns: rows [0, BN / 2) are their gates and rows
// [BN / 2, BN) their values. MAPPED = false compiles the plain kernels (row c for column c, no
// SwiGLU), so the per-head map costs them nothing.
template <int BN, bool MAPPED>
__device__ __forceinline__ int tile_b_col(const GemmProblem& p, int n0, int r) {
  if constexpr (!MAPPED) return n0 + r;
  return n0 + (p.ep.glu && r >= BN / 2 ? r - BN / 2 : r);
}

// B row of tile-local row r (columns past N read the last column's row: their outputs are never
// stored): the logical column, through the per-head row map, plus the value offset.
template <int BN, bool MAPPED>
__device__ __forceinline__ int tile_b_row(const GemmProblem& p, int n0, int r) {
  const int c = min(tile_b_col<BN, MAPPED>(p, n0, r), p.N - 1);
  if constexpr (!MAPPED) return c;
  int row = c;
  if (p.b_head_w > 0) {
    const int h = c / p.b_head_w;
    row = h * p.b_head_pitch + p.b_head_off + (c - h * p.b_head_w);
  }
  if (p.ep.glu && r >= BN / 2) row += p.ep.glu_off;
  return row;
}

// Output element of logical column c in a row (the per-head placement, if any).
__device__ __forceinline__ int64_t head_out_col(const GemmEpilogue& ep, int c) {
  if (ep.c_head_w <= 0) return c;
  const int h = c / ep.c_head_w;
  return (int64_t)h * ep.c_head_pitch + ep.c_head_off + (c - h * ep.c_head_w);
}

// Output-stage modes. A kernel built for one of the fixed modes carries only that path: the
// generic stage's code (GELU, float32 and accumulate, fp8 scales, per-element fallbacks)
// measured 18 us of fixed cost per launch on the 32768 x 3072 GEMM when it is not needed.
constexpr int EPI_GENERIC = 0;    // every mode decided at run time
constexpr int EPI_BF16 = 1;       // bf16 output, no activation, no fp8 scales (bias as given)
constexpr int EPI_BF16_GELU = 2;  // bf16 output, exact GELU, no fp8 scales (bias as given)
constexpr int EPI_FP8_BF16 = 3;   // bf16 output, fp8 row and channel scales, no activation (bias as given)
constexpr int EPI_F32 = 4;        // float32 output, no activation, no fp8 scales (bias and accumulate as given)

// The output is written once and not read back by the kernel: its whole-chunk stores are
// non-temporal (measured 0.5-2% faster than ordinary stores on the GEMM shapes).
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_nt;

// The segment holding local column c: the shift and end of the first segment that ends past
// it, or `none`. Every index is a constant (the loop runs backwards over all TP_MAX_SUBPARAMS
// slots, so the first match is the one kept): a loop-variable index into the kernel argument's
// arrays makes the compiler copy the whole argument block to scratch.
struct SegHit {
  int delta, end;
};
__device__ __forceinline__ SegHit seg_of(const GemmEpilogue& ep, int c, SegHit none) {
  SegHit h = none;
#pragma unroll
  for (int sg = TP_MAX_SUBPARAMS - 1; sg >= 0; --sg)
    if (sg < ep.n_seg && c < ep.seg_end[sg]) h = SegHit{ep.seg_delta[sg], ep.seg_end[sg]};
  return h;
}

// Output columns col .. col + 3 of an epilogue chunk: the segment shift of the first, whether
// all four share its segment and lie below N, and their column scales and bias. Indices past N
// clamp to column N - 1 (N >= 1), so the loads need no per-element branch and issue together;
// values past N are never stored.
struct ChunkCols {
  int col, d;
  bool whole;
  float cs[4], bs[4];
};
template <bool MAY_SCALE>
__device__ __forceinline__ ChunkCols chunk_cols(const GemmEpilogue& ep, int col, int N) {
  ChunkCols c;
  c.col = col;
  c.d = 0;
  const SegHit h = seg_of(ep, col, {0, N});
  c.d = h.delta;
  c.whole = col + 4 <= h.end && col + 4 <= N;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c.cs[e] = 1.0f;
    c.bs[e] = 0.0f;
  }
  if (MAY_SCALE && ep.row_scale != nullptr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c.cs[e] = ep.col_scale[min(col + e, N - 1)];
  }
  if (ep.bias != nullptr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c.bs[e] = bf16_to_f32(ep.bias[min(col + e, N - 1)]);
  }
  return c;
}

// Output stage of the bf16-output modes without fp8 scales (EPI_BF16, EPI_BF16_GELU): bias and
// GELU are applied in registers, each value is rounded once, and the band is parked in LDS as
// bf16, half the bytes of the float32 stage below. Lanes 2c and 2c + 1 hold columns 2c and 2c + 1
// of the same rows, and rows R(v) and R(v + 1) are adjacent for even v: the pair swaps one value
// (a DPP move), then the even lane writes both columns of row R(v) and the odd lane both columns
// of row R(v + 1), one 32-bit word each. The read-back takes eight columns (16 bytes) per thread.
// The values and their rounding are those of the float32 stage, so the outputs are identical.
// Only the paired-row kernels call it: `smem` is their free 160 KB ring, and the stage is the
// kernel's last use of it.
template <int BM, int BN, int WAVES_M, int WAVES_N, int FM, int FN, bool GELU>
__device__ __forceinline__ void gemm_store_tile_bf16(const GemmProblem& p, f32x16_t (&acc)[FM][FN],
                                                     unsigned char* smem, int m0, int n0, int wm, int wn, int lane,
                                                     int tid) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int SROW = BN + 8;        // staged row pitch in bf16 values (a 16-byte bank offset)
  constexpr int SROWS = WAVES_M * 32;  // staged rows per band
  constexpr int C8 = BN / 8;           // eight-column chunks per staged row
  constexpr int Q = SROWS * C8 / NT;   // chunks per thread per band
  static_assert(SROWS * C8 % NT == 0 && NT % C8 == 0, "band chunks must divide evenly, one column per thread");
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
  const GemmEpilogue& ep = p.ep;
  const int M = p.M, N = p.N;
  float bias[FN];  // this lane's bias in each 32-column block
#pragma unroll
  for (int j = 0; j < FN; ++j)
    bias[j] = ep.bias != nullptr ? bf16_to_f32(ep.bias[min(n0 + wn * WN + j * 32 + (lane & 31), N - 1)]) : 0.0f;
  // this thread's read-back columns (the same in every pass): their segment, and whether all
  // eight share it and lie below N
  const int c8 = tid % C8, col = n0 + c8 * 8;
  const SegHit hit = seg_of(ep, col, {0, N});
  const bool whole = col + 8 <= hit.end && col + 8 <= N;
  const int odd = lane & 1;
  const int wr_off = odd * (SROW - 1);  // odd lanes write the next row, one column to the left
  // Every band at once when they fit in the 160 KB the paired-row kernels' ring frees (one
  // barrier per tile instead of two per band), else one band at a time.
  constexpr int BAND = SROWS * SROW;
  constexpr int PASS = FM * BAND * 2 <= 160 * 1024 ? FM : 1;  // bands per pass
  auto park = [&](auto ic, int slot) {
    constexpr int i = decltype(ic)::value;
    static_for<FN>([&](auto j) {
      static_for<8>([&](auto vp) {
        constexpr int v = 2 * decltype(vp)::value;
        float a = acc[i][j][v] + bias[j], b = acc[i][j][v + 1] + bias[j];
        if constexpr (GELU) {
          a = gelu_erf(a);
          b = gelu_erf(b);
        }
        const uint32_t ha = f32_to_bf16(a), hb = f32_to_bf16(b);
        // quad_perm [1, 0, 3, 2]: each lane receives its pair partner's value
        const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? ha : hb), 0xB1, 0xF, 0xF, false);
        const uint32_t word = odd ? (recv | (hb << 16)) : (ha | (recv << 16));
        const int r = wm * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        *reinterpret_cast<uint32_t*>(stage + slot * BAND + r * SROW + wn * WN + j * 32 + (lane & 31) + wr_off) = word;
      });
    });
  };
  // stores band i from stage slot `slot`; returns whether a chunk was left to the element-wise pass
  auto drain = [&](int i, int slot) {
    bool partial = false;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int sr = (tid + q * NT) / C8;
      const int row = m0 + (sr >> 5) * WM + i * 32 + (sr & 31);
      if (row < M && col < N) {
        uint16_t* out = reinterpret_cast<uint16_t*>(ep.C) + (int64_t)row * ep.ldc + col + hit.delta;
        if (whole && (reinterpret_cast<uintptr_t>(out) & 15) == 0)
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(stage + slot * BAND + sr * SROW + c8 * 8),
                                      reinterpret_cast<u32x4_t*>(out));
        else
          partial = true;
      }
    }
    return partial;
  };
  // a chunk crossing a segment end or column N, or a misaligned output row
  auto drain_partial = [&](int i, int slot) {
#pragma unroll 1
    for (int q = 0; q < Q; ++q) {
      const int sr = (tid + q * NT) / C8;
      const int row = m0 + (sr >> 5) * WM + i * 32 + (sr & 31);
      if (row >= M || col >= N) continue;
      uint16_t* out = reinterpret_cast<uint16_t*>(ep.C) + (int64_t)row * ep.ldc;
      if (whole && (reinterpret_cast<uintptr_t>(out + col + hit.delta) & 15) == 0) continue;
      const uint16_t* src = stage + slot * BAND + sr * SROW + c8 * 8;
#pragma unroll 1
      for (int e = 0; e < 8 && col + e < N; ++e) out[col + e + seg_of(ep, col + e, {hit.delta, 0}).delta] = src[e];
    }
  };
  if constexpr (PASS == FM && GELU) {
    // GELU makes parking vector-ALU bound: band i + 1 is parked while band i drains, so the
    // drain's LDS reads and stores overlap the next band's arithmetic (one barrier per band)
    park(std::integral_constant<int, 0>{}, 0);
    __syncthreads();
    static_for<FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + 1 < FM) park(std::integral_constant<int, i + 1>{}, i + 1);
      if (drain(i, i)) drain_partial(i, i);
      if constexpr (i + 1 < FM) __syncthreads();
    });
  } else if constexpr (PASS == FM) {
    static_for<FM>([&](auto i) { park(i, decltype(i)::value); });
    __syncthreads();
    bool partial = false;
#pragma unroll
    for (int i = 0; i < FM; ++i) partial |= drain(i, i);
    if (partial) {
#pragma unroll 1
      for (int i = 0; i < FM; ++i) drain_partial(i, i);
    }
    // nothing reads or writes the stage after this: the kernel ends
  } else {
    static_for<FM>([&](auto i) {
      park(i, 0);
      __syncthreads();
      if (drain(i, 0)) drain_partial(i, 0);
      __syncthreads();
    });
  }
}

// Output stage of a BM x BN tile, one 32-row band of every wave at a time. In a 32x32
// accumulator block, lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4 of
// its sixteen values v. Each wave parks its band (32 rows x WN columns) in LDS; the
// workgroup then reads the staged band back four consecutive columns per thread and
// finishes them: bias, GELU, one rounding, the column remap, and a coalesced store (or a
// float32 add). `smem` must hold WAVES_M * 32 * (BN + 4) floats and be free.
template <int BM, int BN, int WAVES_M, int WAVES_N, int FM, int FN, bool MAPPED, int EPI = EPI_GENERIC>
__device__ __forceinline__ void gemm_store_tile(const GemmProblem& p, f32x16_t (&acc)[FM][FN], unsigned char* smem,
                                                int m0, int n0, int wm, int wn, int lane, int tid) {
  if constexpr (!MAPPED && (EPI == EPI_BF16 || EPI == EPI_BF16_GELU)) {
    gemm_store_tile_bf16<BM, BN, WAVES_M, WAVES_N, FM, FN, EPI == EPI_BF16_GELU>(p, acc, smem, m0, n0, wm, wn, lane,
                                                                                 tid);
    return;
  }
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  const int M = p.M, N = p.N;
  constexpr int SROW = BN + 4;                       // staged row pitch in floats (bank offset)
  constexpr int SROWS = WAVES_M * 32;                // staged rows per band
  float* stage = reinterpret_cast<float*>(smem);
  const GemmEpilogue& ep = p.ep;
  // the epilogue's modes: runtime for EPI_GENERIC, fixed at compile time otherwise
  constexpr bool GEN = EPI == EPI_GENERIC;
  const bool scaled = GEN ? ep.row_scale != nullptr : EPI == EPI_FP8_BF16;
  const bool gelu = GEN ? ep.act == TP_ACT_GELU_ERF : EPI == EPI_BF16_GELU;
  const bool out_f32 = GEN ? ep.out_f32 != 0 : EPI == EPI_F32;
  constexpr int C4 = BN / 4;                         // four-column chunks per staged row
  constexpr int CHUNKS = SROWS * C4;
  static_assert(CHUNKS % NT == 0, "band chunks must divide evenly over the workgroup");
  constexpr int Q = CHUNKS / NT;                     // chunks per thread per band
  // A thread's chunk column c4 = (tid + q NT) % C4 is the same in every pass when NT is a
  // multiple of C4 (every eight-wave tile): its segment, column scales and bias are then
  // fetched once per tile.
  constexpr bool FIXED_COL = NT % C4 == 0;
  ChunkCols fixed_cols{};
  if constexpr (FIXED_COL)
    if (!(MAPPED && ep.glu)) fixed_cols = chunk_cols<GEN || EPI == EPI_FP8_BF16>(ep, n0 + (tid % C4) * 4, N);
  static_for<FM>([&](auto i) {
    // this band's row scales (eight-wave tiles), fetched before the staging so their latency
    // overlaps it; other tiles load each chunk's row scale where it is used
    float rsv[FIXED_COL ? Q : 1];
    if constexpr (FIXED_COL) {
      if (!(MAPPED && ep.glu) && scaled) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const int sr = (tid + q * NT) / C4;
          rsv[q] = ep.row_scale[min(m0 + (sr >> 5) * WM + i * 32 + (sr & 31), M - 1)];
        }
      }
    }
    static_for<FN>([&](auto j) {
      static_for<16>([&](auto v) {
        constexpr int vv = v;
        const int r = wm * 32 + (vv >> 2) * 8 + (lane >> 5) * 4 + (vv & 3);
        stage[r * SROW + wn * WN + j * 32 + (lane & 31)] = acc[i][j][vv];
      });
    });
    __syncthreads();
    if (MAPPED && ep.glu) {
      // SwiGLU: the gate of output column n0 + c is staged at column c, its value at BN / 2 + c
      constexpr int C8 = BN / 8;
      constexpr int GCHUNKS = SROWS * C8;
      static_assert(GCHUNKS % NT == 0, "SwiGLU band chunks must divide evenly over the workgroup");
      for (int q = 0; q < GCHUNKS / NT; ++q) {
        const int id = tid + q * NT;
        const int sr = id / C8, c4 = id - sr * C8;
        const int row = m0 + (sr >> 5) * WM + i * 32 + (sr & 31);
        const int col = n0 + c4 * 4;
        if (row < M && col < N) {
          const f32x4_t g = *reinterpret_cast<const f32x4_t*>(stage + sr * SROW + c4 * 4);
          const f32x4_t u = *reinterpret_cast<const f32x4_t*>(stage + sr * SROW + BN / 2 + c4 * 4);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = swiglu_of(g[e], u[e]);
          uint16_t* out = reinterpret_cast<uint16_t*>(ep.C) + (int64_t)row * ep.ldc;
          const int in_head = ep.c_head_w > 0 ? col % ep.c_head_w : 0;
          const bool whole = col + 4 <= N && (ep.c_head_w <= 0 || in_head + 4 <= ep.c_head_w);
          uint16_t* c = out + head_out_col(ep, col);
          if (whole && (reinterpret_cast<uintptr_t>(c) & 7) == 0) {
            const u32x2_nt pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            __builtin_nontemporal_store(pk, reinterpret_cast<u32x2_nt*>(c));
          } else {
            for (int e = 0; e < 4 && col + e < N; ++e) out[head_out_col(ep, col + e)] = f32_to_bf16(y[e]);
          }
        }
      }
      __syncthreads();
      return;
    }
    // Whole, aligned chunks are finished in this loop. A chunk that crosses a segment end or the
    // last column, or whose output is misaligned, is left to the element-wise pass below, which
    // keeps that rare path's code out of the unrolled loop.
    auto finish = [&](f32x4_t val, float rs, const ChunkCols& cc) {
      if (scaled) {  // fp8: dequantise the product
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] *= rs * cc.cs[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (ep.bias != nullptr) val[e] += cc.bs[e];
        if (gelu) val[e] = gelu_erf(val[e]);
      }
      return val;
    };
    auto vector_ok = [&](const ChunkCols& cc, int64_t off) {
      const uintptr_t a = out_f32 ? reinterpret_cast<uintptr_t>(reinterpret_cast<float*>(ep.C) + off)
                                  : reinterpret_cast<uintptr_t>(reinterpret_cast<uint16_t*>(ep.C) + off);
      return cc.whole && (a & (out_f32 ? 15 : 7)) == 0;
    };
    bool partial = false;
    for (int q = 0; q < Q; ++q) {
      const int id = tid + q * NT;
      const int sr = id / C4, c4 = id - sr * C4;
      const int row = m0 + (sr >> 5) * WM + i * 32 + (sr & 31);
      // output column of the chunk's first column, and whether all four share its segment
      const ChunkCols cc = FIXED_COL ? fixed_cols : chunk_cols<GEN || EPI == EPI_FP8_BF16>(ep, n0 + c4 * 4, N);
      if (row < M && cc.col < N) {
        const int64_t off = (int64_t)row * ep.ldc + cc.col + cc.d;
        if (!vector_ok(cc, off)) {
          partial = true;
          continue;
        }
        const float rs = scaled ? (FIXED_COL ? rsv[FIXED_COL ? q : 0] : ep.row_scale[row]) : 1.0f;
        f32x4_t val = finish(*reinterpret_cast<const f32x4_t*>(stage + sr * SROW + c4 * 4), rs, cc);
        if (out_f32) {
          f32x4_t* c4p = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(ep.C) + off);
          if (ep.accumulate) val += *c4p;
          __builtin_nontemporal_store(val, c4p);
        } else {
          const u32x2_nt pk = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
          __builtin_nontemporal_store(pk, reinterpret_cast<u32x2_nt*>(reinterpret_cast<uint16_t*>(ep.C) + off));
        }
      }
    }
    if (partial) {
#pragma unroll 1
      for (int q = 0; q < Q; ++q) {
        const int id = tid + q * NT;
        const int sr = id / C4, c4 = id - sr * C4;
        const int row = m0 + (sr >> 5) * WM + i * 32 + (sr & 31);
        const ChunkCols cc = FIXED_COL ? fixed_cols : chunk_cols<GEN || EPI == EPI_FP8_BF16>(ep, n0 + c4 * 4, N);
        const int col = cc.col;
        if (row >= M || col >= N || vector_ok(cc, (int64_t)row * ep.ldc + col + cc.d)) continue;
        const f32x4_t val = finish(*reinterpret_cast<const f32x4_t*>(stage + sr * SROW + c4 * 4),
                                   scaled ? ep.row_scale[row] : 1.0f, cc);
        const int64_t base = (int64_t)row * ep.ldc;
#pragma unroll 1
        for (int e = 0; e < 4 && col + e < N; ++e) {
          const int de = seg_of(ep, col + e, {cc.d, 0}).delta;
          if (out_f32) {
            float* ce = reinterpret_cast<float*>(ep.C) + base + col + e + de;
            *ce = ep.accumulate ? *ce + val[e] : val[e];
          } else {
            reinterpret_cast<uint16_t*>(ep.C)[base + col + e + de] = f32_to_bf16(val[e]);
          }
        }
      }
    }
    __syncthreads();
  });
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool NORM, bool MAPPED>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_nt_kernel(GemmProblem p, int tiles_m, int tiles_n,
                                                                        int group_m) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int CA = BM * BK / 8 / NT, CB = BN * BK / 8 / NT;
  constexpr int ROWS_PER_PASS = NT / 8;  // tile rows covered by one 16-byte load per thread
  static_assert(FM * 32 == WM && FN * 32 == WN, "wave tile must be whole 32x32 blocks");
  static_assert(CA * NT * 8 == BM * BK && CB * NT * 8 == BN * BK, "tile not evenly loadable");
  constexpr int STAGE = (BM + BN) * ROW_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // Tile of this workgroup: XCD-local logical order, then groups of group_m tile rows
  // walked column by column so that neighbouring tiles share A rows and B columns.
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = group_m * tiles_n;
  const int grp = lid / per_group, first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int in = lid - grp * per_group;
  const int m0 = (first_m + in % gsz) * BM, n0 = (in / gsz) * (MAPPED && p.ep.glu ? BN / 2 : BN);

  const int M = p.M, N = p.N, K = p.K;
  const int kc = tid & 7;          // this thread's 16-byte chunk within a 64-wide K slab
  const int lrow = tid >> 3;       // first tile row this thread loads

  float rr[NORM ? CA : 1];
  const bool has_t = NORM && p.col_t != nullptr;
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int gm = m0 + lrow + i * ROWS_PER_PASS;
      rr[i] = gm < M ? p.row_r[gm] : 0.0f;
    }
  }

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // Out-of-range rows and K chunks load from a clamped (valid) address and are zeroed when
  // they are written to LDS.
  bool a_ok[CA], b_ok[CB];
  int64_t a_off[CA], b_off[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int gm = m0 + lrow + i * ROWS_PER_PASS;
    a_ok[i] = gm < M;
    a_off[i] = (int64_t)(a_ok[i] ? gm : M - 1) * p.lda + kc * 8;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int r = lrow + i * ROWS_PER_PASS;
    b_ok[i] = tile_b_col<BN, MAPPED>(p, n0, r) < N;
    b_off[i] = (int64_t)tile_b_row<BN, MAPPED>(p, n0, r) * p.ldb + kc * 8;
  }
  // One K step's operand pieces in registers.
  struct Regs {
    u32x4_t a[CA], b[CB], t;
  };
  // Issues the loads of step kt (clamped to the last step, so the call is unconditional and
  // the compiler can count the loads in flight); nothing reads them until lstore.
  const int nk = (K + BK - 1) / BK;
  auto gload = [&](int kt, Regs& r) {
    kt = kt < nk ? kt : nk - 1;
    const int k0 = kt * BK;
    const int kk0 = k0 + kc * 8 < K ? k0 : 0;
#pragma unroll
    for (int i = 0; i < CA; ++i) r.a[i] = *reinterpret_cast<const u32x4_t*>(p.A + a_off[i] + kk0);
#pragma unroll
    for (int i = 0; i < CB; ++i) r.b[i] = *reinterpret_cast<const u32x4_t*>(p.B + b_off[i] + kk0);
    if (has_t) r.t = *reinterpret_cast<const u32x4_t*>(p.col_t + kk0 + kc * 8);
  };
  // Writes step kt's pieces into LDS stage `buf` (zeros outside the matrices).
  auto lstore = [&](int buf, int kt, const Regs& r) {
    const bool kok = kt * BK + kc * 8 < K;
    unsigned char* sa = smem + buf * STAGE;
    unsigned char* sb = sa + BM * ROW_BYTES;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      u32x4_t v = (kok && a_ok[i]) ? r.a[i] : zero;
      if constexpr (NORM) v = rms_apply(v, rr[i], r.t, has_t);
      *reinterpret_cast<u32x4_t*>(sa + lds_off(lrow + i * ROWS_PER_PASS, kc)) = v;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i)
      *reinterpret_cast<u32x4_t*>(sb + lds_off(lrow + i * ROWS_PER_PASS, kc)) = (kok && b_ok[i]) ? r.b[i] : zero;
  };

  f32x16_t acc[FM][FN];
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) {
      static_for<16>([&](auto v) { acc[i][j][decltype(v)::value] = 0.0f; });
    });
  });

  const int a_row0 = wm * WM + (lane & 31), b_row0 = wn * WN + (lane & 31);
  const int khalf = lane >> 5;
  auto compute = [&](int buf) {
    const unsigned char* sa = smem + buf * STAGE;
    const unsigned char* sb = sa + BM * ROW_BYTES;
    static_for<BK / 16>([&](auto kk) {
      bf16x8_t af[FM], bfr[FN];
      static_for<FM>([&](auto i) {
        af[i] = __builtin_bit_cast(bf16x8_t,
                                   *reinterpret_cast<const u32x4_t*>(sa + lds_off(a_row0 + i * 32, kk * 2 + khalf)));
      });
      static_for<FN>([&](auto j) {
        bfr[j] = __builtin_bit_cast(bf16x8_t,
                                    *reinterpret_cast<const u32x4_t*>(sb + lds_off(b_row0 + j * 32, kk * 2 + khalf)));
      });
      static_for<FM>([&](auto i) {
        static_for<FN>([&](auto j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        });
      });
    });
  };

  // Pipeline over K steps: one register set and two LDS stages. While step kt is
  // multiplied out of LDS stage kt % 2, the loads of step kt + 1 are in flight; after the
  // MFMAs they are written to the other stage. One barrier per step: the barrier closing
  // step kt - 1 proves that every wave finished reading the stage step kt + 1 overwrites.
  // Loads are unconditional (clamped to the last step) so the compiler keeps them in flight
  // across the MFMAs.
  Regs r0;
  gload(0, r0);
  lstore(0, 0, r0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    gload(kt + 1, r0);
    compute(kt & 1);
    lstore((kt + 1) & 1, kt + 1, r0);
    __syncthreads();
  }

  static_assert(WAVES_M * 32 * (BN + 4) * 4 <= 2 * STAGE, "band staging must fit in the pipeline's LDS");
  gemm_store_tile<BM, BN, WAVES_M, WAVES_N, FM, FN, MAPPED>(p, acc, smem, m0, n0, wm, wn, lane, tid);
}


// Direct-to-LDS variant for K a multiple of 32 and no A transform. Each K step (32 wide)
// of A and B is fetched with global_load_lds_dwordx4: every lane's 16 bytes go straight
// into LDS (M0 base + 16 x lane), so no VGPRs hold operands in flight and the prefetch
// depth is set by LDS: STAGES stages, STAGES - 1 of them loading while one is multiplied.
// LDS rows are 64 bytes (32 bf16 of K); the 16-byte chunk index is XORed with bits 2..3
// of the row, so the sixteen consecutive rows one ds_read_b128 phase reads fall on
// sixteen distinct bank groups. A 1 KB DMA block is 16 rows; lane q of a block fetches the
// global chunk that belongs at its LDS slot (row q / 4, physical chunk q % 4). Rows beyond
// M or N read a clamped row: they only feed outputs that are never stored.
constexpr int DBK = 32;
constexpr int DROW = DBK * 2;  // 64-byte LDS rows

__device__ __forceinline__ int dma_off(int row, int c) { return row * DROW + ((c ^ ((row >> 2) & 3)) << 4); }

typedef __attribute__((address_space(3))) unsigned char lds_byte;

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma_load16(const void* g, lds_byte* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// Buffer-resource form of the same transfer. The LDS destination is M0 plus the instruction
// offset plus 16 * lane, and the instruction offset also moves the global source, so a wave
// whose blocks sit next to each other in LDS sets M0 once per stage and reaches its next
// three blocks through the offset field (at most 4095 bytes); the K advance rides in the
// scalar offset. Raw-buffer word 3 for gfx9: 32-bit data format, no swizzle, no stride.
constexpr int BUF_BACKOFF = 4096;  // the resource base sits this far below the tile's first row
constexpr int BUF_MAX_BLOCKS = 4;  // 1 KB blocks one M0 covers: offsets 0, 1, 2 and 3 KB
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const unsigned char* base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base - BUF_BACKOFF), (short)0, 0x7FFFFFFF, 0x00020000);
}
template <int IMM>
__device__ __forceinline__ void buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, lds_byte* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)lds, 16, voff, soff, IMM, 0);
}

// How a tile's waves split the 1 KB blocks of a stage for buffer loads, each run of a wave's
// blocks contiguous in LDS, within one operand and within one M0's reach:
// 1 = wave w owns blocks [P w, P (w + 1)), all of one operand (P blocks per wave);
// 2 = wave w owns A blocks [PA w, PA (w + 1)) and B blocks NBLK_A + [PB w, PB (w + 1)) (B
//     blocks past the tile's rows are padding that reads a valid row);
// 0 = neither fits: per-lane global_load_lds.
template <int BM, int BN, int NWAVE>
constexpr int tile_buffer_mode() {
  constexpr int na = BM / 16, nb = BN / 16, per_wave = (na + nb + NWAVE - 1) / NWAVE;
  if (na + nb == NWAVE * per_wave && na % per_wave == 0 && per_wave <= BUF_MAX_BLOCKS) return 1;
  constexpr int pa = na / NWAVE, pb = (nb + NWAVE - 1) / NWAVE;
  if (na % NWAVE == 0 && pa + pb == per_wave && pa <= BUF_MAX_BLOCKS && pb <= BUF_MAX_BLOCKS) return 2;
  return 0;
}
template <int BM, int BN, int NWAVE>
constexpr bool tile_uses_buffer_loads() {
  return tile_buffer_mode<BM, BN, NWAVE>() != 0;
}

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

// SCHED selects the main-loop schedule: 0 = every wave multiplies while its own next reads fly
// (fragments double-buffered in registers); 1 = ping-pong between two groups of four waves (one
// wave per SIMD each, eight waves per workgroup): one group multiplies while the other reads
// its next fragments from LDS and issues the next global loads, and the roles swap at every
// barrier, so each SIMD always has a wave issuing MFMAs.
//
// FP8: A and B are E4M3 codes. A stage still holds 64 bytes of every row (64 K values instead
// of 32) and one v_mfma_f32_32x32x64_f8f6f4 per 32x32 block takes the place of the two bf16
// MFMAs: lane l supplies 32 consecutive K bytes (chunks 2 (l / 32) and 2 (l / 32) + 1 of the
// row), the same for A and B. Only the ping-pong schedule handles it.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int SCHED, bool FP8 = false, bool MAPPED = false>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_nt_dma_kernel(GemmProblem p, int tiles_m, int tiles_n,
                                                                            int group_m) {
  static_assert(!FP8 || SCHED == 1, "the fp8 path runs the ping-pong schedule");
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int NWAVE = NT / 64;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int NBLK_A = BM / 16, NBLK = (BM + BN) / 16;  // 1 KB DMA blocks per stage
  constexpr int BLK_PER_WAVE = (NBLK + NWAVE - 1) / NWAVE;
  // Every wave issues the same number of loads per stage (blocks past NBLK load a valid
  // row into padding), so one vmcnt immediate fits all waves.
  constexpr int STAGE = NWAVE * BLK_PER_WAVE * 1024;
  static_assert(FM * 32 == WM && FN * 32 == WN, "wave tile must be whole 32x32 blocks");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "tile rows must fill DMA blocks");
  constexpr int EPI = WAVES_M * 32 * (BN + 4) * 4;
  constexpr int SMEM = STAGES * STAGE > EPI ? STAGES * STAGE : EPI;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = group_m * tiles_n;
  const int grp = lid / per_group, first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int in = lid - grp * per_group;
  const int m0 = (first_m + in % gsz) * BM, n0 = (in / gsz) * (MAPPED && p.ep.glu ? BN / 2 : BN);
  const int M = p.M, N = p.N, K = p.K;
  constexpr int ESZ = FP8 ? 1 : 2;  // bytes per element
  const int nk = K / (DROW / ESZ);    // a stage is 64 bytes of every row

  // Per DMA block this wave issues: the source of this lane's 16 bytes, addressed from the
  // tile's first row of its operand (rows past M or N clamp to the last row, never below the
  // first). Buffer-load modes 1 and 2 give each wave contiguous runs of blocks (one run per
  // operand it loads, one M0 and one resource each); otherwise blocks w, w + NWAVE, ...
  constexpr int MODE = tile_buffer_mode<BM, BN, NWAVE>();
  constexpr int PA = MODE == 1 ? BLK_PER_WAVE : MODE == 2 ? NBLK_A / NWAVE : 0;  // blocks of the first run
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // first block of each run: mode 1, one run (A or B by wave); mode 2, the A run then the B run
  const int run0 = MODE == 2 ? wave_s * PA : wave_s * BLK_PER_WAVE;
  const int run1 = MODE == 2 ? NBLK_A + wave_s * (BLK_PER_WAVE - PA) : run0;
  const int nb_first = tile_b_row<BN, MAPPED>(p, n0, 0);
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(p.A) + (int64_t)m0 * p.lda * ESZ;
  const unsigned char* bbase = reinterpret_cast<const unsigned char*>(p.B) + (int64_t)nb_first * p.ldb * ESZ;
  const __amdgpu_buffer_rsrc_t rsrc0 = buf_rsrc(MODE == 2 || run0 < NBLK_A ? abase : bbase);
  const __amdgpu_buffer_rsrc_t rsrc1 = buf_rsrc(bbase);
  const unsigned char* src[BLK_PER_WAVE];
  uint32_t voff[BLK_PER_WAVE];
  int dst[BLK_PER_WAVE];
#pragma unroll
  for (int b = 0; b < BLK_PER_WAVE; ++b) {
    const int blk = MODE == 0 ? wave + b * NWAVE : b < PA ? run0 + b : run1 + (b - PA);
    const int row = (blk < NBLK_A ? blk : blk - NBLK_A) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);  // logical chunk stored at this lane's slot
    int64_t off;                                 // bytes from the tile's first row
    if (blk < NBLK_A) {
      const int gm = min(m0 + row, M - 1);
      off = ((int64_t)(gm - m0) * p.lda) * ESZ + c * 16;
      src[b] = abase + off;
    } else {
      const int gn = blk < NBLK ? tile_b_row<BN, MAPPED>(p, n0, row) : nb_first;
      off = ((int64_t)(gn - nb_first) * p.ldb) * ESZ + c * 16;
      src[b] = bbase + off;
    }
    voff[b] = (uint32_t)(off + BUF_BACKOFF - (b < PA ? b : b - PA) * 1024);
    dst[b] = blk * 1024;
  }
  // Stage kt (0 <= kt < nk) into ring slot `slot` (kt % STAGES).
  auto issue_at = [&](int kt, unsigned slot) {
    lds_byte* base = (lds_byte*)smem + slot * STAGE;
    if constexpr (MODE != 0) {
      static_for<BLK_PER_WAVE>([&](auto b) {
        constexpr int bi = decltype(b)::value;
        if constexpr (bi < PA)
          buf_load16<bi * 1024>(rsrc0, voff[bi], kt * DROW, base + run0 * 1024);
        else
          buf_load16<(bi - PA) * 1024>(rsrc1, voff[bi], kt * DROW, base + run1 * 1024);
      });
    } else {
#pragma unroll
      for (int b = 0; b < BLK_PER_WAVE; ++b) dma_load16(src[b] + (int64_t)kt * DROW, base + dst[b]);
    }
  };
  auto issue = [&](int kt) {
    kt = kt < nk ? kt : nk - 1;  // clamped: the loop issues unconditionally
    issue_at(kt, (unsigned)kt % STAGES);
  };

  f32x16_t acc[FM][FN];
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) { static_for<16>([&](auto v) { acc[i][j][decltype(v)::value] = 0.0f; }); });
  });
  const int a_row0 = wm * WM + (lane & 31), b_row0 = wn * WN + (lane & 31);
  const int khalf = lane >> 5;
  // Operand fragments of one 16-wide half of a K step: lane l holds row l % 32 of each
  // 32-row block and K values 8 (l / 32) .. +8 of the half.
  struct Frag {
    bf16x8_t a[FM], b[FN];
  };
  // bf16: fragment `half` is the 16-wide half of the stage (chunk 2 half + l / 32); fp8: it is
  // one of the two 16-byte chunks of the lane's 32 K bytes (chunk 2 (l / 32) + half).
  auto read = [&](Frag& f, int stage, int half) {
    const unsigned char* sa = smem + stage * STAGE;
    const unsigned char* sb = sa + BM * DROW;
    const int chunk = FP8 ? khalf * 2 + half : half * 2 + khalf;
    static_for<FM>([&](auto i) {
      f.a[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(sa + dma_off(a_row0 + i * 32, chunk)));
    });
    static_for<FN>([&](auto j) {
      f.b[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(sb + dma_off(b_row0 + j * 32, chunk)));
    });
  };
  // fp8: one MFMA per 32x32 block over the stage's 64 K values, operands from both fragments
  auto mma8 = [&](const Frag& f0, const Frag& f1) {
    static_for<FM>([&](auto i) {
      static_for<FN>([&](auto j) {
        const i32x8_t a = __builtin_bit_cast(
            i32x8_t, __builtin_shufflevector(__builtin_bit_cast(u32x4_t, f0.a[i]), __builtin_bit_cast(u32x4_t, f1.a[i]),
                                             0, 1, 2, 3, 4, 5, 6, 7));
        const i32x8_t b = __builtin_bit_cast(
            i32x8_t, __builtin_shufflevector(__builtin_bit_cast(u32x4_t, f0.b[j]), __builtin_bit_cast(u32x4_t, f1.b[j]),
                                             0, 1, 2, 3, 4, 5, 6, 7));
        // E4M3 x E4M3 (format selectors 0), unit block scales
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 0, 0, 0);
      });
    });
  };
  auto mma = [&](const Frag& f) {
    static_for<FM>([&](auto i) {
      static_for<FN>([&](auto j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
      });
    });
  };
  // s_waitcnt vmcnt(VM) with expcnt and lgkmcnt left open (gfx9 encoding: vmcnt[3:0] |
  // expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]), then a workgroup barrier without a
  // memory fence: a fence would make the compiler drain every outstanding load (vmcnt 0)
  // and serialise the stages. The empty asm statements keep the compiler from moving LDS
  // accesses across the barrier; the scheduling barriers keep the MFMAs on their side.
  auto wait_barrier = [&](auto vm, auto lgkm) {
    constexpr int VM = decltype(vm)::value, LGKM = decltype(lgkm)::value;
    static_assert(VM >= 0 && VM < 64, "vmcnt immediate is six bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (LGKM << 8) | ((VM >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  if constexpr (SCHED == 1) {
    static_assert(WAVES_M == 2 && NWAVE == 8, "ping-pong needs two groups of four waves");
    // Group g = wm: waves 0-3 and 4-7, one wave of each group per SIMD. Group 1 runs one phase
    // behind group 0. Memory phase k: read both halves of stage k, issue stage k + STAGES - 1
    // into the slot of stage k - 1, then wait until this wave's loads of stage k + 1 have
    // landed (at most the STAGES - 2 newer stages outstanding) and its reads are done, and
    // meet the other group at the barrier. Compute phase k: 16 MFMAs, barrier. A group reads
    // stage k only after both groups waited for their loads of it (its own wait one memory
    // phase earlier, the other group's before the barrier between them), and a slot is
    // overwritten two phases after both groups finished reading it. Every wave executes the
    // same number of barriers: the prologue's, 2 per K step, and one extra (group 1 at the
    // start, group 0 at the end).
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s);
    wait_barrier(std::integral_constant<int, (STAGES - 2) * BLK_PER_WAVE>{}, std::integral_constant<int, 15>{});
    if (wm == 1) {
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    Frag f0, f1;
    // K step kt: read slot rs, stage k_in into slot is
    auto step = [&](unsigned rs, int k_in, unsigned is) {
      read(f0, rs, 0);
      read(f1, rs, 1);
      __builtin_amdgcn_sched_barrier(0);  // the reads first: loads issued ahead of them stall this wave
      issue_at(k_in, is);
      wait_barrier(std::integral_constant<int, (STAGES - 2) * BLK_PER_WAVE>{}, std::integral_constant<int, 0>{});
      __builtin_amdgcn_s_setprio(1);  // the multiplying wave first: the other group only issues memory work
      if constexpr (FP8) {
        mma8(f0, f1);
      } else {
        mma(f0);
        mma(f1);
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // STAGES steps per iteration while no issued stage needs clamping: every ring slot is a
    // constant, so the LDS addresses are immediates and M0 a constant
    int kt = 0;
    for (; kt + 2 * STAGES - 1 <= nk; kt += STAGES)
      static_for<STAGES>([&](auto u) {
        constexpr unsigned U = decltype(u)::value;
        step(U, kt + U + STAGES - 1, (U + STAGES - 1) % STAGES);
      });
    for (; kt < nk; ++kt) {
      const int k_in = kt + STAGES - 1 < nk ? kt + STAGES - 1 : nk - 1;  // clamped past the last stage
      step((unsigned)kt % STAGES, k_in, (unsigned)k_in % STAGES);
    }
    if (wm == 0) {
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    gemm_store_tile<BM, BN, WAVES_M, WAVES_N, FM, FN, MAPPED>(p, acc, smem, m0, n0, wm, wn, lane, tid);
    return;
  }

  if constexpr (!FP8) {
  // Software pipeline over K steps, two register sets of fragments. Step kt enters with the
  // first half of stage kt in f0; it reads the second half into f1 and multiplies f0 (the
  // MFMAs cover the LDS latency); waits until stage kt + 1 has landed in every wave (at most
  // the STAGES - 3 newer stages of this wave outstanding) behind a barrier, which also proves
  // every wave is done with stage kt - 1, whose slot the next DMA overwrites; issues stage
  // kt + STAGES - 1; reads the first half of stage kt + 1 into f0 and multiplies f1.
  static_assert(STAGES >= 3, "the pipeline reads one stage ahead");
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(s);
  wait_barrier(std::integral_constant<int, (STAGES - 2) * BLK_PER_WAVE>{}, std::integral_constant<int, 15>{});
  // Scheduling barriers pin each phase: left alone, the scheduler sinks every read to just
  // before the MFMAs that consume it, which exposes the LDS latency again. Each multiply
  // phase ends with lgkmcnt(0): the reads issued before it have long completed, and with
  // only one set of reads ever outstanding the compiler needs no wait of its own before the
  // next multiply (with two sets, 16 reads, it falls back to draining both).
  Frag f0, f1;
  read(f0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // both edges into the loop arrive with no reads pending
  // K step kt: slot rs holds stage kt, stage k_in goes into slot is, slot rn holds stage kt + 1
  // (past the last step: a slot of clamped data, never multiplied)
  auto step = [&](unsigned rs, int k_in, unsigned is, unsigned rn) {
    read(f1, rs, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    wait_barrier(std::integral_constant<int, (STAGES - 3) * BLK_PER_WAVE>{}, std::integral_constant<int, 0>{});
    issue_at(k_in, is);
    read(f0, rn, 0);
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left open
    __builtin_amdgcn_sched_barrier(0);
  };
  // STAGES steps per iteration while no issued stage needs clamping (constant ring slots)
  int kt = 0;
  for (; kt + 2 * STAGES - 1 <= nk; kt += STAGES)
    static_for<STAGES>([&](auto u) {
      constexpr unsigned U = decltype(u)::value;
      step(U, kt + U + STAGES - 1, (U + STAGES - 1) % STAGES, (U + 1) % STAGES);
    });
  for (; kt < nk; ++kt) {
    const int k_in = kt + STAGES - 1 < nk ? kt + STAGES - 1 : nk - 1;
    step((unsigned)kt % STAGES, k_in, (unsigned)k_in % STAGES, (unsigned)(kt + 1) % STAGES);
  }
  __syncthreads();
  gemm_store_tile<BM, BN, WAVES_M, WAVES_N, FM, FN, MAPPED>(p, acc, smem, m0, n0, wm, wn, lane, tid);
  }
}

// Ping-pong tile (256x256, 128x128, 256x128, 128x256) on paired K steps. An LDS row holds two consecutive K steps (128
// bytes: 64 bf16 or 128 E4M3 values), so the eight lanes that fetch a row of a 1 KB block (8
// rows) read one whole 128-byte line: half the cache requests of 64-byte rows for the same
// bytes. The 16-byte chunk index is XORed with bits 1..3 of the row, so the 16 consecutive rows
// one ds_read_b128 phase reads fall on 16 distinct bank groups (row parity picks the half of
// the 256-byte bank window).
//
// The ring is S slots, each the size of one operand's rows of one pair (a "half": 32 KB for 256
// rows, 16 KB for 128; S = 5 for tiles with a 256-row operand, 10 for 128x128: 160 KB). Half h is
// the A rows (h even) or the B rows (h odd) of K pair h / 2 and lives in slot h % S. Memory phase k (the two groups run the same ping-pong as the
// 64-byte-row kernel) reads step k from halves 2 (k / 2) and 2 (k / 2) + 1, issues half
// k + S - 2 into the slot of half k - 2 (which both groups finished reading at step k - 1 at
// the latest, one barrier earlier), and waits until step k + 1's halves have landed: the
// halves issued after them are k + 2 .. k + S - 2 for even k and k + 3 .. k + S - 2 for odd
// k. Halves past the last pair reload the last pair into its own slot (identical bytes), so
// every phase issues the same loads. Each wave owns a run of BM / 64 A blocks and one of BN / 64
// B blocks (one M0 and one buffer resource each); the waits count each half's own loads.
__device__ __forceinline__ int pair_off(int row, int lc) { return row * 128 + ((lc ^ ((row >> 1) & 7)) << 4); }

// Loads one wave issues for half h + d when h is even (A halves: RA blocks, B halves: RB).
constexpr int pair_loads(int d, int ra, int rb) { return (d & 1) ? rb : ra; }
constexpr int pair_wait(int from, int to, int parity, int ra, int rb) {
  int n = 0;
  for (int d = from; d <= to; ++d) n += pair_loads(d + parity, ra, rb);
  return n;
}

template <int BM, int BN, int SLOTS, bool FP8, bool MAPPED, int EPI = EPI_GENERIC, bool PP = false>
__global__ __launch_bounds__(512) void gemm_nt_pair_kernel(GemmProblem p, int tiles_m, int tiles_n, int group_m) {
  constexpr int WAVES_M = 2, WAVES_N = 4, WM = BM / 2, WN = BN / 4, FM = WM / 32, FN = WN / 32;
  constexpr int HALF = (BM > BN ? BM : BN) * 128;  // slot size: the larger operand's half
  constexpr int RA = BM / 64, RB = BN / 64;          // a wave's blocks per A half and per B half
  // vmcnt after an even step's issue, an odd step's, and the prologue's (see above)
  constexpr int VM_EVEN = pair_wait(2, SLOTS - 2, 0, RA, RB), VM_ODD = pair_wait(3, SLOTS - 2, 1, RA, RB);
  constexpr int VM_PRO = pair_wait(2, SLOTS - 3, 0, RA, RB);
  static_assert((BM == 256 || BM == 128) && (BN == 256 || BN == 128) && SLOTS >= 4 && VM_EVEN < 64, "pair ring shape");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SLOTS * HALF];
  static_assert(SLOTS * HALF >= WAVES_M * 32 * (BN + 4) * 4, "the output stage reuses the ring");
  static_assert((EPI != EPI_BF16 && EPI != EPI_BF16_GELU) || SLOTS * HALF >= 160 * 1024,
                "the bf16 output stage may park every band in the 160 KB ring");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = group_m * tiles_n;
  const int grp = lid / per_group, first_m = grp * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  const int in = lid - grp * per_group;
  const int m0 = (first_m + in % gsz) * BM, n0 = (in / gsz) * (MAPPED && p.ep.glu ? BN / 2 : BN);
  const int M = p.M, K = p.K;
  constexpr int ESZ = FP8 ? 1 : 2;
  const int nk = K / (64 / ESZ);  // 64-byte K steps; K fills whole pairs
  const int np = nk / 2;

  // This wave's blocks: rows 8 (RUN w + b) + lane / 8 of each operand's tile, physical chunk
  // lane % 8 of the 128-byte LDS row, fetched from logical chunk (lane % 8) ^ ((row / 2) % 8).
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int nb_first = tile_b_row<BN, MAPPED>(p, n0, 0);
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(p.A) + (int64_t)m0 * p.lda * ESZ;
  const unsigned char* bbase = reinterpret_cast<const unsigned char*>(p.B) + (int64_t)nb_first * p.ldb * ESZ;
  const __amdgpu_buffer_rsrc_t rsrc_a = buf_rsrc(abase), rsrc_b = buf_rsrc(bbase);
  uint32_t voff_a[RA], voff_b[RB];
#pragma unroll
  for (int b = 0; b < RA; ++b) {
    const int row = (RA * wave_s + b) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ ((row >> 1) & 7);
    const int gm = min(m0 + row, M - 1);
    voff_a[b] = (uint32_t)(((int64_t)(gm - m0) * p.lda) * ESZ + lc * 16 + BUF_BACKOFF - b * 1024);
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int row = (RB * wave_s + b) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ ((row >> 1) & 7);
    const int gn = tile_b_row<BN, MAPPED>(p, n0, row);
    voff_b[b] = (uint32_t)(((int64_t)(gn - nb_first) * p.ldb) * ESZ + lc * 16 + BUF_BACKOFF - b * 1024);
  }
  // Half h (pair h / 2, clamped to the last pair) into slot `slot` (h % S, or the clamped
  // half's slot): A rows for even h, B rows for odd h.
  auto issue_half = [&](int pair, bool b_rows, unsigned slot) {
    lds_byte* base = (lds_byte*)smem + slot * HALF;
    if (b_rows)
      static_for<RB>([&](auto b) {
        constexpr int bi = decltype(b)::value;
        buf_load16<bi * 1024>(rsrc_b, voff_b[bi], pair * 128, base + wave_s * RB * 1024);
      });
    else
      static_for<RA>([&](auto b) {
        constexpr int bi = decltype(b)::value;
        buf_load16<bi * 1024>(rsrc_a, voff_a[bi], pair * 128, base + wave_s * RA * 1024);
      });
  };
  auto issue_clamped = [&](int h) {
    const int hc = h < 2 * np ? h : 2 * (np - 1) + (h & 1);
    issue_half(hc >> 1, hc & 1, (unsigned)hc % SLOTS);
  };

  f32x16_t acc[FM][FN];
  static_for<FM>([&](auto i) {
    static_for<FN>([&](auto j) { static_for<16>([&](auto v) { acc[i][j][decltype(v)::value] = 0.0f; }); });
  });
  const int a_row0 = wm * WM + (lane & 31), b_row0 = wn * WN + (lane & 31);
  const int khalf = lane >> 5;
  struct Frag {
    bf16x8_t a[FM], b[FN];
  };
  // Fragment `half` of step k from slots sa (A) and sb (B): the 64-byte half kp = k % 2 of the
  // rows, then as in the 64-byte-row kernel (bf16: chunk 2 half + l / 32; fp8: 2 (l / 32) + half).
  // Rows 32 apart share the swizzle, so one per-lane offset per (kp, half) serves every block.
  int off_a[2][2], off_b[2][2];
#pragma unroll
  for (int kp = 0; kp < 2; ++kp)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int lc = kp * 4 + (FP8 ? khalf * 2 + hf : hf * 2 + khalf);
      off_a[kp][hf] = pair_off(a_row0, lc);
      off_b[kp][hf] = pair_off(b_row0, lc);
    }
  auto read = [&](Frag& f, unsigned sa, unsigned sb, int kp, int half) {
    const unsigned char* pa = smem + (sa * HALF + off_a[kp][half]);
    const unsigned char* pb = smem + (sb * HALF + off_b[kp][half]);
    static_for<FM>([&](auto i) {
      f.a[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(pa + i * 32 * 128));
    });
    static_for<FN>([&](auto j) {
      f.b[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(pb + j * 32 * 128));
    });
  };
  auto mma8 = [&](const Frag& f0, const Frag& f1) {
    static_for<FM>([&](auto i) {
      static_for<FN>([&](auto j) {
        const i32x8_t a = __builtin_bit_cast(
            i32x8_t, __builtin_shufflevector(__builtin_bit_cast(u32x4_t, f0.a[i]), __builtin_bit_cast(u32x4_t, f1.a[i]),
                                             0, 1, 2, 3, 4, 5, 6, 7));
        const i32x8_t b = __builtin_bit_cast(
            i32x8_t, __builtin_shufflevector(__builtin_bit_cast(u32x4_t, f0.b[j]), __builtin_bit_cast(u32x4_t, f1.b[j]),
                                             0, 1, 2, 3, 4, 5, 6, 7));
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 0, 0, 0);
      });
    });
  };
  auto mma = [&](const Frag& f) {
    static_for<FM>([&](auto i) {
      static_for<FN>([&](auto j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
      });
    });
  };
  // s_waitcnt vmcnt(VM) lgkmcnt(LGKM) (expcnt open) and a fence-free workgroup barrier
  auto wait_barrier = [&](auto vm, auto lgkm) {
    constexpr int VM = decltype(vm)::value, LGKM = decltype(lgkm)::value;
    static_assert(VM >= 0 && VM < 64, "vmcnt immediate is six bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (LGKM << 8) | ((VM >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: halves 0 .. S - 3; pair 0 (halves 0 and 1) landed everywhere. Group 1 runs one
  // phase behind group 0 (an extra barrier at its start, one at group 0's end).
#pragma unroll
  for (int h = 0; h < SLOTS - 2; ++h) issue_clamped(h);
  wait_barrier(std::integral_constant<int, VM_PRO>{}, std::integral_constant<int, 15>{});
  if (wm == 1) {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  Frag f0, f1;
  // memory phase of step k (reads from slots sa, sb at pair half kp; issues `pair`'s A or B
  // rows into slot is), then the compute phase
  auto step = [&](unsigned sa, unsigned sb, int kp, int pair, bool b_rows, unsigned is, auto vm) {
    read(f0, sa, sb, kp, 0);
    read(f1, sa, sb, kp, 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_half(pair, b_rows, is);
    wait_barrier(vm, std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_setprio(1);
    if constexpr (FP8) {
      mma8(f0, f1);
    } else {
      mma(f0);
      mma(f1);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Two steps (one K pair) per iteration: the pair half kp and the waits are constants; slots
  // are scalars kept by increments, so each fragment read adds one slot offset to a per-lane
  // base. Pair j reads slots sa = 2j % S and sa + 1 and issues halves 2j + S - 2 and
  // 2j + S - 1 into slots (sa + S - 2) % S and (sa + S - 1) % S; the last pairs clamp.
  unsigned sa = 0;
  auto next = [](unsigned v, unsigned d) { return v + d >= SLOTS ? v + d - SLOTS : v + d; };
  constexpr int H0 = SLOTS - 2;  // half issued at the first step of pair 0
  int j = 0;
  if constexpr (PP) {
    // PP: one memory phase and one compute phase per K pair instead of per K step (the
    // 128x128 tile, whose few MFMAs per step, four bf16 or two fp8, cannot cover a step's
    // memory phase).
    // Pair j reads all four fragment sets of the pair, issues halves 2j + S - 2 and 2j + S - 1
    // (into pair j - 1's slots, which both groups finished reading one barrier earlier) and
    // waits until pair j + 1 has landed (the halves issued after it: 2j + 4 .. 2j + S - 1).
    constexpr int VM_PAIR = pair_wait(4, SLOTS - 1, 0, RA, RB);
    static_assert(VM_PAIR < 64, "vmcnt immediate is six bits");
    Frag f2, f3;
    auto pair_phase = [&](unsigned sa_, unsigned sb_, int h0, int h1) {
      read(f0, sa_, sb_, 0, 0);
      read(f1, sa_, sb_, 0, 1);
      read(f2, sa_, sb_, 1, 0);
      read(f3, sa_, sb_, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      const int c0 = h0 < 2 * np ? h0 : 2 * (np - 1) + (h0 & 1);
      const int c1 = h1 < 2 * np ? h1 : 2 * (np - 1) + (h1 & 1);
      issue_half(c0 >> 1, c0 & 1, (unsigned)c0 % SLOTS);
      issue_half(c1 >> 1, c1 & 1, (unsigned)c1 % SLOTS);
      wait_barrier(std::integral_constant<int, VM_PAIR>{}, std::integral_constant<int, 0>{});
      __builtin_amdgcn_s_setprio(1);
      if constexpr (FP8) {
        mma8(f0, f1);
        mma8(f2, f3);
      } else {
        mma(f0);
        mma(f1);
        mma(f2);
        mma(f3);
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (; j < np; ++j) {
      pair_phase(sa, sa + 1 == SLOTS ? 0 : sa + 1, 2 * j + H0, 2 * j + H0 + 1);
      sa = next(sa, 2);
    }
  }
  for (; !PP && 2 * j + SLOTS <= 2 * np; ++j) {
    const unsigned sb = sa + 1 == SLOTS ? 0 : sa + 1;
    step(sa, sb, 0, j + (H0 >> 1), H0 & 1, next(sa, SLOTS - 2), std::integral_constant<int, VM_EVEN>{});
    step(sa, sb, 1, j + ((H0 + 1) >> 1), (H0 + 1) & 1, next(sa, SLOTS - 1), std::integral_constant<int, VM_ODD>{});
    sa = next(sa, 2);
  }
  for (; !PP && j < np; ++j) {
    const unsigned sb = sa + 1 == SLOTS ? 0 : sa + 1;
    int h = 2 * j + H0, hc = h < 2 * np ? h : 2 * (np - 1) + (h & 1);
    step(sa, sb, 0, hc >> 1, hc & 1, (unsigned)hc % SLOTS, std::integral_constant<int, VM_EVEN>{});
    h = 2 * j + H0 + 1, hc = h < 2 * np ? h : 2 * (np - 1) + (h & 1);
    step(sa, sb, 1, hc >> 1, hc & 1, (unsigned)hc % SLOTS, std::integral_constant<int, VM_ODD>{});
    sa = next(sa, 2);
  }
  if (wm == 0) {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  gemm_store_tile<BM, BN, WAVES_M, WAVES_N, FM, FN, MAPPED, EPI>(p, acc, smem, m0, n0, wm, wn, lane, tid);
}

// The output-stage mode a launch can be built for (EPI_GENERIC when no fixed mode covers it).
static int epilogue_mode(const GemmEpilogue& ep) {
  if (ep.glu || ep.c_head_w > 0) return EPI_GENERIC;
  if (ep.out_f32) return ep.act == TP_ACT_NONE && ep.row_scale == nullptr ? EPI_F32 : EPI_GENERIC;
  if (ep.row_scale != nullptr) return ep.act == TP_ACT_NONE ? EPI_FP8_BF16 : EPI_GENERIC;
  if (ep.act == TP_ACT_NONE) return EPI_BF16;
  if (ep.act == TP_ACT_GELU_ERF) return EPI_BF16_GELU;
  return EPI_GENERIC;
}

// Whether every buffer-loaded byte of a BM x BN tile lies within the 2^31 - 1 bytes a buffer
// resource covers from the tile's first row: min(BM, M) rows of A; for B, min(BN, N) consecutive
// rows or, through the per-head map (non-decreasing when the head pitch is at least the head
// width and values follow their gates), the rows of BN (SwiGLU: BN / 2) columns plus the value
// offset. Rows past M or N clamp to the last one.
bool buffer_span_ok(const GemmProblem& p, int BM, int BN) {
  const int64_t esz = p.fp8 ? 1 : 2;
  const int64_t tail = (int64_t)p.K * esz + BUF_BACKOFF + DROW;
  if ((int64_t)(std::min(BM, p.M) - 1) * p.lda * esz + tail > INT32_MAX) return false;
  int64_t rows = std::min(BN, p.N);
  if (p.ep.glu || p.b_head_w > 0) {
    if ((p.ep.glu && p.ep.glu_off < 0) || (p.b_head_w > 0 && p.b_head_pitch < p.b_head_w)) return false;
    const int64_t cols = std::min(p.ep.glu ? BN / 2 : BN, p.N);
    rows = cols + (p.ep.glu ? p.ep.glu_off : 0);
    if (p.b_head_w > 0) rows += (cols / p.b_head_w + 1) * (int64_t)(p.b_head_pitch - p.b_head_w);
  }
  return (rows - 1) * p.ldb * esz + tail <= INT32_MAX;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int SCHED = 0>
hipError_t launch_tile(const GemmProblem& p, int path, hipStream_t stream) {
  const int bn_out = p.ep.glu ? BN / 2 : BN;  // output columns per tile
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + bn_out - 1) / bn_out;
  const int nb = tiles_m * tiles_n;
  const int group_m = tiles_m < 4 ? tiles_m : 4;  // 4 M-tiles per group: measured best for L2 reuse
  dim3 grid(nb), block(WAVES_M * WAVES_N * 64);
  const bool dma_ok = p.row_r == nullptr && p.K % DBK == 0 && p.lda % 8 == 0 && p.ldb % 8 == 0 &&
                      (!tile_uses_buffer_loads<BM, BN, WAVES_M * WAVES_N>() || buffer_span_ok(p, BM, BN));
  if (path == GEMM_PATH_DMA && !dma_ok) return hipErrorInvalidValue;
  // the per-head row map and SwiGLU run in their own instantiations (never with RMSNorm staging)
  const bool mapped = p.ep.glu || p.b_head_w > 0;
  if (mapped && p.row_r != nullptr) return hipErrorInvalidValue;
  if (dma_ok && path != GEMM_PATH_REGISTER) {
    if constexpr ((BM == 256 || BM == 128) && (BN == 256 || BN == 128) && WAVES_M == 2 && WAVES_N == 4 &&
                  SCHED == 1) {
      constexpr int S = BM == 256 || BN == 256 ? 5 : 10;  // 160 KB of halves
      constexpr bool PP = BM == 128 && BN == 128;         // one phase per K pair (see the kernel)
      if (p.K % 64 == 0) {                               // whole K pairs: 128-byte LDS rows
        if (mapped)
          hipLaunchKernelGGL((gemm_nt_pair_kernel<BM, BN, S, false, true, EPI_GENERIC, PP>), grid, block, 0, stream, p, tiles_m,
                             tiles_n, group_m);
        else if (epilogue_mode(p.ep) == EPI_BF16)
          hipLaunchKernelGGL((gemm_nt_pair_kernel<BM, BN, S, false, false, EPI_BF16, PP>), grid, block, 0, stream, p,
                             tiles_m, tiles_n, group_m);
        else if (epilogue_mode(p.ep) == EPI_BF16_GELU)
          hipLaunchKernelGGL((gemm_nt_pair_kernel<BM, BN, S, false, false, EPI_BF16_GELU, PP>), grid, block, 0, stream,
                             p, tiles_m, tiles_n, group_m);
        else if (epilogue_mode(p.ep) == EPI_F32)
          hipLaunchKernelGGL((gemm_nt_pair_kernel<BM, BN, S, false, false, EPI_F32, PP>), grid, block, 0, stream, p,
                             tiles_m, tiles_n, group_m);
        else
          hipLaunchKernelGGL((gemm_nt_pair_kernel<BM, BN, S, false, false, EPI_GENERIC, PP>), grid, block, 0, stream, p, tiles_m,
                             tiles_n, group_m);
        return hipGetLastError();
      }
    }
    if (mapped)
      hipLaunchKernelGGL((gemm_nt_dma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, SCHED, false, true>), grid, block, 0,
                         stream, p, tiles_m, tiles_n, group_m);
    else
      hipLaunchKernelGGL((gemm_nt_dma_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, SCHED>), grid, block, 0, stream, p,
                         tiles_m, tiles_n, group_m);
  } else if (p.row_r != nullptr) {
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, true, false>), grid, block, 0, stream, p, tiles_m,
                       tiles_n, group_m);
  } else if (mapped) {
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, false, true>), grid, block, 0, stream, p, tiles_m,
                       tiles_n, group_m);
  } else {
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, false, false>), grid, block, 0, stream, p, tiles_m,
                       tiles_n, group_m);
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_tile_fp8(const GemmProblem& p, hipStream_t stream) {
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int group_m = tiles_m < 4 ? tiles_m : 4;
  static_assert(tile_uses_buffer_loads<BM, BN, 8>(), "the fp8 tiles load through buffer resources");
  if (!buffer_span_ok(p, BM, BN)) return hipErrorNotSupported;
  if (p.K % 128 == 0) {  // whole K pairs: 128-byte LDS rows
    constexpr bool PP = BM == 128;  // one phase per K pair (see the kernel)
    if (epilogue_mode(p.ep) == EPI_FP8_BF16)
      hipLaunchKernelGGL((gemm_nt_pair_kernel<BM, BN, BM == 256 ? 5 : 10, true, false, EPI_FP8_BF16, PP>),
                         dim3(tiles_m * tiles_n), dim3(512), 0, stream, p, tiles_m, tiles_n, group_m);
    else
      hipLaunchKernelGGL((gemm_nt_pair_kernel<BM, BN, BM == 256 ? 5 : 10, true, false, EPI_GENERIC, PP>),
                         dim3(tiles_m * tiles_n), dim3(512), 0, stream, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_nt_dma_kernel<BM, BN, 2, 4, 4, 1, true>), dim3(tiles_m * tiles_n), dim3(512), 0, stream, p,
                     tiles_m, tiles_n, group_m);
  return hipGetLastError();
}

}  // namespace

namespace {
// A launch's modelled time in full-wave units: one workgroup per CU and 256 CUs give
// floor(n / 256) full waves, and r left-over tiles a partial wave that runs at a higher clock
// (power cap) and takes part0 + (1 - part0) r / 256 of a full one.
double wave_units(long long n, double part0) {
  const long long r = n % 256;
  return (double)(n / 256) + (r ? part0 + (1.0 - part0) * (double)r / 256.0 : 0.0);
}
}  // namespace

int gemm_fp8_pick_tile(int M, int N, int K) {
  (void)K;
  // Full-wave times at K = 4096: 256x256 58.9 us, 128x128 24.7 (relative 100, 42); a partial
  // wave costs 0.72 + 0.28 r / 256 of a full one (256x256: 48 tiles 43.9 us, 128 tiles 47.4).
  // 6144x1536x4096: 48.0 us on 144 256x256 tiles against 60.7 on 576 128x128 tiles;
  // 2048x3072x4096: 41.5 us on 384 128x128 tiles against 45.9 on 96 256x256 tiles.
  const long long t256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
  const long long t128 = (long long)((M + 127) / 128) * ((N + 127) / 128);
  return 100.0 * wave_units(t256, 0.72) <= 42.0 * wave_units(t128, 0.72) ? TILE_256x256 : TILE_128x128;
}

hipError_t launch_gemm_fp8(const GemmProblem& p, int tile, hipStream_t stream) {
  if (!p.fp8 || p.K % 64 != 0 || p.lda % 16 != 0 || p.ldb % 16 != 0 || p.row_r != nullptr || p.ep.glu ||
      p.b_head_w > 0)
    return hipErrorInvalidValue;
  if (p.M <= 0 || p.N <= 0) return hipSuccess;  // nothing to write
  if (tile == TILE_AUTO) tile = gemm_fp8_pick_tile(p.M, p.N, p.K);
  switch (tile) {
    case TILE_256x256: return launch_tile_fp8<256, 256>(p, stream);
    case TILE_128x128: return launch_tile_fp8<128, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

int gemm_pick_tile(int M, int N, int K) {
  (void)K;
  auto tiles = [&](int bm, int bn) { return (long long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  // Full-wave times at K = 4096: 256x256 105 us, 128x256 64, 256x128 65.6, 128x128 39.2
  // (relative 100, 61, 62.5, 37.3); a partial wave costs 0.62 + 0.38 r / 256 of a full one
  // (256x256: 48 tiles 67-68 us, 96 tiles 73-75, 128 tiles 82, 224 tiles 96). The least
  // modelled time wins, the larger tile at a tie: 6144x1536x4096 77.9 us on 144 256x256 tiles
  // against 105.9 on 288 128x256 tiles; 2048x3072x4096 56.2 us on 192 256x128 tiles against
  // 69.3 on 384 128x128.
  const long long t128 = tiles(128, 128);
  if (t128 >= 128) {
    const struct {
      int tile;
      long long n;
      double wave;
    } c[] = {{TILE_256x256, tiles(256, 256), 100.0}, {TILE_128x256, tiles(128, 256), 61.0},
             {TILE_256x128, tiles(256, 128), 62.5}, {TILE_128x128, t128, 37.3}};
    int best = 0;
    double best_t = 0.0;
    for (int i = 0; i < 4; ++i) {
      const double t = c[i].wave * wave_units(c[i].n, 0.62);
      if (i == 0 || t < best_t) best = i, best_t = t;
    }
    return c[best].tile;
  }
  // below a full wave of 128x64 tiles the K loop's latency decides: 64x64 tiles keep twice as
  // many CUs busy (1024x512x4096: 21 us against 35 us; 2048x768x4096: 36 against 38)
  if ((long long)((M + 127) / 128) * ((N + 63) / 64) >= 256) return TILE_128x64;
  return TILE_64x64;
}

hipError_t launch_gemm(const GemmProblem& p, int tile, int path, hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;  // nothing to write (the epilogue clamps to row M - 1, column N - 1)
  if (tile == TILE_AUTO) tile = gemm_pick_tile(p.M, p.ep.glu ? 2 * p.N : p.N, p.K);
  switch (tile) {
    case TILE_256x256: return launch_tile<256, 256, 2, 4, 4, 1>(p, path, stream);  // 8 waves, ping-pong
    case TILE_256x128: return launch_tile<256, 128, 2, 4, 4, 1>(p, path, stream);  // 8 waves, ping-pong
    case TILE_128x128: return launch_tile<128, 128, 2, 4, 4, 1>(p, path, stream);  // 8 waves, ping-pong
    case TILE_128x256: return launch_tile<128, 256, 2, 4, 5, 1>(p, path, stream);  // 8 waves, ping-pong
    case TILE_256x224: return launch_tile<256, 224, 4, 1, 5>(p, path, stream);
    case TILE_128x64: return launch_tile<128, 64, 2, 2, 4>(p, path, stream);
    case TILE_64x64: return launch_tile<64, 64, 2, 2, 8>(p, path, stream);  // 8 stages: short-K launches keep every K step in flight
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpk
