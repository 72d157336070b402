// K3 + K4: vocab-sharded decode LM head with the shard's argmax.
//
// [tt] LMHead1D: the shard's projection is split into chunks of at most C rows,
// one linear per chunk, outputs concatenated along the vocab; each device ends
// with complete logits for its own vocab rows. [palm] unembed_manual: float32
// logits. Decode has a few batch rows, so the work is a stream of the weight
// shard from HBM: every weight byte is read once.
//
// Four streaming kernels compute the logits; each gives a workgroup a tile of weight rows
// and finishes with that workgroup's (max, lowest index) candidate per batch row, which a
// second kernel launched right after reduces (a kernel boundary instead of per-workgroup
// device-scope fences, which on gfx950 write back and invalidate the whole L2).
//
// * Row-quad (shapes 11-16; the default): a workgroup owns 64 rows (128: shape 16) over the whole K, x sits
//   in LDS one slice at a time (32 or 64 batch rows per pass), and each weight load
//   instruction reads 4 rows x 256 contiguous bytes into registers; each wave turns its
//   loads into the MFMA operand layout through 4 KB of its own LDS.
// * x-resident (shape 10): the same split with the weight loaded straight in the operand
//   layout (16 rows x 64 bytes per load instruction).
// * LDS ring (shapes 8, 9; the fallback for a K the others cannot take): a workgroup owns 64
//   rows over the whole K; weight, x and block-scale pieces go global -> LDS with
//   global_load_lds into a ring of stages that fills the CU's LDS.
// * Register streaming (shapes 0-7; any K % 8 == 0): a workgroup owns 16 G weight rows and
//   its waves split K; each wave loads its K steps straight into MFMA operand registers and
//   the waves' partials are summed through LDS in wave order.
//
// The 64-row kernels tile the shard in whole 64-row blocks: the chunks only group the
// concatenated output, which is the same rows in the same order, so a chunk boundary inside
// a block changes nothing. The register-streaming shapes tile each chunk on its own.
//
// All multiply with v_mfma_f32_16x16x32_bf16, x as the row operand and the
// weight as the column operand, so every lane's accumulators belong to one weight
// row. E4M3 weights are widened to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8
// with scale 1: exact, every E4M3 value is a bf16 value) and each 128-wide K
// block's partial is multiplied by the row's block scale before it joins the
// float32 accumulator.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int LM_BATCH = 32;  // batch rows per launch pass (two 16-row MFMA groups)
constexpr int LM_FIN_THREADS = 256;

// Launch shapes: G 16-row weight groups per workgroup, W waves splitting the workgroup's K,
// P 32-wide K steps per batch of loads (a multiple of four: whole 128-wide E4M3 blocks), KS
// workgroups splitting K. x is re-read by every workgroup, so its share of the L1 traffic is
// 32 / (16 G): more rows per workgroup (with K split to keep every CU busy) cut it.
struct LmShape {
  int G, W, P, KS;
};
// (Every shape fits the register file at its wave count: {8, 8, 4, 2} spilled in its E4M3 build.)
constexpr LmShape kLmShapes[] = {{4, 8, 8, 1}, {2, 8, 8, 1}, {4, 4, 8, 1}, {2, 4, 8, 1},
                                 {4, 8, 4, 1}, {1, 8, 8, 1}, {4, 8, 4, 2}, {8, 4, 4, 2}};
constexpr int kLmDmaShape = 8;  // 8, 9: the direct-to-LDS kernel (indices past the table)
constexpr int kLmXresShape = 10;  // the x-resident kernel (batch passes of up to 64 rows)
constexpr int kLmQuadShape = 11;  // 11 .. 16: the row-quad kernel (batch passes of 32 or 64 rows)
constexpr int kLmRingShape = 9;  // LDS ring, 128-byte stages (falls back to 4 for a ragged bf16 K)

// Two E4M3 codes (bytes HI ? 2,3 : 0,1 of w) -> two bf16, exactly (scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

template <bool FP8, int G, int LM_WAVES, int LM_P, int KS>
__global__ __launch_bounds__(LM_WAVES * 64) void lm_head_kernel(LmHeadProblem p, int tiles_per_chunk, int n_tiles,
                                                               int b0) {
  constexpr int LM_ROWS = G * 16;
  constexpr int LM_THREADS = LM_WAVES * 64;
  __shared__ __attribute__((aligned(16))) float red[LM_WAVES * LM_BATCH * LM_ROWS];
  __shared__ float red_v[LM_WAVES][LM_BATCH];
  __shared__ int red_i[LM_WAVES][LM_BATCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, V = p.V, C = p.chunk;
  const int nbatch = min(LM_BATCH, p.B - b0);

  // This workgroup's rows: tile t of chunk c, clipped to the chunk's end; and its K slice.
  const int tile = blockIdx.x / KS, kslice = blockIdx.x % KS;
  const int chunk = tile / tiles_per_chunk, tin = tile - chunk * tiles_per_chunk;
  const int row0 = chunk * C + tin * LM_ROWS;
  const int chunk_end = min(V, (chunk + 1) * C);
  const int nrows = max(0, min(LM_ROWS, chunk_end - row0));

  // This wave's K steps [s_begin, s_end) of the ceil(K / 32) steps: the workgroup's K slice
  // split over its waves, in whole 128-wide blocks (four steps) so that an E4M3 scale block
  // never straddles two waves.
  const int nsteps = (K + 31) / 32;
  const int per_wave = ((nsteps + LM_WAVES * KS - 1) / (LM_WAVES * KS) + 3) / 4 * 4;
  const int s_begin = min(nsteps, (kslice * LM_WAVES + wave) * per_wave), s_end = min(nsteps, s_begin + per_wave);
  const int nblk = K / 128;

  // Lane roles in v_mfma_f32_16x16x32_bf16: lane l supplies row (or column) l % 16 and
  // eight K values selected by q = l / 16. Weight rows and x rows beyond the tile read a
  // clamped row: they only feed outputs that are never stored.
  const int r16 = lane & 15, kq = lane >> 4;
  const int64_t ldw = FP8 ? (int64_t)K : 2 * (int64_t)K;  // bytes per weight row
  const unsigned char* wrow[G];
  bool wok[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int r = g * 16 + r16;
    wok[g] = r < nrows;
    wrow[g] = reinterpret_cast<const unsigned char*>(p.w) + (int64_t)(row0 + (wok[g] ? r : 0)) * ldw;
  }
  const uint16_t* xrow[2];
  bool xok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = h * 16 + r16;
    xok[h] = b < nbatch;
    xrow[h] = p.x + (int64_t)(b0 + (xok[h] ? b : 0)) * K;
  }

  // K values of step st seen by this lane (8 consecutive from kofs(st)). bf16: the natural
  // layout, 32 st + 8 q. E4M3: one 16-byte weight piece holds K values 64 (st / 2) + 16 q ..
  // +16; its first eight feed the even step, the other eight the odd step.
  auto kofs = [&](int st) { return FP8 ? (st & ~1) * 32 + kq * 16 + (st & 1) * 8 : st * 32 + kq * 8; };

  constexpr int WPIECES = FP8 ? LM_P / 2 : LM_P;
  struct Batch {
    u32x4_t w[WPIECES][G];
    u32x4_t x[LM_P][2];
    float sc[LM_P / 4][G];
  };
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // Issues the loads of the batch starting at step s0 (clamped to the last steps, so the
  // loads are unconditional and stay in flight; consume ignores steps past s_end).
  auto load = [&](int s0, Batch& bt) {
    static_for<LM_P>([&](auto i) {
      const int st = min(s0 + (int)i, nsteps - 1);
      const int k = kofs(st) < K ? kofs(st) : 0;
      static_for<2>([&](auto h) { bt.x[i][h] = *reinterpret_cast<const u32x4_t*>(xrow[h] + k); });
    });
    static_for<WPIECES>([&](auto i) {
      int off;
      if constexpr (FP8) {
        off = min(s0 + 2 * (int)i, nsteps - 2) * 32 + kq * 16;
      } else {
        const int k = kofs(min(s0 + (int)i, nsteps - 1));
        off = (k < K ? k : 0) * 2;
      }
      static_for<G>([&](auto g) { bt.w[i][g] = *reinterpret_cast<const u32x4_t*>(wrow[g] + off); });
    });
    if constexpr (FP8) {
      static_for<LM_P / 4>([&](auto j) {
        const int blk = min(s0 / 4 + (int)j, nblk - 1);
        static_for<G>([&](auto g) {
          bt.sc[j][g] = p.wscale[(int64_t)(row0 + (wok[g] ? g * 16 + r16 : 0)) * nblk + blk];
        });
      });
    }
  };

  f32x4_t acc[G][2], part[G][2];
  auto clear = [&](f32x4_t(&a)[G][2]) {
    static_for<G>([&](auto g) {
      static_for<2>([&](auto h) { static_for<4>([&](auto v) { a[g][h][decltype(v)::value] = 0.0f; }); });
    });
  };
  clear(acc);
  clear(part);
  // Multiplies the batch starting at step s0. Steps at or past s_end multiply zeros instead
  // of branching around the MFMAs (a branch would make the compiler drain the loads in
  // flight at the join). With E4M3 weights, each 128-wide block's partial (four steps) is
  // scaled by the row's block scale as it joins the float32 accumulator.
  auto consume = [&](int s0, const Batch& bt) {
    static_for<LM_P>([&](auto i) {
      constexpr int ii = i;
      const int st = s0 + ii;
      const bool kok = st < s_end && kofs(st) < K;
      bf16x8_t xa[2];
      static_for<2>([&](auto h) { xa[h] = __builtin_bit_cast(bf16x8_t, (kok && xok[h]) ? bt.x[i][h] : zero); });
      static_for<G>([&](auto g) {
        u32x4_t wv;
        if constexpr (FP8) {
          const u32x4_t q = bt.w[ii / 2][g];
          constexpr int o = (ii % 2) * 2;  // dwords 0,1 feed the even step, 2,3 the odd
          wv[0] = e4m3x2_to_bf16x2<false>(q[o]);
          wv[1] = e4m3x2_to_bf16x2<true>(q[o]);
          wv[2] = e4m3x2_to_bf16x2<false>(q[o + 1]);
          wv[3] = e4m3x2_to_bf16x2<true>(q[o + 1]);
        } else {
          wv = bt.w[i][g];
        }
        const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, wv);
        static_for<2>([&](auto h) {
          if constexpr (FP8)
            part[g][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[h], wb, part[g][h], 0, 0, 0);
          else
            acc[g][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[h], wb, acc[g][h], 0, 0, 0);
        });
      });
      if constexpr (FP8 && ii % 4 == 3) {
        const bool live = s0 + ii - 3 < s_end;
        static_for<G>([&](auto g) {
          const float sc = (live && wok[g]) ? bt.sc[ii / 4][g] : 0.0f;
          static_for<2>([&](auto h) {
            static_for<4>([&](auto v) {
              constexpr int vv = v;
              acc[g][h][vv] = fmaf(part[g][h][vv], sc, acc[g][h][vv]);
            });
          });
        });
        clear(part);
      }
    });
  };

  // One batch in flight per wave, issued whole (eight steps: 48 KB per wave, 384 KB per
  // workgroup), then multiplied. The eight waves of the CU keep HBM busy between them.
  for (int s0 = s_begin; s0 < s_end; s0 += LM_P) {
    Batch bt;
    load(s0, bt);
    // keeps the scheduler from interleaving the batch's loads with its MFMAs (which would
    // leave only a few loads in flight per wave)
    __builtin_amdgcn_sched_barrier(0);
    consume(s0, bt);
  }

  // Sum the eight waves' partials in wave order. 16x16 accumulator layout: lane l holds
  // weight row (block column) l % 16 and batch rows 4 (l / 16) + v of its four values.
  static_for<G>([&](auto g) {
    static_for<2>([&](auto h) {
      static_for<4>([&](auto v) {
        constexpr int vv = v;
        const int b = h * 16 + kq * 4 + vv;
        red[(wave * LM_BATCH + b) * LM_ROWS + g * 16 + r16] = acc[g][h][vv];
      });
    });
  });
  __syncthreads();
  // Thread -> weight row r = tid % LM_ROWS and batch rows bq, bq + BSTEP, ...: the threads
  // cover the 32 x LM_ROWS outputs. Per batch row, the LM_ROWS threads holding it (whole
  // waves, or a wave's aligned quarter/half for 16/32 rows) reduce to this workgroup's
  // (max, lowest index) candidate.
  constexpr int BSTEP = LM_THREADS >= LM_ROWS ? LM_THREADS / LM_ROWS : 1;  // batch rows side by side
  constexpr int BITER = LM_BATCH / BSTEP;
  static_assert(LM_THREADS >= LM_ROWS && BITER * BSTEP == LM_BATCH, "reduction layout");
  static_assert(KS > 1 || LM_ROWS <= 64, "in-kernel candidates need at most 64 rows per workgroup");
  if constexpr (KS > 1) {
    // K split over workgroups: store this slice's partial logits; the finalisation kernel
    // adds the slices in order, writes the logits and takes the argmax.
    float* slice = reinterpret_cast<float*>(p.workspace) + (size_t)kslice * LM_BATCH * V;
    const int r = tid % LM_ROWS, bq = tid / LM_ROWS;
#pragma unroll
    for (int t = 0; t < BITER; ++t) {
      const int b = bq + BSTEP * t;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < LM_WAVES; ++w) sum += red[(w * LM_BATCH + b) * LM_ROWS + r];
      if (r < nrows) slice[(size_t)b * V + row0 + r] = sum;
    }
    return;
  }
  {
    const int r = tid % LM_ROWS, bq = tid / LM_ROWS;
#pragma unroll
    for (int t = 0; t < BITER; ++t) {
      const int b = bq + BSTEP * t;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < LM_WAVES; ++w) sum += red[(w * LM_BATCH + b) * LM_ROWS + r];
      if (r < nrows && b < nbatch) p.logits[(int64_t)(b0 + b) * V + row0 + r] = sum;
      float v = (r < nrows && !(sum != sum)) ? sum : -INFINITY;
      int idx = row0 + r;
#pragma unroll
      for (int off = LM_ROWS / 2; off > 0; off >>= 1) {
        float ov = __shfl_xor(v, off, 64);
        int oi = __shfl_xor(idx, off, 64);
        if (better(ov, oi, v, idx)) {
          v = ov;
          idx = oi;
        }
      }
      if (r == 0) {
        red_v[0][b] = v;
        red_i[0][b] = idx;
      }
    }
  }
  __syncthreads();

  // Publish this workgroup's candidates; the finalisation kernel that follows on the stream
  // reduces them.
  float* part_v = reinterpret_cast<float*>(p.workspace);
  int* part_i = reinterpret_cast<int*>(part_v + (size_t)n_tiles * LM_BATCH);
  if (tid < LM_BATCH) {
    part_v[(size_t)tid * n_tiles + tile] = red_v[0][tid];
    part_i[(size_t)tid * n_tiles + tile] = red_i[0][tid];
  }
}


// ---------------------------------------------------------------------------------------
// Direct-to-LDS variant. The weight, x and (E4M3) block-scale pieces of each K stage are
// fetched with global_load_lds into a ring of STAGES LDS stages, STAGES - 1 of them in flight:
// no VGPRs hold loads in flight, so the prefetch depth is set by LDS (up to 160 KB per CU)
// and does not cost registers. The workgroup owns 64 weight rows over the whole K; wave w
// multiplies rows 16 w .. +16 against the 32 x rows, which the four waves share from LDS.
//
// A stage holds RB bytes of every weight row (RB = 64 or 128: 32 or 64 K values of bf16, 64
// or 128 of E4M3), the same K range of the 32 x rows, and for E4M3 the block scale of every
// row (64 lanes x 4 bytes per wave: lane l holds the scale of its wave's row l % 16). LDS
// rows of n 16-byte chunks store chunk c at c XOR (row / (16 / n)) mod n, so the sixteen
// rows one ds_read_b128 phase reads at the same logical chunk fall on sixteen distinct bank
// groups of the 256-byte bank window. Every 1 KB DMA block is row-major; lane q of a block
// fetches the logical chunk that belongs at its physical slot. Blocks are dealt round-robin
// to the waves and padded with duplicate blocks so that every wave issues the same number
// of loads per stage (one vmcnt immediate fits all waves).
//
// The ring is the kernel's only LDS object: with a second one the compiler cannot tell
// the LDS reads from the DMA writes in flight and drains every load before each read.
constexpr int LMD_ROWS = 64;
constexpr int LMD_THREADS = 256;

typedef __attribute__((address_space(3))) unsigned char lmd_lds;
// cache-policy bits of the global_load_lds aux operand
constexpr int LMD_POLICY_DEFAULT = 0;
template <int POLICY>
__device__ __forceinline__ void lmd_dma16(const void* g, lmd_lds* lds) { __builtin_amdgcn_global_load_lds(g, lds, 16, 0, POLICY); }
__device__ __forceinline__ void lmd_dma4(const void* g, lmd_lds* lds) { __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0); }

// byte offset of logical chunk c of row `row` in an LDS array of ROWB-byte rows
template <int ROWB>
__device__ __forceinline__ int lmd_off(int row, int c) {
  constexpr int NC = ROWB / 16;          // chunks per row: 4, 8 or 16
  constexpr int RPW = 16 / NC;           // rows per 256-byte bank window
  return row * ROWB + ((c ^ ((row / RPW) & (NC - 1))) << 4);
}

template <bool FP8, int RB>
struct LmdStage {
  static constexpr int KW = FP8 ? RB : RB / 2;  // K values per stage
  static constexpr int XB = KW * 2;             // x bytes per row per stage
  static constexpr int NWB = LMD_ROWS * RB / 1024;        // weight DMA blocks (a multiple of 4)
  static constexpr int NXB = LM_BATCH * XB / 1024;        // x DMA blocks
  static constexpr int WPW = NWB / 4;                     // weight blocks per wave
  static constexpr int XPW = (NXB + 3) / 4;               // x blocks per wave (padded)
  static constexpr int X_OFF = NWB * 1024;
  static constexpr int S_OFF = X_OFF + 4 * XPW * 1024;    // E4M3 scales after x and its padding
  static constexpr int BYTES = S_OFF + (FP8 ? 1024 : 0);
  static constexpr int OPS = WPW + XPW + (FP8 ? 1 : 0);   // loads per wave per stage
  static_assert(NWB % 4 == 0, "weight blocks split evenly over the waves");
};

template <bool FP8, int RB, int STAGES>
__global__ __launch_bounds__(LMD_THREADS) void lm_head_dma_kernel(LmHeadProblem p, int n_tiles, int b0) {
  using SG = LmdStage<FP8, RB>;
  constexpr int KW = SG::KW, XB = SG::XB, STAGE = SG::BYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[STAGES * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, V = p.V;
  const int nbatch = min(LM_BATCH, p.B - b0);
  const int tile = blockIdx.x;
  const int row0 = tile * LMD_ROWS;
  const int nrows = max(0, min(LMD_ROWS, V - row0));
  const int nst = K / KW;
  const int nblk = K / 128;
  // Each tile walks K from its own starting stage (tile mod the stage count; E4M3 at
  // 64-byte stages: an even stage, so that 128-wide blocks stay whole) and wraps. Tiles in
  // flight together then read different offsets of their rows instead of the same one,
  // which spreads the requests over the memory channels: with every tile at the same
  // offset, the time depended on where the weight copy sat in memory (29 to 41 us for the
  // same bytes). A row's order depends only on its 64-row block, so the logits do not
  // depend on the chunking.
  const int rot = (FP8 && KW < 128) ? (tile % (nst / 2)) * 2 : tile % nst;
  auto kstage = [&](int st) { return st + rot < nst ? st + rot : st + rot - nst; };

  // This lane's DMA sources: weight block wave + 4 b (b < WPW) and x block wave + 4 b (b < XPW;
  // x blocks past NXB repeat x block 0 into padding). Rows past the tile or the batch read a
  // clamped row: they only feed outputs that are never stored.
  const unsigned char* wsrc[SG::WPW];
  const unsigned char* xsrc[SG::XPW];
#pragma unroll
  for (int b = 0; b < SG::WPW; ++b) {
    const int blk = wave + 4 * b;
    constexpr int RPB = 1024 / RB;  // rows per block
    const int row = blk * RPB + lane / (RB / 16);
    const int c = (lane % (RB / 16)) ^ ((row / (16 / (RB / 16))) & (RB / 16 - 1));
    const int grow = row0 + (row < nrows ? row : 0);
    wsrc[b] = reinterpret_cast<const unsigned char*>(p.w) + (int64_t)grow * (FP8 ? K : 2 * K) + c * 16;
  }
#pragma unroll
  for (int b = 0; b < SG::XPW; ++b) {
    const int blk = (wave + 4 * b) < SG::NXB ? wave + 4 * b : 0;
    constexpr int RPB = 1024 / XB;
    const int xr = blk * RPB + lane / (XB / 16);
    const int c = (lane % (XB / 16)) ^ ((xr / (16 / (XB / 16))) & (XB / 16 - 1));
    xsrc[b] = reinterpret_cast<const unsigned char*>(p.x + (int64_t)(b0 + (xr < nbatch ? xr : 0)) * K) + c * 16;
  }
  const float* ssrc = nullptr;
  if constexpr (FP8) {
    const int row = wave * 16 + (lane & 15);
    ssrc = p.wscale + (int64_t)(row0 + (row < nrows ? row : 0)) * nblk;
  }
  // Both streams use the default cache policy: the non-temporal policy on the weight blocks
  // (read once) measured slower here than the default.
  auto issue = [&](int st) {
    st = st < nst ? st : nst - 1;  // clamped: the loop issues unconditionally
    lmd_lds* base = (lmd_lds*)ring + (st % STAGES) * STAGE;
    const int ks = kstage(st);      // the K stage this ring slot receives
#pragma unroll
    for (int b = 0; b < SG::WPW; ++b)
      lmd_dma16<LMD_POLICY_DEFAULT>(wsrc[b] + (size_t)ks * RB, base + (wave + 4 * b) * 1024);
#pragma unroll
    for (int b = 0; b < SG::XPW; ++b)
      lmd_dma16<LMD_POLICY_DEFAULT>(xsrc[b] + (size_t)ks * XB, base + SG::X_OFF + (wave + 4 * b) * 1024);
    if constexpr (FP8) lmd_dma4(ssrc + ks * KW / 128, base + SG::S_OFF + wave * 256);
  };

  const int r16 = lane & 15, kq = lane >> 4;
  const int myrow = wave * 16 + r16;
  const bool rok = myrow < nrows;
  f32x4_t acc[2], part[2];
  static_for<2>([&](auto h) {
    static_for<4>([&](auto v) {
      acc[h][decltype(v)::value] = 0.0f;
      part[h][decltype(v)::value] = 0.0f;
    });
  });

  // Stage st: KW / 32 MFMA steps. Step j, lane kq: K values 32 j + 8 kq .. +8, i.e. x chunk
  // 4 j + kq; weight chunk 4 j + kq (bf16), or bytes 8 (kq % 2) .. +8 of chunk 2 j + kq / 2
  // (E4M3). The E4M3 partial of a 128-wide block joins the accumulator times the row's scale
  // once the block is complete.
  auto compute = [&](int st) {
    const unsigned char* base = ring + (st % STAGES) * STAGE;
    static_for<KW / 32>([&](auto jj) {
      constexpr int j = jj;
      u32x4_t wv;
      if constexpr (FP8) {
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(base + lmd_off<RB>(myrow, 2 * j + (kq >> 1)));
        const uint32_t lo = (kq & 1) ? q[2] : q[0], hi = (kq & 1) ? q[3] : q[1];
        wv[0] = e4m3x2_to_bf16x2<false>(lo);
        wv[1] = e4m3x2_to_bf16x2<true>(lo);
        wv[2] = e4m3x2_to_bf16x2<false>(hi);
        wv[3] = e4m3x2_to_bf16x2<true>(hi);
      } else {
        wv = *reinterpret_cast<const u32x4_t*>(base + lmd_off<RB>(myrow, 4 * j + kq));
      }
      const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, wv);
      static_for<2>([&](auto h) {
        const bf16x8_t xa = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(base + SG::X_OFF + lmd_off<XB>(h * 16 + r16, 4 * j + kq)));
        if constexpr (FP8)
          part[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, part[h], 0, 0, 0);
        else
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, acc[h], 0, 0, 0);
      });
    });
    if constexpr (FP8) {
      // the block is complete after every stage (KW = 128) or every odd stage (KW = 64)
      const bool done = KW == 128 || (st & 1);
      const float sc = *reinterpret_cast<const float*>(base + SG::S_OFF + wave * 256 + r16 * 4);
      const float m = (done && rok) ? sc : 0.0f;
      static_for<2>([&](auto h) {
        static_for<4>([&](auto v) {
          constexpr int vv = v;
          acc[h][vv] = fmaf(part[h][vv], m, acc[h][vv]);
          part[h][vv] = done ? 0.0f : part[h][vv];
        });
      });
    }
  };

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) issue(st);
  for (int st = 0; st < nst; ++st) {
    // this wave's loads of stage st have landed once at most the loads of the STAGES - 2
    // newer stages are outstanding; the fence-free barrier then covers every wave's loads
    // and proves that all waves finished stage st - 1, whose slot the next issue overwrites
    constexpr int VM = SG::OPS * (STAGES - 2);
    static_assert(VM < 64, "vmcnt immediate is six bits");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(st + STAGES - 1);
    compute(st);
  }
  __syncthreads();  // every load landed (the waitcnt the barrier brings) and every wave is done
                    // with the ring before the candidates reuse it

  // Logits: lane holds weight row myrow and batch rows 4 kq + v (+16 h).
  static_for<2>([&](auto h) {
    static_for<4>([&](auto v) {
      constexpr int vv = v;
      const int b = h * 16 + kq * 4 + vv;
      if (rok && b < nbatch) p.logits[(int64_t)(b0 + b) * V + row0 + myrow] = acc[h][vv];
    });
  });
  // This workgroup's (max, lowest index) candidate per batch row: each wave over its 16 rows
  // (16-lane groups), then the four waves through LDS.
  float* cand_v = reinterpret_cast<float*>(ring);
  int* cand_i = reinterpret_cast<int*>(ring + 4 * LM_BATCH * sizeof(float));
  static_for<2>([&](auto h) {
    static_for<4>([&](auto v) {
      constexpr int vv = v;
      float val = (rok && !(acc[h][vv] != acc[h][vv])) ? acc[h][vv] : -INFINITY;
      int idx = row0 + myrow;
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        const float ov = __shfl_xor(val, off, 64);
        const int oi = __shfl_xor(idx, off, 64);
        if (better(ov, oi, val, idx)) {
          val = ov;
          idx = oi;
        }
      }
      if (r16 == 0) {
        cand_v[wave * LM_BATCH + h * 16 + kq * 4 + vv] = val;
        cand_i[wave * LM_BATCH + h * 16 + kq * 4 + vv] = idx;
      }
    });
  });
  __syncthreads();
  if (tid < LM_BATCH) {
    float val = cand_v[tid];
    int idx = cand_i[tid];
    for (int w = 1; w < 4; ++w)
      if (better(cand_v[w * LM_BATCH + tid], cand_i[w * LM_BATCH + tid], val, idx)) {
        val = cand_v[w * LM_BATCH + tid];
        idx = cand_i[w * LM_BATCH + tid];
      }
    float* part_v = reinterpret_cast<float*>(p.workspace);
    int* part_i = reinterpret_cast<int*>(part_v + (size_t)n_tiles * LM_BATCH);
    part_v[(size_t)tid * n_tiles + tile] = val;
    part_i[(size_t)tid * n_tiles + tile] = idx;
  }
}

// ---------------------------------------------------------------------------------------
// x-resident variant. The decode batch x is small and every weight byte is read once, so a
// workgroup keeps x in LDS and streams only the weight, straight into MFMA operand
// registers with non-temporal 16-byte loads (no LDS round trip for the weight).
//
// A workgroup owns 64 weight rows over the whole K, eight waves: wave w multiplies row group
// g = w % 4 (16 rows) over the K half h = w / 4 of each x slice. x goes to LDS one slice of
// XS_K columns at a time (16 BH rows x XS_K bf16 = 64 KB), double-buffered: slice s + 1 is
// loaded into registers while slice s is multiplied, then written to the other buffer. The
// weight of slice s + 2 is in flight meanwhile (two register sets, each one slice of the
// wave's rows), so a wave keeps about 24 KB of loads in flight with no LDS for them.
//
// Operands of v_mfma_f32_16x16x32_bf16: x is the row operand (16 batch rows x 32 K), the weight
// the column operand (32 K x 16 vocab rows), so lane l's accumulators belong to vocab row
// l % 16 and batch rows 4 (l / 16) + v. bf16: lane l loads row l % 16, K values 8 (l / 16) ..
// +8 of each 32-wide step. E4M3: one 16-byte load covers a pair of steps: K values
// 64 t + 16 (l / 16) .. +16, the first eight feeding step 2 t and the rest step 2 t + 1 (a
// permutation of K inside the pair, applied to x as well); each 128-wide block's partial
// joins the accumulator times the row's block scale. The two K halves of a row group are
// added in a fixed order (half 0 + half 1) at the end, through LDS.
//
// x rows in LDS: row b's 16-byte chunk c sits at chunk c ^ (b % 16), so the 16 lanes that read
// one chunk column of 16 rows hit 16 distinct bank groups.
template <int BH>
struct LmxShape {
  static constexpr int BROWS = 16 * BH;                  // batch rows per pass: 32 or 64
  static constexpr int XS_K = BH == 2 ? 1024 : 512;      // x slice width (K values)
  static constexpr int HALF_K = XS_K / 2;                // a wave's share of a slice
  static constexpr int XBYTES = BROWS * XS_K * 2;        // one x buffer: 64 KB
  static constexpr int XCHUNKS = XBYTES / 16 / 512;      // 16-byte x chunks per thread per slice
  static_assert(XBYTES == 65536 && XCHUNKS == 8, "x slice layout");
};
constexpr int LMX_ROWS = 64;
constexpr int LMX_THREADS = 512;

// End of a 64-row tile computed by eight waves, wave w holding row group w % 4 (16 rows) of K
// half w / 4 for 16 BH batch rows (acc[hb]: lane l has tile row 16 (w % 4) + l % 16 and batch
// rows 16 hb + 4 (l / 16) + v). The two halves are added in a fixed order (half 0 + half 1)
// through `red` (2 x 16 BH x 64 floats of free LDS), then the logits are stored and the
// tile's (max, lowest index) candidate per batch row goes to the workspace, row-major
// [batch row][tile].
template <int BH>
__device__ __forceinline__ void lm_tile64_finish(const LmHeadProblem& p, const f32x4_t (&acc)[BH], float* red,
                                                 int n_tiles, int b0, int nbatch, int tile) {
  constexpr int BROWS = 16 * BH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = wave & 3, hk = wave >> 2, r16 = lane & 15, q = lane >> 4;
  const int row0 = tile * LMX_ROWS, V = p.V;
  static_for<BH>([&](auto hb) {
    static_for<4>([&](auto v) {
      constexpr int vv = v;
      const int b = hb * 16 + q * 4 + vv;
      red[(hk * BROWS + b) * LMX_ROWS + g * 16 + r16] = acc[hb][vv];
    });
  });
  __syncthreads();
  float* part_v = reinterpret_cast<float*>(p.workspace);
  int* part_i = reinterpret_cast<int*>(part_v + (size_t)n_tiles * BROWS);
  const int r = lane;  // row of the tile; each wave takes batch rows wave, wave + 8, ...
  const bool ok_r = row0 + r < V;
#pragma unroll
  for (int b = wave; b < BROWS; b += LMX_THREADS / 64) {
    const float sum = red[b * LMX_ROWS + r] + red[(BROWS + b) * LMX_ROWS + r];
    if (ok_r && b < nbatch) p.logits[(int64_t)(b0 + b) * V + row0 + r] = sum;
    float val = (ok_r && !(sum != sum)) ? sum : -INFINITY;
    int idx = row0 + r;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(val, off, 64);
      const int oi = __shfl_xor(idx, off, 64);
      if (better(ov, oi, val, idx)) {
        val = ov;
        idx = oi;
      }
    }
    if (lane == 0) {
      part_v[(size_t)b * n_tiles + tile] = val;
      part_i[(size_t)b * n_tiles + tile] = idx;
    }
  }
}

template <bool FP8, int BH>
__global__ __launch_bounds__(LMX_THREADS) void lm_head_xres_kernel(LmHeadProblem p, int n_tiles, int b0) {
  using SH = LmxShape<BH>;
  constexpr int XS_K = SH::XS_K, HALF_K = SH::HALF_K, BROWS = SH::BROWS;
  constexpr int XROW = XS_K * 2;                                // bytes per x row in LDS
  constexpr int NLD = FP8 ? HALF_K / 64 : HALF_K / 32;          // weight loads per lane per slice
  constexpr int NBLK = FP8 ? HALF_K / 128 : 1;                  // scale blocks per lane per slice
  __shared__ __attribute__((aligned(16))) unsigned char xs[2 * SH::XBYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, V = p.V;
  const int nbatch = min(BROWS, p.B - b0);
  const int tile = blockIdx.x, row0 = tile * LMX_ROWS;
  const int g = wave & 3, hk = wave >> 2;
  const int r16 = lane & 15, q = lane >> 4;
  const int myrow = row0 + g * 16 + r16;
  const bool rok = myrow < V;
  const int nslice = (K + XS_K - 1) / XS_K;
  const int nkb = K / 128;

  // weight row of this lane (a clamped row past V: its outputs are never stored)
  const unsigned char* wrow = reinterpret_cast<const unsigned char*>(p.w) +
                              (int64_t)(rok ? myrow : row0) * (FP8 ? (int64_t)K : 2 * (int64_t)K);
  const float* srow = FP8 ? p.wscale + (int64_t)(rok ? myrow : row0) * nkb : nullptr;

  struct WRegs {
    u32x4_t w[NLD];
    float sc[NBLK];
  };
  // Loads of slice s for this wave: step / pair i covers K from kbase + i * (FP8 ? 64 : 32).
  // Steps past K load a valid address (the row's first bytes) and are skipped when multiplied.
  auto wload = [&](int s, WRegs& r) {
    const int kbase = s * XS_K + hk * HALF_K;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int k = kbase + i * (FP8 ? 64 : 32);
      const int64_t off = k < K ? (FP8 ? (int64_t)k + 16 * q : 2 * ((int64_t)k + 8 * q)) : 0;
      r.w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wrow + off));
    }
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < NBLK; ++j) {
        const int blk = (kbase >> 7) + j;
        r.sc[j] = blk < nkb ? srow[blk] : 0.0f;
      }
    }
  };
  // x slice s: thread chunk j is chunk id = tid + 512 j of the [BROWS][XS_K] slice (row
  // id / (XS_K / 8), logical chunk id % (XS_K / 8)); rows past the batch and columns past K read a
  // valid address (their products are never stored, or meet skipped steps).
  u32x4_t xr[SH::XCHUNKS];
  auto xload = [&](int s) {
#pragma unroll
    for (int j = 0; j < SH::XCHUNKS; ++j) {
      const int id = tid + LMX_THREADS * j;
      const int b = id / (XS_K / 8), c = id % (XS_K / 8);
      const int k = s * XS_K + c * 8;
      const uint16_t* src = p.x + (int64_t)(b0 + (b < nbatch ? b : 0)) * K + (k < K ? k : 0);
      xr[j] = *reinterpret_cast<const u32x4_t*>(src);
    }
  };
  auto xstore = [&](int buf) {
    unsigned char* base = xs + buf * SH::XBYTES;
#pragma unroll
    for (int j = 0; j < SH::XCHUNKS; ++j) {
      const int id = tid + LMX_THREADS * j;
      const int b = id / (XS_K / 8), c = id % (XS_K / 8);
      *reinterpret_cast<u32x4_t*>(base + b * XROW + ((c ^ (b & 15)) << 4)) = xr[j];
    }
  };

  f32x4_t acc[BH], part[BH];
  static_for<BH>([&](auto h) {
    static_for<4>([&](auto v) {
      acc[h][decltype(v)::value] = 0.0f;
      part[h][decltype(v)::value] = 0.0f;
    });
  });

  // x fragment of batch-row half hb at logical chunk c of the slice in buffer buf
  auto xfrag = [&](int buf, int hb, int c) {
    const int b = hb * 16 + r16;
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + buf * SH::XBYTES + b * XROW +
                                                                           ((c ^ r16) << 4)));
  };
  auto compute = [&](int s, int buf, const WRegs& r) {
    const int kbase = s * XS_K + hk * HALF_K;
    static_for<NLD>([&](auto ii) {
      constexpr int i = ii;
      if constexpr (FP8) {
        const int k = kbase + i * 64;  // pair of steps, uniform validity (K % 128 == 0)
        if (k < K) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t lo = half ? r.w[i][2] : r.w[i][0], hi = half ? r.w[i][3] : r.w[i][1];
            u32x4_t wv;
            wv[0] = e4m3x2_to_bf16x2<false>(lo);
            wv[1] = e4m3x2_to_bf16x2<true>(lo);
            wv[2] = e4m3x2_to_bf16x2<false>(hi);
            wv[3] = e4m3x2_to_bf16x2<true>(hi);
            const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, wv);
            // x values K = k + 16 q + 8 half .. +8: logical chunk (k - slice start) / 8 + 2 q + half
            const int c = (hk * HALF_K + i * 64) / 8 + 2 * q + half;
            static_for<BH>([&](auto hb) {
              part[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xfrag(buf, hb, c), wb, part[hb], 0, 0, 0);
            });
          }
        }
        if constexpr (i % 2 == 1) {  // a 128-wide block is complete: scale it into the sum
          const float sc = rok ? r.sc[i / 2] : 0.0f;
          static_for<BH>([&](auto hb) {
            static_for<4>([&](auto v) {
              constexpr int vv = v;
              acc[hb][vv] = fmaf(part[hb][vv], sc, acc[hb][vv]);
              part[hb][vv] = 0.0f;
            });
          });
        }
      } else {
        const int k = kbase + i * 32;  // uniform validity (K % 32 == 0)
        if (k < K) {
          const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, r.w[i]);
          const int c = (hk * HALF_K + i * 32) / 8 + q;
          static_for<BH>([&](auto hb) {
            acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xfrag(buf, hb, c), wb, acc[hb], 0, 0, 0);
          });
        }
      }
    });
  };

  WRegs w0, w1;
  xload(0);
  wload(0, w0);
  xstore(0);
  if (nslice > 1) {
    xload(1);
    wload(1, w1);
  }
  __syncthreads();
  for (int s = 0; s < nslice; s += 2) {
    // even slice: buffer 0, registers w0
    compute(s, 0, w0);
    if (s + 1 < nslice) xstore(1);
    if (s + 2 < nslice) {
      xload(s + 2);
      wload(s + 2, w0);
    }
    __syncthreads();
    if (s + 1 >= nslice) break;
    // odd slice: buffer 1, registers w1
    compute(s + 1, 1, w1);
    if (s + 2 < nslice) xstore(0);
    if (s + 3 < nslice) {
      xload(s + 3);
      wload(s + 3, w1);
    }
    __syncthreads();
  }

  // every wave passed the loop's last barrier: the x buffers are free for the reduction
  lm_tile64_finish<BH>(p, acc, reinterpret_cast<float*>(xs), n_tiles, b0, nbatch, blockIdx.x);
}

// ---------------------------------------------------------------------------------------
// Row-quad kernel (the default). The work split is the x-resident
// kernel's: a workgroup owns 64 weight rows over the whole K, wave w multiplies row group
// g = w % 4 (16 rows) over K half h = w / 4 of every x slice, x sits in LDS one slice of XS_K
// columns at a time (double-buffered), and the weight goes to registers with non-temporal
// 16-byte loads. What differs is the fetch shape. The operand layout wants 16 rows x 64
// bytes per load instruction, and that shape streamed about 30% slower on this GPU than
// 4 rows x 256 contiguous bytes, the fastest of the shapes measured (as fast as a linear
// sweep of the workgroup's rows; tpt_stream_probe). So here lane l of a load reads row l / 16 at bytes
// 16 (l % 16) of a 256-byte run, and a "window" is four such loads: 16 rows x 256 bytes
// (128 bf16 or 256 E4M3 K values). The wave writes its window to its own 4 KB of LDS and
// reads it back in the operand layout (lane l: row l % 16, 16 bytes at chunk 4 t + l / 16 for
// step t). No other wave touches that memory and a wave's LDS operations complete in
// order, so the round trip needs no barrier.
//
// D windows of weight loads are in flight. A slice's x loads are issued just before the
// weight loads of the slice's first window, so that waiting for them (before they are
// written to LDS at the end of the previous slice) never waits for a weight load that is
// not needed yet; NXS register sets hold them, which bounds D by NXS times the windows per
// slice. With ROT, slices are visited from slice (tile mod slice count) on, wrapping, so that
// the tiles in flight read different offsets of their rows (as in the LDS-ring kernel).
//
// Operand layout for v_mfma_f32_16x16x32_bf16 is the x-resident kernel's: x the row operand,
// the weight the column operand; bf16 step t of a window takes K values 32 t + 8 q .. +8
// (q = lane / 16); an E4M3 16-byte read covers K values 64 t + 16 q .. +16, the first eight
// feeding one MFMA and the rest the next (the same permutation of K applied to x).
constexpr int lm_gcd(int a, int b) { return b == 0 ? a : lm_gcd(b, a % b); }
constexpr int lm_lcm(int a, int b) { return a / lm_gcd(a, b) * b; }

//
// RPW = 2: the workgroup owns two 64-row blocks (128 rows) and wave w multiplies row group g in
// both, rows 16 g and 64 + 16 g of the workgroup's rows, so every x fragment a wave reads from
// LDS feeds two MFMAs and each workgroup's x slices serve twice the weight bytes. A window is
// then one 16-row window per block (eight loads); candidates stay per 64-row block. A tuning
// shape only: on the decode shard its 126 workgroups leave half the CUs idle, and a CU streams no
// faster with the extra rows (1.5x the 64-row kernel's time).
template <bool FP8, int XS_K, int BH, int RPW>
struct LmqShape {
  static constexpr int BROWS = 16 * BH;              // batch rows per pass: 32 or 64
  static constexpr int WIN_K = FP8 ? 256 : 128;      // K values per window (256 bytes of a row)
  static constexpr int WPS = XS_K / 2 / WIN_K;       // windows per slice per wave
  static constexpr int XBYTES = BROWS * XS_K * 2;    // one x buffer
  static constexpr int XCH = XBYTES / 16 / 512;      // 16-byte x chunks per thread per slice
  static constexpr int STAGE = 16 * 256 * RPW;       // one wave's windows in LDS
  static constexpr int LDS = 2 * XBYTES + 8 * STAGE;
  static_assert(WPS >= 1 && XCH >= 1 && LDS <= 160 * 1024 && (RPW == 1 || RPW == 2), "row-quad shape");
};

template <bool FP8, int XS_K, int D, int NXS, bool ROT, int BH, int RPW>
__global__ __launch_bounds__(512) void lm_head_quad_kernel(LmHeadProblem p, int n_tiles, int b0) {
  using SH = LmqShape<FP8, XS_K, BH, RPW>;
  constexpr int WIN_K = SH::WIN_K, WPS = SH::WPS, XROW = XS_K * 2, XCH = SH::XCH;
  static_assert(D >= 1 && D <= NXS * WPS, "NXS x register sets allow D <= NXS windows per slice");
  __shared__ __attribute__((aligned(16))) unsigned char lds[SH::LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, V = p.V;
  const int nbatch = min(SH::BROWS, p.B - b0);
  const int tile = blockIdx.x, row0 = tile * 64 * RPW;
  const int g = wave & 3, hk = wave >> 2;
  const int r16 = lane & 15, q = lane >> 4;
  const int nslice = K / XS_K, nw = nslice * WPS;
  const int rot = ROT ? tile % nslice : 0;
  const int nkb = K / 128;
  unsigned char* const xs = lds;                                  // [2][BROWS][XS_K] bf16
  unsigned char* const stage = lds + 2 * SH::XBYTES + wave * SH::STAGE;

  // Load layout: lane l of quad j in block i reads row 64 i + 16 g + 4 j + l / 16 (a row past V
  // reads row V - 1; its outputs are never stored) at bytes 16 (l % 16) of the window.
  const unsigned char* wq[RPW][4];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = min(row0 + 64 * i + 16 * g + 4 * j + q, V - 1);
      wq[i][j] = reinterpret_cast<const unsigned char*>(p.w) + (int64_t)row * (FP8 ? K : 2 * K) + 16 * r16;
    }
  // Operand layout: lane l holds row 64 i + 16 g + l % 16 of block i.
  bool rok[RPW];
  const float* srow[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int myrow = row0 + 64 * i + 16 * g + r16;
    rok[i] = myrow < V;
    srow[i] = FP8 ? p.wscale + (int64_t)min(myrow, V - 1) * nkb : nullptr;
  }

  auto slice_of = [&](int si) { return si + rot < nslice ? si + rot : si + rot - nslice; };
  // first K value of this wave's window wi
  auto win_k = [&](int wi) { return slice_of(wi / WPS) * XS_K + hk * (XS_K / 2) + (wi % WPS) * WIN_K; };

  struct Win {
    u32x4_t w[RPW][4];
    float sc[RPW][2];
  };
  auto wload = [&](int wi, Win& r) {
    const int k = win_k(wi);
    const int64_t off = FP8 ? (int64_t)k : 2 * (int64_t)k;
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r.w[i][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wq[i][j] + off));
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        r.sc[i][0] = srow[i][k / 128];
        r.sc[i][1] = srow[i][k / 128 + 1];
      }
    }
  };
  // x slice si (in visiting order): thread chunk j is chunk tid + 512 j of the [BROWS][XS_K]
  // slice; batch rows past the pass read row b0 (their outputs are never stored). Row b's
  // chunk c sits at chunk c ^ (b % 16).
  u32x4_t xr[NXS][XCH];  // register sets, by slice index mod NXS
  auto xload = [&](int si, u32x4_t (&d)[XCH]) {
    const int s = slice_of(si);
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int id = tid + 512 * j, b = id / (XS_K / 8), c = id % (XS_K / 8);
      d[j] = *reinterpret_cast<const u32x4_t*>(p.x + (int64_t)(b0 + (b < nbatch ? b : 0)) * K + s * XS_K + c * 8);
    }
  };
  auto xstore = [&](int buf, const u32x4_t (&d)[XCH]) {
    unsigned char* base = xs + buf * SH::XBYTES;
#pragma unroll
    for (int j = 0; j < XCH; ++j) {
      const int id = tid + 512 * j, b = id / (XS_K / 8), c = id % (XS_K / 8);
      *reinterpret_cast<u32x4_t*>(base + b * XROW + ((c ^ (b & 15)) << 4)) = d[j];
    }
  };

  f32x4_t acc[RPW][BH], part[RPW][BH];
  static_for<RPW>([&](auto i) {
    static_for<BH>([&](auto h) {
      static_for<4>([&](auto v) {
        acc[i][h][decltype(v)::value] = 0.0f;
        part[i][h][decltype(v)::value] = 0.0f;
      });
    });
  });

  auto compute = [&](const Win& r, int buf, int w2) {
    // each block's window through this wave's LDS stage (4 KB per block): row R's chunk C at
    // chunk C ^ R
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * j + q;
        *reinterpret_cast<u32x4_t*>(stage + i * 4096 + row * 256 + ((r16 ^ row) << 4)) = r.w[i][j];
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    u32x4_t wf[RPW][4];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        wf[i][t] = *reinterpret_cast<const u32x4_t*>(stage + i * 4096 + r16 * 256 + (((4 * t + q) ^ r16) << 4));
    const unsigned char* xb = xs + buf * SH::XBYTES;
    const int cx0 = hk * (XS_K / 16) + w2 * (WIN_K / 8);  // the window's first x chunk
    auto xfrag = [&](int hb, int c) {
      return __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(xb + (hb * 16 + r16) * XROW + ((c ^ r16) << 4)));
    };
    static_for<4>([&](auto tt) {
      constexpr int t = tt;
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = cx0 + 8 * t + 2 * q + h;
          bf16x8_t xf[BH];
          static_for<BH>([&](auto hb) { xf[hb] = xfrag(hb, c); });
          static_for<RPW>([&](auto i) {
            const uint32_t lo = h ? wf[i][t][2] : wf[i][t][0], hi = h ? wf[i][t][3] : wf[i][t][1];
            u32x4_t wv;
            wv[0] = e4m3x2_to_bf16x2<false>(lo);
            wv[1] = e4m3x2_to_bf16x2<true>(lo);
            wv[2] = e4m3x2_to_bf16x2<false>(hi);
            wv[3] = e4m3x2_to_bf16x2<true>(hi);
            const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, wv);
            static_for<BH>([&](auto hb) {
              part[i][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[hb], wb, part[i][hb], 0, 0, 0);
            });
          });
        }
        if constexpr (t % 2 == 1) {  // a 128-wide block is complete: scale it into the sum
          static_for<RPW>([&](auto i) {
            const float sc = rok[i] ? r.sc[i][t / 2] : 0.0f;
            static_for<BH>([&](auto hb) {
              static_for<4>([&](auto v) {
                constexpr int vv = v;
                acc[i][hb][vv] = fmaf(part[i][hb][vv], sc, acc[i][hb][vv]);
                part[i][hb][vv] = 0.0f;
              });
            });
          });
        }
      } else {
        const int c = cx0 + 4 * t + q;
        static_for<BH>([&](auto hb) {
          const bf16x8_t xf = xfrag(hb, c);
          static_for<RPW>([&](auto i) {
            const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, wf[i][t]);
            acc[i][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, wb, acc[i][hb], 0, 0, 0);
          });
        });
      }
    });
  };

  // The window loop runs in periods of PER windows, a common multiple of D and of two slices,
  // so that every ring slot, x register set and x buffer index is a constant and every load
  // is unconditional: the wait before each use then counts exactly the loads issued after it.
  // The last period issues no loads past the last window.
  constexpr int PER = lm_lcm(lm_lcm(D, NXS * WPS), 2 * WPS);
  Win ring[D];
  xload(0, xr[0]);
  static_for<D>([&](auto jj) {
    constexpr int j = jj;
    if constexpr (j > 0 && j % WPS == 0) xload(j / WPS, xr[(j / WPS) % NXS]);
    wload(j, ring[j]);
  });
  xstore(0, xr[0]);
  __syncthreads();
  auto period = [&](int base, auto last_c) {
    constexpr bool LAST = decltype(last_c)::value;
    static_for<PER>([&](auto jj) {
      constexpr int j = jj;
      constexpr int slot = j % D, w2 = j % WPS, par = (j / WPS) & 1;
      compute(ring[slot], par, w2);
      constexpr int nxj = j + D;  // the window whose loads take this slot
      if constexpr (!LAST || nxj < PER) {
        if constexpr (nxj % WPS == 0) xload((base + nxj) / WPS, xr[(nxj / WPS) % NXS]);
        wload(base + nxj, ring[slot]);
      }
      if constexpr (w2 == WPS - 1) {  // a slice is done: the next one to LDS
        if constexpr (!LAST || j != PER - 1) xstore(par ^ 1, xr[(j / WPS + 1) % NXS]);
        __syncthreads();
      }
    });
  };
  int base = 0;
  for (; base < nw - PER; base += PER) period(base, std::false_type{});
  period(base, std::true_type{});
  // the last window ended a slice: every wave passed that barrier, the x buffers are free.
  // Block i is 64-row tile RPW tile + i; a second block past the shard's last tile has no rows.
  static_for<RPW>([&](auto i) {
    constexpr int ii = i;
    const int t64 = tile * RPW + ii;
    if (t64 < n_tiles) {
      if constexpr (ii > 0) __syncthreads();  // the previous block's reads of the buffer are done
      lm_tile64_finish<BH>(p, acc[ii], reinterpret_cast<float*>(xs), n_tiles, b0, nbatch, t64);
    }
  });
}

// Reduces every workgroup's (max, lowest index) candidate of one batch row (one workgroup
// per row). The candidates are stored row-major, [batch row][tile] (values, then indices after
// stride x n_tiles values), so a row's candidates are contiguous: each thread loads its
// candidates with independent, coalesced loads (one memory round trip),
// then wave and workgroup reductions. Running as its own kernel after the logits kernel makes
// the candidates visible across XCDs without device-scope fences in the streaming kernel.
__global__ __launch_bounds__(LM_FIN_THREADS) void lm_head_argmax_kernel(LmHeadProblem p, int n_tiles, int b0,
                                                                         int stride) {
  __shared__ float sv[LM_FIN_THREADS / 64];
  __shared__ int si[LM_FIN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const float* part_v = reinterpret_cast<const float*>(p.workspace);
  const int* part_i = reinterpret_cast<const int*>(part_v + (size_t)n_tiles * stride);
  float v = -INFINITY;
  int idx = 0x7fffffff;
  for (int t = tid; t < n_tiles; t += LM_FIN_THREADS) {
    const float tv = part_v[(size_t)b * n_tiles + t];
    const int ti = part_i[(size_t)b * n_tiles + t];
    if (better(tv, ti, v, idx)) {
      v = tv;
      idx = ti;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float ov = __shfl_xor(v, off, 64);
    int oi = __shfl_xor(idx, off, 64);
    if (better(ov, oi, v, idx)) {
      v = ov;
      idx = oi;
    }
  }
  if (lane == 0) {
    sv[wave] = v;
    si[wave] = idx;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < LM_FIN_THREADS / 64; ++w)
      if (better(sv[w], si[w], v, idx)) {
        v = sv[w];
        idx = si[w];
      }
    if (idx == 0x7fffffff) idx = 0;  // every logit NaN: index 0, as the lowest index of -inf
    p.argmax[b0 + b] = idx;
    if (p.maxval != nullptr) p.maxval[b0 + b] = v;
  }
}

// K split over KS workgroups: logits = the slices' partial logits added in slice order; then
// the row's (max, lowest index). One workgroup per batch row.
template <int KS>
__global__ __launch_bounds__(LM_FIN_THREADS) void lm_head_sum_argmax_kernel(LmHeadProblem p, int b0) {
  __shared__ float sv[LM_FIN_THREADS / 64];
  __shared__ int si[LM_FIN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, V = p.V;
  const float* part = reinterpret_cast<const float*>(p.workspace);
  float v = -INFINITY;
  int idx = 0x7fffffff;
  for (int j = tid; j < V; j += LM_FIN_THREADS) {
    float sum = part[(size_t)b * V + j];
#pragma unroll
    for (int k = 1; k < KS; ++k) sum += part[((size_t)k * LM_BATCH + b) * V + j];
    p.logits[(int64_t)(b0 + b) * V + j] = sum;
    const float cand = sum != sum ? -INFINITY : sum;
    if (better(cand, j, v, idx)) {
      v = cand;
      idx = j;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float ov = __shfl_xor(v, off, 64);
    int oi = __shfl_xor(idx, off, 64);
    if (better(ov, oi, v, idx)) {
      v = ov;
      idx = oi;
    }
  }
  if (lane == 0) {
    sv[wave] = v;
    si[wave] = idx;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < LM_FIN_THREADS / 64; ++w)
      if (better(sv[w], si[w], v, idx)) {
        v = sv[w];
        idx = si[w];
      }
    if (idx == 0x7fffffff) idx = 0;
    p.argmax[b0 + b] = idx;
    if (p.maxval != nullptr) p.maxval[b0 + b] = v;
  }
}

int lm_tiles(int V, int chunk, int rows, int* tiles_per_chunk) {
  const int n_chunks = (V + chunk - 1) / chunk;
  const int per = (min(chunk, V) + rows - 1) / rows;
  *tiles_per_chunk = per;
  const int last_rows = V - (n_chunks - 1) * chunk;
  return (n_chunks - 1) * per + (last_rows + rows - 1) / rows;
}

template <bool FP8, int S>
void launch_shape(const LmHeadProblem& p, int b0, hipStream_t stream) {
  constexpr LmShape sh = kLmShapes[S];
  int per;
  const int n_tiles = lm_tiles(p.V, p.chunk, sh.G * 16, &per);
  hipLaunchKernelGGL((lm_head_kernel<FP8, sh.G, sh.W, sh.P, sh.KS>), dim3(n_tiles * sh.KS), dim3(sh.W * 64), 0,
                     stream, p, per, n_tiles, b0);
  if constexpr (sh.KS > 1)
    hipLaunchKernelGGL((lm_head_sum_argmax_kernel<sh.KS>), dim3(min(LM_BATCH, p.B - b0)), dim3(LM_FIN_THREADS), 0,
                       stream, p, b0);
  else
    hipLaunchKernelGGL(lm_head_argmax_kernel, dim3(min(LM_BATCH, p.B - b0)), dim3(LM_FIN_THREADS), 0, stream, p,
                       n_tiles, b0, LM_BATCH);
}

// Direct-to-LDS launch shapes (stage row bytes RB, ring depth): the ring fills 160 KB of LDS.
template <bool FP8, int RB, int STAGES>
void launch_dma(const LmHeadProblem& p, int b0, hipStream_t stream) {
  static_assert(STAGES * LmdStage<FP8, RB>::BYTES <= 160 * 1024, "ring exceeds LDS");
  const int n_tiles = (p.V + LMD_ROWS - 1) / LMD_ROWS;  // whole 64-row blocks of the shard
  hipLaunchKernelGGL((lm_head_dma_kernel<FP8, RB, STAGES>), dim3(n_tiles), dim3(LMD_THREADS), 0, stream, p, n_tiles,
                     b0);
  hipLaunchKernelGGL(lm_head_argmax_kernel, dim3(min(LM_BATCH, p.B - b0)), dim3(LM_FIN_THREADS), 0, stream, p, n_tiles,
                     b0, LM_BATCH);
}

// x-resident kernel: batch passes of 32 rows (BH = 2) or, for more than 32 rows, of 64 (BH = 4).
template <bool FP8, int BH>
void launch_xres(const LmHeadProblem& p, int b0, hipStream_t stream) {
  const int n_tiles = (p.V + LMX_ROWS - 1) / LMX_ROWS;
  hipLaunchKernelGGL((lm_head_xres_kernel<FP8, BH>), dim3(n_tiles), dim3(LMX_THREADS), 0, stream, p, n_tiles, b0);
  hipLaunchKernelGGL(lm_head_argmax_kernel, dim3(min(16 * BH, p.B - b0)), dim3(LM_FIN_THREADS), 0, stream, p, n_tiles,
                     b0, 16 * BH);
}

bool xres_ok(const LmHeadProblem& p) { return p.w_fp8 ? p.K % 128 == 0 : p.K % 32 == 0; }
int xres_pass_rows(const LmHeadProblem& p) { return p.B <= 32 ? 32 : 64; }

// Row-quad kernel. Shapes kLmQuadShape + i take variant i: x slice width, windows in flight,
// x register sets, staggered slice order, 16-row batch groups per pass; for bf16 and E4M3.
struct LmQuadCfg {
  int xs_k, d, nxs, rot, bh, rpw;
};
constexpr int kLmQuadCount = 6;
constexpr LmQuadCfg kLmQuad[kLmQuadCount][2] = {
    {{256, 2, 2, 1, 2, 1}, {512, 2, 2, 1, 2, 1}},   // the default up to 32 batch rows
    {{256, 2, 2, 1, 4, 1}, {512, 2, 2, 1, 4, 1}},   // the default above: 64-row passes
    {{256, 4, 4, 1, 2, 1}, {512, 4, 4, 1, 2, 1}},   {{512, 4, 2, 1, 2, 1}, {1024, 2, 2, 1, 2, 1}},
    {{512, 2, 2, 1, 4, 1}, {512, 1, 1, 1, 4, 1}},
    {{256, 2, 2, 1, 2, 2}, {512, 2, 2, 1, 2, 2}}};  // 128 rows per workgroup
bool is_quad(int shape) { return shape >= kLmQuadShape && shape < kLmQuadShape + kLmQuadCount; }
int quad_pass_rows(const LmHeadProblem& p, int shape) { return 16 * kLmQuad[shape - kLmQuadShape][p.w_fp8 ? 1 : 0].bh; }
// K must hold whole periods of windows (see lm_head_quad_kernel).
bool quad_ok(const LmHeadProblem& p, int shape) {
  const int fp8 = p.w_fp8 ? 1 : 0;
  const LmQuadCfg& c = kLmQuad[shape - kLmQuadShape][fp8];
  const int wps = c.xs_k / 2 / (fp8 ? 256 : 128);
  return p.K >= c.xs_k && p.K % c.xs_k == 0 && (p.K / c.xs_k * wps) % lm_lcm(lm_lcm(c.d, c.nxs * wps), 2 * wps) == 0;
}
template <bool FP8, int I>
void launch_quad(const LmHeadProblem& p, int b0, hipStream_t stream) {
  constexpr LmQuadCfg c = kLmQuad[I][FP8];
  const int n_tiles = (p.V + 63) / 64;  // 64-row tiles: one argmax candidate each
  hipLaunchKernelGGL((lm_head_quad_kernel<FP8, c.xs_k, c.d, c.nxs, c.rot != 0, c.bh, c.rpw>),
                     dim3((n_tiles + c.rpw - 1) / c.rpw), dim3(512), 0, stream, p, n_tiles, b0);
  hipLaunchKernelGGL(lm_head_argmax_kernel, dim3(min(16 * c.bh, p.B - b0)), dim3(LM_FIN_THREADS), 0, stream, p, n_tiles,
                     b0, 16 * c.bh);
}

// A row-quad shape whose slice width does not divide K runs the LDS-ring default instead.
int effective_shape(const LmHeadProblem& p, int shape) {
  if (is_quad(shape) && !quad_ok(p, shape)) return kLmRingShape;
  return shape;
}

// The default launch shape: the row-quad kernel, in 32-row batch passes up to 32 rows and in
// 64-row passes above, which stream the weight once per 64 rows. On the decode workload (K 4096,
// 16032 rows; kernel times from a HIP kernel trace): 32 rows 25.1 us bf16 and 19.7 us E4M3
// (512-wide x slices for E4M3: 0.4-0.5 us under 1024-wide ones in four interleaved rounds),
// against 30.3 and 24.3 us for the LDS ring; 64 rows in one pass 30.8 and 28.9 us, against
// 40.2 and 32.7 us for the x-resident kernel. A K that the row-quad kernel cannot take runs the
// x-resident kernel above 32 rows if it can, else the LDS ring.
int default_shape(const LmHeadProblem& p) {
  if (p.B > 32) return quad_ok(p, kLmQuadShape + 1) ? kLmQuadShape + 1 : xres_ok(p) ? kLmXresShape : kLmRingShape;
  return quad_ok(p, kLmQuadShape) ? kLmQuadShape : kLmRingShape;
}

template <bool FP8>
void launch_any(const LmHeadProblem& p, int shape, int b0, hipStream_t stream) {
  switch (shape) {
    case kLmDmaShape:  // 64-byte stages (bf16 needs K % 32 == 0)
      if (FP8) launch_dma<true, 64, 17>(p, b0, stream);
      else if (p.K % 32 == 0) launch_dma<false, 64, 20>(p, b0, stream);
      else launch_shape<FP8, 4>(p, b0, stream);  // ragged K: the register-streaming kernel
      break;
    case kLmDmaShape + 1:  // 128-byte stages (bf16 needs K % 64 == 0)
      if (FP8) launch_dma<true, 128, 9>(p, b0, stream);
      else if (p.K % 64 == 0) launch_dma<false, 128, 13>(p, b0, stream);
      else launch_shape<FP8, 4>(p, b0, stream);
      break;
    case kLmXresShape:  // batch passes of xres_pass_rows rows (see launch_lm_head)
      if (xres_pass_rows(p) == 32) launch_xres<FP8, 2>(p, b0, stream);
      else launch_xres<FP8, 4>(p, b0, stream);
      break;
    case kLmQuadShape: launch_quad<FP8, 0>(p, b0, stream); break;
    case kLmQuadShape + 1: launch_quad<FP8, 1>(p, b0, stream); break;
    case kLmQuadShape + 2: launch_quad<FP8, 2>(p, b0, stream); break;
    case kLmQuadShape + 3: launch_quad<FP8, 3>(p, b0, stream); break;
    case kLmQuadShape + 4: launch_quad<FP8, 4>(p, b0, stream); break;
    case kLmQuadShape + 5: launch_quad<FP8, 5>(p, b0, stream); break;
    case 1: launch_shape<FP8, 1>(p, b0, stream); break;
    case 2: launch_shape<FP8, 2>(p, b0, stream); break;
    case 3: launch_shape<FP8, 3>(p, b0, stream); break;
    case 4: launch_shape<FP8, 4>(p, b0, stream); break;
    case 5: launch_shape<FP8, 5>(p, b0, stream); break;
    case 6: launch_shape<FP8, 6>(p, b0, stream); break;
    case 7: launch_shape<FP8, 7>(p, b0, stream); break;
    default: launch_shape<FP8, 0>(p, b0, stream); break;
  }
}

}  // namespace

int lm_head_shape_count() { return kLmQuadShape + kLmQuadCount; }

// Workspace of one launch shape (-1: the default): per-workgroup candidates, or KS slices of
// partial logits for one batch pass.
size_t lm_head_shape_workspace_bytes(int shape, int B, int V, int K, bool fp8, int chunk) {
  LmHeadProblem q{};
  q.B = B;
  q.K = K;
  q.w_fp8 = fp8;
  if (shape < 0) shape = default_shape(q);
  shape = effective_shape(q, shape);
  if (is_quad(shape))
    return (size_t)((V + 63) / 64) * quad_pass_rows(q, shape) * (sizeof(float) + sizeof(int));
  if (shape == kLmXresShape && xres_ok(q))
    return (size_t)((V + LMX_ROWS - 1) / LMX_ROWS) * xres_pass_rows(q) * (sizeof(float) + sizeof(int));
  if (shape == kLmDmaShape || shape == kLmDmaShape + 1)
    if (fp8 || K % (shape == kLmDmaShape ? 32 : 64) == 0)
      return (size_t)((V + LMD_ROWS - 1) / LMD_ROWS) * LM_BATCH * (sizeof(float) + sizeof(int));
  const LmShape& sh = kLmShapes[shape < (int)(sizeof(kLmShapes) / sizeof(kLmShapes[0])) ? shape : 4];
  int per;
  const size_t cand = (size_t)lm_tiles(V, chunk, sh.G * 16, &per) * LM_BATCH * (sizeof(float) + sizeof(int));
  const size_t slices = sh.KS > 1 ? (size_t)sh.KS * LM_BATCH * V * sizeof(float) : 0;
  return max(cand, slices);
}

size_t lm_head_workspace_bytes(int V) {
  // The largest need over the launch shapes and every chunk size: per-workgroup candidates
  // (the register-streaming shapes tile each chunk, so one-row chunks give V tiles), KS slices
  // of partial logits for one 32-row batch pass, or the 64-row kernels' candidates of up to 64
  // batch rows per 64-row tile.
  size_t need = (size_t)V * LM_BATCH * (sizeof(float) + sizeof(int));
  for (const LmShape& sh : kLmShapes)
    if (sh.KS > 1) need = max(need, (size_t)sh.KS * LM_BATCH * V * sizeof(float));
  need = max(need, (size_t)((V + LMX_ROWS - 1) / LMX_ROWS) * 64 * (sizeof(float) + sizeof(int)));
  return need;
}

// The allocation-free entry point's workspace: a file-scope device array of
// kLmScratchBytes, one copy per GPU, held until the process ends. Host code never names the
// array as an address: its device address is looked up once per device, with that device
// current, and kept.
constexpr size_t kLmScratchBytes = size_t(1) << 20;
static __device__ __align__(256) unsigned char scratch[kLmScratchBytes];

hipError_t lm_head_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* a = addr[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    a = addr[dev].load(std::memory_order_relaxed);
    if (a == nullptr) {
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (a == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(a, std::memory_order_release);
    }
  }
  *ptr = a;
  *bytes = kLmScratchBytes;
  return hipSuccess;
}

hipError_t launch_lm_head(const LmHeadProblem& p, int shape, hipStream_t stream) {
  if (shape < 0) shape = default_shape(p);
  if (shape >= lm_head_shape_count()) return hipErrorInvalidValue;
  shape = effective_shape(p, shape);
  if (shape == kLmXresShape && !xres_ok(p)) shape = 4;  // ragged K: the register-streaming kernel
  const int pass = shape == kLmXresShape ? xres_pass_rows(p) : is_quad(shape) ? quad_pass_rows(p, shape) : LM_BATCH;
  for (int b0 = 0; b0 < p.B; b0 += pass) {
    if (p.w_fp8)
      launch_any<true>(p, shape, b0, stream);
    else
      launch_any<false>(p, shape, b0, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tpk
