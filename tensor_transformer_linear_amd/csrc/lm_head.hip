// K3 + K4: vocab-sharded decode LM head with the shard's argmax.
//
// [tt] LMHead1D: the shard's projection is split into chunks of at most C rows,
// one linear per chunk, outputs concatenated along the vocab; each device ends
// with complete logits for its own vocab rows. [palm] unembed_manual: float32
// logits. Decode has a few batch rows, so the work is a stream of the weight
// shard from HBM: every weight byte is read once.
//
// Two streaming kernels compute the logits; both give a workgroup a tile of weight
// rows and finish with that workgroup's (max, lowest index) candidate per batch
// row, which a second kernel launched right after reduces
// (a kernel boundary instead of per-workgroup device-scope fences, which on gfx950
// write back and invalidate the whole L2).
//
// * Register streaming (shapes 0-7): a workgroup owns 16 G weight rows and its
//   waves split K; each wave loads the 16-byte pieces of its K steps straight into
//   MFMA operand registers, P steps per batch, and the waves' partials are summed
//   through LDS in wave order. Works for any K % 8 == 0.
// * LDS ring (shapes 8, 9; the default): a workgroup owns 64 rows over the whole
//   K; weight, x and block-scale pieces go global -> LDS with global_load_lds into
//   a ring of stages that fills the CU's LDS, so the prefetch depth costs no
//   registers. Needs K % 32 (64-byte stages) or K % 64 (128-byte stages) for bf16.
//   Its tiles are whole 64-row blocks of the shard: the chunks only group the
//   concatenated output, which is the same rows in the same order, so a chunk
//   boundary inside a block changes nothing.
//
// The register-streaming shapes tile each chunk on its own.
//
// Both multiply with v_mfma_f32_16x16x32_bf16, x as the row operand and the
// weight as the column operand, so every lane's accumulators belong to one weight
// row. E4M3 weights are widened to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8
// with scale 1: exact, every E4M3 value is a bf16 value) and each 128-wide K
// block's partial is multiplied by the row's block scale before it joins the
// float32 accumulator.
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
constexpr int kLmDefaultShape = 9;  // LDS ring, 128-byte stages (falls back to 4 for a ragged bf16 K)

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
    part_v[(size_t)tile * LM_BATCH + tid] = red_v[0][tid];
    part_i[(size_t)tile * LM_BATCH + tid] = red_i[0][tid];
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
    part_v[(size_t)tile * LM_BATCH + tid] = val;
    part_i[(size_t)tile * LM_BATCH + tid] = idx;
  }
}

// Reduces every workgroup's (max, lowest index) candidate of one batch row (one workgroup
// per row): each thread loads its candidates with independent loads (one memory round trip),
// then wave and workgroup reductions. Running as its own kernel after the logits kernel makes
// the candidates visible across XCDs without device-scope fences in the streaming kernel.
__global__ __launch_bounds__(LM_FIN_THREADS) void lm_head_argmax_kernel(LmHeadProblem p, int n_tiles, int b0) {
  __shared__ float sv[LM_FIN_THREADS / 64];
  __shared__ int si[LM_FIN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const float* part_v = reinterpret_cast<const float*>(p.workspace);
  const int* part_i = reinterpret_cast<const int*>(part_v + (size_t)n_tiles * LM_BATCH);
  float v = -INFINITY;
  int idx = 0x7fffffff;
  for (int t = tid; t < n_tiles; t += LM_FIN_THREADS) {
    const float tv = part_v[(size_t)t * LM_BATCH + b];
    const int ti = part_i[(size_t)t * LM_BATCH + b];
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
                       n_tiles, b0);
}

// Direct-to-LDS launch shapes (stage row bytes RB, ring depth): the ring fills 160 KB of LDS.
template <bool FP8, int RB, int STAGES>
void launch_dma(const LmHeadProblem& p, int b0, hipStream_t stream) {
  static_assert(STAGES * LmdStage<FP8, RB>::BYTES <= 160 * 1024, "ring exceeds LDS");
  const int n_tiles = (p.V + LMD_ROWS - 1) / LMD_ROWS;  // whole 64-row blocks of the shard
  hipLaunchKernelGGL((lm_head_dma_kernel<FP8, RB, STAGES>), dim3(n_tiles), dim3(LMD_THREADS), 0, stream, p, n_tiles,
                     b0);
  hipLaunchKernelGGL(lm_head_argmax_kernel, dim3(min(LM_BATCH, p.B - b0)), dim3(LM_FIN_THREADS), 0, stream, p, n_tiles,
                     b0);
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

int lm_head_shape_count() { return (int)(sizeof(kLmShapes) / sizeof(kLmShapes[0])) + 2; }

size_t lm_head_workspace_bytes(int B, int V, int chunk) {
  (void)B;
  // the largest need over the launch shapes: per-workgroup candidates, or KS slices of
  // partial logits for one 32-row batch pass
  size_t need = 0;
  int per;
  for (const LmShape& sh : kLmShapes) {
    const size_t cand = (size_t)lm_tiles(V, chunk, sh.G * 16, &per) * LM_BATCH * (sizeof(float) + sizeof(int));
    const size_t slices = sh.KS > 1 ? (size_t)sh.KS * LM_BATCH * V * sizeof(float) : 0;
    need = max(need, max(cand, slices));
  }
  return need;
}

hipError_t launch_lm_head(const LmHeadProblem& p, int shape, hipStream_t stream) {
  if (shape < 0) shape = kLmDefaultShape;
  if (shape >= lm_head_shape_count()) return hipErrorInvalidValue;
  for (int b0 = 0; b0 < p.B; b0 += LM_BATCH) {
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
