// K3 + K4: vocab-sharded decode LM head with the shard's argmax, in one launch.
//
// [tt] LMHead1D: the shard's projection is split into chunks of at most C rows,
// one linear per chunk, outputs concatenated along the vocab; each device ends
// with complete logits for its own vocab rows. [palm] unembed_manual: float32
// logits. Decode has a few batch rows, so the work is a stream of the weight
// shard from HBM: every weight byte is read once.
//
// A workgroup owns 16 G weight rows that lie inside one chunk, over the whole K;
// its waves split K. Each wave streams its K range straight from global
// memory into MFMA operand registers (no LDS staging, no barriers in the loop):
// for every 32-wide K step it loads the 16-byte pieces of the G 16-row weight
// groups and of the two 16-row x groups and issues v_mfma_f32_16x16x32_bf16 with
// x as the row operand and the weight as the column operand, so every lane's
// accumulators belong to one weight row. Steps go in batches of P, each issued
// whole before it is multiplied. E4M3 weights are widened to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact, every E4M3 value is a bf16
// value) and each 128-wide K block's partial is multiplied by the row's block
// scale before it joins the float32 accumulator. The waves' partials are
// summed through LDS in wave order (deterministic), written as logits, and
// reduced to a (max, lowest index) pair per batch row; a second kernel
// launched right after reduces the pairs of all workgroups (a kernel boundary
// instead of per-workgroup device-scope fences, which on gfx950 write back and
// invalidate the whole L2).
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int LM_BATCH = 32;  // batch rows per launch pass (two 16-row MFMA groups)
constexpr int LM_FIN_THREADS = 256;

// Launch shapes: G 16-row weight groups per workgroup, W waves splitting K, P 32-wide K steps
// per batch of loads (a multiple of four: whole 128-wide E4M3 blocks).
struct LmShape {
  int G, W, P;
};
constexpr LmShape kLmShapes[] = {{4, 8, 8}, {2, 8, 8}, {4, 4, 8}, {2, 4, 8}, {4, 8, 4}, {1, 8, 8}};
constexpr int kLmDefaultShape = 4;

// Two E4M3 codes (bytes HI ? 2,3 : 0,1 of w) -> two bf16, exactly (scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

template <bool FP8, int G, int LM_WAVES, int LM_P>
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

  // This workgroup's rows: tile t of chunk c, clipped to the chunk's end.
  const int tile = blockIdx.x;
  const int chunk = tile / tiles_per_chunk, tin = tile - chunk * tiles_per_chunk;
  const int row0 = chunk * C + tin * LM_ROWS;
  const int chunk_end = min(V, (chunk + 1) * C);
  const int nrows = max(0, min(LM_ROWS, chunk_end - row0));

  // This wave's K steps [s_begin, s_end) of the ceil(K / 32) steps, in whole 128-wide
  // blocks (four steps), so that an E4M3 scale block never straddles two waves.
  const int nsteps = (K + 31) / 32;
  const int per_wave = ((nsteps + LM_WAVES - 1) / LM_WAVES + 3) / 4 * 4;
  const int s_begin = min(nsteps, wave * per_wave), s_end = min(nsteps, s_begin + per_wave);
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
  constexpr int BSTEP = LM_THREADS / LM_ROWS;  // batch rows handled side by side
  constexpr int BITER = LM_BATCH / BSTEP;
  static_assert(LM_ROWS <= 64 && BITER * BSTEP == LM_BATCH, "reduction layout");
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
  hipLaunchKernelGGL((lm_head_kernel<FP8, sh.G, sh.W, sh.P>), dim3(n_tiles), dim3(sh.W * 64), 0, stream, p, per,
                     n_tiles, b0);
  hipLaunchKernelGGL(lm_head_argmax_kernel, dim3(min(LM_BATCH, p.B - b0)), dim3(LM_FIN_THREADS), 0, stream, p,
                     n_tiles, b0);
}

template <bool FP8>
void launch_any(const LmHeadProblem& p, int shape, int b0, hipStream_t stream) {
  switch (shape) {
    case 1: launch_shape<FP8, 1>(p, b0, stream); break;
    case 2: launch_shape<FP8, 2>(p, b0, stream); break;
    case 3: launch_shape<FP8, 3>(p, b0, stream); break;
    case 4: launch_shape<FP8, 4>(p, b0, stream); break;
    case 5: launch_shape<FP8, 5>(p, b0, stream); break;
    default: launch_shape<FP8, 0>(p, b0, stream); break;
  }
}

}  // namespace

int lm_head_shape_count() { return (int)(sizeof(kLmShapes) / sizeof(kLmShapes[0])); }

size_t lm_head_workspace_bytes(int B, int V, int chunk) {
  (void)B;
  // sized for the launch shape with the most workgroups (16-row groups: the smallest tiles)
  int per, n_tiles = 0;
  for (const LmShape& sh : kLmShapes) n_tiles = max(n_tiles, lm_tiles(V, chunk, sh.G * 16, &per));
  return (size_t)n_tiles * LM_BATCH * (sizeof(float) + sizeof(int));
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
