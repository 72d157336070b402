// K3 + K4: vocab-sharded decode LM head with the shard's argmax, in one launch.
//
// [tt] LMHead1D: the shard's projection is split into chunks of at most C rows,
// one linear per chunk, outputs concatenated along the vocab; each device ends
// with complete logits for its own vocab rows. [palm] unembed_manual: float32
// logits. Decode has a few batch rows, so the work is a stream of the weight
// shard from HBM: every weight byte is read once.
//
// A workgroup owns ROWS weight rows that lie inside one chunk, over the whole K.
// K is walked in slabs of 256: the weight slab (bf16, or E4M3 widened to bf16 on
// the way in - E4M3 values are exactly bf16 values) and the matching x slab are
// staged in LDS with 16-byte coalesced loads, the next two slabs' loads being in
// flight during the current slab's MFMAs. Each of the eight waves takes 32 of
// the slab's K values for both 32-row blocks (x is the 32-row MFMA operand, the
// weight rows the 32-column operand). With E4M3 weights each wave's 32 K values
// lie inside one 128-wide scale block, so the wave multiplies its block partial
// by the row's scale before adding it to its float32 accumulator. The eight
// waves' partials are summed through LDS in a fixed order, written as logits,
// and reduced to a (max, lowest index) pair per batch row; the last workgroup
// to finish (a device-scope ticket) reduces the pairs of all workgroups and
// resets the ticket.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int LM_ROWS = 64;        // weight rows per workgroup (two 32-row MFMA blocks)
constexpr int LM_BATCH = 32;       // batch rows handled per launch pass (the MFMA's 32-row operand)
constexpr int LM_KS = 256;         // K per slab
constexpr int LM_THREADS = 512;    // eight waves
constexpr int LM_WAVES = LM_THREADS / 64;
constexpr int LM_KW = LM_KS / LM_WAVES;  // K values per wave per slab (32)
constexpr int LM_ROWB = LM_KS * 2;       // LDS bytes per staged row (bf16)
constexpr int LM_WCH = LM_ROWS * LM_KS / 8 / LM_THREADS;    // weight 16-byte chunks per thread (bf16)
constexpr int LM_XCH = LM_BATCH * LM_KS / 8 / LM_THREADS;   // x chunks per thread
constexpr int LM_W8CH = LM_ROWS * LM_KS / 16 / LM_THREADS;  // weight 16-byte chunks per thread (E4M3)
constexpr size_t LM_TICKET_BYTES = 256;

static_assert(LM_WCH == 4 && LM_XCH == 2 && LM_W8CH == 2, "slab partition");

// LDS offset of 16-byte chunk c (0..31) of staged row `row`; the XOR spreads the
// rows read by one ds_read_b128 phase over all banks.
__device__ __forceinline__ int lm_off(int row, int c) { return row * LM_ROWB + ((c ^ (row & 31)) << 4); }

// Two E4M3 codes (bytes HI ? 2,3 : 0,1 of w) -> two bf16, exactly (scale 1).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

template <bool FP8>
__global__ __launch_bounds__(LM_THREADS) void lm_head_kernel(LmHeadProblem p, int tiles_per_chunk, int n_tiles,
                                                             int b0) {
  // Two slab buffers ([64 weight rows][256] + [32 x rows][256] bf16 each, 48 KB); the
  // cross-wave reduction at the end reuses the same memory (64 KB).
  constexpr int SLAB = (LM_ROWS + LM_BATCH) * LM_ROWB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * SLAB];
  __shared__ float red_v[LM_THREADS / 64][LM_BATCH];
  __shared__ int red_i[LM_THREADS / 64][LM_BATCH];
  __shared__ int is_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, V = p.V, C = p.chunk;
  const int nbatch = min(LM_BATCH, p.B - b0);

  // This workgroup's rows: tile t of chunk c, clipped to the chunk's end.
  const int tile = blockIdx.x;
  const int chunk = tile / tiles_per_chunk, tin = tile - chunk * tiles_per_chunk;
  const int row0 = chunk * C + tin * LM_ROWS;
  const int chunk_end = min(V, (chunk + 1) * C);
  const int nrows = max(0, min(LM_ROWS, chunk_end - row0));

  // Global-load assignment.
  // bf16 weight: chunk q = tid + i * 512 -> row q / 32, 16-byte piece q % 32.
  // E4M3 weight: chunk q -> row q / 16, 16-byte piece q % 16 (16 K values).
  // x: chunk q -> batch row q / 32, piece q % 32.
  constexpr int NW = FP8 ? LM_W8CH : LM_WCH;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // Loads of one slab into a register set (weight pieces rw, x pieces rx). Out-of-range
  // pieces load from a valid address; lstore zeroes them, so nothing between the loads
  // and lstore waits on them.
  auto gload = [&](int k0, u32x4_t(&rw)[NW], u32x4_t(&rx)[LM_XCH]) {
    if constexpr (FP8) {
      const uint8_t* w8 = reinterpret_cast<const uint8_t*>(p.w);
#pragma unroll
      for (int i = 0; i < LM_W8CH; ++i) {
        int q = tid + i * LM_THREADS, r = q >> 4, k = k0 + (q & 15) * 16;
        bool ok = r < nrows && k < K;
        rw[i] = *reinterpret_cast<const u32x4_t*>(w8 + (int64_t)(row0 + (ok ? r : 0)) * K + (ok ? k : 0));
      }
    } else {
      const uint16_t* w16 = reinterpret_cast<const uint16_t*>(p.w);
#pragma unroll
      for (int i = 0; i < LM_WCH; ++i) {
        int q = tid + i * LM_THREADS, r = q >> 5, k = k0 + (q & 31) * 8;
        bool ok = r < nrows && k < K;
        rw[i] = *reinterpret_cast<const u32x4_t*>(w16 + (int64_t)(row0 + (ok ? r : 0)) * K + (ok ? k : 0));
      }
    }
#pragma unroll
    for (int i = 0; i < LM_XCH; ++i) {
      int q = tid + i * LM_THREADS, b = q >> 5, k = k0 + (q & 31) * 8;
      bool ok = b < nbatch && k < K;
      rx[i] = *reinterpret_cast<const u32x4_t*>(p.x + (int64_t)(b0 + (ok ? b : 0)) * K + (ok ? k : 0));
    }
  };
  // A register set into slab buffer `buf` (E4M3 widened to bf16 on the way).
  auto lstore = [&](int buf, int k0, u32x4_t(&rw)[NW], u32x4_t(&rx)[LM_XCH]) {
    unsigned char* sw = smem + buf * SLAB;
    unsigned char* sx = sw + LM_ROWS * LM_ROWB;
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < LM_W8CH; ++i) {
        int q = tid + i * LM_THREADS, r = q >> 4, c = (q & 15) * 2;
        const u32x4_t w = (r < nrows && k0 + (q & 15) * 16 < K) ? rw[i] : zero;
        u32x4_t lo, hi;
        lo[0] = e4m3x2_to_bf16x2<false>(w[0]);
        lo[1] = e4m3x2_to_bf16x2<true>(w[0]);
        lo[2] = e4m3x2_to_bf16x2<false>(w[1]);
        lo[3] = e4m3x2_to_bf16x2<true>(w[1]);
        hi[0] = e4m3x2_to_bf16x2<false>(w[2]);
        hi[1] = e4m3x2_to_bf16x2<true>(w[2]);
        hi[2] = e4m3x2_to_bf16x2<false>(w[3]);
        hi[3] = e4m3x2_to_bf16x2<true>(w[3]);
        *reinterpret_cast<u32x4_t*>(sw + lm_off(r, c)) = lo;
        *reinterpret_cast<u32x4_t*>(sw + lm_off(r, c + 1)) = hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < LM_WCH; ++i) {
        int q = tid + i * LM_THREADS, r = q >> 5;
        *reinterpret_cast<u32x4_t*>(sw + lm_off(r, q & 31)) = (r < nrows && k0 + (q & 31) * 8 < K) ? rw[i] : zero;
      }
    }
#pragma unroll
    for (int i = 0; i < LM_XCH; ++i) {
      int q = tid + i * LM_THREADS, b = q >> 5;
      *reinterpret_cast<u32x4_t*>(sx + lm_off(b, q & 31)) = (b < nbatch && k0 + (q & 31) * 8 < K) ? rx[i] : zero;
    }
  };

  f32x16_t acc[2];
  static_for<2>([&](auto j) { static_for<16>([&](auto v) { acc[j][decltype(v)::value] = 0.0f; }); });

  const int nslab = (K + LM_KS - 1) / LM_KS;
  const int nblk = K / 128;
  // This wave's 32 K values of slab s: two k16 steps. Lane l supplies batch row (or weight
  // row) l % 32 and eight K values starting at 8 * (l / 32).
  auto compute = [&](int buf, int s) {
    const unsigned char* sw = smem + buf * SLAB;
    const unsigned char* sx = sw + LM_ROWS * LM_ROWB;
    f32x16_t part[2];
    if constexpr (FP8) static_for<2>([&](auto j) { static_for<16>([&](auto v) { part[j][decltype(v)::value] = 0.0f; }); });
    static_for<LM_KW / 16>([&](auto kk) {
      const int c = (wave * LM_KW + kk * 16) / 8 + (lane >> 5);
      bf16x8_t xa = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(sx + lm_off(lane & 31, c)));
      static_for<2>([&](auto j) {
        bf16x8_t wb =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(sw + lm_off(j * 32 + (lane & 31), c)));
        if constexpr (FP8)
          part[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, wb, part[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, wb, acc[j], 0, 0, 0);
      });
    });
    if constexpr (FP8) {
      const int blk = (s * LM_KS + wave * LM_KW) / 128;
      static_for<2>([&](auto j) {
        const int r = j * 32 + (lane & 31);
        const float sc = (r < nrows && blk < nblk) ? p.wscale[(int64_t)(row0 + r) * nblk + blk] : 0.0f;
        static_for<16>([&](auto v) {
          constexpr int vv = v;
          acc[j][vv] = fmaf(part[j][vv], sc, acc[j][vv]);
        });
      });
    }
  };

  // Pipeline: two register sets carry slabs s + 1 and s + 2 from HBM while slab s is in
  // LDS and being multiplied; one barrier per slab (the barrier of slab s also proves that
  // every wave finished slab s - 2, whose buffer slab s overwrites).
  // Loads are unconditional (slab index clamped to the last slab; the extra loads are
  // in bounds and never stored) so the compiler keeps both sets in flight.
  u32x4_t rw0[NW], rx0[LM_XCH], rw1[NW], rx1[LM_XCH];
  auto slab_k = [&](int s) { return (s < nslab ? s : nslab - 1) * LM_KS; };
  gload(slab_k(0), rw0, rx0);
  gload(slab_k(1), rw1, rx1);
  for (int s = 0; s < nslab; s += 2) {
    lstore(0, s * LM_KS, rw0, rx0);
    __syncthreads();
    gload(slab_k(s + 2), rw0, rx0);
    compute(0, s);
    if (s + 1 >= nslab) break;
    lstore(1, (s + 1) * LM_KS, rw1, rx1);
    __syncthreads();
    gload(slab_k(s + 3), rw1, rx1);
    compute(1, s + 1);
  }
  __syncthreads();

  // Sum the eight waves' partials in wave order. Accumulator layout: lane l holds
  // weight row (column of the 32x32 block) l % 32 and batch rows 8(v/4) + 4(l/32) + v%4.
  float* red = reinterpret_cast<float*>(smem);  // [wave][batch 32][row 64]
  static_for<2>([&](auto j) {
    static_for<16>([&](auto v) {
      constexpr int vv = v;
      const int b = (vv >> 2) * 8 + (lane >> 5) * 4 + (vv & 3);
      red[(wave * LM_BATCH + b) * LM_ROWS + j * 32 + (lane & 31)] = acc[j][vv];
    });
  });
  __syncthreads();
  // Thread -> (batch b, rows r, r + 32 ... ): 512 threads cover 32 x 64 outputs, 4 each.
  {
    const int r = tid & 63, bq = tid >> 6;  // batch rows bq, bq + 8, bq + 16, bq + 24
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int b = bq + 8 * t;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < LM_WAVES; ++w) sum += red[(w * LM_BATCH + b) * LM_ROWS + r];
      if (r < nrows && b < nbatch) p.logits[(int64_t)(b0 + b) * V + row0 + r] = sum;
      float v = (r < nrows && !(sum != sum)) ? sum : -INFINITY;
      int idx = row0 + r;
      // wave-wide (max, lowest index) over the 64 rows of batch row b
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
        red_v[wave][t] = v;
        red_i[wave][t] = idx;
      }
    }
  }
  __syncthreads();

  // Publish this workgroup's candidates: wave w, slot t holds batch row w + 8 t.
  float* part_v = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(p.workspace) + LM_TICKET_BYTES);
  int* part_i = reinterpret_cast<int*>(part_v + (size_t)n_tiles * LM_BATCH);
  if (tid < LM_BATCH) {
    const int w = tid & 7, t = tid >> 3;  // batch row tid = w + 8 t
    part_v[(size_t)tile * LM_BATCH + tid] = red_v[w][t];
    part_i[(size_t)tile * LM_BATCH + tid] = red_i[w][t];
  }
  __threadfence();
  __syncthreads();
  unsigned int* ticket = reinterpret_cast<unsigned int*>(p.workspace);
  if (tid == 0) {
    unsigned int prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == (unsigned int)(n_tiles - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // Last workgroup: reduce every workgroup's candidates. Wave w handles batch rows w, w + 8, ...
  for (int b = wave; b < nbatch; b += LM_WAVES) {
    float v = -INFINITY;
    int idx = 0x7fffffff;
    for (int t = lane; t < n_tiles; t += 64) {
      float tv = __hip_atomic_load(&part_v[(size_t)t * LM_BATCH + b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int ti = __hip_atomic_load(&part_i[(size_t)t * LM_BATCH + b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      if (idx == 0x7fffffff) idx = 0;  // every logit NaN: index 0, as the lowest index of -inf
      p.argmax[b0 + b] = idx;
      if (p.maxval != nullptr) p.maxval[b0 + b] = v;
    }
  }
  if (tid == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

int lm_tiles(int V, int chunk, int* tiles_per_chunk) {
  const int n_chunks = (V + chunk - 1) / chunk;
  const int per = (min(chunk, V) + LM_ROWS - 1) / LM_ROWS;
  *tiles_per_chunk = per;
  const int last_rows = V - (n_chunks - 1) * chunk;
  return (n_chunks - 1) * per + (last_rows + LM_ROWS - 1) / LM_ROWS;
}

}  // namespace

size_t lm_head_workspace_bytes(int B, int V, int chunk) {
  (void)B;
  int per;
  const int n_tiles = lm_tiles(V, chunk, &per);
  return LM_TICKET_BYTES + (size_t)n_tiles * LM_BATCH * (sizeof(float) + sizeof(int));
}

hipError_t launch_lm_head(const LmHeadProblem& p, hipStream_t stream) {
  int per;
  const int n_tiles = lm_tiles(p.V, p.chunk, &per);
  for (int b0 = 0; b0 < p.B; b0 += LM_BATCH) {
    if (p.w_fp8)
      hipLaunchKernelGGL(lm_head_kernel<true>, dim3(n_tiles), dim3(LM_THREADS), 0, stream, p, per, n_tiles, b0);
    else
      hipLaunchKernelGGL(lm_head_kernel<false>, dim3(n_tiles), dim3(LM_THREADS), 0, stream, p, per, n_tiles, b0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tpk
