// K1: bf16 NT GEMM on gfx950 matrix cores with a fused output stage.
//
// C[M,N] = A[M,K] * B[N,K]^T where A is the activation and B a weight shard as
// stored ([out_features, in_features], K contiguous) - the per-rank matmul of a
// column- or row-parallel linear ([deepspeed] SubParamLinearLayer.forward,
// [nanotron] "MLP Module").
//
// Structure: one workgroup owns a BM x BN output tile and walks K in steps of
// 64. Each step's A and B slabs go global -> registers -> LDS (two LDS stages:
// the loads for step k+1 are in flight while step k's MFMAs run). Each wave owns
// a WM x WN sub-tile made of 32x32 blocks, computed with
// v_mfma_f32_32x32x16_bf16 from 16-byte LDS reads. LDS rows are 128 bytes
// (64 bf16 of K); the 16-byte chunk index is XORed with the row's low three
// bits so that the eight rows one ds_read_b128 phase touches hit distinct banks.
// Optionally the A slab is RMS-normalised on its way into LDS.
// The output stage adds the bias, applies GELU, rounds once and stores bf16
// or f32 at the (possibly remapped) output column, or adds into f32.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int BK = 64;
constexpr int ROW_BYTES = BK * 2;

__device__ __forceinline__ int lds_off(int row, int kc) { return row * ROW_BYTES + ((kc ^ (row & 7)) << 4); }

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

template <int BM, int BN, int WAVES_M, int WAVES_N, bool NORM>
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
  const int m0 = (first_m + in % gsz) * BM, n0 = (in / gsz) * BN;

  const int M = p.M, N = p.N, K = p.K;
  const int kc = tid & 7;          // this thread's 16-byte chunk within a 64-wide K slab
  const int lrow = tid >> 3;       // first tile row this thread loads
  const uint16_t* a_base = p.A + (int64_t)(m0 + lrow) * p.lda + kc * 8;
  const uint16_t* b_base = p.B + (int64_t)(n0 + lrow) * p.ldb + kc * 8;
  const int64_t a_step = (int64_t)ROWS_PER_PASS * p.lda, b_step = (int64_t)ROWS_PER_PASS * p.ldb;

  float rr[NORM ? CA : 1];
  const bool has_t = NORM && p.col_t != nullptr;
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      int gm = m0 + lrow + i * ROWS_PER_PASS;
      rr[i] = gm < M ? p.row_r[gm] : 0.0f;
    }
  }

  u32x4_t ra[CA], rb[CB], rt;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
    const bool kok = k0 + kc * 8 < K;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      bool ok = kok && (m0 + lrow + i * ROWS_PER_PASS < M);
      ra[i] = ok ? *reinterpret_cast<const u32x4_t*>(a_base + i * a_step + k0) : zero;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      bool ok = kok && (n0 + lrow + i * ROWS_PER_PASS < N);
      rb[i] = ok ? *reinterpret_cast<const u32x4_t*>(b_base + i * b_step + k0) : zero;
    }
    if (has_t) rt = kok ? *reinterpret_cast<const u32x4_t*>(p.col_t + k0 + kc * 8) : zero;
  };
  auto lstore = [&](int buf) {
    unsigned char* sa = smem + buf * STAGE;
    unsigned char* sb = sa + BM * ROW_BYTES;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      u32x4_t v = ra[i];
      if constexpr (NORM) v = rms_apply(v, rr[i], rt, has_t);
      *reinterpret_cast<u32x4_t*>(sa + lds_off(lrow + i * ROWS_PER_PASS, kc)) = v;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i)
      *reinterpret_cast<u32x4_t*>(sb + lds_off(lrow + i * ROWS_PER_PASS, kc)) = rb[i];
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int a_row0 = wm * WM + (lane & 31), b_row0 = wn * WN + (lane & 31);
  const int khalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload((kt + 1) * BK);
    const unsigned char* sa = smem + (kt & 1) * STAGE;
    const unsigned char* sb = sa + BM * ROW_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t,
                                   *reinterpret_cast<const u32x4_t*>(sa + lds_off(a_row0 + i * 32, kk * 2 + khalf)));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8_t,
                                    *reinterpret_cast<const u32x4_t*>(sb + lds_off(b_row0 + j * 32, kk * 2 + khalf)));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // Output stage. In a 32x32 accumulator block, lane l holds column l % 32 and
  // rows 8 * (v / 4) + 4 * (l / 32) + v % 4 for its sixteen values v.
  const GemmEpilogue& ep = p.ep;
  int ocol[FN];
  float bias[FN];
  bool cok[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int c = n0 + wn * WN + j * 32 + (lane & 31);
    cok[j] = c < N;
    int d = 0;
    for (int s = 0; s < ep.n_seg; ++s)
      if (c < ep.seg_end[s]) {
        d = ep.seg_delta[s];
        break;
      }
    ocol[j] = c + d;
    bias[j] = (ep.bias != nullptr && cok[j]) ? bf16_to_f32(ep.bias[c]) : 0.0f;
  }
  const int rbase = m0 + wm * WM + (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = rbase + i * 32 + (v >> 2) * 8 + (v & 3);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (!cok[j]) continue;
        float val = acc[i][j][v] + bias[j];
        if (ep.act == TP_ACT_GELU_ERF) val = gelu_erf(val);
        const int64_t off = (int64_t)row * ep.ldc + ocol[j];
        if (ep.out_f32) {
          float* c = reinterpret_cast<float*>(ep.C) + off;
          if (ep.accumulate) val = *c + val;
          *c = val;
        } else {
          reinterpret_cast<uint16_t*>(ep.C)[off] = f32_to_bf16(val);
        }
      }
    }
  }
}

struct TileInfo {
  int bm, bn, threads;
};

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_tile(const GemmProblem& p, hipStream_t stream) {
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int nb = tiles_m * tiles_n;
  const int group_m = tiles_m < 8 ? tiles_m : 8;
  dim3 grid(nb), block(WAVES_M * WAVES_N * 64);
  if (p.row_r != nullptr)
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, true>), grid, block, 0, stream, p, tiles_m, tiles_n,
                       group_m);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, false>), grid, block, 0, stream, p, tiles_m,
                       tiles_n, group_m);
  return hipGetLastError();
}

}  // namespace

int gemm_pick_tile(int M, int N, int K) {
  (void)K;
  const long long t256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 512) return TILE_256x256;
  if (N % 224 == 0 && (long long)((M + 255) / 256) * (N / 224) >= 256) return TILE_256x224;
  const long long t256x128 = (long long)((M + 255) / 256) * ((N + 127) / 128);
  if (t256x128 >= 256) return TILE_256x128;
  const long long t128 = (long long)((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= 128) return TILE_128x128;
  if ((long long)((M + 127) / 128) * ((N + 63) / 64) >= 64) return TILE_128x64;
  return TILE_64x64;
}

hipError_t launch_gemm(const GemmProblem& p, int tile, hipStream_t stream) {
  if (tile == TILE_AUTO) tile = gemm_pick_tile(p.M, p.N, p.K);
  switch (tile) {
    case TILE_256x256: return launch_tile<256, 256, 2, 2>(p, stream);
    case TILE_256x128: return launch_tile<256, 128, 2, 2>(p, stream);
    case TILE_128x128: return launch_tile<128, 128, 2, 2>(p, stream);
    case TILE_128x256: return launch_tile<128, 256, 2, 2>(p, stream);
    case TILE_256x224: return launch_tile<256, 224, 4, 1>(p, stream);
    case TILE_128x64: return launch_tile<128, 64, 2, 2>(p, stream);
    case TILE_64x64: return launch_tile<64, 64, 2, 2>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpk
