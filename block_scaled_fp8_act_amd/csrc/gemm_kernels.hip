// Block-scaled FP8 GEMM  y = x * W^T  (bf16 out) and its grouped
// (mixture-of-experts) variant, for gfx950.
//
// The FP8 linear layer of the "Fine-grained FP8" page of the transformers
// docs ("DeepGEMM fast path": (128,128) weight blocks with dynamic
// per-token-group activation scales).  Its value is that of
// dequantize-then-matmul ("BFL (fp8r / nvfp4)" page of the diffusers docs,
// "Kernels"), computed here as
//     y[m,n] = sum_kb x_s[m,kb] * w_s[n/128,kb] * P_kb[m,n],
//     P_kb[m,n] = sum_{k in block kb} dec(x_q[m,k]) * dec(w_q[n,k]),
// where each P_kb is one v_mfma_f32_16x16x128_f8f6f4 (K = 128 = one scale
// block, fp32 result) and the scale pair is applied with one fp32 FMA per
// output per K block ("promotion" into the fp32 accumulator).
//
// Workgroup tile 128x128 (4 waves of 64x64), K step 128, double-buffered
// LDS staging of the fp8 A and B tiles with a 16-byte-chunk XOR swizzle
// (chunk c of row r is stored at c ^ (r & 7)) so that the 16 lanes reading
// the same chunk of 16 consecutive rows spread over the LDS banks.
#include "fp8blk_device.h"
#include "fp8blk_launch.h"

namespace fp8blk {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kGemmThreads = 256;

struct GemmSmem {
  uint8_t a[2][BM * BK];
  uint8_t b[2][BN * BK];
  float as[2][BM];
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ v8i frag_from(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// One BM x BN output tile.
//   A  : x_q at row m0 (row stride K bytes); rows_a valid rows (<= BM)
//   As : x_scale at row m0 (row stride KB floats)
//   B  : w_q at row n0 (row stride K bytes); rows_b valid rows (<= BN)
//   Bs : w_scale row n0/128 (KB floats)
//   Y  : y at (m0, n0), row stride ldy elements
__device__ __forceinline__ void gemm_tile(const uint8_t *__restrict__ A,
                                          const float *__restrict__ As, int rows_a,
                                          const uint8_t *__restrict__ B,
                                          const float *__restrict__ Bs, int rows_b, int64_t K,
                                          uint16_t *__restrict__ Y, int64_t ldy, GemmSmem &sm) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int KB = (int)(K / BK);

  uint4 ga[4], gb[4];
  float gs = 0.0f;
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = t + kGemmThreads * i;
      const int row = j >> 3, ch = j & 7;
      const int64_t off = (int64_t)row * K + (int64_t)kb * BK + ch * 16;
      ga[i] = row < rows_a ? *reinterpret_cast<const uint4 *>(A + off) : make_uint4(0, 0, 0, 0);
      gb[i] = row < rows_b ? *reinterpret_cast<const uint4 *>(B + off) : make_uint4(0, 0, 0, 0);
    }
    gs = (t < rows_a) ? As[(int64_t)t * KB + kb] : 0.0f;
  };
  auto swrite = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = t + kGemmThreads * i;
      const int row = j >> 3, ch = j & 7;
      *reinterpret_cast<uint4 *>(sm.a[st] + swz(row, ch)) = ga[i];
      *reinterpret_cast<uint4 *>(sm.b[st] + swz(row, ch)) = gb[i];
    }
    if (t < BM) sm.as[st][t] = gs;
  };

  v4f acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  gload(0);
  swrite(0);
  __syncthreads();

  const int c0 = (lane >> 4) * 2;
  for (int kb = 0; kb < KB; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < KB) gload(kb + 1);
    const float wsc = Bs[kb];
    v8i af[4], bfr[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = wm * 64 + mi * 16 + (lane & 15);
      af[mi] = frag_from(*reinterpret_cast<const uint4 *>(sm.a[st] + swz(row, c0)),
                         *reinterpret_cast<const uint4 *>(sm.a[st] + swz(row, c0 + 1)));
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int row = wn * 64 + ni * 16 + (lane & 15);
      bfr[ni] = frag_from(*reinterpret_cast<const uint4 *>(sm.b[st] + swz(row, c0)),
                          *reinterpret_cast<const uint4 *>(sm.b[st] + swz(row, c0 + 1)));
    }
    v4f sc[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const float4 s4 =
          *reinterpret_cast<const float4 *>(&sm.as[st][wm * 64 + mi * 16 + 4 * (lane >> 4)]);
      sc[mi] = v4f{s4.x * wsc, s4.y * wsc, s4.z * wsc, s4.w * wsc};
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[mi], bfr[ni], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] = fmaf(p[r], sc[mi][r], acc[mi][ni][r]);
      }
    if (kb + 1 < KB) swrite(st ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds rows 4*(lane/16)+r of each 16x16 tile, column lane%16.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = wn * 64 + ni * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + mi * 16 + 4 * (lane >> 4) + r;
        if (row < rows_a && col < rows_b)
          Y[(int64_t)row * ldy + col] = (uint16_t)bf16_rne(acc[mi][ni][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// Large-tile configuration: 256x256 output tile per workgroup of 8 waves
// (2 along M x 4 along N, 128x64 per wave), K step 128.  At the dense fp8
// rate a 256x256 tile needs 32 bytes per clock per CU from L2 (a 128x128
// tile would need 64), and each wave's 128x64 sub-tile halves the LDS read
// traffic per MFMA compared with 64x64.  Operand tiles go from global memory
// straight into LDS (global_load_lds_dwordx4, no VGPR staging), two stages.
// Per stage: A 256x128 B, B 256x128 B (16-byte chunks XOR-swizzled by row),
// and the 256 activation scales of the K block.
namespace big {
constexpr int TM = 256, TN = 256, TK = 128;
constexpr int kThreads = 512;
constexpr int kStageA = TM * TK;            // bytes
constexpr int kStageB = TN * TK;
struct Smem {
  uint8_t a[2][kStageA];
  uint8_t b[2][kStageB];
  float as[2][TM];
};
}  // namespace big

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void lds_dma16(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 4, 0, 0);
}

// One 256x256 output tile (see above).  Rows past rows_a / rows_b are read
// from the last valid row (never out of bounds); their outputs are not stored.
__device__ __forceinline__ void gemm_tile_256(const uint8_t *__restrict__ A,
                                              const float *__restrict__ As, int rows_a,
                                              const uint8_t *__restrict__ B,
                                              const float *__restrict__ Bs, int rows_b,
                                              int64_t K, uint16_t *__restrict__ Y, int64_t ldy,
                                              big::Smem &sm) {
  using namespace big;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int KB = (int)(K / TK);

  // Global source rows/chunks for this lane's four A and four B DMA loads:
  // load i of wave w fills LDS rows [8r, 8r+8), r = 4w + i; lane l writes
  // bytes [16l, 16l+16) of that 1 KB run = row 8r + l/8, physical chunk l%8,
  // which holds logical chunk (l%8) ^ (row%8).
  const int lchunk = (lane & 7) ^ ((lane >> 3) & 7);
  const uint8_t *pa[4];
  const uint8_t *pb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    pa[i] = A + (int64_t)min(row, rows_a - 1) * K + lchunk * 16;
    pb[i] = B + (int64_t)min(row, rows_b - 1) * K + lchunk * 16;
  }
  // Activation scales of rows 64w + l (waves 0..3).
  const float *ps = As + (int64_t)min(64 * (wave & 3) + lane, rows_a - 1) * KB;
  // Weight-block scale row of this wave's 64 columns (clamped to the last
  // existing block row of a short tile; such columns are not stored).
  const float *pws = Bs + (int64_t)min((wn * 64) / 128, (rows_b - 1) / 128) * KB;

  auto issue = [&](int kb, int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds_dma16(pa[i] + (int64_t)kb * TK, sm.a[st] + (4 * wave + i) * 1024);
      lds_dma16(pb[i] + (int64_t)kb * TK, sm.b[st] + (4 * wave + i) * 1024);
    }
    if (wave < 4) lds_dma4(ps + kb, &sm.as[st][64 * wave]);
  };

  v4f acc[8][4];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int c0 = (lane >> 4) * 2;
  const int r16 = lane & 15;
  for (int kb = 0; kb < KB; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < KB) issue(kb + 1, st ^ 1);
    const float wsc = pws[kb];
    const uint8_t *sa = sm.a[st];
    const uint8_t *sb = sm.b[st];
    v8i bfr[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int row = wn * 64 + ni * 16 + r16;
      bfr[ni] = frag_from(*reinterpret_cast<const uint4 *>(sb + swz(row, c0)),
                          *reinterpret_cast<const uint4 *>(sb + swz(row, c0 + 1)));
    }
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      const int row = wm * 128 + mi * 16 + r16;
      const v8i af = frag_from(*reinterpret_cast<const uint4 *>(sa + swz(row, c0)),
                               *reinterpret_cast<const uint4 *>(sa + swz(row, c0 + 1)));
      const float4 s4 =
          *reinterpret_cast<const float4 *>(&sm.as[st][wm * 128 + mi * 16 + 4 * (lane >> 4)]);
      const float sc[4] = {s4.x * wsc, s4.y * wsc, s4.z * wsc, s4.w * wsc};
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af, bfr[ni], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] = fmaf(p[r], sc[r], acc[mi][ni][r]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = wn * 64 + ni * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 128 + mi * 16 + 4 * (lane >> 4) + r;
        if (row < rows_a && col < rows_b)
          Y[(int64_t)row * ldy + col] = (uint16_t)bf16_rne(acc[mi][ni][r]);
      }
    }
}

// Map a linear workgroup id to (tile_m, tile_n).  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2); consecutive logical
// tiles are made to land on one XCD, and logical tiles are ordered in
// groups of 8 tile rows so that neighbours share A rows and B columns.
__device__ __forceinline__ void tile_coords(int bid, int total, int tiles_m, int tiles_n,
                                            int &tm, int &tn) {
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = bid - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

__global__ __launch_bounds__(kGemmThreads) void block_gemm_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xs, const uint8_t *__restrict__ wq,
    const float *__restrict__ ws, int64_t M, int64_t N, int64_t K, uint16_t *__restrict__ y,
    int tiles_m, int tiles_n) {
  __shared__ GemmSmem sm;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t KB = K / BK;
  gemm_tile(xq + m0 * K, xs + m0 * KB, (int)min<int64_t>(BM, M - m0), wq + n0 * K,
            ws + (n0 / BN) * KB, (int)min<int64_t>(BN, N - n0), K, y + m0 * N + n0, N, sm);
}

__global__ __launch_bounds__(big::kThreads) void block_gemm_256_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xs, const uint8_t *__restrict__ wq,
    const float *__restrict__ ws, int64_t M, int64_t N, int64_t K, uint16_t *__restrict__ y,
    int tiles_m, int tiles_n) {
  __shared__ big::Smem sm;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * big::TM, n0 = (int64_t)tn * big::TN;
  const int64_t KB = K / big::TK;
  gemm_tile_256(xq + m0 * K, xs + m0 * KB, (int)min<int64_t>(big::TM, M - m0), wq + n0 * K,
                ws + (n0 / 128) * KB, (int)min<int64_t>(big::TN, N - n0), K, y + m0 * N + n0, N,
                sm);
}

// Grouped variant.  The logical m-tiles of all experts are numbered
// consecutively (expert e owns ceil(M_e/128) of them); the grid is sized
// for the upper bound ceil(total_M/128) + E, and workgroups past the real
// count exit at once.  Offsets are read on the device (no host sync) and
// clamped to [0, total_M].
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xs, const uint8_t *__restrict__ wq,
    const float *__restrict__ ws, const int32_t *__restrict__ offsets, int E, int64_t total_M,
    int64_t N, int64_t K, uint16_t *__restrict__ y, int tiles_n) {
  __shared__ GemmSmem sm;
  const int tn = blockIdx.x % tiles_n;
  int mt = blockIdx.x / tiles_n;
  int64_t r0 = 0, r1 = 0;
  int e = 0;
  for (; e < E; ++e) {
    int64_t a = offsets[e], b = offsets[e + 1];
    a = a < 0 ? 0 : (a > total_M ? total_M : a);
    b = b < a ? a : (b > total_M ? total_M : b);
    const int cnt = (int)((b - a + BM - 1) / BM);
    if (mt < cnt) {
      r0 = a + (int64_t)mt * BM;
      r1 = b;
      break;
    }
    mt -= cnt;
  }
  if (e == E) return;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t KB = K / BK;
  const int64_t NB = (N + BN - 1) / BN;
  gemm_tile(xq + r0 * K, xs + r0 * KB, (int)min<int64_t>(BM, r1 - r0), wq + (int64_t)e * N * K + n0 * K,
            ws + ((int64_t)e * NB + n0 / BN) * KB, (int)min<int64_t>(BN, N - n0), K,
            y + r0 * N + n0, N, sm);
}

hipError_t launch_block_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                             int64_t M, int64_t N, int64_t K, void *y, hipStream_t stream) {
  const int64_t big_tiles = ((M + big::TM - 1) / big::TM) * ((N + big::TN - 1) / big::TN);
  if (big_tiles >= 128) {
    const int tm = (int)((M + big::TM - 1) / big::TM), tn = (int)((N + big::TN - 1) / big::TN);
    hipLaunchKernelGGL(block_gemm_256_kernel, dim3((unsigned)(tm * tn)), dim3(big::kThreads), 0,
                       stream, static_cast<const uint8_t *>(xq), xs,
                       static_cast<const uint8_t *>(wq), ws, M, N, K, static_cast<uint16_t *>(y),
                       tm, tn);
    return hipGetLastError();
  }
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL(block_gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kGemmThreads),
                     0, stream, static_cast<const uint8_t *>(xq), xs,
                     static_cast<const uint8_t *>(wq), ws, M, N, K, static_cast<uint16_t *>(y),
                     tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *offsets, int32_t E, int64_t total_M, int64_t N,
                               int64_t K, void *y, hipStream_t stream) {
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t tiles_m = (total_M + BM - 1) / BM + E;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kGemmThreads),
                     0, stream, static_cast<const uint8_t *>(xq), xs,
                     static_cast<const uint8_t *>(wq), ws, offsets, (int)E, total_M, N, K,
                     static_cast<uint16_t *>(y), (int)tiles_n);
  return hipGetLastError();
}

}  // namespace fp8blk
