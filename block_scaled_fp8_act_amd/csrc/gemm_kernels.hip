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
// Configurations: 256x256 LDS-staged tiles for M > 64 when they fill the
// chip; 128x128 tiles otherwise (with K split over two wave groups inside
// the workgroup when there is at most one workgroup per CU, and, given a
// caller workspace, over several workgroups when the grid would leave most
// CUs idle, or stream-K over 256x256 tiles for a partly empty last round
// and for small grids with long K); and a weight-streaming kernel with K
// split over its waves for M <= 64 (decode).
//
// With power-of-two scales stored as E8M0 bytes (the "UE8M0 scale format"
// section of the same page) the scale pair is applied by the matrix core
// itself: v_mfma_scale_f32_16x16x128_f8f6f4 multiplies each product by
// 2^(sa-127) * 2^(sb-127), sa taken per A row and sb per B column (each per
// 32 K values; a 128-block scale is simply the same byte for all four), and
// adds into the fp32 accumulator -- no per-block partials, no promotion FMAs.
#include <algorithm>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "fp8blk_device.h"
#include "fp8blk_launch.h"

namespace fp8blk {

__device__ __forceinline__ v8i frag_from(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// ---------------------------------------------------------------------------
// Tiled configurations.  A workgroup of WM x WN waves computes a
// (WM*FM*16) x (WN*64) output tile; each wave owns FM 16-row fragments by
// four 16-column fragments (FM*16 x 64 outputs, FM*16 fp32 accumulators per
// lane), K step 128 = one scale block.
//   Tile<2,4,8>: 256x256, 8 waves.  At the dense fp8 rate a 256x256 tile
//     needs 32 bytes per clock per CU from L2 (a 128x128 tile needs 64), and
//     a 128x64 wave sub-tile halves LDS reads per MFMA against 64x64.
//   Tile<2,2,4>: 128x128, 4 waves, for grids too small to fill 256 CUs with
//     256x256 tiles.
// Operand tiles go from global memory straight into LDS
// (global_load_lds_dwordx4, no VGPR staging), two stages.  Per stage: A
// TMx128 B, B TNx128 B (16-byte chunks XOR-swizzled by row) and the TM
// activation scales of the K block.
template <int WM, int WN, int FM>
struct Tile {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int TM = WM * FM * 16;
  static constexpr int TN = WN * 64;
  static constexpr int kDmaA = TM / 8 / kWaves;  // 1 KB DMA loads per wave per stage
  static constexpr int kDmaB = TN / 8 / kWaves;
  static_assert(kDmaA * 8 * kWaves == TM && kDmaB * 8 * kWaves == TN, "tile/DMA mismatch");
  static_assert(TM / 64 <= kWaves, "scale DMA needs TM/64 waves");
  static_assert(TM / 64 < kWaves, "one wave must be free for the weight-scale DMA");
  struct Smem {
    uint8_t a[2][TM * 128];
    uint8_t b[2][TN * 128];
    float as[2][TM];
    float ws[2][64];  // weight-block scales of the tile's (<= 2) column blocks
    float asc[2][TM * 4];  // activation scales four K blocks at a time, [row][4]
  };
  struct SmemMx {  // E8M0 scale bytes, one zero-extended dword per slot
    uint8_t a[2][TM * 128];
    uint8_t b[2][TN * 128];
    int32_t as[2][TM];  // slot wm*FM*16 + (mi/4)*64 + 4r + mi%4 holds row wm*FM*16 + 16mi + r
    int32_t ws[2][64];  // the tile's (<= 2) 128-column blocks
  };
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void lds_dma16(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 4, 0, 0);
}
// One byte per lane, written zero-extended to LDS dword lds_base + 4*lane.
__device__ __forceinline__ void lds_dma1(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 1, 0, 0);
}

// The same DMAs through a buffer resource: address = base + voff (a 32-bit
// VGPR) + soff (an SGPR), range-checked against the resource's byte count
// (reads past it return zeros).  Keeps per-load addresses at one VGPR.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                           0x00020000);
}
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void buf_dma1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 1, (int)voff, (int)soff, 0, 0);
}

// Chunk swizzle: chunk c of row r is stored at c ^ f(r) with
// f(r) = ((r & 3) << 1) | ((r >> 2) & 1), a permutation of r's low three
// bits.  A fragment read (16 lanes on 16 consecutive rows, one chunk each)
// then runs at the full LDS rate (~220 B/clk/CU measured on gfx950), where
// c ^ (r & 7) or c ^ ((r >> 1) & 7) run at half rate and no swizzle at a
// quarter.
__device__ __forceinline__ int swz_f(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ swz_f(row)) << 4);
}

// Epilogue for a full tile with 16-byte aligned output rows: each wave
// writes its (FM*16) x 64 bf16 sub-tile row-major into its own 2*FM KB of
// LDS (the 32-byte column chunks of rows 4q..4q+3 of a fragment XOR-swizzled
// by q, so the four row groups of a write land in different banks), then
// stores it 16 bytes per lane: 2*FM store instructions of 1 KB per wave
// instead of 16*FM of 128 bytes.  `stage` must be LDS that no other wave
// touches meanwhile.  The global stores are non-temporal: the output is
// not re-read by this kernel, and streaming it keeps it from displacing
// operand lines in L2 and the MALL (measured: Llama prefill step 1755 ->
// 1824 TFLOP/s, gate/up 263 -> 243 us; a dependent chain that quantizes
// each GEMM output for the next GEMM 494 -> 484 us per layer, so a
// consumer reading the output right away loses nothing).
template <int FM>
__device__ __forceinline__ void store_tile_rows16(const v4f (&acc)[FM][4], uint16_t *stage,
                                                  uint16_t *__restrict__ Yw, int64_t ldy,
                                                  int lane) {
  const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mi * 16 + 4 * q + r;
        stage[row * 64 + ((ni ^ q) << 4) + r16] = (uint16_t)bf16_rne(acc[mi][ni][r]);
      }
#pragma unroll
  for (int j = 0; j < FM * 2; ++j) {
    const int e = j * 512 + lane * 8;  // logical element: row e / 64, columns e % 64 .. +8
    const int row = e >> 6, col = e & 63;
    const int phys = row * 64 + ((((col >> 4) ^ ((row >> 2) & 3))) << 4) + (col & 15);
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u v = *reinterpret_cast<const v4u *>(stage + phys);
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(Yw + (int64_t)row * ldy + col));
  }
}

// One output tile.  A: x_q at the tile's first row (row stride K bytes),
// rows_a valid rows; As: x_scale at that row, element (r, kb) at
// As[r*xs_rs + kb*xs_ks] -- (KB, 1) for per-token-group scales, (0, 0) for
// one static scale; B: w_q
// at the tile's first column's row, rows_b valid rows; Bs: w_scale row of
// that first column's 128-block; Y: y at the tile origin (row stride ldy).
// Operand rows past rows_a / rows_b read as zeros (never out of bounds) and
// their scales from the last valid row; their outputs are not stored.
//
// The loop over a wave's FM A fragments is software-pipelined: each MFMA is
// followed by the four promotion FMAs of the MFMA issued two before it
// (whose result is complete), and the LDS reads for fragment mi+2 go out
// right after fragment mi's first MFMA; scheduling barriers pin this order
// so the FMAs fill the MFMA shadow without waiting on a result.  Three MFMA
// results and two sets of scale products are live at a time (the kernel
// fits in 256 VGPRs with room to spare).
//
// KS > 1 splits K inside the workgroup: KS groups of WM x WN waves, each with
// its own two LDS stages (sm0 is the first of KS consecutive Smem), take K
// blocks kg, kg + KS, ... in lockstep (one shared barrier per step); a group
// past the last K block re-reads it with its weight scale zeroed.  At the end
// groups 1.. hand their accumulators to group 0 through LDS, which adds them
// (in group order) and stores the tile.  For grids too small to give a CU
// more than one workgroup, this puts KS waves on each SIMD.
//
// nkb >= 1 runs only the first nkb K blocks from A, As, B, Bs (K stays the
// row stride of A and B, K/128 that of the weight scales); with kPartial
// the tile's fp32 sums go unrounded to Y reinterpreted as float (row
// stride ldy floats), one K range of a split over workgroups.
//
// kChunk (256x256 tiles over all of K; the caller guarantees xs_ks == 1,
// xs_rs and K/128 multiples of 4 and As 16-byte aligned): the activation
// scales travel four K blocks at a time, one 16-byte DMA per row into an
// LDS ring [row][4], a quarter of the rows per step (wave it & 3 loads the
// next chunk's rows 64(it & 3)..+63 during step it).  Per K step the tile
// then asks for 64 scale lines instead of one line per row (256): rows
// [M, K/128] apart are all in different lines, and those requests share the
// per-CU L1 miss slots with the 512 operand lines of the step.  Same
// values, so the same bits.  Measured (same inputs streamed from HBM, one
// launch at a time): 1.4-5.2 % faster on K >= 4096 shapes (q_a
// 8192x1536x7168 120.5 -> 114.2 us, Llama down 243.0 -> 236.6, gate/up
// 280.6 -> 274.8); all rows reading one address instead (a timing bound,
// not the method) measured 3-10 %.  Where it is used: chunked_scales_ok.
template <int WM, int WN, int FM, int KS = 1, bool kPartial = false, bool kChunk = false>
__device__ __forceinline__ void gemm_tile(const uint8_t *__restrict__ A,
                                          const float *__restrict__ As, int64_t xs_rs, int xs_ks,
                                          int rows_a, const uint8_t *__restrict__ B,
                                          const float *__restrict__ Bs, int rows_b, int64_t K,
                                          uint16_t *__restrict__ Y, int64_t ldy,
                                          typename Tile<WM, WN, FM>::Smem &sm0, int nkb = -1) {
  using T = Tile<WM, WN, FM>;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kg = KS == 1 ? 0 : wave_all / T::kWaves;  // K group
  const int wave = KS == 1 ? wave_all : wave_all % T::kWaves;
  auto &sm = (&sm0)[kg];
  const int wm = wave / WN, wn = wave % WN;
  const int KB = (int)(K / 128);           // row stride of the weight scales
  const int NKB = nkb > 0 ? nkb : KB;      // K blocks run by this tile
  const int KI = (NKB + KS - 1) / KS;  // steps (the same for every group)

  // DMA load i of a wave fills LDS rows [8r, 8r+8), r = kDma*w + i; lane l
  // writes bytes [16l, 16l+16) of that 1 KB run = row 8r + l/8, physical
  // chunk l%8, which holds logical chunk (l%8) ^ swz_f(row) (row & 7 = l/8,
  // so the chunk is the same for every i).  The loads go through a buffer
  // resource based at the K block, sized to the tile's valid rows: one VGPR
  // offset per operand, load i adding 8*i*K as a scalar offset (offsets
  // stay below 256 * K <= 2^32), and rows past rows_a / rows_b read as
  // zeros (their outputs are not stored).
  const int drow = lane >> 3;
  const uint32_t dchunk = (uint32_t)(((lane & 7) ^ swz_f(drow)) * 16);
  const uint32_t va = (uint32_t)(8 * T::kDmaA * wave + drow) * (uint32_t)K + dchunk;
  const uint32_t vb = (uint32_t)(8 * T::kDmaB * wave + drow) * (uint32_t)K + dchunk;
  const uint32_t row8 = 8u * (uint32_t)K;
  // Activation scales of rows 64w + l (waves w < TM/64).
  const float *ps = As + (int64_t)min(64 * wave + lane, rows_a - 1) * xs_rs;
  // Weight-block scales of the tile's column blocks (TN / 128 of them),
  // DMA'd with the stage by lanes 0..TN/128-1 of wave TM/64 (clamped to the
  // last existing block row of a short tile; such columns are not stored).
  // Keeping every per-step load on the vector memory path leaves no scalar
  // load in flight, so LDS waits can count partially (LDS returns in order).
  constexpr int kNbTile = T::TN / 128;
  const float *pws = Bs + (int64_t)min(lane, min(kNbTile, (rows_b + 127) / 128) - 1) * KB;
  const int wsel = (wn * 64) / 128;  // this wave's column block within the tile

  auto issue = [&](int kb, int st) {
    const uint64_t ko = (uint64_t)kb * 128u;
    const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(A + ko, (uint64_t)rows_a * (uint64_t)K - ko);
    const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(B + ko, (uint64_t)rows_b * (uint64_t)K - ko);
#pragma unroll
    for (int i = 0; i < T::kDmaA; ++i)
      buf_dma16(rA, va, (uint32_t)i * row8, sm.a[st] + (T::kDmaA * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < T::kDmaB; ++i)
      buf_dma16(rB, vb, (uint32_t)i * row8, sm.b[st] + (T::kDmaB * wave + i) * 1024);
    if constexpr (kChunk) {
      // during step kb - 1: rows 64q..64q+63 (q = (kb - 1) & 3) of the next
      // chunk; past the last chunk the last one is loaded again (its buffer
      // is not the one being read)
      if (kb > 0) {
        const int itc = kb - 1;
        const int q = itc & 3;
        const int ch = min((itc >> 2) + 1, NKB / 4 - 1);
        if (wave == q)
          lds_dma16(As + (int64_t)min(64 * q + lane, rows_a - 1) * xs_rs + 4 * ch,
                    &sm.asc[((itc >> 2) + 1) & 1][64 * q * 4]);
      }
    } else {
      if (wave < T::TM / 64) lds_dma4(ps + (int64_t)kb * xs_ks, &sm.as[st][64 * wave]);
    }
    if (wave == T::TM / 64 && lane < kNbTile) lds_dma4(pws + kb, &sm.ws[st][0]);
  };
  static_assert(!kChunk || (T::TM == 256 && KS == 1 && !kPartial),
                "chunked scales: 256-row tiles over all of K");

  v4f acc[FM][4];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  issue(min(kg, NKB - 1), 0);
  if constexpr (kChunk) {
    // chunk 0 (K blocks 0..3) of every row
    if (wave < 4)
      lds_dma16(As + (int64_t)min(64 * wave + lane, rows_a - 1) * xs_rs, &sm.asc[0][64 * wave * 4]);
  }
  // Y (a kernel argument) is first used by the epilogue; consuming it here
  // makes its scalar load complete before the loop.  With no scalar load in
  // flight the LDS reads of the loop can be waited on partially (LDS
  // returns in order; scalar loads may not).
  asm volatile("" ::"s"(Y));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int c0 = (lane >> 4) * 2;
  const int r16 = lane & 15;
  const int arow0 = wm * FM * 16 + r16;
  const int brow0 = wn * 64 + r16;
  const int srow0 = wm * FM * 16 + 4 * (lane >> 4);
  // MFMA results in flight (result j is promoted after MFMA j+2 is issued)
  // and the scale products of the current and previous A fragment
  v4f pc[3];
  float scp[2][4];

  for (int it = 0; it < KI; ++it) {
    const int st = it & 1;
    const float wsc = (KS == 1 || it * KS + kg < NKB) ? sm.ws[st][wsel] : 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t *sa = sm.a[st];
    const float4 *sas = reinterpret_cast<const float4 *>(&sm.as[st][srow0]);
    const float *sch = &sm.asc[(it >> 2) & 1][srow0 * 4 + (it & 3)];
    // the activation scales of rows srow0 + 16 mi + 0..3 at this K block
    auto rs = [&](int mi) {
      if constexpr (kChunk) {
        const float *p = sch + mi * 64;
        return float4{p[0], p[4], p[8], p[12]};
      } else {
        return sas[mi * 4];
      }
    };
    // Reads in first-use order (B0, A0, B1, B2, B3, scales, then fragment 1),
    // so the first MFMA waits only for the first four; LDS returns in order.
    // A fragments are then fetched two fragments ahead of their MFMAs.
    const uint8_t *sb = sm.b[st];
    v8i bfr[4];
    auto read_a = [&](int mi) {
      const int row = arow0 + mi * 16;
      return frag_from(*reinterpret_cast<const uint4 *>(sa + swz(row, c0)),
                       *reinterpret_cast<const uint4 *>(sa + swz(row, c0 + 1)));
    };
    bfr[0] = frag_from(*reinterpret_cast<const uint4 *>(sb + swz(brow0, c0)),
                       *reinterpret_cast<const uint4 *>(sb + swz(brow0, c0 + 1)));
    v8i af = read_a(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ni = 1; ni < 4; ++ni) {
      const int row = brow0 + ni * 16;
      bfr[ni] = frag_from(*reinterpret_cast<const uint4 *>(sb + swz(row, c0)),
                          *reinterpret_cast<const uint4 *>(sb + swz(row, c0 + 1)));
      __builtin_amdgcn_sched_barrier(0);
    }
    float4 s4 = rs(0);
    v8i afn = read_a(1);
    float4 s4n = rs(1);
    __builtin_amdgcn_sched_barrier(0);
    v8i afn2 = afn;
    float4 s4n2 = s4n;
    // MFMA j = 4*mi + ni; after issuing it, the promotion FMAs of MFMA j-2
    // (issued two MFMAs = 64 cycles earlier, its result complete) fill the
    // matrix core's shadow; scheduling barriers pin this order
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int j = mi * 4 + ni;
        pc[j % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af, bfr[ni], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (ni == 0) {
          if (mi + 2 < FM) {
            afn2 = read_a(mi + 2);
            s4n2 = rs(mi + 2);
          }
          scp[mi & 1][0] = s4.x * wsc;
          scp[mi & 1][1] = s4.y * wsc;
          scp[mi & 1][2] = s4.z * wsc;
          scp[mi & 1][3] = s4.w * wsc;
          __builtin_amdgcn_sched_barrier(0);
        }
        if (j >= 2) {
          const int jj = j - 2, mj = jj / 4, nj = jj % 4;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[mj][nj][r] = fmaf(pc[jj % 3][r], scp[mj & 1][r], acc[mj][nj][r]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (mi == 0) {
        // next stage's DMA goes out once this step's first fragment is
        // running, so the step-start LDS reads can be waited on partially
        if (it + 1 < KI) issue(min((it + 1) * KS + kg, NKB - 1), st ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      af = afn;
      s4 = s4n;
      afn = afn2;
      s4n = s4n2;
    }
    // all MFMAs of this step are issued: publish the next stage, then finish
    // this step's last two promotions
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int jj = 4 * FM - 2; jj < 4 * FM; ++jj) {
      const int mj = jj / 4, nj = jj % 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[mj][nj][r] = fmaf(pc[jj % 3][r], scp[mj & 1][r], acc[mj][nj][r]);
    }
  }

  if constexpr (KS > 1) {
    // The last step's barrier ended every LDS read and DMA: the stages are
    // free.  Groups 1.. write their accumulators (conflict-free: lane-major)
    // into one group-sized slot each, group 0 adds them in order.
    static_assert((size_t)(KS - 1) * T::TM * T::TN * 4 <= KS * sizeof(typename T::Smem),
                  "reduction buffer does not fit in the stages");
    float *red = reinterpret_cast<float *>(&sm0);
    auto slot = [&](int g, int mi, int ni, int r) {
      return (((((g - 1) * T::kWaves + wave) * FM + mi) * 4 + ni) * 4 + r) * 64 + lane;
    };
    if (kg > 0) {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[slot(kg, mi, ni, r)] = acc[mi][ni][r];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KS; ++g)
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mi][ni][r] += red[slot(g, mi, ni, r)];
  }

  // Epilogue: lane holds rows 4*(lane/16)+r of each 16x16 fragment, column lane%16.
  if constexpr (kPartial) {
    // fp32 partial sums; 16 lanes store 64 contiguous bytes of a row
    float *Yf = reinterpret_cast<float *>(Y);
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int col = wn * 64 + ni * 16 + r16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * FM * 16 + mi * 16 + 4 * (lane >> 4) + r;
          if (row < rows_a && col < rows_b) Yf[(int64_t)row * ldy + col] = acc[mi][ni][r];
        }
      }
    return;
  }
  // Full tiles with 16-byte aligned rows go through LDS (free since the last
  // barrier; past the split-K reduction slots), others element by element.
  static_assert((size_t)(KS - 1) * T::TM * T::TN * 4 + (size_t)T::TM * T::TN * 2 <=
                    KS * sizeof(typename T::Smem),
                "epilogue staging does not fit in the stages");
  if (rows_a == T::TM && rows_b == T::TN && (ldy & 7) == 0) {
    uint16_t *stage = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(&sm0) +
                                                   (size_t)(KS - 1) * T::TM * T::TN * 4) +
                      wave * (FM * 16 * 64);
    store_tile_rows16<FM>(acc, stage, Y + (int64_t)(wm * FM * 16) * ldy + wn * 64, ldy, lane);
    return;
  }
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = wn * 64 + ni * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * FM * 16 + mi * 16 + 4 * (lane >> 4) + r;
        if (row < rows_a && col < rows_b)
          Y[(int64_t)row * ldy + col] = (uint16_t)bf16_rne(acc[mi][ni][r]);
      }
    }
}

// The same tile with E8M0 scales.  A: x_q at the tile's first row; As: its
// scale bytes (row stride KB); B, Bs: w_q and the scale-byte row of the
// tile's first 128-column block; the rest as for gemm_tile.  The scale bytes
// travel with each stage by LDS DMA like the operands (VGPR-returning global
// loads in this loop would cost about half its rate), gathered so that the
// four A-row scales of fragments 4q..4q+3 that a lane needs -- rows
// wm*FM*16 + 16*mi + lane%16 -- sit in one aligned 16-byte slot group, and
// the 16 lanes of a row read 256 contiguous bytes (no bank conflict); they
// are the MFMAs' scale operands.
//
// With kScaled = false (row-wise scales) there are no per-block scales: the
// MFMAs accumulate unscaled products over all of K, and the epilogue
// multiplies output (r, c) by xr[r] * wr[c] (fp32 scales of the tile's rows
// and columns); As and Bs are unused.
//
// KS > 1 splits K inside the workgroup as in gemm_tile (KS groups, each with
// its own stages in sm0[0..KS-1], K blocks kg, kg + KS, ...; group 0 sums
// and stores).  Here the MFMAs accumulate directly, so a group cannot sit out
// a step: the caller guarantees KB % KS == 0.
//
// nkb and kPartial as in gemm_tile (one K range of a split over workgroups;
// with KS > 1 the range's block count must be a multiple of KS).
template <int WM, int WN, int FM, bool kDmaAtBarrier, bool kScaled = true, int KS = 1,
          bool kPartial = false>
__device__ __forceinline__ void gemm_tile_mx(const uint8_t *__restrict__ A,
                                             const uint8_t *__restrict__ As, int rows_a,
                                             const uint8_t *__restrict__ B,
                                             const uint8_t *__restrict__ Bs, int rows_b, int64_t K,
                                             uint16_t *__restrict__ Y, int64_t ldy,
                                             typename Tile<WM, WN, FM>::SmemMx &sm0,
                                             const float *__restrict__ xr = nullptr,
                                             const float *__restrict__ wr = nullptr,
                                             int nkb = -1) {
  using T = Tile<WM, WN, FM>;
  static_assert(FM % 4 == 0, "scale slots are read four at a time");
  static_assert(kScaled || !kPartial, "partial sums only with per-block scales");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kg = KS == 1 ? 0 : wave_all / T::kWaves;  // K group
  const int wave = KS == 1 ? wave_all : wave_all % T::kWaves;
  auto &sm = (&sm0)[kg];
  const int wm = wave / WN, wn = wave % WN;
  const int KB = (int)(K / 128);           // row stride of the scale bytes
  const int NKB = nkb > 0 ? nkb : KB;      // K blocks run by this tile
  const int KI = NKB / KS;  // steps (NKB % KS == 0)
  const int r16 = lane & 15;

  uint32_t oa[T::kDmaA];
  uint32_t ob[T::kDmaB];
#pragma unroll
  for (int i = 0; i < T::kDmaA; ++i) {
    const int row = 8 * (T::kDmaA * wave + i) + (lane >> 3);
    const int lchunk = (lane & 7) ^ swz_f(row);
    oa[i] = (uint32_t)min(row, rows_a - 1) * (uint32_t)K + lchunk * 16;
  }
#pragma unroll
  for (int i = 0; i < T::kDmaB; ++i) {
    const int row = 8 * (T::kDmaB * wave + i) + (lane >> 3);
    const int lchunk = (lane & 7) ^ swz_f(row);
    ob[i] = (uint32_t)min(row, rows_b - 1) * (uint32_t)K + lchunk * 16;
  }
  // Scale slot 64*wave + lane (waves < TM/64) <- the byte of row
  // g*FM*16 + 16*mi + r, where g = slot / (FM*16) and, within that group,
  // rem = slot % (FM*16) = 64*(mi/4) + 4r + mi%4.
  uint32_t ps;
  {
    const int slot = 64 * wave + lane;
    const int g = slot / (FM * 16), rem = slot % (FM * 16);
    const int mi = (rem / 64) * 4 + (rem & 3), r = (rem & 63) >> 2;
    const int row = g * FM * 16 + mi * 16 + r;
    ps = (uint32_t)min(row, rows_a - 1) * (uint32_t)KB;
  }
  constexpr int kNbTile = T::TN / 128;
  const int nb_tile = min(kNbTile, (rows_b + 127) / 128);
  const uint32_t pws = (uint32_t)min(lane, nb_tile - 1) * (uint32_t)KB;
  const int wsel = (wn * 64) / 128;
  const __amdgpu_buffer_rsrc_t rAs = buffer_rsrc(As, (uint64_t)rows_a * (uint64_t)KB);
  const __amdgpu_buffer_rsrc_t rBs = buffer_rsrc(Bs, (uint64_t)nb_tile * (uint64_t)KB);

  // Operand resources are based at the K block (offsets then stay below
  // 255*K + 128 < 2^32 for every K <= 2^24).
  auto issue = [&](int kb, int st) {
    const uint64_t ko = (uint64_t)kb * 128u;
    const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(A + ko, (uint64_t)rows_a * (uint64_t)K - ko);
    const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(B + ko, (uint64_t)rows_b * (uint64_t)K - ko);
#pragma unroll
    for (int i = 0; i < T::kDmaA; ++i)
      buf_dma16(rA, oa[i], 0, sm.a[st] + (T::kDmaA * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < T::kDmaB; ++i)
      buf_dma16(rB, ob[i], 0, sm.b[st] + (T::kDmaB * wave + i) * 1024);
    if constexpr (kScaled) {
      if (wave < T::TM / 64) buf_dma1(rAs, ps, (uint32_t)kb, &sm.as[st][64 * wave]);
      if (wave == T::TM / 64 && lane < kNbTile) buf_dma1(rBs, pws, (uint32_t)kb, &sm.ws[st][0]);
    }
  };

  v4f acc[FM][4];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  issue(kg, 0);
  if constexpr (kDmaAtBarrier) issue(min(KS + kg, NKB - 1), 1);
  asm volatile("" ::"s"(Y));  // no scalar load left in flight (see gemm_tile)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int c0 = (lane >> 4) * 2;
  const int arow0 = wm * FM * 16 + r16;
  const int brow0 = wn * 64 + r16;
  const int slot0 = wm * FM * 16 + r16 * 4;
  auto read_a = [&](int st, int mi) {
    const uint8_t *p = sm.a[st];
    const int row = arow0 + mi * 16;
    return frag_from(*reinterpret_cast<const uint4 *>(p + swz(row, c0)),
                     *reinterpret_cast<const uint4 *>(p + swz(row, c0 + 1)));
  };
  auto read_b = [&](int st, int ni) {
    const uint8_t *p = sm.b[st];
    const int row = brow0 + ni * 16;
    return frag_from(*reinterpret_cast<const uint4 *>(p + swz(row, c0)),
                     *reinterpret_cast<const uint4 *>(p + swz(row, c0 + 1)));
  };

  // Step kb reads stage kb&1.  Its barrier sits before the last fragment's
  // MFMAs: every wave has then finished reading stage kb&1 (waitcnt) and
  // block kb+1 has landed in the other stage.  The first reads of stage kb+1
  // go out right after it, their latency hidden under the last fragment's
  // MFMAs instead of idling the matrix core at the step start.  Block kb+2
  // is sent into stage kb&1 either right after that barrier (kDmaAtBarrier:
  // a full step ahead; used where registers are plentiful) or once the
  // first fragment of step kb+1 is running (fewer live registers).  Blocks
  // past KB-1 are clamped to KB-1: an in-bounds re-fetch into a stage that
  // nobody reads again, which keeps the step branch-free.
  v8i b0n = read_b(0, 0);
  v8i a0n = read_a(0, 0);
  for (int it = 0; it < KI; ++it) {
    const int st = it & 1;
    v8i bfr[4];
    bfr[0] = b0n;
    v8i af = a0n;
    int sa[FM] = {}, sb = 0;
    if constexpr (kScaled) {
#pragma unroll
      for (int q = 0; q < FM / 4; ++q) {
        const int4 v = *reinterpret_cast<const int4 *>(&sm.as[st][slot0 + 64 * q]);
        sa[4 * q] = v.x; sa[4 * q + 1] = v.y; sa[4 * q + 2] = v.z; sa[4 * q + 3] = v.w;
      }
      sb = sm.ws[st][wsel];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ni = 1; ni < 4; ++ni) {
      bfr[ni] = read_b(st, ni);
      __builtin_amdgcn_sched_barrier(0);
    }
    v8i afn = read_a(st, 1);
    __builtin_amdgcn_sched_barrier(0);
    v8i afn2 = afn;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
      if (mi == FM - 1) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (kDmaAtBarrier) issue(min((it + 2) * KS + kg, NKB - 1), st);
        // the last step reads the re-fetched block KB-1 here (unused)
        b0n = read_b(st ^ 1, 0);
        a0n = read_a(st ^ 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        if constexpr (kScaled)
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bfr[ni], acc[mi][ni], 0, 0, 0, sa[mi], 0, sb);
        else
          acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bfr[ni], acc[mi][ni], 0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (ni == 0 && mi + 2 < FM) {
          afn2 = read_a(st, mi + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (!kDmaAtBarrier) {
        if (mi == 0) {
          issue(min((it + 1) * KS + kg, NKB - 1), st ^ 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      af = afn;
      afn = afn2;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  if constexpr (KS > 1) {
    // as in gemm_tile: groups 1.. hand their accumulators to group 0
    static_assert((size_t)(KS - 1) * T::TM * T::TN * 4 <= KS * sizeof(typename T::SmemMx),
                  "reduction buffer does not fit in the stages");
    __syncthreads();  // every wave is past its last LDS read and DMA
    float *red = reinterpret_cast<float *>(&sm0);
    auto slot = [&](int g, int mi, int ni, int r) {
      return (((((g - 1) * T::kWaves + wave) * FM + mi) * 4 + ni) * 4 + r) * 64 + lane;
    };
    if (kg > 0) {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[slot(kg, mi, ni, r)] = acc[mi][ni][r];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KS; ++g)
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mi][ni][r] += red[slot(g, mi, ni, r)];
  }

  if constexpr (kPartial) {
    // fp32 partial sums, as in gemm_tile
    float *Yf = reinterpret_cast<float *>(Y);
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int col = wn * 64 + ni * 16 + r16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * FM * 16 + mi * 16 + 4 * (lane >> 4) + r;
          if (row < rows_a && col < rows_b) Yf[(int64_t)row * ldy + col] = acc[mi][ni][r];
        }
      }
    return;
  }
  float cs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if constexpr (!kScaled) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) cs[ni] = wr[min(wn * 64 + ni * 16 + r16, rows_b - 1)];
  }
  static_assert((size_t)(KS - 1) * T::TM * T::TN * 4 + (size_t)T::TM * T::TN * 2 <=
                    KS * sizeof(typename T::SmemMx),
                "epilogue staging does not fit in the stages");
  if (rows_a == T::TM && rows_b == T::TN && (ldy & 7) == 0) {
    // as in gemm_tile; the barrier ends the last step's (unused) reads of
    // the other stage (with KS > 1 the reduction's barriers already did, and
    // groups 1.. have left)
    if constexpr (!kScaled) {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float rs = xr[wm * FM * 16 + mi * 16 + 4 * (lane >> 4) + r];
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) acc[mi][ni][r] = acc[mi][ni][r] * (rs * cs[ni]);
        }
    }
    if constexpr (KS == 1) __syncthreads();
    uint16_t *stage = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(&sm0) +
                                                   (size_t)(KS - 1) * T::TM * T::TN * 4) +
                      wave * (FM * 16 * 64);
    store_tile_rows16<FM>(acc, stage, Y + (int64_t)(wm * FM * 16) * ldy + wn * 64, ldy, lane);
    return;
  }
#pragma unroll
  for (int mi = 0; mi < FM; ++mi) {
    float rs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (!kScaled) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rs[r] = xr[min(wm * FM * 16 + mi * 16 + 4 * (lane >> 4) + r, rows_a - 1)];
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int col = wn * 64 + ni * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * FM * 16 + mi * 16 + 4 * (lane >> 4) + r;
        float v = acc[mi][ni][r];
        if constexpr (!kScaled) v = v * (rs[r] * cs[ni]);
        if (row < rows_a && col < rows_b) Y[(int64_t)row * ldy + col] = (uint16_t)bf16_rne(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-M ("decode") configuration, M <= 64: the GEMM is a stream of W from
// HBM (arithmetic intensity 2..32 flop/byte).  One workgroup owns a slab of
// 16 output columns; its waves (16, or 8 where the register budget calls
// for it) split the K blocks round-robin (wave w of S takes kb = w, w + S,
// ...), so the slab's weight rows are read once,
// straight from global memory into MFMA operand registers (no LDS staging),
// U blocks per wave at a time so that many loads are in flight.  Each wave
// keeps 16x16 partial tiles for up to four 16-row fragments of x; the
// partials are summed through LDS at the end.  Activation codes come from L2
// (x is small and read by every workgroup); activation scales are staged
// once in LDS, transposed to [kb][row], while the first weight loads fly.
constexpr int kDecWaves = 16;
constexpr int kDecThreads = kDecWaves * 64;
// Two row fragments (17-32 rows, fp32 block scales) run 8 waves from this
// many columns on, in the decode GEMM and the fused layer alike (the same K
// split over the same waves, so the two stay bit-identical).  Measured
// against 16 waves, weights streamed from HBM, M = 17-32: the GEMM 14336 x
// 4096 25.2-26.1 -> 22.5-22.7 us; the fused layer 14336 x 4096 33.3-37.5 ->
// 33.1-33.9 us and 7168 x 16384 52.8-61.8 -> 52.0-53.9 us; on narrower
// shapes the fused layer lost up to 12 % (4096 x 14336, 1536 x 7168 at
// M = 17), hence the bound.
constexpr int64_t kDecWide8N = 8192;
constexpr int kDecMaxM = 64;
constexpr int kDecMaxScaleBytes = 32 * 1024;  // x_scale staging limit (KB * MF * 16 * 4)

// NW waves per workgroup (kDecWaves by default; 8 for four row fragments
// with fp32 block scales, for two from kDecWide8N columns on, and for E8M0
// scales past 16 rows: the twice larger register budget per wave holds two
// load buffers, and packed slabs, without spilling).
//
// S = float: fp32 scales, promoted per K block with FMAs as in gemm_tile;
// S = uint8_t: E8M0 scale bytes, loaded with the operands and applied by the
// matrix core (nothing staged in LDS but the final partials).  kRow: fp32
// row-wise scales (xs[M], ws[N]): unscaled MFMAs accumulate over all of K and
// the sum is scaled by xs[m] * ws[n] at the end.  kPartial (fp32 block
// scales only): workgroup (x, s) takes K blocks [s * kb_per, (s + 1) * kb_per)
// and writes its unrounded fp32 sums to part + s * slice (row stride N).
template <int MF, typename S, bool kRow = false, int NS = 1, bool kPartial = false,
          int NW = kDecWaves>
__global__ __launch_bounds__(NW * 64) void decode_gemm_kernel(
    const uint8_t *__restrict__ xq, const S *__restrict__ xs, int64_t xs_rs, int xs_ks,
    const uint8_t *__restrict__ wq, const S *__restrict__ ws, int M, int64_t N, int64_t K,
    uint16_t *__restrict__ y, float *__restrict__ part, int64_t slice, int kb_per) {
  constexpr bool MX = std::is_same<S, uint8_t>::value;
  static_assert(!(kRow && MX), "row-wise scales are fp32");
  static_assert(!kPartial || (!MX && !kRow), "partial sums: fp32 block scales only");
  static_assert(NS == 1 || NS == 2 || NS == 4, "slabs per workgroup: 1, 2 or 4");
  static_assert(NS * MF <= NW, "one wave per (slab, fragment) sums the partials");
  constexpr int R = MF * 16;                          // staged rows
  // register buffers of U K blocks: two (the next batch's loads go out
  // before the current batch's MFMAs) unless four row fragments, four slabs
  // with E8M0 scale operands, or eight (slab, fragment) pairs leave no room
  // in the 128 VGPRs of a 16-wave workgroup (then one, reloaded after its
  // MFMAs; for the four E8M0 slabs that still beats two slabs in two rounds
  // of workgroups: 14336 x 4096 at M = 16 18.2 -> 14.5 us, M = 4 15.2 ->
  // 13.8 us).  With 8 waves (256 VGPRs) every variant keeps two.
  static_assert(NW == kDecWaves || NW == kDecWaves / 2, "16 or 8 waves");
  constexpr bool kRoomy = NW < kDecWaves;
  constexpr int NB = (!kRoomy && (MF >= 4 || (MX && NS == 4) || MF * NS >= 8)) ? 1 : 2;
  constexpr int U = (4 / NB) / (MF * NS) > 0 ? (4 / NB) / (MF * NS) : 1;
  extern __shared__ __align__(16) float dsm[];
  float *s_as = dsm;                                  // [KB][R] (fp32 scales only)
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int KB = (int)(K / 128);
  // this workgroup's K blocks: [kb0, kb0 + kbn)
  const int kb0 = kPartial ? (int)blockIdx.y * kb_per : 0;
  const int kbn = kPartial ? min(KB - kb0, kb_per) : KB;
  v4f *s_part = reinterpret_cast<v4f *>(dsm);  // [waves][NS][MF][64], reuses s_as after the loop
  const int64_t n0 = (int64_t)blockIdx.x * 16 * NS;

  const int r16 = lane & 15;
  const int kc = (lane >> 4) * 32;  // this lane's 32 K bytes within the block
  const uint8_t *pb[NS];            // weight row of this lane's column in slab s (clamped)
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) pb[sl] = wq + min<int64_t>(n0 + 16 * sl + r16, N - 1) * K + kc;
  const uint8_t *pa[MF];
  const S *psa[MF];                 // E8M0: scale row of this lane's A-operand row
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    pa[f] = xq + (int64_t)min(f * 16 + r16, M - 1) * K + kc;
    psa[f] = xs + (int64_t)min(f * 16 + r16, M - 1) * KB;
  }
  // the NS slabs (16 * NS <= 64 columns from a multiple of 16 * NS) share
  // one 128-column weight block
  const S *pws = ws + (n0 / 128) * KB;
  const int nmine = wave < kbn ? (kbn - wave + NW - 1) / NW : 0;

  uint4 bw[NB][U][NS][2];
  v8i af[NB][U][MF];
  int sa[NB][U][MF], sb[NB][U];
  auto load = [&](auto bufc, int j0) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < nmine) {
        const int kb = kb0 + wave + NW * (j0 + u);
        const int64_t ko = (int64_t)kb * 128;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          bw[buf][u][sl][0] = *reinterpret_cast<const uint4 *>(pb[sl] + ko);
          bw[buf][u][sl][1] = *reinterpret_cast<const uint4 *>(pb[sl] + ko + 16);
        }
#pragma unroll
        for (int f = 0; f < MF; ++f)
          af[buf][u][f] = frag_from(*reinterpret_cast<const uint4 *>(pa[f] + ko),
                                    *reinterpret_cast<const uint4 *>(pa[f] + ko + 16));
        if constexpr (MX) {
#pragma unroll
          for (int f = 0; f < MF; ++f) sa[buf][u][f] = psa[f][kb];
          sb[buf][u] = pws[kb];
        }
      }
    }
  };
  load(std::integral_constant<int, 0>{}, 0);

  if constexpr (!MX && !kRow) {
    for (int i = t; i < kbn * R; i += NW * 64) {
      const int kb = kb0 + i / R, m = i % R;
      s_as[i] = xs[(int64_t)min(m, M - 1) * xs_rs + (int64_t)kb * xs_ks];
    }
    __syncthreads();
  }

  v4f acc[NS][MF];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl)
#pragma unroll
    for (int f = 0; f < MF; ++f) acc[sl][f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](auto bufc, int j0) {
    constexpr int buf = decltype(bufc)::value;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < nmine) {
        const int kb = kb0 + wave + NW * (j0 + u);
        float4 s4[MF];
        float wsc = 1.0f;
        if constexpr (!MX && !kRow) {
          wsc = pws[kb];
#pragma unroll
          for (int f = 0; f < MF; ++f)
            s4[f] = *reinterpret_cast<const float4 *>(&s_as[(kb - kb0) * R + f * 16 + 4 * (lane >> 4)]);
        }
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          const v8i bf = frag_from(bw[buf][u][sl][0], bw[buf][u][sl][1]);
#pragma unroll
          for (int f = 0; f < MF; ++f) {
            if constexpr (MX) {
              acc[sl][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  af[buf][u][f], bf, acc[sl][f], 0, 0, 0, sa[buf][u][f], 0, sb[buf][u]);
            } else if constexpr (kRow) {
              acc[sl][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  af[buf][u][f], bf, acc[sl][f], 0, 0, 0, 0, 0, 0);
            } else {
              const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  af[buf][u][f], bf, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
              acc[sl][f][0] = fmaf(p[0], s4[f].x * wsc, acc[sl][f][0]);
              acc[sl][f][1] = fmaf(p[1], s4[f].y * wsc, acc[sl][f][1]);
              acc[sl][f][2] = fmaf(p[2], s4[f].z * wsc, acc[sl][f][2]);
              acc[sl][f][3] = fmaf(p[3], s4[f].w * wsc, acc[sl][f][3]);
            }
          }
        }
      }
    }
  };
  if constexpr (NB == 2) {
    for (int j0 = 0; j0 < nmine; j0 += 2 * U) {
      load(std::integral_constant<int, 1>{}, j0 + U);
      compute(std::integral_constant<int, 0>{}, j0);
      load(std::integral_constant<int, 0>{}, j0 + 2 * U);
      compute(std::integral_constant<int, 1>{}, j0 + U);
    }
  } else {
    for (int j0 = 0; j0 < nmine; j0 += U) {
      compute(std::integral_constant<int, 0>{}, j0);
      load(std::integral_constant<int, 0>{}, j0 + U);
    }
  }
  __syncthreads();  // every wave is done with s_as
#pragma unroll
  for (int sl = 0; sl < NS; ++sl)
#pragma unroll
    for (int f = 0; f < MF; ++f) s_part[((wave * NS + sl) * MF + f) * 64 + lane] = acc[sl][f];
  __syncthreads();
  // wave q (< NS * MF) sums (slab q / MF, fragment q % MF) over the waves
  if (wave < NS * MF) {
    const int sl = wave / MF, f = wave % MF;
    v4f sum = s_part[(sl * MF + f) * 64 + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const v4f v = s_part[((w * NS + sl) * MF + f) * 64 + lane];
      sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
    }
    const int64_t col = n0 + 16 * sl + r16;
    float cs = 1.0f;
    if constexpr (kRow) cs = ws[min<int64_t>(col, N - 1)];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = f * 16 + 4 * (lane >> 4) + r;
      float v = sum[r];
      if constexpr (kRow) v = v * (xs[min(row, M - 1)] * cs);
      if (row < M && col < N) {
        if constexpr (kPartial)
          part[(int64_t)blockIdx.y * slice + (int64_t)row * N + col] = v;
        else
          y[(int64_t)row * N + col] = (uint16_t)bf16_rne(v);
      }
    }
  }
}
// 16-column slabs per decode workgroup: 1, 2 or up to max_ns.  More slabs
// make each workgroup stream more weight bytes per read of x (and, in the
// fused layer, amortize its quantization of x); with one workgroup per CU
// the count is picked for the fullest last round of workgroups (ties: more
// slabs).
static int decode_slabs(int64_t N, int max_ns) {
  const int64_t slabs = (N + 15) / 16;
  int ns_best = 1;
  double best = 0.0;
  for (int ns = 1; ns <= max_ns; ns *= 2) {
    const int64_t wgs = (slabs + ns - 1) / ns;
    const double fill = (double)wgs / (double)(((wgs + 255) / 256) * 256);
    if (fill >= best - 1e-9) { best = fill; ns_best = ns; }
  }
  return ns_best;
}

int linear_decode_slabs(int64_t M, int64_t N) { return decode_slabs(N, M <= 16 ? 4 : 2); }

template <int MF, typename S, bool kRow, int NW>
static hipError_t launch_decode_nw(const void *xq, const S *xs, int64_t xs_rs, int xs_ks,
                                   const void *wq, const S *ws, int64_t M, int64_t N, int64_t K,
                                   void *y, hipStream_t stream) {
  const int64_t KB = K / 128;
  // slabs per workgroup: up to four for one or two row fragments, up to two
  // for four; for more than one fragment with fp32 scales (block or
  // row-wise) and with E8M0 scales on 8 waves (below).  Every workgroup
  // reads all of x (M x K
  // bytes) once per K pass, as many bytes as its slab of weights at M = 16
  // and twice or four times as many at M = 32 or 64, so packing slabs cuts
  // the bytes per output column: measured (weights streamed from HBM)
  // 14336 x 4096 at M = 17-32 27.3-31.8 -> 18.7-20.0 us, M = 48-64 44-51 ->
  // 41-44 us; 7168 x 16384 at M = 17-32 42-52 -> 32-36 us, M = 64 85 -> 71
  // us; row-wise 14336 x 4096 at M = 17-64 22.9-42.4 -> 15.3-29.4 us,
  // 7168 x 16384 37.7-75.5 -> 30.3-48.3 us; shapes that keep one slab
  // unchanged.
  //
  // Four row fragments with fp32 block scales run 8 waves per workgroup:
  // with 16 they had one load buffer and spilled; with 8 (256 VGPRs each)
  // they keep two and none spills.  Measured (M = 24-64, weights streamed
  // from HBM, one launch at a time): 7168 x 16384 at M = 48 / 64 71.0 /
  // 76.6 -> 52.2 / 57.4 us, the other decode shapes within 3 %.  One or
  // two fragments keep 16 waves (8 measured up to 16 % slower at M = 1-16).
  //
  // E8M0 scales past 16 rows (two or four fragments) likewise run 8 waves,
  // which leaves room to pack slabs as the fp32 kernel does (with 16 waves
  // the packed variants spilled, so they kept one slab).  Measured, one
  // slab on 16 waves against packed slabs on 8: 14336 x 4096 at M = 17-32
  // 33.8-42.1 -> 21.8-23.8 us, 7168 x 16384 at M = 17-64 51-112 -> 40-72
  // us, the other Llama and DeepSeek-V3 decode shapes within 3 %.
  //
  // Two fragments with fp32 block scales take 8 waves from kDecWide8N
  // columns on (launch_decode).
  constexpr bool kBlk = std::is_same<S, float>::value;
  constexpr bool kMx8 = !kBlk && MF >= 2;
  const int64_t slabs = (N + 15) / 16;
  const int NS = MF == 1 ? decode_slabs(N, 4)
                         : ((kBlk || kMx8) ? decode_slabs(N, MF == 2 ? 4 : 2) : 1);
  const size_t part = (size_t)NW * NS * MF * 64 * 16;
  const size_t lds = (std::is_same<S, uint8_t>::value || kRow)
                         ? part
                         : std::max((size_t)KB * MF * 16 * 4, part);
  const dim3 grid((unsigned)((slabs + NS - 1) / NS));
  const auto *a = static_cast<const uint8_t *>(xq);
  const auto *b = static_cast<const uint8_t *>(wq);
  auto *out = static_cast<uint16_t *>(y);
  if (NS == 4)
    hipLaunchKernelGGL(
        (decode_gemm_kernel<MF, S, kRow, (MF == 1 || ((kBlk || kMx8) && MF == 2) ? 4 : 1), false,
                            NW>),
        grid, dim3(NW * 64), lds, stream, a, xs, xs_rs, xs_ks, b, ws, (int)M, N, K, out, nullptr,
        (int64_t)0, 0);
  else if (NS == 2)
    hipLaunchKernelGGL((decode_gemm_kernel<MF, S, kRow, (MF == 1 || kBlk || kMx8 ? 2 : 1), false, NW>),
                       grid, dim3(NW * 64), lds, stream, a, xs, xs_rs, xs_ks, b, ws, (int)M, N,
                       K, out, nullptr, (int64_t)0, 0);
  else
    hipLaunchKernelGGL((decode_gemm_kernel<MF, S, kRow, 1, false, NW>), grid, dim3(NW * 64), lds,
                       stream, a, xs, xs_rs, xs_ks, b, ws, (int)M, N, K, out, nullptr,
                       (int64_t)0, 0);
  return hipGetLastError();
}

template <int MF, typename S, bool kRow = false>
static hipError_t launch_decode(const void *xq, const S *xs, int64_t xs_rs, int xs_ks,
                                const void *wq, const S *ws, int64_t M, int64_t N, int64_t K,
                                void *y, hipStream_t stream) {
  constexpr bool kBlk = std::is_same<S, float>::value;
  if constexpr (MF == 2 && kBlk && !kRow) {
    if (N >= kDecWide8N)
      return launch_decode_nw<MF, S, kRow, kDecWaves / 2>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K,
                                                           y, stream);
    return launch_decode_nw<MF, S, kRow, kDecWaves>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y,
                                                    stream);
  } else {
    constexpr int NW = ((MF == 4 && kBlk && !kRow) || (!kBlk && MF >= 2)) ? kDecWaves / 2
                                                                             : kDecWaves;
    return launch_decode_nw<MF, S, kRow, NW>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y, stream);
  }
}

// ---------------------------------------------------------------------------
// Fused decode linear layer (M <= 64): the dynamic activation quantization
// runs inside the weight-streaming GEMM, so one launch turns bf16 x into y.
// Each lane loads the 32 bf16 values whose fp8 codes its A fragment would
// hold (row 16f + lane%16 of K block kb, values 32*(lane/16) .. +32); the
// group amax is the max over the four lanes holding that row's 128 values
// (xor-shuffles by 16 and 32); the element map is make_qparams / quotient,
// bit-identical to the activation quantizer; the codes go straight into the
// MFMA operand and the group scale into the promotion (fetched by shuffle
// from the lane that holds each output row).  x is small and read by every
// workgroup from L2; the redundant quantization hides under the W stream.
// NW waves split the K blocks (16, or 8 for MF = 4, whose four bf16
// fragments need the larger per-wave register budget).
template <int MF, int NW, int NS = 1>
__global__ __launch_bounds__(NW * 64) void decode_linear_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ wq, const float *__restrict__ ws,
    int M, int64_t N, int64_t K, uint16_t *__restrict__ y) {
  static_assert(NS == 1 || NS == 2 || NS == 4, "slabs per workgroup: 1, 2 or 4");
  static_assert(NS * MF <= NW, "one wave per (slab, fragment) sums the partials");
  // K blocks in flight (bf16 x takes 16 VGPRs per fragment)
  constexpr int U = (MF == 1 && NS < 4) ? 2 : 1;
  extern __shared__ __align__(16) float dsm[];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int KB = (int)(K / 128);
  v4f *s_part = reinterpret_cast<v4f *>(dsm);  // [waves][NS][MF][64]
  const int64_t n0 = (int64_t)blockIdx.x * 16 * NS;

  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int kc = g * 32;
  const uint8_t *pb[NS];  // weight row of this lane's column in slab s (clamped)
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) pb[sl] = wq + min<int64_t>(n0 + 16 * sl + r16, N - 1) * K + kc;
  const uint16_t *px[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) px[f] = x + (int64_t)min(f * 16 + r16, M - 1) * K + kc;
  // the NS slabs (16 * NS <= 64 columns from a multiple of 16 * NS) share
  // one 128-column weight block
  const float *pws = ws + (n0 / 128) * KB;
  const int nmine = wave < KB ? (KB - wave + NW - 1) / NW : 0;

  uint4 bw[U][NS][2];
  uint4 xr[U][MF][4];
  auto load = [&](int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < nmine) {
        const int64_t ko = (int64_t)(wave + NW * (j0 + u)) * 128;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          bw[u][sl][0] = *reinterpret_cast<const uint4 *>(pb[sl] + ko);
          bw[u][sl][1] = *reinterpret_cast<const uint4 *>(pb[sl] + ko + 16);
        }
#pragma unroll
        for (int f = 0; f < MF; ++f)
#pragma unroll
          for (int c = 0; c < 4; ++c) xr[u][f][c] = *reinterpret_cast<const uint4 *>(px[f] + ko + 8 * c);
      }
    }
  };
  load(0);

  v4f acc[NS][MF];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl)
#pragma unroll
    for (int f = 0; f < MF; ++f) acc[sl][f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int j0 = 0; j0 < nmine; j0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < nmine) {
        const int kb = wave + NW * (j0 + u);
        const float wsc = pws[kb];
#pragma unroll
        for (int f = 0; f < MF; ++f) {
          float am = 0.0f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float v[8];
            unpack8(xr[u][f][c], v);
            am = fmaxf(am, absmax8(v));
          }
          am = fmaxf(am, __shfl_xor(am, 16));
          am = fmaxf(am, __shfl_xor(am, 32));
          const QParams p = make_qparams(am);
          v8i af;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float v[8];
            unpack8(xr[u][f][c], v);
#pragma unroll
            for (int h = 0; h < 2; ++h)
              af[2 * c + h] = (int)pack4_e4m3(quotient(ldexpf(v[4 * h], p.k), p.sp, p.y),
                                              quotient(ldexpf(v[4 * h + 1], p.k), p.sp, p.y),
                                              quotient(ldexpf(v[4 * h + 2], p.k), p.sp, p.y),
                                              quotient(ldexpf(v[4 * h + 3], p.k), p.sp, p.y));
          }
          // output rows 4g + r of this fragment: their scales live in lanes 4g + r
          float sr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) sr[r] = __shfl(p.s, 4 * g + r) * wsc;
          // the codes are formed once and serve every slab
#pragma unroll
          for (int sl = 0; sl < NS; ++sl) {
            const v8i bf = frag_from(bw[u][sl][0], bw[u][sl][1]);
            const v4f pc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af, bf, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[sl][f][r] = fmaf(pc[r], sr[r], acc[sl][f][r]);
          }
        }
      }
    }
    if (j0 + U < nmine) load(j0 + U);
  }
#pragma unroll
  for (int sl = 0; sl < NS; ++sl)
#pragma unroll
    for (int f = 0; f < MF; ++f) s_part[((wave * NS + sl) * MF + f) * 64 + lane] = acc[sl][f];
  __syncthreads();
  if (wave < NS * MF) {
    const int sl = wave / MF, f = wave % MF;
    v4f sum = s_part[(sl * MF + f) * 64 + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const v4f v = s_part[((w * NS + sl) * MF + f) * 64 + lane];
      sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
    }
    const int64_t col = n0 + 16 * sl + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = f * 16 + 4 * g + r;
      if (row < M && col < N) y[(int64_t)row * N + col] = (uint16_t)bf16_rne(sum[r]);
    }
  }
}

// Slabs per workgroup: up to four for one row fragment, up to two for two
// or four (more would spill: the bf16 x fragments take 16 VGPRs each).
// Every workgroup reads and quantizes all of x (2 M K bytes), twice its
// slab's weight bytes at M = 16, so packing matters more as M grows:
// measured with no workspaces (weights streamed from HBM) 14336 x 4096 at
// M = 17-32 46-49 -> 27-31 us and M = 33-64 85-91 -> 47-49 us, 7168 x 16384
// at M = 17-32 77-82 -> 48-55 us and M = 33-64 149-154 -> 82-85 us;
// bit-identical (same waves per K split).
template <int MF, int NW>
static hipError_t launch_decode_linear(const void *x, const void *wq, const float *ws, int64_t M,
                                       int64_t N, int64_t K, void *y, hipStream_t stream) {
  const int NS = decode_slabs(N, MF == 1 ? 4 : 2);
  const size_t lds = (size_t)NW * NS * MF * 64 * 16;
  const dim3 grid((unsigned)(((N + 15) / 16 + NS - 1) / NS));
  const auto *xp = static_cast<const uint16_t *>(x);
  const auto *wp = static_cast<const uint8_t *>(wq);
  auto *yp = static_cast<uint16_t *>(y);
  if (NS == 4)
    hipLaunchKernelGGL((decode_linear_kernel<MF, NW, (MF == 1 ? 4 : 1)>), grid, dim3(NW * 64), lds,
                       stream, xp, wp, ws, (int)M, N, K, yp);
  else if (NS == 2)
    hipLaunchKernelGGL((decode_linear_kernel<MF, NW, 2>), grid, dim3(NW * 64), lds,
                       stream, xp, wp, ws, (int)M, N, K, yp);
  else
    hipLaunchKernelGGL((decode_linear_kernel<MF, NW, 1>), grid, dim3(NW * 64), lds, stream, xp, wp,
                       ws, (int)M, N, K, yp);
  return hipGetLastError();
}

hipError_t launch_linear_decode(const void *x, const void *wq, const float *ws, int64_t M,
                                int64_t N, int64_t K, void *y, hipStream_t stream) {
  if (M <= 16) return launch_decode_linear<1, 16>(x, wq, ws, M, N, K, y, stream);
  if (M <= 32)
    return N >= kDecWide8N ? launch_decode_linear<2, 8>(x, wq, ws, M, N, K, y, stream)
                           : launch_decode_linear<2, 16>(x, wq, ws, M, N, K, y, stream);
  return launch_decode_linear<4, 8>(x, wq, ws, M, N, K, y, stream);
}

// Map a linear workgroup id to (tile_m, tile_n).  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2); consecutive logical
// tiles are made to land on one XCD, and logical tiles are ordered in
// groups of 8 tile rows so that neighbours share A rows and B columns.
__device__ __forceinline__ void group_coords(int bid, int tiles_m, int tiles_n, int &tm,
                                             int &tn) {
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = bid - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  return (total & 7) == 0 ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
}

__device__ __forceinline__ void tile_coords(int bid, int total, int tiles_m, int tiles_n,
                                            int &tm, int &tn) {
  group_coords(xcd_remap(bid, total), tiles_m, tiles_n, tm, tn);
}

// One tile with either scale type: S = float -> gemm_tile, S = uint8_t
// (E8M0 bytes) -> gemm_tile_mx.
template <int WM, int WN, int FM, typename S>
struct TileSmem {
  using type = typename std::conditional<std::is_same<S, uint8_t>::value,
                                         typename Tile<WM, WN, FM>::SmemMx,
                                         typename Tile<WM, WN, FM>::Smem>::type;
};

// xs_rs / xs_ks address the fp32 activation scales (E8M0 bytes always use
// the per-token-group layout).
template <int WM, int WN, int FM, typename S, bool kChunk = false>
__device__ __forceinline__ void run_tile(const uint8_t *A, const S *As, int64_t xs_rs, int xs_ks,
                                         int rows_a, const uint8_t *B, const S *Bs, int rows_b,
                                         int64_t K, uint16_t *Y, int64_t ldy,
                                         typename TileSmem<WM, WN, FM, S>::type &sm) {
  if constexpr (std::is_same<S, uint8_t>::value)
    gemm_tile_mx<WM, WN, FM, (FM <= 4)>(A, As, rows_a, B, Bs, rows_b, K, Y, ldy, sm);
  else
    gemm_tile<WM, WN, FM, 1, false, kChunk>(A, As, xs_rs, xs_ks, rows_a, B, Bs, rows_b, K, Y,
                                            ldy, sm);
}

template <int WM, int WN, int FM, typename S, bool kChunk = false>
__global__ __launch_bounds__(WM * WN * 64) void block_gemm_kernel(
    const uint8_t *__restrict__ xq, const S *__restrict__ xs, int64_t xs_rs, int xs_ks,
    const uint8_t *__restrict__ wq, const S *__restrict__ ws, int64_t M, int64_t N, int64_t K,
    uint16_t *__restrict__ y, int tiles_m, int tiles_n) {
  using T = Tile<WM, WN, FM>;
  __shared__ typename TileSmem<WM, WN, FM, S>::type sm;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * T::TM, n0 = (int64_t)tn * T::TN;
  const int64_t KB = K / 128;
  run_tile<WM, WN, FM, S, kChunk>(xq + m0 * K, xs + m0 * xs_rs, xs_rs, xs_ks,
                                  (int)min<int64_t>(T::TM, M - m0), wq + n0 * K,
                                  ws + (n0 / 128) * KB, (int)min<int64_t>(T::TN, N - n0), K,
                                  y + m0 * N + n0, N, sm);
}

// Split-K inside the workgroup: KS groups of WM x WN waves on one tile, for
// grids that leave CUs with a single workgroup.  S = float: fp32 scales
// (any K); S = uint8_t: E8M0 bytes (K/128 a multiple of KS); kRow: row-wise
// fp32 scales xs[M], ws[N] (K/128 a multiple of KS).
template <int WM, int WN, int FM, int KS, typename S, bool kRow = false>
__global__ __launch_bounds__(WM * WN * 64 * KS) void block_gemm_ks_kernel(
    const uint8_t *__restrict__ xq, const S *__restrict__ xs, int64_t xs_rs, int xs_ks,
    const uint8_t *__restrict__ wq, const S *__restrict__ ws, int64_t M, int64_t N,
    int64_t K, uint16_t *__restrict__ y, int tiles_m, int tiles_n) {
  using T = Tile<WM, WN, FM>;
  constexpr bool kMx = std::is_same<S, uint8_t>::value || kRow;
  __shared__ typename std::conditional<kMx, typename T::SmemMx, typename T::Smem>::type sm[KS];
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * T::TM, n0 = (int64_t)tn * T::TN;
  const int64_t KB = K / 128;
  const int rows_a = (int)min<int64_t>(T::TM, M - m0), rows_b = (int)min<int64_t>(T::TN, N - n0);
  if constexpr (kRow)
    gemm_tile_mx<WM, WN, FM, (FM <= 4), false, KS>(xq + m0 * K, nullptr, rows_a, wq + n0 * K,
                                                   nullptr, rows_b, K, y + m0 * N + n0, N, sm[0],
                                                   xs + m0, ws + n0);
  else if constexpr (kMx)
    gemm_tile_mx<WM, WN, FM, (FM <= 4), true, KS>(xq + m0 * K, xs + m0 * KB, rows_a, wq + n0 * K,
                                                  ws + (n0 / 128) * KB, rows_b, K, y + m0 * N + n0,
                                                  N, sm[0]);
  else
    gemm_tile<WM, WN, FM, KS>(xq + m0 * K, xs + m0 * xs_rs, xs_rs, xs_ks, rows_a, wq + n0 * K,
                              ws + (n0 / 128) * KB, rows_b, K, y + m0 * N + n0, N, sm[0]);
}

// K split over workgroups, for grids of 128x128 tiles that would leave most
// CUs idle (small M and N, long K: DeepSeek-V3 q_a and kv_a at M = 512 have
// 48 and 20 tiles for 256 CUs).  Workgroup b runs tile b % tiles over K
// blocks [split * kb_per, min(KB, (split + 1) * kb_per)), split = b / tiles,
// with the two wave groups of block_gemm_ks_kernel inside, and writes the
// tile's unrounded fp32 sums to slice `split` of the workspace (slices of
// slice_elems floats, row stride N).  splitk_reduce_kernel then adds the
// slices in split order and rounds once to bf16.
// S = float: fp32 scales (any range length); S = uint8_t: E8M0 scale bytes
// (range lengths multiples of KS).
template <int WM, int WN, int FM, int KS, typename S>
__global__ __launch_bounds__(WM * WN * 64 * KS) void block_gemm_splitk_kernel(
    const uint8_t *__restrict__ xq, const S *__restrict__ xs, const uint8_t *__restrict__ wq,
    const S *__restrict__ ws, int64_t M, int64_t N, int64_t K, float *__restrict__ part,
    int64_t slice_elems, int tiles_m, int tiles_n, int kb_per) {
  using T = Tile<WM, WN, FM>;
  __shared__ typename TileSmem<WM, WN, FM, S>::type sm[KS];
  const int tiles = tiles_m * tiles_n;
  const int split = blockIdx.x / tiles;
  int tm, tn;
  tile_coords(blockIdx.x - split * tiles, tiles, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * T::TM, n0 = (int64_t)tn * T::TN;
  const int64_t KB = K / 128;
  const int64_t kb0 = (int64_t)split * kb_per;
  const int nkb = (int)min<int64_t>(kb_per, KB - kb0);
  uint16_t *out = reinterpret_cast<uint16_t *>(part + split * slice_elems + m0 * N + n0);
  const int rows_a = (int)min<int64_t>(T::TM, M - m0), rows_b = (int)min<int64_t>(T::TN, N - n0);
  if constexpr (std::is_same<S, uint8_t>::value)
    gemm_tile_mx<WM, WN, FM, (FM <= 4), true, KS, true>(
        xq + m0 * K + kb0 * 128, xs + m0 * KB + kb0, rows_a, wq + n0 * K + kb0 * 128,
        ws + (n0 / 128) * KB + kb0, rows_b, K, out, N, sm[0], nullptr, nullptr, nkb);
  else
    gemm_tile<WM, WN, FM, KS, true>(xq + m0 * K + kb0 * 128, xs + m0 * KB + kb0, KB, 1, rows_a,
                                    wq + n0 * K + kb0 * 128, ws + (n0 / 128) * KB + kb0, rows_b,
                                    K, out, N, sm[0], nkb);
}

// y[i] = bf16(sum over s = 0, 1, ... of part[s * slice_elems + i]), i < MN;
// slice_elems is a multiple of 4, so every slice is 16-byte aligned.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part,
                                                            int splits, int64_t slice_elems,
                                                            int64_t MN, uint16_t *__restrict__ y) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t n4 = MN / 4;
  // the first kBatch partials are loaded together (their latencies
  // overlap), then added in split order like any later ones
  constexpr int kBatch = 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    float4 p[kBatch];
#pragma unroll
    for (int sp = 0; sp < kBatch; ++sp)
      if (sp < splits) p[sp] = reinterpret_cast<const float4 *>(part + sp * slice_elems)[i];
    float4 a = p[0];
#pragma unroll
    for (int sp = 1; sp < kBatch; ++sp)
      if (sp < splits) {
        a.x += p[sp].x; a.y += p[sp].y; a.z += p[sp].z; a.w += p[sp].w;
      }
    for (int sp = kBatch; sp < splits; ++sp) {
      const float4 b = reinterpret_cast<const float4 *>(part + sp * slice_elems)[i];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    v2u o;
    o.x = bf16_rne(a.x) | (bf16_rne(a.y) << 16);
    o.y = bf16_rne(a.z) | (bf16_rne(a.w) << 16);
    __builtin_nontemporal_store(o, reinterpret_cast<v2u *>(y) + i);  // as the GEMM epilogue
  }
  for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += stride) {
    float a = part[i];
    for (int sp = 1; sp < splits; ++sp) a += part[sp * slice_elems + i];
    y[i] = (uint16_t)bf16_rne(a);
  }
}

// Stream-K tail of the 256x256 tiled GEMM (fp32 per-token-group scales).
// With T output tiles on kCUs compute units, T % kCUs tiles would run as a
// last, partly empty round.  Here the first t_dp = (T / kCUs) * kCUs tiles
// (in the tiled order: 8-row groups, XCD-aware) run whole as in
// block_gemm_kernel, and the remaining `rem` tiles' K blocks, rem * KB
// (tile, K block) steps taken in tile-major order, are cut into nsk equal
// contiguous ranges of L steps, one per extra workgroup.  A range covers
// the end of one tile and/or the start of the next (L <= KB): each piece is
// one gemm_tile over those K blocks, promoting every 128-long partial sum
// with its scale pair as always, and stores its unrounded fp32 sums to a
// workspace slot (256x256 fp32, tile-local rows).  The piece of tail tile s
// run by range w goes to slot w + s.  sk_reduce_kernel then adds each tail
// tile's pieces in K order and rounds once to bf16.
constexpr int kCUs = 256;  // MI355X compute units

template <int WM, int WN, int FM, bool kChunk = false>
__global__ __launch_bounds__(WM * WN * 64) void block_gemm_sk_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xs, const uint8_t *__restrict__ wq,
    const float *__restrict__ ws, int64_t M, int64_t N, int64_t K, uint16_t *__restrict__ y,
    float *__restrict__ part, int tiles_m, int tiles_n, int t_dp, int rem, int L) {
  using T = Tile<WM, WN, FM>;
  __shared__ typename T::Smem sm;
  const int64_t KB = K / 128;
  const int bid = blockIdx.x;
  int tm, tn;
  if (bid < t_dp) {
    group_coords(xcd_remap(bid, t_dp), tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * T::TM, n0 = (int64_t)tn * T::TN;
    gemm_tile<WM, WN, FM, 1, false, kChunk>(xq + m0 * K, xs + m0 * KB, KB, 1,
                                            (int)min<int64_t>(T::TM, M - m0), wq + n0 * K,
                                            ws + (n0 / 128) * KB,
                                            (int)min<int64_t>(T::TN, N - n0), K, y + m0 * N + n0,
                                            N, sm);
    return;
  }
  const int w = bid - t_dp;
  const int64_t i0 = (int64_t)w * L;
  const int64_t i1 = min<int64_t>(i0 + L, (int64_t)rem * KB);
  const int s0 = (int)(i0 / KB);
#pragma unroll 1
  for (int s = s0; s <= s0 + 1 && s < rem && (int64_t)s * KB < i1; ++s) {
    const int kb0 = (int)(max<int64_t>(i0, (int64_t)s * KB) - (int64_t)s * KB);
    const int kb1 = (int)(min<int64_t>(i1, (int64_t)(s + 1) * KB) - (int64_t)s * KB);
    if (s > s0) __syncthreads();  // the previous piece's last reads of LDS are done
    group_coords(t_dp + s, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * T::TM, n0 = (int64_t)tn * T::TN;
    float *slot = part + (int64_t)(w + s) * (T::TM * T::TN);
    gemm_tile<WM, WN, FM, 1, true>(
        xq + m0 * K + kb0 * 128, xs + m0 * KB + kb0, KB, 1, (int)min<int64_t>(T::TM, M - m0),
        wq + n0 * K + kb0 * 128, ws + (n0 / 128) * KB + kb0, (int)min<int64_t>(T::TN, N - n0), K,
        reinterpret_cast<uint16_t *>(slot), T::TN, sm, kb1 - kb0);
  }
}

// y over tail tile s = sum, in K order, of its pieces' slots (ranges
// floor(s*KB/L) .. floor(((s+1)*KB-1)/L), slot w + s), rounded once to
// bf16.  Workgroup (s, c) covers rows 4c .. 4c+3 of the tile: 256 threads,
// four columns each.
template <int TM, int TN>
__global__ __launch_bounds__(256) void sk_reduce_kernel(const float *__restrict__ part,
                                                        int64_t M, int64_t N, int64_t KB,
                                                        int tiles_m, int tiles_n, int t_dp,
                                                        int L, uint16_t *__restrict__ y) {
  static_assert(TN == 256, "one row of four columns per thread");
  const int s = blockIdx.x / (TM / 4);
  const int r = (blockIdx.x % (TM / 4)) * 4 + threadIdx.x / 64;
  const int c = (threadIdx.x % 64) * 4;
  int tm, tn;
  group_coords(t_dp + s, tiles_m, tiles_n, tm, tn);
  const int64_t row = (int64_t)tm * TM + r, col0 = (int64_t)tn * TN + c;
  if (row >= M) return;
  const int w0 = (int)(((int64_t)s * KB) / L), w1 = (int)(((int64_t)(s + 1) * KB - 1) / L);
  auto piece = [&](int w) {
    return reinterpret_cast<const float4 *>(part + (int64_t)(w + s) * (TM * TN) + r * TN + c)[0];
  };
  // the first kBatch pieces are loaded together (their latencies overlap),
  // then added in K order like any later ones
  constexpr int kBatch = 8;
  const int np = w1 - w0 + 1;
  float4 p[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i)
    if (i < np) p[i] = piece(w0 + i);
  float4 a = p[0];
#pragma unroll
  for (int i = 1; i < kBatch; ++i)
    if (i < np) {
      a.x += p[i].x; a.y += p[i].y; a.z += p[i].z; a.w += p[i].w;
    }
  for (int w = w0 + kBatch; w <= w1; ++w) {
    const float4 b = piece(w);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  if ((N & 3) == 0 && col0 + 3 < N) {
    // four whole columns of a row starting at a multiple of 4: one 8-byte
    // store (non-temporal, as the GEMM epilogue)
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    v2u o;
    o.x = bf16_rne(a.x) | (bf16_rne(a.y) << 16);
    o.y = bf16_rne(a.z) | (bf16_rne(a.w) << 16);
    __builtin_nontemporal_store(o, reinterpret_cast<v2u *>(y + row * N + col0));
    return;
  }
  const float v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (col0 + j < N) y[row * N + col0 + j] = (uint16_t)bf16_rne(v[j]);
}

// Grouped variant.  The logical m-tiles of all experts are numbered
// consecutively (expert e owns ceil(M_e/TM) of them); the grid is sized for
// the upper bound ceil(total_M/TM) + E, and workgroups past the real count
// exit at once.  Offsets are read on the device (no host sync) and clamped
// to [0, total_M].  Batched layout (capacity > 0): expert e owns rows
// [e*capacity, e*capacity + count[e]) with count[e] = offsets[e] clamped to
// [0, capacity]; its tiles are numbered directly (ceil(capacity/TM) per
// expert) and tiles past the count exit.
template <int WM, int WN, int FM, typename S, bool kChunk = false>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(
    const uint8_t *__restrict__ xq, const S *__restrict__ xs, int64_t xs_rs, int xs_ks,
    const uint8_t *__restrict__ wq, const S *__restrict__ ws,
    const int32_t *__restrict__ offsets, int E, int64_t total_M, int64_t N, int64_t K,
    uint16_t *__restrict__ y, int tiles_n, int64_t capacity) {
  using T = Tile<WM, WN, FM>;
  __shared__ typename TileSmem<WM, WN, FM, S>::type sm;
  const int tn = blockIdx.x % tiles_n;
  int mt = blockIdx.x / tiles_n;
  int64_t r0 = 0, r1 = 0;
  int e = 0;
  if (capacity > 0) {
    const int tpe = (int)((capacity + T::TM - 1) / T::TM);
    e = mt / tpe;
    if (e >= E) return;
    const int64_t lt = mt % tpe;
    int64_t c = offsets[e];
    c = c < 0 ? 0 : (c > capacity ? capacity : c);
    if (lt * T::TM >= c) return;
    r0 = (int64_t)e * capacity + lt * T::TM;
    r1 = (int64_t)e * capacity + c;
  } else {
    for (; e < E; ++e) {
      int64_t a = offsets[e], b = offsets[e + 1];
      a = a < 0 ? 0 : (a > total_M ? total_M : a);
      b = b < a ? a : (b > total_M ? total_M : b);
      const int cnt = (int)((b - a + T::TM - 1) / T::TM);
      if (mt < cnt) {
        r0 = a + (int64_t)mt * T::TM;
        r1 = b;
        break;
      }
      mt -= cnt;
    }
    if (e == E) return;
  }
  const int64_t n0 = (int64_t)tn * T::TN;
  const int64_t KB = K / 128;
  const int64_t NB = (N + 127) / 128;
  const uint8_t *wt = wq + (int64_t)e * N * K + n0 * K;
  const S *wst = ws + ((int64_t)e * NB + n0 / 128) * KB;
  const int rows_b = (int)min<int64_t>(T::TN, N - n0);
  if constexpr (FM % 2 == 0) {
    // a row tile with at most half its rows (an expert's ragged last tile)
    // runs the half-height tile: the same waves, half the A fragments each,
    // half the MFMA work
    using H = Tile<WM, WN, FM / 2>;
    if (r1 - r0 <= H::TM) {
      auto &smh = *reinterpret_cast<typename TileSmem<WM, WN, FM / 2, S>::type *>(&sm);
      static_assert(sizeof(typename TileSmem<WM, WN, FM / 2, S>::type) <= sizeof(sm), "LDS");
      run_tile<WM, WN, FM / 2, S>(xq + r0 * K, xs + r0 * xs_rs, xs_rs, xs_ks, (int)(r1 - r0), wt,
                                  wst, rows_b, K, y + r0 * N + n0, N, smh);
      return;
    }
  }
  run_tile<WM, WN, FM, S, kChunk>(xq + r0 * K, xs + r0 * xs_rs, xs_rs, xs_ks,
                                  (int)min<int64_t>(T::TM, r1 - r0), wt, wst, rows_b, K,
                                  y + r0 * N + n0, N, sm);
}

// The chunked activation-scale loads of gemm_tile apply: per-token-group
// scales (K-block stride 1) whose rows and K-block count are multiples of 4
// floats from a 16-byte aligned base, with K >= 4096.  In the bench step
// (same box, runs alternated): the six DeepSeek-V3 GEMMs 3398-3419 ->
// 3351-3381 us (q_a -4 %, MLP down -2.6 %, MLP up -1.7 %), the Llama four
// 577-578 -> 570 us; q_b (K = 1536, three chunks) ~1 % slower, hence the
// bound.
template <typename S>
static bool chunked_scales_ok(const S *xs, int64_t xs_rs, int xs_ks, int64_t K) {
  return std::is_same<S, float>::value && xs_ks == 1 && xs_rs % 4 == 0 && (K / 128) % 4 == 0 &&
         K / 128 >= 32 && (reinterpret_cast<uintptr_t>(xs) & 15) == 0;
}

template <int WM, int WN, int FM, typename S>
static hipError_t launch_tiled(const void *xq, const S *xs, int64_t xs_rs, int xs_ks,
                               const void *wq, const S *ws, int64_t M, int64_t N, int64_t K,
                               void *y, hipStream_t stream) {
  using T = Tile<WM, WN, FM>;
  const int tm = (int)((M + T::TM - 1) / T::TM), tn = (int)((N + T::TN - 1) / T::TN);
  if constexpr (T::TM == 256 && std::is_same<S, float>::value) {
    if (chunked_scales_ok(xs, xs_rs, xs_ks, K)) {
      hipLaunchKernelGGL((block_gemm_kernel<WM, WN, FM, S, true>), dim3((unsigned)(tm * tn)),
                         dim3(T::kThreads), 0, stream, static_cast<const uint8_t *>(xq), xs, xs_rs,
                         xs_ks, static_cast<const uint8_t *>(wq), ws, M, N, K,
                         static_cast<uint16_t *>(y), tm, tn);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((block_gemm_kernel<WM, WN, FM, S>), dim3((unsigned)(tm * tn)),
                     dim3(T::kThreads), 0, stream, static_cast<const uint8_t *>(xq), xs, xs_rs,
                     xs_ks, static_cast<const uint8_t *>(wq), ws, M, N, K,
                     static_cast<uint16_t *>(y), tm, tn);
  return hipGetLastError();
}

constexpr int64_t kKsMaxTiles = 256;

template <int WM, int WN, int FM, int KS, typename S, bool kRow = false>
static hipError_t launch_tiled_ks(const void *xq, const S *xs, int64_t xs_rs, int xs_ks,
                                  const void *wq, const S *ws, int64_t M, int64_t N, int64_t K,
                                  void *y, hipStream_t stream) {
  using T = Tile<WM, WN, FM>;
  const int tm = (int)((M + T::TM - 1) / T::TM), tn = (int)((N + T::TN - 1) / T::TN);
  hipLaunchKernelGGL((block_gemm_ks_kernel<WM, WN, FM, KS, S, kRow>), dim3((unsigned)(tm * tn)),
                     dim3(T::kThreads * KS), 0, stream, static_cast<const uint8_t *>(xq), xs, xs_rs,
                     xs_ks, static_cast<const uint8_t *>(wq), ws, M, N, K,
                     static_cast<uint16_t *>(y), tm, tn);
  return hipGetLastError();
}

// Configuration choice (both scale types): the decode kernel for M <= 64
// (fp32 scales: while its LDS scale staging fits; for 33-64 rows only below
// kDecWideN columns), 256x256 tiles when they fill the chip (>= 192
// tiles), 128x128 otherwise.  With four row fragments every decode
// workgroup reads four times its weight bytes of x, and for wide N the
// tiled kernel (rows padded to 128) wins: measured at M = 33-64, weights
// streamed from HBM, decode against tiled: 14336x4096 38.7-43.8 / 31.7-34.7
// us, 24576x1536 28.2-30.9 / 16.5-18.0, 18432x7168 73.6-101.3 / 52.9-57.3,
// 12288x4096 29.7-38.9 / 31.6-34.2; narrower shapes the other way
// (8192x4096 22.6-24.7 / 31.4-32.6, 8192x7168 30.9-36.1 / 49.9-54.4,
// 4096x4096 11.9-14.1 / 31.2-32.7).  E8M0 scales likewise: 14336x4096
// 45.2-61.1 / 28.4-30.0 us, 24576x1536 29.8-36.3 / 15.7-17.2, 18432x7168
// 77.0-101.6 / 46.1-49.3.
constexpr int64_t kDecWideN = 12288;

template <typename S>
static hipError_t dispatch_gemm(const void *xq, const S *xs, int64_t xs_rs, int xs_ks,
                                const void *wq, const S *ws, int64_t M, int64_t N, int64_t K,
                                void *y, hipStream_t stream) {
  if (M <= kDecMaxM && (M <= 32 || N < kDecWideN)) {
    const int MF = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    if (std::is_same<S, uint8_t>::value || (K / 128) * MF * 16 * 4 <= kDecMaxScaleBytes) {
      if (MF == 1) return launch_decode<1, S>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y, stream);
      if (MF == 2) return launch_decode<2, S>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y, stream);
      return launch_decode<4, S>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y, stream);
    }
  }
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles >= 192)
    return launch_tiled<2, 4, 8, S>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y, stream);
  // at most one 128x128 workgroup per CU: split K over two wave groups
  // (E8M0 scales: only for an even number of K blocks)
  const int64_t small_tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (small_tiles <= kKsMaxTiles && K >= 256 &&
      (std::is_same<S, float>::value || (K / 128) % 2 == 0))
    return launch_tiled_ks<2, 2, 4, 2, S>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y, stream);
  return launch_tiled<2, 2, 4, S>(xq, xs, xs_rs, xs_ks, wq, ws, M, N, K, y, stream);
}

// Split-K over workgroups (fp32 per-token-group scales), for grids of at
// most kSplitMaxTiles 128x128 tiles (at most half the CUs busy).  The split
// count S (2 .. min(256 / tiles, KB / kSplitMinKb)) maximises a time model
// fitted to measurements on MI355X (plain and split times of seven shapes
// with M = 128..1024, K = 2048..7168): the plain kernel spends ~0.85 us per
// step of two K blocks, so S ranges save 0.85 (KB/2)(1 - 1/S) us, and the
// split costs ~4.2 us more of fixed overhead (second launch, prologue and
// tail) plus its traffic (S*M*N fp32 written and read, M*N bf16 written,
// mostly in cache) at ~10 TB/s.  No split unless the model gains more than
// 2 us.  Measured: q_a 512x1536x7168 41.2 -> 21.2 us, kv_a 512x576x7168
// 30.5 -> 18.7 us, 1024x1024x4096 25.3 -> 19.3 us; 256x7168x2048 (12.6 ->
// 19.6) and 300x576x2048 (12.5 -> 13.2) are slower split and stay whole.
//
// fp32 scales with 33-64 rows and K >= kSplitSmallMMinK take this split
// (one padded row tile) instead of the decode kernel: measured at M =
// 33-64, weights streamed from HBM, decode against the split: 4096x14336
// 28.1-39.2 / 23.1-25.0 us, 1536x7168 16.4-21.3 / 14.5-15.8, 576x7168
// 15.5-20.0 / 12.7-13.8, 7168x16384 60.9-70.5 / 39.8-43.5, 7168x18432
// (whose scales do not fit the decode kernel: the plain tiled kernel)
// 118.8-130.3 / 42.0-45.4; at K = 4096 the decode kernel is as fast or
// faster (4096x4096 11.9-14.1 / 14.9-16.6, 1024x4096 11.4-12.9 /
// 11.3-12.4).
constexpr int64_t kSplitMaxTiles = 128;
constexpr int kSplitMinKb = 4;
constexpr int64_t kSplitSmallMMinK = 6144;

// even: every range a multiple of 2 K blocks (the E8M0 tile's two wave
// groups cannot sit a step out), hence K/128 even too.
static int splitk_plan(int64_t M, int64_t N, int64_t K, int &kb_per, int64_t &slice_elems,
                       bool even = false) {
  // (also called before argument validation: sizes past the library's
  // limits are simply not split)
  if (M <= (even ? kDecMaxM : 32) || N <= 0 || K <= 0) return 0;
  if (!even && M <= kDecMaxM && K < kSplitSmallMMinK) return 0;
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 24)) return 0;
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (tiles > kSplitMaxTiles) return 0;
  const int64_t KB = K / 128;
  const int64_t smax = std::min<int64_t>(256 / tiles, KB / kSplitMinKb);
  const double mn = (double)M * (double)N;
  int64_t best = 0;
  double best_gain = 2.0;  // us
  for (int64_t sp = 2; sp <= smax; ++sp) {
    const double saved = 0.85 * 0.5 * (double)KB * (1.0 - 1.0 / (double)sp);
    const double cost = 4.2 + ((double)sp * mn * 8.0 + mn * 2.0) / 1.0e7;
    if (saved - cost > best_gain) {
      best_gain = saved - cost;
      best = sp;
    }
  }
  if (best < 2 || (even && KB % 2 != 0)) return 0;
  kb_per = (int)((KB + best - 1) / best);
  if (even) kb_per += kb_per & 1;
  const int splits = (int)((KB + kb_per - 1) / kb_per);
  slice_elems = (M * N + 3) / 4 * 4;
  return splits >= 2 ? splits : 0;
}

// Decode (9 <= M <= 16, fp32 scales) with long K and few columns: four
// 16-column slabs per workgroup read x once per 64 output columns instead of
// once per 16, and the K blocks are split over gridDim.y so that the grid
// still fills the chip.  Used where one to two slabs per workgroup would
// otherwise be needed to fill it (decode_slabs < 4), with at least 16 K
// blocks per split (one per wave) and at least 192 workgroups.  Partial sums
// as in the tiled split (fp32, reduced in split order by
// splitk_reduce_kernel).  Measured on MI355X, 4096 x 14336 weights streamed
// from HBM: M = 16 17.7 -> 15.6 us; at M = 1 and 4 the x reads saved
// (1/16 and 1/4 of the weight bytes) are worth less than the second launch
// (13.7 -> 15.1, 14.3 -> 15.4 us), hence M > 8.
constexpr int kDecSplitMinKb = kDecWaves;

static int decode_split_plan(int64_t M, int64_t N, int64_t K, int &kb_per,
                             int64_t &slice_elems) {
  if (M <= 8 || M > 16 || N <= 0 || K <= 0) return 0;
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 24)) return 0;
  const int64_t KB = K / 128;
  if (KB * 16 * 4 > kDecMaxScaleBytes) return 0;  // as the unsplit decode path
  if (decode_slabs(N, 4) == 4) return 0;          // four slabs already fill the chip
  const int64_t groups = ((N + 15) / 16 + 3) / 4;
  const int64_t sp = std::min<int64_t>(256 / groups, KB / kDecSplitMinKb);
  if (sp < 2 || groups * sp < 192) return 0;
  kb_per = (int)((KB + sp - 1) / sp);
  const int splits = (int)((KB + kb_per - 1) / kb_per);
  slice_elems = (M * N + 3) / 4 * 4;
  return splits >= 2 ? splits : 0;
}

// The split plan of either kind; dec = true for the decode kernel's.
template <typename S>
static int any_split_plan(int64_t M, int64_t N, int64_t K, int &kb_per, int64_t &slice_elems,
                          bool &dec) {
  dec = false;
  if constexpr (std::is_same<S, float>::value) {
    if (M <= 16) {
      dec = true;
      return decode_split_plan(M, N, K, kb_per, slice_elems);
    }
  }
  return splitk_plan(M, N, K, kb_per, slice_elems, std::is_same<S, uint8_t>::value);
}

// Stream-K tail plan (fp32 scales, the 256x256 tiled path).  A time model
// fitted to measurements on MI355X: a K step of the 256x256 tile takes
// ~1.9 us, so the tail saves (KB - L) steps; the pieces' fp32 sums cost
// their traffic (written, then read by the reduction) at ~4 TB/s plus ~4 us
// for the second launch.  Used only when the model gains more than 8 us
// (DeepSeek-V3 o_proj and MLP down at M = 8192: 3.5 rounds of tiles, the
// last half-empty; a short-K tail such as Llama gate/up's gains nothing).
//
// Grids of fewer than 192 256x256 tiles run the 128x128 kernels; with long
// K (at least 56 blocks), at least 32 such tiles and more than
// kSplitMaxTiles 128x128 tiles (past the split over workgroups), the whole
// grid runs as stream-K on 256x256 tiles (no data-parallel part) when the
// same model of it beats an estimate of the 128x128 kernel by 10 %: ~0.9
// us per K block with one tile per CU (split K inside the workgroup, at
// most 256 tiles), ~1.46 us per K block and round of 512 tiles (two per
// CU) beyond.  The estimates fit measurements on MI355X within ~20 %, and
// the rule took every measured case the faster way but for a few small
// gains forgone; measured (random codes, one launch at a time) DeepSeek-V3
// at M = 512 o_proj 7168x16384 116 -> 98 us, MLP up 18432x7168 139 -> 117,
// MLP down 7168x18432 132 -> 101; at M = 768-1536 o_proj 160-280 ->
// 124-205, MLP down 175-329 -> 126-263, Llama down 4096x14336 101-134 ->
// 72-111; short K (K = 4096 and below) and MLP up at M = 384 (one round of
// 432 128x128 tiles: 82 us against 99) stay on the 128x128 kernels.
constexpr int64_t kSkSmallMinTiles = 32;
constexpr int64_t kSkSmallMinKb = 56;

struct SkPlan {
  int t_dp = 0, rem = 0, L = 0, nsk = 0;
  size_t bytes = 0;
};

static bool sk_plan(int64_t M, int64_t N, int64_t K, SkPlan &p) {
  // (also called before argument validation: sizes past the library's
  // limits are simply not split)
  if (M <= kDecMaxM || N <= 0 || K <= 0) return false;
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 24)) return false;
  using T = Tile<2, 4, 8>;
  const int64_t tiles = ((M + T::TM - 1) / T::TM) * ((N + T::TN - 1) / T::TN);
  if (tiles > (int64_t(1) << 24)) return false;
  const int64_t KB = K / 128;
  const bool small = tiles < 192;  // below the 256x256 path's threshold
  if (small) {
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles < kSkSmallMinTiles || KB < kSkSmallMinKb || t128 <= kSplitMaxTiles) return false;
  }
  const int64_t rem = tiles % kCUs;
  if (rem == 0) return false;
  const int64_t L = (rem * KB + kCUs - 1) / kCUs;
  const int64_t nsk = (rem * KB + L - 1) / L;
  const int64_t pieces = nsk + rem;  // upper bound (and the slot count)
  const double cost = 4.0 + 2.0 * (double)pieces * (double)(T::TM * T::TN * 4) / 4.0e6;
  if (small) {
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const double cur = t128 <= kKsMaxTiles
                           ? 0.9 * (double)KB
                           : 1.46 * (double)KB * (double)((t128 + 2 * kCUs - 1) / (2 * kCUs));
    if (1.9 * (double)L + cost > 0.9 * cur) return false;
  } else {
    const double saved = 1.9 * (double)(KB - L);
    if (saved - cost <= 8.0) return false;
  }
  p.t_dp = (int)(tiles - rem);
  p.rem = (int)rem;
  p.L = (int)L;
  p.nsk = (int)nsk;
  p.bytes = (size_t)pieces * (size_t)(T::TM * T::TN) * sizeof(float);
  return true;
}

template <typename S>
static size_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  int kb_per = 0;
  int64_t slice = 0;
  bool dec = false;
  const int splits = any_split_plan<S>(M, N, K, kb_per, slice, dec);
  return splits ? (size_t)splits * (size_t)slice * sizeof(float) : 0;
}

size_t block_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  SkPlan sk;
  if (sk_plan(M, N, K, sk)) return sk.bytes;
  return splitk_workspace_bytes<float>(M, N, K);
}

size_t block_gemm_split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return splitk_workspace_bytes<float>(M, N, K);
}
size_t block_gemm_e8m0_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return splitk_workspace_bytes<uint8_t>(M, N, K);
}

template <typename S>
static hipError_t launch_splitk(const void *xq, const S *xs, const void *wq, const S *ws,
                                int64_t M, int64_t N, int64_t K, void *y, void *work,
                                size_t work_bytes, hipStream_t stream, bool allow_sk = true) {
  if constexpr (std::is_same<S, float>::value) {
    SkPlan sk;
    if (allow_sk && sk_plan(M, N, K, sk)) {
      if (work == nullptr || work_bytes < sk.bytes)
        return launch_block_gemm(xq, xs, wq, ws, M, N, K, y, stream);
      using T = Tile<2, 4, 8>;
      const int tm = (int)((M + T::TM - 1) / T::TM), tn = (int)((N + T::TN - 1) / T::TN);
      float *part = static_cast<float *>(work);
      if (chunked_scales_ok(xs, K / 128, 1, K))
        hipLaunchKernelGGL((block_gemm_sk_kernel<2, 4, 8, true>),
                           dim3((unsigned)(sk.t_dp + sk.nsk)), dim3(T::kThreads), 0, stream,
                           static_cast<const uint8_t *>(xq), xs, static_cast<const uint8_t *>(wq),
                           ws, M, N, K, static_cast<uint16_t *>(y), part, tm, tn, sk.t_dp,
                           sk.rem, sk.L);
      else
        hipLaunchKernelGGL((block_gemm_sk_kernel<2, 4, 8>), dim3((unsigned)(sk.t_dp + sk.nsk)),
                           dim3(T::kThreads), 0, stream, static_cast<const uint8_t *>(xq), xs,
                           static_cast<const uint8_t *>(wq), ws, M, N, K,
                           static_cast<uint16_t *>(y), part, tm, tn, sk.t_dp, sk.rem, sk.L);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((sk_reduce_kernel<T::TM, T::TN>), dim3((unsigned)(sk.rem * (T::TM / 4))),
                         dim3(256), 0, stream, part, M, N, K / 128, tm, tn, sk.t_dp, sk.L,
                         static_cast<uint16_t *>(y));
      return hipGetLastError();
    }
  }
  int kb_per = 0;
  int64_t slice = 0;
  bool dec = false;
  const int splits = any_split_plan<S>(M, N, K, kb_per, slice, dec);
  if (splits == 0 || work == nullptr ||
      work_bytes < (size_t)splits * (size_t)slice * sizeof(float)) {
    if constexpr (std::is_same<S, uint8_t>::value)
      return launch_block_gemm_e8m0(xq, xs, wq, ws, M, N, K, y, stream);
    else
      return launch_block_gemm(xq, xs, wq, ws, M, N, K, y, stream);
  }
  float *part = static_cast<float *>(work);
  if constexpr (std::is_same<S, float>::value) {
    if (dec) {
      const int64_t groups = ((N + 15) / 16 + 3) / 4;
      const size_t lds =
          std::max((size_t)kb_per * 16 * 4, (size_t)kDecWaves * 4 * 64 * sizeof(v4f));
      hipLaunchKernelGGL((decode_gemm_kernel<1, float, false, 4, true>),
                         dim3((unsigned)groups, (unsigned)splits), dim3(kDecThreads), lds, stream,
                         static_cast<const uint8_t *>(xq), xs, K / 128, 1,
                         static_cast<const uint8_t *>(wq), ws, (int)M, N, K, nullptr, part, slice,
                         kb_per);
    }
  }
  if (!dec) {
    using T = Tile<2, 2, 4>;
    const int tm = (int)((M + T::TM - 1) / T::TM), tn = (int)((N + T::TN - 1) / T::TN);
    hipLaunchKernelGGL((block_gemm_splitk_kernel<2, 2, 4, 2, S>),
                       dim3((unsigned)(tm * tn * splits)), dim3(T::kThreads * 2), 0, stream,
                       static_cast<const uint8_t *>(xq), xs, static_cast<const uint8_t *>(wq), ws,
                       M, N, K, part, slice, tm, tn, kb_per);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n4 = std::max<int64_t>(M * N / 4, 1);
  const unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 256 * 8);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(256), 0, stream, part, splits, slice,
                     M * N, static_cast<uint16_t *>(y));
  return hipGetLastError();
}

hipError_t launch_block_gemm_ws(const void *xq, const float *xs, const void *wq, const float *ws,
                                int64_t M, int64_t N, int64_t K, void *y, void *work,
                                size_t work_bytes, hipStream_t stream) {
  return launch_splitk<float>(xq, xs, wq, ws, M, N, K, y, work, work_bytes, stream);
}

// Device scratch for the K split of fp8_block_gemm_noalloc (callers that
// cannot allocate: graph capture, tight serving loops).  One copy per GPU,
// held until the process ends.  Its size covers every split plan: a tiled
// plan has at most 128 tiles of 128x128 and at most 256 / tiles ranges
// (<= 256 * 128 * 128 fp32 = 16 MiB, plus the rounding of slices to 4
// elements), a decode plan at most 1 MiB.  In host code `scratch` only
// names the symbol; its device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void *g_scratch_addr[kScratchMaxDevices];

hipError_t scratch_address(void **addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_block_gemm_noalloc(const void *xq, const float *xs, const void *wq,
                                     const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                                     hipStream_t stream) {
  // the K splits over workgroups only: a stream-K tail's slots (tens of MB)
  // are not held in the scratch, and such shapes run unsplit
  if (block_gemm_split_workspace_bytes(M, N, K) == 0)
    return launch_block_gemm(xq, xs, wq, ws, M, N, K, y, stream);
  void *p = nullptr;
  hipError_t e = scratch_address(&p);
  if (e != hipSuccess) return e;
  return launch_splitk<float>(xq, xs, wq, ws, M, N, K, y, p, kScratchBytes, stream, false);
}

hipError_t launch_block_gemm_e8m0_ws(const void *xq, const uint8_t *xs, const void *wq,
                                     const uint8_t *ws, int64_t M, int64_t N, int64_t K, void *y,
                                     void *work, size_t work_bytes, hipStream_t stream) {
  return launch_splitk<uint8_t>(xq, xs, wq, ws, M, N, K, y, work, work_bytes, stream);
}

template <typename S>
static hipError_t dispatch_grouped(const void *xq, const S *xs, const void *wq, const S *ws,
                                   const int32_t *offsets, int32_t E, int64_t total_M, int64_t N,
                                   int64_t K, void *y, hipStream_t stream, int64_t capacity = 0) {
  using T = Tile<2, 4, 8>;
  const int64_t tiles_n = (N + T::TN - 1) / T::TN;
  const int64_t tiles_m = capacity > 0 ? (int64_t)E * ((capacity + T::TM - 1) / T::TM)
                                       : (total_M + T::TM - 1) / T::TM + E;
  // full row tiles load the activation scales four K blocks at a time where
  // that applies (any row offset keeps the 16-byte alignment when K / 128
  // is a multiple of 4)
  if constexpr (std::is_same<S, float>::value) {
    if (chunked_scales_ok(xs, K / 128, 1, K)) {
      hipLaunchKernelGGL((grouped_gemm_kernel<2, 4, 8, S, true>),
                         dim3((unsigned)(tiles_m * tiles_n)), dim3(T::kThreads), 0, stream,
                         static_cast<const uint8_t *>(xq), xs, K / 128, 1,
                         static_cast<const uint8_t *>(wq), ws, offsets, (int)E, total_M, N, K,
                         static_cast<uint16_t *>(y), (int)tiles_n, capacity);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<2, 4, 8, S>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(T::kThreads), 0, stream, static_cast<const uint8_t *>(xq), xs, K / 128,
                     1, static_cast<const uint8_t *>(wq), ws, offsets, (int)E, total_M, N, K,
                     static_cast<uint16_t *>(y), (int)tiles_n, capacity);
  return hipGetLastError();
}

hipError_t launch_block_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                             int64_t M, int64_t N, int64_t K, void *y, hipStream_t stream) {
  return dispatch_gemm<float>(xq, xs, K / 128, 1, wq, ws, M, N, K, y, stream);
}

hipError_t launch_block_gemm_static(const void *xq, const float *xs, const void *wq,
                                    const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                                    hipStream_t stream) {
  return dispatch_gemm<float>(xq, xs, 0, 0, wq, ws, M, N, K, y, stream);
}

hipError_t launch_block_gemm_e8m0(const void *xq, const uint8_t *xs, const void *wq,
                                  const uint8_t *ws, int64_t M, int64_t N, int64_t K, void *y,
                                  hipStream_t stream) {
  return dispatch_gemm<uint8_t>(xq, xs, K / 128, 1, wq, ws, M, N, K, y, stream);
}

hipError_t launch_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *offsets, int32_t E, int64_t total_M, int64_t N,
                               int64_t K, void *y, hipStream_t stream) {
  return dispatch_grouped<float>(xq, xs, wq, ws, offsets, E, total_M, N, K, y, stream);
}

hipError_t launch_grouped_gemm_e8m0(const void *xq, const uint8_t *xs, const void *wq,
                                    const uint8_t *ws, const int32_t *offsets, int32_t E,
                                    int64_t total_M, int64_t N, int64_t K, void *y,
                                    hipStream_t stream) {
  return dispatch_grouped<uint8_t>(xq, xs, wq, ws, offsets, E, total_M, N, K, y, stream);
}

// Row-wise scales: the E8M0 tile's loop without scales (unscaled MFMAs
// accumulating over all of K), xs[M] and ws[N] applied in the epilogue.
template <int WM, int WN, int FM>
__global__ __launch_bounds__(WM * WN * 64) void rowwise_gemm_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xs, const uint8_t *__restrict__ wq,
    const float *__restrict__ ws, int64_t M, int64_t N, int64_t K, uint16_t *__restrict__ y,
    int tiles_m, int tiles_n) {
  using T = Tile<WM, WN, FM>;
  __shared__ typename T::SmemMx sm;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * T::TM, n0 = (int64_t)tn * T::TN;
  gemm_tile_mx<WM, WN, FM, (FM <= 4), false>(xq + m0 * K, nullptr, (int)min<int64_t>(T::TM, M - m0),
                                             wq + n0 * K, nullptr, (int)min<int64_t>(T::TN, N - n0),
                                             K, y + m0 * N + n0, N, sm, xs + m0, ws + n0);
}

template <int WM, int WN, int FM>
static hipError_t launch_rowwise_tiled(const void *xq, const float *xs, const void *wq,
                                       const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                                       hipStream_t stream) {
  using T = Tile<WM, WN, FM>;
  const int tm = (int)((M + T::TM - 1) / T::TM), tn = (int)((N + T::TN - 1) / T::TN);
  hipLaunchKernelGGL((rowwise_gemm_kernel<WM, WN, FM>), dim3((unsigned)(tm * tn)),
                     dim3(T::kThreads), 0, stream, static_cast<const uint8_t *>(xq), xs,
                     static_cast<const uint8_t *>(wq), ws, M, N, K, static_cast<uint16_t *>(y),
                     tm, tn);
  return hipGetLastError();
}

hipError_t launch_rowwise_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               int64_t M, int64_t N, int64_t K, void *y, hipStream_t stream) {
  if (M <= kDecMaxM) {
    const int MF = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    if (MF == 1) return launch_decode<1, float, true>(xq, xs, 1, 0, wq, ws, M, N, K, y, stream);
    if (MF == 2) return launch_decode<2, float, true>(xq, xs, 1, 0, wq, ws, M, N, K, y, stream);
    return launch_decode<4, float, true>(xq, xs, 1, 0, wq, ws, M, N, K, y, stream);
  }
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles >= 192) return launch_rowwise_tiled<2, 4, 8>(xq, xs, wq, ws, M, N, K, y, stream);
  const int64_t small_tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (small_tiles <= kKsMaxTiles && K >= 256 && (K / 128) % 2 == 0)
    return launch_tiled_ks<2, 2, 4, 2, float, true>(xq, xs, 0, 0, wq, ws, M, N, K, y, stream);
  return launch_rowwise_tiled<2, 2, 4>(xq, xs, wq, ws, M, N, K, y, stream);
}

hipError_t launch_batched_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *counts, int32_t E, int64_t capacity, int64_t N,
                               int64_t K, void *y, hipStream_t stream) {
  return dispatch_grouped<float>(xq, xs, wq, ws, counts, E, (int64_t)E * capacity, N, K, y,
                                 stream, capacity);
}

}  // namespace fp8blk
