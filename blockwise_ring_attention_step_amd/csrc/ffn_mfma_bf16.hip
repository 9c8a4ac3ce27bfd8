// Blockwise feed-forward for gfx950 (CDNA4): the two projections of the position-wise feed-forward
// that the blockwise method computes after attention (cyberairomania.ro, "Context parallelism",
// section on Ring Attention: attention and the feed-forward are both computed block by block),
//   h = act(x W1^T + b1)   (bf16, one token block at a time),   y = h W2^T + b2,
// each a bf16 GEMM on v_mfma_f32_32x32x16_bf16 with the bias, the activation and the rounding fused
// into the epilogue:
//   out[m, n] = epi(sum_k a[m, k] w[n, k] + bias[n]),
// a [M, K] (tokens x features, row-major), w [N, K] (the weight in nn.Linear layout: one row per
// output feature), both read along k.
//
// A workgroup of 4 waves (one per SIMD, 256 accumulator registers each for 256 x 256 tiles) owns
// BM x BN output tiles, one after the other (persistent: one workgroup per CU, or two with the
// 128 x 128 tiles taken when the large ones would leave CUs idle); each wave a (BM/2) x (BN/2) quarter as
// (BN/64) x (BM/64) accumulators of 32 x 32, held transposed (the lane is the token m, the register
// the feature n, so that 4 consecutive features leave as one 8-byte store).  k advances in steps of
// BK: the a and w rows of a step go HBM -> LDS directly (global_load_lds) into a ring of S buffers.
// The steps of all of a workgroup's tiles form one stream: step s+S is requested into the buffer
// of step s as soon as every wave has read it (one workgroup barrier per step), so S-1 steps are in
// flight while one is multiplied, across tile boundaries too (the next tile's first steps load
// while the current tile's epilogue runs).  Within a step, the LDS fragments of k slice kk+1 are
// read while the products of slice kk run.  Tiles are numbered so that each XCD (workgroup id
// mod 8) sweeps a contiguous range of them, GM m-tiles at a time, so the rows that neighbouring
// workgroups share stay in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "gfx950_tile.h"
#include "internal.h"

namespace ra {
namespace {

using namespace tile;

constexpr int kFfnWaves = 4;
constexpr int kFfnThreads = 64 * kFfnWaves;
constexpr int kFfnGroupM = 4;  // m-tiles per sweep of the n-tiles
// BM x BN output tiles, k steps of BK, S LDS buffers (2 x 64 KiB of the 160 KiB).  Deeper rings of
// shorter steps (BK 32 with 4 or 5 buffers) measured no faster: the rate at which one CU pulls rows
// from L2, not the latency, bounds these loads.
constexpr int kFfnBM = 256, kFfnBN = 256, kFfnBK = 64, kFfnStages = 2;

// Phi(z), the standard normal CDF, from the Chebyshev fit of erfc in Numerical Recipes (Press et al.,
// section 6.2, "erfcc"): erfc(x) = t exp(-x^2 + P(t)), t = 1 / (1 + x/2), x >= 0, with fractional
// error below 1.2e-7 everywhere, the far tails included.  Phi(z) = erfc(-z / sqrt 2) / 2.
__device__ __forceinline__ float normal_cdf(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, x, 1.f));
  float q = 0.17087277f;
  q = __builtin_fmaf(q, t, -0.82215223f);
  q = __builtin_fmaf(q, t, 1.48851587f);
  q = __builtin_fmaf(q, t, -1.13520398f);
  q = __builtin_fmaf(q, t, 0.27886807f);
  q = __builtin_fmaf(q, t, -0.18628806f);
  q = __builtin_fmaf(q, t, 0.09678418f);
  q = __builtin_fmaf(q, t, 0.37409196f);
  q = __builtin_fmaf(q, t, 1.00002368f);
  q = __builtin_fmaf(q, t, -1.26551223f);
  const float e = t * __builtin_amdgcn_exp2f(__builtin_fmaf(-x, x, q) * kLog2e);  // erfc(x)
  return z >= 0.f ? __builtin_fmaf(-0.5f, e, 1.f) : 0.5f * e;
}

template <int ACT>
__device__ __forceinline__ float activate(float z) {
  if constexpr (ACT == RA_FFN_GELU) return z * normal_cdf(z);
  if constexpr (ACT == RA_FFN_RELU) return fmaxf(z, 0.f);
  return z;
}

template <int BM, int BN, int BK, int S, int ACT, int OCC>
__global__ __launch_bounds__(kFfnThreads, OCC) void ffn_gemm_bf16(const FfnGemmParams p) {
  constexpr int R = BK * 2;                  // bytes of one row of a step
  constexpr int C = R / 16;                  // 16-byte chunks per row
  constexpr int RPP = 1024 / R;              // rows per 1 KiB copy
  constexpr int KK = BK / 16;                // k slices of one product per step
  constexpr int kTileA = BM * R;
  constexpr int kStage = (BM + BN) * R;
  constexpr int kPieces = (BM + BN) / RPP / kFfnWaves;  // 1 KiB copies per wave per step
  constexpr int MB = BM / 64, NB = BN / 64;             // 32 x 32 blocks per wave along m and n
  static_assert(R == 64 || R == 128, "step rows of 64 or 128 bytes");
  static_assert(KK % 2 == 0, "fragment double buffer alternates per k slice");
  static_assert(kPieces * kFfnWaves * RPP == BM + BN, "tile rows split evenly over the waves");
  static_assert((S - 1) * kPieces < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * kStage];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  // LDS layout of a step tile: 16-byte chunk c of row r is stored at chunk c ^ swz(r), so that the 16
  // lanes of a row read (16 consecutive rows, one chunk) cover the 16 bank groups of 256 bytes
  auto swz = [](int r) { return (r / (256 / R)) % C; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31, h2 = lane >> 5;

  const int T = p.tiles_m * p.tiles_n;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int nt = (T - b + G - 1) / G;  // tiles of this workgroup: virtual indices b, b + G, ...
  const int KT = p.K / BK;
  const int NS = nt * KT;
  // tile origin of this workgroup's i-th tile; every XCD owns a contiguous range of tiles
  auto tile_of = [&](int i, int& m0, int& n0) {
    const int u = i * G + b;
    const int xcd = u & 7, slot = u >> 3;
    const int t = xcd * (T >> 3) + min(xcd, T & 7) + slot;
    const int sweep = t / (kFfnGroupM * p.tiles_n);
    const int first_m = sweep * kFfnGroupM;
    const int gsize = min(p.tiles_m - first_m, kFfnGroupM);
    const int within = t - sweep * kFfnGroupM * p.tiles_n;
    m0 = (first_m + within % gsize) * BM;
    n0 = (within / gsize) * BN;
  };

  // requests: piece q (0 .. (BM+BN)/RPP) holds tile rows RPP q .. + RPP-1 (a rows, then w rows);
  // lane l copies row RPP q + l / C, chunk (l % C) ^ swz(row) of the source to LDS chunk l % C.
  // Rows past the end of a and w re-read the last row.
  const char* xa = nullptr;
  const char* wa = nullptr;
  uint32_t voff[kPieces];
  int rq_tile = 0, rq_kt = 0;
  auto setup_request_tile = [&](int i) {
    int m0, n0;
    tile_of(i, m0, n0);
    xa = (const char*)p.x + (int64_t)m0 * p.ldx * 2;
    wa = (const char*)p.w + (int64_t)n0 * p.ldw * 2;
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int q = wave + kFfnWaves * k;
      const int row = RPP * q + lane / C;
      const int chunk = ((lane % C) ^ swz(row)) * 16;
      if (RPP * q < BM) {
        voff[k] = (uint32_t)(min(row, p.M - 1 - m0) * p.ldx * 2) + chunk;
      } else {
        voff[k] = (uint32_t)(min(row - BM, p.N - 1 - n0) * p.ldw * 2) + chunk;
      }
    }
  };
  // piece k of the requested step into buffer buf; then move the request on by one step
  auto issue_piece = [&](int k, int buf) {
    const int q = wave + kFfnWaves * k;
    const bool is_a = kFfnWaves * k < BM / RPP;  // the same for every wave (wave < 4, BM/RPP % 4 == 0)
    copy_to_lds16((is_a ? xa : wa) + rq_kt * R, voff[k], (uint32_t)(uintptr_t)(smem + buf * kStage) + q * 1024);
  };
  auto advance_request = [&]() {
    if (++rq_kt == KT) {
      rq_kt = 0;
      if (++rq_tile < nt) setup_request_tile(rq_tile);  // past the end: the last tile again
    }
  };

  // operand reads: lane reads row j of a 32-row block, chunk 2 kk + h2 (k = 16 kk + 8 h2 .. + 7)
  int roff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) roff[kk] = j * R + (((2 * kk + h2) ^ swz(j)) * 16);
  const int wn = wave >> 1, wm = wave & 1;
  const int a_row0 = wm * (BM / 2), w_row0 = kTileA / R + wn * (BN / 2);

  f32x16 acc[NB][MB];
  bf16x8 wf[2][NB], xf[2][MB];  // fragments of two k slices
  // fragment r of k slice kk (r < NB: w rows of block r; else x rows of block r - NB) into `set`
  auto read_one = [&](int buf, int kk, int set, int r) {
    const LDS_AS char* base = smem + buf * kStage + roff[kk];
    if (r < NB)
      wf[set][r] = __builtin_bit_cast(bf16x8, *(const LDS_AS i16x8*)(base + (w_row0 + 32 * r) * R));
    else
      xf[set][r - NB] = __builtin_bit_cast(bf16x8, *(const LDS_AS i16x8*)(base + (a_row0 + 32 * (r - NB)) * R));
  };
  auto mfma_one = [&](int set, int i) {
    const int bn = i / MB, bm = i % MB;
    acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[set][bn], xf[set][bm], acc[bn][bm], 0, 0, 0);
  };

  // epilogue of the tile at (m0, n0): register 4 g + e of block (bn, bm) is feature
  // n = n0 + wn BN/2 + 32 bn + 8 g + 4 h2 + e of token m = m0 + wm BM/2 + 32 bm + j
  const unsigned short* bias = (const unsigned short*)p.bias;
  unsigned short* out = (unsigned short*)p.out;
  auto epilogue = [&](int m0, int n0) {
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) {
      const int nb = n0 + wn * (BN / 2) + 32 * bn + 4 * h2;
      u16x4 bv[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nb + 8 * g;
        bv[g] = n < p.N ? *(const u16x4*)(bias + n) : u16x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int bm = 0; bm < MB; ++bm) {
        const int m = m0 + wm * (BM / 2) + 32 * bm + j;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = nb + 8 * g;
          u16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc[bn][bm][4 * g + e] + __uint_as_float((uint32_t)bv[g][e] << 16);
            o[e] = __builtin_bit_cast(unsigned short, (__bf16)activate<ACT>(z));
          }
          if (m < p.M && n < p.N) *(u16x4*)(out + (int64_t)m * p.ldo + n) = o;
        }
      }
    }
  };

  // One step: KK slices of NB x MB products.  Each product is followed by one slot of other work, in
  // this order (sched_barrier keeps it): while slice kk multiplies, the fragments of slice kk+1 are
  // read; the last slice first meets the other waves at the barrier (step s+1 landed, step s read by
  // all), then reads step s+1's first fragments and requests step s+S into the freed buffer, so that
  // the matrix cores keep running across the barrier and the copies.  Near the end of the stream the
  // same schedule runs on: requests past the last step fetch the last tile's rows again into buffers
  // that no step reads, and the fragments read for a step past the last one are not used.
  constexpr int kProducts = NB * MB;
  constexpr int kReads = NB + MB;
  static_assert(kProducts >= 4, "slots for the barrier, reads and copies");
  auto step = [&](int s) {
    const int buf = s % S;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int set = kk & 1;
#pragma unroll
      for (int i = 0; i < kProducts; ++i) {
        mfma_one(set, i);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < KK) {
#pragma unroll
          for (int r = 0; r < kReads; ++r)
            if (r % kProducts == i) read_one(buf, kk + 1, set ^ 1, r);
        } else if (i == 0) {
          wait_vmem<(S - 2) * kPieces>();  // step s+1 has landed (this wave's copies)
          __syncthreads();                 // ... every wave's, and every wave has read all of step s
        } else {
#pragma unroll
          for (int r = 0; r < kReads; ++r)
            if (1 + r % (kProducts - 1) == i) read_one((s + 1) % S, 0, 0, r);
#pragma unroll
          for (int k = 0; k < kPieces; ++k)
            if (1 + k * (kProducts - 1) / kPieces == i) issue_piece(k, buf);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    advance_request();
  };

  if (NS == 0) return;
  setup_request_tile(0);
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int k = 0; k < kPieces; ++k) issue_piece(k, s);
    advance_request();
  }
  wait_vmem<(S - 1) * kPieces>();  // steps 1 .. S-1 may still fly
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kReads; ++r) read_one(0, 0, 0, r);
  for (int ti = 0; ti < nt; ++ti) {
#pragma unroll
    for (int bn = 0; bn < NB; ++bn)
#pragma unroll
      for (int bm = 0; bm < MB; ++bm) acc[bn][bm] = f32x16{};
    for (int kt = 0; kt < KT; ++kt) step(ti * KT + kt);
    int m0, n0;
    tile_of(ti, m0, n0);
    epilogue(m0, n0);
  }
  wait_vmem<0>();  // no copy into LDS outlives the workgroup
}

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// OCC workgroups per CU (1 for 256 x 256 tiles: 512 registers per lane; 2 for 128 x 128)
template <int BM, int BN, int BK, int S, int ACT, int OCC>
hipError_t launch_tiles(FfnGemmParams p, hipStream_t stream) {
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const int T = p.tiles_m * p.tiles_n;
  // persistent workgroups, OCC per CU; when the tiles outnumber them, a multiple of 8 so that every
  // round of tiles keeps the XCD of each virtual index
  int G = std::min(T, OCC * cu_count());
  if (G < T) G = std::max(8, G / 8 * 8);
  hipLaunchKernelGGL((ffn_gemm_bf16<BM, BN, BK, S, ACT, OCC>), dim3(G), dim3(kFfnThreads), 0, stream, p);
  return hipGetLastError();
}

// 256 x 256 tiles when they fill every CU, else 128 x 128 (four times as many, two workgroups per
// CU): small token blocks and the narrow second projection keep the chip busy
template <int ACT>
hipError_t launch_act(const FfnGemmParams& p, hipStream_t stream) {
  const int64_t big = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256);
  if (big >= cu_count()) return launch_tiles<kFfnBM, kFfnBN, kFfnBK, kFfnStages, ACT, 1>(p, stream);
  return launch_tiles<128, 128, kFfnBK, kFfnStages, ACT, 2>(p, stream);
}

}  // namespace

hipError_t launch_ffn_gemm_bf16(const FfnGemmParams& p, int act, hipStream_t stream) {
  if (p.M <= 0) return hipSuccess;
  switch (act) {
    case kFfnActNone: return launch_act<kFfnActNone>(p, stream);
    case RA_FFN_GELU: return launch_act<RA_FFN_GELU>(p, stream);
    case RA_FFN_RELU: return launch_act<RA_FFN_RELU>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ra
