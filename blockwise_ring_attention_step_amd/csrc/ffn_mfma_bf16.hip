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
// A workgroup owns BM x BN output tiles, one after the other (persistent): 256 x 256 tiles with 8
// waves, two per SIMD, one workgroup per CU; or, when those would leave CUs idle, 128 x 128 tiles with
// 4 waves and two workgroups per CU.  The waves form a (W/2) x 2 grid over the tile, each wave owning
// (BM / (W/2)) x (BN/2) outputs as 32 x 32 accumulators (128 registers with 8 waves, so the 256 x 256
// kernel holds everything in registers without spilling), held transposed (the lane is the token m,
// the register the feature n).  k advances in steps of BK: the a and w rows of a step go HBM -> LDS
// directly (global_load_lds) into a ring of S buffers.  The steps of all of a workgroup's tiles form
// one stream: step s+S is requested into the buffer of step s as soon as every wave has read it (one
// workgroup barrier per step), so S-1 steps are in flight while one is multiplied, across tile
// boundaries too (the next tile's first steps load while the current tile's epilogue runs).  Within a
// step, the LDS fragments of k slice kk+1 are read while the products of slice kk run.  The epilogue
// takes the bias from LDS (copied there during the tile's last steps) and sends each 32 x 32 output
// block through a small LDS area of its wave, so that every store writes 64 contiguous bytes of a
// row.  Tiles are numbered so that each XCD (workgroup id mod 8) sweeps a contiguous range of them,
// GM m-tiles at a time, so the rows that neighbouring workgroups share stay in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "gfx950_tile.h"
#include "internal.h"

namespace ra {
namespace {

using namespace tile;

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

// W waves in a WM x WN grid (WM = W / 2 along m, WN = 2 along n); OCC workgroups per CU.
template <int BM, int BN, int BK, int S, int ACT, int OCC, int W>
__global__ __launch_bounds__(64 * W, OCC) void ffn_gemm_bf16(const FfnGemmParams p) {
  constexpr int kFfnWaves = W;
  constexpr int WN = 2, WM = W / WN;
  constexpr int R = BK * 2;                  // bytes of one row of a step
  constexpr int C = R / 16;                  // 16-byte chunks per row
  constexpr int RPP = 1024 / R;              // rows per 1 KiB copy
  constexpr int KK = BK / 16;                // k slices of one product per step
  constexpr int kTileA = BM * R;
  constexpr int kStage = (BM + BN) * R;
  constexpr int kPieces = (BM + BN) / RPP / kFfnWaves;  // 1 KiB copies per wave per step
  constexpr int MB = BM / (32 * WM), NB = BN / (32 * WN);  // 32 x 32 blocks per wave along m and n
  static_assert(MB >= 1 && NB >= 1 && MB * 32 * WM == BM && NB * 32 * WN == BN, "wave grid covers the tile");
  static_assert(R == 64 || R == 128, "step rows of 64 or 128 bytes");
  static_assert(kPieces * kFfnWaves * RPP == BM + BN, "tile rows split evenly over the waves");
  static_assert((S - 1) * kPieces < 64, "vmcnt range");
  // after the S step buffers, 256 bytes per wave for the bias of its columns of the current tile
  constexpr int kBiasOff = S * kStage;
  static_assert(BN / WN <= 128, "one 256-byte bias copy per wave");
  // then, per wave, a 32 x 32 block of the output on its way to HBM (rows padded from 64 to 80 bytes)
  constexpr int kOutRow = 80;
  constexpr int kOutOff = kBiasOff + 256 * W;
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * kStage + 256 * W + 32 * kOutRow * W];
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
  // A piece covers RPP consecutive rows; its 16-byte chunk swizzle is the same for every piece of this
  // wave (swz(row) depends on row / (256/R) mod C, and pieces of one wave start RPP * kFfnWaves rows
  // apart, a multiple of 256/R * C), so one per-lane offset (lane's row within the piece and chunk)
  // serves them all, with the piece's first row added as a scalar; only a piece that reaches past the
  // last row of a or w takes the per-lane clamp.
  static_assert((RPP * kFfnWaves) % ((256 / R) * C) == 0, "one chunk swizzle for all pieces of a wave");
  const char* xa = nullptr;
  const char* wa = nullptr;
  int lim_a = 0, lim_w = 0;  // last valid row of this tile's a rows and w rows
  const uint32_t lane_row = lane / C;
  const uint32_t lane_chunk = ((lane % C) ^ swz(RPP * wave + lane / C)) * 16;
  int rq_tile = 0, rq_kt = 0;
  auto setup_request_tile = [&](int i) {
    int m0, n0;
    tile_of(i, m0, n0);
    xa = (const char*)p.x + (int64_t)m0 * p.ldx * 2;
    wa = (const char*)p.w + (int64_t)n0 * p.ldw * 2;
    lim_a = p.M - 1 - m0;
    lim_w = p.N - 1 - n0;
  };
  // piece k of the requested step into buffer buf; then move the request on by one step
  auto issue_piece = [&](int k, int buf) {
    const int q = wave + kFfnWaves * k;
    const bool is_a = kFfnWaves * k < BM / RPP;  // the same for every wave (wave < W, BM/RPP % W == 0)
    const int row0 = RPP * q - (is_a ? 0 : BM);  // first row of the piece within the tile's a or w rows
    const int lim = is_a ? lim_a : lim_w;
    const int64_t ld2 = (is_a ? p.ldx : p.ldw) * 2;
    const char* base = (is_a ? xa : wa) + rq_kt * R;
    const uint32_t dst = (uint32_t)(uintptr_t)(smem + buf * kStage) + q * 1024;
    if (row0 + RPP - 1 <= lim) {
      copy_to_lds16(base + row0 * ld2, (uint32_t)(lane_row * ld2) + lane_chunk, dst);
    } else {  // rows past the end re-read the last row
      const int row = min(row0 + (int)lane_row, lim);
      copy_to_lds16(base, (uint32_t)(row * ld2) + lane_chunk, dst);
    }
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
  const int wn = wave / WM, wm = wave % WM;
  const int a_row0 = wm * (BM / WM), w_row0 = kTileA / R + wn * (BN / WN);

  f32x16 acc[NB][MB];
  // Products run bn-major (product i = NB-block i / MB, MB-block i % MB).  The w fragment bn of the next k
  // slice is read right after product MB bn + MB - 1, its last use in the current slice, into the register
  // it frees, at least (NB - 1) MB products before its first use.  Every product of a slice reads all MB
  // x fragments, so they are held twice, by slice parity: the next slice's x fragment bm is read after
  // product bm of the current one, kProducts - 1 products before its first use (one set only would leave
  // a single product between the read and the use, too short for LDS latency).
  static_assert(KK % 2 == 0, "slice parity is the same in every step");
  bf16x8 wf[NB], xf[2][MB];
  // fragment r of k slice kk (r < NB: w rows of block r; else x rows of block r - NB)
  auto read_one = [&](int buf, int kk, int r) {
    const LDS_AS char* base = smem + buf * kStage + roff[kk];
    if (r < NB)
      wf[r] = __builtin_bit_cast(bf16x8, *(const LDS_AS i16x8*)(base + (w_row0 + 32 * r) * R));
    else
      xf[kk & 1][r - NB] = __builtin_bit_cast(bf16x8, *(const LDS_AS i16x8*)(base + (a_row0 + 32 * (r - NB)) * R));
  };
  auto mfma_one = [&](int i, int kk) {
    const int bn = i / MB, bm = i % MB;
    acc[bn][bm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[bn], xf[kk & 1][bm], acc[bn][bm], 0, 0, 0);
  };
  // the fragment reads of slice kk that follow product i of the slice before it
  auto reads_after = [&](int i, int buf, int kk) {
    if (i % MB == MB - 1) read_one(buf, kk, i / MB);  // w fragment bn = i / MB (its last use was product i)
    if (i < MB) read_one(buf, kk, NB + i);            // x fragment bm = i, into the other parity's set
  };

  // The bias of the wave's BN / WN columns of the tile at n0 goes HBM -> LDS (4 bytes per lane, columns past
  // the end re-read the last pair), requested at the start of step KT - S + 1 of the tile: the barrier wait of
  // the tile's last step leaves only the (S - 2) kPieces most recent loads in flight, and the copies of the
  // S - 2 steps between are that many loads younger than the bias copy.  (A tile of fewer steps requests it
  // at its first step and waits for it before the epilogue.)  The epilogue then reads it from LDS: a global
  // load there would wait for every store before it and for the next tile's copies.
  auto request_bias = [&](int n0) {
    const int c = min(n0 + wn * (BN / WN) + 2 * lane, p.N - 2);
    copy_to_lds4((const char*)p.bias, (uint32_t)c * 2, (uint32_t)(uintptr_t)(smem + kBiasOff + wave * 256));
  };
  const LDS_AS char* bias_lds = smem + kBiasOff + wave * 256 + 8 * h2;

  // epilogue of the tile at (m0, n0): register 4 g + e of block (bn, bm) is feature
  // n = n0 + wn BN/WN + 32 bn + 8 g + 4 h2 + e of token m = m0 + wm BM/WM + 32 bm + j
  unsigned short* out = (unsigned short*)p.out;
  // A tile that lies inside [0, M) x [0, N) stores without per-element bounds checks; only the edge
  // tiles take the checked form (its branches would otherwise keep accumulator values live across
  // every store and push the 256 x 256 kernel into scratch).
  // Each 32 x 32 block passes through the wave's LDS staging area: lane (j, h2) writes its 16 values into
  // row j, then every lane reads 16 bytes of one row (four lanes a row, 16 rows a pass) and stores them, so
  // that each store writes 64 contiguous bytes of 16 output rows instead of 16 bytes of 32 rows.  The area
  // belongs to one wave, whose LDS accesses execute in order, so no barrier is needed.
  LDS_AS char* stage_out = smem + kOutOff + wave * (32 * kOutRow);
  auto epilogue_body = [&](int m0, int n0, auto checked_tag) {
    constexpr bool kChecked = decltype(checked_tag)::value;
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) {
      const int nblk = n0 + wn * (BN / WN) + 32 * bn;  // first feature of the block (N % 32 == 0)
      u16x4 bv[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bv[g] = (!kChecked || nblk < p.N) ? *(const LDS_AS u16x4*)(bias_lds + (32 * bn + 8 * g) * 2) : u16x4{0, 0, 0, 0};
#pragma unroll
      for (int bm = 0; bm < MB; ++bm) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc[bn][bm][4 * g + e] + __uint_as_float((uint32_t)bv[g][e] << 16);
            o[e] = __builtin_bit_cast(unsigned short, (__bf16)activate<ACT>(z));
          }
          *(LDS_AS u16x4*)(stage_out + j * kOutRow + 16 * g + 8 * h2) = o;
        }
        const int mblk = m0 + wm * (BM / WM) + 32 * bm;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          const int r = 16 * pass + lane / 4, c = lane % 4;
          const i16x8 v = *(const LDS_AS i16x8*)(stage_out + r * kOutRow + 16 * c);
          if (!kChecked || (mblk + r < p.M && nblk < p.N))
            *(i16x8*)(out + (int64_t)(mblk + r) * p.ldo + nblk + 8 * c) = v;
        }
      }
    }
  };
  auto epilogue = [&](int m0, int n0) {
    if (m0 + BM <= p.M && n0 + BN <= p.N)
      epilogue_body(m0, n0, std::false_type{});
    else
      epilogue_body(m0, n0, std::true_type{});
  };

  // One step: KK slices of NB x MB products.  After each product come the fragment reads it frees
  // (reads_after) and the step's other work in fixed slots (sched_barrier keeps the order).  In the last
  // slice, product 0 first meets the other waves at the barrier (step s+1 landed, step s read by all:
  // the next step's fragments are read from buffer (s+1) % S only after it), and the first half of the
  // copies of step s+S into the freed buffer follows products 1 .. kProducts-1; the second half follows
  // the products of the first slice of step s+1, so that fewer copies queue at the memory pipeline at
  // once and the matrix cores keep running across the barrier and the copies.  (The barrier of step s+1
  // waits for both halves.)  Near the end of the stream the same schedule runs on: requests past the
  // last step fetch the last tile's rows again into buffers that no step reads, and the fragments read
  // for a step past the last one are not used.
  constexpr int kProducts = NB * MB;
  static_assert(kProducts >= 4 && KK >= 2, "slots for the barrier and copies");
  static_assert(S == 2 && kPieces % 2 == 0, "a request split over two steps fills the buffer the second frees");
  auto step = [&](int s) {
    const int buf = s % S;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < kProducts; ++i) {
        mfma_one(i, kk);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < KK) {
          reads_after(i, buf, kk + 1);
          if (kk == 0 && s > 0) {  // the second half of the request begun in step s-1 (the prologue's is whole)
#pragma unroll
            for (int k = kPieces / 2; k < kPieces; ++k)
              if (1 + (k - kPieces / 2) * (kProducts - 1) / (kPieces / 2) == i) issue_piece(k, (s + 1) % S);
            if (i == kProducts - 1) advance_request();
          }
        } else {
          if (i == 0) {
            wait_vmem<(S - 2) * kPieces>();  // step s+1 has landed (this wave's copies)
            __syncthreads();                 // ... every wave's, and every wave has read all of step s
          }
          reads_after(i, (s + 1) % S, 0);
#pragma unroll
          for (int k = 0; k < kPieces / 2; ++k)
            if (1 + k * (kProducts - 1) / (kPieces / 2) == i) issue_piece(k, buf);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
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
  for (int r = 0; r < NB + MB; ++r) read_one(0, 0, r);
  for (int ti = 0; ti < nt; ++ti) {
#pragma unroll
    for (int bn = 0; bn < NB; ++bn)
#pragma unroll
      for (int bm = 0; bm < MB; ++bm) acc[bn][bm] = f32x16{};
    int m0, n0;
    tile_of(ti, m0, n0);
    const int kt_bias = max(KT - S + 1, 0);
    for (int kt = 0; kt < KT; ++kt) {
      if (kt == kt_bias) request_bias(n0);
      step(ti * KT + kt);
    }
    if (KT - S + 1 < 0) wait_vmem<0>();
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

// OCC workgroups of W waves per CU: 256 x 256 tiles with 8 waves (two per SIMD, 64 x 128 outputs and
// 128 accumulator registers each), 128 x 128 tiles with 4 waves and two workgroups per CU
template <int BM, int BN, int BK, int S, int ACT, int OCC, int W>
hipError_t launch_tiles(FfnGemmParams p, hipStream_t stream) {
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const int T = p.tiles_m * p.tiles_n;
  // persistent workgroups, OCC per CU; when the tiles outnumber them, a multiple of 8 so that every
  // round of tiles keeps the XCD of each virtual index
  int G = std::min(T, OCC * cu_count());
  if (G < T) G = std::max(8, G / 8 * 8);
  hipLaunchKernelGGL((ffn_gemm_bf16<BM, BN, BK, S, ACT, OCC, W>), dim3(G), dim3(64 * W), 0, stream, p);
  return hipGetLastError();
}

// 256 x 256 tiles when they fill every CU, else 128 x 128 (four times as many, two workgroups per
// CU): small token blocks and the narrow second projection keep the chip busy
template <int ACT>
hipError_t launch_act(const FfnGemmParams& p, hipStream_t stream) {
  const int64_t big = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256);
  if (big >= cu_count()) return launch_tiles<kFfnBM, kFfnBN, kFfnBK, kFfnStages, ACT, 1, 8>(p, stream);
  return launch_tiles<128, 128, kFfnBK, kFfnStages, ACT, 2, 4>(p, stream);
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
