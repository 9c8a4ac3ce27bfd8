// bf16 ring-attention backward step kernels for gfx950 (CDNA4), head dim 128, on
// v_mfma_f32_32x32x16_bf16.
//
// The pages use ring attention for training (Ultralytics glossary, "Ring Attention", section
// "Aplicações"), and the backward of the ring follows the forward's schedule: device i keeps its
// queries, output gradient and the forward's log-sum-exp, and folds the key/value block it holds at
// each step into its query gradient while that block's key/value gradients travel with the block.
// One step for one (query block, key/value block) pair is the gradient of exact attention restricted
// to that pair; with lse the forward's log-sum-exp of each query row, P is recomputed exactly:
//   x = log2(e) * scale * q.k,  p = 2^(x - lse2),  dp = dO.v,  ds = p * (dp - delta),
//   dq += scale * ds k,  dk += scale * ds q,  dv += p dO,
// where lse2 = log2(e) * lse and delta = sum_d dO * O of the row (the softmax Jacobian term).
//
// Two kernels, so that every output is owned by exactly one workgroup (no atomics, deterministic):
//   bwd_dq:  query-stationary like the forward step: a workgroup holds 256 query rows (8 waves x 32),
//            streams 64-key tiles of K and V through LDS and computes, per 32-key half tile,
//              S^T = K Q^T, dP^T = V dO^T (A = K / V rows from LDS, B = Q^T / dO^T in VGPRs),
//              dS^T = P^T * (dP^T - delta),  dQ^T += K^T dS^T (A = K^T by LDS transpose reads).
//   bwd_dkv: key-stationary: a workgroup holds 128 keys (8 waves: each 32 keys belong to a value
//            wave and a key wave), streams 64-row tiles of Q, dO, lse2 and delta of every query head
//            that reads its key/value head, and computes, per 32-row chunk,
//              S = Q K^T, dP = dO V^T (A = Q / dO rows from LDS, B = K^T / V^T in VGPRs),
//              dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T by LDS transpose reads).
// In both, the lane of an accumulator is its stationary row (query or key), so the per-row scalars
// (lse2, delta) or per-column ones come as one value per lane (bwd_dq) or four 16-byte LDS reads per
// chunk (bwd_dkv).  Tiles go HBM -> LDS directly (global_load_lds) through 3-stage rings in the
// swizzled layout of gfx950_tile.h; tile t+2 is requested while tile t is computed and one
// workgroup barrier per tile makes the next one visible.
#include <type_traits>

#include "gfx950_tile.h"
#include "internal.h"

namespace ra {
namespace {

using namespace tile;

constexpr int kTile = 64;                        // rows per streamed tile (keys or queries)
constexpr int kTileBytes = kTile * kRowBytes;    // 16 KiB
constexpr int kBwdStages = 3;

// A 64-row tile load: the 16 pieces of 1 KiB (4 rows each) are spread over the waves; lane l of a
// piece copies row 4*piece + l/16, 16-byte chunk (l%16) ^ swz(row) of the source, to LDS chunk l%16.
// Rows past `nrows` re-read the last row (finite values; the kernels mask them).
struct TileSrc {
  const char* base;  // row 0 of the tile's rows
  int64_t row_bytes; // bytes between consecutive rows in global memory
  int nrows;         // valid rows in the tile (<= 64)
};

__device__ __forceinline__ void load_tile_pieces(const TileSrc& src, uint32_t lds_tile, int first_piece, int npieces) {
  const int lane = __lane_id();
  for (int i = 0; i < npieces; ++i) {
    const int piece = first_piece + i;
    const int row = piece * 4 + (lane >> 4);
    const int srow = row < src.nrows ? row : src.nrows - 1;
    const uint32_t off = (uint32_t)(srow * src.row_bytes) + (((lane & 15) ^ swz(row)) * 16);
    copy_to_lds16(src.base, off, lds_tile + piece * 1024);
  }
}

// Operand tables for one 64-row tile in LDS (shared by both kernels).
//   rowoff[kk]:   A operand "rows": lane reads row (lane % 32) of a 32-row half, 8 values of the
//                 16-wide k step kk (d = 16 kk + 8 (lane / 32)); add half * 32 * kRowBytes.
//   troff[rr][dt]: A operand "transposed": the two 4-value transpose reads that give lane l the 8
//                 tile rows of 16-row block kb (add kb * 16 * kRowBytes) at column d = 32 dt + l % 32,
//                 in the order in which a 32x32 accumulator holds its rows (row 8 (r/4) + 4 (lane/32)
//                 + r % 4 of register r), so that 8 consecutive accumulator registers converted to
//                 bf16 are the matching B operand.
struct TileOffsets {
  int rowoff[8];
  int troff[2][4];
};

__device__ __forceinline__ TileOffsets tile_offsets() {
  TileOffsets t;
  const int lane = __lane_id();
  const int j = lane & 31, h2 = lane >> 5;
  const int jswz = swz(j);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) t.rowoff[kk] = j * kRowBytes + (((2 * kk + h2) ^ jswz) * 16);
  const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
  const int chunk0 = 2 * (tg & 1) + (tq >> 1);
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = 8 * rr + 4 * (tg >> 1) + te;
    const int rswz = (te << 2) | ((2 * rr + (tg >> 1)) & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) t.troff[rr][dt] = row * kRowBytes + (((4 * dt + chunk0) ^ rswz) * 16) + 8 * (tq & 1);
  }
  return t;
}

__device__ __forceinline__ bf16x8 read_rows(const LDS_AS char* tile, int half, int off) {
  return __builtin_bit_cast(bf16x8, *(const LDS_AS i16x8*)(tile + half * 32 * kRowBytes + off));
}

__device__ __forceinline__ bf16x8 read_transposed(const LDS_AS char* tile, int kb, const TileOffsets& t, int dt) {
  const LDS_AS char* b = tile + kb * 16 * kRowBytes;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(b + t.troff[0][dt]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(b + t.troff[1][dt]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// accumulator registers 8h .. 8h+7 of x, rounded to bf16 (a B operand of a later product)
__device__ __forceinline__ bf16x8 pack_half(const float (&x)[16], int h) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[8 * h + e];
  return r;
}

// ------------------------------------------------------------------------------------------------
// bwd_dq: 256 query rows per workgroup, 8 waves (two per SIMD).
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = 32 * kDqWaves;
constexpr int kDqVRing = kBwdStages * kTileBytes;  // LDS: K ring, then V ring
constexpr int kDqPieces = 16 / kDqWaves;           // 1 KiB pieces per wave per K (and per V) tile

struct DqCtx {
  TileSrc k, v;            // tile 0 of this pair's keys and values
  int64_t tile_stride;     // bytes from one key tile to the next
  int nk;
  int wave;
};

__device__ __forceinline__ void dq_request(const DqCtx& cx, int t, int stage, const LDS_AS char* smem) {
  TileSrc k = cx.k, v = cx.v;
  k.base += t * cx.tile_stride;
  v.base += t * cx.tile_stride;
  k.nrows = v.nrows = min(kTile, cx.nk - t * kTile);
  const uint32_t kl = (uint32_t)(uintptr_t)(smem + stage * kTileBytes);
  load_tile_pieces(k, kl, cx.wave * kDqPieces, kDqPieces);
  load_tile_pieces(v, kl + kDqVRing, cx.wave * kDqPieces, kDqPieces);
}

__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq_bf16_d128(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kDqVRing];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31, h2 = lane >> 5;

  // work item: the workgroups that read one (slot, batch, key/value head)'s keys and values (all its
  // query heads and query tiles) run on one XCD (blockIdx mod 8), so they share its L2; causal:
  // heaviest query tiles first
  const int gsz = p.Hq / p.Hkv;
  const int per_group = gsz * p.n_qtiles;
  const int xcd = blockIdx.x & 7, sl = blockIdx.x >> 3;
  const int gi = sl / per_group, rem = sl - gi * per_group;
  const int grp = gi * 8 + xcd;
  if (grp >= p.groups) return;
  const int qt_rank = rem / gsz, hq = rem - qt_rank * gsz;
  const int kvh = grp % p.Hkv, bt = grp / p.Hkv;
  const int dl = bt / p.B, bb = bt - dl * p.B;
  const int h = kvh * gsz + hq;
  const int qt = p.causal ? p.n_qtiles - 1 - qt_rank : qt_rank;
  const int qdev = p.qslot[dl], kvdev = p.kvslot[dl];
  const int Nq = p.Nq, nk = p.nk[dl], row0 = p.q_row0[dl];
  const int qr = qt * kDqRows + wave * 32 + j;  // this lane's query row within the slot
  const bool qvalid = qr < Nq;
  const int qlast = min(qt * kDqRows + kDqRows, Nq) - 1;

  // causal range: last visible key of this lane's row, of the wave's rows and of the workgroup's
  auto last_key = [&](int row) -> int {
    if (!p.causal) return nk - 1;
    const int64_t d = p.q_off[dl] + (int64_t)row * p.q_stride - p.k_off[dl];
    if (d < 0) return -1;
    const int64_t kk = d / p.k_stride;
    return kk < (int64_t)(nk - 1) ? (int)kk : nk - 1;
  };
  const int kmax_lane = last_key(qvalid ? qr : qlast);
  const int wrow0 = min(qt * kDqRows + wave * 32, qlast), wrow1 = min(qt * kDqRows + wave * 32 + 31, qlast);
  const int kmin_wave = last_key(wrow0), kmax_wave = last_key(wrow1);
  const int kend = last_key(qlast);
  const int ntiles = kend < 0 ? 0 : kend / kTile + 1;

  // this lane's row: Q^T and dO^T fragments (B operands), lse2 and delta
  const size_t qrow_elems = (size_t)p.Hq * kD;
  const size_t qbase = (((size_t)qdev * p.B + bb) * p.NqTot + row0 + (qvalid ? qr : 0)) * qrow_elems + (size_t)h * kD;
  bf16x8 qf[8], df[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const i16x8 zq = {0, 0, 0, 0, 0, 0, 0, 0};
    qf[kk] = __builtin_bit_cast(bf16x8, qvalid ? *(const i16x8*)((const unsigned short*)p.q + qbase + 16 * kk + 8 * h2) : zq);
    df[kk] = __builtin_bit_cast(bf16x8, qvalid ? *(const i16x8*)((const unsigned short*)p.dout + qbase + 16 * kk + 8 * h2) : zq);
  }
  const size_t srow = (((size_t)qdev * p.B + bb) * p.Hq + h) * p.NqTot + row0 + (qvalid ? qr : 0);
  const float lse2 = qvalid ? p.lse2[srow] : INFINITY;  // +inf for a row that saw no key: p = 0
  const float delta = qvalid ? p.delta[srow] : 0.f;
  const float c = p.scale_log2;

  DqCtx cx;
  const int64_t krow_bytes = (int64_t)p.Hkv * kD * 2;
  const size_t kv_off = 2 * ((((size_t)kvdev * p.B + bb) * p.NkTot) * p.Hkv * kD + (size_t)kvh * kD);
  cx.k = TileSrc{(const char*)p.k + kv_off, krow_bytes, kTile};
  cx.v = TileSrc{(const char*)p.v + kv_off, krow_bytes, kTile};
  cx.tile_stride = kTile * krow_bytes;
  cx.nk = nk;
  cx.wave = wave;
  const TileOffsets to = tile_offsets();

  f32x16 dqt[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) dqt[dt] = f32x16{};

  if (ntiles > 0) {
    for (int t = 0; t < 2 && t < ntiles; ++t) dq_request(cx, t, t, smem);
    wait_vmem<0>();
    __syncthreads();
  }
  // one key tile (t, LDS stage ST = t % 3); unrolled by three below so that every LDS address is a
  // per-lane base plus an immediate
  auto tile = [&](auto stage_tag, int t) {
    constexpr int ST = decltype(stage_tag)::value;
    if (t + 2 < ntiles) dq_request(cx, t + 2, (ST + 2) % kBwdStages, smem);
    const int key0 = t * kTile;
    if (key0 <= kmax_wave) {  // else no row of this wave sees the tile
      const LDS_AS char* kt = smem + ST * kTileBytes;
      const LDS_AS char* vt = kt + kDqVRing;
      const bool masked = key0 + kTile - 1 > kmin_wave;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          s = mfma(read_rows(kt, cc, to.rowoff[kk]), qf[kk], s);
          dp = mfma(read_rows(vt, cc, to.rowoff[kk]), df[kk], dp);
        }
        float pr[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
        if (masked) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * cc + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (key > kmax_lane) pr[r] = 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = pr[r] * (dp[r] - delta);
        const bf16x8 b0 = pack_half(ds, 0), b1 = pack_half(ds, 1);
        bf16x8 ta[3];
        ta[0] = read_transposed(kt, 2 * cc, to, 0);
        ta[1] = read_transposed(kt, 2 * cc, to, 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // item i: 16-key block 2 cc + i / 4, d tile i % 4
          if (i + 2 < 8) ta[(i + 2) % 3] = read_transposed(kt, 2 * cc + (i + 2) / 4, to, (i + 2) % 4);
          __builtin_amdgcn_sched_barrier(0);
          dqt[i % 4] = mfma(ta[i % 3], i < 4 ? b0 : b1, dqt[i % 4]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (t + 1 < ntiles) {
      if (t + 2 < ntiles)
        wait_vmem<2 * kDqPieces>();  // all but the request just issued (tile t+2)
      else
        wait_vmem<0>();
      __syncthreads();
    }
  };
  for (int t = 0; t < ntiles; t += kBwdStages) {
    tile(std::integral_constant<int, 0>{}, t);
    if (t + 1 >= ntiles) break;
    tile(std::integral_constant<int, 1>{}, t + 1);
    if (t + 2 >= ntiles) break;
    tile(std::integral_constant<int, 2>{}, t + 2);
  }

  // epilogue: dq (token-major, fp32) += scale * dQ; lane's row, d = 32 dt + 8 g + 4 h2 + i
  if (!qvalid) return;
  float* dqrow = p.dq + (((size_t)qdev * p.B + bb) * p.NqTot + row0 + qr) * qrow_elems + (size_t)h * kD;
  const bool init = p.flags[dl] & kBwdInitDq;
  f32x4 old[16];
#pragma unroll
  for (int cI = 0; cI < 16; ++cI)
    old[cI] = init ? f32x4{0.f, 0.f, 0.f, 0.f} : *(const f32x4*)(dqrow + 32 * (cI >> 2) + 8 * (cI & 3) + 4 * h2);
#pragma unroll
  for (int cI = 0; cI < 16; ++cI) {
    const int dt = cI >> 2, g = cI & 3;
    f32x4 nv;
#pragma unroll
    for (int i = 0; i < 4; ++i) nv[i] = old[cI][i] + p.scale * dqt[dt][4 * g + i];
    *(f32x4*)(dqrow + 32 * dt + 8 * g + 4 * h2) = nv;
  }
}

// ------------------------------------------------------------------------------------------------
// bwd_dkv: 128 keys per workgroup, 8 waves, two per SIMD.  Waves w and w + 4 share the keys
// 32 (w % 4) .. + 31 and split the work, so that each holds one gradient accumulator and two waves
// fit every SIMD.  Per query tile, in two halves separated by a workgroup barrier:
//   value wave (w < 4): S = Q K^T, P = 2^(x - lse2) (kept as bf16, and stored to LDS as bf16) |
//                       dV^T += dO^T P
//   key wave (w >= 4):  dP = dO V^T                                                         |
//                       dS = P (from LDS) * (dP - delta), dK^T += Q^T dS
// Each wave issues 32 products per tile.
constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvKeys = 32 * (kKvWaves / 2);
constexpr int kKvStageBytes = 2 * kTileBytes + 512;  // Q tile, dO tile, lse2 (256 B) + delta (256 B)
constexpr int kKvPBytes = 4 * 4 * 64 * 16;           // P in bf16: 4 wave pairs x 4 packs x 64 lanes x 16 B
constexpr int kKvPieces = 16 / kKvWaves;             // 1 KiB pieces per wave per Q (and per dO) tile

struct KvCtx {
  const char* q;        // row 0 of the slot's query rows of query head 0 (batch bb), bytes
  const char* dout;
  const char* lse2;     // lse2 / delta row 0 of query head 0 (batch bb), bytes
  const char* delta;
  int64_t row_bytes;    // Hq * D * 2
  int64_t head_stat;    // bytes from one query head's lse2 / delta rows to the next (NqTot * 4)
  int nq;
  int wave;
};

// request tile (query head hq, query tile qt) into a stage: 2 Q + 2 dO pieces per wave, and 16 lanes
// of 4 bytes of lse2 (waves 0-3: rows 16 w .. + 15) or delta (waves 4-7)
__device__ __forceinline__ void kv_request(const KvCtx& cx, int stage, int hq, int qt, const LDS_AS char* smem) {
  const uint32_t st = (uint32_t)(uintptr_t)(smem + stage * kKvStageBytes);
  const int nrows = min(kTile, cx.nq - qt * kTile);
  const int64_t rowsel = (int64_t)qt * kTile * cx.row_bytes + (int64_t)hq * kD * 2;
  load_tile_pieces(TileSrc{cx.q + rowsel, cx.row_bytes, nrows}, st, cx.wave * kKvPieces, kKvPieces);
  load_tile_pieces(TileSrc{cx.dout + rowsel, cx.row_bytes, nrows}, st + kTileBytes, cx.wave * kKvPieces, kKvPieces);
  const int lane = __lane_id();
  if (lane < 16) {
    const char* src = (cx.wave < 4 ? cx.lse2 : cx.delta) + hq * cx.head_stat;
    const int row = qt * kTile + (cx.wave & 3) * 16 + lane;
    const int srow = row < cx.nq ? row : cx.nq - 1;  // rows past the end re-read the last (masked)
    copy_to_lds4(src, (uint32_t)(srow * 4), st + 2 * kTileBytes + (cx.wave >> 2) * 256 + (cx.wave & 3) * 64);
  }
}

__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkv_bf16_d128(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kBwdStages * kKvStageBytes + kKvPBytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool key_wave = wave >= kKvWaves / 2;  // accumulates dK (else dV)
  // this pair's P buffer: [pack][lane] bf16x8; pack 2 c2 + hh holds registers 8 hh .. 8 hh + 7 of the
  // 32-row half c2 (the accumulator layout of S and dP, whose lane is the key)
  LDS_AS i16x8* pbuf = (LDS_AS i16x8*)(smem + kBwdStages * kKvStageBytes) + (wave & 3) * 4 * 64;
  const int j = lane & 31, h2 = lane >> 5;

  // work item: (slot, batch, key/value head, key tile of 128); the key tiles of one (slot, batch,
  // key/value head) read the same query rows and run on one XCD (blockIdx mod 8), sharing its L2
  const int xcd = blockIdx.x & 7, sl = blockIdx.x >> 3;
  const int gi = sl / p.n_ktiles, ktile = sl - gi * p.n_ktiles;
  const int grp = gi * 8 + xcd;
  if (grp >= p.groups) return;
  const int kvh = grp % p.Hkv, bt = grp / p.Hkv;
  const int dl = bt / p.B, bb = bt - dl * p.B;
  const int gsz = p.Hq / p.Hkv;
  const int qdev = p.qslot[dl], kvdev = p.kvslot[dl], gdev = p.gslot[dl];
  const int Nq = p.Nq, nk = p.nk[dl], row0 = p.q_row0[dl];
  if (ktile * kKvKeys >= nk) return;
  const int key = ktile * kKvKeys + (wave & 3) * 32 + j;  // this lane's key
  const bool kvalid = key < nk;

  // causal: first query row that sees this lane's key, of the wave's keys and of the workgroup's
  auto first_row = [&](int kk) -> int {
    if (!p.causal) return 0;
    const int64_t d = p.k_off[dl] + (int64_t)kk * p.k_stride - p.q_off[dl];
    if (d <= 0) return 0;
    const int64_t r = (d + p.q_stride - 1) / p.q_stride;
    return r < (int64_t)Nq ? (int)r : Nq;
  };
  const int klast = min(ktile * kKvKeys + kKvKeys, nk) - 1;
  const int qmin_lane = first_row(kvalid ? key : klast);
  const int wk0 = min(ktile * kKvKeys + (wave & 3) * 32, klast), wk1 = min(ktile * kKvKeys + (wave & 3) * 32 + 31, klast);
  const int qmin_wave = first_row(wk0), qmax_wave = first_row(wk1);  // rows >= qmax_wave see every key of the wave
  const int qt_first = first_row(ktile * kKvKeys) / kTile;
  const int nqt = (Nq + kTile - 1) / kTile;
  const int nitems = (nqt - qt_first) * gsz;  // (query head, query tile) pairs, head-major

  // this lane's key: K^T fragments (B operand of S, value wave) or V^T fragments (of dP, key wave)
  const size_t krow_elems = (size_t)p.Hkv * kD;
  const size_t kbase = (((size_t)kvdev * p.B + bb) * p.NkTot + (kvalid ? key : 0)) * krow_elems + (size_t)kvh * kD;
  const unsigned short* frag_src = (const unsigned short*)(key_wave ? p.v : p.k) + kbase;
  bf16x8 kvf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const i16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    kvf[kk] = __builtin_bit_cast(bf16x8, kvalid ? *(const i16x8*)(frag_src + 16 * kk + 8 * h2) : z);
  }

  KvCtx cx;
  cx.row_bytes = (int64_t)p.Hq * kD * 2;
  const size_t q_off = 2 * ((((size_t)qdev * p.B + bb) * p.NqTot + row0) * p.Hq * kD + (size_t)(kvh * gsz) * kD);
  cx.q = (const char*)p.q + q_off;
  cx.dout = (const char*)p.dout + q_off;
  const size_t stat0 = 4 * ((((size_t)qdev * p.B + bb) * p.Hq + kvh * gsz) * p.NqTot + row0);
  cx.lse2 = (const char*)p.lse2 + stat0;
  cx.delta = (const char*)p.delta + stat0;
  cx.head_stat = (int64_t)p.NqTot * 4;
  cx.nq = Nq;
  cx.wave = wave;
  const TileOffsets to = tile_offsets();
  const float c = p.scale_log2;

  f32x16 acc[4];  // dK^T (key wave) or dV^T (value wave): lane's key, d = 32 dt + 8 (r / 4) + 4 h2 + r % 4
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  // items walk (query head, query tile) head-major: the query tile of the current item, and the
  // item requested next
  int qt = qt_first, rhq = 0, rqt = qt_first;
  auto advance = [&](int& h_, int& q_) {
    if (++q_ == nqt) {
      q_ = qt_first;
      ++h_;
    }
  };
  if (nitems > 0) {
    for (int it = 0; it < 2 && it < nitems; ++it) {
      kv_request(cx, it, rhq, rqt, smem);
      advance(rhq, rqt);
    }
    wait_vmem<0>();
    __syncthreads();
  }
  constexpr int kPerRequest = 2 * kKvPieces + 1;  // vector-memory instructions per wave per request
  // one query tile (item it, LDS stage ST = it % 3); unrolled by three below so that every LDS
  // address is a per-lane base plus an immediate
  auto tile = [&](auto stage_tag, int it) {
    constexpr int ST = decltype(stage_tag)::value;
    if (it + 2 < nitems) {
      kv_request(cx, (ST + 2) % kBwdStages, rhq, rqt, smem);
      advance(rhq, rqt);
    }
    const int q0 = qt * kTile;
    qt = qt + 1 == nqt ? qt_first : qt + 1;
    const bool work = q0 + kTile > qmin_wave;  // else no key of this wave (pair) is seen by the tile's rows
    const LDS_AS char* st = smem + ST * kKvStageBytes;
    const LDS_AS char* qtl = st;
    const LDS_AS char* dtl = st + kTileBytes;
    const LDS_AS float* lsel = (const LDS_AS float*)(st + 2 * kTileBytes);
    const LDS_AS float* dell = lsel + kTile;
    const bool masked = q0 < qmax_wave || q0 + kTile > Nq;
    // first half: P (value wave) or dP (key wave) of the two 32-row halves, in the same registers
    f32x16 t2[2];
    if (work) {
      if (!key_wave) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          f32x16 sc = {};
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) sc = mfma(read_rows(qtl, c2, to.rowoff[kk]), kvf[kk], sc);
          // row of register r: 32 c2 + 8 (r / 4) + 4 h2 + r % 4
          f32x4 l4[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) l4[g] = *(const LDS_AS f32x4*)(lsel + 32 * c2 + 8 * g + 4 * h2);
#pragma unroll
          for (int r = 0; r < 16; ++r) t2[c2][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, -l4[r >> 2][r & 3]));
          if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = q0 + 32 * c2 + 8 * (r >> 2) + 4 * h2 + (r & 3);
              if (row < qmin_lane || row >= Nq) t2[c2][r] = 0.f;
            }
          }
          float x[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = t2[c2][r];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) pbuf[(2 * c2 + hh) * 64 + lane] = __builtin_bit_cast(i16x8, pack_half(x, hh));
        }
      } else {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          t2[c2] = f32x16{};
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) t2[c2] = mfma(read_rows(dtl, c2, to.rowoff[kk]), kvf[kk], t2[c2]);
        }
      }
    }
    __syncthreads();  // P of this tile is in LDS
    // second half: dV^T += dO^T P (value wave) or dS = P (dP - delta), dK^T += Q^T dS (key wave)
    if (work) {
      if (!key_wave) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          float x[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = t2[c2][r];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const bf16x8 b = pack_half(x, hh);
            __builtin_amdgcn_sched_barrier(0);  // bounds how far the scheduler hoists operand reads
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(read_transposed(dtl, 2 * c2 + hh, to, dt), b, acc[dt]);
          }
        }
      } else {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          float x[16];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const bf16x8 p8 = __builtin_bit_cast(bf16x8, pbuf[(2 * c2 + hh) * 64 + lane]);
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
              const int g = 2 * hh + g2;
              const f32x4 d4 = *(const LDS_AS f32x4*)(dell + 32 * c2 + 8 * g + 4 * h2);
#pragma unroll
              for (int i = 0; i < 4; ++i) x[4 * g + i] = (float)p8[4 * g2 + i] * (t2[c2][4 * g + i] - d4[i]);
            }
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const bf16x8 b = pack_half(x, hh);
            __builtin_amdgcn_sched_barrier(0);  // bounds how far the scheduler hoists operand reads
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma(read_transposed(qtl, 2 * c2 + hh, to, dt), b, acc[dt]);
          }
        }
      }
    }
    if (it + 1 < nitems) {
      if (it + 2 < nitems)
        wait_vmem<kPerRequest>();  // all but the request just issued (item it+2)
      else
        wait_vmem<0>();
      __syncthreads();
    }
  };
  for (int it = 0; it < nitems; it += kBwdStages) {
    tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 >= nitems) break;
    tile(std::integral_constant<int, 1>{}, it + 1);
    if (it + 2 >= nitems) break;
    tile(std::integral_constant<int, 2>{}, it + 2);
  }

  // epilogue: dk += scale * dK or dv += dV (token-major, fp32); lane's key, d = 32 dt + 8 g + 4 h2 + i
  if (!kvalid) return;
  const size_t grow = (((size_t)gdev * p.B + bb) * p.NkTot + key) * krow_elems + (size_t)kvh * kD;
  float* row = (key_wave ? p.dk : p.dv) + grow;
  const float mul = key_wave ? p.scale : 1.f;
  const bool init = p.flags[dl] & kBwdInitDkv;
  f32x4 old[16];
#pragma unroll
  for (int cI = 0; cI < 16; ++cI)
    old[cI] = init ? f32x4{0.f, 0.f, 0.f, 0.f} : *(const f32x4*)(row + 32 * (cI >> 2) + 8 * (cI & 3) + 4 * h2);
#pragma unroll
  for (int cI = 0; cI < 16; ++cI) {
    const int dt = cI >> 2, g = cI & 3;
    f32x4 nv;
#pragma unroll
    for (int i = 0; i < 4; ++i) nv[i] = old[cI][i] + mul * acc[dt][4 * g + i];
    *(f32x4*)(row + 32 * dt + 8 * g + 4 * h2) = nv;
  }
}

// ------------------------------------------------------------------------------------------------
// delta = sum_d dout * out and lse2 = log2(e) * lse (+inf where lse = -inf) per (device, batch, head,
// row); 16 lanes per row.
template <bool BF16>
__device__ __forceinline__ float load_val(const void* p, size_t i) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)((const unsigned short*)p)[i] << 16);
  else
    return ((const float*)p)[i];
}

template <bool BF16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* __restrict__ out, const void* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ delta,
                                                       float* __restrict__ lse2, int B, int Hq, int Nq, int D,
                                                       size_t rows) {
  const size_t r = (size_t)blockIdx.x * 16 + threadIdx.x / 16;  // row of [n_dev, B, Hq, Nq]
  const int sub = threadIdx.x % 16;
  if (r >= rows) return;
  const int t = (int)(r % Nq);
  const size_t dbh = r / Nq;  // (dev * B + b) * Hq + h
  const int h = (int)(dbh % Hq);
  const size_t db = dbh / Hq;
  const size_t base = ((db * Nq + t) * Hq + h) * (size_t)D;
  float acc = 0.f;
  for (int d = sub; d < D; d += 16) acc = __builtin_fmaf(load_val<BF16>(out, base + d), load_val<BF16>(dout, base + d), acc);
#pragma unroll
  for (int w = 8; w >= 1; w /= 2) acc += __shfl_xor(acc, w, 16);
  if (sub == 0) {
    delta[r] = acc;
    const float l = lse[r];
    lse2[r] = l == -INFINITY ? INFINITY : l * kLog2e;  // a row that saw no key gets p = 2^(x - inf) = 0
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16_d128(const BwdParams& p_in, hipStream_t stream) {
  BwdParams p = p_in;
  p.n_qtiles = (p.Nq + kDqRows - 1) / kDqRows;
  p.groups = p.n_launch * p.B * p.Hkv;
  p.groups_per_xcd = (p.groups + 7) / 8;
  const long long grid = 8LL * p.groups_per_xcd * (p.Hq / p.Hkv) * p.n_qtiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dq_bf16_d128, dim3((unsigned)grid), dim3(kDqThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv_bf16_d128(const BwdParams& p_in, hipStream_t stream) {
  BwdParams p = p_in;
  p.n_ktiles = (p.Nk + kKvKeys - 1) / kKvKeys;
  p.groups = p.n_launch * p.B * p.Hkv;
  p.groups_per_xcd = (p.groups + 7) / 8;
  const long long grid = 8LL * p.groups_per_xcd * p.n_ktiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dkv_bf16_d128, dim3((unsigned)grid), dim3(kKvThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* delta, float* lse2, int n_dev,
                           int B, int Hq, int Nq, int D, int dtype, hipStream_t stream) {
  const size_t rows = (size_t)n_dev * B * Hq * Nq;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 15) / 16));
  if (dtype == RA_BF16)
    hipLaunchKernelGGL(bwd_prep_kernel<true>, grid, dim3(256), 0, stream, out, dout, lse, delta, lse2, B, Hq, Nq, D, rows);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<false>, grid, dim3(256), 0, stream, out, dout, lse, delta, lse2, B, Hq, Nq, D, rows);
  return hipGetLastError();
}

}  // namespace ra
