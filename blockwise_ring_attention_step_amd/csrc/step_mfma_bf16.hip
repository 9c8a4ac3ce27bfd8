// bf16 ring-attention step kernel for gfx950 (CDNA4), head dim 128, on v_mfma_f32_32x32x16_bf16.
//
// One workgroup (8 waves, 512 threads) folds one or two key/value blocks (one or two ring steps) into
// the online-softmax state of 256 query rows of one (device, batch, query head): the blocks form one
// stream of 64-key tiles, and the state stays in registers across the seam.  This is the per-step work of the Ultralytics
// glossary page "Ring Attention", section "Como funciona a atenção em anel" (attend the held block,
// accumulate exponentiated scores and weighted values), with the running-maximum rescaling of
// "Sequence Parallelism and Ring Attention", section "Approfondimento tecnico".
//
// Per 64-key tile t and per wave (32 query rows):
//   S^T[key, query] = K_t . Q^T        32x32x16 MFMA: A = K rows from LDS, B = Q^T held in VGPRs
//   online softmax in registers        lane j (mod 32) owns query j; its 32 keys per tile sit in its
//                                      own registers, the other 32 in lane j^32: a row max needs
//                                      one permlane32 swap, the row sum none (the two halves are
//                                      added once at the end)
//   O^T[d, query] += V_t^T . P^T       A = V^T via ds_read_b64_tr_b16 (LDS transpose read), B = P^T
//                                      straight from the S^T accumulators converted to bf16
// Every lane owns one query row in both accumulators, so rescaling O is a per-lane scalar multiply.
// The reference exponent m of a row moves only when it must (the final quotient does not depend
// on it): a tile is exponentiated against the current m, and the exact row maximum is formed only
// when a tile sum could overflow or a row sees its first keys.
//
// Ping-pong between two wave groups.  Waves 0-3 (group A, rows 0-127) and waves 4-7 (group B,
// rows 128-255) share the SIMDs pairwise and run the same instruction sequence per tile,
//     X_t = [P.V of tile t-1, scores of tile t]  (32 MFMAs)  barrier  Y_t = [softmax of tile t]  barrier
// with B one barrier window behind A: while one group's X keeps the matrix pipe busy, the other
// group's Y runs on the vector ALU.
//
// Memory: K and V tiles go HBM -> LDS directly (global_load_lds, 16 B per lane, no VGPR staging)
// through 4-stage rings (K tiles in the first 64 KiB of LDS, V tiles in the next 64 KiB, so every
// LDS address is a per-lane base plus an immediate); tile t+2 is requested while tile t is
// computed, and a wave waits for its loads only down to one tile still in flight.
//
// The ring hop inside the step (optional, per device): the workgroups of the first query head of
// each key/value head also store the key/value rows they stage in LDS into the successor device's
// receive slot (the same pages: the next block travels while the current one is computed).
//
// LDS layout of a tile: 64 rows (keys) x 256 B, the 16-byte chunk c of row r stored at chunk
// c ^ swz(r) with swz(r) = 4*(r%4) + (r/4)%4.  Both the 16-lane groups of the K reads (16
// consecutive rows, one chunk) and the 32-lane groups of the transpose reads (4 consecutive rows x
// 4 chunks) then hit distinct banks.
#include <hip/hip_ext.h>

#include "gfx950_tile.h"
#include "internal.h"

namespace ra {
namespace {

using namespace tile;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;              // query rows per workgroup
constexpr int kBc = 64;                       // keys per tile
constexpr int kTileBytes = kBc * kRowBytes;   // 16 KiB
constexpr int kStages = 4;
constexpr int kVRing = kStages * kTileBytes;  // LDS: K ring [0, 64 KiB), V ring [64 KiB, 128 KiB)
constexpr int kQStageBytes = 32 * kRowBytes;  // a wave's 32 query rows, staged in the prologue
static_assert(2 * kVRing + 4 * kQStageBytes <= 160 * 1024, "LDS of gfx950");
static_assert(4 * kQStageBytes <= 2 * kTileBytes, "waves 4-7 stage their rows in K stages 2 and 3");
constexpr int kPrefetch = 2;                  // tiles requested ahead of the one being computed
constexpr int kPiecesPerWave = kTileBytes / 1024 / kWaves;  // 1 KiB load instructions per tile per wave

static_assert(kPiecesPerWave == 2, "wait counts below assume 2 K + 2 V loads per wave per tile");
static_assert(kBr == kMfmaRowsPerWg && kBc == kMfmaKeysPerTile, "host view of the work geometry");
static_assert(kStages >= kPrefetch + 2, "a stage is reused only after both groups finished with it");

__device__ __forceinline__ void wait_vmem_all() { wait_vmem<0>(); }
// all but this wave's most recent tile request (2 K + 2 V instructions) have landed in LDS
__device__ __forceinline__ void wait_vmem_but_one_tile() { wait_vmem<4>(); }

// Largest key index of block b visible to the query at local row `row` (causal), clamped to [-1, nk-1].
__device__ __forceinline__ int last_visible_key(const StepParams& p, int dl, int b, int row, int nk) {
  const int64_t pq = p.q_off[dl] + (int64_t)row * p.q_stride;
  const int64_t d = pq - p.k_off[dl][b];
  if (d < 0) return -1;
  const int64_t kk = d / p.k_stride;
  return kk < (int64_t)(nk - 1) ? (int)kk : nk - 1;
}

// One key/value block the workgroup folds, and the loop bounds it sets.
struct Block {
  const char* kbase;  // this (batch, kv head)'s key rows in the block, byte address of key 0
  const char* vbase;
  int nk;             // keys in the block
  int ntiles;         // tiles the workgroup loads
  int ntiles_grp;     // tiles this wave's group computes (causal: group A may stop earlier)
  int nfull;          // tiles [0, nfull) need no mask for any row of the group
  int kmax_lane;      // largest key this lane's query sees
};

// The workgroup's tile stream: virtual tile v < t0 is tile v of block 0, v in [t0, total) tile v - t0
// of block 1 (a slot that folds two ring steps); the online-softmax state runs on across the seam.
struct Ctx {
  int64_t row_bytes;   // bytes between consecutive keys (Hkv * D * 2)
  uint32_t goff[kPiecesPerWave];  // byte offset of this lane's 16 B in each of its tile pieces
  Block b0, b1;  // b1 repeats b0 when the slot folds one block
  int t0, total;
};

// Block and local tile index of virtual tile v (selects, no indexing).
struct TileRef {
  const char* kbase;
  const char* vbase;
  int nk, t;
};
__device__ __forceinline__ TileRef tile_ref(const Ctx& cx, int v) {
  const bool second = v >= cx.t0;
  return TileRef{second ? cx.b1.kbase : cx.b0.kbase, second ? cx.b1.vbase : cx.b0.vbase,
                 second ? cx.b1.nk : cx.b0.nk, second ? v - cx.t0 : v};
}


// This wave's share of one K/V tile request: 2 K + 2 V copies of 1 KiB (the wait counts rely on
// exactly four).  The addresses are prepared ahead (make_request) so that the X phase only issues
// the copies (request_piece).
struct TileRequest {
  const char* kt;               // global rows of the tile's first key, K and V
  const char* vt;
  uint32_t dst;                 // LDS address of this wave's first K piece in the stage
  uint32_t off[kPiecesPerWave]; // per-lane byte offsets of the pieces
};

__device__ __forceinline__ TileRequest make_request(const Ctx& cx, int v, LDS_AS char* smem, int stage, int wave) {
  TileRequest r;
  const TileRef tr = tile_ref(cx, v);
  const int key0 = tr.t * kBc;
  const int64_t tofs = (int64_t)key0 * cx.row_bytes;
  r.kt = tr.kbase + tofs;
  r.vt = tr.vbase + tofs;
  r.dst = (uint32_t)(uintptr_t)(smem + stage * kTileBytes) + wave * kPiecesPerWave * 1024;
  if (key0 + kBc <= tr.nk) {
#pragma unroll
    for (int i = 0; i < kPiecesPerWave; ++i) r.off[i] = cx.goff[i];
  } else {  // ragged last tile: rows past the end re-read the last key (the mask drops them)
    const int lane = __lane_id();
#pragma unroll
    for (int i = 0; i < kPiecesPerWave; ++i) {
      const int row = (wave * kPiecesPerWave + i) * 4 + (lane >> 4);
      const int krow = max(0, min(row, tr.nk - 1 - key0));
      r.off[i] = (uint32_t)(krow * cx.row_bytes) + ((lane & 15) ^ swz(row)) * 16;
    }
  }
  return r;
}

// Copy j (0..3) of a request: piece j / 2, K for even j, V for odd j.
__device__ __forceinline__ void request_piece(const TileRequest& r, int j) {
  const int i = j >> 1;
  if (j & 1)
    copy_to_lds16(r.vt, r.off[i], r.dst + i * 1024 + kVRing);
  else
    copy_to_lds16(r.kt, r.off[i], r.dst + i * 1024);
}

struct Frags {
  bf16x8 q[8];     // Q^T fragments (B operand of S^T = K Q^T)
  int koff[8];     // LDS byte offset of this lane's K fragment for step kk (chunk 0 of the tile)
  int voff[2][4];  // LDS byte offset of this lane's transpose reads [half][d tile] (k step 0, stage 0)
};

struct Softmax {
  float M = -INFINITY;                    // reference exponent (log2 units)
  float lpart[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's partial sums of 2^(x - M) over its keys
};

// Online-softmax update for tile t: mask (diagonal or ragged tiles), then P = 2^(x - M) against
// the row's current reference exponent M, summed in fp32 and rounded to bf16 for P.V.  The final
// division by the normaliser cancels any choice of M, so M need not track the running maximum
// exactly; it only has to keep the sums finite and be set once the row has seen a key.  The exact
// row maximum (and a rescale of O and the normaliser) is therefore computed only when some lane's
// tile sum exceeds 2^64, or a lane without a reference sees a visible key; otherwise the tile costs
// no maximum at all.
constexpr float kSumLimit = 0x1p64f;

__device__ __forceinline__ void tile_softmax(f32x16 (&s)[2], int t, bool masked, int kmax_lane, int h2, float c,
                                             Softmax& sm, f32x16 (&o)[4], bf16x8 (&pf)[4]) {
  const int key_lo = t * kBc + 4 * h2;  // smallest key index this lane holds in the tile
  if (masked) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key_lo + 32 * cc + 8 * (r >> 2) + (r & 3);
        if (key > kmax_lane) s[cc][r] = -INFINITY;
      }
  }
  float e[2][16];
  float ts[4];
  {
    const float negM = sm.M == -INFINITY ? 0.f : -sm.M;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[cc][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cc][r], c, negM));
        ts[r & 3] = (cc == 0 && r < 4) ? e[cc][r] : ts[r & 3] + e[cc][r];
      }
  }
  const float tsum = (ts[0] + ts[1]) + (ts[2] + ts[3]);
  const bool first_keys = sm.M == -INFINITY && key_lo <= kmax_lane;
  if (__builtin_amdgcn_ballot_w64(!(tsum <= kSumLimit) || first_keys)) {
    // new reference: the exact row maximum (both lanes of the row agree on it)
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, partner(mx));
    const float Mn = fmaxf(sm.M, mx * c);
    const float alpha = Mn > sm.M ? __builtin_amdgcn_exp2f(sm.M - Mn) : 1.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.lpart[i] *= alpha;
    sm.M = Mn;
    const float negM = Mn == -INFINITY ? 0.f : -Mn;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[cc][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cc][r], c, negM));
        ts[r & 3] = (cc == 0 && r < 4) ? e[cc][r] : ts[r & 3] + e[cc][r];
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.lpart[i] += ts[i];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[2 * cc + (r >> 3)][r & 7] = (__bf16)e[cc][r];
}

struct Loop {
  int h2;
  float c;
};

// The X phase as one stream of 32 MFMAs: the 16 P.V products of tile t-1 (V fragment (kb, dt) from
// the stage before ST, accumulator o[dt]) and the 16 score products of tile t (K fragment (cc, kk)
// from stage ST, accumulator s[cc]): items 0..15 are the P.V products (consecutive items use
// different accumulators), items 16..31 the score products.  Each item's LDS operand is read
// kAhead items before its MFMA into a small ring of registers, and scheduling barriers keep that
// order, so LDS latency hides behind the MFMAs in flight.  The first kAhead operands (V rows of tile
// t-1, resident since the window before) are read at the end of the previous window (x_preload),
// where the wave would otherwise wait at the barrier, so the stream opens with an MFMA; the K rows
// of tile t are read only after this window's barrier, which is what makes the other group's share
// of that tile visible.  The window's tile request (addresses prepared in the previous window) goes
// out behind the first two products (the hook).
constexpr int kAhead = 3;
constexpr int kRing = kAhead + 2;

template <int ST, int I>
__device__ __forceinline__ bf16x8 x_operand(const Frags& f, const LDS_AS char* smem) {
  constexpr int P = I;
  if constexpr (P < 16) {
    constexpr int kb = P >> 2, dt = P & 3;
    const LDS_AS char* vt = smem + ((ST + kStages - 1) % kStages) * kTileBytes;  // voff includes the V ring base
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vt + kb * 16 * kRowBytes + f.voff[0][dt]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vt + kb * 16 * kRowBytes + f.voff[1][dt]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    constexpr int cc = (P - 16) & 1, kk = (P - 16) >> 1;
    const LDS_AS char* kt = smem + ST * kTileBytes;
    return __builtin_bit_cast(bf16x8, *(const LDS_AS i16x8*)(kt + cc * 32 * kRowBytes + f.koff[kk]));
  }
}

template <int I>
__device__ __forceinline__ void x_product(const Frags& f, bf16x8 a, f32x16 (&s)[2], const bf16x8 (&pf)[4],
                                          f32x16 (&o)[4]) {
  constexpr int P = I;
  if constexpr (P < 16)
    o[P & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[P >> 2], o[P & 3], 0, 0, 0);
  else
    s[(P - 16) & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, f.q[(P - 16) >> 1], s[(P - 16) & 1], 0, 0, 0);
}

// The operands of items 0 .. kAhead-1 of the X phase on stage ST (V rows of the tile before ST).
template <int ST, int I = 0>
__device__ __forceinline__ void x_preload(const Frags& f, const LDS_AS char* smem, bf16x8 (&ring)[kRing]) {
  static_assert(kAhead <= 16, "preloaded operands must all be V rows of the previous tile");
  if constexpr (I < kAhead) {
    ring[I] = x_operand<ST, I>(f, smem);
    x_preload<ST, I + 1>(f, smem, ring);
  }
}

template <int ST, int I, typename Hook>
__device__ __forceinline__ void x_stream_step(const Frags& f, const LDS_AS char* smem, bf16x8 (&ring)[kRing],
                                              f32x16 (&s)[2], const bf16x8 (&pf)[4], f32x16 (&o)[4],
                                              const Hook& hook) {
  if constexpr (I < 32) {
    if constexpr (I + kAhead < 32) ring[(I + kAhead) % kRing] = x_operand<ST, I + kAhead>(f, smem);
    __builtin_amdgcn_sched_barrier(0);
    x_product<I>(f, ring[I % kRing], s, pf, o);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (I == 1) {
      hook();
      __builtin_amdgcn_sched_barrier(0);
    }
    x_stream_step<ST, I + 1>(f, smem, ring, s, pf, o, hook);
  }
}

// X phase on stage ST with items 0 .. kAhead-1 already in the ring.
template <int ST, typename Hook>
__device__ __forceinline__ void x_stream(const Frags& f, const LDS_AS char* smem, bf16x8 (&ring)[kRing],
                                         f32x16 (&s)[2], const bf16x8 (&pf)[4], f32x16 (&o)[4], const Hook& hook) {
  s[0] = f32x16{};
  s[1] = f32x16{};
  x_stream_step<ST, 0>(f, smem, ring, s, pf, o, hook);
}

// Y_v: softmax of virtual tile v.  A tile past this group's last visible key of its block (causal,
// the group of lower rows) is not needed: its P is zero, so the next window's P.V adds nothing; nor
// is the drain position v = total.
__device__ __forceinline__ void phase_y(const Ctx& cx, const Loop& lp, int v, f32x16 (&s)[2], Softmax& sm,
                                        f32x16 (&o)[4], bf16x8 (&pf)[4]) {
  const bool second = v >= cx.t0;
  const int t = second ? v - cx.t0 : v;
  const int ntiles_grp = second ? cx.b1.ntiles_grp : cx.b0.ntiles_grp;
  const int nfull = second ? cx.b1.nfull : cx.b0.nfull;
  const int kmax_lane = second ? cx.b1.kmax_lane : cx.b0.kmax_lane;
  if (v < cx.total && t < ntiles_grp) {
    tile_softmax(s, t, t >= nfull, kmax_lane, lp.h2, lp.c, sm, o, pf);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = bf16x8{};
  }
}

// End of an X window.  While tiles are still being requested, a wave's loads are complete down to
// its most recent tile request: that covers tile t+1, whose K rows the next X phase reads, and every
// older copy or store; once requests stop (drain), everything is waited for.  The barrier then makes
// every wave's share visible.
__device__ __forceinline__ void window_end_x(bool drain) {
  if (drain)
    wait_vmem_all();
  else
    wait_vmem_but_one_tile();
  __syncthreads();
}

// End of a Y window: nothing the next window reads is in flight (tile t+1 completed at the end of
// X_t), so no memory wait; forwarded rows may still be in flight and are covered by the next X end.
__device__ __forceinline__ void window_end_y() { __syncthreads(); }

// The ring hop inside the step: rows of the slot's last key/value block that this workgroup forwards to
// the next device's receive slot (its query tile's 256 keys: virtual tiles [v_lo, v_hi) of the
// stream, tile v - v0 of the block).
struct Fwd {
  char* kdst;  // destination rows of this (batch, key/value head): key 0, K and V
  char* vdst;
  int v_lo, v_hi, v0, nk;
};

// Forward virtual tile v (stage ST): each lane stores back exactly the 16 bytes it copied into LDS, to
// the same offset in the destination block (the lane's copy offset within a tile, cx.goff, from the
// tile's first row there); rows past the end of a ragged tile are not stored.
template <int ST>
__device__ __forceinline__ void forward_tile(const Ctx& cx, const Fwd& fw, const LDS_AS char* smem, int v,
                                             int wave) {
  const int lane = __lane_id();
  const int key0 = (v - fw.v0) * kBc;
  const int64_t tofs = (int64_t)key0 * cx.row_bytes;
  char* const kb = fw.kdst + tofs;
  char* const vb = fw.vdst + tofs;
  const bool full = key0 + kBc <= fw.nk;
#pragma unroll
  for (int i = 0; i < kPiecesPerWave; ++i) {
    const LDS_AS char* src = smem + ST * kTileBytes + (wave * kPiecesPerWave + i) * 1024 + 16 * lane;
    const i16x8 kd = *(const LDS_AS i16x8*)src;
    const i16x8 vd = *(const LDS_AS i16x8*)(src + kVRing);
    if (full) {
      *(i16x8*)(kb + cx.goff[i]) = kd;
      *(i16x8*)(vb + cx.goff[i]) = vd;
    } else if (key0 + (wave * kPiecesPerWave + i) * 4 + (lane >> 4) < fw.nk) {
      *(i16x8*)(kb + cx.goff[i]) = kd;
      *(i16x8*)(vb + cx.goff[i]) = vd;
    }
  }
}

// Both barrier windows of position t (0 <= t <= total, virtual tile t in stage ST): request tile t+2,
// then X_t = scores of tile t and P.V of tile t-1, then Y_t.  Every position runs the same X: at
// position 0 the P.V multiplies a zeroed V stage by P = 0, and at position total the scores are
// computed but never used, so the loop holds one X variant only.  Every wave runs this same
// sequence; group B runs it one window behind group A (one extra barrier before the loop, and
// group A one extra barrier after it), so in each window one group is in X while the other is in Y.
template <int ST>
__device__ __forceinline__ void tile_windows(const Ctx& cx, const Frags& f, const Loop& lp, LDS_AS char* smem,
                                             int t, int wave, bf16x8 (&ring)[kRing], TileRequest& req,
                                             const Fwd& fw, f32x16 (&s)[2], bf16x8 (&pf)[4], Softmax& sm,
                                             f32x16 (&o)[4]) {
  const bool drain = t + kPrefetch >= cx.total;
  x_stream<ST>(f, smem, ring, s, pf, o, [&] {
    if (!drain)
#pragma unroll
      for (int j = 0; j < 4; ++j) request_piece(req, j);
  });
  window_end_x(drain);
  phase_y(cx, lp, t, s, sm, o, pf);
  // the next X phase opens with the P.V of tile t, whose V rows both groups completed a window ago;
  // its tile request (tile t+3) is prepared here too, where the wave would wait at the barrier, and
  // so is the hop of tile t (this wave's copies of it completed at the end of X_{t-1})
  x_preload<(ST + 1) % kStages>(f, smem, ring);
  req = make_request(cx, t + 1 + kPrefetch, smem, (ST + 1 + kPrefetch) % kStages, wave);
  if (t >= fw.v_lo && t < fw.v_hi) forward_tile<ST>(cx, fw, smem, t, wave);
  window_end_y();
}

__global__ __launch_bounds__(kThreads, 1) void step_mfma_bf16_d128(const StepParams p) {
  // the K and V rings, then 32 KiB that (with K stages 2 and 3) stage the query rows in the prologue
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kVRing + 4 * kQStageBytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_b = wave >= kWaves / 2;
  const int j = lane & 31;
  const int h2 = lane >> 5;

  // ---- work item: workgroups that share a key/value head land on one XCD (blockIdx mod 8)
  const int gsz = p.Hq / p.Hkv;
  const int per_group = gsz * p.n_qtiles;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int gi = slot / per_group;
  const int rem = slot - gi * per_group;
  const int g = gi * 8 + xcd;
  if (g >= p.groups) return;
  const int qt_rank = rem / gsz;
  const int hq = rem - qt_rank * gsz;
  const int qt = p.causal ? p.n_qtiles - 1 - qt_rank : qt_rank;  // heaviest causal tiles first
  const int kvh = g % p.Hkv;
  const int bt = g / p.Hkv;
  const int dl = bt / p.B;
  const int bb = bt - dl * p.B;
  const int h = kvh * gsz + hq;
  const int dev = p.slot[dl];
  const int dfl = p.dflags[dl];
  const int Nq = p.Nq, Hq = p.Hq, nsub = p.nsub[dl];
  const int NqT = p.NqTot, NkT = p.NkTot, row0 = p.q_row0[dl];  // array rows; this slot's first row

  const int qrow0 = qt * kBr;
  const int qr = qrow0 + wave * 32 + j;
  const bool qvalid = qr < Nq;
  const int qlast = min(qrow0 + kBr, Nq) - 1;
  const int grow0 = min(qrow0 + (grp_b ? kBr / 2 : 0), qlast);  // this group's first and last rows
  const int grow1 = min(qrow0 + (grp_b ? kBr : kBr / 2) - 1, qlast);

  Loop lp;
  lp.h2 = h2;
  lp.c = p.scale_log2;

  // ---- Q^T fragments (read in the prologue): lane holds q[row qr][16*kk + 8*h2 .. +7]
  Frags f;

  // ---- the blocks this slot folds: rows of this (batch, kv head), and the key ranges: the workgroup
  // loads tiles up to its last row's limit; each group computes up to its own last row's limit; masks
  // apply from the first tile its first row does not fully see
  Ctx cx;
  const size_t kv_in_blk = 2 * ((size_t)bb * NkT * p.Hkv * kD + (size_t)kvh * kD);
  cx.row_bytes = (int64_t)p.Hkv * kD * 2;
  auto setup_block = [&](Block& bk, int bs) {
    const int ref = p.kv[dl][bs];
    const int64_t boff = (int64_t)(ref & 0xffff) * p.kv_block + (int64_t)kv_in_blk;
    bk.kbase = p.kv_base[ref >> 16][0] + boff;
    bk.vbase = p.kv_base[ref >> 16][1] + boff;
    const int nk = p.nk[dl][bs];
    bk.nk = nk;
    bk.kmax_lane = nk - 1;
    int kmin_grp = nk - 1, kend_wg = nk - 1, kend_grp = nk - 1;
    if (p.causal) {
      bk.kmax_lane = last_visible_key(p, dl, bs, qvalid ? qr : qlast, nk);
      kmin_grp = last_visible_key(p, dl, bs, grow0, nk);
      kend_grp = last_visible_key(p, dl, bs, grow1, nk);
      kend_wg = last_visible_key(p, dl, bs, qlast, nk);
    }
    bk.ntiles = kend_wg < 0 ? 0 : kend_wg / kBc + 1;
    bk.ntiles_grp = kend_grp < 0 ? 0 : kend_grp / kBc + 1;
    bk.nfull = kmin_grp < 0 ? 0 : (kmin_grp + 1) / kBc;
  };
  setup_block(cx.b0, 0);
  if (nsub > 1)
    setup_block(cx.b1, 1);
  else
    cx.b1 = cx.b0;  // never reached: the stream ends at t0
  cx.t0 = cx.b0.ntiles;
  cx.total = cx.t0 + (nsub > 1 ? cx.b1.ntiles : 0);
#pragma unroll
  for (int i = 0; i < kPiecesPerWave; ++i) {
    const int row = (wave * kPiecesPerWave + i) * 4 + (lane >> 4);
    cx.goff[i] = (uint32_t)(row * cx.row_bytes + ((lane & 15) ^ swz(row)) * 16);
  }
  // the hop inside the step: the slot's last block, this query tile's 256 keys of it
  Fwd fw;
  fw.kdst = fw.vdst = nullptr;
  fw.v_lo = fw.v_hi = fw.v0 = fw.nk = 0;
  if (p.fwd[dl] >= 0 && hq == 0) {
    const int ref = p.fwd[dl];
    const int64_t boff = (int64_t)(ref & 0xffff) * p.kv_block + (int64_t)kv_in_blk;
    fw.kdst = p.kv_base[ref >> 16][0] + boff;
    fw.vdst = p.kv_base[ref >> 16][1] + boff;
    const bool two = nsub > 1;
    fw.v0 = two ? cx.t0 : 0;
    fw.nk = two ? cx.b1.nk : cx.b0.nk;
    fw.v_lo = fw.v0 + qt * (kBr / kBc);
    fw.v_hi = min(fw.v_lo + kBr / kBc, fw.v0 + (two ? cx.b1.ntiles : cx.b0.ntiles));
  }
  const int kswz = swz(j);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) f.koff[kk] = j * kRowBytes + (((2 * kk + h2) ^ kswz) * 16);
  {
    const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
    const int vchunk0 = 2 * (tg & 1) + (tq >> 1);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int vrow = 8 * rr + 4 * (tg >> 1) + te;
      const int vswz = (te << 2) | ((2 * rr + (tg >> 1)) & 3);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        f.voff[rr][dt] = kVRing + vrow * kRowBytes + (((4 * dt + vchunk0) ^ vswz) * 16) + 8 * (tq & 1);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  Softmax sm;

  if (cx.total > 0) {
    // prologue: the wave's 32 query rows (a row of 256 bytes every Hq * D * 2 bytes) go to LDS in whole
    // rows, row r at qs + r * 256 with its 16-byte chunk c at position c ^ (r & 15), while the first
    // kPrefetch tiles are requested; each lane then reads its fragments from there.  (Waves 0-3 stage in
    // the 32 KiB after the rings, waves 4-7 in K stages 2 and 3, which no request reaches before the
    // barrier below.)
    const int wrow0 = qrow0 + wave * 32;
    const int nqv = max(0, min(32, Nq - wrow0));  // the wave's rows that exist
    const LDS_AS char* qs =
        smem + (wave < kWaves / 2 ? 2 * kVRing + wave * kQStageBytes : 2 * kTileBytes + (wave - kWaves / 2) * kQStageBytes);
    if (nqv > 0) {
      const char* q0 = (const char*)p.q +
                       2 * ((size_t)dev * p.B * NqT * Hq * kD + (((size_t)bb * NqT + row0 + wrow0) * Hq + h) * kD);
      const int qr_l = lane >> 4, qp = lane & 15;  // copy k: row 4 k + qr_l, LDS position qp
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + qr_l;
        const int rs = min(r, nqv - 1);  // rows past the end re-read the last row (zeroed below)
        copy_to_lds16(q0, (uint32_t)(rs * Hq * kD * 2 + ((qp ^ (r & 15)) * 16)), (uint32_t)(uintptr_t)(qs + k * 1024));
      }
    }
#pragma unroll
    for (int t = 0; t < kPrefetch; ++t)
      if (t < cx.total) {
        const TileRequest r = make_request(cx, t, smem, t, wave);
#pragma unroll
        for (int j = 0; j < 4; ++j) request_piece(r, j);
      }
    {  // V stage 3 feeds the P.V of position 0 (with P = 0): it must hold finite values
      LDS_AS i16x8* z = (LDS_AS i16x8*)(smem + kVRing + 3 * kTileBytes);
      z[tid] = i16x8{};
      z[tid + kThreads] = i16x8{};
    }
    wait_vmem_all();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const i16x8 raw = qvalid ? *(const LDS_AS i16x8*)(qs + j * kRowBytes + (((2 * kk + h2) ^ (j & 15)) * 16))
                               : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
      f.q[kk] = __builtin_bit_cast(bf16x8, raw);
    }
    __syncthreads();
    f32x16 s[2];
    bf16x8 pf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = bf16x8{};
    bf16x8 ring[kRing];
    x_preload<0>(f, smem, ring);
    TileRequest req = make_request(cx, kPrefetch, smem, kPrefetch, wave);
    if (grp_b) __builtin_amdgcn_s_barrier();  // group B starts one window late
    // positions 0 .. total (the extra position drains the last P.V); virtual tile t lives in stage t % 4
    for (int t = 0; t <= cx.total; t += kStages) {
      tile_windows<0>(cx, f, lp, smem, t, wave, ring, req, fw, s, pf, sm, o);
      if (t + 1 > cx.total) break;
      tile_windows<1>(cx, f, lp, smem, t + 1, wave, ring, req, fw, s, pf, sm, o);
      if (t + 2 > cx.total) break;
      tile_windows<2>(cx, f, lp, smem, t + 2, wave, ring, req, fw, s, pf, sm, o);
      if (t + 3 > cx.total) break;
      tile_windows<3>(cx, f, lp, smem, t + 3, wave, ring, req, fw, s, pf, sm, o);
    }
    if (!grp_b) __builtin_amdgcn_s_barrier();  // matches group B's extra barrier
  }
  float lsum = (sm.lpart[0] + sm.lpart[1]) + (sm.lpart[2] + sm.lpart[3]);
  const float M = sm.M;

  // ---- epilogue: merge with the incoming state (or finalize).  The wave's 32 rows of o_acc are one
  // contiguous 16 KiB run; they pass through LDS (the rings are free once every wave has left the loop):
  // copied in whole rows, read by each lane in its accumulator layout, merged, written back, and stored
  // in whole rows, so every global access of the state moves full 512-byte rows instead of 32 scattered
  // 32-byte pieces.  The wave's area: row r (0..31) at wave * 16 KiB + r * 512, its 16-byte chunk c at
  // position c ^ (r & 15), which spreads the 32 rows of one lane access over all banks.
  lsum += partner(lsum);
  __syncthreads();  // every wave has left the loop: no LDS read of the rings is outstanding
  const int wrow0 = qrow0 + wave * 32;                       // the wave's first row
  const int nvalid = max(0, min(32, Nq - wrow0));            // its rows that exist
  if (nvalid == 0) return;
  const size_t srow0 = ((size_t)(dev * p.B + bb) * Hq + h) * NqT + row0 + wrow0;
  const size_t srow = srow0 + j;
  LDS_AS char* wl = smem + wave * (32 * kD * 4);
  const bool has_old = !(dfl & kDevInit);
  float* const oacc_wave = p.o_acc + srow0 * kD;
  // lane l of whole-row access k: row 2 k + l / 32, LDS position l % 32, global chunk (l % 32) ^ (row & 15)
  const int xr = lane >> 5, xp = lane & 31;
  if (has_old) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 2 * k + xr;
      const int rs = min(r, nvalid - 1);  // rows past the end re-read the last row (not used)
      copy_to_lds16((const char*)oacc_wave, (uint32_t)(rs * kD * 4 + ((xp ^ (r & 15)) * 16)),
                    (uint32_t)(uintptr_t)(wl + k * 1024));
    }
  }
  float Mo = -INFINITY, lo = 0.f;
  if (has_old && qvalid) {
    Mo = p.m[srow];
    lo = p.l[srow];
  }
  const float Mf = fmaxf(Mo, M);
  const float ao = Mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mo - Mf);
  const float an = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
  const float lf = ao * lo + an * lsum;
  // this lane's chunk (dt, gq): d = 32 dt + 8 gq + 4 h2 .. + 3, global chunk 8 dt + 2 gq + h2 of row j
  auto lane_chunk = [&](int c) -> LDS_AS char* {
    return wl + j * (kD * 4) + ((((8 * (c >> 2) + 2 * (c & 3) + h2)) ^ (j & 15)) * 16);
  };
  f32x4 old[16];
  if (has_old) {
    wait_vmem<0>();  // this wave's copies have landed (the area is the wave's own: no barrier)
#pragma unroll
    for (int c = 0; c < 16; ++c) old[c] = *(const LDS_AS f32x4*)lane_chunk(c);
  } else {
#pragma unroll
    for (int c = 0; c < 16; ++c) old[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (dfl & kDevFinal) {
    // O rows in bf16 (256 bytes each; a wave's rows are Hq * D * 2 bytes apart): staged as 32 rows of
    // 256 bytes, chunk c at position c ^ (row & 15), then stored four whole rows per instruction
    const float inv = lf > 0.f ? 1.0f / lf : 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int dt = c >> 2, gq = c & 3;
      u16x4 outv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float val = (ao * old[c][i] + an * o[dt][4 * gq + i]) * inv;
        outv[i] = __builtin_bit_cast(unsigned short, (__bf16)val);
      }
      // 8-byte piece (dt, gq, h2) of the row: 16-byte chunk 4 dt + gq, half h2
      *(LDS_AS u16x4*)(wl + j * (kD * 2) + (((4 * dt + gq) ^ (j & 15)) * 16) + 8 * h2) = outv;
    }
    unsigned short* const orow0 =
        (unsigned short*)p.o_out + (((size_t)dev * p.B + bb) * NqT + row0 + wrow0) * (size_t)Hq * kD + (size_t)h * kD;
    const int yr = lane >> 4, yp = lane & 15;  // four rows per instruction, 16 chunks of 16 bytes each
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + yr;
      const i16x8 v8 = *(const LDS_AS i16x8*)(wl + r * (kD * 2) + yp * 16);
      if (r < nvalid) *(i16x8*)(orow0 + (size_t)r * Hq * kD + 8 * (yp ^ (r & 15))) = v8;
    }
    if (h2 == 0 && qvalid && p.lse_out) p.lse_out[srow] = lf > 0.f ? (Mf + log2f(lf)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int dt = c >> 2, gq = c & 3;
      f32x4 nv;
#pragma unroll
      for (int i = 0; i < 4; ++i) nv[i] = ao * old[c][i] + an * o[dt][4 * gq + i];
      *(LDS_AS f32x4*)lane_chunk(c) = nv;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = 2 * k + xr;
      const f32x4 v4 = *(const LDS_AS f32x4*)(wl + r * (kD * 4) + xp * 16);
      if (r < nvalid) *(f32x4*)(oacc_wave + r * kD + 4 * (xp ^ (r & 15))) = v4;
    }
    if (h2 == 0 && qvalid) {
      p.m[srow] = Mf;
      p.l[srow] = lf;
    }
  }
}

}  // namespace

hipError_t launch_step_mfma_bf16_d128(const StepParams& p_in, hipStream_t stream, hipEvent_t ev_start,
                                      hipEvent_t ev_stop) {
  StepParams p = p_in;
  p.groups = p.n_launch * p.B * p.Hkv;
  p.groups_per_xcd = (p.groups + 7) / 8;
  p.n_qtiles = (p.Nq + kBr - 1) / kBr;
  const int gsz = p.Hq / p.Hkv;
  const long long grid = 8LL * p.groups_per_xcd * gsz * p.n_qtiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipExtLaunchKernelGGL(step_mfma_bf16_d128, dim3((unsigned)grid), dim3(kThreads), 0, stream, ev_start, ev_stop, 0, p);
  return hipGetLastError();
}

}  // namespace ra
