// bf16 ring-attention step kernel for gfx950 (CDNA4), head dim 128, on v_mfma_f32_32x32x16_bf16.
//
// One workgroup (4 waves, 256 threads) folds one key/value block into the online-softmax state of
// 128 query rows of one (device, batch, query head).  This is the per-step work of the Ultralytics
// glossary page "Ring Attention", section "Como funciona a atenção em anel" (attend the held block,
// accumulate exponentiated scores and weighted values), with the running-maximum rescaling of
// "Sequence Parallelism and Ring Attention", section "Approfondimento tecnico".
//
// Data flow per 64-key tile:
//   HBM --global_load_lds (16 B/lane, no VGPR staging)--> LDS K and V tiles (double-buffered)
//   S^T[key, query] = K . Q^T          32x32x16 MFMA: A = K rows from LDS, B = Q^T held in VGPRs
//   online softmax in registers        lane j (mod 32) owns query j; its 32 keys per tile sit in its
//                                      own registers, the other 32 in lane j^32: a row max needs
//                                      one permlane32 swap, the row sum none (halves are summed once
//                                      at the end)
//   O^T[d, query] += V^T . P^T         A = V^T via ds_read_b64_tr_b16 (LDS transpose read), B = P^T
//                                      straight from the S^T accumulators converted to bf16
// Because every lane owns one query row in both accumulators, rescaling O by exp2(m_old - m_new)
// is a per-lane scalar multiply.  Rescaling is lazy: the reference exponent m only moves when a
// tile's maximum exceeds it by more than 8 (so exponentials stay <= 2^8), which leaves the final
// quotient exact and skips almost every rescale after the first tile.
//
// LDS layout of a tile: 64 rows (keys) x 256 B, the 16-byte chunk c of row r stored at chunk
// c ^ swz(r) with swz(r) = 4*(r%4) + (r/4)%4.  This makes both the 16-lane groups of the K reads
// (16 consecutive rows, one chunk) and the 32-lane groups of the transpose reads (4 consecutive
// rows x 4 chunks) hit distinct banks.
#include "internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kD = 128;
constexpr int kBr = 128;                      // query rows per workgroup
constexpr int kBc = 64;                       // keys per tile
constexpr int kThreads = 256;
constexpr int kRowBytes = kD * 2;             // one key row of K or V in LDS
constexpr int kTileBytes = kBc * kRowBytes;   // 16 KiB
constexpr int kStageBytes = 2 * kTileBytes;   // K tile + V tile
constexpr int kStages = 2;
constexpr float kLazySlack = 8.0f;            // log2 units
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ float partner(float x) {
  // value held by lane (lane ^ 32)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned lane = __lane_id();
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// This wave's quarter of the K and V tiles starting at key0: 4 x 1 KiB pieces each, 16 B per lane.
__device__ __forceinline__ void issue_tile_loads(const char* kbase, const char* vbase, int64_t row_bytes, int key0,
                                                 int nk, LDS_AS char* stage, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int piece = wave * 4 + i;
    const int row = piece * 4 + (lane >> 4);
    const int lchunk = (lane & 15) ^ swz(row);
    int key = key0 + row;
    key = key < nk ? key : nk - 1;  // ragged tail: load a valid row, the mask drops it
    const int64_t off = (int64_t)key * row_bytes + lchunk * 16;
    __builtin_amdgcn_global_load_lds((const void*)(kbase + off), (LDS_AS void*)(stage + piece * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(vbase + off), (LDS_AS void*)(stage + kTileBytes + piece * 1024),
                                     16, 0, 0);
  }
}

// Largest key index visible to the query at local row `row` (causal), clamped to [-1, nk-1].
__device__ __forceinline__ int last_visible_key(const StepParams& p, int dl, int row, int nk) {
  const int64_t pq = p.q_off[dl] + (int64_t)row * p.q_stride;
  const int64_t d = pq - p.k_off[dl];
  if (d < 0) return -1;
  const int64_t kk = d / p.k_stride;
  return kk < (int64_t)(nk - 1) ? (int)kk : nk - 1;
}

__global__ __launch_bounds__(kThreads, 2) void step_mfma_bf16_d128(const StepParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStages * kStageBytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int Nq = p.Nq, Nk = p.Nk, Hq = p.Hq;

  const int qrow0 = qt * kBr;
  const int qr = qrow0 + wave * 32 + j;
  const bool qvalid = qr < Nq;
  const int qlast = min(qrow0 + kBr, Nq) - 1;

  // key range of this workgroup and the per-lane causal limit
  int kmax_lane = Nk - 1, kmin_wg = Nk - 1, kend_wg = Nk - 1;
  if (p.causal) {
    kmax_lane = last_visible_key(p, dl, qvalid ? qr : qlast, Nk);
    kmin_wg = last_visible_key(p, dl, qrow0, Nk);
    kend_wg = last_visible_key(p, dl, qlast, Nk);
  }
  const int ntiles = kend_wg < 0 ? 0 : kend_wg / kBc + 1;
  const int nfull = kmin_wg < 0 ? 0 : (kmin_wg + 1) / kBc;  // tiles [0, nfull) need no mask

  // ---- Q^T fragments (B operand): lane holds q[row qr][16*kk + 8*h2 .. +7]
  const size_t q_dev = (size_t)p.B * Nq * Hq * kD;
  const unsigned short* qrow =
      (const unsigned short*)p.q + dev * q_dev + ((size_t)bb * Nq + (qvalid ? qr : 0)) * Hq * kD + h * kD + 8 * h2;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    i16x8 raw = qvalid ? *(const i16x8*)(qrow + 16 * kk) : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
    qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }

  const size_t kv_dev = (size_t)p.B * Nk * p.Hkv * kD;
  const size_t kv_off = 2 * (dev * kv_dev + (size_t)bb * Nk * p.Hkv * kD + (size_t)kvh * kD);
  const char* kbase = (const char*)p.k + kv_off;
  const char* vbase = (const char*)p.v + kv_off;
  const int64_t row_bytes = (int64_t)p.Hkv * kD * 2;

  // per-lane LDS offsets
  const int kswz = swz(j);  // rows 32c + j share swz(j)
  const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
  // transpose-read row inside a 16-key step: 8*r' + 4*(tg>>1) + te; chunk 4*dt + 2*(tg&1) + (tq>>1)
  int vrow_off[2], vswz[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    vrow_off[rr] = 8 * rr + 4 * (tg >> 1) + te;
    vswz[rr] = (te << 2) | ((2 * rr + (tg >> 1)) & 3);
  }
  const int vchunk0 = 2 * (tg & 1) + (tq >> 1);
  const int vbyte = 8 * (tq & 1);

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float M = -INFINITY;  // reference exponent (log2 units)
  float lsum = 0.f;     // this lane's partial sum of 2^(x - M) over its keys
  const float c = p.scale_log2;

  if (ntiles > 0) issue_tile_loads(kbase, vbase, row_bytes, 0, Nk, smem, wave, lane);

  for (int t = 0; t < ntiles; ++t) {
    LDS_AS char* st = smem + (t & 1) * kStageBytes;
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < ntiles)
      issue_tile_loads(kbase, vbase, row_bytes, (t + 1) * kBc, Nk, smem + ((t + 1) & 1) * kStageBytes, wave, lane);

    // ---- S^T = K Q^T for keys [64t, 64t+64): two 32-key chunks
    f32x16 s[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      s[cc] = f32x16{};
      const LDS_AS char* krow = st + (32 * cc + j) * kRowBytes;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int pch = (2 * kk + h2) ^ kswz;
        bf16x8 kf = __builtin_bit_cast(bf16x8, *(const LDS_AS i16x8*)(krow + pch * 16));
        s[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[cc], 0, 0, 0);
      }
    }

    // ---- mask (diagonal / ragged tiles only): key index of register r of chunk cc
    if (t >= nfull) {
      const int kbase_idx = t * kBc + 4 * h2;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase_idx + 32 * cc + 8 * (r >> 2) + (r & 3);
          if (key > kmax_lane) s[cc][r] = -INFINITY;
        }
    }

    // ---- online softmax
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, partner(mx));
    const float mxs = mx * c;
    const bool need = mxs > M + kLazySlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float Mn = fmaxf(M, mxs);
      const float alpha = Mn > M ? __builtin_amdgcn_exp2f(M - Mn) : 1.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      lsum *= alpha;
      M = Mn;
    }
    const float negM = M == -INFINITY ? 0.f : -M;
    // P = 2^(x - M): summed in fp32 into the normaliser (this keeps the log-sum-exp exact to fp32),
    // rounded to bf16 for the P.V product
    bf16x8 pf[4];
    float lpart[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cc][r], c, negM));
        lpart[r & 3] += e;
        pf[2 * cc + (r >> 3)][r & 7] = (__bf16)e;
      }
    lsum += (lpart[0] + lpart[1]) + (lpart[2] + lpart[3]);

    // ---- O^T += V^T P^T
    const LDS_AS char* vt = st + kTileBytes;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(vt + (16 * kb + vrow_off[0]) * kRowBytes + (((4 * dt + vchunk0) ^ vswz[0]) * 16) + vbyte));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(vt + (16 * kb + vrow_off[1]) * kRowBytes + (((4 * dt + vchunk0) ^ vswz[1]) * 16) + vbyte));
        i16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[kb], o[dt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: merge with the incoming state (or finalize)
  lsum += partner(lsum);
  if (!qvalid) return;
  const size_t srow = ((size_t)(dev * p.B + bb) * Hq + h) * Nq + qr;
  float Mo = -INFINITY, lo = 0.f;
  const bool has_old = !(dfl & kDevInit);
  if (has_old) {
    Mo = p.m[srow];
    lo = p.l[srow];
  }
  const float Mf = fmaxf(Mo, M);
  const float ao = Mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mo - Mf);
  const float an = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
  const float lf = ao * lo + an * lsum;
  float* oacc_row = p.o_acc + srow * kD;

  if (dfl & kDevFinal) {
    const float inv = lf > 0.f ? 1.0f / lf : 0.f;
    unsigned short* orow =
        (unsigned short*)p.o_out + (((size_t)dev * p.B + bb) * Nq + qr) * (size_t)Hq * kD + (size_t)h * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * h2;
        f32x4 old = has_old ? *(const f32x4*)(oacc_row + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
        u16x4 outv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float val = (ao * old[i] + an * o[dt][4 * gq + i]) * inv;
          outv[i] = __builtin_bit_cast(unsigned short, (__bf16)val);
        }
        *(u16x4*)(orow + d0) = outv;
      }
    if (h2 == 0 && p.lse_out) p.lse_out[srow] = lf > 0.f ? (Mf + log2f(lf)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * h2;
        f32x4 old = has_old ? *(const f32x4*)(oacc_row + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 nv;
#pragma unroll
        for (int i = 0; i < 4; ++i) nv[i] = ao * old[i] + an * o[dt][4 * gq + i];
        *(f32x4*)(oacc_row + d0) = nv;
      }
    if (h2 == 0) {
      p.m[srow] = Mf;
      p.l[srow] = lf;
    }
  }
}

}  // namespace

hipError_t launch_step_mfma_bf16_d128(const StepParams& p, hipStream_t stream) {
  const int gsz = p.Hq / p.Hkv;
  const long long grid = 8LL * p.groups_per_xcd * gsz * p.n_qtiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(step_mfma_bf16_d128, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
