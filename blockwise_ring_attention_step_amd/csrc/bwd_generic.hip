// Generic backward step kernels (fp32 arithmetic; fp32 or bf16 storage; any head dim <= 128).
//
// The correctness path beside the bf16 head-dim-128 MFMA kernels, on the same BwdParams and the same
// reading of the backward of the ring (the pages use ring attention for training, Ultralytics
// glossary "Ring Attention", section "Aplicações"): for one (query block, key/value block) pair, the
// exact gradient of attention restricted to the pair, with P recomputed from the forward's
// log-sum-exp:
//   x = log2(e) * scale * q.k,  p = 2^(x - lse2),  dp = dO.v,  ds = p * (dp - delta),
//   dq += scale * ds k,  dk += scale * ds q,  dv += p dO.
// Two kernels, so that every output row has one owner (no atomics): one walks the visible keys of a
// query row (dq), the other the query rows of every query head of the group that see a key (dk, dv).
// Layout as the generic forward step: 16 lanes per row, lane `sub` owns dims sub, sub + 16, ...; the
// dot products are reduced across the 16 lanes with xor shuffles.
#include "internal.h"

namespace ra {
namespace {

constexpr int kLanesPerRow = 16;
constexpr int kRowsPerBlock = 16;
constexpr int kMaxPerLane = RA_MAX_D / kLanesPerRow;  // 8

template <bool BF16>
__device__ __forceinline__ float elem(const void* base, size_t i) {
  if constexpr (BF16)
    return __uint_as_float((unsigned)((const unsigned short*)base)[i] << 16);
  else
    return ((const float*)base)[i];
}

__device__ __forceinline__ float row_sum(float part) {
#pragma unroll
  for (int w = kLanesPerRow / 2; w >= 1; w /= 2) part += __shfl_xor(part, w, kLanesPerRow);
  return part;
}

// grid (query-row groups of 16, Hq, n_launch * B)
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_dq_generic(const BwdParams p) {
  const int sub = threadIdx.x % kLanesPerRow;
  const int r = blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;  // row in the slot's window
  const int h = blockIdx.y;
  const int dl = blockIdx.z / p.B, bb = blockIdx.z % p.B;
  if (r >= p.Nq) return;  // whole 16-lane groups leave together
  const int D = p.D, Hq = p.Hq, Hkv = p.Hkv;
  const int kvh = h / (Hq / Hkv);
  const int qdev = p.qslot[dl], kvdev = p.kvslot[dl];
  const int nk = p.nk[dl], row = p.q_row0[dl] + r;
  int kmax = nk - 1;
  if (p.causal) {
    const int64_t d = p.q_off[dl] + (int64_t)r * p.q_stride - p.k_off[dl];
    kmax = d < 0 ? -1 : (int)(d / p.k_stride < (int64_t)(nk - 1) ? d / p.k_stride : nk - 1);
  }
  const size_t qoff = (((size_t)qdev * p.B + bb) * p.NqTot + row) * Hq * D + (size_t)h * D;
  float q[kMaxPerLane], dout[kMaxPerLane], acc[kMaxPerLane];
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int d = sub + kLanesPerRow * e;
    q[e] = d < D ? elem<BF16>(p.q, qoff + d) : 0.f;
    dout[e] = d < D ? elem<BF16>(p.dout, qoff + d) : 0.f;
    acc[e] = 0.f;
  }
  const size_t srow = (((size_t)qdev * p.B + bb) * Hq + h) * p.NqTot + row;
  const float lse2 = p.lse2[srow], delta = p.delta[srow];
  const size_t kvrow = (size_t)Hkv * D;
  const size_t kvbase = (((size_t)kvdev * p.B + bb) * p.NkTot) * kvrow + (size_t)kvh * D;
  for (int u = 0; u <= kmax; ++u) {
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int d = sub + kLanesPerRow * e;
      if (d < D) {
        s = __builtin_fmaf(q[e], elem<BF16>(p.k, kvbase + u * kvrow + d), s);
        dp = __builtin_fmaf(dout[e], elem<BF16>(p.v, kvbase + u * kvrow + d), dp);
      }
    }
    s = row_sum(s);
    dp = row_sum(dp);
    const float pr = exp2f(s * p.scale_log2 - lse2);  // 0 for a row that saw no key (lse2 = +inf)
    const float ds = pr * (dp - delta);
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int d = sub + kLanesPerRow * e;
      if (d < D) acc[e] = __builtin_fmaf(ds, elem<BF16>(p.k, kvbase + u * kvrow + d), acc[e]);
    }
  }
  float* dq = p.dq + qoff;
  const bool init = p.flags[dl] & kBwdInitDq;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int d = sub + kLanesPerRow * e;
    if (d < D) dq[d] = (init ? 0.f : dq[d]) + p.scale * acc[e];
  }
}

// grid (key-row groups of 16, Hkv, n_launch * B)
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_dkv_generic(const BwdParams p) {
  const int sub = threadIdx.x % kLanesPerRow;
  const int u = blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;  // key row
  const int kvh = blockIdx.y;
  const int dl = blockIdx.z / p.B, bb = blockIdx.z % p.B;
  const int nk = p.nk[dl];
  if (u >= nk) return;
  const int D = p.D, Hq = p.Hq, Hkv = p.Hkv, gsz = Hq / Hkv, Nq = p.Nq;
  const int qdev = p.qslot[dl], kvdev = p.kvslot[dl], gdev = p.gslot[dl];
  int rmin = 0;  // first query row of the window that sees key u
  if (p.causal) {
    const int64_t d = p.k_off[dl] + (int64_t)u * p.k_stride - p.q_off[dl];
    if (d > 0) {
      const int64_t rr = (d + p.q_stride - 1) / p.q_stride;
      rmin = rr < (int64_t)Nq ? (int)rr : Nq;
    }
  }
  const size_t kvrow = (size_t)Hkv * D;
  const size_t koff = (((size_t)kvdev * p.B + bb) * p.NkTot + u) * kvrow + (size_t)kvh * D;
  float k[kMaxPerLane], v[kMaxPerLane], dk[kMaxPerLane], dv[kMaxPerLane];
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int d = sub + kLanesPerRow * e;
    k[e] = d < D ? elem<BF16>(p.k, koff + d) : 0.f;
    v[e] = d < D ? elem<BF16>(p.v, koff + d) : 0.f;
    dk[e] = dv[e] = 0.f;
  }
  for (int hq = 0; hq < gsz; ++hq) {
    const int h = kvh * gsz + hq;
    for (int r = rmin; r < Nq; ++r) {
      const int row = p.q_row0[dl] + r;
      const size_t qoff = (((size_t)qdev * p.B + bb) * p.NqTot + row) * Hq * D + (size_t)h * D;
      const size_t srow = (((size_t)qdev * p.B + bb) * Hq + h) * p.NqTot + row;
      float qv[kMaxPerLane], dov[kMaxPerLane];
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) {
        const int d = sub + kLanesPerRow * e;
        qv[e] = d < D ? elem<BF16>(p.q, qoff + d) : 0.f;
        dov[e] = d < D ? elem<BF16>(p.dout, qoff + d) : 0.f;
        s = __builtin_fmaf(qv[e], k[e], s);
        dp = __builtin_fmaf(dov[e], v[e], dp);
      }
      s = row_sum(s);
      dp = row_sum(dp);
      const float pr = exp2f(s * p.scale_log2 - p.lse2[srow]);
      const float ds = pr * (dp - p.delta[srow]);
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) {
        dv[e] = __builtin_fmaf(pr, dov[e], dv[e]);
        dk[e] = __builtin_fmaf(ds, qv[e], dk[e]);
      }
    }
  }
  const size_t goff = (((size_t)gdev * p.B + bb) * p.NkTot + u) * kvrow + (size_t)kvh * D;
  const bool init = p.flags[dl] & kBwdInitDkv;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int d = sub + kLanesPerRow * e;
    if (d < D) {
      p.dk[goff + d] = (init ? 0.f : p.dk[goff + d]) + p.scale * dk[e];
      p.dv[goff + d] = (init ? 0.f : p.dv[goff + d]) + dv[e];
    }
  }
}

}  // namespace

hipError_t launch_bwd_generic(const BwdParams& p, int dtype, bool dq_pass, hipStream_t stream) {
  const long long z = (long long)p.n_launch * p.B;
  if (z <= 0) return hipSuccess;
  if (z > 65535 || p.Hq > 65535) return hipErrorInvalidConfiguration;
  for (int x = 0; x < p.n_launch; ++x)
    if (p.nk2[x] != 0 || p.two_q[x]) return hipErrorInvalidValue;  // one block, one query device per slot here
  const int rows = dq_pass ? p.Nq : p.Nk;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)(dq_pass ? p.Hq : p.Hkv),
                  (unsigned)z);
  if (dq_pass) {
    if (dtype == RA_BF16)
      hipLaunchKernelGGL(bwd_dq_generic<true>, grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL(bwd_dq_generic<false>, grid, dim3(256), 0, stream, p);
  } else {
    if (dtype == RA_BF16)
      hipLaunchKernelGGL(bwd_dkv_generic<true>, grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL(bwd_dkv_generic<false>, grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace ra
