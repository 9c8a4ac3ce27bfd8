// Generic ring-attention step kernel (fp32 arithmetic; fp32 or bf16 storage; any head dim <= 128),
// plus the finalize and state-initialisation kernels.
//
// The generic step is the straightforward form of the per-step fold on the Ultralytics glossary
// page "Ring Attention", section "Como funciona a atenção em anel", with the exact running maximum
// of "Sequence Parallelism and Ring Attention", section "Approfondimento tecnico": keys are taken
// one at a time, the state is rescaled whenever a key raises the maximum.  It serves the fp32 path,
// head dims other than 128 and small shapes; the bf16 head-dim-128 hot path has its own MFMA kernel.
//
// Layout: 16 lanes cooperate on one query row (lane `sub` owns dims sub, sub+16, ...), 16 rows per
// 256-thread workgroup; the dot product is reduced across the 16 lanes with xor shuffles.
#include <hip/hip_ext.h>

#include <algorithm>

#include "internal.h"

namespace ra {
namespace {

constexpr int kLanesPerRow = 16;
constexpr int kRowsPerBlock = 16;
constexpr int kMaxPerLane = RA_MAX_D / kLanesPerRow;  // 8
constexpr float kLn2 = 0.693147180559945309f;

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
  if constexpr (BF16) {
    const unsigned short b = ((const unsigned short*)base)[i];
    return __uint_as_float((unsigned)b << 16);
  } else {
    return ((const float*)base)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* base, size_t i, float x) {
  if constexpr (BF16) {
    ((unsigned short*)base)[i] = __builtin_bit_cast(unsigned short, (__bf16)x);
  } else {
    ((float*)base)[i] = x;
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void step_generic(const StepParams p) {
  const int sub = threadIdx.x % kLanesPerRow;
  const int qr = blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int h = blockIdx.y;
  const int dl = blockIdx.z / p.B;
  const int bb = blockIdx.z % p.B;
  if (qr >= p.Nq) return;  // whole 16-lane groups leave together
  const int D = p.D, Hq = p.Hq, Hkv = p.Hkv;
  const int dev = p.slot[dl];
  const int Nk = p.nk[dl][0], NqT = p.NqTot, NkT = p.NkTot, row = p.q_row0[dl] + qr;  // array row of this query
  const int dfl = p.dflags[dl];
  const int kvh = h / (Hq / Hkv);

  float q[kMaxPerLane], o[kMaxPerLane];
  const size_t qoff = (((size_t)dev * p.B + bb) * NqT + row) * Hq * D + (size_t)h * D;
#pragma unroll
  for (int e = 0; e < kMaxPerLane; ++e) {
    const int d = sub + kLanesPerRow * e;
    q[e] = d < D ? load_elem<BF16>(p.q, qoff + d) : 0.f;
    o[e] = 0.f;
  }

  int kmax = Nk - 1;
  if (p.causal) {
    const int64_t dpos = p.q_off[dl] + (int64_t)qr * p.q_stride - p.k_off[dl][0];
    if (dpos < 0) {
      kmax = -1;
    } else {
      const int64_t kk = dpos / p.k_stride;
      kmax = kk < (int64_t)(Nk - 1) ? (int)kk : Nk - 1;
    }
  }

  const float c = p.scale_log2;
  float M = -INFINITY, l = 0.f;
  const size_t kvrow = (size_t)Hkv * D;
  const size_t kvbase = (size_t)bb * NkT * kvrow + (size_t)kvh * D;  // elements into this slot's block
  const int ref = p.kv[dl][0];
  const char* kblock = p.kv_base[ref >> 16][0] + (int64_t)(ref & 0xffff) * p.kv_block;
  const char* vblock = p.kv_base[ref >> 16][1] + (int64_t)(ref & 0xffff) * p.kv_block;
  for (int u = 0; u <= kmax; ++u) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int d = sub + kLanesPerRow * e;
      if (d < D) part = __builtin_fmaf(q[e], load_elem<BF16>(kblock, kvbase + u * kvrow + d), part);
    }
#pragma unroll
    for (int w = kLanesPerRow / 2; w >= 1; w /= 2) part += __shfl_xor(part, w, kLanesPerRow);
    const float x = part * c;
    if (x > M) {
      const float alpha = exp2f(M - x);  // 0 when M = -inf
#pragma unroll
      for (int e = 0; e < kMaxPerLane; ++e) o[e] *= alpha;
      l *= alpha;
      M = x;
    }
    const float pr = exp2f(x - M);
    l += pr;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int d = sub + kLanesPerRow * e;
      if (d < D) o[e] = __builtin_fmaf(pr, load_elem<BF16>(vblock, kvbase + u * kvrow + d), o[e]);
    }
  }

  // merge with the incoming state
  const size_t srow = (((size_t)dev * p.B + bb) * Hq + h) * NqT + row;
  const bool has_old = !(dfl & kDevInit);
  const float Mo = has_old ? p.m[srow] : -INFINITY;
  const float lo = has_old ? p.l[srow] : 0.f;
  const float Mf = fmaxf(Mo, M);
  const float ao = Mo == -INFINITY ? 0.f : exp2f(Mo - Mf);
  const float an = M == -INFINITY ? 0.f : exp2f(M - Mf);
  const float lf = ao * lo + an * l;
  float* oacc = p.o_acc + srow * D;
  if (dfl & kDevFinal) {
    const float inv = lf > 0.f ? 1.0f / lf : 0.f;
    const size_t ooff = (((size_t)dev * p.B + bb) * NqT + row) * Hq * D + (size_t)h * D;
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int d = sub + kLanesPerRow * e;
      if (d < D) store_elem<BF16>(p.o_out, ooff + d, (ao * (has_old ? oacc[d] : 0.f) + an * o[e]) * inv);
    }
    if (sub == 0 && p.lse_out) p.lse_out[srow] = lf > 0.f ? (Mf + log2f(lf)) * kLn2 : -INFINITY;
  } else {
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
      const int d = sub + kLanesPerRow * e;
      if (d < D) oacc[d] = ao * (has_old ? oacc[d] : 0.f) + an * o[e];
    }
    if (sub == 0) {
      p.m[srow] = Mf;
      p.l[srow] = lf;
    }
  }
}

// o[dev, b, t, h, :] = o_acc[dev, b, h, t, :] / l ; lse = ln2 * (m + log2 l).  One thread per output element.
template <bool BF16>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ o_acc, const float* __restrict__ m,
                                                       const float* __restrict__ l, void* __restrict__ o,
                                                       float* __restrict__ lse, int B, int Hq, int Nq, int D,
                                                       size_t total) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int d = (int)(i % D);
  size_t r = i / D;
  const int h = (int)(r % Hq);
  r /= Hq;
  const int t = (int)(r % Nq);
  const size_t db = r / Nq;  // dev * B + b
  const size_t srow = (db * Hq + h) * Nq + t;
  const float lv = l[srow];
  const float val = lv > 0.f ? o_acc[srow * D + d] / lv : 0.f;
  store_elem<BF16>(o, i, val);
  if (d == 0 && lse) lse[srow] = lv > 0.f ? (m[srow] + log2f(lv)) * kLn2 : -INFINITY;
}

// The same for D % 4 == 0, four consecutive d per thread: rows are taken in output order (token-major,
// then head), so the D/4 threads of a row store one contiguous run and read one 16 D-byte run of
// o_acc; 256 / (D/4) rows per workgroup.
template <bool BF16>
__global__ __launch_bounds__(256) void finalize_vec_kernel(const float* __restrict__ o_acc, const float* __restrict__ m,
                                                           const float* __restrict__ l, void* __restrict__ o,
                                                           float* __restrict__ lse, int B, int Hq, int Nq, int D,
                                                           size_t rows) {
  const int tpr = D / 4;  // threads per row
  const int rows_per_block = 256 / tpr;
  const int sub = threadIdx.x % tpr;
  const size_t row = (size_t)blockIdx.x * rows_per_block + threadIdx.x / tpr;  // output order: (db, t, h)
  if ((int)threadIdx.x >= rows_per_block * tpr || row >= rows) return;
  const int h = (int)(row % Hq);
  size_t r = row / Hq;
  const int t = (int)(r % Nq);
  const size_t db = r / Nq;
  const size_t srow = (db * Hq + h) * Nq + t;
  const float lv = l[srow];
  const float inv = lv > 0.f ? 1.0f / lv : 0.f;
  const float4 a = *(const float4*)(o_acc + srow * D + 4 * sub);
  const float vals[4] = {a.x * inv, a.y * inv, a.z * inv, a.w * inv};
  const size_t oi = row * D + 4 * sub;
  if constexpr (BF16) {
    ushort4 ov;
    ov.x = __builtin_bit_cast(unsigned short, (__bf16)vals[0]);
    ov.y = __builtin_bit_cast(unsigned short, (__bf16)vals[1]);
    ov.z = __builtin_bit_cast(unsigned short, (__bf16)vals[2]);
    ov.w = __builtin_bit_cast(unsigned short, (__bf16)vals[3]);
    *(ushort4*)((unsigned short*)o + oi) = ov;
  } else {
    *(float4*)((float*)o + oi) = make_float4(vals[0], vals[1], vals[2], vals[3]);
  }
  if (sub == 0 && lse) lse[srow] = lv > 0.f ? (m[srow] + log2f(lv)) * kLn2 : -INFINITY;
}

// The same for D % 16 == 0 with four independent 16-byte loads per thread: D/16 threads per row, a
// thread's four float4 D/16 float4 apart, so that each load instruction of a row's threads still reads
// one contiguous run.  Four times the loads in flight per wave, which this HBM-bound kernel needs to
// approach the bandwidth.
template <bool BF16>
__global__ __launch_bounds__(256) void finalize_vec16_kernel(const float* __restrict__ o_acc, const float* __restrict__ m,
                                                             const float* __restrict__ l, void* __restrict__ o,
                                                             float* __restrict__ lse, int B, int Hq, int Nq, int D,
                                                             size_t rows) {
  const int tpr = D / 16;  // threads per row
  const int rows_per_block = 256 / tpr;
  const int sub = threadIdx.x % tpr;
  const size_t row = (size_t)blockIdx.x * rows_per_block + threadIdx.x / tpr;  // output order: (db, t, h)
  if ((int)threadIdx.x >= rows_per_block * tpr || row >= rows) return;
  const int h = (int)(row % Hq);
  size_t r = row / Hq;
  const int t = (int)(r % Nq);
  const size_t db = r / Nq;
  const size_t srow = (db * Hq + h) * Nq + t;
  float4 a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = *(const float4*)(o_acc + srow * D + 4 * (sub + k * tpr));
  const float lv = l[srow];
  const float inv = lv > 0.f ? 1.0f / lv : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float vals[4] = {a[k].x * inv, a[k].y * inv, a[k].z * inv, a[k].w * inv};
    const size_t oi = row * D + 4 * (sub + k * tpr);
    if constexpr (BF16) {
      ushort4 ov;
      ov.x = __builtin_bit_cast(unsigned short, (__bf16)vals[0]);
      ov.y = __builtin_bit_cast(unsigned short, (__bf16)vals[1]);
      ov.z = __builtin_bit_cast(unsigned short, (__bf16)vals[2]);
      ov.w = __builtin_bit_cast(unsigned short, (__bf16)vals[3]);
      *(ushort4*)((unsigned short*)o + oi) = ov;
    } else {
      *(float4*)((float*)o + oi) = make_float4(vals[0], vals[1], vals[2], vals[3]);
    }
  }
  if (sub == 0 && lse) lse[srow] = lv > 0.f ? (m[srow] + log2f(lv)) * kLn2 : -INFINITY;
}

// Empty state (m = -inf, l = 0, o_acc = 0) for the listed device slots.
__global__ __launch_bounds__(256) void init_state_kernel(float* o_acc, float* m, float* l, int slot, size_t rows,
                                                         int D) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t base = (size_t)slot * rows;
  if (i < rows) {
    m[base + i] = -INFINITY;
    l[base + i] = 0.f;
  }
  if (i < rows * D) o_acc[base * D + i] = 0.f;
}

// Every 16-bit word of [p, p + n) set to `value` (grid-stride loop).
__global__ __launch_bounds__(256) void fill_u16_kernel(uint16_t* __restrict__ p, size_t n, uint16_t value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// One wave that sleeps for `rounds` rounds of the longest s_sleep (64 x 127 clocks each) and exits.
__global__ __launch_bounds__(64) void spin_kernel(unsigned rounds) {
  for (unsigned r = 0; r < rounds; ++r) __builtin_amdgcn_s_sleep(127);
}

}  // namespace

hipError_t launch_fill_u16(void* p, size_t n_words, uint16_t value, hipStream_t stream) {
  if (n_words == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n_words + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_u16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint16_t*)p, n_words, value);
  return hipGetLastError();
}

hipError_t launch_spin(unsigned rounds, hipStream_t stream) {
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, stream, rounds);
  return hipGetLastError();
}

hipError_t launch_step_generic(const StepParams& p, int dtype, hipStream_t stream, hipEvent_t ev_start,
                               hipEvent_t ev_stop) {
  if (p.Nq == 0 || p.n_launch == 0) return hipSuccess;
  dim3 grid((p.Nq + kRowsPerBlock - 1) / kRowsPerBlock, p.Hq, p.n_launch * p.B);
  if (dtype == RA_BF16)
    hipExtLaunchKernelGGL(step_generic<true>, grid, dim3(256), 0, stream, ev_start, ev_stop, 0, p);
  else
    hipExtLaunchKernelGGL(step_generic<false>, grid, dim3(256), 0, stream, ev_start, ev_stop, 0, p);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* o_acc, const float* m, const float* l, void* o, float* lse, int n_dev, int B,
                           int Hq, int Nq, int D, int out_dtype, hipStream_t stream) {
  const size_t total = (size_t)n_dev * B * Nq * Hq * D;
  if (total == 0) return hipSuccess;
  const size_t align = out_dtype == RA_BF16 ? 8 : 16;  // bytes of one thread's 4 outputs
  if (D % 16 == 0 && (uintptr_t)o_acc % 16 == 0 && (uintptr_t)o % align == 0) {
    const size_t rows = total / D;
    const size_t rows_per_block = 256 / (D / 16);
    const size_t vblocks = (rows + rows_per_block - 1) / rows_per_block;
    if (out_dtype == RA_BF16)
      hipLaunchKernelGGL(finalize_vec16_kernel<true>, dim3((unsigned)vblocks), dim3(256), 0, stream, o_acc, m, l, o,
                         lse, B, Hq, Nq, D, rows);
    else
      hipLaunchKernelGGL(finalize_vec16_kernel<false>, dim3((unsigned)vblocks), dim3(256), 0, stream, o_acc, m, l, o,
                         lse, B, Hq, Nq, D, rows);
    return hipGetLastError();
  }
  if (D % 4 == 0 && (uintptr_t)o_acc % 16 == 0 && (uintptr_t)o % align == 0) {
    const size_t rows = total / D;
    const size_t rows_per_block = 256 / (D / 4);
    const size_t vblocks = (rows + rows_per_block - 1) / rows_per_block;
    if (out_dtype == RA_BF16)
      hipLaunchKernelGGL(finalize_vec_kernel<true>, dim3((unsigned)vblocks), dim3(256), 0, stream, o_acc, m, l, o, lse,
                         B, Hq, Nq, D, rows);
    else
      hipLaunchKernelGGL(finalize_vec_kernel<false>, dim3((unsigned)vblocks), dim3(256), 0, stream, o_acc, m, l, o,
                         lse, B, Hq, Nq, D, rows);
    return hipGetLastError();
  }
  const size_t blocks = (total + 255) / 256;
  if (out_dtype == RA_BF16)
    hipLaunchKernelGGL(finalize_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, o_acc, m, l, o, lse, B, Hq,
                       Nq, D, total);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, o_acc, m, l, o, lse, B,
                       Hq, Nq, D, total);
  return hipGetLastError();
}

hipError_t launch_init_state(float* o_acc, float* m, float* l, int /*n_dev_total*/, const int* slots, int n_slots,
                             int B, int Hq, int Nq, int D, hipStream_t stream) {
  const size_t rows = (size_t)B * Hq * Nq;
  if (rows == 0) return hipSuccess;
  const size_t blocks = (rows * D + 255) / 256;
  for (int i = 0; i < n_slots; ++i) {
    hipLaunchKernelGGL(init_state_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o_acc, m, l, slots[i], rows,
                       D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ra
