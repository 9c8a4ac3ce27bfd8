// Shared host/device definitions of the ring-attention HIP library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ring_attn.h"
#include "step_params.h"

namespace ra {

// Per-slot flags of a backward step launch.
enum : uint8_t {
  kBwdInitDq = 1,   // overwrite this slot's query-gradient rows instead of adding to them
  kBwdInitDkv = 2,  // overwrite this slot's key/value-gradient rows instead of adding to them
};

// Everything one backward step launch needs (both kernels of it).  Launch slot t pairs the query
// rows [q_row0[t], q_row0[t] + Nq) of device qslot[t] (q, dout, lse2, delta, dq at that index of
// their leading dimension; NqTot rows per (device, batch)) with the keys [0, nk[t]) of the block
// in kvslot[t] of k and v, whose gradients accumulate at index gslot[t] of dk and dv (NkTot rows per
// (block, batch)).  Positions and masking as in StepParams.
struct BwdParams {
  const void* q;       // [.., B, NqTot, Hq, D]
  const void* k;       // [.., B, NkTot, Hkv, D]
  const void* v;
  const void* dout;    // like q: gradient of the attention output
  const float* lse2;   // [.., B, Hq, NqTot]: log2 of sum_u 2^(x_u), x = log2(e) * scale * q.k (forward)
  const float* delta;  // [.., B, Hq, NqTot]: sum_d dout * out of the row
  float* dq;           // [.., B, NqTot, Hq, D] fp32
  float* dk;           // [.., B, NkTot, Hkv, D] fp32
  float* dv;
  void* fwd_k;         // the next step's receive slot (like k), filled by bwd_dq where fwd[t] >= 0
  void* fwd_v;
  int n_launch;
  int B, Hq, Hkv, Nq, Nk, NqTot, NkTot, D;  // Nq: query rows per slot; Nk: the largest nk[t]
  int causal;
  float scale, scale_log2;
  int64_t q_stride, k_stride;
  int groups, groups_per_xcd, n_qtiles, n_ktiles;  // filled in by the launchers
  int qslot[RA_MAX_DEV];
  int kvslot[RA_MAX_DEV];
  int gslot[RA_MAX_DEV];
  int q_row0[RA_MAX_DEV];
  int nk[RA_MAX_DEV];
  int64_t q_off[RA_MAX_DEV];
  int64_t k_off[RA_MAX_DEV];
  uint8_t flags[RA_MAX_DEV];
  int fwd[RA_MAX_DEV];  // bwd_dq: device position in fwd_k / fwd_v that slot t's block is handed to, or -1
  // bwd_dq only: a second key/value block folded after the first in the same launch (two ring steps;
  // nk2[t] = 0: none).  With a second block, fwd[t] hands on the second block.
  int kvslot2[RA_MAX_DEV];
  int nk2[RA_MAX_DEV];
  int64_t k_off2[RA_MAX_DEV];
  // bwd_dkv only: where two_q[t] != 0, the query rows of device qslot2[t] (the same q_row0, position
  // q_off2[t]) also see slot t's block, folded after those of qslot[t] in the same launch
  uint8_t two_q[RA_MAX_DEV];
  int qslot2[RA_MAX_DEV];
  int64_t q_off2[RA_MAX_DEV];
};

// One projection of the blockwise feed-forward: out[m, n] = act(sum_k x[m, k] w[n, k] + bias[n]) in
// bf16, fp32 accumulation.  Rows are strided (elements); K and N are multiples of 64.
struct FfnGemmParams {
  const void* x;     // [M, K] bf16, row stride ldx
  const void* w;     // [N, K] bf16, row stride ldw
  const void* bias;  // [N] bf16
  void* out;         // [M, N] bf16, row stride ldo
  int M, N, K;
  int64_t ldx, ldw, ldo;
  int tiles_m, tiles_n;  // filled in by the launcher
};
constexpr int kFfnActNone = -1;  // activation code of the second projection (bias only)

// Launchers (defined in the kernel sources); return a hipError_t.
// ev_start / ev_stop (may be null): timing events stamped by the launch itself (no extra packets)
hipError_t launch_step_mfma_bf16_d128(const StepParams& p, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_step_generic(const StepParams& p, int dtype, hipStream_t stream, hipEvent_t ev_start,
                               hipEvent_t ev_stop);
hipError_t launch_bwd_dq_bf16_d128(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dkv_bf16_d128(const BwdParams& p, hipStream_t stream);
// the same two passes for every other (dtype, head dim): dq_pass selects the query-gradient kernel
hipError_t launch_bwd_generic(const BwdParams& p, int dtype, bool dq_pass, hipStream_t stream);
// delta[row] = sum_d dout * out and lse2[row] = log2(e) * lse[row], rows of [n_dev, B, Hq, Nq]
hipError_t launch_bwd_prep(const void* out, const void* dout, const float* lse, float* delta, float* lse2, int n_dev,
                           int B, int Hq, int Nq, int D, int dtype, hipStream_t stream);
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t stream);
// act: RA_FFN_GELU, RA_FFN_RELU or kFfnActNone
hipError_t launch_ffn_gemm_bf16(const FfnGemmParams& p, int act, hipStream_t stream);
hipError_t launch_finalize(const float* o_acc, const float* m, const float* l, void* o, float* lse, int n_dev,
                           int B, int Hq, int Nq, int D, int out_dtype, hipStream_t stream);
// Test hooks of the ring drivers: every 16-bit word of [p, p + 2 n_words) set to `value`; one wave
// that sleeps `rounds` x 8128 clocks (bounded) and exits.
hipError_t launch_fill_u16(void* p, size_t n_words, uint16_t value, hipStream_t stream);
hipError_t launch_spin(unsigned rounds, hipStream_t stream);
hipError_t launch_init_state(float* o_acc, float* m, float* l, int n_dev_total, const int* slots, int n_slots,
                             int B, int Hq, int Nq, int D, hipStream_t stream);

}  // namespace ra
