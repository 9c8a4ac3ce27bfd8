// Shared host/device definitions of the ring-attention HIP library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ring_attn.h"

namespace ra {

// Per-device flags inside one step launch.
enum : uint8_t {
  kDevInit = 1,   // ignore incoming state (first block folded by this device)
  kDevFinal = 2,  // last block of this device: write o = o_acc / l and lse instead of the state
};

// Key/value blocks a step launch reads or writes are named by a reference: source index * 65536 +
// block index, the block's keys at kv_base[source][0] + block * kv_block and its values at
// kv_base[source][1] + block * kv_block (each a [B, NkTot, Hkv, D] array).
constexpr int kMaxSub = 2;  // key/value blocks one launch slot folds in sequence (ring steps per launch)
__host__ __device__ inline int kv_ref(int source, int block) { return source * 65536 + block; }

// Everything one step launch needs.  Passed by value as the kernel argument (about 3.6 KiB).
// Launch slot t addresses q, state and outputs at index slot[t] of their leading [n_dev] dimension.
// Within it, slot t works on the query rows [q_row0[t], q_row0[t] + Nq) of the NqTot rows that the q,
// o_acc, m, l, o_out and lse_out arrays hold per (device, batch), and folds nsub[t] key/value blocks
// in order: block kv_ref[t][b] with keys [0, nk[t][b]) of its NkTot rows and first key position
// k_off[t][b].  The running state stays in registers from one block to the next and is merged with
// the incoming state once.
struct StepParams {
  const void* q;       // [n_dev, B, NqTot, Hq, D]
  char* kv_base[3][2];  // key/value block sources (see kv_ref); written only through fwd_ref
  int64_t kv_block;    // bytes of one block: B * NkTot * Hkv * D * element size
  float* o_acc;        // [n_dev, B, Hq, NqTot, D]
  float* m;            // [n_dev, B, Hq, NqTot]
  float* l;            // [n_dev, B, Hq, NqTot]
  void* o_out;         // [n_dev, B, NqTot, Hq, D] (slots with kDevFinal)
  float* lse_out;      // [n_dev, B, Hq, NqTot] or null
  int n_launch;
  int B, Hq, Hkv, Nq, Nk, D;  // Nq: query rows per slot; Nk: the largest nk[t][b]
  int NqTot, NkTot;
  int causal;
  float scale_log2;  // scale * log2(e)
  int64_t q_stride, k_stride;
  // XCD-aware work decomposition, filled in by the MFMA kernel's launcher: groups = n_launch*B*Hkv
  int groups, groups_per_xcd, n_qtiles;
  int slot[RA_MAX_DEV];
  int64_t q_off[RA_MAX_DEV];
  int q_row0[RA_MAX_DEV];
  uint8_t dflags[RA_MAX_DEV];
  uint8_t nsub[RA_MAX_DEV];  // 1 or 2 (2 only in the bf16 D=128 kernel)
  int kv[RA_MAX_DEV][kMaxSub];
  int64_t k_off[RA_MAX_DEV][kMaxSub];
  int nk[RA_MAX_DEV][kMaxSub];
  // Ring hop inside the step (bf16 D=128 kernel; -1: none).  The key/value rows of the slot's last
  // block that it stages for its computation are also written to block fwd[t] (the next device's
  // receive slot), by the workgroups of the first query head of each key/value head, each the 256 keys
  // that line up with its query tile.
  int fwd[RA_MAX_DEV];
};
static_assert(sizeof(StepParams) <= 4096, "kernel argument block");

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

// Work geometry of the bf16 D=128 step kernel that the host also needs (the in-step hop): query rows
// per workgroup and keys per tile.
constexpr int kMfmaRowsPerWg = 256;
constexpr int kMfmaKeysPerTile = 64;

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
