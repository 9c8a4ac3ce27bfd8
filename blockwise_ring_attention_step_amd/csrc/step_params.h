// Argument block of the forward step kernels (bf16 D=128 MFMA and generic): one launch folds one or
// two key/value blocks into the running state of each launch slot.  Shared by the host driver and the
// kernels (not part of the public ABI).
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

// Work geometry of the bf16 D=128 step kernel that the host also needs (the in-step hop): query rows
// per workgroup and keys per tile.
constexpr int kMfmaRowsPerWg = 256;
constexpr int kMfmaKeysPerTile = 64;

}  // namespace ra
