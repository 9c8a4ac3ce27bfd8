// C ABI of the ring-attention library: argument validation, the ring schedule (planner), the step
// and finalize entry points and the whole-ring driver with its copy/compute overlap.
//
// The schedule follows the Ultralytics glossary page "Ring Attention", section "Como funciona a
// atenção em anel": P steps; in step s device i holds key/value block j = (i - s) mod P, which it
// received from device i - 1 (the block that device held one step earlier).  The hop for step s+1
// runs on a second stream while step s computes, as "Ring Attention Là Gì?" (thienlv.com), section
// "Ring Attention Hoạt Động Thế Nào?", describes (the next block is already being sent during the
// current computation).  Causal blocks that are fully masked are skipped, which is the idle time of
// the first devices that the Ultralytics page attributes to causal masking.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace {

using ra::StepParams;

constexpr double kLog2e = 1.4426950408889634;

size_t elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

bool valid_dtype(int dtype) { return dtype == RA_F32 || dtype == RA_BF16; }

// [a, a + na) and [b, b + nb) overlap (empty ranges never overlap)
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

// product of non-negative sizes, or -1 on overflow past 2^62
int64_t mul_sizes(std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x < 0) return -1;
    if (x != 0 && r > ((int64_t)1 << 62) / x) return -1;
    r *= x;
  }
  return r;
}

// Position of the first and last row of a block: off + r * stride.
struct Span {
  int64_t lo, hi;
};

// Classification of a (query block, key block) pair from positions.
// 0: no key visible to any query; 1: every key visible to every query; 2: partially visible.
int classify(bool causal, int64_t q_off, int64_t q_stride, int Nq, int64_t k_off, int64_t k_stride, int Nk) {
  if (Nq <= 0 || Nk <= 0) return 0;
  if (!causal) return 1;
  const Span q{q_off, q_off + (int64_t)(Nq - 1) * q_stride};
  const Span k{k_off, k_off + (int64_t)(Nk - 1) * k_stride};
  if (k.lo > q.hi) return 0;
  if (k.hi <= q.lo) return 1;
  return 2;
}

int64_t block_offset(int layout, int P, int n, int block) {
  return layout == RA_LAYOUT_STRIPED ? (int64_t)block : (int64_t)block * n;
}

// Whether the bf16 D=128 step kernel stages every key/value row of a block it computes on in the
// workgroups that forward it (query tile qt forwards key tiles [4 qt, 4 qt + 4), which it must load):
// the last row of each query tile has to see up to the last of those tiles.
bool step_forward_covers(bool causal, int64_t q_off, int64_t q_stride, int Nq, int64_t k_off, int64_t k_stride,
                         int Nk) {
  const int br = ra::kMfmaRowsPerWg, bc = ra::kMfmaKeysPerTile;
  const int ktiles = (Nk + bc - 1) / bc;
  for (int qt = 0; qt * br < Nq; ++qt) {
    const int last_row = std::min(qt * br + br - 1, Nq - 1);
    int64_t kend = Nk - 1;
    if (causal) {
      const int64_t d = q_off + (int64_t)last_row * q_stride - k_off;
      kend = d < 0 ? -1 : std::min<int64_t>(d / k_stride, Nk - 1);
    }
    const int loaded = kend < 0 ? 0 : (int)(kend / bc) + 1;
    if (loaded < std::min(qt * (br / bc) + br / bc, ktiles)) return false;
  }
  return true;
}

int64_t layout_stride(int layout, int P) { return layout == RA_LAYOUT_STRIPED ? (int64_t)P : 1; }

bool valid_layout(int layout) {
  return layout == RA_LAYOUT_CONTIGUOUS || layout == RA_LAYOUT_STRIPED || layout == RA_LAYOUT_ZIGZAG;
}

// Global position of local row r of block b (n rows per block).  Zigzag: the sequence is cut into
// 2P chunks of n/2 tokens and block b holds chunks b and 2P-1-b, in that order.
int64_t token_pos(int layout, int P, int n, int b, int64_t r) {
  if (layout == RA_LAYOUT_STRIPED) return r * P + b;
  if (layout == RA_LAYOUT_ZIGZAG) {
    const int64_t c = n / 2;
    return r < c ? (int64_t)b * c + r : (2 * (int64_t)P - 1 - b) * c + (r - c);
  }
  return (int64_t)b * n + r;
}

// Number of key rows of block j whose position is <= pos.
int64_t keys_upto(int layout, int P, int n, int j, int64_t pos) {
  auto clampn = [](int64_t x, int64_t hi) { return x < 0 ? 0 : (x > hi ? hi : x); };
  if (layout == RA_LAYOUT_STRIPED) return pos < j ? 0 : clampn((pos - j) / P + 1, n);
  if (layout == RA_LAYOUT_ZIGZAG) {
    const int64_t c = n / 2;
    return clampn(pos - (int64_t)j * c + 1, c) + clampn(pos - (2 * (int64_t)P - 1 - j) * c + 1, c);
  }
  return clampn(pos - (int64_t)j * n + 1, n);
}

// Visible (query, key) pairs between query block i and key block j: sum over query rows r of the
// keys at or before the row's position.
int64_t count_visible(int P, int n, int mask, int layout, int i, int j) {
  if (n <= 0) return 0;
  if (mask == RA_MASK_NONE) return (int64_t)n * n;
  int64_t total = 0;
  for (int r = 0; r < n; ++r) total += keys_upto(layout, P, n, j, token_pos(layout, P, n, i, r));
  return total;
}

// Class of the block pair (i, j) of a ring (0 / 1 / 2 as in classify), for any layout.
int block_class(bool causal, int P, int n, int layout, int i, int j) {
  if (n <= 0) return 0;
  if (layout != RA_LAYOUT_ZIGZAG) {
    const int64_t st = layout_stride(layout, P);
    return classify(causal, block_offset(layout, P, n, i), st, n, block_offset(layout, P, n, j), st, n);
  }
  const int64_t v = count_visible(P, n, causal ? RA_MASK_CAUSAL : RA_MASK_NONE, layout, i, j);
  return v == 0 ? 0 : (v == (int64_t)n * n ? 1 : 2);
}

// One launch slot of the ring driver: query rows [row0, row0 + nq) of local device t against the
// keys [0, nk) of the block it holds, with the positions of the first query row and first key (the
// rows and keys are consecutive positions with stride `stride`).  The contiguous and striped layouts
// use one unit per device (the whole block, positions of the layout); zigzag uses two, one per
// query chunk:
//   first chunk (positions i*c + r): the keys of chunk j (the first n/2 rows of block j);
//   second chunk (positions (2P-1-i)*c + r): for j < i only chunk j is visible (all of it), so the
//   unit reads the first n/2 rows; for j >= i it reads the whole block [chunk j | chunk 2P-1-j] as
//   one run of consecutive positions ending at the true positions of chunk 2P-1-j.  Chunk j's keys
//   then carry positions below their true ones, but still below every query of the unit (their
//   true positions are too), so exactly the visible keys stay visible.
struct Unit {
  int row0, nk;
  int64_t q_off, k_off, stride;
};

Unit ring_unit(bool causal, int layout, int P, int n, int i, int j, int half) {
  if (layout == RA_LAYOUT_ZIGZAG && !causal) return Unit{half * (n / 2), n, 0, 0, 1};
  if (layout != RA_LAYOUT_ZIGZAG) {
    const int64_t st = layout_stride(layout, P);
    return Unit{0, n, block_offset(layout, P, n, i), block_offset(layout, P, n, j), st};
  }
  const int c = n / 2;
  if (half == 0) return Unit{0, c, (int64_t)i * c, (int64_t)j * c, 1};
  const int64_t qo = (2 * (int64_t)P - 1 - i) * c;
  if (j >= i) return Unit{c, n, qo, (2 * (int64_t)P - 2 - j) * c, 1};
  return Unit{c, c, qo, (int64_t)j * c, 1};
}

struct Shape {
  int n_dev, B, Hq, Hkv, Nq, Nk, D, dtype;
};

int validate_shape(const Shape& s) {
  if (s.n_dev < 1 || s.n_dev > RA_MAX_DEV) return RA_ERR_INVALID_ARG;
  if (s.B < 1 || s.Hq < 1 || s.Hkv < 1 || s.Nq < 0 || s.Nk < 0 || s.D < 1) return RA_ERR_INVALID_ARG;
  if (s.Hq % s.Hkv) return RA_ERR_INVALID_ARG;
  if (!valid_dtype(s.dtype)) return RA_ERR_INVALID_ARG;
  if (s.D > RA_MAX_D) return RA_ERR_UNSUPPORTED;
  if (mul_sizes({s.n_dev, s.B, s.Nq, s.Hq, s.D}) < 0 || mul_sizes({s.n_dev, s.B, s.Nk, s.Hkv, s.D}) < 0)
    return RA_ERR_INVALID_ARG;
  return RA_OK;
}

// Fill the work decomposition fields and launch the right kernel for the devices in p.
// The bf16 D = 128 steps run on the MFMA kernel; everything else on the generic one.
bool uses_mfma_kernel(int dtype, int D) { return dtype == RA_BF16 && D == 128; }

// ev_start / ev_stop (may be null) are stamped by the kernel launch itself; when nothing is
// launched they are recorded on the stream so that they are still valid.
hipError_t launch_step(StepParams& p, int dtype, hipStream_t stream, hipEvent_t ev_start = nullptr,
                       hipEvent_t ev_stop = nullptr) {
  if (p.n_launch == 0 || p.Nq == 0) {
    hipError_t e = hipSuccess;
    if (ev_start) e = hipEventRecord(ev_start, stream);
    if (e == hipSuccess && ev_stop) e = hipEventRecord(ev_stop, stream);
    return e;
  }
  if (uses_mfma_kernel(dtype, p.D)) return ra::launch_step_mfma_bf16_d128(p, stream, ev_start, ev_stop);
  return ra::launch_step_generic(p, dtype, stream, ev_start, ev_stop);
}

// One pass of a backward step launch (query gradients, or key/value gradients) on the kernel for
// the dtype and head dim, as launch_step chooses the forward's.
hipError_t launch_bwd(const ra::BwdParams& p, int dtype, bool dq_pass, hipStream_t stream) {
  if (uses_mfma_kernel(dtype, p.D))
    return dq_pass ? ra::launch_bwd_dq_bf16_d128(p, stream) : ra::launch_bwd_dkv_bf16_d128(p, stream);
  return ra::launch_bwd_generic(p, dtype, dq_pass, stream);
}

int hip_status(hipError_t e) { return e == hipSuccess ? RA_OK : RA_ERR_HIP; }

// Some non-null pointer is not a multiple of `align` bytes.  The kernels move 16-byte vectors of
// the tensors (and per-row scalars of the fp32 row arrays), so tensors must be 16-byte aligned and
// row arrays 4-byte aligned.
bool misaligned(std::initializer_list<const void*> ps, uintptr_t align) {
  for (const void* p : ps)
    if (p && (uintptr_t)p % align) return true;
  return false;
}

// Test hooks of the ring drivers, read from the environment at every call (documented in
// ring_attn.h): RING_ATTN_HOP_STRESS = comma-separated "poison", "jitter-copy", "jitter-compute";
// RING_ATTN_FAIL_AT_STEP = k (ring_attn_local stops before step k).
struct HopStress {
  bool poison = false;          // NaN-fill every receive-slot range just before it is written
  bool jitter_copy = false;     // a bounded sleep kernel before each step's hop copies
  bool jitter_compute = false;  // a bounded sleep kernel before each step kernel
  int fail_at = -1;             // stop before this step (-1: run the whole ring)
};

HopStress read_hop_stress() {
  HopStress h;
  if (const char* e = std::getenv("RING_ATTN_HOP_STRESS")) {
    const std::string v(e);
    h.poison = v.find("poison") != std::string::npos;
    h.jitter_copy = v.find("jitter-copy") != std::string::npos;
    h.jitter_compute = v.find("jitter-compute") != std::string::npos;
  }
  if (const char* e = std::getenv("RING_ATTN_FAIL_AT_STEP")) {
    char* end = nullptr;
    const long k = std::strtol(e, &end, 10);
    if (end != e && k >= 0 && k < (1L << 30)) h.fail_at = (int)k;
  }
  return h;
}

constexpr unsigned kJitterRounds = 48;  // ~0.2 ms of sleep per jitter kernel at 2 GHz
constexpr uint16_t kPoison = 0xFFFF;    // NaN as bf16 and, in pairs, as fp32

// NaN-fill `bytes` (a whole number of 16-bit words) at p on `stream` when poisoning.
hipError_t poison(const HopStress& hs, void* p, size_t bytes, hipStream_t stream) {
  return hs.poison ? ra::launch_fill_u16(p, bytes / 2, kPoison, stream) : hipSuccess;
}

hipError_t jitter(bool on, hipStream_t stream) { return on ? ra::launch_spin(kJitterRounds, stream) : hipSuccess; }

// Fixed device scratch of ring_attn_local_noalloc: the ring's receive slots and running state live
// here instead of in a caller workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never the device memory: kernel
// arguments and copies use the address hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxGpus = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxGpus] = {};

// Device address of `scratch` on the current device (looked up once per device); null on failure.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxGpus) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Ring steps folded per launch of the bf16 D=128 kernel when the whole ring is local (1 or 2;
// RING_ATTN_STEPS_PER_LAUNCH overrides the default of 2).
int steps_per_launch() {
  if (const char* e = std::getenv("RING_ATTN_STEPS_PER_LAUNCH")) {
    if (e[0] == '1' && e[1] == 0) return 1;
  }
  return 2;
}

// Everything the whole-ring drivers share once the arguments are validated.
struct LocalRing {
  const void* q;
  const char* ksrc;
  const char* vsrc;
  void* o;
  float* lse;
  int P, B, Hq, Hkv, n, D, dtype, layout;
  bool causal;
  float scale_log2;
  size_t blk;
  char* stage_k[2];
  char* stage_v[2];
  float* o_acc;
  float* m;
  float* l;
  hipStream_t cs, xs;
  void* const* step_events;
  HopStress hs;
};

// The whole ring with two steps per launch (every device local, key/value source in device memory,
// the bf16 D=128 kernel).  Launch L folds steps s = 2L and s + 1: device i first folds the block it
// holds (receive slot L & 1 of device i, or its own shard at L = 0) and then the block its
// predecessor holds at step s (slot L & 1 of device i - 1, or shard i - 1 at L = 0; one hop, pulled
// by the reader), with the running state in registers across both; the second block is what device i
// holds at step s + 1, and it also passes it on: stored from inside the kernel into the successor's
// slot (L + 1) & 1 (one hop, pushed), or, where the kernel cannot (the block is not computed, the
// forwarding workgroups do not stage all of it, or zigzag's half-block units), copied there on the
// copy stream.  Slot L & 1 is only read and slot (L + 1) & 1 only written during launch L, so a
// launch never waits on another workgroup; two hops per launch is the most a neighbour-only ring
// allows without such waits.  Returns a hipError_t.
hipError_t ring_two_step(const LocalRing& r, const std::vector<int>& cls, const std::vector<int>& first_step,
                         const std::vector<int>& last_step, int nh) {
  const int P = r.P, n = r.n;
  const int n_units = P * nh;
  const int NL = (P + 1) / 2;
  const int64_t st = layout_stride(r.layout, P);
  const hipStream_t cs = r.cs, xs = r.xs;
  const bool two_streams = xs != cs;
  auto blockj = [&](int i, int s) { return ((i - s) % P + P) % P; };

  // in-kernel push of launch L by device i (its step-(2L+1) block into device i+1's slot (L+1) & 1)
  std::vector<uint8_t> push((size_t)NL * P, 0);
  for (int L = 0; L + 1 < NL; ++L)
    for (int i = 0; i < P && nh == 1; ++i) {
      const int s1 = 2 * L + 1;
      if (cls[(size_t)s1 * n_units + i] == 0) continue;
      const int j = blockj(i, s1);
      if (step_forward_covers(r.causal, block_offset(r.layout, P, n, i), st, n, block_offset(r.layout, P, n, j), st, n))
        push[(size_t)L * P + i] = 1;
    }
  auto needs_copy = [&](int L) -> bool {  // launch L's slot L & 1 has a block not pushed by launch L-1
    if (L <= 0 || L >= NL) return false;
    for (int x = 0; x < P; ++x)
      if (!push[(size_t)(L - 1) * P + (x + P - 1) % P]) return true;
    return false;
  };
  // copies that fill slot L & 1 for launch L >= 1: device x's block of step 2L is the step-(2L-1)
  // block of device x-1, which it read from slot (L-1) & 1 of device x-2 (or shard x-2 when L = 1)
  auto enqueue_copies = [&](int L) -> hipError_t {
    hipError_t e;
    for (int x = 0; x < P; ++x) {
      if (push[(size_t)(L - 1) * P + (x + P - 1) % P]) continue;
      const int from = (x + P - 2) % P;
      const char* ks = (L == 1 ? r.ksrc : r.stage_k[(L - 1) & 1]) + (size_t)from * r.blk;
      const char* vs = (L == 1 ? r.vsrc : r.stage_v[(L - 1) & 1]) + (size_t)from * r.blk;
      char* kd = r.stage_k[L & 1] + (size_t)x * r.blk;
      char* vd = r.stage_v[L & 1] + (size_t)x * r.blk;
      if ((e = poison(r.hs, kd, r.blk, xs)) != hipSuccess) return e;
      if ((e = poison(r.hs, vd, r.blk, xs)) != hipSuccess) return e;
      if ((e = hipMemcpyAsync(kd, ks, r.blk, hipMemcpyDeviceToDevice, xs)) != hipSuccess) return e;
      if ((e = hipMemcpyAsync(vd, vs, r.blk, hipMemcpyDeviceToDevice, xs)) != hipSuccess) return e;
    }
    return hipSuccess;
  };

  hipEvent_t ev_copy[2] = {nullptr, nullptr}, ev_comp[2] = {nullptr, nullptr}, ev_fork = nullptr;
  hipError_t err = hipSuccess;
  auto cleanup = [&]() {
    for (int a = 0; a < 2; ++a) {
      if (ev_copy[a]) (void)hipEventDestroy(ev_copy[a]);
      if (ev_comp[a]) (void)hipEventDestroy(ev_comp[a]);
    }
    if (ev_fork) (void)hipEventDestroy(ev_fork);
  };
#define RA_TRY(x)               \
  do {                          \
    if ((err = (x)) != hipSuccess) { \
      cleanup();                \
      return err;               \
    }                           \
  } while (0)
  if (two_streams) {
    for (int a = 0; a < 2; ++a) {
      RA_TRY(hipEventCreateWithFlags(&ev_copy[a], hipEventDisableTiming));
      RA_TRY(hipEventCreateWithFlags(&ev_comp[a], hipEventDisableTiming));
    }
    RA_TRY(hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming));
    RA_TRY(hipEventRecord(ev_fork, cs));
    RA_TRY(hipStreamWaitEvent(xs, ev_fork, 0));
  }
  for (int L = 0; L < NL; ++L) {
    const int s0 = 2 * L, s1 = 2 * L + 1;
    // copies for launch L+1 into the slot launch L-1 read (they may read blocks it pushed)
    if (needs_copy(L + 1)) {
      if (L >= 1 && two_streams) RA_TRY(hipStreamWaitEvent(xs, ev_comp[(L + 1) & 1], 0));
      RA_TRY(jitter(r.hs.jitter_copy, xs));
      RA_TRY(enqueue_copies(L + 1));
      if (two_streams) RA_TRY(hipEventRecord(ev_copy[(L + 1) & 1], xs));
    }
    if (needs_copy(L) && two_streams) RA_TRY(hipStreamWaitEvent(cs, ev_copy[L & 1], 0));

    StepParams p{};
    p.q = r.q;
    // source 0: the shards in place; 1: the slot of this launch; 2: the slot of the next
    p.kv_base[0][0] = (char*)r.ksrc;
    p.kv_base[0][1] = (char*)r.vsrc;
    p.kv_base[1][0] = r.stage_k[L & 1];
    p.kv_base[1][1] = r.stage_v[L & 1];
    p.kv_base[2][0] = r.stage_k[(L + 1) & 1];
    p.kv_base[2][1] = r.stage_v[(L + 1) & 1];
    p.kv_block = (int64_t)r.blk;
    p.o_acc = r.o_acc;
    p.m = r.m;
    p.l = r.l;
    p.o_out = r.o;
    p.lse_out = r.lse;
    p.B = r.B;
    p.Hq = r.Hq;
    p.Hkv = r.Hkv;
    p.Nq = n / nh;
    p.NqTot = n;
    p.NkTot = n;
    p.D = r.D;
    p.causal = r.causal ? 1 : 0;
    p.scale_log2 = r.scale_log2;
    std::vector<int> todo;
    for (int u = 0; u < n_units; ++u) {
      const bool c0 = cls[(size_t)s0 * n_units + u] != 0;
      const bool c1 = s1 < P && cls[(size_t)s1 * n_units + u] != 0;
      if (c0 || c1) todo.push_back(u);
    }
    const size_t n_chunks = todo.empty() ? 1 : (todo.size() + RA_MAX_DEV - 1) / RA_MAX_DEV;
    for (size_t ch = 0; ch < n_chunks; ++ch) {
      p.n_launch = 0;
      p.Nk = 0;
      for (size_t a = ch * RA_MAX_DEV; a < todo.size() && a < (ch + 1) * RA_MAX_DEV; ++a) {
        const int u = todo[a], i = u / nh;
        const int x = p.n_launch++;
        p.slot[x] = i;
        p.nsub[x] = 0;
        for (int s = s0; s <= s1 && s < P; ++s) {
          if (cls[(size_t)s * n_units + u] == 0) continue;
          const int j = blockj(i, s);
          const Unit un = ring_unit(r.causal, r.layout, P, n, i, j, u % nh);
          const int b = p.nsub[x]++;
          // step s0: the block device i holds; step s1: the block device i - 1 holds at step s0
          const int holder = s == s0 ? i : (i + P - 1) % P;
          p.kv[x][b] = L == 0 ? ra::kv_ref(0, holder) : ra::kv_ref(1, holder);
          p.nk[x][b] = un.nk;
          p.k_off[x][b] = un.k_off;
          p.Nk = std::max(p.Nk, un.nk);
          p.q_row0[x] = un.row0;
          p.q_off[x] = un.q_off;
          p.q_stride = un.stride;  // the same for every unit of a layout
          p.k_stride = un.stride;
        }
        const bool first = first_step[u] == s0 || first_step[u] == s1;
        const bool last = last_step[u] == s0 || last_step[u] == s1;
        p.dflags[x] = (first ? ra::kDevInit : 0) | (last ? ra::kDevFinal : 0);
        const bool pushes = push[(size_t)L * P + i] != 0;
        p.fwd[x] = pushes ? ra::kv_ref(2, (i + 1) % P) : -1;
        if (pushes) {  // slot (L+1) & 1 was last read by launch L-1, earlier on this stream
          RA_TRY(poison(r.hs, r.stage_k[(L + 1) & 1] + (size_t)((i + 1) % P) * r.blk, r.blk, cs));
          RA_TRY(poison(r.hs, r.stage_v[(L + 1) & 1] + (size_t)((i + 1) % P) * r.blk, r.blk, cs));
        }
      }
      RA_TRY(jitter(r.hs.jitter_compute, cs));
      hipEvent_t e0 = r.step_events && ch == 0 ? (hipEvent_t)r.step_events[2 * s0] : nullptr;
      hipEvent_t e1 = r.step_events && ch + 1 == n_chunks ? (hipEvent_t)r.step_events[2 * s0 + 1] : nullptr;
      RA_TRY(launch_step(p, r.dtype, cs, e0, e1));
    }
    if (r.step_events && s1 < P) {  // the second step's events: right after the launch that folded it
      RA_TRY(hipEventRecord((hipEvent_t)r.step_events[2 * s1], cs));
      RA_TRY(hipEventRecord((hipEvent_t)r.step_events[2 * s1 + 1], cs));
    }
    if (needs_copy(L + 2) && two_streams) RA_TRY(hipEventRecord(ev_comp[L & 1], cs));
  }
  // devices that never computed (no visible block): empty output
  for (int t = 0; t < P && nh == 1; ++t)
    if (first_step[t] < 0) {
      int slot_t = t;
      RA_TRY(ra::launch_init_state(r.o_acc, r.m, r.l, P, &slot_t, 1, r.B, r.Hq, n, r.D, cs));
      const size_t per = (size_t)r.B * r.Hq * n;
      RA_TRY(ra::launch_finalize(r.o_acc + t * per * r.D, r.m + t * per, r.l + t * per,
                                 (char*)r.o + t * per * r.D * elem_size(r.dtype), r.lse ? r.lse + t * per : nullptr, 1,
                                 r.B, r.Hq, n, r.D, r.dtype, cs));
    }
  if (two_streams) {
    RA_TRY(hipEventRecord(ev_copy[0], xs));
    RA_TRY(hipStreamWaitEvent(cs, ev_copy[0], 0));
    RA_TRY(hipEventRecord(ev_comp[0], cs));
    RA_TRY(hipStreamWaitEvent(xs, ev_comp[0], 0));
  }
  cleanup();
#undef RA_TRY
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* ring_attn_strerror(int code) {
  switch (code) {
    case RA_OK: return "ok";
    case RA_ERR_INVALID_ARG: return "invalid argument";
    case RA_ERR_UNSUPPORTED: return "unsupported configuration";
    case RA_ERR_HIP: return "HIP runtime error";
    case RA_ERR_WORKSPACE: return "workspace too small";
    case RA_ERR_INJECTED: return "stopped by RING_ATTN_FAIL_AT_STEP";
    case RA_ERR_SCRATCH: return "needs more than the fixed scratch of ring_attn_local_noalloc";
    default: return "unknown status";
  }
}

int64_t ring_attn_visible_pairs(int P, int n, int mask, int layout, int i, int j) {
  if (P < 1 || P > RA_MAX_DEV || n < 0 || i < 0 || j < 0 || i >= P || j >= P) return -1;
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return -1;
  if (!valid_layout(layout) || (layout == RA_LAYOUT_ZIGZAG && n % 2)) return -1;
  return count_visible(P, n, mask, layout, i, j);
}

int ring_attn_plan(int P, int dev0, int n_local, int n, int mask, int layout, int32_t* out_rows) {
  if (P < 1 || P > RA_MAX_DEV || dev0 < 0 || dev0 >= P || n_local < 1 || dev0 + n_local > P || n < 0)
    return RA_ERR_INVALID_ARG;
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return RA_ERR_INVALID_ARG;
  if (!valid_layout(layout) || (layout == RA_LAYOUT_ZIGZAG && n % 2)) return RA_ERR_INVALID_ARG;
  if (!out_rows) return RA_ERR_INVALID_ARG;
  int32_t* row = out_rows;
  for (int s = 0; s < P; ++s)
    for (int i = dev0; i < dev0 + n_local; ++i) {
      const int j = ((i - s) % P + P) % P;
      row[0] = s;
      row[1] = i;
      row[2] = j;
      row[3] = s & 1;
      row[4] = block_class(mask == RA_MASK_CAUSAL, P, n, layout, i, j);
      row += 5;
    }
  return RA_OK;
}

int ring_attn_step(const void* q, const void* k, const void* v, float* o_acc, float* m, float* l, int n_dev, int B,
                   int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale, int mask, const int64_t* q_off,
                   int64_t q_stride, const int64_t* k_off, int64_t k_stride, int flags, void* stream) {
  const Shape sh{n_dev, B, Hq, Hkv, Nq, Nk, D, dtype};
  int rc = validate_shape(sh);
  if (rc != RA_OK) return rc;
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return RA_ERR_INVALID_ARG;
  if (flags & ~RA_STEP_INIT) return RA_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.f)) return RA_ERR_INVALID_ARG;
  const bool causal = mask == RA_MASK_CAUSAL;
  if (causal && (!q_off || !k_off || q_stride <= 0 || k_stride <= 0)) return RA_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  const size_t q_bytes = (size_t)n_dev * B * Nq * Hq * D * es;
  const size_t kv_bytes = (size_t)n_dev * B * Nk * Hkv * D * es;
  const size_t rows = (size_t)n_dev * B * Hq * Nq;
  if (rows > 0 && (!q || !o_acc || !m || !l)) return RA_ERR_INVALID_ARG;
  if (kv_bytes > 0 && (!k || !v)) return RA_ERR_INVALID_ARG;
  if (misaligned({q, k, v, o_acc}, 16) || misaligned({m, l}, 4)) return RA_ERR_INVALID_ARG;
  // the state is written: it may not alias the inputs or itself
  const void* outs[3] = {o_acc, m, l};
  const size_t out_sz[3] = {rows * D * 4, rows * 4, rows * 4};
  const void* ins[3] = {q, k, v};
  const size_t in_sz[3] = {q_bytes, kv_bytes, kv_bytes};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 3; ++b)
      if (overlaps(outs[a], out_sz[a], ins[b], in_sz[b])) return RA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], out_sz[a], outs[b], out_sz[b])) return RA_ERR_INVALID_ARG;
  }
  if (rows == 0) return RA_OK;

  StepParams p{};
  p.q = q;
  p.kv_base[0][0] = (char*)k;  // read only: no slot of this launch forwards
  p.kv_base[0][1] = (char*)v;
  p.kv_block = (int64_t)B * Nk * Hkv * D * es;
  p.o_acc = o_acc;
  p.m = m;
  p.l = l;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.NqTot = Nq;
  p.NkTot = Nk;
  p.D = D;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = (float)(scale * kLog2e);
  p.q_stride = causal ? q_stride : 1;
  p.k_stride = causal ? k_stride : 1;
  std::vector<int> skipped_init;
  for (int t = 0; t < n_dev; ++t) {
    const int64_t qo = q_off ? q_off[t] : 0, ko = k_off ? k_off[t] : 0;
    const int cls = classify(causal, qo, p.q_stride, Nq, ko, p.k_stride, Nk);
    if (cls == 0) {
      if (flags & RA_STEP_INIT) skipped_init.push_back(t);
      continue;
    }
    const int i = p.n_launch++;
    p.slot[i] = t;
    p.q_row0[i] = 0;
    p.q_off[i] = qo;
    p.nsub[i] = 1;
    p.kv[i][0] = ra::kv_ref(0, t);
    p.nk[i][0] = Nk;
    p.k_off[i][0] = ko;
    p.fwd[i] = -1;
    p.dflags[i] = (flags & RA_STEP_INIT) ? ra::kDevInit : 0;
  }
  hipStream_t st = (hipStream_t)stream;
  if (!skipped_init.empty()) {
    rc = hip_status(ra::launch_init_state(o_acc, m, l, n_dev, skipped_init.data(), (int)skipped_init.size(), B, Hq,
                                          Nq, D, st));
    if (rc != RA_OK) return rc;
  }
  return hip_status(launch_step(p, dtype, st));
}

int ring_attn_finalize(const float* o_acc, const float* m, const float* l, void* o, float* lse, int n_dev, int B,
                       int Hq, int Nq, int D, int out_dtype, void* stream) {
  if (n_dev < 1 || n_dev > RA_MAX_DEV || B < 1 || Hq < 1 || Nq < 0 || D < 1) return RA_ERR_INVALID_ARG;
  if (!valid_dtype(out_dtype)) return RA_ERR_INVALID_ARG;
  if (D > RA_MAX_D) return RA_ERR_UNSUPPORTED;
  const size_t rows = (size_t)n_dev * B * Hq * Nq;
  if (rows == 0) return RA_OK;
  if (!o_acc || !m || !l || !o) return RA_ERR_INVALID_ARG;
  if (misaligned({o_acc, o}, 16) || misaligned({m, l, lse}, 4)) return RA_ERR_INVALID_ARG;
  const size_t o_bytes = rows * D * elem_size(out_dtype);
  if (overlaps(o, o_bytes, o_acc, rows * D * 4) || overlaps(o, o_bytes, m, rows * 4) ||
      overlaps(o, o_bytes, l, rows * 4) || overlaps(lse, rows * 4, o, o_bytes) ||
      overlaps(lse, rows * 4, o_acc, rows * D * 4) || overlaps(lse, rows * 4, l, rows * 4))
    return RA_ERR_INVALID_ARG;
  return hip_status(ra::launch_finalize(o_acc, m, l, o, lse, n_dev, B, Hq, Nq, D, out_dtype, (hipStream_t)stream));
}

size_t ring_attn_local_workspace_bytes(int P, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype) {
  if (P < 1 || P > RA_MAX_DEV || n_local < 1 || n_local > P || B < 1 || Hq < 1 || Hkv < 1 || n < 0 || D < 1 ||
      D > RA_MAX_D || Hq % Hkv || !valid_dtype(dtype))
    return 0;
  const size_t align = 256;
  auto up = [&](size_t x) { return (x + align - 1) / align * align; };
  const size_t blk = (size_t)B * n * Hkv * D * elem_size(dtype);
  const size_t rows = (size_t)n_local * B * Hq * n;
  return 4 * up((size_t)n_local * blk) + up(rows * D * 4) + 2 * up(rows * 4);
}

int ring_attn_local(const void* q_local, const void* k_src, const void* v_src, int kv_src_is_host, void* o,
                    float* lse, int P, int dev0, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype,
                    float scale, int mask, int layout, void* workspace, size_t workspace_bytes,
                    void* compute_stream, void* copy_stream, void* const* step_events) {
  if (P < 1 || P > RA_MAX_DEV || dev0 < 0 || dev0 >= P || n_local < 1 || dev0 + n_local > P) return RA_ERR_INVALID_ARG;
  const Shape sh{n_local, B, Hq, Hkv, n, n, D, dtype};
  int rc = validate_shape(sh);
  if (rc != RA_OK) return rc;
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return RA_ERR_INVALID_ARG;
  if (!valid_layout(layout) || (layout == RA_LAYOUT_ZIGZAG && n % 2)) return RA_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.f)) return RA_ERR_INVALID_ARG;
  if (n == 0) return RA_OK;
  if (!q_local || !k_src || !v_src || !o || !workspace) return RA_ERR_INVALID_ARG;
  if (misaligned({q_local, k_src, v_src, o, workspace}, 16) || misaligned({lse}, 4)) return RA_ERR_INVALID_ARG;
  const size_t need = ring_attn_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, dtype);
  if (need == 0) return RA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return RA_ERR_WORKSPACE;

  const size_t es = elem_size(dtype);
  const size_t blk = (size_t)B * n * Hkv * D * es;  // one device's K (or V) block
  const size_t rows = (size_t)n_local * B * Hq * n;
  const size_t q_bytes = rows * D * es;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* ws = (char*)workspace;
  char* stage_k[2] = {ws, ws + up((size_t)n_local * blk)};
  char* stage_v[2] = {ws + 2 * up((size_t)n_local * blk), ws + 3 * up((size_t)n_local * blk)};
  float* o_acc = (float*)(ws + 4 * up((size_t)n_local * blk));
  float* m_st = (float*)((char*)o_acc + up(rows * D * 4));
  float* l_st = (float*)((char*)m_st + up(rows * 4));
  // outputs may not alias inputs or the workspace
  const size_t src_bytes = (size_t)P * blk;
  const void* ro[4] = {q_local, kv_src_is_host ? nullptr : k_src, kv_src_is_host ? nullptr : v_src, workspace};
  const size_t ro_sz[4] = {q_bytes, src_bytes, src_bytes, need};
  for (int a = 0; a < 4; ++a)
    if (overlaps(o, q_bytes, ro[a], ro_sz[a]) || overlaps(lse, rows * 4, ro[a], ro_sz[a])) return RA_ERR_INVALID_ARG;
  if (overlaps(o, q_bytes, lse, rows * 4)) return RA_ERR_INVALID_ARG;
  if (overlaps(workspace, need, q_local, q_bytes) ||
      (!kv_src_is_host && (overlaps(workspace, need, k_src, src_bytes) || overlaps(workspace, need, v_src, src_bytes))))
    return RA_ERR_INVALID_ARG;

  hipStream_t cs = (hipStream_t)compute_stream;
  hipStream_t xs = (hipStream_t)copy_stream;
  const bool causal = mask == RA_MASK_CAUSAL;
  const int64_t st = layout_stride(layout, P);
  const HopStress hs = read_hop_stress();
  const int stop = hs.fail_at >= 0 && hs.fail_at < P ? hs.fail_at : P;  // steps run: [0, stop)

  // per-unit schedule (a unit is a device's whole query block, or one of its two zigzag chunks):
  // class of every (step, unit) and each unit's first and last computed step
  const int nh = layout == RA_LAYOUT_ZIGZAG ? 2 : 1;
  const int n_units = n_local * nh;
  std::vector<int> first_step(n_units, -1), last_step(n_units, -1);
  std::vector<int> cls((size_t)P * n_units);
  for (int s = 0; s < P; ++s)
    for (int u = 0; u < n_units; ++u) {
      const int i = dev0 + u / nh;
      const int j = ((i - s) % P + P) % P;
      const Unit un = ring_unit(causal, layout, P, n, i, j, u % nh);
      const int c = classify(causal, un.q_off, un.stride, n / nh, un.k_off, un.stride, un.nk);
      cls[(size_t)s * n_units + u] = c;
      if (c != 0) {
        if (first_step[u] < 0) first_step[u] = s;
        last_step[u] = s;
      }
    }

  // whole ring local, device source, MFMA kernel: two ring steps per launch
  if (!kv_src_is_host && uses_mfma_kernel(dtype, D) && n_local == P && P >= 2 && stop == P &&
      steps_per_launch() == 2) {
    LocalRing r{};
    r.q = q_local;
    r.ksrc = (const char*)k_src;
    r.vsrc = (const char*)v_src;
    r.o = o;
    r.lse = lse;
    r.P = P, r.B = B, r.Hq = Hq, r.Hkv = Hkv, r.n = n, r.D = D, r.dtype = dtype, r.layout = layout;
    r.causal = causal;
    r.scale_log2 = (float)(scale * kLog2e);
    r.blk = blk;
    for (int a = 0; a < 2; ++a) {
      r.stage_k[a] = stage_k[a];
      r.stage_v[a] = stage_v[a];
    }
    r.o_acc = o_acc, r.m = m_st, r.l = l_st;
    r.cs = cs, r.xs = xs;
    r.step_events = step_events;
    r.hs = hs;
    return hip_status(ring_two_step(r, cls, first_step, last_step, nh));
  }

  hipEvent_t ev_copy[2] = {nullptr, nullptr}, ev_comp[2] = {nullptr, nullptr}, ev_fork = nullptr;
  auto cleanup = [&]() {
    for (int a = 0; a < 2; ++a) {
      if (ev_copy[a]) (void)hipEventDestroy(ev_copy[a]);
      if (ev_comp[a]) (void)hipEventDestroy(ev_comp[a]);
    }
    if (ev_fork) (void)hipEventDestroy(ev_fork);
  };
#define RA_CHECK(x)            \
  do {                         \
    hipError_t e_ = (x);       \
    if (e_ != hipSuccess) {    \
      cleanup();               \
      return RA_ERR_HIP;       \
    }                          \
  } while (0)

  // cross-stream ordering needs events only when the copies have a stream of their own; on one
  // stream, stream order alone separates every copy from the kernels around it
  const bool two_streams = xs != cs;
  if (two_streams) {
    for (int a = 0; a < 2; ++a) {
      RA_CHECK(hipEventCreateWithFlags(&ev_copy[a], hipEventDisableTiming));
      RA_CHECK(hipEventCreateWithFlags(&ev_comp[a], hipEventDisableTiming));
    }
    RA_CHECK(hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming));
    RA_CHECK(hipEventRecord(ev_fork, cs));
    RA_CHECK(hipStreamWaitEvent(xs, ev_fork, 0));
  }
  const hipMemcpyKind kind = kv_src_is_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice;
  const char* ksrc = (const char*)k_src;
  const char* vsrc = (const char*)v_src;

  // Hop plan.  With a device-resident source and the bf16 D=128 kernel, a device that computes at
  // step s hands its block to its local successor inside the step-s kernel (the rows it stages in
  // LDS are stored into the successor's slot); every other block of step s+1 is copied on the copy
  // stream.  fwd_to[s*n_local+t]: successor fed by device t's step-s kernel (-1: none);
  // by_kernel[s*n_local+t]: device t's step-s block arrives that way.
  const bool in_step_hop = !kv_src_is_host && uses_mfma_kernel(dtype, D) && nh == 1;
  std::vector<int> fwd_to((size_t)P * n_local, -1);
  std::vector<uint8_t> by_kernel((size_t)P * n_local, 0);
  if (in_step_hop)
    for (int s = 0; s + 1 < P; ++s)
      for (int t = 0; t < n_local; ++t) {
        if (cls[(size_t)s * n_local + t] == 0) continue;
        const int succ = t + 1 < n_local ? t + 1 : (n_local == P ? 0 : -1);
        if (succ < 0) continue;
        const int i = dev0 + t, j = ((i - s) % P + P) % P;
        if (!step_forward_covers(causal, block_offset(layout, P, n, i), st, n, block_offset(layout, P, n, j), st, n))
          continue;
        fwd_to[(size_t)s * n_local + t] = succ;
        by_kernel[(size_t)(s + 1) * n_local + succ] = 1;
      }
  // whether the blocks of step s need any copy
  auto needs_copy = [&](int s) -> bool {
    if (s < 0 || s >= P) return false;
    if (kv_src_is_host) return true;
    if (s == 0) return false;  // device mode: step 0 reads the source in place
    for (int t = 0; t < n_local; ++t)
      if (!by_kernel[(size_t)s * n_local + t]) return true;
    return false;
  };
  // device mode, s >= 1: where device t's step-s block comes from (what its predecessor held)
  auto hop_src = [&](int s, int t, const char* src, char* const* stage) -> const char* {
    if (t == 0 && n_local < P) return src + (size_t)(((dev0 - s) % P + P) % P) * blk;  // remote predecessor
    const int pred = t >= 1 ? t - 1 : n_local - 1;
    return (s == 1 ? src + (size_t)dev0 * blk : stage[(s - 1) & 1]) + (size_t)pred * blk;
  };

  // copies that bring the blocks of step s not handed over by a kernel into staging slot s & 1
  auto enqueue_hop = [&](int s) -> hipError_t {
    const int sl = s & 1;
    hipError_t e;
    if (kv_src_is_host) {
      // every device receives block (i - s) mod P from the source (pinned host memory here)
      for (int t = 0; t < n_local; ++t) {
        const int j = ((dev0 + t - s) % P + P) % P;
        if ((e = poison(hs, stage_k[sl] + t * blk, blk, xs)) != hipSuccess) return e;
        if ((e = poison(hs, stage_v[sl] + t * blk, blk, xs)) != hipSuccess) return e;
        if ((e = hipMemcpyAsync(stage_k[sl] + t * blk, ksrc + j * blk, blk, kind, xs)) != hipSuccess) return e;
        if ((e = hipMemcpyAsync(stage_v[sl] + t * blk, vsrc + j * blk, blk, kind, xs)) != hipSuccess) return e;
      }
      return hipSuccess;
    }
    for (int t = 0; t < n_local;) {
      if (by_kernel[(size_t)s * n_local + t]) {
        ++t;
        continue;
      }
      // a run of devices whose sources are contiguous too
      const char* k0 = hop_src(s, t, ksrc, stage_k);
      const char* v0 = hop_src(s, t, vsrc, stage_v);
      int t2 = t + 1;
      while (t2 < n_local && !by_kernel[(size_t)s * n_local + t2] &&
             hop_src(s, t2, ksrc, stage_k) == k0 + (size_t)(t2 - t) * blk &&
             hop_src(s, t2, vsrc, stage_v) == v0 + (size_t)(t2 - t) * blk)
        ++t2;
      const size_t bytes = (size_t)(t2 - t) * blk;
      if ((e = poison(hs, stage_k[sl] + t * blk, bytes, xs)) != hipSuccess) return e;
      if ((e = poison(hs, stage_v[sl] + t * blk, bytes, xs)) != hipSuccess) return e;
      if ((e = hipMemcpyAsync(stage_k[sl] + t * blk, k0, bytes, hipMemcpyDeviceToDevice, xs)) != hipSuccess) return e;
      if ((e = hipMemcpyAsync(stage_v[sl] + t * blk, v0, bytes, hipMemcpyDeviceToDevice, xs)) != hipSuccess) return e;
      t = t2;
    }
    return hipSuccess;
  };

  if (kv_src_is_host && stop > 0) {
    RA_CHECK(jitter(hs.jitter_copy, xs));
    RA_CHECK(enqueue_hop(0));
    if (two_streams) RA_CHECK(hipEventRecord(ev_copy[0], xs));
  }
  for (int s = 0; s < stop; ++s) {
    // copies for step s+1, into the slot that step s-1 read; they may read blocks that kernel s-1
    // handed over, so they wait for it
    if (s + 1 < stop && needs_copy(s + 1)) {
      if (s >= 1 && two_streams) RA_CHECK(hipStreamWaitEvent(xs, ev_comp[(s + 1) & 1], 0));
      RA_CHECK(jitter(hs.jitter_copy, xs));
      RA_CHECK(enqueue_hop(s + 1));
      if (two_streams) RA_CHECK(hipEventRecord(ev_copy[(s + 1) & 1], xs));
    }
    const bool staged = kv_src_is_host || s > 0;
    if (needs_copy(s) && two_streams) RA_CHECK(hipStreamWaitEvent(cs, ev_copy[s & 1], 0));

    StepParams p{};
    p.q = q_local;
    // source 0: the blocks of step s (receive slot s & 1, or the shards in place); source 1: the other
    // receive slot, which the in-step hop fills for step s + 1
    p.kv_base[0][0] = staged ? stage_k[s & 1] : (char*)(ksrc + (size_t)dev0 * blk);
    p.kv_base[0][1] = staged ? stage_v[s & 1] : (char*)(vsrc + (size_t)dev0 * blk);
    p.kv_base[1][0] = stage_k[(s + 1) & 1];
    p.kv_base[1][1] = stage_v[(s + 1) & 1];
    p.kv_block = (int64_t)blk;
    p.o_acc = o_acc;
    p.m = m_st;
    p.l = l_st;
    p.o_out = o;
    p.lse_out = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = n / nh;
    p.NqTot = n;
    p.NkTot = n;
    p.D = D;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = (float)(scale * kLog2e);
    // the units of step s, RA_MAX_DEV per launch (one launch unless zigzag with more than 32 devices)
    std::vector<int> todo;
    for (int u = 0; u < n_units; ++u)
      if (cls[(size_t)s * n_units + u] != 0) todo.push_back(u);
    const size_t n_chunks = todo.empty() ? 1 : (todo.size() + RA_MAX_DEV - 1) / RA_MAX_DEV;
    for (size_t ch = 0; ch < n_chunks; ++ch) {
      p.n_launch = 0;
      p.Nk = 0;
      for (size_t a = ch * RA_MAX_DEV; a < todo.size() && a < (ch + 1) * RA_MAX_DEV; ++a) {
        const int u = todo[a], t = u / nh;
        const int i = dev0 + t;
        const int j = ((i - s) % P + P) % P;
        const Unit un = ring_unit(causal, layout, P, n, i, j, u % nh);
        const int x = p.n_launch++;
        p.slot[x] = t;
        p.q_row0[x] = un.row0;
        p.q_off[x] = un.q_off;
        p.nsub[x] = 1;
        p.kv[x][0] = ra::kv_ref(0, t);
        p.nk[x][0] = un.nk;
        p.k_off[x][0] = un.k_off;
        p.Nk = std::max(p.Nk, un.nk);
        p.q_stride = un.stride;  // the same for every unit of a layout
        p.k_stride = un.stride;
        p.dflags[x] = (s == first_step[u] ? ra::kDevInit : 0) |
                      (s == last_step[u] && stop == P ? ra::kDevFinal : 0);
        const int succ = in_step_hop ? fwd_to[(size_t)s * n_local + t] : -1;
        p.fwd[x] = succ >= 0 ? ra::kv_ref(1, succ) : -1;
        if (succ >= 0) {  // the slot this kernel fills was last read by step s-1, earlier on this stream
          RA_CHECK(poison(hs, stage_k[(s + 1) & 1] + (size_t)succ * blk, blk, cs));
          RA_CHECK(poison(hs, stage_v[(s + 1) & 1] + (size_t)succ * blk, blk, cs));
        }
      }
      RA_CHECK(jitter(hs.jitter_compute, cs));
      hipEvent_t e0 = step_events && ch == 0 ? (hipEvent_t)step_events[2 * s] : nullptr;
      hipEvent_t e1 = step_events && ch + 1 == n_chunks ? (hipEvent_t)step_events[2 * s + 1] : nullptr;
      RA_CHECK(launch_step(p, dtype, cs, e0, e1));
    }
    if (s + 2 < stop && needs_copy(s + 2) && two_streams) RA_CHECK(hipEventRecord(ev_comp[s & 1], cs));
  }
  if (stop < P) {
    // stopped before step `stop`: the workspace state is the fold of steps [0, stop); devices that
    // have not computed yet get the empty state so that every device's state is a valid checkpoint
    // (a zigzag unit computes at step 0, so only stop == 0 leaves zigzag devices untouched)
    for (int t = 0; t < n_local; ++t)
      if (stop == 0 || (nh == 1 && (first_step[t] < 0 || first_step[t] >= stop))) {
        int slot_t = t;
        RA_CHECK(ra::launch_init_state(o_acc, m_st, l_st, n_local, &slot_t, 1, B, Hq, n, D, cs));
      }
    if (two_streams) {
      RA_CHECK(hipEventRecord(ev_copy[0], xs));
      RA_CHECK(hipStreamWaitEvent(cs, ev_copy[0], 0));
      RA_CHECK(hipEventRecord(ev_comp[0], cs));
      RA_CHECK(hipStreamWaitEvent(xs, ev_comp[0], 0));
    }
    cleanup();
    return RA_ERR_INJECTED;
  }
  // devices that never computed (no visible block): empty output (a zigzag unit always computes:
  // its own block holds keys at or before each of its queries)
  for (int t = 0; t < n_local && nh == 1; ++t)
    if (first_step[t] < 0) {
      int slot_t = t;
      RA_CHECK(ra::launch_init_state(o_acc, m_st, l_st, n_local, &slot_t, 1, B, Hq, n, D, cs));
      const size_t per = (size_t)B * Hq * n;
      RA_CHECK(ra::launch_finalize(o_acc + t * per * D, m_st + t * per, l_st + t * per, (char*)o + t * per * D * es,
                                   lse ? lse + t * per : nullptr, 1, B, Hq, n, D, dtype, cs));
    }
  // join: both streams ordered after all work of this call
  if (two_streams) {
    RA_CHECK(hipEventRecord(ev_copy[0], xs));
    RA_CHECK(hipStreamWaitEvent(cs, ev_copy[0], 0));
    RA_CHECK(hipEventRecord(ev_comp[0], cs));
    RA_CHECK(hipStreamWaitEvent(xs, ev_comp[0], 0));
  }
  cleanup();
#undef RA_CHECK
  return RA_OK;
}

size_t ring_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int ring_attn_local_noalloc(const void* q_local, const void* k_src, const void* v_src, int kv_src_is_host, void* o,
                            float* lse, int P, int dev0, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype,
                            float scale, int mask, int layout, void* compute_stream, void* copy_stream,
                            void* const* step_events) {
  const size_t need = ring_attn_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, dtype);
  if (need == 0)  // invalid arguments, or nothing to do: ring_attn_local says which, before any HIP call
    return ring_attn_local(q_local, k_src, v_src, kv_src_is_host, o, lse, P, dev0, n_local, B, Hq, Hkv, n, D, dtype,
                           scale, mask, layout, nullptr, 0, compute_stream, copy_stream, step_events);
  if (need > kNoAllocScratchBytes) return RA_ERR_SCRATCH;
  void* ws = device_scratch();
  if (!ws) return RA_ERR_HIP;
  return ring_attn_local(q_local, k_src, v_src, kv_src_is_host, o, lse, P, dev0, n_local, B, Hq, Hkv, n, D, dtype,
                         scale, mask, layout, ws, kNoAllocScratchBytes, compute_stream, copy_stream, step_events);
}

// ------------------------------------------------------------------------------------------------
// Backward pass of the ring (gradients of exact attention).

int ring_attn_bwd_prep(const void* o, const void* dout, const float* lse, float* delta, float* lse2, int n_dev, int B,
                       int Hq, int Nq, int D, int dtype, void* stream) {
  if (n_dev < 1 || n_dev > RA_MAX_DEV || B < 1 || Hq < 1 || Nq < 0 || D < 1) return RA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return RA_ERR_INVALID_ARG;
  if (D > RA_MAX_D) return RA_ERR_UNSUPPORTED;
  const size_t rows = (size_t)n_dev * B * Hq * Nq;
  if (rows == 0) return RA_OK;
  if (!o || !dout || !lse || !delta || !lse2) return RA_ERR_INVALID_ARG;
  if (misaligned({o, dout}, 16) || misaligned({lse, delta, lse2}, 4)) return RA_ERR_INVALID_ARG;
  const size_t in_bytes = rows * D * elem_size(dtype);
  const void* ins[3] = {o, dout, lse};
  const size_t in_sz[3] = {in_bytes, in_bytes, rows * 4};
  for (int a = 0; a < 3; ++a)
    if (overlaps(delta, rows * 4, ins[a], in_sz[a]) || overlaps(lse2, rows * 4, ins[a], in_sz[a])) return RA_ERR_INVALID_ARG;
  if (overlaps(delta, rows * 4, lse2, rows * 4)) return RA_ERR_INVALID_ARG;
  return hip_status(ra::launch_bwd_prep(o, dout, lse, delta, lse2, n_dev, B, Hq, Nq, D, dtype, (hipStream_t)stream));
}

int ring_attn_bwd_step(const void* q, const void* k, const void* v, const void* dout, const float* lse2,
                       const float* delta, float* dq, float* dk, float* dv, int n_dev, int B, int Hq, int Hkv, int Nq,
                       int Nk, int D, int dtype, float scale, int mask, const int64_t* q_off, int64_t q_stride,
                       const int64_t* k_off, int64_t k_stride, int flags, void* stream) {
  const Shape sh{n_dev, B, Hq, Hkv, Nq, Nk, D, dtype};
  int rc = validate_shape(sh);
  if (rc != RA_OK) return rc;
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return RA_ERR_INVALID_ARG;
  if (flags & ~(RA_BWD_INIT_DQ | RA_BWD_INIT_DKV)) return RA_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.f)) return RA_ERR_INVALID_ARG;
  const bool causal = mask == RA_MASK_CAUSAL;
  if (causal && (!q_off || !k_off || q_stride <= 0 || k_stride <= 0)) return RA_ERR_INVALID_ARG;
  const size_t qrows = (size_t)n_dev * B * Nq * Hq, krows = (size_t)n_dev * B * Nk * Hkv;
  if (qrows + krows == 0) return RA_OK;
  if ((qrows > 0 && (!q || !dout || !lse2 || !delta || !dq)) || (krows > 0 && (!k || !v || !dk || !dv)))
    return RA_ERR_INVALID_ARG;
  if (misaligned({q, k, v, dout, dq, dk, dv}, 16) || misaligned({lse2, delta}, 4)) return RA_ERR_INVALID_ARG;
  // the gradients are written: they may not alias the inputs or each other
  const void* outs[3] = {dq, dk, dv};
  const size_t out_sz[3] = {qrows * D * 4, krows * D * 4, krows * D * 4};
  const void* ins[6] = {q, k, v, dout, lse2, delta};
  const size_t es = elem_size(dtype);
  const size_t in_sz[6] = {qrows * D * es, krows * D * es, krows * D * es, qrows * D * es, qrows * 4, qrows * 4};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], out_sz[a], ins[b], in_sz[b])) return RA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], out_sz[a], outs[b], out_sz[b])) return RA_ERR_INVALID_ARG;
  }
  hipStream_t st = (hipStream_t)stream;
  ra::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.lse2 = lse2;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = p.NqTot = Nq;
  p.Nk = p.NkTot = Nk;
  p.D = D;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = (float)(scale * kLog2e);
  p.q_stride = causal ? q_stride : 1;
  p.k_stride = causal ? k_stride : 1;
  for (int t = 0; t < n_dev; ++t) {
    const int64_t qo = q_off ? q_off[t] : 0, ko = k_off ? k_off[t] : 0;
    if (classify(causal, qo, p.q_stride, Nq, ko, p.k_stride, Nk) == 0) {
      // nothing visible: only an initialisation to do
      const size_t qn = (size_t)B * Nq * Hq * D, kn = (size_t)B * Nk * Hkv * D;
      hipError_t e = hipSuccess;
      if (flags & RA_BWD_INIT_DQ) e = ra::launch_zero_f32(dq + t * qn, qn, st);
      if (e == hipSuccess && (flags & RA_BWD_INIT_DKV)) e = ra::launch_zero_f32(dk + t * kn, kn, st);
      if (e == hipSuccess && (flags & RA_BWD_INIT_DKV)) e = ra::launch_zero_f32(dv + t * kn, kn, st);
      if (e != hipSuccess) return RA_ERR_HIP;
      continue;
    }
    const int x = p.n_launch++;
    p.qslot[x] = p.kvslot[x] = p.gslot[x] = t;
    p.q_row0[x] = 0;
    p.nk[x] = Nk;
    p.q_off[x] = qo;
    p.k_off[x] = ko;
    p.flags[x] = (uint8_t)(((flags & RA_BWD_INIT_DQ) ? ra::kBwdInitDq : 0) |
                           ((flags & RA_BWD_INIT_DKV) ? ra::kBwdInitDkv : 0));
    p.fwd[x] = -1;  // a single step hands nothing on
  }
  if (p.n_launch == 0) return RA_OK;
  rc = hip_status(launch_bwd(p, dtype, true, st));
  if (rc != RA_OK) return rc;
  return hip_status(launch_bwd(p, dtype, false, st));
}

size_t ring_attn_bwd_local_workspace_bytes(int P, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype) {
  if (P < 1 || P > RA_MAX_DEV || n_local < 1 || n_local > P || B < 1 || Hq < 1 || Hkv < 1 || n < 0 || D < 1 ||
      D > RA_MAX_D || Hq % Hkv || !valid_dtype(dtype))
    return 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t blk = (size_t)B * n * Hkv * D * elem_size(dtype);
  const size_t rows = (size_t)n_local * B * Hq * n;
  return 4 * up((size_t)n_local * blk) + 2 * up(rows * 4);
}

int ring_attn_bwd_local(const void* q_local, const void* k_src, const void* v_src, const void* o_local,
                        const void* dout_local, const float* lse_local, float* dq_local, float* dk, float* dv, int P,
                        int dev0, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype, float scale, int mask,
                        int layout, void* workspace, size_t workspace_bytes, void* compute_stream, void* copy_stream) {
  if (P < 1 || P > RA_MAX_DEV || dev0 < 0 || dev0 >= P || n_local < 1 || dev0 + n_local > P) return RA_ERR_INVALID_ARG;
  const Shape sh{n_local, B, Hq, Hkv, n, n, D, dtype};
  int rc = validate_shape(sh);
  if (rc != RA_OK) return rc;
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return RA_ERR_INVALID_ARG;
  if (!valid_layout(layout)) return RA_ERR_INVALID_ARG;
  if (!(std::isfinite(scale) && scale > 0.f)) return RA_ERR_INVALID_ARG;
  if (layout == RA_LAYOUT_ZIGZAG && n % 2) return RA_ERR_INVALID_ARG;
  if (n == 0) return RA_OK;
  if (!q_local || !k_src || !v_src || !o_local || !dout_local || !lse_local || !dq_local || !dk || !dv || !workspace)
    return RA_ERR_INVALID_ARG;
  if (misaligned({q_local, k_src, v_src, o_local, dout_local, dq_local, dk, dv, workspace}, 16) ||
      misaligned({lse_local}, 4))
    return RA_ERR_INVALID_ARG;
  const size_t need = ring_attn_bwd_local_workspace_bytes(P, n_local, B, Hq, Hkv, n, D, dtype);
  if (need == 0) return RA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return RA_ERR_WORKSPACE;

  const size_t es = elem_size(dtype);
  const size_t blk = (size_t)B * n * Hkv * D * es;  // one device's K (or V) block
  const size_t rows = (size_t)n_local * B * Hq * n;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* ws = (char*)workspace;
  char* stage_k[2] = {ws, ws + up((size_t)n_local * blk)};
  char* stage_v[2] = {ws + 2 * up((size_t)n_local * blk), ws + 3 * up((size_t)n_local * blk)};
  float* delta = (float*)(ws + 4 * up((size_t)n_local * blk));
  float* lse2 = (float*)((char*)delta + up(rows * 4));
  // outputs may not alias the inputs, the workspace or each other
  const size_t q_bytes = rows * D * es, src_bytes = (size_t)P * blk;
  const size_t dq_bytes = rows * D * 4, dkv_bytes = (size_t)P * B * n * Hkv * D * 4;
  const void* ins[7] = {q_local, k_src, v_src, o_local, dout_local, lse_local, workspace};
  const size_t in_sz[7] = {q_bytes, src_bytes, src_bytes, q_bytes, q_bytes, rows * 4, need};
  const void* outs[3] = {dq_local, dk, dv};
  const size_t out_sz[3] = {dq_bytes, dkv_bytes, dkv_bytes};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 7; ++b)
      if (overlaps(outs[a], out_sz[a], ins[b], in_sz[b])) return RA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], out_sz[a], outs[b], out_sz[b])) return RA_ERR_INVALID_ARG;
  }
  for (int b = 0; b < 6; ++b)
    if (overlaps(workspace, need, ins[b], in_sz[b])) return RA_ERR_INVALID_ARG;

  hipStream_t cs = (hipStream_t)compute_stream;
  hipStream_t xs = (hipStream_t)copy_stream;
  const bool causal = mask == RA_MASK_CAUSAL;
  const HopStress hs = read_hop_stress();

  // schedule over units (a device's whole query block, or one of its two zigzag chunks, as in the
  // forward): class of every (step, unit), the first computed step of each unit's query gradient and
  // the first visit of each block's key/value gradient.  Zigzag units of one device read overlapping
  // key rows of the same block, so their key/value gradients start from zero and always accumulate.
  const int nh = layout == RA_LAYOUT_ZIGZAG ? 2 : 1;
  const int n_units = n_local * nh;
  std::vector<int> cls((size_t)P * n_units);
  std::vector<int> dq_first(n_units, -1), dkv_first(P, -1);
  std::vector<uint8_t> first_flags((size_t)P * n_units, 0);
  for (int s = 0; s < P; ++s)
    for (int u = 0; u < n_units; ++u) {
      const int i = dev0 + u / nh, j = ((i - s) % P + P) % P;
      const Unit un = ring_unit(causal, layout, P, n, i, j, u % nh);
      const int c = classify(causal, un.q_off, un.stride, n / nh, un.k_off, un.stride, un.nk);
      cls[(size_t)s * n_units + u] = c;
      if (c == 0) continue;
      uint8_t f = 0;
      if (dq_first[u] < 0) {
        dq_first[u] = s;
        f |= ra::kBwdInitDq;
      }
      if (dkv_first[j] < 0) {
        dkv_first[j] = s;
        if (nh == 1) f |= ra::kBwdInitDkv;
      }
      first_flags[(size_t)s * n_units + u] = f;
    }

  hipEvent_t ev_copy[2] = {nullptr, nullptr}, ev_comp[2] = {nullptr, nullptr}, ev_fork = nullptr;
  auto cleanup = [&]() {
    for (int a = 0; a < 2; ++a) {
      if (ev_copy[a]) (void)hipEventDestroy(ev_copy[a]);
      if (ev_comp[a]) (void)hipEventDestroy(ev_comp[a]);
    }
    if (ev_fork) (void)hipEventDestroy(ev_fork);
  };
#define RA_CHECK(x)            \
  do {                         \
    hipError_t e_ = (x);       \
    if (e_ != hipSuccess) {    \
      cleanup();               \
      return RA_ERR_HIP;       \
    }                          \
  } while (0)
  for (int a = 0; a < 2; ++a) {
    RA_CHECK(hipEventCreateWithFlags(&ev_copy[a], hipEventDisableTiming));
    RA_CHECK(hipEventCreateWithFlags(&ev_comp[a], hipEventDisableTiming));
  }
  RA_CHECK(hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming));
  const bool two_streams = xs != cs;
  if (two_streams) {
    RA_CHECK(hipEventRecord(ev_fork, cs));
    RA_CHECK(hipStreamWaitEvent(xs, ev_fork, 0));
  }
  const char* ksrc = (const char*)k_src;
  const char* vsrc = (const char*)v_src;
  // Hop plan, as in the forward: with the bf16 D=128 kernels a device that computes at step s hands its
  // block to its local successor inside the step-s bwd_dq kernel (the rows it stages in LDS are stored
  // into the successor's part of slot (s+1) & 1), where every forwarded row is staged by its workgroup.
  // fwd_to[s*n_local+t]: successor fed by device t's step-s kernel (-1: none); by_kernel[s*n_local+t]:
  // device t's step-s block arrives that way.
  const bool in_step_hop = uses_mfma_kernel(dtype, D) && nh == 1;
  std::vector<int> fwd_to((size_t)P * n_local, -1);
  std::vector<uint8_t> by_kernel((size_t)P * n_local, 0);
  if (in_step_hop) {
    const int64_t st = layout_stride(layout, P);
    for (int s = 0; s + 1 < P; ++s)
      for (int t = 0; t < n_local; ++t) {
        if (cls[(size_t)s * n_units + t] == 0) continue;
        const int succ = t + 1 < n_local ? t + 1 : (n_local == P ? 0 : -1);
        if (succ < 0) continue;
        const int i = dev0 + t, j = ((i - s) % P + P) % P;
        if (!step_forward_covers(causal, block_offset(layout, P, n, i), st, n, block_offset(layout, P, n, j), st, n))
          continue;
        fwd_to[(size_t)s * n_local + t] = succ;
        by_kernel[(size_t)(s + 1) * n_local + succ] = 1;
      }
  }
  auto needs_copy = [&](int s) -> bool {  // step s >= 1 has a block that no kernel hands over
    if (s < 1 || s >= P) return false;
    for (int t = 0; t < n_local; ++t)
      if (!by_kernel[(size_t)s * n_local + t]) return true;
    return false;
  };
  // the blocks of step s >= 1 not handed over by a kernel arrive by copy into staging slot s & 1 (block
  // (i - s) mod P of the local device, copied from its source shard); step 0 reads each device's own
  // shard in place
  auto enqueue_hop = [&](int s) -> hipError_t {
    const int sl = s & 1;
    for (int t = 0; t < n_local;) {
      if (by_kernel[(size_t)s * n_local + t]) {
        ++t;
        continue;
      }
      const int j0 = ((dev0 + t - s) % P + P) % P;
      int t2 = t + 1;
      while (t2 < n_local && !by_kernel[(size_t)s * n_local + t2] && ((dev0 + t2 - s) % P + P) % P == j0 + (t2 - t))
        ++t2;  // contiguous source run
      const size_t bytes = (size_t)(t2 - t) * blk;
      hipError_t e = poison(hs, stage_k[sl] + t * blk, bytes, xs);
      if (e == hipSuccess) e = poison(hs, stage_v[sl] + t * blk, bytes, xs);
      if (e == hipSuccess)
        e = hipMemcpyAsync(stage_k[sl] + t * blk, ksrc + (size_t)j0 * blk, bytes, hipMemcpyDeviceToDevice, xs);
      if (e == hipSuccess)
        e = hipMemcpyAsync(stage_v[sl] + t * blk, vsrc + (size_t)j0 * blk, bytes, hipMemcpyDeviceToDevice, xs);
      if (e != hipSuccess) return e;
      t = t2;
    }
    return hipSuccess;
  };

  RA_CHECK(ra::launch_bwd_prep(o_local, dout_local, lse_local, delta, lse2, n_local, B, Hq, n, D, dtype, cs));
  if (nh == 2) {
    RA_CHECK(ra::launch_zero_f32(dk, dkv_bytes / 4, cs));
    RA_CHECK(ra::launch_zero_f32(dv, dkv_bytes / 4, cs));
  }
  // the fields every launch shares
  ra::BwdParams base{};
  base.q = q_local;
  base.dout = dout_local;
  base.lse2 = lse2;
  base.delta = delta;
  base.dq = dq_local;
  base.dk = dk;
  base.dv = dv;
  base.B = B;
  base.Hq = Hq;
  base.Hkv = Hkv;
  base.Nq = n / nh;
  base.NqTot = n;
  base.NkTot = n;
  base.D = D;
  base.causal = causal ? 1 : 0;
  base.scale = scale;
  base.scale_log2 = (float)(scale * kLog2e);

  // Whole ring local (dev0 = 0) with the bf16 D=128 kernels: two ring steps per query-gradient launch,
  // as in the forward.  Pair L covers steps s0 = 2L and s1 = 2L + 1.  Device i's block of s0 is in its
  // part of slot L & 1 (its own shard at L = 0); its block of s1 is what its predecessor holds at s0,
  // in device i - 1's part of the same slot (shard i - 1 at L = 0).  One bwd_dq launch folds both
  // blocks into each device's query gradient, writing it once, and hands the s1 block on to device
  // i + 1's part of slot (L + 1) & 1 where its workgroups stage all of it (push); one bwd_dkv launch
  // folds, into each block's key/value gradient, the queries of the device that holds it at s0 and of
  // that device's successor (which sees the block at s1), writing it once.  Blocks not pushed arrive
  // by copy from their source shard.  Slot L & 1 is only read and slot (L + 1) & 1 only written during
  // pair L.
  const bool two_step = in_step_hop && n_local == P && P >= 2 && steps_per_launch() == 2;
  if (two_step) {
    const int NL = (P + 1) / 2;
    const int64_t st = layout_stride(layout, P);
    auto blockj = [&](int i, int s) { return ((i - s) % P + P) % P; };
    std::vector<uint8_t> push((size_t)NL * P, 0);
    for (int L = 0; L + 1 < NL; ++L)
      for (int i = 0; i < P; ++i) {
        const int s1 = 2 * L + 1;
        if (cls[(size_t)s1 * n_units + i] == 0) continue;
        if (step_forward_covers(causal, block_offset(layout, P, n, i), st, n,
                                block_offset(layout, P, n, blockj(i, s1)), st, n))
          push[(size_t)L * P + i] = 1;
      }
    auto pair_needs_copy = [&](int L) -> bool {  // pair L's slot L & 1 has a block not pushed by pair L-1
      if (L <= 0 || L >= NL) return false;
      for (int x = 0; x < P; ++x)
        if (!push[(size_t)(L - 1) * P + (x + P - 1) % P]) return true;
      return false;
    };
    auto pair_copies = [&](int L) -> hipError_t {  // device x's block of step 2L, from its source shard
      const int sl = L & 1;
      for (int x = 0; x < P;) {
        if (push[(size_t)(L - 1) * P + (x + P - 1) % P]) {
          ++x;
          continue;
        }
        const int j0 = blockj(x, 2 * L);
        int x2 = x + 1;
        while (x2 < P && !push[(size_t)(L - 1) * P + x2 - 1] && blockj(x2, 2 * L) == j0 + (x2 - x)) ++x2;
        const size_t bytes = (size_t)(x2 - x) * blk;
        hipError_t e = poison(hs, stage_k[sl] + x * blk, bytes, xs);
        if (e == hipSuccess) e = poison(hs, stage_v[sl] + x * blk, bytes, xs);
        if (e == hipSuccess)
          e = hipMemcpyAsync(stage_k[sl] + x * blk, ksrc + (size_t)j0 * blk, bytes, hipMemcpyDeviceToDevice, xs);
        if (e == hipSuccess)
          e = hipMemcpyAsync(stage_v[sl] + x * blk, vsrc + (size_t)j0 * blk, bytes, hipMemcpyDeviceToDevice, xs);
        if (e != hipSuccess) return e;
        x = x2;
      }
      return hipSuccess;
    };
    for (int L = 0; L < NL; ++L) {
      const int s0 = 2 * L, s1 = 2 * L + 1;
      if (pair_needs_copy(L + 1)) {  // copies for pair L+1, into the slot that pair L-1 read
        if (L >= 1) RA_CHECK(hipStreamWaitEvent(xs, ev_comp[(L + 1) & 1], 0));
        RA_CHECK(jitter(hs.jitter_copy, xs));
        RA_CHECK(pair_copies(L + 1));
        RA_CHECK(hipEventRecord(ev_copy[(L + 1) & 1], xs));
      }
      if (pair_needs_copy(L)) RA_CHECK(hipStreamWaitEvent(cs, ev_copy[L & 1], 0));
      ra::BwdParams p = base;
      p.k = L == 0 ? (const void*)ksrc : (const void*)stage_k[L & 1];
      p.v = L == 0 ? (const void*)vsrc : (const void*)stage_v[L & 1];
      p.fwd_k = stage_k[(L + 1) & 1];
      p.fwd_v = stage_v[(L + 1) & 1];
      // query gradients of both steps
      p.n_launch = 0;
      for (int i = 0; i < P; ++i) {
        const bool c0 = cls[(size_t)s0 * n_units + i] != 0, c1 = s1 < P && cls[(size_t)s1 * n_units + i] != 0;
        if (!c0 && !c1) continue;
        const int x = p.n_launch++;
        const Unit u0 = ring_unit(causal, layout, P, n, i, blockj(i, s0), 0);
        p.qslot[x] = i;
        p.kvslot[x] = i;
        p.kvslot2[x] = (i + P - 1) % P;
        p.gslot[x] = blockj(i, s0);
        p.q_row0[x] = u0.row0;
        p.q_off[x] = u0.q_off;
        p.q_stride = p.k_stride = u0.stride;
        p.nk[x] = c0 ? u0.nk : 0;
        p.k_off[x] = u0.k_off;
        if (c1) {
          const Unit u1 = ring_unit(causal, layout, P, n, i, blockj(i, s1), 0);
          p.nk2[x] = u1.nk;
          p.k_off2[x] = u1.k_off;
        }
        p.Nk = std::max({p.Nk, p.nk[x], p.nk2[x]});
        p.flags[x] = dq_first[i] == s0 || dq_first[i] == s1 ? ra::kBwdInitDq : 0;
        const bool pushes = push[(size_t)L * P + i] != 0;
        p.fwd[x] = pushes ? (i + 1) % P : -1;
        if (pushes) {  // slot (L+1) & 1 was last read by pair L-1, earlier on this stream
          RA_CHECK(poison(hs, stage_k[(L + 1) & 1] + (size_t)((i + 1) % P) * blk, blk, cs));
          RA_CHECK(poison(hs, stage_v[(L + 1) & 1] + (size_t)((i + 1) % P) * blk, blk, cs));
        }
      }
      RA_CHECK(jitter(hs.jitter_compute, cs));
      if (p.n_launch > 0) RA_CHECK(launch_bwd(p, dtype, true, cs));
      // key/value gradients of both steps in one launch: block j meets the queries of a = j + s0 (step
      // s0, the device that holds it) and of b = j + s1 (step s1, which reads it from a's part of the
      // slot), and its gradient rows are written once
      ra::BwdParams pk = base;
      pk.k = p.k;
      pk.v = p.v;
      pk.n_launch = 0;
      for (int j = 0; j < P; ++j) {
        const int a = (j + s0) % P, b = (j + s1) % P;
        const bool ca = cls[(size_t)s0 * n_units + a] != 0, cb = s1 < P && cls[(size_t)s1 * n_units + b] != 0;
        if (!ca && !cb) continue;
        const int x = pk.n_launch++;
        const Unit ua = ring_unit(causal, layout, P, n, a, j, 0), ub = ring_unit(causal, layout, P, n, b, j, 0);
        const Unit& u0 = ca ? ua : ub;
        pk.qslot[x] = ca ? a : b;
        pk.kvslot[x] = a;
        pk.gslot[x] = j;
        pk.q_row0[x] = u0.row0;
        pk.q_off[x] = u0.q_off;
        pk.q_stride = pk.k_stride = u0.stride;
        pk.nk[x] = u0.nk;
        pk.k_off[x] = u0.k_off;
        pk.Nk = std::max(pk.Nk, u0.nk);
        if (ca && cb) {
          pk.two_q[x] = 1;
          pk.qslot2[x] = b;
          pk.q_off2[x] = ub.q_off;
        }
        pk.flags[x] = dkv_first[j] == s0 || dkv_first[j] == s1 ? ra::kBwdInitDkv : 0;
        pk.fwd[x] = -1;
      }
      if (pk.n_launch > 0) RA_CHECK(launch_bwd(pk, dtype, false, cs));
      if (pair_needs_copy(L + 2)) RA_CHECK(hipEventRecord(ev_comp[L & 1], cs));
    }
  }
  for (int s = 0; s < P && !two_step; ++s) {
    if (needs_copy(s + 1)) {  // copies for step s+1, into the slot that step s-1 read
      if (s >= 1) RA_CHECK(hipStreamWaitEvent(xs, ev_comp[(s + 1) & 1], 0));
      RA_CHECK(jitter(hs.jitter_copy, xs));
      RA_CHECK(enqueue_hop(s + 1));
      RA_CHECK(hipEventRecord(ev_copy[(s + 1) & 1], xs));
    }
    if (needs_copy(s)) RA_CHECK(hipStreamWaitEvent(cs, ev_copy[s & 1], 0));
    ra::BwdParams p{};
    p.q = q_local;
    p.k = s > 0 ? (const void*)stage_k[s & 1] : (const void*)(ksrc + (size_t)dev0 * blk);
    p.v = s > 0 ? (const void*)stage_v[s & 1] : (const void*)(vsrc + (size_t)dev0 * blk);
    p.dout = dout_local;
    p.lse2 = lse2;
    p.delta = delta;
    p.dq = dq_local;
    p.dk = dk;
    p.dv = dv;
    p.fwd_k = stage_k[(s + 1) & 1];
    p.fwd_v = stage_v[(s + 1) & 1];
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Nq = n / nh;
    p.NqTot = n;
    p.NkTot = n;
    p.D = D;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    p.scale_log2 = (float)(scale * kLog2e);
    // launches of step s: the query gradients of every unit (RA_MAX_DEV slots per launch), then the
    // key/value gradients, one launch per zigzag half (the two halves of a device touch the same rows)
    auto launch_units = [&](int half_sel, bool dq_pass) -> hipError_t {
      std::vector<int> todo;
      for (int u = 0; u < n_units; ++u)
        if (cls[(size_t)s * n_units + u] != 0 && (half_sel < 0 || u % nh == half_sel)) todo.push_back(u);
      for (size_t a0 = 0; a0 < todo.size(); a0 += RA_MAX_DEV) {
        p.n_launch = 0;
        p.Nk = 0;
        for (size_t a = a0; a < todo.size() && a < a0 + RA_MAX_DEV; ++a) {
          const int u = todo[a], t = u / nh;
          const int i = dev0 + t, j = ((i - s) % P + P) % P;
          const Unit un = ring_unit(causal, layout, P, n, i, j, u % nh);
          const int x = p.n_launch++;
          p.qslot[x] = p.kvslot[x] = t;
          p.gslot[x] = j;
          p.q_row0[x] = un.row0;
          p.nk[x] = un.nk;
          p.Nk = std::max(p.Nk, un.nk);
          p.q_off[x] = un.q_off;
          p.k_off[x] = un.k_off;
          p.q_stride = un.stride;  // the same for every unit of a layout
          p.k_stride = un.stride;
          p.flags[x] = first_flags[(size_t)s * n_units + u];
          const int succ = dq_pass && in_step_hop ? fwd_to[(size_t)s * n_local + t] : -1;
          p.fwd[x] = succ;
          if (succ >= 0) {  // the slot this kernel fills was last read by step s-1, earlier on this stream
            hipError_t e = poison(hs, stage_k[(s + 1) & 1] + (size_t)succ * blk, blk, cs);
            if (e == hipSuccess) e = poison(hs, stage_v[(s + 1) & 1] + (size_t)succ * blk, blk, cs);
            if (e != hipSuccess) return e;
          }
        }
        const hipError_t e = launch_bwd(p, dtype, dq_pass, cs);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    };
    RA_CHECK(jitter(hs.jitter_compute, cs));
    RA_CHECK(launch_units(-1, true));
    if (nh == 1) {
      RA_CHECK(launch_units(-1, false));
    } else {
      RA_CHECK(launch_units(0, false));
      RA_CHECK(launch_units(1, false));
    }
    if (needs_copy(s + 2)) RA_CHECK(hipEventRecord(ev_comp[s & 1], cs));
  }
  // gradients nothing contributed to: zero (a zigzag unit always sees its own block's keys)
  const size_t qn = (size_t)B * n * Hq * D, kn = (size_t)B * n * Hkv * D;
  for (int t = 0; t < n_local && nh == 1; ++t)
    if (dq_first[t] < 0) RA_CHECK(ra::launch_zero_f32(dq_local + t * qn, qn, cs));
  for (int j = 0; j < P && nh == 1; ++j)
    if (dkv_first[j] < 0) {
      RA_CHECK(ra::launch_zero_f32(dk + j * kn, kn, cs));
      RA_CHECK(ra::launch_zero_f32(dv + j * kn, kn, cs));
    }
  if (two_streams) {
    RA_CHECK(hipEventRecord(ev_copy[0], xs));
    RA_CHECK(hipStreamWaitEvent(cs, ev_copy[0], 0));
    RA_CHECK(hipEventRecord(ev_comp[0], cs));
    RA_CHECK(hipStreamWaitEvent(xs, ev_comp[0], 0));
  }
  cleanup();
#undef RA_CHECK
  return RA_OK;
}

// ------------------------------------------------------------------------------------------------
// Blockwise feed-forward after attention.

size_t ring_attn_ffn_workspace_bytes(int64_t n_tokens, int d_model, int d_ff, int64_t block_tokens) {
  if (n_tokens < 0 || block_tokens < 1) return 0;
  if (d_model < 64 || d_model > 65536 || d_model % 64 || d_ff < 64 || d_ff > 65536 || d_ff % 64) return 0;
  const int64_t rows = std::max<int64_t>(1, std::min(n_tokens, block_tokens));  // one block's tokens
  if (rows > ((int64_t)1 << 30)) return 0;  // keeps the kernels' 32-bit row indices (row + tile) in range
  return (size_t)rows * d_ff * 2;
}

int ring_attn_ffn(const void* x, const void* w1, const void* b1, const void* w2, const void* b2, void* y,
                  int64_t n_tokens, int d_model, int d_ff, int64_t block_tokens, int activation, void* workspace,
                  size_t workspace_bytes, void* stream) {
  const size_t need = ring_attn_ffn_workspace_bytes(n_tokens, d_model, d_ff, block_tokens);
  if (need == 0) return RA_ERR_INVALID_ARG;
  if (activation != RA_FFN_GELU && activation != RA_FFN_RELU) return RA_ERR_INVALID_ARG;
  if (mul_sizes({n_tokens, d_model, 2}) < 0) return RA_ERR_INVALID_ARG;
  if (n_tokens == 0) return RA_OK;
  if (!x || !w1 || !b1 || !w2 || !b2 || !y || !workspace) return RA_ERR_INVALID_ARG;
  if (misaligned({x, w1, w2, y, workspace}, 16) || misaligned({b1, b2}, 8)) return RA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return RA_ERR_WORKSPACE;
  const size_t act_bytes = (size_t)n_tokens * d_model * 2;
  const size_t w_bytes = (size_t)d_ff * d_model * 2;
  const void* ins[5] = {x, w1, b1, w2, b2};
  const size_t in_sz[5] = {act_bytes, w_bytes, (size_t)d_ff * 2, w_bytes, (size_t)d_model * 2};
  for (int a = 0; a < 5; ++a) {
    if (overlaps(workspace, need, ins[a], in_sz[a])) return RA_ERR_INVALID_ARG;
    if (a > 0 && overlaps(y, act_bytes, ins[a], in_sz[a])) return RA_ERR_INVALID_ARG;
  }
  if (y != x && overlaps(y, act_bytes, x, act_bytes)) return RA_ERR_INVALID_ARG;
  if (overlaps(y, act_bytes, workspace, need)) return RA_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  for (int64_t t0 = 0; t0 < n_tokens; t0 += block_tokens) {
    const int M = (int)std::min(block_tokens, n_tokens - t0);
    ra::FfnGemmParams up{};
    up.x = (const char*)x + t0 * d_model * 2;
    up.w = w1;
    up.bias = b1;
    up.out = workspace;
    up.M = M, up.N = d_ff, up.K = d_model;
    up.ldx = d_model, up.ldw = d_model, up.ldo = d_ff;
    hipError_t e = ra::launch_ffn_gemm_bf16(up, activation, st);
    if (e != hipSuccess) return RA_ERR_HIP;
    ra::FfnGemmParams down{};
    down.x = workspace;
    down.w = w2;
    down.bias = b2;
    down.out = (char*)y + t0 * d_model * 2;
    down.M = M, down.N = d_model, down.K = d_ff;
    down.ldx = d_ff, down.ldw = d_ff, down.ldo = d_model;
    e = ra::launch_ffn_gemm_bf16(down, ra::kFfnActNone, st);
    if (e != hipSuccess) return RA_ERR_HIP;
  }
  return RA_OK;
}

}  // extern "C"
