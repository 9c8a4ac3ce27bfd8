/*
 * ring_attn.h — C ABI of the per-device hot path of blockwise ring attention on MI355X (gfx950).
 *
 * The method (sources are cited by page title and section):
 *   - Ultralytics glossary, "Ring Attention", section "Como funciona a atenção em anel": a sequence
 *     is split into N blocks, one per device.  Each device keeps its query block for the whole
 *     computation; in each of N steps it computes attention between its queries and the key/value
 *     block it holds, sends that block to the next device and receives one from the previous device.
 *     Partial results are combined with the accumulated softmax of flash attention: a running sum of
 *     exponentiated scores and of score-weighted values, divided one by the other at the end.  The
 *     same section notes that production kernels subtract a running maximum before exponentiating,
 *     that a causal mask leaves the devices holding the first query blocks mostly idle, and that
 *     Striped Attention evens this out by spreading the tokens uniformly over the devices.
 *   - "Sequence Parallelism and Ring Attention" (aiunderstanding.org), section "Approfondimento
 *     tecnico": online softmax keeps a running maximum and normaliser and rescales earlier partial
 *     sums when a larger value appears, so the blockwise result equals full attention.
 *   - "Ring Attention Là Gì?" (thienlv.com), section "Ring Attention Hoạt Động Thế Nào?": while a
 *     device computes with the current block it is already sending the next one.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller, except where marked "host".
 *     The caller keeps them alive until the work enqueued on the given stream(s) has completed.
 *     Tensors (q, k, v, outputs, gradients, fp32 accumulators, workspaces) are 16-byte aligned and
 *     per-row fp32 arrays (m, l, lse, lse2, delta) 4-byte aligned (biases of ring_attn_ffn 8-byte);
 *     a misaligned non-null pointer is RA_ERR_INVALID_ARG.
 *   - `stream` arguments are hipStream_t values passed as void* (NULL = the default stream).
 *     Every call only enqueues work and returns; kernel faults surface at the caller's
 *     synchronisation.  Launch failures are reported as RA_ERR_HIP.
 *   - Every call returns RA_OK (0) or a negative RA_ERR_* code.  Arguments are validated before any
 *     HIP call, so validation errors are reported without touching the GPU.  No C++ exception
 *     crosses this boundary.
 *   - bf16 tensors hold raw bfloat16 bit patterns (uint16).  Shapes are row-major, last index fastest.
 *   - Token positions: local row r of device t has global position  off[t] + r * stride.  With
 *     contiguous sharding off[t] = t*n, stride = 1; with striped sharding (token p on shard p mod P)
 *     off[t] = t, stride = P.  Under RA_MASK_CAUSAL key u is visible to query t iff pos(u) <= pos(t).
 *     The zigzag layout of ring_attn_local (shard i holds the chunks i and 2P-1-i of n/2 tokens, the
 *     second of the balancing variants named next to striped attention on "Ukulandelana
 *     Ukuhambisana Nokunakwa Kwendandatho" (aiunderstanding.org), section "Ikusasa Lokulandelana
 *     Ukufana Nokunakwa Kwendandatho") is two such runs per shard; the driver handles it.
 *   - Grouped-query attention: query head h reads key/value head h / (Hq / Hkv).
 *
 * Running state between ring steps (fp32, caller-owned, persistent across calls): the running
 * maximum and normaliser of "Sequence Parallelism and Ring Attention", section "Approfondimento
 * tecnico", kept in base 2:
 *   o_acc[dev, b, h, t, :] = sum_u 2^(x_u - m[dev,b,h,t]) * v_u
 *   l[dev, b, h, t]        = sum_u 2^(x_u - m[dev,b,h,t])
 *   where x_u = log2(e) * scale * <q_t, k_u> over the visible keys folded so far (N of them) and
 *   m is a reference exponent, or -inf while no visible key has been folded (then o_acc = 0 and
 *   l = 0).  The quotient o_acc / l and the log-sum-exp (m + log2 l) * ln 2 do not depend on which
 *   reference is used, so m need not be the running maximum X = max_u x_u.  Bounds every state
 *   written by this library satisfies (up to fp32 rounding of x):
 *     m <= X <= m + 64         m is the exact maximum of some of the folded scores; the MFMA kernel
 *                              moves it only when a 64-key tile's partial sum of 2^(x - m) over one
 *                              lane's 32 keys would pass 2^64 (the generic kernel keeps m = X)
 *     1 <= l <= N * 2^64       every folded term is at most 2^64, the largest at least 1
 *     |o_acc| <= l * max_u |v_u| (elementwise over d)
 *   A state that satisfies these bounds (for example one merged from other states by the same rule:
 *   m = max(m1, m2), l = 2^(m1 - m) l1 + 2^(m2 - m) l2, likewise o_acc) may be passed back in.
 *   Shapes: o_acc [n_dev, B, Hq, Nq, D], m and l [n_dev, B, Hq, Nq].
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define RA_F32 0  /* float32 */
#define RA_BF16 1 /* bfloat16 bit patterns */

/* mask modes */
#define RA_MASK_NONE 0
#define RA_MASK_CAUSAL 1

/* token layouts (ring_attn_local, ring_attn_plan, ring_attn_visible_pairs) */
#define RA_LAYOUT_CONTIGUOUS 0 /* shard i holds tokens [i*n, (i+1)*n) */
#define RA_LAYOUT_STRIPED 1    /* token p on shard p mod P, local row p div P */
#define RA_LAYOUT_ZIGZAG 2     /* 2P chunks of n/2 tokens; shard i holds chunk i, then chunk 2P-1-i
                                  (n must be even) */

/* status codes */
#define RA_OK 0
#define RA_ERR_INVALID_ARG (-1) /* null pointer, bad size, inconsistent shape, overlapping buffers */
#define RA_ERR_UNSUPPORTED (-2) /* valid but not implemented (e.g. head dim > 128) */
#define RA_ERR_HIP (-3)         /* a HIP runtime call or kernel launch failed */
#define RA_ERR_WORKSPACE (-4)   /* workspace too small */
#define RA_ERR_INJECTED (-5)    /* ring_attn_local stopped early by RING_ATTN_FAIL_AT_STEP (test hook) */
#define RA_ERR_SCRATCH (-6)     /* larger than the fixed scratch of ring_attn_local_noalloc */

/* ring_attn_step flags */
#define RA_STEP_INIT 1 /* ignore the incoming state: treat it as m = -inf, l = 0, o_acc = 0 */

/* ring_attn_bwd_step flags */
#define RA_BWD_INIT_DQ 1  /* overwrite dq instead of adding to it */
#define RA_BWD_INIT_DKV 2 /* overwrite dk and dv instead of adding to them */

/* ring_attn_ffn activations */
#define RA_FFN_GELU 0 /* exact gelu: z * Phi(z), Phi the standard normal CDF */
#define RA_FFN_RELU 1 /* max(z, 0) */

#define RA_MAX_DEV 64 /* largest ring size / number of devices batched into one call */
#define RA_MAX_D 128  /* largest head dimension */

/*
 * ring_attn_step — fold one key/value block into the running online-softmax state of a query
 * block, for n_dev independent (query block, key/value block) pairs at once (n_dev = 1 for one
 * device; n_dev = P to process one ring step of P emulated devices in a single launch).
 * Defining passage: the per-step attention and accumulation of the Ultralytics "Ring Attention"
 * page, section "Como funciona a atenção em anel", with the running-maximum rescaling of
 * "Sequence Parallelism and Ring Attention", section "Approfondimento tecnico".
 *
 *   q      [n_dev, B, Nq, Hq, D]  (dtype)      query block of each device (read only)
 *   k, v   [n_dev, B, Nk, Hkv, D] (dtype)      the key/value block each device holds (read only)
 *   o_acc, m, l                                running state (read unless RA_STEP_INIT, written)
 *   scale                                      multiplies q.k (pass 1/sqrt(D))
 *   mask                                       RA_MASK_NONE or RA_MASK_CAUSAL
 *   q_off, k_off  host int64[n_dev]            position offsets (may be NULL when mask is NONE)
 *   q_stride, k_stride                         position strides (> 0 under RA_MASK_CAUSAL)
 *   flags                                      RA_STEP_INIT or 0
 * Key/value blocks that are fully masked for a device (min key position > max query position)
 * are skipped without a launch; the state of that device is left as it was (or initialised to
 * the empty state under RA_STEP_INIT).  Supported: 1 <= D <= 128; bf16 with D == 128 runs the
 * MFMA kernel, every other case the generic fp32-arithmetic kernel.  Nq or Nk may be 0.
 */
int ring_attn_step(const void* q, const void* k, const void* v, float* o_acc, float* m, float* l,
                   int n_dev, int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale,
                   int mask, const int64_t* q_off, int64_t q_stride, const int64_t* k_off,
                   int64_t k_stride, int flags, void* stream);

/*
 * ring_attn_finalize — divide the accumulated numerator by the denominator after the last block
 * and produce the log-sum-exp (Ultralytics "Ring Attention", "Como funciona a atenção em anel":
 * the division happens once, at the end).
 *   o   [n_dev, B, Nq, Hq, D] (out_dtype)  o = o_acc / l, written in token-major layout
 *   lse [n_dev, B, Hq, Nq] fp32 (may be NULL)  natural log of sum_u exp(scale * <q_t, k_u>)
 * Rows with l == 0 (no visible key) get o = 0 and lse = -inf.
 */
int ring_attn_finalize(const float* o_acc, const float* m, const float* l, void* o, float* lse, int n_dev,
                       int B, int Hq, int Nq, int D, int out_dtype, void* stream);

/*
 * ring_attn_local — the whole ring schedule for the devices [dev0, dev0 + n_local) of a P-way
 * ring, run on this GPU (Ultralytics "Ring Attention", "Como funciona a atenção em anel": P steps;
 * in step s device i holds block (i - s) mod P, received from device i - 1; "Ring Attention Là
 * Gì?", "Ring Attention Hoạt Động Thế Nào?": the next block is in flight during compute).
 *
 *   q_local [n_local, B, n, Hq, D]   queries of the local devices, in shard order (dtype)
 *   k_src, v_src [P, B, n, Hkv, D]   every shard's keys/values in shard order (dtype); device
 *                                    memory, or pinned host memory when kv_src_is_host != 0
 *   o   [n_local, B, n, Hq, D]       output (dtype), token-major, in shard order
 *   lse [n_local, B, Hq, n] fp32     log-sum-exp (may be NULL)
 *   layout                           RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED or RA_LAYOUT_ZIGZAG
 *                                    (sets positions; zigzag needs n even)
 *   workspace                        device buffer of >= ring_attn_local_workspace_bytes(...) bytes:
 *                                    two staging slots of K and V for the local devices, and the
 *                                    fp32 running state
 *   compute_stream, copy_stream      hipStream_t; the step kernels run on compute_stream, the hops
 *                                    that are copies on copy_stream, double-buffered against them
 *                                    (the two may be equal)
 *   step_events  (may be NULL)       host array of 2*P hipEvent_t handles created by the caller;
 *                                    events 2s and 2s+1 carry the start and end time of the step-s
 *                                    kernel, stamped by its launch on compute_stream (no extra
 *                                    stream packets); a step with nothing to launch records both
 *                                    on compute_stream
 * Hops: a local device whose ring predecessor is also local receives the block its predecessor
 * held; otherwise the block comes from k_src/v_src.  With a device-resident source and the bf16
 * D = 128 kernel, a device that computes in step s hands its block to a local successor inside the
 * step-s kernel (the rows it stages for its own computation are stored into the successor's slot;
 * the host checks that every row of the block is staged, else it copies); every other hop is a
 * device-to-device (or, from pinned host memory, host-to-device) copy on copy_stream (always so under
 * the zigzag layout, whose query chunks are folded as two units of n/2 rows).  With a
 * device-resident source a device's own block (step 0) is read in place.  Under RA_MASK_CAUSAL,
 * fully masked blocks are still passed on but not computed.  The last step of each device writes
 * o and lse directly.  The call returns after enqueueing; both streams are left ordered after all
 * of its work.
 *
 * Workspace layout (R(x) = x rounded up to 256 bytes, blk = B*n*Hkv*D*sizeof(dtype)): K slots 0 and
 * 1 and V slots 0 and 1 of n_local blocks each (R(n_local*blk) bytes apiece), then the running state
 * of the local devices as ring_attn_step keeps it: o_acc (R(rows*D*4) bytes), m and l (R(rows*4)
 * bytes each), rows = n_local*B*Hq*n.
 *
 * Test hooks (environment variables read at every call; unset in normal use):
 *   RING_ATTN_HOP_STRESS  comma-separated: "poison" fills every receive-slot range with NaN on the
 *                         stream that is about to write it, just before the write (a read of a slot
 *                         before its block has landed, or a row the in-step hop failed to store,
 *                         then shows as NaN); "jitter-copy" / "jitter-compute" put a bounded sleep
 *                         kernel (about 0.2 ms) before each step's hop copies / each step kernel.
 *                         Results must not change.  ring_attn_bwd_local honours the same three.
 *   RING_ATTN_STEPS_PER_LAUNCH=1  one ring step per kernel launch where the whole ring is local
 *                         (n_local == P, device source, bf16, D = 128), instead of two: the second
 *                         block of a launch is pulled from the predecessor's slot and pushed on to
 *                         the successor's next slot.  The same switch applies to ring_attn_bwd_local.
 *   RING_ATTN_FAIL_AT_STEP=k  (0 <= k < P) enqueue steps [0, k) only, without the fused final
 *                         division, give every local device that has not computed yet the empty
 *                         state, join the streams and return RA_ERR_INJECTED.  The workspace state is
 *                         then the ring's checkpoint after k steps: folding the remaining blocks
 *                         with ring_attn_step and calling ring_attn_finalize completes the ring.
 */
int ring_attn_local(const void* q_local, const void* k_src, const void* v_src, int kv_src_is_host, void* o,
                    float* lse, int P, int dev0, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype,
                    float scale, int mask, int layout, void* workspace, size_t workspace_bytes,
                    void* compute_stream, void* copy_stream, void* const* step_events);

/* Workspace size in bytes for ring_attn_local with these arguments (0 on invalid arguments): the
 * device memory one device's share of the ring needs besides its inputs and outputs, namely the two
 * receive slots of key/value blocks that double-buffer the hop ("Ring Attention Là Gì?",
 * "Ring Attention Hoạt Động Thế Nào?": the next block arrives while the current one is used) and
 * the persistent fp32 running state of the local query blocks (Ultralytics "Ring Attention",
 * "Como funciona a atenção em anel": the accumulated sums each device keeps).  Pure host
 * arithmetic; no HIP call. */
size_t ring_attn_local_workspace_bytes(int P, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype);

/*
 * ring_attn_local_noalloc — ring_attn_local without a workspace argument and without any device
 * memory allocation, for callers that cannot allocate: code recorded under HIP graph capture, tight
 * serving loops, and harnesses that forbid hipMalloc.  Same arguments, schedule, kernels and results
 * as ring_attn_local, except that the receive slots and the running state live in a fixed device
 * array inside the library (ring_attn_noalloc_scratch_bytes() bytes, 64 MiB, one copy per GPU, held
 * until the process ends); the caller still passes every input and output.
 *   - Returns RA_ERR_SCRATCH when ring_attn_local_workspace_bytes(...) for these arguments exceeds
 *     that size, RA_ERR_INVALID_ARG / RA_ERR_UNSUPPORTED as ring_attn_local, RA_ERR_HIP if the array's
 *     device address cannot be obtained.
 *   - The first call on a device looks up the array's address there (hipGetSymbolAddress); no call
 *     allocates device memory.  With compute_stream == copy_stream no HIP event is created either.
 *   - Every call on one GPU uses the same array and nothing in it needs clearing between calls (each
 *     ring initialises the state it reads).  Calls that overlap on one GPU (concurrent streams, or
 *     another thread) race on it: the caller serialises them.
 */
int ring_attn_local_noalloc(const void* q_local, const void* k_src, const void* v_src, int kv_src_is_host, void* o,
                            float* lse, int P, int dev0, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype,
                            float scale, int mask, int layout, void* compute_stream, void* copy_stream,
                            void* const* step_events);

/* Size in bytes of the fixed scratch ring_attn_local_noalloc works in (host constant). */
size_t ring_attn_noalloc_scratch_bytes(void);

/*
 * ring_attn_plan — the ring schedule as a table, computed on the host (no HIP call): the N steps of
 * Ultralytics "Ring Attention", "Como funciona a atenção em anel" (in step s device i holds the
 * block its predecessor held one step earlier, i.e. block (i - s) mod P), with the block classes
 * behind the causal idling that page describes (a fully masked block is not computed).
 * For each step s in [0, P) and each local device i in [dev0, dev0 + n_local), one row of 5 int32:
 *   { s, i, j = (i - s) mod P, staging slot (s mod 2), class }
 * class: 0 = fully masked (skipped), 1 = fully visible, 2 = partially visible (masked tiles).
 * Returns RA_ERR_INVALID_ARG for an unknown layout, or zigzag with n odd.
 * out_rows (host) must hold P * n_local * 5 int32.
 */
int ring_attn_plan(int P, int dev0, int n_local, int n, int mask, int layout, int32_t* out_rows);

/* Visible (query, key) pairs between query block i and key block j of a P-way ring with n tokens
 * per block under the given mask and layout (host arithmetic; -1 on invalid arguments). */
int64_t ring_attn_visible_pairs(int P, int n, int mask, int layout, int i, int j);

/*
 * Backward pass.  The pages use ring attention to train (Ultralytics "Ring Attention", section
 * "Aplicações"; section "Como funciona a atenção em anel": striped attention raises training
 * throughput) without writing the backward out; it is read here as the exact gradient of the same
 * attention, run on the forward's ring schedule: device i keeps q_i, dO_i and the forward's lse_i and
 * accumulates dq_i; the key/value block it holds carries its own dk, dv accumulators.  For one
 * (query block, key/value block) pair, with x = log2(e) * scale * q.k:
 *   p = 2^(x - lse2), lse2 = log2(e) * lse;  dp = dO . v;  ds = p * (dp - delta), delta = sum dO * O;
 *   dq += scale * ds k;  dk += scale * ds^T q;  dv += p^T dO.
 * Supported: bf16 or fp32 inputs, 1 <= D <= 128; gradients are fp32.  bf16 with D == 128 runs the
 * MFMA kernels, every other case a plain fp32 kernel pair (correctness path, not tuned).
 */

/*
 * ring_attn_bwd_prep — per-row quantities of the backward from the forward's results.
 *   o, dout  [n_dev, B, Nq, Hq, D] (dtype)   forward output and its gradient
 *   lse      [n_dev, B, Hq, Nq] fp32         forward log-sum-exp (natural log)
 *   delta    [n_dev, B, Hq, Nq] fp32 out     sum_d dout * o
 *   lse2     [n_dev, B, Hq, Nq] fp32 out     log2(e) * lse, and +inf where lse = -inf (a row that
 *                                            sees no key: its p is then 2^(x - inf) = 0)
 * Any dtype and D <= RA_MAX_D.
 */
int ring_attn_bwd_prep(const void* o, const void* dout, const float* lse, float* delta, float* lse2, int n_dev,
                       int B, int Hq, int Nq, int D, int dtype, void* stream);

/*
 * ring_attn_bwd_step — add the gradient contributions of n_dev independent (query block, key/value
 * block) pairs: device t's queries q[t] against the block k[t], v[t], whose gradient accumulators
 * are dk[t], dv[t] (they travel with the block; the caller moves them with it).
 *   q, dout  [n_dev, B, Nq, Hq, D] dtype      lse2, delta [n_dev, B, Hq, Nq] fp32 (ring_attn_bwd_prep)
 *   k, v     [n_dev, B, Nk, Hkv, D] dtype
 *   dq       [n_dev, B, Nq, Hq, D] fp32       dk, dv [n_dev, B, Nk, Hkv, D] fp32  (in/out)
 *   flags    RA_BWD_INIT_DQ | RA_BWD_INIT_DKV, or 0 to accumulate
 * Positions, masking, scale and grouped-query heads as in ring_attn_step.  Fully masked pairs launch
 * nothing (their outputs are only zeroed when an INIT flag asks for it).  Deterministic: each output
 * row is written by one workgroup, without atomics.
 */
int ring_attn_bwd_step(const void* q, const void* k, const void* v, const void* dout, const float* lse2,
                       const float* delta, float* dq, float* dk, float* dv, int n_dev, int B, int Hq, int Hkv, int Nq,
                       int Nk, int D, int dtype, float scale, int mask, const int64_t* q_off, int64_t q_stride,
                       const int64_t* k_off, int64_t k_stride, int flags, void* stream);

/*
 * ring_attn_bwd_local — the backward ring for devices [dev0, dev0 + n_local) of a P-way ring
 * (same schedule as ring_attn_local: in step s device i holds block (i - s) mod P).
 *   q_local, o_local, dout_local [n_local, B, n, Hq, D] dtype   lse_local [n_local, B, Hq, n] fp32
 *   k_src, v_src [P, B, n, Hkv, D] dtype, device memory
 *   dq_local [n_local, B, n, Hq, D] fp32 out     gradient of the local devices' queries
 *   dk, dv   [P, B, n, Hkv, D] fp32 out          gradient of every shard's keys and values from the
 *                                                local devices' queries (the whole gradient when
 *                                                n_local == P; otherwise this GPU's share, summed over
 *                                                GPUs by the caller)
 *   layout   RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED or RA_LAYOUT_ZIGZAG (n even; the two chunks of a
 *            device run as two units, as in ring_attn_local)
 *   workspace >= ring_attn_bwd_local_workspace_bytes(...): two staging slots of K and V for the
 *             local devices, and delta / lse2
 * The blocks of steps s >= 1 arrive in a staging slot double-buffered against the kernels on
 * compute_stream (step 0 reads the shards in place).  With bf16 inputs and D = 128 (not zigzag), a
 * device that computes at step s hands its block to its local successor inside the step-s query-
 * gradient kernel, as the forward does (the rows it stages in LDS are stored into the successor's
 * slot; the host checks that every row of the block is staged); every other block is copied from its
 * source shard on copy_stream.  When, in addition, the whole ring is local (n_local == P), each pair of
 * steps 2L, 2L + 1 runs as one query-gradient and one key/value-gradient launch, with the schedule of
 * ring_attn_local's two-step launches (the gradients are the same up to fp32 summation order).  Each block's dk, dv accumulators are addressed where the block came
 * from rather than copied along (same arithmetic, no traffic).  RING_ATTN_HOP_STRESS (see
 * ring_attn_local) applies here too.  Both streams are left ordered after all of the call's work.
 */
int ring_attn_bwd_local(const void* q_local, const void* k_src, const void* v_src, const void* o_local,
                        const void* dout_local, const float* lse_local, float* dq_local, float* dk, float* dv, int P,
                        int dev0, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype, float scale, int mask,
                        int layout, void* workspace, size_t workspace_bytes, void* compute_stream, void* copy_stream);

/* Workspace size in bytes for ring_attn_bwd_local with these arguments (0 on invalid arguments). */
size_t ring_attn_bwd_local_workspace_bytes(int P, int n_local, int B, int Hq, int Hkv, int n, int D, int dtype);

/*
 * ring_attn_ffn — the position-wise feed-forward that follows attention, computed one block of
 * tokens at a time.  The context-parallelism article on cyberairomania.ro (section on Ring
 * Attention) has the method compute attention and the feed-forward block by block; the pages give no
 * formula, and the one used is the transformer's feed-forward of each token's attention output:
 *   y = act(x W1^T + b1) W2^T + b2
 *   x      [n_tokens, d_model] bf16     tokens as rows, e.g. ring_attn_local's output viewed as
 *                                       [n_local * B * n, Hq * D]
 *   w1     [d_ff, d_model] bf16         b1 [d_ff] bf16     (weights as nn.Linear stores them:
 *   w2     [d_model, d_ff] bf16         b2 [d_model] bf16   one row per output feature)
 *   y      [n_tokens, d_model] bf16 out  may be x itself (in place); no other overlap
 *   block_tokens  tokens per block (>= 1): one block's hidden activations act(x W1^T + b1),
 *                 [min(block_tokens, n_tokens), d_ff] bf16, live in the workspace; at most 2^30
 *                 tokens per block
 *   activation    RA_FFN_GELU or RA_FFN_RELU
 *   workspace     device memory, >= ring_attn_ffn_workspace_bytes(...)
 * d_model and d_ff are multiples of 64 in [64, 65536].  Products accumulate in fp32; the hidden
 * activations are rounded to bf16 before the second product, the output when stored.  Per block,
 * two kernels on `stream` (bias, activation and rounding fused into their epilogues).
 */
int ring_attn_ffn(const void* x, const void* w1, const void* b1, const void* w2, const void* b2, void* y,
                  int64_t n_tokens, int d_model, int d_ff, int64_t block_tokens, int activation, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Workspace size in bytes for ring_attn_ffn with these arguments (0 on invalid arguments). */
size_t ring_attn_ffn_workspace_bytes(int64_t n_tokens, int d_model, int d_ff, int64_t block_tokens);

/* Human-readable text for a status code (static storage; never NULL, "unknown status" for codes
 * this library does not return).  Not an operation of the method: the pages define no interface, and
 * this only names the RA_* codes above. */
const char* ring_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
