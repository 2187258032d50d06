/*
 * bca.h -- block-causal / staircase attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbca.so.  Plain pointers and sizes only; no HIP, torch or C++
 * types appear in the signatures.  A `stream` argument is a hipStream_t passed
 * as void* (NULL = the default stream).
 *
 * The attention computed is the one of "On-Policy Residual Learning for
 * Diffusion Language Models":
 *   - block-causal attention (thread page, highlight 3): with block size B,
 *     query i of a sequence attends to key j iff floor(j/B) <= floor(i/B),
 *     i.e. bidirectionally inside its own block and to every earlier block;
 *   - staircase packed replay (paper cards page, Figure 3 caption; thread page,
 *     Insight 3): a trajectory is a clean prefix of P tokens followed by S
 *     copies of one B-token block.  Prefix queries are block-causal inside the
 *     prefix; a query of copy c attends to the whole prefix and to copy c only;
 *   - the decode step (thread page, Result 4: each block's denoising loop):
 *     the B queries of the current block attend, unmasked, to a prefix KV cache
 *     followed by the block's own B keys/values.
 * O = softmax(scale * Q K^T restricted to admitted keys) V, and
 * LSE = ln(sum over admitted keys of exp(scale * q.k)) per query row.
 *
 * Layouts (all row-major, contiguous, every pointer 16-byte aligned):
 *   q, o, dout, dq : [total, hq,  d]
 *   k, v, dk, dv   : [total, hkv, d]
 *   lse            : [hq, total] float32
 *   cu_seqlens     : int32 [nseq + 1] on the device, cu_seqlens[0] = 0,
 *                    non-decreasing, cu_seqlens[nseq] = total; segment s holds
 *                    tokens [cu_seqlens[s], cu_seqlens[s+1]).  Segments never
 *                    attend to each other and block indices restart at the
 *                    start of every segment.
 *   s_copies       : int32 [nseq] on the device (S per segment) or NULL (all 0).
 *                    With S > 0 a segment of L tokens must satisfy
 *                    L - S*B >= 0 and (L - S*B) % B == 0.
 * GQA head map: query head h reads KV head h / (hq / hkv); hq % hkv == 0.
 * Element type: BCA_BF16 (bfloat16 inputs and outputs, float32 accumulation)
 * or BCA_F32 (float32 throughout; forward only).  LSE is always float32.
 *
 * Ownership: the caller allocates and frees every buffer, workspaces
 * included.  The library never allocates, frees or synchronises: each call
 * only enqueues kernels on `stream` and returns.  Inputs are read-only and
 * outputs must not alias inputs.  Device-array contents (cu_seqlens,
 * s_copies, the copy-group tables) and max_seqlen >= every segment length
 * are the caller's contract: they are not read on the host unless
 * BCA_VALIDATE is set (below).  A max_seqlen below a segment's length leaves
 * that segment's first query tiles unwritten.
 *
 * Device: as with HIP itself, the calling thread's current device must be
 * the device that holds the pointers and owns `stream` (the no-allocation
 * decode finds its scratch array, and the graph entry points create their
 * capture stream, on the current device).
 *
 * Errors and exceptions: no C++ exception leaves the library; a host
 * allocation that fails returns BCA_ERR_HOST_MEMORY.
 *
 * Errors: every host-detectable fault (NULL pointer, bad shape or size,
 * unsupported head_dim or dtype, scale not finite or not > 0, workspace too
 * small) is reported by the return value before anything is enqueued.  A
 * failed kernel launch returns BCA_ERR_HIP.  bca_last_error() gives a message
 * for the calling thread's most recent failure.  Faults inside kernels
 * surface at the caller's next synchronisation, as with any asynchronous GPU
 * work.
 *
 * Environment switches (read at every call; on = set and not "0"):
 *   BCA_VALIDATE  the packed entry points copy cu_seqlens, s_copies and the
 *                 copy-group tables to the host (synchronising `stream`) and
 *                 check them before any launch: cu_seqlens[0] = 0,
 *                 non-decreasing, cu_seqlens[nseq] = total, every length
 *                 <= max_seqlen; per segment S >= 0, P = L - S*B >= 0 and,
 *                 with copies, P % B == 0; group_start[0] = 0 and
 *                 non-decreasing, every pe a multiple of B in [0, P] and
 *                 non-decreasing within its segment, copies >= 0.  A table
 *                 that fails returns BCA_ERR_SHAPE and nothing is enqueued.
 *                 Not for use under graph capture (it synchronises).
 *   BCA_POISON    workspaces are filled with NaN words (by a fill kernel on
 *                 `stream`) before the kernels that use them, so that reading
 *                 a word no kernel wrote shows up in the outputs.
 */
#ifndef BCA_H
#define BCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BCA_ABI_VERSION 1

typedef enum {
  BCA_OK = 0,
  BCA_ERR_NULL = 1,        /* a required pointer is NULL */
  BCA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  BCA_ERR_DTYPE = 3,       /* element type not supported by this entry point */
  BCA_ERR_UNSUPPORTED = 4, /* head_dim or head grouping not implemented */
  BCA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  BCA_ERR_HIP = 6,         /* the HIP runtime refused a launch */
  BCA_ERR_HOST_MEMORY = 7  /* host memory for the library's own small host-side
                              arrays (validation copies, packing, graph handles)
                              could not be allocated; nothing was enqueued */
} bca_status_t;

typedef enum { BCA_F32 = 0, BCA_BF16 = 1 } bca_dtype_t;

/* Version of this ABI (BCA_ABI_VERSION of the built library). */
int32_t bca_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" for values
 * outside the enumeration). */
const char* bca_status_string(bca_status_t status);

/* Message describing the calling thread's most recent failure ("" if none).
 * The string is owned by the library and valid until the next call from the
 * same thread. */
const char* bca_last_error(void);

/*
 * Block-causal forward over packed variable-length sequences.
 *   q, k, v     : inputs (layouts above), element type `dtype`
 *   o           : output [total, hq, d], element type `dtype`
 *   lse         : output [hq, total] float32
 *   cu_seqlens  : device int32 [nseq + 1]
 *   nseq        : number of segments (>= 0; 0 enqueues nothing)
 *   max_seqlen  : an upper bound on every segment length (> 0 when total > 0)
 *   total       : number of packed tokens (cu_seqlens[nseq])
 *   hq, hkv, d  : query heads, KV heads, head_dim; d in {64, 128}
 *   block_size  : B >= 1
 *   scale       : multiplies q.k before the softmax (typically 1/sqrt(d));
 *                 finite and > 0
 * Every row of o and lse for the `total` tokens is written.
 * Equivalent to bca_staircase_fwd with s_copies = NULL.
 */
bca_status_t bca_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu_seqlens, int32_t nseq, int32_t max_seqlen,
                     int32_t total, int32_t hq, int32_t hkv, int32_t d, int32_t block_size,
                     float scale, bca_dtype_t dtype, void* stream);

/*
 * Staircase packed-replay forward.  As bca_fwd, plus
 *   s_copies : device int32 [nseq], copies S of the last block per segment
 *              (NULL = no copies, i.e. plain block-causal).
 */
bca_status_t bca_staircase_fwd(const void* q, const void* k, const void* v, void* o,
                               float* lse, const int32_t* cu_seqlens, const int32_t* s_copies,
                               int32_t nseq, int32_t max_seqlen, int32_t total, int32_t hq,
                               int32_t hkv, int32_t d, int32_t block_size, float scale,
                               bca_dtype_t dtype, void* stream);

/* Bytes of workspace bca_staircase_bwd needs: two float32 arrays of row
 * terms, [hq, total] each (each rounded up to 256 bytes): rowsum(dO * O) and
 * LSE * log2(e). */
size_t bca_staircase_bwd_workspace(int32_t total, int32_t hq, int32_t hkv, int32_t d);

/*
 * Staircase (and, with s_copies = NULL, block-causal) backward, bf16 only.
 *   q, k, v, o, lse : the forward's inputs and outputs (o and lse exactly as
 *                     produced by bca_staircase_fwd for the same inputs)
 *   dout            : dO [total, hq, d] bf16
 *   dq              : output [total, hq, d] bf16
 *   dk, dv          : outputs [total, hkv, d] bf16, summed over the hq/hkv
 *                     query heads that share each KV head
 *   workspace       : device buffer of at least
 *                     bca_staircase_bwd_workspace(total, hq, hkv, d) bytes;
 *                     contents undefined on entry and on exit
 * Other arguments as bca_staircase_fwd.
 */
bca_status_t bca_staircase_bwd(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk,
                               void* dv, const int32_t* cu_seqlens, const int32_t* s_copies,
                               int32_t nseq, int32_t max_seqlen, int32_t total, int32_t hq,
                               int32_t hkv, int32_t d, int32_t block_size, float scale,
                               bca_dtype_t dtype, void* workspace, size_t ws_bytes,
                               void* stream);

/*
 * One stage of bca_staircase_bwd, same arguments (the same formulas:
 * dS = P * (dP - delta) with delta = rowsum(dO * O), dK = scale dS^T Q,
 * dV = P^T dO, dQ = scale dS K):
 *   stage 1 : the row terms -- delta and LSE * log2(e) -- into the workspace
 *   stage 2 : dK and dV (reads the row terms)
 *   stage 3 : dQ (reads the row terms)
 *   stage 0 : all three in order (= bca_staircase_bwd)
 * Stages 2 and 3 need stage 1's workspace contents and are independent of
 * each other: after stage 1 has completed they may run in either order, or
 * concurrently on two streams.  This lets a caller time the kernels one by
 * one or overlap them with other work.  stage outside 0..3: BCA_ERR_SHAPE.
 */
bca_status_t bca_staircase_bwd_stage(int32_t stage, const void* q, const void* k, const void* v,
                                     const void* o, const float* lse, const void* dout, void* dq,
                                     void* dk, void* dv, const int32_t* cu_seqlens,
                                     const int32_t* s_copies, int32_t nseq, int32_t max_seqlen,
                                     int32_t total, int32_t hq, int32_t hkv, int32_t d,
                                     int32_t block_size, float scale, bca_dtype_t dtype,
                                     void* workspace, size_t ws_bytes, void* stream);

/*
 * General trajectory staircase (paper cards page, Figure 3 caption; thread
 * page, Insight 3: a trajectory's captured denoising states are replayed
 * together).  A segment is a clean prefix of P tokens followed by groups of
 * block copies; the copies of group g are noisy states of one block and see
 * the clean keys [0, pe_g) -- the tokens before that block -- and,
 * bidirectionally, their own B tokens; clean rows stay block-causal.
 *   group_start  : device int32 [nseq + 1]; segment s owns groups
 *                  [group_start[s], group_start[s+1])
 *   group_pe     : device int32 [groups], prefix end pe_g of each group
 *                  (a multiple of B, 0 <= pe_g <= P, non-decreasing within a
 *                  segment)
 *   group_copies : device int32 [groups], copies of each group (>= 0)
 * Group g's copies follow group g-1's, and P = L - B * (sum of the segment's
 * copies) must be >= 0 and a multiple of B when there are copies.  A segment
 * with one group whose pe is P is the plain staircase.  Other arguments,
 * layouts and errors as bca_staircase_fwd / bca_staircase_bwd (the table
 * contents, like cu_seqlens, are the caller's contract).
 */
bca_status_t bca_staircase_groups_fwd(const void* q, const void* k, const void* v, void* o,
                                      float* lse, const int32_t* cu_seqlens,
                                      const int32_t* group_start, const int32_t* group_pe,
                                      const int32_t* group_copies, int32_t nseq,
                                      int32_t max_seqlen, int32_t total, int32_t hq, int32_t hkv,
                                      int32_t d, int32_t block_size, float scale,
                                      bca_dtype_t dtype, void* stream);

bca_status_t bca_staircase_groups_bwd(const void* q, const void* k, const void* v,
                                      const void* o, const float* lse, const void* dout,
                                      void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                                      const int32_t* group_start, const int32_t* group_pe,
                                      const int32_t* group_copies, int32_t nseq,
                                      int32_t max_seqlen, int32_t total, int32_t hq, int32_t hkv,
                                      int32_t d, int32_t block_size, float scale,
                                      bca_dtype_t dtype, void* workspace, size_t ws_bytes,
                                      void* stream);

/* Bytes of workspace bca_decode needs for `num_splits` key chunks
 * (num_splits = 0: the count bca_decode would choose itself).  Returns 0 for
 * invalid sizes. */
size_t bca_decode_workspace(int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                            int32_t num_splits);

/*
 * Decode step: one block of q_len noisy queries against a KV cache, bf16 only.
 *   q          : [q_len, hq, d] bf16 (the current block's queries)
 *   k, v       : [kv_len, hkv, d] bf16; rows [0, kv_len - q_len) are the prefix
 *                cache and the last q_len rows the block's own keys/values
 *   o          : output [q_len, hq, d] bf16
 *   lse        : output [hq, q_len] float32
 *   num_splits : number of key chunks processed in parallel (split-KV) and
 *                merged by log-sum-exp weights, in [0, 256]; 0 = chosen by
 *                the library; a count above ceil(kv_len / 64) is lowered to it
 *   workspace  : device buffer of at least
 *                bca_decode_workspace(q_len, kv_len, hq, hkv, d, num_splits)
 *                bytes (may be NULL when that size is 0); contents undefined
 *                on entry and on exit
 * Every query attends to all kv_len keys (no mask).
 */
bca_status_t bca_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                        float scale, bca_dtype_t dtype, int32_t num_splits, void* workspace,
                        size_t ws_bytes, void* stream);

/*
 * bca_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as bca_decode minus
 * the workspace: the split partials go to a scratch array the library holds
 * per GPU -- 32 MiB, allocated when the library's code is loaded on that GPU
 * and kept until the process ends -- whose address is looked up on the first
 * call on each device (that device must be current).  This call itself
 * allocates and frees nothing.
 *   - A call whose partials need more than 32 MiB
 *     (bca_decode_workspace(q_len, kv_len, hq, hkv, d, num_splits) bytes)
 *     returns BCA_ERR_WORKSPACE before anything is enqueued; ask for fewer
 *     num_splits or use bca_decode with a workspace.
 *   - All calls on one GPU share its scratch array, which keeps the last
 *     call's contents: calls that overlap on one GPU (several streams or
 *     host threads with work in flight at once) race on it and may return
 *     wrong results.  Order them on one stream, or use bca_decode.
 * Nothing in the scratch array needs to start at zero.
 */
bca_status_t bca_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t q_len, int32_t kv_len, int32_t hq, int32_t hkv, int32_t d,
                                float scale, bca_dtype_t dtype, int32_t num_splits, void* stream);

/*
 * Decode step against an FP8 KV cache (the pages serve with an FP8 KV cache:
 * paper cards page, Table 11 configurations).  As bca_decode, except
 *   k8, v8            : [kv_len, hkv, d] bytes, OCP FP8 E4M3 (bias 7, no
 *                       infinities, S.1111.111 is NaN), 16-byte aligned
 *   k_scale, v_scale  : the cache holds K / k_scale and V / v_scale: the keys
 *                       and values attended are k_scale * e4m3(k8) and
 *                       v_scale * e4m3(v8) (finite, > 0)
 * q, o stay bf16; the workspace is bca_decode_workspace's (same partials).
 */
bca_status_t bca_decode_fp8(const void* q, const void* k8, const void* v8, float k_scale,
                            float v_scale, void* o, float* lse, int32_t q_len, int32_t kv_len,
                            int32_t hq, int32_t hkv, int32_t d, float scale, int32_t num_splits,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * Captured denoising loop (thread page, Result 4: each block's denoising loop
 * runs on the GPU as one captured graph, so per-step launch and scheduling
 * costs vanish at batch 1).  bca_decode_graph_create checks its arguments as
 * bca_decode does, then records `steps` consecutive bca_decode calls on these
 * buffers into a HIP graph (through a private capture stream) and
 * instantiates it.  Each bca_decode_graph_launch enqueues one replay of all
 * `steps` calls on `stream`, ordered after earlier work on that stream.
 *   steps  : 1 .. 4096
 *   graph  : receives an opaque handle (set to NULL on failure)
 * The graph keeps the raw pointers: the buffers (workspace included) must
 * stay allocated, at the same addresses and sizes, until the graph is
 * destroyed; their contents may change between launches (the caller writes a
 * step's new queries or the block's own K/V rows, then launches).  Replays of
 * one graph that overlap (two streams) race on o, lse and the workspace.
 * Unlike the other entry points, create allocates the HIP runtime's graph
 * objects; it allocates no device buffer of its own.  Launch and destroy do
 * not synchronise; destroy a graph only after its last replay has finished.
 */
typedef struct bca_decode_graph bca_decode_graph_t;

bca_status_t bca_decode_graph_create(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int32_t q_len, int32_t kv_len, int32_t hq,
                                     int32_t hkv, int32_t d, float scale, bca_dtype_t dtype,
                                     int32_t num_splits, void* workspace, size_t ws_bytes,
                                     int32_t steps, bca_decode_graph_t** graph);

/*
 * A block's whole denoising loop captured once and reused for every block
 * of a generation (thread page, Result 4; the pages time one denoising round
 * as the median over graph replays, paper cards page, Table 10 caption).  As
 * bca_decode_graph_create, except that
 *   q          : [steps, q_len, hq, d] bf16 -- step i reads q[i]
 *   o, lse     : [steps, q_len, hq, d] bf16 and [steps, hq, q_len] float32 --
 *                step i writes o[i], lse[i]
 *   k, v       : [kv_capacity, hkv, d] bf16 cache storage
 *   kv_len_dev : device int32, read by every step when the graph runs: the
 *                number of cache rows attended (the prefix so far plus the
 *                current block's own q_len rows, which are its last rows);
 *                values outside [q_len, kv_capacity] are clamped into it
 *   steps_dev  : device int32 or NULL: the number of steps a replay runs
 *                (a block that stops denoising early); the kernels of
 *                steps i >= *steps_dev return at once and leave o[i], lse[i]
 *                as they were.  NULL: all `steps` run
 * The split plan and the workspace are those of bca_decode for kv_capacity
 * keys (bca_decode_workspace(q_len, kv_capacity, ...)); splits that a
 * shorter cache leaves empty contribute nothing.  The caller updates
 * *kv_len_dev (and the cache rows, and q) between replays, with ordinary
 * device work ordered before the launch.  Launch with
 * bca_decode_graph_launch, release with bca_decode_graph_destroy.
 * Errors as bca_decode_graph_create; kv_len_dev NULL: BCA_ERR_NULL; a pointer
 * not 4-byte aligned: BCA_ERR_SHAPE.
 */
bca_status_t bca_decode_loop_create(const void* q, const void* k, const void* v, void* o,
                                    float* lse, const int32_t* kv_len_dev,
                                    const int32_t* steps_dev, int32_t q_len,
                                    int32_t kv_capacity, int32_t hq, int32_t hkv, int32_t d,
                                    float scale, bca_dtype_t dtype, int32_t num_splits,
                                    void* workspace, size_t ws_bytes, int32_t steps,
                                    bca_decode_graph_t** graph);

bca_status_t bca_decode_graph_launch(bca_decode_graph_t* graph, void* stream);

/* Releases the graph (NULL is ignored). */
void bca_decode_graph_destroy(bca_decode_graph_t* graph);

/*
 * Compute-balanced packing (paper cards page, abstract and Figure 3 caption:
 * captured states are packed and balanced by compute across GPUs; thread
 * page, Insight 3).  Host-only: these calls touch no GPU and may run anywhere.
 *
 * bca_trajectory_cost: pairs of (query, key) admitted per query head by one
 * trajectory of `seqlen` tokens with `s_copies` copies of its last block:
 * with P = seqlen - s_copies * B, n = P / B, r = P % B,
 *   B^2 n (n+1) / 2 + r (n B + r) + s_copies * B * (P + B).
 * Returns -1 for invalid arguments (P < 0, or P % B != 0 with copies).
 */
int64_t bca_trajectory_cost(int32_t seqlen, int32_t s_copies, int32_t block_size);

/*
 * Assigns `ntraj` trajectories to `nbins` bins so that the largest bin cost
 * stays small: longest-processing-time greedy -- trajectories by decreasing
 * cost (ties: lower index first), each to the bin of least cost so far (ties:
 * lower bin index).  All arrays are host memory owned by the caller:
 *   seqlens   : [ntraj] lengths in tokens;  s_copies : [ntraj] or NULL (all 0)
 *   bin_of    : out [ntraj], the bin of each trajectory
 *   bin_cost  : out [nbins], summed costs
 *   order     : out [ntraj], trajectory indices grouped by bin, each bin's in
 *               assignment order (costliest first)
 *   bin_start : out [nbins + 1], bin b's members are order[bin_start[b] ..
 *               bin_start[b+1])
 * Errors: BCA_ERR_SHAPE (ntraj < 0, nbins < 1, block_size < 1, a bad
 * trajectory), BCA_ERR_NULL; bca_pack_last_error() gives the message.
 */
bca_status_t bca_pack_balanced(const int32_t* seqlens, const int32_t* s_copies, int32_t ntraj,
                               int32_t block_size, int32_t nbins, int32_t* bin_of,
                               int64_t* bin_cost, int32_t* order, int32_t* bin_start);

/*
 * The same for general trajectory staircases (copy groups, as in
 * bca_staircase_groups_fwd).  Host arrays:
 *   bca_trajectory_cost_groups: one trajectory of `seqlen` tokens with
 *     `ngroups` groups (group_pe[g], group_copies[g]); its cost is the clean
 *     prefix's B^2 n (n+1)/2 + r (n B + r) plus group_copies[g] * B *
 *     (group_pe[g] + B) per group.  -1 for an invalid trajectory (a group's pe
 *     not a multiple of B, outside [0, P] or decreasing, copies < 0, P < 0, or
 *     P % B != 0 with copies).
 *   bca_pack_balanced_groups: trajectory t owns groups
 *     [group_start[t], group_start[t+1]) of group_pe / group_copies; outputs
 *     and errors as bca_pack_balanced.
 */
int64_t bca_trajectory_cost_groups(int32_t seqlen, const int32_t* group_pe,
                                   const int32_t* group_copies, int32_t ngroups,
                                   int32_t block_size);

bca_status_t bca_pack_balanced_groups(const int32_t* seqlens, const int32_t* group_start,
                                      const int32_t* group_pe, const int32_t* group_copies,
                                      int32_t ntraj, int32_t block_size, int32_t nbins,
                                      int32_t* bin_of, int64_t* bin_cost, int32_t* order,
                                      int32_t* bin_start);

/* Message of the calling thread's last packing failure ("" if none). */
const char* bca_pack_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BCA_H */
