/*
 * ra.h -- C ABI of the MI355X (gfx950) ring-attention per-device library.
 *
 * What is computed.  Exact softmax attention of a device's local query chunk
 * against a sequence of key/value blocks, as in Ring Attention: every block
 * step produces a block-normalised output together with its softmax
 * log-sum-exp ("softmax_lse"), and the step results are combined through
 * their lse into an fp32 running output ("Ring Flash Attention" README on
 * github.com/zhuzilin/ring-flash-attention: the lse of each block is what
 * makes blockwise results combinable; its "Limits" section: combining bf16
 * block outputs loses accuracy, hence fp32 accumulation here).  The ring
 * itself is virtual: all N steps of one rank's share run one after another on
 * this GPU, with every rank's K/V block resident in device memory.
 *
 * Conventions (apply to every entry point):
 *  - Every call returns ra_status.  Arguments are validated before anything is
 *    enqueued: on RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED or RA_ERR_WORKSPACE
 *    nothing has been enqueued and no output written.  RA_ERR_HIP reports a
 *    failed launch, after which launches enqueued before it may still run.
 *    ra_last_error() returns a thread-local message describing the failure.
 *  - Tensors are caller-owned DEVICE memory.  The library never allocates or
 *    frees device memory; calls that need scratch take a caller workspace.
 *  - Calls are asynchronous on the caller's stream (a hipStream_t passed as
 *    void*, NULL = the null stream).  Buffers must stay alive and unmodified
 *    until the stream has finished the work.  A call enqueues kernel launches
 *    only (plus event record/wait for the fp32 per-sequence rings), with no
 *    allocation, memset or synchronisation, so it may be captured into a HIP
 *    graph and replayed; kernel timing (ra_timing_begin) must be off then, and
 *    the fp32 per-sequence rings need one eager call on the thread first (it
 *    creates their side streams and events).
 *  - Q/K/V/dO and outputs are token-major [batch, tokens, heads, head_dim]
 *    described by ra_tensor: element strides for batch, token and head; the
 *    head_dim axis is contiguous.  Base pointers and all strides must keep
 *    every row 16-byte aligned.  lse/delta buffers are dense [batch, heads, tokens].
 *  - Token positions are GLOBAL positions in the full sequence (a posmap maps
 *    a local token index to its global position).  Masks are evaluated on
 *    global positions: key j is visible to query i iff
 *      (!causal || pos_k(j) <= pos_q(i)) && seq(pos_k(j)) == seq(pos_q(i)),
 *    where seq() is the packed-sequence index given by cu_seqlens (a single
 *    array shared by q and k/v, as the reference's varlen API has it).
 *  - A row with no visible key gets out = 0 and lse = -inf.
 *  - lse is the natural log of sum_j exp(scale * <q_i, k_j>) over visible j.
 *  - Supported: head_dim 64 or 128; dtype bf16 (MFMA bf16, fp32 accumulate)
 *    or fp32 (fp32 MFMA throughout).  seq_len < 2^31.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_ABI_VERSION 3
#define RA_MAX_TIMED_LAUNCHES 65536

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1, /* a pointer, size, stride or enum is not acceptable */
  RA_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (e.g. head_dim 96) */
  RA_ERR_HIP = 3,         /* a HIP runtime call failed (message has the HIP error) */
  RA_ERR_WORKSPACE = 4    /* workspace missing or smaller than required */
} ra_status;

/* Token-to-device layouts.
 *  CONTIGUOUS: rank r owns the r-th of N equal consecutive chunks.
 *  ZIGZAG:     the sequence is cut into 2N equal chunks; rank r owns chunk r
 *              followed by chunk 2N-1-r (balances causal work; "zigzag ring"
 *              of the ring-flash-attention README).
 *  STRIPE:     token t lives on rank t mod N ("Striped Ring Attention" section
 *              of the guijiagi.com Ring Attention article; Striped Attention
 *              abstract on briefgpt.xyz). */
/* Token-to-rank layouts.  The *_VARLEN layouts apply zigzag / stripe to every
 * packed sequence of cu_seqlens on its own (the README lists zigzag and stripe
 * forms of the varlen ring function): rank r holds its part of sequence 0,
 * then of sequence 1, and so on.  They need cu_seqlens (with its host copy),
 * and every sequence length divisible by 2*world (zigzag) or world (stripe). */
typedef enum {
  RA_LAYOUT_CONTIGUOUS = 0,
  RA_LAYOUT_ZIGZAG = 1,
  RA_LAYOUT_STRIPE = 2,
  RA_LAYOUT_ZIGZAG_VARLEN = 3,
  RA_LAYOUT_STRIPE_VARLEN = 4
} ra_layout;

typedef enum { RA_DTYPE_F32 = 0, RA_DTYPE_BF16 = 1 } ra_dtype;

/* One arithmetic run of a posmap: `len` local tokens whose global positions
 * are begin, begin+stride, ...  */
typedef struct { int64_t begin, stride, len; } ra_seg;

/* Local token index -> global position: the segments are concatenated in
 * local order.  Positions must be strictly increasing over the whole map
 * (true for all three layouts), stride >= 1, nseg in {1, 2}. */
typedef struct { int32_t nseg; ra_seg seg[2]; } ra_posmap;

/* A token-major tensor: element (b, t, h, d) lives at
 * ptr + b*stride_b + t*stride_t + h*stride_h + d (in elements).  Pointer and strides
 * keep every row 16-byte aligned.  The operands read through buffer descriptors
 * (q, k, v, dout) must have (batch, head) slices below 2 GiB counting 256 rows past
 * the last one (RA_ERR_UNSUPPORTED otherwise: 32-bit offsets); results and
 * accumulators (out, dq, dk, dv and the bf16 copies) have no size limit. */
typedef struct { void* ptr; int64_t stride_b, stride_t, stride_h; } ra_tensor;

typedef struct {
  int32_t batch, heads, head_dim; /* q and k/v share `heads` (no GQA) */
  ra_dtype dtype;                 /* element type of q, k, v, dout */
  float softmax_scale;            /* <= 0 selects 1/sqrt(head_dim) */
  int32_t causal;                 /* nonzero: mask by global positions */
  const int32_t* cu_seqlens;      /* DEVICE int32 [num_seqs+1] global offsets, or NULL (one sequence) */
  const int32_t* cu_seqlens_host; /* optional HOST copy of the same array: when given it is validated
                                     (cu[0]=0, non-decreasing, cu[num_seqs]=seq_len) and used to skip
                                     ring steps with no visible pair; may be NULL */
  int32_t num_seqs;               /* entries of cu_seqlens minus one; batch must be 1 when > 0 */
  int64_t seq_len;                /* S: global tokens of the whole (virtual) ring */
} ra_problem;

/* ---- block level ------------------------------------------------------------------------ */

/* Attention of q (lq local tokens, positions qmap) against one K/V block (lk tokens,
 * positions kmap).  out_b (fp32 [b, lq, h, d]) and lse_b (fp32 [b, h, lq]) are
 * OVERWRITTEN with the block-normalised output and its lse (natural log).
 * This is one step of the ring ("Ring Flash Attention" README: each block's kernel
 * returns out and softmax_lse). */
ra_status ra_block_attn_fwd(const ra_problem* prob,
                            ra_tensor q, int64_t lq, ra_posmap qmap,
                            ra_tensor k, ra_tensor v, int64_t lk, ra_posmap kmap,
                            ra_tensor out_b, float* lse_b, void* stream);

/* In place, fp32: (out, lse) <- merge((out, lse), (out_b, lse_b)) with
 *   lse' = log(exp(lse) + exp(lse_b)),
 *   out' = exp(lse - lse') * out + exp(lse_b - lse') * out_b,
 * a side with lse = -inf contributing nothing (online-softmax update of the
 * guijiagi.com Ring Attention article, section on online softmax, written with
 * each side's (max, sum) state taken as (lse, 1)).  out/out_b fp32 [b, lq, h, d];
 * lse/lse_b fp32 [b, h, lq]. */
ra_status ra_lse_merge(const ra_problem* prob, int64_t lq,
                       ra_tensor out, float* lse, ra_tensor out_b, const float* lse_b,
                       void* stream);

/* delta[b, h, i] = sum_d dout[b, i, h, d] * out[b, i, h, d] (out fp32 final output,
 * dout in prob->dtype).  First step of the backward (textbook softmax gradient;
 * the pages give no backward). */
ra_status ra_bwd_preprocess(const ra_problem* prob, int64_t lq, ra_tensor out, ra_tensor dout,
                            float* delta, void* stream);

/* Backward of one block step using the FINAL lse and delta of the rows:
 *   P = exp(scale*q.k - lse) on visible pairs, dV += P^T dO, dS = P*(dO.V^T - delta),
 *   dQ += scale*dS K, dK += scale*dS^T Q
 * (the textbook gradient of softmax attention; the pages give no backward).
 * dq_acc (fp32 [b, lq, h, d]), dk_acc and dv_acc (fp32 [b, lk, h, d]) are ACCUMULATED
 * (+=).  For bf16 all three are updated by plain read-modify-write (no atomics);
 * for fp32 dq_acc is updated with fp32 atomics and dk_acc/dv_acc by plain
 * read-modify-write.  Calls that may run concurrently (other streams) must not
 * share any rows of these buffers. */
ra_status ra_block_attn_bwd(const ra_problem* prob,
                            ra_tensor q, int64_t lq, ra_posmap qmap,
                            ra_tensor k, ra_tensor v, int64_t lk, ra_posmap kmap,
                            ra_tensor dout, const float* lse, const float* delta,
                            ra_tensor dq_acc, ra_tensor dk_acc, ra_tensor dv_acc,
                            void* stream);

/* ---- virtual ring (one rank's share) ----------------------------------------------------- */

/* Forward of rank `rank`'s share of an N-rank ring in `layout` ("Ring Attention"
 * article on guijiagi.com, detailed-flow section: at step s the rank attends to the
 * block of rank (rank - s) mod N).
 *  q_local: [b, S/N, h, d] in prob->dtype, local tokens in layout order.
 *  k_ring, v_ring: block n of rank n at ptr + n*stride_rank elements, each [b, S/N, h, d].
 *  out: fp32 [b, S/N, h, d] and lse: fp32 [b, h, S/N], OVERWRITTEN.
 *  out_lowp: optional copy of the final output in prob->dtype (ptr NULL = none).
 * Each step's block result is folded into out/lse by the lse merge inside the
 * attention kernel's epilogue (fp32 throughout); steps without any visible pair
 * are not launched.  With a *_VARLEN layout (cu_seqlens and its host copy
 * required) the sequences never attend to each other, so each sequence's rows
 * (a contiguous run of the local tokens) run as a ring of their own.  For bf16,
 * each ring step is one launch over every sequence with visible pairs at that
 * step (up to 16 sequences per launch).  For fp32 the sequences' rings run
 * concurrently on up to 4 side streams that the library creates per host thread
 * and device on first use (default priority, kept until the process ends),
 * forked from `stream` and joined back into it with events: the work is
 * ordered on `stream` as if it ran there. */
ra_status ra_ring_fwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                      ra_tensor q_local, ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank,
                      ra_tensor out, float* lse, ra_tensor out_lowp, void* stream);

/* Backward of rank `rank`'s share.  out/lse are that rank's FINAL forward results
 * (as written by ra_ring_fwd), dout its output gradient (prob->dtype).
 *  dq: fp32 [b, S/N, h, d], OVERWRITTEN.
 *  dk_ring, dv_ring: fp32, block n at ptr + n*stride_rank_grad elements, each
 *  [b, S/N, h, d]; ACCUMULATED (+=) with this rank's contribution, so that running
 *  every rank into the same buffers yields the full gradients.
 *  workspace: device memory, 16-byte aligned, of at least ra_ring_workspace_min_bytes()
 *  bytes.  It holds delta = rowsum(dO * O) (the row term of the textbook softmax-attention
 *  gradient; the pages give no backward) and, for bf16, the bf16 dS^T of the current step
 *  when the rest of the workspace holds it: the dK/dV kernel then stores dS and dQ = dS K
 *  is one product per pair instead of a recompute of S, P and dP.  When the rest holds
 *  the dS^T of only part of a step's keys (at least 1024 keys, in whole 128-key tiles),
 *  each step runs in chunks of keys: the dK/dV kernel and the dQ-from-dS kernel once per
 *  chunk (dK/dV are the same bit for bit; dQ adds the chunks in turn, so it agrees to
 *  fp32 rounding).  With less than that, dQ is computed by the recompute kernel.
 *  The per-sequence layouts run their sequences as ra_ring_fwd does (bf16: grouped
 *  launches, every sequence with its own dS^T region side by side; no chunks). */
ra_status ra_ring_bwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                      ra_tensor q_local, ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank,
                      ra_tensor out, const float* lse, ra_tensor dout,
                      ra_tensor dq, ra_tensor dk_ring, ra_tensor dv_ring, int64_t stride_rank_grad,
                      void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ra_ring_bwd without a workspace
 * argument.  Its scratch (delta and, when it also fits, the bf16 dS^T of a step) lives in
 * a fixed device array of ra_noalloc_scratch_bytes() (32 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends; the call itself allocates
 * nothing, and nothing in the scratch needs clearing between calls (every value read is
 * written earlier in the same call).  A problem whose delta (4 * batch * heads * S/N bytes,
 * rounded up to 256) exceeds the array is rejected with RA_ERR_WORKSPACE before anything
 * is enqueued; when delta fits, the rest of the array takes the dS^T as ra_ring_bwd's
 * workspace would (whole steps, or chunks of at least 1024 keys), and with room for
 * less than that dQ comes from the recompute kernel (the minimal-workspace path).  The fp32 per-sequence layouts run their
 * sequences one after another on `stream` (no side streams).  Every call on a GPU uses
 * that GPU's one array: calls that may overlap on one GPU (other streams or threads)
 * race and must be serialised by the caller.  Other arguments and results as ra_ring_bwd. */
ra_status ra_ring_bwd_noalloc(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                              ra_tensor q_local, ra_tensor k_ring, ra_tensor v_ring, int64_t stride_rank,
                              ra_tensor out, const float* lse, ra_tensor dout,
                              ra_tensor dq, ra_tensor dk_ring, ra_tensor dv_ring, int64_t stride_rank_grad,
                              void* stream);
size_t ra_noalloc_scratch_bytes(void);

/* Bytes of device workspace for ra_ring_bwd's fastest path (0 on invalid input):
 * delta (b*h*L fp32) and, for bf16, dS^T (b*h*round_up(L, 128)^2 bf16), L = S/N.  When
 * one (batch, head) slice of that dS^T would reach 4 GiB (what a buffer descriptor
 * addresses; L above 46340), the dS^T of a chunk of keys instead: the most whole
 * 128-key tiles that keep a slice below 4 GiB and all slices within 32 GiB (the
 * backward then runs each step in chunks, see ra_ring_bwd).  For a per-sequence layout,
 * the sum of the whole dS^T size over the sequences, each with its own local length.
 * Never smaller than ra_ring_workspace_min_bytes(). */
size_t ra_ring_workspace_bytes(const ra_problem* prob, ra_layout layout, int32_t world);

/* Smallest workspace ra_ring_bwd accepts (delta only; 0 on invalid input). */
size_t ra_ring_workspace_min_bytes(const ra_problem* prob, ra_layout layout, int32_t world);

/* ---- gathered K/V share (llama3-style context parallelism) ------------------------------- */

/* Rank `rank`'s share when every rank holds the whole K/V (all-gathered) instead of
 * receiving it block by block: its local queries attend to all keys in ONE block step
 * (SourcePulse page on ring-flash-attention, "How It Works" and "Highlighted Details":
 * the llama3 variant gathers K/V first; the page recommends it for varlen use).
 *  layout: CONTIGUOUS, ZIGZAG or STRIPE (which local queries the rank holds; the
 *          per-sequence layouts are RA_ERR_UNSUPPORTED here).
 *  q_local: [b, S/N, h, d] in prob->dtype, local tokens in layout order.
 *  k_all, v_all: [b, S, h, d] in GLOBAL token order.  Only the keys the rank's queries
 *          can see are read: none past the last query position when causal, and with
 *          cu_seqlens (and its host copy) none outside the sequences of the first and
 *          last query.
 *  out: fp32 [b, S/N, h, d] and lse: fp32 [b, h, S/N], OVERWRITTEN; out_lowp optional
 *          (ptr NULL = none), the output in prob->dtype.
 * Masks as everywhere: global positions, causal flag, cu_seqlens. */
ra_status ra_gathered_fwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                          ra_tensor q_local, ra_tensor k_all, ra_tensor v_all,
                          ra_tensor out, float* lse, ra_tensor out_lowp, void* stream);

/* Backward of ra_gathered_fwd's share with its FINAL out/lse: dq fp32 [b, S/N, h, d]
 * OVERWRITTEN; dk_all, dv_all fp32 [b, S, h, d] in global order ACCUMULATED (+=) over the
 * keys the share sees, so that running every rank into the same buffers gives the full
 * gradients (a reduce-scatter on a real ring).  Workspace as for ra_ring_bwd: at least
 * ra_gathered_workspace_min_bytes() (delta; dQ then recomputes S and dP), or
 * ra_gathered_workspace_bytes() for the stored-dS path (bf16 only; the visible keys in
 * chunks when the workspace, or a 4 GiB (batch, head) slice, holds only part of them). */
ra_status ra_gathered_bwd(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank,
                          ra_tensor q_local, ra_tensor k_all, ra_tensor v_all,
                          ra_tensor out, const float* lse, ra_tensor dout,
                          ra_tensor dq, ra_tensor dk_all, ra_tensor dv_all,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of ra_gathered_bwd: its fastest path / the least it accepts (0 on invalid input). */
size_t ra_gathered_workspace_bytes(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank);
size_t ra_gathered_workspace_min_bytes(const ra_problem* prob, ra_layout layout, int32_t world, int32_t rank);

/* ---- utilities ---------------------------------------------------------------------------- */

/* host_pos_out[a] = global position of local token a of `rank` (S/N entries, host memory). */
ra_status ra_layout_positions(ra_layout layout, int64_t seq_len, int32_t world, int32_t rank,
                              int64_t* host_pos_out);

/* As ra_layout_positions, for any layout including the *_VARLEN ones:
 * cu_host[0..num_seqs] are the packed sequences' global offsets (host memory;
 * ignored by the other layouts, seq_len = cu_host[num_seqs]). */
ra_status ra_layout_positions_cu(ra_layout layout, const int32_t* cu_host, int32_t num_seqs, int32_t world,
                                 int32_t rank, int64_t* host_pos_out);

/* The posmap ra_ring_fwd/bwd use for `rank` (host struct; not for *_VARLEN layouts,
 * whose posmaps have a pair of segments per sequence). */
ra_status ra_layout_posmap(ra_layout layout, int64_t seq_len, int32_t world, int32_t rank,
                           ra_posmap* out);

/* dst[i] = bf16 of src[i] for i < n (device pointers, no alignment needed; faster when
 * both are 16-byte aligned): round to nearest, ties to even, subnormals included; a NaN
 * stays a NaN (sign and top payload bits kept, quiet bit set).  The optional low-precision
 * copies of out, dQ, dK and dV that the autograd forms return are made with it. */
ra_status ra_cast_f32_to_bf16(const float* src, void* dst, int64_t n, void* stream);

/* Kernel timing.  Between ra_timing_begin and ra_timing_end every kernel the library
 * launches from the calling thread is bracketed by a pair of HIP events recorded on the
 * launch stream.  ra_timing_end waits for the last event and writes, per launch, the
 * kernel id, the ring step (-1 outside a ring call) and the elapsed milliseconds.
 * At most `capacity` (<= RA_MAX_TIMED_LAUNCHES) launches are recorded. */
typedef struct { int32_t kernel_id; int32_t step; float ms; } ra_launch_time;
ra_status ra_timing_begin(int32_t capacity);
ra_status ra_timing_end(ra_launch_time* out, int32_t capacity, int32_t* n_out);
const char* ra_kernel_name(int32_t kernel_id);

const char* ra_status_str(ra_status s);
const char* ra_last_error(void);
int ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
